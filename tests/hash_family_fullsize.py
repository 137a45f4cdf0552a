#!/usr/bin/env python3
"""Estimation error of the two hash families at the workloads' full size (CPU, oracle only).

For each workload, on its own seeded (index, value) lists, the fp64 oracle compresses every
worker, aggregates and decodes twice: with the library's default partitioned bucket hash
(h_j(i) = P(i) 2^K + Q_j(i), all rows of an item in one partition of 2^K buckets per row)
and with independent rows (K = L).  It prints the relative l2 error of the decoded aggregate
against the exact sum of the workers' gradients, ||g_hat - sum_k g_k|| / ||sum_k g_k||, over
the merged non-zeros, for several hash seeds (the workload's own seed and the next ones), so
the difference between the families can be read against the spread over seeds.

S2 Reducer Section 3.1 and Appendix A.1 ask only that each row map items uniformly with
Pr[same bucket] = 1/m; this measures what grouping the rows does to the median estimate at
the sizes the benchmark runs.

Usage: python tests/hash_family_fullsize.py [--workloads embedding,...] [--seeds 3] [--jobs 4]
Prints a markdown table on stdout.
"""
from __future__ import annotations

import argparse
import os
import sys
import time
from multiprocessing import Pool

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as WL  # noqa: E402

DEFAULT_TILE_BYTES = 64 * 1024  # the library's default partition tile: d x 2^K fp32


def default_K(d: int, L: int) -> int:
    K = L
    while K > 0 and (d << K) * 4 > DEFAULT_TILE_BYTES:
        K -= 1
    return K


def rel_error(job):
    cid, K, seed_offset = job
    wl = WL.workload(cid)
    t0 = time.perf_counter()
    p = oracle.params_from_seed(wl.hash_seed + seed_offset, wl.d, wl.log2_w, K)
    lists = [WL.worker_sparse(cid, k) for k in range(wl.W)]
    S = np.zeros((wl.d, wl.w))
    A = np.zeros((wl.d, wl.w))
    bm = np.zeros(oracle.bitmap_words(p, wl.N), dtype=np.uint64)
    for idx, val in lists:
        e = oracle.encode_sparse(p, idx, val, wl.N)
        # the aggregation of section 3.1, one worker at a time (the running sum starts at 0)
        bm, S, A = oracle.reduce(np.stack([bm, e["bitmap"]]), np.stack([S, e["S"]]),
                                 np.stack([A, e["A"]]))
    oi, ov, _ = oracle.decode(p, wl.N, bm, S, A)
    allidx = np.concatenate([i for i, _ in lists]).astype(np.int64)
    allval = np.concatenate([v for _, v in lists]).astype(np.float64)
    sup, inv = np.unique(allidx, return_inverse=True)
    exact = np.zeros(sup.size)
    np.add.at(exact, inv, allval)
    assert np.array_equal(oi.astype(np.int64), sup)
    err = float(np.linalg.norm(ov - exact) / np.linalg.norm(exact))
    return cid, K, seed_offset, err, time.perf_counter() - t0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--workloads", default="embedding,resnet50_blocktopk,transformer_mixed,large")
    ap.add_argument("--seeds", type=int, default=3)
    ap.add_argument("--jobs", type=int, default=4)
    args = ap.parse_args()
    names = {w.name: w for w in WL.WORKLOADS}
    jobs = []
    for name in args.workloads.split(","):
        wl = names[name]
        for K in (default_K(wl.d, wl.log2_w), wl.log2_w):
            for s in range(args.seeds):
                jobs.append((wl.cid, K, s))
    with Pool(args.jobs) as pool:
        res = pool.map(rel_error, jobs, chunksize=1)
    print("| workload | d | w | K (partitioned) | rel. l2 error, partitioned | rel. l2 error, "
          "independent rows (K = L) | ratio of means |")
    print("|---|---|---|---|---|---|---|")
    for name in args.workloads.split(","):
        wl = names[name]
        Kp = default_K(wl.d, wl.log2_w)
        part = [e for c, K, _, e, _ in res if c == wl.cid and K == Kp]
        ind = [e for c, K, _, e, _ in res if c == wl.cid and K == wl.log2_w]
        fmt = lambda v: ", ".join(f"{x:.4f}" for x in v)
        print(f"| {wl.name} | {wl.d} | 2^{wl.log2_w} | {Kp} | {fmt(part)} | {fmt(ind)} | "
              f"{np.mean(part) / np.mean(ind):.4f} |")
    print(f"\n(hash seeds: each workload's own and the next {args.seeds - 1}; "
          f"oracle time per run {min(r[4] for r in res):.0f}-{max(r[4] for r in res):.0f} s)")
    return 0


if __name__ == "__main__":
    sys.exit(main())
