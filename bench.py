#!/usr/bin/env python3
"""Throughput of the sparse-sketch aggregation hot path on one MI355X.

One step = s2r_encode (all W workers) -> s2r_reduce -> s2r_decode over one batch of
synthetic gradients already resident in HBM.  The metric is gradient elements per second,
W * N / t_step, in units of 1e9, plus the fraction of the 8 TB/s HBM roofline that the
dominant phase reaches on its algorithmic bytes:

  encode  W * (4N + 8 words + 4 d w)        read gradients, write bitmaps and sketches
  reduce  (W + 1) * (4 d w + 8 words)       read W sketches/bitmaps, write one of each
  decode  8 words + min(4 d w, 4 d U) + 4N  read bitmap and sketch cells, write g_hat

(words = bitmap words, ceil(N/64) at the default per-element granularity; U = elements
queried by the decode, the set bits of the merged bitmap).  List writes and any extra
traffic of the implementation are not credited.

Besides `value` (K steps back to back, host-timed), the line reports the median and minimum
of the per-step event times, the same for `--cold-reps` steps each timed alone after an
untimed 512 MiB write that evicts L2 and the Infinity Cache, a plain streaming read of
2 GiB measured on the same GPU (the achievable read ceiling) with the step's fraction of it,
the estimation error of the decoded aggregate against the exact sum, and the CPU oracle's
rate on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload embedding]
Prints ONE JSON line on stdout; progress goes to stderr.

`python bench.py --copy-reference` instead runs a plain 1 GiB device copy (an elementwise
kernel that reads 1 GiB and writes 1 GiB), the known-size reference that scales the
FETCH_SIZE / WRITE_SIZE hardware counters into bytes.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
COPY_REF_BYTES = 1 << 30


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def build_inputs(wl, dev, hash_family: str, log2_block: int = 0, log2_part: int | None = None):
    import numpy as np
    import torch

    import count_sketch_aggregation_amd as s2r
    import workloads as WL

    if hash_family == "independent":
        K = wl.log2_w
    elif log2_part is not None:
        K = log2_part
    else:
        K = s2r.s2r_default_log2_part(wl.d, wl.log2_w)
    p = s2r.s2r_params_from_seed(wl.hash_seed, wl.d, wl.log2_w, K, log2_block=log2_block)
    ld = (wl.N + 3) // 4 * 4
    grad = torch.zeros((wl.W, ld), dtype=torch.float32, device=dev)
    nnz_max = 0
    sparse = []
    for k in range(wl.W):
        idx, val = WL.worker_sparse(wl.cid, k)
        nnz_max = max(nnz_max, idx.size)
        grad[k].index_copy_(0, torch.from_numpy(idx.astype(np.int64)).to(dev),
                            torch.from_numpy(val).to(dev))
        sparse.append((idx, val))
        log(f"  worker {k}: nnz={idx.size}")
    cap = nnz_max
    return p, grad, ld, cap, sparse


def estimation_error(wl, sparse, out_dev) -> dict:
    """Relative l2 error of the decoded aggregate against the exact sum of the workers'
    gradients, sum_k g_k, formed in fp64 with numpy from the same seeded (index, value) lists:
    ||g_hat - sum_k g_k|| / ||sum_k g_k||, over all N elements, and over the union of the
    workers' non-zeros.  Measured after the timed region."""
    import numpy as np

    idx_all = np.concatenate([x[0] for x in sparse]).astype(np.int64)
    val_all = np.concatenate([x[1] for x in sparse]).astype(np.float64)
    sup, inv = np.unique(idx_all, return_inverse=True)
    gsum = np.zeros(sup.size, dtype=np.float64)
    np.add.at(gsum, inv, val_all)
    ghat = out_dev.cpu().numpy().astype(np.float64)
    on_sup = ghat[sup] - gsum
    err2_sup = float(np.dot(on_sup, on_sup))
    off = ghat.copy()
    off[sup] = 0.0
    err2_all = err2_sup + float(np.dot(off, off))
    ref2 = float(np.dot(gsum, gsum))
    return {"rel_l2_all": round((err2_all / ref2) ** 0.5, 6) if ref2 else None,
            "rel_l2_support": round((err2_sup / ref2) ** 0.5, 6) if ref2 else None,
            "union_nnz": int(sup.size)}


def library_source_sha256() -> str:
    """sha256 over the library's sources (kernels, launchers, C header), by file name."""
    import glob
    import hashlib

    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "count_sketch_aggregation_amd", "csrc", "*")))
    files.append(os.path.join(ROOT, "include", "s2r.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str, phase: str):
    """HBM bytes per call of `phase` from the committed counter summary
    (profiles/<workload>_traffic.md: FETCH_SIZE and WRITE_SIZE passes scaled by the copy
    reference), or None if there is none or the library sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.md")
    if phase != "encode" or not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.split(":", 1)[0] in ("traffic_bytes_per_call", "source_sha256"):
                k, v = line.split(":", 1)
                vals[k] = v.strip()
    if vals.get("source_sha256") != library_source_sha256() or "traffic_bytes_per_call" not in vals:
        return None
    return int(vals["traffic_bytes_per_call"])


def cpu_baseline(wl, sparse, p_dict, budget_s: float = 20.0):
    """The fp64 oracle, single-threaded, on the first workers of the same workload until
    about `budget_s` seconds of oracle work are done (at least one worker)."""
    import numpy as np

    import oracle
    import workloads as WL

    op = oracle.params_from_constants(p_dict["d"], p_dict["log2_w"], p_dict["log2_part"],
                                      p_dict["pA"], p_dict["pB"], p_dict["hA"], p_dict["hB"],
                                      p_dict["sA"], p_dict["sB"])
    elapsed = 0.0
    encs = []
    for k in range(wl.W):
        g = WL.dense_from_sparse(wl.N, *sparse[k])
        t0 = time.perf_counter()
        encs.append(oracle.encode_dense(op, g))
        elapsed += time.perf_counter() - t0
        del g
        est_total = elapsed / len(encs) * (len(encs) + 1) * 1.5
        if est_total > budget_s:
            break
    Wp = len(encs)
    t0 = time.perf_counter()
    bm, S, A = oracle.reduce(np.stack([e["bitmap"] for e in encs]), np.stack([e["S"] for e in encs]),
                             np.stack([e["A"] for e in encs]))
    oracle.decode(op, wl.N, bm, S, A)
    elapsed += time.perf_counter() - t0
    return {
        "value": round(Wp * wl.N / elapsed / 1e9, 6),
        "unit": "G gradient-elements/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{Wp} of {wl.W} workers of the {wl.name} workload (full N={wl.N} each): "
                  f"fp64 encode of each, reduce and decode over them; {elapsed:.1f} s",
    }


def copy_reference() -> int:
    import torch

    dev = torch.device("cuda:0")
    src = torch.ones(COPY_REF_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / 3
    print(json.dumps({"copy_reference_bytes_read": COPY_REF_BYTES,
                      "copy_reference_bytes_written": COPY_REF_BYTES,
                      "GBs": round(2 * COPY_REF_BYTES / dt / 1e9, 1)}), flush=True)
    return 0


def topk_stage(args) -> int:
    """Block-wise Top-K with error feedback on the ResNet-50 workload's dense gradients
    (W=16, N=25,557,032, blocks of 256, K = 1% of the blocks), residual carried across steps.
    Algorithmic bytes: 16 per element (read gradient and residual, write output and
    residual)."""
    import numpy as np
    import torch

    import count_sketch_aggregation_amd as s2r
    import workloads as WL

    if args.gpus != 1:
        print("bench.py runs on one GPU only", file=sys.stderr)
        return 2
    cid, block = 2, 256
    wl = WL.workload(cid)
    nb = -(-wl.N // block)
    K = -(-nb // 100)
    dev = torch.device("cuda:0")
    ld = (wl.N + 3) // 4 * 4
    log(f"topk stage {wl.name}: W={wl.W} N={wl.N} block={block} K={K}")
    grad = torch.zeros((wl.W, ld), dtype=torch.float32, device=dev)
    for k in range(wl.W):
        grad[k, :wl.N] = torch.from_numpy(WL.worker_dense(cid, k)).to(dev)
    res = torch.zeros_like(grad)
    out = torch.empty_like(grad)
    sel = torch.empty((wl.W, (nb + 63) // 64), dtype=torch.int64, device=dev)
    ws = torch.empty((s2r.s2r_topk_workspace_bytes(wl.W, wl.N, block),), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream()

    def step():
        s2r.s2r_topk_ef(wl.W, grad, res, wl.N, ld, block, K, out, sel, ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for _ in range(args.steps):
        step()
    ev[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_ev = ev[0].elapsed_time(ev[1]) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    alg = 16 * wl.W * wl.N
    achieved = alg / (ms_ev * 1e-3) / 1e9
    result = {
        "metric": "G gradient-elements/s (block-wise Top-K with error feedback)",
        "value": round(wl.W * wl.N / (ms_per_step * 1e-3) / 1e9, 3),
        "unit": "G gradient-elements/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "resnet50_blocktopk dense gradients", "W": wl.W, "N": wl.N,
                   "block": block, "K": K, "error_feedback": True},
        "roofline": {"bound": "hbm", "kernel": "s2r_topk_ef", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        import oracle
        g0 = WL.worker_dense(cid, 0)
        r0 = np.zeros_like(g0)
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < 10.0 or reps == 0:
            o = oracle.topk_ef(g0, r0, block, K)
            r0 = o["residual"]
            reps += 1
        el = time.perf_counter() - t0
        result["cpu_baseline"] = {
            "value": round(reps * wl.N / el / 1e9, 6), "unit": "G gradient-elements/s",
            "cores": 1, "kind": "oracle",
            "sample": f"{reps} error-feedback steps of worker 0 (N={wl.N}), {el:.1f} s"}
    print(json.dumps(result), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="embedding",
                    help="tiny | embedding | resnet50_blocktopk | transformer_mixed | large")
    ap.add_argument("--hash", dest="hash_family", default="partitioned",
                    choices=["partitioned", "independent"])
    ap.add_argument("--block", type=int, default=0, metavar="LOG2_B",
                    help="bitmap granularity: one bit per 2^LOG2_B elements (default 0: per element)")
    ap.add_argument("--log2-part", type=int, default=None, metavar="K",
                    help="partitioned hash: 2^K buckets per partition and row (default: the "
                         "library's s2r_default_log2_part)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-reps", type=int, default=20,
                    help="extra steps timed alone after flushing the caches (0 to skip)")
    ap.add_argument("--no-error", action="store_true",
                    help="skip the estimation-error report (relative l2 error vs the exact sum)")
    ap.add_argument("--stage", default="aggregate", choices=["aggregate", "topk"],
                    help="aggregate: encode+reduce+decode (default); topk: the block-wise Top-K "
                         "with error feedback that precedes it (ResNet-50 workload)")
    ap.add_argument("--copy-reference", action="store_true",
                    help="run the 1 GiB copy that calibrates the traffic counters, then exit")
    args = ap.parse_args()
    if args.copy_reference:
        return copy_reference()
    if args.stage == "topk":
        return topk_stage(args)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the W data-parallel "
              "workers are simulated as W buffers on that GPU.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import count_sketch_aggregation_amd as s2r
    import workloads as WL

    names = {w.name: w for w in WL.WORKLOADS}
    if args.workload not in names:
        print(f"unknown workload {args.workload}; choose from {sorted(names)}", file=sys.stderr)
        return 2
    wl = names[args.workload]
    dev = torch.device("cuda:0")
    log(f"workload {wl.name}: W={wl.W} N={wl.N} d={wl.d} w=2^{wl.log2_w} hash={args.hash_family}")
    p, grad, ld, cap, sparse = build_inputs(wl, dev, args.hash_family, args.block, args.log2_part)
    buf = s2r.alloc_encode_buffers(p, wl.W, wl.N, cap, dev)
    words = s2r.s2r_block_bitmap_words(wl.N, args.block)
    bm = torch.empty(max(words, 1), dtype=torch.int64, device=dev)
    sk = torch.empty((wl.d, 1 << wl.log2_w), dtype=torch.float32, device=dev)
    out = torch.empty(wl.N, dtype=torch.float32, device=dev)
    # the merged query set holds at most every worker's touched blocks
    max_set = min(wl.N, sum(np.unique(x[0] >> args.block).size << args.block for x in sparse))
    dws = s2r.alloc_decode_workspace(p, wl.N, max_set, dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        s2r.s2r_encode(p, wl.W, grad, wl.N, ld, buf["bitmaps"], buf["sketches"], buf["idx"],
                       buf["val"], cap, buf["nnz"], buf["workspace"], stream=stream)
        if ev is not None:
            ev[1].record(stream)
        s2r.s2r_reduce(p, wl.W, wl.N, buf["bitmaps"], buf["sketches"], bm, sk, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        s2r.s2r_decode(p, wl.N, bm, sk, out, max_set=max_set, workspace=dws, stream=stream)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    nnz = buf["nnz"].cpu().numpy()
    assert all(int(x) <= cap for x in nnz), "list capacity exceeded"
    # U = elements queried by the decode (every element of every set block)
    B = 1 << args.block
    nblocks = (wl.N + B - 1) // B
    setb = np.flatnonzero(np.unpackbits(bm.cpu().numpy().view(np.uint8), bitorder="little")[:nblocks])
    U = int(setb.size) * B - ((nblocks * B - wl.N) if setb.size and setb[-1] == nblocks - 1 else 0)

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    phase_ms = {"encode": 0.0, "reduce": 0.0, "decode": 0.0}
    for ev in events:
        phase_ms["encode"] += ev[0].elapsed_time(ev[1])
        phase_ms["reduce"] += ev[1].elapsed_time(ev[2])
        phase_ms["decode"] += ev[2].elapsed_time(ev[3])
    for k in phase_ms:
        phase_ms[k] /= args.steps
    ms_per_step = wall * 1e3 / args.steps
    value = wl.W * wl.N / (ms_per_step * 1e-3) / 1e9

    dw = wl.d * (1 << wl.log2_w)
    b_alg = {
        "encode": wl.W * (4 * wl.N + 8 * words + 4 * dw),
        "reduce": (wl.W + 1) * (4 * dw + 8 * words),
        "decode": 8 * words + min(4 * dw, 4 * wl.d * U) + 4 * wl.N,
    }
    phases = {k: {"ms": round(phase_ms[k], 4), "alg_bytes": b_alg[k],
                  "alg_GBs": round(b_alg[k] / (phase_ms[k] * 1e-3) / 1e9, 1)} for k in phase_ms}
    step_ev = sorted(ev[0].elapsed_time(ev[3]) for ev in events)

    # Cold-cache repetitions: before each, an untimed 512 MiB write evicts L2 and the
    # Infinity Cache; each step is timed alone with events.  Then a plain streaming read of
    # 2 GiB on the same GPU for the measured read ceiling.
    flush = torch.empty(512 << 18, dtype=torch.float32, device=dev)
    cold = []
    for _ in range(args.cold_reps):
        flush.fill_(1.0)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        step(ev)
        torch.cuda.synchronize()
        cold.append(ev[0].elapsed_time(ev[3]))
    del flush
    cold.sort()
    big = torch.ones(512 << 20, dtype=torch.float32, device=dev)
    sink = torch.zeros(1, dtype=torch.float32, device=dev)
    nbytes = big.numel() * 4
    s2r.s2r_diag_stream_read(big, nbytes, sink, stream=stream)
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record(stream)
    for _ in range(5):
        s2r.s2r_diag_stream_read(big, nbytes, sink, stream=stream)
    r1.record(stream)
    torch.cuda.synchronize()
    read_GBs = 5 * nbytes / (r0.elapsed_time(r1) * 1e-3) / 1e9
    del big
    dom = max(phase_ms, key=phase_ms.get)
    achieved = b_alg[dom] / (phase_ms[dom] * 1e-3) / 1e9
    step_alg = sum(b_alg.values()) / (ms_per_step * 1e-3) / 1e9
    log(f"ms/step {ms_per_step:.3f}  phases {phases}  step alg GB/s {step_alg:.0f}")

    result = {
        "metric": "G gradient-elements/s (encode+reduce+decode) and % of peak HBM GB/s",
        "value": round(value, 3),
        "unit": "G gradient-elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "W": wl.W, "N": wl.N, "d": wl.d, "w": 1 << wl.log2_w,
                   "log2_part": p.log2_part, "log2_block": args.block, "hash": args.hash_family,
                   "nnz_per_worker": int(nnz.max()),
                   "set_bits_merged": U},
        "roofline": {"bound": "hbm", "kernel": f"s2r_{dom}", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(wl.name, dom)},
        "step_alg_GBs": round(step_alg, 1),
        "step_hbm_frac": round(step_alg / HBM_PEAK_GBS, 4),
        "step_ms_events": {"median": round(step_ev[len(step_ev) // 2], 4), "min": round(step_ev[0], 4)},
        "cold_cache_step_ms": ({"median": round(cold[len(cold) // 2], 4), "min": round(cold[0], 4),
                                "reps": len(cold)} if cold else None),
        "measured_read_GBs": round(read_GBs, 1),
        "step_frac_of_measured_read": round(step_alg / read_GBs, 4),
        "phases": phases,
    }
    if not args.no_error:
        log("estimation error vs the exact sum ...")
        result["estimation_error"] = estimation_error(wl, sparse, out)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(wl, sparse, p.as_dict())
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
