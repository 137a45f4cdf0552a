#!/usr/bin/env python3
"""Throughput of the sparse-sketch aggregation hot path on one MI355X.

One step = s2r_encode (all W workers) -> s2r_reduce -> s2r_decode over one batch of
synthetic gradients already resident in HBM.  The metric is gradient elements per second,
W * N / t_step, in units of 1e9, and the fraction of the 8 TB/s HBM peak the step reaches
on its algorithmic bytes:

  encode  W * (4N + 8 words + 4 d w)        read gradients, write bitmaps and sketches
  reduce  (W + 1) * (4 d w + 8 words)       read W sketches/bitmaps, write one of each
  decode  8 words + min(4 d w, 4 d U) + 4N  read bitmap and sketch cells, write g_hat

(words = bitmap words, ceil(N/64) at the default per-element granularity; U = elements
queried by the decode, the set bits of the merged bitmap).  List writes and any extra
traffic of the implementation are not credited.  The default workload is `large`
(W = 8, N = 1e9), the largest configuration.

`value` and `ms_per_step` come from K steps back to back, host-timed, with nothing else on
the stream.  K more steps with events between the three calls give the phase split
(`phases`) and the per-step event times, and the same K steps are then run again with the
library's kernel trace attached (HIP events recorded on the
library's stream around every launch, include/s2r_diag.h): `kernels` lists each kernel's
average launch time and its algorithmic bytes per launch, and `roofline` is the dominant
kernel's algorithmic bytes per launch over its average launch time against the 8 TB/s
peak.  The line also carries the median and minimum per-step event times, cold-cache steps
(each timed alone after an untimed 512 MiB write that evicts L2 and the Infinity Cache), a
plain streaming read and a plain streaming write of 2 GiB on the same GPU (the achievable
read and write rates), the same plain read over the gradient rows themselves (the read rate
at the size the encode streams, which falls with size), the sketch
ratio lambda both ways, the estimation error of the decoded aggregate against the exact sum
formed on the GPU by the lossless comparator (s2r_gather_sum, which is timed too), and the
CPU oracle's rate on a bounded sample of the same workload with the host's identity.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload large]
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


def kernel_alg_bytes(name: str, wl, W: int, ewords: int, bwords: int, nnz_total: int, U: int):
    """Algorithmic bytes of one launch of a library kernel (what its step must move at
    least; list writes, partition round trips and atomic read-modify-writes are not
    credited).  None for kernels whose work is not a byte stream (scans, list expansion)."""
    N, dw = wl.N, wl.d * wl.w
    table = {
        "k_stream": W * (4 * N + 8 * ewords),            # read gradient, write bitmap
        "k_blockbits": W * 8 * (ewords + bwords),
        "k_bin": 16 * nnz_total,                         # read and write (index, value)
        "k_accumulate": 8 * nnz_total + 4 * W * dw,      # read pairs, write sketch
        "k_scatter": 8 * nnz_total,
        "k_fill_zero": 4 * W * dw,
        "k_reduce": (W + 1) * (4 * dw + 8 * bwords),     # W sketches + bitmaps in, one out
        "k_dcount": 8 * bwords,
        "k_dbin": 8 * bwords + 6 * U,                    # bitmap in, index + rank slot out
        "k_dmedian": 4 * dw + 8 * U,                     # cells once, index in, median out
        "k_dunsort": 10 * U,
        "k_dwrite": 8 * bwords + 4 * N + 4 * U,          # bitmap and medians in, g_hat out
        "k_dwrite_direct": 8 * bwords + 4 * N + min(4 * dw, 4 * wl.d * U),
    }
    return table.get(name)


def library_source_sha256(files) -> str:
    """sha256 over the named library sources (relative to the repository root)."""
    import hashlib

    h = hashlib.sha256()
    for f in sorted(files):
        h.update(os.path.basename(f).encode())
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary
    profiles/<kernel>_<workload>_traffic.md (FETCH_SIZE and WRITE_SIZE passes, each scaled by
    what the counter reads for a plain copy of known size), or None if there is none or the
    sources it names have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line:
                k, v = line.split(":", 1)
                if k in ("traffic_bytes_per_launch", "source_sha256", "source_files"):
                    vals[k] = v.strip()
    if not {"traffic_bytes_per_launch", "source_sha256", "source_files"} <= set(vals):
        return None
    if library_source_sha256(vals["source_files"].split()) != vals["source_sha256"]:
        return None
    return int(vals["traffic_bytes_per_launch"])


def host_identity() -> dict:
    """CPU model and core counts of the host the CPU baseline ran on."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": len(os.sched_getaffinity(0)),
            "cpu_count": os.cpu_count()}


def cpu_baseline(wl, sparse, p_dict, budget_s: float = 20.0):
    """The fp64 oracle, single-threaded, on the first workers of the same workload (each at
    its full N) until about `budget_s` seconds of oracle work are done (at least one
    worker): encode of each, then reduce and decode over them."""
    import numpy as np

    import oracle
    import workloads as WL

    op = oracle.params_from_constants(p_dict["d"], p_dict["log2_w"], p_dict["log2_part"],
                                      p_dict["pA"], p_dict["pB"], p_dict["hA"], p_dict["hB"],
                                      p_dict["sA"], p_dict["sB"], log2_block=p_dict["log2_block"])
    elapsed = 0.0
    encs = []
    for k in range(wl.W):
        g = WL.dense_from_sparse(wl.N, *sparse[k])
        t0 = time.perf_counter()
        # the list capacity the GPU path gets: the largest worker's non-zero count
        encs.append(oracle.encode_dense(op, g, cap=max(x[0].size for x in sparse)))
        elapsed += time.perf_counter() - t0
        del g
        # reduce + decode cost about as much again as the encodes (more for sparse bitmaps)
        est_total = elapsed / len(encs) * (len(encs) + 1) * 2.0
        if est_total > budget_s:
            break
    Wp = len(encs)
    t0 = time.perf_counter()
    bm, S, A = oracle.reduce(np.stack([e["bitmap"] for e in encs]), np.stack([e["S"] for e in encs]),
                             np.stack([e["A"] for e in encs]))
    del encs
    oracle.decode(op, wl.N, bm, S, A)
    elapsed += time.perf_counter() - t0
    return {
        "value": round(Wp * wl.N / elapsed / 1e9, 6),
        "unit": "G gradient-elements/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{Wp} of {wl.W} workers of the {wl.name} workload (full N={wl.N} each): "
                  f"fp64 encode of each, reduce and decode over them; {elapsed:.1f} s",
        "host": host_identity(),
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
    Algorithmic bytes of the step: 16 per element (read gradient and residual, write output
    and residual); the roofline names the dominant kernel with the bytes of its own pass."""
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus})", file=sys.stderr)
        return 2
    import numpy as np
    import torch

    import count_sketch_aggregation_amd as s2r
    import workloads as WL

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
    # per-kernel durations from the library's kernel trace; the two streaming passes are
    # credited with the bytes their design moves (the norm pass reads the gradient and the
    # residual and writes g = gradient + residual back into the residual; the apply pass
    # reads g and writes the output, plus 4 B per element of a kept block for its residual)
    kernels = {}
    if not args.no_trace:
        per, _ = traced_steps(step, args.steps, stream)
        kb = {"k_tk_norm": 12 * wl.W * wl.N, "k_tk_apply": 8 * wl.W * wl.N + 4 * wl.W * K * block}
        for name, (nl, ms) in sorted(per.items(), key=lambda kv: -kv[1][1]):
            us = ms * 1e3 / nl
            ab = kb.get(name)
            kernels[name] = {"avg_us": round(us, 2), "launches_per_step": round(nl / args.steps, 3),
                             "alg_bytes_per_launch": ab,
                             "alg_GBs": round(ab / (us * 1e-6) / 1e9, 1) if ab else None}
    if kernels:
        dom = max(kernels, key=lambda k: kernels[k]["avg_us"] * kernels[k]["launches_per_step"])
        kd = kernels[dom]
        roofline = {"bound": "hbm", "kernel": dom, "achieved": kd["alg_GBs"],
                    "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(kd["alg_GBs"] / HBM_PEAK_GBS, 4) if kd["alg_GBs"] else None,
                    "traffic": measured_traffic("resnet50_topk", dom),
                    "alg_bytes_per_launch": kd["alg_bytes_per_launch"],
                    "avg_launch_us": kd["avg_us"],
                    "timing": "HIP events recorded by the library on its stream around each "
                              f"launch of {dom} over {args.steps} traced steps"}
    else:  # no trace: the call as a whole
        roofline = {"bound": "hbm", "kernel": "s2r_topk_ef (a call, not one kernel)",
                    "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None}
    result = {
        "metric": "G gradient-elements/s (block-wise Top-K with error feedback)",
        "value": round(wl.W * wl.N / (ms_per_step * 1e-3) / 1e9, 3),
        "unit": "G gradient-elements/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "resnet50_blocktopk dense gradients", "W": wl.W, "N": wl.N,
                   "block": block, "K": K, "error_feedback": True},
        "roofline": roofline,
        "step_alg_GBs": round(achieved, 1), "step_hbm_frac": round(achieved / HBM_PEAK_GBS, 4),
        "kernels": kernels,
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


def traced_steps(step, steps: int, stream):
    """Runs `steps` more steps with a kernel trace attached (include/s2r_diag.h): the library
    records a HIP event on its stream before every kernel it launches and after each call's
    last launch.  Returns {kernel: (launches, total ms)} over those steps and their wall ms."""
    import torch

    import count_sketch_aggregation_amd as s2r

    traces = []
    for _ in range(steps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(s2r.TRACE_MAX)]
        for e in evs:
            e.record(stream)  # creates the event; the library records it again below
        t = s2r.s2r_trace()
        t.capacity = s2r.TRACE_MAX
        t.count = 0
        for i, e in enumerate(evs):
            t.events[i] = e.cuda_event
        traces.append((t, evs))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t, _ in traces:
        s2r.s2r_diag_trace_attach(t)
        try:
            step()
        finally:
            s2r.s2r_diag_trace_attach(None)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    per = {}
    for t, evs in traces:
        for i in range(t.count - 1):
            name = t.names[i].decode()
            if name == "end":
                continue
            n, ms = per.get(name, (0, 0.0))
            per[name] = (n + 1, ms + evs[i].elapsed_time(evs[i + 1]))
    return per, wall_ms


def gpu_estimation_error(s2r, wl, cap, buf, out, stream) -> dict:
    """Relative l2 error of the decoded aggregate against the exact sum of the workers'
    gradients, ||g_hat - sum_k g_k|| / ||sum_k g_k||, with the exact sum formed on the GPU by
    the lossless comparator (s2r_gather_sum over the encode's own lists, an fp32 sum in worker
    order, within (W - 1) 2^-24 relative of the exact real sum) and both norms accumulated
    in fp64 on the device.  Also times the comparator: HIP events around 20 calls (ms), and
    its kernels alone from the library's per-launch events over 5 more (kernel_ms)."""
    import torch

    exact = torch.empty(wl.N, dtype=torch.float32, device=out.device)

    def gather():
        s2r.s2r_gather_sum(wl.W, buf["idx"], buf["val"], cap, buf["nnz"], wl.N, exact, stream=stream)

    gather()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record(stream)
    for _ in range(reps):
        gather()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    # the comparator's kernels alone: the library's per-launch events over 5 more calls
    traced = 5
    per, _ = traced_steps(gather, traced, stream)
    kernel_ms = sum(t for _, t in per.values()) / traced
    err2 = ref2 = err2_listed = 0.0
    listed = 0
    chunk = 1 << 27
    for a in range(0, wl.N, chunk):
        x = exact[a:a + chunk].double()
        y = out[a:a + chunk].double()
        dif = y - x
        on = x != 0
        err2 += float((dif * dif).sum())
        err2_listed += float((dif[on] * dif[on]).sum())
        ref2 += float((x * x).sum())
        listed += int(on.sum())
    nnz_total = int(buf["nnz"].sum())
    return {
        "rel_l2_all": round((err2 / ref2) ** 0.5, 6) if ref2 else None,
        "rel_l2_on_nonzero_sum": round((err2_listed / ref2) ** 0.5, 6) if ref2 else None,
        "nonzero_sum_elements": listed,
        "exact_sum": "s2r_gather_sum (lossless comparator) on the device",
        "lossless_comparator": {
            "ms": round(ms, 4),
            "kernel_ms": round(kernel_ms, 4),
            "kernels_avg_us": {k: round(t / n * 1e3, 2) for k, (n, t) in per.items()},
            "G_elem_s": round(wl.W * wl.N / (ms * 1e-3) / 1e9, 3),
            # zero-fill of the dense output, then W list reads and scattered adds
            "alg_bytes": 4 * wl.N + 8 * nnz_total,
            "note": "consumes the compacted lists the encode writes; the sketch step's time "
                    "includes producing them",
        },
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="large",
                    help="tiny | embedding | resnet50_blocktopk | transformer_mixed | large "
                         "(default: large, the largest single-GPU configuration)")
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
                    help="skip the estimation error and the lossless comparator")
    ap.add_argument("--no-trace", action="store_true",
                    help="skip the per-kernel event trace (the roofline then falls back to the "
                         "dominant call)")
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
    ewords = s2r.s2r_bitmap_words(wl.N)
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
    nnz_total = int(nnz.sum())
    # U = elements queried by the decode (every element of every set block)
    B = 1 << args.block
    nblocks = (wl.N + B - 1) // B
    setb = np.flatnonzero(np.unpackbits(bm.cpu().numpy().view(np.uint8), bitorder="little")[:nblocks])
    U = int(setb.size) * B - ((nblocks * B - wl.N) if setb.size and setb[-1] == nblocks - 1 else 0)

    # --- the timed region: K steps back to back, host clock around them -----------------
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # --- phase split: K more steps with events between the calls (outside the timed region:
    # on this stack an event between two kernels costs several microseconds of the step)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
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
    step_alg = sum(b_alg.values()) / (ms_per_step * 1e-3) / 1e9

    # --- per-kernel durations: the same steps again with the kernel trace attached -------
    kernels = {}
    traced_ms = None
    if not args.no_trace:
        per, traced_wall = traced_steps(step, args.steps, stream)
        traced_ms = traced_wall / args.steps
        for name, (n, ms) in sorted(per.items(), key=lambda kv: -kv[1][1]):
            us = ms * 1e3 / n
            ab = kernel_alg_bytes(name, wl, wl.W, ewords, words, nnz_total, U)
            kernels[name] = {"avg_us": round(us, 2), "launches_per_step": round(n / args.steps, 3),
                             "alg_bytes_per_launch": ab,
                             "alg_GBs": round(ab / (us * 1e-6) / 1e9, 1) if ab else None}
    if kernels:
        dom = max(kernels, key=lambda k: kernels[k]["avg_us"] * kernels[k]["launches_per_step"])
        kd = kernels[dom]
        achieved = kd["alg_GBs"]
        roofline = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4) if achieved else None,
                    "traffic": measured_traffic(wl.name, dom),
                    "alg_bytes_per_launch": kd["alg_bytes_per_launch"], "avg_launch_us": kd["avg_us"],
                    "timing": "HIP events recorded by the library on its stream around each launch "
                              f"of {dom} over {args.steps} traced steps"}
    else:  # no trace: the dominant call, as a whole
        domc = max(phase_ms, key=phase_ms.get)
        achieved = b_alg[domc] / (phase_ms[domc] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": f"s2r_{domc} (a call, not one kernel)",
                    "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None}

    # --- cold-cache repetitions and the measured read and write ceilings -----------------
    # Before each cold step an untimed 512 MiB write evicts L2 and the Infinity Cache; each
    # step is timed alone with events.  Then a plain streaming read and write of 2 GiB.
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
    s2r.s2r_diag_stream_write(big, nbytes, 0.0, stream=stream)
    r0.record(stream)
    for _ in range(5):
        s2r.s2r_diag_stream_write(big, nbytes, 0.0, stream=stream)
    r1.record(stream)
    torch.cuda.synchronize()
    write_GBs = 5 * nbytes / (r0.elapsed_time(r1) * 1e-3) / 1e9
    del big
    # the same plain read over the W gradient rows themselves: the read rate at the size the
    # encode streams (it falls with the size read)
    gbytes = grad.numel() * grad.element_size()
    r0.record(stream)
    for _ in range(3):
        s2r.s2r_diag_stream_read(grad, gbytes, sink, stream=stream)
    r1.record(stream)
    torch.cuda.synchronize()
    grad_read_GBs = 3 * gbytes / (r0.elapsed_time(r1) * 1e-3) / 1e9
    log(f"ms/step {ms_per_step:.3f}  phases {phases}  step alg GB/s {step_alg:.0f}  "
        f"roofline {roofline['kernel']} {roofline['achieved']} GB/s")

    lam = {"dw_over_nnz": s2r.s2r_sketch_lambda(wl.d, wl.log2_w, int(nnz.max())),
           "w_over_nnz": s2r.s2r_sketch_lambda(wl.d, wl.log2_w, int(nnz.max()), per_row=True),
           "dw_over_merged": s2r.s2r_sketch_lambda(wl.d, wl.log2_w, U),
           "w_over_merged": s2r.s2r_sketch_lambda(wl.d, wl.log2_w, U, per_row=True)}
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
                   "nnz_per_worker": int(nnz.max()), "set_bits_merged": U,
                   "lambda": {k: round(v, 4) for k, v in lam.items()}},
        "roofline": roofline,
        "step_alg_GBs": round(step_alg, 1),
        "step_hbm_frac": round(step_alg / HBM_PEAK_GBS, 4),
        "step_ms_events": {"median": round(step_ev[len(step_ev) // 2], 4), "min": round(step_ev[0], 4)},
        "traced_ms_per_step": round(traced_ms, 4) if traced_ms else None,
        "cold_cache_step_ms": ({"median": round(cold[len(cold) // 2], 4), "min": round(cold[0], 4),
                                "reps": len(cold)} if cold else None),
        "measured_read_GBs": round(read_GBs, 1),
        "measured_write_GBs": round(write_GBs, 1),
        "measured_read_GBs_gradient_size": {
            "GBs": round(grad_read_GBs, 1), "bytes": gbytes,
            "k_stream_ratio": (round(kernels["k_stream"]["alg_GBs"] / grad_read_GBs, 4)
                               if "k_stream" in kernels and kernels["k_stream"]["alg_GBs"]
                               else None)},
        "step_frac_of_measured_read": round(step_alg / read_GBs, 4),
        "phases": phases,
        "kernels": kernels,
    }
    if not args.no_error:
        log("estimation error against the lossless comparator ...")
        result["estimation_error"] = gpu_estimation_error(s2r, wl, cap, buf, out, stream)
    del grad
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(wl, sparse, p.as_dict())
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
