"""Run the HIP path through the C ABI on numpy inputs and compare with the fp64 oracle.

Used by the GPU parity tests.  Inputs always come from the seeded generators in
``workloads``; expected values always come from ``oracle``; the two sides share only those
inputs.

Comparison rules (per the tolerance the method's fp32 arithmetic allows):
  * hash buckets and signs, bitmaps (pad bits included), nnz, list indices and list value
    bit patterns: bit-exact;
  * sketch cells: |gpu - S| <= 1e-5 * A + 1e-12, with A the cell's absolute mass
    sum |contribution| (any-order fp32 summation of c terms errs by at most
    (c-1) * 2^-24 * A, which stays below 1e-5 * A for c <= 168 contributions per cell);
  * decoded values: |gpu - g_hat| <= 1e-5 * max_j A[j, h_j(i)] + 1e-12 (the median is
    1-Lipschitz in the max-norm of its inputs); clear bits exactly +0.0.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import count_sketch_aggregation_amd as s2r
import oracle

DEV = torch.device("cuda:0")


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def params_pair(seed: int, d: int, L: int, K: int | None = None, log2_block: int = 0):
    """(library params, oracle params) derived independently from one seed."""
    if K is None:
        K = s2r.s2r_default_log2_part(d, L)
    p = s2r.s2r_params_from_seed(seed, d, L, K, log2_block=log2_block)
    op = oracle.params_from_seed(seed, d, L, K, log2_block=log2_block)
    assert p.as_dict() == op.as_dict()
    return p, op


def _u64(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint64)


def run_encode(p, grads: np.ndarray, n: int, cap: int | None = None):
    """grads: [W][ld] float32 host array.  Returns numpy outputs of s2r_encode."""
    W, ld = grads.shape
    cap = n if cap is None else cap
    g = torch.from_numpy(np.ascontiguousarray(grads)).to(DEV)
    buf = s2r.alloc_encode_buffers(p, W, n, cap, DEV)
    # poison the outputs so that anything the kernels fail to write shows up
    buf["bitmaps"].fill_(-1)
    buf["sketches"].fill_(float("nan"))
    buf["idx"].fill_(-1)
    buf["nnz"].fill_(-1)
    buf["workspace"].fill_(0xAB)
    s2r.s2r_encode(p, W, g, n, ld, buf["bitmaps"], buf["sketches"], buf["idx"], buf["val"], cap,
                   buf["nnz"], buf["workspace"])
    torch.cuda.synchronize()
    words = s2r.s2r_block_bitmap_words(n, p.log2_block)
    return {
        "bitmaps": _u64(buf["bitmaps"])[:, :words] if words else np.zeros((W, 0), np.uint64),
        "sketches": buf["sketches"].cpu().numpy(),
        "idx": buf["idx"].cpu().numpy().view(np.uint32),
        "val": buf["val"].cpu().numpy(),
        "nnz": buf["nnz"].cpu().numpy().astype(np.int64),
    }


def run_reduce(p, n: int, bitmaps: np.ndarray, sketches: np.ndarray, inplace: bool = False):
    W = sketches.shape[0]
    bm = torch.from_numpy(np.ascontiguousarray(bitmaps).view(np.int64)).to(DEV)
    sk = torch.from_numpy(np.ascontiguousarray(sketches, dtype=np.float32)).to(DEV)
    if inplace:
        bo, so = bm, sk
    else:
        bo = torch.full((max(bitmaps.shape[1], 1),), -1, dtype=torch.int64, device=DEV)
        so = torch.full(sketches.shape[1:], float("nan"), dtype=torch.float32, device=DEV)
    s2r.s2r_reduce(p, W, n, bm, sk, bo, so)
    torch.cuda.synchronize()
    words = bitmaps.shape[1]
    return _u64(bo.reshape(-1))[:words], so.reshape(sketches.shape[1:]).cpu().numpy() if not inplace \
        else sk[0].cpu().numpy()


def run_decode(p, n: int, bitmap: np.ndarray, sketch: np.ndarray, path: str = "partitioned",
               max_set: int | None = None) -> np.ndarray:
    """path: "direct" (no workspace), "partitioned" (workspace for max_set set bits,
    default n), or "overflow" (workspace far smaller than the set bits: the device must
    fall back to direct gathers)."""
    bm = torch.from_numpy(np.ascontiguousarray(bitmap).view(np.int64)).to(DEV) if bitmap.size else \
        torch.zeros(1, dtype=torch.int64, device=DEV)
    sk = torch.from_numpy(np.ascontiguousarray(sketch, dtype=np.float32)).to(DEV)
    out = torch.full((max(n, 1),), float("nan"), dtype=torch.float32, device=DEV)
    ws = None
    if path != "direct":
        if max_set is None:
            max_set = n if path == "partitioned" else 1
        ws = s2r.alloc_decode_workspace(p, n, max_set, DEV)
        if ws is not None:
            ws.fill_(0xCD)  # contents on entry must not matter
    s2r.s2r_decode(p, n, bm, sk, out, max_set=max_set or 0, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()[:n]


def run_hash(p, keys: np.ndarray):
    k = torch.from_numpy(np.ascontiguousarray(keys, dtype=np.uint32).view(np.int32)).to(DEV)
    m = keys.size
    b = torch.empty((p.d, max(m, 1)), dtype=torch.int32, device=DEV)
    s = torch.empty((p.d, max(m, 1)), dtype=torch.int8, device=DEV)
    s2r.s2r_hash(p, k, m, b, s)
    torch.cuda.synchronize()
    return b.cpu().numpy().view(np.uint32)[:, :m], s.cpu().numpy()[:, :m]


# ---------------------------------------------------------------------------------------
# comparisons


def assert_sketch_close(gpu: np.ndarray, S: np.ndarray, A: np.ndarray, what: str) -> None:
    gpu = gpu.astype(np.float64)
    err = np.abs(gpu - S)
    tol = 1e-5 * A + 1e-12
    bad = ~(err <= tol)  # NaN counts as bad
    if bad.any():
        i = np.flatnonzero(bad.reshape(-1))[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} cells outside tolerance, e.g. flat "
                             f"{i.tolist()} gpu={gpu.reshape(-1)[i]} oracle={S.reshape(-1)[i]} "
                             f"A={A.reshape(-1)[i]}")


def assert_encode_matches(op, grads: np.ndarray, n: int, res: dict, cap: int | None = None,
                          exact_sketch: bool = False) -> list:
    """Compare every worker's outputs with the oracle.  Returns the oracle encodings."""
    cap = n if cap is None else cap
    encs = []
    for k in range(grads.shape[0]):
        e = oracle.encode_dense(op, grads[k, :n], cap=cap)
        encs.append(e)
        assert np.array_equal(res["bitmaps"][k], e["bitmap"]), f"worker {k}: bitmap differs"
        assert res["nnz"][k] == e["nnz"], f"worker {k}: nnz {res['nnz'][k]} vs {e['nnz']}"
        m = min(e["nnz"], cap)
        assert np.array_equal(res["idx"][k, :m], e["idx"]), f"worker {k}: list indices differ"
        assert np.array_equal(res["val"][k, :m].view(np.uint32), e["val"].view(np.uint32)), \
            f"worker {k}: list values differ"
        if e["nnz"] <= cap:
            if exact_sketch:
                assert np.array_equal(res["sketches"][k].astype(np.float64), e["S"]), \
                    f"worker {k}: sketch not exact"
            else:
                assert_sketch_close(res["sketches"][k], e["S"], e["A"], f"worker {k} sketch")
    return encs


def assert_decode_matches(gpu: np.ndarray, want: np.ndarray, tol: np.ndarray, setmask: np.ndarray,
                          exact: bool = False) -> None:
    g = gpu.astype(np.float64)
    clear = ~setmask
    assert np.all(gpu[clear].view(np.uint32) == 0), "clear bits must decode to +0.0"
    if exact:
        bad = setmask & ~(g == want)
    else:
        bad = setmask & ~(np.abs(g - want) <= tol)
    if bad.any():
        i = np.flatnonzero(bad)[:5]
        raise AssertionError(f"{int(bad.sum())} decoded values off, e.g. i={i.tolist()} "
                             f"gpu={g[i]} oracle={want[i]} tol={tol[i]}")


def bits_of(bitmap: np.ndarray, n: int) -> np.ndarray:
    return np.unpackbits(np.ascontiguousarray(bitmap).view(np.uint8), bitorder="little")[:n] \
        .astype(bool)


def set_elements(bitmap: np.ndarray, n: int, log2_block: int) -> np.ndarray:
    """Elements i < n whose block bit is set (the elements a decode queries)."""
    B = 1 << log2_block
    blocks = bits_of(bitmap, (n + B - 1) // B)
    return np.repeat(blocks, B)[:n]


def run_topk(grads: np.ndarray, residual: np.ndarray | None, n: int, block: int, K: int):
    """grads, residual: [W][ld] host arrays.  Returns (out, residual, selected) as numpy."""
    W, ld = grads.shape
    g = torch.from_numpy(np.ascontiguousarray(grads)).to(DEV)
    r = None if residual is None else torch.from_numpy(np.ascontiguousarray(residual)).to(DEV)
    out = torch.full((W, ld), float("nan"), dtype=torch.float32, device=DEV)
    nb = -(-n // block)
    sw = max((nb + 63) // 64, 1)
    sel = torch.full((W, sw), -1, dtype=torch.int64, device=DEV)
    ws = torch.empty((max(s2r.s2r_topk_workspace_bytes(W, n, block), 1),), dtype=torch.uint8,
                     device=DEV)
    ws.fill_(0xAB)
    s2r.s2r_topk_ef(W, g, r, n, ld, block, K, out, sel, ws)
    torch.cuda.synchronize()
    return (out.cpu().numpy(), None if r is None else r.cpu().numpy(),
            sel.cpu().numpy().view(np.uint64)[:, : (nb + 63) // 64])


def assert_topk_matches(grads, residual, n, block, K, out, res_out, sel, what=""):
    """Every worker against the oracle.  The kept set must equal the oracle's unless the
    K-th and (K+1)-th squared norms tie to within fp64 rounding (1e-12 relative); then the
    GPU's set must still be a valid Top-K of the oracle's norms.  Given the kept set, out and
    the residual are bit-exact (the same fp32 addition g = grad + residual on both sides)."""
    W = grads.shape[0]
    nb = -(-n // block)
    for k in range(W):
        o = oracle.topk_ef(grads[k, :n], None if residual is None else residual[k, :n], block, K)
        gbits = np.unpackbits(sel[k].view(np.uint8), bitorder="little")
        assert not gbits[nb:].any(), f"{what} worker {k}: selection pad bits"
        gkept = gbits[:nb].astype(bool)
        okept = np.unpackbits(o["selected"].view(np.uint8), bitorder="little")[:nb].astype(bool)
        assert int(gkept.sum()) == min(K, nb), f"{what} worker {k}: {gkept.sum()} kept"
        if not np.array_equal(gkept, okept):
            nrm = o["norm2"]
            srt = np.sort(nrm)[::-1]
            tie = srt[min(K, nb) - 1]
            close = np.abs(nrm - tie) <= 1e-12 * max(tie, 1e-300)
            diff = gkept != okept
            assert np.all(close[diff]), f"{what} worker {k}: kept set differs beyond ties"
            # recompute the expected output with the GPU's (valid) kept set
            em = np.repeat(gkept, block)[:n]
            g = grads[k, :n] + (0 if residual is None else residual[k, :n])
            want_out = np.where(em, g, np.float32(0))
            want_res = np.where(em, np.float32(0), g)
        else:
            want_out, want_res = o["out"], o["residual"]
        assert np.array_equal(out[k, :n].view(np.uint32), want_out.astype(np.float32).view(np.uint32)), \
            f"{what} worker {k}: out"
        assert np.all(np.isnan(out[k, n:])), f"{what} worker {k}: wrote beyond n"
        if residual is not None:
            assert np.array_equal(res_out[k, :n].view(np.uint32),
                                  want_res.astype(np.float32).view(np.uint32)), f"{what} worker {k}: residual"
            assert np.array_equal(res_out[k, n:].view(np.uint32), residual[k, n:].view(np.uint32)), \
                f"{what} worker {k}: residual beyond n"
