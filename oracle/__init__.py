"""fp64 CPU oracle for sparse-sketch gradient aggregation (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import this
package.  The GPU library never imports, links or calls it.  The arithmetic lives in
``s2r_oracle.cpp`` (plain C++, fp64); this module compiles it with g++ and marshals numpy
arrays through ctypes.

What the oracle computes follows "S2 Reducer: High-Performance Sparse Communication to
Accelerate Distributed Deep Learning" (arXiv 2110.02140), Section 3.1 and Algorithm 1:
bitmap + count-sketch compression of each worker's gradient, element-wise sum of the
sketches with OR of the bitmaps, and a median-of-rows query at every set bit.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "s2r_oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")
MAX_ROWS = 16


class OrcParams(ctypes.Structure):
    """Mirror of ``struct orc_params`` in s2r_oracle.cpp."""

    _fields_ = [
        ("d", ctypes.c_uint32),
        ("log2_w", ctypes.c_uint32),
        ("log2_part", ctypes.c_uint32),
        ("log2_block", ctypes.c_uint32),
        ("pA", ctypes.c_uint64),
        ("pB", ctypes.c_uint64),
        ("hA", ctypes.c_uint64 * MAX_ROWS),
        ("hB", ctypes.c_uint64 * MAX_ROWS),
        ("sA", ctypes.c_uint64 * MAX_ROWS),
        ("sB", ctypes.c_uint64 * MAX_ROWS),
    ]

    @property
    def w(self) -> int:
        return 1 << self.log2_w

    def as_dict(self) -> dict:
        d = self.d
        return {
            "d": d, "log2_w": self.log2_w, "log2_part": self.log2_part,
            "log2_block": self.log2_block, "pA": self.pA, "pB": self.pB,
            "hA": list(self.hA)[:d], "hB": list(self.hB)[:d],
            "sA": list(self.sA)[:d], "sB": list(self.sB)[:d],
        }


def build(force: bool = False) -> str:
    """Compile liboracle.so with g++ (fp64, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fPIC", "-shared",
               "-o", tmp, _SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(L: ctypes.CDLL) -> ctypes.CDLL:
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    u64, u32 = ctypes.c_uint64, ctypes.c_uint32
    L.orc_splitmix64_next.argtypes = [P(u64)]
    L.orc_splitmix64_next.restype = u64
    L.orc_params_from_seed.argtypes = [u64, u32, u32, u32, P(OrcParams)]
    L.orc_params_from_seed.restype = ctypes.c_int
    L.orc_bucket.argtypes = [P(OrcParams), u32, u32]
    L.orc_bucket.restype = u32
    L.orc_sign.argtypes = [P(OrcParams), u32, u32]
    L.orc_sign.restype = ctypes.c_int
    L.orc_hash.argtypes = [P(OrcParams), vp, u64, vp, vp]
    L.orc_hash.restype = None
    L.orc_encode_dense.argtypes = [P(OrcParams), vp, u64, vp, vp, vp, vp, vp, u64, P(u64)]
    L.orc_encode_dense.restype = ctypes.c_int
    L.orc_encode_sparse.argtypes = [P(OrcParams), vp, vp, u64, u64, vp, vp, vp]
    L.orc_encode_sparse.restype = ctypes.c_int
    L.orc_reduce.argtypes = [u32, u64, u64, vp, vp, vp, vp, vp, vp]
    L.orc_reduce.restype = None
    L.orc_decode.argtypes = [P(OrcParams), u64, vp, vp, vp, vp, vp, vp, u64]
    L.orc_decode.restype = u64
    L.orc_gather_sum.argtypes = [u32, vp, vp, vp, u64, u64, vp, vp]
    L.orc_gather_sum.restype = None
    L.orc_topk_ef.argtypes = [vp, vp, u64, u64, u64, vp, vp, vp]
    L.orc_topk_ef.restype = ctypes.c_int
    L.orc_bitmap_words.argtypes = [P(OrcParams), u64]
    L.orc_bitmap_words.restype = u64
    return L


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


@contextlib.contextmanager
def using(path: str):
    """Temporarily route every call of this module to another build of the oracle source
    (the pin suite uses this to show that altered copies of the oracle fail it)."""
    global _lib
    old = _lib
    _lib = _bind(ctypes.CDLL(os.path.abspath(path)))
    try:
        yield
    finally:
        _lib = old


def compile_source(src_path: str, out_path: str) -> str:
    subprocess.run(["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fPIC", "-shared",
                    "-o", out_path, src_path], check=True)
    return out_path


def source_path() -> str:
    return _SRC


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def splitmix64(seed: int, count: int) -> list[int]:
    st = ctypes.c_uint64(seed)
    return [lib().orc_splitmix64_next(ctypes.byref(st)) for _ in range(count)]


def params_from_seed(seed: int, d: int, log2_w: int, log2_part: int | None = None,
                     log2_block: int = 0) -> OrcParams:
    """Hash constants from SplitMix64; log2_block sets the bitmap granularity (one bit per
    2^log2_block elements)."""
    if log2_part is None:
        log2_part = log2_w
    p = OrcParams()
    rc = lib().orc_params_from_seed(seed, d, log2_w, log2_part, ctypes.byref(p))
    if rc != 0:
        raise ValueError(f"oracle: bad params d={d} log2_w={log2_w} log2_part={log2_part}")
    p.log2_block = log2_block
    return p


def params_from_constants(d, log2_w, log2_part, pA, pB, hA, hB, sA, sB,
                          log2_block: int = 0) -> OrcParams:
    p = OrcParams()
    p.d, p.log2_w, p.log2_part, p.log2_block = d, log2_w, log2_part, log2_block
    p.pA, p.pB = pA, pB
    for j in range(d):
        p.hA[j], p.hB[j], p.sA[j], p.sB[j] = hA[j], hB[j], sA[j], sB[j]
    return p


def bucket(p: OrcParams, j: int, i: int) -> int:
    return lib().orc_bucket(ctypes.byref(p), j, i)


def sign(p: OrcParams, j: int, i: int) -> int:
    return lib().orc_sign(ctypes.byref(p), j, i)


def hash_keys(p: OrcParams, keys: np.ndarray):
    keys = np.ascontiguousarray(keys, dtype=np.uint32)
    m = keys.size
    b = np.empty((p.d, m), dtype=np.uint32)
    s = np.empty((p.d, m), dtype=np.int8)
    lib().orc_hash(ctypes.byref(p), _ptr(keys), m, _ptr(b), _ptr(s))
    return b, s


def words(n: int) -> int:
    """uint64 words of an element-granular bitmap of n bits."""
    return (n + 63) // 64


def bitmap_words(p: OrcParams, n: int) -> int:
    """uint64 words of the bitmap for n elements at p's granularity."""
    return int(lib().orc_bitmap_words(ctypes.byref(p), n))


def encode_dense(p: OrcParams, g: np.ndarray, cap: int | None = None):
    """Returns dict(bitmap, S, A, idx, val, nnz) for one worker's dense fp32 gradient."""
    g = np.ascontiguousarray(g, dtype=np.float32)
    n = g.size
    cap = n if cap is None else cap
    bm = np.empty(bitmap_words(p, n), dtype=np.uint64)
    S = np.empty((p.d, p.w), dtype=np.float64)
    A = np.empty((p.d, p.w), dtype=np.float64)
    idx = np.empty(max(cap, 1), dtype=np.uint32)
    val = np.empty(max(cap, 1), dtype=np.float32)
    nnz = ctypes.c_uint64(0)
    rc = lib().orc_encode_dense(ctypes.byref(p), _ptr(g), n, _ptr(bm), _ptr(S), _ptr(A),
                                _ptr(idx), _ptr(val), cap, ctypes.byref(nnz))
    if rc:
        raise ValueError(f"oracle encode_dense failed rc={rc}")
    k = min(nnz.value, cap)
    return {"bitmap": bm, "S": S, "A": A, "idx": idx[:k].copy(), "val": val[:k].copy(),
            "nnz": nnz.value}


def encode_sparse(p: OrcParams, idx: np.ndarray, val: np.ndarray, n: int):
    """Compression from Sparse(g) (index, value) pairs.  Returns dict(bitmap, S, A)."""
    idx = np.ascontiguousarray(idx, dtype=np.uint32)
    val = np.ascontiguousarray(val, dtype=np.float32)
    bm = np.empty(bitmap_words(p, n), dtype=np.uint64)
    S = np.empty((p.d, p.w), dtype=np.float64)
    A = np.empty((p.d, p.w), dtype=np.float64)
    rc = lib().orc_encode_sparse(ctypes.byref(p), _ptr(idx), _ptr(val), idx.size, n,
                                 _ptr(bm), _ptr(S), _ptr(A))
    if rc:
        raise ValueError(f"oracle encode_sparse failed rc={rc}")
    return {"bitmap": bm, "S": S, "A": A}


def reduce(bitmaps: np.ndarray, S: np.ndarray, A: np.ndarray):
    """bitmaps [W][words] u64, S/A [W][...] f64 -> (bitmap, S_sum, A_sum)."""
    bitmaps = np.ascontiguousarray(bitmaps, dtype=np.uint64)
    S = np.ascontiguousarray(S, dtype=np.float64)
    A = np.ascontiguousarray(A, dtype=np.float64)
    W = bitmaps.shape[0]
    nwords = bitmaps.shape[1]
    cells = S[0].size
    bm_out = np.empty(nwords, dtype=np.uint64)
    S_out = np.empty(S.shape[1:], dtype=np.float64)
    A_out = np.empty(A.shape[1:], dtype=np.float64)
    lib().orc_reduce(W, cells, nwords, _ptr(bitmaps), _ptr(S), _ptr(A), _ptr(bm_out),
                     _ptr(S_out), _ptr(A_out))
    return bm_out, S_out, A_out


def decode(p: OrcParams, n: int, bitmap: np.ndarray, S: np.ndarray, A: np.ndarray | None = None):
    """Sparse decode: (idx u32, val f64, tol f64) over the elements < n whose block bit is
    set, ascending."""
    bitmap = np.ascontiguousarray(bitmap, dtype=np.uint64)
    S = np.ascontiguousarray(S, dtype=np.float64)
    A = np.abs(S) if A is None else np.ascontiguousarray(A, dtype=np.float64)
    B = 1 << p.log2_block
    nblocks = (n + B - 1) // B
    nb = bitmap[: bitmap_words(p, n)]
    # the elements of the set blocks below n bound the output
    cap = 0
    if n:
        setb = np.flatnonzero(np.unpackbits(nb.view(np.uint8), bitorder="little")[:nblocks])
        cap = int(setb.size) * B - (B * nblocks - n if nblocks - 1 in setb else 0)
    out_idx = np.empty(max(cap, 1), dtype=np.uint32)
    out_val = np.empty(max(cap, 1), dtype=np.float64)
    out_tol = np.empty(max(cap, 1), dtype=np.float64)
    cnt = lib().orc_decode(ctypes.byref(p), n, _ptr(bitmap), _ptr(S), _ptr(A), _ptr(out_idx),
                           _ptr(out_val), _ptr(out_tol), cap)
    assert cnt == cap, (cnt, cap)
    return out_idx[:cnt].copy(), out_val[:cnt].copy(), out_tol[:cnt].copy()


def decode_dense(p: OrcParams, n: int, bitmap, S, A=None):
    """Dense fp64 g_hat[n] (zero at clear bits) and dense tolerance."""
    i, v, t = decode(p, n, bitmap, S, A)
    out = np.zeros(n, dtype=np.float64)
    tol = np.zeros(n, dtype=np.float64)
    out[i] = v
    tol[i] = t
    return out, tol


def gather_sum(lists, n: int):
    """Exact aggregate of W workers' (index, value) lists, worker by worker: dense fp64
    out[n] and the absolute mass[n] (sum of |value| per element)."""
    W = len(lists)
    stride = max([max(int(i.size), 1) for i, _ in lists] + [1])
    idx = np.zeros((W, stride), dtype=np.uint32)
    val = np.zeros((W, stride), dtype=np.float32)
    ln = np.zeros(W, dtype=np.uint64)
    for k, (i, v) in enumerate(lists):
        idx[k, :i.size] = i
        val[k, :v.size] = v
        ln[k] = i.size
    out = np.empty(max(n, 1), dtype=np.float64)
    mass = np.empty(max(n, 1), dtype=np.float64)
    lib().orc_gather_sum(W, _ptr(idx), _ptr(val), _ptr(ln), stride, n, _ptr(out), _ptr(mass))
    return out[:n], mass[:n]


def topk_ef(grad: np.ndarray, residual: np.ndarray | None, block: int, K: int):
    """Block-wise Top-K with error feedback on one worker's gradient.  Returns
    dict(out, residual (None without error feedback), selected (uint64 bitmap of kept blocks),
    norm2 (fp64 squared block norms))."""
    grad = np.ascontiguousarray(grad, dtype=np.float32)
    n = grad.size
    nb = -(-n // block)
    res = None if residual is None else np.array(residual, dtype=np.float32, copy=True)
    out = np.empty(max(n, 1), dtype=np.float32)
    sel = np.empty(max((nb + 63) // 64, 1), dtype=np.uint64)
    norm2 = np.empty(max(nb, 1), dtype=np.float64)
    rc = lib().orc_topk_ef(_ptr(grad), None if res is None else _ptr(res), n, block, K, _ptr(out),
                           _ptr(sel), _ptr(norm2))
    if rc:
        raise ValueError(f"oracle topk_ef failed rc={rc}")
    return {"out": out[:n], "residual": res, "selected": sel[: (nb + 63) // 64],
            "norm2": norm2[:nb]}

