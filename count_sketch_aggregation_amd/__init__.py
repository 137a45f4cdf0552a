"""Python binding of libs2r: sparse-sketch gradient aggregation on MI355X (gfx950).

Thin ctypes marshalling over the C ABI in include/s2r.h -- the functions below carry the
same names as the C entry points, take torch tensors (device memory) and the current torch
stream, and do no arithmetic of their own.  Every step of the path runs in the HIP kernels
of libs2r.so; there is no CPU or PyTorch fallback: if the library is not built, importing
the binding's entry points raises.

The method is the data-parallel hot path of S2 Reducer (arXiv 2110.02140, Section 3.1 and
Algorithm 1): encode (bitmap + count-sketch per worker), reduce (sum of sketches, OR of
bitmaps) and decode (median over rows at every set bit).
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libs2r.so")
MAX_ROWS = 16

(S2R_OK, S2R_ERR_NULL, S2R_ERR_DIM, S2R_ERR_ALIGN, S2R_ERR_WORKSPACE, S2R_ERR_HIP,
 S2R_ERR_SCRATCH) = range(7)
NOALLOC_SCRATCH_BYTES = 256 << 20


class S2RError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class s2r_params(ctypes.Structure):
    """Mirror of ``s2r_params`` in include/s2r.h."""

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


_lib = None


def lib() -> ctypes.CDLL:
    """Load libs2r.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"libs2r.so not found at {LIB_PATH}: build it with "
                "`python -c 'import __graft_entry__ as g; g.build()'` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        vp, u64, u32, sz = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_size_t
        st = ctypes.c_int
        L.s2r_params_from_seed.argtypes = [u64, u32, u32, u32, P(s2r_params)]
        L.s2r_params_from_seed.restype = st
        L.s2r_default_log2_part.argtypes = [u32, u32]
        L.s2r_default_log2_part.restype = u32
        L.s2r_sketch_lambda.argtypes = [u32, u32, u64, ctypes.c_int]
        L.s2r_sketch_lambda.restype = ctypes.c_double
        L.s2r_log2_w_for_lambda.argtypes = [u32, u64, ctypes.c_double, ctypes.c_int]
        L.s2r_log2_w_for_lambda.restype = u32
        L.s2r_bitmap_words.argtypes = [u64]
        L.s2r_bitmap_words.restype = u64
        L.s2r_block_bitmap_words.argtypes = [u64, u32]
        L.s2r_block_bitmap_words.restype = u64
        L.s2r_encode_workspace_bytes.argtypes = [P(s2r_params), u32, u64, u64]
        L.s2r_encode_workspace_bytes.restype = sz
        L.s2r_encode.argtypes = [P(s2r_params), u32, vp, u64, u64, vp, vp, vp, vp, u64, vp, vp, sz,
                                 vp]
        L.s2r_encode.restype = st
        L.s2r_encode_noalloc.argtypes = [P(s2r_params), u32, vp, u64, u64, vp, vp, vp, vp, u64,
                                         vp, vp]
        L.s2r_encode_noalloc.restype = st
        L.s2r_reduce.argtypes = [P(s2r_params), u32, u64, vp, vp, vp, vp, vp]
        L.s2r_reduce.restype = st
        L.s2r_decode_workspace_bytes.argtypes = [P(s2r_params), u64, u64]
        L.s2r_decode_workspace_bytes.restype = sz
        L.s2r_decode.argtypes = [P(s2r_params), u64, vp, vp, vp, u64, vp, sz, vp]
        L.s2r_decode.restype = st
        L.s2r_hash.argtypes = [P(s2r_params), vp, u64, vp, vp, vp]
        L.s2r_hash.restype = st
        L.s2r_gather_sum.argtypes = [u32, vp, vp, u64, vp, u64, vp, vp]
        L.s2r_gather_sum.restype = st
        L.s2r_diag_trace_attach.argtypes = [vp]
        L.s2r_diag_trace_attach.restype = st
        L.s2r_topk_workspace_bytes.argtypes = [u32, u64, u64]
        L.s2r_topk_workspace_bytes.restype = sz
        L.s2r_topk_ef.argtypes = [u32, vp, vp, u64, u64, u64, u64, vp, vp, vp, sz, vp]
        L.s2r_topk_ef.restype = st
        L.s2r_diag_stream_write.argtypes = [vp, sz, ctypes.c_float, vp]
        L.s2r_diag_stream_write.restype = st
        L.s2r_diag_stream_read.argtypes = [vp, sz, vp, vp]
        L.s2r_diag_stream_read.restype = st
        L.s2r_status_string.argtypes = [st]
        L.s2r_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().s2r_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != S2R_OK:
        raise S2RError(status, where)


def _ptr(t) -> int | None:
    """Device pointer of a tensor (None for None), or an int passed through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ---------------------------------------------------------------------------------------
# entry points (same names as the C ABI)


def s2r_params_from_seed(seed: int, d: int, log2_w: int, log2_part: int | None = None,
                         log2_block: int = 0) -> s2r_params:
    """Hash constants from a seed (SplitMix64).  log2_part defaults to the largest partition
    that fits the LDS accumulator (s2r_default_log2_part); log2_part == log2_w gives
    independent rows.  log2_block sets the bitmap granularity (one bit per 2^log2_block
    elements; 0 = per element)."""
    if log2_part is None:
        log2_part = s2r_default_log2_part(d, log2_w)
    p = s2r_params()
    _check(lib().s2r_params_from_seed(seed, d, log2_w, log2_part, ctypes.byref(p)),
           "s2r_params_from_seed")
    p.log2_block = log2_block
    return p


def s2r_default_log2_part(d: int, log2_w: int) -> int:
    return int(lib().s2r_default_log2_part(d, log2_w))


def s2r_sketch_lambda(rows: int, log2_w: int, nnz: int, per_row: bool = False) -> float:
    """Sketch size over the non-zero count: rows * 2^log2_w / nnz, or 2^log2_w / nnz with
    per_row (see include/s2r.h)."""
    return float(lib().s2r_sketch_lambda(rows, log2_w, nnz, 1 if per_row else 0))


def s2r_log2_w_for_lambda(rows: int, nnz: int, lam: float, per_row: bool = False) -> int:
    """Smallest log2_w reaching the ratio `lam`; 2^32 - 1 when none can."""
    return int(lib().s2r_log2_w_for_lambda(rows, nnz, lam, 1 if per_row else 0))


def s2r_bitmap_words(n: int) -> int:
    return int(lib().s2r_bitmap_words(n))


def s2r_block_bitmap_words(n: int, log2_block: int) -> int:
    return int(lib().s2r_block_bitmap_words(n, log2_block))


def s2r_encode_workspace_bytes(p: s2r_params, W: int, n: int, cap: int) -> int:
    return int(lib().s2r_encode_workspace_bytes(ctypes.byref(p), W, n, cap))


def s2r_encode(p: s2r_params, W: int, grad, n: int, ld: int, bitmaps, sketches, idx, val, cap: int,
               nnz, workspace, ws_bytes: int | None = None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().s2r_encode(ctypes.byref(p), W, _ptr(grad), n, ld, _ptr(bitmaps), _ptr(sketches),
                            _ptr(idx), _ptr(val), cap, _ptr(nnz), _ptr(workspace), ws_bytes,
                            _stream(stream)), "s2r_encode")


def s2r_encode_noalloc(p: s2r_params, W: int, grad, n: int, ld: int, bitmaps, sketches, idx, val,
                       cap: int, nnz, stream=None) -> None:
    """s2r_encode with the library's static scratch as its workspace (allocates nothing)."""
    _check(lib().s2r_encode_noalloc(ctypes.byref(p), W, _ptr(grad), n, ld, _ptr(bitmaps),
                                    _ptr(sketches), _ptr(idx), _ptr(val), cap, _ptr(nnz),
                                    _stream(stream)), "s2r_encode_noalloc")


def s2r_reduce(p: s2r_params, W: int, n: int, bitmaps, sketches, bitmap_out, sketch_out,
               stream=None) -> None:
    _check(lib().s2r_reduce(ctypes.byref(p), W, n, _ptr(bitmaps), _ptr(sketches), _ptr(bitmap_out),
                            _ptr(sketch_out), _stream(stream)), "s2r_reduce")


def s2r_decode_workspace_bytes(p: s2r_params, n: int, max_set: int) -> int:
    return int(lib().s2r_decode_workspace_bytes(ctypes.byref(p), n, max_set))


def s2r_decode(p: s2r_params, n: int, bitmap, sketch, out, max_set: int = 0, workspace=None,
               ws_bytes: int | None = None, stream=None) -> None:
    """workspace=None selects direct gathers; otherwise pass a buffer of
    s2r_decode_workspace_bytes(p, n, max_set) bytes (see include/s2r.h)."""
    if ws_bytes is None:
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().s2r_decode(ctypes.byref(p), n, _ptr(bitmap), _ptr(sketch), _ptr(out), max_set,
                            _ptr(workspace), ws_bytes, _stream(stream)), "s2r_decode")


def s2r_hash(p: s2r_params, keys, m: int, buckets, signs, stream=None) -> None:
    _check(lib().s2r_hash(ctypes.byref(p), _ptr(keys), m, _ptr(buckets), _ptr(signs),
                          _stream(stream)), "s2r_hash")


def s2r_gather_sum(W: int, idx, val, cap: int, nnz, n: int, out, stream=None) -> None:
    """Exact sum of the workers' (index, value) lists into dense out[n] (worker order)."""
    _check(lib().s2r_gather_sum(W, _ptr(idx), _ptr(val), cap, _ptr(nnz), n, _ptr(out),
                                _stream(stream)), "s2r_gather_sum")


def s2r_topk_workspace_bytes(W: int, n: int, block: int) -> int:
    return int(lib().s2r_topk_workspace_bytes(W, n, block))


def s2r_topk_ef(W: int, grad, residual, n: int, ld: int, block: int, K: int, out, selected,
                workspace, ws_bytes: int | None = None, stream=None) -> None:
    """Block-wise Top-K with error feedback (residual may be None: no error feedback;
    selected may be None)."""
    if ws_bytes is None:
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().s2r_topk_ef(W, _ptr(grad), _ptr(residual), n, ld, block, K, _ptr(out),
                             _ptr(selected), _ptr(workspace), ws_bytes, _stream(stream)),
           "s2r_topk_ef")


TRACE_MAX = 64


class s2r_trace(ctypes.Structure):
    """Mirror of ``s2r_trace`` in include/s2r_diag.h."""

    _fields_ = [
        ("capacity", ctypes.c_uint32),
        ("count", ctypes.c_uint32),
        ("events", ctypes.c_void_p * TRACE_MAX),
        ("names", ctypes.c_char_p * TRACE_MAX),
    ]


def s2r_diag_trace_attach(trace) -> None:
    """Attach an s2r_trace (or None to detach) to the calling thread (include/s2r_diag.h)."""
    _check(lib().s2r_diag_trace_attach(None if trace is None else ctypes.addressof(trace)),
           "s2r_diag_trace_attach")


def s2r_diag_stream_write(buf, nbytes: int, value: float = 0.0, stream=None) -> None:
    """Measurement helper (include/s2r_diag.h): fill `nbytes` of `buf` with `value` once."""
    _check(lib().s2r_diag_stream_write(_ptr(buf), nbytes, value, _stream(stream)),
           "s2r_diag_stream_write")


def s2r_diag_stream_read(buf, nbytes: int, sink, stream=None) -> None:
    """Measurement helper (include/s2r_diag.h): stream `nbytes` of `buf` once."""
    _check(lib().s2r_diag_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)),
           "s2r_diag_stream_read")


# ---------------------------------------------------------------------------------------
# allocation helper (torch supplies device memory; no arithmetic here)


def alloc_decode_workspace(p: s2r_params, n: int, max_set: int, device="cuda"):
    """A workspace tensor for the partitioned decode, or None when it does not apply."""
    import torch
    nb = s2r_decode_workspace_bytes(p, n, max_set)
    return torch.empty((nb,), dtype=torch.uint8, device=device) if nb else None


def alloc_encode_buffers(p: s2r_params, W: int, n: int, cap: int, device="cuda") -> dict:
    """torch tensors for every s2r_encode output plus its workspace."""
    import torch
    words = s2r_block_bitmap_words(n, p.log2_block)
    ws = s2r_encode_workspace_bytes(p, W, n, cap)
    if ws == 0:
        raise S2RError(S2R_ERR_DIM, "s2r_encode_workspace_bytes")
    return {
        "bitmaps": torch.empty((W, max(words, 1)), dtype=torch.int64, device=device),
        "sketches": torch.empty((W, p.d, p.w), dtype=torch.float32, device=device),
        "idx": torch.empty((W, max(cap, 1)), dtype=torch.int32, device=device),
        "val": torch.empty((W, max(cap, 1)), dtype=torch.float32, device=device),
        "nnz": torch.empty((W,), dtype=torch.int64, device=device),
        "workspace": torch.empty((ws,), dtype=torch.uint8, device=device),
    }


__all__ = [
    "s2r_params", "S2RError", "s2r_params_from_seed", "s2r_default_log2_part", "s2r_bitmap_words",
    "s2r_sketch_lambda", "s2r_log2_w_for_lambda",
    "s2r_block_bitmap_words",
    "s2r_encode_workspace_bytes", "s2r_encode", "s2r_encode_noalloc", "s2r_reduce", "s2r_decode_workspace_bytes",
    "s2r_decode", "s2r_hash", "s2r_gather_sum", "s2r_topk_workspace_bytes", "s2r_topk_ef",
    "s2r_trace", "s2r_diag_trace_attach",
    "alloc_encode_buffers", "status_string", "lib",
]
