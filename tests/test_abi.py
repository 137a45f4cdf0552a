"""The C ABI on the CPU: symbols, host-only calls and argument checks (no GPU needed).

Every call here returns before anything is enqueued, so no device is touched.
"""
import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "s2r.h")


@pytest.fixture(scope="module")
def s2r():
    import count_sketch_aggregation_amd as m
    if not os.path.exists(m.LIB_PATH):
        from count_sketch_aggregation_amd import _build
        _build.build()
    return m


def _declared():
    """Every function declared in include/*.h."""
    import glob
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(s2r_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_symbols_exported(s2r):
    names = _declared()
    assert {"s2r_encode", "s2r_reduce", "s2r_decode", "s2r_hash", "s2r_topk_ef",
            "s2r_diag_stream_read"} <= set(names)
    L = ctypes.CDLL(s2r.LIB_PATH)
    for name in names:
        assert hasattr(L, name), f"{name} declared in s2r.h but not exported"


def test_params_match_oracle(s2r):
    for (seed, d, L, K) in [(0, 1, 0, 0), (1, 3, 14, 13), (2**64 - 1, 16, 31, 11), (7, 5, 20, 20)]:
        p = s2r.s2r_params_from_seed(seed, d, L, K)
        assert p.as_dict() == oracle.params_from_seed(seed, d, L, K).as_dict()


def test_params_range_checks(s2r):
    for args in [(0, 0, 10, 10), (0, 17, 10, 10), (0, 3, 32, 10), (0, 3, 10, 11)]:
        with pytest.raises(s2r.S2RError) as e:
            s2r.s2r_params_from_seed(*args)
        assert e.value.status == s2r.S2R_ERR_DIM


def test_small_helpers(s2r):
    assert [s2r.s2r_bitmap_words(n) for n in (0, 1, 64, 65, 2**32 - 1)] == [0, 1, 1, 2, 2**26]
    # partition tile = d x 2^K fp32 must fit 64 KiB of LDS
    assert s2r.s2r_default_log2_part(5, 23) == 11
    assert s2r.s2r_default_log2_part(3, 19) == 12
    assert s2r.s2r_default_log2_part(1, 10) == 10
    assert s2r.s2r_default_log2_part(1, 20) == 14
    assert s2r.s2r_default_log2_part(16, 31) == 10
    p = s2r.s2r_params_from_seed(1, 3, 14, 13)
    assert s2r.s2r_encode_workspace_bytes(p, 4, 1 << 20, 1 << 20) > 0
    assert s2r.s2r_encode_workspace_bytes(p, 0, 1 << 20, 1 << 20) == 0
    assert s2r.s2r_encode_workspace_bytes(p, 1, 1 << 32, 1) == 0
    assert s2r.status_string(s2r.S2R_ERR_WORKSPACE) == "workspace too small"


def test_sketch_lambda(s2r):
    """lambda = sketch size / non-zeros, both readings (whole table, one row)."""
    assert s2r.s2r_sketch_lambda(5, 20, 2_097_152) == 5 * 2**20 / 2_097_152
    assert s2r.s2r_sketch_lambda(5, 20, 2_097_152, per_row=True) == 0.5
    assert s2r.s2r_sketch_lambda(3, 0, 3) == 1.0
    for bad in [(0, 10, 5), (17, 10, 5), (3, 32, 5), (3, 10, 0)]:
        assert s2r.s2r_sketch_lambda(*bad) == 0.0
    # the smallest width reaching the target, checked against every width by brute force
    for rows, nnz, lam, per_row in [(5, 2_097_152, 0.5, True), (5, 2_097_152, 0.5, False),
                                    (3, 255_744, 1.0, False), (1, 1, 1.0, True),
                                    (3, 1000, 0.05, False), (16, 7, 3.0, True),
                                    (2, 10**9, 0.5, True)]:
        L = s2r.s2r_log2_w_for_lambda(rows, nnz, lam, per_row)
        cells = lambda k: (1 if per_row else rows) * 2**k
        ok = [k for k in range(32) if cells(k) / nnz >= lam]
        assert L == ok[0]
        got = s2r.s2r_sketch_lambda(rows, L, nnz, per_row)
        assert got >= lam and (L == 0 or got < 2 * lam)
    assert s2r.s2r_log2_w_for_lambda(5, 2_097_152, 0.5, True) == 20  # the embedding workload
    assert s2r.s2r_log2_w_for_lambda(3, 0, 0.5, False) == 0
    none = 2**32 - 1
    assert s2r.s2r_log2_w_for_lambda(1, 2**63, 1.0, True) == none  # needs more than 2^31
    for bad in [(0, 10, 0.5), (17, 10, 0.5), (3, 10, 0.0), (3, 10, -1.0), (3, 10, float("nan")),
                (3, 10, float("inf"))]:
        assert s2r.s2r_log2_w_for_lambda(*bad) == none


def test_encode_noalloc_host_checks(s2r):
    """The allocation-free encode refuses, before touching any device, a request larger
    than its static scratch, and checks its arguments like s2r_encode."""
    p = s2r.s2r_params_from_seed(1, 5, 22, 11)
    L = s2r.lib()
    W, n, cap = 8, 160_000_000, 8_000_512
    assert s2r.s2r_encode_workspace_bytes(p, W, n, cap) > s2r.NOALLOC_SCRATCH_BYTES
    args = [ctypes.byref(p), W, FAKE, n, n, FAKE, FAKE, FAKE, FAKE, cap, FAKE, 0]
    assert L.s2r_encode_noalloc(*args) == s2r.S2R_ERR_SCRATCH
    bad = list(args)
    bad[5] = None
    assert L.s2r_encode_noalloc(*bad) == s2r.S2R_ERR_NULL
    bad = list(args)
    bad[1] = 0
    assert L.s2r_encode_noalloc(*bad) == s2r.S2R_ERR_DIM
    bad = list(args)
    bad[2] = FAKE + 4
    assert L.s2r_encode_noalloc(*bad) == s2r.S2R_ERR_ALIGN
    assert "static scratch" in s2r.status_string(s2r.S2R_ERR_SCRATCH)


FAKE = 1 << 20  # a 256-byte aligned non-null address; never dereferenced on these paths


def _encode(s2r, p, **kw):
    a = dict(W=2, grad=FAKE, n=1000, ld=1000, bitmaps=FAKE, sketches=FAKE, idx=FAKE, val=FAKE,
             cap=1000, nnz=FAKE, workspace=FAKE, ws_bytes=1 << 40, stream=0)
    a.update(kw)
    return s2r.lib().s2r_encode(ctypes.byref(p), a["W"], a["grad"], a["n"], a["ld"], a["bitmaps"],
                                a["sketches"], a["idx"], a["val"], a["cap"], a["nnz"],
                                a["workspace"], a["ws_bytes"], a["stream"])


def test_encode_argument_errors(s2r):
    p = s2r.s2r_params_from_seed(3, 3, 10, 10)
    assert _encode(s2r, p, grad=None) == s2r.S2R_ERR_NULL
    assert _encode(s2r, p, nnz=None) == s2r.S2R_ERR_NULL
    assert _encode(s2r, p, idx=None) == s2r.S2R_ERR_NULL          # cap > 0 needs a list
    assert _encode(s2r, p, W=0) == s2r.S2R_ERR_DIM
    assert _encode(s2r, p, n=2**32, ld=2**32) == s2r.S2R_ERR_DIM
    assert _encode(s2r, p, ld=996) == s2r.S2R_ERR_DIM              # ld < n
    assert _encode(s2r, p, ld=1002) == s2r.S2R_ERR_ALIGN           # ld % 4
    assert _encode(s2r, p, grad=FAKE + 4) == s2r.S2R_ERR_ALIGN     # grad not 16-byte aligned
    assert _encode(s2r, p, bitmaps=FAKE + 4) == s2r.S2R_ERR_ALIGN
    need = s2r.s2r_encode_workspace_bytes(p, 2, 1000, 1000)
    assert _encode(s2r, p, ws_bytes=need - 1) == s2r.S2R_ERR_WORKSPACE
    bad = s2r.s2r_params_from_seed(3, 3, 10, 10)
    bad.log2_block = 17                                            # beyond S2R_MAX_LOG2_BLOCK
    assert _encode(s2r, bad) == s2r.S2R_ERR_DIM
    bad = s2r.s2r_params_from_seed(3, 3, 10, 10)
    bad.log2_part = 11
    assert _encode(s2r, bad) == s2r.S2R_ERR_DIM


def test_reduce_decode_hash_argument_errors(s2r):
    L = s2r.lib()
    p = s2r.s2r_params_from_seed(3, 3, 10, 10)
    pr = ctypes.byref(p)
    assert L.s2r_reduce(pr, 2, 100, FAKE, None, FAKE, FAKE, 0) == s2r.S2R_ERR_NULL
    assert L.s2r_reduce(pr, 0, 100, FAKE, FAKE, FAKE, FAKE, 0) == s2r.S2R_ERR_DIM
    assert L.s2r_reduce(pr, 2, 100, FAKE + 4, FAKE, FAKE, FAKE, 0) == s2r.S2R_ERR_ALIGN
    assert L.s2r_decode(pr, 100, None, FAKE, FAKE, 0, None, 0, 0) == s2r.S2R_ERR_NULL
    assert L.s2r_decode(pr, 2**32, FAKE, FAKE, FAKE, 0, None, 0, 0) == s2r.S2R_ERR_DIM
    assert L.s2r_decode(pr, 100, FAKE, FAKE, FAKE + 4, 0, None, 0, 0) == s2r.S2R_ERR_ALIGN
    q = s2r.s2r_params_from_seed(3, 3, 14, 12)
    need = s2r.s2r_decode_workspace_bytes(q, 100_000, 5000)
    assert need > 0
    assert L.s2r_decode(ctypes.byref(q), 100_000, FAKE, FAKE, FAKE, 5000, FAKE, need - 1, 0) == \
        s2r.S2R_ERR_WORKSPACE
    # no partitioned decode for a table beyond the LDS budget with independent rows
    assert s2r.s2r_decode_workspace_bytes(s2r.s2r_params_from_seed(3, 5, 20, 20), 1000, 1000) == 0
    assert L.s2r_hash(pr, None, 10, FAKE, FAKE, 0) == s2r.S2R_ERR_NULL
    assert L.s2r_hash(None, FAKE, 10, FAKE, FAKE, 0) == s2r.S2R_ERR_NULL


def test_binding_refuses_without_library(s2r, tmp_path, monkeypatch):
    monkeypatch.setattr(s2r, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(s2r, "_lib", None)
    with pytest.raises(ImportError):
        s2r.lib()


def test_block_bitmap_words(s2r):
    """ceil(ceil(n / 2^lb) / 64), computed by the library on the host."""
    for n in (0, 1, 63, 64, 65, 4095, 4096, 4097, 137_084_928, 25_557_032, 2**32 - 1):
        for lb in (0, 1, 5, 6, 8, 9, 12, 16):
            B = 1 << lb
            assert s2r.s2r_block_bitmap_words(n, lb) == ((n + B - 1) // B + 63) // 64, (n, lb)
    assert s2r.s2r_block_bitmap_words(1000, 0) == s2r.s2r_bitmap_words(1000)


def test_block_workspace_grows(s2r):
    """A block-granular encode keeps the element bitmaps in its workspace."""
    p = s2r.s2r_params_from_seed(3, 3, 10, 10)
    q = s2r.s2r_params_from_seed(3, 3, 10, 10, log2_block=9)
    a = s2r.s2r_encode_workspace_bytes(p, 2, 100_000, 1000)
    b = s2r.s2r_encode_workspace_bytes(q, 2, 100_000, 1000)
    assert b >= a + 2 * s2r.s2r_bitmap_words(100_000) * 8



def test_topk_argument_errors(s2r):
    """s2r_topk_ef rejects bad arguments on the host, before any enqueue."""
    FAKE = 1 << 20
    L = s2r.lib()
    need = s2r.s2r_topk_workspace_bytes(2, 1000, 64)
    assert need > 0 and s2r.s2r_topk_workspace_bytes(0, 1000, 64) == 0
    assert s2r.s2r_topk_workspace_bytes(2, 1000, 0) == 0

    def call(W=2, grad=FAKE, res=FAKE * 2, n=1000, ld=1000, block=64, K=3, out=FAKE * 3,
             sel=FAKE * 4, ws=FAKE * 5, ws_bytes=None):
        return L.s2r_topk_ef(W, grad, res, n, ld, block, K, out, sel, ws,
                             need if ws_bytes is None else ws_bytes, None)

    assert call(grad=None) == s2r.S2R_ERR_NULL
    assert call(out=None) == s2r.S2R_ERR_NULL
    assert call(ws=None) == s2r.S2R_ERR_NULL
    assert call(W=0) == s2r.S2R_ERR_DIM
    assert call(block=0) == s2r.S2R_ERR_DIM
    assert call(ld=996) == s2r.S2R_ERR_DIM
    assert call(n=2**32, ld=2**32) == s2r.S2R_ERR_DIM
    assert call(res=FAKE) == s2r.S2R_ERR_DIM          # residual may not be the gradient
    assert call(ld=1002) == s2r.S2R_ERR_ALIGN
    assert call(grad=FAKE + 4) == s2r.S2R_ERR_ALIGN
    assert call(out=FAKE * 3 + 8) == s2r.S2R_ERR_ALIGN
    assert call(sel=FAKE * 4 + 4) == s2r.S2R_ERR_ALIGN
    assert call(ws_bytes=need - 1) == s2r.S2R_ERR_WORKSPACE


def test_diag_argument_errors(s2r):
    L = s2r.lib()
    assert L.s2r_diag_stream_read(None, 16, 1 << 20, None) == s2r.S2R_ERR_NULL
    assert L.s2r_diag_stream_read(1 << 20, 16, None, None) == s2r.S2R_ERR_NULL
    assert L.s2r_diag_stream_read((1 << 20) + 4, 16, 1 << 21, None) == s2r.S2R_ERR_ALIGN
    assert L.s2r_diag_stream_read(1 << 20, 20, 1 << 21, None) == s2r.S2R_ERR_ALIGN
    assert L.s2r_diag_stream_read(1 << 20, 0, 1 << 21, None) == s2r.S2R_OK  # nothing to read

