"""The allocation-free encode, s2r_encode_noalloc, through the C ABI: its outputs equal
those of s2r_encode on the same inputs (bitmaps, nnz and lists bit-exact; sketch cells both
within the oracle's bound |gpu - S| <= 1e-5 A + 1e-12), over two calls in a row whose second
is smaller (the static scratch keeps the first call's contents), on both accumulation paths;
an oversize request is refused with S2R_ERR_SCRATCH and writes nothing."""
import numpy as np
import pytest
import torch

import count_sketch_aggregation_amd as s2r
import oracle
import workloads as WL

pytestmark = pytest.mark.gpu

gp = pytest.importorskip("gpu_path")


def _outputs(p, W, n, cap):
    words = max(s2r.s2r_block_bitmap_words(n, p.log2_block), 1)
    return {
        "bitmaps": torch.full((W, words), -1, dtype=torch.int64, device=gp.DEV),
        "sketches": torch.full((W, p.d, p.w), float("nan"), dtype=torch.float32, device=gp.DEV),
        "idx": torch.full((W, max(cap, 1)), -1, dtype=torch.int32, device=gp.DEV),
        "val": torch.full((W, max(cap, 1)), float("nan"), dtype=torch.float32, device=gp.DEV),
        "nnz": torch.full((W,), -1, dtype=torch.int64, device=gp.DEV),
    }


def _run_both(p, grads, n, cap):
    W, ld = grads.shape
    g = torch.from_numpy(np.ascontiguousarray(grads)).to(gp.DEV)
    a = _outputs(p, W, n, cap)
    ws = torch.empty(s2r.s2r_encode_workspace_bytes(p, W, n, cap), dtype=torch.uint8, device=gp.DEV)
    s2r.s2r_encode(p, W, g, n, ld, a["bitmaps"], a["sketches"], a["idx"], a["val"], cap, a["nnz"], ws)
    b = _outputs(p, W, n, cap)
    s2r.s2r_encode_noalloc(p, W, g, n, ld, b["bitmaps"], b["sketches"], b["idx"], b["val"], cap,
                           b["nnz"])
    torch.cuda.synchronize()
    return a, b


def _compare(op, grads, n, cap, a, b):
    W = grads.shape[0]
    assert torch.equal(a["bitmaps"], b["bitmaps"])
    assert torch.equal(a["nnz"], b["nnz"])
    nnz = a["nnz"].cpu().numpy()
    for k in range(W):
        m = min(int(nnz[k]), cap)
        assert torch.equal(a["idx"][k, :m], b["idx"][k, :m])
        assert torch.equal(a["val"][k, :m].view(torch.int32), b["val"][k, :m].view(torch.int32))
        e = oracle.encode_dense(op, grads[k, :n], cap=cap)
        assert int(nnz[k]) == e["nnz"]
        if e["nnz"] > cap:  # past the list capacity the sketch is unspecified
            continue
        for name, res in (("s2r_encode", a), ("s2r_encode_noalloc", b)):
            gp.assert_sketch_close(res["sketches"][k].cpu().numpy(), e["S"], e["A"],
                                   f"{name} worker {k}")


@pytest.mark.parametrize("K", [None, 14])
def test_noalloc_matches_encode_twice(K):
    """Two calls in a row, the second on a smaller input, each against s2r_encode."""
    d, L = 3, 14
    p, op = gp.params_pair(808, d, L, K)
    for (W, n, density, seed) in [(4, 1 << 20, 0.01, 10), (2, 100_003, 0.05, 20)]:
        gp.say(f"encode_noalloc K={K} W={W} n={n}")
        ld = (n + 3) // 4 * 4
        grads = np.stack([WL.dense_from_sparse(n, *WL.uniform_sparse(n, density, seed + k), ld=ld)
                          for k in range(W)])
        cap = n
        a, b = _run_both(p, grads, n, cap)
        _compare(op, grads, n, cap, a, b)


def test_noalloc_block_bitmap_and_capacity_cut():
    """A block-granular bitmap (the scratch holds the element bitmaps) and a list cut by
    its capacity (bitmaps, nnz and the listed entries still exact), after a larger call."""
    d, L = 5, 18
    p, op = gp.params_pair(909, d, L, log2_block=8)
    n, W = 300_000, 3
    grads = np.stack([WL.dense_from_sparse(n, *WL.blocks_sparse(n, 256, 0.05, 30 + k))
                      for k in range(W)])
    gp.say("encode_noalloc block bitmap")
    a, b = _run_both(p, grads, n, n)
    _compare(op, grads, n, n, a, b)
    gp.say("encode_noalloc capacity cut")
    a, b = _run_both(p, grads, n, 5000)
    _compare(op, grads, n, 5000, a, b)


def test_noalloc_refuses_oversize():
    p = s2r.s2r_params_from_seed(1, 5, 22, 11)
    W, n, cap = 8, 160_000_000, 8_000_512  # the 160M-element workload's shape
    assert s2r.s2r_encode_workspace_bytes(p, W, n, cap) > s2r.NOALLOC_SCRATCH_BYTES
    g = torch.zeros((1, 4), dtype=torch.float32, device=gp.DEV)  # never read
    out = _outputs(p, 1, 4, 4)
    with pytest.raises(s2r.S2RError) as e:
        s2r.s2r_encode_noalloc(p, W, g, n, n, out["bitmaps"], out["sketches"], out["idx"],
                               out["val"], cap, out["nnz"])
    assert e.value.status == s2r.S2R_ERR_SCRATCH
    torch.cuda.synchronize()
    assert int(out["nnz"][0]) == -1  # nothing was enqueued
