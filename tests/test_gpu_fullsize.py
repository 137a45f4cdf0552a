"""Full-size parity: each large workload at its real shape, in the launch configuration the
benchmark times (default partitioned hash, list capacity = the largest worker's nnz,
partitioned decode with max_set = sum of nnz), against the fp64 oracle.

Every output is compared, not a sample:
  * per-worker bitmaps, nnz and lists: bit-exact (the lists against the generator's own
    ascending (index, value) pairs, which are exactly Sparse(g_k));
  * per-worker and merged sketch cells: |gpu - S| <= 1e-5 * A + 1e-12;
  * merged bitmap: bit-exact;
  * decoded values at every set bit within tol(i), every clear bit exactly +0.0.
The oracle compresses each worker from Sparse(g_k), the input form of Algorithm 1.
The block-granular cases use the workloads' own row or block size as the bitmap block
(embedding rows of 512, ResNet-50 blocks of 256, Transformer blocks of 512).
"""
import gc

import numpy as np
import pytest
import torch

import count_sketch_aggregation_amd as s2r
import oracle
import workloads as WL

pytestmark = pytest.mark.gpu

gp = pytest.importorskip("gpu_path")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cid,lb", [(1, 0), (2, 0), (3, 0), (4, 0), (1, 9), (2, 8), (3, 9)])
def test_fullsize_pipeline(cid, lb):
    wl = WL.workload(cid)
    dev = gp.DEV
    gp.say(f"fullsize {wl.name}: W={wl.W} N={wl.N} d={wl.d} w=2^{wl.log2_w} B=2^{lb}")
    p, op = gp.params_pair(wl.hash_seed, wl.d, wl.log2_w, log2_block=lb)
    ld = (wl.N + 3) // 4 * 4
    grad = torch.zeros((wl.W, ld), dtype=torch.float32, device=dev)
    sparse = []
    for k in range(wl.W):
        idx, val = WL.worker_sparse(cid, k)
        grad[k].index_copy_(0, torch.from_numpy(idx.astype(np.int64)).to(dev),
                            torch.from_numpy(val).to(dev))
        sparse.append((idx, val))
    cap = max(x[0].size for x in sparse)
    # the merged query set holds at most every worker's touched blocks
    max_set = min(wl.N, sum(np.unique(x[0] >> lb).size << lb for x in sparse))
    buf = s2r.alloc_encode_buffers(p, wl.W, wl.N, cap, dev)
    words = s2r.s2r_block_bitmap_words(wl.N, lb)
    bm = torch.empty(words, dtype=torch.int64, device=dev)
    sk = torch.empty((wl.d, wl.w), dtype=torch.float32, device=dev)
    out = torch.full((wl.N,), float("nan"), dtype=torch.float32, device=dev)
    dws = s2r.alloc_decode_workspace(p, wl.N, max_set, dev)
    s2r.s2r_encode(p, wl.W, grad, wl.N, ld, buf["bitmaps"], buf["sketches"], buf["idx"], buf["val"],
                   cap, buf["nnz"], buf["workspace"])
    s2r.s2r_reduce(p, wl.W, wl.N, buf["bitmaps"], buf["sketches"], bm, sk)
    s2r.s2r_decode(p, wl.N, bm, sk, out, max_set=max_set, workspace=dws)
    torch.cuda.synchronize()
    del grad
    gp.say("  gpu done; checking workers")

    nnz = buf["nnz"].cpu().numpy()
    bitmaps = np.empty((wl.W, words), dtype=np.uint64)
    S_all = np.empty((wl.W, wl.d, wl.w))
    A_all = np.empty((wl.W, wl.d, wl.w))
    for k in range(wl.W):
        idx, val = sparse[k]
        e = oracle.encode_sparse(op, idx, val, wl.N)
        gbm = buf["bitmaps"][k].cpu().numpy().view(np.uint64)
        assert np.array_equal(gbm, e["bitmap"]), f"worker {k}: bitmap"
        assert int(nnz[k]) == idx.size, f"worker {k}: nnz {nnz[k]} vs {idx.size}"
        assert np.array_equal(buf["idx"][k, : idx.size].cpu().numpy().view(np.uint32), idx), \
            f"worker {k}: list indices"
        assert np.array_equal(buf["val"][k, : idx.size].cpu().numpy().view(np.uint32),
                              val.view(np.uint32)), f"worker {k}: list values"
        gp.assert_sketch_close(buf["sketches"][k].cpu().numpy(), e["S"], e["A"], f"worker {k} sketch")
        bitmaps[k], S_all[k], A_all[k] = e["bitmap"], e["S"], e["A"]
        del e
        gc.collect()
    gp.say("  checking merge")
    obm, oS, oA = oracle.reduce(bitmaps, S_all, A_all)
    del S_all, A_all, bitmaps
    gc.collect()
    assert np.array_equal(bm.cpu().numpy().view(np.uint64), obm), "merged bitmap"
    gp.assert_sketch_close(sk.cpu().numpy(), oS, oA, "merged sketch")
    gp.say("  checking decode")
    oi, ov, ot = oracle.decode(op, wl.N, obm, oS, oA)
    got = out.cpu().numpy()
    setmask = np.zeros(wl.N, dtype=bool)
    setmask[oi] = True
    assert np.array_equal(setmask, gp.set_elements(obm, wl.N, lb))
    assert np.all(got[~setmask].view(np.uint32) == 0), "clear bits must decode to +0.0"
    g = got[oi].astype(np.float64)
    bad = ~(np.abs(g - ov) <= ot)
    assert not bad.any(), f"{int(bad.sum())} decoded values outside tolerance, e.g. " \
        f"i={oi[bad][:5].tolist()} gpu={g[bad][:5]} oracle={ov[bad][:5]} tol={ot[bad][:5]}"
    gp.say(f"  ok: nnz/worker max {int(nnz.max())}, set bits {oi.size}")


@pytest.mark.timeout(900)
def test_fullsize_topk_resnet():
    """Block-wise Top-K with error feedback at the ResNet-50 workload's size (W=16,
    N=25,557,032, blocks of 256, K = 999), two steps with the residual carried: kept sets,
    outputs and residuals against the oracle; the first step's kept blocks are exactly the
    workload's own Top-1% blocks."""
    wl = WL.workload(2)
    block = 256
    nb = -(-wl.N // block)
    K = -(-nb // 100)
    gp.say(f"fullsize topk {wl.name}: W={wl.W} N={wl.N} K={K}")
    ld = (wl.N + 3) // 4 * 4
    grads = np.zeros((wl.W, ld), dtype=np.float32)
    for k in range(wl.W):
        grads[k, :wl.N] = WL.worker_dense(2, k)
    res = np.zeros_like(grads)
    for step in range(2):
        out, res_new, sel = gp.run_topk(grads, res, wl.N, block, K)
        gp.say(f"  step {step}: gpu done")
        gp.assert_topk_matches(grads, res, wl.N, block, K, out, res_new, sel, f"step {step}")
        if step == 0:
            for k in range(3):
                idx, val = WL.worker_sparse(2, k)
                nzi = np.flatnonzero(out[k, :wl.N])
                assert np.array_equal(nzi, idx.astype(np.int64)), f"worker {k}: kept elements"
        res = res_new


@pytest.mark.timeout(900)
def test_maxsize_pipeline():
    """n = 2^32 - 1, the largest size the boundary accepts (indices are 32-bit): W = 2
    workers of about a million uniform non-zeros each plus the 32-bit edge indices (0, 2^31
    and the last element n - 1), a non-zero pad element at index n inside the row stride
    (it must be ignored), d = 5, w = 2^23.  Lists, bitmaps and nnz bit-exact, sketches within
    1e-5 * A + 1e-12, and the decode checked on the device: every set element within tol(i)
    and every other one of the 2^32 - 1 outputs exactly +0.0."""
    W, n, d, L = 2, 2**32 - 1, 5, 23
    ld = 2**32
    dev = gp.DEV
    gp.say(f"maxsize: W={W} n={n} d={d} w=2^{L}")
    p, op = gp.params_pair(4243, d, L)
    grad = torch.zeros((W, ld), dtype=torch.float32, device=dev)
    grad[:, n] = 3.0  # the pad element past n
    edges = np.array([0, 1, 63, 64, 4095, 4096, 2**31 - 1, 2**31, 2**32 - 8193, 2**32 - 65,
                      2**32 - 3, n - 1], dtype=np.uint64)
    sparse = []
    for k in range(W):
        rng = np.random.Generator(np.random.PCG64(4300 + k))
        idx = np.unique(np.concatenate([rng.integers(0, n, 1_000_000, dtype=np.uint64), edges]))
        val = rng.standard_normal(idx.size).astype(np.float32)
        val[val == 0] = 1.0
        idx = idx.astype(np.uint32)
        grad[k].index_copy_(0, torch.from_numpy(idx.astype(np.int64)).to(dev),
                            torch.from_numpy(val).to(dev))
        sparse.append((idx, val))
    cap = max(x[0].size for x in sparse)
    max_set = sum(x[0].size for x in sparse)
    buf = s2r.alloc_encode_buffers(p, W, n, cap, dev)
    words = s2r.s2r_block_bitmap_words(n, 0)
    bm = torch.empty(words, dtype=torch.int64, device=dev)
    sk = torch.empty((d, 1 << L), dtype=torch.float32, device=dev)
    dws = s2r.alloc_decode_workspace(p, n, max_set, dev)
    s2r.s2r_encode(p, W, grad, n, ld, buf["bitmaps"], buf["sketches"], buf["idx"], buf["val"],
                   cap, buf["nnz"], buf["workspace"])
    torch.cuda.synchronize()
    del grad
    out = torch.full((n,), float("nan"), dtype=torch.float32, device=dev)
    s2r.s2r_reduce(p, W, n, buf["bitmaps"], buf["sketches"], bm, sk)
    s2r.s2r_decode(p, n, bm, sk, out, max_set=max_set, workspace=dws)
    torch.cuda.synchronize()
    gp.say("  gpu done; checking workers")
    nnz = buf["nnz"].cpu().numpy()
    bitmaps = np.empty((W, words), dtype=np.uint64)
    S_all = np.empty((W, d, 1 << L))
    A_all = np.empty((W, d, 1 << L))
    for k in range(W):
        idx, val = sparse[k]
        e = oracle.encode_sparse(op, idx, val, n)
        assert np.array_equal(buf["bitmaps"][k].cpu().numpy().view(np.uint64), e["bitmap"]), \
            f"worker {k}: bitmap"
        assert int(nnz[k]) == idx.size, f"worker {k}: nnz {nnz[k]} vs {idx.size}"
        assert np.array_equal(buf["idx"][k, : idx.size].cpu().numpy().view(np.uint32), idx), \
            f"worker {k}: list indices"
        assert np.array_equal(buf["val"][k, : idx.size].cpu().numpy().view(np.uint32),
                              val.view(np.uint32)), f"worker {k}: list values"
        gp.assert_sketch_close(buf["sketches"][k].cpu().numpy(), e["S"], e["A"], f"worker {k} sketch")
        bitmaps[k], S_all[k], A_all[k] = e["bitmap"], e["S"], e["A"]
        del e
        gc.collect()
    gp.say("  checking merge")
    obm, oS, oA = oracle.reduce(bitmaps, S_all, A_all)
    del S_all, A_all, bitmaps
    gc.collect()
    assert np.array_equal(bm.cpu().numpy().view(np.uint64), obm), "merged bitmap"
    gp.assert_sketch_close(sk.cpu().numpy(), oS, oA, "merged sketch")
    gp.say("  checking decode")
    oi, ov, ot = oracle.decode(op, n, obm, oS, oA)
    assert np.array_equal(oi, np.unique(np.concatenate([x[0] for x in sparse])))
    at = torch.from_numpy(oi.astype(np.int64)).to(dev)
    g = out.index_select(0, at).cpu().numpy().astype(np.float64)
    bad = ~(np.abs(g - ov) <= ot)
    assert not bad.any(), f"{int(bad.sum())} decoded values outside tolerance, e.g. " \
        f"i={oi[bad][:5].tolist()} gpu={g[bad][:5]} oracle={ov[bad][:5]} tol={ot[bad][:5]}"
    out.index_fill_(0, at, 0.0)
    assert int(torch.count_nonzero(out.view(torch.int32))) == 0, \
        "clear bits must decode to +0.0"
    gp.say(f"  ok: set bits {oi.size}")
