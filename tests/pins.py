"""Checks that tie the fp64 oracle to what the S2 Reducer pages and mathematics fix.

Each ``pin_*`` function raises AssertionError when the oracle (whichever build the
``oracle`` module currently routes to) disagrees with an independent fact:

  * published SplitMix64 outputs;
  * closed forms of the multiply-add-shift hash for hand-picked constants;
  * statistical properties the method relies on ("randomly mapped" buckets and "random
    sign", S2 Reducer Section 3.1; uniform pairwise mapping, Appendix A.1);
  * the linear-projection view of the sketch, S = A^T g with an explicit mapping matrix
    A in {-1,0,+1}^{N x w} (Section 3.1, "Collecting Sparse-Sketch with AllReduce"), built
    and multiplied here with numpy;
  * zeros leave the sketch unchanged (Section 3.1, "Compressing Sparse Gradient");
  * the sum of sketches equals the sketch of the sum (same passage);
  * the query as the median over rows of (A_j A_j^T g)(i), taken with numpy.median
    (Section 3.1, "Decompressing Sparse Gradient"; Algorithm 1);
  * exact recovery when a majority of an item's buckets hold no other item;
  * block-granular bitmaps (one bit per embedding row or gradient block, Section 3.1): the
    bit of a block is the OR of its elements' non-zero tests, the sketch does not depend
    on the granularity, and every element of a set block is queried;
  * block-wise Top-K with error feedback (Section 2.2; Appendix A.2): numpy's block norms
    and ordering, out + residual = g, the kept mass bound of Theorem 2's proof, and the
    telescoping sum of the error sequence;
  * unbiasedness of the single-row estimate over random hash constants (Theorem 1);
  * the decode bound tol(i) = 1e-5 max_j (mass of row j's cell) + 1e-12, recomputed from the
    explicit |A_j|^T |g| of every worker;
  * the lossless gathered sum (Section 1; Section 2.2, Fig. 1(b)) as numpy's dense sum.

The test modules run every pin against the real oracle and against altered copies of it.
"""
from __future__ import annotations

import os

import numpy as np

import oracle as O
import workloads as WL

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TWO64 = 1 << 64


def _golden_ints(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                out.append(int(line, 0))
    return out


def _mapping_matrices(p, n):
    """Explicit A_j in {-1,0,+1}^{n x w}: A_j[i, h_j(i)] = s_j(i)."""
    keys = np.arange(n, dtype=np.uint32)
    b, s = O.hash_keys(p, keys)
    mats = []
    for j in range(p.d):
        A = np.zeros((n, p.w), dtype=np.float64)
        A[np.arange(n), b[j].astype(np.int64)] = s[j]
        mats.append(A)
    return mats


def _int_grad(n, density, seed):
    idx, val = WL.uniform_sparse(n, density, seed, integer=True)
    return WL.dense_from_sparse(n, idx, val)


# ---------------------------------------------------------------------------------------


def pin_splitmix64():
    assert O.splitmix64(0, 3) == _golden_ints("splitmix64_seed0.txt")


def pin_params_draw_order():
    """Constants are SplitMix64 draws in the order pA, pB, then (hA, hB, sA, sB) per row."""
    seed, d = 12345, 4
    draws = O.splitmix64(seed, 2 + 4 * d)
    p = O.params_from_seed(seed, d, 20, 12)
    assert (p.pA, p.pB) == (draws[0], draws[1])
    for j in range(d):
        assert (p.hA[j], p.hB[j], p.sA[j], p.sB[j]) == tuple(draws[2 + 4 * j: 6 + 4 * j])


def pin_hash_closed_forms():
    keys = np.concatenate([np.arange(0, 4096), [2**31 - 1, 2**31, 2**32 - 2, 2**32 - 1]]).astype(np.uint32)
    k64 = keys.astype(np.int64)
    # (1) K = L = 6; a = c*2^58, b = e*2^58  =>  h(i) = (c*i + e) mod 64
    L = 6
    p = O.params_from_constants(2, L, L, 0, 0, [1 << 58, 3 << 58], [0, 5 << 58], [0, 0], [0, 0])
    b, _ = O.hash_keys(p, keys)
    assert np.array_equal(b[0], (k64 % 64).astype(np.uint32))
    assert np.array_equal(b[1], ((3 * k64 + 5) % 64).astype(np.uint32))
    # (2) a = 2^64-1, b = 1: (1 - i) mod 2^64 -> bucket 0 for i in {0,1}, 2^L-1 for i >= 2;
    #     the add happens before the shift and wraps mod 2^64.
    L = 10
    p = O.params_from_constants(1, L, L, 0, 0, [TWO64 - 1], [1], [0], [0])
    b, _ = O.hash_keys(p, keys)
    want = np.where(k64 >= 2, (1 << L) - 1, 0).astype(np.uint32)
    assert np.array_equal(b[0], want)
    # (3) signs: the top bit of (sA*i + sB) mod 2^64 set means -1
    p = O.params_from_constants(3, 4, 4, 0, 0, [0] * 3, [0] * 3,
                                [0, 0, 1 << 63], [1 << 63, (1 << 63) - 1, 0])
    _, s = O.hash_keys(p, keys)
    assert np.all(s[0] == -1)
    assert np.all(s[1] == 1)
    assert np.array_equal(s[2], np.where(k64 % 2 == 0, 1, -1).astype(np.int8))
    # (4) partitioned buckets, L = 8, K = 3: P(i) = (i + 7) mod 32 in the high 5 bits,
    #     Q_j(i) = ((2j+1) i) mod 8 in the low 3 bits
    L, K = 8, 3
    p = O.params_from_constants(2, L, K, 1 << 59, 7 << 59, [1 << 61, 3 << 61], [0, 0],
                                [0, 0], [0, 0])
    b, _ = O.hash_keys(p, keys)
    for j in range(2):
        want = (((k64 + 7) % 32) << 3) | (((2 * j + 1) * k64) % 8)
        assert np.array_equal(b[j], want.astype(np.uint32))
    # (5) K = 0: every row's bucket is the partition hash alone
    p = O.params_from_constants(2, 5, 0, 1 << 59, 0, [123, 456], [7, 8], [0, 0], [0, 0])
    b, _ = O.hash_keys(p, keys)
    assert np.array_equal(b[0], (k64 % 32).astype(np.uint32))
    assert np.array_equal(b[1], b[0])
    # (6) w = 1: every bucket is 0
    p = O.params_from_seed(99, 3, 0, 0)
    b, _ = O.hash_keys(p, keys)
    assert np.all(b == 0)


def pin_hash_statistics():
    """Buckets look uniform, signs balanced, pair collisions at rate 1/w (Section 3.1's
    random mapping; Appendix A.1 assumes Pr[same bucket] = 1/m)."""
    rng = np.random.Generator(np.random.PCG64(7))
    keys = np.unique(rng.integers(0, 2**32, size=1 << 18, dtype=np.uint64)).astype(np.uint32)
    m = keys.size
    for (L, K) in [(8, 8), (8, 5), (12, 12)]:
        p = O.params_from_seed(2024 + L + K, 3, L, K)
        b, s = O.hash_keys(p, keys)
        w = 1 << L
        for j in range(3):
            cnt = np.bincount(b[j], minlength=w)
            assert cnt.size == w
            exp = m / w
            chi2 = float(((cnt - exp) ** 2 / exp).sum())
            assert chi2 < (w - 1) + 6 * np.sqrt(2 * (w - 1)), (L, K, j, chi2)
            assert abs(int(s[j].astype(np.int64).sum())) < 6 * np.sqrt(m)
        # pair collisions in row 0 at rate 1/w
        x = rng.integers(0, m, size=1 << 20)
        y = rng.integers(0, m, size=1 << 20)
        ok = x != y
        coll = (b[0][x[ok]] == b[0][y[ok]]).mean()
        se = np.sqrt((1 / w) * (1 - 1 / w) / ok.sum())
        assert abs(coll - 1 / w) < 6 * se, (L, K, coll)
        # signs of the same key in two rows are uncorrelated
        assert abs(float((s[0].astype(np.int64) * s[1]).mean())) < 6 / np.sqrt(m)


def pin_bitmap_and_list():
    """Bit i is set exactly where g(i) != 0 (IEEE comparison: -0 == 0, subnormals count);
    the list holds those indices ascending with their exact values; pad bits are 0."""
    n = 200
    rng = np.random.Generator(np.random.PCG64(3))
    g = np.zeros(n, dtype=np.float32)
    pos = rng.choice(n, size=60, replace=False)
    g[pos] = rng.standard_normal(60).astype(np.float32)
    g[5] = -0.0
    g[6] = np.float32(1e-45)   # smallest subnormal
    g[7] = -np.float32(1e-45)
    g[63], g[64], g[127], g[128], g[199] = 1.0, -2.0, 3.0, 4.0, 5.0
    p = O.params_from_seed(1, 2, 6)
    e = O.encode_dense(p, g)
    nz = np.flatnonzero(g != 0)
    bits = np.unpackbits(e["bitmap"].view(np.uint8), bitorder="little")
    assert bits.size == 256
    assert np.array_equal(np.flatnonzero(bits), nz)
    assert e["nnz"] == nz.size
    assert np.array_equal(e["idx"], nz.astype(np.uint32))
    assert np.array_equal(e["val"].view(np.uint32), g[nz].view(np.uint32))
    # list capacity: the count stays exact, the list is cut
    e2 = O.encode_dense(p, g, cap=10)
    assert e2["nnz"] == nz.size and np.array_equal(e2["idx"], nz[:10].astype(np.uint32))


def pin_sketch_projection():
    """S_j = A_j^T g and the absolute mass = |A_j|^T |g|, for every row (Section 3.1)."""
    n = 96
    for (d, L, K, seed) in [(3, 5, 5, 11), (4, 6, 3, 12), (1, 4, 4, 13)]:
        p = O.params_from_seed(seed, d, L, K)
        g = _int_grad(n, 0.4, seed).astype(np.float32)
        e = O.encode_dense(p, g)
        mats = _mapping_matrices(p, n)
        for j in range(d):
            assert np.array_equal(e["S"][j], mats[j].T @ g.astype(np.float64))
            assert np.array_equal(e["A"][j], np.abs(mats[j]).T @ np.abs(g.astype(np.float64)))


def pin_zeros_do_not_matter():
    """Compressing only the non-zeros gives the sketch of the dense vector (Section 3.1)."""
    n = 500
    p = O.params_from_seed(77, 3, 7, 4)
    idx, val = WL.uniform_sparse(n, 0.1, 5)
    g = WL.dense_from_sparse(n, idx, val)
    dense = O.encode_dense(p, g)
    sparse = O.encode_sparse(p, idx, val, n)
    assert np.array_equal(dense["bitmap"], sparse["bitmap"])
    assert np.array_equal(dense["S"], sparse["S"])
    mats = _mapping_matrices(p, n)
    for j in range(3):
        assert np.allclose(dense["S"][j], mats[j].T @ g.astype(np.float64), rtol=0, atol=1e-15)


def pin_linearity():
    """sketch(g1 + g2) = sketch(g1) + sketch(g2), exactly on integer-valued data."""
    n = 300
    p = O.params_from_seed(5, 3, 6, 6)
    g1 = _int_grad(n, 0.2, 1)
    g2 = _int_grad(n, 0.2, 2)
    s12 = O.encode_dense(p, (g1 + g2).astype(np.float32))["S"]
    assert np.array_equal(s12, O.encode_dense(p, g1)["S"] + O.encode_dense(p, g2)["S"])


def pin_signed_permutation():
    """One row whose hash is injective on the indices: the sketch is g with signs."""
    n = 64
    L = 6
    # h(i) = (5 i + 3) mod 64 is a bijection; s(i) = +1 for even i, -1 for odd i
    p = O.params_from_constants(1, L, L, 0, 0, [5 << 58], [3 << 58], [1 << 63], [0])
    g = np.random.Generator(np.random.PCG64(4)).standard_normal(n).astype(np.float32)
    S = O.encode_dense(p, g)["S"][0]
    i = np.arange(n)
    want = np.zeros(1 << L)
    want[(5 * i + 3) % 64] = np.where(i % 2 == 0, 1.0, -1.0) * g.astype(np.float64)
    assert np.array_equal(S, want)


def pin_reduce():
    """The sum of workers' sketches is the sketch of the summed gradient, and the merged
    bitmap marks the union of their non-zeros (Section 3.1, AllReduce step)."""
    n, W = 400, 3
    p = O.params_from_seed(8, 3, 7, 5)
    gs = [_int_grad(n, 0.15, 100 + k) for k in range(W)]
    encs = [O.encode_dense(p, g) for g in gs]
    bm, S, A = O.reduce(np.stack([e["bitmap"] for e in encs]), np.stack([e["S"] for e in encs]),
                        np.stack([e["A"] for e in encs]))
    total = np.sum(np.stack(gs).astype(np.float64), axis=0).astype(np.float32)
    assert np.array_equal(S, O.encode_dense(p, total)["S"])
    assert np.array_equal(A, sum(e["A"] for e in encs))
    union = np.flatnonzero(np.any(np.stack(gs) != 0, axis=0))
    bits = np.unpackbits(bm.view(np.uint8), bitorder="little")[:n]
    assert np.array_equal(np.flatnonzero(bits), union)


def pin_median_query():
    """g_hat(i) = median_j (A_j A_j^T g)(i) at the set bits, 0 elsewhere (Section 3.1)."""
    n = 80
    for d in (1, 2, 3, 4, 5, 7):
        p = O.params_from_seed(300 + d, d, 4, 4 if d % 2 else 2)
        g = _int_grad(n, 0.3, d)
        e = O.encode_dense(p, g)
        out, _ = O.decode_dense(p, n, e["bitmap"], e["S"], e["A"])
        mats = _mapping_matrices(p, n)
        est = np.stack([mats[j] @ (mats[j].T @ g.astype(np.float64)) for j in range(d)])
        want = np.where(g != 0, np.median(est, axis=0), 0.0)
        assert np.array_equal(out, want), d


def pin_exact_recovery():
    """If more than half of an item's rows hold it alone in its bucket, the query returns
    its exact aggregated value (no collision, Section 3.1)."""
    n, W = 2048, 2
    p = O.params_from_seed(42, 5, 9, 9)
    gs = [WL.dense_from_sparse(n, *WL.uniform_sparse(n, 0.05, 10 + k)) for k in range(W)]
    encs = [O.encode_dense(p, g) for g in gs]
    bm, S, A = O.reduce(np.stack([e["bitmap"] for e in encs]), np.stack([e["S"] for e in encs]),
                        np.stack([e["A"] for e in encs]))
    out, _ = O.decode_dense(p, n, bm, S, A)
    total = gs[0].astype(np.float64) + gs[1].astype(np.float64)
    sup = np.flatnonzero(np.any(np.stack(gs) != 0, axis=0))
    b, _ = O.hash_keys(p, sup.astype(np.uint32))
    alone = np.zeros(sup.size, dtype=int)
    for j in range(p.d):
        cnt = np.bincount(b[j], minlength=p.w)
        alone += cnt[b[j]] == 1
    good = sup[alone > p.d // 2]
    assert good.size > sup.size // 2
    assert np.array_equal(out[good], total[good])


def pin_unbiased_single_row():
    """E[g_hat] = g over random hash constants (Theorem 1), single row."""
    n = 48
    g = _int_grad(n, 0.5, 9).astype(np.float64)
    T = 3000
    errs = np.zeros((T, n))
    for t in range(T):
        p = O.params_from_seed(10_000 + t, 1, 3, 3 if t % 2 else 1)
        e = O.encode_dense(p, g.astype(np.float32))
        out, _ = O.decode_dense(p, n, e["bitmap"], e["S"])
        errs[t] = out - g
    sup = g != 0
    mean = errs[:, sup].mean(axis=0)
    se = errs[:, sup].std(axis=0, ddof=1) / np.sqrt(T)
    assert np.all(np.abs(mean) < 5 * se + 1e-12)
    # and the estimate is not trivially exact: collisions do occur with 8 buckets
    assert np.abs(errs[:, sup]).mean() > 0.1


def _block_bits(g, B):
    """numpy: one flag per block of B elements (last block ragged), True if any is non-zero."""
    n = g.size
    nb = (n + B - 1) // B
    pad = np.zeros(nb * B, dtype=np.float32)
    pad[:n] = g
    return (pad.reshape(nb, B) != 0).any(axis=1)


def pin_block_bitmap():
    """Block bit = OR of the block's non-zero tests (ragged last block included); pad bits 0;
    list and sketch unchanged by the granularity (zeros add nothing, Section 3.1)."""
    for (n, lb, seed) in [(200, 2, 31), (333, 3, 32), (1000, 6, 33), (130, 7, 34), (5000, 9, 35)]:
        B = 1 << lb
        rng = np.random.Generator(np.random.PCG64(seed))
        g = np.zeros(n, dtype=np.float32)
        pos = rng.choice(n, size=max(1, n // 25), replace=False)
        g[pos] = rng.standard_normal(pos.size).astype(np.float32)
        g[n - 1] = 1.5   # the ragged last block is set
        g[min(B, n - 1) - 1] = -0.0  # a negative zero sets nothing
        p = O.params_from_seed(seed, 3, 6, 3, log2_block=lb)
        e = O.encode_dense(p, g)
        want = _block_bits(g, B)
        bits = np.unpackbits(e["bitmap"].view(np.uint8), bitorder="little")
        assert e["bitmap"].size == (want.size + 63) // 64
        assert np.array_equal(bits[: want.size].astype(bool), want)
        assert not bits[want.size:].any()
        nz = np.flatnonzero(g != 0)
        assert e["nnz"] == nz.size and np.array_equal(e["idx"], nz.astype(np.uint32))
        mats = _mapping_matrices(p, n)
        for j in range(p.d):
            assert np.array_equal(e["S"][j], mats[j].T @ g.astype(np.float64))


def pin_block_query():
    """Every element of a set block -- zeros inside it too -- decodes to
    median_j (A_j A_j^T g)(i); elements of clear blocks decode to 0 (Section 3.1)."""
    n = 90
    for (d, lb) in [(1, 1), (3, 2), (4, 3), (5, 4)]:
        B = 1 << lb
        p = O.params_from_seed(700 + d, d, 4, 2, log2_block=lb)
        g = _int_grad(n, 0.08, 40 + d)
        e = O.encode_dense(p, g)
        out, tol = O.decode_dense(p, n, e["bitmap"], e["S"], e["A"])
        mats = _mapping_matrices(p, n)
        est = np.stack([mats[j] @ (mats[j].T @ g.astype(np.float64)) for j in range(d)])
        inset = np.repeat(_block_bits(g, B), B)[:n]
        assert inset.sum() > (g != 0).sum()  # some zeros lie inside set blocks
        want = np.where(inset, np.median(est, axis=0), 0.0)
        assert np.array_equal(out, want), (d, lb)
        assert np.array_equal(tol > 0, inset)


def pin_decode_tolerance():
    """The decode bound the parity tests use, tol(i) = 1e-5 * max_j M_j[h_j(i)] + 1e-12 with
    M_j = sum_k |A_j|^T |g_k| the absolute mass of row j after aggregation (the sum of the
    magnitudes of every contribution to the cell, Section 3.1's projection A^T g with |A|
    and |g|), recomputed here from explicit mapping matrices at every queried element:
    rows d = 1..7, two workers, an element-granular and a block-granular bitmap.  Integer
    data make every mass exact, so the bound must match bit for bit."""
    n, W = 120, 2
    for (d, L, K, lb) in [(1, 4, 4, 0), (2, 5, 2, 0), (3, 4, 1, 0), (4, 6, 6, 0), (5, 5, 3, 0),
                          (6, 4, 4, 0), (7, 5, 2, 0), (3, 5, 3, 2)]:
        p = O.params_from_seed(900 + 10 * d + lb, d, L, K, log2_block=lb)
        gs = [_int_grad(n, 0.2, 60 + 7 * d + k) for k in range(W)]
        # one large-magnitude element, so the bound differs from cell to cell by orders
        gs[1][17] = np.float32(3000.0)
        encs = [O.encode_dense(p, g) for g in gs]
        bm, S, A = O.reduce(np.stack([e["bitmap"] for e in encs]), np.stack([e["S"] for e in encs]),
                            np.stack([e["A"] for e in encs]))
        idx, _, tol = O.decode(p, n, bm, S, A)
        mats = _mapping_matrices(p, n)
        absg = sum(np.abs(g.astype(np.float64)) for g in gs)
        mass = np.stack([np.abs(mats[j]).T @ absg for j in range(d)])  # [d][w]
        keys = idx.astype(np.int64)
        per_row = np.stack([mass[j][np.argmax(np.abs(mats[j][keys]), axis=1)] for j in range(d)])
        want = 1e-5 * per_row.max(axis=0) + 1e-12
        assert idx.size > 0 and np.array_equal(tol, want), (d, lb)


def pin_gather_sum():
    """The lossless aggregate (Section 1; Section 2.2, Fig. 1(b)): gathering every worker's
    (index, value) list and adding gives numpy's sum of the dense gradients; the mass is the
    sum of magnitudes; indices at or beyond n are skipped; an empty list adds nothing."""
    n, W = 700, 4
    gs = [_int_grad(n, 0.15, 500 + k) for k in range(W)]
    gs[2][:] = 0  # one worker with an empty list
    lists = [(np.flatnonzero(g).astype(np.uint32), g[g != 0]) for g in gs]
    out, mass = O.gather_sum(lists, n)
    dense = np.stack(gs).astype(np.float64)
    assert np.array_equal(out, dense.sum(axis=0))
    assert np.array_equal(mass, np.abs(dense).sum(axis=0))
    # entries at or beyond n change nothing
    extra = [(np.append(i, np.uint32(n + k)), np.append(v, np.float32(5.0))) for k, (i, v) in
             enumerate(lists)]
    out2, _ = O.gather_sum(extra, n)
    assert np.array_equal(out2, out)
    # one worker alone: its gradient back
    out1, _ = O.gather_sum(lists[:1], n)
    assert np.array_equal(out1, gs[0].astype(np.float64))


def _topk_numpy(g, block, K):
    """numpy: squared block norms (fp64), kept blocks by (norm desc, id asc), out, residual."""
    n = g.size
    nb = -(-n // block)
    pad = np.zeros(nb * block, dtype=np.float64)
    pad[:n] = g.astype(np.float64)
    norm2 = (pad.reshape(nb, block) ** 2).sum(axis=1)
    order = np.lexsort((np.arange(nb), -norm2))
    kept = np.zeros(nb, dtype=bool)
    kept[order[:K]] = True
    em = np.repeat(kept, block)[:n]
    return norm2, kept, np.where(em, g, np.float32(0)), np.where(em, np.float32(0), g)


def pin_topk_numpy():
    """Integer-valued data (every square and sum exact): norms, kept set with planted ties
    (identical blocks, zero blocks), out and residual equal numpy's (Section 2.2)."""
    for (n, block, seed) in [(1000, 10, 1), (1001, 16, 2), (257, 256, 3), (5000, 64, 4), (7, 3, 5)]:
        rng = np.random.Generator(np.random.PCG64(seed))
        nb = -(-n // block)
        grad = rng.integers(-8, 9, size=n).astype(np.float32)
        grad[rng.random(n) < 0.5] = 0
        if nb >= 4:  # a tie between two identical blocks and a run of zero blocks
            grad[block:2 * block] = grad[:block]
            grad[2 * block:min(n, 4 * block)] = 0
        res = rng.integers(-2, 3, size=n).astype(np.float32)
        for K in sorted({0, 1, nb // 3, nb // 2, nb - 1, nb, nb + 5}):
            if K < 0:
                continue
            o = O.topk_ef(grad, res, block, K)
            g = grad + res
            norm2, kept, out, resid = _topk_numpy(g, block, K)
            assert np.array_equal(o["norm2"], norm2), (n, block, K)
            bits = np.unpackbits(o["selected"].view(np.uint8), bitorder="little")
            assert np.array_equal(bits[:nb].astype(bool), kept), (n, block, K)
            assert not bits[nb:].any()
            assert np.array_equal(o["out"], out) and np.array_equal(o["residual"], resid)
            o2 = O.topk_ef(grad, None, block, K)  # no error feedback: g = grad
            _, kept2, out2, _ = _topk_numpy(grad, block, K)
            assert o2["residual"] is None and np.array_equal(o2["out"], out2)


def pin_topk_identities():
    """Float data: out + residual = g exactly with disjoint supports; the kept squared mass
    is at least K/b of the total (the bound in the proof of Theorem 2)."""
    rng = np.random.Generator(np.random.PCG64(21))
    n, block = 20_000, 100
    nb = n // block
    grad = (rng.standard_normal(n) * rng.exponential(1.0, size=n)).astype(np.float32)
    res = (rng.standard_normal(n) * 0.1).astype(np.float32)
    g = grad + res
    for K in (1, 7, 50, 199):
        o = O.topk_ef(grad, res, block, K)
        assert np.array_equal(o["out"] + o["residual"], g)
        assert not np.any((o["out"] != 0) & (o["residual"] != 0))
        kept_mass = float((o["out"].astype(np.float64) ** 2).sum())
        assert kept_mass >= K / nb * float((g.astype(np.float64) ** 2).sum()) * (1 - 1e-12)
        assert np.allclose(o["norm2"], _topk_numpy(g, block, K)[0], rtol=1e-12, atol=0)


def pin_topk_error_feedback():
    """Over T steps with the residual carried, sum_t out_t + e_T = sum_t gradient_t exactly
    (integer data): the error sequence loses nothing (Appendix A.2)."""
    rng = np.random.Generator(np.random.PCG64(31))
    n, block, K, T = 3000, 30, 9, 12
    e = np.zeros(n, dtype=np.float32)
    sent = np.zeros(n, dtype=np.float64)
    total = np.zeros(n, dtype=np.float64)
    for t in range(T):
        grad = rng.integers(-5, 6, size=n).astype(np.float32)
        o = O.topk_ef(grad, e, block, K)
        e = o["residual"]
        sent += o["out"]
        total += grad
        assert int((o["out"] != 0).sum()) <= K * block
    assert np.array_equal(sent + e, total)


ALL_PINS = [
    pin_splitmix64, pin_params_draw_order, pin_hash_closed_forms, pin_hash_statistics,
    pin_bitmap_and_list, pin_sketch_projection, pin_zeros_do_not_matter, pin_linearity,
    pin_signed_permutation, pin_reduce, pin_median_query, pin_exact_recovery,
    pin_unbiased_single_row, pin_decode_tolerance, pin_block_bitmap, pin_block_query,
    pin_gather_sum, pin_topk_numpy,
    pin_topk_identities, pin_topk_error_feedback,
]
