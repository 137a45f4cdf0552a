"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on seeded inputs.

Sizes are ones the oracle finishes in seconds while still spanning several 8192-element
tiles, several 8192-entry list chunks and ragged tails.  Both hash families are covered:
log2_part == log2_w (independent rows; the global-atomic path whenever the d x w table
exceeds the LDS accumulator) and the LDS-partitioned default.
"""
import numpy as np
import pytest

import oracle
import workloads as WL

pytestmark = pytest.mark.gpu

gp = pytest.importorskip("gpu_path")


def _grads(W, n, ld, density, seed, integer=False, pad=0.0, block=None):
    rows = []
    for k in range(W):
        if block:
            idx, val = WL.blocks_sparse(n, block, density, seed + k)
        else:
            idx, val = WL.uniform_sparse(n, density, seed + k, integer=integer)
        rows.append(WL.dense_from_sparse(n, idx, val, ld=ld, fill_pad=pad))
    return np.stack(rows)


# ---------------------------------------------------------------------------------------
# hash


@pytest.mark.parametrize("d,L,K", [(1, 0, 0), (3, 14, 14), (3, 14, 13), (5, 22, 12), (16, 31, 11),
                                   (4, 31, 31), (2, 9, 0), (7, 17, 5)])
def test_hash_bit_exact(d, L, K):
    gp.say(f"hash d={d} L={L} K={K}")
    p, op = gp.params_pair(1234 + L, d, L, K)
    rng = np.random.Generator(np.random.PCG64(L))
    keys = np.concatenate([np.arange(1 << 16), rng.integers(0, 2**32, 1 << 16),
                           [2**32 - 1, 2**31, 2**31 - 1]]).astype(np.uint32)
    b, s = gp.run_hash(p, keys)
    ob, os_ = oracle.hash_keys(op, keys)
    assert np.array_equal(b, ob)
    assert np.array_equal(s, os_)


# ---------------------------------------------------------------------------------------
# encode


ENCODE_CASES = [
    # (name, W, n, ld, density, d, L, K or None, extra)
    ("tiny_cfg_atomic", 4, 1 << 20, 1 << 20, 0.01, 3, 14, 14, {}),
    ("tiny_cfg_partitioned", 4, 1 << 20, 1 << 20, 0.01, 3, 14, None, {}),
    ("n1", 1, 1, 4, 1.0, 3, 10, None, {}),
    ("n63", 2, 63, 64, 0.5, 3, 10, None, {}),
    ("n64", 2, 64, 64, 0.5, 3, 10, 10, {}),
    ("n65_pad_garbage", 3, 65, 72, 0.5, 2, 8, None, {"pad": 7.0}),
    ("tile_edges", 2, 8193, 8196, 0.3, 5, 16, None, {}),
    ("tile_edge_4097", 3, 4097, 4100, 0.6, 3, 12, None, {}),
    ("ragged_many_tiles", 3, 100_003, 100_008, 0.05, 3, 15, None, {"pad": float("nan")}),
    ("dense_all", 2, 20_000, 20_000, 1.0, 3, 12, None, {}),
    # every element non-zero over 37 list chunks per worker: only dense spans, full segments
    ("dense_all_chunks", 2, 300_007, 300_008, 1.0, 5, 20, None, {}),
    ("all_zero", 2, 30_000, 30_000, 0.0, 3, 12, None, {}),
    ("blocks_partitioned", 4, 300_000, 300_000, 0.05, 5, 18, None, {"block": 256}),
    ("blocks_atomic", 2, 300_000, 300_000, 0.05, 5, 18, 18, {"block": 256}),
    ("d1", 2, 50_000, 50_000, 0.1, 1, 12, None, {}),
    ("d16", 2, 50_000, 50_000, 0.1, 16, 12, None, {}),
    ("d2_w1", 2, 5_000, 5_000, 0.1, 2, 0, 0, {}),
    ("w2_K0", 2, 5_000, 5_000, 0.1, 3, 1, 0, {}),
    ("K0_many_partitions", 2, 200_000, 200_000, 0.05, 3, 13, 0, {}),
    # 201 x 4 (worker, partition) items on a walking accumulation grid: two rounds, an item
    # count that is not a multiple of 8, workgroups with one and with two items
    ("walk_ragged_items", 201, 4096, 4096, 0.2, 5, 13, None, {}),
    # 402 tiles x 3 workers: one whole group of 8 XCD runs of 128 tiles, then a ragged tail
    # of 182 tiles in launch order
    ("xcd_runs_ragged", 3, 1_642_497, 1_642_500, 0.01, 3, 15, None, {}),
    # the walking accumulation with 16 and with 7 rows (list capacity / partitions <= 2048)
    ("d16_walk", 3, 20_000, 20_000, 0.1, 16, 14, None, {}),
    ("d7_walk", 3, 30_000, 30_000, 0.1, 7, 15, None, {}),
]


@pytest.mark.parametrize("case", ENCODE_CASES, ids=[c[0] for c in ENCODE_CASES])
def test_encode(case):
    name, W, n, ld, density, d, L, K, extra = case
    gp.say(f"encode {name}: W={W} n={n} ld={ld} d={d} L={L} K={K}")
    p, op = gp.params_pair(WL.HASH_SEED_BASE + len(name), d, L, K)
    grads = _grads(W, n, ld, density, 10 + len(name), pad=extra.get("pad", 0.0),
                   block=extra.get("block"))
    res = gp.run_encode(p, grads, n)
    gp.assert_encode_matches(op, grads, n, res)


@pytest.mark.parametrize("K", [None, 14])
def test_encode_reduce_decode_empty_gradient(K):
    """n == 0 (regression: the list scan once read the word before its tile counts when a
    worker had no tiles): nnz = 0, all-zero sketches, and reduce and decode are no-ops."""
    gp.say(f"encode n=0 K={K}")
    W, d, L = 3, 3, 14  # K = 14: a 192 KiB table, the global-atomic path
    p, op = gp.params_pair(606, d, L, K)
    res = gp.run_encode(p, np.zeros((W, 4), np.float32), 0)
    assert np.array_equal(res["nnz"], np.zeros(W, np.int64))
    assert np.array_equal(res["sketches"], np.zeros((W, d, 1 << L), np.float32))
    gp.assert_encode_matches(op, np.zeros((W, 4), np.float32), 0, res)
    bm, S = gp.run_reduce(p, 0, res["bitmaps"], res["sketches"])
    assert bm.size == 0 and np.array_equal(S, np.zeros((d, 1 << L), np.float32))
    assert gp.run_decode(p, 0, bm, S).size == 0


@pytest.mark.parametrize("K", [None, 15])
def test_encode_integer_values_exact(K):
    """Integer values: every fp32 partial sum is exact, so the sketch must be bit-exact."""
    gp.say(f"encode integer K={K}")
    W, n, d, L = 3, 200_000, 3, 15
    p, op = gp.params_pair(77, d, L, K)
    grads = _grads(W, n, n, 0.2, 5, integer=True)
    res = gp.run_encode(p, grads, n)
    gp.assert_encode_matches(op, grads, n, res, exact_sketch=True)


def test_encode_special_values():
    """+0/-0 are zero; subnormals are non-zero and kept bit-exact."""
    gp.say("encode special values")
    n = 10_000
    g = np.zeros((1, n), np.float32)
    g[0, 1::7] = -0.0
    g[0, 2::11] = np.float32(1e-45)
    g[0, 3::13] = -np.float32(3e-39)
    g[0, 5::17] = np.float32(1.5)
    p, op = gp.params_pair(5, 3, 11)
    res = gp.run_encode(p, g, n)
    gp.assert_encode_matches(op, g, n, res)


@pytest.mark.parametrize("K", [None, 12])
def test_encode_reduce_non_finite_values(K):
    """+Inf, -Inf and NaN have non-zero magnitude bits, so the bitmap and the lists keep them
    with their exact bits like any other value.  A sketch cell they reach is non-finite, and
    of the same kind as the oracle's (NaN where contributions of both infinite signs or a NaN
    meet, else the infinity's signed direction), whatever the order of the adds; every other
    cell is within the tolerance.  The reduce keeps each cell's kind (K = L: the global-atomic
    scatter; default K: the LDS tiles)."""
    gp.say(f"encode/reduce non-finite values K={K}")
    W, n, d, L = 3, 60_000, 3, 12
    p, op = gp.params_pair(808, d, L, K)
    grads = _grads(W, n, n, 0.1, 31)
    rng = np.random.Generator(np.random.PCG64(32))
    special = np.array([np.inf, -np.inf, np.nan, np.inf, -np.inf, np.nan, np.inf], np.float32)
    for k in range(W):
        grads[k, rng.choice(n, special.size, replace=False)] = special
    res = gp.run_encode(p, grads, n)
    for k in range(W):
        e = oracle.encode_dense(op, grads[k, :n], cap=n)
        assert np.array_equal(res["bitmaps"][k], e["bitmap"]), f"worker {k}: bitmap differs"
        assert res["nnz"][k] == e["nnz"]
        m = e["nnz"]
        assert np.array_equal(res["idx"][k, :m], e["idx"])
        assert np.array_equal(res["val"][k, :m].view(np.uint32), e["val"].view(np.uint32))
        S, g = e["S"], res["sketches"][k].astype(np.float64)
        for kind in (np.isnan, np.isposinf, np.isneginf):
            assert np.array_equal(kind(g), kind(S)), f"worker {k}: {kind.__name__} cells differ"
        assert np.isnan(S).any() and np.isinf(S).any()  # the case is exercised
        fin = np.isfinite(S)
        gp.assert_sketch_close(res["sketches"][k][fin], S[fin], e["A"][fin], f"worker {k} sketch")
    _, red = gp.run_reduce(p, n, res["bitmaps"], res["sketches"])
    want = res["sketches"][0].copy()
    for k in range(1, W):
        want = want + res["sketches"][k]  # fp32, worker order
    for kind in (np.isnan, np.isposinf, np.isneginf):
        assert np.array_equal(kind(red), kind(want)), f"reduce: {kind.__name__} cells differ"
    fin = np.isfinite(want)
    assert np.array_equal(red[fin].view(np.uint32), want[fin].view(np.uint32))


@pytest.mark.parametrize("cap", [0, 1, 1000, 8192, 8193])
def test_encode_capacity(cap):
    """nnz beyond cap: bitmap and nnz exact, the first cap list entries exact."""
    gp.say(f"encode capacity cap={cap}")
    W, n = 2, 300_000
    p, op = gp.params_pair(9, 3, 14)
    grads = _grads(W, n, n, 0.05, 3)
    res = gp.run_encode(p, grads, n, cap=cap)
    gp.assert_encode_matches(op, grads, n, res, cap=cap)


def test_encode_reduce_max_workers():
    """W = 65535, the most workers one encode call accepts (one grid row per worker): 100
    elements each at 30% density, d = 3, w = 2^9 in 4 partitions (262,140 (worker,
    partition) items on the walking accumulation grid); then the reduce over all 65535
    sketches and bitmaps against the oracle's."""
    W, n, d, L, K = 65535, 100, 3, 9, 7
    gp.say(f"encode + reduce W={W} n={n} d={d} L={L} K={K}")
    p, op = gp.params_pair(65535, d, L, K)
    rng = np.random.Generator(np.random.PCG64(65535))
    grads = np.zeros((W, n), np.float32)
    mask = rng.random((W, n)) < 0.3
    grads[mask] = rng.standard_normal(int(mask.sum())).astype(np.float32)
    res = gp.run_encode(p, grads, n)
    encs = gp.assert_encode_matches(op, grads, n, res)
    bm, S = gp.run_reduce(p, n, res["bitmaps"], res["sketches"])
    obm, oS, oA = oracle.reduce(np.stack([e["bitmap"] for e in encs]),
                                np.stack([e["S"] for e in encs]), np.stack([e["A"] for e in encs]))
    assert np.array_equal(bm, obm)
    gp.assert_sketch_close(S, oS, oA, "reduced sketch")


def test_encode_deterministic_integer_parts():
    """Two runs give identical bitmaps and lists (catches races in the compaction)."""
    gp.say("encode twice")
    W, n = 4, 400_000
    p, _ = gp.params_pair(21, 5, 18)
    grads = _grads(W, n, n, 0.03, 8, block=512)
    a = gp.run_encode(p, grads, n)
    b = gp.run_encode(p, grads, n)
    for key in ("bitmaps", "idx", "nnz"):
        assert np.array_equal(a[key], b[key])
    assert np.array_equal(a["val"].view(np.uint32), b["val"].view(np.uint32))


# ---------------------------------------------------------------------------------------
# reduce (on tables that do not come from an encode)


@pytest.mark.parametrize("W,d,L,n,inplace", [(1, 3, 10, 1000, False), (4, 3, 14, 1 << 20, False),
                                             (16, 3, 12, 99_999, False), (8, 5, 16, 640, True),
                                             (3, 3, 1, 70, False), (5, 1, 0, 1, False)])
def test_reduce(W, d, L, n, inplace):
    gp.say(f"reduce W={W} d={d} L={L} n={n} inplace={inplace}")
    p, _ = gp.params_pair(3, d, L)
    sk = np.stack([WL.random_sketch((d, 1 << L), 100 + k) for k in range(W)])
    bms = np.stack([WL.random_bitmap(n, 0.1, 200 + k) for k in range(W)])
    bm, S = gp.run_reduce(p, n, bms, sk, inplace=inplace)
    obm, oS, oA = oracle.reduce(bms, sk.astype(np.float64), np.abs(sk.astype(np.float64)))
    assert np.array_equal(bm, obm)
    gp.assert_sketch_close(S, oS, oA, "reduced sketch")
    # the sum runs in worker order: it equals a left-to-right fp32 replay
    replay = sk[0].copy()
    for k in range(1, W):
        replay = replay + sk[k]
    assert np.array_equal(S.view(np.uint32), replay.view(np.uint32))


def test_reduce_integer_exact():
    gp.say("reduce integer")
    W, d, L, n = 8, 5, 13, 5000
    p, _ = gp.params_pair(4, d, L)
    sk = np.stack([WL.random_sketch((d, 1 << L), 300 + k, integer=True) for k in range(W)])
    bms = np.stack([WL.random_bitmap(n, 0.3, 400 + k) for k in range(W)])
    bm, S = gp.run_reduce(p, n, bms, sk)
    obm, oS, _ = oracle.reduce(bms, sk.astype(np.float64), np.abs(sk.astype(np.float64)))
    assert np.array_equal(bm, obm) and np.array_equal(S.astype(np.float64), oS)


# ---------------------------------------------------------------------------------------
# decode (on a generated bitmap and sketch)


DECODE_CASES = [(3, 14, 13, 1 << 20, 0.04), (5, 16, 12, 100_003, 0.3), (1, 10, 10, 4097, 0.5),
                (2, 10, 4, 5000, 0.5), (4, 12, 12, 65, 1.0), (7, 9, 3, 9000, 0.2),
                (16, 11, 11, 3000, 0.2), (5, 20, 12, 1, 1.0), (3, 18, 0, 300_000, 0.6),
                (5, 22, 12, 200_000, 0.02), (3, 20, 20, 50_000, 0.1),
                # 2076 output tiles of 8192: whole groups of 8 XCD runs (64 tiles of the
                # output pass, 256 workgroups of the count pass) and ragged tails
                (5, 20, None, 17_000_003, 0.01),
                # the most partitions the binning allows (2^13) with even d: odd-length
                # rows of 16-bit partition offsets, 8192 median workgroups
                (2, 21, 8, 2_000_003, 0.05),
                # the most rows (16, even: mean of the middle two) and an odd count past the
                # median-of-five network (7) on the partitioned path (tables over 4 MiB)
                (16, 17, 10, 500_003, 0.1), (7, 19, 11, 400_001, 0.1),
                # every bit set: all-ones words in every round of the rank expansion, 37
                # chunks of 8192 set bits and a ragged last chunk, word and tile
                (5, 20, 11, 300_007, 1.0)]


@pytest.mark.parametrize("path", ["direct", "partitioned", "overflow"])
@pytest.mark.parametrize("d,L,K,n,density", DECODE_CASES)
def test_decode(d, L, K, n, density, path):
    gp.say(f"decode d={d} L={L} K={K} n={n} path={path}")
    p, op = gp.params_pair(55 + d, d, L, K)
    sketch = WL.random_sketch((d, 1 << L), 7 * d)
    bm = WL.random_bitmap(n, density, 9 * d)
    # set bits beyond n in the input: they must be ignored
    if n % 64:
        bm[-1] |= np.uint64(~((1 << (n % 64)) - 1) & 0xFFFFFFFFFFFFFFFF)
    out = gp.run_decode(p, n, bm, sketch, path=path)
    want, tol = oracle.decode_dense(op, n, bm, sketch.astype(np.float64))
    setmask = gp.bits_of(bm, n)
    # odd d: the median selects one of the fp32 inputs, so the result is exact
    gp.assert_decode_matches(out, want, tol, setmask, exact=(d % 2 == 1))


@pytest.mark.parametrize("path", ["direct", "partitioned"])
def test_decode_empty_bitmap(path):
    gp.say(f"decode empty {path}")
    p, op = gp.params_pair(1, 3, 12)
    n = 10_000
    out = gp.run_decode(p, n, np.zeros((n + 63) // 64, np.uint64), WL.random_sketch((3, 1 << 12), 2),
                        path=path)
    assert np.all(out.view(np.uint32) == 0)


def test_decode_capacity_boundary():
    """max_set exactly U, and U + 1, and U - 1 (the last falls back on the device)."""
    d, L, n = 5, 16, 200_000
    p, op = gp.params_pair(8, d, L)
    sketch = WL.random_sketch((d, 1 << L), 3)
    bm = WL.random_bitmap(n, 0.25, 4)
    U = int(gp.bits_of(bm, n).sum())
    want, tol = oracle.decode_dense(op, n, bm, sketch.astype(np.float64))
    for ms in (U - 1, U, U + 1, 8192, 8193):
        gp.say(f"decode capacity U={U} max_set={ms}")
        out = gp.run_decode(p, n, bm, sketch, path="partitioned", max_set=ms)
        gp.assert_decode_matches(out, want, tol, gp.bits_of(bm, n), exact=True)


@pytest.mark.parametrize("n,density", [(3_000_000, 0.003), (1_000_003, 0.0004)])
def test_decode_sparse_bitmap_tight_capacity(n, density):
    """A sparse bitmap (fewer set bits than bitmap words) with max_set = U: the partitioned
    decode bins each rank chunk with the wide 1024-thread kernel, over many rounds of
    bitmap words per chunk."""
    d, L = 5, 20  # a 20 MiB table: the partitioned path
    p, op = gp.params_pair(77, d, L)
    sketch = WL.random_sketch((d, 1 << L), 5)
    bm = WL.random_bitmap(n, density, 6)
    U = int(gp.bits_of(bm, n).sum())
    assert U < (n + 63) // 64
    gp.say(f"decode sparse bitmap n={n} U={U}")
    want, tol = oracle.decode_dense(op, n, bm, sketch.astype(np.float64))
    out = gp.run_decode(p, n, bm, sketch, path="partitioned", max_set=U)
    gp.assert_decode_matches(out, want, tol, gp.bits_of(bm, n), exact=True)


@pytest.mark.parametrize("set_bits", [9_999, 10_000, 10_001, 96_000])
def test_decode_unsort_threshold(set_bits):
    """The partitioned decode on both sides of the density where the medians stop being put
    in rank order by a separate pass (fewer than n / 32 set bits: k_dwrite reads each median
    through its rank's slot instead), with exactly `set_bits` set bits out of n = 320,000."""
    d, L, n = 5, 20, 320_000  # a 20 MiB table: the partitioned path; n / 32 = 10,000
    p, op = gp.params_pair(91, d, L)
    sketch = WL.random_sketch((d, 1 << L), 12)
    rng = np.random.Generator(np.random.PCG64(set_bits))
    pos = rng.choice(n, size=set_bits, replace=False)
    bits = np.zeros(((n + 63) // 64) * 64, dtype=np.uint8)
    bits[pos] = 1
    bm = np.packbits(bits, bitorder="little").view(np.uint64).copy()
    assert int(gp.bits_of(bm, n).sum()) == set_bits
    gp.say(f"decode unsort threshold U={set_bits} n={n}")
    want, tol = oracle.decode_dense(op, n, bm, sketch.astype(np.float64))
    for ms in (n, set_bits):
        out = gp.run_decode(p, n, bm, sketch, path="partitioned", max_set=ms)
        gp.assert_decode_matches(out, want, tol, gp.bits_of(bm, n), exact=True)


@pytest.mark.parametrize("pattern,density", [("uniform", 0.0152), ("uniform", 0.0160),
                                             ("runs", 0.30), ("runs", 0.012)])
def test_decode_binning_kernels(pattern, density):
    """The partitioned decode with max_set = U on both sides of the density (one set bit in
    64 elements) where the rank expansion changes from four consecutive bitmap words per
    thread (1024 threads) to four words a round apart (512 threads), a chunk then spanning
    about four rounds; and with the set bits in aligned runs of 1024 (all-ones words), dense
    and sparse.  n = 2,000,003: a ragged last word and tile."""
    d, L, n = 5, 20, 2_000_003
    p, op = gp.params_pair(93, d, L)
    sketch = WL.random_sketch((d, 1 << L), 14)
    if pattern == "uniform":
        bm = WL.random_bitmap(n, density, 15)
    else:
        rng = np.random.Generator(np.random.PCG64(16))
        rows = (n + 1023) // 1024
        pick = rng.random(rows) < density
        bits = np.zeros(((n + 63) // 64) * 64, dtype=np.uint8)
        run = np.repeat(pick, 1024).astype(np.uint8)
        m = min(run.size, bits.size)
        bits[:m] = run[:m]
        bits[n:] = 0
        bm = np.packbits(bits, bitorder="little").view(np.uint64).copy()
    U = int(gp.bits_of(bm, n).sum())
    gp.say(f"decode binning kernels {pattern} density={density} U={U} n={n}")
    want, tol = oracle.decode_dense(op, n, bm, sketch.astype(np.float64))
    out = gp.run_decode(p, n, bm, sketch, path="partitioned", max_set=U)
    gp.assert_decode_matches(out, want, tol, gp.bits_of(bm, n), exact=True)


# ---------------------------------------------------------------------------------------
# end to end


@pytest.mark.parametrize("K", [None, 14])
def test_pipeline_tiny_config(K):
    """The tiny workload end to end (W=4, N=2^20, 1% uniform, d=3, w=2^14)."""
    wl = WL.workload(0)
    gp.say(f"pipeline tiny K={K}")
    p, op = gp.params_pair(wl.hash_seed, wl.d, wl.log2_w, K)
    grads = np.stack([WL.dense_from_sparse(wl.N, *WL.worker_sparse(0, k)) for k in range(wl.W)])
    res = gp.run_encode(p, grads, wl.N)
    encs = gp.assert_encode_matches(op, grads, wl.N, res)
    bm, S = gp.run_reduce(p, wl.N, res["bitmaps"], res["sketches"])
    obm, oS, oA = oracle.reduce(np.stack([e["bitmap"] for e in encs]),
                                np.stack([e["S"] for e in encs]), np.stack([e["A"] for e in encs]))
    assert np.array_equal(bm, obm)
    gp.assert_sketch_close(S, oS, oA, "reduced sketch")
    out = gp.run_decode(p, wl.N, bm, S)
    want, tol = oracle.decode_dense(op, wl.N, obm, oS, oA)
    gp.assert_decode_matches(out, want, tol, gp.bits_of(obm, wl.N))


def test_encode_span_classes():
    """Tile pairs (8192 elements) with exactly 1024 non-zeros (listed one wave per pair), 1025
    (a workgroup per pair), a full pair, and a pair whose non-zeros straddle its two tiles,
    plus a ragged tail: every list entry in place."""
    gp.say("encode span classes")
    n = 8192 * 6 + 777
    ld = (n + 3) // 4 * 4
    rng = np.random.Generator(np.random.PCG64(17))
    g = np.zeros((2, ld), dtype=np.float32)
    for k in range(2):
        for span, cnt in ((0, 1024), (1, 1025), (2, 8192), (4, 1)):
            pos = rng.choice(8192, size=cnt, replace=False) + 8192 * span
            g[k, pos] = rng.standard_normal(cnt).astype(np.float32) + 3.0
        g[k, 8192 * 3 + 4090:8192 * 3 + 4102] = 1.5   # across the tile boundary inside pair 3
        g[k, n - 5:] = -2.0                            # the ragged last pair
    p, op = gp.params_pair(4242, 3, 14)
    res = gp.run_encode(p, g, n)
    gp.assert_encode_matches(op, g, n, res)
    # and with a list capacity that cuts inside the dense pair
    res = gp.run_encode(p, g, n, cap=1500)
    gp.assert_encode_matches(op, g, n, res, cap=1500)
