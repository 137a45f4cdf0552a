"""GPU parity of block-granular bitmaps (one bit per embedding row or gradient block,
S2 Reducer Section 3.1) against the fp64 oracle at the same granularity.

The bitmap of worker k has one bit per block of B = 2^log2_block elements, set when any
element of the block is non-zero; the list and the sketch are those of the element
granularity; decoding queries every element of every set block (zeros inside a set block
get a median estimate too).  Bit-exact bitmaps and lists, sketch and decode tolerances as
in the element-granular tests.
"""
import numpy as np
import pytest

import oracle
import workloads as WL

pytestmark = pytest.mark.gpu

gp = pytest.importorskip("gpu_path")


def _grads(W, n, ld, seed, block, keep):
    rows = []
    for k in range(W):
        idx, val = WL.blocks_sparse(n, block, keep, seed + k)
        rows.append(WL.dense_from_sparse(n, idx, val, ld=ld))
    return np.stack(rows)


BLOCK_ENCODE = [
    # (name, W, n, ld, data block, keep fraction, d, L, K, log2_block)
    ("b2_ragged", 3, 100_003, 100_008, 64, 0.05, 3, 15, None, 1),
    ("b8_ragged", 3, 100_003, 100_008, 64, 0.05, 3, 15, None, 3),
    ("b64_aligned", 2, 8193, 8196, 64, 0.2, 5, 16, None, 6),
    ("b256_misaligned_data", 4, 300_000, 300_000, 200, 0.03, 5, 18, None, 8),
    ("b512_rows", 4, 1 << 20, 1 << 20, 512, 0.02, 5, 18, None, 9),
    ("b512_atomic", 2, 300_000, 300_000, 512, 0.05, 5, 18, 18, 9),
    ("b4096_tile", 3, 50_000, 50_000, 300, 0.05, 3, 12, None, 12),
    ("b65536_bigger_than_n", 2, 50_000, 50_000, 300, 0.02, 3, 12, None, 16),
]


@pytest.mark.parametrize("case", BLOCK_ENCODE, ids=[c[0] for c in BLOCK_ENCODE])
def test_block_encode(case):
    name, W, n, ld, blk, keep, d, L, K, lb = case
    gp.say(f"block encode {name}: W={W} n={n} B=2^{lb}")
    p, op = gp.params_pair(WL.HASH_SEED_BASE + 7 * lb, d, L, K, log2_block=lb)
    grads = _grads(W, n, ld, 100 + lb, blk, keep)
    res = gp.run_encode(p, grads, n)
    gp.assert_encode_matches(op, grads, n, res)


@pytest.mark.parametrize("path", ["direct", "partitioned", "overflow"])
@pytest.mark.parametrize("lb,d,L,K,n,density", [(1, 3, 14, 13, 100_003, 0.1), (2, 5, 16, 12, 65_537, 0.2),
                                                (5, 4, 12, 12, 9000, 0.3), (6, 3, 20, 12, 300_000, 0.05),
                                                (9, 5, 22, 12, 1 << 20, 0.03), (12, 1, 10, 10, 40_000, 0.5),
                                                # the largest block (2^16), a ragged last block
                                                (16, 3, 20, 12, 1_000_003, 0.4)])
def test_block_decode(lb, d, L, K, n, density, path):
    gp.say(f"block decode B=2^{lb} d={d} L={L} K={K} n={n} path={path}")
    p, op = gp.params_pair(60 + lb, d, L, K, log2_block=lb)
    B = 1 << lb
    nblocks = (n + B - 1) // B
    sketch = WL.random_sketch((d, 1 << L), 5 * lb)
    bm = WL.random_bitmap(nblocks, density, 3 * lb)
    if nblocks % 64:  # bits of blocks beyond the last must be ignored
        bm[-1] |= np.uint64(~((1 << (nblocks % 64)) - 1) & 0xFFFFFFFFFFFFFFFF)
    setmask = gp.set_elements(bm, n, lb)
    out = gp.run_decode(p, n, bm, sketch, path=path, max_set=int(setmask.sum()) if path == "partitioned" else None)
    want, tol = oracle.decode_dense(op, n, bm, sketch.astype(np.float64))
    assert np.array_equal(tol > 0, setmask)
    gp.assert_decode_matches(out, want, tol, setmask, exact=(d % 2 == 1))


@pytest.mark.parametrize("lb", [6, 9])
def test_block_pipeline(lb):
    """Encode -> reduce -> decode with row-like data blocks of 200 elements, so set bitmap
    blocks hold zeros as well: every element of a set block is decoded."""
    W, n, d, L = 4, 1 << 20, 5, 20
    gp.say(f"block pipeline B=2^{lb}")
    p, op = gp.params_pair(909, d, L, None, log2_block=lb)
    grads = _grads(W, n, n, 300, 200, 0.01)
    res = gp.run_encode(p, grads, n)
    encs = gp.assert_encode_matches(op, grads, n, res)
    bm, S = gp.run_reduce(p, n, res["bitmaps"], res["sketches"])
    obm, oS, oA = oracle.reduce(np.stack([e["bitmap"] for e in encs]),
                                np.stack([e["S"] for e in encs]), np.stack([e["A"] for e in encs]))
    assert np.array_equal(bm, obm)
    gp.assert_sketch_close(S, oS, oA, "reduced sketch")
    setmask = gp.set_elements(obm, n, lb)
    assert setmask.sum() > (np.stack(grads) != 0).any(axis=0).sum()  # zeros inside set blocks
    for path in ("direct", "partitioned"):
        out = gp.run_decode(p, n, bm, S, path=path)
        want, tol = oracle.decode_dense(op, n, obm, oS, oA)
        gp.assert_decode_matches(out, want, tol, setmask)
