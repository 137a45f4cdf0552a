"""GPU parity of block-wise Top-K sparsification with error feedback (S2 Reducer Section 2.2;
Appendix A.2) against the fp64 oracle on seeded inputs.

The kept-block set must equal the oracle's (unless two squared norms tie to within fp64
rounding, where any valid Top-K is accepted); given the kept set, the sparse output and the
new residual are bit-exact.  Cases cover ragged last blocks, block sizes that are and are not
multiples of 4, K = 0 / 1 / nb - 1 / nb / more, exact ties decided by block id (integer data
with identical blocks), running without error feedback, and several steps with the residual
carried.
"""
import numpy as np
import pytest

import workloads as WL

pytestmark = pytest.mark.gpu

gp = pytest.importorskip("gpu_path")


def _dense(W, n, ld, seed, scale=1.0, integer=False, pad=0.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = np.full((W, ld), pad, dtype=np.float32)
    if integer:
        x[:, :n] = rng.integers(-6, 7, size=(W, n)).astype(np.float32)
    else:
        x[:, :n] = (rng.standard_normal((W, n)) * scale).astype(np.float32)
    return x


CASES = [
    # (name, W, n, ld, block, K, error feedback)
    ("resnet_like_ragged", 3, 100_003, 100_004, 256, 4, True),
    ("block512_no_ef", 2, 300_000, 300_000, 512, 6, False),
    ("block37_scalar", 2, 50_001, 50_004, 37, 40, True),
    ("block1_elements", 2, 20_000, 20_000, 1, 1000, True),
    ("K0", 2, 10_000, 10_000, 64, 0, True),
    ("K1", 2, 10_000, 10_000, 64, 1, True),
    ("K_nb_minus_1", 2, 10_000, 10_000, 64, 156, True),
    ("K_all", 2, 10_000, 10_000, 64, 157, True),
    ("K_more", 2, 10_000, 10_000, 64, 10_000, False),
    ("n_small", 3, 5, 8, 2, 2, True),
    ("many_blocks", 2, 2_000_000, 2_000_000, 16, 12_500, True),
    ("block3", 2, 30_001, 30_004, 3, 2_000, True),
    ("block1000", 2, 250_000, 250_000, 1000, 25, True),
    ("block_beyond_n", 2, 100_000, 100_000, 1 << 31, 1, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_topk(case):
    name, W, n, ld, block, K, ef = case
    gp.say(f"topk {name}: W={W} n={n} block={block} K={K} ef={ef}")
    grads = _dense(W, n, ld, 11 + len(name), pad=float("nan"))
    res = _dense(W, n, ld, 99 + len(name), scale=0.1, pad=5.0) if ef else None
    out, res_out, sel = gp.run_topk(grads, res, n, block, K)
    gp.assert_topk_matches(grads, res, n, block, K, out, res_out, sel, name)


@pytest.mark.parametrize("K", [3, 5, 8])
def test_topk_ties_by_block_id(K):
    """Integer data with identical blocks and zero blocks: equal squared norms are exact on
    both sides, and the lower block ids must win."""
    W, n, block = 2, 64 * 40, 64
    gp.say(f"topk ties K={K}")
    grads = _dense(W, n, n, 5, integer=True)
    for k in range(W):
        grads[k, 64 * 3:64 * 4] = grads[k, 0:64]          # blocks 0, 3, 7 identical
        grads[k, 64 * 7:64 * 8] = grads[k, 0:64]
        grads[k, 64 * 10:64 * 40] = 0                     # 30 zero blocks
        grads[k, 0:64] *= 3                               # now block 0 is the largest
        grads[k, 64 * 3:64 * 4] *= 2                      # blocks 3 and 7 differ again ...
        grads[k, 64 * 7:64 * 8] *= 2                      # ... but tie with each other
    res = np.zeros_like(grads)
    out, res_out, sel = gp.run_topk(grads, res, n, block, K)
    gp.assert_topk_matches(grads, res, n, block, K, out, res_out, sel, f"ties K={K}")


@pytest.mark.parametrize("K", [100, 5_000, 59_000])
def test_topk_large_tie_group(K):
    """60,000 blocks, all but 100 of them with one identical norm: more equal keys than any
    candidate list holds, so the select ranks the whole tie group from the keys themselves;
    K inside the group keeps the lowest block ids, K = 100 keeps exactly the distinct ones."""
    W, n, block = 2, 240_000, 4
    gp.say(f"topk large tie group K={K}")
    grads = np.ones((W, n), dtype=np.float32)
    for k in range(W):
        rows = np.random.default_rng(70 + k).choice(n // block, 100, replace=False)
        for r in rows:
            grads[k, r * block:(r + 1) * block] = 2.0
    res = np.zeros_like(grads)
    out, res_out, sel = gp.run_topk(grads, res, n, block, K)
    gp.assert_topk_matches(grads, res, n, block, K, out, res_out, sel, f"tie group K={K}")


def test_topk_zero_blocks_fill_K():
    """Fewer non-zero blocks than K: the zero blocks tie at 0 and the lowest ids fill K."""
    W, n, block, K = 2, 6400, 64, 30
    gp.say("topk zero fill")
    grads = np.zeros((W, n), dtype=np.float32)
    grads[:, 64 * 50:64 * 52] = 1.0
    out, res_out, sel = gp.run_topk(grads, np.zeros_like(grads), n, block, K)
    gp.assert_topk_matches(grads, np.zeros_like(grads), n, block, K, out, res_out, sel, "zero fill")


def test_topk_error_feedback_steps():
    """Five steps with the residual carried on both sides, ResNet-50-like blocks of 256."""
    W, n, block, K = 4, 1 << 20, 256, 41
    grads_all = [_dense(W, n, n, 300 + t) for t in range(5)]
    res_gpu = np.zeros((W, n), dtype=np.float32)
    res_ref = np.zeros((W, n), dtype=np.float32)
    for t, grads in enumerate(grads_all):
        gp.say(f"topk ef step {t}")
        out, res_gpu_new, sel = gp.run_topk(grads, res_gpu, n, block, K)
        gp.assert_topk_matches(grads, res_ref, n, block, K, out, res_gpu_new, sel, f"step {t}")
        res_gpu = res_gpu_new
        res_ref = res_gpu_new.copy()  # equal to the oracle's residual (just asserted)


def test_topk_feeds_encode():
    """The sparse output goes straight into s2r_encode; its block bitmap at the Top-K block
    size equals the kept set wherever a kept block has a non-zero."""
    import oracle
    W, n, block, K, lb = 2, 1 << 18, 256, 10, 8
    gp.say("topk -> encode")
    grads = _dense(W, n, n, 77)
    out, _, sel = gp.run_topk(grads, None, n, block, K)
    p, op = gp.params_pair(123, 3, 16, None, log2_block=lb)
    res = gp.run_encode(p, out, n)
    gp.assert_encode_matches(op, out, n, res)
    for k in range(W):
        assert np.array_equal(res["bitmaps"][k], sel[k])
