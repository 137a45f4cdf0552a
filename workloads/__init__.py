"""Seeded synthetic gradient generators for sparse-sketch aggregation.

This module only draws inputs: it holds none of the method's arithmetic (no hashing, no
sketching, no medians) and is shared by the tests, the benchmark and the smoke check.

Each workload stands in for a gradient shape the S2 Reducer pages train on (arXiv
2110.02140, Section 4 and Table 1: embedding-layer gradients of LSTM/GNMT over 94% sparse,
and block-wise Top-K sparsified ResNet-50 / Transformer gradients).  No dataset or trained
model is used: positions and values are drawn from seeded numpy PCG64 generators.

Conventions:
  * values are float32; N(mu, s) uses s as the standard deviation, Laplace(0, b) b as the
    scale; a draw that is exactly zero is redrawn, so the non-zero count is exact;
  * worker k of workload c uses seed 1000*c + k; the hash seed of workload c is
    HASH_SEED_BASE + c;
  * every generator returns one worker's gradient as ascending uint32 indices and their
    float32 values (the dense gradient is zero elsewhere).
"""
from __future__ import annotations

import dataclasses

import numpy as np

HASH_SEED_BASE = 0x5332524544554345


@dataclasses.dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    W: int          # simulated data-parallel workers
    N: int          # gradient elements per worker
    d: int          # sketch rows
    log2_w: int     # log2 of sketch columns
    nnz_hint: int   # upper bound of non-zeros per worker (exact where the recipe fixes it)
    recipe: str

    @property
    def w(self) -> int:
        return 1 << self.log2_w

    @property
    def hash_seed(self) -> int:
        return HASH_SEED_BASE + self.cid


# The five workloads.  Sizes follow the pages' model shapes (Table 1) and sparsity levels.
WORKLOADS = [
    Workload(0, "tiny", 4, 1 << 20, 3, 14, 10486,
             "N=2^20; 1% positions uniform without replacement; values N(0,1e-3)"),
    Workload(1, "embedding", 8, 267744 * 512, 5, 20, 4096 * 512,
             "267,744x512 table; 4,096 distinct rows by finite Zipf(1.1); rows N(0,1e-2)"),
    Workload(2, "resnet50_blocktopk", 16, 25557032, 3, 19, 999 * 256,
             "blocks of 256 (last 40); keep top 1% blocks by l2 norm of N(0,1) draws"),
    Workload(3, "transformer_mixed", 8, 160_000_000, 5, 22, 4688 * 1024 + 6250 * 512,
             "96M embedding (rows of 1024, 5% rows by Zipf(1.05)) + 64M dense part, "
             "top 5% blocks of 512 by l2 norm; values N(0,1e-3)"),
    Workload(4, "large", 8, 1_000_000_000, 5, 23, 1_000_000,
             "N=1e9; 15,625 runs of 64 at uniform non-overlapping starts; Laplace(0,1e-3)"),
]


def workload(cid: int) -> Workload:
    return WORKLOADS[cid]


def rng_for(cid: int, k: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * cid + k))


# ----------------------------------------------------------------------------------------
# value draws


def _nonzero(draw, size: int) -> np.ndarray:
    """Draw `size` float32 values with `draw(m)`, redrawing exact zeros."""
    v = np.asarray(draw(size), dtype=np.float32)
    bad = v == 0
    while bad.any():
        v[bad] = np.asarray(draw(int(bad.sum())), dtype=np.float32)
        bad = v == 0
    return v


def normal(rng: np.random.Generator, size: int, std: float) -> np.ndarray:
    return _nonzero(lambda m: rng.standard_normal(m, dtype=np.float32) * np.float32(std), size)


def laplace(rng: np.random.Generator, size: int, scale: float) -> np.ndarray:
    return _nonzero(lambda m: rng.laplace(0.0, scale, m), size)


# ----------------------------------------------------------------------------------------
# structure draws


def finite_zipf_distinct(rng: np.random.Generator, support: int, s: float, count: int) -> np.ndarray:
    """Draw ranks r in 1..support with p(r) ∝ r^-s (with replacement) until `count` distinct
    values were seen; rank r maps to row r-1.  Returns the distinct rows, ascending."""
    if count > support:
        raise ValueError("count exceeds support")
    p = np.arange(1, support + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(p)
    cdf /= cdf[-1]
    seen: dict[int, None] = {}
    batch = max(1024, 2 * count)
    while len(seen) < count:
        u = rng.random(batch)
        rows = np.searchsorted(cdf, u, side="right")
        rows = np.minimum(rows, support - 1)
        for r in rows.tolist():
            if r not in seen:
                seen[r] = None
                if len(seen) == count:
                    break
    return np.sort(np.fromiter(seen.keys(), dtype=np.int64, count=count))


def topk_blocks(rng: np.random.Generator, n: int, block: int, keep: int, std: float,
                base: int = 0):
    """Dense N(0,std) draws over n elements in blocks of `block` (last block may be short);
    keep the `keep` blocks of largest l2 norm (ties to the lower block id).  Returns
    (indices, values) of the kept elements, ascending, offset by `base`."""
    dense = normal(rng, n, std)
    nblocks = -(-n // block)
    sq = dense.astype(np.float64) ** 2
    pad = nblocks * block - n
    if pad:
        sq = np.concatenate([sq, np.zeros(pad)])
    norms = sq.reshape(nblocks, block).sum(axis=1)
    order = np.argsort(-norms, kind="stable")[:keep]
    blocks = np.sort(order)
    starts = blocks * block
    lens = np.minimum(block, n - starts)
    idx = np.concatenate([np.arange(s, s + l) for s, l in zip(starts, lens)]) if keep else \
        np.empty(0, dtype=np.int64)
    return (idx + base).astype(np.uint32), dense[idx]


def rows_block(rows: np.ndarray, width: int, base: int = 0) -> np.ndarray:
    """Element indices of whole rows of a row-major table."""
    return (base + (rows[:, None] * width + np.arange(width)[None, :]).reshape(-1)).astype(np.uint32)


def runs(rng: np.random.Generator, n: int, run: int, count: int) -> np.ndarray:
    """`count` non-overlapping runs of `run` elements; starts uniform on [0, n-run], draws
    that overlap an accepted run are rejected.  Returns element indices, ascending."""
    starts: list[int] = []
    taken = np.zeros(0, dtype=np.int64)
    while len(starts) < count:
        cand = rng.integers(0, n - run + 1, size=2 * (count - len(starts)) + 16)
        for s in cand.tolist():
            if len(starts) == count:
                break
            # reject if [s, s+run) overlaps an accepted run
            pos = np.searchsorted(taken, s)
            ok = True
            if pos > 0 and taken[pos - 1] + run > s:
                ok = False
            if pos < taken.size and s + run > taken[pos]:
                ok = False
            if ok:
                starts.append(s)
                taken = np.insert(taken, pos, s)
    st = np.sort(np.array(starts, dtype=np.int64))
    return (st[:, None] + np.arange(run)[None, :]).reshape(-1).astype(np.uint32)


# ----------------------------------------------------------------------------------------
# the five workloads


def worker_sparse(cid: int, k: int):
    """Worker k's gradient of workload `cid` as (ascending uint32 indices, float32 values)."""
    wl = WORKLOADS[cid]
    rng = rng_for(cid, k)
    if cid == 0:
        K = round(0.01 * wl.N)
        idx = np.sort(rng.choice(wl.N, size=K, replace=False)).astype(np.uint32)
        return idx, normal(rng, K, 1e-3)
    if cid == 1:
        rows = finite_zipf_distinct(rng, 267744, 1.1, 4096)
        idx = rows_block(rows, 512)
        return idx, normal(rng, idx.size, 1e-2)
    if cid == 2:
        nblocks = -(-wl.N // 256)
        keep = -(-nblocks // 100)  # ceil(1% of blocks)
        return topk_blocks(rng, wl.N, 256, keep, 1.0)
    if cid == 3:
        emb_rows = 93_750
        rows = finite_zipf_distinct(rng, emb_rows, 1.05, -(-emb_rows * 5 // 100))
        i1 = rows_block(rows, 1024)
        v1 = normal(rng, i1.size, 1e-3)
        i2, v2 = topk_blocks(rng, 64_000_000, 512, 6250, 1e-3, base=96_000_000)
        return np.concatenate([i1, i2]), np.concatenate([v1, v2])
    if cid == 4:
        idx = runs(rng, wl.N, 64, 15_625)
        return idx, laplace(rng, idx.size, 1e-3)
    raise ValueError(cid)


def worker_dense(cid: int, k: int) -> np.ndarray:
    """Worker k's dense gradient before block-wise Top-K, for the block-sparsified workload
    (cid 2: N(0,1) over all N elements, the same draws worker_sparse(2, k) keeps 1% of)."""
    if cid != 2:
        raise ValueError("dense pre-sparsification gradients exist for the ResNet-50 workload")
    return normal(rng_for(cid, k), WORKLOADS[cid].N, 1.0)


# ----------------------------------------------------------------------------------------
# small generators for edge cases and parity at oracle-friendly sizes


def uniform_sparse(n: int, density: float, seed: int, std: float = 1e-3, integer: bool = False):
    """Uniform random positions at the given density.  With integer=True values are
    non-zero integers in [-64, 64] (every fp32 sum of them below 2^24 is exact)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    K = int(round(density * n))
    K = min(max(K, 0), n)
    idx = np.sort(rng.choice(n, size=K, replace=False)).astype(np.uint32) if K else \
        np.empty(0, dtype=np.uint32)
    if integer:
        v = rng.integers(1, 65, size=K) * rng.choice([-1, 1], size=K)
        return idx, v.astype(np.float32)
    return idx, normal(rng, K, std)


def blocks_sparse(n: int, block: int, keep_frac: float, seed: int, std: float = 1e-3):
    """Block-wise Top-K shaped input at arbitrary size (ragged last block allowed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    nblocks = -(-n // block)
    keep = max(1, int(round(keep_frac * nblocks)))
    return topk_blocks(rng, n, block, keep, std)


def dense_from_sparse(n: int, idx: np.ndarray, val: np.ndarray, ld: int | None = None,
                      fill_pad: float = 0.0) -> np.ndarray:
    """Dense float32 row of length ld (>= n); entries [n, ld) hold `fill_pad`."""
    ld = n if ld is None else ld
    g = np.zeros(ld, dtype=np.float32)
    if ld > n:
        g[n:] = fill_pad
    g[idx.astype(np.int64)] = val
    return g


def random_sketch(shape, seed: int, integer: bool = False, scale: float = 1.0) -> np.ndarray:
    """A float32 table of the given shape, for testing aggregation and decompression on
    their own (inputs that do not come from a compression step)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if integer:
        return rng.integers(-512, 513, size=shape).astype(np.float32)
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(scale))


def random_bitmap(n: int, density: float, seed: int) -> np.ndarray:
    """A bitmap of ceil(n/64) uint64 words with bits >= n clear."""
    rng = np.random.Generator(np.random.PCG64(seed))
    bits = rng.random(n) < density
    nwords = (n + 63) // 64
    padded = np.zeros(nwords * 64, dtype=np.uint8)
    padded[:n] = bits
    return np.packbits(padded, bitorder="little").view(np.uint64).copy()
