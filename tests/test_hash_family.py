"""The partitioned bucket hash versus fully independent rows (CPU, oracle only).

S2 Reducer (Section 3.1; Appendix A.1) needs each row's bucket map to be uniformly random
with Pr[two items share a bucket] = 1/m, and random signs; it does not say how the rows
relate to each other.  The library's default groups all rows of an item into one
partition of 2^K buckets per row (h_j(i) = P(i) 2^K + Q_j(i)), which keeps every row a
uniform 2-independent map.  These checks show the median estimate behaves the same as with
independent rows (K = L) on the same gradients: same per-row collision rate, and an error
distribution that matches within Monte-Carlo noise.
"""
import numpy as np

import oracle as O
import workloads as WL


def _errors(K, seeds, g_sparse, n, d, L):
    idx, val = g_sparse
    g = WL.dense_from_sparse(n, idx, val).astype(np.float64)
    errs = []
    for s in seeds:
        p = O.params_from_seed(s, d, L, K)
        e = O.encode_sparse(p, idx, val, n)
        oi, ov, _ = O.decode(p, n, e["bitmap"], e["S"], e["A"])
        errs.append(ov - g[oi])
    return np.concatenate(errs)


def test_partitioned_rows_match_independent_rows():
    n, d, L = 1 << 16, 5, 10
    g_sparse = WL.blocks_sparse(n, 64, 0.05, seed=11, std=1.0)   # 3,264 non-zeros in blocks
    seeds = range(100, 140)
    e_ind = _errors(L, seeds, g_sparse, n, d, L)
    e_part = _errors(4, seeds, g_sparse, n, d, L)                  # 64 partitions of 16 buckets
    m_ind, m_part = np.abs(e_ind).mean(), np.abs(e_part).mean()
    assert 0.9 < m_part / m_ind < 1.1, (m_ind, m_part)
    for q in (0.5, 0.9, 0.99):
        a, b = np.quantile(np.abs(e_ind), q), np.quantile(np.abs(e_part), q)
        assert 0.85 < b / a < 1.15, (q, a, b)
    # both estimators are centred (Theorem 1 concerns the per-row estimate; the median of a
    # symmetric noise is centred as well)
    for e in (e_ind, e_part):
        assert abs(e.mean()) < 5 * e.std() / np.sqrt(e.size)


def test_partitioned_pair_collision_rates():
    """Per row: Pr[same bucket] = 1/w for both families; across rows the partitioned family
    makes a second-row collision 2^(L-K) times likelier given a first (the grouping), and
    independent rows give 1/w again."""
    rng = np.random.Generator(np.random.PCG64(5))
    keys = np.unique(rng.integers(0, 2**32, size=1 << 17, dtype=np.uint64)).astype(np.uint32)
    L, K = 12, 6
    x = rng.integers(0, keys.size, size=1 << 21)
    y = rng.integers(0, keys.size, size=1 << 21)
    ok = x != y
    for fam_K, cond_rate in ((L, 1 / (1 << L)), (K, 1 / (1 << K))):
        p = O.params_from_seed(77, 2, L, fam_K)
        b, _ = O.hash_keys(p, keys)
        c0 = b[0][x[ok]] == b[0][y[ok]]
        c1 = b[1][x[ok]] == b[1][y[ok]]
        w = 1 << L
        se = np.sqrt(c0.size * (1 / w)) / c0.size
        assert abs(c0.mean() - 1 / w) < 6 * se
        assert abs(c1.mean() - 1 / w) < 6 * se
        # P(collide in row 1 | collide in row 0)
        cond = c1[c0].mean()
        assert abs(cond - cond_rate) < 6 * np.sqrt(cond_rate / max(c0.sum(), 1)) + 1e-3, \
            (fam_K, cond, cond_rate)


def test_partitioned_rows_at_the_workloads_partition_geometry():
    """The benchmark's partition shape: d = 5 rows, 2^11 buckets per partition and row (the
    default K for d = 5), about 10 items per bucket as in the embedding and Transformer
    workloads (U / w = 10.1 and 10.4).  Here w = 2^13 (4 partitions) and U = 81,920 items in
    runs of 64, so every partition holds about 20K items as the embedding workload's do; the
    median's error matches that of independent rows within Monte-Carlo noise."""
    n, d, L, K = 1 << 20, 5, 13, 11
    g_sparse = WL.blocks_sparse(n, 64, 0.078125, seed=21, std=1.0)
    assert abs(g_sparse[0].size / (1 << L) - 10.0) < 0.1
    seeds = range(300, 324)
    e_ind = _errors(L, seeds, g_sparse, n, d, L)
    e_part = _errors(K, seeds, g_sparse, n, d, L)
    m_ind, m_part = np.abs(e_ind).mean(), np.abs(e_part).mean()
    assert 0.95 < m_part / m_ind < 1.05, (m_ind, m_part)
    r_ind = np.sqrt((e_ind ** 2).mean())
    r_part = np.sqrt((e_part ** 2).mean())
    assert 0.95 < r_part / r_ind < 1.05, (r_ind, r_part)
    for q in (0.5, 0.9, 0.99):
        a, b = np.quantile(np.abs(e_ind), q), np.quantile(np.abs(e_part), q)
        assert 0.9 < b / a < 1.1, (q, a, b)
