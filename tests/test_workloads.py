"""Structure of the seeded synthetic gradients (CPU only)."""
import numpy as np
import pytest

import workloads as WL


def _check(idx, val, n):
    assert idx.dtype == np.uint32 and val.dtype == np.float32
    assert idx.size == val.size
    assert np.all(np.diff(idx.astype(np.int64)) > 0)
    assert idx.size == 0 or int(idx.max()) < n
    assert not np.any(val == 0)


@pytest.mark.parametrize("cid", [0, 1, 2, 4])
def test_workload_worker0(cid):
    wl = WL.workload(cid)
    idx, val = WL.worker_sparse(cid, 0)
    _check(idx, val, wl.N)
    assert idx.size == wl.nnz_hint
    # deterministic
    idx2, val2 = WL.worker_sparse(cid, 0)
    assert np.array_equal(idx, idx2) and np.array_equal(val.view(np.uint32), val2.view(np.uint32))


def test_embedding_rows_are_whole():
    idx, _ = WL.worker_sparse(1, 1)
    rows = idx.astype(np.int64) // 512
    u, c = np.unique(rows, return_counts=True)
    assert u.size == 4096 and np.all(c == 512)
    # Zipf(1.1) head: the first rows are almost always touched
    assert np.isin(np.arange(8), u).all()


def test_blocktopk_last_block_ragged():
    wl = WL.workload(2)
    assert wl.N % 256 == 40
    idx, val = WL.blocks_sparse(1000, 256, 1.0, 3)  # keep every block
    assert idx.size == 1000


def test_runs_non_overlapping():
    rng = np.random.Generator(np.random.PCG64(1))
    idx = WL.runs(rng, 10_000, 64, 100)
    assert idx.size == 6400 and np.unique(idx).size == 6400


def test_small_generators():
    idx, val = WL.uniform_sparse(1000, 0.1, 1, integer=True)
    _check(idx, val, 1000)
    assert np.all(np.abs(val) <= 64) and np.all(val == np.round(val))
    bm = WL.random_bitmap(130, 0.5, 2)
    assert bm.size == 3
    bits = np.unpackbits(bm.view(np.uint8), bitorder="little")
    assert not bits[130:].any()
    g = WL.dense_from_sparse(10, np.array([1, 3], np.uint32), np.array([2, -1], np.float32), ld=12,
                             fill_pad=7.0)
    assert g.tolist() == [0, 2, 0, -1, 0, 0, 0, 0, 0, 0, 7, 7]
