"""GPU parity of the lossless comparator s2r_gather_sum (the exact sum of the workers'
(index, value) lists, S2 Reducer Section 1 and Section 2.2 with Fig. 1(b)).

Checks, on seeded lists:
  * against the fp64 oracle: |gpu - exact| <= 1e-5 * mass + 1e-12 at every element, where
    mass is the sum of the magnitudes of the element's contributions (an fp32 sum of c terms
    in any order errs by at most (c - 1) 2^-24 mass), and +0.0 bit-exact where no worker
    lists the element;
  * bit-exact against a numpy fp32 replay in worker order (out = 0; out[idx_k] += val_k for
    k = 0, 1, ...), the order the call promises;
  * bit-exact against the oracle on integer-valued data, where every fp32 sum is exact.
"""
import numpy as np
import pytest
import torch

import count_sketch_aggregation_amd as s2r
import oracle
import workloads as WL

pytestmark = pytest.mark.gpu

gp = pytest.importorskip("gpu_path")


def _device_lists(lists, cap):
    W = len(lists)
    idx = torch.full((W, max(cap, 1)), -1, dtype=torch.int32)
    val = torch.full((W, max(cap, 1)), float("nan"), dtype=torch.float32)
    nnz = torch.zeros(W, dtype=torch.int64)
    for k, (i, v) in enumerate(lists):
        m = min(i.size, cap)
        idx[k, :m] = torch.from_numpy(i[:m].view(np.int32))
        val[k, :m] = torch.from_numpy(v[:m])
        nnz[k] = i.size  # may exceed cap: only the first cap entries are listed
    return idx.to(gp.DEV), val.to(gp.DEV), nnz.to(gp.DEV)


def run_gather(lists, n, cap=None):
    cap = max([x[0].size for x in lists] + [0]) if cap is None else cap
    idx, val, nnz = _device_lists(lists, cap)
    out = torch.full((max(n, 1),), float("nan"), dtype=torch.float32, device=gp.DEV)
    s2r.s2r_gather_sum(len(lists), idx, val, cap, nnz, n, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()[:n]


def replay_fp32(lists, n, cap=None):
    out = np.zeros(n, dtype=np.float32)
    for i, v in lists:
        m = i.size if cap is None else min(i.size, cap)
        keep = i[:m] < n
        out[i[:m][keep].astype(np.int64)] += v[:m][keep]
    return out


def check(lists, n, cap=None, integer=False):
    got = run_gather(lists, n, cap)
    cut = [(i[:cap], v[:cap]) for i, v in lists] if cap is not None else lists
    want, mass = oracle.gather_sum(cut, n)
    listed = np.zeros(n, dtype=bool)
    for i, _ in cut:
        listed[i[i < n].astype(np.int64)] = True
    assert np.all(got[~listed].view(np.uint32) == 0), "unlisted elements must be +0.0"
    g = got.astype(np.float64)
    if integer:
        assert np.array_equal(g, want)
    bad = ~(np.abs(g - want) <= 1e-5 * mass + 1e-12)
    assert not bad.any(), f"{int(bad.sum())} elements off the exact sum"
    assert np.array_equal(got.view(np.uint32), replay_fp32(lists, n, cap).view(np.uint32))


CASES = [  # (W, n, density, seed, integer)
    (1, 1, 1.0, 1, False), (2, 1000, 0.3, 2, False), (4, 1 << 20, 0.01, 3, False),
    (8, 100_003, 0.2, 4, True), (16, 65_537, 0.05, 5, False), (3, 5, 1.0, 6, True),
]


@pytest.mark.parametrize("W,n,density,seed,integer", CASES)
def test_gather_sum(W, n, density, seed, integer):
    gp.say(f"gather W={W} n={n} density={density} integer={integer}")
    lists = [WL.uniform_sparse(n, density, 1000 * seed + k, integer=integer) for k in range(W)]
    check(lists, n, integer=integer)


def test_gather_sum_edges():
    gp.say("gather edges: empty worker, capacity cut, indices beyond n, n = 0")
    n = 50_000
    lists = [WL.uniform_sparse(n, 0.1, 70 + k) for k in range(4)]
    lists[1] = (np.zeros(0, np.uint32), np.zeros(0, np.float32))  # a worker with nothing
    check(lists, n)
    check(lists, n, cap=777)  # nnz beyond the list capacity: the first cap entries count
    check(lists, n, cap=0)
    beyond = [(np.append(i, np.uint32(n + 3 + k)), np.append(v, np.float32(9.0)))
              for k, (i, v) in enumerate(lists)]
    check(beyond, n)
    assert run_gather(lists, 0).size == 0


def test_gather_sum_from_encode_lists():
    """The comparator on the lists s2r_encode itself wrote (device to device)."""
    gp.say("gather from encode lists")
    W, n, d, L = 4, 300_001, 5, 16
    p, _ = gp.params_pair(31, d, L)
    lists = [WL.blocks_sparse(n, 256, 0.05, 40 + k) for k in range(W)]
    ld = (n + 3) // 4 * 4
    grad = torch.from_numpy(np.stack([WL.dense_from_sparse(n, i, v, ld=ld) for i, v in lists]))
    grad = grad.to(gp.DEV)
    cap = max(x[0].size for x in lists)
    buf = s2r.alloc_encode_buffers(p, W, n, cap, gp.DEV)
    s2r.s2r_encode(p, W, grad, n, ld, buf["bitmaps"], buf["sketches"], buf["idx"], buf["val"], cap,
                   buf["nnz"], buf["workspace"])
    out = torch.full((n,), float("nan"), dtype=torch.float32, device=gp.DEV)
    s2r.s2r_gather_sum(W, buf["idx"], buf["val"], cap, buf["nnz"], n, out)
    torch.cuda.synchronize()
    want, mass = oracle.gather_sum(lists, n)
    got = out.cpu().numpy()
    assert np.all(np.abs(got.astype(np.float64) - want) <= 1e-5 * mass + 1e-12)
    assert np.array_equal(got.view(np.uint32), replay_fp32(lists, n).view(np.uint32))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cid", [1, 2, 3, 4])
def test_fullsize_gather_sum(cid):
    """Each workload's seeded lists at full size, in the shape the benchmark passes them
    (list capacity = the largest worker's nnz)."""
    wl = WL.workload(cid)
    gp.say(f"fullsize gather {wl.name}: W={wl.W} N={wl.N}")
    lists = [WL.worker_sparse(cid, k) for k in range(wl.W)]
    got = run_gather(lists, wl.N)
    gp.say("  gpu done; checking")
    want, mass = oracle.gather_sum(lists, wl.N)
    sup = np.unique(np.concatenate([i for i, _ in lists])).astype(np.int64)
    listed = np.zeros(wl.N, dtype=bool)
    listed[sup] = True
    assert np.all(got[~listed].view(np.uint32) == 0)
    del listed
    g = got[sup].astype(np.float64)
    assert np.all(np.abs(g - want[sup]) <= 1e-5 * mass[sup] + 1e-12)
    del want, mass
    assert np.array_equal(got[sup].view(np.uint32), replay_fp32(lists, wl.N)[sup].view(np.uint32))
