"""Calls from several host threads, each on its own stream with its own buffers, give the
same results as one thread alone (the library keeps no global state)."""
import threading

import numpy as np
import pytest
import torch

import count_sketch_aggregation_amd as s2r
import workloads as WL

pytestmark = pytest.mark.gpu

gp = pytest.importorskip("gpu_path")


def _pipeline(p, g, W, n, d, L, stream, reps):
    dev = gp.DEV
    with torch.cuda.stream(stream):
        buf = s2r.alloc_encode_buffers(p, W, n, n, dev)
        bm = torch.empty(s2r.s2r_bitmap_words(n), dtype=torch.int64, device=dev)
        sk = torch.empty((d, 1 << L), dtype=torch.float32, device=dev)
        out = torch.empty(n, dtype=torch.float32, device=dev)
        dws = s2r.alloc_decode_workspace(p, n, n, dev)
    for _ in range(reps):
        s2r.s2r_encode(p, W, g, n, n, buf["bitmaps"], buf["sketches"], buf["idx"], buf["val"], n,
                       buf["nnz"], buf["workspace"], stream=stream)
        s2r.s2r_reduce(p, W, n, buf["bitmaps"], buf["sketches"], bm, sk, stream=stream)
        s2r.s2r_decode(p, n, bm, sk, out, max_set=n, workspace=dws, stream=stream)
    stream.synchronize()
    return bm.cpu(), sk.cpu(), out.cpu()


def test_threads_on_separate_streams():
    W, n, d, L = 3, 200_000, 5, 20
    p, _ = gp.params_pair(777, d, L)
    inputs = []
    for t in range(4):
        grads = np.stack([WL.dense_from_sparse(n, *WL.uniform_sparse(n, 0.05, 100 * t + k,
                                                                      integer=True))
                          for k in range(W)])
        inputs.append(torch.from_numpy(grads).to(gp.DEV))
    gp.say("concurrency: one thread")
    want = [_pipeline(p, g, W, n, d, L, torch.cuda.Stream(), 1) for g in inputs]
    gp.say("concurrency: four threads")
    got = [None] * 4
    errors = []

    def run(t):
        try:
            got[t] = _pipeline(p, inputs[t], W, n, d, L, torch.cuda.Stream(), 3)
        except Exception as e:  # surfaced below
            errors.append(e)

    threads = [threading.Thread(target=run, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    for t in range(4):
        for a, b in zip(got[t], want[t]):
            assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                               b.view(torch.int32) if b.dtype == torch.float32 else b), t
