"""The three calls inside a captured HIP graph (through torch.cuda.graph): none of them
allocates, synchronises or depends on host state, so a replayed graph must give the same
outputs as the eager calls.  Integer-valued gradients make every fp32 sum exact, so the
comparison is bit-exact even though the sketch additions happen in no fixed order.  Each
replay is checked, with eager work in between."""
import numpy as np
import pytest
import torch

import count_sketch_aggregation_amd as s2r
import workloads as WL

pytestmark = pytest.mark.gpu

gp = pytest.importorskip("gpu_path")


def test_graph_replays_match_eager():
    W, n, d, L = 3, 300_000, 5, 20
    dev = gp.DEV
    p, _ = gp.params_pair(31337, d, L)
    grads = np.stack([WL.dense_from_sparse(n, *WL.uniform_sparse(n, 0.03, 50 + k, integer=True))
                      for k in range(W)])
    g = torch.from_numpy(grads).to(dev)
    buf = s2r.alloc_encode_buffers(p, W, n, n, dev)
    words = s2r.s2r_bitmap_words(n)
    bm = torch.empty(words, dtype=torch.int64, device=dev)
    sk = torch.empty((d, 1 << L), dtype=torch.float32, device=dev)
    out = torch.empty(n, dtype=torch.float32, device=dev)
    dws = s2r.alloc_decode_workspace(p, n, n, dev)

    def step(stream):
        s2r.s2r_encode(p, W, g, n, n, buf["bitmaps"], buf["sketches"], buf["idx"], buf["val"], n,
                       buf["nnz"], buf["workspace"], stream=stream)
        s2r.s2r_reduce(p, W, n, buf["bitmaps"], buf["sketches"], bm, sk, stream=stream)
        s2r.s2r_decode(p, n, bm, sk, out, max_set=n, workspace=dws, stream=stream)

    def snapshot():
        torch.cuda.synchronize()
        return [t.clone() for t in (buf["bitmaps"], buf["sketches"], buf["idx"], buf["val"],
                                    buf["nnz"], bm, sk, out)]

    gp.say("graph: eager reference")
    for t in (buf["bitmaps"], buf["sketches"], buf["idx"], buf["val"], buf["nnz"], bm, sk, out):
        t.fill_(7)  # list entries beyond nnz are never written: same filler on both sides
    step(torch.cuda.current_stream())
    want = snapshot()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the launch path on the capture stream
        step(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(torch.cuda.current_stream())
    for rep in range(3):
        gp.say(f"graph: replay {rep}")
        for t in (buf["bitmaps"], buf["sketches"], buf["idx"], buf["val"], buf["nnz"], bm, sk, out):
            t.fill_(7)  # stale contents must not matter
        torch.cuda.synchronize()
        graph.replay()
        got = snapshot()
        for a, b in zip(got, want):
            assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                               b.view(torch.int32) if b.dtype == torch.float32 else b)
        step(torch.cuda.current_stream())  # eager work between replays
        torch.cuda.synchronize()
