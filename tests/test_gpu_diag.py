"""The measurement helper of include/s2r_diag.h on the GPU: it reads every byte it is given
(the sink receives the sum when that sum is exactly 1)."""
import pytest
import torch

import count_sketch_aggregation_amd as s2r

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [4, 1024, (1 << 22) + 4])
def test_stream_read_touches_everything(n):
    buf = torch.zeros(n, dtype=torch.float32, device="cuda")
    buf[-1] = 1.0   # the last float4 must be read for the sum to reach 1
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    s2r.s2r_diag_stream_read(buf, n * 4, sink)
    torch.cuda.synchronize()
    assert float(sink) == 1.0


def _trace(n_events):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_events)]
    stream = torch.cuda.current_stream()
    for e in evs:
        e.record(stream)
    t = s2r.s2r_trace()
    t.capacity = n_events
    t.count = 0
    for i, e in enumerate(evs):
        t.events[i] = e.cuda_event
    return t, evs


def test_kernel_trace_names_and_times():
    """With a trace attached, an encode + reduce + decode records one event before each
    kernel and one after each call; results equal an untraced run; nothing is recorded once
    the trace is detached or full."""
    import numpy as np

    import workloads as WL
    W, n, d, L = 3, 300_000, 5, 20   # a 20 MiB table: the partitioned decode
    p = s2r.s2r_params_from_seed(5, d, L)
    grads = np.stack([WL.dense_from_sparse(n, *WL.uniform_sparse(n, 0.02, 9 + k)) for k in range(W)])
    g = torch.from_numpy(grads).cuda()
    buf = s2r.alloc_encode_buffers(p, W, n, n, "cuda")
    bm = torch.empty(s2r.s2r_bitmap_words(n), dtype=torch.int64, device="cuda")
    sk = torch.empty((d, 1 << L), dtype=torch.float32, device="cuda")
    dws = s2r.alloc_decode_workspace(p, n, n, "cuda")

    def run():
        out = torch.empty(n, dtype=torch.float32, device="cuda")
        s2r.s2r_encode(p, W, g, n, n, buf["bitmaps"], buf["sketches"], buf["idx"], buf["val"], n,
                       buf["nnz"], buf["workspace"])
        s2r.s2r_reduce(p, W, n, buf["bitmaps"], buf["sketches"], bm, sk)
        s2r.s2r_decode(p, n, bm, sk, out, max_set=n, workspace=dws)
        return out

    plain = run()
    t, evs = _trace(s2r.TRACE_MAX)
    s2r.s2r_diag_trace_attach(t)
    try:
        traced = run()
    finally:
        s2r.s2r_diag_trace_attach(None)
    torch.cuda.synchronize()
    names = [t.names[i].decode() for i in range(t.count)]
    assert names.count("end") == 3 and names[-1] == "end"
    for k in ("k_stream", "k_scan", "k_bin", "k_accumulate", "k_reduce", "k_dcount", "k_dbin",
              "k_dmedian", "k_dwrite"):
        assert k in names, (k, names)
    assert names.index("k_stream") < names.index("k_reduce") < names.index("k_dwrite")
    times = [evs[i].elapsed_time(evs[i + 1]) for i in range(t.count - 1)]
    assert all(x >= 0 for x in times)
    assert torch.equal(plain.view(torch.int32), traced.view(torch.int32))
    # detached: nothing more is recorded
    before = t.count
    run()
    torch.cuda.synchronize()
    assert t.count == before
    # a full trace records nothing more and the calls still run
    t2, _ = _trace(2)
    s2r.s2r_diag_trace_attach(t2)
    try:
        again = run()
    finally:
        s2r.s2r_diag_trace_attach(None)
    torch.cuda.synchronize()
    assert t2.count == 2 and torch.equal(plain.view(torch.int32), again.view(torch.int32))


def test_trace_attach_rejects_bad_capacity():
    t = s2r.s2r_trace()
    t.capacity = s2r.TRACE_MAX + 1
    with pytest.raises(s2r.S2RError):
        s2r.s2r_diag_trace_attach(t)
    t.capacity, t.count = 4, 5
    with pytest.raises(s2r.S2RError):
        s2r.s2r_diag_trace_attach(t)


@pytest.mark.parametrize("n", [4, 1024, (1 << 22) + 4])
def test_stream_write_fills_everything(n):
    buf = torch.full((n,), -1.0, dtype=torch.float32, device="cuda")
    s2r.s2r_diag_stream_write(buf, n * 4, 2.5)
    torch.cuda.synchronize()
    assert bool((buf == 2.5).all())
