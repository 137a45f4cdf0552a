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
