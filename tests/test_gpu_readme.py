"""The usage example of README.md runs as written, and its decoded gradient matches the
oracle at every element."""
import os
import re

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

gp = pytest.importorskip("gpu_path")


def test_readme_example():
    gp.say("readme example")
    src = open(os.path.join(os.path.dirname(__file__), "..", "README.md")).read()
    code = re.search(r"```python\n(.*?)```", src, re.S).group(1)
    env: dict = {}
    exec(compile(code, "README.md", "exec"), env)
    import torch
    torch.cuda.synchronize()
    s2r, p, n = env["s2r"], env["p"], env["n"]
    op = oracle.params_from_seed(1234, p.d, p.log2_w, p.log2_part)
    assert op.as_dict() == p.as_dict()
    grads = env["grads"].cpu().numpy()
    encs = [oracle.encode_dense(op, grads[k, :n]) for k in range(grads.shape[0])]
    obm, oS, oA = oracle.reduce(np.stack([e["bitmap"] for e in encs]),
                                np.stack([e["S"] for e in encs]), np.stack([e["A"] for e in encs]))
    want, tol = oracle.decode_dense(op, n, obm, oS, oA)
    got = env["g_hat"].cpu().numpy()
    gp.assert_decode_matches(got, want, tol, gp.bits_of(obm, n))
