"""The README's Python example runs as written and gives the oracle's result
(quantise on the GPU, GEMM, grouped GEMM), so the documented use stays true."""
import re
import os

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_example(gpu):
    text = open(os.path.join(ROOT, "README.md")).read()
    code = re.search(r"```python\n(.*?)```", text, re.S).group(1)
    torch.manual_seed(0)
    env = {}
    exec(compile(code, "README.md", "exec"), env)
    torch.cuda.synchronize()
    A, a_s, B, b_s, C, Cg = (env[k] for k in ("A", "a_s", "B", "b_s", "C", "Cg"))
    qa, sa = A.view(torch.uint8).cpu().numpy(), a_s.cpu().numpy()
    qb, sb = B.view(torch.uint8).cpu().numpy(), b_s.cpu().numpy()
    ref = oracle.block_gemm(qa, sa, qb, sb)
    got = C.float().cpu().double().numpy()
    assert np.all(np.abs(got - ref) <= oracle.tolerance(ref, "bf16"))
    # the grouped call with the same expert weight twice equals the plain GEMM
    assert torch.equal(Cg.view(torch.int16), C.view(torch.int16)) or \
        np.all(np.abs(Cg.float().cpu().double().numpy() - ref) <= oracle.tolerance(ref, "bf16"))
