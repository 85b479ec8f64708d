"""The README's usage example runs as written (forward, backward, autograd and
the DilatedAttention module on the GPU) and produces finite results."""
import os
import re

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch


def test_readme_example_runs(torch_cuda):
    torch = torch_cuda
    text = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```python\n(.*?)```", text, re.S)
    assert len(blocks) == 1
    scope = {}
    exec(compile(blocks[0], "README.md", "exec"), scope)
    torch.cuda.synchronize()
    for name in ("out", "lse", "dq", "dk", "dv", "y"):
        assert torch.isfinite(scope[name].float()).all(), name
    assert scope["q"].grad is not None and torch.isfinite(scope["q"].grad.float()).all()
    assert scope["y"].shape == (32, 8192, 512)
