"""The usage example of README.md runs as written (on the GPU)."""
import os
import re

import pytest
import torch

pytestmark = pytest.mark.gpu


def test_readme_usage_example_runs():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    text = open(os.path.join(root, "README.md")).read()
    blocks = re.findall(r"```python\n(.*?)```", text, re.S)
    assert len(blocks) == 1
    scope = {}
    exec(compile(blocks[0], "README.md", "exec"), scope)
    torch.cuda.synchronize()
    B, L, H, P, N = (scope[k] for k in ("B", "L", "H", "P", "N"))
    assert scope["y"].shape == (B, L, H, P) and scope["ssm_state"].shape == (B, H, P, N)
    assert scope["y_t"].shape == (B, H, P)
    for k in ("y", "ssm_state", "y_t", "conv_next"):
        assert torch.isfinite(scope[k].float()).all(), k
