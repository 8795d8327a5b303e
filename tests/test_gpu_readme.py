"""The Python examples of README.md run as written (GPU), and their outputs are finite."""
import os
import re

import pytest
import torch

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_python_example_runs():
    src = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```python\n(.*?)```", src, re.S)
    assert blocks, "README.md has no python example"
    env = {}
    for b in blocks:
        exec(compile(b, "README.md", "exec"), env)
    torch.cuda.synchronize()
    for name in ("o", "lse", "dq", "dk", "dv", "o16", "od", "lsed"):
        t = env[name]
        assert torch.isfinite(t.float()).all(), name
