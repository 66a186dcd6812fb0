"""The usage example in README.md runs as written and gives what it says."""

import os
import re

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_python_example_runs():
    text = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```python\n(.*?)```", text, flags=re.S)
    assert len(blocks) == 1
    ns = {}
    exec(compile(blocks[0], "README.md", "exec"), ns)
    torch.cuda.synchronize()
    w, q, w_hat, y = ns["w"], ns["q"], ns["w_hat"], ns["y"]
    assert w_hat.shape == w.shape and w_hat.dtype == torch.float32
    assert q.codes.shape == (4096, 2048) and q.scales.shape == (4096, 256)
    rel = float((w_hat - w.float()).norm() / w.float().norm())
    assert rel < 0.2, rel  # FP4: a few percent of the weight's norm
    assert y.shape == (8192, 4096) and y.dtype == torch.bfloat16 and bool(torch.isfinite(y).all())
