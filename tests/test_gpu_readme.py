"""The README's usage snippet runs as written and gives finite outputs (its
pools are zero apart from the tokens the step writes, so every row is an
average of those rows' V with weights from q.K)."""
import os
import re

import pytest
import torch

from tests.gpu_util import announce, require_gpu

pytestmark = pytest.mark.gpu

README = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")


def test_readme_decode_snippet_runs():
    require_gpu()
    text = open(README).read()
    blocks = re.findall(r"```python\n(.*?)```", text, re.S)
    assert blocks, "no python block in README.md"
    env = {}
    exec(compile(blocks[0], "README.md", "exec"), env)
    torch.cuda.synchronize()
    out = env["out"]
    assert torch.isfinite(out).all()
    # only the current token is stored beyond zeros: with K = 0 elsewhere every
    # key scores 0 except the new one, so each row mixes zeros and v_new
    announce(f"README snippet: out max |x| {out.abs().max().item():.3e}")
