"""The usage example in README.md runs as written (GPU)."""
import os
import re

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_example_runs():
    text = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```python\n(.*?)```", text, re.S)
    assert len(blocks) == 1
    ns = {}
    exec(compile(blocks[0], "README.md", "exec"), ns)
    import torch
    torch.cuda.synchronize()
    pool, seqs, out = ns["pool"], ns["seqs"], ns["out"]
    assert all(pool.seq_len(int(s)) == 1 for s in seqs)
    assert pool.seq_len(ns["child"]) == 0
    # one visible key per sequence: every head's output is its kv head's V row
    v = ns["v"]
    expect = v.view(4, 8, 1, 128).expand(4, 8, 4, 128).reshape(4, 32 * 128)
    assert torch.equal(out, expect)
