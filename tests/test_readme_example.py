"""The usage example in README.md runs as written (every public entry it shows:
compress/decompress, batched decode, a shared codebook, the dominant-range codec,
K/V slots and the layer pipeline), and its claims hold."""
import os
import re
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_readme_example_runs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("readme example", file=sys.stderr, flush=True)
    text = open(os.path.join(ROOT, "README.md")).read()
    code = re.search(r"```python\n(.*?)```", text, re.S).group(1)
    ns = {}
    exec(compile(code, "README.md", "exec"), ns)
    torch.cuda.synchronize()
    x, c, y = ns["x"], ns["c"], ns["y"]
    assert torch.equal(y.view(torch.int16), x.view(torch.int16))
    for t in ns["ys"]:
        assert torch.equal(t.view(torch.int16), x.view(torch.int16))
    assert 0.6 < c.nbytes() / (x.numel() * 2) < 0.75
    assert torch.equal(ns["zx"].decompress(ns["c2"]).view(torch.int16), (2 * x).view(torch.int16))
    assert ns["status"].tolist() == [0, 0, 0, 0]
    assert torch.equal(ns["kv"].view(torch.int16), ns["blocks"].view(torch.int16))
