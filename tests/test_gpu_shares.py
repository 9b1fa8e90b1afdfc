"""GPU: how a batch decode splits segments among workgroups.

A per-tensor batch is split into contiguous workgroup ranges, one range per tensor,
each workgroup taking an equal run of its tensor's segments.  Whatever the split,
every segment must be decoded exactly once: each case decodes a batch under a
different cap on the resident workgroups (one segment per wavefront, several per
wavefront, one workgroup per tensor) and compares every output with its input bit
for bit (lossless: DFloat11 article, 实验结果).
"""
import sys

import numpy as np
import pytest
import torch

import lossless_float_compression_amd as zx
from lossless_float_compression_amd import zx as zxm

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def batch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g = torch.Generator(device="cuda")
    g.manual_seed(4242)
    shapes = [(4096, 4096), (2048, 4096), (1000, 999)]
    xs = [(torch.randn(s, generator=g, device="cuda") * 0.02).to(torch.bfloat16) for s in shapes]
    cs = [zx.compress(x) for x in xs]
    torch.cuda.synchronize()
    return xs, cs


# 0: every resident slot (about one segment per wavefront); 1 and 3: one workgroup
# per tensor; 100, 300, 340: several segments per wavefront
@pytest.mark.parametrize("max_wg", [0, 1, 3, 100, 300, 340])
def test_batch_split_decodes_every_segment_once(batch, max_wg):
    xs, cs = batch
    say(f"batch decode, max_workgroups={max_wg}, segments {[c.nsegs for c in cs]}")
    outs = [torch.full_like(x, float("nan")) for x in xs]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    zxm.zx_decode_block_batch([c.container() for c in cs], outs, err=err, max_workgroups=max_wg)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for x, y in zip(xs, outs):
        assert torch.equal(y.view(torch.int16), x.view(torch.int16))
