"""Layer-ahead decode into reused scratch buffers (lossless_float_compression_amd.pipeline).

* CPU: the constructor's argument checks (layer shapes must match, depth >= 2,
  at most 16 tensors per layer).
* GPU: several small layers decoded one ahead of a consumer on another stream; the
  consumer copies each layer's weights out, and every copy must equal the input bit
  for bit (so no decode overwrote a buffer set the consumer was still reading, and
  no consumer read a set before its decode finished).  The consumer also runs a
  GEMM per tensor to keep its stream busy while the next layer decodes.
"""
import sys
from types import SimpleNamespace

import pytest
import torch

from lossless_float_compression_amd.pipeline import LayerPipeline


def _fake(shape, dtype=0):
    return SimpleNamespace(shape=shape, dtype=dtype)


def test_rejects_depth_below_two():
    with pytest.raises(ValueError):
        LayerPipeline([[_fake((4, 4))]], depth=1)


def test_rejects_mismatched_layers():
    with pytest.raises(ValueError):
        LayerPipeline([[_fake((4, 4))], [_fake((4, 8))]])
    with pytest.raises(ValueError):
        LayerPipeline([[_fake((4, 4))], [_fake((4, 4), dtype=1)]])


def test_rejects_more_than_sixteen_tensors():
    with pytest.raises(ValueError):
        LayerPipeline([[_fake((4, 4))] * 17])


def test_rejects_no_layers():
    with pytest.raises(ValueError):
        LayerPipeline([])


@pytest.mark.gpu
@pytest.mark.parametrize("depth", [2, 3])
def test_pipeline_round_trip(depth):
    import lossless_float_compression_amd as zx
    print(f"pipeline depth {depth}", file=sys.stderr, flush=True)
    shapes = [(700, 512), (256, 512), (512, 1400)]   # ragged: last blocks and segments partial
    n_layers = 5
    g = torch.Generator(device="cuda")
    inputs, layers = [], []
    for l in range(n_layers):
        g.manual_seed(9100 + l)
        ts = [(torch.randn(s, generator=g, device="cuda") * (0.02 * (l + 1))).to(torch.bfloat16) for s in shapes]
        inputs.append(ts)
        layers.append([zx.compress(t) for t in ts])
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    pipe = LayerPipeline(layers, depth=depth, err=err)
    consumer_stream = torch.cuda.Stream()
    copies = [[None] * len(shapes) for _ in range(n_layers)]
    x = [torch.randn((64, s[1]), device="cuda").to(torch.bfloat16) for s in shapes]
    sink = [torch.empty((64, s[0]), device="cuda", dtype=torch.bfloat16) for s in shapes]

    def consumer(l, w):
        for j, t in enumerate(w):
            torch.matmul(x[j], t.t(), out=sink[j])   # keep the stream busy with reads of t
            copies[l][j] = t.clone()

    with torch.cuda.stream(consumer_stream):
        pipe.run(consumer, consumer_stream)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for l in range(n_layers):
        for j in range(len(shapes)):
            assert torch.equal(copies[l][j].view(torch.int16), inputs[l][j].view(torch.int16)), (l, j)
