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


def _late_copy(c, busy_a, busy_b):
    """A copy of container c whose arrays are written on the current stream behind a
    queue of long matmuls, so they are finished only well after this call returns."""
    import dataclasses
    for _ in range(6):
        torch.mm(busy_a, busy_a, out=busy_b)
    kw = {f.name: getattr(c, f.name) for f in dataclasses.fields(c)}
    for f, v in list(kw.items()):
        if torch.is_tensor(v):
            kw[f] = v.clone()
    return type(c)(**kw)


@pytest.mark.gpu
def test_side_stream_decodes_wait_for_the_producer_stream():
    """decompress(stream=side), decompress_batch(stream=side), KVSlotPool.decode(stream=
    side) and LayerPipeline start their side-stream work only after what the current
    stream has queued: here the containers themselves are still being written there."""
    import lossless_float_compression_amd as zx
    from lossless_float_compression_amd.kvslots import KVSlotPool
    print("side stream waits for the producer", file=sys.stderr, flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    xs = [(torch.randn(s, generator=g, device="cuda") * 0.03).to(torch.bfloat16) for s in [(1000, 700), (300, 4096)]]
    cs = [zx.compress(x) for x in xs]
    a = torch.randn(4096, 4096, device="cuda")
    b = torch.empty_like(a)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    torch.cuda.synchronize()

    late = _late_copy(cs[0], a, b)
    y = zx.decompress(late, err=err, stream=side)
    late2 = [_late_copy(c, a, b) for c in cs]
    ys = zx.decompress_batch(late2, err=err, stream=side)
    late3 = [[_late_copy(c, a, b) for c in cs] for _ in range(2)]
    pipe = LayerPipeline(late3, err=err)
    got = []
    pipe.run(lambda l, w: got.append([t.clone() for t in w]))

    pool = KVSlotPool(4, zx.BF16, cap_words=8192)
    blocks = (torch.randn(2 * 65536, generator=g, device="cuda") * 0.5).to(torch.bfloat16)
    pool.append(blocks, torch.tensor([2, 0], dtype=torch.int32, device="cuda"))
    for _ in range(6):
        torch.mm(a, a, out=b)
    ids = torch.tensor([0, 2], dtype=torch.int32, device="cuda")   # written behind the matmuls
    rows = pool.decode(ids, err=err, stream=side)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(y.view(torch.int16), xs[0].view(torch.int16))
    for x, t in zip(xs, ys):
        assert torch.equal(t.view(torch.int16), x.view(torch.int16))
    for layer in got:
        for x, t in zip(xs, layer):
            assert torch.equal(t.view(torch.int16), x.view(torch.int16))
    assert torch.equal(rows.view(torch.int16), blocks.view(2, 65536)[[1, 0]].view(torch.int16))


@pytest.mark.gpu
def test_decompress_rejects_wrong_outputs():
    import lossless_float_compression_amd as zx
    x = (torch.randn(5000, device="cuda") * 0.1).to(torch.bfloat16)
    c = zx.compress(x)
    for bad in (torch.empty(5000, dtype=torch.uint8, device="cuda"),          # FP8-sized
                torch.empty(4999, dtype=torch.bfloat16, device="cuda"),        # short
                torch.empty((100, 100), dtype=torch.bfloat16, device="cuda").t()[:50],   # not contiguous
                torch.empty(5000, dtype=torch.bfloat16)):                      # host
        with pytest.raises(ValueError):
            zx.decompress(c, out=bad)
        with pytest.raises(ValueError):
            zx.decompress_batch([c], outs=[bad])


@pytest.mark.gpu
def test_side_stream_encodes_wait_for_the_producer_stream():
    """compress, compress_zf, build_shared_codebook and KVSlotPool.append given
    stream=side read their input only
    after what the current stream has queued: here the input itself is still being
    written there, behind long matmuls."""
    import lossless_float_compression_amd as zx
    from lossless_float_compression_amd.kvslots import KVSlotPool
    print("side-stream encodes wait for the producer", file=sys.stderr, flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(78)
    x = (torch.randn((2000, 1000), generator=g, device="cuda") * 0.03).to(torch.bfloat16)
    blocks = (torch.randn(3 * 65536, generator=g, device="cuda") * 0.5).to(torch.bfloat16)
    a = torch.randn(4096, 4096, device="cuda")
    b = torch.empty_like(a)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()

    for _ in range(6):
        torch.mm(a, a, out=b)
    x_late = x.clone()                       # written behind the matmuls
    c = zx.compress(x_late, stream=side)
    pool = KVSlotPool(4, zx.BF16, cap_words=8192)
    for _ in range(6):
        torch.mm(a, a, out=b)
    blocks_late = blocks.clone()
    ids = torch.tensor([3, 1, 0], dtype=torch.int32, device="cuda")
    status = pool.append(blocks_late, ids, stream=side)
    for _ in range(6):
        torch.mm(a, a, out=b)
    x_late2 = x.clone()
    cz = zx.compress_zf(x_late2, stream=side)
    for _ in range(6):
        torch.mm(a, a, out=b)
    x_late3 = x.clone()
    cb = zx.build_shared_codebook([x_late3], stream=side)
    torch.cuda.synchronize()
    assert torch.equal(zx.decompress_zf(cz).view(torch.int16), x.view(torch.int16))
    assert torch.equal(cb.lengths.cpu(), c.lengths.cpu()), "one tensor's shared codebook is its own"
    assert int(c._err.item()) == 0
    assert torch.equal(zx.decompress(c).view(torch.int16), x.view(torch.int16))
    assert torch.equal(status.cpu(), torch.zeros(3, dtype=torch.int32))
    rows = pool.decode(ids)
    torch.cuda.synchronize()
    assert torch.equal(rows.view(torch.int16), blocks.view(3, 65536).view(torch.int16))
