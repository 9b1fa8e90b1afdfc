"""GPU: the decode launches captured in a HIP graph and replayed.

A decode call allocates nothing, sets no memory with a fill command and waits for
nothing on the host, so a layer's batched decode (and a single decode, and a
per-block-codebook one) can be captured once and replayed per use.  Each replay runs
after eager work that overwrites the outputs, and every replay is checked against
the input bit for bit (lossless: DFloat11 article, 实验结果)."""
import sys

import pytest
import torch

import lossless_float_compression_amd as zx

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def layer():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g = torch.Generator(device="cuda").manual_seed(9090)
    shapes = [(1024, 1024), (1024, 256), (2048, 1024), (300, 777)]
    xs = [(torch.randn(s, generator=g, device="cuda") * 0.02).to(torch.bfloat16) for s in shapes]
    cs = [zx.compress(x) for x in xs]
    torch.cuda.synchronize()
    return xs, cs


def check(xs, outs, err):
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for x, y in zip(xs, outs):
        assert torch.equal(y.view(torch.int16), x.view(torch.int16))


def replay_and_check(graph, xs, outs, err, times=4):
    for r in range(times):
        for o in outs:                      # eager work between the replays
            o.fill_(float("nan"))
        err.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        check(xs, outs, err)


def test_batch_decode_in_a_graph(layer):
    xs, cs = layer
    say("graph: batched decode of", len(cs), "tensors")
    outs = [zx.empty_output(c) for c in cs]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    zx.decompress_batch(cs, outs, err=err)          # eager first
    check(xs, outs, err)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        zx.decompress_batch(cs, outs, err=err)
    replay_and_check(graph, xs, outs, err)


def test_single_and_per_block_decodes_in_one_graph(layer):
    xs, cs = layer
    say("graph: single per-tensor decode and per-block decode")
    x0 = xs[2]
    cb = zx.compress(x0, per_block=True)
    outs = [zx.empty_output(cs[0]), zx.empty_output(cb)]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        zx.decompress(cs[0], out=outs[0], err=err)
        zx.decompress(cb, out=outs[1], err=err)
    replay_and_check(graph, [xs[0], x0], outs, err)


def test_kv_append_and_slot_decode_in_a_graph():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_float_compression_amd.kvslots import KVSlotPool
    say("graph: K/V fused append + slot decode, new blocks before every replay")
    k = 8
    pool = KVSlotPool(32, zx.BF16, bits_per_elem=4.0)
    slots = torch.arange(3, 3 + 2 * k, 2, dtype=torch.int32, device="cuda")
    blocks = torch.empty((k, zx.BLOCK_ELEMS), dtype=torch.bfloat16, device="cuda")
    status = torch.empty(k, dtype=torch.int32, device="cuda")
    out = torch.empty((k, zx.BLOCK_ELEMS), dtype=torch.bfloat16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(515)
    blocks.copy_(torch.randn(blocks.shape, generator=g, device="cuda") * 0.5)
    pool.append(blocks, slots, status=status, err=err)          # eager first
    pool.decode(slots, out=out, err=err)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), blocks.view(torch.int16))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pool.append(blocks, slots, status=status, err=err)
        pool.decode(slots, out=out, err=err)
    for r in range(4):
        # new K/V blocks (eager), then the captured append and decode
        blocks.copy_(torch.randn(blocks.shape, generator=g, device="cuda") * (0.25 + r))
        out.fill_(float("nan"))
        status.fill_(-1)
        err.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert torch.equal(status.cpu(), torch.zeros(k, dtype=torch.int32))
        assert torch.equal(out.view(torch.int16), blocks.view(torch.int16))
