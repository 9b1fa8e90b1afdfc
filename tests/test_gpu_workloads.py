"""Full-size workloads through the C ABI, in the launch configuration bench.py times.

* Llama-3-8B-shaped weight set: layer 0's seven tensors and the lm_head are
  compared with the oracle container byte for byte; every tensor of the set
  round-trips on the device through the batched one-layer decode.
* K/V cache [2, 32, 8, 32768, 128] (2^31 elements, one codebook per block): the
  whole cache round-trips on the device; sampled blocks are compared with the
  oracle encoding each block on its own (per-block codebooks make blocks
  independent, so a block's bits, gaps, segment entries and bytes must equal
  those of a one-block container).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
import lossless_float_compression_amd as zx
from gpu_util import assert_same_container, np_u, raw, to_oracle

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)
    zx.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def stream_bits(words_u32: np.ndarray, start: int, nbits: int) -> np.ndarray:
    """Bits [start, start + nbits) of a MSB-first u32 word stream, as 0/1 bytes."""
    w0 = start // 32
    w1 = (start + nbits + 31) // 32
    by = words_u32[w0:w1].astype(">u4").view(np.uint8)
    bits = np.unpackbits(by)
    off = start - 32 * w0
    return bits[off:off + nbits]


def test_c3_layer0_and_lm_head_match_oracle():
    names = workloads.c3_names()
    idx = list(range(7)) + [len(names) - 1]
    comps, xs = [], []
    for i in idx:
        say("c3 tensor", names[i][0])
        x = workloads.c3_tensor(i)
        c = zx.compress(x)
        torch.cuda.synchronize()
        assert int(c._err.item()) == 0
        o = oracle.encode(0, raw(x))
        assert_same_container(to_oracle(c), o)
        comps.append(c)
        xs.append(x)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    outs = zx.decompress_batch(comps[:7], err=err)
    head = zx.decompress(comps[7], err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for x, y in zip(xs[:7], outs):
        assert torch.equal(y.view(torch.int16), x)
    assert torch.equal(head.view(torch.int16), xs[7])


def test_c3_all_layers_round_trip():
    names = workloads.c3_names()
    per_layer = len(workloads.C3_SHAPES)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for layer in range(workloads.C3_LAYERS):
        ids = range(layer * per_layer, (layer + 1) * per_layer)
        xs = [workloads.c3_tensor(i) for i in ids]
        cs = [zx.compress(x) for x in xs]
        outs = zx.decompress_batch(cs, err=err)
        torch.cuda.synchronize()
        for x, y, i in zip(xs, outs, ids):
            assert torch.equal(y.view(torch.int16), x), names[i][0]
        del xs, cs, outs
    assert int(err.item()) == 0


def test_c5_kv_cache_round_trip_and_sampled_blocks():
    say("c5 generate")
    x = workloads.c5()
    n = x.numel()
    assert n == 1 << 31
    c = zx.compress(x, per_block=True)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = zx.decompress(c, err=err)
    torch.cuda.synchronize()
    assert int(c._err.item()) == 0 and int(err.item()) == 0
    assert torch.equal(y.view(torch.int16), x)
    del y
    nb = n // 65536
    bitoff = np_u(c.block_bitoff, np.uint64)
    bseg = np_u(c.block_seg, np.uint32)
    rng = np.random.default_rng(5)
    # the block scan runs in tiles of 8192 blocks: include the blocks around the tile seams
    seams = [8191, 8192, 8193, 16383, 16384, 24575, 24576]
    sample = sorted(set([0, 1, nb // 2, nb - 1] + seams + list(rng.integers(0, nb, 8))))
    stream = np_u(c.stream, np.uint32)
    for b in sample:
        say("c5 block", b)
        xb = raw(x.reshape(-1)[b * 65536:(b + 1) * 65536])
        o = oracle.encode(0, xb, per_block=True)
        assert np.array_equal(np_u(c.lengths[b], np.uint8), o.lengths[0])
        assert int(np_u(c.degenerate[b:b + 1], np.uint16)[0]) == int(o.degenerate[0])
        assert np.array_equal(np_u(c.signmant[b * 65536:(b + 1) * 65536], np.uint8), o.signmant)
        g0, g1 = int(bitoff[b]), int(bitoff[b + 1])
        assert g1 - g0 == o.total_bits
        ob = stream_bits(o.stream, 0, o.total_bits)
        assert np.array_equal(stream_bits(stream, g0, g1 - g0), ob)
        s0, s1 = int(bseg[b]), int(bseg[b + 1])
        assert s1 - s0 == o.nsegs
        sd = np_u(c.seg_desc[s0:s1], np.uint32).reshape(-1, 2)
        assert (sd[:, 0] == b).all() and np.array_equal(sd[:, 1], o.seg_desc[:, 1])
        assert np.array_equal(np_u(c.gaps[s0:s1], np.uint8), o.gaps)
