"""GPU: zx_encode writes every word of its outputs, whatever the buffers held.

The stream words two blocks share (the first and last word of a block) are set by
each block in the bits it owns, and the stream's last block owns everything after
its own bits, the zero padding included.  So a stream, gap table, segment table and
sign/mantissa array allocated over old contents must come out byte for byte as the
oracle's container (the stored layout; DFloat11 article, 方法介绍, Fig. 2).  Each case
takes its codebook and block geometry from the oracle and fills the output buffers
with a non-zero pattern first; the cases cover full and ragged last blocks,
zero-bit blocks in the middle and at the end, and the empty tensor.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import lossless_float_compression_amd as zx
from gpu_util import assert_same_container, np_u

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


def data(dtype, n, seed, flat_blocks=()):
    """Seeded bits; blocks listed in flat_blocks hold one exponent only (0 bits each
    under a per-block codebook)."""
    rng = np.random.default_rng(seed)
    if dtype == zx.BF16:
        x = (rng.standard_normal(n) * 0.02).astype(np.float32)
        b = (x.view(np.uint32) >> 16).astype(np.uint16)
        for k in flat_blocks:
            s = slice(k * 65536, min((k + 1) * 65536, n))
            b[s] = (b[s] & 0x807F) | (120 << 7)
        return b
    if dtype == zx.FP8_E4M3FN:
        e = rng.integers(2, 12, n).astype(np.uint8)
        nib = rng.integers(0, 16, n).astype(np.uint8)
        for k in flat_blocks:
            e[k * 65536:(k + 1) * 65536] = 7
        return (((nib & 8) << 4) | (e << 3) | (nib & 7)).astype(np.uint8)
    e = rng.integers(110, 140, n).astype(np.uint8)   # E8M0 scale bytes
    for k in flat_blocks:
        e[k * 65536:(k + 1) * 65536] = 127
    return e


def up(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a).view(dt).copy()).cuda()


CASES = [
    # dtype, n, per_block, zero-bit blocks
    (zx.BF16, 4 * 65536, False, ()),                 # full blocks only
    (zx.BF16, 3 * 65536 + 5, False, ()),             # ragged last block
    (zx.BF16, 5 * 65536 + 777, True, (1, 3)),        # zero-bit blocks in the middle
    (zx.BF16, 4 * 65536 + 100, True, (4,)),          # a zero-bit last block
    (zx.BF16, 3 * 65536, True, (0, 1, 2)),           # every block zero-bit: padding only
    (zx.FP8_E4M3FN, 1_000_003, False, ()),
    (zx.FP8_E4M3FN, 6 * 65536, True, (2, 5)),
    (zx.E8M0, 70_000, False, ()),
    (zx.BF16, 0, False, ()),
]


@pytest.mark.parametrize("fill", [0xFF, 0xA5])
@pytest.mark.parametrize("dtype,n,per_block,flat", CASES)
def test_encode_over_old_contents_equals_oracle(dtype, n, per_block, flat, fill):
    say(f"encode over filled buffers: dtype {dtype} n {n} per_block {per_block} zero-bit blocks {flat} fill {fill:#x}")
    x = data(dtype, n, seed=n % 997 + 7 * dtype, flat_blocks=flat)
    o = oracle.encode(dtype, x, per_block=per_block, max_len=32)
    for k in flat:
        assert o.block_bitoff[k + 1] == o.block_bitoff[k], "the case must hold a zero-bit block"
    xd = up(x, np.int16 if dtype == zx.BF16 else np.uint8)
    sm_bytes = o.signmant.size
    signmant = torch.full((max(sm_bytes, 1),), fill, dtype=torch.uint8, device="cuda")
    words = torch.full((o.stream.size,), fill * 0x01010101 - (1 << 32 if fill >= 0x80 else 0), dtype=torch.int32,
                       device="cuda")
    seg_desc = torch.full((max(o.nsegs, 1), 2), -1, dtype=torch.int32, device="cuda")
    gaps = torch.full((max(o.nsegs, 1), 64), fill, dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    zx.zx_encode(dtype, xd, n, per_block, up(o.lengths, np.uint8), up(o.degenerate, np.int16),
                 up(o.block_bitoff, np.int64), up(o.block_seg, np.int32), o.total_bits, o.nsegs,
                 signmant, words, seg_desc, gaps, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    g = oracle.Container(
        dtype=dtype, per_block=int(per_block), n=n, lengths=o.lengths, degenerate=o.degenerate,
        signmant=np_u(signmant, np.uint8)[:sm_bytes], stream=np_u(words, np.uint32),
        block_bitoff=o.block_bitoff, block_seg=o.block_seg,
        seg_desc=np_u(seg_desc, np.uint32)[:o.nsegs], gaps=np_u(gaps, np.uint8)[:o.nsegs])
    assert_same_container(g, o)
