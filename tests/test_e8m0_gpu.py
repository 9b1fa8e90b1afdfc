"""FP4 block scale factors (E8M0 bytes) through the Huffman path on the GPU, against
the oracle byte for byte (Intel summary, FP4 results; blog on the same paper, FP4
section: the scales of FP4 blocks are Huffman-compressible).  Every byte is a bare
exponent and is coded whole; the container has no sign/mantissa array.  Inputs are
MX-style scales of N(0, 1/sqrt(fan_in)) weights (blocks of 32), every byte pattern,
constant scales (0-bit blocks), ragged sizes across the 65536-element block seam,
and the scales of the whole Llama-3-8B-shaped weight set."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
import lossless_float_compression_amd as zx
from gpu_util import assert_same_container, from_oracle, np_u, raw, to_oracle

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


def e8m0(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda().view(torch.float8_e8m0fnu)


def check(x: torch.Tensor, per_block=False, oracle_too=True):
    c = zx.compress(x, per_block=per_block)
    y = zx.decompress(c)
    torch.cuda.synchronize()
    assert c.dtype == zx.E8M0 and c.signmant.numel() == 0
    assert int(c._err.item()) == 0
    assert y.dtype == torch.float8_e8m0fnu
    r = raw(x)
    assert np.array_equal(raw(y), r)
    if oracle_too:
        o = oracle.encode(oracle.E8M0, r, per_block=per_block)
        assert_same_container(to_oracle(c), o)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        y2 = zx.decompress(from_oracle(o), out=torch.empty_like(y).reshape(-1), err=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0 and np.array_equal(raw(y2), r)
    return c


@pytest.mark.parametrize("n", [1, 2, 3, 15, 16, 17, 4097, 65535, 65536, 65537, 300_001])
@pytest.mark.parametrize("per_block", [False, True])
def test_mx_scales_parity(n, per_block):
    say("e8m0 mx scales", n, per_block)
    s = workloads.fp4_scales(-(-n // 128), 4096, idx=n).reshape(-1)[:n]
    c = check(e8m0(s), per_block)
    if n >= 65536:
        assert c.nbytes() < 0.3 * n      # a few exponents dominate


@pytest.mark.parametrize("per_block", [False, True])
def test_every_byte_pattern(per_block):
    say("e8m0 patterns", per_block)
    u = np.arange(256, dtype=np.uint8)
    for x in (u, np.tile(u, 700), np.random.default_rng(3).permutation(np.tile(u, 300))):
        check(e8m0(x), per_block)


def test_constant_and_empty():
    say("e8m0 constant/empty")
    for n in (1, 65536, 65537, 200_000):
        for pb in (False, True):
            c = check(e8m0(np.full(n, 120, np.uint8)), pb)
            assert c.total_bits == 0
    c = zx.compress(torch.empty(0, dtype=torch.float8_e8m0fnu, device="cuda"))
    assert c.n == 0 and zx.decompress(c).numel() == 0


def test_batch_and_shared_codebook():
    say("e8m0 batch/shared")
    parts = [e8m0(workloads.fp4_scales(r, 4096, idx=50 + r).reshape(-1)) for r in (64, 4096, 1024)]
    cb = zx.build_shared_codebook(parts)
    cs = [zx.compress(p, codebook=cb) for p in parts]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    outs = zx.decompress_batch(cs, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    h = sum(np.bincount(raw(p), minlength=256) for p in parts).astype(np.uint64)
    ln, dg = oracle.code_lengths(h, 32)
    for p, c, y in zip(parts, cs, outs):
        assert int(c._err.item()) == 0
        assert_same_container(to_oracle(c), oracle.encode(oracle.E8M0, raw(p), lengths=ln, degenerate=dg))
        assert np.array_equal(raw(y), raw(p))


def test_llama_shaped_scale_set_whole():
    """The scales of every tensor of the Llama-3-8B-shaped set (2.3e8 bytes), as the
    bench encodes and decodes them, compared whole with the oracle's container."""
    say("e8m0 llama scale set")
    s = workloads.fp4_scales_c3().view(torch.float8_e8m0fnu)
    check(s, per_block=False)


def test_unsupported_entry_points_reject_e8m0():
    x = e8m0(np.full(4096, 120, np.uint8))
    with pytest.raises(TypeError):
        zx.compress_zf(x)
    with pytest.raises(zx.ZxError):
        zx.KVSlotPool(4, dtype=zx.E8M0, bits_per_elem=2.0)
