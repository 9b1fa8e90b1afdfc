"""Dominant-range codec on the GPU (csrc/zx_zf.hip) through the C ABI, against the
oracle (oracle/zf_oracle.c) byte for byte: per-block l_b, the three bit planes, the
record offsets and records, and the sign/mantissa bytes; then the decode must give
the input back bit for bit.  Sizes span several blocks and ragged tails, the record
scan's tile seam (8192 blocks), every BF16 and FP8 bit pattern, and the empty tensor.
A record offset past the record array is reported, not followed.  The 4096x4096 BF16,
8192x8192 FP8 and 1 GiB BF16 K/V workloads are compared whole.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import lossless_float_compression_amd as zx
from gpu_util import np_u

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


def check(x_dev, dtype):
    n = x_dev.numel()
    c = zx.compress_zf(x_dev)
    xb = np_u(x_dev.reshape(-1), np.uint16 if dtype == 0 else np.uint8)
    o = oracle.zf_encode(dtype, xb)
    assert c.nrecords == o.records.size
    assert np.array_equal(np_u(c.lb, np.uint8), o.lb)
    assert np.array_equal(np_u(c.planes, np.uint8).reshape(-1, 3, 256), o.planes)
    assert np.array_equal(np_u(c.rec_off, np.uint64), o.rec_off)
    assert np.array_equal(np_u(c.records, np.uint16)[:c.nrecords], o.records)
    assert np.array_equal(np_u(c.signmant, np.uint8), o.signmant)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = zx.decompress_zf(c, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(y.reshape(-1).view(x_dev.dtype), x_dev.reshape(-1)), f"n={n} did not round-trip"
    return c


def kv_like(n, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn(n, generator=g, device="cuda") / torch.sqrt(torch.rand(n, generator=g, device="cuda") + 0.05)
    x[::37] *= 20.0
    return (x * 0.5).to(torch.bfloat16).view(torch.int16)


@pytest.mark.parametrize("n", [1, 2, 3, 7, 8, 9, 2047, 2048, 2049, 5000, 65553, 1 << 20])
def test_bf16_parity(n):
    say("zf bf16", n)
    check(kv_like(n, n), 0)
    g = torch.Generator(device="cuda")
    g.manual_seed(7 + n)
    w = (torch.randn(n, generator=g, device="cuda") / 64).to(torch.bfloat16).view(torch.int16)
    check(w, 0)


@pytest.mark.parametrize("n", [1, 2, 3, 7, 9, 2047, 2049, 5001, 1 << 20])
def test_fp8_parity(n):
    say("zf fp8", n)
    g = torch.Generator(device="cuda")
    g.manual_seed(n)
    x = torch.randn(n, generator=g, device="cuda")
    q = (x / (x.abs().max() / 448)).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    check(q, 1)


def test_every_pattern():
    say("zf all patterns")
    x = torch.arange(1 << 16, dtype=torch.int32, device="cuda").to(torch.int16)
    check(x, 0)
    perm = torch.randperm(1 << 16, generator=torch.Generator().manual_seed(1)).cuda()
    check(x[perm].contiguous(), 0)
    y = torch.arange(256, dtype=torch.int32, device="cuda").to(torch.uint8).repeat(33)
    check(y, 1)


def test_record_scan_spans_two_tiles():
    say("zf two scan tiles")
    n = 8192 * 2048 + 3 * 2048 + 5                      # 8196 blocks
    check(kv_like(n, 5), 0)


def test_empty_tensor():
    c = zx.compress_zf(torch.empty(0, dtype=torch.bfloat16, device="cuda"))
    assert c.nrecords == 0 and int(c.rec_off[0].item()) == 0
    assert zx.decompress_zf(c).numel() == 0


def test_corrupt_record_offset_is_reported():
    say("zf corrupt offset")
    x = kv_like(4 * 2048, 3)
    c = zx.compress_zf(x)
    assert c.nrecords > 0
    bad = c.rec_off.clone()
    bad[2] = c.nrecords + 1000
    c2 = zx.ZfCompressed(dtype=c.dtype, n=c.n, shape=c.shape, nrecords=c.nrecords, lb=c.lb, planes=c.planes,
                         rec_off=bad, records=c.records, signmant=c.signmant)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    zx.decompress_zf(c2, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 4


@pytest.mark.parametrize("cfg", ["c2", "c4", "c5"])
def test_full_size_workloads(cfg):
    """The 4096x4096 BF16, 8192x8192 FP8 and [2,32,8,32768,128] BF16 K/V workloads
    whole, as the bench encodes and decodes them."""
    import workloads
    say("zf full", cfg)
    if cfg == "c2":
        check(workloads.c2().cuda().view(torch.int16).reshape(-1), 0)
    elif cfg == "c4":
        q, _ = workloads.c4(device="cuda")
        check(q.reshape(-1), 1)
    else:
        check(workloads.c5().reshape(-1), 0)
