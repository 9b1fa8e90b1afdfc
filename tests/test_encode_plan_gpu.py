"""zx_encode_plan (histogram, codebook, block geometry, totals and decode table in as
few launches as the tensor allows) against the separate calls it stands for and
against the oracle: every output bit for bit, and the totals published to pinned
host memory with their tag.  Both of its paths run: the one planning workgroup (up
to 2048 blocks) and the separate steps for larger tensors."""
import sys

import numpy as np
import pytest
import torch

import oracle
import lossless_float_compression_amd as zx

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


def bits_of(dtype, n, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    x = torch.randn(n, generator=g, device="cuda", dtype=torch.float32)
    if dtype == zx.BF16:
        return (x * 0.02).to(torch.bfloat16).view(torch.int16)
    if dtype == zx.FP8_E4M3FN:
        return (x * 30).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    return torch.randint(100, 140, (n,), generator=g, device="cuda", dtype=torch.int32).to(torch.uint8)   # E8M0 bytes


def separate_calls(dtype, flat, n, max_len):
    A, nb = zx.alphabet(dtype), zx.nblocks_of(n)
    th = torch.empty(A, dtype=torch.int32, device="cuda")
    bh = torch.empty((max(nb, 1), A), dtype=torch.int32, device="cuda")
    ln = torch.empty((1, A), dtype=torch.uint8, device="cuda")
    dg = torch.empty(1, dtype=torch.int16, device="cuda")
    bo = torch.empty(nb + 1, dtype=torch.int64, device="cuda")
    bs = torch.empty(nb + 1, dtype=torch.int32, device="cuda")
    tot = torch.empty(2, dtype=torch.int64, device="cuda")
    dt = torch.empty(zx.zx_decode_table_bytes(), dtype=torch.uint8, device="cuda")
    zx.zx_histogram(dtype, flat, n, th, bh)
    zx.zx_build_codebook(dtype, th, 1, max_len, ln, dg)
    zx.zx_encode_size(dtype, flat, n, False, ln, bh, bo, bs, tot)
    zx.zx_build_decode_table(dtype, ln, dt)
    return dict(ln=ln, dg=dg, bo=bo, bs=bs, tot=tot, dt=dt, th=th)


@pytest.mark.parametrize("dtype,n,max_len", [
    (zx.BF16, 0, 32), (zx.BF16, 1, 32), (zx.BF16, 3 * 65536 + 5, 32), (zx.BF16, 300_001, 12),
    (zx.FP8_E4M3FN, 1_000_003, 15), (zx.FP8_E4M3FN, 2048 * 65536, 8), (zx.E8M0, 70_000, 32),
    (zx.BF16, 2048 * 65536, 32),            # the largest tensor of the one-workgroup plan
    (zx.BF16, 2048 * 65536 + 1, 32),        # one block more: the separate steps
])
def test_plan_equals_separate_calls_and_oracle(dtype, n, max_len):
    say("encode plan", dtype, n, max_len)
    flat = bits_of(dtype, n, seed=n % 1000 + dtype)
    A, nb = zx.alphabet(dtype), zx.nblocks_of(n)
    ref = separate_calls(dtype, flat, n, max_len)
    bh = torch.empty((max(nb, 1), A), dtype=torch.int32, device="cuda")
    th = torch.empty(A, dtype=torch.int32, device="cuda")
    ln = torch.empty((1, A), dtype=torch.uint8, device="cuda")
    dg = torch.empty(1, dtype=torch.int16, device="cuda")
    bo = torch.empty(nb + 1, dtype=torch.int64, device="cuda")
    bs = torch.empty(nb + 1, dtype=torch.int32, device="cuda")
    tot = torch.empty(2, dtype=torch.int64, device="cuda")
    dt = torch.empty(zx.zx_decode_table_bytes(), dtype=torch.uint8, device="cuda")
    err = torch.full((1,), 77, dtype=torch.int32, device="cuda")
    host = torch.full((4,), -1, dtype=torch.int64, pin_memory=True)
    cd = torch.full((A,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    zx.zx_encode_plan(dtype, flat, n, max_len, bh, th, ln, dg, bo, bs, tot, host, 4242 + n, dt, err, codes=cd)
    torch.cuda.synchronize()
    for name, mine in (("ln", ln), ("dg", dg), ("bo", bo), ("bs", bs), ("tot", tot), ("dt", dt)):
        assert torch.equal(mine, ref[name]), name
    assert int(err.item()) == 0
    # the canonical codes (RFC 1951 order) for the lengths, by the oracle's own assignment
    lens = ln.cpu().numpy().reshape(-1)
    want = oracle.canonical_codes(lens).astype(np.uint32)
    got = cd.cpu().numpy().view(np.uint32)
    assert np.array_equal(got[lens > 0], want[lens > 0])
    h = host.numpy()
    assert (int(h[0]), int(h[1]), int(h[2])) == (int(tot[0]), int(tot[1]), 4242 + n)
    if n <= 4_000_000:
        # the oracle's code lengths from its own histogram of the same bits
        x = flat.cpu().numpy()
        x = x.view(np.uint16) if dtype == zx.BF16 else x
        exps = oracle.split(dtype, x)[0]
        hist = oracle.histogram(exps, A)
        ol, od = oracle.code_lengths(hist, max_len)
        assert np.array_equal(ln.cpu().numpy().reshape(-1), ol)
        assert int(dg.cpu().item()) & 0xFFFF == int(od)
        o = oracle.encode(dtype, x, per_block=False, max_len=max_len)
        assert np.array_equal(bo.cpu().numpy(), o.block_bitoff.astype(np.int64))
        assert np.array_equal(bs.cpu().numpy(), o.block_seg.astype(np.int32))


def test_compress_waits_for_the_published_totals_behind_earlier_work():
    """compress() waits for the totals on a pinned host word; with a long kernel ahead
    of it on the stream it falls back to waiting for the stream, and the container is
    the same."""
    x = bits_of(zx.BF16, 4 * 65536 + 77, seed=5)
    c0 = zx.compress(x)
    big = torch.empty(1 << 28, dtype=torch.uint8, device="cuda")
    for _ in range(20):
        big.add_(1)                      # about 20 x 0.1 ms of earlier work on the stream
    c1 = zx.compress(x)
    torch.cuda.synchronize()
    assert c0.total_bits == c1.total_bits and c0.nsegs == c1.nsegs
    for f in ("stream", "gaps", "seg_desc", "signmant", "lengths", "block_bitoff", "block_seg", "dtab"):
        assert torch.equal(getattr(c0, f), getattr(c1, f)), f


@pytest.mark.parametrize("dtype,n,max_len", [
    (zx.BF16, 1, 32), (zx.BF16, 3 * 65536 + 5, 32), (zx.BF16, 300_001, 12), (zx.BF16, 16 * 65536, 32),
    (zx.FP8_E4M3FN, 1_000_003, 15), (zx.E8M0, 70_000, 32), (zx.E8M0, 4 * 65536, 9),
])
def test_encode_coded_equals_encode(dtype, n, max_len):
    """zx_encode_coded with the codes zx_encode_plan wrote produces exactly what
    zx_encode produces from the lengths, into buffers that held other bytes."""
    say("encode coded", dtype, n, max_len)
    flat = bits_of(dtype, n, seed=n % 997 + 3 * dtype)
    A, nb = zx.alphabet(dtype), zx.nblocks_of(n)
    bh = torch.empty((max(nb, 1), A), dtype=torch.int32, device="cuda")
    th = torch.empty(A, dtype=torch.int32, device="cuda")
    ln = torch.empty((1, A), dtype=torch.uint8, device="cuda")
    dg = torch.empty(1, dtype=torch.int16, device="cuda")
    bo = torch.empty(nb + 1, dtype=torch.int64, device="cuda")
    bs = torch.empty(nb + 1, dtype=torch.int32, device="cuda")
    tot = torch.empty(2, dtype=torch.int64, device="cuda")
    cd = torch.empty(A, dtype=torch.int32, device="cuda")
    zx.zx_encode_plan(dtype, flat, n, max_len, bh, th, ln, dg, bo, bs, tot, codes=cd)
    total_bits, nsegs = (int(v) for v in tot.cpu().tolist())
    smn = n if dtype == zx.BF16 else (n + 1) // 2 if dtype == zx.FP8_E4M3FN else 0
    outs = []
    for fill in (0x00, 0xA5):
        sm = torch.full((max(smn, 16),), fill, dtype=torch.uint8, device="cuda")
        st = torch.full((zx.zx_stream_words(total_bits),), fill * 0x01010101 - (1 << 32 if fill >= 0x80 else 0),
                        dtype=torch.int32, device="cuda")
        sd = torch.full((nsegs, 2), fill, dtype=torch.int32, device="cuda")
        gp = torch.full((nsegs, 64), fill, dtype=torch.uint8, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        outs.append((sm, st, sd, gp, err))
    (sm0, st0, sd0, gp0, e0), (sm1, st1, sd1, gp1, e1) = outs
    zx.zx_encode(dtype, flat, n, False, ln, dg, bo, bs, total_bits, nsegs, sm0, st0, sd0, gp0, e0)
    zx.zx_encode_coded(dtype, flat, n, ln, cd, dg, bo, bs, total_bits, nsegs, sm1, st1, sd1, gp1, e1)
    torch.cuda.synchronize()
    assert int(e0.item()) == 0 and int(e1.item()) == 0
    assert torch.equal(st0, st1) and torch.equal(sd0, sd1) and torch.equal(gp0, gp1)
    assert torch.equal(sm0[:smn], sm1[:smn])
