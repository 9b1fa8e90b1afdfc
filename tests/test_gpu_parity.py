"""GPU parity: the HIP path through the C ABI against the CPU oracle.

All of this is integer/bit work, so the bar is bit-exactness: identical histograms,
identical code lengths, identical container bytes from encode, and decode output
equal to the input bit for bit (DFloat11 article, 实验结果: lossless means the
decompressed weights equal the originals bit for bit).
"""
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
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def rand_bf16(n, seed, scale=0.05):
    g = np.random.default_rng(seed)
    x = torch.from_numpy(g.standard_normal(n).astype(np.float32) * scale).to(torch.bfloat16)
    return x


def rand_fp8(n, seed):
    g = np.random.default_rng(seed)
    x = torch.from_numpy(g.standard_normal(n).astype(np.float32) * 20).clamp(-448, 448).to(torch.float8_e4m3fn)
    return x


def gpu_roundtrip_and_parity(x_cpu: torch.Tensor, per_block=False, max_len=32, check_oracle=True):
    """Compress on the GPU, compare every container array with the oracle's, decode
    on the GPU, compare with the input; also decode the oracle's container."""
    x = x_cpu.cuda()
    c = zx.compress(x, per_block=per_block, max_len=max_len)
    y = zx.decompress(c)
    torch.cuda.synchronize()
    assert int(c._err.item()) == 0
    r_in = raw(x_cpu)
    assert np.array_equal(raw(y), r_in)
    if check_oracle:
        o = oracle.encode(c.dtype, r_in, per_block=per_block, max_len=max_len)
        assert_same_container(to_oracle(c), o)
        # the GPU decoder reads the oracle's container too
        co = from_oracle(o)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        y2 = zx.decompress(co, out=torch.empty_like(y).reshape(-1), err=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert np.array_equal(raw(y2), r_in)
    return c


# ------------------------------------------------------------------ histogram

@pytest.mark.parametrize("dtype", [0, 1])
@pytest.mark.parametrize("n", [1, 1000, 65536, 65537, 300_001])
def test_histogram(dtype, n):
    say("hist", dtype, n)
    x = rand_bf16(n, n) if dtype == 0 else rand_fp8(n, n)
    r = raw(x)
    e = ((r >> 7) & 0xFF) if dtype == 0 else ((r >> 3) & 0xF)
    A = 256 if dtype == 0 else 16
    nb = (n + 65535) // 65536
    th = torch.empty(A, dtype=torch.int32, device="cuda")
    bh = torch.empty((nb, A), dtype=torch.int32, device="cuda")
    flat = x.cuda().reshape(-1).view(torch.int16 if dtype == 0 else torch.uint8)
    zx.zx_histogram(dtype, flat, n, th, bh)
    torch.cuda.synchronize()
    assert np.array_equal(np_u(th, np.uint32), np.bincount(e, minlength=A))
    for b in range(nb):
        assert np.array_equal(np_u(bh[b], np.uint32), np.bincount(e[b * 65536:(b + 1) * 65536], minlength=A))


@pytest.mark.parametrize("dtype", [zx.BF16, zx.FP8_E4M3FN, zx.E8M0])
@pytest.mark.parametrize("pattern", ["one value", "lane-shifted sweep", "random bits"])
def test_histogram_value_layouts(dtype, pattern):
    """Counts per block, per tensor and accumulated in 64 bits, for value patterns that
    stress the per-lane LDS counters: every lane on one value, and a sweep of every
    value shifted by the lane (neighbouring lanes on neighbouring values); three full
    blocks and a ragged tail."""
    say("hist layouts", dtype, pattern)
    n = 3 * 65536 + 4101
    A = zx.alphabet(dtype)
    i = np.arange(n, dtype=np.int64)
    g = np.random.default_rng(5)
    if pattern == "one value":
        sym = np.full(n, A // 2 + 1, dtype=np.int64)
    elif pattern == "lane-shifted sweep":
        sym = (i + i // 64) % A
    else:
        sym = g.integers(0, A, n)
    other = g.integers(0, 1 << 16, n)          # the bits outside the exponent field, at random
    if dtype == zx.BF16:
        words = ((other & 0x807F) | (sym << 7)).astype(np.uint16)
        x = torch.from_numpy(words.view(np.int16))
    elif dtype == zx.FP8_E4M3FN:
        words = ((other & 0x87) | (sym << 3)).astype(np.uint8)
        x = torch.from_numpy(words)
    else:
        words = sym.astype(np.uint8)
        x = torch.from_numpy(words)
    want = np.bincount(sym, minlength=A)
    nb = (n + 65535) // 65536
    xd = x.cuda()
    th = torch.empty(A, dtype=torch.int32, device="cuda")
    bh = torch.empty((nb, A), dtype=torch.int32, device="cuda")
    zx.zx_histogram(dtype, xd, n, th, bh)
    h64 = torch.zeros(A, dtype=torch.int64, device="cuda")
    L = zx.lib()
    s = torch.cuda.current_stream().cuda_stream
    for _ in range(2):
        assert L.zx_histogram_accumulate(dtype, xd.data_ptr(), n, h64.data_ptr(), s) == 0
    torch.cuda.synchronize()
    assert np.array_equal(np_u(th, np.uint32), want)
    for b in range(nb):
        assert np.array_equal(np_u(bh[b], np.uint32), np.bincount(sym[b * 65536:(b + 1) * 65536], minlength=A))
    assert np.array_equal(h64.cpu().numpy(), 2 * want)


# ------------------------------------------------------------------ codebook

@pytest.mark.parametrize("dtype", [0, 1])
def test_codebook_random(dtype):
    say("codebook", dtype)
    A = 256 if dtype == 0 else 16
    g = np.random.default_rng(11 + dtype)
    hists = []
    for i in range(96):
        h = np.zeros(A, np.uint32)
        k = int(g.integers(0, min(A, 60) + 1)) if i % 4 else int(g.integers(0, A + 1))
        syms = g.choice(A, size=k, replace=False)
        kind = i % 3
        if kind == 0:
            h[syms] = g.integers(1, 1000, size=k)
        elif kind == 1:
            h[syms] = np.minimum(g.zipf(1.2, size=k), 1 << 24)
        else:
            h[syms] = 1 + (np.arange(k) % 3)   # many ties
        hists.append(h)
    H = np.stack(hists)
    for max_len in ([32, 12, 8] if dtype == 0 else [32, 6, 4]):
        ln = torch.empty(H.shape, dtype=torch.uint8, device="cuda")
        dg = torch.empty(H.shape[0], dtype=torch.int16, device="cuda")
        zx.zx_build_codebook(dtype, torch.from_numpy(H.view(np.int32)).cuda(), H.shape[0], max_len, ln, dg)
        torch.cuda.synchronize()
        gl = np_u(ln, np.uint8)
        gd = np_u(dg, np.uint16)
        for i, h in enumerate(H):
            if (h > 0).sum() > (1 << max_len):
                continue
            ol, od = oracle.code_lengths(h.astype(np.uint64), max_len)
            assert np.array_equal(gl[i], ol), (max_len, i)
            assert gd[i] == od


def test_codebook_fibonacci_package_merge():
    say("codebook fib")
    fib = [1, 1]
    while len(fib) < 40:
        fib.append(fib[-1] + fib[-2])
    h = np.zeros(256, np.uint32)
    h[10:50] = fib
    for L in (32, 20, 9):
        ln = torch.empty((1, 256), dtype=torch.uint8, device="cuda")
        dg = torch.empty(1, dtype=torch.int16, device="cuda")
        zx.zx_build_codebook(0, torch.from_numpy(h.view(np.int32)).cuda(), 1, L, ln, dg)
        torch.cuda.synchronize()
        ol, _ = oracle.code_lengths(h.astype(np.uint64), L)
        assert np.array_equal(np_u(ln, np.uint8)[0], ol)
        assert ol.max() == L


# ------------------------------------------------------------------ encode/decode parity, small

@pytest.mark.parametrize("n", [1, 2, 3, 777, 65535, 65536, 65537, 200_001])
@pytest.mark.parametrize("per_block", [False, True])
def test_bf16_parity(n, per_block):
    say("bf16", n, per_block)
    gpu_roundtrip_and_parity(rand_bf16(n, 7 * n + 1), per_block)


@pytest.mark.parametrize("n", [1, 2, 3, 4097, 65536, 131073, 300_001])
@pytest.mark.parametrize("per_block", [False, True])
def test_fp8_parity(n, per_block):
    say("fp8", n, per_block)
    gpu_roundtrip_and_parity(rand_fp8(n, 3 * n + 2), per_block)


def test_all_bf16_patterns():
    say("all bf16")
    u = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    perm = torch.from_numpy(np.random.default_rng(0).permutation(65536)).long()
    for x in (u, u[perm], u.repeat(3)):
        for pb in (False, True):
            gpu_roundtrip_and_parity(x, pb)


def test_all_fp8_patterns():
    say("all fp8")
    u = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    for x in (u, u.repeat(700)):
        for pb in (False, True):
            gpu_roundtrip_and_parity(x, pb)


@pytest.mark.parametrize("dtype", [0, 1])
def test_constant_and_mixed_degenerate(dtype):
    say("constant", dtype)
    for n in (1, 65536, 65537, 300_000):
        x = torch.full((n,), 0x3F80 if dtype == 0 else 0x38, dtype=torch.int16 if dtype == 0 else torch.uint8)
        for pb in (False, True):
            gpu_roundtrip_and_parity(x, pb)
    if dtype == 0:
        parts = []
        for b in range(6):
            if b % 2:
                parts.append(torch.full((65536,), 0x4000 + b, dtype=torch.int16))
            else:
                parts.append(rand_bf16(65536, b).view(torch.int16))
        parts.append(torch.full((100,), 0x3C00, dtype=torch.int16))
        gpu_roundtrip_and_parity(torch.cat(parts), True)


def test_forced_package_merge():
    say("forced pm")
    fib = [1, 1]
    while len(fib) < 24:
        fib.append(fib[-1] + fib[-2])
    g = np.random.default_rng(4)
    e = g.permutation(np.repeat(np.arange(100, 124), fib))
    x = ((e.astype(np.uint16) << 7) | g.integers(0, 128, e.size).astype(np.uint16)).astype(np.uint16)
    c = gpu_roundtrip_and_parity(torch.from_numpy(x.view(np.int16)), False, max_len=12)
    assert int(c.lengths.max()) == 12


def test_encode_is_deterministic():
    say("determinism")
    x = rand_bf16(1 << 20, 5).cuda()
    a = to_oracle(zx.compress(x))
    for _ in range(3):
        assert_same_container(to_oracle(zx.compress(x)), a)


def test_encode_on_a_busy_side_stream():
    """compress, compress_zf and build_shared_codebook given a stream other than the
    current one: torch's fills and the size readback run on that stream too, so the
    sizes are read only after its kernels wrote them.  A long matmul queued first on
    the side stream delays those kernels while the current stream stays idle."""
    say("side stream")
    x = rand_bf16(1 << 20, 8).cuda()
    ref = to_oracle(zx.compress(x))
    refz = zx.compress_zf(x)
    a = torch.randn(4096, 4096, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()

    def busy():
        with torch.cuda.stream(s):
            for _ in range(8):
                torch.mm(a, a, out=b)

    busy()
    c = zx.compress(x, stream=s)
    busy()
    cz = zx.compress_zf(x, stream=s)
    busy()
    cb = zx.build_shared_codebook([x], stream=s)
    c2 = zx.compress(x, stream=s, codebook=cb)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        y = zx.decompress(c, err=err, stream=s)
    s.synchronize()
    assert int(c._err.item()) == 0 and int(c2._err.item()) == 0 and int(err.item()) == 0
    assert_same_container(to_oracle(c), ref)
    assert_same_container(to_oracle(c2), ref)      # one tensor's shared codebook is its own
    assert torch.equal(y.view(torch.int16), x.view(torch.int16))
    assert cz.nrecords == refz.nrecords
    for f in ("lb", "planes", "rec_off", "signmant"):
        assert torch.equal(getattr(cz, f), getattr(refz, f)), f
    assert torch.equal(cz.records[:cz.nrecords], refz.records[:refz.nrecords])


# ------------------------------------------------------------------ batch decode

def test_batch_equals_single():
    say("batch")
    xs = [rand_bf16(n, i).cuda() for i, n in enumerate([1, 65536, 1000, 300_001, 65537, 5, 131072])]
    cs = [zx.compress(x, per_block=(i % 2 == 1)) for i, x in enumerate(xs)]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    outs = zx.decompress_batch(cs, err=err)
    singles = [zx.decompress(c) for c in cs]
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for x, o, s in zip(xs, outs, singles):
        assert torch.equal(o.view(torch.int16), x.view(torch.int16))
        assert torch.equal(s.view(torch.int16), x.view(torch.int16))


# ------------------------------------------------------------------ corruption

def test_corrupt_container_is_reported_and_bounded():
    say("corrupt")
    n = 300_001
    x = rand_bf16(n, 99).cuda()
    for field, mutate in [
        # a gap moved by one bit: Huffman codes resynchronise, so only the check that
        # a chunk's codes end where the next chunk's first code starts catches it
        ("gaps", lambda c: c.gaps.__setitem__((3, 7), (int(c.gaps[3, 7]) + 1) % 32)),
        ("gaps_range", lambda c: c.gaps.__setitem__((4, 9), 40)),
        ("seg_desc", lambda c: c.seg_desc.__setitem__((2, 1), c.seg_desc[2, 1] + 1)),
        ("block_bitoff", lambda c: c.block_bitoff.__setitem__(2, c.block_bitoff[2] + 3)),
        ("gaps_ff", lambda c: c.gaps.__setitem__((1, 0), 0xFF)),
    ]:
        c = zx.compress(x)
        mutate(c)
        guard = torch.full((n + 2048,), 0x5A5A, dtype=torch.int16, device="cuda")
        out = guard[1024:1024 + n]
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        zx.zx_decode(c.container(), out, err)
        torch.cuda.synchronize()
        assert int(err.item()) == 4, field
        assert bool((guard[:1024] == 0x5A5A).all()) and bool((guard[1024 + n:] == 0x5A5A).all()), field


# ------------------------------------------------------------------ full-size workloads

def test_c1_full():
    say("c1")
    gpu_roundtrip_and_parity(workloads.c1())


def test_c2_full():
    say("c2")
    gpu_roundtrip_and_parity(workloads.c2())


def test_c4_full():
    say("c4")
    q, scale = workloads.c4()
    c = gpu_roundtrip_and_parity(q)
    assert c.dtype == 1
