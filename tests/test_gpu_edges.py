"""GPU parity at the edges of the code: the longest codes the length limit allows, and
exponent streams of very low entropy.

Lossless means bit for bit (DFloat11 article, 实验结果), for every codebook the limit
allows, including 32-bit codes; and the pages report K/V caches whose exponents
compress to a fifth or less (edgentiq blog, "Compressing Key-Value Caches in LLMs";
Intel summary, 关键结果: FP8 exponent ratios down to 0.07), i.e. mean code lengths
near one bit.  Each case checks, from the oracle's container, that it really reaches
the regime it is named for, then compares the GPU container with the oracle's byte for
byte and decodes both ways.
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import lossless_float_compression_amd as zx
from gpu_util import assert_same_container, from_oracle, np_u, raw, to_oracle

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


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


def fib(k):
    f = [1, 1]
    while len(f) < k:
        f.append(f[-1] + f[-2])
    return f[:k]


def bf16_from_exps(e, rng):
    """BF16 bit patterns with the given exponent bytes and random sign and mantissa."""
    sm = rng.integers(0, 256, e.size).astype(np.uint16)
    return (((sm & 0x80) << 8) | (e.astype(np.uint16) << 7) | (sm & 0x7F)).astype(np.uint16)


def fp8_from_exps(e, rng):
    nib = rng.integers(0, 16, e.size).astype(np.uint8)
    return (((nib & 8) << 4) | (e.astype(np.uint8) << 3) | (nib & 7)).astype(np.uint8)


def code_starts(o: oracle.Container, exps: np.ndarray):
    """Per block, the stream position (block-relative) of every element's code, from
    the oracle container's code lengths: used only to check which decode regime a
    workload reaches (chunk fill, segment size), not for parity."""
    A = o.lengths.shape[1]
    out = []
    for b in range(o.nblocks):
        ln = o.lengths[b if o.per_block else 0].astype(np.int64)
        eb = exps[b * 65536:(b + 1) * 65536]
        lens = ln[eb]
        out.append(np.concatenate([[0], np.cumsum(lens)[:-1]]) if eb.size else np.zeros(0, np.int64))
    return out


def regime(o: oracle.Container, exps: np.ndarray):
    """(most codes starting in one 128-bit chunk, most elements in one 64-chunk segment)."""
    mx_chunk = mx_seg = 0
    for st in code_starts(o, exps):
        if st.size == 0:
            continue
        ch = st // 128
        mx_chunk = max(mx_chunk, int(np.bincount(ch).max()))
        mx_seg = max(mx_seg, int(np.bincount(ch // 64).max()))
    return mx_chunk, mx_seg


def exps_of(dtype, x):
    return ((x >> 7) & 0xFF).astype(np.uint8) if dtype == 0 else ((x >> 3) & 0xF).astype(np.uint8)


def parity(dtype, x: np.ndarray, per_block: bool, max_len: int = 32, batch_with_other: bool = True):
    """GPU container == oracle container; GPU decode of both equals the input; the
    batched decode (next to an ordinary tensor) too.  Returns the oracle container."""
    xt = torch.from_numpy(x.view(np.int16) if dtype == 0 else x).cuda()
    c = zx.compress(xt, per_block=per_block, max_len=max_len)
    o = oracle.encode(dtype, x, per_block=per_block, max_len=max_len)
    torch.cuda.synchronize()
    assert int(c._err.item()) == 0
    assert_same_container(to_oracle(c), o)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = zx.decompress(c, err=err)
    co = from_oracle(o)
    y2 = zx.decompress(co, out=torch.empty_like(y).reshape(-1), err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert np.array_equal(raw(y), x)
    assert np.array_equal(raw(y2), x)
    if batch_with_other:
        other = torch.from_numpy(np.random.default_rng(1).standard_normal(70_001).astype(np.float32) * 0.02)
        other = other.to(torch.bfloat16 if dtype == 0 else torch.float8_e4m3fn).cuda()
        c2 = zx.compress(other)
        outs = zx.decompress_batch([c2, c, c2], err=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert np.array_equal(raw(outs[1]), x)
        assert torch.equal(raw_t(outs[0]), raw_t(other)) and torch.equal(raw_t(outs[2]), raw_t(other))
    return o


def raw_t(t):
    return t.reshape(-1).view(torch.int16 if t.element_size() == 2 else torch.uint8)


# ------------------------------------------------------------------ tie rules on the device

def tie_cases():
    rows = []
    for line in open(os.path.join(GOLDEN, "huffman_tie_rules.txt")):
        if line.strip() and not line.startswith("#"):
            name, limit, counts, lengths, _flip, _cost = line.split()
            rows.append((name, int(limit), [int(v) for v in counts.split(",")], [int(v) for v in lengths.split(",")]))
    return rows


@pytest.mark.parametrize("dtype", [0, 1])
def test_codebook_tie_rules(dtype):
    """The device codebook builds the hand-derived lengths of the tie cases (leaf queue
    first on equal weight; in package-merge a leaf before a package)."""
    say("tie rules", dtype)
    A = 256 if dtype == 0 else 16
    lo = 8 if dtype == 0 else 4
    for name, limit, counts, lengths in tie_cases():
        if limit < lo:
            continue
        for off in (0, A - len(counts)):
            h = np.zeros(A, np.uint32)
            h[off:off + len(counts)] = counts
            ln = torch.empty((1, A), dtype=torch.uint8, device="cuda")
            dg = torch.empty(1, dtype=torch.int16, device="cuda")
            zx.zx_build_codebook(dtype, torch.from_numpy(h.view(np.int32)).cuda(), 1, limit, ln, dg)
            torch.cuda.synchronize()
            want = np.zeros(A, np.uint8)
            want[off:off + len(lengths)] = lengths
            assert np.array_equal(np_u(ln, np.uint8)[0], want), (name, off)


# ------------------------------------------------------------------ the longest codes

@pytest.mark.parametrize("max_len", [32, 28, 24])
def test_fibonacci_exponents_up_to_32_bit_codes(max_len):
    """33 exponents with Fibonacci counts F(1..33) (9,227,464 elements): the Huffman
    tree is a path, so the two rarest exponents get 32-bit codes.  At limit 32 that is
    the code itself; at 28 and 24 package-merge redistributes the lengths."""
    say("fib33", max_len)
    rng = np.random.default_rng(33)
    e = rng.permutation(np.repeat(np.arange(100, 133, dtype=np.uint8), fib(33)))
    x = bf16_from_exps(e, rng)
    o = parity(0, x, per_block=False, max_len=max_len, batch_with_other=(max_len == 32))
    assert int(o.lengths.max()) == max_len
    assert int(o.lengths[0, 100]) == max_len and int(o.lengths[0, 101]) == max_len


@pytest.mark.parametrize("dtype", [0, 1])
def test_fibonacci_blocks_per_block_codebooks(dtype):
    """Per-block scope: every 65536-element block holds its own Fibonacci histogram
    (21 symbols, F(1..21), padded with the commonest), so each block's code reaches 20
    bits under its own codebook; a forced limit of 12 (BF16) / 8 (FP8) runs
    package-merge per block.  Four blocks and a ragged tail."""
    say("fib blocks", dtype)
    rng = np.random.default_rng(21 + dtype)
    k = 21 if dtype == 0 else 15
    base = 90 if dtype == 0 else 0
    parts = []
    for b in range(5):
        cnt = np.array(fib(k), np.int64)
        cnt[-1] += 65536 - cnt.sum()
        e = np.repeat(np.arange(base, base + k, dtype=np.uint8), cnt)
        e = rng.permutation(e)
        if b == 4:
            e = e[:12_345]
        parts.append(e)
    e = np.concatenate(parts)
    x = bf16_from_exps(e, rng) if dtype == 0 else fp8_from_exps(e, rng)
    o = parity(dtype, x, per_block=True)
    assert int(o.lengths[:4].max()) >= (20 if dtype == 0 else 14)
    parity(dtype, x, per_block=True, max_len=12 if dtype == 0 else 8, batch_with_other=False)


# ------------------------------------------------------------------ low entropy

def low_entropy(dtype, n, p_top, seed):
    """One exponent with probability p_top, the rest spread geometrically over the
    exponents below it (a K/V-like or scale-like skew)."""
    rng = np.random.default_rng(seed)
    top = 120 if dtype == 0 else 7
    tail = rng.geometric(0.45, n).clip(1, 40 if dtype == 0 else 7)
    e = np.where(rng.random(n) < p_top, top, top - tail).astype(np.uint8)
    return (bf16_from_exps(e, rng) if dtype == 0 else fp8_from_exps(e, rng)), e


@pytest.mark.parametrize("dtype", [0, 1])
@pytest.mark.parametrize("per_block", [False, True])
@pytest.mark.parametrize("p_top", [0.9, 0.85, 0.75])
def test_low_entropy(dtype, per_block, p_top):
    """Mean code length 1.1-1.6 bits: 128-bit chunks hold more codes than the
    decoder's register rounds, and segments more elements than its stage.  Six blocks
    and a ragged tail, so several segments per block and a partial last block."""
    say("low entropy", dtype, per_block, p_top)
    n = 6 * 65536 + 4_321
    x, e = low_entropy(dtype, n, p_top, seed=int(p_top * 100) + 7 * dtype + per_block)
    o = parity(dtype, x, per_block=per_block)
    bbar = o.total_bits / n
    assert 1.0 < bbar < 1.7, bbar
    mx_chunk, mx_seg = regime(o, e)
    assert mx_chunk > 84 and mx_seg > 3616 - 16, (mx_chunk, mx_seg)


@pytest.mark.parametrize("dtype", [0, 1])
@pytest.mark.parametrize("p_top", [0.97, 0.99])
def test_low_entropy_segments_beyond_one_stage_window(dtype, p_top):
    """Mean code length about 1.02-1.07 bits: segments of 7700-8100 elements, more than
    the low-entropy decode's stage window (7552 positions), so their exponents are
    replayed and written in two windows; chunks of 128 one-bit codes fill every count
    round."""
    say("low entropy, two stage windows", dtype, p_top)
    n = 6 * 65536 + 4_321
    x, e = low_entropy(dtype, n, p_top, seed=3)
    o = parity(dtype, x, per_block=False)
    assert 1.0 < o.total_bits / n < 1.1
    mx_chunk, mx_seg = regime(o, e)
    assert mx_chunk == 128 and mx_seg > 7552, (mx_chunk, mx_seg)


@pytest.mark.parametrize("dtype", [0, 1])
def test_dense_runs_in_ordinary_data(dtype):
    """Runs of the one exponent that has a 1-bit code inside otherwise spread data:
    chunks inside a run hold 128 codes (beyond the register rounds) while whole
    segments stay within the stage, so the count and stage are done code by code for
    those segments only."""
    say("dense runs", dtype)
    rng = np.random.default_rng(5 + dtype)
    n = 4 * 65536 + 999
    top = 120 if dtype == 0 else 7
    if dtype == 0:
        e = (top - 1 - rng.integers(0, 24, n)).astype(np.uint8)
    else:                              # the other 15 FP8 exponents, evenly
        e = rng.integers(0, 15, n).astype(np.uint8)
        e += (e >= top).astype(np.uint8)
    run, lo, hi = 600, 100, 1400
    i = 0
    while i < n:                       # runs at random spacing: about 45% of the elements
        j = i + int(rng.integers(lo, hi))
        e[j:j + run] = top
        i = j + run
    x = bf16_from_exps(e, rng) if dtype == 0 else fp8_from_exps(e, rng)
    o = parity(dtype, x, per_block=False)
    assert int(o.lengths[0, top]) == 1
    mx_chunk, mx_seg = regime(o, e)
    assert mx_chunk > 84 and mx_seg < 3600, (mx_chunk, mx_seg)


@pytest.mark.parametrize("dtype", [0, 1])
def test_dense_stretch_in_ordinary_data(dtype):
    """Mean code length above 2.3 bits overall (the decode that shares one LDS region
    between a wavefront's words and its stage), with a stretch of one short-coded
    exponent in the middle: those segments hold more elements than the stage, so
    several wavefronts of one workgroup take the spare stage in turn."""
    say("dense stretch", dtype)
    rng = np.random.default_rng(17 + dtype)
    n = 7 * 65536 + 333
    top = 120 if dtype == 0 else 12
    e = (top - rng.geometric(0.3, n).clip(1, 30 if dtype == 0 else 12)).astype(np.uint8)
    e[150_000:190_000] = top - 1       # the commonest exponent: a code of two bits or less
    x = bf16_from_exps(e, rng) if dtype == 0 else fp8_from_exps(e, rng)
    o = parity(dtype, x, per_block=False)
    assert int(o.lengths[0, top - 1]) <= 2
    assert o.total_bits * 10 >= 23 * n, o.total_bits / n
    mx_chunk, mx_seg = regime(o, e)
    assert mx_seg > 3616, (mx_chunk, mx_seg)
