"""One codebook for many tensors (a model-wide Huffman tree, DFloat11 article, 方法介绍).

* CPU, the oracle's encode with a given codebook: given the tensor's own codebook it
  writes exactly the bytes of the plain encode; given a shared one, the stream holds
  exactly sum(count * length) bits (a closed form from a library histogram) and the
  container round-trips; an exponent without a code is rejected.
* GPU: the device's shared codebook (64-bit histogram sum, then one codebook) equals
  the oracle's codebook of the summed library histogram; every tensor's container
  equals the oracle's encode with that codebook byte for byte; all tensors decode in
  one batched launch through the one shared table; a tensor holding an exponent the
  codebook lacks is reported through the container's error word.
"""
import sys

import numpy as np
import pytest
import torch

import oracle


def bf16_bits(rng, n, std):
    x = torch.from_numpy((rng.standard_normal(n) * std).astype(np.float32)).to(torch.bfloat16)
    return x.view(torch.int16).numpy().view(np.uint16)


def exps(b):
    return ((b >> 7) & 0xFF).astype(np.int64)


def test_own_codebook_gives_the_plain_bytes():
    rng = np.random.default_rng(1)
    b = bf16_bits(rng, 200001, 0.02)
    plain = oracle.encode(0, b)
    given = oracle.encode(0, b, lengths=plain.lengths[0], degenerate=int(plain.degenerate[0]))
    for f in ("lengths", "degenerate", "signmant", "stream", "block_bitoff", "block_seg", "seg_desc", "gaps"):
        assert np.array_equal(getattr(plain, f), getattr(given, f)), f


def test_shared_codebook_bits_and_round_trip():
    rng = np.random.default_rng(2)
    ts = [bf16_bits(rng, 70000 + 1000 * i, s) for i, s in enumerate((1 / 64, 1 / 120, 0.05, 0.002))]
    h = sum(np.bincount(exps(b), minlength=256) for b in ts).astype(np.uint64)
    ln, dg = oracle.code_lengths(h, 32)
    for b in ts:
        c = oracle.encode(0, b, lengths=ln, degenerate=dg)
        assert c.total_bits == int((np.bincount(exps(b), minlength=256) * ln.astype(np.int64)).sum())
        assert np.array_equal(oracle.decode(c), b)


def test_exponent_without_a_code_is_rejected():
    rng = np.random.default_rng(3)
    a = bf16_bits(rng, 5000, 0.02)
    ln, dg = oracle.code_lengths(np.bincount(exps(a), minlength=256).astype(np.uint64), 32)
    b = a.copy()
    missing = int(np.nonzero(ln == 0)[0][0])
    b[17] = np.uint16(missing << 7)
    with pytest.raises(ValueError):
        oracle.encode(0, b, lengths=ln, degenerate=dg)


# ------------------------------------------------------------------------- GPU

@pytest.mark.gpu
def test_shared_codebook_on_the_device():
    import lossless_float_compression_amd as zx
    from gpu_util import assert_same_container, np_u, raw, to_oracle
    print("shared codebook", file=sys.stderr, flush=True)
    g = torch.Generator(device="cuda")
    ts = []
    for i, (shape, std) in enumerate((((1024, 4096), 1 / 64), ((4096, 1024), 1 / 64), ((700, 14336), 1 / 120),
                                      ((333, 4096), 0.05))):
        g.manual_seed(40 + i)
        ts.append((torch.randn(shape, generator=g, device="cuda") * std).to(torch.bfloat16))
    cb = zx.build_shared_codebook(ts)
    h = sum(np.bincount(exps(raw(t)), minlength=256) for t in ts).astype(np.uint64)
    ln, dg = oracle.code_lengths(h, 32)
    assert np.array_equal(np_u(cb.lengths, np.uint8).reshape(-1), ln)
    assert int(np_u(cb.degenerate, np.uint16)[0]) == dg
    cs = [zx.compress(t, codebook=cb) for t in ts]
    torch.cuda.synchronize()
    for t, c in zip(ts, cs):
        assert int(c._err.item()) == 0
        assert_same_container(to_oracle(c), oracle.encode(0, raw(t), lengths=ln, degenerate=dg))
        assert c.dtab.data_ptr() == cb.dtab.data_ptr()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    outs = zx.decompress_batch(cs, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for t, y in zip(ts, outs):
        assert torch.equal(y.view(torch.int16), t.view(torch.int16))


@pytest.mark.gpu
def test_shared_codebook_missing_exponent_is_reported():
    import lossless_float_compression_amd as zx
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    a = (torch.randn(100000, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    cb = zx.build_shared_codebook([a])
    b = a.clone()
    b[12345] = 1.0e30          # an exponent far outside a's range
    c = zx.compress(b, codebook=cb)
    torch.cuda.synchronize()
    assert int(c._err.item()) == 3
