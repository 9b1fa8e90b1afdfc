"""Pins of the dominant-range exponent codec's oracle (oracle/zf_oracle.c), each
against something other than the oracle itself:

* worked blocks derived by hand from the ZipFloat page (sections 3.2-3.3), in
  tests/golden/zipfloat_block_example.txt, byte for byte;
* MD equals a library argmax of a library histogram (ties to the smallest);
* the record set is exactly the elements whose exponent lies outside
  [MD - 6, MD + 2) modulo the field, and the exponent bytes of a full block equal the
  layout's closed form 768 + 2 * outliers (3 dense bits per element, 16 bits per
  outlier record: the cost model of the page's Eq. 2 with the dense bits stored for
  every element);
* every BF16 and FP8 bit pattern, and random tensors of ragged sizes, round-trip.
"""
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "zipfloat_block_example.txt")


def golden_cases():
    cases, cur = [], None
    for line in open(GOLD):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        if key == "case":
            cur = {"name": vals[0], "dtype": int(vals[1])}
            cases.append(cur)
        elif key == "bits":
            cur["bits"] = np.array([int(v, 16) for v in vals], np.uint16 if cur["dtype"] == 0 else np.uint8)
        elif key in ("lb", "rec_off", "records"):
            cur[key] = [int(v) for v in vals]
        elif key == "planes":
            cur["planes"] = {(int(a), int(b)): int(h, 16) for a, rest in (v.split(":") for v in vals)
                             for b, h in [rest.split("=")]}
        elif key == "signmant":
            cur["signmant"] = [int(v, 16) for v in vals]
    return cases


@pytest.mark.parametrize("case", golden_cases(), ids=lambda c: c["name"])
def test_worked_blocks(case):
    c = oracle.zf_encode(case["dtype"], case["bits"])
    assert c.lb.tolist() == case["lb"]
    assert c.rec_off.tolist() == case["rec_off"]
    assert c.records.tolist() == case["records"]
    want = np.zeros((1, 3, 256), np.uint8)
    for (p, k), v in case["planes"].items():
        want[0, p, k] = v
    assert np.array_equal(c.planes, want)
    assert c.signmant.tolist() == case["signmant"]
    assert np.array_equal(oracle.zf_decode(c), case["bits"])


def exps_of(dtype, x):
    return ((x >> 7) & 0xFF).astype(np.int64) if dtype == 0 else ((x >> 3) & 0xF).astype(np.int64)


@pytest.mark.parametrize("dtype", [0, 1])
def test_mode_is_library_argmax(dtype):
    rng = np.random.default_rng(11)
    A = 256 if dtype == 0 else 16
    for t in range(200):
        e = rng.integers(0, A, size=int(rng.integers(1, 3000)), dtype=np.int64)
        if t % 3 == 0:
            e = np.minimum(e, 3 + t % 5)        # many ties
        assert oracle.zf_mode(e.astype(np.uint8), A) == int(np.argmax(np.bincount(e, minlength=A)))


def kv_like_bf16(rng, n):
    """Student-t values scaled like K/V entries, with a few channels much larger."""
    import torch
    x = rng.standard_t(5, size=n).astype(np.float32) * 0.5
    x[::37] *= 20.0
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("dtype", [0, 1])
def test_records_are_the_out_of_range_exponents_and_size_is_the_closed_form(dtype):
    rng = np.random.default_rng(3)
    A = 256 if dtype == 0 else 16
    if dtype == 0:
        x = kv_like_bf16(rng, 7 * 2048)
    else:
        x = rng.integers(0, 256, size=7 * 2048, dtype=np.uint8)
        x = np.where(x == 0x7F, 0x7E, np.where(x == 0xFF, 0xFE, x)).astype(np.uint8)
    c = oracle.zf_encode(dtype, x)
    e = exps_of(dtype, x)
    total_out = 0
    for b in range(c.nblocks):
        eb = e[b * 2048:(b + 1) * 2048]
        md = int(np.argmax(np.bincount(eb, minlength=A)))
        lb = (md - 6) % A
        assert int(c.lb[b]) == lb
        out = [(i, int((v - lb) % A)) for i, v in enumerate(eb) if not ((v - lb) % A) < 8]
        recs = c.records[int(c.rec_off[b]):int(c.rec_off[b + 1])]
        assert [(int(r) >> 5, int(r) & 31) for r in recs] == [(i, r >> 3) for i, r in out]
        total_out += len(out)
    # exponent bytes: 3 dense bits for every element plus a 16-bit record per outlier
    assert c.planes.nbytes + c.records.nbytes == 7 * (3 * 2048 // 8) + 2 * total_out
    assert np.array_equal(oracle.zf_decode(c), x)


def test_every_pattern_round_trips():
    rng = np.random.default_rng(0)
    x = np.arange(1 << 16, dtype=np.uint16)
    for order in (x, rng.permutation(x)):
        assert np.array_equal(oracle.zf_decode(oracle.zf_encode(0, order)), order)
    y = np.arange(256, dtype=np.uint8)
    for order in (y, rng.permutation(y), np.repeat(y, 9)):
        assert np.array_equal(oracle.zf_decode(oracle.zf_encode(1, order)), order)


@pytest.mark.parametrize("n", [0, 1, 2, 3, 2047, 2048, 2049, 4096, 10001])
def test_ragged_sizes_round_trip(n):
    rng = np.random.default_rng(n)
    x = kv_like_bf16(rng, n) if n else np.zeros(0, np.uint16)
    c = oracle.zf_encode(0, x)
    assert c.nblocks == (n + 2047) // 2048 and c.planes.shape == (c.nblocks, 3, 256)
    assert np.array_equal(oracle.zf_decode(c), x)
    f = rng.integers(0, 256, size=n, dtype=np.uint8)
    assert np.array_equal(oracle.zf_decode(oracle.zf_encode(1, f)), f)
