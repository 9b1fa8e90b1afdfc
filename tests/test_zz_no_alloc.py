"""The K/V append that allocates nothing (zx_kv_encode_slots_noalloc), through the C
ABI, against the append with a caller workspace (zx_kv_encode_slots) on the same
blocks: every pool array and every block status equal, on two calls in a row, the
second with fewer blocks (the library's scratch keeps the first call's contents), for
BF16 K/V blocks and FP8 blocks; and the blocks decode back bit for bit."""
import ctypes as C
import sys

import numpy as np
import pytest
import torch

import lossless_float_compression_amd as zx
from lossless_float_compression_amd.kvslots import KVSlotPool

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def kv_blocks(k, dtype, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    z = torch.randn((k, 65536), generator=g, device="cuda")
    chi = torch.randn((k, 65536, 5), generator=g, device="cuda").pow(2).sum(-1) / 5.0
    t = 0.5 * z / chi.sqrt()                         # Student-t with 5 degrees of freedom, x0.5
    t[:, ::32] *= 20.0                               # outlier channels
    if dtype == zx.BF16:
        return t.to(torch.bfloat16)
    return (t * (448.0 / t.abs().max())).clamp(-448, 448).to(torch.float8_e4m3fn)


def pool_arrays(p):
    return {f: getattr(p, f).clone() for f in ("signmant", "stream", "gaps", "seg_desc", "lengths", "degenerate",
                                               "block_bitoff", "block_seg")}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    zx.lib()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", [zx.BF16, zx.FP8_E4M3FN])
def test_noalloc_append_equals_workspace_append(dtype):
    say("noalloc append", dtype)
    n_slots = 96
    a = KVSlotPool(n_slots, dtype, cap_words=7168)
    b = KVSlotPool(n_slots, dtype, cap_words=7168)
    for p in (a, b):                                 # identical starting contents
        for f in pool_arrays(p):
            getattr(p, f).zero_()
    err_a = torch.zeros(1, dtype=torch.int32, device="cuda")
    err_b = torch.zeros(1, dtype=torch.int32, device="cuda")
    calls = [(40, 11), (7, 12)]                      # the second call smaller than the first
    used = []
    rng = np.random.default_rng(3 + dtype)
    for k, seed in calls:
        blocks = kv_blocks(k, dtype, seed)
        ids = rng.choice([s for s in range(n_slots) if s not in used], size=k, replace=False)
        used += ids.tolist()
        sid = torch.tensor(ids, dtype=torch.int32, device="cuda")
        st_a = a.append(blocks, sid, err=err_a, fused=False)   # zx_kv_encode_slots, with a workspace
        st_b = b.append(blocks, sid, err=err_b, noalloc=True)
        torch.cuda.synchronize()
        assert torch.equal(st_a, st_b)
        assert int(err_a.item()) == int(err_b.item())
        for f, t in pool_arrays(a).items():
            assert torch.equal(t, getattr(b, f)), (k, f)
        ok = (st_b == 0).nonzero().flatten()
        if ok.numel():
            rows = b.decode(sid[ok])
            torch.cuda.synchronize()
            want = blocks.reshape(k, 65536)[ok.long()]
            nbits = torch.int16 if dtype == zx.BF16 else torch.uint8
            assert torch.equal(rows.view(nbits), want.view(nbits))


def test_noalloc_append_rejects_past_its_limit():
    pool = KVSlotPool(4, zx.BF16, cap_words=7168)
    blocks = torch.zeros((zx.zx.KV_NOALLOC_MAX_BLOCKS + 1) * 65536, dtype=torch.bfloat16, device="cuda")
    sid = torch.zeros(zx.zx.KV_NOALLOC_MAX_BLOCKS + 1, dtype=torch.int32, device="cuda")
    with pytest.raises(zx.ZxError) as e:
        pool.append(blocks, sid, noalloc=True)
    assert e.value.status == zx.zx.ZX_E_LIMIT
