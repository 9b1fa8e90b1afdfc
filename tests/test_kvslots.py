"""K/V cache in fixed compressed slots (lossless_float_compression_amd.kvslots).

* CPU: slot strides and per-slot containers are plain pointer arithmetic on the
  host; bad arguments are rejected before anything is launched.
* GPU: blocks appended into slots (histograms, codebooks, sizes and packing all on
  the device) are compared with the oracle encoding each block on its own as a
  one-block container with a per-block codebook: code lengths, degenerate symbol,
  sign/mantissa bytes, stream bits (zero after the last code up to the end of the
  slot), segment entries and gap bytes must be equal byte for byte.  Slots decoded on
  demand, in any order, give the input back bit for bit.  A block that needs more
  bits than its slot holds is reported and leaves the slot empty; a slot written
  twice holds the second block only.
"""
import ctypes as C
import sys

import numpy as np
import pytest
import torch

import lossless_float_compression_amd as zx
from lossless_float_compression_amd import zx as Z
from lossless_float_compression_amd.kvslots import KVSlotPool

BLOCK = 65536


def sizes(dtype, cap):
    sz = Z.zx_kv_sizes()
    st = Z.lib().zx_kv_slot_sizes(dtype, cap, C.byref(sz))
    return st, sz


def test_slot_sizes():
    for dtype, sm in ((0, 65536), (1, 32768)):
        for cap in (256, 512, 768, 8192):
            st, sz = sizes(dtype, cap)
            assert st == 0
            assert sz.sm_bytes == sm
            assert sz.stream_words == Z.zx_stream_words(cap * 32) == cap + 260
            assert sz.max_segs == cap // 256
            assert sz.seg_stride % 2 == 0 and sz.seg_stride - sz.max_segs in (0, 1)
            assert sz.alphabet == (256 if dtype == 0 else 16)
    for cap in (0, 100, 255, 257, 8192 + 256, 1 << 20):
        assert sizes(0, cap)[0] == 1
    assert sizes(5, 256)[0] == 2


def fake_pool(dtype=0, n_slots=10, cap=768):
    base = 1 << 24
    return Z.zx_kv_pool(dtype, n_slots, cap, 0, base, 2 * base, 3 * base, 4 * base, 5 * base, 6 * base, 7 * base,
                        8 * base)


def test_slot_container_offsets():
    for dtype in (0, 1):
        p = fake_pool(dtype)
        st, sz = sizes(dtype, 768)
        c = Z.zx_container()
        assert Z.lib().zx_kv_slot_container(C.byref(p), 3, C.byref(c)) == 0
        A = 256 if dtype == 0 else 16
        assert (c.dtype, c.per_block, c.n) == (dtype, 1, BLOCK)
        assert c.nsegs == 3 and c.total_bits == 768 * 32 and c.stream_words == 768 + 260
        assert c.signmant == p.signmant + 3 * sz.sm_bytes
        assert c.stream == p.stream + 3 * sz.stream_words * 4
        assert c.gaps == p.gaps + 3 * sz.seg_stride * 64
        assert c.seg_desc == p.seg_desc + 3 * sz.seg_stride * 8
        assert c.lengths == p.lengths + 3 * A
        assert c.degenerate == p.degenerate + 3 * 2
        assert c.block_bitoff == p.block_bitoff + 3 * 16
        assert c.block_seg == p.block_seg + 3 * 8
        assert c.dtab is None
    p = fake_pool()
    assert Z.lib().zx_kv_slot_container(C.byref(p), 10, C.byref(Z.zx_container())) == 1


def test_encode_slots_argument_errors():
    L = Z.lib()
    P = C.c_void_p
    p = fake_pool()
    ws = int(L.zx_kv_workspace_bytes(0, 4))
    assert ws > 4 * 256 * 4
    assert L.zx_kv_encode_slots(None, P(0x1000), 4, P(0x2000), 32, P(0x3000), ws, P(0x4000), None, None) == 1
    assert L.zx_kv_encode_slots(C.byref(p), P(0x1001), 4, P(0x2000), 32, P(0x3000), ws, P(0x4000), None, None) == 1
    assert L.zx_kv_encode_slots(C.byref(p), P(0x1000), 4, P(0x2000), 32, P(0x3000), ws - 1, P(0x4000), None, None) == 1
    assert L.zx_kv_encode_slots(C.byref(p), P(0x1000), 4, None, 32, P(0x3000), ws, P(0x4000), None, None) == 1
    bad = fake_pool(cap=300)
    assert L.zx_kv_encode_slots(C.byref(bad), P(0x1000), 4, P(0x2000), 32, P(0x3000), ws, P(0x4000), None, None) == 1
    assert L.zx_kv_encode_slots(C.byref(p), P(0x1000), 0, P(0x2000), 32, P(0x3000), ws, P(0x4000), None, None) == 0
    assert L.zx_status_string(6)


def test_pool_arguments():
    with pytest.raises(ValueError):
        KVSlotPool(4, cap_words=256, bits_per_elem=1.0)
    with pytest.raises(ValueError):
        KVSlotPool(4)
    with pytest.raises(ValueError):
        KVSlotPool(0, cap_words=256)
    with pytest.raises(Z.ZxError):
        KVSlotPool(4, cap_words=300)


# ------------------------------------------------------------------------- GPU

def say(*a):
    print(*a, file=sys.stderr, flush=True)


def slot_matches_oracle(pool, slot, block_bits_np, dtype):
    import oracle
    from gpu_util import np_u
    o = oracle.encode(dtype, block_bits_np, per_block=True)
    A = 256 if dtype == 0 else 16
    assert np.array_equal(np_u(pool.lengths[slot], np.uint8), o.lengths[0])
    assert int(np_u(pool.degenerate[slot:slot + 1], np.uint16)[0]) == int(o.degenerate[0])
    assert np.array_equal(np_u(pool.signmant[slot], np.uint8), o.signmant)
    bo = np_u(pool.block_bitoff[slot], np.uint64)
    bs = np_u(pool.block_seg[slot], np.uint32)
    assert (int(bo[0]), int(bo[1])) == (0, o.total_bits)
    assert (int(bs[0]), int(bs[1])) == (0, o.nsegs)
    st = np_u(pool.stream[slot], np.uint32)
    nw = (o.total_bits + 31) // 32
    assert np.array_equal(st[:nw], o.stream[:nw])
    assert not st[nw:].any(), "slot stream not zero after the block's codes"
    assert np.array_equal(np_u(pool.seg_desc[slot, :o.nsegs], np.uint32), o.seg_desc)
    assert np.array_equal(np_u(pool.gaps[slot, :o.nsegs], np.uint8), o.gaps)
    assert A == pool.lengths.shape[1]


def kv_blocks(kv, layer, tokens=512):
    import workloads
    return workloads.c5_slab(kv, layer, device="cuda", tokens=tokens).reshape(-1, BLOCK).contiguous()


@pytest.mark.gpu
def test_append_matches_oracle_and_decodes_on_demand():
    from gpu_util import np_u
    x = kv_blocks(0, 3)                               # 8 blocks: 512 tokens of 8 heads
    pool = KVSlotPool(16, bits_per_elem=4.0)
    slots = [5, 0, 11, 3, 7, 9, 2, 14]
    sid = torch.tensor(slots, dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("kv append 8 blocks")
    status = pool.append(x, sid, err=err)
    torch.cuda.synchronize()
    assert status.tolist() == [0] * 8 and int(err.item()) == 0
    xb = np_u(x, np.uint16)
    for j, s in enumerate(slots):
        slot_matches_oracle(pool, s, xb[j], 0)
    order = [3, 14, 5, 2, 0, 9, 11, 7, 3]               # any order, repeats allowed
    derr = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("kv decode 9 slots, slot list")
    y = pool.decode(order, err=derr)
    say("kv decode 9 slots, containers")
    y2 = pool.decode_containers(order, err=derr)
    torch.cuda.synchronize()
    assert int(derr.item()) == 0
    for i, s in enumerate(order):
        assert torch.equal(y[i].view(torch.int16), x[slots.index(s)]), s
    assert torch.equal(y2.view(torch.int16), y.view(torch.int16))


@pytest.mark.gpu
def test_append_more_than_a_batch_and_rewrite_a_slot():
    from gpu_util import np_u
    x = torch.cat([kv_blocks(1, 0), kv_blocks(1, 1), kv_blocks(0, 31)])   # 24 blocks
    pool = KVSlotPool(40, bits_per_elem=3.5)
    slots = list(range(39, 15, -1))
    status = pool.append(x, torch.tensor(slots, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert status.tolist() == [0] * 24
    y = pool.decode(slots)
    assert torch.equal(y.view(torch.int16), x)
    assert torch.equal(pool.decode_containers(slots).view(torch.int16), x)   # 16 per launch, then 8
    # overwrite slot 20 with another block: the slot holds that block only
    z = kv_blocks(0, 7)[5:6].contiguous()
    say("kv rewrite slot 20")
    assert pool.append(z, torch.tensor([20], dtype=torch.int32, device="cuda")).tolist() == [0]
    torch.cuda.synchronize()
    slot_matches_oracle(pool, 20, np_u(z, np.uint16)[0], 0)
    assert torch.equal(pool.decode([20]).view(torch.int16), z)


@pytest.mark.gpu
def test_block_that_does_not_fit_leaves_its_slot_empty():
    x = kv_blocks(0, 0)[:2]                             # ~2.9 bits per element each
    c = torch.full((1, BLOCK), 0x3C00, dtype=torch.int16, device="cuda")   # one symbol: 0 bits
    blocks = torch.cat([x, c]).contiguous()
    pool = KVSlotPool(4, cap_words=256)                 # 1/8 bit per element
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("kv overflow")
    status = pool.append(blocks, torch.tensor([0, 1, 2], dtype=torch.int32, device="cuda"), err=err)
    torch.cuda.synchronize()
    assert status.tolist() == [6, 6, 0]
    assert int(err.item()) == 6
    assert pool.block_seg[0].tolist() == [0, 0] and pool.block_seg[1].tolist() == [0, 0]
    assert torch.equal(pool.decode([2]).view(torch.int16), c)
    # a slot id past the pool is reported and its row left alone
    derr = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = torch.zeros((2, BLOCK), dtype=torch.bfloat16, device="cuda")
    pool.decode([2, 4], out=y, err=derr)
    torch.cuda.synchronize()
    assert int(derr.item()) == 4
    assert torch.equal(y[0].view(torch.int16), c[0]) and not y[1].view(torch.int16).any()


@pytest.mark.gpu
def test_fp8_slots():
    import workloads
    from gpu_util import np_u
    q, _ = workloads.c4(device="cuda")
    x = q.reshape(-1)[:5 * BLOCK].reshape(5, BLOCK).contiguous()
    pool = KVSlotPool(6, dtype=zx.FP8_E4M3FN, bits_per_elem=3.0)
    slots = [4, 1, 0, 5, 2]
    say("kv fp8 append")
    status = pool.append(x, torch.tensor(slots, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert status.tolist() == [0] * 5
    xb = np_u(x, np.uint8)
    for j, s in enumerate(slots):
        slot_matches_oracle(pool, s, xb[j], 1)
    y = pool.decode(slots)
    assert torch.equal(y.view(torch.uint8), x)
    assert torch.equal(pool.decode_containers(slots).view(torch.uint8), x)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,max_len", [(zx.BF16, 32), (zx.BF16, 12), (zx.FP8_E4M3FN, 15), (zx.FP8_E4M3FN, 6)])
def test_fused_append_equals_workspace_append(dtype, max_len):
    """zx_kv_encode_slots_fused (one launch: each block's histogram, codebook and size
    in its workgroup) against zx_kv_encode_slots (separate launches, workspace): every
    pool array, status and error word equal.  The blocks include ones that do not fit
    their slot, a one-symbol block, and a slot id past the pool; max_len 12 / 6 force
    length-limited codes."""
    import workloads
    say("kv fused append", dtype, max_len)
    g = torch.Generator(device="cuda").manual_seed(17)
    if dtype == zx.BF16:
        x = torch.cat([kv_blocks(0, 4), kv_blocks(1, 9)[:2]])                           # 10 blocks, ~2.9 bits
        one = torch.full((1, BLOCK), 0x3C00, dtype=torch.int16, device="cuda")
        noise = torch.randint(-32768, 32767, (1, BLOCK), generator=g, device="cuda", dtype=torch.int32).to(torch.int16)
    else:
        q, _ = workloads.c4(device="cuda")
        x = q.reshape(-1)[:10 * BLOCK].reshape(10, BLOCK)                                  # ~2.6 bits
        one = torch.full((1, BLOCK), 0x38, dtype=torch.uint8, device="cuda")
        noise = torch.randint(0, 255, (1, BLOCK), generator=g, device="cuda", dtype=torch.int32).to(torch.uint8)
    blocks = torch.cat([x, noise, one]).contiguous()   # noise: 4+ bits per element, past any 3-bit slot
    pools = [KVSlotPool(16, dtype=dtype, cap_words=6144) for _ in range(2)]
    for p in pools:
        for f in ("signmant", "stream", "gaps", "seg_desc", "lengths", "degenerate", "block_bitoff", "block_seg"):
            getattr(p, f).zero_()
    slots = torch.tensor([15, 3, 7, 0, 12, 9, 1, 4, 16, 2, 11, 6], dtype=torch.int32, device="cuda")   # 16: past the pool
    errs = [torch.zeros(1, dtype=torch.int32, device="cuda") for _ in range(2)]
    st_ws = pools[0].append(blocks, slots, err=errs[0], max_len=max_len, fused=False)
    st_fu = pools[1].append(blocks, slots, err=errs[1], max_len=max_len)
    torch.cuda.synchronize()
    assert st_ws.tolist() == st_fu.tolist()
    assert st_fu.tolist()[8] == 1 and st_fu.tolist()[10] == 6 and st_fu.tolist()[11] == 0   # bad id, noise, one symbol
    assert st_fu.tolist().count(0) >= 6
    # the error word keeps the first report, and the order in which workgroups report
    # is not fixed: each holds one of the statuses reported
    reported = {v for v in st_fu.tolist() if v}
    assert int(errs[0].item()) in reported and int(errs[1].item()) in reported
    for f in ("signmant", "stream", "gaps", "seg_desc", "lengths", "degenerate", "block_bitoff", "block_seg"):
        assert torch.equal(getattr(pools[0], f), getattr(pools[1], f)), f
    ok = [int(s) for s, st in zip(slots.tolist(), st_fu.tolist()) if st == 0]
    y = pools[1].decode(ok)
    torch.cuda.synchronize()
    rows = [slots.tolist().index(s) for s in ok]
    assert torch.equal(y.reshape(len(ok), -1).view(blocks.dtype if blocks.dtype != torch.bfloat16 else torch.int16),
                       blocks[rows])
