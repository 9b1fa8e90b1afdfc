"""Helpers for the GPU parity tests: move containers between the HIP library's
device tensors and the oracle's numpy arrays (no codec arithmetic here)."""
import numpy as np
import torch

import oracle
import lossless_float_compression_amd as zx


def np_u(t: torch.Tensor, dt) -> np.ndarray:
    """Device tensor -> numpy array reinterpreted as unsigned dtype `dt`."""
    return t.detach().cpu().contiguous().numpy().view(dt)


def to_oracle(c: zx.Compressed) -> oracle.Container:
    return oracle.Container(
        dtype=c.dtype, per_block=c.per_block, n=c.n,
        lengths=np_u(c.lengths, np.uint8).reshape(-1, 16 if c.dtype == 1 else 256),
        degenerate=np_u(c.degenerate, np.uint16),
        signmant=np_u(c.signmant, np.uint8),
        stream=np_u(c.stream, np.uint32),
        block_bitoff=np_u(c.block_bitoff, np.uint64),
        block_seg=np_u(c.block_seg, np.uint32),
        seg_desc=np_u(c.seg_desc, np.uint32).reshape(-1, 2),
        gaps=np_u(c.gaps, np.uint8).reshape(-1, 64),
    )


def from_oracle(o: oracle.Container, device="cuda") -> zx.Compressed:
    """Upload an oracle container and build its decode table on the device."""
    def up(a, dt):
        return torch.from_numpy(np.ascontiguousarray(a).view(dt).copy()).to(device)
    nb = (o.n + 65535) // 65536
    lengths = up(o.lengths.reshape(-1, 16 if o.dtype == 1 else 256), np.uint8)
    c = zx.Compressed(
        dtype=o.dtype, per_block=o.per_block, n=o.n, shape=(o.n,), total_bits=o.total_bits, nsegs=o.nsegs,
        lengths=lengths, degenerate=up(o.degenerate, np.int16), signmant=up(o.signmant, np.uint8),
        stream=up(o.stream, np.int32), block_bitoff=up(o.block_bitoff, np.int64), block_seg=up(o.block_seg, np.int32),
        seg_desc=up(o.seg_desc.reshape(-1, 2), np.int32), gaps=up(o.gaps.reshape(-1, 64), np.uint8),
    )
    if not o.per_block and nb:
        c.dtab = torch.empty(zx.zx_decode_table_bytes(), dtype=torch.uint8, device=device)
        zx.zx_build_decode_table(o.dtype, c.lengths, c.dtab)
    return c


def assert_same_container(g: oracle.Container, o: oracle.Container):
    assert g.n == o.n and g.dtype == o.dtype
    for f in ("lengths", "degenerate", "block_bitoff", "block_seg", "signmant", "seg_desc", "gaps", "stream"):
        a, b = getattr(g, f), getattr(o, f)
        assert a.shape == b.shape, (f, a.shape, b.shape)
        if not np.array_equal(a, b):
            bad = np.nonzero(a.reshape(-1) != b.reshape(-1))[0]
            raise AssertionError(f"{f} differs at {bad.size} places, first {bad[:8]}: gpu {a.reshape(-1)[bad[:8]]} "
                                 f"oracle {b.reshape(-1)[bad[:8]]}")


def raw(x: torch.Tensor) -> np.ndarray:
    """Raw bits of a bf16/int16 (-> uint16) or fp8/uint8 (-> uint8) tensor."""
    if x.dtype in (torch.bfloat16, torch.int16):
        return np_u(x.reshape(-1).view(torch.int16), np.uint16)
    return np_u(x.reshape(-1).view(torch.uint8), np.uint8)
