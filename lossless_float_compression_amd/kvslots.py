"""K/V cache in fixed-size compressed slots, one 65536-element block per slot.

New blocks are compressed into preallocated slots as they fill, and reused blocks are
decompressed on demand (ZipFloat page, section 4.2: slot-based K/V layout with
incremental compressed writes; section 3.3: K/V blocks go to fixed per-block slots
without locks).  Fast online compression is what makes a compressed K/V cache usable
at all (ZipFloat page, 4.2; Intel summary, 局限性).

The compression runs on the device from end to end (zx_kv_encode_slots): histograms,
codebooks, block sizes and the bit-packing of every block are enqueued with no host
synchronisation, so an append can sit inside a decode loop.  Each slot is a complete
container (one block, its own codebook) at fixed offsets in the pool's arrays; the
stream part has a fixed capacity of `cap_words` words.  A block whose codes need more
bits than that is not stored: its status is ZX_E_NOSPACE and the caller keeps it some
other way (for instance uncompressed).

For a K/V cache laid out [kv, layer, head, token, channel] with 128 channels, one
block is 512 tokens of one (kv, layer, head); after every 512 generated tokens each
of the 2 * layers * heads slabs completes one block, and all of them are appended in
one call.
"""
from __future__ import annotations

import ctypes as C
from typing import Dict, List, Optional, Sequence

import torch

from . import zx as _zx

BLOCK = _zx.BLOCK_ELEMS


class KVSlotPool:
    """`n_slots` compressed slots of one dtype (BF16 or FP8 E4M3) on `device`.

    cap_words: code-stream capacity of a slot in u32 words (a multiple of 256, at
    most 8192, i.e. up to 4 bits per element); `bits_per_elem` gives it instead as a
    bit budget per element, rounded up to a multiple of 256 words."""

    def __init__(self, n_slots: int, dtype: int = _zx.BF16, cap_words: Optional[int] = None,
                 bits_per_elem: Optional[float] = None, device="cuda"):
        if n_slots <= 0:
            raise ValueError("n_slots must be positive")
        if (cap_words is None) == (bits_per_elem is None):
            raise ValueError("give exactly one of cap_words and bits_per_elem")
        if cap_words is None:
            cap_words = -(-int(bits_per_elem * BLOCK) // (32 * 256)) * 256
        sz = _zx.zx_kv_sizes()
        st = _zx.lib().zx_kv_slot_sizes(int(dtype), int(cap_words), C.byref(sz))
        if st != 0:
            raise _zx.ZxError("zx_kv_slot_sizes", st)
        self.dtype = int(dtype)
        self.n_slots = int(n_slots)
        self.cap_words = int(cap_words)
        self.sizes = sz
        u8 = dict(dtype=torch.uint8, device=device)
        i32 = dict(dtype=torch.int32, device=device)
        A = sz.alphabet
        self.signmant = torch.empty((n_slots, sz.sm_bytes), **u8)
        self.stream = torch.zeros((n_slots, sz.stream_words), **i32)
        self.gaps = torch.zeros((n_slots, sz.seg_stride, _zx.SEG_CHUNKS), **u8)
        self.seg_desc = torch.zeros((n_slots, sz.seg_stride, 2), **i32)
        self.lengths = torch.zeros((n_slots, A), **u8)
        self.degenerate = torch.zeros(n_slots, dtype=torch.int16, device=device)
        self.block_bitoff = torch.zeros((n_slots, 2), dtype=torch.int64, device=device)
        self.block_seg = torch.zeros((n_slots, 2), **i32)   # {0, 0}: an empty slot
        self.pool = _zx.zx_kv_pool(self.dtype, self.n_slots, self.cap_words, 0,
                                   self.signmant.data_ptr(), self.stream.data_ptr(), self.gaps.data_ptr(),
                                   self.seg_desc.data_ptr(), self.lengths.data_ptr(), self.degenerate.data_ptr(),
                                   self.block_bitoff.data_ptr(), self.block_seg.data_ptr())
        self._conts: Dict[int, _zx.zx_container] = {}
        self._ws: Optional[torch.Tensor] = None
        self._streams = set()   # side streams the pool's arrays are recorded on

    def _on_side(self, side: torch.cuda.Stream) -> None:
        """Mark the pool's arrays as used on `side` (once per stream), so that their
        memory is not handed out again before work there is done."""
        key = side.cuda_stream
        if key in self._streams:
            return
        self._streams.add(key)
        for t in (self.signmant, self.stream, self.gaps, self.seg_desc, self.lengths, self.degenerate,
                  self.block_bitoff, self.block_seg):
            t.record_stream(side)

    # ---- sizes
    def nbytes(self) -> int:
        """Device bytes the pool holds (all slots, whether used or not)."""
        return sum(t.numel() * t.element_size() for t in (self.signmant, self.stream, self.gaps, self.seg_desc,
                                                          self.lengths, self.degenerate, self.block_bitoff,
                                                          self.block_seg))

    def raw_bytes(self) -> int:
        """Bytes the same number of blocks takes uncompressed."""
        return self.n_slots * BLOCK * (2 if self.dtype == _zx.BF16 else 1)

    # ---- append
    def workspace(self, nblk: int) -> torch.Tensor:
        need = int(_zx.lib().zx_kv_workspace_bytes(self.dtype, int(nblk)))
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 16), dtype=torch.uint8, device=self.signmant.device)
        return self._ws

    def append(self, blocks: torch.Tensor, slot_ids: torch.Tensor, status: Optional[torch.Tensor] = None,
               err: Optional[torch.Tensor] = None, max_len: int = 32, stream=None, noalloc: bool = False,
               fused: bool = True) -> torch.Tensor:
        """Compress `blocks` (k * 65536 elements, contiguous; bf16/int16 for a BF16
        pool, float8_e4m3fn/uint8 for FP8) into slots `slot_ids` (device int32 [k],
        distinct).  Returns the per-block status (device int32 [k]: 0, or 6 when the
        block did not fit and its slot was left empty).  Nothing waits for the GPU.
        By default one launch builds each block's histogram, codebook and stream
        (zx_kv_encode_slots_fused); fused=False takes the separate histogram, codebook
        and size launches with a workspace (zx_kv_encode_slots), noalloc=True those
        launches with the library's fixed scratch.  All three write the same bytes.
        With a torch `stream` other than the current one, the append (and `status`,
        when allocated here) runs on it after the work already enqueued on the current
        stream, the producer of `blocks`.  Appends with fused=False share the pool's
        workspace, and noalloc=True ones the device's scratch: such calls must not
        overlap, on any stream."""
        side = _zx._side_stream(stream)
        if side is not None:
            side.wait_stream(torch.cuda.current_stream())
            self._on_side(side)
            with torch.cuda.stream(side):
                return self.append(blocks, slot_ids, status, err, max_len, None, noalloc, fused)
        dt, flat = _zx._as_bits(blocks)
        if dt != self.dtype:
            raise TypeError("blocks have another dtype than the pool")
        if not flat.is_contiguous() or flat.numel() % BLOCK:
            raise ValueError("blocks must be contiguous whole 65536-element blocks")
        k = flat.numel() // BLOCK
        if slot_ids.dtype != torch.int32 or slot_ids.numel() != k or not slot_ids.is_cuda:
            raise ValueError("slot_ids must be a device int32 tensor with one entry per block")
        if status is None:
            status = torch.empty(k, dtype=torch.int32, device=flat.device)
        if noalloc:
            # the library's own fixed scratch (zx_kv_encode_slots_noalloc): at most
            # KV_NOALLOC_MAX_BLOCKS blocks per call, no workspace, and calls on one
            # device must not overlap
            st = _zx.lib().zx_kv_encode_slots_noalloc(C.byref(self.pool), _zx._ptr(flat), k, _zx._ptr(slot_ids),
                                                      int(max_len), _zx._ptr(status), _zx._ptr(err), _zx._stream(stream))
            if st != 0:
                raise _zx.ZxError("zx_kv_encode_slots_noalloc", st)
            return status
        if fused:
            st = _zx.lib().zx_kv_encode_slots_fused(C.byref(self.pool), _zx._ptr(flat), k, _zx._ptr(slot_ids),
                                                    int(max_len), _zx._ptr(status), _zx._ptr(err), _zx._stream(stream))
            if st != 0:
                raise _zx.ZxError("zx_kv_encode_slots_fused", st)
            return status
        ws = self.workspace(k)
        st = _zx.lib().zx_kv_encode_slots(C.byref(self.pool), _zx._ptr(flat), k, _zx._ptr(slot_ids), int(max_len),
                                          _zx._ptr(ws), ws.numel(), _zx._ptr(status), _zx._ptr(err),
                                          _zx._stream(stream))
        if st != 0:
            raise _zx.ZxError("zx_kv_encode_slots", st)
        return status

    # ---- decode on demand
    def container(self, slot: int) -> _zx.zx_container:
        c = self._conts.get(slot)
        if c is None:
            c = _zx.zx_container()
            st = _zx.lib().zx_kv_slot_container(C.byref(self.pool), int(slot), C.byref(c))
            if st != 0:
                raise _zx.ZxError("zx_kv_slot_container", st)
            self._conts[slot] = c
        return c

    def _out(self, k: int, out: Optional[torch.Tensor]) -> torch.Tensor:
        if out is None:
            tdt = torch.bfloat16 if self.dtype == _zx.BF16 else torch.float8_e4m3fn
            out = torch.empty((k, BLOCK), dtype=tdt, device=self.signmant.device)
        esz = 2 if self.dtype == _zx.BF16 else 1
        if (out.dim() < 1 or out.shape[0] != k or out.numel() != k * BLOCK or not out.is_contiguous()
                or not out.is_cuda or out.element_size() != esz):
            raise ValueError(f"out must be a contiguous device tensor [len(slots), 65536] of {esz}-byte elements")
        return out

    def decode(self, slots, out: Optional[torch.Tensor] = None, err: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
        """Decompress the blocks in `slots` (a device int32 tensor, or host ints) into
        out[j] (shape [k, 65536], bf16 or float8_e4m3fn) with one launch, one
        workgroup per slot (zx_kv_decode_slots).  A slot whose block did not fit holds
        no segments and leaves its row unwritten.  With a torch `stream` other than the
        current one, everything (the slot-id copy, the output, the decode) runs on it
        after the work already enqueued on the current stream."""
        side = _zx._side_stream(stream)
        if side is not None:
            side.wait_stream(torch.cuda.current_stream())
            self._on_side(side)
            with torch.cuda.stream(side):
                return self.decode(slots, out, err, None)
        if not torch.is_tensor(slots):
            slots = torch.tensor(list(slots), dtype=torch.int32).to(self.signmant.device, non_blocking=True)
        if slots.dtype != torch.int32 or not slots.is_cuda:
            raise ValueError("slots must be a device int32 tensor or a sequence of ints")
        k = slots.numel()
        out = self._out(k, out)
        st = _zx.lib().zx_kv_decode_slots(C.byref(self.pool), _zx._ptr(slots), k, _zx._ptr(out), _zx._ptr(err),
                                          _zx._stream(stream))
        if st != 0:
            raise _zx.ZxError("zx_kv_decode_slots", st)
        return out

    def decode_containers(self, slots: Sequence[int], out: Optional[torch.Tensor] = None,
                          err: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        """As `decode`, through the per-slot containers and the tensor-batch decode
        (up to 16 slots per launch)."""
        side = _zx._side_stream(stream)
        if side is not None:
            side.wait_stream(torch.cuda.current_stream())
            self._on_side(side)
            with torch.cuda.stream(side):
                return self.decode_containers(slots, out, err, None)
        k = len(slots)
        out = self._out(k, out)
        rows = list(out.view(k, BLOCK))
        for i in range(0, k, _zx.MAX_BATCH):
            _zx.zx_decode_block_batch([self.container(s) for s in slots[i:i + _zx.MAX_BATCH]],
                                      rows[i:i + _zx.MAX_BATCH], err=err, stream=stream)
        return out
