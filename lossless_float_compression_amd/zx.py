"""Python binding of libzx (ctypes).

This is argument marshalling only.  Every step of the codec runs in the HIP kernels
behind the C ABI in include/zx.h.  PyTorch supplies device memory and the current
stream.  If libzx.so is missing, this module raises: there is no CPU fallback.

Low-level names mirror the C ABI (zx_histogram, zx_build_codebook, zx_encode_size,
zx_encode, zx_build_decode_table, zx_decode, zx_decode_block_batch).  `compress`,
`decompress` and `decompress_batch` chain them and allocate the outputs.
"""
from __future__ import annotations

import ctypes as C
import itertools
import threading
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

import torch

BF16 = 0
FP8_E4M3FN = 1
E8M0 = 2   # FP4 block scale factors: every byte a bare exponent, coded whole
BLOCK_ELEMS = 65536
SEG_CHUNKS = 64
MAX_BATCH = 16

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzx.so")
_lib = None

_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported dtype", 3: "codebook error",
           4: "corrupt container", 5: "HIP launch failure", 6: "block does not fit its slot",
           7: "request larger than the library's fixed scratch"}
ZX_E_NOSPACE = 6
ZX_E_LIMIT = 7
KV_NOALLOC_MAX_BLOCKS = 1024


class ZxError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)} ({status})")
        self.status = status


class zx_container(C.Structure):
    _fields_ = [
        ("dtype", C.c_int32), ("per_block", C.c_int32),
        ("n", C.c_uint64), ("nsegs", C.c_uint64), ("total_bits", C.c_uint64), ("stream_words", C.c_uint64),
        ("lengths", C.c_void_p), ("degenerate", C.c_void_p), ("signmant", C.c_void_p), ("stream", C.c_void_p),
        ("block_bitoff", C.c_void_p), ("block_seg", C.c_void_p), ("seg_desc", C.c_void_p), ("gaps", C.c_void_p),
        ("dtab", C.c_void_p),
    ]


class zx_kv_pool(C.Structure):
    _fields_ = [
        ("dtype", C.c_int32), ("n_slots", C.c_uint32), ("cap_words", C.c_uint32), ("reserved_", C.c_uint32),
        ("signmant", C.c_void_p), ("stream", C.c_void_p), ("gaps", C.c_void_p), ("seg_desc", C.c_void_p),
        ("lengths", C.c_void_p), ("degenerate", C.c_void_p), ("block_bitoff", C.c_void_p), ("block_seg", C.c_void_p),
    ]


class zx_kv_sizes(C.Structure):
    _fields_ = [
        ("sm_bytes", C.c_uint64), ("stream_words", C.c_uint64), ("max_segs", C.c_uint32), ("seg_stride", C.c_uint32),
        ("alphabet", C.c_uint32), ("reserved_", C.c_uint32),
    ]


class zx_zf_container(C.Structure):
    _fields_ = [
        ("dtype", C.c_int32), ("reserved_", C.c_int32), ("n", C.c_uint64), ("nrecords", C.c_uint64),
        ("lb", C.c_void_p), ("planes", C.c_void_p), ("rec_off", C.c_void_p), ("records", C.c_void_p),
        ("signmant", C.c_void_p),
    ]


EXPORTS = ("zx_histogram", "zx_build_codebook", "zx_encode_size", "zx_encode", "zx_build_decode_table",
           "zx_decode_table_bytes", "zx_decode", "zx_decode_block_batch", "zx_decode_block_batch_wg", "zx_stream_words",
           "zx_status_string", "zx_version", "zx_kv_slot_sizes", "zx_kv_workspace_bytes", "zx_kv_encode_slots",
           "zx_kv_slot_container", "zx_kv_decode_slots", "zx_zf_scan_workspace_bytes", "zx_zf_encode_size",
           "zx_zf_encode", "zx_zf_decode", "zx_histogram_accumulate", "zx_build_codebook_u64",
           "zx_kv_encode_slots_noalloc", "zx_encode_plan", "zx_kv_encode_slots_fused", "zx_encode_coded")


def lib():
    """Load libzx.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "`python -m lossless_float_compression_amd._build` (there is no fallback)")
        L = C.CDLL(LIB_PATH)
        P, U64, U32, I = C.c_void_p, C.c_uint64, C.c_uint32, C.c_int
        L.zx_histogram.argtypes = [I, P, U64, P, P, P]
        L.zx_build_codebook.argtypes = [I, P, U32, U32, P, P, P]
        L.zx_encode_size.argtypes = [I, P, U64, I, P, P, P, P, P, P]
        L.zx_encode.argtypes = [I, P, U64, I, P, P, P, P, U64, U64, P, P, P, P, P, P]
        L.zx_build_decode_table.argtypes = [I, P, P, P]
        L.zx_decode_table_bytes.argtypes = []
        L.zx_decode_table_bytes.restype = C.c_size_t
        L.zx_decode.argtypes = [C.POINTER(zx_container), P, P, P]
        L.zx_decode_block_batch.argtypes = [C.POINTER(zx_container), C.POINTER(C.c_void_p), U32, P, P]
        L.zx_decode_block_batch_wg.argtypes = [C.POINTER(zx_container), C.POINTER(C.c_void_p), U32, U32, P, P]
        L.zx_stream_words.argtypes = [U64]
        L.zx_stream_words.restype = U64
        L.zx_status_string.argtypes = [I]
        L.zx_status_string.restype = C.c_char_p
        L.zx_version.restype = C.c_char_p
        L.zx_kv_slot_sizes.argtypes = [I, U32, C.POINTER(zx_kv_sizes)]
        L.zx_kv_workspace_bytes.argtypes = [I, U32]
        L.zx_kv_workspace_bytes.restype = C.c_size_t
        L.zx_kv_encode_slots.argtypes = [C.POINTER(zx_kv_pool), P, U32, P, U32, P, C.c_size_t, P, P, P]
        L.zx_kv_encode_slots_noalloc.argtypes = [C.POINTER(zx_kv_pool), P, U32, P, U32, P, P, P]
        L.zx_kv_encode_slots_fused.argtypes = [C.POINTER(zx_kv_pool), P, U32, P, U32, P, P, P]
        L.zx_kv_slot_container.argtypes = [C.POINTER(zx_kv_pool), U32, C.POINTER(zx_container)]
        L.zx_kv_decode_slots.argtypes = [C.POINTER(zx_kv_pool), P, U32, P, P, P]
        L.zx_zf_scan_workspace_bytes.argtypes = [U64]
        L.zx_zf_scan_workspace_bytes.restype = C.c_size_t
        L.zx_zf_encode_size.argtypes = [I, P, U64, P, P, P, C.c_size_t, P, P]
        L.zx_zf_encode.argtypes = [I, P, U64, P, P, P, U64, P, P, P, P]
        L.zx_zf_decode.argtypes = [C.POINTER(zx_zf_container), P, P, P]
        L.zx_histogram_accumulate.argtypes = [I, P, U64, P, P]
        L.zx_build_codebook_u64.argtypes = [I, P, U32, U32, P, P, P]
        L.zx_encode_plan.argtypes = [I, P, U64, U32, P, P, P, P, P, P, P, P, U64, P, P, P, P]
        L.zx_encode_coded.argtypes = [I, P, U64, P, P, P, P, P, U64, U64, P, P, P, P, P, P]
        for f in ("zx_histogram", "zx_build_codebook", "zx_encode_size", "zx_encode", "zx_build_decode_table",
                  "zx_decode", "zx_decode_block_batch", "zx_decode_block_batch_wg", "zx_kv_slot_sizes",
                  "zx_kv_encode_slots", "zx_kv_slot_container", "zx_kv_decode_slots", "zx_zf_encode_size",
                  "zx_zf_encode", "zx_zf_decode", "zx_histogram_accumulate", "zx_build_codebook_u64",
                  "zx_kv_encode_slots_noalloc", "zx_encode_plan", "zx_kv_encode_slots_fused", "zx_encode_coded"):
            getattr(L, f).restype = I
        _lib = L
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    if isinstance(stream, C.c_void_p):      # already marshalled
        return stream
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _raw_stream(dev) -> int:
    """The current torch stream of `dev` as a raw handle (the cheap accessor when this
    torch build has it)."""
    get = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    return get(dev.index) if get is not None else torch.cuda.current_stream(dev).cuda_stream


def _check(fn: str, st: int):
    if st != 0:
        raise ZxError(fn, st)


def alphabet(dtype: int) -> int:
    return 16 if dtype == FP8_E4M3FN else 256


def nblocks_of(n: int) -> int:
    return (n + BLOCK_ELEMS - 1) // BLOCK_ELEMS


# ----------------------------------------------------------------- C ABI mirrors

def zx_histogram(dtype, inp, n, tensor_hist=None, block_hist=None, stream=None):
    _check("zx_histogram", lib().zx_histogram(dtype, _ptr(inp), n, _ptr(tensor_hist), _ptr(block_hist), _stream(stream)))


def zx_build_codebook(dtype, hist, n_codebooks, max_len, lengths, degenerate, stream=None):
    _check("zx_build_codebook", lib().zx_build_codebook(dtype, _ptr(hist), n_codebooks, max_len, _ptr(lengths),
                                                        _ptr(degenerate), _stream(stream)))


def zx_encode_size(dtype, inp, n, per_block, lengths, block_hist, block_bitoff, block_seg, totals, stream=None):
    _check("zx_encode_size", lib().zx_encode_size(dtype, _ptr(inp), n, int(per_block), _ptr(lengths), _ptr(block_hist),
                                                  _ptr(block_bitoff), _ptr(block_seg), _ptr(totals), _stream(stream)))


def zx_encode_plan(dtype, inp, n, max_len, block_hist, tensor_hist, lengths, degenerate, block_bitoff, block_seg,
                   totals, totals_host=None, tag=0, dtab=None, err=None, stream=None, codes=None):
    """totals_host: a pinned host int64 tensor of at least 3 entries, or None; codes: an
    int32 device tensor of A entries that receives the canonical codes, or None."""
    _check("zx_encode_plan", lib().zx_encode_plan(dtype, _ptr(inp), n, max_len, _ptr(block_hist), _ptr(tensor_hist),
                                                  _ptr(lengths), _ptr(degenerate), _ptr(block_bitoff), _ptr(block_seg),
                                                  _ptr(totals), _ptr(totals_host), int(tag), _ptr(dtab), _ptr(codes),
                                                  _ptr(err), _stream(stream)))


def zx_encode(dtype, inp, n, per_block, lengths, degenerate, block_bitoff, block_seg, total_bits, nsegs,
              signmant, stream_words, seg_desc, gaps, err=None, stream=None):
    _check("zx_encode", lib().zx_encode(dtype, _ptr(inp), n, int(per_block), _ptr(lengths), _ptr(degenerate),
                                        _ptr(block_bitoff), _ptr(block_seg), total_bits, nsegs, _ptr(signmant),
                                        _ptr(stream_words), _ptr(seg_desc), _ptr(gaps), _ptr(err), _stream(stream)))


def zx_encode_coded(dtype, inp, n, lengths, codes, degenerate, block_bitoff, block_seg, total_bits, nsegs,
                    signmant, stream_words, seg_desc, gaps, err=None, stream=None):
    _check("zx_encode_coded", lib().zx_encode_coded(dtype, _ptr(inp), n, _ptr(lengths), _ptr(codes), _ptr(degenerate),
                                                    _ptr(block_bitoff), _ptr(block_seg), total_bits, nsegs,
                                                    _ptr(signmant), _ptr(stream_words), _ptr(seg_desc), _ptr(gaps),
                                                    _ptr(err), _stream(stream)))


def zx_build_decode_table(dtype, lengths, dtab, stream=None):
    _check("zx_build_decode_table", lib().zx_build_decode_table(dtype, _ptr(lengths), _ptr(dtab), _stream(stream)))


def zx_decode_table_bytes() -> int:
    return int(lib().zx_decode_table_bytes())


def zx_stream_words(total_bits: int) -> int:
    return int(lib().zx_stream_words(int(total_bits)))


def zx_decode(container: zx_container, out, err=None, stream=None):
    _check("zx_decode", lib().zx_decode(C.byref(container), _ptr(out), _ptr(err), _stream(stream)))


def zx_decode_block_batch(containers: Sequence[zx_container], outs: Sequence[torch.Tensor], err=None, stream=None,
                          max_workgroups: int = 0):
    k = len(containers)
    arr = (zx_container * k)(*containers)
    optrs = (C.c_void_p * k)(*[o.data_ptr() for o in outs])
    if max_workgroups:
        _check("zx_decode_block_batch_wg",
               lib().zx_decode_block_batch_wg(arr, optrs, k, int(max_workgroups), _ptr(err), _stream(stream)))
    else:
        _check("zx_decode_block_batch", lib().zx_decode_block_batch(arr, optrs, k, _ptr(err), _stream(stream)))


# ----------------------------------------------------------------- compressed tensor

@dataclass
class Compressed:
    """A compressed tensor: container v1 arrays as device tensors."""
    dtype: int
    per_block: int
    n: int
    shape: tuple
    total_bits: int
    nsegs: int
    lengths: torch.Tensor      # uint8 [ncb, A]
    degenerate: torch.Tensor   # int16 (u16 bits) [ncb]
    signmant: torch.Tensor     # uint8
    stream: torch.Tensor       # int32 (u32 bits) [stream_words]
    block_bitoff: torch.Tensor # int64 (u64 bits) [nblocks+1]
    block_seg: torch.Tensor    # int32 (u32 bits) [nblocks+1]
    seg_desc: torch.Tensor     # int32 (u32 bits) [nsegs, 2]
    gaps: torch.Tensor         # uint8 [nsegs, 64]
    dtab: Optional[torch.Tensor] = None  # uint8 decode table (per-tensor scope)
    fp8_scale: Optional[float] = None    # carried raw for FP8 tensors, never applied

    def container(self) -> zx_container:
        c = zx_container()
        c.dtype, c.per_block, c.n = self.dtype, self.per_block, self.n
        c.nsegs, c.total_bits, c.stream_words = self.nsegs, self.total_bits, self.stream.numel()
        c.lengths, c.degenerate = self.lengths.data_ptr(), self.degenerate.data_ptr()
        c.signmant, c.stream = self.signmant.data_ptr(), self.stream.data_ptr()
        c.block_bitoff, c.block_seg = self.block_bitoff.data_ptr(), self.block_seg.data_ptr()
        c.seg_desc, c.gaps = self.seg_desc.data_ptr(), self.gaps.data_ptr()
        c.dtab = self.dtab.data_ptr() if self.dtab is not None else None
        return c

    def nbytes(self) -> int:
        """All container bytes (arrays + a 64-byte header), excluding the decode
        table, which is derived from the lengths."""
        return int(64 + sum(t.numel() * t.element_size() for t in (
            self.lengths, self.degenerate, self.signmant, self.stream, self.block_bitoff,
            self.block_seg, self.seg_desc, self.gaps)))

    def raw_bytes(self) -> int:
        return self.n * (2 if self.dtype == BF16 else 1)


def _as_bits(x: torch.Tensor):
    """(dtype code, flat raw-bit view) of a bf16 / float8_e4m3fn / float8_e8m0fnu / int16 /
    uint8 tensor (int16 reads as BF16 bits, uint8 as FP8 E4M3FN bits)."""
    if x.dtype == torch.float8_e8m0fnu:
        return E8M0, x.reshape(-1).view(torch.uint8)
    if x.dtype in (torch.bfloat16, torch.int16):
        return BF16, x.reshape(-1).view(torch.int16)
    if x.dtype in (torch.float8_e4m3fn, torch.uint8):
        return FP8_E4M3FN, x.reshape(-1).view(torch.uint8)
    raise TypeError(f"unsupported dtype {x.dtype}")


@dataclass
class SharedCodebook:
    """One codebook for many tensors (device tensors): lengths u8 [1, A], degenerate
    int16 [1], and its decode table."""
    dtype: int
    lengths: torch.Tensor
    degenerate: torch.Tensor
    dtab: torch.Tensor


def build_shared_codebook(tensors, max_len: int = 32, stream=None) -> SharedCodebook:
    """A model-wide codebook: the exponent counts of all `tensors` (any iterable, read
    once) summed in 64 bits (zx_histogram_accumulate), then one Huffman codebook and
    one decode table.  Everything runs on `stream` (a torch stream; default the
    current one), after the work already enqueued on the current stream (the producers
    of the tensors) when it is another one."""
    side = _side_stream(stream)
    if side is not None:
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            return build_shared_codebook(tensors, max_len, None)
    L = lib()
    s = _stream(None)
    hist = None
    dtype = dev = None
    for t in tensors:
        dt, flat = _as_bits(t)
        if hist is None:
            dtype, dev = dt, t.device
            hist = torch.zeros(alphabet(dtype), dtype=torch.int64, device=dev)
        elif dt != dtype:
            raise TypeError("all tensors of a shared codebook must have one dtype")
        flat = flat.contiguous()
        _check("zx_histogram_accumulate", L.zx_histogram_accumulate(dtype, _ptr(flat), flat.numel(), _ptr(hist), s))
    if hist is None:
        raise ValueError("no tensors")
    A = alphabet(dtype)
    lengths = torch.empty((1, A), dtype=torch.uint8, device=dev)
    degenerate = torch.empty(1, dtype=torch.int16, device=dev)
    _check("zx_build_codebook_u64", L.zx_build_codebook_u64(dtype, _ptr(hist), 1, int(max_len), _ptr(lengths),
                                                            _ptr(degenerate), s))
    dtab = torch.empty(zx_decode_table_bytes(), dtype=torch.uint8, device=dev)
    zx_build_decode_table(dtype, lengths, dtab, s)
    return SharedCodebook(dtype=dtype, lengths=lengths, degenerate=degenerate, dtab=dtab)


def compress(x: torch.Tensor, per_block: bool = False, max_len: int = 32, fp8_scale: Optional[float] = None,
             stream=None, codebook: Optional[SharedCodebook] = None) -> Compressed:
    """Encode a device tensor (bf16 or int16 bits -> BF16; float8_e4m3fn or uint8 bits -> FP8;
    float8_e8m0fnu -> E8M0, the block scales of FP4 formats, coded whole byte).

    Runs histogram -> codebook -> block sizes (and the decode table), reads back the
    two totals (the single host synchronisation) to size the outputs, then encodes.
    With `codebook` (from build_shared_codebook), the tensor is coded with that
    codebook and shares its decode table; an exponent without a code sets the
    container's error word to ZX_E_CODEBOOK.

    `stream` (a torch stream; default the current one) carries every kernel, torch's
    own fills and the synchronisation of the readback; a stream other than the current
    one first waits for the work already enqueued on the current stream (the producer
    of `x`)."""
    side = _side_stream(stream)
    if side is not None:
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            return compress(x, per_block, max_len, fp8_scale, None, codebook)
    dtype, flat = _as_bits(x)
    if not flat.is_cuda:
        raise ValueError("compress expects a device tensor")
    if codebook is not None and (per_block or codebook.dtype != dtype):
        raise ValueError("a shared codebook needs per-tensor scope and the codebook's dtype")
    flat = flat.contiguous()
    dev = flat.device
    n = flat.numel()
    A = alphabet(dtype)
    nb = nblocks_of(n)
    ncb = nb if per_block else 1
    if not per_block and codebook is None and n < (1 << 32):
        return _compress_planned(x, dtype, flat, n, A, nb, max_len, fp8_scale, _raw_stream(dev))
    stream = _stream(None)
    u8 = dict(dtype=torch.uint8, device=dev)
    i32 = dict(dtype=torch.int32, device=dev)
    # each kernel is enqueued as soon as its buffers exist, so the GPU starts while
    # the host allocates the rest
    block_hist = torch.empty((max(nb, 1), A), **i32)
    tensor_hist = None if (per_block or codebook is not None) else torch.empty(A, **i32)
    zx_histogram(dtype, flat, n, tensor_hist, block_hist, stream)
    if codebook is None:
        lengths = torch.empty((max(ncb, 1), A), **u8)
        degenerate = torch.empty(max(ncb, 1), dtype=torch.int16, device=dev)
        zx_build_codebook(dtype, block_hist if per_block else tensor_hist, ncb, max_len, lengths, degenerate, stream)
    else:
        lengths, degenerate = codebook.lengths, codebook.degenerate
    if per_block and nb == 0:
        lengths = lengths[:0]
        degenerate = degenerate[:0]
    block_bitoff = torch.empty(nb + 1, dtype=torch.int64, device=dev)
    block_seg = torch.empty(nb + 1, **i32)
    totals = torch.empty(2, dtype=torch.int64, device=dev)
    zx_encode_size(dtype, flat, n, per_block, lengths, block_hist, block_bitoff, block_seg, totals, stream)
    # work that does not depend on the sizes goes before the readback: the decode
    # table (it needs only the code lengths) and the outputs of known size
    dtab = None
    if codebook is not None:
        dtab = codebook.dtab
    elif not per_block:
        dtab = torch.empty(zx_decode_table_bytes(), **u8)
        zx_build_decode_table(dtype, lengths, dtab, stream)
    signmant = torch.empty(n if dtype == BF16 else (n + 1) // 2 if dtype == FP8_E4M3FN else 0, **u8)
    err = torch.zeros(1, **i32)
    total_bits, nsegs = (int(v) for v in totals.cpu().tolist())
    words = torch.empty(zx_stream_words(total_bits), **i32)
    seg_desc = torch.empty((nsegs, 2), **i32)
    gaps = torch.empty((nsegs, SEG_CHUNKS), **u8)
    zx_encode(dtype, flat, n, per_block, lengths, degenerate, block_bitoff, block_seg, total_bits, nsegs,
              signmant, words, seg_desc, gaps, err, stream)
    c = Compressed(dtype=dtype, per_block=int(per_block), n=n, shape=tuple(x.shape), total_bits=total_bits,
                   nsegs=nsegs, lengths=lengths, degenerate=degenerate, signmant=signmant, stream=words,
                   block_bitoff=block_bitoff, block_seg=block_seg, seg_desc=seg_desc, gaps=gaps, dtab=dtab,
                   fp8_scale=fp8_scale)
    c._err = err  # device word set by the encoder on a data/codebook mismatch
    return c


_plan_tags = itertools.count(1)   # next() is atomic: concurrent compress() calls get distinct tags
# device index -> (pinned int64 [_PLAN_SLOTS, 4] where zx_encode_plan publishes the totals,
# its numpy view, its address)
_plan_ring = {}
_plan_ring_lock = threading.Lock()
_PLAN_SLOTS = 256


def _plan_slot(dev):
    """A pinned 4-word host slot for one compress() call, as (address, numpy view, tag)
    (slots are reused round-robin; each call's unique tag tells its own publication
    from an older one)."""
    ring = _plan_ring.get(dev.index)
    if ring is None:
        with _plan_ring_lock:
            ring = _plan_ring.get(dev.index)
            if ring is None:
                t = torch.full((_PLAN_SLOTS, 4), -1, dtype=torch.int64, pin_memory=True)
                ring = _plan_ring[dev.index] = (t, t.numpy(), t.data_ptr())
    tag = next(_plan_tags)
    i = tag % _PLAN_SLOTS
    return ring[2] + 32 * i, ring[1][i], tag


def _layout(sizes):
    """16-byte-aligned offsets of (bytes, dtype) pieces in one arena, and its size."""
    offs, off = [], 0
    for nbytes, _ in sizes:
        offs.append(off)
        off += (nbytes + 15) // 16 * 16
    return offs, off


def _compress_planned(x, dtype, flat, n, A, nb, max_len, fp8_scale, stream):
    """Per-tensor codebook: zx_encode_plan (histogram, codebook, sizes and totals in
    as few launches as the tensor allows; the canonical codes and the decode table
    after the totals), a wait for the totals on a pinned host word instead of the
    stream, then zx_encode_coded with those codes.  The
    launches take raw addresses in one arena; the container's tensor views of it are
    made while the kernels run."""
    dev = flat.device
    L = lib()
    u8 = dict(dtype=torch.uint8, device=dev)
    nbw = max(nb, 1)
    sizes = [(zx_decode_table_bytes(), torch.uint8), (8 * (nb + 1), torch.int64), (4 * (nb + 1), torch.int32),
             (16, torch.int64), (4, torch.int32), (A, torch.uint8), (2, torch.int16)]
    offs, total = _layout(sizes)
    ws = torch.empty(nbw * A + 2 * A, dtype=torch.int32, device=dev)   # block histograms, tensor histogram, codes
    arena = torch.empty(total, **u8)
    base, wsp = arena.data_ptr(), ws.data_ptr()
    o_dtab, o_bo, o_bs, o_tot, o_err, o_len, o_deg = offs
    host_ptr, hv, tag = _plan_slot(dev)
    _check("zx_encode_plan", L.zx_encode_plan(dtype, flat.data_ptr(), n, max_len, wsp, wsp + 4 * nbw * A, base + o_len,
                                              base + o_deg, base + o_bo, base + o_bs, base + o_tot, host_ptr, tag,
                                              base + o_dtab, wsp + 4 * (nbw * A + A), base + o_err, stream))
    signmant = torch.empty(n if dtype == BF16 else (n + 1) // 2 if dtype == FP8_E4M3FN else 0, **u8)
    dtab, block_bitoff, block_seg, totals, err, lengths, degenerate = (
        arena[o:o + nbytes].view(dt) for o, (nbytes, dt) in zip(offs, sizes))
    spins = 0
    while hv[2] != tag:
        spins += 1
        if spins == 20000:          # the stream is busy with earlier work: block on it instead
            torch.cuda.current_stream().synchronize()
            if hv[2] != tag:
                raise RuntimeError("zx_encode_plan did not publish its totals")
    total_bits, nsegs = int(hv[0]), int(hv[1])
    nwords = zx_stream_words(total_bits)
    # one allocation: stream words, segment table, gaps (16-byte aligned pieces)
    o_sd = (4 * nwords + 15) // 16 * 16
    o_gp = o_sd + (8 * nsegs + 15) // 16 * 16
    out = torch.empty(o_gp + SEG_CHUNKS * nsegs, **u8)
    ob = out.data_ptr()
    _check("zx_encode_coded", L.zx_encode_coded(dtype, flat.data_ptr(), n, base + o_len, wsp + 4 * (nbw * A + A),
                                                base + o_deg, base + o_bo, base + o_bs, total_bits, nsegs,
                                                signmant.data_ptr(), ob, ob + o_sd, ob + o_gp, base + o_err, stream))
    # the container's views of it, made while the encode runs (as few tensor operations
    # as possible: this is the host's share of back-to-back calls)
    out32 = out.view(torch.int32)
    c = Compressed(dtype=dtype, per_block=0, n=n, shape=tuple(x.shape), total_bits=total_bits,
                   nsegs=nsegs, lengths=lengths.view(1, A), degenerate=degenerate, signmant=signmant,
                   stream=out32[:nwords], block_bitoff=block_bitoff, block_seg=block_seg,
                   seg_desc=out32.as_strided((nsegs, 2), (2, 1), o_sd // 4),
                   gaps=out.as_strided((nsegs, SEG_CHUNKS), (SEG_CHUNKS, 1), o_gp), dtab=dtab, fp8_scale=fp8_scale)
    c._err = err
    return c


def empty_output(c: Compressed, device=None) -> torch.Tensor:
    dev = device if device is not None else c.signmant.device
    if c.dtype == BF16:
        return torch.empty(c.shape, dtype=torch.bfloat16, device=dev)
    if c.dtype == E8M0:
        return torch.empty(c.shape, dtype=torch.float8_e8m0fnu, device=dev)
    return torch.empty(c.shape, dtype=torch.float8_e4m3fn, device=dev)


def _elem_bytes(dtype: int) -> int:
    return 2 if dtype == BF16 else 1


def check_out(out: torch.Tensor, n: int, dtype: int, what: str = "out") -> None:
    """A decode writes n elements of the container's width through out's pointer:
    reject anything that is not exactly that (another width, size or layout would
    make the kernel write past or across the buffer)."""
    if not out.is_cuda or not out.is_contiguous() or out.numel() != n or out.element_size() != _elem_bytes(dtype):
        raise ValueError(f"{what} must be a contiguous device tensor of {n} elements of "
                         f"{_elem_bytes(dtype)} bytes (got {tuple(out.shape)}, {out.dtype}, "
                         f"{'device' if out.is_cuda else 'host'}, contiguous={out.is_contiguous()})")


def _side_stream(stream):
    """A torch stream other than the current one, or None.  Work given such a stream
    first makes it wait for everything already enqueued on the current stream (the
    producers of the containers and of caller-supplied outputs), then runs with it as
    the current stream so that any output is allocated on it."""
    if stream is None or isinstance(stream, C.c_void_p):   # a raw handle: ordering is the caller's
        return None
    cur = torch.cuda.current_stream()
    return None if stream == cur else stream


def decompress(c: Compressed, out: Optional[torch.Tensor] = None, err: Optional[torch.Tensor] = None, stream=None):
    """Decode into `out` (allocated when None).  `err` is an optional int32 device
    word that receives 4 (corrupt) if the decoder finds an inconsistency.  With a
    torch `stream` other than the current one the decode runs on it after the work
    already enqueued on the current stream."""
    side = _side_stream(stream)
    if side is not None:
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            return decompress(c, out, err, None)
    if out is None:
        out = empty_output(c)
    check_out(out, c.n, c.dtype)
    zx_decode(c.container(), out, err, stream)
    return out


def decompress_batch(cs: Sequence[Compressed], outs: Optional[List[torch.Tensor]] = None,
                     err: Optional[torch.Tensor] = None, stream=None):
    """Decode up to 16 tensors (e.g. one transformer layer) with one kernel launch
    (stream ordering as `decompress`)."""
    side = _side_stream(stream)
    if side is not None:
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            return decompress_batch(cs, outs, err, None)
    if outs is None:
        outs = [empty_output(c) for c in cs]
    if len(outs) != len(cs):
        raise ValueError("one output per container")
    for i, (c, o) in enumerate(zip(cs, outs)):
        check_out(o, c.n, c.dtype, f"outs[{i}]")
    zx_decode_block_batch([c.container() for c in cs], outs, err, stream)
    return outs


# ----------------------------------------------------------------- dominant-range codec

ZF_BLOCK = 2048


@dataclass
class ZfCompressed:
    """A tensor in the dominant-range layout (device tensors)."""
    dtype: int
    n: int
    shape: tuple
    nrecords: int
    lb: torch.Tensor         # uint8 [nblocks]
    planes: torch.Tensor     # uint8 [nblocks, 3, 256]
    rec_off: torch.Tensor    # int64 [nblocks + 1]
    records: torch.Tensor    # int16 [max(nrecords, 1)]
    signmant: torch.Tensor   # uint8
    fp8_scale: Optional[float] = None

    def container(self) -> zx_zf_container:
        return zx_zf_container(self.dtype, 0, self.n, self.nrecords, self.lb.data_ptr(), self.planes.data_ptr(),
                               self.rec_off.data_ptr(), self.records.data_ptr(), self.signmant.data_ptr())

    def nbytes(self) -> int:
        """All container bytes: the arrays (records counted as stored) plus a 64-byte header."""
        return int(64 + self.lb.numel() + self.planes.numel() + self.rec_off.numel() * 8 + 2 * self.nrecords
                   + self.signmant.numel())

    def raw_bytes(self) -> int:
        return self.n * (2 if self.dtype == BF16 else 1)


def compress_zf(x: torch.Tensor, fp8_scale: Optional[float] = None, stream=None) -> ZfCompressed:
    """Encode a device tensor with the dominant-range codec: block parameters and
    record offsets, one 8-byte read of the record total, then planes and records.
    Everything runs on `stream` (a torch stream; default the current one), after the
    work already enqueued on the current stream (the producer of `x`) when it is
    another one."""
    side = _side_stream(stream)
    if side is not None:
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            return compress_zf(x, fp8_scale, None)
    dtype, flat = _as_bits(x)
    if dtype == E8M0:
        raise TypeError("the dominant-range codec takes BF16 and FP8 E4M3FN tensors")
    if not flat.is_cuda:
        raise ValueError("compress_zf expects a device tensor")
    flat = flat.contiguous()
    dev = flat.device
    n = flat.numel()
    nb = (n + ZF_BLOCK - 1) // ZF_BLOCK
    L = lib()
    ws = torch.empty(max(int(L.zx_zf_scan_workspace_bytes(n)), 16), dtype=torch.uint8, device=dev)
    lb = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    rec_off = torch.empty(nb + 1, dtype=torch.int64, device=dev)
    total = torch.empty(1, dtype=torch.int64, device=dev)
    s = _stream(None)
    _check("zx_zf_encode_size", L.zx_zf_encode_size(dtype, _ptr(flat), n, _ptr(lb), _ptr(rec_off), _ptr(ws), ws.numel(),
                                                    _ptr(total), s))
    planes = torch.empty((max(nb, 1), 3, 256), dtype=torch.uint8, device=dev)
    signmant = torch.empty(max(n if dtype == BF16 else (n + 1) // 2, 1), dtype=torch.uint8, device=dev)
    nrec = int(total.item())
    records = torch.empty(max(nrec, 1), dtype=torch.int16, device=dev)
    _check("zx_zf_encode", L.zx_zf_encode(dtype, _ptr(flat), n, _ptr(lb), _ptr(rec_off), _ptr(ws), nrec, _ptr(planes),
                                          _ptr(records), _ptr(signmant), s))
    return ZfCompressed(dtype=dtype, n=n, shape=tuple(x.shape), nrecords=nrec, lb=lb[:nb], planes=planes[:nb],
                        rec_off=rec_off, records=records, signmant=signmant[:n if dtype == BF16 else (n + 1) // 2],
                        fp8_scale=fp8_scale)


def decompress_zf(c: ZfCompressed, out: Optional[torch.Tensor] = None, err: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """Decode a dominant-range container (stream ordering as `decompress`)."""
    side = _side_stream(stream)
    if side is not None:
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            return decompress_zf(c, out, err, None)
    if out is None:
        tdt = torch.bfloat16 if c.dtype == BF16 else torch.float8_e4m3fn
        out = torch.empty(c.shape, dtype=tdt, device=c.signmant.device)
    check_out(out, c.n, c.dtype)
    cont = c.container()
    _check("zx_zf_decode", lib().zx_zf_decode(C.byref(cont), _ptr(out), _ptr(err), _stream(stream)))
    return out
