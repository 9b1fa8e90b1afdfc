"""ctypes marshalling for the C oracle in zx_oracle.c and zf_oracle.c (test
infrastructure only).

Every computation happens in the C files.  This module only converts between numpy
arrays and the C structures.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

BF16 = 0
FP8 = 1
E8M0 = 2     # FP4 block scale factors: bare 8-bit exponents, the whole byte is coded
BLOCK = 65536
CHUNK_BITS = 128
SEG_CHUNKS = 64

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "zx_oracle.c")
_SRC_ZF = os.path.join(_HERE, "zf_oracle.c")
ZF_BLOCK = 2048
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile zx_oracle.c and zf_oracle.c with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-shared", "-fPIC",
                               "-o", tmp, _SRC, _SRC_ZF])
        os.replace(tmp, _LIB)
    return _LIB


class _CContainer(C.Structure):
    _fields_ = [
        ("dtype", C.c_int32), ("per_block", C.c_int32),
        ("n", C.c_uint64), ("nblocks", C.c_uint64), ("ncb", C.c_uint64), ("nsegs", C.c_uint64),
        ("total_bits", C.c_uint64), ("stream_words", C.c_uint64), ("signmant_bytes", C.c_uint64),
        ("lengths", C.POINTER(C.c_uint8)), ("degenerate", C.POINTER(C.c_uint16)),
        ("signmant", C.POINTER(C.c_uint8)), ("stream", C.POINTER(C.c_uint32)),
        ("block_bitoff", C.POINTER(C.c_uint64)), ("block_seg", C.POINTER(C.c_uint32)),
        ("seg_desc", C.POINTER(C.c_uint32)), ("gaps", C.POINTER(C.c_uint8)),
    ]


class _ZfContainer(C.Structure):
    _fields_ = [
        ("dtype", C.c_int32), ("reserved_", C.c_int32),
        ("n", C.c_uint64), ("nblocks", C.c_uint64), ("nrecords", C.c_uint64), ("signmant_bytes", C.c_uint64),
        ("lb", C.POINTER(C.c_uint8)), ("planes", C.POINTER(C.c_uint8)), ("rec_off", C.POINTER(C.c_uint64)),
        ("records", C.POINTER(C.c_uint16)), ("signmant", C.POINTER(C.c_uint8)),
    ]


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = C.CDLL(_LIB)
        if lib.zxo_sizeof_container() != C.sizeof(_CContainer):
            raise RuntimeError("oracle struct layout mismatch; rebuild oracle")
        P = C.c_void_p
        lib.zxo_split.argtypes = [C.c_int, P, C.c_uint64, P, P]
        lib.zxo_histogram.argtypes = [P, C.c_uint64, C.c_uint32, P]
        lib.zxo_huffman_lengths.argtypes = [P, C.c_int, P]
        lib.zxo_package_merge.argtypes = [P, C.c_int, C.c_int, P]
        lib.zxo_code_lengths.argtypes = [P, C.c_int, C.c_int, P, P]
        lib.zxo_canonical_codes.argtypes = [P, C.c_int, P]
        lib.zxo_stream_words.argtypes = [C.c_uint64]
        lib.zxo_stream_words.restype = C.c_uint64
        lib.zxo_encode.argtypes = [C.c_int, P, C.c_uint64, C.c_int, C.c_int, C.POINTER(_CContainer)]
        lib.zxo_encode_with_lengths.argtypes = [C.c_int, P, C.c_uint64, P, C.c_uint16, C.POINTER(_CContainer)]
        lib.zxo_decode.argtypes = [C.POINTER(_CContainer), P]
        lib.zxo_decode_blocks.argtypes = [C.POINTER(_CContainer), C.c_uint64, C.c_uint64, P]
        lib.zxo_free.argtypes = [C.POINTER(_CContainer)]
        if lib.zfo_sizeof_container() != C.sizeof(_ZfContainer):
            raise RuntimeError("oracle struct layout mismatch; rebuild oracle")
        lib.zfo_mode.argtypes = [P, C.c_uint64, C.c_uint32]
        lib.zfo_mode.restype = C.c_uint32
        lib.zfo_encode.argtypes = [C.c_int, P, C.c_uint64, C.POINTER(_ZfContainer)]
        lib.zfo_decode.argtypes = [C.POINTER(_ZfContainer), P]
        lib.zfo_free.argtypes = [C.POINTER(_ZfContainer)]
        _lib = lib
    return _lib


def _alphabet(dtype: int) -> int:
    return 16 if dtype == FP8 else 256


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


@dataclass
class Container:
    """One compressed tensor in container v1 layout (all arrays are numpy)."""
    dtype: int
    per_block: int
    n: int
    lengths: np.ndarray        # uint8 [ncb, A]
    degenerate: np.ndarray     # uint16 [ncb]
    signmant: np.ndarray       # uint8 [n] or [ceil(n/2)]
    stream: np.ndarray         # uint32 [stream_words]
    block_bitoff: np.ndarray   # uint64 [nblocks+1]
    block_seg: np.ndarray      # uint32 [nblocks+1]
    seg_desc: np.ndarray       # uint32 [nsegs, 2]
    gaps: np.ndarray           # uint8 [nsegs, 64]
    extra: dict = field(default_factory=dict)

    @property
    def nblocks(self) -> int:
        return (self.n + BLOCK - 1) // BLOCK

    @property
    def nsegs(self) -> int:
        return int(self.block_seg[-1])

    @property
    def total_bits(self) -> int:
        return int(self.block_bitoff[-1])

    def nbytes(self) -> int:
        """All container bytes: every array plus a 64-byte header."""
        return int(64 + self.lengths.nbytes + self.degenerate.nbytes + self.signmant.nbytes
                   + self.stream.nbytes + self.block_bitoff.nbytes + self.block_seg.nbytes
                   + self.seg_desc.nbytes + self.gaps.nbytes)


def split(dtype: int, x: np.ndarray):
    lib = load()
    x = np.ascontiguousarray(x)
    n = x.size
    exps = np.empty(max(n, 1), np.uint8)
    nsm = n if dtype == BF16 else (n + 1) // 2 if dtype == FP8 else 0
    sm = np.empty(max(nsm, 1), np.uint8)
    lib.zxo_split(dtype, _p(x), n, _p(exps), _p(sm))
    return exps[:n], sm[:nsm]


def histogram(exps: np.ndarray, alphabet: int) -> np.ndarray:
    lib = load()
    exps = np.ascontiguousarray(exps, dtype=np.uint8)
    h = np.zeros(alphabet, np.uint64)
    lib.zxo_histogram(_p(exps), exps.size, alphabet, _p(h))
    return h


def huffman_lengths(hist) -> np.ndarray:
    lib = load()
    h = np.ascontiguousarray(hist, dtype=np.uint64)
    ln = np.zeros(h.size, np.uint8)
    lib.zxo_huffman_lengths(_p(h), h.size, _p(ln))
    return ln


def package_merge(hist, L: int) -> np.ndarray:
    lib = load()
    h = np.ascontiguousarray(hist, dtype=np.uint64)
    ln = np.zeros(h.size, np.uint8)
    if lib.zxo_package_merge(_p(h), h.size, int(L), _p(ln)) < 0:
        raise ValueError("package-merge infeasible")
    return ln


def code_lengths(hist, max_len: int):
    """(lengths uint8[A], degenerate symbol or 0xFFFF)."""
    lib = load()
    h = np.ascontiguousarray(hist, dtype=np.uint64)
    ln = np.zeros(h.size, np.uint8)
    d = np.zeros(1, np.uint16)
    if lib.zxo_code_lengths(_p(h), h.size, int(max_len), _p(ln), _p(d)) < 0:
        raise ValueError("length limit infeasible")
    return ln, int(d[0])


def canonical_codes(lengths) -> np.ndarray:
    lib = load()
    ln = np.ascontiguousarray(lengths, dtype=np.uint8)
    code = np.zeros(ln.size, np.uint32)
    lib.zxo_canonical_codes(_p(ln), ln.size, _p(code))
    return code


def stream_words(total_bits: int) -> int:
    return int(load().zxo_stream_words(int(total_bits)))


def _arr(ptr, count, dtype):
    if count == 0:
        return np.zeros(0, dtype)
    return np.ctypeslib.as_array(ptr, shape=(int(count),)).copy().astype(dtype, copy=False)


def encode(dtype: int, x: np.ndarray, per_block: bool = False, max_len: int = 32, lengths=None,
           degenerate: int = 0xFFFF) -> Container:
    """Encode raw bits (uint16 for BF16, uint8 for FP8) into a container; with
    `lengths` (and `degenerate`), use that codebook for the whole tensor."""
    lib = load()
    x = np.ascontiguousarray(x).reshape(-1)
    want = np.uint16 if dtype == BF16 else np.uint8
    if x.dtype != want:
        x = x.view(want)
    cc = _CContainer()
    if lengths is not None:
        ln = np.ascontiguousarray(lengths, dtype=np.uint8)
        rc = lib.zxo_encode_with_lengths(dtype, _p(x) if x.size else None, x.size, _p(ln), int(degenerate), C.byref(cc))
    else:
        rc = lib.zxo_encode(dtype, _p(x) if x.size else None, x.size, int(per_block), int(max_len), C.byref(cc))
    if rc != 0:
        raise ValueError(f"oracle encode failed rc={rc}")
    try:
        A = _alphabet(dtype)
        ncb = int(cc.ncb)
        c = Container(
            dtype=dtype, per_block=int(per_block), n=int(cc.n),
            lengths=_arr(cc.lengths, ncb * A, np.uint8).reshape(ncb, A),
            degenerate=_arr(cc.degenerate, ncb, np.uint16),
            signmant=_arr(cc.signmant, cc.signmant_bytes, np.uint8),
            stream=_arr(cc.stream, cc.stream_words, np.uint32),
            block_bitoff=_arr(cc.block_bitoff, cc.nblocks + 1, np.uint64),
            block_seg=_arr(cc.block_seg, cc.nblocks + 1, np.uint32),
            seg_desc=_arr(cc.seg_desc, 2 * cc.nsegs, np.uint32).reshape(-1, 2),
            gaps=_arr(cc.gaps, SEG_CHUNKS * cc.nsegs, np.uint8).reshape(-1, SEG_CHUNKS),
        )
    finally:
        lib.zxo_free(C.byref(cc))
    return c


def _marshal(c: Container):
    """(C container, arrays kept alive for its pointers, output array) for a decode."""
    lib = load()
    A = _alphabet(c.dtype)
    keep = [np.ascontiguousarray(a) for a in (c.lengths.reshape(-1), c.degenerate, c.signmant, c.stream,
                                               c.block_bitoff, c.block_seg, c.seg_desc.reshape(-1),
                                               c.gaps.reshape(-1))]
    ln, dg, sm, st, bo, bs, sd, gp = keep
    assert ln.dtype == np.uint8 and dg.dtype == np.uint16 and sm.dtype == np.uint8 and st.dtype == np.uint32
    assert bo.dtype == np.uint64 and bs.dtype == np.uint32 and sd.dtype == np.uint32 and gp.dtype == np.uint8
    nb = (c.n + BLOCK - 1) // BLOCK
    cc = _CContainer()
    cc.dtype = c.dtype
    cc.per_block = int(c.per_block)
    cc.n = c.n
    cc.nblocks = nb
    cc.ncb = ln.size // A
    cc.nsegs = int(bs[-1])
    cc.total_bits = int(bo[-1])
    cc.stream_words = st.size
    cc.signmant_bytes = sm.size

    def ptr(a, t):
        if a.size == 0:
            a = np.zeros(1, a.dtype)
            keep.append(a)
        return a.ctypes.data_as(C.POINTER(t))

    cc.lengths = ptr(ln, C.c_uint8)
    cc.degenerate = ptr(dg, C.c_uint16)
    cc.signmant = ptr(sm, C.c_uint8)
    cc.stream = ptr(st, C.c_uint32)
    cc.block_bitoff = ptr(bo, C.c_uint64)
    cc.block_seg = ptr(bs, C.c_uint32)
    cc.seg_desc = ptr(sd, C.c_uint32)
    cc.gaps = ptr(gp, C.c_uint8)
    out = np.empty(max(c.n, 1), np.uint16 if c.dtype == BF16 else np.uint8)
    return lib, cc, keep, out


def decode(c: Container) -> np.ndarray:
    """Decode a container (from the oracle or from anywhere else); raises on any
    inconsistency the oracle's checks find."""
    lib, cc, keep, out = _marshal(c)
    rc = lib.zxo_decode(C.byref(cc), _p(out))
    if rc != 0:
        raise ValueError(f"oracle decode rejected the container rc={rc}")
    return out[: c.n]


def decode_blocks(c: Container, ranges) -> np.ndarray:
    """Decode the blocks of each (b0, b1) range in `ranges` into one output array
    (elements of blocks outside the ranges are left unset); raises on any
    inconsistency in those blocks."""
    lib, cc, keep, out = _marshal(c)
    for b0, b1 in ranges:
        rc = lib.zxo_decode_blocks(C.byref(cc), int(b0), int(b1), _p(out))
        if rc != 0:
            raise ValueError(f"oracle decode rejected blocks [{b0}, {b1}) rc={rc}")
    return out[: c.n]


def decode_threaded(c: Container, threads: int) -> np.ndarray:
    """The same decode with the blocks split into `threads` contiguous ranges, each
    decoded on its own host thread (the calls release the interpreter lock)."""
    import threading
    lib, cc, keep, out = _marshal(c)
    nb = c.nblocks
    bounds = [nb * t // threads for t in range(threads + 1)]
    rcs = [0] * threads

    def run(t):
        rcs[t] = lib.zxo_decode_blocks(C.byref(cc), bounds[t], bounds[t + 1], _p(out))

    ths = [threading.Thread(target=run, args=(t,)) for t in range(threads)]
    for th in ths:
        th.start()
    for th in ths:
        th.join()
    if any(rcs):
        raise ValueError(f"oracle decode rejected the container rc={rcs}")
    return out[: c.n]


# ---------------------------------------------------------------- dominant-range codec

@dataclass
class ZfContainer:
    """One tensor in the dominant-range layout (2048-element blocks; numpy arrays)."""
    dtype: int
    n: int
    lb: np.ndarray          # uint8 [nblocks]
    planes: np.ndarray      # uint8 [nblocks, 3, 256]
    rec_off: np.ndarray     # uint64 [nblocks + 1]
    records: np.ndarray     # uint16 [nrecords]
    signmant: np.ndarray    # uint8 [n] or [ceil(n/2)]

    @property
    def nblocks(self) -> int:
        return (self.n + ZF_BLOCK - 1) // ZF_BLOCK

    def nbytes(self) -> int:
        """All container bytes: every array plus a 64-byte header."""
        return int(64 + self.lb.nbytes + self.planes.nbytes + self.rec_off.nbytes + self.records.nbytes
                   + self.signmant.nbytes)


def zf_mode(exps: np.ndarray, alphabet: int) -> int:
    e = np.ascontiguousarray(exps, dtype=np.uint8)
    return int(load().zfo_mode(_p(e), e.size, alphabet))


def zf_encode(dtype: int, x: np.ndarray) -> ZfContainer:
    """Encode raw bits (uint16 for BF16, uint8 for FP8) with the dominant-range codec."""
    lib = load()
    x = np.ascontiguousarray(x).reshape(-1)
    want = np.uint16 if dtype == BF16 else np.uint8
    if x.dtype != want:
        x = x.view(want)
    cc = _ZfContainer()
    rc = lib.zfo_encode(dtype, _p(x) if x.size else None, x.size, C.byref(cc))
    if rc != 0:
        raise ValueError(f"oracle zf encode failed rc={rc}")
    try:
        nb = int(cc.nblocks)
        c = ZfContainer(dtype=dtype, n=int(cc.n), lb=_arr(cc.lb, nb, np.uint8),
                        planes=_arr(cc.planes, nb * 3 * 256, np.uint8).reshape(nb, 3, 256),
                        rec_off=_arr(cc.rec_off, nb + 1, np.uint64), records=_arr(cc.records, cc.nrecords, np.uint16),
                        signmant=_arr(cc.signmant, cc.signmant_bytes, np.uint8))
    finally:
        lib.zfo_free(C.byref(cc))
    return c


def zf_decode(c: ZfContainer) -> np.ndarray:
    lib = load()
    # converted arrays are bound here, so that every pointer below stays valid until
    # the call returns
    keep = [np.ascontiguousarray(c.lb, dtype=np.uint8), np.ascontiguousarray(c.planes, dtype=np.uint8),
            np.ascontiguousarray(c.rec_off, dtype=np.uint64), np.ascontiguousarray(c.records, dtype=np.uint16),
            np.ascontiguousarray(c.signmant, dtype=np.uint8)]
    cc = _ZfContainer()
    cc.dtype, cc.n, cc.nblocks, cc.nrecords = c.dtype, c.n, c.nblocks, keep[3].size
    cc.signmant_bytes = keep[4].size
    cc.lb = keep[0].ctypes.data_as(C.POINTER(C.c_uint8))
    cc.planes = keep[1].ctypes.data_as(C.POINTER(C.c_uint8))
    cc.rec_off = keep[2].ctypes.data_as(C.POINTER(C.c_uint64))
    cc.records = keep[3].ctypes.data_as(C.POINTER(C.c_uint16))
    cc.signmant = keep[4].ctypes.data_as(C.POINTER(C.c_uint8))
    out = np.empty(max(c.n, 1), np.uint16 if c.dtype == BF16 else np.uint8)
    rc = lib.zfo_decode(C.byref(cc), _p(out))
    if rc != 0:
        raise ValueError(f"oracle zf decode failed rc={rc}")
    return out[:c.n]
