"""Host-only checks of the C-ABI library: it loads, exports every entry point that
include/zx.h declares, and rejects bad arguments before touching a GPU."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zx.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zx_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def zx():
    import lossless_float_compression_amd as m
    return m


def test_header_lists_the_api():
    names = declared_functions()
    for f in ("zx_histogram", "zx_build_codebook", "zx_encode_size", "zx_encode", "zx_build_decode_table",
              "zx_decode", "zx_decode_block_batch", "zx_decode_block_batch_wg", "zx_stream_words", "zx_status_string",
              "zx_version"):
        assert f in names


def test_library_exports_every_declared_symbol(zx):
    lib = zx.lib()
    for f in declared_functions():
        assert hasattr(lib, f), f
    assert b"container v1" in lib.zx_version()


def test_stream_words_rule(zx):
    # round_up(ceil(bits/32), 4) + 260 (one segment's rows, 256 + 2 words, and a
    # multiple of four: a decoder reads a segment's rows from any start unchecked)
    for bits, want in [(0, 260), (1, 264), (32, 264), (128, 264), (129, 268), (1000, 292)]:
        assert zx.zx_stream_words(bits) == want


def test_status_strings(zx):
    lib = zx.lib()
    for s in range(8):
        assert lib.zx_status_string(s)
    assert lib.zx_status_string(7) != lib.zx_status_string(99)


def test_argument_errors_return_before_any_launch(zx):
    lib = zx.lib()
    P = C.c_void_p
    # unknown dtype
    assert lib.zx_histogram(7, None, 0, P(16), None, None) == 2
    # no output at all
    assert lib.zx_histogram(0, None, 0, None, None, None) == 1
    # misaligned pointer
    assert lib.zx_histogram(0, P(0x1001), 10, P(0x2000), None, None) == 1
    # tensor scope limited to n < 2^32
    assert lib.zx_histogram(0, P(0x1000), 1 << 32, P(0x2000), None, None) == 1
    # max_len below log2(alphabet) or above 32
    assert lib.zx_build_codebook(0, P(0x1000), 1, 7, P(0x2000), P(0x3000), None) == 3
    assert lib.zx_build_codebook(1, P(0x1000), 1, 3, P(0x2000), P(0x3000), None) == 3
    assert lib.zx_build_codebook(0, P(0x1000), 1, 33, P(0x2000), P(0x3000), None) == 3
    # decode: null container, too many tensors in a batch
    assert lib.zx_decode(None, P(0x1000), None, None) == 1
    arr = (zx.zx.zx_container * 17)()
    outs = (C.c_void_p * 17)()
    assert lib.zx_decode_block_batch(arr, outs, 17, None, None) == 1
    # per-tensor container without its decode table
    c = zx.zx.zx_container()
    c.dtype, c.per_block, c.n, c.nsegs, c.total_bits, c.stream_words = 0, 0, 10, 1, 20, 264
    for f in ("lengths", "degenerate", "signmant", "stream", "block_bitoff", "block_seg", "seg_desc", "gaps"):
        setattr(c, f, 0x10000)
    c.dtab = None
    assert lib.zx_decode(C.byref(c), P(0x20000), None, None) == 1
    # stream length must follow the padding rule
    c.dtab = 0x30000
    c.stream_words = 5
    assert lib.zx_decode(C.byref(c), P(0x20000), None, None) == 1
    # the encode plan: dtype, length limit, missing workspace, n >= 2^32, misaligned host word
    ok = [P(0x1000 * (k + 1)) for k in range(8)]   # in, block_hist, tensor_hist, lengths, degenerate, bitoff, seg, totals
    def plan(dtype=0, n=10, max_len=32, bufs=ok, host=None, codes=None):
        return lib.zx_encode_plan(dtype, bufs[0], n, max_len, bufs[1], bufs[2], bufs[3], bufs[4], bufs[5], bufs[6],
                                  bufs[7], host, 0, None, codes, None, None)
    assert plan(dtype=5) == 2
    assert plan(max_len=7) == 3 and plan(dtype=1, max_len=3) == 3 and plan(max_len=33) == 3
    assert plan(bufs=ok[:1] + [None] + ok[2:]) == 1
    assert plan(n=1 << 32) == 1
    assert plan(host=P(0x5004)) == 1
    assert plan(codes=P(0x6002)) == 1          # the codes must be u32-aligned
    # zx_encode_coded: the codes are required and u32-aligned
    def coded(codes):
        return lib.zx_encode_coded(0, P(0x1000), 10, P(0x2000), codes, P(0x3000), P(0x4000), P(0x5000), 20, 1,
                                   P(0x6000), P(0x7000), P(0x8000), P(0x9000), None, None)
    assert coded(None) == 1 and coded(P(0xA002)) == 1
    # the K/V append without allocation takes at most ZX_KV_NOALLOC_MAX_BLOCKS blocks
    pool = zx.zx.zx_kv_pool()
    assert zx.zx.KV_NOALLOC_MAX_BLOCKS == 1024
    assert "#define ZX_KV_NOALLOC_MAX_BLOCKS 1024u" in open(HEADER).read()
    assert lib.zx_kv_encode_slots_noalloc(C.byref(pool), P(0x1000), 1025, P(0x2000), 32, P(0x3000), None, None) == 7


def test_element_type_codes_agree():
    """The element-type enum of include/zx.h, the binding's constants and the oracle's
    are one numbering (BF16 0, FP8 E4M3FN 1, E8M0 block scales 2)."""
    import oracle
    import lossless_float_compression_amd as zx
    text = open(HEADER).read()
    enum = dict((k, int(v)) for k, v in re.findall(r"\b(ZX_BF16|ZX_FP8_E4M3FN|ZX_E8M0)\s*=\s*(\d+)", text))
    assert enum == {"ZX_BF16": 0, "ZX_FP8_E4M3FN": 1, "ZX_E8M0": 2}
    assert (zx.BF16, zx.FP8_E4M3FN, zx.E8M0) == (0, 1, 2)
    assert (oracle.BF16, oracle.FP8, oracle.E8M0) == (0, 1, 2)
    src = open(os.path.join(ROOT, "oracle", "zx_oracle.c")).read()
    assert re.search(r"#define ZXO_E8M0 2\b", src) and re.search(r"#define ZXO_FP8 1\b", src)
    from lossless_float_compression_amd.zx import alphabet
    assert alphabet(zx.E8M0) == 256 and alphabet(zx.BF16) == 256 and alphabet(zx.FP8_E4M3FN) == 16
