"""Lossless canonical-Huffman exponent coding of BF16/FP8 tensors on AMD MI355X.

The compute path is the HIP library libzx.so (C ABI in include/zx.h); the module
`zx` is its ctypes binding.
"""
from .zx import (  # noqa: F401
    BF16, FP8_E4M3FN, E8M0, BLOCK_ELEMS, Compressed, ZxError, compress, decompress, decompress_batch,
    empty_output, lib, zx_build_codebook, zx_build_decode_table, zx_decode, zx_decode_block_batch,
    zx_decode_table_bytes, zx_encode, zx_encode_coded, zx_encode_size, zx_encode_plan, zx_histogram, zx_stream_words, zx_container,
    alphabet, nblocks_of, check_out,
    ZF_BLOCK, ZfCompressed, compress_zf, decompress_zf, SharedCodebook, build_shared_codebook,
)
from .kvslots import KVSlotPool  # noqa: F401,E402
from .pipeline import LayerPipeline  # noqa: F401,E402
