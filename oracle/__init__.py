"""CPU oracle for canonical-Huffman exponent coding (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg import
this package.  The library's product path never does.  The oracle shares no code
with the HIP library.  The C sources `zx_oracle.c` (Huffman codec) and `zf_oracle.c` (dominant-range
codec) hold every step of the methods.
This module only marshals numpy arrays in and out of it through ctypes.
"""
from .oracle import (  # noqa: F401
    BF16, FP8, E8M0, BLOCK, CHUNK_BITS, SEG_CHUNKS, Container, build, load,
    split, histogram, huffman_lengths, package_merge, code_lengths,
    canonical_codes, stream_words, encode, decode, decode_blocks, decode_threaded,
    ZF_BLOCK, ZfContainer, zf_mode, zf_encode, zf_decode,
)
