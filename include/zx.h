/*
 * zx.h -- C ABI of libzx: lossless canonical-Huffman coding of the exponent field
 * of BF16 and FP8-E4M3FN tensors on AMD MI355X (gfx950).
 *
 * Method (from the pages this library follows):
 *   - each float is split into its exponent field and the raw sign+mantissa bits;
 *     only the exponent is entropy coded, with Huffman coding
 *     (Intel paper summary "Lossless Compression of Neural Network Components:
 *      Weights, Checkpoints, and K/V Caches in Low-Precision Formats", sections
 *      方法论 / 方法详解 and the English abstract);
 *   - the Huffman tree comes from the exponent distribution; coded exponents are
 *     tightly bit-packed into one byte array (EncodedExponent) and sign+mantissa go
 *     into a separate byte array (PackedSignMantissa)
 *     (DFloat11 article "70% Size, 100% Accuracy ...", section 方法介绍, Fig. 2);
 *   - a tensor is coded in fixed-size blocks (Intel summary, section 实验设计);
 *   - the GPU decoder uses small lookup tables, a two-phase kernel whose auxiliary
 *     variables tell each thread where to read and write, and block-level decode
 *     (DFloat11 article, 方法介绍: three components);
 *   - decoding is lossless bit for bit (DFloat11 article, 实验结果).
 *
 * Container v1 (all multi-byte values little-endian; every array is device memory):
 *   block      65536 elements; block b = elements [65536 b, min(65536 (b+1), n)).
 *   codebook   one per tensor (per_block = 0) or one per block (per_block = 1);
 *              stored as code lengths only (lengths[cb][A], A = 256 for BF16,
 *              16 for FP8), 0 = symbol absent.  A scope with a single exponent
 *              value has all lengths 0 and degenerate[cb] = that value (0 bits per
 *              element); otherwise degenerate[cb] = 0xFFFF.
 *   lengths    Huffman lengths by two-queue merging (leaf queue in (count, symbol)
 *              order wins weight ties), redone with package-merge when deeper than
 *              max_len; canonical codes in (length, symbol) order (RFC 1951 3.2.2).
 *   signmant   BF16: byte i = sign<<7 | mantissa7 of element i (n bytes).
 *              FP8: nibble sign<<3 | mantissa3; element i in the low nibble of
 *              byte i/2 when i is even, high nibble when odd (ceil(n/2) bytes).
 *   stream     codes of all elements in order, MSB first; stream bit j is bit
 *              31 - j%32 of u32 word j/32; blocks follow each other with no gap;
 *              stream_words = round_up(ceil(total_bits/32), 4) + 260, zero padded
 *              (a decoder may read a segment's 258 words from any segment start).
 *   block_bitoff[nblocks+1]  u64 stream bit where block b starts; last = total_bits.
 *   block_seg[nblocks+1]     u32 first segment of block b; last = nsegs.
 *              A block's bits are cut into 128-bit chunks (block-relative),
 *              64 chunks per segment; a block has max(1, ceil(chunks/64)) segments.
 *   seg_desc[nsegs][2]       u32 {block, index (in the block) of the first element
 *              whose code starts at or after the segment's first bit}.
 *   gaps[nsegs][64]          u8 per chunk: offset of the first code starting in the
 *              chunk, 0xFF if none starts there or the chunk does not exist.
 *
 * Conventions for every entry point:
 *   - every pointer argument is a device pointer unless stated otherwise; the
 *     caller owns and allocates all memory (the library allocates nothing);
 *   - device pointers must be 16-byte aligned;
 *   - work is enqueued on `stream` and the call returns without synchronising;
 *   - argument errors are detected on the host and returned synchronously before
 *     anything is enqueued; data errors found on the device are written to the
 *     optional device word `err` (first error wins, 0 = no error; the caller
 *     clears it);
 *   - the library keeps no global mutable state; calls on different streams may
 *     run concurrently.
 */
#ifndef ZX_H
#define ZX_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZX_BLOCK_ELEMS 65536u
#define ZX_CHUNK_BITS 128u
#define ZX_SEG_CHUNKS 64u
#define ZX_MAX_CODE_LEN 32u
#define ZX_NO_DEGENERATE 0xFFFFu
#define ZX_NO_GAP 0xFFu

typedef enum {
    ZX_OK = 0,
    ZX_E_INVAL = 1,        /* bad argument (null, misaligned, size out of range)   */
    ZX_E_UNSUPPORTED = 2,  /* unknown dtype                                        */
    ZX_E_CODEBOOK = 3,     /* max_len infeasible, or data/codebook mismatch        */
    ZX_E_CORRUPT = 4,      /* container inconsistent (device-detected)             */
    ZX_E_HIP = 5,          /* a HIP launch failed                                  */
    ZX_E_NOSPACE = 6,      /* K/V slots: a block's code bits exceed its slot         */
    ZX_E_LIMIT = 7         /* request larger than the fixed scratch of an entry point
                              that allocates nothing                                 */
} zx_status;

typedef enum {
    ZX_BF16 = 0,           /* 8-bit exponent, alphabet 256 */
    ZX_FP8_E4M3FN = 1,     /* 4-bit exponent, alphabet 16  */
    ZX_E8M0 = 2            /* FP4 block scale factors (Intel summary, FP4 results; blog,
                              FP4 section): one byte per element that is a bare biased
                              exponent (value 2^(b-127)); the whole byte is coded, alphabet
                              256, and there is no sign/mantissa array (signmant may be
                              NULL).  Not supported by the K/V slot and dominant-range
                              entry points. */
} zx_dtype;

/* One compressed tensor (a host struct holding device pointers). */
typedef struct zx_container {
    int32_t dtype;                 /* zx_dtype                                          */
    int32_t per_block;             /* 0: one codebook, 1: one codebook per block        */
    uint64_t n;                    /* elements                                          */
    uint64_t nsegs;                /* block_seg[nblocks]                                */
    uint64_t total_bits;           /* block_bitoff[nblocks]                             */
    uint64_t stream_words;         /* length of `stream` in u32 words                   */
    const uint8_t *lengths;        /* [ncb][A]                                          */
    const uint16_t *degenerate;    /* [ncb]                                             */
    const uint8_t *signmant;       /* [n] (BF16) or [ceil(n/2)] (FP8)                   */
    const uint32_t *stream;        /* [stream_words]                                    */
    const uint64_t *block_bitoff;  /* [nblocks+1]                                       */
    const uint32_t *block_seg;     /* [nblocks+1]                                       */
    const uint32_t *seg_desc;      /* [nsegs][2]                                        */
    const uint8_t *gaps;           /* [nsegs][64]                                       */
    const uint32_t *dtab;          /* per_block = 0: decode table from
                                      zx_build_decode_table (required); per_block = 1:
                                      ignored (tables are built in the kernel)          */
} zx_container;

/* Exponent histogram (Intel summary, 方法论: the exponent distribution is what makes
 * it compressible; DFloat11, 方法介绍: the tree is built from that distribution).
 *   in           n elements: BF16 as u16 bits, FP8 as u8 bits.
 *   tensor_hist  u32[A] or NULL: counts over the whole tensor (requires n < 2^32).
 *   block_hist   u32[nblocks][A] or NULL: counts per 65536-element block.
 * At least one output must be given. */
zx_status zx_histogram(zx_dtype dtype, const void *in, uint64_t n,
                       uint32_t *tensor_hist, uint32_t *block_hist, hipStream_t stream);

/* Add the exponent counts of n elements to hist64 (u64[A], device, 8-byte aligned; the
 * caller clears it before the first tensor).  Summed over all linear weights of a
 * model it gives one model-wide codebook (DFloat11 article, 方法介绍: a Huffman tree
 * built from the exponents of the model's weights), which every tensor then uses
 * through zx_encode_size/zx_encode and one shared decode table. */
zx_status zx_histogram_accumulate(zx_dtype dtype, const void *in, uint64_t n, uint64_t *hist64,
                                  hipStream_t stream);

/* Code lengths for n_codebooks histograms (DFloat11, 方法介绍: Huffman tree from the
 * exponent distribution; the length limit and tie rules are container v1).
 *   hist        u32[n_codebooks][A]
 *   max_len     length limit, 8..32 for BF16, 4..32 for FP8 (else ZX_E_CODEBOOK)
 *   lengths     u8[n_codebooks][A] out;  degenerate u16[n_codebooks] out. */
zx_status zx_build_codebook(zx_dtype dtype, const uint32_t *hist, uint32_t n_codebooks,
                            uint32_t max_len, uint8_t *lengths, uint16_t *degenerate,
                            hipStream_t stream);

/* zx_build_codebook for u64 counts (histograms summed over many tensors; counts must
 * stay below 2^48). */
zx_status zx_build_codebook_u64(zx_dtype dtype, const uint64_t *hist, uint32_t n_codebooks,
                                uint32_t max_len, uint8_t *lengths, uint16_t *degenerate,
                                hipStream_t stream);

/* Block geometry for encoding: per-block stream bits and segment counts, scanned.
 * (Auxiliary read/write positions: DFloat11, 方法介绍, second component.)
 *   lengths      u8[ncb][A] (ncb = 1, or nblocks when per_block)
 *   block_hist   u32[nblocks][A] from zx_histogram, or NULL to read `in` instead
 *   block_bitoff u64[nblocks+1] out;  block_seg u32[nblocks+1] out
 *   totals       u64[2] out: {total_bits, nsegs}; the caller reads these back to
 *                size the stream (zx_stream_words) and the segment arrays. */
zx_status zx_encode_size(zx_dtype dtype, const void *in, uint64_t n, int per_block,
                         const uint8_t *lengths, const uint32_t *block_hist,
                         uint64_t *block_bitoff, uint32_t *block_seg, uint64_t *totals,
                         hipStream_t stream);

/* Everything a per-tensor-codebook encode needs before its outputs are sized:
 * histogram, codebook, block geometry and totals (zx_histogram + zx_build_codebook +
 * zx_encode_size in as few launches as the tensor allows), then the decode table.
 * Same tie rules and limits as those calls (DFloat11, 方法介绍: Huffman tree from the
 * exponent distribution, position data for the two-phase decode).
 *   block_hist    u32[max(nblocks,1)][A] device workspace
 *   tensor_hist   u32[A] device workspace
 *   lengths u8[A], degenerate u16[1], block_bitoff u64[nblocks+1], block_seg
 *                 u32[nblocks+1], totals u64[2] = {total_bits, nsegs}: device out
 *   totals_host   NULL, or 3 u64 of pinned host memory: {total_bits, nsegs, tag} are
 *                 written there, the tag last, as soon as the totals are known (before
 *                 the decode table), so a host thread may wait for the tag instead of
 *                 the stream
 *   dtab          NULL, or zx_decode_table_bytes() device bytes: the decode table
 *   codes         NULL, or u32[A] device out: the canonical code of each symbol
 *                 (right-aligned, 0 for a symbol without a code), for zx_encode_coded
 *   err           NULL, or a device word set to 0 (the error word zx_encode reports to)
 * Errors: ZX_E_UNSUPPORTED (dtype), ZX_E_CODEBOOK (max_len out of range), ZX_E_INVAL
 * (null or misaligned buffers, n >= 2^32), ZX_E_HIP (launch). */
zx_status zx_encode_plan(zx_dtype dtype, const void *in, uint64_t n, uint32_t max_len,
                         uint32_t *block_hist, uint32_t *tensor_hist, uint8_t *lengths,
                         uint16_t *degenerate, uint64_t *block_bitoff, uint32_t *block_seg,
                         uint64_t *totals, uint64_t *totals_host, uint64_t tag, uint32_t *dtab,
                         uint32_t *codes, uint32_t *err, hipStream_t stream);

/* Encode: split fields, bit-pack exponent codes, write gaps and segment table
 * (Intel summary, 方法论; DFloat11, 方法介绍 Fig. 2).
 *   in, n, per_block, lengths, degenerate   as above
 *   block_bitoff, block_seg                  from zx_encode_size
 *   total_bits, nsegs                        the totals read back
 *   signmant   u8 out [n] (BF16) or [ceil(n/2)] (FP8)
 *   stream     u32 out [zx_stream_words(total_bits)]: every word is written (the padding
 *              as zeros), whatever the buffer held, so it needs no clearing
 *   seg_desc   u32 out [nsegs][2];  gaps  u8 out [nsegs][64]
 *   err        optional: ZX_E_CODEBOOK if an element's exponent has no code. */
zx_status zx_encode(zx_dtype dtype, const void *in, uint64_t n, int per_block,
                    const uint8_t *lengths, const uint16_t *degenerate,
                    const uint64_t *block_bitoff, const uint32_t *block_seg,
                    uint64_t total_bits, uint64_t nsegs,
                    uint8_t *signmant, uint32_t *stream, uint32_t *seg_desc, uint8_t *gaps,
                    uint32_t *err, hipStream_t stream_);

/* zx_encode of a per-tensor codebook whose canonical codes are already known, as
 * zx_encode_plan writes them (the codes of RFC 1951, section 3.2.2, that zx_encode
 * would derive from the lengths in every workgroup).  Same outputs and errors as
 * zx_encode with per_block = 0.
 *   codes  u32[A] device: the canonical code of each symbol for these lengths (the
 *          caller guarantees they match; other codes make an undecodable stream);
 *          NULL or misaligned: ZX_E_INVAL. */
zx_status zx_encode_coded(zx_dtype dtype, const void *in, uint64_t n, const uint8_t *lengths,
                          const uint32_t *codes, const uint16_t *degenerate,
                          const uint64_t *block_bitoff, const uint32_t *block_seg,
                          uint64_t total_bits, uint64_t nsegs,
                          uint8_t *signmant, uint32_t *stream, uint32_t *seg_desc, uint8_t *gaps,
                          uint32_t *err, hipStream_t stream_);

/* Decode table for one codebook (per-tensor scope): the small lookup tables the
 * decoder keeps in LDS (DFloat11, 方法介绍: one large prefix-free table split into
 * compact tables that fit on-chip memory).
 *   lengths  u8[A];  dtab  out, zx_decode_table_bytes() bytes. */
zx_status zx_build_decode_table(zx_dtype dtype, const uint8_t *lengths, uint32_t *dtab,
                                hipStream_t stream);
size_t zx_decode_table_bytes(void);

/* Decode one container into out (n u16 BF16 bits, or n u8 FP8 bits): count pass,
 * wavefront prefix scan of output positions, fused write pass (DFloat11, 方法介绍:
 * two-phase kernel).  err: optional device word, ZX_E_CORRUPT on inconsistency;
 * out is never written outside [0, n). */
zx_status zx_decode(const zx_container *c, void *out, uint32_t *err, hipStream_t stream);

/* Decode `count` containers (host array) into outs[i] (host array of device
 * pointers) with one kernel launch: block-level decode of a group of tensors such
 * as one transformer layer (DFloat11, 方法介绍: decompression at transformer-block
 * level; 消融研究: its cost does not depend on batch size).  count <= 16. */
zx_status zx_decode_block_batch(const zx_container *cs, void *const *outs, uint32_t count,
                                uint32_t *err, hipStream_t stream);

/* zx_decode_block_batch with the per-tensor-codebook decode spread over at most
 * max_workgroups resident workgroups (0: all resident slots, as zx_decode_block_batch).  For
 * decoding the next layer while the current layer's GEMMs run on another stream
 * (DFloat11 article, 方法介绍: block-level decode into a temporary buffer): fewer
 * decode workgroups leave CUs, and their LDS, to the GEMM.  Containers with
 * per-block codebooks still take one workgroup per block. */
zx_status zx_decode_block_batch_wg(const zx_container *cs, void *const *outs, uint32_t count,
                                   uint32_t max_workgroups, uint32_t *err, hipStream_t stream);

/* ---- K/V slot pool --------------------------------------------------------------
 * A K/V cache kept in preallocated fixed-size slots, one 65536-element block per
 * slot: new blocks are compressed into their slots as they fill, and reused blocks
 * are decompressed on demand (ZipFloat page, section 4.2: slot-based K/V layout with
 * incremental compressed writes; section 3.3: K/V blocks written to fixed per-block
 * slots, without locks or a shared allocation counter).
 *
 * Every slot holds one block as a complete container with its own codebook
 * (per_block = 1, n = 65536) at fixed offsets in the pool's arrays; its code stream
 * has a fixed capacity of cap_words words, chosen by the caller (cap_words * 32 /
 * 65536 bits per element).  A block whose code bits exceed the capacity is not
 * stored (status ZX_E_NOSPACE for that block); the caller keeps it another way.
 * Slot s of each array starts at s times the stride that zx_kv_slot_sizes gives.
 * All pointers are caller-allocated device memory. */
typedef struct zx_kv_pool {
    int32_t dtype;             /* zx_dtype                                              */
    uint32_t n_slots;
    uint32_t cap_words;        /* stream capacity per slot: a multiple of 256, 256..8192 */
    uint32_t reserved_;        /* 0                                                     */
    uint8_t *signmant;         /* [n_slots][sm_bytes]                                   */
    uint32_t *stream;          /* [n_slots][stream_words]                               */
    uint8_t *gaps;             /* [n_slots][seg_stride][64]                             */
    uint32_t *seg_desc;        /* [n_slots][seg_stride][2]                              */
    uint8_t *lengths;          /* [n_slots][A]                                          */
    uint16_t *degenerate;      /* [n_slots]                                             */
    uint64_t *block_bitoff;    /* [n_slots][2]: {0, code bits of the slot's block}      */
    uint32_t *block_seg;       /* [n_slots][2]: {0, segments of the slot's block}       */
} zx_kv_pool;

typedef struct zx_kv_sizes {
    uint64_t sm_bytes;         /* 65536 (BF16) or 32768 (FP8)                           */
    uint64_t stream_words;     /* zx_stream_words(cap_words * 32): capacity + padding   */
    uint32_t max_segs;         /* segments a full slot uses: cap_words / 256            */
    uint32_t seg_stride;       /* max_segs rounded up to even (16-byte slot alignment)  */
    uint32_t alphabet;         /* 256 or 16                                             */
    uint32_t reserved_;
} zx_kv_sizes;

/* Per-slot strides for a pool of the given dtype and capacity (ZX_E_INVAL if
 * cap_words is not a multiple of 256 in 256..8192). */
zx_status zx_kv_slot_sizes(zx_dtype dtype, uint32_t cap_words, zx_kv_sizes *out);

/* Workspace bytes that zx_kv_encode_slots needs for nblk blocks. */
size_t zx_kv_workspace_bytes(zx_dtype dtype, uint32_t nblk);

/* Compress nblk full blocks into their slots with no host synchronisation: per-block
 * histograms, codebooks and sizes are computed on the device, and each block is
 * written into slot slot_ids[j] (ZipFloat page, 4.2: new K/V entries compressed
 * into preallocated slots as they are produced).
 *   src        nblk * 65536 elements (BF16 as u16 bits, FP8 as u8 bits), 16-byte aligned
 *   slot_ids   device u32[nblk], distinct slots < n_slots
 *   max_len    code length limit, as zx_build_codebook
 *   workspace  device, zx_kv_workspace_bytes(dtype, nblk) bytes, 16-byte aligned
 *   status     device u32[nblk] out: ZX_OK, ZX_E_NOSPACE (block left out, its slot
 *              marked empty), ZX_E_INVAL (slot id out of range) or ZX_E_CODEBOOK
 *   err        optional device word: the first non-zero block status
 * The slot contents equal what zx_encode writes for that block alone with
 * per_block = 1 (stream bits after the block's last code and up to the end of the
 * slot's stream are zero).  Blocks written by one call must go to distinct slots;
 * calls that write the same slot race. */
zx_status zx_kv_encode_slots(const zx_kv_pool *pool, const void *src, uint32_t nblk,
                             const uint32_t *slot_ids, uint32_t max_len, void *workspace,
                             size_t ws_bytes, uint32_t *status, uint32_t *err, hipStream_t stream);

/* zx_kv_encode_slots in one launch and without a workspace: each block's workgroup
 * builds its histogram, its code lengths (same tie rules and limits) and its size
 * from the block it holds, then encodes it into its slot (ZipFloat page, 4.2: online
 * compression of new entries into preallocated slots; DFloat11, 方法介绍: the tree from
 * the exponent distribution).  Same arguments, statuses and bytes as
 * zx_kv_encode_slots, with no workspace; ZX_E_CODEBOOK for max_len out of range. */
zx_status zx_kv_encode_slots_fused(const zx_kv_pool *pool, const void *src, uint32_t nblk,
                                   const uint32_t *slot_ids, uint32_t max_len, uint32_t *status,
                                   uint32_t *err, hipStream_t stream);

/* zx_kv_encode_slots for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same work with no
 * workspace argument.  The workspace is a file-scope device array of the library,
 * sized for ZX_KV_NOALLOC_MAX_BLOCKS blocks (1,325,088 bytes, held on each device the
 * library runs on until the process ends); nblk above that returns ZX_E_LIMIT before
 * anything is enqueued.  The entry point calls no hipMalloc, hipFree or other
 * allocating routine; on its first call on a device it looks up the array's address
 * there (hipGetSymbolAddress; ZX_E_HIP if that fails).  Every call on one device uses
 * the same array: calls that overlap in time on one device (other streams, other host
 * threads) race, and must be ordered by the caller.  Results equal zx_kv_encode_slots'
 * for the same arguments. */
#define ZX_KV_NOALLOC_MAX_BLOCKS 1024u
zx_status zx_kv_encode_slots_noalloc(const zx_kv_pool *pool, const void *src, uint32_t nblk,
                                     const uint32_t *slot_ids, uint32_t max_len, uint32_t *status,
                                     uint32_t *err, hipStream_t stream);

/* The container of slot `slot` (host struct of device pointers into the pool), for
 * zx_decode / zx_decode_block_batch: decoding reused K/V blocks on demand (ZipFloat
 * page, 4.2).  Its nsegs and total_bits are the slot's capacities; the block's own
 * segment count and bit length are read on the device from block_seg and
 * block_bitoff, so no host copy of them is needed. */
zx_status zx_kv_slot_container(const zx_kv_pool *pool, uint32_t slot, zx_container *out);

/* Decode the blocks in slots slot_ids[0..count) (device u32 array) into rows of
 * `out` (count * 65536 elements: row j holds slot slot_ids[j]) with one kernel
 * launch, one workgroup per slot: reused K/V blocks decompressed on demand (ZipFloat
 * page, 4.2).  A slot whose block did not fit holds no segments and leaves its row
 * unwritten; a slot id >= n_slots sets err to ZX_E_CORRUPT and leaves its row
 * unwritten. */
zx_status zx_kv_decode_slots(const zx_kv_pool *pool, const uint32_t *slot_ids, uint32_t count,
                             void *out, uint32_t *err, hipStream_t stream);

/* ---- dominant-range codec ---------------------------------------------------------
 * A second codec behind the same conventions (ZipFloat page, sections 3.1-3.3): blocks
 * of 2048 elements; per block, MD is the most frequent exponent (ties to the smallest)
 * and l_b = MD - 6; every exponent is remapped to v = e - l_b modulo the exponent
 * field; the low 3 bits of every v go into three 256-byte bit planes (plane p, byte k,
 * bit i = bit p of element 8k+i's v), and each element with v >= 8 gets a 2-byte record
 * (index << 5) | (v >> 3), in element order.  Sign and mantissa are stored as in
 * zx_container (n bytes BF16, ceil(n/2) nibble bytes FP8).  No entropy coding: every
 * element encodes and decodes on its own. */
typedef struct zx_zf_container {
    int32_t dtype;             /* zx_dtype                                            */
    int32_t reserved_;
    uint64_t n;                /* elements                                            */
    uint64_t nrecords;         /* rec_off[nblocks]                                    */
    const uint8_t *lb;         /* [nblocks], nblocks = ceil(n / 2048)                 */
    const uint8_t *planes;     /* [nblocks][3][256]                                   */
    const uint64_t *rec_off;   /* [nblocks + 1] exclusive prefix of records per block */
    const uint16_t *records;   /* [nrecords]                                          */
    const uint8_t *signmant;   /* as zx_container                                     */
} zx_zf_container;

/* Workspace bytes zx_zf_encode_size and zx_zf_encode need for n elements. */
size_t zx_zf_scan_workspace_bytes(uint64_t n);

/* Per-block l_b and record offsets, and the record total the caller reads back to size
 * the record array (ZipFloat page, 3.2: MD and l_b = MD - 6; 3.3: the records).
 *   in        n elements (BF16 u16 bits / FP8 u8 bits), 16-byte aligned
 *   lb        out u8[nblocks];  rec_off  out u64[nblocks+1] (finished by zx_zf_encode)
 *   workspace device, zx_zf_scan_workspace_bytes(n) bytes, kept for zx_zf_encode
 *   total     out u64[1] (device): the number of records */
zx_status zx_zf_encode_size(zx_dtype dtype, const void *in, uint64_t n, uint8_t *lb, uint64_t *rec_off,
                            void *workspace, size_t ws_bytes, uint64_t *total, hipStream_t stream);

/* Planes, records and sign/mantissa bytes; turns rec_off into the exclusive offsets.
 *   planes  out u8[nblocks][3][256];  records  out u16[total_records];  signmant out */
zx_status zx_zf_encode(zx_dtype dtype, const void *in, uint64_t n, const uint8_t *lb, uint64_t *rec_off,
                       const void *workspace, uint64_t total_records, uint8_t *planes, uint16_t *records,
                       uint8_t *signmant, hipStream_t stream);

/* Decode (ZipFloat page, 3.3: reverse bit-matrix unpacking, every block on its own).
 * err: optional device word, ZX_E_CORRUPT if a block's records run past nrecords. */
zx_status zx_zf_decode(const zx_zf_container *c, void *out, uint32_t *err, hipStream_t stream);

/* Stream length in u32 words for a given number of code bits. */
uint64_t zx_stream_words(uint64_t total_bits);
const char *zx_status_string(zx_status s);
const char *zx_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ZX_H */
