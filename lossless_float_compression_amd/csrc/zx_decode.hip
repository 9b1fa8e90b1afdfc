// zx_decode.hip -- massively parallel decode of container v1 back to BF16 / FP8.
//
// Prior art on the DFloat11 article (方法介绍, three components) is a kernel with
// (1) compact lookup tables in on-chip memory, (2) two phases coordinated by small
// auxiliary variables that tell each thread where to read and write, and (3)
// decode of a whole transformer block per call.  The gfx950 design here:
//   * one wavefront decodes one segment: 64 chunks of 128 stream bits, lane l owns
//     chunk l and starts at the chunk's stored gap (the first code starting in it);
//   * count pass: a lane refreshes a 32-bit window from its LDS word rows with one
//     funnel shift, then takes three lookups from it; each lookup indexes a
//     2048-entry LDS table with the next 11 bits (one 8-byte entry, one 64-bit LDS
//     read) and yields up to four symbols.  The entries stay in registers.  A
//     running "256 - position" value gives the funnel-shift amount and the word row
//     directly, and accumulates the code count;
//   * a wavefront prefix scan of the per-lane counts, plus the segment's stored first
//     element, gives each lane its output offset;
//   * replay: the register entries are dropped into a wavefront-private LDS stage in
//     output order; the write pass then fuses the staged exponents with the
//     sign/mantissa bytes, which were requested before the decode started, into
//     16-byte coalesced stores.
// Per-tensor codebooks load a prepared table; per-block codebooks (one workgroup
// per block) build theirs in LDS from the block's code lengths.
#include <cstring>

#include "zx_common.h"

namespace zxk {

constexpr int kDecWaves = 8;                  // wavefronts per decode workgroup (at most)
constexpr int kDecThreads = kDecWaves * kWave;
constexpr int kMinDecWaves = 6;               // a per-tensor launch may use 6..8 (see the host)
constexpr int kMaxBatch = 16;

// Per-wavefront LDS: the lanes' stream words and the exponent stage.
constexpr uint32_t kSlots = 7;                 // word slots per lane
// Slot 6 is only ever read as the upper word of a zero-bit shift (a position of
// exactly kPosBase), so it holds the lanes' gap bytes instead; the word after the
// slots holds the next segment's first gap.
constexpr uint32_t kGapSlot = 6;
constexpr uint32_t kSegWords = kSlots * kWave + 4;
constexpr uint32_t kStageBytes = 3616;         // one byte per output position, 16-byte multiple
// A segment whose exponents do not fit the stage at once (mean code length under
// about 2.3 bits) is written in rounds of kRoundElems output positions.
constexpr uint32_t kRoundElems = 3584;
// Register path: up to kRounds rounds of three lookups per lane (kLowRounds in the
// low-entropy mode); the symbol counts of the lookups are kept one byte each, four to
// a register.
constexpr int kRounds = 7;
constexpr int kWriteBatch = 7;                 // write-pass pieces per lane whose loads go out together (at most)
// pieces per lane in one batch: 7 x 64 x 8 BF16 elements cover a stage; FP8 pieces hold
// 16 elements, so 4 x 64 x 16 do (and fewer registers are live in the write pass)
template <int DT> constexpr int write_batch() { return DT == ZX_FP8_E4M3FN ? 4 : kWriteBatch; }
// Bit positions within a lane's rows: row r holds bits [32 r, 32 r + 32); row 1 is
// the word holding the chunk's first bit, so the chunk starts at kPosBase + b0.
constexpr uint32_t kPosBase = 32;
// A lane's position stays below kPosBase + 31 (block start within its word) + 128
// (chunk) + kMaxLen (a code started before the chunk end): the "256 - position" byte
// and the first-three-codes field summed into the byte above it never borrow.
static_assert(kPosBase + 31 + kChunkBits + kMaxLen < 256, "lane position must fit one byte");

struct DecTensor {
    const uint8_t *signmant;
    const uint32_t *stream;
    const uint64_t *block_bitoff;
    const uint32_t *block_seg;
    const uint32_t *seg_desc;
    const uint8_t *gaps;
    const uint8_t *lengths;
    const uint16_t *degenerate;
    const DTab *dtab;
    void *out;
    uint64_t n;
    uint64_t total_bits;
    uint64_t stream_words;
    uint32_t nsegs;
    uint32_t nblocks;
    uint32_t per_block;
    uint32_t wg_begin;
    uint32_t wg_count;
    uint32_t segs_per_wg;
};

// Slot-list decode: workgroup g decodes the one-block container in slot
// slot_ids[g] of a K/V slot pool.  t[0] then describes slot 0's container and the
// strides below give every other slot's arrays; workgroup g's output is row g.
struct DecSlots {
    const uint32_t *slot_ids;   // null: no slot list
    uint64_t sm_bytes;          // sign/mantissa bytes per slot
    uint64_t stream_words;      // stream words per slot
    uint64_t seg_stride;        // segment entries per slot
    uint64_t out_bytes;         // output bytes per row
    uint32_t alphabet;
    uint32_t n_slots;
};

struct DecBatch {
    DecTensor t[kMaxBatch];
    uint32_t count;
    DecSlots slots;
};

typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

// Lane index computed where it is used.  The segment loop runs each wavefront over
// many segments; if the lane index were a plain value the compiler would hoist every
// lane-derived address out of that loop and keep them all live across it, which
// costs more registers than recomputing them per segment.
__device__ __forceinline__ uint32_t lane_now()
{
    uint32_t r;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(r));
    return r;
}

// True if the predicate holds in any lane (the lane mask itself, not a ballot
// materialised through vector registers).
__device__ __forceinline__ bool any_lane(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }


__device__ __forceinline__ uint2 lds_pair(const uint2 *base, uint32_t byte_off)
{
    return *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint8_t *>(base) + byte_off);
}

// ---- stream words of the lanes' chunks --------------------------------------
//
// Lane l needs the six words w0(l) .. w0(l)+5 from the one holding its chunk's first
// bit: the chunk starts less than 32 bits into w0 and the lane never reads a window
// starting at or past the chunk end.  They are its rows 1..6; row r sits in slot
// 7 - r, i.e. at sw[(6 - r) * 64 + l], one column per lane so that every window read
// of the wavefront hits 64 distinct banks.  Row 0 is never stored: it is read only
// with a zero funnel shift, which takes the other word whole.

// 16 bytes of stream words per lane (the lane's rows 1..4, the previous lane's rows 5
// and 6) plus, in lanes 0 and 1, lane 63's rows 5 and 6 (the other lanes load a word
// they do not use).  W0 is at most the last code word, and the stream has
// kStreamPadWords zero words after it: every read is in bounds, and none needs a
// condition.
__device__ __forceinline__ void rows_load(const uint32_t *stream, uint64_t W0, uint32_t lane, u32x4_a4 &v,
                                          uint32_t &tail)
{
    v = *reinterpret_cast<const u32x4_a4 *>(stream + W0 + 4u * lane);
    tail = stream[W0 + 256u + (lane & 1u)];
}

__device__ __forceinline__ void rows_store(uint32_t *sw, uint32_t lane, const u32x4_a4 &v, uint32_t tail)
{
    sw[5 * 64 + lane] = v.x;
    sw[4 * 64 + lane] = v.y;
    sw[3 * 64 + lane] = v.z;
    sw[2 * 64 + lane] = v.w;
    if (lane > 0) {
        sw[1 * 64 + lane - 1] = v.x;
        sw[0 * 64 + lane - 1] = v.y;
    }
    if (lane < 2) sw[(1 - lane) * 64 + 63] = tail;
}

// The 32 stream bits starting at position p of this lane's rows, given q with low
// byte 256 - p.  For p in [32, 190] the slots read are this lane's; any p up to 223
// (a lane past its chunk end after a long code) still reads inside the LDS
// allocation, one slot below, which only idle lanes do.  Slot (q >> 5) & 7 holds the row with the
// window's first bit (or, when p is a multiple of 32, the row before it, which a
// zero funnel shift then drops), the next slot down holds the row after it, and the
// low five bits of q are the funnel shift.
// `col` is window_col(): the LDS address two slots below this lane's slot 0 column,
// kept opaque to the compiler so that both words come from one two-address LDS read
// with immediate offsets.
typedef __attribute__((address_space(3))) const uint32_t lds_cu32;

__device__ __forceinline__ uint32_t window(lds_cu32 *col, uint32_t q)
{
    lds_cu32 *w = col + (__builtin_amdgcn_ubfe(q, 5, 3) << 6);
    return __builtin_amdgcn_alignbit(w[64], w[0], q);
}

__device__ __forceinline__ lds_cu32 *window_col(uint32_t *sw, uint32_t lane)
{
    lds_cu32 *p = (lds_cu32 *)(sw + lane);
    uint32_t a = (uint32_t)(uintptr_t)p - 2u * 64u * 4u;
    asm volatile("" : "+v"(a));
    return (lds_cu32 *)(uintptr_t)a;
}

// Codes longer than the lookup window: canonical length limits, kept out of line.
__device__ __forceinline__ uint32_t slow_len(const DTab &tab, uint32_t v)
{
    uint32_t L = kLutBits + 1;
#pragma unroll 1
    while (L <= kMaxLen && (uint64_t)v >= tab.lim[L]) ++L;
    return L;
}

__device__ __forceinline__ uint32_t slow_sym(const DTab &tab, uint32_t v, uint32_t L)
{
    return tab.sym[(uint32_t)(tab.base[L] + (int32_t)(v >> (32 - L))) & 0xFFu];
}

// Length and stage form of the code at the front of window v.
__device__ __forceinline__ uint32_t one_code(const DTab &tab, uint32_t v, uint32_t &sym)
{
    const uint32_t x = v >> (32 - kLutBits);
    const uint32_t lo = tab.e[x].x;
    if (lo != 0) {
        sym = tab.e[x].y & 0xFFu;
        return (lo >> 24) & 0xFu;
    }
    const uint32_t L = slow_len(tab, v);
    sym = L <= kMaxLen ? slow_sym(tab, v, L) : 0u;
    return L;
}

// ---- write pass ---------------------------------------------------------------

// 8 BF16 or 16 FP8 elements per lane per piece: 8 bytes of sign/mantissa in and one
// 16-byte store out.
template <int DT>
struct Piece {
    static constexpr uint32_t kElems = DT == ZX_BF16 ? 8 : 16;
};

template <int DT>
__device__ __forceinline__ uint2 load_sm(const uint8_t *sm_block, uint32_t i)
{
    if constexpr (DT == ZX_E8M0) return make_uint2(0, 0);   // no sign/mantissa array
    return *reinterpret_cast<const uint2 *>(sm_block + (DT == ZX_BF16 ? i : i / 2));
}

// The element of [i_begin, i_end) this lane writes in one of the (at most two) cut
// pieces at the range ends, or ~0u: lane t (< P) takes element t of the head piece,
// lane P + t element t of the tail piece.
template <int DT>
__device__ __forceinline__ uint32_t cut_elem(uint32_t i_begin, uint32_t i_end)
{
    constexpr uint32_t P = Piece<DT>::kElems;
    if (i_begin >= i_end) return ~0u;
    const uint32_t lane = lane_now();
    const uint32_t q_head = i_begin / P;
    const uint32_t q_tail = (i_end - 1) / P;
    const bool head_cut = (i_begin % P) != 0 || (q_head == q_tail && (i_end % P) != 0);
    const bool tail_cut = (i_end % P) != 0 && q_tail != q_head;
    uint32_t ii = ~0u;
    if (lane < P && head_cut) ii = q_head * P + lane;
    if (lane >= P && lane < 2 * P && tail_cut) ii = q_tail * P + (lane - P);
    return (ii != ~0u && ii >= i_begin && ii < i_end) ? ii : ~0u;
}

template <int DT>
__device__ __forceinline__ uint32_t load_cut_sm(const uint8_t *sm_block, uint32_t ii)
{
    if constexpr (DT == ZX_E8M0) return 0u;
    return ii != ~0u ? (uint32_t)sm_block[DT == ZX_BF16 ? ii : ii / 2] : 0u;
}

// Sign/mantissa bytes of the first batch of whole pieces of [i_begin, i_end)
// (piece q = first + lane + 64 k) and of this lane's cut-piece element.  Every load
// is issued, and nothing else writes its register: a piece (or cut element) the
// lane does not have reads `dummy` instead, any 16 readable bytes (the stream, which
// has at least kStreamPadWords words).  (A default
// value written to the register would first wait for the previous segment's load
// into it, and so, with one counter for loads and stores, for all its stores.)
template <int DT>
__device__ __forceinline__ void prefetch_sm(const uint8_t *sm_block, uint32_t i_begin, uint32_t i_end,
                                            const uint8_t *dummy, uint2 (&smv)[kWriteBatch], uint32_t &smcut)
{
    if constexpr (DT == ZX_E8M0) {   // nothing to read: the symbol is the whole element
        smcut = 0;
#pragma unroll
        for (int k = 0; k < write_batch<DT>(); ++k) smv[k] = make_uint2(0, 0);
        return;
    }
    const uint32_t ii = cut_elem<DT>(i_begin, i_end);
    smcut = *(ii != ~0u ? sm_block + (DT == ZX_BF16 ? ii : ii / 2) : dummy);
    constexpr uint32_t P = Piece<DT>::kElems;
    const uint32_t lane = lane_now();
    const uint32_t qf_begin = (i_begin + P - 1) / P;
    const uint32_t qf_end = i_end / P;
#pragma unroll
    for (int k = 0; k < write_batch<DT>(); ++k) {
        const uint32_t q = qf_begin + lane + k * kWave;
        const uint8_t *a = q < qf_end ? sm_block + (DT == ZX_BF16 ? q * P : q * P / 2) : dummy;
        smv[k] = *reinterpret_cast<const uint2 *>(a);
    }
}

// Mark the prefetched bytes as used on every path, at a point where they have
// arrived and no store of the segment is out yet.  A register the loads target
// that looks still pending on some path would make the next segment's first write
// to it wait for all memory operations, this segment's stores included.
template <int DT>
__device__ __forceinline__ void settle_sm(const uint2 (&smv)[kWriteBatch], uint32_t smcut)
{
#pragma unroll
    for (int k = 0; k < write_batch<DT>(); ++k) asm volatile("" ::"v"(smv[k].x), "v"(smv[k].y));
    asm volatile("" ::"v"(smcut));
}

// Staged exponents of one piece, or a 0-bit block's single symbol.
template <int DT>
__device__ __forceinline__ uint4 piece_exps(const uint8_t *ex, bool degen, uint32_t dsplat)
{
    if (degen) return make_uint4(dsplat, dsplat, dsplat, dsplat);
    if (DT == ZX_BF16) {
        const uint2 e = *reinterpret_cast<const uint2 *>(ex);
        return make_uint4(e.x, e.y, 0, 0);
    }
    return *reinterpret_cast<const uint4 *>(ex);
}

// BF16: from four sign/mantissa bytes S and four staged exponents E (each rotated
// right by one bit) make the output word of two elements: byte-permute into
// [e, s, e, s] and [s, e, s, e], then take bit 7 of each byte from the first and
// bits 0..6 from the second.  Low byte: exponent bit 0 | mantissa; high byte:
// sign | exponent bits 7..1.
__device__ __forceinline__ uint32_t fuse_bf16_pair(uint32_t S, uint32_t E, uint32_t sel_a, uint32_t sel_b)
{
    const uint32_t a = __builtin_amdgcn_perm(E, S, sel_a);
    const uint32_t b = __builtin_amdgcn_perm(E, S, sel_b);
    return (a & 0x80808080u) | (b & 0x7F7F7F7Fu);
}
constexpr uint32_t kSelA01 = 0x01050004u, kSelB01 = 0x05010400u;   // elements 0, 1

// BF16, four elements at once: bit-select every low byte (exponent bit 0 | mantissa)
// and every high byte (sign | exponent bits 7..1), then interleave them into the
// two output words.  Four operations for four elements.
__device__ __forceinline__ uint2 fuse_bf16_quad(uint32_t S, uint32_t E)
{
    const uint32_t lo = (E & 0x80808080u) | (S & 0x7F7F7F7Fu);
    const uint32_t hi = (S & 0x80808080u) | (E & 0x7F7F7F7Fu);
    return make_uint2(__builtin_amdgcn_perm(hi, lo, 0x05010400u), __builtin_amdgcn_perm(hi, lo, 0x07030602u));
}

// FP8: four sign|mantissa nibbles N (element k at bits 4k..4k+3) and four staged
// exponents E3 (already at bits 3..6).  Each output byte is sign << 7 | exp << 3 | mant.
__device__ __forceinline__ uint32_t fuse_fp8_quad(uint32_t N, uint32_t E3)
{
    const uint32_t t = __builtin_amdgcn_perm(0u, N, 0x01010000u);       // [n01, n01, n23, n23]
    const uint32_t x = (t & 0x000F000Fu) | ((t >> 4) & 0x0F000F00u);    // one nibble per byte
    return x + (x & 0x08080808u) * 15u + E3;                             // sign bit 3 -> bit 7
}

// E8M0: four staged symbols (each rotated right by one bit, the form of a 256-symbol
// alphabet) back to the bytes themselves.
__device__ __forceinline__ uint32_t unrotate_quad(uint32_t E)
{
    return ((E << 1) & 0xFEFEFEFEu) | ((E >> 7) & 0x01010101u);
}

// Output words of one piece.
template <int DT>
__device__ __forceinline__ uint4 fuse_piece(uint2 smv, uint4 e)
{
    uint4 r;
    if constexpr (DT == ZX_E8M0) {
        (void)smv;
        r = make_uint4(unrotate_quad(e.x), unrotate_quad(e.y), unrotate_quad(e.z), unrotate_quad(e.w));
    } else if (DT == ZX_BF16) {
        const uint2 w01 = fuse_bf16_quad(smv.x, e.x);
        const uint2 w23 = fuse_bf16_quad(smv.y, e.y);
        r = make_uint4(w01.x, w01.y, w23.x, w23.y);
    } else {
        r.x = fuse_fp8_quad(smv.x & 0xFFFFu, e.x);
        r.y = fuse_fp8_quad(smv.x >> 16, e.y);
        r.z = fuse_fp8_quad(smv.y & 0xFFFFu, e.z);
        r.w = fuse_fp8_quad(smv.y >> 16, e.w);
    }
    return r;
}

// SO: a streaming (non-temporal) store, for launches whose output is small next to
// the Infinity Cache (the host picks the kernel instantiation).  (A run-time choice
// between the two stores is merged by the compiler into one plain store.)
template <int DT, bool SO>
__device__ __forceinline__ void store_piece(void *out_block, uint32_t i, uint4 r)
{
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    v4u *p = DT == ZX_BF16 ? reinterpret_cast<v4u *>(reinterpret_cast<uint16_t *>(out_block) + i)
                           : reinterpret_cast<v4u *>(reinterpret_cast<uint8_t *>(out_block) + i);
    const v4u v = {r.x, r.y, r.z, r.w};
    if constexpr (SO)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// One batch of whole pieces.  Every piece is fused before the first store goes out:
// the stores are conditional, and once one is in flight the outstanding-access
// count no longer tells when a given load has returned, so any wait after it would
// have to drain all stores first.  (Fusing and storing piece by piece after one
// wait for all loads was measured slower: each piece then waits for its own LDS
// read.)
template <int DT, bool SO>
__device__ __forceinline__ void store_batch(void *out_block, uint32_t qb, uint32_t qf_end, const uint2 (&smv)[kWriteBatch],
                                            const uint8_t *stage, uint32_t sbase, bool degen, uint32_t dsplat)
{
    constexpr uint32_t P = Piece<DT>::kElems;
    const uint32_t lane = lane_now();
    uint4 r[kWriteBatch];
#pragma unroll
    for (int k = 0; k < write_batch<DT>(); ++k) {
        const uint32_t q = qb + lane + k * kWave;
        r[k] = make_uint4(0, 0, 0, 0);
        asm volatile("" ::"v"(smv[k].x), "v"(smv[k].y));
        if (q < qf_end) r[k] = fuse_piece<DT>(smv[k], piece_exps<DT>(stage + (q * P - sbase), degen, dsplat));
    }
#pragma unroll
    for (int k = 0; k < write_batch<DT>(); ++k) {
        const uint32_t q = qb + lane + k * kWave;
        if (q < qf_end) store_piece<DT, SO>(out_block, q * P, r[k]);
    }
}

// This lane's cut-piece element (see cut_elem), from its sign/mantissa byte smb.
template <int DT>
__device__ __forceinline__ void write_cut_pieces(void *out_block, uint32_t i_begin, uint32_t i_end, const uint8_t *stage,
                                                 uint32_t sbase, bool degen, uint32_t dform, uint32_t smb)
{
    const uint32_t ii = cut_elem<DT>(i_begin, i_end);
    asm volatile("" ::"v"(smb));
    if (ii != ~0u) {
        const uint32_t ex = degen ? dform : stage[ii - sbase];
        if constexpr (DT == ZX_E8M0) {
            reinterpret_cast<uint8_t *>(out_block)[ii] = (uint8_t)(unrotate_quad(ex) & 0xFFu);
        } else if (DT == ZX_BF16) {
            reinterpret_cast<uint16_t *>(out_block)[ii] = (uint16_t)fuse_bf16_pair(smb, ex, kSelA01, kSelB01);
        } else {
            const uint32_t nn = (ii & 1) ? (smb >> 4) : (smb & 0xFu);
            reinterpret_cast<uint8_t *>(out_block)[ii] = (uint8_t)(fuse_fp8_quad(nn, ex) & 0xFFu);
        }
    }
}

// Write block elements [i_begin, i_end); the staged exponent of element i is
// stage[i - sbase] (or `dform` for a 0-bit block).  Whole pieces go in batches of
// kWriteBatch per lane, whose sign/mantissa loads are all issued before any is used;
// with kPre the first batch's bytes and the cut-piece byte are `smv0` and `smcut0`,
// loaded by prefetch_sm on the same range.  The (at most two) cut pieces at the range
// ends go one element per lane; their byte is loaded before any store goes out.
template <int DT, bool kPre, bool SO>
__device__ __forceinline__ void write_range(void *out_block, const uint8_t *sm_block, uint32_t i_begin, uint32_t i_end,
                                            const uint8_t *stage, uint32_t sbase, bool degen, uint32_t dform,
                                            const uint2 (&smv0)[kWriteBatch], uint32_t smcut0)
{
    constexpr uint32_t P = Piece<DT>::kElems;
    if (i_begin >= i_end) return;
    const uint32_t lane = lane_now();
    const uint32_t smcut = kPre ? smcut0 : load_cut_sm<DT>(sm_block, cut_elem<DT>(i_begin, i_end));
    const uint32_t qf_begin = (i_begin + P - 1) / P;
    const uint32_t qf_end = i_end / P;
    const uint32_t dsplat = dform * 0x01010101u;
    uint32_t qb = qf_begin;
    if (kPre && qb < qf_end) {
        store_batch<DT, SO>(out_block, qb, qf_end, smv0, stage, sbase, degen, dsplat);
        qb += kWave * write_batch<DT>();
    }
    for (; qb < qf_end; qb += kWave * write_batch<DT>()) {
        uint2 smv[kWriteBatch];
#pragma unroll
        for (int k = 0; k < write_batch<DT>(); ++k) {
            const uint32_t q = qb + lane + k * kWave;
            smv[k] = make_uint2(0, 0);
            if (q < qf_end) smv[k] = load_sm<DT>(sm_block, q * P);
        }
        store_batch<DT, SO>(out_block, qb, qf_end, smv, stage, sbase, degen, dsplat);
    }
    write_cut_pieces<DT>(out_block, i_begin, i_end, stage, sbase, degen, dform, smcut);
}

// ---- fallback passes, one code at a time ------------------------------------

// Count the codes starting in [start, lim): whole lookups while the window lies
// inside the chunk, single codes near its end.
__device__ uint32_t count_generic(const DTab &tab, lds_cu32 *col, uint32_t start, uint32_t lim, bool work,
                                  bool &lane_bad, uint32_t &pos_out)
{
    uint32_t cnt = 0;
    uint32_t p = start;
    if (work) {
        while (p < lim) {
            const uint32_t v = window(col, 256u - p);
            const uint32_t lo = tab.e[v >> (32 - kLutBits)].x;
            if (lo != 0 && p + kLutBits <= lim) {
                cnt += (lo >> 16) & 0xFFu;
                p += lo & 0xFFu;
            } else if (lo != 0) {
                cnt += 1;
                p += (lo >> 24) & 0xFu;
            } else {
                const uint32_t L = slow_len(tab, v);
                if (L > kMaxLen) { lane_bad = true; break; }
                cnt += 1;
                p += L;
            }
        }
    }
    pos_out = p;
    return cnt;
}

// Store this lane's `cnt` symbols, decoded again from `start`, at stage[wp ...].
__device__ void store_generic(const DTab &tab, lds_cu32 *col, uint8_t *stage, uint32_t start, uint32_t cnt, uint32_t wp)
{
    uint32_t p = start;
    for (uint32_t i = 0; i < cnt; ++i) {
        uint32_t sy;
        p += one_code(tab, window(col, 256u - p), sy);
        stage[wp + i] = (uint8_t)sy;
    }
}

// Segments whose exponents do not fit the stage: rounds of WIN stage positions
// (a multiple of 16), one code per step, exact writes.
template <int DT, bool SO, uint32_t WIN = kRoundElems>
__device__ void write_rounds(const DTab &tab, lds_cu32 *col, uint8_t *stage, uint32_t start, uint32_t cnt,
                             uint32_t off, uint32_t t0, uint32_t total, void *out_block, const uint8_t *sm_block,
                             uint32_t sbase)
{
    static_assert(WIN % 16 == 0, "stage rounds keep 16-element pieces whole");
    const uint2 none[kWriteBatch] = {};
    for (uint32_t r0 = 0; r0 < t0 + total; r0 += WIN) {
        const uint32_t r1 = r0 + WIN;
        uint32_t p = start;
        uint32_t t = t0 + off;
        for (uint32_t i = 0; i < cnt && t < r1; ++i, ++t) {
            uint32_t sy;
            p += one_code(tab, window(col, 256u - p), sy);
            if (t >= r0) stage[t - r0] = (uint8_t)sy;
        }
        wave_sync();
        const uint32_t ib = sbase + (r0 > t0 ? r0 : t0);
        const uint32_t ie = sbase + (r1 < t0 + total ? r1 : t0 + total);
        write_range<DT, false, SO>(out_block, sm_block, ib, ie, stage, sbase + r0, false, 0, none, 0u);
        wave_sync();
    }
}

// ---- segment descriptors and requests issued one segment ahead ---------------

// A segment's descriptor, validated.  Each lane of a wavefront loads the descriptor
// of one of the wavefront's segments (lane k: its k-th segment), so the dependent
// loads (segment -> block -> bit offset) are paid once per 64 segments.  The
// descriptors are then kept in LDS (not in registers, which the decode needs) and
// read back one segment at a time as wavefront-uniform values.
struct __align__(16) SegMeta {
    uint32_t b;          // block
    uint32_t e0;         // first element, within the block
    uint32_t e_end;      // end element, within the block
    uint32_t bits;       // stream bits of the block
    uint32_t j;          // segment index within the block
    uint32_t wlo, whi;   // stream word holding the segment's first bit
    uint32_t b0bad;      // bits 0..4: bit offset of the block start within its word;
                         // bit 8: the descriptor is inconsistent with the block arrays
};

__device__ __forceinline__ void load_meta(const DecTensor &T, uint32_t s, bool valid, SegMeta &m)
{
    m.b = 0; m.e0 = 0; m.e_end = 0; m.bits = 0; m.j = 0; m.wlo = 0; m.whi = 0;
    m.b0bad = valid ? 0u : 0x100u;
    if (!valid) return;
    const uint32_t b = T.seg_desc[2 * (uint64_t)s];
    const uint32_t e0 = T.seg_desc[2 * (uint64_t)s + 1];
    // the next descriptor's first element is requested with this one, before it is
    // known to be needed (it is when segment s + 1 is in the same block)
    const uint32_t e0n = T.seg_desc[2 * (uint64_t)(s + 1 < T.nsegs ? s + 1 : s) + 1];
    if (b >= T.nblocks) { m.b0bad = 0x100u; return; }
    const uint64_t G = T.block_bitoff[b];
    const uint64_t Gn = T.block_bitoff[b + 1];
    const uint32_t sb = T.block_seg[b];
    const uint32_t sbn = T.block_seg[b + 1];
    const uint64_t lo = (uint64_t)b * kBlock;
    const uint32_t nb = (uint32_t)(((lo + kBlock < T.n) ? lo + kBlock : T.n) - lo);
    // (a segment after a block's first starts inside the block's bits: its rows are
    // then read within the stream and its padding)
    if (Gn < G || Gn > T.total_bits || s < sb || s >= sbn || sbn > T.nsegs || Gn - G > (uint64_t)nb * kMaxLen ||
        (s != sb && (uint64_t)(s - sb) * kSegBits >= Gn - G)) {
        m.b0bad = 0x100u;
        return;
    }
    const uint32_t e_end = (s + 1 < sbn) ? e0n : nb;
    if (e0 > e_end || e_end > nb) { m.b0bad = 0x100u; return; }
    const uint64_t W0 = (G >> 5) + (uint64_t)(s - sb) * (kSegBits / 32);
    m.b = b;
    m.e0 = e0;
    m.e_end = e_end;
    m.bits = (uint32_t)(Gn - G);
    m.j = s - sb;
    m.wlo = (uint32_t)W0;
    m.whi = (uint32_t)(W0 >> 32);
    m.b0bad = (uint32_t)(G & 31);
}

// Descriptor i of a wavefront's LDS copy, as wavefront-uniform values.
__device__ __forceinline__ SegMeta meta_get(const SegMeta *ms, uint32_t i)
{
    const SegMeta v = ms[i];   // one address for the whole wavefront
    SegMeta u;
    u.b = __builtin_amdgcn_readfirstlane(v.b);
    u.e0 = __builtin_amdgcn_readfirstlane(v.e0);
    u.e_end = __builtin_amdgcn_readfirstlane(v.e_end);
    u.bits = __builtin_amdgcn_readfirstlane(v.bits);
    u.j = __builtin_amdgcn_readfirstlane(v.j);
    u.wlo = __builtin_amdgcn_readfirstlane(v.wlo);
    u.whi = __builtin_amdgcn_readfirstlane(v.whi);
    u.b0bad = __builtin_amdgcn_readfirstlane(v.b0bad);
    return u;
}

// Descriptor held by lane i, as wavefront-uniform values.
__device__ __forceinline__ SegMeta meta_at(const SegMeta &m, uint32_t i)
{
    SegMeta u;
    u.b = __builtin_amdgcn_readlane(m.b, i);
    u.e0 = __builtin_amdgcn_readlane(m.e0, i);
    u.e_end = __builtin_amdgcn_readlane(m.e_end, i);
    u.bits = __builtin_amdgcn_readlane(m.bits, i);
    u.j = __builtin_amdgcn_readlane(m.j, i);
    u.wlo = __builtin_amdgcn_readlane(m.wlo, i);
    u.whi = __builtin_amdgcn_readlane(m.whi, i);
    u.b0bad = __builtin_amdgcn_readlane(m.b0bad, i);
    return u;
}

// Loads a segment needs before it can decode: its lanes' stream words and gap bytes
// (and the next segment's first gap, for lane 63), with which of the gaps are real.
//
// Every load here is unconditional and its register is written by nothing else:
// gfx9 counts stores and loads in one counter, so a register write that has to
// wait for an earlier load into the same register (a default value, say) waits for
// every store issued since as well.  Values that some lanes do not need are still
// marked used on all lanes where they are stored, for the same reason.
struct SegIn {
    u32x4_a4 rv;
    uint32_t rtail;
    uint32_t gap;
    uint32_t gapn;
    uint32_t nch;        // the segment's block has nch chunks and the segment's
    uint32_t ch0;        // first is chunk ch0 (wavefront-uniform values)
};

// Put a segment's requested words and gap bytes into the wavefront's LDS rows.
__device__ __forceinline__ void rows_store_in(uint32_t *sw, uint32_t lane, const SegIn &in)
{
    asm volatile("" ::"v"(in.rtail), "v"(in.gapn));
    rows_store(sw, lane, in.rv, in.rtail);
    const uint32_t ch = in.ch0 + lane;
    sw[kGapSlot * kWave + lane] = ch < in.nch ? in.gap : (uint32_t)ZX_NO_GAP;
    if (lane == kWave - 1) sw[kGapSlot * kWave + kWave] = ch + 1 < in.nch ? in.gapn : (uint32_t)ZX_NO_GAP;
}

// Request segment s; unless `want` (and a valid descriptor) the loads read the
// stream's and the gap table's first entries, and no gap counts as real.
__device__ __forceinline__ void issue_seg(const DecTensor &T, uint32_t s, const SegMeta &m, uint32_t lane, SegIn &in,
                                          bool want)
{
    const bool ok = want && (m.b0bad & 0x100u) == 0 && m.bits != 0;
    const uint64_t W0 = ok ? (((uint64_t)m.whi << 32) | m.wlo) : 0ull;
    rows_load(T.stream, W0, lane, in.rv, in.rtail);
    const uint32_t sv = ok ? s : 0u;
    const uint32_t svn = sv + 1 < T.nsegs ? sv + 1 : sv;
    in.gap = T.gaps[(uint64_t)sv * kSegChunks + lane];
    in.gapn = T.gaps[(uint64_t)svn * kSegChunks];
    in.nch = ok ? (m.bits + kChunkBits - 1) / kChunkBits : 0u;
    in.ch0 = m.j * kSegChunks;
}

// ---- the spare stage of the fast decode ---------------------------------------
//
// One wavefront at a time may use the workgroup's spare stage, for a segment that
// needs the code-by-code passes.  The holder waits for no other wavefront while it
// holds it, so every waiting wavefront gets it in the end; the wait is capped anyway
// (about a second, far beyond any holder's work), after which the segment is
// reported corrupt and skipped.
__device__ __forceinline__ bool spare_acquire(uint32_t *lock)
{
    for (uint32_t spin = 0; spin < (1u << 24); ++spin) {
        uint32_t got = 0;
        if (lane_now() == 0) got = atomicCAS(lock, 0u, 1u) == 0u ? 1u : 0u;
        if (__builtin_amdgcn_readfirstlane(got)) {
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            return true;
        }
        __builtin_amdgcn_s_sleep(2);
    }
    return false;
}

__device__ __forceinline__ void spare_release(uint32_t *lock)
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    if (lane_now() == 0) atomicExch(lock, 0u);
}

// ---- one segment per wavefront ------------------------------------------------

// ---- the low-entropy fast decode's stage geometry ------------------------------
//
// Below about 2.3 bits per code a segment holds more elements than the 3616-byte
// stage and a chunk more codes than seven rounds.  The low-entropy mode runs eleven
// rounds (33 lookups of up to four codes: a 128-bit chunk holds at most 128 codes,
// and every lookup but a stalled third one takes four codes or more than 5.5 bits on
// average) and gives each wavefront a region of kLowRegion bytes.  The rows sit at its
// start during the count pass; the replay then writes the stage at kLowGuard, in
// windows of kLowWin positions when a segment holds more elements than that (below
// about 1.09 bits per code).  The 16 guard bytes before the stage take the up to
// three bytes an entry that straddles a window's start writes before it, and the 16
// after it those an entry writes past its end.  The code-by-code passes (a lane
// that needs more than eleven rounds) keep the rows and use the rest of the region.
constexpr int kLowRounds = 11;
constexpr uint32_t kLowRegion = 7584;
constexpr uint32_t kLowGuard = 16;
constexpr uint32_t kLowWin = kLowRegion - 2 * kLowGuard;
constexpr uint32_t kLowGenOff = (kSegWords * 4 + 15) & ~15u;
constexpr uint32_t kLowGenWin = (kLowRegion - kLowGenOff) & ~15u;
static_assert(kLowWin % 16 == 0 && kLowGenWin % 16 == 0 && kLowGenWin >= 4096, "low-entropy stage windows");

// Low-entropy mode: replay a lane's `cnt` symbols (register entries `ent`, counts in
// the bytes of `nsb`), which go to stage positions t0 + off ..., into `st` one window
// of kLowWin positions at a time, and write each window out.  In a window starting at
// position w0 an entry at p stores its four bytes at st + p - w0 when any of them can
// fall inside (p - w0 >= -3), then the lane's first three symbols are stored again
// over the bytes the lane before it wrote past its end.  Windows start at 16-aligned
// elements, so the cut pieces are only at the segment's ends; the first window's
// sign/mantissa bytes come from prefetch_sm over the whole segment.
template <int DT, bool SO, int kE, int kNs>
__device__ __forceinline__ void replay_windows(const uint32_t (&ent)[kE], const uint32_t (&nsb)[kNs], uint32_t cnt,
                                               uint32_t off, uint32_t t0, uint32_t total, uint8_t *st,
                                               void *out_block, const uint8_t *sm_block, uint32_t e0, uint32_t sbase,
                                               const uint2 (&smv)[kWriteBatch], uint32_t smcut)
{
    const uint2 none[kWriteBatch] = {};
    // first three symbols: the first entry's, topped up from the entries after it (a
    // stalled lookup leaves an empty entry; three rounds hold at least three symbols)
    uint32_t f3 = ent[0];
    uint32_t nf = nsb[0] & 0xFFu;
    const uint32_t need = cnt < 3u ? cnt : 3u;
#pragma unroll
    for (int k = 1; k < 7; ++k) {
        if (__builtin_amdgcn_ballot_w64(nf < need) == 0) break;
        if (nf < need) {
            f3 = (f3 & ((1u << (8 * nf)) - 1u)) | (ent[k] << (8 * nf));
            nf += (nsb[k >> 2] >> (8 * (k & 3))) & 0xFFu;
        }
    }
    const uint32_t tend = t0 + total;
    for (uint32_t w0 = 0;; w0 += kLowWin) {
        const int32_t base = (int32_t)(t0 + off) - (int32_t)w0;   // the lane's first position in the window
        const int32_t pend = base + (int32_t)cnt;
        const int32_t plim = pend < (int32_t)kLowWin ? pend : (int32_t)kLowWin;
        int32_t pp = base;
#pragma unroll
        for (int k = 0; k < kE; ++k) {
            if (__builtin_amdgcn_ballot_w64(pp < plim) == 0) break;
            if (pp < plim) {
                if (pp >= -3) {
                    uint8_t *a = st + pp;
                    // two pairs of non-adjacent bytes, kept apart: four adjacent byte
                    // stores would be merged into one unaligned dword store
                    a[0] = (uint8_t)ent[k];
                    a[2] = (uint8_t)(ent[k] >> 16);
                    asm volatile("" ::: "memory");
                    a[1] = (uint8_t)(ent[k] >> 8);
                    a[3] = (uint8_t)(ent[k] >> 24);
                }
                pp += (int32_t)((nsb[k >> 2] >> (8 * (k & 3))) & 0xFFu);
            }
        }
        wave_sync();
        if (base > -3 && base < (int32_t)kLowWin) {
            uint8_t *const a0 = st + base;
            if (cnt >= 3) {
                a0[0] = (uint8_t)f3;
                a0[1] = (uint8_t)(f3 >> 8);
                a0[2] = (uint8_t)(f3 >> 16);
            } else if (cnt == 2) {
                a0[0] = (uint8_t)f3;
                a0[1] = (uint8_t)(f3 >> 8);
            } else if (cnt == 1) {
                a0[0] = (uint8_t)f3;
            }
        }
        wave_sync();
        const uint32_t wend = w0 + kLowWin < tend ? w0 + kLowWin : tend;
        if (w0 == 0) {
            settle_sm<DT>(smv, smcut);
            write_range<DT, true, SO>(out_block, sm_block, e0, sbase + wend, st, sbase, false, 0, smv, smcut);
        } else {
            write_range<DT, false, SO>(out_block, sm_block, sbase + w0, sbase + wend, st, sbase + w0, false, 0, none, 0u);
        }
        if (wend >= tend) break;
        wave_sync();
    }
}

// Byte selector that puts byte 2 of the first v_perm operand into byte j and keeps
// the second operand's other bytes.
__host__ __device__ constexpr uint32_t ns_sel(int j)
{
    return j == 0 ? 0x03020106u : j == 1 ? 0x03020600u : j == 2 ? 0x03060100u : 0x06020100u;
}
// Symbol count of lookup k, from the packed count bytes.
#define ZX_NS(k) ((nsb[(k) >> 2] >> (8 * ((k) & 3))) & 0xFFu)

// One table lookup at the front of `win` for the lanes in `a`; the others read the
// zero entry and keep their state.  `xsym` and `xns` add a symbol decoded before
// the lookup (a long code in slot 0) to the entry and to its count.
#define ZX_LOOKUP(a, slot, xsym, xns)                                                    \
    do {                                                                                 \
        const uint32_t x_ = (a) ? ((win >> (29 - kLutBits)) & ((kLutSize - 1u) << 3))    \
                                : (kLutSize * 8u);                                       \
        const uint2 e_ = lds_pair(tab.e, x_);                                            \
        const uint32_t lo_ = e_.x;                                                       \
        const uint32_t hi_ = e_.y;                                                       \
        win <<= (lo_ & 31u);                                                             \
        Bprev = (a) ? B : Bprev;                                                         \
        B -= lo_;                                                                        \
        ent[slot] = hi_ | (xsym);                                                        \
        nsb[(slot) >> 2] = __builtin_amdgcn_perm(lo_ | (xns), nsb[(slot) >> 2], ns_sel((slot) & 3)); \
    } while (0)

// Decode segment s.  The wavefront's word rows and its stage share one region: the
// segment's stream words and gap bytes, requested into `in` while the segment before
// it decoded, are put in at its start (after that segment's write pass has read the
// stage), and the next segment's are requested into `in` (when has_next).  A segment
// that needs the code-by-code passes borrows the workgroup's spare stage under `lock`.
// LOW: the low-entropy mode above; no spare stage.
template <int DT, bool SO, bool LOW>
__device__ __forceinline__ bool decode_segment_body(const DecTensor &T, const DTab &tab, uint8_t *stage, uint32_t *sw,
                                                    uint32_t s, const SegMeta &m, SegIn &in, bool has_next, uint32_t sn,
                                                    const SegMeta &mn, uint32_t *err, uint8_t *spare = nullptr,
                                                    uint32_t *lock = nullptr)
{
    constexpr uint32_t A = alphabet_of(DT);
    const uint32_t lane = lane_now();
    const bool bad = (m.b0bad & 0x100u) != 0;
    const uint32_t b = m.b;
    const uint32_t e0 = m.e0;
    const uint32_t e_end = m.e_end;
    const uint32_t bits = m.bits;
    const uint32_t j = m.j;
    const uint64_t lo = (uint64_t)b * kBlock;
    const uint32_t nb = (uint32_t)(((lo + kBlock < T.n) ? lo + kBlock : T.n) - lo);
    const uint8_t *sm_block = DT == ZX_E8M0 ? T.signmant : T.signmant + (DT == ZX_BF16 ? lo : lo / 2);
    void *out_block = reinterpret_cast<uint8_t *>(T.out) + lo * (DT == ZX_BF16 ? 2 : 1);
    const uint32_t sbase = e0 & ~15u;   // 16-aligned element that stage byte 0 stands for

    // the next segment's words and gaps, and this segment's sign/mantissa bytes for
    // its first write batch, are requested first; they arrive while this segment
    // decodes.  The bytes are requested only on the path that uses them, so that no
    // path from their request to the next segment skips their use.
    rows_store_in(sw, lane, in);
    wave_sync();
    const uint32_t gap = sw[kGapSlot * kWave + lane];
    const uint32_t gap_next = sw[kGapSlot * kWave + lane + 1];
    issue_seg(T, sn, mn, lane, in, has_next);
    if (bad) { report(err, ZX_E_CORRUPT); return false; }
    if (bits == 0) {
        const uint32_t d = T.degenerate[T.per_block ? b : 0];
        if (d >= A || e0 != 0 || e_end != nb) { report(err, ZX_E_CORRUPT); return false; }
        uint2 smv[kWriteBatch];
        uint32_t smcut;
        prefetch_sm<DT>(sm_block, e0, e_end, reinterpret_cast<const uint8_t *>(T.stream), smv, smcut);
        settle_sm<DT>(smv, smcut);
        write_range<DT, true, SO>(out_block, sm_block, e0, e_end, stage, sbase, true, stage_form(A, d), smv, smcut);
        return false;
    }
    if (!tab.ok) { report(err, ZX_E_CORRUPT); return false; }

    const uint32_t nch = (bits + kChunkBits - 1) / kChunkBits;
    const uint32_t ch = j * kSegChunks + lane;
    bool work = gap != ZX_NO_GAP;
    bool lane_bad = false;
    if (work && gap >= kMaxLen) { work = false; lane_bad = true; }
    const uint32_t cend = (ch * kChunkBits + kChunkBits < bits) ? kChunkBits : bits - ch * kChunkBits;
    if (work && gap >= cend) { work = false; lane_bad = true; }
    const uint32_t b0 = m.b0bad & 31u;
    // codes of one chunk must end exactly where the next chunk's first code starts
    // (or at the block end), as the stored gaps claim
    const uint32_t expect = (ch + 1 < nch && gap_next != ZX_NO_GAP) ? kPosBase + b0 + kChunkBits + gap_next
                                                                    : kPosBase + b0 + (bits - ch * kChunkBits);
    wave_sync();
    lds_cu32 *col = window_col(sw, lane);
    const uint32_t start = kPosBase + b0 + gap;
    const uint32_t lim = kPosBase + b0 + cend;
    // B: low byte 256 - position, bits 8..15 absorb the entries' third-code field,
    // bits 16..23 minus the code count; a lane is active while its position is below
    // lim, i.e. while B's low byte exceeds thr (a lane without a chunk, or one found
    // damaged, gets thr = 255: never active)
    uint32_t thr = work ? 256u - lim : 255u;
    constexpr uint32_t kIdleQ = 256u - kPosBase;   // a harmless window for idle lanes
    uint32_t B = 0xFF00u | (work ? 256u - start : kIdleQ);
    uint32_t Bprev = B;
    const uint32_t lim_short = tab.lim_short;

    // ---- count pass, register path
    // entries of rounds that do not run are never read: the replay stops once no lane
    // has symbols left
    static_assert(LOW || DT != ZX_E8M0, "E8M0 takes the low-entropy mode only");
    constexpr int kR = LOW ? kLowRounds : kRounds, kE = 3 * kR, kNs = (kE + 3) / 4;
    uint32_t ent[kE];
    uint32_t nsb[kNs];
#pragma unroll
    for (int k = 0; k < kE; ++k) ent[k] = __builtin_nondeterministic_value(0u);
#pragma unroll
    for (int k = 0; k < kNs; ++k) nsb[k] = __builtin_nondeterministic_value(0u);
#pragma unroll
    for (int r = 0; r < kR; ++r) {
        bool act = (B & 0xFFu) > thr;
        const uint64_t am = __builtin_amdgcn_ballot_w64(act);
        if (am == 0) break;
        uint32_t win = window(col, B);
        uint32_t Bw = B;                           // B when win was read
        const bool lng = act && win > lim_short;   // the next code is longer than the table window
        uint32_t eslow = 0, nslow = 0;
        // (a divergent branch: skipped as a whole when no lane has a long code)
        if (lng) {
            const uint32_t L = slow_len(tab, win);
            if (L > kMaxLen) {
                thr = 255u;
                lane_bad = true;
                act = false;
            } else {
                eslow = slow_sym(tab, win, L);
                nslow = 1u << 16;
                Bprev = B;
                B -= L | (1u << 16);
                act = (B & 0xFFu) > thr;
                win = window(col, B);
                Bw = B;
            }
        }
        const bool a0 = act && !lng;   // a long code took slot 0
        ZX_LOOKUP(a0, 3 * r, eslow, nslow);
        act = act && (B & 0xFFu) > thr;
        ZX_LOOKUP(act, 3 * r + 1, 0u, 0u);
        // the third lookup needs kLutBits valid window bits: two lookups may have
        // taken up to 2 kLutBits of the 32 (a lane that lacks them waits a round)
        act = act && (B & 0xFFu) > thr && ((Bw - B) & 0xFFu) + kLutBits <= 32u;
        ZX_LOOKUP(act, 3 * r + 2, 0u, 0u);
    }
    const bool more = __builtin_amdgcn_ballot_w64((B & 0xFFu) > thr) != 0;

    uint32_t cnt = 0;
    if (!more) {
        if (work && !lane_bad) {
            // the last lookup may hold codes that start in the next chunk: drop them
            const uint32_t el = Bprev - B;
            const uint32_t pl = 256u - (Bprev & 0xFFu);
            const uint32_t ns = (el >> 16) & 0xFFu;
            uint32_t endp = pl + (el & 0xFFu);
            uint32_t drop = 0;
            if (ns >= 2 && pl + ((el >> 24) & 0xFu) >= lim) {
                drop = ns - 1;
                endp = pl + ((el >> 24) & 0xFu);
            } else if (ns >= 3 && pl + (el >> 28) >= lim) {
                drop = ns - 2;
                endp = pl + (el >> 28);
            } else if ((el & (4u << 16)) != 0 && pl + ((el >> 8) & 0xFu) >= lim) {   // ns == 4
                drop = 1;
                endp = pl + ((el >> 8) & 0xFu);
            }
            cnt = ((0u - (B >> 16)) & 0xFFu) - drop;
            if (endp != expect) lane_bad = true;
        }
    } else {
        // some lane needs more lookups than the registers hold: count again, one code at a time near the end
        uint32_t pos = 0;
        cnt = count_generic(tab, col, start, lim, work, lane_bad, pos);
        if (work && !lane_bad && pos != expect) lane_bad = true;
    }
    uint32_t total;
    const uint32_t off = wave_excl_scan(cnt, total);
    if (any_lane(lane_bad) || e0 + total != e_end) { report(err, ZX_E_CORRUPT); return false; }

    const uint32_t t0 = e0 - sbase;   // stage position of the segment's first element
    if constexpr (LOW) {
        if (more) {
            write_rounds<DT, SO, kLowGenWin>(tab, col, stage + kLowGenOff, start, cnt, off, t0, total, out_block,
                                             sm_block, sbase);
            return false;
        }
        uint2 smv[kWriteBatch];
        uint32_t smcut;
        prefetch_sm<DT>(sm_block, e0, e_end, reinterpret_cast<const uint8_t *>(T.stream), smv, smcut);
        replay_windows<DT, SO, kE, kNs>(ent, nsb, cnt, off, t0, total, stage + kLowGuard, out_block, sm_block, e0,
                                        sbase, smv, smcut);
        return true;
    }
    if (t0 + total + 3 > kStageBytes) {
        if (!spare_acquire(lock)) { report(err, ZX_E_CORRUPT); return false; }
        write_rounds<DT, SO>(tab, col, spare, start, cnt, off, t0, total, out_block, sm_block, sbase);
        spare_release(lock);
        return false;
    }
    // some lane needed more lookups than the registers hold: its symbols go to the
    // stage one code at a time, and no entry is replayed.  The rows are still needed
    // for that, so the symbols go to the spare stage.
    if (more) {
        if (!spare_acquire(lock)) { report(err, ZX_E_CORRUPT); return false; }
        stage = spare;
        store_generic(tab, col, stage, start, cnt, t0 + off);
    }
    const uint32_t rcnt = more ? 0u : cnt;

    // the sign/mantissa bytes of the first write batch are requested now: they arrive
    // during the replay, and their registers are free during the count pass.  From
    // here to their use below there is no exit, so every path uses them before any
    // store goes out.
    uint2 smv[kWriteBatch];
    uint32_t smcut;
    prefetch_sm<DT>(sm_block, e0, e_end, reinterpret_cast<const uint8_t *>(T.stream), smv, smcut);

    // ---- replay the entries into the stage: each entry stores its four symbol bytes
    //      and advances by its symbol count (byte stores: unaligned dword stores to LDS
    //      stall).  A lane's last entry may store up to three bytes past its end, onto
    //      the first positions of the lanes after it, so after a barrier every lane
    //      rewrites its first three positions.
    // first three symbols: the first entry's, topped up from the entries after it (a
    // stalled lookup leaves an empty entry; a long code fills one slot; three rounds
    // hold at least three symbols)
    uint32_t f3 = ent[0];
    uint32_t nf = ZX_NS(0);
    const uint32_t need = rcnt < 3u ? rcnt : 3u;
#pragma unroll
    for (int k = 1; k < 7; ++k) {
        if (__builtin_amdgcn_ballot_w64(nf < need) == 0) break;
        if (nf < need) {
            f3 = (f3 & ((1u << (8 * nf)) - 1u)) | (ent[k] << (8 * nf));
            nf += ZX_NS(k);
        }
    }
    uint8_t *a = stage + t0 + off;
    uint8_t *const aend = a + rcnt;
#pragma unroll
    for (int k = 0; k < kE; ++k) {
        if (__builtin_amdgcn_ballot_w64(a < aend) == 0) break;
        if (a < aend) {
            // two pairs of non-adjacent bytes, kept apart: four adjacent byte stores
            // would be merged into one unaligned dword store
            a[0] = (uint8_t)ent[k];
            a[2] = (uint8_t)(ent[k] >> 16);
            asm volatile("" ::: "memory");
            a[1] = (uint8_t)(ent[k] >> 8);
            a[3] = (uint8_t)(ent[k] >> 24);
            a += ZX_NS(k);
        }
    }
    wave_sync();
    uint8_t *const a0 = stage + t0 + off;
    if (rcnt >= 3) {
        a0[0] = (uint8_t)f3;
        a0[1] = (uint8_t)(f3 >> 8);
        a0[2] = (uint8_t)(f3 >> 16);
    } else if (rcnt == 2) {
        a0[0] = (uint8_t)f3;
        a0[1] = (uint8_t)(f3 >> 8);
    } else if (rcnt == 1) {
        a0[0] = (uint8_t)f3;
    }
    wave_sync();
    settle_sm<DT>(smv, smcut);
    write_range<DT, true, SO>(out_block, sm_block, e0, e_end, stage, sbase, false, 0, smv, smcut);
    if (more) spare_release(lock);
    return true;
}
#undef ZX_LOOKUP
#undef ZX_NS

// Issue priority of this wavefront from the share of its segments still ahead: 3 at
// the start, down to 0 for its last quarter.  A SIMD issues from its oldest wavefront
// first among equal priorities, so without this the workgroups a CU received first run
// ahead and the last one is left to finish its segments alone with few wavefronts
// beside it; with it, wavefronts that are behind go first and the CU's wavefronts end
// close together, at full occupancy until near the end.
__device__ __forceinline__ void set_priority_by_remaining(uint32_t remaining, uint32_t total)
{
    const uint32_t p = __builtin_amdgcn_readfirstlane((4u * remaining - 1u) / total);   // 0..3
    if (p >= 3) __builtin_amdgcn_s_setprio(3);
    else if (p == 2) __builtin_amdgcn_s_setprio(2);
    else if (p == 1) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
}

// ---- the decode kernels ---------------------------------------------------------
//
// Three 512-thread workgroups per CU (six wavefronts per SIMD): each wavefront's
// stream words and its stage share one region (3616 bytes), descriptors are
// refreshed sixteen at a time, and the code-by-code passes borrow one spare stage
// per workgroup.  A tensor of 5376 segments (4096 x 4096 BF16) gets one segment per
// wavefront, and every wavefront has five others on its SIMD to hide its memory and
// LDS waits behind.  Segments of mean code length below about 2.3 bits overflow the
// stage and would take the spare one wavefront at a time, so such containers (and
// all E8M0 ones) take the low-entropy mode (LOW): two workgroups per CU, eleven count
// rounds and a larger region per wavefront (see kLowRegion), no spare.
// k_decode_fast takes per-tensor codebooks, persistent over a share of the segments;
// k_decode_fast_blocks per-block ones (and K/V slot lists), one workgroup per block.
constexpr int kFastWgPerCu = 3;
constexpr int kLowWgPerCu = 2;
constexpr uint32_t kFastMeta = 16;   // descriptors per wavefront refresh
static_assert(kSegWords * 4 <= kStageBytes, "the word rows fit the stage region");

template <bool LOW>
struct FastShared {
    static constexpr uint32_t kRegion = LOW ? kLowRegion : kStageBytes;
    DTab tab;
    uint8_t region[kDecWaves][kRegion];       // rows during the count pass, then the stage
    SegMeta meta[kDecWaves][kFastMeta];
    uint8_t spare[LOW ? 16u : kStageBytes];   // the code-by-code passes' stage (not LOW)
    uint32_t lock;
};
static_assert(sizeof(FastShared<false>) <= 160u * 1024u / kFastWgPerCu, "fast decode workgroup LDS budget");
static_assert(sizeof(FastShared<true>) <= 160u * 1024u / kLowWgPerCu, "low-entropy decode workgroup LDS budget");

// The segment loop of a fast-decode wavefront: its segments s0 + nw k, k < nk (nw:
// the workgroup's wavefronts), whose first descriptors (up to kFastMeta) are already
// in the wavefront's LDS copy
// and whose first words were requested into `in`.  On return `in` holds the last
// request (a dummy, or the words of a segment this wavefront does not decode).
template <int DT, bool SO, bool LOW>
__device__ __forceinline__ void fast_segment_loop(const DecTensor &T, FastShared<LOW> &sh, uint32_t wave, uint32_t nw,
                                                  uint32_t s0, uint32_t nk, SegIn &in, uint32_t *err)
{
    uint8_t *reg = sh.region[wave];
    uint32_t *sw = reinterpret_cast<uint32_t *>(reg);
    SegMeta *metas = sh.meta[wave];
    for (uint32_t k = 0; k < nk; ++k) {
        set_priority_by_remaining(nk - k, nk);
        const uint32_t i = k & (kFastMeta - 1);
        const uint32_t s = s0 + nw * k;
        const bool has_next = k + 1 < nk && i + 1 < kFastMeta;
        const SegMeta mu = meta_get(metas, i);
        const SegMeta mn = meta_get(metas, has_next ? i + 1 : i);
        decode_segment_body<DT, SO, LOW>(T, sh.tab, reg, sw, s, mu, in, has_next, s + nw, mn, err, sh.spare,
                                               &sh.lock);
        if (i == kFastMeta - 1 && k + 1 < nk) {
            // next group of 16 descriptors, and the words of its first segment (put
            // in at that segment's start)
            const uint32_t lane = lane_now();
            SegMeta m2;
            load_meta(T, s + nw + nw * lane, lane < kFastMeta && k + 1 + lane < nk, m2);
            issue_seg(T, s + nw, meta_at(m2, 0), lane, in, true);
            wave_sync();
            if (lane < kFastMeta) metas[lane] = m2;
            wave_sync();
        }
    }
}

// Per-block codebooks: one workgroup per block, all eight wavefronts on its segments,
// the block's table built in LDS first.  The build's scratch (the canonical
// description and the single-code table) lives in the wavefronts' regions, which no
// wavefront uses before the table is built.  The block's descriptors and first words
// are requested before the build, so that they arrive while it runs; the other
// workgroups resident on the CU (three, or two in the low-entropy mode) keep the
// memory busy meanwhile.
constexpr uint32_t kCanonBytes = (sizeof(Canon) + 15u) & ~15u;

template <int DT, bool SO, bool LOW>
__device__ __forceinline__ void fast_block(const DecTensor &T, uint32_t b, FastShared<LOW> &sh, uint32_t *err)
{
    constexpr uint32_t A = alphabet_of(DT);
    static_assert(kCanonBytes + kLutSize * 2 <= sizeof(sh.region), "table scratch fits the regions");
    const uint32_t tid = threadIdx.x;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const uint32_t lane = lane_now();
    const uint32_t len = tid < A ? T.lengths[(uint64_t)b * A + tid] : 0u;
    const uint32_t s_begin = T.block_seg[b];
    uint32_t s_end = T.block_seg[b + 1];
    if (s_end > T.nsegs || s_begin > s_end) {
        s_end = s_begin;
        if (tid == 0) report(err, ZX_E_CORRUPT);
    }
    const uint32_t s0 = s_begin + wave;
    const uint32_t nk = __builtin_amdgcn_readfirstlane(s0 < s_end ? (s_end - s0 + kDecWaves - 1) / kDecWaves : 0);
    SegMeta mine;
    load_meta(T, s0 + kDecWaves * lane, lane < kFastMeta && lane < nk, mine);
    SegIn in;
    issue_seg(T, s0, meta_at(mine, 0), lane, in, nk != 0);
    Canon &c = *reinterpret_cast<Canon *>(&sh.region[0][0]);
    canon_build_from(len, A, c);
    dtab_fill(c, A, sh.tab, reinterpret_cast<uint16_t *>(&sh.region[0][0] + kCanonBytes));
    if (lane < kFastMeta) sh.meta[wave][lane] = mine;
    if (tid == 0) sh.lock = 0;
    __syncthreads();
    fast_segment_loop<DT, SO, LOW>(T, sh, wave, kDecWaves, s0, nk, in, err);
    asm volatile("" ::"v"(in.rv.x), "v"(in.rtail), "v"(in.gap), "v"(in.gapn));
}

template <int DT, bool SO, bool LOW>
__global__ __launch_bounds__(kDecThreads, (LOW ? kLowWgPerCu : kFastWgPerCu) * kDecWaves / 4) void k_decode_fast(
    const DecBatch batch, uint32_t *err)
{
    static_assert(DT == ZX_BF16 || DT == ZX_FP8_E4M3FN || (DT == ZX_E8M0 && LOW), "fast decode: BF16, FP8; E8M0 in LOW");
    __shared__ FastShared<LOW> sh;
    const uint32_t g = blockIdx.x;
    uint32_t t = 0;
    while (t + 1 < batch.count && g >= batch.t[t + 1].wg_begin) ++t;
    const DecTensor &T = batch.t[t];
    const uint32_t lg = g - T.wg_begin;
    const uint32_t tid = threadIdx.x;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const uint32_t nw = __builtin_amdgcn_readfirstlane(blockDim.x / kWave);   // kMinDecWaves..kDecWaves
    const uint32_t lane = lane_now();
    const uint32_t s_begin = lg * T.segs_per_wg;
    const uint32_t s_end = s_begin + T.segs_per_wg < T.nsegs ? s_begin + T.segs_per_wg : T.nsegs;
    // the wavefront's segments are s_begin + wave + nw k, k < nk; lane i < 16 loads
    // the descriptor of the i-th (in groups of 16)
    const uint32_t s0 = s_begin + wave;
    const uint32_t nk = __builtin_amdgcn_readfirstlane(s0 < s_end ? (s_end - s0 + nw - 1) / nw : 0);
    // the prepared table is requested first, the descriptors and first words next; the
    // table is stored to LDS once it arrives
    const uint4 *src = reinterpret_cast<const uint4 *>(T.dtab);
    uint4 *dst = reinterpret_cast<uint4 *>(&sh.tab);
    constexpr uint32_t kTabPieces = sizeof(DTab) / 16;
    constexpr uint32_t kPer = (kTabPieces + kMinDecWaves * kWave - 1) / (kMinDecWaves * kWave);
    uint4 pc[kPer];
#pragma unroll
    for (uint32_t k = 0; k < kPer; ++k) {
        const uint32_t i = tid + k * blockDim.x;
        pc[k] = i < kTabPieces ? src[i] : make_uint4(0, 0, 0, 0);
    }
    SegMeta mine;
    load_meta(T, s0 + nw * lane, lane < kFastMeta && lane < nk, mine);
    SegIn in;
    issue_seg(T, s0, meta_at(mine, 0), lane, in, nk != 0);
#pragma unroll
    for (uint32_t k = 0; k < kPer; ++k) {
        const uint32_t i = tid + k * blockDim.x;
        if (i < kTabPieces) dst[i] = pc[k];
    }
    if (lane < kFastMeta) sh.meta[wave][lane] = mine;
    if (tid == 0) sh.lock = 0;
    __syncthreads();
    fast_segment_loop<DT, SO, LOW>(T, sh, wave, nw, s0, nk, in, err);
    // the last request into `in` is used here, so that no load is left unused in flight
    asm volatile("" ::"v"(in.rv.x), "v"(in.rtail), "v"(in.gap), "v"(in.gapn));
}

// The batch of per-block-codebook containers, one workgroup per block (see fast_block).
// SLOTS: the batch is a slot list (DecSlots): workgroup g decodes the one-block
// container in slot slot_ids[g] of a K/V slot pool into row g of the output; t[0]
// describes slot 0's container and the strides give every other slot's arrays.
template <int DT, bool SO, bool LOW, bool SLOTS>
__global__ __launch_bounds__(kDecThreads, (LOW ? kLowWgPerCu : kFastWgPerCu) * kDecWaves / 4) void k_decode_fast_blocks(
    const DecBatch batch, uint32_t *err)
{
    __shared__ FastShared<LOW> sh;
    const uint32_t g = blockIdx.x;
    if constexpr (SLOTS) {
        const DecSlots &S = batch.slots;
        const uint64_t slot = S.slot_ids[g];
        if (slot >= S.n_slots) {
            if (threadIdx.x == 0) report(err, ZX_E_CORRUPT);
            return;
        }
        DecTensor T = batch.t[0];
        T.signmant += slot * S.sm_bytes;
        T.stream += slot * S.stream_words;
        T.block_bitoff += 2 * slot;
        T.block_seg += 2 * slot;
        T.seg_desc += 2 * slot * S.seg_stride;
        T.gaps += slot * S.seg_stride * kSegChunks;
        T.lengths += slot * S.alphabet;
        T.degenerate += slot;
        T.out = static_cast<uint8_t *>(T.out) + (uint64_t)g * S.out_bytes;
        fast_block<DT, SO, LOW>(T, 0, sh, err);
    } else {
        uint32_t t = 0;
        while (t + 1 < batch.count && g >= batch.t[t + 1].wg_begin) ++t;
        fast_block<DT, SO, LOW>(batch.t[t], g - batch.t[t].wg_begin, sh, err);
    }
}

__global__ __launch_bounds__(1024) void k_build_dtab(const uint8_t *__restrict__ lengths, uint32_t A, DTab *__restrict__ out)
{
    __shared__ Canon c;
    __shared__ uint16_t t1[kLutSize];
    canon_build(lengths, A, c);
    dtab_fill(c, A, *out, t1);
}

}  // namespace zxk

using namespace zxk;

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

extern "C" size_t zx_decode_table_bytes(void) { return sizeof(DTab); }

extern "C" zx_status zx_build_decode_table(zx_dtype dtype, const uint8_t *lengths, uint32_t *dtab, hipStream_t stream)
{
    if (dtype != ZX_BF16 && dtype != ZX_FP8_E4M3FN && dtype != ZX_E8M0) return ZX_E_UNSUPPORTED;
    if (!lengths || !dtab || !aligned16(dtab)) return ZX_E_INVAL;
    // one table entry per thread
    hipLaunchKernelGGL(k_build_dtab, dim3(1), dim3(1024), 0, stream, lengths, alphabet_of(dtype), reinterpret_cast<DTab *>(dtab));
    return hipGetLastError() == hipSuccess ? ZX_OK : ZX_E_HIP;
}

static zx_status check_container(const zx_container *c, const void *out)
{
    if (!c) return ZX_E_INVAL;
    if (c->dtype != ZX_BF16 && c->dtype != ZX_FP8_E4M3FN && c->dtype != ZX_E8M0) return ZX_E_UNSUPPORTED;
    if (c->n == 0) return ZX_OK;
    const uint64_t nblocks = (c->n + kBlock - 1) / kBlock;
    if (nblocks > 0x7FFFFFFFull || c->nsegs > 0xFFFFFFFFull || c->nsegs < nblocks) return ZX_E_INVAL;
    if (!out || !c->lengths || !c->degenerate || (!c->signmant && c->dtype != ZX_E8M0) || !c->stream || !c->block_bitoff || !c->block_seg || !c->seg_desc ||
        !c->gaps)
        return ZX_E_INVAL;
    if (!c->per_block && !c->dtab) return ZX_E_INVAL;
    if (!aligned16(out) || !aligned16(c->signmant) || !aligned16(c->stream) || !aligned16(c->dtab) || !aligned16(c->seg_desc))
        return ZX_E_INVAL;
    if (c->stream_words != zx_stream_words(c->total_bits)) return ZX_E_INVAL;
    return ZX_OK;
}

// One fast-decode launch over containers idx[0..m) of a batch, all of one codebook
// scope (per_block) and one dtype.
static zx_status launch_fast(const zx_container *all, void *const *all_outs, const uint32_t *idx, uint32_t m,
                             bool per_block, int dt, int cus, uint32_t max_workgroups, uint32_t *err, hipStream_t stream)
{
    zx_container cs[kMaxBatch];
    void *outs[kMaxBatch];
    const uint32_t count = m;
    for (uint32_t j = 0; j < m; ++j) {
        cs[j] = all[idx[j]];
        outs[j] = all_outs[idx[j]];
    }
    // the fast decode takes every batch; in its low-entropy mode when any container's
    // mean code length is below 2.3 bits (its segments then average over 3562
    // elements, beyond the ordinary stage), and always for E8M0 scales (mean codes near
    // 1.5 bits).  Per-block codebooks are decoded block by block, each block's table
    // built in LDS.
    bool low = dt == ZX_E8M0;
    for (uint32_t i = 0; i < count; ++i)
        if (cs[i].n && 10 * cs[i].total_bits < 23 * cs[i].n) low = true;
    // resident 512-thread workgroups
    uint64_t slots = (uint64_t)cus * (low ? kLowWgPerCu : kFastWgPerCu);
    if (max_workgroups != 0 && max_workgroups < slots) slots = max_workgroups;
    // resident workgroup slots for each container: its share of the slots by segment
    // count, rounded down, then the slots left over go to the largest remainders.  The
    // total never exceeds the resident slots, so every workgroup starts at once: one
    // more workgroup than fits would run its whole share after the others.
    uint64_t seg_total = 0;
    uint32_t nshare = 0;
    for (uint32_t i = 0; i < count; ++i)
        if (cs[i].n) { seg_total += cs[i].nsegs; ++nshare; }
    uint64_t share[kMaxBatch] = {};
    if (nshare) {
        if (slots < nshare) slots = nshare;
        uint64_t given = 0;
        uint64_t rem[kMaxBatch] = {};
        for (uint32_t i = 0; i < count; ++i) {
            if (cs[i].n == 0) continue;
            const uint64_t num = slots * cs[i].nsegs;
            share[i] = num / seg_total;
            rem[i] = num % seg_total;
            if (share[i] == 0) { share[i] = 1; rem[i] = 0; }
            given += share[i];
        }
        while (given < slots) {
            uint32_t best = count;
            for (uint32_t i = 0; i < count; ++i)
                if (cs[i].n && (best == count || rem[i] > rem[best])) best = i;
            if (best == count || rem[best] == 0) break;
            share[best] += 1;
            rem[best] = 0;
            given += 1;
        }
    }
    // Per-tensor codebooks whose shares hold at most 8 segments per slot: workgroups of
    // nw = 6..8 wavefronts, the fewest that give every wavefront one segment, so that
    // the resident slots fill evenly (BF16 4096 x 4096: 768 workgroups of 7 instead of
    // 672 of 8, which left 160 CUs with three workgroups and 96 with two).  Larger
    // shares take 8 and loop.
    uint32_t nw = kDecWaves;
    if (!per_block) {
        uint64_t need = kMinDecWaves;
        for (uint32_t i = 0; i < count; ++i) {
            if (cs[i].n == 0) continue;
            const uint64_t q = (cs[i].nsegs + share[i] - 1) / share[i];
            if (q > need) need = q;
        }
        if (need <= kDecWaves) nw = (uint32_t)need;
    }
    DecBatch batch;
    memset(&batch, 0, sizeof(batch));
    uint32_t wg = 0;
    uint32_t used = 0;
    for (uint32_t i = 0; i < count; ++i) {
        const zx_container &c = cs[i];
        if (c.n == 0) continue;
        DecTensor &T = batch.t[used++];
        T.signmant = c.signmant;
        T.stream = c.stream;
        T.block_bitoff = c.block_bitoff;
        T.block_seg = c.block_seg;
        T.seg_desc = c.seg_desc;
        T.gaps = c.gaps;
        T.lengths = c.lengths;
        T.degenerate = c.degenerate;
        T.dtab = reinterpret_cast<const DTab *>(c.dtab);
        T.out = outs[i];
        T.n = c.n;
        T.total_bits = c.total_bits;
        T.stream_words = c.stream_words;
        T.nsegs = (uint32_t)c.nsegs;
        T.nblocks = (uint32_t)((c.n + kBlock - 1) / kBlock);
        T.per_block = c.per_block ? 1u : 0u;
        T.wg_begin = wg;
        if (c.per_block) {
            T.wg_count = T.nblocks;   // one workgroup per block
            T.segs_per_wg = 0;
        } else {
            // at least one segment per wavefront of the workgroup
            uint64_t want = share[i];
            const uint64_t cap = (c.nsegs + nw - 1) / nw;
            if (want > cap) want = cap;
            if (want == 0) want = 1;
            T.segs_per_wg = (uint32_t)((c.nsegs + want - 1) / want);
            T.wg_count = (uint32_t)((c.nsegs + T.segs_per_wg - 1) / T.segs_per_wg);
        }
        wg += T.wg_count;
    }
    batch.count = used;
    if (used == 0) return ZX_OK;
    // Output at most half the 256 MB Infinity Cache goes out with streaming stores:
    // measured faster there (BF16 4096 x 4096: 19.2 -> 16.1 us; FP8 8192 x 8192:
    // 40.2 -> 38.3 us), while plain stores measured 2% faster on a 436 MB Llama-shaped
    // layer call.
    uint64_t out_bytes = 0;
    for (uint32_t i = 0; i < count; ++i) out_bytes += cs[i].n * (cs[i].dtype == ZX_BF16 ? 2u : 1u);
    const bool stream_out = out_bytes <= (128ull << 20);
    void (*kern)(const DecBatch, uint32_t *);
    if (per_block) {
        if (dt == ZX_E8M0)
            kern = stream_out ? k_decode_fast_blocks<ZX_E8M0, true, true, false> : k_decode_fast_blocks<ZX_E8M0, false, true, false>;
        else if (dt == ZX_BF16)
            kern = low ? (stream_out ? k_decode_fast_blocks<ZX_BF16, true, true, false> : k_decode_fast_blocks<ZX_BF16, false, true, false>)
                       : (stream_out ? k_decode_fast_blocks<ZX_BF16, true, false, false>
                                     : k_decode_fast_blocks<ZX_BF16, false, false, false>);
        else
            kern = low ? (stream_out ? k_decode_fast_blocks<ZX_FP8_E4M3FN, true, true, false>
                                     : k_decode_fast_blocks<ZX_FP8_E4M3FN, false, true, false>)
                       : (stream_out ? k_decode_fast_blocks<ZX_FP8_E4M3FN, true, false, false>
                                     : k_decode_fast_blocks<ZX_FP8_E4M3FN, false, false, false>);
    } else {
        if (dt == ZX_E8M0)
            kern = stream_out ? k_decode_fast<ZX_E8M0, true, true> : k_decode_fast<ZX_E8M0, false, true>;
        else if (dt == ZX_BF16)
            kern = low ? (stream_out ? k_decode_fast<ZX_BF16, true, true> : k_decode_fast<ZX_BF16, false, true>)
                       : (stream_out ? k_decode_fast<ZX_BF16, true, false> : k_decode_fast<ZX_BF16, false, false>);
        else
            kern = low ? (stream_out ? k_decode_fast<ZX_FP8_E4M3FN, true, true> : k_decode_fast<ZX_FP8_E4M3FN, false, true>)
                       : (stream_out ? k_decode_fast<ZX_FP8_E4M3FN, true, false>
                                     : k_decode_fast<ZX_FP8_E4M3FN, false, false>);
    }
    hipLaunchKernelGGL(kern, dim3(wg), dim3(nw * kWave), 0, stream, batch, err);
    return hipGetLastError() == hipSuccess ? ZX_OK : ZX_E_HIP;
}

extern "C" zx_status zx_decode_block_batch_wg(const zx_container *cs, void *const *outs, uint32_t count,
                                              uint32_t max_workgroups, uint32_t *err, hipStream_t stream)
{
    if (count == 0) return ZX_OK;
    if (!cs || !outs || count > (uint32_t)kMaxBatch) return ZX_E_INVAL;
    const int dt = cs[0].dtype;
    for (uint32_t i = 0; i < count; ++i) {
        const zx_status st = check_container(&cs[i], outs[i]);
        if (st != ZX_OK) return st;
        if (cs[i].dtype != dt) return ZX_E_INVAL;
    }
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    // per-tensor and per-block codebooks take separate kernels: a batch that holds both
    // is two launches on the stream
    uint32_t pt[kMaxBatch], pb[kMaxBatch];
    uint32_t npt = 0, npb = 0;
    for (uint32_t i = 0; i < count; ++i) {
        if (cs[i].per_block) pb[npb++] = i;
        else pt[npt++] = i;
    }
    if (npt) {
        const zx_status st = launch_fast(cs, outs, pt, npt, false, dt, cus, max_workgroups, err, stream);
        if (st != ZX_OK) return st;
    }
    if (npb) return launch_fast(cs, outs, pb, npb, true, dt, cus, max_workgroups, err, stream);
    return ZX_OK;
}

extern "C" zx_status zx_kv_decode_slots(const zx_kv_pool *pool, const uint32_t *slot_ids, uint32_t count, void *out,
                                        uint32_t *err, hipStream_t stream)
{
    zx_container c;
    zx_kv_sizes sz;
    if (!pool || zx_kv_slot_container(pool, 0, &c) != ZX_OK || zx_kv_slot_sizes((zx_dtype)pool->dtype, pool->cap_words, &sz) != ZX_OK)
        return ZX_E_INVAL;
    if (count == 0) return ZX_OK;
    if (!slot_ids || !out || !aligned16(out) || count > 0x7FFFFFFFu) return ZX_E_INVAL;
    DecBatch batch;
    memset(&batch, 0, sizeof(batch));
    DecTensor &T = batch.t[0];
    T.signmant = c.signmant;
    T.stream = c.stream;
    T.block_bitoff = c.block_bitoff;
    T.block_seg = c.block_seg;
    T.seg_desc = c.seg_desc;
    T.gaps = c.gaps;
    T.lengths = c.lengths;
    T.degenerate = c.degenerate;
    T.dtab = nullptr;
    T.out = out;
    T.n = c.n;
    T.total_bits = c.total_bits;
    T.stream_words = c.stream_words;
    T.nsegs = (uint32_t)c.nsegs;
    T.nblocks = 1;
    T.per_block = 1;
    T.wg_begin = 0;
    T.wg_count = count;
    T.segs_per_wg = 0;
    batch.count = 1;
    batch.slots.slot_ids = slot_ids;
    batch.slots.sm_bytes = sz.sm_bytes;
    batch.slots.stream_words = sz.stream_words;
    batch.slots.seg_stride = sz.seg_stride;
    batch.slots.out_bytes = pool->dtype == ZX_BF16 ? 2ull * kBlock : (uint64_t)kBlock;
    batch.slots.alphabet = sz.alphabet;
    batch.slots.n_slots = pool->n_slots;
    // a pool whose slots hold under 2.3 bits per element only has low-entropy blocks:
    // the low-entropy mode; otherwise the ordinary one (whose spare stage takes any
    // low-entropy segment)
    const bool low = 10ull * 32ull * pool->cap_words < 23ull * kBlock;
    void (*kern)(const DecBatch, uint32_t *) =
        pool->dtype == ZX_BF16 ? (low ? k_decode_fast_blocks<ZX_BF16, false, true, true>
                                      : k_decode_fast_blocks<ZX_BF16, false, false, true>)
                               : (low ? k_decode_fast_blocks<ZX_FP8_E4M3FN, false, true, true>
                                      : k_decode_fast_blocks<ZX_FP8_E4M3FN, false, false, true>);
    hipLaunchKernelGGL(kern, dim3(count), dim3(kDecThreads), 0, stream, batch, err);
    return hipGetLastError() == hipSuccess ? ZX_OK : ZX_E_HIP;
}

extern "C" zx_status zx_decode_block_batch(const zx_container *cs, void *const *outs, uint32_t count, uint32_t *err,
                                           hipStream_t stream)
{
    return zx_decode_block_batch_wg(cs, outs, count, 0, err, stream);
}

extern "C" zx_status zx_decode(const zx_container *c, void *out, uint32_t *err, hipStream_t stream)
{
    return zx_decode_block_batch_wg(c, &out, 1, 0, err, stream);
}

extern "C" const char *zx_status_string(zx_status s)
{
    switch (s) {
    case ZX_OK: return "ok";
    case ZX_E_INVAL: return "invalid argument";
    case ZX_E_UNSUPPORTED: return "unsupported dtype";
    case ZX_E_CODEBOOK: return "codebook error (length limit infeasible or data without a code)";
    case ZX_E_CORRUPT: return "corrupt container";
    case ZX_E_HIP: return "HIP launch failure";
    case ZX_E_NOSPACE: return "block does not fit its slot";
    case ZX_E_LIMIT: return "request larger than the library's fixed scratch";
    }
    return "unknown status";
}

extern "C" const char *zx_version(void) { return "zx 0.1 (container v1, gfx950)"; }
