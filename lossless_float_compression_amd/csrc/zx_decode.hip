// zx_decode.hip -- massively parallel decode of container v1 back to BF16 / FP8.
//
// Prior art on the DFloat11 article (方法介绍, three components) is a kernel with
// (1) compact lookup tables in on-chip memory, (2) two phases coordinated by small
// auxiliary variables that tell each thread where to read and write, and (3)
// decode of a whole transformer block per call.  The gfx950 design here:
//   * one wavefront decodes one segment: 64 chunks of 128 stream bits, lane l owns
//     chunk l and starts at the chunk's stored gap (the first code starting in it);
//   * lookup: the next 10 stream bits index a 1024-entry LDS table that yields up to
//     three whole codes; longer codes fall back to the canonical length limits;
//   * count pass, then a wavefront prefix scan of per-lane counts gives each lane
//     its output offset (the segment's first element is stored in the container);
//   * the lane decodes again, dropping exponents into a wavefront-private LDS stage
//     in output order; the write pass then streams sign/mantissa bytes, fuses them
//     with the staged exponents and issues 16-byte coalesced stores.
// Per-tensor codebooks load a prepared table; per-block codebooks (one workgroup
// per block) build theirs in LDS from the block's code lengths.
#include <cstring>

#include "zx_common.h"

namespace zxk {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = kDecWaves * kWave;
constexpr uint32_t kStageBytes = 4000;   // exponent stage per wavefront
// A segment whose exponents do not fit the stage at once (mean code length under
// two bits) is written in rounds of kRoundElems output positions.
constexpr uint32_t kRoundElems = 3968;
constexpr int kDecWgPerCu = 3;
constexpr int kDecMinWavesPerSimd = kDecWgPerCu * kDecWaves / 4;
constexpr int kMaxBatch = 16;

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

struct DecBatch {
    DecTensor t[kMaxBatch];
    uint32_t count;
};

typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

// Stream words of a lane's chunk, staged in LDS one column per lane: word t of
// lane l (the t-th word from the one holding the chunk's first bit) sits at
// 64 t + l.  In every window read each lane then hits its own bank.  A chunk
// starts less than 32 bits into its first word and a lane reads at most a 64-bit
// window starting inside its chunk, so 7 words per lane suffice.
constexpr uint32_t kLaneWords = 7;
constexpr uint32_t kSegWords = kLaneWords * 64;

struct SegWords {
    const uint32_t *w;   // LDS, this lane's column
    // 64 bits starting at chunk-relative bit p (counted from the first word's MSB)
    __device__ __forceinline__ uint64_t win(uint32_t p) const
    {
        const uint32_t t = p >> 5;
        const uint64_t v = ((uint64_t)w[t * 64] << 32) | w[(t + 1) * 64];
        return v << (p & 31);
    }
};

// Stage the segment's words: the wavefront loads stream words [W0, W0 + 260) with
// one coalesced 16-byte load per lane (plus the tail words), and each word goes to
// the lanes that need it: lane l needs words 4 l .. 4 l + 6.
__device__ __forceinline__ void stage_seg_words(uint32_t *sw, const uint32_t *stream, uint64_t words, uint64_t W0)
{
    const uint32_t lane = lane_id();
    const uint64_t k = W0 + 4ull * lane;
    u32x4_a4 v;
    if (k + 4 <= words) {
        v = *reinterpret_cast<const u32x4_a4 *>(stream + k);
    } else {
        v.x = k < words ? stream[k] : 0u;
        v.y = k + 1 < words ? stream[k + 1] : 0u;
        v.z = k + 2 < words ? stream[k + 2] : 0u;
        v.w = k + 3 < words ? stream[k + 3] : 0u;
    }
    uint32_t *own = sw + lane;                    // words 4l .. 4l+3 are this lane's 0..3
    own[0] = v.x; own[64] = v.y; own[128] = v.z; own[192] = v.w;
    if (lane > 0) {                               // and the previous lane's 4..6
        uint32_t *prev = sw + lane - 1;
        prev[256] = v.x; prev[320] = v.y; prev[384] = v.z;
    }
    if (lane < 3) {                               // words 256..258 finish lane 63
        const uint64_t t = W0 + 256 + lane;
        sw[64 * (4 + lane) + 63] = t < words ? stream[t] : 0u;
    }
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

// Write pass pieces: 8 BF16 or 16 FP8 elements per lane per step, i.e. 8 bytes of
// sign/mantissa in and one 16-byte store out.
template <int DT>
struct Piece {
    static constexpr uint32_t kElems = DT == ZX_BF16 ? 8 : 16;
};

template <int DT>
__device__ __forceinline__ uint2 load_sm(const uint8_t *sm_block, uint32_t i)
{
    return *reinterpret_cast<const uint2 *>(sm_block + (DT == ZX_BF16 ? i : i / 2));
}

// Exponents of one piece, from the stage or a 0-bit block's single symbol.
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

// BF16: from sign/mantissa bytes S and exponent bytes E (4 elements each) make the
// two output words of elements (2h, 2h+1): byte-permute S into [s,s] per element
// (sign lands on bit 15, mantissa on bits 0..6 after the mask) and E into
// [0,e] per element, shifted to bits 7..14.
__device__ __forceinline__ uint32_t fuse_bf16_pair(uint32_t S, uint32_t E, uint32_t sel_s, uint32_t sel_e)
{
    const uint32_t sd = __builtin_amdgcn_perm(0u, S, sel_s);
    const uint32_t ed = __builtin_amdgcn_perm(0u, E, sel_e);
    return (sd & 0x807F807Fu) | (ed << 7);
}

// FP8: four sign|mantissa nibbles N (element k at bits 4k..4k+3) and four exponent
// bytes E.  Each output byte is (sign << 7) | (exp << 3) | mant.
__device__ __forceinline__ uint32_t fuse_fp8_quad(uint32_t N, uint32_t E)
{
    const uint32_t t = __builtin_amdgcn_perm(0u, N, 0x01010000u);       // [n23, n23, n01, n01]
    const uint32_t x = (t & 0x000F000Fu) | ((t >> 4) & 0x0F000F00u);    // one nibble per byte
    return x + (x & 0x08080808u) * 15u + (E << 3);                       // sign bit 3 -> bit 7
}

template <int DT>
__device__ __forceinline__ void store_piece(void *out_block, uint32_t i, uint2 smv, uint4 e)
{
    if (DT == ZX_BF16) {
        uint4 r;
        r.x = fuse_bf16_pair(smv.x, e.x, 0x01010000u, 0x0C010C00u);
        r.y = fuse_bf16_pair(smv.x, e.x, 0x03030202u, 0x0C030C02u);
        r.z = fuse_bf16_pair(smv.y, e.y, 0x01010000u, 0x0C010C00u);
        r.w = fuse_bf16_pair(smv.y, e.y, 0x03030202u, 0x0C030C02u);
        *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(out_block) + i) = r;
    } else {
        uint4 r;
        r.x = fuse_fp8_quad(smv.x & 0xFFFFu, e.x);
        r.y = fuse_fp8_quad(smv.x >> 16, e.y);
        r.z = fuse_fp8_quad(smv.y & 0xFFFFu, e.z);
        r.w = fuse_fp8_quad(smv.y >> 16, e.w);
        *reinterpret_cast<uint4 *>(reinterpret_cast<uint8_t *>(out_block) + i) = r;
    }
}



// Elements of the cut pieces at the two range ends, one element per lane: lane t
// (< P) takes element t of the head piece, lane P + t element t of the tail piece.
template <int DT>
__device__ __forceinline__ void write_cut_pieces(void *out_block, const uint8_t *sm_block, uint32_t i_begin, uint32_t i_end,
                                                 const uint8_t *stage, uint32_t sbase, bool degen, uint32_t degen_sym)
{
    constexpr uint32_t P = Piece<DT>::kElems;
    const uint32_t lane = lane_id();
    const uint32_t q_head = i_begin / P;
    const uint32_t q_tail = (i_end - 1) / P;
    const bool head_cut = (i_begin % P) != 0 || (q_head == q_tail && (i_end % P) != 0);
    const bool tail_cut = (i_end % P) != 0 && q_tail != q_head;
    uint32_t ii = ~0u;
    if (lane < P && head_cut) ii = q_head * P + lane;
    if (lane >= P && lane < 2 * P && tail_cut) ii = q_tail * P + (lane - P);
    if (ii != ~0u && ii >= i_begin && ii < i_end) {
        const uint32_t smb = sm_block[DT == ZX_BF16 ? ii : ii / 2];
        const uint32_t ex = degen ? degen_sym : stage[ii - sbase];
        if (DT == ZX_BF16) {
            reinterpret_cast<uint16_t *>(out_block)[ii] = (uint16_t)fuse_bf16_pair(smb, ex, 0x0C0C0000u, 0x0C0C0C00u);
        } else {
            const uint32_t nn = (ii & 1) ? (smb >> 4) : (smb & 0xFu);
            reinterpret_cast<uint8_t *>(out_block)[ii] = (uint8_t)(fuse_fp8_quad(nn, ex) & 0xFFu);
        }
    }
}

constexpr int kWriteBatch = 7;   // whole pieces per lane whose loads are issued together
// Whole pieces of [i_begin, i_end) for this lane: q = qf_begin + lane + 64 k.
__device__ __forceinline__ uint32_t first_whole(uint32_t i_begin, uint32_t P) { return (i_begin + P - 1) / P; }

// Write block elements [i_begin, i_end); the exponent of element i is stage[i - sbase]
// (or `degen_sym` for a 0-bit block).  Whole pieces: sign/mantissa loads of
// kWriteBatch pieces per lane are issued before any is used, then each piece is
// fused and written with one 16-byte store.  The (at most two) cut pieces at the
// range ends are written one element per lane.
template <int DT>
__device__ __forceinline__ void write_range(void *out_block, const uint8_t *sm_block, uint32_t i_begin, uint32_t i_end,
                                            const uint8_t *stage, uint32_t sbase, bool degen, uint32_t degen_sym)
{
    constexpr uint32_t P = Piece<DT>::kElems;
    if (i_begin >= i_end) return;
    const uint32_t lane = lane_id();
    const uint32_t qf_begin = first_whole(i_begin, P);
    const uint32_t qf_end = i_end / P;
    const uint32_t dsplat = degen_sym * 0x01010101u;
    for (uint32_t qb = qf_begin; qb < qf_end; qb += kWave * kWriteBatch) {
        uint2 smv[kWriteBatch];
#pragma unroll
        for (int k = 0; k < kWriteBatch; ++k) {
            const uint32_t q = qb + lane + k * kWave;
            smv[k] = make_uint2(0, 0);
            if (q < qf_end) smv[k] = load_sm<DT>(sm_block, q * P);
        }
#pragma unroll
        for (int k = 0; k < kWriteBatch; ++k) {
            const uint32_t q = qb + lane + k * kWave;
            if (q < qf_end) store_piece<DT>(out_block, q * P, smv[k], piece_exps<DT>(stage + (q * P - sbase), degen, dsplat));
        }
    }
    write_cut_pieces<DT>(out_block, sm_block, i_begin, i_end, stage, sbase, degen, degen_sym);
}

__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Decode one segment with one wavefront.
template <int DT>
__device__ void decode_segment(const DecTensor &T, const DTab &tab, uint8_t *stage, uint32_t *swords, uint32_t s,
                               uint32_t *err)
{
    constexpr uint32_t A = alphabet_of(DT);
    constexpr uint32_t P = Piece<DT>::kElems;
    const uint32_t lane = lane_id();
    const uint32_t b = T.seg_desc[2 * (uint64_t)s];
    const uint32_t e0 = T.seg_desc[2 * (uint64_t)s + 1];
    if (b >= T.nblocks) { report(err, ZX_E_CORRUPT); return; }
    const uint64_t G = T.block_bitoff[b];
    const uint64_t Gn = T.block_bitoff[b + 1];
    const uint32_t sb = T.block_seg[b];
    const uint32_t sbn = T.block_seg[b + 1];
    const uint64_t lo = (uint64_t)b * kBlock;
    const uint32_t nb = (uint32_t)(((lo + kBlock < T.n) ? lo + kBlock : T.n) - lo);
    if (Gn < G || Gn > T.total_bits || s < sb || s >= sbn || sbn > T.nsegs || Gn - G > (uint64_t)nb * kMaxLen) {
        report(err, ZX_E_CORRUPT);
        return;
    }
    const uint32_t bits = (uint32_t)(Gn - G);
    const uint32_t j = s - sb;
    const uint32_t e_end = (s + 1 < sbn) ? T.seg_desc[2 * (uint64_t)(s + 1) + 1] : nb;
    if (e0 > e_end || e_end > nb) { report(err, ZX_E_CORRUPT); return; }
    const uint8_t *sm_block = T.signmant + (DT == ZX_BF16 ? lo : lo / 2);
    void *out_block = reinterpret_cast<uint8_t *>(T.out) + lo * (DT == ZX_BF16 ? 2 : 1);
    const uint32_t sbase = e0 & ~15u;   // 16-aligned element that stage byte 0 stands for

    if (bits == 0) {
        const uint32_t d = T.degenerate[T.per_block ? b : 0];
        if (d >= A || e0 != 0 || e_end != nb) { report(err, ZX_E_CORRUPT); return; }
        write_range<DT>(out_block, sm_block, e0, e_end, stage, sbase, true, d);
        return;
    }
    if (!tab.ok) { report(err, ZX_E_CORRUPT); return; }

    const uint32_t nch = (bits + kChunkBits - 1) / kChunkBits;
    const uint32_t ch = j * kSegChunks + lane;
    const uint32_t gap = (ch < nch) ? T.gaps[(uint64_t)s * kSegChunks + lane] : ZX_NO_GAP;
    bool work = gap != ZX_NO_GAP;
    bool lane_bad = false;
    if (work && gap >= kMaxLen) { work = false; lane_bad = true; }
    // chunk-relative end: the lane decodes the codes starting in [gap, cend)
    const uint32_t cend = (ch * kChunkBits + kChunkBits < bits) ? kChunkBits : bits - ch * kChunkBits;
    if (work && gap >= cend) { work = false; lane_bad = true; }
    // chunk-relative bit coordinates from the MSB of the word holding the chunk's
    // first bit: the chunk starts at b0 < 32
    const uint64_t cbit = G + (uint64_t)ch * kChunkBits;
    const uint32_t b0 = (uint32_t)(cbit & 31);
    stage_seg_words(swords, T.stream, T.stream_words, (G >> 5) + (uint64_t)j * (kSegBits / 32));
    wave_sync();
    const SegWords sw{swords + lane};
    const uint32_t start = work ? b0 + gap : 0;
    const uint32_t lim = work ? b0 + cend : 0;

    // ---- count pass.  Main phase: while a whole window lies inside the chunk, every
    //      code the table returns starts inside it.  Tail phase: one code at a time.
    //      A code longer than the window reads as a zero entry, so its lane stalls;
    //      the inner loops run while some lane progresses, then stalled lanes take
    //      their long code from the canonical length limits.
    uint32_t cnt = 0;
    uint32_t pos = work ? start : 0;
    for (;;) {
        bool act = pos + kLutBits <= lim;
        if (__ballot(act) == 0) break;
        bool progress;
        do {
            const uint32_t idx = act ? (uint32_t)(sw.win(pos) >> (64 - kLutBits)) : kLutSize;
            const uint32_t e = tab.lut[idx];
            const uint32_t adv = (e >> 24) & 0xFu;
            progress = adv != 0;   // a zero advance (long code, or a damaged table) stalls
            cnt += e >> 28;
            pos += adv;
            act = pos + kLutBits <= lim;
        } while (__ballot(progress && act) != 0);
        if (act && !progress) {   // stalled at a long code
            uint32_t L = slow_len(tab, (uint32_t)(sw.win(pos) >> 32));
            if (L > kMaxLen) { lane_bad = true; L = lim - pos; }
            cnt += 1;
            pos += L;
        }
    }
    for (;;) {
        bool act = pos < lim;
        if (__ballot(act) == 0) break;
        bool progress;
        do {
            const uint32_t idx = act ? (uint32_t)(sw.win(pos) >> (64 - kLutBits)) : kLutSize;
            const uint32_t L = tab.first_len[idx];
            progress = L != 0;
            cnt += progress ? 1u : 0u;
            pos += L;
            act = pos < lim;
        } while (__ballot(progress && act) != 0);
        if (act && !progress) {
            uint32_t L = slow_len(tab, (uint32_t)(sw.win(pos) >> 32));
            if (L > kMaxLen) { lane_bad = true; L = lim - pos; }
            cnt += 1;
            pos += L;
        }
    }
    // codes of one chunk must end exactly where the next chunk's first code
    // starts (or at the block end), as the stored gaps claim
    uint32_t gap_next = __shfl_down(gap, 1, kWave);
    if (lane == kWave - 1) gap_next = (ch + 1 < nch) ? T.gaps[(uint64_t)(s + 1) * kSegChunks] : ZX_NO_GAP;
    if (work && !lane_bad) {
        const uint32_t expect = (ch + 1 < nch && gap_next != ZX_NO_GAP) ? b0 + kChunkBits + gap_next : b0 + (bits - ch * kChunkBits);
        if (pos != expect) lane_bad = true;
    }
    uint32_t total;
    const uint32_t off = wave_excl_scan(cnt, total);
    if (__ballot(lane_bad) != 0 || e0 + total != e_end) { report(err, ZX_E_CORRUPT); return; }

    const uint32_t t0 = e0 - sbase;   // stage position of the segment's first element
    if (t0 + total + 2 <= kStageBytes - 4) {   // the last 4 bytes are the dummy store slot
        // ---- decode pass, one round: each lookup stores all its symbols; a lane's
        //      last lookup may spill up to two bytes onto the next lanes' first
        //      positions, which those lanes restore right after
        uint32_t wp = t0 + off;
        uint32_t done = 0;
        pos = start;
        uint8_t *const dummy = stage + kStageBytes - 4;   // where lanes that are done store
        for (;;) {
            bool act = done < cnt;
            if (__ballot(act) == 0) break;
            bool progress;
            do {
                const uint32_t idx = act ? (uint32_t)(sw.win(pos) >> (64 - kLutBits)) : kLutSize;
                const uint32_t e = tab.lut[idx];
                uint8_t *const d = act ? stage + wp : dummy;
                d[0] = (uint8_t)e;
                d[1] = (uint8_t)(e >> 8);
                d[2] = (uint8_t)(e >> 16);
                const uint32_t adv = (e >> 24) & 0xFu;
                progress = adv != 0;
                const uint32_t ns = e >> 28;
                wp += ns;
                done += ns;
                pos += adv;
                act = done < cnt;
            } while (__ballot(progress && act) != 0);
            if (act && !progress) {
                const uint32_t v = (uint32_t)(sw.win(pos) >> 32);
                const uint32_t L = slow_len(tab, v);
                stage[wp] = (uint8_t)slow_sym(tab, v, L);
                wp += 1;
                done += 1;
                pos += L;
            }
        }
        wave_sync();
        if (cnt) {
            uint32_t p = start;
            const uint32_t first = cnt < 2 ? cnt : 2;
            for (uint32_t k = 0; k < first; ++k) {
                const uint64_t x = sw.win(p);
                const uint32_t idx = (uint32_t)(x >> (64 - kLutBits));
                uint32_t L = tab.first_len[idx];
                uint32_t sy;
                if (L) {
                    sy = tab.lut[idx] & 0xFFu;
                } else {
                    const uint32_t v = (uint32_t)(x >> 32);
                    L = slow_len(tab, v);
                    sy = slow_sym(tab, v, L);
                }
                stage[t0 + off + k] = (uint8_t)sy;
                p += L;
            }
        }
        wave_sync();
        write_range<DT>(out_block, sm_block, e0, e_end, stage, sbase, false, 0);
    } else {
        // ---- several rounds of kRoundElems stage positions; exact writes
        for (uint32_t r0 = 0; r0 < t0 + total; r0 += kRoundElems) {
            const uint32_t r1 = r0 + kRoundElems;
            if (cnt) {
                uint32_t p = start;
                uint32_t t = t0 + off;
                uint32_t done = 0;
                while (done < cnt && t < r1) {
                    const uint64_t x = sw.win(p);
                    const uint32_t idx = (uint32_t)(x >> (64 - kLutBits));
                    uint32_t L = tab.first_len[idx];
                    uint32_t sy;
                    if (L) {
                        sy = tab.lut[idx] & 0xFFu;
                    } else {
                        const uint32_t v = (uint32_t)(x >> 32);
                        L = slow_len(tab, v);
                        sy = slow_sym(tab, v, L);
                    }
                    if (t >= r0) stage[t - r0] = (uint8_t)sy;
                    p += L;
                    ++t;
                    ++done;
                }
            }
            wave_sync();
            const uint32_t ib = sbase + (r0 > t0 ? r0 : t0);
            const uint32_t ie = sbase + (r1 < t0 + total ? r1 : t0 + total);
            write_range<DT>(out_block, sm_block, ib, ie, stage, sbase + r0, false, 0);
            wave_sync();
        }
    }
}

template <int DT>
__global__ __launch_bounds__(kDecThreads, kDecMinWavesPerSimd) void k_decode(const DecBatch batch, uint32_t *err)
{
    constexpr uint32_t A = alphabet_of(DT);
    __shared__ DTab tab;
    __shared__ __align__(16) uint8_t stage_all[kDecWaves * kStageBytes];
    __shared__ __align__(16) uint32_t words_all[kDecWaves * kSegWords];
    // three workgroups of this size were measured to fit a CU; 54 KB ones were not
    static_assert(sizeof(DTab) + sizeof(stage_all) + sizeof(words_all) <= 52224, "decode workgroup LDS budget");
    static_assert(sizeof(Canon) <= sizeof(stage_all), "Canon is built inside the stage area");

    const uint32_t g = blockIdx.x;
    uint32_t t = 0;
    while (t + 1 < batch.count && g >= batch.t[t + 1].wg_begin) ++t;
    const DecTensor &T = batch.t[t];
    const uint32_t lg = g - T.wg_begin;
    const uint32_t tid = threadIdx.x;
    uint32_t s_begin, s_end;
    if (T.per_block) {
        const uint32_t b = lg;
        s_begin = T.block_seg[b];
        s_end = T.block_seg[b + 1];
        if (s_end > T.nsegs || s_begin > s_end) { s_end = s_begin; if (tid == 0) report(err, ZX_E_CORRUPT); }
        Canon &c = *reinterpret_cast<Canon *>(stage_all);
        canon_build(T.lengths + (uint64_t)b * A, A, c);
        dtab_fill(c, tab);
        __syncthreads();
    } else {
        s_begin = lg * T.segs_per_wg;
        s_end = s_begin + T.segs_per_wg;
        if (s_end > T.nsegs) s_end = T.nsegs;
        const uint4 *src = reinterpret_cast<const uint4 *>(T.dtab);
        uint4 *dst = reinterpret_cast<uint4 *>(&tab);
        for (uint32_t i = tid; i < sizeof(DTab) / 16; i += kDecThreads) dst[i] = src[i];
        __syncthreads();
    }
    const uint32_t wave = tid / kWave;
    uint8_t *stage = stage_all + wave * kStageBytes;
    uint32_t *swords = words_all + wave * kSegWords;
    for (uint32_t s = s_begin + wave; s < s_end; s += kDecWaves) decode_segment<DT>(T, tab, stage, swords, s, err);
}

__global__ __launch_bounds__(256) void k_build_dtab(const uint8_t *__restrict__ lengths, uint32_t A, DTab *__restrict__ out)
{
    __shared__ Canon c;
    canon_build(lengths, A, c);
    dtab_fill(c, *out);
}

}  // namespace zxk

using namespace zxk;

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

extern "C" size_t zx_decode_table_bytes(void) { return sizeof(DTab); }

extern "C" zx_status zx_build_decode_table(zx_dtype dtype, const uint8_t *lengths, uint32_t *dtab, hipStream_t stream)
{
    if (dtype != ZX_BF16 && dtype != ZX_FP8_E4M3FN) return ZX_E_UNSUPPORTED;
    if (!lengths || !dtab || !aligned16(dtab)) return ZX_E_INVAL;
    hipLaunchKernelGGL(k_build_dtab, dim3(1), dim3(256), 0, stream, lengths, alphabet_of(dtype), reinterpret_cast<DTab *>(dtab));
    return hipGetLastError() == hipSuccess ? ZX_OK : ZX_E_HIP;
}

static zx_status check_container(const zx_container *c, const void *out)
{
    if (!c) return ZX_E_INVAL;
    if (c->dtype != ZX_BF16 && c->dtype != ZX_FP8_E4M3FN) return ZX_E_UNSUPPORTED;
    if (c->n == 0) return ZX_OK;
    const uint64_t nblocks = (c->n + kBlock - 1) / kBlock;
    if (nblocks > 0x7FFFFFFFull || c->nsegs > 0xFFFFFFFFull || c->nsegs < nblocks) return ZX_E_INVAL;
    if (!out || !c->lengths || !c->degenerate || !c->signmant || !c->stream || !c->block_bitoff || !c->block_seg || !c->seg_desc ||
        !c->gaps)
        return ZX_E_INVAL;
    if (!c->per_block && !c->dtab) return ZX_E_INVAL;
    if (!aligned16(out) || !aligned16(c->signmant) || !aligned16(c->stream) || !aligned16(c->dtab) || !aligned16(c->seg_desc))
        return ZX_E_INVAL;
    if (c->stream_words != zx_stream_words(c->total_bits)) return ZX_E_INVAL;
    return ZX_OK;
}

extern "C" zx_status zx_decode_block_batch(const zx_container *cs, void *const *outs, uint32_t count, uint32_t *err,
                                           hipStream_t stream)
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
    if (hipGetDevice(&dev) == hipSuccess) hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const uint64_t slots = (uint64_t)cus * kDecWgPerCu;   // resident 512-thread workgroups per CU
    uint64_t seg_total = 0;
    for (uint32_t i = 0; i < count; ++i)
        if (!cs[i].per_block) seg_total += cs[i].nsegs;
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
            T.wg_count = T.nblocks;
            T.segs_per_wg = 0;
        } else {
            // share the resident workgroup slots in proportion to segment counts,
            // with at least one wavefront's worth of segments per workgroup
            uint64_t want = (slots * c.nsegs + seg_total - 1) / (seg_total ? seg_total : 1);
            const uint64_t cap = (c.nsegs + kDecWaves - 1) / kDecWaves;
            if (want > cap) want = cap;
            if (want == 0) want = 1;
            T.segs_per_wg = (uint32_t)((c.nsegs + want - 1) / want);
            T.wg_count = (uint32_t)((c.nsegs + T.segs_per_wg - 1) / T.segs_per_wg);
        }
        wg += T.wg_count;
    }
    batch.count = used;
    if (used == 0) return ZX_OK;
    if (dt == ZX_BF16)
        hipLaunchKernelGGL(k_decode<ZX_BF16>, dim3(wg), dim3(kDecThreads), 0, stream, batch, err);
    else
        hipLaunchKernelGGL(k_decode<ZX_FP8_E4M3FN>, dim3(wg), dim3(kDecThreads), 0, stream, batch, err);
    return hipGetLastError() == hipSuccess ? ZX_OK : ZX_E_HIP;
}

extern "C" zx_status zx_decode(const zx_container *c, void *out, uint32_t *err, hipStream_t stream)
{
    return zx_decode_block_batch(c, &out, 1, err, stream);
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
    }
    return "unknown status";
}

extern "C" const char *zx_version(void) { return "zx 0.1 (container v1, gfx950)"; }
