// zx_decode.hip -- massively parallel decode of container v1 back to BF16 / FP8.
//
// Prior art on the DFloat11 article (方法介绍, three components) is a kernel with
// (1) compact lookup tables in on-chip memory, (2) two phases coordinated by small
// auxiliary variables that tell each thread where to read and write, and (3)
// decode of a whole transformer block per call.  The gfx950 design here:
//   * one wavefront decodes one segment: 64 chunks of 128 stream bits, lane l owns
//     chunk l and starts at the chunk's stored gap (the first code starting in it);
//   * lookup: the next 11 stream bits index a 2048-entry LDS table that yields up to
//     two whole codes; longer codes fall back to the canonical length limits;
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
constexpr uint32_t kStageBytes = kSegChunks * kChunkBits + 16;   // <= 8192 codes + alignment slack
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

// Left-aligned 64-bit bit buffer over the stream: bit 63 is the next stream bit.
struct BitReader {
    uint64_t buf;
    uint32_t nbits;
    uint64_t next;
    const uint32_t *s;
    uint64_t wmax;
    __device__ __forceinline__ void init(const uint32_t *stream, uint64_t words, uint64_t pos)
    {
        s = stream;
        wmax = words - 1;
        const uint64_t w = pos >> 5;
        const uint32_t off = (uint32_t)(pos & 31);
        const uint64_t w0 = s[w < wmax ? w : wmax];
        const uint64_t w1 = s[w + 1 < wmax ? w + 1 : wmax];
        buf = ((w0 << 32) | w1) << off;
        nbits = 64 - off;
        next = w + 2;
    }
    __device__ __forceinline__ void refill()
    {
        if (nbits < 32) {
            const uint64_t wd = s[next < wmax ? next : wmax];
            buf |= wd << (32 - nbits);
            nbits += 32;
            ++next;
        }
    }
    __device__ __forceinline__ void skip(uint32_t k)
    {
        buf <<= k;
        nbits -= k;
    }
};

__device__ __forceinline__ uint32_t fuse2_bf16(uint32_t s16, uint32_t e16)
{
    // element a in the low half, b in the high half: sign -> bit 15, exponent -> bits 7..14
    const uint32_t s2 = (s16 & 0xFFu) | ((s16 & 0xFF00u) << 8);
    const uint32_t e2 = (e16 & 0xFFu) | ((e16 & 0xFF00u) << 8);
    return ((s2 * 0x0101u) & 0x807F807Fu) | (e2 << 7);
}

__device__ __forceinline__ uint32_t fuse4_fp8(uint32_t nib16, uint32_t e4)
{
    // four sign|mantissa nibbles (element k at bits 4k..4k+3) and four exponent bytes
    const uint32_t x = (nib16 & 0xFu) | ((nib16 & 0xF0u) << 4) | ((nib16 & 0xF00u) << 8) | ((nib16 & 0xF000u) << 12);
    return ((x & 0x08080808u) << 4) | (x & 0x07070707u) | (e4 << 3);
}

// Decode one segment with one wavefront.
template <int DT>
__device__ void decode_segment(const DecTensor &T, const DTab &tab, uint8_t *stage, uint32_t s, uint32_t *err)
{
    constexpr uint32_t A = alphabet_of(DT);
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

    uint32_t total = 0;
    uint32_t degen_sym = 0;
    const bool degen = (bits == 0);
    if (degen) {
        const uint32_t d = T.degenerate[T.per_block ? b : 0];
        if (d >= A || e0 != 0 || e_end != nb) { report(err, ZX_E_CORRUPT); return; }
        degen_sym = d;
        total = nb;
    } else {
        if (!tab.ok) { report(err, ZX_E_CORRUPT); return; }
        const uint32_t nch = (bits + kChunkBits - 1) / kChunkBits;
        const uint32_t ch = j * kSegChunks + lane;
        const uint32_t gap = (ch < nch) ? T.gaps[(uint64_t)s * kSegChunks + lane] : ZX_NO_GAP;
        bool work = gap != ZX_NO_GAP;
        bool lane_bad = false;
        if (work && gap >= kMaxLen) { work = false; lane_bad = true; }
        const uint64_t start = G + (uint64_t)ch * kChunkBits + gap;
        const uint64_t cend = (uint64_t)ch * kChunkBits + kChunkBits;
        const uint64_t end = G + (cend < bits ? cend : bits);
        if (work && start >= end) { work = false; lane_bad = true; }
        // ---- count pass
        uint32_t cnt = 0;
        uint64_t pos_end = start;
        if (work) {
            BitReader br;
            br.init(T.stream, T.stream_words, start);
            uint64_t pos = start;
            while (pos < end) {
                br.refill();
                const uint32_t e = tab.lut[br.buf >> (64 - kLutBits)];
                const uint32_t ns = e >> 24;
                uint32_t adv;
                if (ns == 0) {
                    const uint32_t L = canon_len(tab.lim, (uint32_t)(br.buf >> 32), kLutBits + 1);
                    if (L > kMaxLen) { lane_bad = true; break; }
                    adv = L;
                    cnt += 1;
                } else {
                    const uint32_t L0 = (e >> 16) & 0xFu;
                    const bool two = (ns == 2) && (pos + L0 < end);
                    adv = two ? ((e >> 20) & 0xFu) : L0;
                    cnt += two ? 2u : 1u;
                    if (L0 == 0 || adv < L0) { lane_bad = true; break; }   // a damaged table must not stall
                }
                br.skip(adv);
                pos += adv;
            }
            pos_end = pos;
        }
        // codes of one chunk must end exactly where the next chunk's first code
        // starts (or at the block end), as the stored gaps claim
        uint32_t gap_next = __shfl_down(gap, 1, kWave);
        if (lane == kWave - 1) gap_next = (ch + 1 < nch) ? T.gaps[(uint64_t)(s + 1) * kSegChunks] : ZX_NO_GAP;
        if (work && !lane_bad) {
            const uint64_t expect = (ch + 1 < nch && gap_next != ZX_NO_GAP) ? G + (uint64_t)(ch + 1) * kChunkBits + gap_next
                                                                              : G + bits;
            if (pos_end != expect) lane_bad = true;
        }
        uint32_t off = wave_excl_scan(cnt, total);
        if (__ballot(lane_bad) != 0 || e0 + total != e_end) { report(err, ZX_E_CORRUPT); return; }
        // ---- decode pass: exponents into the stage, in output order
        if (work) {
            BitReader br;
            br.init(T.stream, T.stream_words, start);
            uint64_t pos = start;
            uint32_t wp = (e0 & 7u) + off;
            while (pos < end) {
                br.refill();
                const uint32_t e = tab.lut[br.buf >> (64 - kLutBits)];
                const uint32_t ns = e >> 24;
                uint32_t adv;
                if (ns == 0) {
                    const uint32_t v = (uint32_t)(br.buf >> 32);
                    const uint32_t L = canon_len(tab.lim, v, kLutBits + 1);
                    adv = L;
                    stage[wp++] = tab.sym[(uint32_t)(tab.base[L] + (int32_t)(v >> (32 - L))) & 0xFFu];
                } else {
                    const uint32_t L0 = (e >> 16) & 0xFu;
                    const bool two = (ns == 2) && (pos + L0 < end);
                    stage[wp++] = (uint8_t)e;
                    if (two) stage[wp++] = (uint8_t)(e >> 8);
                    adv = two ? ((e >> 20) & 0xFu) : L0;
                }
                br.skip(adv);
                pos += adv;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    // ---- write pass over block elements [e0, e_end)
    const uint32_t sbase = e0 & ~7u;   // stage byte k holds element sbase + k
    const uint32_t g_begin = e0 >> 3;
    const uint32_t g_end = (e_end + 7) >> 3;
    const uint32_t dsplat = degen_sym * 0x01010101u;
    if (DT == ZX_BF16) {
        uint16_t *out = reinterpret_cast<uint16_t *>(T.out) + lo;
        const uint8_t *sm = T.signmant + lo;
        for (uint32_t g = g_begin + lane; g < g_end; g += kWave) {
            const uint32_t i = g * 8;
            if (i >= e0 && i + 8 <= e_end) {
                const uint2 s8 = *reinterpret_cast<const uint2 *>(sm + i);
                uint32_t ea, eb;
                if (degen) {
                    ea = eb = dsplat;
                } else {
                    const uint2 e8 = *reinterpret_cast<const uint2 *>(stage + (i - sbase));
                    ea = e8.x;
                    eb = e8.y;
                }
                uint4 o;
                o.x = fuse2_bf16(s8.x & 0xFFFFu, ea & 0xFFFFu);
                o.y = fuse2_bf16(s8.x >> 16, ea >> 16);
                o.z = fuse2_bf16(s8.y & 0xFFFFu, eb & 0xFFFFu);
                o.w = fuse2_bf16(s8.y >> 16, eb >> 16);
                *reinterpret_cast<uint4 *>(out + i) = o;
            } else {
                for (uint32_t k = 0; k < 8; ++k) {
                    const uint32_t ii = i + k;
                    if (ii >= e0 && ii < e_end) {
                        const uint32_t ex = degen ? degen_sym : stage[ii - sbase];
                        out[ii] = (uint16_t)(fuse2_bf16(sm[ii], ex) & 0xFFFFu);
                    }
                }
            }
        }
    } else {
        uint8_t *out = reinterpret_cast<uint8_t *>(T.out) + lo;
        const uint8_t *nib = T.signmant + lo / 2;
        for (uint32_t g = g_begin + lane; g < g_end; g += kWave) {
            const uint32_t i = g * 8;
            if (i >= e0 && i + 8 <= e_end) {
                const uint32_t n8 = *reinterpret_cast<const uint32_t *>(nib + i / 2);
                uint32_t ea, eb;
                if (degen) {
                    ea = eb = dsplat;
                } else {
                    const uint2 e8 = *reinterpret_cast<const uint2 *>(stage + (i - sbase));
                    ea = e8.x;
                    eb = e8.y;
                }
                uint2 o;
                o.x = fuse4_fp8(n8 & 0xFFFFu, ea);
                o.y = fuse4_fp8(n8 >> 16, eb);
                *reinterpret_cast<uint2 *>(out + i) = o;
            } else {
                for (uint32_t k = 0; k < 8; ++k) {
                    const uint32_t ii = i + k;
                    if (ii >= e0 && ii < e_end) {
                        const uint32_t nb2 = nib[ii / 2];
                        const uint32_t nn = (ii & 1) ? (nb2 >> 4) : (nb2 & 0xFu);
                        const uint32_t ex = degen ? degen_sym : stage[ii - sbase];
                        out[ii] = (uint8_t)(fuse4_fp8(nn, ex) & 0xFFu);
                    }
                }
            }
        }
    }
}

template <int DT>
__global__ __launch_bounds__(kDecThreads) void k_decode(const DecBatch batch, uint32_t *err)
{
    constexpr uint32_t A = alphabet_of(DT);
    __shared__ DTab tab;
    __shared__ __align__(16) uint8_t stage_all[kDecWaves * kStageBytes];
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
    for (uint32_t s = s_begin + wave; s < s_end; s += kDecWaves) decode_segment<DT>(T, tab, stage, s, err);
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
    const uint64_t slots = (uint64_t)cus * 2;   // two 512-thread workgroups fit a CU's LDS
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
