// zx_zf.hip -- the dominant-range exponent codec: 2048-element blocks, the
// exponent remapped against the block's most frequent one, three dense bit planes
// and 2-byte outlier records (ZipFloat page, sections 3.1-3.3).
//
// Per block of Ne = 2048 elements: MD is the most frequent exponent (ties to the
// smallest), the dominant range starts at l_b = MD - 6 (section 3.2, Delta* = 6,
// L* = 8), and every exponent is remapped to v = e - l_b modulo the exponent field
// (Eq. 4).  The low three bits of v of every element go into three bit planes of 256
// bytes (plane p, byte k, bit i = bit p of element 8k+i's v); the elements whose v is
// 8 or more get a record (i << 5) | (v >> 3), in element order (section 3.3).  Sign
// and mantissa stay raw, in the same byte (BF16) or nibble (FP8) array as the
// Huffman codec's.  Record offsets come from a prefix sum over blocks (the page
// reserves space with an atomic add; the sum gives the same sizes and fixed bytes).
//
// Every step is element-parallel: a thread owns 8 consecutive elements, which are
// exactly one byte of each plane.  Decode scatters a block's records into an LDS
// array of high bits and then fuses each thread's 8 elements with one 16-byte (BF16)
// or 8-byte (FP8) store, so it is bound by memory traffic alone.  The analysis and
// decode passes run grid-stride, one block per workgroup step.
#include "zx_common.h"

namespace zxk {

constexpr uint32_t kZfBlock = 2048;
constexpr uint32_t kZfThreads = 256;               // 8 elements per thread
constexpr uint32_t kZfPlaneBytes = kZfBlock / 8;   // 256
constexpr uint32_t kZfScanTile = 8192;             // record-count scan tile (1024 threads x 8)

// One thread's 8 exponents (element 8t+k in byte k) and sign/mantissa bits.
template <int DT>
struct ZfIn {
    uint32_t e[2];    // exponents, one per byte
    uint32_t sm[2];   // BF16: sign/mantissa bytes, one per byte; FP8: nibble word in sm[0]
};

template <int DT>
__device__ __forceinline__ ZfIn<DT> zf_load(const void *__restrict__ in, uint64_t e0, uint32_t cnt)
{
    ZfIn<DT> r;
    if (DT == ZX_BF16) {
        uint32_t w[4] = {0, 0, 0, 0};
        const uint16_t *src = reinterpret_cast<const uint16_t *>(in) + e0;
        if (cnt == 8) {
            const uint4 q = *reinterpret_cast<const uint4 *>(src);
            w[0] = q.x; w[1] = q.y; w[2] = q.z; w[3] = q.w;
        } else {
            for (uint32_t k = 0; k < cnt; ++k) w[k / 2] |= (uint32_t)src[k] << (16 * (k % 2));
        }
        // x >> 7 holds the first element's exponent in byte 0 and the second's in byte 2
        r.e[0] = __builtin_amdgcn_perm(w[1] >> 7, w[0] >> 7, 0x06040200u);
        r.e[1] = __builtin_amdgcn_perm(w[3] >> 7, w[2] >> 7, 0x06040200u);
        uint32_t t[4];
        for (uint32_t k = 0; k < 4; ++k) t[k] = (w[k] & 0x007F007Fu) | ((w[k] >> 8) & 0x00800080u);
        r.sm[0] = __builtin_amdgcn_perm(t[1], t[0], 0x06040200u);
        r.sm[1] = __builtin_amdgcn_perm(t[3], t[2], 0x06040200u);
    } else {
        uint32_t w[2] = {0, 0};
        const uint8_t *src = reinterpret_cast<const uint8_t *>(in) + e0;
        if (cnt == 8) {
            const uint2 q = *reinterpret_cast<const uint2 *>(src);
            w[0] = q.x; w[1] = q.y;
        } else {
            for (uint32_t k = 0; k < cnt; ++k) w[k / 4] |= (uint32_t)src[k] << (8 * (k % 4));
        }
        r.e[0] = (w[0] >> 3) & 0x0F0F0F0Fu;
        r.e[1] = (w[1] >> 3) & 0x0F0F0F0Fu;
        uint32_t t[2];
        for (uint32_t k = 0; k < 2; ++k) {
            const uint32_t nb4 = (w[k] & 0x07070707u) | ((w[k] >> 4) & 0x08080808u);   // one nibble per byte
            t[k] = (nb4 | (nb4 >> 4)) & 0x00FF00FFu;                                    // two nibbles per half
        }
        r.sm[0] = __builtin_amdgcn_perm(t[1], t[0], 0x06040200u);
        r.sm[1] = 0;
    }
    return r;
}

__device__ __forceinline__ uint32_t zf_byte(const uint32_t (&v)[2], uint32_t k) { return (v[k / 4] >> (8 * (k % 4))) & 0xFFu; }

// ---- analyze: l_b and the outlier count of every block, one block per 256-thread
// workgroup step (grid-stride, the next block's input requested before this one is
// counted).  Exponents cluster on a few values, so one shared histogram would
// serialise its atomics; lane l adds into copy l % C (C = 16 for BF16, 64 for FP8,
// copies A + 1 words apart so one instruction's atomics on one value fall in
// different banks), and thread t then sums bin t over the copies.

template <int DT>
__global__ __launch_bounds__(kZfThreads) void k_zf_analyze(const void *__restrict__ in, uint64_t n, uint64_t nb,
                                                           uint8_t *__restrict__ lb_out, uint64_t *__restrict__ counts)
{
    constexpr uint32_t A = alphabet_of(DT);
    constexpr uint32_t C = DT == ZX_BF16 ? 16 : 64;   // histogram copies
    constexpr uint32_t S = A + 1;                     // copy stride in words
    __shared__ uint32_t hist[C * S];
    __shared__ uint32_t wbest[kZfThreads / kWave];
    __shared__ uint32_t part[kZfThreads / kWave];
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = lane_id();
    const uint32_t wave = tid / kWave;
    uint32_t *const mine = hist + (lane % C) * S;
    uint64_t b = blockIdx.x;
    ZfIn<DT> x;
    uint32_t cnt = 0;
    if (b < nb) {
        const uint64_t e0 = b * kZfBlock + (uint64_t)tid * 8;
        cnt = e0 >= n ? 0u : (n - e0 < 8 ? (uint32_t)(n - e0) : 8u);
        x = zf_load<DT>(in, e0, cnt);
    }
    for (; b < nb; b += gridDim.x) {
        for (uint32_t i = tid; i < C * S; i += kZfThreads) hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (uint32_t k = 0; k < 8; ++k)
            if (k < cnt) atomicAdd(&mine[zf_byte(x.e, k)], 1u);
        // request the next block's input while this one is summed
        const ZfIn<DT> cur = x;
        const uint32_t ccur = cnt;
        const uint64_t bn = b + gridDim.x;
        cnt = 0;
        if (bn < nb) {
            const uint64_t e0 = bn * kZfBlock + (uint64_t)tid * 8;
            cnt = e0 >= n ? 0u : (n - e0 < 8 ? (uint32_t)(n - e0) : 8u);
            x = zf_load<DT>(in, e0, cnt);
        }
        __syncthreads();
        // most frequent exponent, ties to the smallest: maximise count << 8 | (255 - symbol)
        uint32_t best = 0;
        if (tid < A) {
            uint32_t c = 0;
#pragma unroll 8
            for (uint32_t cp = 0; cp < C; ++cp) c += hist[cp * S + tid];
            best = (c << 8) | (255u - tid);
        }
        for (int o = kWave / 2; o >= 1; o >>= 1) {
            const uint32_t y = (uint32_t)__shfl_xor((int)best, o, kWave);
            best = y > best ? y : best;
        }
        if (lane == 0) wbest[wave] = best;
        __syncthreads();
        best = wbest[0];
        for (uint32_t w = 1; w < kZfThreads / kWave; ++w) best = wbest[w] > best ? wbest[w] : best;
        const uint32_t lb = ((255u - (best & 0xFFu)) + A - 6u) % A;
        uint32_t outl = 0;
#pragma unroll
        for (uint32_t k = 0; k < 8; ++k) outl += (k < ccur && ((zf_byte(cur.e, k) + A - lb) % A) >= 8u) ? 1u : 0u;
        uint32_t tot;
        wave_excl_scan(outl, tot);
        if (lane == 0) part[wave] = tot;
        __syncthreads();
        if (tid == 0) {
            uint32_t sum = 0;
            for (uint32_t w = 0; w < kZfThreads / kWave; ++w) sum += part[w];
            lb_out[b] = (uint8_t)lb;
            counts[b + 1] = sum;   // scanned into offsets afterwards
        }
    }
}

// ---- record offsets: tiles of 8192 counts scanned in place (inclusive, entries
// 1..nb), then the tile totals; the encode kernel adds the tile offsets.
__global__ __launch_bounds__(1024) void k_zf_scan_tiles(uint64_t nb, uint64_t *__restrict__ off, uint64_t *__restrict__ tiles)
{
    __shared__ uint64_t wsum[16];
    const uint32_t tid = threadIdx.x;
    const uint64_t base = 1 + (uint64_t)blockIdx.x * kZfScanTile + (uint64_t)tid * 8;
    uint64_t v[8];
    uint64_t s = 0;
    for (uint32_t k = 0; k < 8; ++k) {
        v[k] = base + k <= nb ? off[base + k] : 0ull;
        s += v[k];
    }
    uint64_t x = s;
    const uint32_t lane = lane_id();
    for (int d = 1; d < kWave; d <<= 1) {
        const uint64_t y = __shfl_up(x, d, kWave);
        if (lane >= (uint32_t)d) x += y;
    }
    if (lane == kWave - 1) wsum[tid / kWave] = x;
    __syncthreads();
    uint64_t o = x - s, tile = 0;
    for (uint32_t w = 0; w < 16; ++w) {
        if (w < tid / kWave) o += wsum[w];
        tile += wsum[w];
    }
    for (uint32_t k = 0; k < 8; ++k) {
        o += v[k];
        if (base + k <= nb) off[base + k] = o;
    }
    if (tid == 0) tiles[blockIdx.x] = tile;
}

__global__ __launch_bounds__(1024) void k_zf_scan_top(uint32_t ntiles, uint64_t *__restrict__ tiles, uint64_t *__restrict__ total)
{
    __shared__ uint64_t wsum[16];
    const uint32_t tid = threadIdx.x;
    uint64_t v[8];
    uint64_t s = 0;
    for (uint32_t k = 0; k < 8; ++k) {
        const uint32_t i = tid * 8 + k;
        v[k] = i < ntiles ? tiles[i] : 0ull;
        s += v[k];
    }
    uint64_t x = s;
    const uint32_t lane = lane_id();
    for (int d = 1; d < kWave; d <<= 1) {
        const uint64_t y = __shfl_up(x, d, kWave);
        if (lane >= (uint32_t)d) x += y;
    }
    if (lane == kWave - 1) wsum[tid / kWave] = x;
    __syncthreads();
    uint64_t o = x - s, all = 0;
    for (uint32_t w = 0; w < 16; ++w) {
        if (w < tid / kWave) o += wsum[w];
        all += wsum[w];
    }
    for (uint32_t k = 0; k < 8; ++k) {   // exclusive offset of each tile
        const uint32_t i = tid * 8 + k;
        if (i < ntiles) tiles[i] = o;
        o += v[k];
    }
    if (tid == 0) total[0] = all;
}

// ---- encode: planes, records, sign/mantissa, and the block's final record offset
template <int DT>
__global__ __launch_bounds__(kZfThreads) void k_zf_encode(const void *__restrict__ in, uint64_t n, const uint8_t *__restrict__ lbs,
                                                          uint64_t *__restrict__ off, const uint64_t *__restrict__ tiles,
                                                          uint8_t *__restrict__ planes, uint16_t *__restrict__ records,
                                                          uint8_t *__restrict__ signmant)
{
    constexpr uint32_t A = alphabet_of(DT);
    __shared__ uint32_t part[kZfThreads / kWave];
    const uint32_t tid = threadIdx.x;
    const uint32_t wave = tid / kWave;
    const uint64_t b = blockIdx.x;
    const uint64_t e0 = b * kZfBlock + (uint64_t)tid * 8;
    const uint32_t cnt = e0 >= n ? 0u : (n - e0 < 8 ? (uint32_t)(n - e0) : 8u);
    const ZfIn<DT> x = zf_load<DT>(in, e0, cnt);
    const uint32_t lb = lbs[b];
    // this block's first record: the in-tile inclusive count of the previous block plus
    // the tile's offset (entry 0, the first block's, is 0)
    const uint64_t rbase = (b == 0 ? 0ull : off[b] + tiles[(b - 1) / kZfScanTile]);
    uint32_t pl[3] = {0, 0, 0};
    uint32_t outl = 0;
    uint32_t hi[8];
#pragma unroll
    for (uint32_t k = 0; k < 8; ++k) {
        const uint32_t v = k < cnt ? (zf_byte(x.e, k) + A - lb) % A : 0u;
        for (uint32_t p = 0; p < 3; ++p) pl[p] |= ((v >> p) & 1u) << k;
        hi[k] = v >> 3;
        outl += hi[k] ? 1u : 0u;
    }
    uint8_t *pb = planes + b * 3 * kZfPlaneBytes;
    for (uint32_t p = 0; p < 3; ++p) pb[p * kZfPlaneBytes + tid] = (uint8_t)pl[p];
    if (DT == ZX_BF16) {
        if (cnt == 8)
            *reinterpret_cast<uint2 *>(signmant + e0) = make_uint2(x.sm[0], x.sm[1]);
        else
            for (uint32_t k = 0; k < cnt; ++k) signmant[e0 + k] = (uint8_t)zf_byte(x.sm, k);
    } else {
        if (cnt == 8)
            *reinterpret_cast<uint32_t *>(signmant + e0 / 2) = x.sm[0];
        else
            for (uint32_t k = 0; k < cnt; k += 2) signmant[(e0 + k) / 2] = (uint8_t)(x.sm[0] >> (4 * k));
    }
    // records in element order: a workgroup exclusive scan of the per-thread counts
    uint32_t tot;
    uint32_t o = wave_excl_scan(outl, tot);
    if (lane_id() == 0) part[wave] = tot;
    __syncthreads();
    uint32_t blk = 0;
    for (uint32_t w = 0; w < kZfThreads / kWave; ++w) {
        if (w < wave) o += part[w];
        blk += part[w];
    }
    if (outl) {
        uint16_t *dst = records + rbase + o;
        uint32_t j = 0;
#pragma unroll
        for (uint32_t k = 0; k < 8; ++k)
            if (hi[k]) dst[j++] = (uint16_t)(((tid * 8 + k) << 5) | hi[k]);
    }
    __syncthreads();   // every thread has read off[b] before it is overwritten
    if (tid == 0) {
        off[b] = rbase;
        if (b + 1 == gridDim.x) off[b + 1] = rbase + blk;   // the total
    }
}

// ---- decode arithmetic, four elements per 32-bit word (one per byte)

// Bits 0..3 of q to bits 0, 8, 16, 24: the shifted copies q, q << 7, q << 14, q << 21
// do not overlap, so the product has no carries.
__device__ __forceinline__ uint32_t zf_spread4(uint32_t q) { return (q * 0x00204081u) & 0x01010101u; }

// Remapped exponents of 4 elements (byte k = element k) from their plane nibbles and
// high bits: the three plane bits below, the high bits above.
__device__ __forceinline__ uint32_t zf_v4(uint32_t q0, uint32_t q1, uint32_t q2, uint32_t hi)
{
    return zf_spread4(q0) | (zf_spread4(q1) << 1) | (zf_spread4(q2) << 2) | (hi << 3);
}

// Byte-wise (a + b) mod 256.
__device__ __forceinline__ uint32_t zf_add_bytes(uint32_t a, uint32_t b)
{
    return ((a & 0x7F7F7F7Fu) + (b & 0x7F7F7F7Fu)) ^ ((a ^ b) & 0x80808080u);
}

// Four BF16 values (two words) from 4 exponents and 4 sign/mantissa bytes: the
// exponent rotated right by one bit per byte puts its low bit at bit 7 (next to the
// mantissa, low byte) and its upper seven bits at 0..6 (next to the sign, high byte);
// two bit-selects build all low and all high bytes, two byte permutes interleave them.
__device__ __forceinline__ void zf_fuse_bf16(uint32_t e, uint32_t S, uint32_t &w0, uint32_t &w1)
{
    const uint32_t er = ((e >> 1) & 0x7F7F7F7Fu) | ((e << 7) & 0x80808080u);
    const uint32_t lo = (er & 0x80808080u) | (S & 0x7F7F7F7Fu);
    const uint32_t hi = (S & 0x80808080u) | (er & 0x7F7F7F7Fu);
    w0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    w1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

// ---- decode: one block per 256-thread workgroup step, grid-stride; thread t owns
// elements 8t..8t+7 (one byte of each plane, 8 sign/mantissa bytes or 4 nibble bytes,
// one 16- or 8-byte store), so every load and store instruction of a wavefront covers
// one contiguous range.  A step requests everything it reads at once, including one
// record per thread (blocks with more than 256 records loop for the rest), scatters
// the records into an LDS array of high bits (two arrays used in turn, so a step
// needs two barriers), then fuses and stores.
template <int DT>
__global__ __launch_bounds__(kZfThreads) void k_zf_decode(uint64_t n, uint64_t nb, uint64_t nrec, const uint8_t *__restrict__ lbs,
                                                          const uint8_t *__restrict__ planes, const uint64_t *__restrict__ off,
                                                          const uint16_t *__restrict__ records,
                                                          const uint8_t *__restrict__ signmant, void *__restrict__ out,
                                                          uint32_t *__restrict__ err)
{
    constexpr uint32_t A = alphabet_of(DT);
    __shared__ __align__(16) uint8_t high_all[2][kZfBlock];
    const uint32_t tid = threadIdx.x;
    uint32_t par = 0;
    for (uint64_t b = blockIdx.x; b < nb; b += gridDim.x, par ^= 1u) {
        uint8_t *high = high_all[par];
        const uint64_t e0 = b * kZfBlock + (uint64_t)tid * 8;
        const uint32_t cnt = e0 >= n ? 0u : (n - e0 < 8 ? (uint32_t)(n - e0) : 8u);
        const uint32_t lb = lbs[b];
        const uint64_t r0 = off[b], r1 = off[b + 1];
        const bool rec_ok = r1 > r0 && r1 <= nrec;   // uniform
        const uint32_t rv = (rec_ok && r0 + tid < r1) ? records[r0 + tid] : 0xFFFFFFFFu;
        const uint8_t *pb = planes + b * 3 * kZfPlaneBytes;
        const uint32_t p0 = pb[tid], p1 = pb[kZfPlaneBytes + tid], p2 = pb[2 * kZfPlaneBytes + tid];
        uint32_t smw[2] = {0, 0};
        if (DT == ZX_BF16) {
            if (cnt == 8) {
                const uint2 q = *reinterpret_cast<const uint2 *>(signmant + e0);
                smw[0] = q.x; smw[1] = q.y;
            } else {
                for (uint32_t k = 0; k < cnt; ++k) smw[k / 4] |= (uint32_t)signmant[e0 + k] << (8 * (k % 4));
            }
        } else {
            if (cnt == 8)
                smw[0] = *reinterpret_cast<const uint32_t *>(signmant + e0 / 2);
            else
                for (uint32_t k = 0; k < cnt; k += 2) smw[0] |= (uint32_t)signmant[(e0 + k) / 2] << (4 * k);
        }
        if (r1 > r0 && r1 > nrec && tid == 0) report(err, ZX_E_CORRUPT);
        uint32_t hw[2] = {0, 0};
        if (rec_ok) {
            reinterpret_cast<uint2 *>(high)[tid] = make_uint2(0, 0);
            __syncthreads();
            if (rv != 0xFFFFFFFFu) high[rv >> 5] = (uint8_t)(rv & 31u);
            for (uint64_t k = r0 + kZfThreads + tid; k < r1; k += kZfThreads) {
                const uint32_t r = records[k];
                high[r >> 5] = (uint8_t)(r & 31u);
            }
            __syncthreads();
            const uint2 h = reinterpret_cast<const uint2 *>(high)[tid];
            hw[0] = h.x; hw[1] = h.y;
        }
        uint32_t o[4];
        const uint32_t lrep = lb * 0x01010101u;
#pragma unroll
        for (uint32_t h = 0; h < 2; ++h) {
            const uint32_t v = zf_v4((p0 >> (4 * h)) & 0xFu, (p1 >> (4 * h)) & 0xFu, (p2 >> (4 * h)) & 0xFu, hw[h]);
            if (DT == ZX_BF16) {
                zf_fuse_bf16(zf_add_bytes(v, lrep), smw[h], o[2 * h], o[2 * h + 1]);
            } else {
                // 4-bit field: v, l_b <= 15, so a plain add never carries out of a byte
                const uint32_t e = (v + lrep) & 0x0F0F0F0Fu;
                // sign/mantissa nibbles of elements 4h..4h+3, one per byte
                const uint32_t nw = (smw[0] >> (16 * h)) & 0xFFFFu;
                const uint32_t N = ((nw & 0x000Fu) | ((nw & 0x00F0u) << 4) | ((nw & 0x0F00u) << 8) | ((nw & 0xF000u) << 12));
                o[h] = ((N & 0x08080808u) << 4) | (e << 3) | (N & 0x07070707u);
            }
        }
        (void)A;
        if (DT == ZX_BF16) {
            uint16_t *dst = reinterpret_cast<uint16_t *>(out) + e0;
            if (cnt == 8)
                *reinterpret_cast<uint4 *>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
            else
                for (uint32_t k = 0; k < cnt; ++k) dst[k] = (uint16_t)(o[k / 2] >> (16 * (k % 2)));
        } else {
            uint8_t *dst = reinterpret_cast<uint8_t *>(out) + e0;
            if (cnt == 8)
                *reinterpret_cast<uint2 *>(dst) = make_uint2(o[0], o[1]);
            else
                for (uint32_t k = 0; k < cnt; ++k) dst[k] = (uint8_t)(o[k / 4] >> (8 * (k % 4)));
        }
    }
}

}  // namespace zxk

using namespace zxk;

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Analysis and decode: one block per workgroup step, 8 resident 256-thread workgroups
// per CU.
static uint64_t zf_grid_waves(uint64_t nb)
{
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    return nb < (uint64_t)cus * 8 ? nb : (uint64_t)cus * 8;
}

extern "C" size_t zx_zf_scan_workspace_bytes(uint64_t n)
{
    const uint64_t nb = (n + kZfBlock - 1) / kZfBlock;
    return (size_t)(((nb + kZfScanTile - 1) / kZfScanTile + 1) * 8);
}

extern "C" zx_status zx_zf_encode_size(zx_dtype dtype, const void *in, uint64_t n, uint8_t *lb, uint64_t *rec_off,
                                       void *workspace, size_t ws_bytes, uint64_t *total, hipStream_t stream)
{
    if (dtype != ZX_BF16 && dtype != ZX_FP8_E4M3FN) return ZX_E_UNSUPPORTED;
    const uint64_t nb = (n + kZfBlock - 1) / kZfBlock;
    const uint64_t ntiles = (nb + kZfScanTile - 1) / kZfScanTile;
    if (!rec_off || !total || !workspace || ws_bytes < zx_zf_scan_workspace_bytes(n) || !aligned16(in) || (n && (!in || !lb)))
        return ZX_E_INVAL;
    if (nb > 0x7FFFFFFFull || ntiles > 1024 * 8) return ZX_E_INVAL;
    uint64_t *tiles = static_cast<uint64_t *>(workspace);
    if (nb == 0) {
        hipLaunchKernelGGL(k_zf_scan_top, dim3(1), dim3(1024), 0, stream, 0u, tiles, total);
        if (hipGetLastError() != hipSuccess) return ZX_E_HIP;
        return hipMemsetAsync(rec_off, 0, 8, stream) == hipSuccess ? ZX_OK : ZX_E_HIP;
    }
    const uint64_t agrid = zf_grid_waves(nb);   // one block per workgroup step
    if (dtype == ZX_BF16)
        hipLaunchKernelGGL(k_zf_analyze<ZX_BF16>, dim3((uint32_t)agrid), dim3(kZfThreads), 0, stream, in, n, nb, lb, rec_off);
    else
        hipLaunchKernelGGL(k_zf_analyze<ZX_FP8_E4M3FN>, dim3((uint32_t)agrid), dim3(kZfThreads), 0, stream, in, n, nb, lb, rec_off);
    hipLaunchKernelGGL(k_zf_scan_tiles, dim3((uint32_t)ntiles), dim3(1024), 0, stream, nb, rec_off, tiles);
    hipLaunchKernelGGL(k_zf_scan_top, dim3(1), dim3(1024), 0, stream, (uint32_t)ntiles, tiles, total);
    return hipGetLastError() == hipSuccess ? ZX_OK : ZX_E_HIP;
}

extern "C" zx_status zx_zf_encode(zx_dtype dtype, const void *in, uint64_t n, const uint8_t *lb, uint64_t *rec_off,
                                  const void *workspace, uint64_t total_records, uint8_t *planes, uint16_t *records,
                                  uint8_t *signmant, hipStream_t stream)
{
    if (dtype != ZX_BF16 && dtype != ZX_FP8_E4M3FN) return ZX_E_UNSUPPORTED;
    const uint64_t nb = (n + kZfBlock - 1) / kZfBlock;
    if (nb == 0) return ZX_OK;
    if (!in || !lb || !rec_off || !workspace || !planes || !signmant || (total_records && !records) || !aligned16(in) ||
        !aligned16(signmant) || nb > 0x7FFFFFFFull)
        return ZX_E_INVAL;
    const uint64_t *tiles = static_cast<const uint64_t *>(workspace);
    if (dtype == ZX_BF16)
        hipLaunchKernelGGL(k_zf_encode<ZX_BF16>, dim3((uint32_t)nb), dim3(kZfThreads), 0, stream, in, n, lb, rec_off, tiles,
                           planes, records, signmant);
    else
        hipLaunchKernelGGL(k_zf_encode<ZX_FP8_E4M3FN>, dim3((uint32_t)nb), dim3(kZfThreads), 0, stream, in, n, lb, rec_off, tiles,
                           planes, records, signmant);
    return hipGetLastError() == hipSuccess ? ZX_OK : ZX_E_HIP;
}

extern "C" zx_status zx_zf_decode(const zx_zf_container *c, void *out, uint32_t *err, hipStream_t stream)
{
    if (!c) return ZX_E_INVAL;
    if (c->dtype != ZX_BF16 && c->dtype != ZX_FP8_E4M3FN) return ZX_E_UNSUPPORTED;
    const uint64_t nb = (c->n + kZfBlock - 1) / kZfBlock;
    if (nb == 0) return ZX_OK;
    if (!out || !c->lb || !c->planes || !c->rec_off || !c->signmant || (c->nrecords && !c->records) || !aligned16(out) ||
        !aligned16(c->signmant) || nb > 0x7FFFFFFFull)
        return ZX_E_INVAL;
    const uint64_t grid = zf_grid_waves(nb);
    if (c->dtype == ZX_BF16)
        hipLaunchKernelGGL(k_zf_decode<ZX_BF16>, dim3((uint32_t)grid), dim3(kZfThreads), 0, stream, c->n, nb, c->nrecords, c->lb,
                           c->planes, c->rec_off, c->records, c->signmant, out, err);
    else
        hipLaunchKernelGGL(k_zf_decode<ZX_FP8_E4M3FN>, dim3((uint32_t)grid), dim3(kZfThreads), 0, stream, c->n, nb, c->nrecords,
                           c->lb, c->planes, c->rec_off, c->records, c->signmant, out, err);
    return hipGetLastError() == hipSuccess ? ZX_OK : ZX_E_HIP;
}
