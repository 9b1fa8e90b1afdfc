// zx_common.h -- device-side helpers shared by the libzx kernels (gfx950, wave64).
//
// Canonical code tables are rebuilt on the device from code lengths alone, which
// is all the container stores (DFloat11 article, 方法介绍: the Huffman tree comes
// from the exponent distribution; container v1 keeps only its lengths).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zx.h"

namespace zxk {

constexpr uint32_t kBlock = 65536;       // elements per block
constexpr uint32_t kChunkBits = 128;     // stream bits per decode chunk
constexpr uint32_t kSegChunks = 64;      // chunks per segment (one wavefront lane each)
constexpr uint32_t kSegBits = kChunkBits * kSegChunks;
constexpr uint32_t kMaxLen = 32;
// Zero words after the last stream word (a multiple of four): one segment's words
// and the two a lane's window may reach past them.
constexpr uint32_t kStreamPadWords = 260;
static_assert(kStreamPadWords % 4 == 0 && kStreamPadWords >= kSegBits / 32 + 2 + 2, "stream padding");
constexpr int kWave = 64;

// Decode lookup table index width: the primary table maps the next kLutBits
// stream bits to up to four symbols.
constexpr int kLutBits = 11;
constexpr uint32_t kLutSize = 1u << kLutBits;

__host__ __device__ constexpr uint32_t alphabet_of(int dtype) { return dtype == ZX_FP8_E4M3FN ? 16u : 256u; }

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }
__device__ __forceinline__ uint64_t lanemask_lt() { return (1ull << lane_id()) - 1ull; }

__device__ __forceinline__ void report(uint32_t *err, uint32_t code)
{
    if (err) atomicCAS(err, 0u, code);
}

// Exclusive prefix sum across the 64 lanes of a wavefront; `total` gets the sum.
// Data-parallel-primitive lane moves: shifts by 1, 2, 4, 8 inside each row of 16
// lanes, then the last lane of each row is broadcast into the following rows.  No
// address registers are needed, unlike a permute-based scan.
__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t v, uint32_t &total)
{
    // dpp_ctrl encodings: row_shr:n = 0x110 + n, row_bcast:15 = 0x142, row_bcast:31 = 0x143
    int x = (int)v;
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);
    total = (uint32_t)__builtin_amdgcn_readlane(x, kWave - 1);
    return (uint32_t)x - v;
}

// Canonical-code description of one codebook, built in LDS by a whole workgroup.
// Codes of length L are the consecutive integers first[L] .. first[L]+count[L]-1,
// assigned to symbols in (length, symbol) order (RFC 1951, section 3.2.2).
// Order the LDS accesses of one wavefront around this point (all its lanes).
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct Canon {
    uint32_t count[kMaxLen + 1];
    uint32_t first[kMaxLen + 1];
    uint32_t offset[kMaxLen + 1];       // position of the first length-L symbol in `sym`
    uint32_t wcnt[16][kMaxLen + 1];     // per-wave symbol counts by length
    uint64_t lim[kMaxLen + 2];          // (first[L]+count[L]) << (32-L), left-justified
    uint32_t code[256];
    uint8_t len[256];
    uint8_t sym[256];
    uint32_t nsym;
    uint32_t maxlen;
    uint32_t ok;                        // 1 if the lengths form a complete prefix code
};

// Build `c` from the code lengths of symbols 0..A-1, thread t holding symbol t's
// length in `l` (threads t >= A pass anything).  Every thread of the workgroup must
// call it; blockDim.x must be a multiple of 64, >= A and <= 1024.
__device__ inline void canon_build_from(uint32_t l, uint32_t A, Canon &c)
{
    const uint32_t tid = threadIdx.x;
    const uint32_t wave = tid / kWave;
    const uint32_t nsw = (A + kWave - 1) / kWave;   // waves that hold symbols
    if (tid >= A) l = 0;
    if (tid < A) c.len[tid] = (uint8_t)l;
    // per-wave count and in-wave rank of each symbol among symbols of its length,
    // for the lengths up to the wave's longest (the counts above it are zero)
    uint32_t rank = 0;
    if (wave < nsw) {
        uint32_t mx = l;
        for (int o = kWave / 2; o >= 1; o >>= 1) {
            const uint32_t y = (uint32_t)__shfl_xor((int)mx, o, kWave);
            mx = y > mx ? y : mx;
        }
        mx = __builtin_amdgcn_readfirstlane(mx);
        const uint64_t lt = lanemask_lt();
        for (uint32_t L = 1; L <= mx; ++L) {
            const uint64_t m = __ballot(l == L);
            if (l == L) rank = (uint32_t)__popcll(m & lt);
            if (lane_id() == 0) c.wcnt[wave][L] = (uint32_t)__popcll(m);
        }
        const uint32_t L = lane_id();
        if (L > mx && L <= kMaxLen) c.wcnt[wave][L] = 0;
    }
    __syncthreads();
    if (wave == 0) {
        // lane L (1..32): the number of codes of length L, then by prefix scans its
        // first canonical code and first symbol index.  Left-justified to 32 bits, the
        // first code of length L is the sum over shorter lengths j of count[j] << (32 - j)
        // (each length's codes follow the shorter ones, one bit longer).
        const uint32_t L = lane_id();
        const bool isl = L >= 1 && L <= kMaxLen;
        uint32_t cnt = 0;
        if (isl)
            for (uint32_t w = 0; w < nsw; ++w) cnt += c.wcnt[w][L];
        uint32_t nsym;
        const uint32_t idx = wave_excl_scan(cnt, nsym);
        const uint64_t t = isl ? (uint64_t)cnt << (kMaxLen - L) : 0ull;
        uint64_t x = t;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const uint64_t y = __shfl_up(x, d, kWave);
            if (L >= (uint32_t)d) x += y;
        }
        const uint64_t F = x - t;                      // exclusive: left-justified first code
        const uint64_t kraft = __shfl(x, kWave - 1, kWave);
        const uint64_t nz = __builtin_amdgcn_ballot_w64(isl && cnt != 0);
        if (isl) {
            c.count[L] = cnt;
            c.first[L] = (uint32_t)(F >> (kMaxLen - L));
            c.offset[L] = idx;
            c.lim[L] = F + t;
        }
        if (L == 0) {
            c.lim[kMaxLen + 1] = ~0ull;
            c.count[0] = 0;
            c.first[0] = 0;
            c.offset[0] = 0;
            c.lim[0] = 0;
            c.nsym = nsym;
            c.maxlen = nz ? 63u - (uint32_t)__builtin_clzll(nz) : 0u;
            c.ok = (nsym >= 2 && kraft == (1ull << 32)) ? 1u : 0u;
        }
    }
    __syncthreads();
    if (tid < A) {
        uint32_t code = 0;
        if (l) {
            uint32_t r = rank;
            for (uint32_t w = 0; w < wave; ++w) r += c.wcnt[w][l];
            code = c.first[l] + r;
            c.sym[c.offset[l] + r] = (uint8_t)tid;
        }
        c.code[tid] = code;
    }
    __syncthreads();
}

__device__ inline void canon_build(const uint8_t *__restrict__ lengths_g, uint32_t A, Canon &c)
{
    const uint32_t tid = threadIdx.x;
    canon_build_from(tid < A ? lengths_g[tid] : 0u, A, c);
}

// Length of the code at the front of a left-justified 32-bit window, searching
// lengths from `from` upward; returns kMaxLen+1 when nothing matches.
__device__ __forceinline__ uint32_t canon_len(const uint64_t *lim, uint32_t v, uint32_t from)
{
    uint32_t L = from;
    while (L <= kMaxLen && (uint64_t)v >= lim[L]) ++L;
    return L;
}

// Form in which the decoder stages an exponent symbol for the write pass.
//   BF16: the 8-bit exponent rotated right by one bit.  Bit 7 is then the exponent's
//         low bit, which belongs in the low byte of the BF16 value next to the 7
//         mantissa bits, and bits 0..6 are the exponent's upper seven bits, which
//         belong in the high byte next to the sign: one bit-select per byte pair.
//   FP8:  the 4-bit exponent already shifted to its place, bits 3..6.
__host__ __device__ constexpr uint32_t stage_form(uint32_t A, uint32_t e)
{
    return A == 16u ? (e << 3) : (((e >> 1) | (e << 7)) & 0xFFu);
}

// Decoder tables kept in LDS.  For every value x of the next kLutBits stream bits one
// 8-byte entry e[x] = {lo, hi}, read with one 64-bit LDS load:
//   lo[x]  bits  0..3   bits taken by the whole codes that fit in the window (adv)
//          bits  8..11  length of the first three codes together (0 if fewer)
//          bits 16..23  number of those codes, at most four (ns)
//          bits 24..27  length of the first code
//          bits 28..31  length of the first two codes together
//          lo[x] == 0   the first code is longer than the window
//   hi[x]  bytes 0..3   stage forms of the decoded symbols, in stream order
// The fields of lo are placed so that a lane can keep its bit position in the low
// byte and its code count in bits 16..23 of one register and subtract whole entries
// from it, and so that the low five bits of lo are exactly the shift that consumes
// the entry from a 32-bit window.  Bits 8..15 of that register start at 255 and
// absorb the first-three-codes field of every entry subtracted: each field is at most
// the bits its entry consumes, so their sum never exceeds the bits a lane consumes,
// which is below 256 (a lane stops before position kPosBase + 31 + 128 + 32).
// Entry kLutSize is all zero.
//   lim/base/sym: canonical description for codes longer than the window.
//   lim_short: the largest left-justified 32-bit window that starts with a code of at
//   most kLutBits bits (canonical codes of length <= L fill [0, lim[L]) in order).
constexpr uint32_t kLutSymMax = 4;

struct __align__(16) DTab {
    uint2 e[kLutSize + 4];              // {lo, hi}
    uint64_t lim[kMaxLen + 2];
    int32_t base[kMaxLen + 1];          // offset[L] - first[L]
    uint8_t sym[256];                   // stage form by canonical index
    uint32_t lim_short;
    uint32_t ok;
    uint32_t nsym;
    uint32_t maxlen;
    uint32_t pad_[3];
};
static_assert(sizeof(DTab) % 16 == 0, "DTab must copy in 16-byte pieces");

// Fill a DTab for alphabet size A from a built Canon; every thread of the workgroup
// calls it.  `t1` is LDS scratch of kLutSize entries: first the code at the front of
// every kLutBits-bit window (its length, and its symbol's stage form in the high
// byte; 0 when that code is longer than the window), then each entry of the table
// chains up to four lookups of it.  Shifting a window left by the bits already used
// fills it with zeros, and a code no longer than the bits left is decided by real
// bits alone (codes are prefix-free), so the chained lookups read the same codes as
// a search of the shifted window would.
__device__ inline void dtab_fill(const Canon &c, uint32_t A, DTab &t, uint16_t *t1)
{
    const uint32_t tid = threadIdx.x;
    for (uint32_t i = tid; i < kMaxLen + 2; i += blockDim.x) t.lim[i] = (i == 0) ? 0ull : c.lim[i];
    for (uint32_t i = tid; i <= kMaxLen; i += blockDim.x) t.base[i] = (int32_t)c.offset[i] - (int32_t)c.first[i];
    // (entries past the present symbols are never read; zero keeps the table's bytes
    // a function of the lengths alone)
    for (uint32_t i = tid; i < 256; i += blockDim.x) t.sym[i] = i < c.nsym ? (uint8_t)stage_form(A, c.sym[i]) : 0u;
    if (tid == 0) {
        t.ok = c.ok;
        t.nsym = c.nsym;
        t.maxlen = c.maxlen;
        const uint64_t l = c.lim[kLutBits];
        t.lim_short = l == 0 ? 0u : (l >= (1ull << 32) ? 0xFFFFFFFFu : (uint32_t)(l - 1));
        t.pad_[0] = t.pad_[1] = t.pad_[2] = 0;
    }
    // the limits of lengths 1..kLutBits, read once: the length of the code at the front
    // of a window is one more than the number of those limits the window reaches (they
    // do not decrease with the length), when that is at most kLutBits
    uint64_t lim_s[kLutBits];
#pragma unroll
    for (int L = 0; L < kLutBits; ++L) lim_s[L] = c.lim[L + 1];
    for (uint32_t x = tid; x < kLutSize; x += blockDim.x) {
        uint32_t e = 0;
        if (c.ok) {
            const uint32_t v = x << (32 - kLutBits);   // window, left-justified, zero filled
            uint32_t L = 1;
#pragma unroll
            for (int j = 0; j < kLutBits; ++j) L += (uint64_t)v >= lim_s[j] ? 1u : 0u;
            if (L <= (uint32_t)kLutBits)
                e = L | (stage_form(A, c.sym[c.offset[L] + ((v >> (32 - L)) - c.first[L])]) << 8);
        }
        t1[x] = (uint16_t)e;
    }
    __syncthreads();
    for (uint32_t x = tid; x < kLutSize; x += blockDim.x) {
        uint32_t lo = 0, hi = 0;
        if (c.ok) {
            uint32_t used = 0, ns = 0, syms = 0, l1 = 0, l12 = 0, l123 = 0;
            while (ns < kLutSymMax) {
                // a code is fully inside the window if its length fits in the bits left
                const uint32_t e = t1[(x << used) & (kLutSize - 1)];
                const uint32_t L = e & 0xFFu;
                if (L == 0 || L > kLutBits - used) break;
                syms |= (e >> 8) << (8 * ns);
                used += L;
                ++ns;
                if (ns == 1) l1 = used;
                if (ns == 2) l12 = used;
                if (ns == 3) l123 = used;
            }
            if (ns) {
                lo = used | (l123 << 8) | (ns << 16) | (l1 << 24) | (l12 << 28);
                hi = syms;
            }
        }
        t.e[x] = make_uint2(lo, hi);
    }
    if (tid < 4) t.e[kLutSize + tid] = make_uint2(0u, 0u);
}

}  // namespace zxk
