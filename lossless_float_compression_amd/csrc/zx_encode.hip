// zx_encode.hip -- field split, exponent bit-packing and the decoder's auxiliary
// arrays, one workgroup per 65536-element block.
//
// Method: sign+mantissa stay raw in their own byte array, exponents are replaced by
// their canonical Huffman codes, tightly bit-packed (DFloat11 article, 方法介绍,
// Fig. 2; Intel summary, 方法论), tensor processed in fixed-size blocks (Intel
// summary, 实验设计).  Fast online encode matters for K/V caches (ZipFloat page,
// section 4.2; Intel summary, 局限性), so the whole encode runs on the GPU.
//
// Positions come from prefix sums, never from atomics: per-block bit counts are
// scanned into block offsets, and inside a block each round of 2048 elements scans
// its per-thread code lengths.  Codes are ORed into an LDS staging area aligned to
// global stream words; whole words are then written with plain stores.  The only
// words two blocks can share are a block's first and last word.  Each block owns the
// stream bits from its first bit up to the next block's (the last block: up to the end
// of the stream, padding included) and sets exactly those bits of a shared word with
// two atomics (clear its bits, then OR its code bits in); the owners' bits are disjoint
// and cover the word, so the word ends the same in any order, whatever it held before.
#include <mutex>

#include "zx_codebook.h"

namespace zxk {

constexpr int kEncThreads = 1024;
constexpr uint32_t kEncPerThread = 8;
constexpr uint32_t kRound = kEncThreads * kEncPerThread;   // 8192 elements per round
constexpr uint32_t kStageWords = kRound + 2;               // up to 32 bits per element + carry

// -------------------------------------------------------------------- block sizes
constexpr int kSizeThreads = 256;

template <int DT>
__global__ __launch_bounds__(kSizeThreads) void k_block_bits(const void *__restrict__ in, uint64_t n, int per_block,
                                                            const uint8_t *__restrict__ lengths,
                                                            const uint32_t *__restrict__ block_hist,
                                                            uint64_t *__restrict__ block_bitoff,
                                                            uint32_t *__restrict__ block_seg)
{
    constexpr uint32_t A = alphabet_of(DT);
    __shared__ uint8_t len[256];
    __shared__ uint32_t part[kSizeThreads / kWave];
    const uint32_t tid = threadIdx.x;
    const uint64_t b = blockIdx.x;
    const uint64_t cb = per_block ? b : 0;
    if (tid < A) len[tid] = lengths[cb * A + tid];
    __syncthreads();
    uint32_t bits = 0;
    if (block_hist) {
        if (tid < A) bits = block_hist[b * A + tid] * (uint32_t)len[tid];
    } else {
        const uint64_t lo = b * kBlock;
        const uint64_t hi = (lo + kBlock < n) ? lo + kBlock : n;
        for (uint64_t i = lo + tid; i < hi; i += kSizeThreads) {
            uint32_t e;
            if (DT == ZX_BF16)
                e = (reinterpret_cast<const uint16_t *>(in)[i] >> 7) & 0xFFu;
            else if (DT == ZX_E8M0)
                e = reinterpret_cast<const uint8_t *>(in)[i];
            else
                e = (reinterpret_cast<const uint8_t *>(in)[i] >> 3) & 0xFu;
            bits += len[e];
        }
    }
    uint32_t tot;
    wave_excl_scan(bits, tot);
    if (lane_id() == 0) part[tid / kWave] = tot;
    __syncthreads();
    if (tid == 0) {
        uint32_t s = 0;
        for (uint32_t w = 0; w < kSizeThreads / kWave; ++w) s += part[w];
        const uint32_t nch = (s + kChunkBits - 1) / kChunkBits;
        uint32_t nseg = (nch + kSegChunks - 1) / kSegChunks;
        if (nseg == 0) nseg = 1;
        block_bitoff[b + 1] = s;   // raw counts; k_scan_blocks turns them into offsets
        block_seg[b + 1] = nseg;
    }
}

// In-place inclusive scan over [1..nblocks] of both arrays; one workgroup.  The
// arrays pass through LDS in tiles of 8192 entries: loaded and stored with
// consecutive threads on consecutive entries, scanned with each thread owning eight
// consecutive entries (the LDS index is padded by one slot per eight, so those
// eight-entry runs start on different banks), and a running carry links the tiles.
constexpr uint32_t kScanPer = 8;
constexpr uint32_t kScanTile = 1024 * kScanPer;
__device__ __forceinline__ uint32_t scan_pad(uint32_t i) { return i + (i >> 3); }

__global__ __launch_bounds__(1024) void k_scan_blocks(uint64_t nblocks, uint64_t *__restrict__ block_bitoff,
                                                      uint32_t *__restrict__ block_seg, uint64_t *__restrict__ totals)
{
    __shared__ uint64_t tb[kScanTile + kScanTile / 8];
    __shared__ uint32_t tsg[kScanTile + kScanTile / 8];
    __shared__ uint64_t wb[16];
    __shared__ uint32_t ws[16];
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = lane_id();
    const uint32_t wave = tid / kWave;
    uint64_t carry_b = 0;
    uint32_t carry_s = 0;
    for (uint64_t base = 1; base <= nblocks; base += kScanTile) {
        const uint32_t cnt = (uint32_t)(nblocks + 1 - base < kScanTile ? nblocks + 1 - base : kScanTile);
#pragma unroll
        for (uint32_t j = 0; j < kScanPer; ++j) {
            const uint32_t i = tid + 1024 * j;
            tb[scan_pad(i)] = i < cnt ? block_bitoff[base + i] : 0ull;
            tsg[scan_pad(i)] = i < cnt ? block_seg[base + i] : 0u;
        }
        __syncthreads();
        uint64_t vb[kScanPer];
        uint32_t vs[kScanPer];
        uint64_t sb = 0;
        uint32_t ss = 0;
#pragma unroll
        for (uint32_t j = 0; j < kScanPer; ++j) {
            vb[j] = tb[scan_pad(kScanPer * tid + j)];
            vs[j] = tsg[scan_pad(kScanPer * tid + j)];
            sb += vb[j];
            ss += vs[j];
        }
        // exclusive scan of (sb, ss) over the workgroup
        uint64_t xb = sb;
        uint32_t xs = ss;
        for (int d = 1; d < kWave; d <<= 1) {
            const uint64_t yb = __shfl_up(xb, d, kWave);
            const uint32_t ys = __shfl_up(xs, d, kWave);
            if (lane >= (uint32_t)d) { xb += yb; xs += ys; }
        }
        if (lane == kWave - 1) { wb[wave] = xb; ws[wave] = xs; }
        __syncthreads();
        uint64_t ob = carry_b + (xb - sb), tile_b = 0;
        uint32_t os = carry_s + (xs - ss), tile_s = 0;
        for (uint32_t w = 0; w < 16; ++w) {
            if (w < wave) { ob += wb[w]; os += ws[w]; }
            tile_b += wb[w];
            tile_s += ws[w];
        }
#pragma unroll
        for (uint32_t j = 0; j < kScanPer; ++j) {
            ob += vb[j];
            os += vs[j];
            tb[scan_pad(kScanPer * tid + j)] = ob;
            tsg[scan_pad(kScanPer * tid + j)] = os;
        }
        __syncthreads();
#pragma unroll
        for (uint32_t j = 0; j < kScanPer; ++j) {
            const uint32_t i = tid + 1024 * j;
            if (i < cnt) {
                block_bitoff[base + i] = tb[scan_pad(i)];
                block_seg[base + i] = tsg[scan_pad(i)];
            }
        }
        carry_b += tile_b;
        carry_s += tile_s;
        __syncthreads();   // LDS and the wave totals are reused by the next tile
    }
    if (tid == 0) {
        block_bitoff[0] = 0;
        block_seg[0] = 0;
        totals[0] = carry_b;
        totals[1] = carry_s;
    }
}

// The stream of an empty tensor: padding only, all zero.
__global__ void k_zero_stream(uint64_t stream_words, uint32_t *__restrict__ stream)
{
    for (uint64_t w = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; w < stream_words; w += (uint64_t)gridDim.x * blockDim.x)
        stream[w] = 0;
}

// Stream word gw gets value v in the bits a block owns, global stream bits [own_lo,
// own_hi) (bit 0 of a word is its most significant): a plain store when it owns the
// whole word, otherwise its bits cleared and then ORed in, so that the other owner of
// the word may do the same at any time.
__device__ __forceinline__ void put_word(uint32_t *stream, uint64_t gw, uint32_t v, uint64_t own_lo, uint64_t own_hi)
{
    const uint64_t wb = gw * 32;
    const uint32_t lo = own_lo > wb ? (uint32_t)(own_lo - wb) : 0u;              // < 32
    const uint32_t hi = own_hi >= wb + 32 ? 32u : (uint32_t)(own_hi - wb);      // > lo
    if (lo == 0 && hi == 32) {
        stream[gw] = v;
        return;
    }
    const uint32_t m = (0xFFFFFFFFu >> lo) & (hi == 32 ? 0xFFFFFFFFu : ~(0xFFFFFFFFu >> hi));
    atomicAnd(&stream[gw], ~m);
    atomicOr(&stream[gw], v & m);
}

// The last block of a stream also owns the words after its own, up to the stream's
// end (its padding): they are cleared (the first of them only from the block's end on,
// when the block ends inside it).
__device__ __forceinline__ void zero_stream_tail(uint32_t *stream, uint64_t from_word, uint64_t zero_to, uint64_t own_lo)
{
    for (uint64_t w = from_word + threadIdx.x; w < zero_to; w += kEncThreads) put_word(stream, w, 0u, own_lo, ~0ull);
}

// -------------------------------------------------------------------- bit packing
// A full block whose bits fit the LDS stage (at most 8192 words: any mean code length
// up to about 4 bits) is packed in one pass.  The whole block's input (8 loads per
// thread) is requested at the kernel's start together with the code lengths, so it
// arrives while the code table is built.  Round r splits its own 16 bytes per thread
// (sign/mantissa bytes or nibbles straight to memory, exponent symbols kept in
// registers) and so waits only for its own loads: the rounds start while the later
// rounds' input is still arriving.  Each round looks up its threads' codes in a table
// of (code, length) pairs, scans their bit counts over the workgroup and places the
// codes, gap bytes and segment entries in LDS; the stream words a round completes
// are stored during the next one, gaps and segment entries at the end.  The rounds
// are bound by vector-ALU issue (about 20 instructions per element), not by memory.  Other
// blocks (the last, partial block of a tensor, or very long codes) take the
// round-by-round path in k_encode.
constexpr uint32_t kOnePassBits = (kStageWords - 2) * 32;
constexpr uint32_t kOnePassChunks = kOnePassBits / kChunkBits;
constexpr uint32_t kOnePassSegs = kOnePassChunks / kSegChunks;
constexpr uint32_t kRoundsPerBlock = kBlock / kRound;
constexpr uint32_t kEncBadFlag = 0x100;   // code table: symbol not allowed in this block

// A full block's input, one thread's share: 16 bytes (BF16) or 8 bytes (FP8) per
// round, i.e. 8 elements at block element r * kRound + tid * kEncPerThread.
template <int DT>
struct BlockIn {
    static constexpr uint32_t RW = DT == ZX_BF16 ? 4 : 2;
    uint32_t w[kRoundsPerBlock][RW];
};

// Request round r of a full block's input for this thread.  A block that is not full
// requests the same 16 bytes of `dummy` instead, so the number of loads in flight is
// the same on every path.
template <int DT>
__device__ __forceinline__ void load_round(const void *__restrict__ in, uint64_t lo, bool full, const void *dummy, uint32_t r,
                                           BlockIn<DT> &x)
{
    const uint64_t e = lo + (uint64_t)r * kRound + threadIdx.x * kEncPerThread;
    if (DT == ZX_BF16) {
        const uint4 *a = full ? reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(in) + e)
                              : reinterpret_cast<const uint4 *>(dummy);
        const uint4 q = *a;
        x.w[r][0] = q.x; x.w[r][1] = q.y; x.w[r][2 % BlockIn<DT>::RW] = q.z; x.w[r][3 % BlockIn<DT>::RW] = q.w;
    } else {
        const uint2 *a = full ? reinterpret_cast<const uint2 *>(reinterpret_cast<const uint8_t *>(in) + e)
                              : reinterpret_cast<const uint2 *>(dummy);
        const uint2 q = *a;
        x.w[r][0] = q.x; x.w[r][1] = q.y;
    }
}

// Request the first NR rounds of a block's input.
template <int DT, uint32_t NR>
__device__ __forceinline__ void load_block_in(const void *__restrict__ in, uint64_t lo, bool full, const void *dummy,
                                              BlockIn<DT> &x)
{
#pragma unroll
    for (uint32_t r = 0; r < NR; ++r) load_round<DT>(in, lo, full, dummy, r, x);
}

// Rounds of input a workgroup has requested before its first round; each round then
// requests the one this many rounds after it.  The whole block at once would keep
// every round's input in registers through the rounds.
constexpr uint32_t kEncAhead = 4;

// D: rounds of input the caller requested (load_block_in<DT, D>) before the call; with
// the whole block requested, every round is split at once.
template <int DT, uint32_t D>
__device__ __forceinline__ void encode_onepass(BlockIn<DT> &x, const void *__restrict__ blk_in, uint64_t lo, uint64_t b,
                                               const Canon &c,
                                               uint32_t degen, uint64_t G, uint32_t bits, uint32_t s0, uint32_t nsb, uint32_t nch,
                                               uint64_t own_hi, uint64_t zero_to, uint8_t *__restrict__ signmant,
                                               uint32_t *__restrict__ stream, uint32_t *__restrict__ seg_desc,
                                               uint8_t *__restrict__ gaps, uint32_t *__restrict__ err, uint32_t *stage,
                                               uint2 *ctab, uint8_t *gapbuf, uint32_t *segbuf,
                                               uint32_t (*part2)[kEncThreads / kWave], uint32_t &s_bad)
{
    const uint32_t tid = threadIdx.x;
    for (uint32_t i = tid; i < kStageWords; i += kEncThreads) stage[i] = 0;
    if (tid == 0) s_bad = 0;
    // code table: the code, and its length with a flag for a symbol the block may not
    // hold (no code, or in a block of zero bits any symbol but the degenerate one)
    if (tid < alphabet_of(DT)) {
        const uint32_t l = c.len[tid];
        const bool flag = bits ? l == 0 : tid != degen;
        ctab[tid] = make_uint2(c.code[tid], l | (flag ? kEncBadFlag : 0u));
    }
    __syncthreads();

    // ---- split of round r, just before its lookups (so a round waits for its own
    //      input only, and the rounds start while the later input is still arriving):
    //      sign/mantissa bytes (nibbles) stored at once, the exponent symbols kept,
    //      one byte per element
    auto split = [&](uint32_t r) -> uint2 {
        const uint32_t i0 = r * kRound + tid * kEncPerThread;
        if (DT == ZX_E8M0) return make_uint2(x.w[r][0], x.w[r][1]);
        if (DT == ZX_BF16) {
            uint32_t t[4];
#pragma unroll
            for (uint32_t w = 0; w < 4; ++w) {
                const uint32_t v = x.w[r][w];
                t[w] = (v & 0x007F007Fu) | ((v >> 8) & 0x00800080u);   // [sm, 0, sm, 0]
            }
            *reinterpret_cast<uint2 *>(signmant + lo + i0) =
                make_uint2(__builtin_amdgcn_perm(t[1], t[0], 0x06040200u), __builtin_amdgcn_perm(t[3], t[2], 0x06040200u));
            // x >> 7 holds the first element's exponent in byte 0 and the second's in byte 2
            return make_uint2(__builtin_amdgcn_perm(x.w[r][1] >> 7, x.w[r][0] >> 7, 0x06040200u),
                              __builtin_amdgcn_perm(x.w[r][3 % BlockIn<DT>::RW] >> 7, x.w[r][2 % BlockIn<DT>::RW] >> 7, 0x06040200u));
        }
        uint32_t t[2];
#pragma unroll
        for (uint32_t w = 0; w < 2; ++w) {
            const uint32_t v = x.w[r][w];
            const uint32_t nb4 = (v & 0x07070707u) | ((v >> 4) & 0x08080808u);   // one nibble per byte
            t[w] = (nb4 | (nb4 >> 4)) & 0x00FF00FFu;                              // two nibbles per half
        }
        *reinterpret_cast<uint32_t *>(signmant + (lo + i0) / 2) = __builtin_amdgcn_perm(t[1], t[0], 0x06040200u);
        return make_uint2((x.w[r][0] >> 3) & 0x0F0F0F0Fu, (x.w[r][1] >> 3) & 0x0F0F0F0Fu);
    };

    const uint32_t a0 = (uint32_t)(G & 31);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    // A round is split at its barrier: `pre` looks up the codes of the thread's 8
    // elements and publishes the wave's bit count; after the barrier `xscan` turns
    // the wave counts into this thread's offset; `post` places the codes and the
    // auxiliary entries.  Round r's `pre` and round r-1's `post` share one barrier
    // interval, so the table lookups of one overlap the stage writes of the other.
    struct Rd {
        uint64_t acc;      // the thread's codes, concatenated (exact while tb <= 64)
        uint64_t starts;   // bit j: a code starts j bits into them (exact while j < 64)
        uint2 sv;          // the 8 symbols, one byte each
        uint32_t tb;       // their total length
        uint32_t o;        // bits before them in the round
        uint32_t R;        // bits in the round
    };
    uint2 pres[D >= kRoundsPerBlock ? kRoundsPerBlock : 1];
    if constexpr (D >= kRoundsPerBlock) {
#pragma unroll
        for (uint32_t r = 0; r < kRoundsPerBlock; ++r) pres[r] = split(r);
    }
    auto pre = [&](uint32_t r, Rd &d) {
        uint2 sv;
        if constexpr (D >= kRoundsPerBlock) {
            sv = pres[r];
        } else {
            sv = split(r);
            if (r + D < kRoundsPerBlock) load_round<DT>(blk_in, 0, true, nullptr, r + D, x);
        }
        d.sv = sv;
        uint32_t flags = 0;
        d.tb = 0;
        d.acc = 0;
        d.starts = 0;
#pragma unroll
        for (uint32_t k = 0; k < kEncPerThread; ++k) {
            const uint32_t sy = ((k < 4 ? sv.x : sv.y) >> (8 * (k & 3))) & 0xFFu;
            const uint2 e = ctab[sy];
            flags |= e.y;
            d.acc = (d.acc << (e.y & 63u)) | e.x;
            d.starts |= 1ull << (d.tb & 63u);
            d.tb += e.y & 0xFFu;
        }
        // (a store, so that each round's flags are reduced in that round and not all
        // kept for the end)
        if (flags & kEncBadFlag) s_bad = 1;
        uint32_t wtot;
        d.o = wave_excl_scan(d.tb, wtot);
        if (lane_id() == 0) part2[r & 1][wave] = wtot;   // double-buffered by round
    };
    auto xscan = [&](uint32_t r, Rd &d) {
        // lanes 0..15 of every wave scan the 16 wave totals
        int pv = (int)part2[r & 1][lane_id() & 15u];
        pv += __builtin_amdgcn_update_dpp(0, pv, 0x111, 0xF, 0xF, true);   // row_shr:1
        pv += __builtin_amdgcn_update_dpp(0, pv, 0x112, 0xF, 0xF, true);   // row_shr:2
        pv += __builtin_amdgcn_update_dpp(0, pv, 0x114, 0xF, 0xF, true);   // row_shr:4
        pv += __builtin_amdgcn_update_dpp(0, pv, 0x118, 0xF, 0xF, true);   // row_shr:8
        d.R = (uint32_t)__builtin_amdgcn_readlane(pv, kEncThreads / kWave - 1);
        if (wave) d.o += (uint32_t)__builtin_amdgcn_readlane(pv, wave - 1);
    };
    auto post = [&](uint32_t r, const Rd &d, uint32_t P) {
        const uint32_t i0 = r * kRound + tid * kEncPerThread;
        const uint32_t tb = d.tb;
        const uint32_t p0 = P + d.o;     // block-relative bit of this thread's first code
        const uint32_t q0 = a0 + p0;     // its stage bit
        const uint32_t bnd = (p0 + kChunkBits - 1) & ~(kChunkBits - 1);   // first chunk boundary >= p0
        if (tb <= 64) {
            // ---- codes into the stage: up to three words, shared with the
            //      neighbouring threads only at the ends
            if (tb) {
                const uint32_t sh = q0 & 31;
                const uint64_t X = d.acc << (64 - tb);
                uint32_t *w = &stage[q0 >> 5];
                atomicOr(&w[0], (uint32_t)(X >> (32 + sh)));
                if (sh + tb > 32) atomicOr(&w[1], (uint32_t)(X >> sh));
                if (sh + tb > 64) atomicOr(&w[2], (uint32_t)(X << (32 - sh)));
            }
            // ---- gap byte of the chunk boundary these bits cover, if any: the distance
            //      to the first code that starts at or after it (the next thread's first
            //      code starts at tb)
            if (bnd < p0 + tb) {
                const uint32_t rel = bnd - p0;
                const uint64_t after = d.starts >> rel;
                const uint32_t m = after ? (uint32_t)__builtin_ctzll(after) : tb - rel;
                gapbuf[bnd / kChunkBits] = (uint8_t)(bnd + m < bits ? m : ZX_NO_GAP);
                if (bnd % (kChunkBits * kSegChunks) == 0 && bnd > 0)   // first element of a segment
                    segbuf[bnd / (kChunkBits * kSegChunks)] = i0 + (uint32_t)__builtin_popcountll(d.starts & ((1ull << rel) - 1));
            }
        } else {
            // ---- long codes: code by code
            const uint2 sv = d.sv;
            uint32_t pk = p0;
#pragma unroll
            for (uint32_t k = 0; k < kEncPerThread; ++k) {
                const uint32_t sy = ((k < 4 ? sv.x : sv.y) >> (8 * (k & 3))) & 0xFFu;
                const uint32_t lk = c.len[sy];
                if (lk == 0) continue;
                const uint32_t q = a0 + pk;
                const uint32_t sh = q & 31;
                const uint64_t x = (uint64_t)c.code[sy] << (64 - lk - sh);
                atomicOr(&stage[q >> 5], (uint32_t)(x >> 32));
                if (sh + lk > 32) atomicOr(&stage[(q >> 5) + 1], (uint32_t)x);
                const uint32_t cd = (pk + kChunkBits - 1) / kChunkBits;
                if (cd * kChunkBits < pk + lk) {
                    uint32_t gap;
                    if (cd * kChunkBits == pk)
                        gap = 0;
                    else
                        gap = (pk + lk < bits) ? pk + lk - cd * kChunkBits : ZX_NO_GAP;
                    gapbuf[cd] = (uint8_t)gap;
                    if (cd % kSegChunks == 0 && cd > 0) segbuf[cd / kSegChunks] = (cd * kChunkBits == pk) ? (i0 + k) : (i0 + k + 1);
                }
                pk += lk;
            }
        }
    };
    // Stream words are stored as soon as they are complete: after round r-1's codes
    // are placed (the barrier of round r), every stage word below round r's first bit.
    const uint64_t W0 = G >> 5;
    uint32_t wdone = 0;   // stage words stored so far
    Rd cur, prev;
    uint32_t P = 0;    // block-relative bit of round r-1's first code
    pre(0, cur);
    __syncthreads();
    xscan(0, cur);
    // unrolled: each round names its own input registers, so it waits for its own loads only
#pragma unroll
    for (uint32_t r = 1; r < kRoundsPerBlock; ++r) {
        prev = cur;
        pre(r, cur);
        post(r - 1, prev, P);
        P += prev.R;
        __syncthreads();
        xscan(r, cur);
        const uint32_t wfin = (a0 + P) >> 5;
        for (uint32_t i = wdone + tid; i < wfin; i += kEncThreads) put_word(stream, W0 + i, stage[i], G, own_hi);
        wdone = wfin;
    }
    post(kRoundsPerBlock - 1, cur, P);
    __syncthreads();
    // ---- the remaining stores
    const uint32_t nw = bits ? (a0 + bits + 31) >> 5 : 0;
    for (uint32_t i = wdone + tid; i < nw; i += kEncThreads) put_word(stream, W0 + i, stage[i], G, own_hi);
    if (zero_to) zero_stream_tail(stream, W0 + nw, zero_to, G);
    for (uint32_t ch = tid; ch < nsb * kSegChunks; ch += kEncThreads)
        gaps[(uint64_t)s0 * kSegChunks + ch] = ch < nch ? gapbuf[ch] : (uint8_t)ZX_NO_GAP;
    for (uint32_t j = tid; j < nsb; j += kEncThreads) {
        seg_desc[2 * (uint64_t)(s0 + j)] = (uint32_t)b;
        seg_desc[2 * (uint64_t)(s0 + j) + 1] = j ? segbuf[j] : 0u;
    }
    if (tid == 0 && s_bad) report(err, ZX_E_CODEBOOK);
}

template <int DT>
__global__ __launch_bounds__(kEncThreads) void k_encode(const void *__restrict__ in, uint64_t n, int per_block,
                                                        const uint8_t *__restrict__ lengths,
                                                        const uint16_t *__restrict__ degenerate,
                                                        const uint64_t *__restrict__ block_bitoff,
                                                        const uint32_t *__restrict__ block_seg,
                                                        uint8_t *__restrict__ signmant, uint32_t *__restrict__ stream,
                                                        uint32_t *__restrict__ seg_desc, uint8_t *__restrict__ gaps,
                                                        uint64_t total_bits, uint64_t nsegs, uint64_t stream_words,
                                                        const uint32_t *__restrict__ codes, uint32_t *__restrict__ err)
{
    constexpr uint32_t A = alphabet_of(DT);
    __shared__ Canon c;
    __shared__ uint32_t stage[kStageWords];
    __shared__ uint32_t part[kEncThreads / kWave];
    __shared__ uint32_t s_bad;
    __shared__ uint8_t gapbuf[kOnePassChunks];
    __shared__ uint32_t segbuf[kOnePassSegs];
    __shared__ uint32_t part2[2][kEncThreads / kWave];
    __shared__ uint2 ctab[256];

    const uint32_t tid = threadIdx.x;
    const uint64_t b = blockIdx.x;
    const uint64_t cb = per_block ? b : 0;
    // the code lengths and, for a full block, its first two rounds of input are
    // requested together, so the input arrives while the code table is built
    // (every vector load that the code table needs goes before the input: loads
    // complete in order, so waiting for one waits for all those issued before it)
    const uint32_t lsym = lengths[cb * A + (tid < A ? tid : A - 1)];
    const uint32_t lcode = codes ? codes[tid < A ? tid : A - 1] : 0u;
    const uint32_t degen = degenerate[cb];
    BlockIn<DT> x;
    load_block_in<DT, kEncAhead>(in, b * kBlock, (b + 1) * (uint64_t)kBlock <= n, block_bitoff, x);
    if (codes) {
        // the canonical codes came with the lengths: only the two arrays the encoder
        // reads are filled (each thread's own symbol; a barrier follows before any
        // thread reads another's)
        if (tid < A) {
            c.len[tid] = (uint8_t)lsym;
            c.code[tid] = lcode;
        }
    } else {
        canon_build_from(lsym, A, c);
    }
    const uint64_t G = block_bitoff[b];
    const uint64_t bits = block_bitoff[b + 1] - G;
    const uint32_t s0 = block_seg[b];
    const uint32_t nsb = block_seg[b + 1] - s0;
    const uint64_t lo = b * kBlock;
    const uint32_t nb = (uint32_t)(((lo + kBlock < n) ? lo + kBlock : n) - lo);
    const uint32_t nch = (uint32_t)((bits + kChunkBits - 1) / kChunkBits);
    // the geometry must be the one zx_encode_size produced for these sizes
    if (block_bitoff[b + 1] < G || block_bitoff[b + 1] > total_bits || block_seg[b + 1] < s0 || block_seg[b + 1] > nsegs ||
        bits > (uint64_t)nb * kMaxLen || (uint64_t)nsb * kSegChunks < nch || nsb == 0) {
        if (tid == 0) report(err, ZX_E_CORRUPT);
        return;
    }
    // the stream bits this block owns: up to the next block's first, or for the last
    // block to the end of the stream, padding included
    const bool last = lo + kBlock >= n;
    const uint64_t own_hi = last ? ~0ull : G + bits;
    const uint64_t zero_to = last ? stream_words : 0ull;
    if (nb == kBlock && (G & 31) + bits <= kOnePassBits) {
        const void *blk_in = reinterpret_cast<const uint8_t *>(in) + lo * (DT == ZX_BF16 ? 2 : 1);
        encode_onepass<DT, kEncAhead>(x, blk_in, lo, b, c, degen, G, (uint32_t)bits, s0, nsb, nch, own_hi, zero_to, signmant, stream, seg_desc,
                           gaps, err, stage, ctab, gapbuf, segbuf, part2, s_bad);
        return;
    }

    if (tid == 0) {
        s_bad = 0;
        seg_desc[2 * (uint64_t)s0] = (uint32_t)b;
        seg_desc[2 * (uint64_t)s0 + 1] = 0;
    }
    // chunks past the block's last chunk, in its last segment
    for (uint32_t ch = nch + tid; ch < nsb * kSegChunks; ch += kEncThreads) gaps[(uint64_t)s0 * kSegChunks + ch] = (uint8_t)ZX_NO_GAP;
    for (uint32_t i = tid; i < kStageWords; i += kEncThreads) stage[i] = 0;
    __syncthreads();

    uint32_t a0 = (uint32_t)(G & 31);   // stage bit of the round's first code
    uint64_t W = G >> 5;                // global word held by stage[0]
    uint32_t P = 0;                     // block-relative bit of the round's first code
    bool bad = false;
    const uint32_t nrounds = (nb + kRound - 1) / kRound;
    // raw 16 (BF16) or 8 (FP8) input bytes of this thread, loaded one round ahead
    constexpr uint32_t RW = BlockIn<DT>::RW;
    auto load_raw = [&](uint32_t r, uint32_t (&w)[RW]) {
        const uint32_t i0 = r * kRound + tid * kEncPerThread;
        if (i0 + kEncPerThread <= nb) {
            if (DT == ZX_BF16) {
                const uint4 q = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(in) + lo + i0);
                w[0] = q.x; w[1] = q.y; w[2 % RW] = q.z; w[3 % RW] = q.w;
            } else {
                const uint2 q = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint8_t *>(in) + lo + i0);
                w[0] = q.x; w[1] = q.y;
            }
        }
    };
    uint32_t nxt[RW];
    if (nrounds) load_raw(0, nxt);
    for (uint32_t r = 0; r < nrounds; ++r) {
        const uint32_t i0 = r * kRound + tid * kEncPerThread;   // block-relative element
        const uint32_t have = (i0 < nb) ? ((nb - i0 < kEncPerThread) ? nb - i0 : kEncPerThread) : 0;
        uint32_t cur[RW];
#pragma unroll
        for (uint32_t k = 0; k < RW; ++k) cur[k] = nxt[k];
        if (r + 1 < nrounds) load_raw(r + 1, nxt);
        uint32_t u[kEncPerThread];
        // ---- split
        if (DT == ZX_E8M0) {
            const uint8_t *src = reinterpret_cast<const uint8_t *>(in) + lo + i0;
            if (have == kEncPerThread) {
#pragma unroll
                for (uint32_t k = 0; k < kEncPerThread; ++k) u[k] = (cur[k >> 2] >> (8 * (k & 3))) & 0xFFu;
            } else {
#pragma unroll
                for (uint32_t k = 0; k < kEncPerThread; ++k) u[k] = (k < have) ? src[k] : 0u;
            }
        } else if (DT == ZX_BF16) {
            const uint16_t *src = reinterpret_cast<const uint16_t *>(in) + lo + i0;
            if (have == kEncPerThread) {
#pragma unroll
                for (uint32_t k = 0; k < kEncPerThread; ++k) u[k] = (cur[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
                uint64_t smv = 0;
#pragma unroll
                for (uint32_t k = 0; k < kEncPerThread; ++k) smv |= (uint64_t)(((u[k] >> 8) & 0x80u) | (u[k] & 0x7Fu)) << (8 * k);
                *reinterpret_cast<uint64_t *>(signmant + lo + i0) = smv;
            } else {
#pragma unroll
                for (uint32_t k = 0; k < kEncPerThread; ++k) {
                    u[k] = 0;
                    if (k < have) {
                        u[k] = src[k];
                        signmant[lo + i0 + k] = (uint8_t)(((u[k] >> 8) & 0x80u) | (u[k] & 0x7Fu));
                    }
                }
            }
        } else {
            const uint8_t *src = reinterpret_cast<const uint8_t *>(in) + lo + i0;
            if (have == kEncPerThread) {
#pragma unroll
                for (uint32_t k = 0; k < kEncPerThread; ++k) u[k] = (cur[k >> 2] >> (8 * (k & 3))) & 0xFFu;
                uint32_t nib = 0;
#pragma unroll
                for (uint32_t k = 0; k < kEncPerThread; ++k) nib |= (((u[k] >> 4) & 0x8u) | (u[k] & 0x7u)) << (4 * k);
                *reinterpret_cast<uint32_t *>(signmant + (lo + i0) / 2) = nib;
            } else {
#pragma unroll
                for (uint32_t k = 0; k < kEncPerThread; ++k) u[k] = (k < have) ? src[k] : 0u;
                for (uint32_t k = 0; k < have; k += 2) {
                    uint32_t lo_n = ((u[k] >> 4) & 0x8u) | (u[k] & 0x7u);
                    uint32_t hi_n = (k + 1 < have) ? (((u[k + 1] >> 4) & 0x8u) | (u[k + 1] & 0x7u)) : 0u;
                    signmant[(lo + i0 + k) / 2] = (uint8_t)(lo_n | (hi_n << 4));
                }
            }
        }
        // ---- code lengths of this thread's elements
        uint32_t sym[kEncPerThread];
        uint32_t tb = 0;
#pragma unroll
        for (uint32_t k = 0; k < kEncPerThread; ++k) {
            sym[k] = (DT == ZX_BF16) ? ((u[k] >> 7) & 0xFFu) : (DT == ZX_E8M0) ? u[k] : ((u[k] >> 3) & 0xFu);
            if (k < have) {
                const uint32_t l = c.len[sym[k]];
                if (bits ? (l == 0) : (sym[k] != degen)) bad = true;
                tb += l;
            }
        }
        // ---- workgroup exclusive scan of code bits
        uint32_t wtot;
        uint32_t o = wave_excl_scan(tb, wtot);
        if (lane_id() == 0) part[tid / kWave] = wtot;
        __syncthreads();
        uint32_t R = 0;
        for (uint32_t w = 0; w < kEncThreads / kWave; ++w) {
            const uint32_t pw = part[w];
            if (w < tid / kWave) o += pw;
            R += pw;
        }
        // ---- place codes, write gaps and segment entries
        uint32_t q = a0 + o;     // stage bit
        uint32_t p = P + o;      // block-relative stream bit
        const bool packed = tb <= 64;   // this thread's codes fit one 64-bit register
        uint64_t acc = 0;
#pragma unroll
        for (uint32_t k = 0; k < kEncPerThread; ++k) {
            // (elements past `have`, and symbols without a code, place nothing; the
            // loop keeps a fixed trip count so that sym[] stays in registers)
            const uint32_t l = k < have ? c.len[sym[k]] : 0u;
            if (l == 0) continue;
            const uint32_t cd = (p + kChunkBits - 1) / kChunkBits;   // first chunk boundary >= p
            if (cd * kChunkBits < p + l) {
                // this code covers the first bit of chunk cd
                uint32_t gap;
                if (cd * kChunkBits == p)
                    gap = 0;
                else
                    gap = (p + l < bits) ? p + l - cd * kChunkBits : ZX_NO_GAP;
                const uint64_t seg = s0 + cd / kSegChunks;
                gaps[seg * kSegChunks + (cd % kSegChunks)] = (uint8_t)gap;
                if (cd % kSegChunks == 0 && cd > 0) {
                    seg_desc[2 * seg] = (uint32_t)b;
                    seg_desc[2 * seg + 1] = (cd * kChunkBits == p) ? (i0 + k) : (i0 + k + 1);
                }
            }
            const uint32_t code = c.code[sym[k]];
            if (packed) {
                acc = (acc << l) | code;
            } else {
                const uint32_t sh = q & 31;
                const uint64_t x = (uint64_t)code << (64 - l - sh);
                atomicOr(&stage[q >> 5], (uint32_t)(x >> 32));
                if (sh + l > 32) atomicOr(&stage[(q >> 5) + 1], (uint32_t)x);
            }
            q += l;
            p += l;
        }
        if (packed && tb) {
            // the thread's tb bits, left-justified, placed at stage bit q0: up to
            // three words, shared with the neighbouring threads only at the ends
            const uint32_t q0 = a0 + o;
            const uint32_t sh = q0 & 31;
            const uint64_t X = acc << (64 - tb);
            uint32_t *w = &stage[q0 >> 5];
            atomicOr(&w[0], (uint32_t)(X >> (32 + sh)));
            if (sh + tb > 32) atomicOr(&w[1], (uint32_t)(X >> sh));
            if (sh + tb > 64) atomicOr(&w[2], (uint32_t)(X << (32 - sh)));
        }
        __syncthreads();
        // ---- flush whole words, keep the partial last word as the next carry
        const uint32_t nw = (a0 + R) >> 5;
        for (uint32_t i = tid; i < nw; i += kEncThreads) put_word(stream, W + i, stage[i], G, own_hi);
        const uint32_t carry = stage[nw];
        __syncthreads();
        for (uint32_t i = tid; i < kStageWords; i += kEncThreads) stage[i] = (i == 0) ? carry : 0u;
        __syncthreads();
        W += nw;
        a0 = (a0 + R) & 31;
        P += R;
    }
    if (tid == 0 && bits && a0) put_word(stream, W, stage[0], G, own_hi);
    if (zero_to) zero_stream_tail(stream, (bits && a0) ? W + 1 : W, zero_to, G);
    if (bad) s_bad = 1;
    __syncthreads();
    if (tid == 0 && s_bad) report(err, ZX_E_CODEBOOK);
    // Nothing of this path is left in flight: the compiler joins its end with the
    // one-pass path's entry, and a memory operation pending here would make the first
    // round there wait for input it does not need yet.
    __builtin_amdgcn_s_waitcnt(0);
}

// -------------------------------------------------------------------- K/V slots
// One workgroup per block: the block (always full) is encoded exactly as in
// k_encode's one-pass path, as a container of its own (block 0, stream bit 0,
// segment 0) inside slot slot_ids[j]; its codebook, sizes and descriptors go to the
// slot's entries of the pool arrays.  The code lengths, code table and block sizes
// come from the workspace filled by the histogram, codebook and block-size kernels.
struct KvSlots {
    uint8_t *signmant;
    uint32_t *stream;
    uint8_t *gaps;
    uint32_t *seg_desc;
    uint8_t *lengths;
    uint16_t *degenerate;
    uint64_t *block_bitoff;
    uint32_t *block_seg;
    uint32_t n_slots;
    uint32_t cap_bits;
    uint32_t max_segs;
    uint32_t seg_stride;
    uint64_t stream_words;
};

template <int DT>
__global__ __launch_bounds__(kEncThreads) void k_encode_slots(KvSlots P, const void *__restrict__ src,
                                                              const uint32_t *__restrict__ slot_ids,
                                                              const uint8_t *__restrict__ wlen,
                                                              const uint16_t *__restrict__ wdeg,
                                                              const uint64_t *__restrict__ wbits,
                                                              const uint32_t *__restrict__ wnseg,
                                                              uint32_t *__restrict__ status, uint32_t *__restrict__ err)
{
    constexpr uint32_t A = alphabet_of(DT);
    constexpr uint32_t kSmBytes = DT == ZX_BF16 ? kBlock : kBlock / 2;
    __shared__ Canon c;
    __shared__ uint32_t stage[kStageWords];
    __shared__ uint32_t s_bad;
    __shared__ uint8_t gapbuf[kOnePassChunks];
    __shared__ uint32_t segbuf[kOnePassSegs];
    __shared__ uint32_t part2[2][kEncThreads / kWave];
    __shared__ uint2 ctab[256];

    const uint32_t tid = threadIdx.x;
    const uint64_t j = blockIdx.x;
    // (the loads the code table and the sizes need go before the input, which
    // completes in order after them)
    const uint32_t lsym = wlen[j * A + (tid < A ? tid : A - 1)];
    const uint32_t slot = slot_ids[j];
    const uint32_t degen = wdeg[j];
    const uint64_t bits = wbits[j + 1];
    const uint32_t nsb = wnseg[j + 1];
    BlockIn<DT> x;
    load_block_in<DT, kEncAhead>(src, j * kBlock, true, nullptr, x);
    canon_build_from(lsym, A, c);
    if (slot >= P.n_slots) {
        if (tid == 0) {
            status[j] = ZX_E_INVAL;
            report(err, ZX_E_INVAL);
        }
        return;
    }
    if (bits > P.cap_bits || nsb > P.max_segs) {
        // the block does not fit: the slot is left holding no segments
        if (tid == 0) {
            P.block_bitoff[2 * (uint64_t)slot] = 0;
            P.block_bitoff[2 * (uint64_t)slot + 1] = 0;
            P.block_seg[2 * (uint64_t)slot] = 0;
            P.block_seg[2 * (uint64_t)slot + 1] = 0;
            status[j] = ZX_E_NOSPACE;
            report(err, ZX_E_NOSPACE);
        }
        return;
    }
    uint8_t *sm = P.signmant + (uint64_t)slot * kSmBytes;
    uint32_t *st = P.stream + (uint64_t)slot * P.stream_words;
    uint8_t *gp = P.gaps + (uint64_t)slot * P.seg_stride * kSegChunks;
    uint32_t *sd = P.seg_desc + (uint64_t)slot * P.seg_stride * 2;
    if (tid < A) P.lengths[(uint64_t)slot * A + tid] = (uint8_t)lsym;
    if (tid == 0) {
        P.degenerate[slot] = (uint16_t)degen;
        P.block_bitoff[2 * (uint64_t)slot] = 0;
        P.block_bitoff[2 * (uint64_t)slot + 1] = bits;
        P.block_seg[2 * (uint64_t)slot] = 0;
        P.block_seg[2 * (uint64_t)slot + 1] = nsb;
    }
    const uint32_t nch = (uint32_t)((bits + kChunkBits - 1) / kChunkBits);
    const void *blk_in = reinterpret_cast<const uint8_t *>(src) + j * kBlock * (DT == ZX_BF16 ? 2 : 1);
    encode_onepass<DT, kEncAhead>(x, blk_in, 0, 0, c, degen, 0, (uint32_t)bits, 0, nsb, nch, ~0ull, 0ull, sm, st, sd, gp, err, stage,
                       ctab, gapbuf, segbuf, part2, s_bad);
    // the rest of the slot's stream, padding included, is zero
    const uint32_t nw = (uint32_t)((bits + 31) / 32);
    for (uint64_t w = nw + tid; w < P.stream_words; w += kEncThreads) st[w] = 0;
    if (tid == 0) status[j] = s_bad ? ZX_E_CODEBOOK : ZX_OK;
}

// The same append in one launch, with no workspace: each workgroup builds its block's
// histogram from the input it holds in registers (32 lane copies in LDS), its code lengths in one wavefront (the codebook's
// LDS in the stage, which the rounds overwrite later), and its bits and segment count,
// then encodes exactly as k_encode_slots.
constexpr uint32_t kFusedHistCopies = 32;
static_assert((kFusedHistCopies & (kFusedHistCopies - 1)) == 0 && kFusedHistCopies <= kWave, "copies: a power of two, at most a wavefront");

template <int DT>
__device__ __forceinline__ uint32_t block_exp(const BlockIn<DT> &x, uint32_t r, uint32_t e)
{
    if constexpr (DT == ZX_BF16) return (x.w[r][e >> 1] >> (16 * (e & 1) + 7)) & 0xFFu;
    return (x.w[r][e >> 2] >> (8 * (e & 3) + 3)) & 0xFu;
}

template <int DT>
__global__ __launch_bounds__(kEncThreads) void k_encode_slots_fused(KvSlots P, const void *__restrict__ src,
                                                                    const uint32_t *__restrict__ slot_ids, uint32_t max_len,
                                                                    uint32_t *__restrict__ status, uint32_t *__restrict__ err)
{
    constexpr uint32_t A = alphabet_of(DT);
    constexpr uint32_t kSmBytes = DT == ZX_BF16 ? kBlock : kBlock / 2;
    __shared__ Canon c;
    __shared__ __align__(16) uint32_t stage[kStageWords];
    __shared__ uint32_t s_bad;
    __shared__ uint8_t gapbuf[kOnePassChunks];
    __shared__ uint32_t segbuf[kOnePassSegs];
    __shared__ uint32_t part2[2][kEncThreads / kWave];
    __shared__ uint32_t hbuf[A * kFusedHistCopies];
    __shared__ uint2 ctab[256];
    __shared__ uint8_t lenbuf[256];
    __shared__ uint16_t degbuf;
    static_assert(sizeof(CodebookLds<uint32_t>) <= sizeof(stage), "the codebook's LDS fits the stage");

    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid % kWave;
    const uint32_t wave = tid / kWave;
    const uint64_t j = blockIdx.x;
    BlockIn<DT> x;
    load_block_in<DT, kRoundsPerBlock>(src, j * kBlock, true, nullptr, x);
    const uint32_t slot = slot_ids[j];
    // histogram: lane l counts into copy l % 32, laid out bin-major (copy k's count of
    // value v at 32 v + k), so the bank of a counter depends on the lane alone and
    // lanes l and l + 32 are the only ones an instruction's atomics pair up
    uint32_t *h = hbuf;
    for (uint32_t i = tid; i < A * kFusedHistCopies; i += kEncThreads) h[i] = 0;
    __syncthreads();
    uint32_t *mine = h + lane % kFusedHistCopies;
#pragma unroll
    for (uint32_t r = 0; r < kRoundsPerBlock; ++r) {
#pragma unroll
        for (uint32_t e = 0; e < kEncPerThread; ++e) atomicAdd(&mine[block_exp<DT>(x, r, e) * kFusedHistCopies], 1u);
    }
    __syncthreads();
    CodebookLds<uint32_t> &L = *reinterpret_cast<CodebookLds<uint32_t> *>(stage);
    if (tid < A) {
        // the copies of value tid, read rotated by tid so that a wavefront's reads fall
        // in distinct banks
        uint32_t t = 0;
        for (uint32_t k = 0; k < kFusedHistCopies; ++k) t += h[tid * kFusedHistCopies + ((k + tid) & (kFusedHistCopies - 1))];
        L.cnt[tid] = t;
    }
    __syncthreads();
    if (wave == 0) codebook_wave<A, uint32_t>(L, max_len, lenbuf, &degbuf);
    __syncthreads();
    const uint32_t lsym = tid < A ? lenbuf[tid] : 0u;
    // the block's bits: count x length summed over the workgroup
    {
        uint32_t tot;
        wave_excl_scan(tid < A ? L.cnt[tid] * lsym : 0u, tot);
        if (lane == 0) part2[0][wave] = tot;
    }
    __syncthreads();
    uint32_t bits32 = 0;
    for (uint32_t w = 0; w < kEncThreads / kWave; ++w) bits32 += part2[0][w];
    const uint64_t bits = bits32;
    const uint32_t nch = (uint32_t)((bits + kChunkBits - 1) / kChunkBits);
    const uint32_t nsb = nch ? (nch + kSegChunks - 1) / kSegChunks : 1u;
    const uint32_t degen = degbuf;
    canon_build_from(lsym, A, c);   // (its barriers also end every read of the codebook's LDS)
    if (slot >= P.n_slots) {
        if (tid == 0) {
            status[j] = ZX_E_INVAL;
            report(err, ZX_E_INVAL);
        }
        return;
    }
    if (bits > P.cap_bits || nsb > P.max_segs) {
        // the block does not fit: the slot is left holding no segments
        if (tid == 0) {
            P.block_bitoff[2 * (uint64_t)slot] = 0;
            P.block_bitoff[2 * (uint64_t)slot + 1] = 0;
            P.block_seg[2 * (uint64_t)slot] = 0;
            P.block_seg[2 * (uint64_t)slot + 1] = 0;
            status[j] = ZX_E_NOSPACE;
            report(err, ZX_E_NOSPACE);
        }
        return;
    }
    uint8_t *sm = P.signmant + (uint64_t)slot * kSmBytes;
    uint32_t *st = P.stream + (uint64_t)slot * P.stream_words;
    uint8_t *gp = P.gaps + (uint64_t)slot * P.seg_stride * kSegChunks;
    uint32_t *sd = P.seg_desc + (uint64_t)slot * P.seg_stride * 2;
    if (tid < A) P.lengths[(uint64_t)slot * A + tid] = (uint8_t)lsym;
    if (tid == 0) {
        P.degenerate[slot] = (uint16_t)degen;
        P.block_bitoff[2 * (uint64_t)slot] = 0;
        P.block_bitoff[2 * (uint64_t)slot + 1] = bits;
        P.block_seg[2 * (uint64_t)slot] = 0;
        P.block_seg[2 * (uint64_t)slot + 1] = nsb;
    }
    encode_onepass<DT, kRoundsPerBlock>(x, nullptr, 0, 0, c, degen, 0, (uint32_t)bits, 0, nsb, nch, ~0ull, 0ull, sm, st, sd, gp, err, stage,
                       ctab, gapbuf, segbuf, part2, s_bad);
    // the rest of the slot's stream, padding included, is zero
    const uint32_t nw = (uint32_t)((bits + 31) / 32);
    for (uint64_t w = nw + tid; w < P.stream_words; w += kEncThreads) st[w] = 0;
    if (tid == 0) status[j] = s_bad ? ZX_E_CODEBOOK : ZX_OK;
}

// -------------------------------------------------------------------- planning
// Everything a per-tensor-codebook encode needs before its outputs can be sized, in
// one workgroup after the block histograms: the tensor histogram (the sum of the
// block ones), the code lengths (one wavefront), each block's bits and segments
// (sum of count x length over its histogram), their scan, and the two totals.  The
// totals are then published (to a pinned host word if the caller gave one, with a
// tag written last, so a host thread can wait on it without waiting for the whole
// kernel), the error word cleared, and the decode table built while the host sizes
// the outputs.  For tensors of at most kPlanMaxBlocks blocks (and their histograms
// at most kPlanMaxHistWords words, read by this one workgroup).
constexpr uint32_t kPlanThreads = 1024;
constexpr uint32_t kPlanMaxBlocks = 2048;
constexpr uint64_t kPlanMaxHistWords = 1u << 17;

__device__ __forceinline__ void publish_totals(uint64_t total_bits, uint64_t nsegs, uint64_t *totals,
                                               uint64_t *totals_host, uint64_t tag, uint32_t *err)
{
    totals[0] = total_bits;
    totals[1] = nsegs;
    if (err) *err = 0;
    if (totals_host) {
        totals_host[0] = total_bits;
        totals_host[1] = nsegs;
        __hip_atomic_store(&totals_host[2], tag, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }
}

template <int DT>
__global__ __launch_bounds__(kPlanThreads) void k_plan(const uint32_t *__restrict__ block_hist, uint32_t nb,
                                                       uint32_t max_len, uint8_t *__restrict__ lengths,
                                                       uint16_t *__restrict__ degenerate, uint64_t *__restrict__ block_bitoff,
                                                       uint32_t *__restrict__ block_seg, uint64_t *__restrict__ totals,
                                                       uint64_t *totals_host, uint64_t tag, DTab *__restrict__ dtab,
                                                       uint32_t *__restrict__ codes, uint32_t *__restrict__ err)
{
    constexpr uint32_t A = alphabet_of(DT);
    struct TableLds {
        Canon c;
        uint16_t t1[kLutSize];
    };
    __shared__ union {
        CodebookLds<uint32_t> cb;
        TableLds tb;
    } u;
    __shared__ uint32_t part[kPlanThreads * 4];
    __shared__ uint32_t bbits[kPlanMaxBlocks];
    __shared__ uint32_t bsegs[kPlanMaxBlocks];
    __shared__ uint64_t wsum_b[kPlanThreads / kWave];
    __shared__ uint32_t wsum_s[kPlanThreads / kWave];
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = lane_id();
    const uint32_t wave = tid / kWave;

    // The block histograms as 16-byte pieces: piece j holds bins 4 (j % (A/4)) .. +3
    // of block j / (A/4).  Thread t takes pieces t + 1024 k, so it always sees the same
    // four bins (of blocks t / (A/4) + G4 k), and the pieces go out eight at a time.
    constexpr uint32_t Q = A / 4;                  // pieces per block
    static_assert(Q == kWave || Q == 4, "a block's pieces are one wavefront or one quad of lanes");
    constexpr uint32_t G4 = kPlanThreads / Q;      // blocks per sweep of the workgroup
    const uint4 *hp = reinterpret_cast<const uint4 *>(block_hist);
    const uint32_t npieces = nb * Q;
    const uint32_t q = tid % Q;
    // Up to kKeep pieces per thread (every tensor of up to 16384 pieces: 256 BF16
    // blocks, 4096 FP8 ones) stay in registers from the histogram sum to the block
    // bits; larger plans read them again.
    constexpr uint32_t kKeep = 16;
    const bool keep = npieces <= kKeep * kPlanThreads;
    uint4 kept[kKeep];
    // tensor histogram: per-thread sums of its four bins, then the G4 groups summed
    {
        uint4 acc = make_uint4(0, 0, 0, 0);
        if (keep) {
#pragma unroll
            for (uint32_t k = 0; k < kKeep; ++k) {
                const uint32_t j = tid + k * kPlanThreads;
                kept[k] = j < npieces ? hp[j] : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (uint32_t k = 0; k < kKeep; ++k) {
                acc.x += kept[k].x; acc.y += kept[k].y; acc.z += kept[k].z; acc.w += kept[k].w;
            }
        } else {
            for (uint32_t j0 = 0; j0 < npieces; j0 += 8 * kPlanThreads) {   // (the same trip count on every lane)
                uint4 v[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const uint32_t j = j0 + tid + k * kPlanThreads;
                    v[k] = j < npieces ? hp[j] : make_uint4(0, 0, 0, 0);
                }
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    acc.x += v[k].x; acc.y += v[k].y; acc.z += v[k].z; acc.w += v[k].w;
                }
            }
        }
        const uint32_t g = tid / Q;
        part[g * A + 4 * q + 0] = acc.x;
        part[g * A + 4 * q + 1] = acc.y;
        part[g * A + 4 * q + 2] = acc.z;
        part[g * A + 4 * q + 3] = acc.w;
    }
    __syncthreads();
    if constexpr (A == 256) {   // 16 partial sums per bin
        if (tid < A) {
            uint32_t t = 0;
            for (uint32_t g = 0; g < G4; ++g) t += part[g * A + tid];
            u.cb.cnt[tid] = t;
        }
    } else {                    // 256 partial sums per bin: wavefront w sums bin w
        if (wave < A) {
            uint32_t t = 0;
            for (uint32_t g = lane; g < G4; g += kWave) t += part[g * A + wave];
            uint32_t tot;
            wave_excl_scan(t, tot);
            if (lane == 0) u.cb.cnt[wave] = tot;
        }
    }
    __syncthreads();
    if (wave == 0) codebook_wave<A, uint32_t>(u.cb, max_len, lengths, degenerate);
    __syncthreads();

    // each block's bits: every piece weighted by its four lengths and summed over the
    // Q threads (adjacent lanes) that hold one block
    {
        const uint32_t l0 = u.cb.out_len[4 * q], l1 = u.cb.out_len[4 * q + 1];
        const uint32_t l2 = u.cb.out_len[4 * q + 2], l3 = u.cb.out_len[4 * q + 3];
        auto block_bits = [&](const uint4 v, const uint32_t j) {
            uint32_t bits = v.x * l0 + v.y * l1 + v.z * l2 + v.w * l3;
            if constexpr (Q == kWave) {
                uint32_t tot;
                wave_excl_scan(bits, tot);
                bits = tot;
            } else {                    // a quad of lanes: DPP quad permutes [1,0,3,2], then [2,3,0,1]
                bits += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)bits, 0xB1, 0xF, 0xF, false);
                bits += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)bits, 0x4E, 0xF, 0xF, false);
            }
            if (q == 0 && j < npieces) {
                const uint32_t b = j / Q;
                const uint32_t nch = (bits + kChunkBits - 1) / kChunkBits;
                const uint32_t ns = (nch + kSegChunks - 1) / kSegChunks;
                bbits[b] = bits;
                bsegs[b] = ns ? ns : 1u;
            }
        };
        if (keep) {
#pragma unroll
            for (uint32_t k = 0; k < kKeep; ++k) block_bits(kept[k], tid + k * kPlanThreads);
        } else {
            for (uint32_t j0 = 0; j0 < npieces; j0 += 8 * kPlanThreads) {   // (every lane shuffles: same trip count)
                uint4 v[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const uint32_t j = j0 + tid + k * kPlanThreads;
                    v[k] = j < npieces ? hp[j] : make_uint4(0, 0, 0, 0);
                }
#pragma unroll
                for (int k = 0; k < 8; ++k) block_bits(v[k], j0 + tid + k * kPlanThreads);
            }
        }
    }
    // the table build below reuses the codebook's LDS: each thread keeps its
    // symbol's length
    const uint32_t mylen = tid < A ? u.cb.out_len[tid] : 0u;
    __syncthreads();

    // inclusive scan: thread t owns blocks 2t and 2t + 1
    uint64_t vb0 = 0, vb1 = 0;
    uint32_t vs0 = 0, vs1 = 0;
    if (2 * tid < nb) { vb0 = bbits[2 * tid]; vs0 = bsegs[2 * tid]; }
    if (2 * tid + 1 < nb) { vb1 = bbits[2 * tid + 1]; vs1 = bsegs[2 * tid + 1]; }
    uint64_t xb = vb0 + vb1;
    uint32_t xs = vs0 + vs1;
    for (int d = 1; d < kWave; d <<= 1) {
        const uint64_t yb = __shfl_up(xb, d, kWave);
        const uint32_t ys = __shfl_up(xs, d, kWave);
        if (lane >= (uint32_t)d) { xb += yb; xs += ys; }
    }
    if (lane == kWave - 1) { wsum_b[wave] = xb; wsum_s[wave] = xs; }
    __syncthreads();
    uint64_t ob = 0, total_b = 0;
    uint32_t os = 0, total_s = 0;
    for (uint32_t w = 0; w < kPlanThreads / kWave; ++w) {
        if (w < wave) { ob += wsum_b[w]; os += wsum_s[w]; }
        total_b += wsum_b[w];
        total_s += wsum_s[w];
    }
    ob += xb - (vb0 + vb1);   // exclusive prefix of this thread's pair
    os += xs - (vs0 + vs1);
    if (2 * tid < nb) { block_bitoff[2 * tid + 1] = ob + vb0; block_seg[2 * tid + 1] = os + vs0; }
    if (2 * tid + 1 < nb) { block_bitoff[2 * tid + 2] = ob + vb0 + vb1; block_seg[2 * tid + 2] = os + vs0 + vs1; }
    if (tid == 0) {
        block_bitoff[0] = 0;
        block_seg[0] = 0;
        publish_totals(total_b, total_s, totals, totals_host, tag, err);
    }
    if (!dtab && !codes) return;
    // the canonical codes and the decode table, once the totals are out
    canon_build_from(mylen, A, u.tb.c);
    if (codes && tid < A) codes[tid] = u.tb.c.code[tid];
    if (dtab) dtab_fill(u.tb.c, A, *dtab, u.tb.t1);
}

// The canonical code of each symbol, for zx_encode_coded (the larger-tensor planning
// path; k_plan writes them itself).
__global__ __launch_bounds__(1024) void k_canon_codes(const uint8_t *__restrict__ lengths, uint32_t A, uint32_t *__restrict__ codes)
{
    __shared__ Canon c;
    canon_build(lengths, A, c);
    if (threadIdx.x < A) codes[threadIdx.x] = c.code[threadIdx.x];
}

// The planning steps' last one for larger tensors (after k_scan_blocks).
__global__ void k_publish(uint64_t *totals, uint64_t *totals_host, uint64_t tag, uint32_t *err)
{
    if (threadIdx.x == 0) publish_totals(totals[0], totals[1], totals, totals_host, tag, err);
}

}  // namespace zxk

using namespace zxk;

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Whole 16-byte groups of code words, then kStreamPadWords zero words: a decoder
// may read one segment's rows (256 words and two more) from any segment start
// without a bounds check.
extern "C" uint64_t zx_stream_words(uint64_t total_bits)
{
    uint64_t w = (total_bits + 31) / 32;
    w = (w + 3) / 4 * 4;
    return w + kStreamPadWords;
}

extern "C" zx_status zx_encode_size(zx_dtype dtype, const void *in, uint64_t n, int per_block,
                                    const uint8_t *lengths, const uint32_t *block_hist,
                                    uint64_t *block_bitoff, uint32_t *block_seg, uint64_t *totals,
                                    hipStream_t stream)
{
    if (dtype != ZX_BF16 && dtype != ZX_FP8_E4M3FN && dtype != ZX_E8M0) return ZX_E_UNSUPPORTED;
    if (!block_bitoff || !block_seg || !totals) return ZX_E_INVAL;
    const uint64_t nblocks = (n + kBlock - 1) / kBlock;
    if (nblocks > 0x7FFFFFFFull) return ZX_E_INVAL;
    if (nblocks && (!lengths || (!block_hist && !in))) return ZX_E_INVAL;
    if (!aligned16(in) || !aligned16(block_hist)) return ZX_E_INVAL;
    if (nblocks) {
        if (dtype == ZX_BF16)
            hipLaunchKernelGGL(k_block_bits<ZX_BF16>, dim3((uint32_t)nblocks), dim3(kSizeThreads), 0, stream, in, n, per_block, lengths,
                               block_hist, block_bitoff, block_seg);
        else if (dtype == ZX_E8M0)
            hipLaunchKernelGGL(k_block_bits<ZX_E8M0>, dim3((uint32_t)nblocks), dim3(kSizeThreads), 0, stream, in, n, per_block, lengths,
                               block_hist, block_bitoff, block_seg);
        else
            hipLaunchKernelGGL(k_block_bits<ZX_FP8_E4M3FN>, dim3((uint32_t)nblocks), dim3(kSizeThreads), 0, stream, in, n, per_block,
                               lengths, block_hist, block_bitoff, block_seg);
        if (hipGetLastError() != hipSuccess) return ZX_E_HIP;
    }
    hipLaunchKernelGGL(k_scan_blocks, dim3(1), dim3(1024), 0, stream, nblocks, block_bitoff, block_seg, totals);
    return hipGetLastError() == hipSuccess ? ZX_OK : ZX_E_HIP;
}

extern "C" zx_status zx_encode_plan(zx_dtype dtype, const void *in, uint64_t n, uint32_t max_len,
                                    uint32_t *block_hist, uint32_t *tensor_hist, uint8_t *lengths,
                                    uint16_t *degenerate, uint64_t *block_bitoff, uint32_t *block_seg,
                                    uint64_t *totals, uint64_t *totals_host, uint64_t tag, uint32_t *dtab,
                                    uint32_t *codes, uint32_t *err, hipStream_t stream)
{
    if (dtype != ZX_BF16 && dtype != ZX_FP8_E4M3FN && dtype != ZX_E8M0) return ZX_E_UNSUPPORTED;
    const uint32_t A = alphabet_of(dtype);
    if (max_len < (A == 256 ? 8u : 4u) || max_len > kMaxLen) return ZX_E_CODEBOOK;
    if (!block_hist || !tensor_hist || !lengths || !degenerate || !block_bitoff || !block_seg || !totals) return ZX_E_INVAL;
    if ((n && !in) || n >= (1ull << 32)) return ZX_E_INVAL;
    if (!aligned16(in) || !aligned16(block_hist) || !aligned16(tensor_hist) || !aligned16(dtab) ||
        ((uintptr_t)totals & 7u) || ((uintptr_t)block_bitoff & 7u) || ((uintptr_t)totals_host & 7u) || ((uintptr_t)codes & 3u))
        return ZX_E_INVAL;
    const uint64_t nblocks = (n + kBlock - 1) / kBlock;
    zx_status st;
    if (nblocks <= kPlanMaxBlocks && nblocks * A <= kPlanMaxHistWords) {
        // block histograms, then the one planning workgroup
        if (nblocks && (st = zx_histogram(dtype, in, n, nullptr, block_hist, stream)) != ZX_OK) return st;
        DTab *t = reinterpret_cast<DTab *>(dtab);
        if (A == 256)
            hipLaunchKernelGGL(k_plan<ZX_BF16>, dim3(1), dim3(kPlanThreads), 0, stream, block_hist, (uint32_t)nblocks, max_len,
                               lengths, degenerate, block_bitoff, block_seg, totals, totals_host, tag, t, codes, err);
        else
            hipLaunchKernelGGL(k_plan<ZX_FP8_E4M3FN>, dim3(1), dim3(kPlanThreads), 0, stream, block_hist, (uint32_t)nblocks,
                               max_len, lengths, degenerate, block_bitoff, block_seg, totals, totals_host, tag, t, codes, err);
        return hipGetLastError() == hipSuccess ? ZX_OK : ZX_E_HIP;
    }
    // larger tensors: the separate steps, then the totals published and the table built
    if ((st = zx_histogram(dtype, in, n, tensor_hist, block_hist, stream)) != ZX_OK) return st;
    if ((st = zx_build_codebook(dtype, tensor_hist, 1, max_len, lengths, degenerate, stream)) != ZX_OK) return st;
    if ((st = zx_encode_size(dtype, in, n, 0, lengths, block_hist, block_bitoff, block_seg, totals, stream)) != ZX_OK)
        return st;
    hipLaunchKernelGGL(k_publish, dim3(1), dim3(64), 0, stream, totals, totals_host, tag, err);
    if (hipGetLastError() != hipSuccess) return ZX_E_HIP;
    if (codes) {
        hipLaunchKernelGGL(k_canon_codes, dim3(1), dim3(1024), 0, stream, lengths, A, codes);
        if (hipGetLastError() != hipSuccess) return ZX_E_HIP;
    }
    if (dtab) return zx_build_decode_table(dtype, lengths, dtab, stream);
    return ZX_OK;
}

static zx_status encode_impl(zx_dtype dtype, const void *in, uint64_t n, int per_block, const uint8_t *lengths,
                             const uint16_t *degenerate, const uint64_t *block_bitoff, const uint32_t *block_seg,
                             uint64_t total_bits, uint64_t nsegs, uint8_t *signmant, uint32_t *stream, uint32_t *seg_desc,
                             uint8_t *gaps, const uint32_t *codes, uint32_t *err, hipStream_t stream_)
{
    if (dtype != ZX_BF16 && dtype != ZX_FP8_E4M3FN && dtype != ZX_E8M0) return ZX_E_UNSUPPORTED;
    const uint64_t nblocks = (n + kBlock - 1) / kBlock;
    if (nblocks > 0x7FFFFFFFull || nsegs > 0xFFFFFFFFull) return ZX_E_INVAL;
    if (!stream || !block_bitoff) return ZX_E_INVAL;
    if (nblocks && (!in || !lengths || !degenerate || !block_seg || (!signmant && dtype != ZX_E8M0) || !seg_desc || !gaps))
        return ZX_E_INVAL;
    if (!aligned16(in) || !aligned16(signmant) || !aligned16(stream)) return ZX_E_INVAL;
    if (nsegs < nblocks) return ZX_E_INVAL;
    const uint64_t words = zx_stream_words(total_bits);
    if (nblocks == 0) {   // no block to clear the padding
        hipLaunchKernelGGL(k_zero_stream, dim3(1), dim3(256), 0, stream_, words, stream);
        return hipGetLastError() == hipSuccess ? ZX_OK : ZX_E_HIP;
    }
    if (dtype == ZX_BF16)
        hipLaunchKernelGGL(k_encode<ZX_BF16>, dim3((uint32_t)nblocks), dim3(kEncThreads), 0, stream_, in, n, per_block, lengths,
                           degenerate, block_bitoff, block_seg, signmant, stream, seg_desc, gaps, total_bits, nsegs, words, codes, err);
    else if (dtype == ZX_E8M0)
        hipLaunchKernelGGL(k_encode<ZX_E8M0>, dim3((uint32_t)nblocks), dim3(kEncThreads), 0, stream_, in, n, per_block, lengths,
                           degenerate, block_bitoff, block_seg, signmant, stream, seg_desc, gaps, total_bits, nsegs, words, codes, err);
    else
        hipLaunchKernelGGL(k_encode<ZX_FP8_E4M3FN>, dim3((uint32_t)nblocks), dim3(kEncThreads), 0, stream_, in, n, per_block, lengths,
                           degenerate, block_bitoff, block_seg, signmant, stream, seg_desc, gaps, total_bits, nsegs, words, codes, err);
    return hipGetLastError() == hipSuccess ? ZX_OK : ZX_E_HIP;
}

extern "C" zx_status zx_encode(zx_dtype dtype, const void *in, uint64_t n, int per_block,
                               const uint8_t *lengths, const uint16_t *degenerate,
                               const uint64_t *block_bitoff, const uint32_t *block_seg,
                               uint64_t total_bits, uint64_t nsegs,
                               uint8_t *signmant, uint32_t *stream, uint32_t *seg_desc, uint8_t *gaps,
                               uint32_t *err, hipStream_t stream_)
{
    return encode_impl(dtype, in, n, per_block, lengths, degenerate, block_bitoff, block_seg, total_bits, nsegs, signmant,
                       stream, seg_desc, gaps, nullptr, err, stream_);
}

extern "C" zx_status zx_encode_coded(zx_dtype dtype, const void *in, uint64_t n, const uint8_t *lengths,
                                     const uint32_t *codes, const uint16_t *degenerate,
                                     const uint64_t *block_bitoff, const uint32_t *block_seg,
                                     uint64_t total_bits, uint64_t nsegs,
                                     uint8_t *signmant, uint32_t *stream, uint32_t *seg_desc, uint8_t *gaps,
                                     uint32_t *err, hipStream_t stream_)
{
    if (!codes || ((uintptr_t)codes & 3u)) return ZX_E_INVAL;
    return encode_impl(dtype, in, n, 0, lengths, degenerate, block_bitoff, block_seg, total_bits, nsegs, signmant, stream,
                       seg_desc, gaps, codes, err, stream_);
}

// ---- K/V slot pool
static constexpr uint32_t kv_alphabet(zx_dtype d) { return d == ZX_BF16 ? 256u : 16u; }

extern "C" zx_status zx_kv_slot_sizes(zx_dtype dtype, uint32_t cap_words, zx_kv_sizes *out)
{
    if (dtype != ZX_BF16 && dtype != ZX_FP8_E4M3FN) return ZX_E_UNSUPPORTED;
    if (!out || cap_words < 256 || cap_words > kStageWords - 2 || cap_words % 256 != 0) return ZX_E_INVAL;
    out->sm_bytes = dtype == ZX_BF16 ? kBlock : kBlock / 2;
    out->stream_words = zx_stream_words((uint64_t)cap_words * 32);
    out->max_segs = cap_words / (kSegBits / 32);
    out->seg_stride = (out->max_segs + 1) & ~1u;
    out->alphabet = kv_alphabet(dtype);
    out->reserved_ = 0;
    return ZX_OK;
}

// workspace: hist u32[nblk][A], lengths u8[nblk][A], degenerate u16[nblk],
// bits u64[nblk+1], segments u32[nblk+1]; each part 16-byte aligned
static constexpr size_t kv_round16(size_t x) { return (x + 15) & ~(size_t)15; }
struct KvWs {
    size_t hist, len, deg, bits, nseg, total;
};
static constexpr KvWs kv_ws(zx_dtype dtype, uint32_t nblk)
{
    const size_t A = kv_alphabet(dtype);
    KvWs w{};
    w.hist = 0;
    w.len = w.hist + kv_round16((size_t)nblk * A * 4);
    w.deg = w.len + kv_round16((size_t)nblk * A);
    w.bits = w.deg + kv_round16((size_t)nblk * 2);
    w.nseg = w.bits + kv_round16(((size_t)nblk + 1) * 8);
    w.total = w.nseg + kv_round16(((size_t)nblk + 1) * 4);
    return w;
}

extern "C" size_t zx_kv_workspace_bytes(zx_dtype dtype, uint32_t nblk) { return kv_ws(dtype, nblk).total; }

static bool kv_pool_ok(const zx_kv_pool *p, zx_kv_sizes *sz)
{
    if (!p || zx_kv_slot_sizes((zx_dtype)p->dtype, p->cap_words, sz) != ZX_OK) return false;
    if (!p->signmant || !p->stream || !p->gaps || !p->seg_desc || !p->lengths || !p->degenerate || !p->block_bitoff ||
        !p->block_seg)
        return false;
    return aligned16(p->signmant) && aligned16(p->stream) && aligned16(p->seg_desc) && aligned16(p->block_bitoff) &&
           ((uintptr_t)p->block_seg & 7u) == 0;
}

extern "C" zx_status zx_kv_encode_slots(const zx_kv_pool *pool, const void *src, uint32_t nblk, const uint32_t *slot_ids,
                                        uint32_t max_len, void *workspace, size_t ws_bytes, uint32_t *status, uint32_t *err,
                                        hipStream_t stream)
{
    if (pool && pool->dtype != ZX_BF16 && pool->dtype != ZX_FP8_E4M3FN) return ZX_E_UNSUPPORTED;
    zx_kv_sizes sz;
    if (!kv_pool_ok(pool, &sz)) return ZX_E_INVAL;
    if (nblk == 0) return ZX_OK;
    const zx_dtype dtype = (zx_dtype)pool->dtype;
    const KvWs w = kv_ws(dtype, nblk);
    if (!src || !slot_ids || !status || !workspace || !aligned16(src) || !aligned16(workspace) || ws_bytes < w.total ||
        nblk > 0x7FFFFFFFu)
        return ZX_E_INVAL;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    uint32_t *hist = reinterpret_cast<uint32_t *>(ws + w.hist);
    uint8_t *len = ws + w.len;
    uint16_t *deg = reinterpret_cast<uint16_t *>(ws + w.deg);
    uint64_t *bits = reinterpret_cast<uint64_t *>(ws + w.bits);
    uint32_t *nseg = reinterpret_cast<uint32_t *>(ws + w.nseg);
    const uint64_t n = (uint64_t)nblk * kBlock;
    zx_status st = zx_histogram(dtype, src, n, nullptr, hist, stream);
    if (st != ZX_OK) return st;
    st = zx_build_codebook(dtype, hist, nblk, max_len, len, deg, stream);
    if (st != ZX_OK) return st;
    if (dtype == ZX_BF16)
        hipLaunchKernelGGL(k_block_bits<ZX_BF16>, dim3(nblk), dim3(kSizeThreads), 0, stream, src, n, 1, len, hist, bits, nseg);
    else
        hipLaunchKernelGGL(k_block_bits<ZX_FP8_E4M3FN>, dim3(nblk), dim3(kSizeThreads), 0, stream, src, n, 1, len, hist, bits,
                           nseg);
    if (hipGetLastError() != hipSuccess) return ZX_E_HIP;
    KvSlots P;
    P.signmant = pool->signmant;
    P.stream = pool->stream;
    P.gaps = pool->gaps;
    P.seg_desc = pool->seg_desc;
    P.lengths = pool->lengths;
    P.degenerate = pool->degenerate;
    P.block_bitoff = pool->block_bitoff;
    P.block_seg = pool->block_seg;
    P.n_slots = pool->n_slots;
    P.cap_bits = pool->cap_words * 32;
    P.max_segs = sz.max_segs;
    P.seg_stride = sz.seg_stride;
    P.stream_words = sz.stream_words;
    if (dtype == ZX_BF16)
        hipLaunchKernelGGL(k_encode_slots<ZX_BF16>, dim3(nblk), dim3(kEncThreads), 0, stream, P, src, slot_ids, len, deg, bits,
                           nseg, status, err);
    else
        hipLaunchKernelGGL(k_encode_slots<ZX_FP8_E4M3FN>, dim3(nblk), dim3(kEncThreads), 0, stream, P, src, slot_ids, len, deg,
                           bits, nseg, status, err);
    return hipGetLastError() == hipSuccess ? ZX_OK : ZX_E_HIP;
}

extern "C" zx_status zx_kv_encode_slots_fused(const zx_kv_pool *pool, const void *src, uint32_t nblk,
                                              const uint32_t *slot_ids, uint32_t max_len, uint32_t *status, uint32_t *err,
                                              hipStream_t stream)
{
    if (pool && pool->dtype != ZX_BF16 && pool->dtype != ZX_FP8_E4M3FN) return ZX_E_UNSUPPORTED;
    zx_kv_sizes sz;
    if (!kv_pool_ok(pool, &sz)) return ZX_E_INVAL;
    const uint32_t A = alphabet_of(pool->dtype);
    if (max_len < (A == 256 ? 8u : 4u) || max_len > kMaxLen) return ZX_E_CODEBOOK;
    if (nblk == 0) return ZX_OK;
    if (!src || !slot_ids || !status || !aligned16(src) || nblk > 0x7FFFFFFFu) return ZX_E_INVAL;
    KvSlots P;
    P.signmant = pool->signmant;
    P.stream = pool->stream;
    P.gaps = pool->gaps;
    P.seg_desc = pool->seg_desc;
    P.lengths = pool->lengths;
    P.degenerate = pool->degenerate;
    P.block_bitoff = pool->block_bitoff;
    P.block_seg = pool->block_seg;
    P.n_slots = pool->n_slots;
    P.cap_bits = pool->cap_words * 32;
    P.max_segs = sz.max_segs;
    P.seg_stride = sz.seg_stride;
    P.stream_words = sz.stream_words;
    if (pool->dtype == ZX_BF16)
        hipLaunchKernelGGL(k_encode_slots_fused<ZX_BF16>, dim3(nblk), dim3(kEncThreads), 0, stream, P, src, slot_ids, max_len,
                           status, err);
    else
        hipLaunchKernelGGL(k_encode_slots_fused<ZX_FP8_E4M3FN>, dim3(nblk), dim3(kEncThreads), 0, stream, P, src, slot_ids,
                           max_len, status, err);
    return hipGetLastError() == hipSuccess ? ZX_OK : ZX_E_HIP;
}

// ---- K/V append with no allocation ---------------------------------------------
//
// For callers that cannot allocate (code under HIP graph capture, serving loops,
// harnesses that forbid it): the workspace of zx_kv_encode_slots lives in a
// file-scope device array of fixed size instead of coming from the caller.  Each
// device holds its own copy at its own address, found once per device with
// hipGetSymbolAddress; the array's name is only a host-side stand-in and is never
// handed to a kernel.  Every part of the workspace is written in full by the kernel
// that produces it before any kernel reads it, so nothing is cleared between calls.
// Calls on one device share the array: calls that overlap in time on one device race.
constexpr uint32_t kKvNoAllocMaxBlocks = ZX_KV_NOALLOC_MAX_BLOCKS;
constexpr size_t kKvScratchBytes = kv_ws(ZX_BF16, kKvNoAllocMaxBlocks).total;
static_assert(kv_ws(ZX_FP8_E4M3FN, kKvNoAllocMaxBlocks).total <= kKvScratchBytes, "scratch sized for the larger alphabet");
static __device__ __align__(256) uint8_t scratch[kKvScratchBytes];

constexpr int kScratchDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[kScratchDevices];

// Device address of `scratch` on the current device (looked up on the first call per
// device), or null with *st set.
static void *scratch_on_current_device(zx_status *st)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) {
        *st = ZX_E_HIP;
        return nullptr;
    }
    std::lock_guard<std::mutex> guard(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            *st = ZX_E_HIP;
            return nullptr;
        }
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

extern "C" zx_status zx_kv_encode_slots_noalloc(const zx_kv_pool *pool, const void *src, uint32_t nblk,
                                                const uint32_t *slot_ids, uint32_t max_len, uint32_t *status,
                                                uint32_t *err, hipStream_t stream)
{
    if (nblk > kKvNoAllocMaxBlocks) return ZX_E_LIMIT;
    if (nblk == 0) return zx_kv_encode_slots(pool, src, 0, slot_ids, max_len, nullptr, 0, status, err, stream);
    zx_status st = ZX_OK;
    void *ws = scratch_on_current_device(&st);
    if (!ws) return st;
    return zx_kv_encode_slots(pool, src, nblk, slot_ids, max_len, ws, kKvScratchBytes, status, err, stream);
}

extern "C" zx_status zx_kv_slot_container(const zx_kv_pool *pool, uint32_t slot, zx_container *out)
{
    zx_kv_sizes sz;
    if (!kv_pool_ok(pool, &sz) || !out || slot >= pool->n_slots) return ZX_E_INVAL;
    const uint64_t A = sz.alphabet;
    out->dtype = pool->dtype;
    out->per_block = 1;
    out->n = kBlock;
    out->nsegs = sz.max_segs;
    out->total_bits = (uint64_t)pool->cap_words * 32;
    out->stream_words = sz.stream_words;
    out->lengths = pool->lengths + slot * A;
    out->degenerate = pool->degenerate + slot;
    out->signmant = pool->signmant + slot * sz.sm_bytes;
    out->stream = pool->stream + slot * sz.stream_words;
    out->block_bitoff = pool->block_bitoff + 2 * (uint64_t)slot;
    out->block_seg = pool->block_seg + 2 * (uint64_t)slot;
    out->seg_desc = pool->seg_desc + 2 * (uint64_t)slot * sz.seg_stride;
    out->gaps = pool->gaps + (uint64_t)slot * sz.seg_stride * kSegChunks;
    out->dtab = nullptr;
    return ZX_OK;
}
