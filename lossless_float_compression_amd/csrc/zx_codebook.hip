// zx_codebook.hip -- Huffman code lengths on the device, one wavefront per codebook.
//
// Huffman tree from the exponent distribution (DFloat11 article, 方法介绍; Intel
// summary, 方法论).  The pages fix neither tie-breaks nor a length limit; container
// v1 fixes them: two-queue merging where the leaf queue (ordered by count, then
// symbol) wins weight ties, and, when the tree is deeper than max_len, the optimal
// length-limited code by package-merge (coin-collector form), leaves before
// packages on weight ties.
//
// The wavefront sorts the present symbols in parallel.  The Huffman merge is a chain
// of dependent steps: with up to 64 present symbols it runs in registers (lane i
// holds leaf i and internal node i, queue heads are read across lanes) and the
// depths come from pointer jumping; larger alphabets and package-merge run on one
// lane over LDS.  Per-block scope launches one
// workgroup per block, so thousands of codebooks are built at once.
#include "zx_common.h"

namespace zxk {

constexpr uint32_t kPmWords = 16;  // 512 bits: one flag per merged-list item

// 64-bit value held by lane i (i wavefront-uniform).
__device__ __forceinline__ uint64_t read_u64(uint64_t v, uint32_t i)
{
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, i);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), i);
    return ((uint64_t)hi << 32) | lo;
}

// H: the count type of the histograms (u32 per tensor or block, u64 for counts summed
// over many tensors; the packed sort key needs counts below 2^48).
template <int DT, typename H>
__global__ __launch_bounds__(64) void k_codebook(const H *__restrict__ hist, uint32_t max_len,
                                                 uint8_t *__restrict__ lengths, uint16_t *__restrict__ degenerate)
{
    constexpr uint32_t A = alphabet_of(DT);
    __shared__ H cnt[256];
    __shared__ uint16_t present[256];
    __shared__ uint16_t leaf_sym[256];
    __shared__ uint64_t w[512];          // leaves 0..k-1 (sorted), merged nodes k..2k-2
    __shared__ uint64_t pm_a[512];
    __shared__ uint64_t pm_b[512];
    __shared__ uint16_t parent[512];
    __shared__ uint8_t depth[512];
    __shared__ uint8_t out_len[256];
    __shared__ uint32_t isleaf[kMaxLen + 1][kPmWords];
    __shared__ uint32_t s_maxd;

    const uint32_t lane = threadIdx.x;
    const uint64_t cb = blockIdx.x;
    for (uint32_t i = lane; i < A; i += kWave) {
        cnt[i] = hist[cb * A + i];
        out_len[i] = 0;
    }
    __syncthreads();
    // present symbols in symbol order
    uint32_t base = 0;
    for (uint32_t q = 0; q < (A + kWave - 1) / kWave; ++q) {
        const uint32_t s = q * kWave + lane;
        const bool p = s < A && cnt[s] != 0;
        const uint64_t m = __ballot(p);
        if (p) present[base + (uint32_t)__popcll(m & lanemask_lt())] = (uint16_t)s;
        base += (uint32_t)__popcll(m);
    }
    const uint32_t k = base;
    __syncthreads();
    if (k < 2) {
        for (uint32_t i = lane; i < A; i += kWave) lengths[cb * A + i] = 0;
        if (lane == 0) degenerate[cb] = (k == 1) ? present[0] : (uint16_t)ZX_NO_DEGENERATE;
        return;
    }
    // leaves ordered by (count, symbol): each present symbol's rank, comparing packed
    // keys count << 16 | symbol (distinct, so the ranks are a permutation)
    uint64_t *key = pm_a;    // free until package-merge
    for (uint32_t i = lane; i < k; i += kWave) {
        const uint32_t s = present[i];
        key[i] = ((uint64_t)cnt[s] << 16) | s;
    }
    __syncthreads();
    for (uint32_t i = lane; i < k; i += kWave) {
        const uint64_t mine = key[i];
        uint32_t r = 0;
        for (uint32_t j = 0; j < k; ++j) r += key[j] < mine ? 1u : 0u;
        leaf_sym[r] = (uint16_t)(mine & 0xFFFFu);
        w[r] = mine >> 16;
    }
    __syncthreads();
    if (k <= kWave) {
        // ---- register path (up to 64 leaves, e.g. every FP8 code and most BF16 ones):
        // lane i holds leaf i's weight and, once it is made, internal node i's; the
        // queue heads are read with readlane, so a merge step touches no memory
        const uint64_t lw = lane < k ? w[lane] : ~0ull;
        uint64_t nw = ~0ull;               // weight of internal node `lane`
        uint32_t lpar = 0, npar = 0;       // parent (internal node index) of leaf / node `lane`
        uint32_t q1 = 0, q2 = 0, made = 0;
        for (uint32_t step = 0; step + 1 < k; ++step) {
            uint64_t val[2];
            for (int t = 0; t < 2; ++t) {
                const uint64_t a = q1 < k ? read_u64(lw, q1) : ~0ull;
                const uint64_t b = q2 < made ? read_u64(nw, q2) : ~0ull;
                // the leaf queue wins weight ties
                const bool take_leaf = q1 < k && (q2 >= made || a <= b);
                if (take_leaf) {
                    if (lane == q1) lpar = made;
                    val[t] = a;
                    ++q1;
                } else {
                    if (lane == q2) npar = made;
                    val[t] = b;
                    ++q2;
                }
            }
            if (lane == made) nw = val[0] + val[1];
            ++made;
        }
        // depths by pointer jumping: each internal node's distance to the root (the
        // last node made, its own parent at distance 0), then one more hop for leaves
        const uint32_t root = made - 1;
        uint32_t dn = lane < root ? 1u : 0u;
        uint32_t pn = lane < root ? npar : root;
        for (int it = 0; it < 6; ++it) {
            const uint32_t dpn = (uint32_t)__shfl((int)dn, (int)pn, kWave);
            const uint32_t ppn = (uint32_t)__shfl((int)pn, (int)pn, kWave);
            dn += dpn;
            pn = ppn;
        }
        const uint32_t dleaf = (uint32_t)__shfl((int)dn, (int)lpar, kWave) + 1u;
        uint32_t maxd = lane < k ? dleaf : 0u;
        for (int o = 32; o >= 1; o >>= 1) {
            const uint32_t y = (uint32_t)__shfl_xor((int)maxd, o, kWave);
            maxd = y > maxd ? y : maxd;
        }
        if (lane < k) depth[lane] = (uint8_t)dleaf;
        if (lane == 0) s_maxd = maxd;
    } else if (lane == 0) {
        // two queues: leaves [q1, k), merged nodes [q2, made)
        uint32_t q1 = 0, q2 = k, made = k;
        for (uint32_t step = 0; step + 1 < k; ++step) {
            uint32_t id[2];
            for (int t = 0; t < 2; ++t) {
                bool take_leaf;
                if (q1 >= k)
                    take_leaf = false;
                else if (q2 >= made)
                    take_leaf = true;
                else
                    take_leaf = w[q1] <= w[q2];
                id[t] = take_leaf ? q1++ : q2++;
            }
            w[made] = w[id[0]] + w[id[1]];
            parent[id[0]] = (uint16_t)made;
            parent[id[1]] = (uint16_t)made;
            ++made;
        }
        const uint32_t root = made - 1;
        depth[root] = 0;
        uint32_t maxd = 0;
        for (int id = (int)root - 1; id >= 0; --id) {
            const uint32_t d = depth[parent[id]] + 1u;
            depth[id] = (uint8_t)(d > 255 ? 255 : d);
            if (id < (int)k && d > maxd) maxd = d;
        }
        s_maxd = maxd;
    }
    __syncthreads();
    if (s_maxd <= max_len) {
        for (uint32_t i = lane; i < k; i += kWave) out_len[leaf_sym[i]] = depth[i];
    } else if (lane == 0) {
        // package-merge at limit L = max_len over the sorted leaf weights w[0..k)
        const int L = (int)max_len;
        // merged lists: level L is the leaves; level lv merges the leaves with the
        // packages made by pairing neighbours of level lv+1 (odd last item dropped)
        uint64_t *prev = pm_a;   // weights of the list one level deeper
        uint64_t *cur = pm_b;
        for (uint32_t i = 0; i < k; ++i) prev[i] = w[i];
        for (uint32_t i = 0; i < kPmWords; ++i) isleaf[L][i] = 0;
        for (uint32_t i = 0; i < k; ++i) isleaf[L][i >> 5] |= 1u << (i & 31);
        uint32_t nprev = k;
        for (int lv = L - 1; lv >= 1; --lv) {
            for (uint32_t i = 0; i < kPmWords; ++i) isleaf[lv][i] = 0;
            const uint32_t np = nprev / 2;
            uint32_t a = 0, b = 0, o = 0;
            while (a < k || b < np) {
                bool take_leaf;
                uint64_t pw = 0;
                if (b < np) pw = prev[2 * b] + prev[2 * b + 1];
                if (a >= k)
                    take_leaf = false;
                else if (b >= np)
                    take_leaf = true;
                else
                    take_leaf = w[a] <= pw;
                if (take_leaf) {
                    cur[o] = w[a++];
                    isleaf[lv][o >> 5] |= 1u << (o & 31);
                } else {
                    cur[o] = pw;
                    ++b;
                }
                ++o;
            }
            uint64_t *t = prev;
            prev = cur;
            cur = t;
            nprev = o;
        }
        // keep the 2(k-1) lightest items of level 1; kept packages expand into the
        // first items of the level below.  Leaves sit in a merged list in their
        // sorted order, so the kept leaves of a level are the lightest ones, and
        // each of them gains one bit of length.
        for (uint32_t i = 0; i < k; ++i) depth[i] = 0;
        uint32_t keep = 2 * (k - 1);
        for (int lv = 1; lv <= L && keep > 0; ++lv) {
            uint32_t nleaf = 0;
            for (uint32_t i = 0; i < keep; ++i) nleaf += (isleaf[lv][i >> 5] >> (i & 31)) & 1u;
            for (uint32_t i = 0; i < nleaf; ++i) depth[i] = (uint8_t)(depth[i] + 1);
            keep = 2 * (keep - nleaf);
        }
        for (uint32_t i = 0; i < k; ++i) out_len[leaf_sym[i]] = depth[i];
    }
    __syncthreads();
    for (uint32_t i = lane; i < A; i += kWave) lengths[cb * A + i] = out_len[i];
    if (lane == 0) degenerate[cb] = (uint16_t)ZX_NO_DEGENERATE;
}

}  // namespace zxk

using namespace zxk;

template <typename H>
static zx_status build_codebook(zx_dtype dtype, const H *hist, uint32_t n_codebooks, uint32_t max_len, uint8_t *lengths,
                                uint16_t *degenerate, hipStream_t stream)
{
    if (dtype != ZX_BF16 && dtype != ZX_FP8_E4M3FN && dtype != ZX_E8M0) return ZX_E_UNSUPPORTED;
    const uint32_t minlen = alphabet_of(dtype) == 256 ? 8 : 4;
    if (max_len < minlen || max_len > kMaxLen) return ZX_E_CODEBOOK;
    if (n_codebooks == 0) return ZX_OK;
    if (!hist || !lengths || !degenerate) return ZX_E_INVAL;
    if (n_codebooks > 0x7FFFFFFFu) return ZX_E_INVAL;
    if (alphabet_of(dtype) == 256)   // BF16 and E8M0: the kernel depends on the alphabet only
        hipLaunchKernelGGL((k_codebook<ZX_BF16, H>), dim3(n_codebooks), dim3(64), 0, stream, hist, max_len, lengths, degenerate);
    else
        hipLaunchKernelGGL((k_codebook<ZX_FP8_E4M3FN, H>), dim3(n_codebooks), dim3(64), 0, stream, hist, max_len, lengths,
                           degenerate);
    return hipGetLastError() == hipSuccess ? ZX_OK : ZX_E_HIP;
}

extern "C" zx_status zx_build_codebook(zx_dtype dtype, const uint32_t *hist, uint32_t n_codebooks,
                                       uint32_t max_len, uint8_t *lengths, uint16_t *degenerate,
                                       hipStream_t stream)
{
    return build_codebook<uint32_t>(dtype, hist, n_codebooks, max_len, lengths, degenerate, stream);
}

extern "C" zx_status zx_build_codebook_u64(zx_dtype dtype, const uint64_t *hist, uint32_t n_codebooks,
                                           uint32_t max_len, uint8_t *lengths, uint16_t *degenerate,
                                           hipStream_t stream)
{
    return build_codebook<uint64_t>(dtype, hist, n_codebooks, max_len, lengths, degenerate, stream);
}
