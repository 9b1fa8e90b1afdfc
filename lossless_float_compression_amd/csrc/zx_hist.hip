// zx_hist.hip -- exponent histogram per 65536-element block.
//
// The exponent distribution is what the Huffman tree is built from (DFloat11
// article, 方法介绍; Intel summary, 方法论).  Exponents of weights and K/V values
// cluster on a few values (ZipFloat page, section 2, Tables 1-2), so lanes of a
// wavefront mostly hold the same handful of values: a single shared histogram would
// serialise its atomics on those few bins.  Each lane therefore owns a private copy
// of the histogram in LDS (shared by the lane of the same index in every wavefront
// of the workgroup), laid out with a stride of A + 1 words so that lane l's bin v
// sits in bank (l + v) mod 64: the 64 LDS atomics of one instruction fall in 64
// distinct banks whatever the values.  The 64 copies are summed at the end.
#include "zx_common.h"

namespace zxk {

constexpr int kHistThreads = 1024;
constexpr uint32_t kHistUnroll = 4;   // 16-byte loads in flight per lane

template <int DT>
__global__ __launch_bounds__(kHistThreads) void k_histogram(const void *__restrict__ in, uint64_t n,
                                                            uint32_t *__restrict__ tensor_hist,
                                                            uint32_t *__restrict__ block_hist,
                                                            unsigned long long *__restrict__ hist64)
{
    constexpr uint32_t A = alphabet_of(DT);
    constexpr uint32_t S = A + 1;                 // copy stride in words
    __shared__ uint32_t h[kWave * S];
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid % kWave;
    const uint64_t b = blockIdx.x;
    for (uint32_t i = tid; i < kWave * S; i += kHistThreads) h[i] = 0;
    __syncthreads();
    uint32_t *const mine = h + lane * S;
    const uint64_t lo = b * kBlock;
    const uint64_t hi = (lo + kBlock < n) ? lo + kBlock : n;
    const uint32_t nb = (uint32_t)(hi - lo);
    // 16 bytes per lane per step: 8 BF16 or 16 FP8 elements
    constexpr uint32_t EPV = DT == ZX_BF16 ? 8 : 16;
    const uint32_t nvec = (nb + EPV - 1) / EPV;
    const uint4 *src = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint8_t *>(in) + lo * (DT == ZX_BF16 ? 2 : 1));
    constexpr uint32_t kStep = kHistThreads * kHistUnroll;
    for (uint32_t base = 0; base < nvec; base += kStep) {
        uint32_t words[kHistUnroll][4];
        uint32_t have[kHistUnroll];
        // issue every load of this step before counting
#pragma unroll
        for (uint32_t u = 0; u < kHistUnroll; ++u) {
            const uint32_t v = base + u * kHistThreads + tid;
            words[u][0] = words[u][1] = words[u][2] = words[u][3] = 0;
            have[u] = 0;
            if (v < nvec) {
                const uint32_t first = v * EPV;
                have[u] = (nb - first < EPV) ? nb - first : EPV;
                if (have[u] == EPV) {
                    const uint4 q = src[v];
                    words[u][0] = q.x; words[u][1] = q.y; words[u][2] = q.z; words[u][3] = q.w;
                } else {
                    const uint8_t *bytes = reinterpret_cast<const uint8_t *>(src) + (uint64_t)first * (DT == ZX_BF16 ? 2 : 1);
                    const uint32_t nbytes = have[u] * (DT == ZX_BF16 ? 2 : 1);
                    for (uint32_t k = 0; k < nbytes; ++k) words[u][k >> 2] |= (uint32_t)bytes[k] << (8 * (k & 3));
                }
            }
        }
#pragma unroll
        for (uint32_t u = 0; u < kHistUnroll; ++u) {
            if (have[u] == EPV) {
#pragma unroll
                for (uint32_t k = 0; k < EPV; ++k) {
                    uint32_t e;
                    if (DT == ZX_BF16) e = (words[u][k >> 1] >> (16 * (k & 1) + 7)) & 0xFFu;
                    else if (DT == ZX_E8M0) e = (words[u][k >> 2] >> (8 * (k & 3))) & 0xFFu;
                    else e = (words[u][k >> 2] >> (8 * (k & 3) + 3)) & 0xFu;
                    atomicAdd(&mine[e], 1u);
                }
            } else {
                for (uint32_t k = 0; k < have[u]; ++k) {
                    uint32_t e;
                    if (DT == ZX_BF16) e = (words[u][k >> 1] >> (16 * (k & 1) + 7)) & 0xFFu;
                    else if (DT == ZX_E8M0) e = (words[u][k >> 2] >> (8 * (k & 3))) & 0xFFu;
                    else e = (words[u][k >> 2] >> (8 * (k & 3) + 3)) & 0xFu;
                    atomicAdd(&mine[e], 1u);
                }
            }
        }
    }
    __syncthreads();
    // sum the 64 copies: thread t adds copies t/A, t/A + 1024/A, ... of bin t % A
    constexpr uint32_t kGroups = kHistThreads / A;          // 4 (BF16) or 64 (FP8)
    const uint32_t bin = tid % A;
    const uint32_t grp = tid / A;
    uint32_t c = 0;
    for (uint32_t cp = grp; cp < kWave; cp += kGroups) c += h[cp * S + bin];
    __syncthreads();
    h[grp * S + bin] = c;
    __syncthreads();
    if (tid < A) {
        uint32_t t = 0;
        for (uint32_t g = 0; g < kGroups; ++g) t += h[g * S + tid];
        if (block_hist) block_hist[b * A + tid] = t;
        if (tensor_hist && t) atomicAdd(&tensor_hist[tid], t);
        if (hist64 && t) atomicAdd(&hist64[tid], (unsigned long long)t);
    }
}

__global__ void k_zero_u32(uint32_t *p, uint64_t count)
{
    for (uint64_t i = blockIdx.x * (uint64_t)blockDim.x + threadIdx.x; i < count; i += (uint64_t)gridDim.x * blockDim.x) p[i] = 0;
}

}  // namespace zxk

using namespace zxk;

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

extern "C" zx_status zx_histogram(zx_dtype dtype, const void *in, uint64_t n, uint32_t *tensor_hist,
                                  uint32_t *block_hist, hipStream_t stream)
{
    if (dtype != ZX_BF16 && dtype != ZX_FP8_E4M3FN && dtype != ZX_E8M0) return ZX_E_UNSUPPORTED;
    if (!tensor_hist && !block_hist) return ZX_E_INVAL;
    if (n && !in) return ZX_E_INVAL;
    if (!aligned16(in) || !aligned16(tensor_hist) || !aligned16(block_hist)) return ZX_E_INVAL;
    if (tensor_hist && n >= (1ull << 32)) return ZX_E_INVAL;
    const uint32_t A = alphabet_of(dtype);
    const uint64_t nblocks = (n + kBlock - 1) / kBlock;
    if (nblocks > 0x7FFFFFFFull) return ZX_E_INVAL;
    if (tensor_hist) {
        hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(256), 0, stream, tensor_hist, (uint64_t)A);
        if (hipGetLastError() != hipSuccess) return ZX_E_HIP;
    }
    if (nblocks == 0) return ZX_OK;
    if (dtype == ZX_BF16)
        hipLaunchKernelGGL(k_histogram<ZX_BF16>, dim3((uint32_t)nblocks), dim3(kHistThreads), 0, stream, in, n, tensor_hist, block_hist,
                           nullptr);
    else if (dtype == ZX_E8M0)
        hipLaunchKernelGGL(k_histogram<ZX_E8M0>, dim3((uint32_t)nblocks), dim3(kHistThreads), 0, stream, in, n, tensor_hist, block_hist,
                           nullptr);
    else
        hipLaunchKernelGGL(k_histogram<ZX_FP8_E4M3FN>, dim3((uint32_t)nblocks), dim3(kHistThreads), 0, stream, in, n, tensor_hist,
                           block_hist, nullptr);
    return hipGetLastError() == hipSuccess ? ZX_OK : ZX_E_HIP;
}

extern "C" zx_status zx_histogram_accumulate(zx_dtype dtype, const void *in, uint64_t n, uint64_t *hist64, hipStream_t stream)
{
    if (dtype != ZX_BF16 && dtype != ZX_FP8_E4M3FN && dtype != ZX_E8M0) return ZX_E_UNSUPPORTED;
    if (!hist64 || (n && !in) || !aligned16(in) || ((uintptr_t)hist64 & 7u)) return ZX_E_INVAL;
    const uint64_t nblocks = (n + kBlock - 1) / kBlock;
    if (nblocks > 0x7FFFFFFFull) return ZX_E_INVAL;
    if (nblocks == 0) return ZX_OK;
    unsigned long long *h = reinterpret_cast<unsigned long long *>(hist64);
    if (dtype == ZX_BF16)
        hipLaunchKernelGGL(k_histogram<ZX_BF16>, dim3((uint32_t)nblocks), dim3(kHistThreads), 0, stream, in, n, nullptr, nullptr, h);
    else if (dtype == ZX_E8M0)
        hipLaunchKernelGGL(k_histogram<ZX_E8M0>, dim3((uint32_t)nblocks), dim3(kHistThreads), 0, stream, in, n, nullptr, nullptr, h);
    else
        hipLaunchKernelGGL(k_histogram<ZX_FP8_E4M3FN>, dim3((uint32_t)nblocks), dim3(kHistThreads), 0, stream, in, n, nullptr, nullptr, h);
    return hipGetLastError() == hipSuccess ? ZX_OK : ZX_E_HIP;
}
