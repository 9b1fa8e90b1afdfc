// zx_hist.hip -- exponent histogram per 65536-element block.
//
// The exponent distribution is what the Huffman tree is built from (DFloat11
// article, 方法介绍; Intel summary, 方法论).  Exponents of weights and K/V values
// cluster on a few values (ZipFloat page, section 2, Tables 1-2), so lanes of a
// wavefront mostly hold the same handful of values: a single shared histogram would
// serialise its atomics on those few bins.  Each lane therefore owns a private copy
// of the histogram in LDS (shared by the lane of the same index in every wavefront
// of the workgroup), laid out bin-major: lane l's count of value v is word 64 v + l.
// The bank of a lane's counter then depends on the lane alone, so the atomics of
// one instruction never meet in a bank because of the values the lanes hold (a
// lane-major layout with an odd stride spreads one value over the banks, but two
// lanes holding neighbouring values collide).  The 64 copies are summed at the end.
#include "zx_common.h"

namespace zxk {

constexpr int kHistThreads = 1024;

template <int DT>
__global__ __launch_bounds__(kHistThreads) void k_histogram(const void *__restrict__ in, uint64_t n,
                                                            uint32_t *__restrict__ tensor_hist,
                                                            uint32_t *__restrict__ block_hist,
                                                            unsigned long long *__restrict__ hist64)
{
    constexpr uint32_t A = alphabet_of(DT);
    __shared__ uint32_t h[A * kWave];             // lane l's count of value v at 64 v + l
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid % kWave;
    const uint64_t b = blockIdx.x;
    uint32_t *const mine = h + lane;
    const uint64_t lo = b * kBlock;
    const uint32_t nb = (uint32_t)(((lo + kBlock < n) ? lo + kBlock : n) - lo);
    auto exp_of = [](uint32_t word, uint32_t k) -> uint32_t {   // k-th element of a 32-bit word
        if (DT == ZX_BF16) return (word >> (16 * (k & 1) + 7)) & 0xFFu;
        if (DT == ZX_E8M0) return (word >> (8 * (k & 3))) & 0xFFu;
        return (word >> (8 * (k & 3) + 3)) & 0xFu;
    };
    if (nb == kBlock) {
        // a full block: every 16-byte load of the thread in flight at once (straight-line
        // code, so that no wait falls between them), issued before the copies are
        // cleared so that the clearing and its barrier overlap them
        constexpr uint32_t kVecs = kBlock * (DT == ZX_BF16 ? 2 : 1) / 16 / kHistThreads;   // 8 or 4
        constexpr uint32_t EPW = DT == ZX_BF16 ? 2 : 4;                                    // elements per word
        const uint4 *src = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint8_t *>(in) + lo * (DT == ZX_BF16 ? 2 : 1));
        // (the scheduling barriers keep the loads in this order and everything that
        // reads them below the workgroup barrier: each vector is then counted as soon as
        // it arrives, and the barrier waits for none of them)
        uint4 q[kVecs];
#pragma unroll
        for (uint32_t u = 0; u < kVecs; ++u) {
            q[u] = src[u * kHistThreads + tid];
            __builtin_amdgcn_sched_barrier(0);
        }
        for (uint32_t i = tid; i < A * kWave; i += kHistThreads) h[i] = 0;
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (uint32_t u = 0; u < kVecs; ++u) {
            const uint32_t wv[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
            for (uint32_t k = 0; k < 4 * EPW; ++k) atomicAdd(&mine[exp_of(wv[k / EPW], k) * kWave], 1u);
        }
    } else {
        // the last, partial block of a tensor: element by element
        for (uint32_t i = tid; i < A * kWave; i += kHistThreads) h[i] = 0;
        __syncthreads();
        for (uint32_t i = tid; i < nb; i += kHistThreads) {
            const uint32_t word = DT == ZX_BF16 ? (uint32_t)reinterpret_cast<const uint16_t *>(in)[lo + i]
                                                : (uint32_t)reinterpret_cast<const uint8_t *>(in)[lo + i];
            atomicAdd(&mine[exp_of(word, 0) * kWave], 1u);
        }
    }
    __syncthreads();
    // sum the 64 copies: G threads per value, each adding C of its copies (rotated by
    // the value, so that a wavefront's reads fall in distinct banks), then the G
    // partial sums of a value are added across neighbouring lanes
    constexpr uint32_t G = kHistThreads / A;                // 4 (alphabet 256) or 64 (alphabet 16)
    constexpr uint32_t C = kWave / G;                       // 16 or 1
    static_assert(G * A == kHistThreads && C * G == kWave, "histogram sum shape");
    const uint32_t v = tid / G;
    const uint32_t g = tid % G;
    uint32_t c = 0;
#pragma unroll
    for (uint32_t j = 0; j < C; ++j) c += h[v * kWave + g * C + ((j + v) & (C - 1))];
#pragma unroll
    for (uint32_t o = 1; o < G; o <<= 1) c += __shfl_xor(c, o);
    if (g == 0) {
        if (block_hist) block_hist[b * A + v] = c;
        if (tensor_hist && c) atomicAdd(&tensor_hist[v], c);
        if (hist64 && c) atomicAdd(&hist64[v], (unsigned long long)c);
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
