// zx_codebook.hip -- Huffman code lengths on the device, one wavefront per codebook
// (the construction is in zx_codebook.h).  Per-block scope launches one workgroup per
// block, so thousands of codebooks are built at once.
#include "zx_codebook.h"

namespace zxk {

template <int DT, typename H>
__global__ __launch_bounds__(64) void k_codebook(const H *__restrict__ hist, uint32_t max_len,
                                                 uint8_t *__restrict__ lengths, uint16_t *__restrict__ degenerate)
{
    constexpr uint32_t A = alphabet_of(DT);
    __shared__ CodebookLds<H> L;
    const uint64_t cb = blockIdx.x;
    for (uint32_t i = threadIdx.x; i < A; i += kWave) L.cnt[i] = hist[cb * A + i];
    wave_sync();
    codebook_wave<A, H>(L, max_len, lengths + cb * A, degenerate + cb);
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
