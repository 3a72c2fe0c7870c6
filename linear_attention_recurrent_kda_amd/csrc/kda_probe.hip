// kda_probe.hip -- a streaming copy that bounds what the memory system
// delivers to a kernel that reads and writes equal amounts (as the decode
// does), used to calibrate memory-traffic counters (bytes per dispatch of a
// kernel of known size) and as a copy ceiling next to the KDA kernels.
//
// It moves memory the way the decode moves its state tiles: one 64 KiB tile
// per workgroup (16 loads of 16 bytes per lane, all in flight, then 16
// stores), at most three workgroups per CU, and the tiles of one 2 MiB
// granule on consecutive workgroups while the granules themselves are
// visited in a scrambled order (a linear sweep measured 3-6% slower on
// MI355X: the concurrent tiles then crowd fewer memory channels).  Loads and
// stores are raw buffer operations with the non-temporal policy (the stores
// also device scope), so a copy larger than the caches streams through them.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int kProbeThreads = 256;
constexpr int kProbeTileF4 = 4096;                  // 64 KiB per workgroup
constexpr int kProbeGranuleTiles = 32;              // 2 MiB granules
constexpr unsigned long long kProbeScramble = 2654435761ull;   // prime: a bijection mod any smaller count
constexpr int kProbePolicyNT = 2, kProbePolicySC1 = 16;
constexpr int kProbeBufferWord3 = 0x00020000;       // raw 32-bit buffer resource

// Workgroup w copies tile t(w) of n4 float4 elements (the last tile may be
// partial).  t(w) keeps w's position inside its granule and scrambles the
// granule: granule (w / 32 * P) mod n_granules for the whole granules, the
// tiles of a last partial granule in order.  dst may equal src (an in-place
// read and rewrite: each lane stores only the elements it has loaded).
__global__ __launch_bounds__(kProbeThreads) __attribute__((amdgpu_waves_per_eu(1, 3)))
void kda_copy_probe_kernel(float4 *dst, const float4 *src, size_t n4) {
    typedef float v4 __attribute__((ext_vector_type(4)));
    const size_t n_tiles = (n4 + kProbeTileF4 - 1) / kProbeTileF4;
    const size_t full_granules = n_tiles / kProbeGranuleTiles;
    const size_t w = blockIdx.x;
    size_t tile = w;
    if (w / kProbeGranuleTiles < full_granules)
        tile = ((w / kProbeGranuleTiles) * kProbeScramble % full_granules) * kProbeGranuleTiles + w % kProbeGranuleTiles;
    const size_t a = tile * kProbeTileF4;
    const int n = (int)(n4 - a < (size_t)kProbeTileF4 ? n4 - a : kProbeTileF4);   // elements of this tile
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float4 *>(src + a), 0, n * 16, kProbeBufferWord3);
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(dst + a, 0, n * 16, kProbeBufferWord3);
    v4 x[kProbeTileF4 / kProbeThreads];
#pragma unroll
    for (int u = 0; u < kProbeTileF4 / kProbeThreads; ++u) {
        const int i = u * kProbeThreads + (int)threadIdx.x;
        if (i < n) x[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, i * 16, 0, kProbePolicyNT);
    }
#pragma unroll
    for (int u = 0; u < kProbeTileF4 / kProbeThreads; ++u) {
        const int i = u * kProbeThreads + (int)threadIdx.x;
        if (i < n) __builtin_amdgcn_raw_buffer_store_b128(x[u], rd, i * 16, 0, kProbePolicyNT | kProbePolicySC1);
    }
}

__global__ void kda_copy_tail_kernel(float *dst, const float *src, size_t start, size_t n) {
    const size_t i = start + threadIdx.x;
    if (i < n) dst[i] = src[i];
}

kda_status launch_copy_probe(float *dst, const float *src, size_t n, hipStream_t stream) {
    const size_t n4 = n / 4;
    if (n4) {
        const size_t tiles = (n4 + kProbeTileF4 - 1) / kProbeTileF4;
        if (tiles > 0x7fffffffu) return KDA_ERR_SHAPE;
        hipLaunchKernelGGL(kda_copy_probe_kernel, dim3((unsigned)tiles), dim3(kProbeThreads), 0, stream,
                           reinterpret_cast<float4 *>(dst), reinterpret_cast<const float4 *>(src), n4);
    }
    if (n % 4)
        hipLaunchKernelGGL(kda_copy_tail_kernel, dim3(1), dim3(4), 0, stream, dst, src, n4 * 4, n);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // namespace kda
