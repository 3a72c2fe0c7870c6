// kda_probe.hip -- a streaming copy that bounds what the memory system
// delivers to a kernel that reads and writes equal amounts (as the decode
// does), used to calibrate memory-traffic counters (bytes per dispatch of a
// kernel of known size) and as the practical copy ceiling next to the KDA
// kernels.
//
// The grid is one round (every workgroup resident at once), each workgroup
// copies one contiguous range, and every lane keeps kProbeUnroll 16-byte
// loads in flight before it stores them.  Loads and stores are raw buffer
// operations with the non-temporal policy (the stores also device scope), so
// a copy larger than the caches streams through them instead of evicting
// and re-fetching lines.
#include "kda_device.h"
#include "kda_internal.h"

#ifndef KDA_PROBE_UNROLL
#define KDA_PROBE_UNROLL 8
#endif
#ifndef KDA_PROBE_WG_PER_CU
#define KDA_PROBE_WG_PER_CU 4
#endif

namespace kda {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = KDA_PROBE_UNROLL;
constexpr int kProbeWorkgroups = 256 * KDA_PROBE_WG_PER_CU;   // 256 CUs
constexpr int kProbePolicyNT = 2, kProbePolicySC1 = 16;
constexpr int kProbeBufferWord3 = 0x00020000;   // raw 32-bit buffer resource

// Workgroup w copies float4 elements [w * per, min((w + 1) * per, n4)).
// A buffer resource per workgroup keeps every byte offset below 2^32
// (per * 16 bytes, checked by the launcher).
// dst may equal src (an in-place read and rewrite: each lane stores only the
// elements it has loaded).
__global__ __launch_bounds__(kProbeThreads) void kda_copy_probe_kernel(float4 *dst, const float4 *src,
                                                                       size_t n4, size_t per) {
    typedef float v4 __attribute__((ext_vector_type(4)));
    const size_t a = (size_t)blockIdx.x * per;
    if (a >= n4) return;
    const int n = (int)(n4 - a < per ? n4 - a : per);   // elements of this workgroup
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float4 *>(src + a), 0, n * 16, kProbeBufferWord3);
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(dst + a, 0, n * 16, kProbeBufferWord3);
    constexpr int kStep = kProbeThreads * kProbeUnroll;
    for (int base = 0; base < n; base += kStep) {
        v4 x[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const int i = base + u * kProbeThreads + (int)threadIdx.x;
            if (i < n) x[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, i * 16, 0, kProbePolicyNT);
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const int i = base + u * kProbeThreads + (int)threadIdx.x;
            if (i < n) __builtin_amdgcn_raw_buffer_store_b128(x[u], rd, i * 16, 0, kProbePolicyNT | kProbePolicySC1);
        }
    }
}

__global__ void kda_copy_tail_kernel(float *dst, const float *src, size_t start, size_t n) {
    const size_t i = start + threadIdx.x;
    if (i < n) dst[i] = src[i];
}

kda_status launch_copy_probe(float *dst, const float *src, size_t n, hipStream_t stream) {
    const size_t n4 = n / 4;
    if (n4) {
        const size_t per = (n4 + kProbeWorkgroups - 1) / kProbeWorkgroups;
        if (per * 16 >= ((size_t)1 << 31)) return KDA_ERR_SHAPE;   // int byte offsets per workgroup
        const size_t blocks = (n4 + per - 1) / per;
        hipLaunchKernelGGL(kda_copy_probe_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, stream,
                           reinterpret_cast<float4 *>(dst), reinterpret_cast<const float4 *>(src), n4, per);
    }
    if (n % 4)
        hipLaunchKernelGGL(kda_copy_tail_kernel, dim3(1), dim3(4), 0, stream, dst, src, n4 * 4, n);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // namespace kda
