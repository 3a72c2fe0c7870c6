// kda_probe.hip -- a plain streaming copy, used to calibrate memory-traffic
// counters (bytes per dispatch of a kernel of known size) and to measure the
// practical HBM copy ceiling next to the KDA kernels.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

__global__ __launch_bounds__(256) void kda_copy_probe_kernel(float4 *__restrict__ dst,
                                                             const float4 *__restrict__ src,
                                                             size_t n4) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
        dst[i] = src[i];
}

__global__ void kda_copy_tail_kernel(float *__restrict__ dst, const float *__restrict__ src,
                                     size_t start, size_t n) {
    const size_t i = start + threadIdx.x;
    if (i < n) dst[i] = src[i];
}

kda_status launch_copy_probe(float *dst, const float *src, size_t n, hipStream_t stream) {
    const size_t n4 = n / 4;
    if (n4) {
        // enough workgroups to cover every CU several times over, capped so
        // each lane still streams a few float4s
        size_t blocks = (n4 + 255) / 256;
        if (blocks > 256 * 32) blocks = 256 * 32;
        hipLaunchKernelGGL(kda_copy_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                           reinterpret_cast<float4 *>(dst), reinterpret_cast<const float4 *>(src), n4);
    }
    if (n % 4)
        hipLaunchKernelGGL(kda_copy_tail_kernel, dim3(1), dim3(4), 0, stream, dst, src, n4 * 4, n);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // namespace kda
