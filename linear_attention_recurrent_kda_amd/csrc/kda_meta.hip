// kda_meta.hip -- per-step batch metadata built on the device in one launch.
//
// "vLLM Kimi K3 support", section "Fused kernels and metadata optimisation"
// (metadata builder bullet): the tables the KDA kernels read each step are
// built by one fused kernel rather than a chain of small tensor operations
// (the page's figure is 870 -> 34 us at batch 1 on its hardware).  Here the
// tables are the ones this library's calls take: from the scheduler's
// per-request token counts and state slots, the packed token offsets
// (cu_seqlens), the slot table (slot_idx, -1 for rows with nothing to do),
// the 64-token chunk offsets of the chunked prefill and the batch counts.
//
// One workgroup of 1024 lanes walks the requests 1024 at a time: per pass a
// wave-level inclusive scan (DPP row shifts via __shfl_up), the 16 wave
// totals scanned by one wave through LDS, and a carry from pass to pass.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int kMetaThreads = 1024;
constexpr int kMetaWaves = kMetaThreads / kWave;
constexpr int kMetaChunk = 64;   // the chunk of kda_chunk_prefill

__device__ __forceinline__ int wave_scan_incl(int v, int lane) {
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
        const int u = __shfl_up(v, m, kWave);
        if (lane >= m) v += u;
    }
    return v;
}

// Inclusive scan of v over the workgroup; every lane also gets the total.
__device__ __forceinline__ int block_scan_incl(int v, int lane, int wave, int (*wtot)[kMetaWaves], int which,
                                               int &total) {
    int x = wave_scan_incl(v, lane);
    if (lane == kWave - 1) wtot[which][wave] = x;
    __syncthreads();
    if (wave == 0) {
        const int w = lane < kMetaWaves ? wtot[which][lane] : 0;
        const int s = wave_scan_incl(w, lane);
        if (lane < kMetaWaves) wtot[which][lane] = s;   // inclusive wave prefix
    }
    __syncthreads();
    if (wave > 0) x += wtot[which][wave - 1];
    total = wtot[which][kMetaWaves - 1];
    return x;
}

__global__ __launch_bounds__(kMetaThreads) void kda_build_metadata_kernel(MetaParams p) {
    __shared__ int wtot[4][kMetaWaves];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    int tok_carry = 0, ch_carry = 0, ones = 0, pres = 0;
    bool err = false;
    if (tid == 0) {
        p.cu_seqlens[0] = 0;
        p.chunk_start[0] = 0;
    }
    for (int base = 0; base < p.n_req; base += kMetaThreads) {
        const int r = base + tid;
        int t = 0, ch = 0, one = 0, pre = 0;
        if (r < p.n_req) {
            t = p.num_tokens[r];
            const int s = p.req_slot[r];
            if (t < 0) {
                err = true;
                t = 0;
            }
            const bool valid = s >= 0 && s < p.n_slots;
            if (!valid && s != -1) err = true;
            const bool has = t > 0 && valid;
            p.slot_idx[r] = has ? s : -1;
            one = has && t == 1;
            pre = has && t >= 2;
            ch = pre ? (t + kMetaChunk - 1) / kMetaChunk : 0;
        }
        int tok_tot, ch_tot, one_tot, pre_tot;
        const int tok_incl = block_scan_incl(t, lane, wave, wtot, 0, tok_tot);
        const int ch_incl = block_scan_incl(ch, lane, wave, wtot, 1, ch_tot);
        block_scan_incl(one, lane, wave, wtot, 2, one_tot);
        block_scan_incl(pre, lane, wave, wtot, 3, pre_tot);
        if (r < p.n_req) {
            p.cu_seqlens[r + 1] = tok_carry + tok_incl;
            p.chunk_start[r + 1] = ch_carry + ch_incl;
        }
        tok_carry += tok_tot;
        ch_carry += ch_tot;
        ones += one_tot;
        pres += pre_tot;
        __syncthreads();   // wtot is rewritten by the next pass
    }
    if (tid == 0) {
        p.counts[0] = tok_carry;
        p.counts[1] = ones;
        p.counts[2] = pres;
        p.counts[3] = ch_carry;
    }
    if (__any(err) && lane == 0) flag_error(p.err_flag);
}

kda_status launch_build_metadata(const MetaParams &p, hipStream_t stream) {
    hipLaunchKernelGGL(kda_build_metadata_kernel, dim3(1), dim3(kMetaThreads), 0, stream, p);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // namespace kda
