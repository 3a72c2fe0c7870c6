// kda_device.h -- device helpers shared by the KDA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kWave = 64;

// Inputs are either fp32 or bf16 (carried as raw uint16_t bit patterns).
template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

__device__ __forceinline__ float sigmoid(float x) { return 1.0f / (1.0f + expf(-x)); }

// softplus without a linear cut-off: max(x, 0) + log(1 + e^-|x|)
__device__ __forceinline__ float softplus(float x) {
    return fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x)));
}

// Cross-lane sums on the VALU: DPP moves (a few cycles each) instead of LDS
// permutes.  dpp_add adds the value of the lane the DPP control selects
// (0 where that lane is masked off by the row mask).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add(float v) {
    const int x = __builtin_bit_cast(int, v);
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xF, false));
}

// Sum of v over lanes 0 .. N-1 of the wave (N = 16, 32 or 64; those lanes
// active), returned as one wave-uniform value: pair and quad sums inside
// each row of 16 lanes (quad permutes, half-row and row mirrors), then row
// broadcasts carry the row sums up to lane N-1, which is read back.
template <int N>
__device__ __forceinline__ float lane_sum(float v) {
    static_assert(N == 16 || N == 32 || N == 64, "rows of 16 lanes");
    v = dpp_add<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
    v = dpp_add<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
    v = dpp_add<0x141, 0xF>(v);   // row_half_mirror
    v = dpp_add<0x140, 0xF>(v);   // row_mirror
    if (N >= 32) v = dpp_add<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
    if (N == 64) v = dpp_add<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), N - 1));
}

// x[l] + x[l + 32] in lanes l = 0..31 (a VALU lane swap between the two
// halves of the wave; lanes 32..63 get 2 x[l], for callers that read only
// the lower half).  The same sum as x + __shfl_xor(x, 32) there.
__device__ __forceinline__ float add_upper_half(float x) {
    const unsigned v = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return x + __uint_as_float(r[1]);
}

// Sum over the 64 lanes of a wave (all active); every lane gets the same value.
__device__ __forceinline__ float wave_sum(float v) { return lane_sum<kWave>(v); }

__device__ __forceinline__ float4 operator*(float4 a, float s) {
    return make_float4(a.x * s, a.y * s, a.z * s, a.w * s);
}

__device__ __forceinline__ float4 fma4(float s, float4 a, float4 c) {
    return make_float4(fmaf(s, a.x, c.x), fmaf(s, a.y, c.y), fmaf(s, a.z, c.z), fmaf(s, a.w, c.w));
}

__device__ __forceinline__ void flag_error(int32_t *err_flag) {
    if (err_flag) atomicOr(err_flag, 1);
}

}  // namespace kda

// ---------------------------------------------------------------------------
// MFMA helpers (gfx950, v_mfma_f32_16x16x32_bf16).  Lane l of a wave holds
//   A operand: A[l % 16][8 (l / 16) + e], e < 8    (16 x 32 tile)
//   B operand: B[8 (l / 16) + e][l % 16], e < 8    (32 x 16 tile)
//   result   : D[4 (l / 16) + r][l % 16], r < 4    (16 x 16 fp32)
// "bf16x3": an fp32 operand x is split as hi = bf16(x), lo = bf16(x - hi);
// a.b ~ ah.bh + ah.bl + al.bh keeps about 16 significant bits per operand
// (relative error ~1e-5), with fp32 accumulation.
// ---------------------------------------------------------------------------
namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

struct Split8 {
    bf16x8 hi, lo;
};

__device__ __forceinline__ Split8 split8(const float *x, float sign = 1.0f) {
    Split8 s;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float v = sign * x[e];
        const __bf16 h = (__bf16)v;
        s.hi[e] = h;
        s.lo[e] = (__bf16)(v - (float)h);
    }
    return s;
}

__device__ __forceinline__ f32x4 mma3(const Split8 &a, const Split8 &b, f32x4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
    return acc;
}

}  // namespace kda
