// kda_prefill.hip -- chunked prefill of the KDA recurrence (gfx950).
//
// Many tokens per sequence are processed in chunks of C = 64.  Inside a chunk
// the delta-rule recurrence has a closed form (the WY/UT form): with the
// per-key-channel log-decay prefix G_t = sum_{r<=t} log alpha_r and start
// state S0,
//   A[t][s] = beta_t sum_c k^_tc k^_sc e^(G_tc - G_sc)        (s < t)
//   P[t][s] = sum_c q^_tc k^_sc e^(G_tc - G_sc)                (s <= t)
//   X = (I + A)^-1 [diag(beta) (K^ * e^G) | diag(beta) V] = [W | U~]
//   U = U~ - W S0,   O = (Q^ * e^G) S0 + P U,
//   S_C = diag(e^G_C) S0 + (K^ * e^(G_C - G))^T U
// (unrolling the recurrence over the chunk; the rows of U are the per-token
// corrections beta_t (v_t - (diag(alpha_t) S_{t-1})^T k^_t)).  Every exponent
// is a difference G_t - G_s with s <= t, so it is <= 0 and nothing overflows.
//
// Kernels, in stream order:
//   meta   one workgroup: validates cu_seqlens, chunk offsets per sequence
//   intra  persistent, one workgroup per CU working through the chunks of one
//          head: conv + SiLU, L2 norms and gates of the chunk's tokens, prefix
//          sums, A, P, the triangular solve for W and U~, the decayed Q and K
//          factors
//   scan   persistent, one workgroup per (sequence, head, 16 or 64 columns of
//          d_v) at a time: the fp32 state carried from chunk to chunk (state
//          columns are independent given the chunk factors) and the outputs:
//          O, then RMSNorm over d_v (the column workgroups of a head exchange
//          per-row partial sums of squares), weight and sigmoid gate
//   repair after 16-column scans: rows whose sums came too late (marked by
//          the scan), normalised once every sum is in; exits when none are
//   norm   after 64-column scans: RMSNorm, weight and gate of every row
#include <algorithm>
#include <cstdlib>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int kChunk = 64;
constexpr int kColBlock = 16;
constexpr int kBufferWord3 = 0x00020000;   // raw 32-bit buffer resource
constexpr float kLog2e = 1.4426950408889634f;
// An empty slot of the scan's row-sum exchange: a NaN bit pattern that no sum
// of squares is stored as (a NaN sum is stored as the canonical quiet NaN).
constexpr uint32_t kXpEmpty = 0xFFFFFFFFu;

// Device pointers into the caller's workspace.  The per-chunk factors the
// scan multiplies on MFMA are stored pre-split as bf16 pairs (hi = bf16(x),
// lo = bf16(x - hi)), each matrix in MFMA operand order (opnd_off below).
struct PrefillWs {
    int32_t *meta;            // [0]: 1 if cu_seqlens is valid; [1 + s]: first chunk of s, s <= N;
                              // [N + 2]: number of chunk-path sequences; [N + 3 + k]: the k-th;
                              // [2N + 3]: number of one-token sequences (decode kernel);
                              // [2N + 4]: nonzero if rows were left for the repair kernel
    uint16_t *Wn_hi, *Wn_lo;  // [G, H] x (64 x d_k)  -W
    uint16_t *Q_hi, *Q_lo;    // [G, H] x (64 x d_k)  Q^ e^G
    uint16_t *K_hi, *K_lo;    // [G, H] x (d_k x 64)  (K^ e^(G_C - G))^T
    uint16_t *P_hi, *P_lo;    // [G, H] x (64 x 64)
    float *Ut;                // [G, H, 64, d_v]
    float *gC;                // [G, H, d_k]  e^(G_C)
    uint32_t *Xp;             // [G, H, 64, d_v / 16]  sums of squares of O rows over 16 columns
    uint32_t *Xf;             // [G, H, d_v / 16, 4]  nonzero: the 16 rows of a wave left unnormalised
    int G_max;
    int xp_spin;              // polls of the exchange before a wave stops waiting
};

// Offset of element (row, k) of an R x K matrix stored in MFMA A-operand
// order: 16 x 32 tiles (row tile major, then k step), each tile as 64 lanes x
// 8 consecutive elements with lane = row % 16 + 16 ((k % 32) / 8), the
// layout of v_mfma_f32_16x16x32_bf16's A operand.  A wave's load of one
// tile is one contiguous kilobyte (eight whole 128-byte lines).
template <int K>
__device__ __forceinline__ size_t opnd_off(int row, int k) {
    return ((size_t)((row / 16) * (K / 32) + k / 32) * kWave + row % 16 + 16 * ((k % 32) / 8)) * 8 + k % 8;
}

struct WsLayout {
    size_t meta, Wn_hi, Wn_lo, Q_hi, Q_lo, K_hi, K_lo, P_hi, P_lo, Ut, gC, Xp, Xf, total;
};

static size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

static WsLayout ws_layout(int H, int dk, int dv, int total_T, int N_seq) {
    const size_t G = (size_t)total_T / kChunk + (size_t)N_seq;
    const size_t GH = G * H;
    WsLayout l{};
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
    l.meta = take(sizeof(int32_t) * (2 * (size_t)N_seq + 5));
    l.Wn_hi = take(2 * GH * kChunk * dk);
    l.Wn_lo = take(2 * GH * kChunk * dk);
    l.Q_hi = take(2 * GH * kChunk * dk);
    l.Q_lo = take(2 * GH * kChunk * dk);
    l.K_hi = take(2 * GH * dk * kChunk);
    l.K_lo = take(2 * GH * dk * kChunk);
    l.P_hi = take(2 * GH * kChunk * kChunk);
    l.P_lo = take(2 * GH * kChunk * kChunk);
    l.Ut = take(4 * GH * kChunk * dv);
    l.gC = take(4 * GH * dk);
    l.Xp = take(4 * GH * kChunk * (dv / 16));
    l.Xf = take(4 * GH * (dv / 16) * 4);
    l.total = off;
    return l;
}

size_t prefill_workspace_bytes(int H, int d_k, int d_v, int total_T, int N_seq, int chunk) {
    if (chunk != kChunk || total_T < 0 || N_seq < 1) return 0;
    return ws_layout(H, d_k, d_v, total_T, N_seq).total;
}

// A load through the scalar unit, for tables no kernel of the call writes
// after its launch (metadata, cu_seqlens, slot tables): scalar loads keep
// off the vector memory counter, which also counts outstanding stores.
__device__ __forceinline__ int32_t ld_const(const int32_t *a) {
    typedef __attribute__((address_space(4))) const int32_t cint32;
    return *reinterpret_cast<cint32 *>(reinterpret_cast<uintptr_t>(a));
}

// Largest s in [0, n) with a[s] <= v (a non-decreasing, a[0] <= v).
__device__ __forceinline__ int upper_index(const int32_t *a, int n, int v) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (ld_const(a + mid) <= v) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ bool slot_ok(int slot, int n_slots) { return slot >= 0 && slot < n_slots; }

// ---------------------------------------------------------------------------
// meta: one wave.  Validates cu_seqlens, gives each sequence that takes the
// chunk path (two or more tokens and a valid slot) its run of chunk slots,
// and lists those sequences in order, so the intra and scan grids can put
// all real work ahead of the workgroups that only exit.  One-token
// sequences take the decode kernel; empty sequences and padding rows take
// nothing.  64 sequences per step, prefix sums across the wave.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
        const int u = __shfl_up(v, m, kWave);
        if (lane >= m) v += u;
    }
    return v;
}

__global__ __launch_bounds__(64) void kda_prefill_meta_kernel(PrefillParams p, PrefillWs ws) {
    const int lane = threadIdx.x, N = p.N_seq;
    int32_t *cs = ws.meta + 1;
    int32_t *list = ws.meta + N + 3;
    bool ok = true, bad_slot = false;
    int chunks = 0, longs = 0, ones = 0;
    if (lane == 0) cs[0] = 0;
    for (int base = 0; base < N; base += kWave) {
        const int s = base + lane;
        int nch = 0, isl = 0;
        if (s < N) {
            const int a0 = p.cu_seqlens[s], a1 = p.cu_seqlens[s + 1];
            ok = ok && a1 >= a0;
            const int sl = p.slot_idx[s];
            bad_slot = bad_slot || (sl != -1 && !slot_ok(sl, p.n_slots));
            if (a1 - a0 >= 2 && slot_ok(sl, p.n_slots)) {
                nch = (a1 - a0 + kChunk - 1) / kChunk;
                isl = 1;
            }
            ones += a1 - a0 == 1 && slot_ok(sl, p.n_slots);
        }
        const int ic = wave_incl_scan(nch, lane), il = wave_incl_scan(isl, lane);
        if (s < N) {
            cs[s + 1] = chunks + ic;
            if (isl) list[longs + il - 1] = s;
        }
        chunks += __shfl(ic, kWave - 1, kWave);
        longs += __shfl(il, kWave - 1, kWave);
    }
    ok = __all(ok) && p.cu_seqlens[0] == 0 && p.cu_seqlens[N] == p.total_T;
    bad_slot = __any(bad_slot);
    ones = wave_incl_scan(ones, lane);
    if (lane == kWave - 1) ws.meta[2 * N + 3] = ok ? ones : 0;
    if (lane == 0) ws.meta[2 * N + 4] = 0;
    if (lane == 0) {
        ws.meta[0] = ok ? 1 : 0;
        ws.meta[N + 2] = ok ? longs : 0;
        if (!ok || bad_slot) flag_error(p.err_flag);
    }
}

// ---------------------------------------------------------------------------
// intra: persistent workgroups of 16 waves, one per CU; workgroup w works
// through every (CUs / H)-th chunk of head w mod H.  Per chunk: the tokens are
// brought in (conv + SiLU, L2 norms, gates; the inputs were requested while
// the previous chunk was computed), then the Gram matrices A and P, the
// diagonal 16 x 16 blocks of T = (I + A)^-1 and [W | U~] = T [diag(beta) K^ e^G
// | diag(beta) V]; every contraction runs on MFMA in bf16x3.
//
// Gram tiles are 16 x 16 token blocks.  For t in block bt (first row r) and s
// in block bs (last row e), e^(G_t - G_s) = e^(G_t - G_r) M e^(G_e - G_s) with
// M = e^(G_r - G_e) per channel: each row is scaled once to its own block's
// start and end, and a tile multiplies one of them by its pair's factor.  Off
// the diagonal every factor is <= 1.  On the diagonal M >= 1; it is used only
// when the block's decay span is at most 2^60 (checked per block), otherwise
// the tile is summed directly with one exponential per term.
//
// [W | U~] is the solution X of (I + A) X = R, found block by block: X_b =
// T_bb (R_b - sum_{m < b} A_bm X_m), each wave for its own 16 columns.
//
// LDS holds the token rows (q^, k^, G, then their scaled forms), -A and the
// diagonal blocks of T split into bf16 pairs, the block factors and the
// head's constants: about 152 KiB at d_k = 128, one workgroup per CU.  v is
// convolved from its raw inputs where [W | U~] needs it.  The factors for the
// scan (P, Q^ e^G, Kd^T, -W as bf16 hi/lo; U~ in fp32) are written in the
// order its loads read.
// ---------------------------------------------------------------------------
constexpr int kIntraThreads = 1024;
constexpr int kIntraWaves = kIntraThreads / kWave;

template <int DK, int DV>
struct __align__(16) IntraLds {
    static constexpr int RW = DK + 4;   // row pitch: 16-byte rows
    static constexpr int NPAIR = 10;    // token-block pairs (bt, bs), bs <= bt
    // Token rows.  Phase 1 writes q^, k^ and the log2-decay prefix sums G in
    // fp32; the conversion then rewrites each row in place: Q and K hold
    // q^ e^(G - G_r) and k^ e^(G - G_r) (r: the row's block start) split into
    // bf16 pairs, for each 8 channels their 8 hi halves then their 8 lo halves
    // (the 32 bytes the 8 fp32 values held), and G holds the fp32
    // k^ e^(G_e - G) (e: the row's block end).
    float Q[kChunk][RW];
    float K[kChunk][RW];
    float G[kChunk][RW];
    float M[NPAIR][DK];                 // e^(G_{16 bt} - G_{16 bs + 15}) per block pair
    float Fq[4][DK];                    // e^(G_{16 b}): block start -> chunk start
    float Fk[4][DK];                    // e^(G_last - G_{16 b + 15}): block end -> chunk end
    // -A (A_ts = beta_t k^_t k^_s decay, s < t; zero on and above the
    // diagonal) and the diagonal 16 x 16 blocks of T = (I + A)^-1, split into
    // bf16 pairs: rows of 4 consecutive elements are operands of
    // v_mfma_f32_16x16x16_bf16
    __bf16 NAh[kChunk][kChunk + 4], NAl[kChunk][kChunk + 4];
    __bf16 Th[4][16][20], Tl[4][16][20];
    float Gb[9][DK];                    // G at the block starts, block ends, the last token
    float D[10][16][17];                // per-wave scratch of waves 0..9: direct tiles, tile stores
    float beta[kChunk];
    int safe[4];
    // the head's constants: conv taps of the q and k channels and of the v
    // channels, e^A per key channel
    float4 Cw[2 * DK];
    float4 Cv[DV];
    float Cea[DK];
};

// The value of the lane the DPP control selects inside each quad of lanes.
template <int CTRL>
__device__ __forceinline__ float quad_get(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Hardware exp2 / log2 / reciprocal forms for the per-token preparation
// (about 1 ulp each; the chunk algebra's bf16x3 contractions are ~1e-5).
__device__ __forceinline__ float silu_hw(float x) {
    return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
}
// 2^x by the hardware instruction, for the decay factors of the chunk
// algebra: every argument is a difference of log2-decay prefix sums (<= 0,
// or <= 60 on a diagonal tile that passed the span check), so the library
// form's range handling is not needed (a result below 2^-126 flushes to 0,
// far under the products it scales).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// log2(alpha) = -e^A softplus(g) / ln 2, softplus(g) = max(g, 0) + ln(1 + e^-|g|)
__device__ __forceinline__ float log2_alpha_hw(float ea, float g) {
    const float sp2 = fmaxf(g, 0.f) * kLog2e + __builtin_amdgcn_logf(1.0f + __builtin_amdgcn_exp2f(-fabsf(g) * kLog2e));
    return -ea * sp2;
}

// NC consecutive input channels of one row, fetched in one load
template <typename Tin, int NC> struct ChRaw;
template <> struct ChRaw<uint16_t, 2> {
    using T = uint32_t;
    __device__ static float get(T r, int e) { return __uint_as_float(e ? (r & 0xffff0000u) : (r << 16)); }
};
template <> struct ChRaw<uint16_t, 1> {
    using T = uint16_t;
    __device__ static float get(T r, int) { return __uint_as_float((uint32_t)r << 16); }
};
template <> struct ChRaw<float, 2> {
    using T = float2;
    __device__ static float get(T r, int e) { return e ? r.y : r.x; }
};
template <> struct ChRaw<float, 1> {
    using T = float;
    __device__ static float get(T r, int) { return r; }
};

template <typename Tin> struct Vec8 {
    typedef Tin T __attribute__((ext_vector_type(8)));
};

// A workgroup works through the chunks of one head and requests the next
// chunk's token inputs while it computes the current one; each wave keeps
// what its role needs of them in registers.
//
// q or k rows 8 part .. 8 part + 7 of a chunk and the three inputs before
// them (from the conv window at chunk 0, else from the sequence; rows past
// the chunk's end repeat its last row); the lane owns channels NC lane ..
// NC lane + NC - 1.
template <typename Tin, int NC>
__device__ __forceinline__ void rows_issue(const PrefillParams &p, const Tin *x, const Tin *win, int choff, int CH,
                                           int c, int t0, int n, int h, int lane, int part,
                                           typename ChRaw<Tin, NC>::T (&raw)[11]) {
    using RT = typename ChRaw<Tin, NC>::T;
    constexpr int D = NC * kWave;
    const int H = p.H, cb = NC * lane;
#pragma unroll
    for (int j = 0; j < 11; ++j) {
        const int q = 8 * part - 3 + j;   // chunk row of the input (wave-uniform)
        const Tin *src;
        if (q < 0)
            src = c == 0 ? win + (q + 3) * CH + choff + cb : x + ((size_t)(t0 + q) * H + h) * D + cb;
        else
            src = x + ((size_t)(t0 + min(q, n - 1)) * H + h) * D + cb;
        raw[j] = *reinterpret_cast<const RT *>(src);
    }
}

// Conv + SiLU, L2 norm (times `scale`) of those rows into LDS (zero past n).
template <typename Tin, int NC>
__device__ __forceinline__ void rows_compute(const PrefillParams &p, const typename ChRaw<Tin, NC>::T (&raw)[11],
                                             const float4 *wt, float scale, int n, int lane, int part,
                                             float *out, int ostride) {
    using R = ChRaw<Tin, NC>;
    const int cb = NC * lane;
    float w[NC][4];
#pragma unroll
    for (int e = 0; e < NC; ++e) {
        const float4 v = wt[e];
        w[e][0] = v.x; w[e][1] = v.y; w[e][2] = v.z; w[e][3] = v.w;
    }
    float y[8][NC], ss[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int e = 0; e < NC; ++e) {
            float acc = w[e][0] * R::get(raw[j], e);
            acc = fmaf(w[e][1], R::get(raw[j + 1], e), acc);
            acc = fmaf(w[e][2], R::get(raw[j + 2], e), acc);
            acc = fmaf(w[e][3], R::get(raw[j + 3], e), acc);
            y[j][e] = p.silu ? silu_hw(acc) : acc;
        }
        ss[j] = 0.f;
#pragma unroll
        for (int e = 0; e < NC; ++e) ss[j] = fmaf(y[j][e], y[j][e], ss[j]);
    }
    // The eight row sums over the wave, by halving exchanges: at each step a
    // lane keeps the half of its partial sums that its lane bit selects and
    // adds the partner's partials of that half (the partner lane differs in
    // that bit), so after lane bits 0, 1 and 2 it holds one row, l % 8, and
    // the sums over lane bits 3, 4 and 5 complete it.  One rsqrt per lane
    // instead of one per row.
    const bool b0 = lane & 1, b1 = lane & 2, b2 = lane & 4;
    float r1[4], r2[2];
#pragma unroll
    for (int k = 0; k < 4; ++k)   // partner lane ^ 1: quad_perm [1,0,3,2]
        r1[k] = (b0 ? ss[2 * k + 1] : ss[2 * k]) + quad_get<0xB1>(b0 ? ss[2 * k] : ss[2 * k + 1]);
#pragma unroll
    for (int k = 0; k < 2; ++k)   // partner lane ^ 2: quad_perm [2,3,0,1]
        r2[k] = (b1 ? r1[2 * k + 1] : r1[2 * k]) + quad_get<0x4E>(b1 ? r1[2 * k] : r1[2 * k + 1]);
    float r3 = (b2 ? r2[1] : r2[0]) + __shfl_xor(b2 ? r2[0] : r2[1], 4, kWave);
    r3 += __shfl_xor(r3, 8, kWave);
    r3 += __shfl_xor(r3, 16, kWave);
    r3 += __shfl_xor(r3, 32, kWave);
    const float scl = 8 * part + (lane & 7) < n ? scale * __builtin_amdgcn_rsqf(r3 + p.l2_eps) : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int row = 8 * part + j;
        const float sc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, scl), j));
        float *dst = out + row * ostride + cb;
        if (NC == 2) *reinterpret_cast<float2 *>(dst) = make_float2(y[j][0] * sc, y[j][NC - 1] * sc);
        else dst[0] = y[j][0] * sc;
    }
}

// Gate inputs of the 16 rows of block qt for channels ch0 .. ch0 + 63: the
// lane fetches 8 channels of rows 16 qt + lane / 8 and 16 qt + lane / 8 + 8.
template <int DK, typename Tin>
__device__ __forceinline__ void gates_issue(const PrefillParams &p, int t0, int n, int h, int lane, int ch0, int qt,
                                            typename Vec8<Tin>::T (&raw)[2]) {
    using V8 = typename Vec8<Tin>::T;
    const int row0 = 16 * qt + lane / 8, cl = ch0 + 8 * (lane % 8);
    const Tin *g = static_cast<const Tin *>(p.g);
#pragma unroll
    for (int i = 0; i < 2; ++i)
        raw[i] = *reinterpret_cast<const V8 *>(g + ((size_t)(t0 + min(row0 + 8 * i, n - 1)) * p.H + h) * DK + cl);
}

// log2(alpha) of those tokens into G, then each lane turns its channel's
// 16 entries into prefix sums from the block's first row (rows past n add
// nothing).  Block sums start again at each block; the block totals link
// them where a factor spans blocks.
template <int DK, typename Tin>
__device__ __forceinline__ void gates_compute(const typename Vec8<Tin>::T (&raw)[2], const float *ea, int n,
                                              int lane, int ch0, int qt, float (*G)[DK + 4]) {
    const int row0 = 16 * qt + lane / 8, cl = ch0 + 8 * (lane % 8);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = row0 + 8 * i;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            // alpha below 2^-200 is 0 in fp32 either way; the floor keeps the
            // prefix sums finite (g = +inf would give -inf - -inf = NaN later)
            const float la = fmaxf(log2_alpha_hw(ea[e], to_f32(raw[i][e])), -200.f);
            G[row][cl + e] = row < n ? la : 0.f;
        }
    }
    // the column a lane sums was written by other lanes of this wave
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int ch = ch0 + lane;
    float acc = 0.f;
#pragma unroll
    for (int j = 16 * qt; j < 16 * qt + 16; ++j) {
        acc += G[j][ch];
        G[j][ch] = acc;
    }
}

constexpr float kSafeSpan = 60.f;

// bf16x3 splits with the paired conversion (v_cvt_pk_bf16_f32 rounds two
// fp32 values to nearest even in one instruction): x = hi + lo, hi = bf16(x),
// lo = bf16(x - hi), three instructions per value.
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
typedef unsigned u32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
    const f32x2v v = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2v));
}
__device__ __forceinline__ void split_pair(float a, float b, unsigned &hi, unsigned &lo) {
    hi = pack_bf16(a, b);
    lo = pack_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}
__device__ __forceinline__ Split8 split8p(const float *x) {
    u32x4v h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        unsigned a, b;
        split_pair(x[2 * i], x[2 * i + 1], a, b);
        h[i] = a;
        l[i] = b;
    }
    Split8 s;
    s.hi = __builtin_bit_cast(bf16x8, h);
    s.lo = __builtin_bit_cast(bf16x8, l);
    return s;
}

// A 16 x 16 fp32 tile in the MFMA result layout (lane l holds rows
// 4 (l / 16) + r, column l % 16) written to a split bf16 matrix with K
// columns in operand order, as 16-byte stores: through the wave's LDS
// scratch, lanes 0..31 each take 8 consecutive columns of one row.
template <int K>
__device__ __forceinline__ void store_tile_split(float (*scr)[17], const f32x4 &v, int lane, uint16_t *hi,
                                                 uint16_t *lo, int row0, int col0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) scr[4 * (lane / 16) + r][lane % 16] = v[r];
    __builtin_amdgcn_wave_barrier();
    if (lane < 32) {
        const int row = lane % 16, kq = lane / 16;
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = scr[row][8 * kq + e];
        const Split8 sx = split8p(x);
        const size_t o = opnd_off<K>(row0 + row, col0 + 8 * kq);
        *reinterpret_cast<bf16x8 *>(hi + o) = sx.hi;
        *reinterpret_cast<bf16x8 *>(lo + o) = sx.lo;
    }
    __builtin_amdgcn_wave_barrier();
}

// 8 consecutive fp32 values of an LDS row (16-byte aligned)
__device__ __forceinline__ void lds8(const float *src, float *x) {
    const float4 a = *reinterpret_cast<const float4 *>(src);
    const float4 b = *reinterpret_cast<const float4 *>(src + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// Sum over the four 16-lane rows of a wave (lanes l, l ^ 16, l ^ 32,
// l ^ 48), every lane receiving it: VALU lane-row swaps.
__device__ __forceinline__ float row4_sum(float v) {
    const unsigned u = __float_as_uint(v);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const unsigned us = __float_as_uint(s);
    const auto b = __builtin_amdgcn_permlane32_swap(us, us, false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// One element through a raw buffer load (an offset past the buffer's range
// reads 0).
template <typename Tin> __device__ __forceinline__ Tin buffer_load_elem(__amdgpu_buffer_rsrc_t r, unsigned off);
template <> __device__ __forceinline__ uint16_t buffer_load_elem<uint16_t>(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
template <> __device__ __forceinline__ float buffer_load_elem<float>(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

// bf16x3 on v_mfma_f32_16x16x16_bf16 (4 operand elements per lane)
typedef short s16x4 __attribute__((ext_vector_type(4)));
struct Split4 {
    s16x4 hi, lo;
};
__device__ __forceinline__ Split4 split4(const float *x) {
    u32x2v h, l;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        unsigned a, b;
        split_pair(x[2 * i], x[2 * i + 1], a, b);
        h[i] = a;
        l[i] = b;
    }
    Split4 s;
    s.hi = __builtin_bit_cast(s16x4, h);
    s.lo = __builtin_bit_cast(s16x4, l);
    return s;
}
__device__ __forceinline__ f32x4 mma3k16(const Split4 &a, const Split4 &b, f32x4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.lo, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.lo, b.hi, acc, 0, 0, 0);
    return acc;
}

template <int DK, int DV, typename Tin>
__global__ __launch_bounds__(kIntraThreads, 1) void kda_prefill_intra_kernel(PrefillParams p, PrefillWs ws) {
    constexpr int KS = DK / 32, NC = DK / 64, CH = 2 * DK + DV;
    constexpr int RW = IntraLds<DK, DV>::RW;
    constexpr int NCT = (DK + DV) / 16;          // column tiles of [W | U~], one per wave
    static_assert(NCT <= kIntraWaves && DK / 16 <= 10, "one column tile per wave; W tiles on waves with scratch");
    using RT = typename ChRaw<Tin, NC>::T;
    using V8 = typename Vec8<Tin>::T;
    __shared__ IntraLds<DK, DV> L;
    // the wave index as a scalar: role branches are uniform
    const int tid = threadIdx.x, lane = tid % kWave, wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lr = lane % 16;
    const int H = p.H;
    if (ws.meta[0] != 1) return;
    const int32_t *cs = ws.meta + 1;
    const int nchunks = cs[p.N_seq];   // chunk slots, all of sequences on the chunk path
    // workgroup w works through chunk slots w / H, w / H + wph, ... of head w % H
    const int h = (int)(blockIdx.x % (unsigned)H), wph = (int)(gridDim.x / (unsigned)H);
    int gidx = (int)(blockIdx.x / (unsigned)H);
    if (gidx >= nchunks) return;

    // roles in step 1: waves 0-7 q^ rows and 8-15 k^ rows, 8 rows each;
    // waves 0 .. DK / 16 - 1 the decay sums of one 16-row block for 64
    // channels each; the last wave beta.  In step 5 wave w takes column tile w.
    const bool isq = wave < 8;
    const int part = wave % 8;
    const Tin *xr = static_cast<const Tin *>(isq ? p.x_q : p.x_k);
    const int choff = isq ? 0 : DK;
    const int gcg = wave / 4, gqt = wave % 4;
    const bool gate_wave = wave < 8 && 64 * gcg < DK;   // wave-uniform
    const bool u_wave = wave >= DK / 16 && wave < NCT;   // wave-uniform
    const int vcol = 16 * wave + lr - DK;                // a U~ wave's v channel
    // the head's constants into LDS (read by step 1 and step 5)
    for (int e = tid; e < CH; e += kIntraThreads) {
        const float4 v = *reinterpret_cast<const float4 *>(p.conv_wt + ((size_t)h * CH + e) * 4);
        if (e < 2 * DK) L.Cw[e] = v;
        else L.Cv[e - 2 * DK] = v;
    }
    if (tid < DK) L.Cea[tid] = expf(p.A[h * DK + tid]);

    // chunk slot g: chunk c of its sequence, its first token t0, n tokens,
    // the sequence's conv window
    auto locate = [&](int g, int &c_, int &t0_, int &n_, const Tin *&win_) {
        const int sq = upper_index(cs, p.N_seq + 1, g);
        const int slot = ld_const(p.slot_idx + sq);
        c_ = g - ld_const(cs + sq);
        t0_ = ld_const(p.cu_seqlens + sq) + c_ * kChunk;
        n_ = min(kChunk, ld_const(p.cu_seqlens + sq + 1) - t0_);
        win_ = static_cast<const Tin *>(p.window) + ((size_t)slot * H + h) * 3 * CH;
    };
    RT rraw[11];
    V8 graw[2];
    auto issue_rows = [&](int c_, int t0_, int n_, const Tin *win_, int ln) {
        rows_issue<Tin, NC>(p, xr, win_, choff, CH, c_, t0_, n_, h, ln, part, rraw);
        if (gate_wave) gates_issue<DK, Tin>(p, t0_, n_, h, ln, 64 * gcg, gqt, graw);
    };
    int c, t0, n;
    const Tin *win;
    locate(gidx, c, t0, n, win);
    issue_rows(c, t0, n, win, lane);
    __syncthreads();

    for (;;) {
    // fresh copies of the lane indices for each chunk: what is derived from
    // them (LDS and workspace addresses) is formed where it is used instead
    // of being kept live in registers across the whole loop
    int tid;
    asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
    const int lane = tid % kWave, lr = lane % 16, lk = lane / 16;
    const size_t gh = (size_t)gidx * H + h;
    // 1. the chunk's tokens: q^, k^ rows (conv + SiLU + L2 norm), the decay
    //    prefix sums and beta into LDS (beta requested here: one value)
    Tin bv = Tin(0);
    if (wave == kIntraWaves - 1) bv = static_cast<const Tin *>(p.b)[(size_t)(t0 + min(lane, n - 1)) * H + h];
    rows_compute<Tin, NC>(p, rraw, &L.Cw[choff + NC * lane], isq ? p.q_scale : 1.0f, n, lane, part,
                          isq ? &L.Q[0][0] : &L.K[0][0], RW);
    if (gate_wave) gates_compute<DK, Tin>(graw, &L.Cea[64 * gcg + 8 * (lane % 8)], n, lane, 64 * gcg, gqt, L.G);
    if (wave == kIntraWaves - 1) L.beta[lane] = lane < n ? sigmoid(to_f32(bv)) : 0.f;
    __syncthreads();

    // 2. per 16-token block: may its diagonal tile use scaled factors
    //    (waves 0-3)?  G (block-local) at the block starts, the block ends
    //    (the block totals) and the last token (the other waves).
    const int last = max(n - 1, 0);
    constexpr int NPAIR = IntraLds<DK, DV>::NPAIR;
    if (wave < 4) {
        float span = 0.f;
        for (int i = lane; i < DK; i += kWave) span = fmaxf(span, L.G[16 * wave][i] - L.G[16 * wave + 15][i]);
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) span = fmaxf(span, __shfl_xor(span, m, kWave));
        if (lane == 0) L.safe[wave] = span <= kSafeSpan ? 1 : 0;
    } else {
        for (int e = tid - 4 * kWave; e < 9 * DK; e += kIntraThreads - 4 * kWave) {
            const int j = e / DK, i = e % DK;
            const int row = j < 4 ? 16 * j : j < 8 ? 16 * (j - 4) + 15 : last;
            L.Gb[j][i] = L.G[row][i];
        }
    }
    __syncthreads();

    // A (times beta, strictly lower) to LDS and P (lower, diagonal included)
    // split to the workspace, from a tile pair in the MFMA result layout
    uint16_t *Ph = ws.P_hi + gh * kChunk * kChunk, *Pl = ws.P_lo + gh * kChunk * kChunk;
    auto gram_out = [&](int bt, int bs, f32x4 aA, f32x4 aP) {
        float na[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int t = 16 * bt + 4 * lk + rr, sv = 16 * bs + lr;
            na[rr] = sv < t ? -L.beta[t] * aA[rr] : 0.f;
            const __bf16 hb = (__bf16)na[rr];
            L.NAh[t][sv] = hb;
            L.NAl[t][sv] = (__bf16)(na[rr] - (float)hb);
            aP[rr] = sv <= t ? aP[rr] : 0.f;
        }
        store_tile_split<kChunk>(L.D[wave], aP, lane, Ph, Pl, 16 * bt, 16 * bs);
        if (bt == bs) {
            // the diagonal block of T = (I + A)^-1 from this wave's own A
            // tile (in fp32 through its scratch): column lr of (I + A_bb)^-1
            // by forward substitution
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) L.D[wave][4 * lk + rr][lr] = na[rr];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // (the sum over earlier rows is split over the four lane rows,
            // m = 4 m' + lk, and combined by lane-row swaps; A_bb is zero on
            // and above its diagonal)
            float xs[4] = {0.f, 0.f, 0.f, 0.f};   // x_m, m = 4 m' + lk
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float part = 0.f;
#pragma unroll
                for (int mp = 0; mp < 4; ++mp)
                    if (4 * mp < i) part = fmaf(L.D[wave][i][4 * mp + lk], xs[mp], part);
                const float xi = (i == lr ? 1.f : 0.f) + row4_sum(part);
                if (lk == i % 4) xs[i / 4] = xi;
                if (lk == 0) {
                    const __bf16 hb = (__bf16)xi;
                    L.Th[bt][i][lr] = hb;
                    L.Tl[bt][i][lr] = (__bf16)(xi - (float)hb);
                }
            }
        }
    };

    // 2b. a block whose decay span is too wide for scaled factors has its
    //     diagonal tiles summed directly (one exponential per term), from the
    //     plain rows, before they are rewritten: lane owns row t = r + lr and
    //     columns s = r + 4 lk + j
    if (!(L.safe[0] & L.safe[1] & L.safe[2] & L.safe[3])) {
        if (wave < 4 && !L.safe[wave]) {
            const int r = 16 * wave, t = r + lr;
            float da[4] = {0.f, 0.f, 0.f, 0.f}, dp[4] = {0.f, 0.f, 0.f, 0.f};
            for (int ch = 0; ch < DK; ++ch) {
                const float kv = L.K[t][ch], qv = L.Q[t][ch], gt = L.G[t][ch];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int sv = r + 4 * lk + j;
                    const float e = exp2_hw(fminf(gt - L.G[sv][ch], 0.f)) * L.K[sv][ch];
                    da[j] = fmaf(kv, e, da[j]);
                    dp[j] = fmaf(qv, e, dp[j]);
                }
            }
            // to the MFMA result layout through this wave's scratch
            f32x4 aA, aP;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                L.D[wave + 4][lr][4 * lk + j] = da[j];
                L.D[wave][lr][4 * lk + j] = dp[j];
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                aA[rr] = L.D[wave + 4][4 * lk + rr][lr];
                aP[rr] = L.D[wave][4 * lk + rr][lr];
            }
            __builtin_amdgcn_wave_barrier();
            gram_out(wave, wave, aA, aP);
        }
        __syncthreads();
    }

    // 3. the rows rewritten for the Gram operands, each lane converting the
    //    8-channel groups it reads (e^(G - G_r) and e^(G_e - G) are <= 1:
    //    G falls along the chunk); then the per-channel block factors
    for (int u = tid; u < kChunk * DK / 8; u += kIntraThreads) {
        const int t = u / (DK / 8), c0 = 8 * (u % (DK / 8)), b = t / 16;
        float q[8], k[8], g[8], gr[8], ge[8], ko[8];
        lds8(&L.Q[t][c0], q);
        lds8(&L.K[t][c0], k);
        lds8(&L.G[t][c0], g);
        lds8(&L.Gb[b][c0], gr);
        lds8(&L.Gb[4 + b][c0], ge);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float ein = exp2_hw(g[e] - gr[e]);
            ko[e] = k[e] * exp2_hw(ge[e] - g[e]);
            q[e] *= ein;
            k[e] *= ein;
        }
        const Split8 sq = split8p(q), sk = split8p(k);
        bf16x8 *dq = reinterpret_cast<bf16x8 *>(&L.Q[t][c0]), *dk = reinterpret_cast<bf16x8 *>(&L.K[t][c0]);
        dq[0] = sq.hi;
        dq[1] = sq.lo;
        dk[0] = sk.hi;
        dk[1] = sk.lo;
        float4 *dg = reinterpret_cast<float4 *>(&L.G[t][c0]);
        dg[0] = make_float4(ko[0], ko[1], ko[2], ko[3]);
        dg[1] = make_float4(ko[4], ko[5], ko[6], ko[7]);
    }
    // Exponents across blocks are sums of block totals Tb (G of a block's
    // last row) and block-local values: with S_b = G at row 16 b and GL = G
    // at the last token (block lb),
    //   M (bt, bs) = e^(S_bt + sum_{bs < b < bt} T_b), or e^(S_b - T_b) on the diagonal;
    //   Fq (b) = e^(sum_{b' < b} T_b' + S_b)  (block start -> chunk start);
    //   Fk (b) = e^(sum_{b < b' < lb} T_b' + GL), e^(GL - T_b) for b = lb, 1 past lb;
    //   e^(G_C) = e^(sum_{b < lb} T_b + GL).
    if (tid < DK) {
        const int i = tid, lb = last / 16;
        float S[4], T[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            S[b] = L.Gb[b][i];
            T[b] = L.Gb[4 + b][i];
        }
        const float GL = L.Gb[8][i];
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) {
            float x = S[bt];
#pragma unroll
            for (int bs = bt; bs >= 0; --bs) {
                // on the diagonal the factor is >= 1 (<= 2^60 where it is
                // used: the block passed the span check)
                L.M[bt * (bt + 1) / 2 + bs][i] = exp2_hw(bs == bt ? S[bt] - T[bt] : x);
                if (bs < bt && bs > 0) x += T[bs];
            }
        }
        float off = 0.f;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            L.Fq[b][i] = exp2_hw(off + S[b]);
            off += T[b];
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            float x = 0.f;
            if (b == lb) {
                x = GL - T[b];
            } else if (b < lb) {
                x = GL;
#pragma unroll
                for (int b2 = 0; b2 < 4; ++b2)
                    if (b2 > b && b2 < lb) x += T[b2];
            }
            L.Fk[b][i] = exp2_hw(x);
        }
        float gc = GL;
#pragma unroll
        for (int b = 0; b < 4; ++b)
            if (b < lb) gc += T[b];
        ws.gC[gh * DK + i] = exp2_hw(gc);
    }
    __syncthreads();

    // the raw v inputs of step 5 (U~ columns): a lane's channel vcol for
    // rows 16 b + 4 lk .. + 3 and the three rows before each run (rows past
    // the chunk's end repeat its last row; their beta is 0)
    //    As raw buffer loads over rows t0 - sh .. t0 + n - 1 (sh = 3, or 0 at
    //    chunk 0): a row outside that range reads 0 (past the chunk's end
    //    beta is 0; before the sequence the conv window supplies it).
    Tin vraw[4][7];
    if (u_wave) {
        const int sh = c == 0 ? 0 : 3;
        const unsigned rowb = (unsigned)(H * DV * sizeof(Tin));
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<Tin *>(static_cast<const Tin *>(p.x_v) + ((size_t)(t0 - sh) * H + h) * DV + 16 * wave - DK), 0,
            (int)((unsigned)(n + sh) * rowb), kBufferWord3);
        const unsigned vo = (unsigned)(4 * lk) * rowb + (unsigned)(lr * sizeof(Tin));
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int j = 0; j < 7; ++j) {
                // chunk row 16 b + 4 lk + j - 3; negative offsets wrap past the range
                const unsigned off = vo + (unsigned)(16 * b + j - 3 + sh) * rowb;
                vraw[b][j] = buffer_load_elem<Tin>(rs, off);
            }
        if (c == 0 && lk == 0) {   // rows -3 .. -1 of the first chunk
#pragma unroll
            for (int j = 0; j < 3; ++j) vraw[0][j] = win[j * CH + 2 * DK + vcol];
        }
    }
    // 4. A and P by token-block pair (bt, bs), bs <= bt: for t in block bt
    //    and s in block bs, e^(G_t - G_s) = e^(G_t - G_r) M_(bt,bs) e^(G_e - G_s)
    //    (r = 16 bt, e = 16 bs + 15): the rewritten q and k rows are the A
    //    operands, the rewritten k rows times the pair's factor the shared B
    //    operand.  Ten pairs (a diagonal pair also inverts its block of
    //    I + A) and the six zero P tiles above the diagonal, one item per wave.
    // items by wave: the diagonal pairs 0 2 5 9 on waves 0-3, the other
    // pairs on 4-9, the zero tiles on 10-15 (waves 8-15 also request the v
    // inputs of step 5)
    {
        const int j = (int)((0xFEDCBA8764319520ull >> (4 * wave)) & 15u);
        if (j >= NPAIR) {
            const int u = j - NPAIR, bt = u < 3 ? 0 : u < 5 ? 1 : 2, bs = u < 3 ? u + 1 : u < 5 ? u - 1 : 3;
            if (lane < 32) {
                const bf16x8 z = {};
                const size_t o = opnd_off<kChunk>(16 * bt + lane % 16, 16 * bs + 8 * (lane / 16));
                *reinterpret_cast<bf16x8 *>(Ph + o) = z;
                *reinterpret_cast<bf16x8 *>(Pl + o) = z;
            }
            // the chunk's slots of the scan's row-sum exchange, marked empty
            // (waves 10 and 11; the scan runs after this kernel)
            const int e4 = (wave - NPAIR) * kWave + lane;
            if (e4 < kChunk * (DV / 16) / 4)
                reinterpret_cast<uint4 *>(ws.Xp + gh * kChunk * (DV / 16))[e4] =
                    make_uint4(kXpEmpty, kXpEmpty, kXpEmpty, kXpEmpty);
            // and its marks of rows left for the repair kernel cleared
            else if (e4 < kChunk * (DV / 16) / 4 + DV / 16)
                reinterpret_cast<uint4 *>(ws.Xf + gh * (DV / 16) * 4)[e4 - kChunk * (DV / 16) / 4] = make_uint4(0, 0, 0, 0);
        } else {
        const int bt = j < 1 ? 0 : j < 3 ? 1 : j < 6 ? 2 : 3, bs = j - bt * (bt + 1) / 2;
        if (!(bt == bs && !L.safe[bt])) {   // else summed directly above
        const int t = 16 * bt + lr, sr = 16 * bs + lr;
        f32x4 aA = {0.f, 0.f, 0.f, 0.f}, aP = aA;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            const int c0 = 32 * kk + 8 * lk;
            const bf16x8 *ka = reinterpret_cast<const bf16x8 *>(&L.K[t][c0]);
            const bf16x8 *qa = reinterpret_cast<const bf16x8 *>(&L.Q[t][c0]);
            float kb[8], m[8];
            lds8(&L.G[sr][c0], kb);
            lds8(&L.M[j][c0], m);
#pragma unroll
            for (int e = 0; e < 8; ++e) kb[e] *= m[e];
            const Split8 b = split8p(kb);
            aA = mma3(Split8{ka[0], ka[1]}, b, aA);
            aP = mma3(Split8{qa[0], qa[1]}, b, aP);
        }
        gram_out(bt, bs, aA, aP);
        }
        }
    }
    // decayed factors for the scan: Q^ e^G (rows), (K^ e^(G_C - G))^T, by
    //    waves 4-15 (waves 0-3, which invert the diagonal blocks, are the
    //    last to finish their items).  Unit e8 (8 elements) is stored at 8 e8
    //    in operand order, so each wave writes whole lines: tile e8 / 64,
    //    lane e8 % 64 of that tile.
    for (int e8 = tid - 4 * kWave; e8 < kChunk * DK / 8; e8 += kIntraThreads - 4 * kWave) {
        if (e8 < 0) break;
        const int tl = e8 / kWave, ln = e8 % kWave;
        const int r = 16 * (tl / KS) + ln % 16, i0 = 32 * (tl % KS) + 8 * (ln / 16);
        const bf16x8 *src = reinterpret_cast<const bf16x8 *>(&L.Q[r][i0]);
        const bf16x8 h8 = src[0], l8 = src[1];
        float f[8], x[8];
        lds8(&L.Fq[r / 16][i0], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = ((float)h8[e] + (float)l8[e]) * f[e];
        const Split8 sx = split8p(x);
        const size_t o = gh * kChunk * DK + (size_t)8 * e8;   // = opnd_off<DK>(r, i0)
        *reinterpret_cast<bf16x8 *>(ws.Q_hi + o) = sx.hi;
        *reinterpret_cast<bf16x8 *>(ws.Q_lo + o) = sx.lo;
    }
    for (int e8 = tid - 4 * kWave; e8 < kChunk * DK / 8; e8 += kIntraThreads - 4 * kWave) {
        if (e8 < 0) break;
        const int tl = e8 / kWave, ln = e8 % kWave;
        const int i = 16 * (tl / 2) + ln % 16, r0 = 32 * (tl % 2) + 8 * (ln / 16);
        const float fk = L.Fk[r0 / 16][i];
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = L.G[r0 + e][i] * fk;   // k^ rows past n are zero
        const Split8 sx = split8p(x);
        const size_t o = gh * DK * kChunk + (size_t)8 * e8;   // = opnd_off<kChunk>(i, r0)
        *reinterpret_cast<bf16x8 *>(ws.K_hi + o) = sx.hi;
        *reinterpret_cast<bf16x8 *>(ws.K_lo + o) = sx.lo;
    }
    __syncthreads();

    const int gnext = gidx + wph;
    const bool more = gnext < nchunks;
    int c2 = 0, t02 = 0, n2 = 0;
    const Tin *win2 = win;

    // 5. [W | U~] = (I + A)^-1 R with R = [diag(beta) K^ e^G | diag(beta) V],
    //    by block forward substitution in each wave's 16 columns:
    //    X_b = T_bb (R_b - sum_{m < b} A_bm X_m).  A result tile of
    //    v_mfma_f32_16x16x16_bf16 is laid out as its B operand (lane l: rows
    //    4 (l / 16) .. + 3 of column l % 16), so the blocks chain in
    //    registers.  -W is stored split in operand order, U~ in fp32.
    if (wave >= NCT && more) {   // wave-uniform: no column tile
        locate(gnext, c2, t02, n2, win2);
        issue_rows(c2, t02, n2, win2, lane);
    }
    if (wave < NCT) {   // wave-uniform
        const int ct = wave, col = 16 * ct + lr;
        const bool isw = ct < DK / 16;   // wave-uniform
        // conv (+ SiLU) of v for the U~ columns, as the q and k rows were
        // formed, times beta: the R rows of this lane (the raw inputs die here)
        float ru[4][4];
        if (!isw) {
            const float4 vwt = L.Cv[col - DK];
            const float vw[4] = {vwt.x, vwt.y, vwt.z, vwt.w};
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float a = vw[0] * to_f32(vraw[b][j]);
                    a = fmaf(vw[1], to_f32(vraw[b][j + 1]), a);
                    a = fmaf(vw[2], to_f32(vraw[b][j + 2]), a);
                    a = fmaf(vw[3], to_f32(vraw[b][j + 3]), a);
                    ru[b][j] = L.beta[16 * b + 4 * lk + j] * (p.silu ? silu_hw(a) : a);
                }
        }
        // the next chunk's rows, gates and beta, in flight through the rest
        // of step 5 (issued once the raw v inputs are used: the registers
        // are shared)
        if (more) {
            locate(gnext, c2, t02, n2, win2);
            issue_rows(c2, t02, n2, win2, lane);
        }
        Split4 xs[3];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            f32x4 acc;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int sv = 16 * b + 4 * lk + j;
                float r;
                if (isw) {
                    // beta_s k^_s e^(G_s): the rewritten k row (hi + lo) times
                    // e^(G_r) of its block
                    const __bf16 *kr = reinterpret_cast<const __bf16 *>(&L.K[sv][0]) + 2 * (col & ~7) + (col & 7);
                    r = ((float)kr[0] + (float)kr[8]) * L.Fq[b][col];
                    acc[j] = L.beta[sv] * r;
                } else {
                    acc[j] = ru[b][j];
                }
            }
#pragma unroll
            for (int m = 0; m < b; ++m) {
                Split4 na;
                na.hi = *reinterpret_cast<const s16x4 *>(&L.NAh[16 * b + lr][16 * m + 4 * lk]);
                na.lo = *reinterpret_cast<const s16x4 *>(&L.NAl[16 * b + lr][16 * m + 4 * lk]);
                acc = mma3k16(na, xs[m], acc);
            }
            float y4[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) y4[j] = acc[j];
            Split4 tt;
            tt.hi = *reinterpret_cast<const s16x4 *>(&L.Th[b][lr][4 * lk]);
            tt.lo = *reinterpret_cast<const s16x4 *>(&L.Tl[b][lr][4 * lk]);
            const f32x4 x = mma3k16(tt, split4(y4), f32x4{0.f, 0.f, 0.f, 0.f});
            if (b < 3) {
                float x4[4] = {x[0], x[1], x[2], x[3]};
                xs[b] = split4(x4);
            }
            if (isw) {
                store_tile_split<DK>(L.D[wave], -x, lane, ws.Wn_hi + gh * kChunk * DK, ws.Wn_lo + gh * kChunk * DK,
                                     16 * b, 16 * ct);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    ws.Ut[gh * kChunk * DV + (16 * b + 4 * lk + j) * DV + (col - DK)] = x[j];
            }
        }
    }
    if (!more) break;
    __syncthreads();   // the next chunk's step 1 rewrites what step 5 reads
    gidx = gnext;
    c = c2;
    t0 = t02;
    n = n2;
    win = win2;
    }
}

// ---------------------------------------------------------------------------
// scan: persistent workgroups, each taking one (sequence, head, CB state
// columns) item at a time, two teams of 4 waves.  Team 0 computes the even
// chunks and team 1 the odd ones; while one team computes a chunk, the other
// loads the operands of the next one into its registers, so the operand
// traffic (bound by the L1's outstanding-miss capacity) runs under the other
// team's MFMA work.  Inside a team, wave w owns rows 16w..16w+15 of the chunk
// and state row tiles TS*w .. TS*w+TS-1; all products run on MFMA in bf16x3
// with fp32 accumulation.  The state is handed from team to team through LDS
// (two buffers).
//
// Outputs with 16-column blocks: the RMSNorm of a row of O needs all d_v
// columns, which the d_v / 16 workgroups of a (sequence, head) hold between
// them.  Each wave keeps its 16 rows of O of the team's last two chunks in
// LDS (4 consecutive columns per lane) and publishes, for every row, the sum
// of squares of its 16 columns into the chunk's exchange slots (marked empty
// by the intra kernel) with relaxed device-scope atomic stores.  Two team
// chunks later it reads the row's d_v / 16 slots of that chunk with relaxed
// device-scope atomic loads until none is empty: each slot is written once
// per call, so a value that is not the empty mark is the final one, and no
// fence is needed.  The row sum adds the slots as a pairwise tree (the same
// bits in every workgroup); then the rows are scaled, weighted, gated and
// stored.  The workgroups of one (sequence, head) must run at the same time:
// items are ordered so that its d_v / CB items are 8 apart inside an aligned
// run of 8 d_v / CB items (all on one XCD, as workgroups go to XCDs
// round-robin), and the grid is a multiple of that run and at most one
// workgroup per CU.  The wait is bounded: if it ever runs out (other work
// holding compute units), the wave waits no more, stores its rows of that and
// its later chunks unnormalised and marks them; the repair kernel after the
// scan normalises them with the same arithmetic.  With 64-column blocks the
// LDS is full:
// the scan writes O and the norm kernel below normalises it with the same
// arithmetic (both give the same bits).
// ---------------------------------------------------------------------------
constexpr int kScanThreads = 512;
template <typename Tin> struct Vec4 {
    typedef Tin T __attribute__((ext_vector_type(4)));
};
typedef float v4f __attribute__((ext_vector_type(4)));

// RMSNorm arithmetic shared by the scan's in-place normalisation (16-column
// blocks) and the norm kernel (64-column blocks), so both give the same bits:
// a lane holds 4 consecutive columns of a row and a quad of lanes one
// 16-column tile.  The tile's sum of squares: the lane's columns in order,
// then the quad's lanes as (0 + 1) + (2 + 3).  The row's sum adds the tiles
// as a pairwise tree, ((0 + 1) + (2 + 3)) + ((4 + 5) + (6 + 7)).
__device__ __forceinline__ float tile_sumsq(v4f y) {
    float s = y.x * y.x;
    s = fmaf(y.y, y.y, s);
    s = fmaf(y.z, y.z, s);
    s = fmaf(y.w, y.w, s);
    s = dpp_add<0xB1, 0xF>(s);      // quad_perm [1,0,3,2]
    return dpp_add<0x4E, 0xF>(s);   // quad_perm [2,3,0,1]
}
// y / sqrt(mean(y^2) + eps) * (w * sigmoid(z)) for the lane's 4 columns:
// the gate factors g = w * sigmoid(z), then the row's scale
__device__ __forceinline__ float sigmoid_hw(float x) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
}
template <typename Tin>
__device__ __forceinline__ v4f gate4(v4f w, typename Vec4<Tin>::T z) {
    return v4f{w.x * sigmoid_hw(to_f32(z[0])), w.y * sigmoid_hw(to_f32(z[1])), w.z * sigmoid_hw(to_f32(z[2])),
               w.w * sigmoid_hw(to_f32(z[3]))};
}
template <int DV>
__device__ __forceinline__ v4f rms_apply(v4f y, float ss, float eps, v4f g) {
    const float rn = __builtin_amdgcn_rsqf(ss * (1.0f / DV) + eps);
    return v4f{y.x * rn * g.x, y.y * rn * g.y, y.z * rn * g.z, y.w * rn * g.w};
}
// Polls of the exchange slots before a wave stops waiting (each a sleep and
// a load, ~1.5 us: about 25 ms in all, thousands of times the usual wait of
// a few chunks; rows left then are finished by the repair kernel)
constexpr int kXpSpin = 1 << 14;

template <int DK, int NCB>
struct ScanOps {
    static constexpr int KS = DK / 32, TS = DK / 64;
    Split8 w[KS];          // -W rows (A operand, K = d_k), pre-split
    Split8 q[KS];          // Q^ e^G rows
    Split8 pm[2];          // P rows (K = token)
    Split8 kd[TS][2];      // Kd^T rows (K = token)
    float ut[NCB][4];      // U~ of each 16-column tile (result layout)
    float gc[TS][4];       // e^(G_C) of the state rows this lane updates
};

__device__ __forceinline__ Split8 load_split8(const uint16_t *hi, const uint16_t *lo, size_t off) {
    Split8 v;
    v.hi = *reinterpret_cast<const bf16x8 *>(hi + off);
    v.lo = *reinterpret_cast<const bf16x8 *>(lo + off);
    return v;
}

// first half of a chunk's operands: the d_k-contraction rows (-W, Q^ e^G)
// and the P rows
template <int DK, int NCB>
__device__ __forceinline__ void scan_load_a(const PrefillWs &ws, size_t gh, int w4, int lr, int lk,
                                            ScanOps<DK, NCB> &o) {
    constexpr int KS = DK / 32;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        const size_t rw = gh * kChunk * DK + opnd_off<DK>(16 * w4 + lr, 32 * k + 8 * lk);
        o.w[k] = load_split8(ws.Wn_hi, ws.Wn_lo, rw);
        o.q[k] = load_split8(ws.Q_hi, ws.Q_lo, rw);
    }
#pragma unroll
    for (int k = 0; k < 2; ++k)   // rows below 32 have P = 0 in tokens 32..63
        if (w4 >= 2 || k == 0)
            o.pm[k] = load_split8(ws.P_hi, ws.P_lo, gh * kChunk * kChunk + opnd_off<kChunk>(16 * w4 + lr, 32 * k + 8 * lk));
}

// second half: Kd^T, U~ and e^(G_C)
template <int DK, int DV, int NCB>
__device__ __forceinline__ void scan_load_b(const PrefillWs &ws, size_t gh, int w4, int lr, int lk, int j0,
                                            ScanOps<DK, NCB> &o) {
    constexpr int TS = DK / 64;
#pragma unroll
    for (int m = 0; m < TS; ++m) {
#pragma unroll
        for (int k = 0; k < 2; ++k)
            o.kd[m][k] = load_split8(ws.K_hi, ws.K_lo,
                                     gh * DK * kChunk + opnd_off<kChunk>(16 * (TS * w4 + m) + lr, 32 * k + 8 * lk));
#pragma unroll
        for (int r = 0; r < 4; ++r) o.gc[m][r] = ws.gC[gh * DK + 16 * (TS * w4 + m) + 4 * lk + r];
    }
#pragma unroll
    for (int ct = 0; ct < NCB; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            o.ut[ct][r] = ws.Ut[gh * kChunk * DV + (16 * w4 + 4 * lk + r) * DV + j0 + 16 * ct + lr];
}

template <int DK, int DV, typename Tin, int CB>
__global__ __launch_bounds__(kScanThreads) void kda_prefill_scan_kernel(PrefillParams p, PrefillWs ws) {
    constexpr int CH = 2 * DK + DV, KS = DK / 32, TS = DK / 64, NCB = CB / 16, NZ = DV / CB, NT = DV / 16;
    // 16-column blocks normalise their outputs in place (row sums exchanged);
    // 64-column blocks write O and the norm kernel follows (no LDS to spare)
    constexpr bool FUSE = CB == kColBlock;
    static_assert(CH <= kScanThreads, "one thread per conv channel");
    // S in fp32 (two buffers) and, for the MFMA B operands, S and U split into
    // bf16 hi / lo and transposed (a lane's 8 consecutive rows are one 16-byte
    // read); rows padded by 8 to spread the transposed 2-byte writes over banks
    __shared__ __align__(16) float S[2][DK][CB];
    __shared__ __align__(16) __bf16 Sh[2][CB][DK + 8], Sl[2][CB][DK + 8];
    __shared__ __align__(16) __bf16 Uh[CB][kChunk + 8], Ul[CB][kChunk + 8];
    // per wave: its 16 rows of O of the team's last two chunks (by the team's
    // chunk count mod 2), written in the MFMA result layout, read as 4
    // consecutive columns per lane
    __shared__ __align__(16) float Yst[FUSE ? kScanThreads / kWave : 1][2][16][CB + 4];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int team = wave / 4, w4 = wave % 4;
    const int lr = lane % 16, lk = lane / 16;
    const int H = p.H, H8 = (H + 7) / 8;
    // false once a wait for the exchange ran out (a negative bound: at once)
    bool xp_live = ws.xp_spin >= 0;
    if (ws.meta[0] != 1) {
        // tables that failed validation: every output row is zero
        v4f *y4 = reinterpret_cast<v4f *>(p.y);
        const size_t n4 = (size_t)p.total_T * H * DV / 4;
        for (size_t e = (size_t)blockIdx.x * kScanThreads + tid; e < n4; e += (size_t)gridDim.x * kScanThreads)
            y4[e] = v4f{0.f, 0.f, 0.f, 0.f};
        return;
    }
    // persistent: item hl + 8 (zb + NZ (h8 + H8 k)) is head 8 h8 + hl, column
    // block zb of the k-th chunk-path sequence (counted on the device);
    // workgroup w takes items w, w + grid, ...  (a batch of one-token rows
    // costs one exit per workgroup, not one per item)
    const int nitems = 8 * NZ * H8 * ws.meta[p.N_seq + 2];
    for (int item = (int)blockIdx.x; item < nitems; item += (int)gridDim.x) {
    const int hl = item % 8, zb = (item / 8) % NZ, rest = item / (8 * NZ);
    const int h = 8 * (rest % H8) + hl, k = rest / H8, j0 = zb * CB;
    if (h >= H) continue;   // heads padded to a multiple of 8
    const int s = ws.meta[p.N_seq + 3 + k];
    const int slot = p.slot_idx[s];
    if (!slot_ok(slot, p.n_slots)) continue;
    const int32_t *cs = ws.meta + 1;
    const int g0 = cs[s], nch = cs[s + 1] - cs[s];
    const int len = p.cu_seqlens[s + 1] - p.cu_seqlens[s];
    if (len == 1) continue;   // a one-token sequence: decode kernel (state, window, output)

    // the window after the sequence: the last 3 raw inputs (older rows from
    // the previous window when len < 3); read everything, then write
    if (zb == 0) {
        Tin *win = static_cast<Tin *>(p.window) + ((size_t)slot * H + h) * 3 * CH;
        const int ch = tid;
        Tin nv[3];
        if (ch < CH) {
            const Tin *src;
            int stride, off;
            if (ch < DK) { src = static_cast<const Tin *>(p.x_q); stride = DK; off = ch; }
            else if (ch < 2 * DK) { src = static_cast<const Tin *>(p.x_k); stride = DK; off = ch - DK; }
            else { src = static_cast<const Tin *>(p.x_v); stride = DV; off = ch - 2 * DK; }
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const int q = len + j - 3;   // sequence position of new row j
                nv[j] = q >= 0 ? src[((size_t)(p.cu_seqlens[s] + q) * H + h) * stride + off]
                               : win[(q + 3) * CH + ch];
            }
        }
        __syncthreads();
        if (ch < CH) {
#pragma unroll
            for (int j = 0; j < 3; ++j) win[j * CH + ch] = nv[j];
            // checkpoint windows: the three raw inputs before each checkpoint
            // position (every position is >= 64, so all rows are inputs)
            const int nck = p.ckpt_slots ? min(p.ckpt_per_seq, len / p.ckpt_interval) : 0;
            for (int j = 0; j < nck; ++j) {
                const int ck = p.ckpt_slots[(size_t)s * p.ckpt_per_seq + j];
                if (!slot_ok(ck, p.n_slots)) continue;
                const Tin *src;
                int stride, off;
                if (ch < DK) { src = static_cast<const Tin *>(p.x_q); stride = DK; off = ch; }
                else if (ch < 2 * DK) { src = static_cast<const Tin *>(p.x_k); stride = DK; off = ch - DK; }
                else { src = static_cast<const Tin *>(p.x_v); stride = DV; off = ch - 2 * DK; }
                Tin *cw = static_cast<Tin *>(p.window) + ((size_t)ck * H + h) * 3 * CH;
                const int pos = (j + 1) * p.ckpt_interval;
#pragma unroll
                for (int r = 0; r < 3; ++r)
                    cw[r * CH + ch] = src[((size_t)(p.cu_seqlens[s] + pos - 3 + r) * H + h) * stride + off];
            }
        }
    }

    float *Sg = p.state + ((size_t)slot * H + h) * DK * DV;
    for (int e = tid; e < DK * CB; e += kScanThreads) {
        const int row = e / CB, col = e % CB;
        const float x = Sg[row * DV + j0 + col];
        const __bf16 hb = (__bf16)x;
        S[0][row][col] = x;
        Sh[0][col][row] = hb;
        Sl[0][col][row] = (__bf16)(x - (float)hb);
    }

    // bf16x3 product with the three partial products in separate
    // accumulators (short dependency chains), summed at the end
    struct Acc3 {
        f32x4 hh, hl, lh;
    };
    auto zero3 = [](Acc3 &a) {
        a.hh = f32x4{0.f, 0.f, 0.f, 0.f};
        a.hl = a.hh;
        a.lh = a.hh;
    };
    auto mma3s = [](const Split8 &x, const Split8 &y, Acc3 &a) {
        a.hh = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x.hi, y.hi, a.hh, 0, 0, 0);
        a.hl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x.hi, y.lo, a.hl, 0, 0, 0);
        a.lh = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x.lo, y.hi, a.lh, 0, 0, 0);
    };
    auto sum3 = [](const Acc3 &a, int r) { return a.hh[r] + (a.hl[r] + a.lh[r]); };

    const int seq_t0 = p.cu_seqlens[s], seq_t1 = p.cu_seqlens[s + 1];
    // in-place RMSNorm (16-column blocks): the lane's row of the wave's 16
    // (rho) and columns 4 qd .. 4 qd + 3 of each 16-column tile
    const int rho = lane / 4, qd = lane % 4;
    using ZT = typename Vec4<Tin>::T;
    v4f nw[NCB];   // the norm weights of those columns
    if constexpr (FUSE) {
#pragma unroll
        for (int ct = 0; ct < NCB; ++ct) nw[ct] = *reinterpret_cast<const v4f *>(p.norm_w + h * DV + j0 + 16 * ct + 4 * qd);
    }
    // the team's two previous chunks, older first (-1: none); their rows of O
    // wait in the wave's scratch
    int pc1 = -1, pc2 = -1;
    // the first of the team's chunks whose rows the wave left unnormalised
    // (-1: none); every later one of the item is left too
    int miss = -1;
    // The older one's RMSNorm in two steps: fin_issue requests the gate inputs and the
    // row-sum slots (the quad of the row reads PL slots per lane), fin_done
    // waits until no slot is empty and stores the results.  The chunk's own
    // products run in between.
    constexpr int PL = NT / 4;
    struct Fin {
        ZT z[NCB];
        uint64_t sl;
        const uint32_t *src;
    };
    auto fin_src = [&](int cc) {
        return ws.Xp + (((size_t)(g0 + cc) * H + h) * kChunk + 16 * w4 + rho) * NT + PL * qd;
    };
    auto poll = [&](const uint32_t *src) -> uint64_t {
        if constexpr (PL == 2)
            return __hip_atomic_load(reinterpret_cast<const uint64_t *>(src), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else   // (the second word a stand-in that is never empty)
            return (uint64_t)__hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) |
                   ((uint64_t)0x7FC00000u << 32);
    };
    auto fin_issue = [&](int cc, Fin &f) {
        const int t0c = seq_t0 + cc * kChunk, nc = min(kChunk, seq_t1 - t0c);
        const size_t row = (size_t)(t0c + min(16 * w4 + rho, nc - 1)) * H + h;
#pragma unroll
        for (int ct = 0; ct < NCB; ++ct)
            f.z[ct] = *reinterpret_cast<const ZT *>(static_cast<const Tin *>(p.z) + row * DV + j0 + 16 * ct + 4 * qd);
        f.src = fin_src(cc);
        f.sl = poll(f.src);
    };
    auto fin_done = [&](int cc, Fin &f) {
        const int t0c = seq_t0 + cc * kChunk, nc = min(kChunk, seq_t1 - t0c);
        // the gate factors and the lane's rows of O do not wait for the sums
        v4f gz[NCB], yo[NCB];
#pragma unroll
        for (int ct = 0; ct < NCB; ++ct) {
            gz[ct] = gate4<Tin>(nw[ct], f.z[ct]);
            yo[ct] = *reinterpret_cast<const v4f *>(&Yst[wave][(cc / 2) & 1][rho][16 * ct + 4 * qd]);
        }
        auto full = [](uint64_t v) { return (uint32_t)v != kXpEmpty && (uint32_t)(v >> 32) != kXpEmpty; };
        // (a wave vote: one path for all lanes; once a wait runs out, this
        // chunk's rows and those of the wave's later chunks stay unnormalised)
        for (int tries = 0; xp_live && !__all(full(f.sl)); ++tries) {
            xp_live = tries < ws.xp_spin;
            __builtin_amdgcn_s_sleep(8);
            f.sl = poll(f.src);
        }
        const bool got = xp_live && __all(full(f.sl));
        if (!got && miss < 0) miss = cc;
        // the row's sum over its tiles, in the tree order, on its quad
        float a = __uint_as_float((uint32_t)f.sl);
        if (PL == 2) a += __uint_as_float((uint32_t)(f.sl >> 32));
        a = dpp_add<0xB1, 0xF>(a);   // quad_perm [1,0,3,2]
        a = dpp_add<0x4E, 0xF>(a);   // quad_perm [2,3,0,1]
        const int t = 16 * w4 + rho;
        if (t < nc) {
#pragma unroll
            for (int ct = 0; ct < NCB; ++ct)
                __builtin_nontemporal_store(got ? rms_apply<DV>(yo[ct], a, p.rms_eps, gz[ct]) : yo[ct],
                                            reinterpret_cast<v4f *>(p.y + ((size_t)(t0c + t) * H + h) * DV + j0 +
                                                                    16 * ct + 4 * qd));
        }
    };
    ScanOps<DK, NCB> ops;
    if (team == 0 && nch > 0) {
        scan_load_a<DK, NCB>(ws, (size_t)g0 * H + h, w4, lr, lk, ops);
        scan_load_b<DK, DV, NCB>(ws, (size_t)g0 * H + h, w4, lr, lk, j0, ops);
    }
    __syncthreads();
    Acc3 ao[NCB];
    for (int c = 0; c < nch; ++c) {
        const int cur = c & 1;
        const bool mine = cur == team;            // wave-uniform
        const size_t gnext = (size_t)(g0 + c + 1) * H + h;
        // segment 1: U = U~ - W S and O = Q^e^G S  |  the other team loads
        if (mine) {
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this chunk's operands have landed
#pragma unroll
            for (int ct = 0; ct < NCB; ++ct) {
                const int cl = 16 * ct + lr;   // this lane's state column in the block
                Split8 sb[KS];
#pragma unroll
                for (int k = 0; k < KS; ++k) {
                    sb[k].hi = *reinterpret_cast<const bf16x8 *>(&Sh[cur][cl][32 * k + 8 * lk]);
                    sb[k].lo = *reinterpret_cast<const bf16x8 *>(&Sl[cur][cl][32 * k + 8 * lk]);
                }
                Acc3 au;
                zero3(au);
                zero3(ao[ct]);
#pragma unroll
                for (int k = 0; k < KS; ++k) {
                    mma3s(ops.w[k], sb[k], au);
                    mma3s(ops.q[k], sb[k], ao[ct]);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float u = ops.ut[ct][r] + sum3(au, r);
                    const __bf16 hb = (__bf16)u;
                    Uh[cl][16 * w4 + 4 * lk + r] = hb;
                    Ul[cl][16 * w4 + 4 * lk + r] = (__bf16)(u - (float)hb);
                }
            }
        } else if (c + 1 < nch) {
            scan_load_a<DK, NCB>(ws, gnext, w4, lr, lk, ops);
        }
        __syncthreads();
        // segment 2: O += P U, S' = diag(e^G_C) S + Kd^T U  |  the other team loads
        if (mine) {
            const size_t ghc = (size_t)(g0 + c) * H + h;
            const int t0 = seq_t0 + c * kChunk;
            const int n = min(kChunk, seq_t1 - t0);
            // the team's chunk before last: its inputs requested now, its rows
            // finished after this chunk's products (their sums are in by then,
            // as a rule).  The operands landed before segment 1; saying so
            // here keeps the compiler from waiting for these new loads before
            // the products (it cannot tell that the loads of the other team's
            // branch are not pending on this one).
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
            Fin f;
            if (FUSE && pc1 >= 0) fin_issue(pc1, f);
            float yv[NCB][4];
#pragma unroll
            for (int ct = 0; ct < NCB; ++ct) {
                const int cl = 16 * ct + lr;
                Split8 ub[2];
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    ub[k].hi = *reinterpret_cast<const bf16x8 *>(&Uh[cl][32 * k + 8 * lk]);
                    ub[k].lo = *reinterpret_cast<const bf16x8 *>(&Ul[cl][32 * k + 8 * lk]);
                }
                // P rows beyond the chunk and above the diagonal are 0
#pragma unroll
                for (int k = 0; k < 2; ++k)
                    if (w4 >= 2 || k == 0) mma3s(ops.pm[k], ub[k], ao[ct]);
#pragma unroll
                for (int m = 0; m < TS; ++m) {
                    Acc3 as;
                    zero3(as);
#pragma unroll
                    for (int k = 0; k < 2; ++k) mma3s(ops.kd[m][k], ub[k], as);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = 16 * (TS * w4 + m) + 4 * lk + r;
                        const float x = ops.gc[m][r] * S[cur][row][cl] + sum3(as, r);
                        const __bf16 hb = (__bf16)x;
                        S[cur ^ 1][row][cl] = x;
                        Sh[cur ^ 1][cl][row] = hb;
                        Sl[cur ^ 1][cl][row] = (__bf16)(x - (float)hb);
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) yv[ct][r] = sum3(ao[ct], r);
            }
            if constexpr (FUSE) {
                // (the previous chunk finishes before this one's stores: with
                // no store issued after its loads, the wait for them is exact)
                if (pc1 >= 0) fin_done(pc1, f);
                pc1 = pc2;   // this chunk's rows wait for the team's chunk after next
                pc2 = c;
                // into the wave's scratch (the slot just finished: its reads
                // by other lanes come first); each quad's tile sum of squares
                // into the exchange
                const int sb = (c / 2) & 1;
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
                for (int ct = 0; ct < NCB; ++ct)
#pragma unroll
                    for (int r = 0; r < 4; ++r) Yst[wave][sb][4 * lk + r][16 * ct + lr] = yv[ct][r];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
                for (int ct = 0; ct < NCB; ++ct) {
                    const float ps = tile_sumsq(*reinterpret_cast<const v4f *>(&Yst[wave][sb][rho][16 * ct + 4 * qd]));
                    const uint32_t bits = ps != ps ? 0x7FC00000u : __float_as_uint(ps);
                    if (qd == 0)
                        __hip_atomic_store(ws.Xp + (ghc * kChunk + 16 * w4 + rho) * NT + zb * NCB + ct, bits,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            } else {
#pragma unroll
                for (int ct = 0; ct < NCB; ++ct)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = 16 * w4 + 4 * lk + r;
                        if (t < n) p.y[((size_t)(t0 + t) * H + h) * DV + j0 + 16 * ct + lr] = yv[ct][r];
                    }
            }
        } else if (c + 1 < nch) {
            scan_load_b<DK, DV, NCB>(ws, gnext, w4, lr, lk, j0, ops);
        }
        __syncthreads();
        // interval checkpoint: the state after this chunk is in S[(c + 1) & 1],
        // which is not written again before two more barriers
        if (p.ckpt_slots) {
            const int pos = min((c + 1) * kChunk, len);
            const int j = pos / p.ckpt_interval - 1;
            if (pos % p.ckpt_interval == 0 && j < p.ckpt_per_seq) {
                const int ck = p.ckpt_slots[(size_t)s * p.ckpt_per_seq + j];
                if (slot_ok(ck, p.n_slots)) {
                    float *D = p.state + ((size_t)ck * H + h) * DK * DV;
                    const int nxt = (c + 1) & 1;
                    for (int e = tid; e < DK * CB; e += kScanThreads)
                        D[(e / CB) * DV + j0 + e % CB] = S[nxt][e / CB][e % CB];
                } else if (ck != -1 && tid == 0 && zb == 0) {
                    flag_error(p.err_flag);
                }
            }
        }
    }
    if (FUSE) {   // each team's last two chunks
        for (int i = 0; i < 2; ++i) {
            const int cc = i ? pc2 : pc1;
            if (cc >= 0) {
                Fin f;
                fin_issue(cc, f);
                fin_done(cc, f);
            }
        }
        if (miss >= 0 && lane == 0) {
            // rows whose sums did not come in time stay unnormalised: the
            // wave's rows in chunks miss, miss + 2, ... to the end of the
            // sequence, marked for the repair kernel (which runs after this
            // one, when every sum is in); the marks are stored here, not in
            // the chunk loop, so that its waits for loads stay loose
#pragma unroll
            for (int ct = 0; ct < NCB; ++ct)
                ws.Xf[(((size_t)(g0 + miss) * H + h) * NT + zb * NCB + ct) * 4 + w4] = 1;
            ws.meta[2 * p.N_seq + 4] = 1;
        }
    }
    const int fin = nch & 1;
    for (int e = tid; e < DK * CB; e += kScanThreads) Sg[(e / CB) * DV + j0 + e % CB] = S[fin][e / CB][e % CB];
    __syncthreads();   // the next item's state load rewrites S
    }
    // rows of sequences that no kernel computes (padding, a bad slot) are zero
    for (int sq = (int)(blockIdx.x * kScanThreads) + tid; sq < p.N_seq; sq += (int)(gridDim.x * kScanThreads)) {
        const int a0 = p.cu_seqlens[sq], a1 = p.cu_seqlens[sq + 1];
        if (a1 > a0 && !slot_ok(p.slot_idx[sq], p.n_slots)) {
            v4f *d = reinterpret_cast<v4f *>(p.y + (size_t)a0 * H * DV);
            for (size_t e = 0; e < (size_t)(a1 - a0) * H * DV / 4; ++e) d[e] = v4f{0.f, 0.f, 0.f, 0.f};
        }
    }
}

// ---------------------------------------------------------------------------
// norm (after the scan with 64-column blocks): y = O / sqrt(mean(O^2) + eps)
// * w * sigmoid(z) over rows r = t*H + h of y (contiguous), with the scan's
// in-place arithmetic (tile sums, then the tiles as a pairwise tree).  A lane
// holds 4 consecutive columns, a row spans d_v/4 lanes (a wave covers 2 rows
// at d_v = 128, 4 at d_v = 64); a workgroup walks kNormRows consecutive rows.
// ---------------------------------------------------------------------------
constexpr int kNormRows = 64;

template <int DV, typename Tin>
__global__ __launch_bounds__(256) void kda_prefill_norm_kernel(PrefillParams p, PrefillWs ws) {
    constexpr int LPR = DV / 4, RPW = kWave / LPR, RPB = 4 * RPW;   // lanes per row, rows per wave / block pass
    constexpr int NP = kNormRows / RPB;                               // passes, all loads issued first
    using ZT = typename Vec4<Tin>::T;
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int H = p.H, c0 = 4 * (lane % LPR);
    const size_t nrows = (size_t)p.total_T * H;
    const bool valid = ws.meta[0] == 1;
    const bool ones = ws.meta[2 * p.N_seq + 3] > 0;   // any rows already final
    v4f o[NP];
    ZT zr[NP];
    size_t rr[NP];
    bool in[NP];
#pragma unroll
    for (int pass = 0; pass < NP; ++pass) {
        const size_t r = (size_t)blockIdx.x * kNormRows + pass * RPB + wave * RPW + lane / LPR;
        in[pass] = r < nrows;
        rr[pass] = in[pass] ? r : 0;
        // y is read once and rewritten: streamed past the caches
        o[pass] = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(p.y + rr[pass] * DV + c0));
        zr[pass] = *reinterpret_cast<const ZT *>(static_cast<const Tin *>(p.z) + rr[pass] * DV + c0);
    }
#pragma unroll
    for (int pass = 0; pass < NP; ++pass) {
        const int t = (int)(rr[pass] / H), h = (int)(rr[pass] % H);
        bool live = in[pass] && valid, done = false;
        if (live) {
            const int sq = p.N_seq == 1 ? 0 : upper_index(p.cu_seqlens, p.N_seq + 1, t);
            live = slot_ok(p.slot_idx[sq], p.n_slots);
            // rows of one-token sequences are already final (decode kernel)
            if (ones) done = live && p.cu_seqlens[sq + 1] - p.cu_seqlens[sq] == 1;
        }
        // tile sums (quads), then the tiles pairwise: quads 4 and 8 (and 16) lanes apart
        float ss = tile_sumsq(o[pass]);
        ss += __shfl_xor(ss, 4, kWave);
        ss += __shfl_xor(ss, 8, kWave);
        if (LPR == 32) ss += __shfl_xor(ss, 16, kWave);
        const v4f w = *reinterpret_cast<const v4f *>(p.norm_w + h * DV + c0);
        v4f out = rms_apply<DV>(o[pass], ss, p.rms_eps, gate4<Tin>(w, zr[pass]));
        if (!live) out = v4f{0.f, 0.f, 0.f, 0.f};
        if (in[pass] && !done) __builtin_nontemporal_store(out, reinterpret_cast<v4f *>(p.y + rr[pass] * DV + c0));
    }
}

// ---------------------------------------------------------------------------
// repair (after the 16-column scan): rows whose row sums did not reach their
// wave in time (other work holding compute units, so that a group's
// workgroups did not all run at once) were stored unnormalised, and the wave
// marked the first chunk it left so.  Once the scan has ended every sum is
// in, so they are normalised here with the scan's arithmetic (the same bits).
// Without marks the workgroups exit at once.
// ---------------------------------------------------------------------------
constexpr int kRepairBlocks = 64;

template <int DV, typename Tin>
__global__ __launch_bounds__(256) void kda_prefill_repair_kernel(PrefillParams p, PrefillWs ws) {
    constexpr int NT = DV / 16, PL = NT / 4;
    using ZT = typename Vec4<Tin>::T;
    if (ws.meta[0] != 1 || ws.meta[2 * p.N_seq + 4] == 0) return;
    const int lane = threadIdx.x % kWave, H = p.H;
    const int32_t *cs = ws.meta + 1;
    const size_t nmarks = (size_t)cs[p.N_seq] * H * NT * 4;
    const size_t nwaves = (size_t)gridDim.x * (blockDim.x / kWave);
    const int rho = lane / 4, qd = lane % 4;
    // mark e = ((g H + h) NT + tile) 4 + w4: rows 16 w4 .. + 15 of head h,
    // columns 16 tile .. + 15, in chunk slot g and every second chunk after it
    // in its sequence; a mark per wave, a lane taking row 16 w4 + lane / 4 and
    // 4 columns as in the scan
    for (size_t e = (size_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave; e < nmarks; e += nwaves) {
        if (ws.Xf[e] == 0) continue;   // the same word on every lane
        const int w4 = (int)(e % 4), tile = (int)((e / 4) % NT);
        const int g = (int)(e / (4 * NT) / H), h = (int)(e / (4 * NT) % H);
        const int sq = upper_index(cs, p.N_seq + 1, g);
        const int t = 16 * w4 + rho;
        for (int gc = g; gc < cs[sq + 1]; gc += 2) {
            const int t0 = p.cu_seqlens[sq] + (gc - cs[sq]) * kChunk, n = min(kChunk, p.cu_seqlens[sq + 1] - t0);
            const uint32_t *src = ws.Xp + (((size_t)gc * H + h) * kChunk + t) * NT + PL * qd;
            float a = __uint_as_float(src[0]);
            if (PL == 2) a += __uint_as_float(src[1]);
            a = dpp_add<0xB1, 0xF>(a);   // quad_perm [1,0,3,2]
            a = dpp_add<0x4E, 0xF>(a);   // quad_perm [2,3,0,1]
            if (t < n) {
                const size_t off = ((size_t)(t0 + t) * H + h) * DV + 16 * tile + 4 * qd;
                const v4f y = *reinterpret_cast<const v4f *>(p.y + off);
                const v4f w = *reinterpret_cast<const v4f *>(p.norm_w + h * DV + 16 * tile + 4 * qd);
                const ZT z = *reinterpret_cast<const ZT *>(static_cast<const Tin *>(p.z) + off);
                *reinterpret_cast<v4f *>(p.y + off) = rms_apply<DV>(y, a, p.rms_eps, gate4<Tin>(w, z));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
template <int DK, int DV, typename Tin>
static kda_status launch_prefill_typed(const PrefillParams &p, hipStream_t stream) {
    const WsLayout l = ws_layout(p.H, DK, DV, p.total_T, p.N_seq);
    unsigned char *base = static_cast<unsigned char *>(p.workspace);
    PrefillWs ws{};
    ws.meta = reinterpret_cast<int32_t *>(base + l.meta);
    ws.Wn_hi = reinterpret_cast<uint16_t *>(base + l.Wn_hi);
    ws.Wn_lo = reinterpret_cast<uint16_t *>(base + l.Wn_lo);
    ws.Q_hi = reinterpret_cast<uint16_t *>(base + l.Q_hi);
    ws.Q_lo = reinterpret_cast<uint16_t *>(base + l.Q_lo);
    ws.K_hi = reinterpret_cast<uint16_t *>(base + l.K_hi);
    ws.K_lo = reinterpret_cast<uint16_t *>(base + l.K_lo);
    ws.P_hi = reinterpret_cast<uint16_t *>(base + l.P_hi);
    ws.P_lo = reinterpret_cast<uint16_t *>(base + l.P_lo);
    ws.Ut = reinterpret_cast<float *>(base + l.Ut);
    ws.gC = reinterpret_cast<float *>(base + l.gC);
    ws.Xp = reinterpret_cast<uint32_t *>(base + l.Xp);
    ws.Xf = reinterpret_cast<uint32_t *>(base + l.Xf);
    ws.xp_spin = kXpSpin;
    if (const char *e = getenv("KDA_XP_SPIN")) ws.xp_spin = atoi(e);   // testing: a short bound (negative: no row in time)
    ws.G_max = p.total_T / kChunk + p.N_seq;

    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return KDA_ERR_LAUNCH;
    hipLaunchKernelGGL(kda_prefill_meta_kernel, dim3(1), dim3(64), 0, stream, p, ws);
    if (p.total_T > 0) {
        // one-token sequences (decode rows of a mixed batch) take the decode
        // kernel: one state read and write instead of a chunk's workspace
        // round trip; the chunk kernels below skip them
        RecParams r{};
        r.A = p.A; r.conv_wt = p.conv_wt; r.norm_w = p.norm_w;
        r.q_scale = p.q_scale; r.l2_eps = p.l2_eps; r.rms_eps = p.rms_eps;
        r.silu = p.silu;
        r.state = p.state; r.window = p.window; r.n_slots = p.n_slots;
        r.slot_idx = p.slot_idx;
        r.x_q = p.x_q; r.x_k = p.x_k; r.x_v = p.x_v; r.g = p.g; r.b = p.b; r.z = p.z;
        r.y = p.y;
        r.B = p.N_seq; r.H = p.H; r.T = 1;
        r.seq_start = p.cu_seqlens;
        r.seq_ok = ws.meta;
        // (a single sequence of two or more tokens has no such row)
        if (!(p.N_seq == 1 && p.total_T >= 2)) {
            const kda_status st = launch_recurrent(r, DK, DV, sizeof(Tin) == 2 ? KDA_BF16 : KDA_F32, RecKind::decode,
                                                   stream);
            if (st != KDA_OK) return st;
        }
        // one workgroup per compute unit (the LDS of one), each working
        // through the chunks of one head
        const int wph = std::max(1, std::min(ws.G_max, cus / p.H));
        hipLaunchKernelGGL((kda_prefill_intra_kernel<DK, DV, Tin>), dim3((unsigned)((size_t)p.H * wph)),
                           dim3(kIntraThreads), 0, stream, p, ws);
    }
    // the scan's column blocks: 64 columns per workgroup load the chunk's
    // shared operands once for four times the columns (about 2.4x the
    // columns per CU and second), when the batch has the prompts and heads to
    // fill the GPU with them (by the host's view: enough rows, and on average
    // four chunks per row, so that one-token rows are not counted as
    // prompts); else 16 (a single long prompt: all CUs busy).  The grid: a
    // multiple of the aligned run of 8 d_v / CB items that holds whole
    // (sequence, head) groups, at most one workgroup per CU (all resident at
    // once: a group's workgroups exchange row sums), at least one run.
    const size_t H8 = ((size_t)p.H + 7) / 8;
    auto scan_grid = [&](int nz) {
        const size_t run = 8 * (size_t)nz, items = run * H8 * (size_t)p.N_seq;
        return (unsigned)std::min(items, std::max(run, (size_t)cus / run * run));
    };
    if ((size_t)p.H * (DV / 64) * p.N_seq >= (size_t)cus && (size_t)p.total_T >= (size_t)4 * kChunk * p.N_seq) {
        hipLaunchKernelGGL((kda_prefill_scan_kernel<DK, DV, Tin, 64>), dim3(scan_grid(DV / 64)), dim3(kScanThreads), 0,
                           stream, p, ws);
        if (p.total_T > 0) {
            const size_t rows = (size_t)p.total_T * p.H;
            hipLaunchKernelGGL((kda_prefill_norm_kernel<DV, Tin>), dim3((unsigned)((rows + kNormRows - 1) / kNormRows)),
                               dim3(256), 0, stream, p, ws);
        }
    } else {
        hipLaunchKernelGGL((kda_prefill_scan_kernel<DK, DV, Tin, kColBlock>), dim3(scan_grid(DV / kColBlock)),
                           dim3(kScanThreads), 0, stream, p, ws);
        if (p.total_T > 0)
            hipLaunchKernelGGL((kda_prefill_repair_kernel<DV, Tin>), dim3(kRepairBlocks), dim3(256), 0, stream, p, ws);
    }
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

template <int DK, int DV>
static kda_status launch_prefill_dt(const PrefillParams &p, kda_dtype dt, hipStream_t s) {
    return dt == KDA_BF16 ? launch_prefill_typed<DK, DV, uint16_t>(p, s)
                          : launch_prefill_typed<DK, DV, float>(p, s);
}

kda_status launch_prefill(const PrefillParams &p, int d_k, int d_v, kda_dtype dt, hipStream_t stream) {
    if (d_k == 128 && d_v == 128) return launch_prefill_dt<128, 128>(p, dt, stream);
    if (d_k == 64 && d_v == 64) return launch_prefill_dt<64, 64>(p, dt, stream);
    if (d_k == 128 && d_v == 64) return launch_prefill_dt<128, 64>(p, dt, stream);
    if (d_k == 64 && d_v == 128) return launch_prefill_dt<64, 128>(p, dt, stream);
    return KDA_ERR_UNSUPPORTED;
}

}  // namespace kda
