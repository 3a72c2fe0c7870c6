// kda_recurrent.hip -- token-recurrent KDA kernels for gfx950: fused decode,
// speculative verification with per-token snapshots, and the commit copy.
//
// One workgroup owns one (sequence, head).  Its d_k x d_v fp32 state tile is
// loaded from HBM once, at kernel entry, into registers (float4 per lane,
// d_v contiguous so each wave instruction moves whole 512 B rows), and it is
// written back once.  The delta rule is independent per state column given
// (alpha, beta, k^, v), so the only cross-lane work per token is the
// reduction over the d_k rows for u = S'^T k^ and p = S'^T q^ (wave butterfly
// + one LDS exchange between waves) and the RMSNorm over d_v.
//
// Per token (see include/kda.h for the definition):
//   conv + SiLU of the q|k|v channels (one lane per channel; the window of
//   raw inputs lives in the cache and is shifted in place), L2 norms and the
//   gates (one wave per token), then
//     S' = diag(alpha) S,  u = S'^T k^,  p = S'^T q^          (one pass)
//     d  = beta (v - u),   S = S' + k^ d^T,  o = p + (k^.q^) d  (= S^T q^)
//     y  = o / sqrt(mean(o^2) + eps_r) * w * sigmoid(z)
// Decode and verify instantiate the same code, so verify + commit(L) equals
// L decode launches bit for bit.  Verify keeps either a full state snapshot
// per token, or (delta mode) the token's replay record (alpha, k^, d and the
// raw conv inputs); the delta commit re-applies S = diag(alpha) S + k^ d^T
// with the same fp32 operations, so it reaches the same bits.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// State tile traffic: read once, written once per launch, as float4 at float
// offset row + col of the d_k x d_v tile at `tile` (a workgroup-uniform
// base; row a multiple of d_v, col the lane's column).
// With STREAM the accesses are raw buffer operations carrying the
// non-temporal policy (stores also the device-scope bit sc1), so a working
// set larger than the caches does not thrash them (and a small, re-used one
// is not kept either).  In the buffer form, with sc1 on the stores, a
// batch-64 step over states that miss the Infinity Cache ran 4% faster than
// with non-temporal global loads and stores.  Only the cache policy differs:
// the values are the same.
constexpr int kPolicyNT = 2, kPolicySC1 = 16;   // CDNA3/4 cache-policy bits
constexpr int kBufferWord3 = 0x00020000;        // raw 32-bit buffer resource

template <bool STREAM, int TILE>
__device__ __forceinline__ float4 load_state4(const float *tile, size_t row, int col) {
    if (STREAM) {
        const size_t off = row + col;
        typedef float v4 __attribute__((ext_vector_type(4)));
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(tile), 0, TILE * 4, kBufferWord3);
        const v4 x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off * 4), 0, kPolicyNT);
        return make_float4(x[0], x[1], x[2], x[3]);
    }
    return *reinterpret_cast<const float4 *>(tile + row + col);
}
template <bool STREAM, int TILE>
__device__ __forceinline__ void store_state4(float *tile, size_t row, int col, float4 v) {
    if (STREAM) {
        const size_t off = row + col;
        typedef float v4 __attribute__((ext_vector_type(4)));
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(tile, 0, TILE * 4, kBufferWord3);
        const v4 x = {v.x, v.y, v.z, v.w};
        __builtin_amdgcn_raw_buffer_store_b128(x, r, (int)(off * 4), 0, kPolicyNT | kPolicySC1);
        return;
    }
    *reinterpret_cast<float4 *>(tile + row + col) = v;
}

template <int DK, int DV, int NT>
struct RecGeo {
    static constexpr int CG = DV / 4;      // float4 column groups
    static constexpr int RG = NT / CG;     // row groups
    static constexpr int RPT = DK / RG;    // state rows per lane
    static constexpr int NW = NT / kWave;  // waves per workgroup
    static constexpr int CH = 2 * DK + DV; // conv channels per head
    static_assert(NT % CG == 0 && DK % RG == 0 && RPT >= 1, "tile does not divide");
    static_assert(CG <= kWave && kWave % CG == 0, "a wave must hold whole rows");
};

// Per-token values shared through LDS.  conv[] holds the conv outputs
// q | k | v; the norm pass overwrites q and k with q^ and k^ in place.
// With LR, rows[0..2] hold alpha, k^ and q^ again, ordered for the
// recurrence: the RPT rows a lane owns (rg, rg + RG, ...) are consecutive,
// at rg * RPT, so a lane reads them with 16-byte loads.  Verify launches
// whose grid fits the GPU at once use it (the token chain is then the
// critical path): up to 8 tokens at three workgroups per CU, 16 tokens at
// two (its LDS allows no more).  Larger grids measured slower with the extra
// LDS, and the one-token decode no faster.

template <int DK, int DV, bool LR>
struct alignas(16) TokenLds {
    float rows[LR ? 3 : 1][LR ? DK : 4];
    float conv[2 * DK + DV + 1];   // + 1: sink for lanes without a channel
    float alpha[DK];
    float gate[DV];   // norm_w * sigmoid(z)
    float beta;
    float kq;         // k^ . q^
};

// Replay record of one (sequence, token, head) in delta mode, at byte offset
// ((b*T + t)*H + h) * rec_bytes of the record buffer:
//   float alpha[DK]; float khat[DK]; float d[DV]; Tin x[2*DK + DV]
// (x = the raw, pre-conv inputs q|k|v of the token: the conv window of a
// later commit is rebuilt from them).
template <int DK, int DV, typename Tin>
struct DeltaRec {
    static constexpr int CH = 2 * DK + DV;
    static constexpr int kFloats = 2 * DK + DV;
    static constexpr size_t kBytes = (size_t)CH * (4 + sizeof(Tin));
    static_assert(kBytes % 16 == 0, "records must stay 16-byte aligned");
    __device__ static float *f(void *base, size_t rec) {
        return reinterpret_cast<float *>(static_cast<char *>(base) + rec * kBytes);
    }
    __device__ static const float *f(const void *base, size_t rec) {
        return reinterpret_cast<const float *>(static_cast<const char *>(base) + rec * kBytes);
    }
    __device__ static Tin *x(void *base, size_t rec) {
        return reinterpret_cast<Tin *>(f(base, rec) + kFloats);
    }
    __device__ static const Tin *x(const void *base, size_t rec) {
        return reinterpret_cast<const Tin *>(f(base, rec) + kFloats);
    }
};

// Raw operands of the conv for the channels one lane owns (c = tid + NT*k):
// the tap weights, the three window entries and the T new inputs.
template <int DK, int DV, int NT, typename Tin, int TMAX>
struct ConvRegs {
    static constexpr int CH = 2 * DK + DV;
    static constexpr int CPT = (CH + NT - 1) / NT;
    float4 w[CPT];
    Tin x[CPT][3 + TMAX];
};

// A global-memory pointer that is the same on every lane, held in scalar
// registers and typed as global (address space 1), so loads through it stay
// global loads (a generic pointer would make them flat loads, which the
// compiler can only wait for with a full drain of the load counter).
template <typename T>
using gptr = const __attribute__((address_space(1))) T *;
template <typename T>
__device__ __forceinline__ gptr<T> uniform_ptr(const T *ptr) {
    const uint64_t v = reinterpret_cast<uint64_t>(ptr);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<gptr<T>>(((uint64_t)hi << 32) | lo);
}

// All loads are unconditional (out-of-range channel slots and tokens re-read a
// valid element) so the compiler issues them back to back, ahead of the state
// tile, without branches that would force waits.  Requires T >= 1.
template <int DK, int DV, int NT, typename Tin, int TMAX, bool VERIFY>
__device__ __forceinline__ void conv_fetch(const RecParams &p, int tid, int b, int row, int h, int slot, int T,
                                           ConvRegs<DK, DV, NT, Tin, TMAX> &cr) {
    constexpr int CH = 2 * DK + DV;
    const Tin *win = static_cast<const Tin *>(p.window) + ((size_t)slot * p.H + h) * 3 * CH;
    // the three input bases as wave-uniform (scalar) values: a per-lane
    // choice among the kernel-argument fields themselves would be compiled
    // as a vector load of the pointer, a memory round trip before any input
    // (and the state tile after them) could be requested
    const gptr<Tin> xq = uniform_ptr(static_cast<const Tin *>(p.x_q));
    const gptr<Tin> xk = uniform_ptr(static_cast<const Tin *>(p.x_k));
    const gptr<Tin> xv = uniform_ptr(static_cast<const Tin *>(p.x_v));
#pragma unroll
    for (int k = 0; k < cr.CPT; ++k) {
        const int c = min(tid + NT * k, CH - 1);
        cr.w[k] = *reinterpret_cast<const float4 *>(p.conv_wt + ((size_t)h * CH + c) * 4);
        cr.x[k][0] = win[c];
        cr.x[k][1] = win[CH + c];
        cr.x[k][2] = win[2 * CH + c];
        const bool isq = c < DK, isk = !isq && c < 2 * DK;
        const gptr<Tin> src = isq ? xq : (isk ? xk : xv);
        const int stride = isq || isk ? DK : DV;
        const int off = isq ? c : (isk ? c - DK : c - 2 * DK);
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            const int tt = min(t, T - 1);
            const size_t n = VERIFY ? (size_t)b * p.T + tt : (size_t)row;
            cr.x[k][3 + t] = src[(n * p.H + h) * stride + off];
        }
    }
}

// Conv (+ activation) of the owned channels for every token into LDS; the
// window rows after each token go to the live slot (decode) or to the
// token's snapshot slot (verify); delta mode keeps the raw inputs in the
// token's record instead.
template <int DK, int DV, int NT, typename Tin, int TMAX, bool VERIFY, bool DELTA, bool LR>
__device__ __forceinline__ void conv_compute(const RecParams &p, int tid, int b, int h, int slot, int T,
                                             const ConvRegs<DK, DV, NT, Tin, TMAX> &cr,
                                             TokenLds<DK, DV, LR> *tok) {
    constexpr int CH = 2 * DK + DV;
#pragma unroll
    for (int k = 0; k < cr.CPT; ++k) {
        // computed by every lane (a lane without a channel writes to the sink
        // entry), so no branch separates the loads from their first use
        const int c = tid + NT * k;
        const bool own = c < CH;
        const int cs = own ? c : CH;
        const float4 w = cr.w[k];
#pragma unroll
        for (int t = 0; t < TMAX; ++t) {
            if (t >= T) continue;
            float acc = w.x * to_f32(cr.x[k][t]);
            acc = fmaf(w.y, to_f32(cr.x[k][t + 1]), acc);
            acc = fmaf(w.z, to_f32(cr.x[k][t + 2]), acc);
            acc = fmaf(w.w, to_f32(cr.x[k][t + 3]), acc);
            tok[t].conv[cs] = p.silu ? acc * sigmoid(acc) : acc;
            if (DELTA && own) {
                DeltaRec<DK, DV, Tin>::x(p.delta, ((size_t)b * p.T + t) * p.H + h)[c] = cr.x[k][t + 3];
            } else if (VERIFY && own) {
                const int ss = p.snap_slots[(size_t)b * p.T + t];
                if (ss >= 0 && ss < p.n_slots) {
                    Tin *sw = static_cast<Tin *>(p.window) + ((size_t)ss * p.H + h) * 3 * CH;
                    sw[c] = cr.x[k][t + 1];
                    sw[CH + c] = cr.x[k][t + 2];
                    sw[2 * CH + c] = cr.x[k][t + 3];
                }
            }
        }
        if (!VERIFY && own) {
            Tin *win = static_cast<Tin *>(p.window) + ((size_t)slot * p.H + h) * 3 * CH;
            win[c] = cr.x[k][1];
            win[CH + c] = cr.x[k][2];
            win[2 * CH + c] = cr.x[k][3];
        }
    }
}

// Raw gate operands of the tokens one wave prepares (t = wave + NW*j).
template <int DK, int DV, typename Tin, int TPW>
struct PrepRegs {
    static constexpr int EK = DK / kWave, EV = DV / kWave;
    float A[EK], w[EV];
    Tin g[TPW][EK], z[TPW][EV], b[TPW];
};

template <int DK, int DV, int NW, typename Tin, int TPW, bool VERIFY>
__device__ __forceinline__ void prep_fetch(const RecParams &p, int wave, int lane, int b, int row, int h, int T,
                                           PrepRegs<DK, DV, Tin, TPW> &pr) {
#pragma unroll
    for (int e = 0; e < pr.EK; ++e) pr.A[e] = p.A[h * DK + lane + kWave * e];
#pragma unroll
    for (int e = 0; e < pr.EV; ++e) pr.w[e] = p.norm_w[h * DV + lane + kWave * e];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
        const int t = min(wave + NW * j, T - 1);
        const size_t n = VERIFY ? (size_t)b * p.T + t : (size_t)row;
        const Tin *g = static_cast<const Tin *>(p.g) + (n * p.H + h) * DK;
        const Tin *z = static_cast<const Tin *>(p.z) + (n * p.H + h) * DV;
#pragma unroll
        for (int e = 0; e < pr.EK; ++e) pr.g[j][e] = g[lane + kWave * e];
#pragma unroll
        for (int e = 0; e < pr.EV; ++e) pr.z[j][e] = z[lane + kWave * e];
        pr.b[j] = static_cast<const Tin *>(p.b)[n * p.H + h];
    }
}

// L2 norms, k^.q^ and gates of one token, by one whole wave (PART < 0), or
// one independent part of them (PART 0: norms and k^.q^, 1: the decay
// alpha, 2: the output gate and beta), so that a single token's preparation
// runs on three waves at once.  Either way every value is formed by the same
// operations.
template <int DK, int DV, typename Tin, int TPW, int RG, int RPT, bool LR, int PART = -1>
__device__ __forceinline__ void prep_token(const RecParams &p, int lane, int j,
                                           const PrepRegs<DK, DV, Tin, TPW> &pr,
                                           TokenLds<DK, DV, LR> &tk) {
    constexpr int EK = DK / kWave, EV = DV / kWave;
    if (PART < 0 || PART == 0) {
        float qv[EK], kv[EK];
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int e = 0; e < EK; ++e) {
            qv[e] = tk.conv[lane + kWave * e];
            kv[e] = tk.conv[DK + lane + kWave * e];
            sq = fmaf(qv[e], qv[e], sq);
            sk = fmaf(kv[e], kv[e], sk);
        }
        sq = wave_sum(sq);
        sk = wave_sum(sk);
        const float rq = p.q_scale / sqrtf(sq + p.l2_eps);
        const float rk = 1.0f / sqrtf(sk + p.l2_eps);
        float kq = 0.f;
#pragma unroll
        for (int e = 0; e < EK; ++e) {
            qv[e] *= rq;
            kv[e] *= rk;
            kq = fmaf(qv[e], kv[e], kq);
            tk.conv[lane + kWave * e] = qv[e];
            tk.conv[DK + lane + kWave * e] = kv[e];
            if (LR) {
                const int r = lane + kWave * e, pos = (r % RG) * RPT + r / RG;
                tk.rows[1][pos] = kv[e];
                tk.rows[2][pos] = qv[e];
            }
        }
        kq = wave_sum(kq);
        if (lane == 0) tk.kq = kq;
    }
    if (PART < 0 || PART == 1) {
#pragma unroll
        for (int e = 0; e < EK; ++e) {
            const float a = expf(-expf(pr.A[e]) * softplus(to_f32(pr.g[j][e])));
            const int r = lane + kWave * e;
            tk.alpha[r] = a;
            if (LR) tk.rows[0][(r % RG) * RPT + r / RG] = a;
        }
    }
    if (PART < 0 || PART == 2) {
#pragma unroll
        for (int e = 0; e < EV; ++e)
            tk.gate[lane + kWave * e] = pr.w[e] * sigmoid(to_f32(pr.z[j][e]));
        if (lane == 0) tk.beta = sigmoid(to_f32(pr.b[j]));
    }
}

// y = o / sqrt(mean(o^2) + eps_r) * gate for the 4 columns 4c..4c+3 of one
// token, by lanes 0 .. d_v/4 - 1 of one wave (a DPP sum over those lanes).
template <int DV>
__device__ __forceinline__ void output_row(const RecParams &p, float4 o, const float *gate, int c,
                                           float *yrow) {
    float ss2 = o.x * o.x;
    ss2 = fmaf(o.y, o.y, ss2);
    ss2 = fmaf(o.z, o.z, ss2);
    ss2 = fmaf(o.w, o.w, ss2);
    ss2 = lane_sum<DV / 4>(ss2);
    const float r = 1.0f / sqrtf(ss2 * (1.0f / DV) + p.rms_eps);
    const float4 gt = make_float4(gate[4 * c], gate[4 * c + 1], gate[4 * c + 2], gate[4 * c + 3]);
    *reinterpret_cast<float4 *>(yrow + 4 * c) =
        make_float4(o.x * r * gt.x, o.y * r * gt.y, o.z * r * gt.z, o.w * r * gt.w);
}

enum RecMode { kDecode = 0, kVerify = 1, kVerifyDelta = 2 };

// LDS of one (sequence, head) item.
// red[]: per-wave partial sums of u and p.  Double-buffered (token t uses
// half t & 1) where LDS allows, so no barrier is needed after a token; at
// TMAX = 16 the second half would cost a workgroup per CU.
// obuf[]: unnormalised outputs of a multi-token call, normalised after the
// recurrence (one wave per token) so the RMSNorm reduction is not on the
// token chain.
template <int DK, int DV, int NT, int TMAX, bool LR_>
struct RecShared {
    using G = RecGeo<DK, DV, NT>;
    static constexpr int NRB = TMAX <= 8 ? 2 : 1;
    static constexpr bool DEFER = TMAX > 1;
    static constexpr bool LR = LR_;
    TokenLds<DK, DV, LR> tok[TMAX];
    float4 red[NRB][G::NW][2][G::CG];
    float4 obuf[DEFER ? TMAX : 1][G::CG];
};

// Registers of one item between its loads and its computation.
template <int DK, int DV, int NT, typename Tin, int TMAX>
struct RecItem {
    using G = RecGeo<DK, DV, NT>;
    static constexpr int TPW = (TMAX + G::NW - 1) / G::NW;
    int b, h, T, slot;
    int row;       // input / output row of a decode item
    bool run;
    bool routed;   // a one-token row of a packed prefill call
    float *yb, *S;
    ConvRegs<DK, DV, NT, Tin, TMAX> cr;
    PrepRegs<DK, DV, Tin, TPW> pr;
    float4 s[G::RPT];
};

// Slot resolution of item `item` = b * H + h (scalar reads only, so that a
// workgroup can resolve all of its items before it stores anything).
template <int DK, int DV, int NT, typename Tin, int TMAX, int MODE>
__device__ __forceinline__ void rec_resolve(const RecParams &p, int item, RecItem<DK, DV, NT, Tin, TMAX> &it) {
    constexpr bool VERIFY = MODE != kDecode;
    const int b = item / p.H, h = item % p.H;
    it.b = b;
    it.h = h;
    int T = 1;
    if (VERIFY) T = p.draft_len ? min(max(p.draft_len[b], 0), p.T) : p.T;
    it.T = T;
    it.slot = p.slot_idx[b];
    int row = b;
    bool take = true;
    it.routed = !VERIFY && p.seq_start != nullptr;
    if (it.routed) {
        const int a0 = p.seq_start[b];
        row = a0;
        take = *p.seq_ok == 1 && p.seq_start[b + 1] - a0 == 1;
    }
    it.row = row;
    const int y_rows = VERIFY ? p.T : 1;
    it.yb = p.y + ((size_t)row * y_rows * p.H + h) * DV;   // token t at + t*H*DV
    it.run = take && !(it.slot < 0 || it.slot >= p.n_slots || T == 0);
}

// Rows that will not be computed (padding, a bad slot, no draft tokens):
// their outputs are zeroed and a bad slot is flagged.  Computed rows get
// zeros for the draft tokens past their length.
template <int DK, int DV, int NT, typename Tin, int TMAX, int MODE>
__device__ __forceinline__ void rec_side(const RecParams &p, const RecItem<DK, DV, NT, Tin, TMAX> &it) {
    constexpr bool VERIFY = MODE != kDecode;
    // the prefill call flags bad slots and writes every row it does not compute
    if (it.routed) return;
    const int tid = threadIdx.x;
    const bool bad = it.slot < 0 || it.slot >= p.n_slots;
    if (bad && it.slot != -1 && tid == 0) flag_error(p.err_flag);
    const int y_rows = VERIFY ? p.T : 1;
    for (int t = bad ? 0 : it.T; t < y_rows; ++t)
        for (int j = tid; j < DV; j += NT) it.yb[(size_t)t * p.H * DV + j] = 0.f;
}

// Every load of a resolved item that will be computed: the small operands
// first, then the single read of the state tile, so the conv/gate math waits
// only for the former.
template <int DK, int DV, int NT, typename Tin, int TMAX, int MODE, bool STREAM>
__device__ __forceinline__ void rec_loads(const RecParams &p, RecItem<DK, DV, NT, Tin, TMAX> &it) {
    using G = RecGeo<DK, DV, NT>;
    constexpr bool VERIFY = MODE != kDecode;
    if (!it.run) return;
    const int tid = threadIdx.x;
    const int lane = tid % kWave, wave = tid / kWave;
    const int cg = tid % G::CG, rg = tid / G::CG;
    const int slot = it.slot, T = it.T;
    conv_fetch<DK, DV, NT, Tin, TMAX, VERIFY>(p, tid, it.b, it.row, it.h, slot, T, it.cr);
    prep_fetch<DK, DV, G::NW, Tin, RecItem<DK, DV, NT, Tin, TMAX>::TPW, VERIFY>(p, wave, lane, it.b, it.row, it.h, T,
                                                                              it.pr);
    it.S = p.state + ((size_t)slot * p.H + it.h) * DK * DV;
    // the small operands are requested before the state tile (loads return
    // in issue order, so the conv/gate math then waits only for them)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < G::RPT; ++i) it.s[i] = load_state4<STREAM, DK * DV>(it.S, (size_t)(rg + G::RG * i) * DV, 4 * cg);
    // and nothing that waits for them is scheduled above them
    __builtin_amdgcn_sched_barrier(0);
}

// The computation of a fetched item (it.run must be true; uniform over the
// workgroup): conv, norms and gates, the recurrence with the state in
// registers, the outputs and the state write.
template <int DK, int DV, int NT, typename Tin, int TMAX, int MODE, bool STREAM, bool LR_>
__device__ __forceinline__ void rec_run(const RecParams &p, RecItem<DK, DV, NT, Tin, TMAX> &it,
                                        RecShared<DK, DV, NT, TMAX, LR_> &sh) {
    using G = RecGeo<DK, DV, NT>;
    using SH = RecShared<DK, DV, NT, TMAX, LR_>;
    constexpr bool VERIFY = MODE != kDecode;
    constexpr bool DELTA = MODE == kVerifyDelta;
    constexpr int TPW = RecItem<DK, DV, NT, Tin, TMAX>::TPW;
    constexpr bool LR = SH::LR;
    TokenLds<DK, DV, LR> *tok = sh.tok;
    const int tid = threadIdx.x;
    const int lane = tid % kWave, wave = tid / kWave;
    const int cg = tid % G::CG, rg = tid / G::CG;
    const int b = it.b, h = it.h, T = it.T, slot = it.slot;
    float *yb = it.yb;
    float4 *s = it.s;

    // 2. conv (+ window update / window snapshots)
    conv_compute<DK, DV, NT, Tin, TMAX, VERIFY, DELTA, LR>(p, tid, b, h, slot, T, it.cr, tok);
    __syncthreads();
    // 3. norms and gates: one wave per token, or for a single token its
    //    three independent parts on three waves (every wave fetched the gate
    //    operands of token 0)
    if (TMAX == 1 && G::NW >= 3) {
        if (wave == 0) prep_token<DK, DV, Tin, TPW, G::RG, G::RPT, LR, 0>(p, lane, 0, it.pr, tok[0]);
        else if (wave == 1) prep_token<DK, DV, Tin, TPW, G::RG, G::RPT, LR, 1>(p, lane, 0, it.pr, tok[0]);
        else if (wave == 2) prep_token<DK, DV, Tin, TPW, G::RG, G::RPT, LR, 2>(p, lane, 0, it.pr, tok[0]);
    } else {
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int t = wave + G::NW * j;
            if (t < T) prep_token<DK, DV, Tin, TPW, G::RG, G::RPT, LR>(p, lane, j, it.pr, tok[t]);
        }
    }
    __syncthreads();
    // delta mode: alpha and k^ of every token into its record
    if (DELTA) {
        constexpr int NI = (TMAX * 2 * DK + NT - 1) / NT;
        float v[NI];
#pragma unroll
        for (int k = 0; k < NI; ++k) {   // all LDS reads first, then the stores
            const int i = min(tid + NT * k, T * 2 * DK - 1);
            const int t = i / (2 * DK), e = i % (2 * DK);
            v[k] = e < DK ? tok[t].alpha[e] : tok[t].conv[e];
        }
#pragma unroll
        for (int k = 0; k < NI; ++k) {
            const int i = tid + NT * k;
            if (i < T * 2 * DK)
                DeltaRec<DK, DV, Tin>::f(p.delta, ((size_t)b * p.T + i / (2 * DK)) * p.H + h)[i % (2 * DK)] = v[k];
        }
    }

    // 4. the recurrence, tokens in order, state in registers
    for (int t = 0; t < T; ++t) {
        const TokenLds<DK, DV, LR> &tk = tok[t];
        float4 u = make_float4(0.f, 0.f, 0.f, 0.f), pq = u;
        static_assert(!LR || G::RPT % 4 == 0, "a lane's rows are read four at a time");
        const float4 *rk = reinterpret_cast<const float4 *>(&tk.rows[LR ? 1 : 0][LR ? rg * G::RPT : 0]);
        if (LR) {
            const float4 *ra = reinterpret_cast<const float4 *>(&tk.rows[0][rg * G::RPT]);
            const float4 *rq = reinterpret_cast<const float4 *>(&tk.rows[LR ? 2 : 0][LR ? rg * G::RPT : 0]);
#pragma unroll
            for (int i4 = 0; i4 < G::RPT / 4; ++i4) {
                const float4 a4 = ra[i4], k4 = rk[i4], q4 = rq[i4];
                const float av[4] = {a4.x, a4.y, a4.z, a4.w}, kv[4] = {k4.x, k4.y, k4.z, k4.w},
                            qv[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int i = 4 * i4 + c;   // row rg + RG * i
                    s[i] = s[i] * av[c];
                    u = fma4(kv[c], s[i], u);
                    pq = fma4(qv[c], s[i], pq);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < G::RPT; ++i) {
                const int r = rg + G::RG * i;
                s[i] = s[i] * tk.alpha[r];
                u = fma4(tk.conv[DK + r], s[i], u);
                pq = fma4(tk.conv[r], s[i], pq);
            }
        }
        // sum over the row groups inside the wave (into lanes 0 .. CG-1),
        // then across waves
#pragma unroll
        for (int m = G::CG; m < kWave; m <<= 1) {
            if (m == 32) {
                u.x = add_upper_half(u.x); u.y = add_upper_half(u.y);
                u.z = add_upper_half(u.z); u.w = add_upper_half(u.w);
                pq.x = add_upper_half(pq.x); pq.y = add_upper_half(pq.y);
                pq.z = add_upper_half(pq.z); pq.w = add_upper_half(pq.w);
            } else {
                u.x += __shfl_xor(u.x, m, kWave); u.y += __shfl_xor(u.y, m, kWave);
                u.z += __shfl_xor(u.z, m, kWave); u.w += __shfl_xor(u.w, m, kWave);
                pq.x += __shfl_xor(pq.x, m, kWave); pq.y += __shfl_xor(pq.y, m, kWave);
                pq.z += __shfl_xor(pq.z, m, kWave); pq.w += __shfl_xor(pq.w, m, kWave);
            }
        }
        const int rb = SH::NRB == 2 ? (t & 1) : 0;
        if (lane < G::CG) { sh.red[rb][wave][0][cg] = u; sh.red[rb][wave][1][cg] = pq; }
        __syncthreads();
        float4 U = sh.red[rb][0][0][cg], P = sh.red[rb][0][1][cg];
#pragma unroll
        for (int w = 1; w < G::NW; ++w) {
            const float4 a = sh.red[rb][w][0][cg], c = sh.red[rb][w][1][cg];
            U.x += a.x; U.y += a.y; U.z += a.z; U.w += a.w;
            P.x += c.x; P.y += c.y; P.z += c.z; P.w += c.w;
        }
        const float beta = tk.beta;
        const float4 v = *reinterpret_cast<const float4 *>(&tk.conv[2 * DK + 4 * cg]);
        const float4 d = make_float4(beta * (v.x - U.x), beta * (v.y - U.y),
                                     beta * (v.z - U.z), beta * (v.w - U.w));
        if (LR) {
#pragma unroll
            for (int i4 = 0; i4 < G::RPT / 4; ++i4) {
                const float4 k4 = rk[i4];
                s[4 * i4] = fma4(k4.x, d, s[4 * i4]);
                s[4 * i4 + 1] = fma4(k4.y, d, s[4 * i4 + 1]);
                s[4 * i4 + 2] = fma4(k4.z, d, s[4 * i4 + 2]);
                s[4 * i4 + 3] = fma4(k4.w, d, s[4 * i4 + 3]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < G::RPT; ++i) s[i] = fma4(tk.conv[DK + rg + G::RG * i], d, s[i]);
        }

        if (DELTA) {
            if (tid < G::CG)
                *reinterpret_cast<float4 *>(DeltaRec<DK, DV, Tin>::f(p.delta, ((size_t)b * p.T + t) * p.H + h) +
                                            2 * DK + 4 * cg) = d;
        } else if (VERIFY) {
            const int ss = p.snap_slots[(size_t)b * p.T + t];
            if (ss >= 0 && ss < p.n_slots) {
                float *D = p.state + ((size_t)ss * p.H + h) * DK * DV;
#pragma unroll
                for (int i = 0; i < G::RPT; ++i) store_state4<STREAM, DK * DV>(D, (size_t)(rg + G::RG * i) * DV, 4 * cg, s[i]);
            } else if (ss != -1 && tid == 0) {
                flag_error(p.err_flag);
            }
        }
        // output: o = p + (k^.q^) d (= S^T q^ of the new state)
        if (tid < G::CG) {
            const float kq = tk.kq;
            const float4 o = make_float4(fmaf(kq, d.x, P.x), fmaf(kq, d.y, P.y),
                                         fmaf(kq, d.z, P.z), fmaf(kq, d.w, P.w));
            if (SH::DEFER) sh.obuf[t][cg] = o;
            else output_row<DV>(p, o, tk.gate, cg, yb);
        }
        if (SH::NRB == 1) __syncthreads();   // red[] is rewritten by the next token
    }
    // RMSNorm + gate of the deferred outputs: token t by lanes 0 .. CG-1 of
    // wave t % NW, the lanes and reduction order of the inline form
    if (SH::DEFER) {
        __syncthreads();
        for (int t = wave; t < T; t += G::NW)
            if (lane < G::CG) output_row<DV>(p, sh.obuf[t][lane], tok[t].gate, lane, yb + (size_t)t * p.H * DV);
    }

    // 5. the single write of the state tile (decode only: verify leaves S0)
    if (!VERIFY) {
#pragma unroll
        for (int i = 0; i < G::RPT; ++i) store_state4<STREAM, DK * DV>(it.S, (size_t)(rg + G::RG * i) * DV, 4 * cg, s[i]);
    }
}

#ifndef KDA_DECODE_WPE
#define KDA_DECODE_WPE 3
#endif
// One workgroup per (sequence, head) item.  Decode is held to three
// workgroups per CU (its registers would allow four): with four, the
// batch-64 step measured about 2% slower (more tiles contending for the same
// bandwidth), while single-round launches gain nothing from the fourth.
template <int DK, int DV, int NT, typename Tin, int TMAX, int MODE, bool STREAM, bool LR>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, MODE == kDecode ? KDA_DECODE_WPE : 8)))
void kda_recurrent_kernel(RecParams p) {
    __shared__ RecShared<DK, DV, NT, TMAX, LR> sh;
    RecItem<DK, DV, NT, Tin, TMAX> it;
    rec_resolve<DK, DV, NT, Tin, TMAX, MODE>(p, blockIdx.x, it);
    rec_side<DK, DV, NT, Tin, TMAX, MODE>(p, it);
    rec_loads<DK, DV, NT, Tin, TMAX, MODE, STREAM>(p, it);
    if (it.run) rec_run<DK, DV, NT, Tin, TMAX, MODE, STREAM, LR>(p, it, sh);
}

// Commit: copy the snapshot of the last accepted token into the live slot.
__global__ __launch_bounds__(256) void kda_commit_kernel(CommitParams p) {
    const int b = blockIdx.x / p.H, h = blockIdx.x % p.H;
    const int L = p.accepted_len[b];
    const int dst = p.slot_idx[b];
    if (L == 0 || dst == -1) return;
    const bool bad_len = L < 0 || L > p.T;
    const int src = bad_len ? -1 : p.snap_slots[(size_t)b * p.T + L - 1];
    if (bad_len || dst < 0 || dst >= p.n_slots || src < 0 || src >= p.n_slots) {
        if (threadIdx.x == 0) flag_error(p.err_flag);
        return;
    }
    const float4 *s4 = reinterpret_cast<const float4 *>(p.state + ((size_t)src * p.H + h) * p.state_elems);
    float4 *d4 = reinterpret_cast<float4 *>(p.state + ((size_t)dst * p.H + h) * p.state_elems);
    for (int i = threadIdx.x; i < p.state_elems / 4; i += blockDim.x) d4[i] = s4[i];
    const uint32_t *sw = static_cast<const uint32_t *>(p.window) + ((size_t)src * p.H + h) * p.window_words;
    uint32_t *dw = static_cast<uint32_t *>(p.window) + ((size_t)dst * p.H + h) * p.window_words;
    for (int i = threadIdx.x; i < p.window_words; i += blockDim.x) dw[i] = sw[i];
}

// Delta commit: replay the first L = accepted_len[b] records of sequence b
// onto its live state, S <- diag(alpha_t) S + k^_t d_t^T for t < L (the same
// two fp32 roundings per element as the verify and decode kernels), and
// rebuild the conv window as rows L, L+1, L+2 of [window rows 0..2, x_1..x_T].
// One workgroup per (sequence, head), the decode kernel's tile geometry.
template <int DK, int DV, int NT, typename Tin, bool STREAM>
__global__ __launch_bounds__(NT) void kda_commit_delta_kernel(CommitDeltaParams p) {
    using G = RecGeo<DK, DV, NT>;
    using R = DeltaRec<DK, DV, Tin>;
    constexpr int CH = 2 * DK + DV;
    constexpr int NF = R::kFloats;
    __shared__ float rec[kMaxDraft][NF];

    const int tid = threadIdx.x;
    const int cg = tid % G::CG, rg = tid / G::CG;
    const int b = blockIdx.x / p.H, h = blockIdx.x % p.H;
    const int L = p.accepted_len[b];
    const int dst = p.slot_idx[b];
    if (L == 0 || dst == -1) return;
    if (L < 0 || L > p.T || dst < 0 || dst >= p.n_slots) {
        if (tid == 0) flag_error(p.err_flag);
        return;
    }
    float *S = p.state + ((size_t)dst * p.H + h) * DK * DV;
    float4 s[G::RPT];
#pragma unroll
    for (int i = 0; i < G::RPT; ++i) s[i] = load_state4<STREAM, DK * DV>(S, (size_t)(rg + G::RG * i) * DV, 4 * cg);

    // the float part of the L records into LDS (16-byte loads)
    for (int i = tid; i < L * (NF / 4); i += NT) {
        const int t = i / (NF / 4), e = 4 * (i % (NF / 4));
        const float4 v = *reinterpret_cast<const float4 *>(R::f(p.delta, ((size_t)b * p.T + t) * p.H + h) + e);
        rec[t][e] = v.x; rec[t][e + 1] = v.y; rec[t][e + 2] = v.z; rec[t][e + 3] = v.w;
    }
    // conv window: per channel, read the three source rows, then write
    Tin *win = static_cast<Tin *>(p.window) + ((size_t)dst * p.H + h) * 3 * CH;
    for (int c = tid; c < CH; c += NT) {
        Tin x[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int r = L + j;   // row of [w0, w1, w2, x_1 .. x_T]
            x[j] = r < 3 ? win[r * CH + c] : R::x(p.delta, ((size_t)b * p.T + (r - 3)) * p.H + h)[c];
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) win[j * CH + c] = x[j];
    }
    __syncthreads();

    for (int t = 0; t < L; ++t) {
        const float *a = rec[t];
        const float4 d = make_float4(a[2 * DK + 4 * cg], a[2 * DK + 4 * cg + 1],
                                     a[2 * DK + 4 * cg + 2], a[2 * DK + 4 * cg + 3]);
#pragma unroll
        for (int i = 0; i < G::RPT; ++i) {
            const int r = rg + G::RG * i;
            s[i] = s[i] * a[r];
            s[i] = fma4(a[DK + r], d, s[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < G::RPT; ++i) store_state4<STREAM, DK * DV>(S, (size_t)(rg + G::RG * i) * DV, 4 * cg, s[i]);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
#ifndef KDA_REC_THREADS
#define KDA_REC_THREADS 256
#endif
constexpr int kRecThreads = KDA_REC_THREADS;   // lanes per (sequence, head) workgroup

// Workgroups resident at once on the 256 CUs: three per CU for verify
// kernels of up to 8 tokens, two for 16 tokens with the lane-ordered rows.
// A grid up to that size is one round and takes the lane-ordered rows.
constexpr long long kOneRoundWorkgroups = 3 * 256, kOneRoundWorkgroups16 = 2 * 256;

template <int DK, int DV, typename Tin, bool STREAM, int MODE>
static void launch_rec_mode(const RecParams &p, hipStream_t stream) {
    const dim3 grid((unsigned)(p.B * p.H)), block(kRecThreads);
    if (MODE == kDecode) {
        hipLaunchKernelGGL((kda_recurrent_kernel<DK, DV, kRecThreads, Tin, 1, kDecode, STREAM, false>), grid,
                           block, 0, stream, p);
    } else if (p.T <= 8 && (long long)p.B * p.H <= kOneRoundWorkgroups) {
        hipLaunchKernelGGL((kda_recurrent_kernel<DK, DV, kRecThreads, Tin, 8, MODE, STREAM, true>), grid, block,
                           0, stream, p);
    } else if (p.T <= 8) {
        hipLaunchKernelGGL((kda_recurrent_kernel<DK, DV, kRecThreads, Tin, 8, MODE, STREAM, false>), grid,
                           block, 0, stream, p);
    } else if ((long long)p.B * p.H <= kOneRoundWorkgroups16) {
        hipLaunchKernelGGL((kda_recurrent_kernel<DK, DV, kRecThreads, Tin, kMaxDraft, MODE, STREAM, true>),
                           grid, block, 0, stream, p);
    } else {
        hipLaunchKernelGGL((kda_recurrent_kernel<DK, DV, kRecThreads, Tin, kMaxDraft, MODE, STREAM, false>),
                           grid, block, 0, stream, p);
    }
}

template <int DK, int DV, typename Tin, bool STREAM>
static kda_status launch_rec_typed(const RecParams &p, RecKind kind, hipStream_t stream) {
    switch (kind) {
        case RecKind::decode: launch_rec_mode<DK, DV, Tin, STREAM, kDecode>(p, stream); break;
        case RecKind::verify: launch_rec_mode<DK, DV, Tin, STREAM, kVerify>(p, stream); break;
        case RecKind::verify_delta: launch_rec_mode<DK, DV, Tin, STREAM, kVerifyDelta>(p, stream); break;
    }
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

template <int DK, int DV>
static kda_status launch_rec_dt(const RecParams &p, kda_dtype dt, RecKind kind, hipStream_t s) {
    if (p.stream_state)
        return dt == KDA_BF16 ? launch_rec_typed<DK, DV, uint16_t, true>(p, kind, s)
                              : launch_rec_typed<DK, DV, float, true>(p, kind, s);
    return dt == KDA_BF16 ? launch_rec_typed<DK, DV, uint16_t, false>(p, kind, s)
                          : launch_rec_typed<DK, DV, float, false>(p, kind, s);
}

kda_status launch_recurrent(const RecParams &p, int d_k, int d_v, kda_dtype dt, RecKind kind,
                            hipStream_t stream) {
    if (p.B == 0) return KDA_OK;
    if (d_k == 128 && d_v == 128) return launch_rec_dt<128, 128>(p, dt, kind, stream);
    if (d_k == 64 && d_v == 64) return launch_rec_dt<64, 64>(p, dt, kind, stream);
    if (d_k == 128 && d_v == 64) return launch_rec_dt<128, 64>(p, dt, kind, stream);
    if (d_k == 64 && d_v == 128) return launch_rec_dt<64, 128>(p, dt, kind, stream);
    return KDA_ERR_UNSUPPORTED;
}

kda_status launch_commit(const CommitParams &p, hipStream_t stream) {
    if (p.B == 0) return KDA_OK;
    hipLaunchKernelGGL(kda_commit_kernel, dim3((unsigned)(p.B * p.H)), dim3(256), 0, stream, p);
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

template <int DK, int DV>
static void launch_commit_delta_shape(const CommitDeltaParams &p, kda_dtype dt, hipStream_t s) {
    const dim3 grid((unsigned)(p.B * p.H)), block(kRecThreads);
    if (p.stream_state) {
        if (dt == KDA_BF16)
            hipLaunchKernelGGL((kda_commit_delta_kernel<DK, DV, kRecThreads, uint16_t, true>), grid, block, 0, s, p);
        else
            hipLaunchKernelGGL((kda_commit_delta_kernel<DK, DV, kRecThreads, float, true>), grid, block, 0, s, p);
    } else {
        if (dt == KDA_BF16)
            hipLaunchKernelGGL((kda_commit_delta_kernel<DK, DV, kRecThreads, uint16_t, false>), grid, block, 0, s, p);
        else
            hipLaunchKernelGGL((kda_commit_delta_kernel<DK, DV, kRecThreads, float, false>), grid, block, 0, s, p);
    }
}

kda_status launch_commit_delta(const CommitDeltaParams &p, int d_k, int d_v, kda_dtype dt,
                               hipStream_t stream) {
    if (p.B == 0) return KDA_OK;
    if (d_k == 128 && d_v == 128) launch_commit_delta_shape<128, 128>(p, dt, stream);
    else if (d_k == 64 && d_v == 64) launch_commit_delta_shape<64, 64>(p, dt, stream);
    else if (d_k == 128 && d_v == 64) launch_commit_delta_shape<128, 64>(p, dt, stream);
    else if (d_k == 64 && d_v == 128) launch_commit_delta_shape<64, 128>(p, dt, stream);
    else return KDA_ERR_UNSUPPORTED;
    return hipGetLastError() == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

size_t spec_delta_record_bytes(int d_k, int d_v, kda_dtype dt) {
    return (size_t)(2 * d_k + d_v) * (4 + (dt == KDA_BF16 ? 2 : 4));
}

}  // namespace kda
