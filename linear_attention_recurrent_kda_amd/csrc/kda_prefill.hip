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
//   prep   one wave per (token, head): conv + SiLU, L2 norms, log2(alpha), beta
//   intra  one workgroup per (chunk, head): prefix sums, A, P, the triangular
//          solve for W and U~, the decayed Q and K factors
//   scan   one workgroup per (sequence, head, 16 columns of d_v): the fp32 state
//          carried from chunk to chunk (state columns are independent given the
//          chunk factors), unnormalised outputs O written to y
//   norm   one wave per (token, head): RMSNorm over d_v, weight, sigmoid gate
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int kChunk = 64;
constexpr int kColBlock = 16;
constexpr float kLog2e = 1.4426950408889634f;

// Device pointers into the caller's workspace (fp32 unless noted).
struct PrefillWs {
    int32_t *meta;        // [0]: 1 if cu_seqlens is valid; [1 + s]: first chunk of s, s <= N
    float *qh, *kh, *vv;  // [T, H, d]
    float *la;            // [T, H, d_k]  log2(alpha)
    float *beta;          // [T, H]
    float *W, *Ut, *Qg;   // [G, H, 64, d]
    float *KdT;           // [G, H, d_k, 64]
    float *P;             // [G, H, 64, 64]
    float *gC;            // [G, H, d_k]  e^(G_C)
    int G_max;
};

struct WsLayout {
    size_t meta, qh, kh, vv, la, beta, W, Ut, Qg, KdT, P, gC, total;
};

static size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

static WsLayout ws_layout(int H, int dk, int dv, int total_T, int N_seq) {
    const size_t G = (size_t)total_T / kChunk + (size_t)N_seq;
    const size_t TH = (size_t)total_T * H, GH = G * H;
    WsLayout l{};
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
    l.meta = take(sizeof(int32_t) * (N_seq + 2));
    l.qh = take(4 * TH * dk);
    l.kh = take(4 * TH * dk);
    l.vv = take(4 * TH * dv);
    l.la = take(4 * TH * dk);
    l.beta = take(4 * TH);
    l.W = take(4 * GH * kChunk * dk);
    l.Ut = take(4 * GH * kChunk * dv);
    l.Qg = take(4 * GH * kChunk * dk);
    l.KdT = take(4 * GH * dk * kChunk);
    l.P = take(4 * GH * kChunk * kChunk);
    l.gC = take(4 * GH * dk);
    l.total = off;
    return l;
}

size_t prefill_workspace_bytes(int H, int d_k, int d_v, int total_T, int N_seq, int chunk) {
    if (chunk != kChunk || total_T < 0 || N_seq < 1) return 0;
    return ws_layout(H, d_k, d_v, total_T, N_seq).total;
}

// Largest s in [0, n) with a[s] <= v (a non-decreasing, a[0] <= v).
__device__ __forceinline__ int upper_index(const int32_t *a, int n, int v) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a[mid] <= v) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ bool slot_ok(int slot, int n_slots) { return slot >= 0 && slot < n_slots; }

// ---------------------------------------------------------------------------
// meta: validate cu_seqlens and count chunks (one lane; N_seq is small)
// ---------------------------------------------------------------------------
__global__ void kda_prefill_meta_kernel(PrefillParams p, PrefillWs ws) {
    if (threadIdx.x != 0) return;
    const int N = p.N_seq;
    bool ok = p.cu_seqlens[0] == 0 && p.cu_seqlens[N] == p.total_T;
    for (int s = 0; s < N && ok; ++s) ok = p.cu_seqlens[s + 1] >= p.cu_seqlens[s];
    int32_t *cs = ws.meta + 1;
    cs[0] = 0;
    for (int s = 0; s < N; ++s) {
        const int len = ok ? p.cu_seqlens[s + 1] - p.cu_seqlens[s] : 0;
        cs[s + 1] = cs[s] + (len + kChunk - 1) / kChunk;
    }
    ws.meta[0] = ok ? 1 : 0;
    if (!ok) flag_error(p.err_flag);
    for (int s = 0; s < N && ok; ++s) {
        const int sl = p.slot_idx[s];
        if (sl != -1 && !slot_ok(sl, p.n_slots)) flag_error(p.err_flag);
    }
}

// ---------------------------------------------------------------------------
// prep: one wave per (token, head)
// ---------------------------------------------------------------------------
template <int DK, int DV, typename Tin>
__global__ __launch_bounds__(256) void kda_prefill_prep_kernel(PrefillParams p, PrefillWs ws) {
    constexpr int CH = 2 * DK + DV, EC = CH / kWave, EK = DK / kWave, EV = DV / kWave;
    const int lane = threadIdx.x % kWave;
    const int t = blockIdx.x * 4 + threadIdx.x / kWave;
    const int h = blockIdx.y, H = p.H;
    if (t >= p.total_T || ws.meta[0] != 1) return;
    const int s = upper_index(p.cu_seqlens, p.N_seq + 1, t);   // cu[s] <= t < cu[s+1]
    const int slot = p.slot_idx[s];
    if (!slot_ok(slot, p.n_slots)) return;
    const int pos = t - p.cu_seqlens[s];
    const Tin *win = static_cast<const Tin *>(p.window) + ((size_t)slot * H + h) * 3 * CH;
    float conv[EC];
#pragma unroll
    for (int e = 0; e < EC; ++e) {
        const int c = lane + kWave * e;
        const Tin *src;
        int stride, off;
        if (c < DK) { src = static_cast<const Tin *>(p.x_q); stride = DK; off = c; }
        else if (c < 2 * DK) { src = static_cast<const Tin *>(p.x_k); stride = DK; off = c - DK; }
        else { src = static_cast<const Tin *>(p.x_v); stride = DV; off = c - 2 * DK; }
        const float4 w = *reinterpret_cast<const float4 *>(p.conv_wt + ((size_t)h * CH + c) * 4);
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int q = pos - 3 + j;   // position of tap j's input in the sequence
            x[j] = q >= 0 ? to_f32(src[((size_t)(t - 3 + j) * H + h) * stride + off])
                          : to_f32(win[(q + 3) * CH + c]);
        }
        float acc = w.x * x[0];
        acc = fmaf(w.y, x[1], acc);
        acc = fmaf(w.z, x[2], acc);
        acc = fmaf(w.w, x[3], acc);
        conv[e] = p.silu ? acc * sigmoid(acc) : acc;
    }
    // channels c = lane + 64 e: e < EK are q, EK <= e < 2 EK are k, the rest v
    float sq = 0.f, sk = 0.f;
#pragma unroll
    for (int e = 0; e < EK; ++e) {
        sq = fmaf(conv[e], conv[e], sq);
        sk = fmaf(conv[EK + e], conv[EK + e], sk);
    }
    sq = wave_sum(sq);
    sk = wave_sum(sk);
    const float rq = p.q_scale / sqrtf(sq + p.l2_eps);
    const float rk = 1.0f / sqrtf(sk + p.l2_eps);
    const size_t th = (size_t)t * H + h;
    const Tin *g = static_cast<const Tin *>(p.g) + th * DK;
#pragma unroll
    for (int e = 0; e < EK; ++e) {
        const int i = lane + kWave * e;
        ws.qh[th * DK + i] = conv[e] * rq;
        ws.kh[th * DK + i] = conv[EK + e] * rk;
        // alpha below 2^-200 is 0 in fp32 either way; the floor keeps the
        // prefix sums finite (g = +inf would give -inf - -inf = NaN later)
        ws.la[th * DK + i] = fmaxf(-expf(p.A[h * DK + i]) * softplus(to_f32(g[i])) * kLog2e, -200.f);
    }
#pragma unroll
    for (int e = 0; e < EV; ++e) ws.vv[th * DV + lane + kWave * e] = conv[2 * EK + e];
    if (lane == 0) ws.beta[th] = sigmoid(to_f32(static_cast<const Tin *>(p.b)[th]));
}

// ---------------------------------------------------------------------------
// intra: one workgroup (4 waves) per (chunk, head).  The Gram matrices A, P,
// the triangular inverse T = (I + A)^-1 and [W | U~] = T [diag(beta) K^ e^G |
// diag(beta) V] are formed here; every contraction runs on MFMA in bf16x3.
//
// Gram tiles are 16 x 16 token blocks.  For a t-block starting at token r,
// e^(G_t - G_s) = e^(G_t - G_r) e^(G_r - G_s): the first factor is <= 1 for
// t >= r and the second is <= 1 for s < r, so an off-diagonal tile is a plain
// product of two scaled operands.  In a diagonal tile s >= r makes the second
// factor >= 1; it is used only when the block's decay span is at most 2^60
// (checked per block), otherwise the tile is summed directly with one
// exponential per term.
// ---------------------------------------------------------------------------
// Rows of q, k and G are padded by one word so that lanes reading down a
// column (different tokens, same channel) hit different LDS banks.
template <int DK, int DV>
struct __align__(16) IntraLds {
    static constexpr int KW = DK + 1;
    static constexpr int QW = KW >= 68 ? KW : 68;
    float q[kChunk][QW];           // q^, later T = (I + A)^-1
    float k[kChunk][KW];           // k^
    float G[kChunk][KW];           // log2-decay prefix sums
    float A[kChunk][kChunk + 1];   // beta_t (K K^T * decay), strictly lower part used
    float Z[3][16][17];            // block-inverse scratch
    float D[4][16][17];            // per-wave scratch of the direct tile path
    float beta[kChunk];
    int safe[4];
};

constexpr float kSafeSpan = 60.f;

template <int DK, int DV>
__global__ __launch_bounds__(256) void kda_prefill_intra_kernel(PrefillParams p, PrefillWs ws) {
    constexpr int KS = DK / 32, QW = IntraLds<DK, DV>::QW;
    __shared__ IntraLds<DK, DV> L;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int lr = lane % 16, lk = lane / 16;
    const int gidx = blockIdx.x, h = blockIdx.y, H = p.H;
    if (ws.meta[0] != 1) return;
    const int32_t *cs = ws.meta + 1;
    if (gidx >= cs[p.N_seq]) return;
    const int s = upper_index(cs, p.N_seq + 1, gidx);
    if (!slot_ok(p.slot_idx[s], p.n_slots)) return;
    const int c = gidx - cs[s];
    const int t0 = p.cu_seqlens[s] + c * kChunk;
    const int n = min(kChunk, p.cu_seqlens[s + 1] - t0);
    const size_t gh = (size_t)gidx * H + h;

    // 1. k^, q^ and beta of the chunk (rows >= n are zero); lanes < d_k also
    //    form the log2-decay prefix sums of their channel straight from memory
    for (int e = tid; e < kChunk * DK / 4; e += 256) {
        const int r = e / (DK / 4), i = 4 * (e % (DK / 4));
        float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), qv = kv;
        if (r < n) {
            const size_t src = ((size_t)(t0 + r) * H + h) * DK + i;
            kv = *reinterpret_cast<const float4 *>(ws.kh + src);
            qv = *reinterpret_cast<const float4 *>(ws.qh + src);
        }
        L.k[r][i] = kv.x; L.k[r][i + 1] = kv.y; L.k[r][i + 2] = kv.z; L.k[r][i + 3] = kv.w;
        L.q[r][i] = qv.x; L.q[r][i + 1] = qv.y; L.q[r][i + 2] = qv.z; L.q[r][i + 3] = qv.w;
    }
    if (tid < DK) {
        const float *la = ws.la + ((size_t)t0 * H + h) * DK + tid;
        float acc = 0.f;
#pragma unroll 8
        for (int r = 0; r < kChunk; ++r) {
            acc += r < n ? la[(size_t)r * H * DK] : 0.f;   // non-increasing in r
            L.G[r][tid] = acc;
        }
    }
    if (tid < kChunk) L.beta[tid] = tid < n ? ws.beta[(size_t)(t0 + tid) * H + h] : 0.f;
    // the V operand of step 7 is read now, so its latency hides behind steps 3-6
    constexpr int NU = DV / 64;                  // U~ column tiles per wave
    float vpre[NU][2][8];
#pragma unroll
    for (int m = 0; m < NU; ++m) {
        const int col = 16 * (wave + 4 * (DK / 64 + m)) + lr - DK;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int sv = 32 * k2 + 8 * lk + e;
                vpre[m][k2][e] = sv < n ? ws.vv[((size_t)(t0 + sv) * H + h) * DV + col] : 0.f;
            }
    }
    __syncthreads();
    // 3. per 16-token block: may the diagonal tile use the scaled factors?
    {
        float span = 0.f;
        for (int i = lane; i < DK; i += kWave) span = fmaxf(span, L.G[16 * wave][i] - L.G[16 * wave + 15][i]);
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) span = fmaxf(span, __shfl_xor(span, m, kWave));
        if (lane == 0) L.safe[wave] = span <= kSafeSpan ? 1 : 0;
    }
    __syncthreads();

    // 4. A and P in 16 x 16 tiles; tile (bt, bs) covers t in block bt, s in
    //    block bs.  The 10 tiles on or below the diagonal go 3,3,2,2 to the
    //    waves; the 6 above it (P = 0 there, A is never read there) 2,2,1,1.
    float *Pg = ws.P + gh * kChunk * kChunk;
    for (int tile = wave; tile < 16; tile += 4) {
        // lower tiles 0..9 in row order, then the upper ones
        const int lbt[16] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3, 0, 0, 0, 1, 1, 2};
        const int lbs[16] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3, 1, 2, 3, 2, 3, 3};
        const int bt = lbt[tile], bs = lbs[tile];
        f32x4 aA = {0.f, 0.f, 0.f, 0.f}, aP = aA;
        if (bs > bt) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) Pg[(16 * bt + 4 * lk + rr) * kChunk + 16 * bs + lr] = 0.f;
            continue;
        }
        const int r = 16 * bt;
        if (bs < bt || L.safe[bt]) {
            const int t = 16 * bt + lr, sr = 16 * bs + lr;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                float ka[8], qa[8], kb[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int ch = 32 * kk + 8 * lk + e;
                    const float gr = L.G[r][ch];
                    const float et = exp2f(L.G[t][ch] - gr);
                    const float es = exp2f(gr - L.G[sr][ch]);
                    ka[e] = L.k[t][ch] * et;
                    qa[e] = L.q[t][ch] * et;
                    kb[e] = L.k[sr][ch] * es;
                }
                const Split8 b = split8(kb);
                aA = mma3(split8(ka), b, aA);
                aP = mma3(split8(qa), b, aP);
            }
        } else {
            // direct: lane owns row t = r + lr and columns s = r + 4 lk + j
            float da[4] = {0.f, 0.f, 0.f, 0.f}, dp[4] = {0.f, 0.f, 0.f, 0.f};
            const int t = r + lr;
            for (int ch = 0; ch < DK; ++ch) {
                const float gt = L.G[t][ch], kt = L.k[t][ch], qt = L.q[t][ch];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int sv = r + 4 * lk + j;
                    const float e = exp2f(fminf(gt - L.G[sv][ch], 0.f)) * L.k[sv][ch];
                    da[j] = fmaf(kt, e, da[j]);
                    dp[j] = fmaf(qt, e, dp[j]);
                }
            }
            // move to the MFMA result layout through this wave's scratch
            // (the tile's block of A is written only by this wave)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                L.A[t][r + 4 * lk + j] = da[j];
                L.D[wave][lr][4 * lk + j] = dp[j];
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                aA[rr] = L.A[r + 4 * lk + rr][r + lr];
                aP[rr] = L.D[wave][4 * lk + rr][lr];
            }
            __builtin_amdgcn_wave_barrier();
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int t = 16 * bt + 4 * lk + rr, sv = 16 * bs + lr;
            L.A[t][sv] = sv < t ? L.beta[t] * aA[rr] : 0.f;
            Pg[t * kChunk + sv] = sv <= t ? aP[rr] : 0.f;
        }
    }
    // 5. decayed factors for the scan: Q^ e^G, (K^ e^(G_C - G))^T, e^(G_C)
    const int last = max(n - 1, 0);
    for (int e = tid; e < kChunk * DK; e += 256) {
        const int r = e / DK, i = e % DK;
        ws.Qg[gh * kChunk * DK + r * DK + i] = L.q[r][i] * exp2f(L.G[r][i]);
    }
    for (int e = tid; e < kChunk * DK; e += 256) {
        const int i = e / kChunk, r = e % kChunk;
        ws.KdT[gh * DK * kChunk + e] = L.k[r][i] * exp2f(fminf(L.G[last][i] - L.G[r][i], 0.f));
    }
    if (tid < DK) ws.gC[gh * DK + tid] = exp2f(L.G[last][tid]);
    __syncthreads();   // q^ is free from here on: T lives in its place

    // 6. T = (I + A)^-1 by 16 x 16 blocks
    float(*T)[QW] = L.q;
    for (int e = tid; e < kChunk * kChunk; e += 256) T[e / kChunk][e % kChunk] = 0.f;
    __syncthreads();
    if (tid < 64) {   // diagonal blocks: column j of (I + A_bb)^-1
        const int b = tid / 16, j = tid % 16, o = 16 * b;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float acc = i == j ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m) acc = fmaf(-L.A[o + i][o + m], x[m], acc);
            x[i] = acc;
            T[o + i][o + j] = i >= j ? acc : 0.f;
        }
    }
    __syncthreads();
    for (int b = 1; b < 4; ++b) {
        // Z_b' = sum_{b' <= m < b} A_bm T_mb'  for every b' < b
        for (int e = tid; e < b * 256; e += 256) {
            const int bp = e / 256, i = (e / 16) % 16, j = e % 16;
            float acc = 0.f;
            for (int m = 16 * bp; m < 16 * b; ++m) acc = fmaf(L.A[16 * b + i][m], T[m][16 * bp + j], acc);
            L.Z[bp][i][j] = acc;
        }
        __syncthreads();
        // T_bb' = -T_bb Z_b'
        for (int e = tid; e < b * 256; e += 256) {
            const int bp = e / 256, i = (e / 16) % 16, j = e % 16;
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < 16; ++m) acc = fmaf(T[16 * b + i][16 * b + m], L.Z[bp][m][j], acc);
            T[16 * b + i][16 * bp + j] = -acc;
        }
        __syncthreads();
    }

    // 7. [W | U~] = T R with R = [diag(beta) K^ e^G | diag(beta) V]  (MFMA)
    Split8 ta[4][2];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = T[16 * rt + lr][32 * k2 + 8 * lk + e];
            ta[rt][k2] = split8(x);
        }
    constexpr int NCT = (DK + DV) / 16;
#pragma unroll
    for (int ci = 0; ci < NCT / 4; ++ci) {
        const int ct = wave + 4 * ci;
        const int col = 16 * ct + lr;
        const bool isw = ci < DK / 64;             // wave-uniform
        Split8 rb[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int sv = 32 * k2 + 8 * lk + e;
                if (isw) x[e] = L.beta[sv] * L.k[sv][col] * exp2f(L.G[sv][col]);
                else x[e] = L.beta[sv] * vpre[ci - DK / 64][k2][e];
            }
            rb[k2] = split8(x);
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma3(ta[rt][0], rb[0], acc);
            if (rt >= 2) acc = mma3(ta[rt][1], rb[1], acc);   // T is lower triangular
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int t = 16 * rt + 4 * lk + rr;
                if (isw) ws.W[gh * kChunk * DK + t * DK + col] = acc[rr];
                else ws.Ut[gh * kChunk * DV + t * DV + (col - DK)] = acc[rr];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// scan: one workgroup (4 waves) per (sequence, head, 16 state columns).
// Per chunk, wave w owns rows 16w..16w+15 of the chunk and state row tiles
// TS*w .. TS*w+TS-1; all products run on MFMA in bf16x3 with fp32
// accumulation.  The next chunk's operands are loaded while the current one
// is computed (two register buffers).
// ---------------------------------------------------------------------------
template <int DK>
struct ScanOps {
    static constexpr int KS = DK / 32, TS = DK / 64;
    float w[KS][8];        // W rows (A operand, K = d_k)
    float q[KS][8];        // Q^ e^G rows
    float pm[2][8];        // P rows (K = token)
    float kd[TS][2][8];    // Kd^T rows (K = token)
    float ut[4];           // U~ (result layout)
    float gc[TS][4];       // e^(G_C) of the state rows this lane updates
};

template <int DK, int DV>
__device__ __forceinline__ void scan_load(const PrefillWs &ws, size_t gh, int wave, int lr, int lk, int j0,
                                          ScanOps<DK> &o) {
    constexpr int KS = DK / 32, TS = DK / 64;
    const float *W = ws.W + gh * kChunk * DK + (16 * wave + lr) * DK + 8 * lk;
    const float *Q = ws.Qg + gh * kChunk * DK + (16 * wave + lr) * DK + 8 * lk;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        *reinterpret_cast<float4 *>(&o.w[k][0]) = *reinterpret_cast<const float4 *>(W + 32 * k);
        *reinterpret_cast<float4 *>(&o.w[k][4]) = *reinterpret_cast<const float4 *>(W + 32 * k + 4);
        *reinterpret_cast<float4 *>(&o.q[k][0]) = *reinterpret_cast<const float4 *>(Q + 32 * k);
        *reinterpret_cast<float4 *>(&o.q[k][4]) = *reinterpret_cast<const float4 *>(Q + 32 * k + 4);
    }
    const float *P = ws.P + gh * kChunk * kChunk + (16 * wave + lr) * kChunk + 8 * lk;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        *reinterpret_cast<float4 *>(&o.pm[k][0]) = *reinterpret_cast<const float4 *>(P + 32 * k);
        *reinterpret_cast<float4 *>(&o.pm[k][4]) = *reinterpret_cast<const float4 *>(P + 32 * k + 4);
    }
#pragma unroll
    for (int m = 0; m < TS; ++m) {
        const float *K = ws.KdT + gh * DK * kChunk + (16 * (TS * wave + m) + lr) * kChunk + 8 * lk;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            *reinterpret_cast<float4 *>(&o.kd[m][k][0]) = *reinterpret_cast<const float4 *>(K + 32 * k);
            *reinterpret_cast<float4 *>(&o.kd[m][k][4]) = *reinterpret_cast<const float4 *>(K + 32 * k + 4);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) o.gc[m][r] = ws.gC[gh * DK + 16 * (TS * wave + m) + 4 * lk + r];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) o.ut[r] = ws.Ut[gh * kChunk * DV + (16 * wave + 4 * lk + r) * DV + j0 + lr];
}

template <int DK, int DV, typename Tin>
__global__ __launch_bounds__(256) void kda_prefill_scan_kernel(PrefillParams p, PrefillWs ws) {
    constexpr int CB = kColBlock, CH = 2 * DK + DV, KS = DK / 32, TS = DK / 64;
    __shared__ __align__(16) float S[2][DK][CB];
    __shared__ __align__(16) float U[kChunk][CB];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int lr = lane % 16, lk = lane / 16;
    const int s = blockIdx.x, h = blockIdx.y, j0 = blockIdx.z * CB, H = p.H;
    if (ws.meta[0] != 1) return;
    const int slot = p.slot_idx[s];
    if (!slot_ok(slot, p.n_slots)) return;
    const int32_t *cs = ws.meta + 1;
    const int g0 = cs[s], nch = cs[s + 1] - cs[s];
    const int len = p.cu_seqlens[s + 1] - p.cu_seqlens[s];

    // the window after the sequence: the last 3 raw inputs (older rows from
    // the previous window when len < 3); read everything, then write
    if (blockIdx.z == 0) {
        Tin *win = static_cast<Tin *>(p.window) + ((size_t)slot * H + h) * 3 * CH;
        Tin nv[2][3];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            const int ch = tid + 256 * k2;
            if (ch >= CH) continue;
            const Tin *src;
            int stride, off;
            if (ch < DK) { src = static_cast<const Tin *>(p.x_q); stride = DK; off = ch; }
            else if (ch < 2 * DK) { src = static_cast<const Tin *>(p.x_k); stride = DK; off = ch - DK; }
            else { src = static_cast<const Tin *>(p.x_v); stride = DV; off = ch - 2 * DK; }
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const int q = len + j - 3;   // sequence position of new row j
                nv[k2][j] = q >= 0 ? src[((size_t)(p.cu_seqlens[s] + q) * H + h) * stride + off]
                                   : win[(q + 3) * CH + ch];
            }
        }
        __syncthreads();
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            const int ch = tid + 256 * k2;
            if (ch >= CH) continue;
#pragma unroll
            for (int j = 0; j < 3; ++j) win[j * CH + ch] = nv[k2][j];
        }
    }

    float *Sg = p.state + ((size_t)slot * H + h) * DK * DV;
    for (int e = tid; e < DK * CB; e += 256) S[0][e / CB][e % CB] = Sg[(e / CB) * DV + j0 + e % CB];
    __syncthreads();

    auto load_sb = [&](int buf, Split8 (&sb)[KS]) {
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = S[buf][32 * k + 8 * lk + e][lr];
            sb[k] = split8(x);
        }
    };
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

    // sequence bounds in registers: a load inside the chunk loop would have
    // to wait behind the prefetch of the next chunk
    const int seq_t0 = p.cu_seqlens[s], seq_t1 = p.cu_seqlens[s + 1];
    float ypend[4];          // outputs of the previous chunk, stored one step late
    int ypend_t0 = 0, ypend_n = 0;
    auto flush_y = [&]() {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * wave + 4 * lk + r;
            if (t < ypend_n) p.y[((size_t)(ypend_t0 + t) * H + h) * DV + j0 + lr] = ypend[r];
        }
    };

    // chunk c reads the state from S[c & 1] and writes the next one to
    // S[(c + 1) & 1]; two barriers per chunk
    auto chunk_step = [&](int c, const ScanOps<DK> &o, Split8 (&sb)[KS]) {
        const int cur = c & 1;
        const int t0 = seq_t0 + c * kChunk;
        const int n = min(kChunk, seq_t1 - t0);
        // U = U~ - W S ; O = Q^e^G S
        Acc3 au, ao;
        zero3(au);
        zero3(ao);
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            mma3s(split8(o.w[k], -1.0f), sb[k], au);
            mma3s(split8(o.q[k]), sb[k], ao);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) U[16 * wave + 4 * lk + r][lr] = o.ut[r] + sum3(au, r);
        __syncthreads();
        Split8 ub[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = U[32 * k + 8 * lk + e][lr];
            ub[k] = split8(x);
        }
        // O += P U  (P rows beyond the chunk and above the diagonal are 0)
#pragma unroll
        for (int k = 0; k < 2; ++k) mma3s(split8(o.pm[k]), ub[k], ao);
#pragma unroll
        for (int r = 0; r < 4; ++r) ypend[r] = sum3(ao, r);
        ypend_t0 = t0;
        ypend_n = n;
        // S' = diag(e^G_C) S + Kd^T U  into the other buffer
#pragma unroll
        for (int m = 0; m < TS; ++m) {
            Acc3 as;
            zero3(as);
#pragma unroll
            for (int k = 0; k < 2; ++k) mma3s(split8(o.kd[m][k]), ub[k], as);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * (TS * wave + m) + 4 * lk + r;
                S[cur ^ 1][row][lr] = o.gc[m][r] * S[cur][row][lr] + sum3(as, r);
            }
        }
        __syncthreads();
        load_sb(cur ^ 1, sb);
    };

    Split8 sb[KS];
    load_sb(0, sb);
    ScanOps<DK> cur, nxt;
    if (nch > 0) scan_load<DK, DV>(ws, (size_t)g0 * H + h, wave, lr, lk, j0, cur);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the loop starts with nothing in flight
    for (int c = 0; c < nch; ++c) {
        // the next chunk's operands load while this chunk computes
        if (c + 1 < nch) scan_load<DK, DV>(ws, (size_t)(g0 + c + 1) * H + h, wave, lr, lk, j0, nxt);
        flush_y();
        chunk_step(c, cur, sb);
        // all of them (and the output stores issued above) have landed by
        // now; an explicit vmcnt(0) tells the compiler so, instead of
        // conservative waits inside the next step
        __builtin_amdgcn_s_waitcnt(0x0F70);
        cur = nxt;
    }
    flush_y();
    const int fin = nch & 1;
    for (int e = tid; e < DK * CB; e += 256) Sg[(e / CB) * DV + j0 + e % CB] = S[fin][e / CB][e % CB];
}

// ---------------------------------------------------------------------------
// norm: one wave per (token, head): y = O / sqrt(mean(O^2) + eps) * w * sigmoid(z)
// ---------------------------------------------------------------------------
template <int DK, int DV, typename Tin>
__global__ __launch_bounds__(256) void kda_prefill_norm_kernel(PrefillParams p, PrefillWs ws) {
    constexpr int EV = DV / kWave;
    const int lane = threadIdx.x % kWave;
    const int t = blockIdx.x * 4 + threadIdx.x / kWave;
    const int h = blockIdx.y, H = p.H;
    if (t >= p.total_T) return;
    float *yr = p.y + ((size_t)t * H + h) * DV;
    bool live = ws.meta[0] == 1;
    if (live) {
        const int s = upper_index(p.cu_seqlens, p.N_seq + 1, t);
        live = slot_ok(p.slot_idx[s], p.n_slots);
    }
    if (!live) {
#pragma unroll
        for (int e = 0; e < EV; ++e) yr[lane + kWave * e] = 0.f;
        return;
    }
    float o[EV];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < EV; ++e) { o[e] = yr[lane + kWave * e]; ss = fmaf(o[e], o[e], ss); }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss * (1.0f / DV) + p.rms_eps);
    const Tin *z = static_cast<const Tin *>(p.z) + ((size_t)t * H + h) * DV;
#pragma unroll
    for (int e = 0; e < EV; ++e) {
        const int j = lane + kWave * e;
        yr[j] = o[e] * r * (p.norm_w[h * DV + j] * sigmoid(to_f32(z[j])));
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
    ws.qh = reinterpret_cast<float *>(base + l.qh);
    ws.kh = reinterpret_cast<float *>(base + l.kh);
    ws.vv = reinterpret_cast<float *>(base + l.vv);
    ws.la = reinterpret_cast<float *>(base + l.la);
    ws.beta = reinterpret_cast<float *>(base + l.beta);
    ws.W = reinterpret_cast<float *>(base + l.W);
    ws.Ut = reinterpret_cast<float *>(base + l.Ut);
    ws.Qg = reinterpret_cast<float *>(base + l.Qg);
    ws.KdT = reinterpret_cast<float *>(base + l.KdT);
    ws.P = reinterpret_cast<float *>(base + l.P);
    ws.gC = reinterpret_cast<float *>(base + l.gC);
    ws.G_max = p.total_T / kChunk + p.N_seq;

    hipLaunchKernelGGL(kda_prefill_meta_kernel, dim3(1), dim3(64), 0, stream, p, ws);
    if (p.total_T > 0) {
        const dim3 tok_grid((unsigned)((p.total_T + 3) / 4), (unsigned)p.H);
        hipLaunchKernelGGL((kda_prefill_prep_kernel<DK, DV, Tin>), tok_grid, dim3(256), 0, stream, p, ws);
        hipLaunchKernelGGL((kda_prefill_intra_kernel<DK, DV>), dim3((unsigned)ws.G_max, (unsigned)p.H),
                           dim3(256), 0, stream, p, ws);
    }
    hipLaunchKernelGGL((kda_prefill_scan_kernel<DK, DV, Tin>),
                       dim3((unsigned)p.N_seq, (unsigned)p.H, (unsigned)(DV / kColBlock)), dim3(256), 0,
                       stream, p, ws);
    if (p.total_T > 0) {
        const dim3 tok_grid((unsigned)((p.total_T + 3) / 4), (unsigned)p.H);
        hipLaunchKernelGGL((kda_prefill_norm_kernel<DK, DV, Tin>), tok_grid, dim3(256), 0, stream, p, ws);
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
