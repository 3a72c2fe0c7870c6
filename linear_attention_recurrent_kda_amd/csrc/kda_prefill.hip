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
// intra: one workgroup (256 lanes) per (chunk, head)
// ---------------------------------------------------------------------------
template <int DK, int DV>
struct __align__(16) IntraLds {
    static constexpr int DM = DK > DV ? DK : DV;
    float G[kChunk][DK];        // log2-decay prefix sums
    float k[kChunk][DK];        // k^, later the W right-hand side / solution
    float q[kChunk][DM];        // q^, later beta v / U~ (row stride DV then)
    float A[kChunk][kChunk + 1];
    float beta[kChunk];
};

template <int DK, int DV>
__global__ __launch_bounds__(256) void kda_prefill_intra_kernel(PrefillParams p, PrefillWs ws) {
    __shared__ IntraLds<DK, DV> L;
    const int tid = threadIdx.x;
    const int gidx = blockIdx.x, h = blockIdx.y, H = p.H;
    if (ws.meta[0] != 1) return;
    const int32_t *cs = ws.meta + 1;
    if (gidx >= cs[p.N_seq]) return;
    const int s = upper_index(cs, p.N_seq + 1, gidx);
    if (!slot_ok(p.slot_idx[s], p.n_slots)) return;
    const int c = gidx - cs[s];
    const int t0 = p.cu_seqlens[s] + c * kChunk;
    const int n = min(kChunk, p.cu_seqlens[s + 1] - t0);

    // 1. load k^, q^, log2 alpha, beta of the chunk (rows >= n are zero)
    for (int e = tid; e < kChunk * DK; e += 256) {
        const int r = e / DK, i = e % DK;
        const bool in = r < n;
        const size_t src = ((size_t)(t0 + r) * H + h) * DK + i;
        L.k[r][i] = in ? ws.kh[src] : 0.f;
        L.q[r][i] = in ? ws.qh[src] : 0.f;
        L.G[r][i] = in ? ws.la[src] : 0.f;
    }
    if (tid < kChunk) L.beta[tid] = tid < n ? ws.beta[(size_t)(t0 + tid) * H + h] : 0.f;
    __syncthreads();
    // 2. prefix sums over the chunk, per key channel (non-increasing in t)
    if (tid < DK) {
        float acc = 0.f;
        for (int r = 0; r < kChunk; ++r) { acc += L.G[r][tid]; L.G[r][tid] = acc; }
    }
    __syncthreads();
    // 3. A (s < t) and P (s <= t), 4x4 tiles of (t, s) per lane, lower tiles only
    float *P = ws.P + ((size_t)gidx * H + h) * kChunk * kChunk;
    for (int tile = tid; tile < 256; tile += 256) {
        const int ti = tile / 16, si = tile % 16;
        float a[4][4] = {}, pq[4][4] = {};
        if (si <= ti) {
            for (int i = 0; i < DK; ++i) {
                float gt[4], kt[4], qt[4], gs[4], ks[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    gt[u] = L.G[4 * ti + u][i]; kt[u] = L.k[4 * ti + u][i]; qt[u] = L.q[4 * ti + u][i];
                    gs[u] = L.G[4 * si + u][i]; ks[u] = L.k[4 * si + u][i];
                }
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        // only s <= t is used; clamp the exponent so unused
                        // entries (s > t) stay finite
                        const float e = exp2f(fminf(gt[u] - gs[v], 0.f)) * ks[v];
                        a[u][v] = fmaf(kt[u], e, a[u][v]);
                        pq[u][v] = fmaf(qt[u], e, pq[u][v]);
                    }
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int t = 4 * ti + u, sv = 4 * si + v;
                L.A[t][sv] = sv < t ? L.beta[t] * a[u][v] : 0.f;
                P[t * kChunk + sv] = sv <= t ? pq[u][v] : 0.f;
            }
    }
    __syncthreads();
    // 4. decayed factors for the state recurrence and the outputs
    const size_t gh = (size_t)gidx * H + h;
    const int last = max(n - 1, 0);
    for (int e = tid; e < kChunk * DK; e += 256) {
        const int r = e / DK, i = e % DK;
        const float gl = L.G[last][i];
        ws.Qg[gh * kChunk * DK + r * DK + i] = L.q[r][i] * exp2f(L.G[r][i]);
        ws.KdT[gh * DK * kChunk + i * kChunk + r] = L.k[r][i] * exp2f(fminf(gl - L.G[r][i], 0.f));
    }
    if (tid < DK) ws.gC[gh * DK + tid] = exp2f(L.G[last][tid]);
    __syncthreads();   // q and G are free from here on
    // 5. right-hand sides in place: k <- beta k e^G (for W), q <- beta v (for U~)
    for (int e = tid; e < kChunk * DK; e += 256) {
        const int r = e / DK, i = e % DK;
        L.k[r][i] = L.beta[r] * L.k[r][i] * exp2f(L.G[r][i]);
    }
    for (int e = tid; e < kChunk * DV; e += 256) {
        const int r = e / DV, j = e % DV;
        reinterpret_cast<float *>(L.q)[r * DV + j] =
            r < n ? L.beta[r] * ws.vv[((size_t)(t0 + r) * H + h) * DV + j] : 0.f;
    }
    __syncthreads();
    // 6. forward substitution (I + A) X = R, in place, one lane per column
    for (int col = tid; col < DK + DV; col += 256) {
        float *x = col < DK ? &L.k[0][col] : reinterpret_cast<float *>(L.q) + (col - DK);
        const int ld = col < DK ? DK : DV;
        for (int t = 1; t < kChunk; ++t) {
            float acc = x[t * ld];
            for (int sv = 0; sv < t; ++sv) acc = fmaf(-L.A[t][sv], x[sv * ld], acc);
            x[t * ld] = acc;
        }
    }
    __syncthreads();
    for (int e = tid; e < kChunk * DK; e += 256)
        ws.W[gh * kChunk * DK + e] = L.k[e / DK][e % DK];
    for (int e = tid; e < kChunk * DV; e += 256)
        ws.Ut[gh * kChunk * DV + e] = reinterpret_cast<float *>(L.q)[e];
}

// ---------------------------------------------------------------------------
// scan: one workgroup per (sequence, head, 16 state columns)
// ---------------------------------------------------------------------------
template <int DK, int DV, typename Tin>
__global__ __launch_bounds__(256) void kda_prefill_scan_kernel(PrefillParams p, PrefillWs ws) {
    constexpr int CB = kColBlock, CH = 2 * DK + DV;
    constexpr int EPT = DK * CB / 256;          // state entries per lane in the update
    static_assert(EPT >= 1 && CB % EPT == 0, "state block does not divide");
    __shared__ __align__(16) float S[DK][CB];
    __shared__ __align__(16) float U[kChunk][CB];
    const int tid = threadIdx.x;
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
    for (int e = tid; e < DK * CB; e += 256) S[e / CB][e % CB] = Sg[(e / CB) * DV + j0 + e % CB];
    __syncthreads();

    const int ut = tid / 4, uq = tid % 4;        // U / O: row ut, columns 4uq..4uq+3
    const int si = tid / (CB / EPT), sc0 = (tid % (CB / EPT)) * EPT;   // S update: row si, EPT columns
    for (int c = 0; c < nch; ++c) {
        const size_t gh = (size_t)(g0 + c) * H + h;
        const int t0 = p.cu_seqlens[s] + c * kChunk;
        const int n = min(kChunk, p.cu_seqlens[s + 1] - t0);
        // U = U~ - W S
        const float *Wr = ws.W + gh * kChunk * DK + ut * DK;
        float4 u = *reinterpret_cast<const float4 *>(ws.Ut + gh * kChunk * DV + ut * DV + j0 + 4 * uq);
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        const float *Qr = ws.Qg + gh * kChunk * DK + ut * DK;
        for (int i = 0; i < DK; i += 4) {
            const float4 w4 = *reinterpret_cast<const float4 *>(Wr + i);
            const float4 q4 = *reinterpret_cast<const float4 *>(Qr + i);
            const float wv[4] = {w4.x, w4.y, w4.z, w4.w}, qv[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float4 sv = *reinterpret_cast<const float4 *>(&S[i + m][4 * uq]);
                u = fma4(-wv[m], sv, u);
                o = fma4(qv[m], sv, o);
            }
        }
        *reinterpret_cast<float4 *>(&U[ut][4 * uq]) = u;
        __syncthreads();
        // O = Q^e^G S + P U (rows >= n of P and U are zero)
        const float *Pr = ws.P + gh * kChunk * kChunk + ut * kChunk;
        for (int sv = 0; sv <= ut; ++sv) o = fma4(Pr[sv], *reinterpret_cast<const float4 *>(&U[sv][4 * uq]), o);
        if (ut < n)
            *reinterpret_cast<float4 *>(p.y + ((size_t)(t0 + ut) * H + h) * DV + j0 + 4 * uq) = o;
        // S = diag(e^G_C) S + Kd^T U
        const float gcv = ws.gC[gh * DK + si];
        const float *Kr = ws.KdT + gh * DK * kChunk + si * kChunk;
        float acc[EPT];
#pragma unroll
        for (int m = 0; m < EPT; ++m) acc[m] = gcv * S[si][sc0 + m];
        for (int t = 0; t < kChunk; t += 4) {
            const float4 k4 = *reinterpret_cast<const float4 *>(Kr + t);
            const float kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
            for (int m2 = 0; m2 < 4; ++m2)
#pragma unroll
                for (int m = 0; m < EPT; ++m) acc[m] = fmaf(kv[m2], U[t + m2][sc0 + m], acc[m]);
        }
        __syncthreads();   // every lane has read S and U of this chunk
#pragma unroll
        for (int m = 0; m < EPT; ++m) S[si][sc0 + m] = acc[m];
        __syncthreads();
    }
    for (int e = tid; e < DK * CB; e += 256) Sg[(e / CB) * DV + j0 + e % CB] = S[e / CB][e % CB];
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
