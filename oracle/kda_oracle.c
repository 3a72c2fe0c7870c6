/*
 * kda_oracle.c -- plain fp64 CPU oracle of the KDA recurrent-state update.
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU baseline); never part of
 * the product path.  Each step follows one passage of the pages:
 *   - fixed-size recurrent state per head: "vLLM Kimi K3 support",
 *     section "Kimi K3 architecture overview" (the KDA bullet);
 *   - conv -> recurrent update -> RMSNorm, in that order: same page,
 *     section "Fused kernels and metadata optimisation" (the KDA decode bullet);
 *   - fp32 state storage ("FP32 SSM cache"): "Kimi K3 vLLM GPU inference
 *     benchmark", section on the time breakdown.  The oracle keeps the state
 *     in double; callers pass the fp32 values widened exactly.
 * Where the pages are silent, the plainest reading is taken (see the header).
 * No blocking, fusion or reordering: every step of the definition is its own
 * loop over plain arrays.
 */
#include "kda_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double softplus(double x) { return fmax(x, 0.0) + log1p(exp(-fabs(x))); }
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* One token of one (sequence, head).  S is d_k x d_v row-major, win is
 * (W-1) x C_h.  xq, xk, g have d_k entries, xv, z have d_v, b is a scalar.
 * y (d_v entries) may be NULL. */
static void oracle_token(const kda_oracle_layer *L, int h, double *S, double *win,
                         const double *xq, const double *xk, const double *xv,
                         const double *g, double bl, const double *z, double *y,
                         double *conv_out, double *Sd, double *u, double *o)
{
    const int dk = L->d_k, dv = L->d_v, W = L->conv_w;
    const int Ch = 2 * dk + dv;
    const double *wt = L->conv_wt + (size_t)h * Ch * W;

    /* 1. short causal conv over the raw inputs, then the window shift */
    for (int c = 0; c < Ch; ++c) {
        double x_now = c < dk ? xq[c] : (c < 2 * dk ? xk[c - dk] : xv[c - 2 * dk]);
        double acc = 0.0;
        for (int j = 0; j < W - 1; ++j) acc += wt[c * W + j] * win[j * Ch + c];
        acc += wt[c * W + (W - 1)] * x_now;
        conv_out[c] = L->conv_silu ? acc * sigmoid(acc) : acc;
        for (int j = 0; j + 1 < W - 1; ++j) win[j * Ch + c] = win[(j + 1) * Ch + c];
        if (W > 1) win[(W - 2) * Ch + c] = x_now;
    }
    const double *q = conv_out, *k = conv_out + dk, *v = conv_out + 2 * dk;

    /* 2. L2 normalisation over d_k (q also takes the scale s) */
    double qq = 0.0, kk = 0.0;
    for (int i = 0; i < dk; ++i) { qq += q[i] * q[i]; kk += k[i] * k[i]; }
    const double rq = L->q_scale / sqrt(qq + L->l2_eps);
    const double rk = 1.0 / sqrt(kk + L->l2_eps);

    /* 3. gates */
    const double beta = sigmoid(bl);

    /* 4. decay: S' = diag(alpha) S, alpha per key channel i */
    for (int i = 0; i < dk; ++i) {
        const double alpha = exp(-exp(L->A[(size_t)h * dk + i]) * softplus(g[i]));
        for (int j = 0; j < dv; ++j) Sd[i * dv + j] = alpha * S[i * dv + j];
    }
    /* 5. prediction u = S'^T k^ */
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += Sd[i * dv + j] * (k[i] * rk);
        u[j] = acc;
    }
    /* 6. delta update S = S' + beta k^ (v - u)^T */
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            S[i * dv + j] = Sd[i * dv + j] + beta * (k[i] * rk) * (v[j] - u[j]);
    /* 7. read-out from the updated state, o = S^T q^ */
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += S[i * dv + j] * (q[i] * rq);
        o[j] = acc;
    }
    /* 8. RMSNorm over d_v, weight, sigmoid output gate */
    if (y) {
        double ms = 0.0;
        for (int j = 0; j < dv; ++j) ms += o[j] * o[j];
        ms /= dv;
        const double r = 1.0 / sqrt(ms + L->rms_eps);
        for (int j = 0; j < dv; ++j)
            y[j] = o[j] * r * L->norm_w[(size_t)h * dv + j] * sigmoid(z[j]);
    }
}

int kda_oracle_threads(int n_threads)
{
#ifdef _OPENMP
    if (n_threads > 0) return n_threads;
    return omp_get_max_threads();
#else
    (void)n_threads;
    return 1;
#endif
}

int kda_oracle_run(const kda_oracle_layer *L, int B, int T,
                   double *state, double *window,
                   const double *x_q, const double *x_k, const double *x_v,
                   const double *g, const double *b, const double *z,
                   const int *lens, double *y, int y_tokens,
                   double *snap_state, double *snap_window, int n_threads)
{
    if (!L || !state || !window || !x_q || !x_k || !x_v || !g || !b || !z) return -1;
    if (B < 0 || T < 0 || L->H <= 0 || L->d_k <= 0 || L->d_v <= 0 || L->conv_w < 1) return -1;
    if (y && (y_tokens < 0 || y_tokens > T)) return -1;
    const int H = L->H, dk = L->d_k, dv = L->d_v, W = L->conv_w;
    const int Ch = 2 * dk + dv;
    const size_t sS = (size_t)dk * dv, sW = (size_t)(W - 1) * Ch;
    const int nthr = kda_oracle_threads(n_threads);
    int bad = 0;

#ifdef _OPENMP
#pragma omp parallel for collapse(2) schedule(dynamic, 1) num_threads(nthr) reduction(| : bad)
#endif
    for (int bi = 0; bi < B; ++bi) {
        for (int h = 0; h < H; ++h) {
            double *scratch = (double *)malloc(sizeof(double) * (Ch + sS + 2 * (size_t)dv));
            if (!scratch) { bad = 1; continue; }
            double *conv_out = scratch, *Sd = scratch + Ch, *u = Sd + sS, *o = u + dv;
            double *S = state + ((size_t)bi * H + h) * sS;
            double *win = window + ((size_t)bi * H + h) * sW;
            const int Tb = lens ? lens[bi] : T;
            for (int t = 0; t < Tb && t < T; ++t) {
                const size_t tok = (size_t)bi * T + t;          /* [B, T] flat */
                double *yt = (y && t < y_tokens)
                    ? y + (((size_t)bi * y_tokens + t) * H + h) * dv : NULL;
                oracle_token(L, h, S, win,
                             x_q + (tok * H + h) * dk, x_k + (tok * H + h) * dk,
                             x_v + (tok * H + h) * dv, g + (tok * H + h) * dk,
                             b[tok * H + h], z + (tok * H + h) * dv, yt,
                             conv_out, Sd, u, o);
                if (snap_state) memcpy(snap_state + (tok * H + h) * sS, S, sizeof(double) * sS);
                if (snap_window) memcpy(snap_window + (tok * H + h) * sW, win, sizeof(double) * sW);
            }
            free(scratch);
        }
    }
    (void)nthr;
    return bad ? -1 : 0;
}
