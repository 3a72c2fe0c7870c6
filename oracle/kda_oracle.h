/*
 * kda_oracle.h -- plain fp64 CPU oracle for the Kimi Delta Attention (KDA)
 * recurrent-state update.  TEST INFRASTRUCTURE ONLY: it exists so that tests,
 * the smoke check and the CPU-baseline leg of the benchmark can check the HIP
 * library against an obviously correct reference.  No product code path may
 * link, load or call it.
 *
 * What it computes (one token, one sequence b, one head h):
 *   The pages ("vLLM Kimi K3 support", section "Kimi K3 architecture overview")
 *   describe KDA as a linear-attention layer that keeps a fixed-size recurrent
 *   state; section "Fused kernels and metadata optimisation" says the decode
 *   step runs a causal convolution, the recurrent update and an RMSNorm, in
 *   that order.  The pages give no formulas; the readings below are the
 *   plainest ones the rest supports (decay first, then the delta rule;
 *   read-out from the updated state; depthwise width-4 conv + SiLU; L2-normed
 *   q/k; RMSNorm over d_v times a sigmoid output gate).
 *
 *   1. conv   : for every channel c of the head (q | k | v):
 *               y_c = sum_j w[c][j] * x_c(t - (W-1) + j), tap 0 the oldest,
 *               zero history before the first token; optional SiLU.
 *               The window then drops its oldest raw input, appends x_c(t).
 *   2. l2 norm: k^ = k / sqrt(|k|^2 + eps2),  q^ = s * q / sqrt(|q|^2 + eps2)
 *   3. gates  : alpha_i = exp(-exp(A_i) * softplus(g_i)),  beta = sigmoid(b)
 *   4. decay  : S' = diag(alpha) S                    (S is d_k x d_v)
 *   5. predict: u = S'^T k^
 *   6. update : S = S' + beta * k^ (v - u)^T
 *   7. readout: o = S^T q^                            (the updated S)
 *   8. output : y = o / sqrt(mean(o^2) + eps_r) * w_norm * sigmoid(z)
 *
 * All arithmetic is in double precision.  Inputs are given as doubles (the
 * exact values of whatever narrower type the caller rounded them to).
 */
#ifndef KDA_ORACLE_H
#define KDA_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kda_oracle_layer {
    int H, d_k, d_v, conv_w;
    const double *A;        /* [H, d_k]  decay log-rate                      */
    const double *conv_wt;  /* [H, 2*d_k + d_v, conv_w]  q|k|v, tap 0 oldest  */
    const double *norm_w;   /* [H, d_v]  RMSNorm weight                      */
    double q_scale;         /* s in step 2                                   */
    double l2_eps;          /* eps2 in step 2                                */
    double rms_eps;         /* eps_r in step 8                               */
    int conv_silu;          /* nonzero: SiLU after the conv                  */
} kda_oracle_layer;

/*
 * Runs T tokens of B independent sequences.
 *   state  [B, H, d_k, d_v]            in/out
 *   window [B, H, conv_w-1, C_h]       in/out, C_h = 2*d_k + d_v, row 0 oldest
 *   x_q, x_k, g [B, T, H, d_k];  x_v, z [B, T, H, d_v];  b [B, T, H]
 *   lens   [B] or NULL: sequence b runs only its first lens[b] tokens
 *   y      [B, y_tokens, H, d_v]: outputs of tokens t < y_tokens (NULL: none)
 *   snap_state  [B, T, H, d_k, d_v] or NULL: state after each token
 *   snap_window [B, T, H, conv_w-1, C_h] or NULL: window after each token
 *   n_threads: OpenMP threads over (b, h); <= 0 uses the OpenMP default.
 * Returns 0, or -1 on a bad argument.
 */
int kda_oracle_run(const kda_oracle_layer *L, int B, int T,
                   double *state, double *window,
                   const double *x_q, const double *x_k, const double *x_v,
                   const double *g, const double *b, const double *z,
                   const int *lens, double *y, int y_tokens,
                   double *snap_state, double *snap_window, int n_threads);

/* Number of OpenMP threads a parallel region would use with n_threads. */
int kda_oracle_threads(int n_threads);

#ifdef __cplusplus
}
#endif
#endif
