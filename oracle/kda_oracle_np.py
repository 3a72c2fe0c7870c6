"""NumPy fp64 twin of the KDA oracle, plus the chunked (WY/UT) form of the core.

TEST INFRASTRUCTURE ONLY: used by tests, the smoke check and the CPU-baseline
leg of the benchmark.  Nothing in the product path may import it.

This file is written independently of ``kda_oracle.c`` (vectorised over
sequences and heads, library routines where they exist: ``np.logaddexp`` for
softplus, ``scipy.special.expit`` for the logistic function, ``einsum`` for
the contractions) so that the two can check each other.

The method: the pages ("vLLM Kimi K3 support", section "Kimi K3 architecture
overview") call KDA a linear-attention layer with a fixed-size recurrent state,
and (section "Fused kernels and metadata optimisation") say its decode step
fuses the causal convolution, the recurrent update and RMSNorm.  The formulas
are not on the pages; the readings used here are:

  conv     y_c = sum_j w[c, j] x_c(t-W+1+j)  (tap 0 oldest, zero history), SiLU
  norms    k^ = k/sqrt(|k|^2+eps2), q^ = s q/sqrt(|q|^2+eps2)
  gates    alpha = exp(-exp(A) softplus(g)) per key channel, beta = sigmoid(b)
  state    S_t = (I - beta k^ k^T) diag(alpha) S_{t-1} + beta k^ v^T
  readout  o_t = S_t^T q^
  output   y = o / sqrt(mean(o^2) + eps_r) * w_norm * sigmoid(z)

The chunked form (``core_chunked``) restates the same recurrence over a chunk
of C tokens with the start state S0, per key channel log-decay prefix sums
G_t = sum_{r<=t} log alpha_r:
  A[t,s] = beta_t sum_c k_tc k_sc exp(G_tc - G_sc)       (s < t)
  P[t,s] = sum_c q_tc k_sc exp(G_tc - G_sc)               (s <= t)
  T = (I + A)^-1,  W = T diag(beta) (K * exp(G)),  U~ = T diag(beta) V
  U = U~ - W S0,   O = (Q * exp(G)) S0 + P U
  S_C = diag(exp(G_C)) S0 + (K * exp(G_C - G))^T U
It is derived from the recurrence by unrolling it over the chunk (the U rows
are the per-token corrections beta_t (v_t - (diag(alpha_t) S_{t-1})^T k^_t)).
parity: pinned against the sequential recurrence by brute force in the tests.
"""
from __future__ import annotations

import numpy as np
from scipy.special import expit


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


class Layer:
    """Parameters of one KDA layer, in fp64.

    A [H, d_k], conv_wt [H, 2 d_k + d_v, W] (q | k | v channels, tap 0 the
    oldest), norm_w [H, d_v]."""

    def __init__(self, A, conv_wt, norm_w, q_scale=None, l2_eps=1e-6,
                 rms_eps=1e-6, conv_silu=True):
        self.A = _f64(A)
        self.conv_wt = _f64(conv_wt)
        self.norm_w = _f64(norm_w)
        self.H, self.d_k = self.A.shape
        self.d_v = self.norm_w.shape[1]
        self.conv_w = self.conv_wt.shape[2]
        assert self.conv_wt.shape[:2] == (self.H, 2 * self.d_k + self.d_v)
        self.q_scale = float(self.d_k ** -0.5 if q_scale is None else q_scale)
        self.l2_eps = float(l2_eps)
        self.rms_eps = float(rms_eps)
        self.conv_silu = bool(conv_silu)

    def heads(self, idx):
        """The same layer restricted to the heads in ``idx`` (heads are
        independent, so a head subset is an exact sub-problem)."""
        idx = np.asarray(idx)
        return Layer(self.A[idx], self.conv_wt[idx], self.norm_w[idx], self.q_scale,
                     self.l2_eps, self.rms_eps, self.conv_silu)


def preprocess(layer: Layer, window, x_q, x_k, x_v, g, b):
    """Conv + activation, L2 norms and gates for every token.

    window [B, H, W-1, C_h]; x_q, x_k, g [B, T, H, d_k]; x_v [B, T, H, d_v];
    b [B, T, H].  Returns q^, k^ [B, T, H, d_k], v [B, T, H, d_v],
    log_alpha [B, T, H, d_k], beta [B, T, H] and the window after all T tokens.
    """
    dk, W = layer.d_k, layer.conv_w
    x = np.concatenate([_f64(x_q), _f64(x_k), _f64(x_v)], axis=-1)    # [B,T,H,Ch]
    hist = np.concatenate([np.moveaxis(_f64(window), 2, 1), x], axis=1)  # [B,W-1+T,H,Ch]
    T = x.shape[1]
    conv = np.zeros_like(x)
    for j in range(W):
        # tap j multiplies the input W-1-j tokens before the current one
        conv += layer.conv_wt[None, None, :, :, j] * hist[:, j:j + T]
    act = conv * expit(conv) if layer.conv_silu else conv
    q, k, v = act[..., :dk], act[..., dk:2 * dk], act[..., 2 * dk:]
    qn = q * (layer.q_scale / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + layer.l2_eps))
    kn = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + layer.l2_eps)
    log_alpha = -np.exp(layer.A)[None, None] * np.logaddexp(0.0, _f64(g))
    beta = expit(_f64(b))
    new_window = np.moveaxis(hist[:, T:], 1, 2).copy() if W > 1 else _f64(window).copy()
    return qn, kn, v, log_alpha, beta, new_window


def output_norm(layer: Layer, o, z):
    """RMSNorm over d_v, weight, sigmoid output gate.  o, z [..., H, d_v]."""
    ms = np.mean(o * o, axis=-1, keepdims=True)
    return o / np.sqrt(ms + layer.rms_eps) * layer.norm_w * expit(_f64(z))


def core_sequential(qn, kn, v, log_alpha, beta, S0, lens=None, snapshots=False):
    """Token-by-token recurrence, vectorised over (B, H).

    Shapes as returned by ``preprocess``; S0 [B, H, d_k, d_v].  Returns
    o [B, T, H, d_v], the final state and (optionally) the state after every
    token [B, T, H, d_k, d_v].  Sequence b stops after lens[b] tokens."""
    B, T = qn.shape[:2]
    S = _f64(S0).copy()
    o = np.zeros(v.shape, dtype=np.float64)
    snaps = np.zeros((B, T) + S.shape[1:]) if snapshots else None
    for t in range(T):
        alpha = np.exp(log_alpha[:, t])                               # [B,H,dk]
        Sd = alpha[..., :, None] * S
        u = np.einsum('bhij,bhi->bhj', Sd, kn[:, t])
        Snew = Sd + beta[:, t, :, None, None] * np.einsum('bhi,bhj->bhij', kn[:, t], v[:, t] - u)
        if lens is not None:
            live = (t < np.asarray(lens))[:, None, None, None]
            Snew = np.where(live, Snew, S)
        S = Snew
        o[:, t] = np.einsum('bhij,bhi->bhj', S, qn[:, t])
        if snapshots:
            snaps[:, t] = S
    return o, S, snaps


def core_chunked(qn, kn, v, log_alpha, beta, S0, chunk):
    """The same recurrence for ONE (sequence, head) in the chunked WY/UT form.

    qn, kn, log_alpha [T, d_k]; v [T, d_v]; beta [T]; S0 [d_k, d_v].
    Returns o [T, d_v], the final state and the per-chunk intermediates of the
    last chunk (A, P, Tinv, W, Ut, U) for stage-by-stage debugging."""
    T = qn.shape[0]
    S = _f64(S0).copy()
    o = np.zeros((T, v.shape[1]))
    inter = {}
    for c0 in range(0, T, chunk):
        n = min(chunk, T - c0)
        q, k, vv, la, bt = (qn[c0:c0 + n], kn[c0:c0 + n], v[c0:c0 + n],
                            log_alpha[c0:c0 + n], beta[c0:c0 + n])
        G = np.cumsum(la, axis=0)                                     # [n, dk]
        D = G[:, None, :] - G[None, :, :]                             # [t, s, dk]
        tt, ss = np.meshgrid(np.arange(n), np.arange(n), indexing='ij')
        E_lt = np.exp(np.where((ss < tt)[..., None], D, -np.inf))
        E_le = np.exp(np.where((ss <= tt)[..., None], D, -np.inf))
        A = bt[:, None] * np.einsum('tc,sc,tsc->ts', k, k, E_lt)
        P = np.einsum('tc,sc,tsc->ts', q, k, E_le)
        Tinv = np.linalg.inv(np.eye(n) + A)
        Wm = Tinv @ (bt[:, None] * (k * np.exp(G)))
        Ut = Tinv @ (bt[:, None] * vv)
        U = Ut - Wm @ S
        o[c0:c0 + n] = (q * np.exp(G)) @ S + P @ U
        S = np.exp(G[-1])[:, None] * S + (k * np.exp(G[-1][None, :] - G)).T @ U
        inter = dict(A=A, P=P, Tinv=Tinv, W=Wm, Ut=Ut, U=U)
    return o, S, inter


def run(layer: Layer, state, window, x_q, x_k, x_v, g, b, z, lens=None,
        snapshots=False, chunk=None):
    """Full pipeline.  With ``chunk`` set, the core runs in the chunked form
    (one (sequence, head) at a time; ``lens`` is not supported there)."""
    qn, kn, v, la, beta, new_window = preprocess(layer, window, x_q, x_k, x_v, g, b)
    if chunk is None:
        o, S, snaps = core_sequential(qn, kn, v, la, beta, state, lens, snapshots)
    else:
        assert lens is None and not snapshots
        B, T, H = qn.shape[:3]
        o = np.zeros(v.shape)
        S = np.zeros(_f64(state).shape)
        for bi in range(B):
            for h in range(H):
                o[bi, :, h], S[bi, h], _ = core_chunked(
                    qn[bi, :, h], kn[bi, :, h], v[bi, :, h], la[bi, :, h],
                    beta[bi, :, h], _f64(state)[bi, h], chunk)
        snaps = None
    y = output_norm(layer, o, z)
    if lens is not None:
        # window of a shortened sequence: redo the preprocessing on its prefix
        new_window = new_window.copy()
        for bi, n in enumerate(lens):
            _, _, _, _, _, wb = preprocess(layer, _f64(window)[bi:bi + 1],
                                           x_q[bi:bi + 1, :n], x_k[bi:bi + 1, :n],
                                           x_v[bi:bi + 1, :n], g[bi:bi + 1, :n],
                                           b[bi:bi + 1, :n])
            new_window[bi] = wb[0]
    return dict(y=y, o=o, state=S, window=new_window, snap_state=snaps)
