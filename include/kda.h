/*
 * kda.h -- C ABI of libkda.so: the Kimi Delta Attention (KDA) recurrent-state
 * update on AMD MI355X (gfx950).
 *
 * What the operation is.  "vLLM Kimi K3 support" (section "Kimi K3
 * architecture overview", KDA bullet) describes KDA as a linear-attention
 * layer that keeps a fixed-size recurrent state per head; its section "Fused
 * kernels and metadata optimisation" (KDA decode bullet) says one decode
 * launch runs the short causal convolution, the recurrent update and RMSNorm
 * so that the state is not re-read; "Kimi K3 vLLM GPU inference benchmark"
 * (time-breakdown section) keeps that state in fp32 ("FP32 SSM cache").  The
 * pages give no formulas.  Per (sequence b, head h, token t) this library
 * computes:
 *
 *   conv     y_c = sum_{j<4} w[h][c][j] * x_c(t-3+j)   (tap 0 oldest), SiLU
 *            over the 2*d_k + d_v channels q | k | v of the head;
 *   norms    k^ = k / sqrt(|k|^2 + l2_eps),  q^ = q_scale * q / sqrt(|q|^2 + l2_eps)
 *   gates    alpha_i = exp(-exp(A[h][i]) * softplus(g_i)),  beta = sigmoid(b)
 *   state    S <- (I - beta k^ k^T) diag(alpha) S + beta k^ v^T   (d_k x d_v)
 *   readout  o = S^T q^   (the updated state)
 *   output   y = o / sqrt(mean(o^2) + rms_eps) * norm_w[h] * sigmoid(z)
 *
 * The compact per-request state blocks of the hybrid cache ("vLLM Kimi K3
 * support", section "Hybrid KV-cache management") are modelled as a pool of
 * fp32 state slots plus a pool of conv windows, addressed by an int32 slot
 * table.
 *
 * Conventions for every call
 *   - Tensor pointers are DEVICE pointers to row-major, contiguous arrays;
 *     the caller owns them.  The library allocates nothing, keeps no pointer
 *     after a call returns and holds no mutable global state (reentrant),
 *     except for kda_chunk_prefill_static and its static workspace.
 *   - Calls are asynchronous on `hip_stream` (a hipStream_t; NULL = the
 *     default stream).  The returned status covers host-side validation,
 *     done before any HIP call, and the launch itself; it never waits for
 *     the GPU.
 *   - Base pointers of state, conv_state, x_q, x_k, x_v, g, z, y, A, conv_wt,
 *     norm_w and workspace must be 16-byte aligned; int32 tables 4-byte.
 *   - Slot tables: -1 marks a padding row (nothing read or written except
 *     zeros to its outputs).  Any other index outside [0, n_slots) is a caller
 *     error found on the device: the row is skipped (outputs zeroed) and, if
 *     cache->err_flag is set, 1 is stored there.  Two rows of one call naming
 *     the same slot, or snapshot slots that alias live slots, are undefined.
 *   - Shapes: d_k, d_v in {64, 128}; conv_w = 4; H >= 1.
 *   - Debug validation: with the environment variable KDA_CHECK=1 every call
 *     first copies its slot tables (slot_idx, snap_slots, ckpt_slots) to the
 *     host on hip_stream, synchronising it, and returns KDA_ERR_SHAPE for an
 *     entry outside [-1, n_slots) or KDA_ERR_ALIAS when two non-negative
 *     entries coincide (two rows on one slot; a snapshot or checkpoint slot
 *     on a live slot or on another one); nothing is launched then.  Not for
 *     serving or graph capture (it synchronises).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 2

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,        /* a required pointer is NULL                     */
    KDA_ERR_SHAPE = 2,       /* a size is out of range                         */
    KDA_ERR_DTYPE = 3,       /* unknown input dtype                            */
    KDA_ERR_ALIGN = 4,       /* a pointer breaks the alignment rule            */
    KDA_ERR_UNSUPPORTED = 5, /* valid but not built (d_k, d_v, conv_w, flags)   */
    KDA_ERR_WORKSPACE = 6,   /* workspace smaller than the size query returns  */
    KDA_ERR_LAUNCH = 7,      /* the HIP launch reported an error               */
    KDA_ERR_ALIAS = 8        /* KDA_CHECK only: slot tables alias (see below)  */
} kda_status;

typedef enum kda_dtype {
    KDA_F32 = 0,             /* float32 inputs and conv window                 */
    KDA_BF16 = 1             /* bfloat16 inputs and conv window                */
} kda_dtype;

/* flags */
#define KDA_CONV_SILU 1u     /* SiLU after the conv (the usual setting)        */
#define KDA_STREAM_STATE 2u  /* decode, verify, delta commit: non-temporal
                                state loads and stores (raw buffer operations
                                with the streaming cache policy).  Results are
                                bitwise identical under every cache policy.
                                Verify and the delta commit stream only when
                                it is set; for kda_decode see below.          */
#define KDA_STATE_RESIDENT 4u /* decode only, a residency hint: the states of
                                the call stay cache-resident until the same
                                slots are decoded again (e.g. one layer re-run
                                back to back whose state fits the 256 MB
                                Infinity Cache), so keep them in the caches.
                                kda_decode's cache policy for the state tiles:
                                  - KDA_STREAM_STATE set: streamed;
                                  - else a call of at most 4 MiB of state
                                    (B * H * d_k * d_v * 4 bytes; one or two
                                    sequences at H = 32, d = 128, whose states
                                    across all layers of a model fit the
                                    Infinity Cache together): cached;
                                  - else KDA_STATE_RESIDENT set and at most
                                    256 MiB of state: cached;
                                  - else streamed: in a serving step over many
                                    KDA layers each layer's states are evicted
                                    before its next step.
                                On MI355X at B = 64, H = 32, d = 128 a step
                                over evicted states took 51 us streamed and
                                61 us cached; a cache-resident one 44 us
                                cached and 51 us streamed.                     */

/* Parameters of one KDA layer (device pointers, fp32). */
typedef struct kda_layer {
    int32_t H, d_k, d_v, conv_w;
    const float *A;          /* [H, d_k]  decay log-rate                        */
    const float *conv_wt;    /* [H, 2*d_k + d_v, conv_w]  q|k|v, tap 0 oldest    */
    const float *norm_w;     /* [H, d_v]  RMSNorm weight                        */
    float q_scale;           /* usually d_k^-1/2                                */
    float l2_eps;            /* usually 1e-6                                    */
    float rms_eps;           /* usually 1e-6                                    */
    uint32_t flags;          /* KDA_CONV_SILU | KDA_STREAM_STATE | KDA_STATE_RESIDENT */
} kda_layer;

/* The recurrent-state pools (device pointers). */
typedef struct kda_cache {
    float *state;            /* [n_slots, H, d_k, d_v] fp32                     */
    void *conv_state;        /* [n_slots, H, conv_w-1, 2*d_k + d_v], input dtype;
                                row 0 oldest; holds raw (pre-conv) inputs      */
    int32_t n_slots;
    int32_t *err_flag;       /* optional device int32; 1 on a bad slot index   */
} kda_cache;

/* Per-token inputs (device pointers, all of `dtype`), N tokens:
 * x_q, x_k, g [N, H, d_k]; x_v, z [N, H, d_v]; b [N, H]. */
typedef struct kda_inputs {
    const void *x_q, *x_k, *x_v, *g, *b, *z;
    kda_dtype dtype;
} kda_inputs;

/*
 * kda_decode -- one token for each of B sequences (the fused decode launch of
 * "vLLM Kimi K3 support", section "Fused kernels and metadata optimisation").
 *   slot_idx [B] int32: the state/window slot of each sequence.
 *   inputs: N = B tokens, token b belongs to sequence b.
 *   y [B, H, d_v] fp32 output.
 * The state and window at slot_idx[b] are read once and updated in place.
 * B = 0 is a no-op.
 */
kda_status kda_decode(const kda_layer *layer, const kda_cache *cache,
                      const int32_t *slot_idx, int32_t B,
                      const kda_inputs *inputs, float *y, void *hip_stream);

/*
 * kda_spec_verify -- target-side verification of T draft tokens per sequence
 * (the speculative decoding of "vLLM Kimi K3 support", section "Speculative
 * decoding with DSpark"; 3-7 and 8 draft tokens per step are quoted there and
 * in "Kimi K3 vLLM GPU inference benchmark").  The T tokens of a sequence
 * are processed in order from the state at slot_idx[b], which is NOT modified.
 *   snap_slots [B, T] int32: after token t the state and window are written
 *     to slot snap_slots[b*T + t] (-1: not kept).
 *   draft_len [B] int32 or NULL (= T): sequence b processes its first
 *     draft_len[b] tokens; y of the remaining tokens is zeroed.
 *   inputs: N = B*T tokens, token (b, t) at row b*T + t.
 *   y [B, T, H, d_v] fp32.
 * 1 <= T <= 16.  The per-token arithmetic is the same code as kda_decode, so
 * verify + commit(L) is bitwise equal to L decode calls.
 */
kda_status kda_spec_verify(const kda_layer *layer, const kda_cache *cache,
                           const int32_t *slot_idx, const int32_t *snap_slots,
                           int32_t B, int32_t T, const int32_t *draft_len,
                           const kda_inputs *inputs, float *y, void *hip_stream);

/*
 * kda_spec_commit -- keep the accepted prefix of a verification: after the
 * target model has checked the draft tokens ("vLLM Kimi K3 support", section
 * "Speculative decoding with DSpark"), the KDA state of each sequence must be
 * the state after its accepted tokens (the pages do not say how a rejected
 * suffix is undone; here the accepted token's snapshot is copied back).
 *   accepted_len [B] int32 (device), each in [0, T]: copies the state and
 *   window snapshot of token accepted_len[b]-1 (snap_slots[b*T + L-1]) into
 *   slot_idx[b]; L = 0 keeps the pre-verify state (no copy).  A length
 *   outside [0, T], or a needed snapshot slot of -1 / out of range, sets
 *   err_flag and leaves that sequence untouched.
 *   L must not exceed the draft_len[b] the verification ran with: snapshots
 *   past it were not written by that verification, and the copy cannot tell
 *   (it would copy whatever the slot holds).  snap_slots and T must be the
 *   ones the verification used; window_dtype is the conv_state dtype.
 */
kda_status kda_spec_commit(const kda_layer *layer, const kda_cache *cache,
                           const int32_t *slot_idx, const int32_t *snap_slots,
                           const int32_t *accepted_len, int32_t B, int32_t T,
                           kda_dtype window_dtype, void *hip_stream);

/*
 * Replayable-delta verification: the same verification as kda_spec_verify,
 * but instead of a full state snapshot per token (d_k*d_v*4 bytes) it keeps a
 * small replay record per (sequence, token, head), and the commit re-applies
 * the accepted records to the live state.  The verification of draft tokens
 * is that of "vLLM Kimi K3 support", section "Speculative decoding with
 * DSpark"; the pages do not say how a rejected suffix is rolled back, and
 * this form moves about a sixth of the snapshot form's bytes per verified
 * token at d_k = d_v = 128.
 *
 * Record layout.  The record buffer is [B, T, H] records of
 * kda_spec_delta_bytes(layer, 1, 1, dtype) / H bytes each = (2 d_k + d_v) *
 * (4 + sizeof(input)) bytes, record (b, t, h) at index (b*T + t)*H + h:
 *   float alpha[d_k];    per-channel decay of the token
 *   float khat[d_k];     the normalised key k^
 *   float d[d_v];        beta * (v - S'^T k^): the rank-one update's row
 *   input x[2d_k + d_v]; the token's raw (pre-conv) inputs q | k | v
 * so that the state after the token is diag(alpha) S + khat d^T, evaluated
 * in fp32 with the same two roundings per element as kda_decode.
 */

/* Bytes of the record buffer for B sequences x T draft tokens (0 on invalid
 * sizes: 1 <= T <= 16, B >= 0, a valid layer and dtype). */
size_t kda_spec_delta_bytes(const kda_layer *layer, int32_t B, int32_t T, kda_dtype dtype);

/*
 * kda_spec_verify_delta -- verify T draft tokens per sequence from the state
 * at slot_idx[b] (NOT modified), writing y [B, T, H, d_v] fp32 exactly as
 * kda_spec_verify does (bitwise) and one replay record per processed token
 * into `delta` (delta_bytes >= kda_spec_delta_bytes(layer, B, T, dtype),
 * 16-byte aligned).  draft_len [B] or NULL as in kda_spec_verify: records of
 * tokens past draft_len[b] are not written.  Padding (-1) and bad slots as for
 * decode.  Errors: KDA_ERR_WORKSPACE when delta_bytes is too small.
 */
kda_status kda_spec_verify_delta(const kda_layer *layer, const kda_cache *cache,
                                 const int32_t *slot_idx, int32_t B, int32_t T,
                                 const int32_t *draft_len, const kda_inputs *inputs,
                                 float *y, void *delta, size_t delta_bytes,
                                 void *hip_stream);

/*
 * kda_spec_commit_delta -- keep the accepted prefix of a delta verification.
 *   accepted_len [B] int32 (device), each in [0, T]: replays records
 *   0 .. L-1 of sequence b onto the state at slot_idx[b] and sets its conv
 *   window to the last three raw inputs of (window, accepted tokens).  The
 *   result is bitwise equal to L kda_decode calls (and to kda_spec_commit
 *   after kda_spec_verify).  L = 0 and slot -1 are no-ops; a length outside
 *   [0, T] or a bad slot sets err_flag and leaves that sequence untouched.
 *   L must not exceed the draft_len the verification ran with (later records
 *   were not written).  `dtype` is the input (and window) dtype of the
 *   verification; T, B and `delta` must be the ones it was called with.
 *   The live slot must not have changed since the verification.
 */
kda_status kda_spec_commit_delta(const kda_layer *layer, const kda_cache *cache,
                                 const int32_t *slot_idx, const void *delta,
                                 size_t delta_bytes, const int32_t *accepted_len,
                                 int32_t B, int32_t T, kda_dtype dtype,
                                 void *hip_stream);

/*
 * kda_chunk_prefill -- many tokens per sequence in chunks (the prefill path,
 * "vLLM Kimi K3 support", section "Fused kernels and metadata optimisation",
 * KDA prefill bullet).  Same result as running the tokens one by one; inside
 * a chunk the recurrence is solved in closed form (WY/UT form) with the
 * contractions on MFMA, and the fp32 state is carried from chunk to chunk.
 *   slot_idx [N_seq] int32; cu_seqlens [N_seq + 1] int32 (device) with
 *   cu_seqlens[0] = 0, non-decreasing, cu_seqlens[N_seq] = total_T.
 *   inputs: total_T tokens; y [total_T, H, d_v] fp32.
 *   chunk: 64.  workspace: >= kda_chunk_prefill_workspace_bytes(...).
 * The state and window at slot_idx[s] are the start state (zero them for a
 * fresh sequence) and are replaced by the final ones.  A batch may mix
 * prompts with one-token (decode) rows: sequences of exactly one token take
 * the decode kernel of kda_decode inside this call (bitwise the results of
 * kda_decode on those rows), so a mixed prefill + decode batch is one call.  total_T = 0 is
 * allowed: inputs' pointers and y are then not read and may be NULL (the
 * dtype must still be valid); cu_seqlens is still checked.
 * Concurrency: the workgroups that hold one head's output columns exchange
 * row sums for the RMSNorm and wait for each other (at most one workgroup
 * per compute unit is launched, so on a GPU free of other work they all run
 * at once).  Each wait is bounded (about 25 ms): rows whose sums did not
 * come in time are normalised by a small kernel after the scan, with the
 * same arithmetic (bitwise the same results), so other work on the GPU
 * (another prefill call on another stream, say) costs time, not
 * correctness.  The bound is read from the environment variable KDA_XP_SPIN
 * at each call if set (polls; a negative value takes no row as in time):
 * a testing knob.
 */
kda_status kda_chunk_prefill(const kda_layer *layer, const kda_cache *cache,
                             const int32_t *slot_idx, const int32_t *cu_seqlens,
                             int32_t N_seq, int32_t total_T, int32_t chunk,
                             const kda_inputs *inputs, float *y,
                             void *workspace, size_t workspace_bytes,
                             void *hip_stream);

/*
 * kda_chunk_prefill_ckpt -- kda_chunk_prefill that also keeps interval
 * checkpoints of each sequence's state.  The interval-based retention of
 * "vLLM Kimi K3 support" (section "Agentic cache retention policies")
 * checkpoints the KDA state at a fixed token interval (32K tokens is its
 * example) and at prompt boundaries; the prompt-boundary state is the final
 * state this call leaves in the live slot, and this call adds the interval
 * ones (read here as: a later request that shares the first (j+1)*interval
 * tokens can start from checkpoint j).
 *   ckpt_interval: tokens between checkpoints, a positive multiple of chunk.
 *   ckpt_slots [N_seq, ckpt_per_seq] int32 (device): after the first
 *     (j+1)*ckpt_interval tokens of sequence s, its state and conv window are
 *     written to slot ckpt_slots[s*ckpt_per_seq + j] (-1: not kept), for
 *     j < min(ckpt_per_seq, len_s / ckpt_interval).  Other indices outside
 *     [0, n_slots) set err_flag and are skipped.  Checkpoint slots must not
 *     alias each other or any live slot of the call.
 * Everything else (outputs, final state, errors) is exactly kda_chunk_prefill;
 * a checkpoint equals the state a prefill of that many tokens would leave.
 * Errors: KDA_ERR_NULL for a NULL ckpt_slots, KDA_ERR_SHAPE for ckpt_per_seq
 * < 1 or an interval that is not a positive multiple of chunk.
 */
kda_status kda_chunk_prefill_ckpt(const kda_layer *layer, const kda_cache *cache,
                                  const int32_t *slot_idx, const int32_t *cu_seqlens,
                                  int32_t N_seq, int32_t total_T, int32_t chunk,
                                  const kda_inputs *inputs, float *y,
                                  const int32_t *ckpt_slots, int32_t ckpt_interval,
                                  int32_t ckpt_per_seq, void *workspace,
                                  size_t workspace_bytes, void *hip_stream);

/*
 * kda_chunk_prefill_static -- kda_chunk_prefill for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It takes no workspace: the call runs in
 * a device array of KDA_STATIC_WORKSPACE_BYTES inside the library (one per
 * GPU the library runs on, held until the process ends; its address is
 * looked up on the first call on each device, which must be the current
 * device).  Nothing is allocated or freed.  A call whose workspace
 * (kda_chunk_prefill_workspace_bytes) exceeds the array returns
 * KDA_ERR_WORKSPACE before any HIP call (at H = 32, d_k = d_v = 128 the array
 * holds one sequence of up to about 3500 tokens, or somewhat fewer tokens
 * over several sequences).  Every call on one GPU shares that GPU's array: calls
 * that overlap on one GPU (several streams, several host threads) race and
 * must be serialised by the caller.  Arguments, results and errors are
 * otherwise exactly those of kda_chunk_prefill.
 */
#define KDA_STATIC_WORKSPACE_BYTES ((size_t)256 << 20)
kda_status kda_chunk_prefill_static(const kda_layer *layer, const kda_cache *cache,
                                    const int32_t *slot_idx, const int32_t *cu_seqlens,
                                    int32_t N_seq, int32_t total_T, int32_t chunk,
                                    const kda_inputs *inputs, float *y, void *hip_stream);

/* Bytes of device workspace kda_chunk_prefill and kda_chunk_prefill_ckpt
 * need for total_T tokens in N_seq sequences (0 on invalid sizes: chunk must
 * be 64, total_T >= 0, N_seq >= 1, a valid layer).  The workspace holds the
 * per-chunk factors of the chunked form of the prefill ("vLLM Kimi K3
 * support", section "Fused kernels and metadata optimisation", KDA prefill
 * bullet) between its kernels; its contents need no initialisation and are
 * of no use after the call. */
size_t kda_chunk_prefill_workspace_bytes(const kda_layer *layer, int32_t total_T,
                                         int32_t N_seq, int32_t chunk);

/*
 * kda_build_metadata -- the per-step tables of a batch, built on the device
 * in one launch ("vLLM Kimi K3 support", section "Fused kernels and metadata
 * optimisation", metadata builder bullet: one fused kernel instead of a chain
 * of eager tensor operations).  The tables depend on the batch only, so one
 * build serves every KDA layer of the step.  Inputs, per request r of the
 * step (device int32 [n_req]):
 *   num_tokens[r]  tokens scheduled for r this step (0: none; below 0 is a
 *                  caller error, taken as 0);
 *   req_slot[r]    r's state / conv-window slot, or -1.
 * Outputs (device int32, written in full):
 *   cu_seqlens[n_req + 1]   packed token offsets: cu_seqlens[0] = 0,
 *                           cu_seqlens[r + 1] = cu_seqlens[r] + tokens of r
 *                           (the kda_chunk_prefill argument);
 *   slot_idx[n_req]         req_slot[r] when r has tokens and its slot is in
 *                           [0, n_slots), else -1 (a padding row: its tokens'
 *                           outputs are zeroed, no state is touched);
 *   chunk_start[n_req + 1]  first 64-token chunk of r in the chunked prefill:
 *                           requests of two or more tokens with a slot take
 *                           ceil(tokens / 64) chunks, all others none;
 *   counts[4]               total tokens, one-token requests with a slot (the
 *                           decode rows of a mixed batch), requests of two or
 *                           more tokens with a slot, total chunks.
 * A negative count or a slot outside [-1, n_slots) stores 1 to err_flag
 * (optional device int32).  The total token count must fit in int32.
 * n_req = 0 writes cu_seqlens[0] = chunk_start[0] = 0 and zero counts (the
 * input pointers and slot_idx may then be NULL).  Errors: KDA_ERR_SHAPE for
 * n_req < 0 or n_slots <= 0, KDA_ERR_NULL, KDA_ERR_ALIGN (4-byte tables).
 */
kda_status kda_build_metadata(const int32_t *num_tokens, const int32_t *req_slot, int32_t n_req,
                              int32_t n_slots, int32_t *cu_seqlens, int32_t *slot_idx,
                              int32_t *chunk_start, int32_t *counts, int32_t *err_flag,
                              void *hip_stream);

/* Measurement helper: dst[i] = src[i] for n floats, moved the way the
 * decode moves its state tiles (64 KiB per workgroup, 16-byte non-temporal
 * loads and stores, at most three workgroups per CU, 2 MiB granules in a
 * scrambled order): a streaming copy of known size that calibrates
 * memory-traffic counters and gives a copy ceiling next to the KDA kernels.
 * dst may equal src: the data is then read and rewritten in place, the
 * decode's own access pattern.  Other overlaps are undefined.  n = 0 is a
 * no-op. */
kda_status kda_copy_probe(float *dst, const float *src, size_t n, void *hip_stream);

/* Static text for a status code. */
const char *kda_status_string(kda_status status);

/* KDA_ABI_VERSION of the built library. */
int32_t kda_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
