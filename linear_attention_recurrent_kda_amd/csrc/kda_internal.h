// kda_internal.h -- launch parameters and launchers shared between the C-ABI
// front end (kda_api.hip) and the kernel files.  Host-side only types.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

// Everything a token-recurrent kernel (decode, verify) needs, flattened.
struct RecParams {
    // layer
    const float *A, *conv_wt, *norm_w;
    float q_scale, l2_eps, rms_eps;
    int silu;
    int stream_state;           // non-temporal state loads / stores
    // cache
    float *state;
    void *window;
    int n_slots;
    int32_t *err_flag;
    // tables
    const int32_t *slot_idx;    // [B]
    const int32_t *snap_slots;  // [B, T] (verify)
    const int32_t *draft_len;   // [B] or null (verify)
    void *delta;                // replay records (verify, delta mode)
    // inputs, rows n = b (decode) or b*T + t (verify)
    const void *x_q, *x_k, *x_v, *g, *b, *z;
    float *y;
    int B, H, T;
    // decode of the one-token sequences of a packed prefill call: sequence b
    // is token row seq_start[b] (inputs and y); only sequences with
    // seq_start[b + 1] - seq_start[b] == 1 are processed, and only when
    // *seq_ok == 1 (null: plain decode)
    const int32_t *seq_start;
    const int32_t *seq_ok;
};

struct CommitParams {
    float *state;
    void *window;
    int n_slots;
    int32_t *err_flag;
    const int32_t *slot_idx, *snap_slots, *accepted_len;
    int B, H, T;
    int state_elems;   // d_k * d_v
    int window_words;  // (conv_w - 1) * C_h * sizeof(input) / 4
};

// Delta commit: replay accepted records onto the live slots.
struct CommitDeltaParams {
    float *state;
    void *window;
    int n_slots;
    int32_t *err_flag;
    int stream_state;
    const int32_t *slot_idx, *accepted_len;
    const void *delta;          // records of kda_spec_verify_delta
    int B, H, T;
};

struct PrefillParams {
    // layer
    const float *A, *conv_wt, *norm_w;
    float q_scale, l2_eps, rms_eps;
    int silu;
    // cache
    float *state;
    void *window;
    int n_slots;
    int32_t *err_flag;
    const int32_t *slot_idx, *cu_seqlens;
    int N_seq, total_T, chunk, H;
    const void *x_q, *x_k, *x_v, *g, *b, *z;
    float *y;
    void *workspace;
    size_t workspace_bytes;
    // interval checkpoints: state and window after every ckpt_interval tokens
    // of sequence s go to ckpt_slots[s * ckpt_per_seq + j] (null: none)
    const int32_t *ckpt_slots;
    int ckpt_interval, ckpt_per_seq;
};

// Per-step batch metadata (kda_build_metadata).
struct MetaParams {
    const int32_t *num_tokens, *req_slot;   // [n_req]
    int n_req, n_slots;
    int32_t *cu_seqlens;    // [n_req + 1]
    int32_t *slot_idx;      // [n_req]
    int32_t *chunk_start;   // [n_req + 1]
    int32_t *counts;        // [4]
    int32_t *err_flag;      // optional
};

// most draft tokens per verification
constexpr int kMaxDraft = 16;

enum class RecKind { decode, verify, verify_delta };

kda_status launch_recurrent(const RecParams &p, int d_k, int d_v, kda_dtype dt, RecKind kind,
                            hipStream_t stream);
kda_status launch_commit(const CommitParams &p, hipStream_t stream);
kda_status launch_commit_delta(const CommitDeltaParams &p, int d_k, int d_v, kda_dtype dt,
                               hipStream_t stream);
// bytes of one (sequence, token, head) replay record
size_t spec_delta_record_bytes(int d_k, int d_v, kda_dtype dt);
kda_status launch_prefill(const PrefillParams &p, int d_k, int d_v, kda_dtype dt,
                          hipStream_t stream);
size_t prefill_workspace_bytes(int H, int d_k, int d_v, int total_T, int N_seq, int chunk);
kda_status launch_copy_probe(float *dst, const float *src, size_t n, hipStream_t stream);
kda_status launch_build_metadata(const MetaParams &p, hipStream_t stream);

}  // namespace kda
