// kda_api.hip -- the extern "C" entry points of libkda.so (declared in
// include/kda.h): host-side argument validation, then dispatch to the
// launchers.  Validation runs before any HIP call, so every error status is
// returned without touching the device.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "kda_internal.h"

#define KDA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

using namespace kda;

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool finite_nonneg(float x) { return isfinite(x) && x >= 0.f; }

size_t elem_size(kda_dtype dt) { return dt == KDA_BF16 ? 2 : 4; }

// size of the static workspace of kda_chunk_prefill_static (KDA_STATIC_WORKSPACE_BYTES)
constexpr size_t kStaticWorkspaceBytes = KDA_STATIC_WORKSPACE_BYTES;

// states of one call above this size cannot stay in the 256 MB Infinity
// Cache: kda_decode streams them even under KDA_STATE_RESIDENT
constexpr size_t kResidentMaxBytes = (size_t)256 << 20;
// kda_decode keeps calls of at most this many state bytes cached by default:
// a few sequences' states of every layer of a model fit the Infinity Cache
// together (256 MB holds 128 layers of one sequence at H = 32, d = 128)
constexpr size_t kCachedDefaultBytes = (size_t)4 << 20;

kda_status check_layer(const kda_layer *L) {
    if (!L) return KDA_ERR_NULL;
    if (!L->A || !L->conv_wt || !L->norm_w) return KDA_ERR_NULL;
    if (L->H <= 0 || L->d_k <= 0 || L->d_v <= 0 || L->conv_w <= 0) return KDA_ERR_SHAPE;
    if (!((L->d_k == 64 || L->d_k == 128) && (L->d_v == 64 || L->d_v == 128))) return KDA_ERR_UNSUPPORTED;
    if (L->conv_w != 4) return KDA_ERR_UNSUPPORTED;
    if (L->flags & ~(KDA_CONV_SILU | KDA_STREAM_STATE | KDA_STATE_RESIDENT)) return KDA_ERR_UNSUPPORTED;
    if (!isfinite(L->q_scale) || !finite_nonneg(L->l2_eps) || !finite_nonneg(L->rms_eps))
        return KDA_ERR_SHAPE;
    if (!aligned(L->A, 16) || !aligned(L->conv_wt, 16) || !aligned(L->norm_w, 16)) return KDA_ERR_ALIGN;
    return KDA_OK;
}

kda_status check_cache(const kda_cache *C) {
    if (!C) return KDA_ERR_NULL;
    if (!C->state || !C->conv_state) return KDA_ERR_NULL;
    if (C->n_slots <= 0) return KDA_ERR_SHAPE;
    if (!aligned(C->state, 16) || !aligned(C->conv_state, 16)) return KDA_ERR_ALIGN;
    if (C->err_flag && !aligned(C->err_flag, 4)) return KDA_ERR_ALIGN;
    return KDA_OK;
}

kda_status check_inputs(const kda_inputs *in) {
    if (!in) return KDA_ERR_NULL;
    if (in->dtype != KDA_F32 && in->dtype != KDA_BF16) return KDA_ERR_DTYPE;
    if (!in->x_q || !in->x_k || !in->x_v || !in->g || !in->b || !in->z) return KDA_ERR_NULL;
    if (!aligned(in->x_q, 16) || !aligned(in->x_k, 16) || !aligned(in->x_v, 16) ||
        !aligned(in->g, 16) || !aligned(in->z, 16) || !aligned(in->b, elem_size(in->dtype)))
        return KDA_ERR_ALIGN;
    return KDA_OK;
}

// ---------------------------------------------------------------------------
// KDA_CHECK=1: debug validation of the slot tables on the host.  The tables
// are copied from the device on the call's stream (which is synchronised, so
// this mode is for debugging, not for serving or graph capture) and checked
// for what the kernels cannot detect: two rows naming the same slot, and
// snapshot / checkpoint slots that alias a live slot or each other.
// ---------------------------------------------------------------------------
bool check_mode() {
    const char *e = getenv("KDA_CHECK");
    return e && strcmp(e, "0") != 0 && e[0] != '\0';
}

// Copy n int32 from the device; false on a HIP error.
bool fetch_table(const int32_t *dev, size_t n, std::vector<int32_t> &host, hipStream_t stream) {
    host.resize(n);
    if (n == 0) return true;
    if (hipMemcpyAsync(host.data(), dev, n * sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess)
        return false;
    return hipStreamSynchronize(stream) == hipSuccess;
}

// Every entry of `live` and `extra` in [-1, n_slots) (KDA_ERR_SHAPE), and the
// non-negative entries distinct across both tables (KDA_ERR_ALIAS).
kda_status check_distinct(const std::vector<int32_t> &live, const std::vector<int32_t> &extra, int n_slots) {
    std::vector<int32_t> all;
    all.reserve(live.size() + extra.size());
    for (const auto *t : {&live, &extra})
        for (int32_t v : *t) {
            if (v < -1 || v >= n_slots) return KDA_ERR_SHAPE;
            if (v >= 0) all.push_back(v);
        }
    std::sort(all.begin(), all.end());
    return std::adjacent_find(all.begin(), all.end()) == all.end() ? KDA_OK : KDA_ERR_ALIAS;
}

kda_status debug_check(const int32_t *live_dev, size_t n_live, const int32_t *extra_dev, size_t n_extra,
                       int n_slots, void *hip_stream) {
    if (!check_mode()) return KDA_OK;
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    std::vector<int32_t> live, extra;
    if (!fetch_table(live_dev, n_live, live, st)) return KDA_ERR_LAUNCH;
    if (extra_dev && !fetch_table(extra_dev, n_extra, extra, st)) return KDA_ERR_LAUNCH;
    return check_distinct(live, extra, n_slots);
}

#define KDA_TRY(expr)                      \
    do {                                   \
        const kda_status st_ = (expr);     \
        if (st_ != KDA_OK) return st_;     \
    } while (0)

RecParams rec_params(const kda_layer *L, const kda_cache *C, const kda_inputs *in, float *y) {
    RecParams p{};
    p.A = L->A; p.conv_wt = L->conv_wt; p.norm_w = L->norm_w;
    p.q_scale = L->q_scale; p.l2_eps = L->l2_eps; p.rms_eps = L->rms_eps;
    p.silu = (L->flags & KDA_CONV_SILU) ? 1 : 0;
    p.stream_state = (L->flags & KDA_STREAM_STATE) ? 1 : 0;
    p.state = C->state; p.window = C->conv_state; p.n_slots = C->n_slots; p.err_flag = C->err_flag;
    p.x_q = in->x_q; p.x_k = in->x_k; p.x_v = in->x_v; p.g = in->g; p.b = in->b; p.z = in->z;
    p.y = y;
    p.H = L->H;
    return p;
}

}  // namespace

KDA_EXPORT kda_status kda_decode(const kda_layer *layer, const kda_cache *cache,
                                 const int32_t *slot_idx, int32_t B, const kda_inputs *inputs,
                                 float *y, void *hip_stream) {
    KDA_TRY(check_layer(layer));
    KDA_TRY(check_cache(cache));
    if (B < 0) return KDA_ERR_SHAPE;
    if (B == 0) return KDA_OK;
    KDA_TRY(check_inputs(inputs));
    if ((size_t)B * layer->H > 0x7fffffffu) return KDA_ERR_SHAPE;
    if (!slot_idx || !y) return KDA_ERR_NULL;
    if (!aligned(slot_idx, 4)) return KDA_ERR_ALIGN;
    if (!aligned(y, 16)) return KDA_ERR_ALIGN;
    KDA_TRY(debug_check(slot_idx, B, nullptr, 0, cache->n_slots, hip_stream));
    RecParams p = rec_params(layer, cache, inputs, y);
    p.slot_idx = slot_idx;
    p.B = B;
    p.T = 1;
    // cached for small calls or when the caller says its states stay
    // cache-resident (a call over more than the Infinity Cache holds streams
    // anyway); streamed otherwise, and always under KDA_STREAM_STATE
    const size_t sbytes = (size_t)B * layer->H * layer->d_k * layer->d_v * sizeof(float);
    const bool cached = !(layer->flags & KDA_STREAM_STATE) &&
                        (sbytes <= kCachedDefaultBytes ||
                         ((layer->flags & KDA_STATE_RESIDENT) && sbytes <= kResidentMaxBytes));
    p.stream_state = cached ? 0 : 1;
    return launch_recurrent(p, layer->d_k, layer->d_v, inputs->dtype, RecKind::decode,
                            static_cast<hipStream_t>(hip_stream));
}

KDA_EXPORT kda_status kda_spec_verify(const kda_layer *layer, const kda_cache *cache,
                                      const int32_t *slot_idx, const int32_t *snap_slots,
                                      int32_t B, int32_t T, const int32_t *draft_len,
                                      const kda_inputs *inputs, float *y, void *hip_stream) {
    KDA_TRY(check_layer(layer));
    KDA_TRY(check_cache(cache));
    if (B < 0 || T < 1 || T > kMaxDraft) return KDA_ERR_SHAPE;
    if (B == 0) return KDA_OK;
    KDA_TRY(check_inputs(inputs));
    if ((size_t)B * layer->H > 0x7fffffffu) return KDA_ERR_SHAPE;
    if (!slot_idx || !snap_slots || !y) return KDA_ERR_NULL;
    if (!aligned(slot_idx, 4) || !aligned(snap_slots, 4) || (draft_len && !aligned(draft_len, 4)))
        return KDA_ERR_ALIGN;
    if (!aligned(y, 16)) return KDA_ERR_ALIGN;
    KDA_TRY(debug_check(slot_idx, B, snap_slots, (size_t)B * T, cache->n_slots, hip_stream));
    RecParams p = rec_params(layer, cache, inputs, y);
    p.slot_idx = slot_idx;
    p.snap_slots = snap_slots;
    p.draft_len = draft_len;
    p.B = B;
    p.T = T;
    return launch_recurrent(p, layer->d_k, layer->d_v, inputs->dtype, RecKind::verify,
                            static_cast<hipStream_t>(hip_stream));
}

KDA_EXPORT kda_status kda_spec_commit(const kda_layer *layer, const kda_cache *cache,
                                      const int32_t *slot_idx, const int32_t *snap_slots,
                                      const int32_t *accepted_len, int32_t B, int32_t T,
                                      kda_dtype window_dtype, void *hip_stream) {
    KDA_TRY(check_layer(layer));
    KDA_TRY(check_cache(cache));
    if (window_dtype != KDA_F32 && window_dtype != KDA_BF16) return KDA_ERR_DTYPE;
    if (B < 0 || T < 1 || T > kMaxDraft) return KDA_ERR_SHAPE;
    if (B == 0) return KDA_OK;
    if ((size_t)B * layer->H > 0x7fffffffu) return KDA_ERR_SHAPE;
    if (!slot_idx || !snap_slots || !accepted_len) return KDA_ERR_NULL;
    if (!aligned(slot_idx, 4) || !aligned(snap_slots, 4) || !aligned(accepted_len, 4))
        return KDA_ERR_ALIGN;
    KDA_TRY(debug_check(slot_idx, B, snap_slots, (size_t)B * T, cache->n_slots, hip_stream));
    CommitParams p{};
    p.state = cache->state;
    p.window = cache->conv_state;
    p.n_slots = cache->n_slots;
    p.err_flag = cache->err_flag;
    p.slot_idx = slot_idx;
    p.snap_slots = snap_slots;
    p.accepted_len = accepted_len;
    p.B = B;
    p.H = layer->H;
    p.T = T;
    p.state_elems = layer->d_k * layer->d_v;
    p.window_words = (int)((size_t)(layer->conv_w - 1) * (2 * layer->d_k + layer->d_v) *
                           elem_size(window_dtype) / 4);
    return launch_commit(p, static_cast<hipStream_t>(hip_stream));
}

KDA_EXPORT size_t kda_spec_delta_bytes(const kda_layer *layer, int32_t B, int32_t T, kda_dtype dtype) {
    if (check_layer(layer) != KDA_OK || B < 0 || T < 1 || T > kMaxDraft) return 0;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return 0;
    return (size_t)B * T * layer->H * spec_delta_record_bytes(layer->d_k, layer->d_v, dtype);
}

KDA_EXPORT kda_status kda_spec_verify_delta(const kda_layer *layer, const kda_cache *cache,
                                            const int32_t *slot_idx, int32_t B, int32_t T,
                                            const int32_t *draft_len, const kda_inputs *inputs,
                                            float *y, void *delta, size_t delta_bytes,
                                            void *hip_stream) {
    KDA_TRY(check_layer(layer));
    KDA_TRY(check_cache(cache));
    if (B < 0 || T < 1 || T > kMaxDraft) return KDA_ERR_SHAPE;
    if (B == 0) return KDA_OK;
    KDA_TRY(check_inputs(inputs));
    if ((size_t)B * layer->H > 0x7fffffffu) return KDA_ERR_SHAPE;
    if (!slot_idx || !y || !delta) return KDA_ERR_NULL;
    if (!aligned(slot_idx, 4) || (draft_len && !aligned(draft_len, 4))) return KDA_ERR_ALIGN;
    if (!aligned(y, 16) || !aligned(delta, 16)) return KDA_ERR_ALIGN;
    if (delta_bytes < kda_spec_delta_bytes(layer, B, T, inputs->dtype)) return KDA_ERR_WORKSPACE;
    KDA_TRY(debug_check(slot_idx, B, nullptr, 0, cache->n_slots, hip_stream));
    RecParams p = rec_params(layer, cache, inputs, y);
    p.slot_idx = slot_idx;
    p.draft_len = draft_len;
    p.delta = delta;
    p.B = B;
    p.T = T;
    return launch_recurrent(p, layer->d_k, layer->d_v, inputs->dtype, RecKind::verify_delta,
                            static_cast<hipStream_t>(hip_stream));
}

KDA_EXPORT kda_status kda_spec_commit_delta(const kda_layer *layer, const kda_cache *cache,
                                            const int32_t *slot_idx, const void *delta,
                                            size_t delta_bytes, const int32_t *accepted_len,
                                            int32_t B, int32_t T, kda_dtype dtype,
                                            void *hip_stream) {
    KDA_TRY(check_layer(layer));
    KDA_TRY(check_cache(cache));
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_DTYPE;
    if (B < 0 || T < 1 || T > kMaxDraft) return KDA_ERR_SHAPE;
    if (B == 0) return KDA_OK;
    if ((size_t)B * layer->H > 0x7fffffffu) return KDA_ERR_SHAPE;
    if (!slot_idx || !delta || !accepted_len) return KDA_ERR_NULL;
    if (!aligned(slot_idx, 4) || !aligned(accepted_len, 4)) return KDA_ERR_ALIGN;
    if (!aligned(delta, 16)) return KDA_ERR_ALIGN;
    if (delta_bytes < kda_spec_delta_bytes(layer, B, T, dtype)) return KDA_ERR_WORKSPACE;
    KDA_TRY(debug_check(slot_idx, B, nullptr, 0, cache->n_slots, hip_stream));
    CommitDeltaParams p{};
    p.state = cache->state;
    p.window = cache->conv_state;
    p.n_slots = cache->n_slots;
    p.err_flag = cache->err_flag;
    p.stream_state = (layer->flags & KDA_STREAM_STATE) ? 1 : 0;
    p.slot_idx = slot_idx;
    p.accepted_len = accepted_len;
    p.delta = delta;
    p.B = B;
    p.H = layer->H;
    p.T = T;
    return launch_commit_delta(p, layer->d_k, layer->d_v, dtype, static_cast<hipStream_t>(hip_stream));
}

KDA_EXPORT size_t kda_chunk_prefill_workspace_bytes(const kda_layer *layer, int32_t total_T,
                                                    int32_t N_seq, int32_t chunk) {
    if (check_layer(layer) != KDA_OK || total_T < 0 || N_seq < 1 || chunk != 64) return 0;
    return prefill_workspace_bytes(layer->H, layer->d_k, layer->d_v, total_T, N_seq, chunk);
}

namespace {

kda_status static_workspace(void **ptr, size_t *bytes);

// With use_static the workspace arguments are ignored: the call runs in the
// library's static workspace (looked up after every other check passed).
kda_status prefill_common(const kda_layer *layer, const kda_cache *cache, const int32_t *slot_idx,
                          const int32_t *cu_seqlens, int32_t N_seq, int32_t total_T, int32_t chunk,
                          const kda_inputs *inputs, float *y, const int32_t *ckpt_slots,
                          int32_t ckpt_interval, int32_t ckpt_per_seq, void *workspace,
                          size_t workspace_bytes, void *hip_stream, bool use_static = false) {
    KDA_TRY(check_layer(layer));
    KDA_TRY(check_cache(cache));
    if (N_seq < 1 || total_T < 0 || chunk <= 0) return KDA_ERR_SHAPE;
    if (chunk != 64) return KDA_ERR_UNSUPPORTED;
    // one-dimensional grids: heads x chunk slots, heads x column blocks x sequences
    const size_t slots = (size_t)total_T / 64 + (size_t)N_seq;
    if ((size_t)layer->H * slots > 0x7fffffffu || (size_t)layer->H * (layer->d_v / 16) * N_seq > 0x7fffffffu)
        return KDA_ERR_SHAPE;
    // with no tokens the inputs and y are never read (and may be NULL)
    if (!inputs) return KDA_ERR_NULL;
    if (inputs->dtype != KDA_F32 && inputs->dtype != KDA_BF16) return KDA_ERR_DTYPE;
    if (total_T > 0) {
        KDA_TRY(check_inputs(inputs));
        if (!y) return KDA_ERR_NULL;
        if (!aligned(y, 16)) return KDA_ERR_ALIGN;
    }
    if (!slot_idx || !cu_seqlens) return KDA_ERR_NULL;
    if (!aligned(slot_idx, 4) || !aligned(cu_seqlens, 4)) return KDA_ERR_ALIGN;
    const size_t need = prefill_workspace_bytes(layer->H, layer->d_k, layer->d_v, total_T, N_seq, chunk);
    if (use_static) {
        if (need > kStaticWorkspaceBytes) return KDA_ERR_WORKSPACE;
    } else {
        if (need && !workspace) return KDA_ERR_NULL;
        if (workspace_bytes < need) return KDA_ERR_WORKSPACE;
        if (workspace && !aligned(workspace, 16)) return KDA_ERR_ALIGN;
    }
    KDA_TRY(debug_check(slot_idx, N_seq, ckpt_slots, ckpt_slots ? (size_t)N_seq * ckpt_per_seq : 0,
                        cache->n_slots, hip_stream));
    if (use_static) KDA_TRY(static_workspace(&workspace, &workspace_bytes));
    PrefillParams p{};
    p.A = layer->A; p.conv_wt = layer->conv_wt; p.norm_w = layer->norm_w;
    p.q_scale = layer->q_scale; p.l2_eps = layer->l2_eps; p.rms_eps = layer->rms_eps;
    p.silu = (layer->flags & KDA_CONV_SILU) ? 1 : 0;
    p.state = cache->state; p.window = cache->conv_state; p.n_slots = cache->n_slots;
    p.err_flag = cache->err_flag;
    p.slot_idx = slot_idx; p.cu_seqlens = cu_seqlens;
    p.N_seq = N_seq; p.total_T = total_T; p.chunk = chunk; p.H = layer->H;
    p.x_q = inputs->x_q; p.x_k = inputs->x_k; p.x_v = inputs->x_v;
    p.g = inputs->g; p.b = inputs->b; p.z = inputs->z;
    p.y = y;
    p.workspace = workspace;
    p.workspace_bytes = workspace_bytes;
    p.ckpt_slots = ckpt_slots;
    p.ckpt_interval = ckpt_interval;
    p.ckpt_per_seq = ckpt_per_seq;
    return launch_prefill(p, layer->d_k, layer->d_v, inputs->dtype,
                          static_cast<hipStream_t>(hip_stream));
}

}  // namespace

KDA_EXPORT kda_status kda_chunk_prefill(const kda_layer *layer, const kda_cache *cache,
                                        const int32_t *slot_idx, const int32_t *cu_seqlens,
                                        int32_t N_seq, int32_t total_T, int32_t chunk,
                                        const kda_inputs *inputs, float *y, void *workspace,
                                        size_t workspace_bytes, void *hip_stream) {
    return prefill_common(layer, cache, slot_idx, cu_seqlens, N_seq, total_T, chunk, inputs, y,
                          nullptr, 0, 0, workspace, workspace_bytes, hip_stream);
}

KDA_EXPORT kda_status kda_chunk_prefill_ckpt(const kda_layer *layer, const kda_cache *cache,
                                             const int32_t *slot_idx, const int32_t *cu_seqlens,
                                             int32_t N_seq, int32_t total_T, int32_t chunk,
                                             const kda_inputs *inputs, float *y,
                                             const int32_t *ckpt_slots, int32_t ckpt_interval,
                                             int32_t ckpt_per_seq, void *workspace,
                                             size_t workspace_bytes, void *hip_stream) {
    if (!ckpt_slots) return KDA_ERR_NULL;
    if (!aligned(ckpt_slots, 4)) return KDA_ERR_ALIGN;
    if (ckpt_per_seq < 1 || ckpt_interval < chunk || chunk <= 0 || ckpt_interval % chunk != 0)
        return KDA_ERR_SHAPE;
    return prefill_common(layer, cache, slot_idx, cu_seqlens, N_seq, total_T, chunk, inputs, y,
                          ckpt_slots, ckpt_interval, ckpt_per_seq, workspace, workspace_bytes,
                          hip_stream);
}

// ---------------------------------------------------------------------------
// The static workspace of kda_chunk_prefill_static: a device array of the
// library, one copy per GPU (each device holds its own instance of the code
// object's globals), alive until the process ends.  Host code never uses the
// array's name as an address: the first call on a device, with that device
// current, looks its device address up and keeps it per device.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[KDA_STATIC_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

kda_status static_workspace(void **ptr, size_t *bytes) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return KDA_ERR_LAUNCH;
    if (dev < 0 || dev >= kMaxDevices) return KDA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KDA_ERR_LAUNCH;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    *bytes = kStaticWorkspaceBytes;
    return KDA_OK;
}

}  // namespace

KDA_EXPORT kda_status kda_chunk_prefill_static(const kda_layer *layer, const kda_cache *cache,
                                               const int32_t *slot_idx, const int32_t *cu_seqlens,
                                               int32_t N_seq, int32_t total_T, int32_t chunk,
                                               const kda_inputs *inputs, float *y, void *hip_stream) {
    return prefill_common(layer, cache, slot_idx, cu_seqlens, N_seq, total_T, chunk, inputs, y, nullptr, 0, 0,
                          nullptr, 0, hip_stream, true);
}

KDA_EXPORT kda_status kda_copy_probe(float *dst, const float *src, size_t n, void *hip_stream) {
    if (n == 0) return KDA_OK;
    if (!dst || !src) return KDA_ERR_NULL;
    if (!aligned(dst, 16) || !aligned(src, 16)) return KDA_ERR_ALIGN;
    return launch_copy_probe(dst, src, n, static_cast<hipStream_t>(hip_stream));
}

KDA_EXPORT kda_status kda_build_metadata(const int32_t *num_tokens, const int32_t *req_slot, int32_t n_req,
                                         int32_t n_slots, int32_t *cu_seqlens, int32_t *slot_idx,
                                         int32_t *chunk_start, int32_t *counts, int32_t *err_flag,
                                         void *hip_stream) {
    if (n_req < 0 || n_slots <= 0) return KDA_ERR_SHAPE;
    if (!cu_seqlens || !chunk_start || !counts) return KDA_ERR_NULL;
    if (n_req > 0 && (!num_tokens || !req_slot || !slot_idx)) return KDA_ERR_NULL;
    for (const void *q : {(const void *)num_tokens, (const void *)req_slot, (const void *)cu_seqlens,
                          (const void *)slot_idx, (const void *)chunk_start, (const void *)counts,
                          (const void *)err_flag})
        if (q && !aligned(q, 4)) return KDA_ERR_ALIGN;
    MetaParams p{};
    p.num_tokens = num_tokens;
    p.req_slot = req_slot;
    p.n_req = n_req;
    p.n_slots = n_slots;
    p.cu_seqlens = cu_seqlens;
    p.slot_idx = slot_idx;
    p.chunk_start = chunk_start;
    p.counts = counts;
    p.err_flag = err_flag;
    return launch_build_metadata(p, static_cast<hipStream_t>(hip_stream));
}

KDA_EXPORT const char *kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_NULL: return "a required pointer is null";
        case KDA_ERR_SHAPE: return "a size or scalar parameter is out of range";
        case KDA_ERR_DTYPE: return "unknown input dtype";
        case KDA_ERR_ALIGN: return "a pointer is not aligned as required";
        case KDA_ERR_UNSUPPORTED: return "unsupported configuration (d_k, d_v, conv_w, chunk or flags)";
        case KDA_ERR_WORKSPACE: return "workspace too small";
        case KDA_ERR_LAUNCH: return "kernel launch failed";
        case KDA_ERR_ALIAS: return "slot tables alias (KDA_CHECK): two rows name the same slot, or "
                                   "snapshot/checkpoint slots alias live slots or each other";
    }
    return "unknown status";
}

KDA_EXPORT int32_t kda_abi_version(void) { return KDA_ABI_VERSION; }
