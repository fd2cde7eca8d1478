// api.hip -- the C ABI declared in include/gdn_mi355x.h: host-side argument
// validation (before any HIP call) and kernel launches on the caller's
// stream. No allocation, no synchronisation, no global mutable state apart
// from the thread-local last HIP error.

#include <limits.h>

#include <cmath>

#include "attention_launch.hpp"
#include "gdn_device.hpp"
#include "gdn_mi355x.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kMaxLog = 16;  // log capacity the decode kernels hold on chip

bool head_dim_ok(int d) { return d == 32 || d == 64 || d == 128; }
bool dtype_ok(int t) { return t == GDN_F32 || t == GDN_BF16; }
bool variant_ok(int v) { return v == GDN_SCALAR || v == GDN_KDA || v == GDN_RWKV6; }

int from_hip(hipError_t e) {
    if (e == hipSuccess) return GDN_OK;
    g_last_hip_error = static_cast<int>(e);
    return GDN_ERR_HIP;
}

int check_decode_common(const void *q, const void *k, const void *v, const float *log_alpha,
                        const float *beta, const void *state, const int32_t *slot_idx,
                        const void *o, int B, int H, int d_k, int d_v, int n_slots,
                        int variant, int io_dtype, int o_dtype) {
    if (!q || !k || !v || !log_alpha || !state || !o) return GDN_ERR_INVALID_ARG;
    if (!variant_ok(variant) || !dtype_ok(io_dtype) || !dtype_ok(o_dtype))
        return GDN_ERR_INVALID_ARG;
    if (variant != GDN_RWKV6 && !beta) return GDN_ERR_INVALID_ARG;
    if (B < 0 || H < 1 || n_slots < 0) return GDN_ERR_INVALID_ARG;
    if ((long long)B * H > INT_MAX) return GDN_ERR_INVALID_ARG;
    if (!slot_idx && B > n_slots) return GDN_ERR_INVALID_ARG;
    if (!head_dim_ok(d_k) || !head_dim_ok(d_v)) return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

}  // namespace

extern "C" {

const char *gdn_status_string(int status) {
    switch (status) {
        case GDN_OK: return "ok";
        case GDN_ERR_INVALID_ARG: return "invalid argument";
        case GDN_ERR_UNSUPPORTED: return "unsupported shape or option";
        case GDN_ERR_WORKSPACE: return "workspace missing or too small";
        case GDN_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

int gdn_last_hip_error(void) { return g_last_hip_error; }

int gdn_max_log_capacity(void) { return kMaxLog; }

int gdn_decode_eager(const void *q, const void *k, const void *v, const float *log_alpha,
                     const float *beta, float *state, const int32_t *slot_idx, void *o, int B,
                     int H, int d_k, int d_v, int n_slots, int variant, int io_dtype, int o_dtype,
                     void *stream) {
    const int st = check_decode_common(q, k, v, log_alpha, beta, state, slot_idx, o, B, H, d_k,
                                       d_v, n_slots, variant, io_dtype, o_dtype);
    if (st != GDN_OK) return st;
    gdn::DecodeArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.log_alpha = log_alpha;
    a.beta = beta;
    a.state = state;
    a.slot_idx = slot_idx;
    a.o = o;
    a.B = B;
    a.H = H;
    a.n_slots = n_slots;
    return from_hip(gdn::launch_decode(0, d_k, d_v, variant, io_dtype, o_dtype, a,
                                       static_cast<hipStream_t>(stream)));
}

int deltalog_append_decode(const void *q, const void *k, const void *v, const float *log_alpha,
                           const float *beta, float *base, float *log_u, void *log_k,
                           float *log_lambda, int32_t *log_len, const int32_t *slot_idx, void *o,
                           int B, int H, int d_k, int d_v, int n_slots, int Mcap, int merge_at,
                           int variant, int io_dtype, int o_dtype, void *stream) {
    const int st = check_decode_common(q, k, v, log_alpha, beta, base, slot_idx, o, B, H, d_k,
                                       d_v, n_slots, variant, io_dtype, o_dtype);
    if (st != GDN_OK) return st;
    if (!log_u || !log_k || !log_lambda || !log_len) return GDN_ERR_INVALID_ARG;
    if (Mcap < 1 || merge_at < 0 || merge_at > Mcap) return GDN_ERR_INVALID_ARG;
    if (Mcap > kMaxLog) return GDN_ERR_UNSUPPORTED;
    gdn::DecodeArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.log_alpha = log_alpha;
    a.beta = beta;
    a.state = base;
    a.log_u = log_u;
    a.log_k = log_k;
    a.log_lam = log_lambda;
    a.log_len = log_len;
    a.slot_idx = slot_idx;
    a.o = o;
    a.B = B;
    a.H = H;
    a.n_slots = n_slots;
    a.Mcap = Mcap;
    a.merge_at = merge_at;
    return from_hip(gdn::launch_decode(1, d_k, d_v, variant, io_dtype, o_dtype, a,
                                       static_cast<hipStream_t>(stream)));
}

int deltalog_merge(float *base, const float *log_u, const void *log_k, const float *log_lambda,
                   int32_t *log_len, const int32_t *slot_idx, int B, int H, int d_k, int d_v,
                   int n_slots, int Mcap, int min_len, int variant, int io_dtype, void *stream) {
    if (!base || !log_u || !log_k || !log_lambda || !log_len) return GDN_ERR_INVALID_ARG;
    if (!variant_ok(variant) || !dtype_ok(io_dtype)) return GDN_ERR_INVALID_ARG;
    if (B < 0 || H < 1 || n_slots < 0 || Mcap < 1) return GDN_ERR_INVALID_ARG;
    if ((long long)B * H > INT_MAX) return GDN_ERR_INVALID_ARG;
    if (!slot_idx && B > n_slots) return GDN_ERR_INVALID_ARG;
    if (!head_dim_ok(d_k) || !head_dim_ok(d_v)) return GDN_ERR_UNSUPPORTED;
    if (Mcap > kMaxLog) return GDN_ERR_UNSUPPORTED;
    gdn::DecodeArgs a{};
    a.state = base;
    a.log_u = const_cast<float *>(log_u);
    a.log_k = const_cast<void *>(log_k);
    a.log_lam = const_cast<float *>(log_lambda);
    a.log_len = log_len;
    a.slot_idx = slot_idx;
    a.B = B;
    a.H = H;
    a.n_slots = n_slots;
    a.Mcap = Mcap;
    a.min_len = min_len < 1 ? 1 : min_len;
    return from_hip(gdn::launch_decode(2, d_k, d_v, variant, io_dtype, GDN_F32, a,
                                       static_cast<hipStream_t>(stream)));
}

size_t gdn_prefill_workspace_bytes(int n_tokens, int n_seq, int H, int d_k, int d_v, int chunk,
                                   int variant) {
    if (n_tokens < 0 || n_seq < 0 || H < 1 || chunk < 1 || !variant_ok(variant)) return 0;
    if (!head_dim_ok(d_k) || !head_dim_ok(d_v)) return 0;
    return gdn::prefill_workspace_bytes(n_tokens, n_seq, H, d_k, d_v, chunk, variant);
}

static int prefill_common(const void *q, const void *k, const void *v, const float *log_alpha,
                          const float *beta, const int32_t *cu, const int32_t *parent, int n_seq,
                          int n_parent, int n_tokens, int H, int d_k, int d_v, int chunk,
                          const float *conv_w, int qk_l2norm, const float *state_in,
                          const void *win_in, void *o, float *state_out, void *win_out,
                          int variant, int io_dtype, int o_dtype, void *workspace,
                          size_t ws_bytes, void *stream, int ckpt_every = 0, int ckpt_cap = 0,
                          float *ckpt_state = nullptr, void *ckpt_window = nullptr) {
    if (!q || !k || !v || !log_alpha || !cu) return GDN_ERR_INVALID_ARG;
    if (!variant_ok(variant) || !dtype_ok(io_dtype) || !dtype_ok(o_dtype))
        return GDN_ERR_INVALID_ARG;
    if (variant != GDN_RWKV6 && !beta) return GDN_ERR_INVALID_ARG;
    if (n_seq < 0 || n_tokens < 0 || H < 1 || n_parent < 0) return GDN_ERR_INVALID_ARG;
    if (chunk != 16 && chunk != 32 && chunk != 64) return GDN_ERR_INVALID_ARG;
    if (!head_dim_ok(d_k) || !head_dim_ok(d_v)) return GDN_ERR_UNSUPPORTED;
    if (chunk != 64) return GDN_ERR_UNSUPPORTED;
    const size_t need =
        gdn::prefill_workspace_bytes(n_tokens, n_seq, H, d_k, d_v, chunk, variant);
    if (need > 0 && (!workspace || ws_bytes < need)) return GDN_ERR_WORKSPACE;
    gdn::PrefillArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.log_alpha = log_alpha;
    a.beta = beta;
    a.cu = cu;
    a.parent = parent;
    a.conv_w = conv_w;
    a.state_in = state_in;
    a.win_in = win_in;
    a.o = o;
    a.state_out = state_out;
    a.win_out = win_out;
    a.ws = workspace;
    a.ws_bytes = ws_bytes;
    a.n_seq = n_seq;
    a.n_parent = n_parent;
    a.n_tokens = n_tokens;
    a.H = H;
    a.qk_norm = qk_l2norm ? 1 : 0;
    a.chunk = chunk;
    a.dv = d_v;
    a.variant = variant;
    a.ckpt_every = ckpt_every;
    a.ckpt_cap = ckpt_cap;
    a.ckpt_state = ckpt_state;
    a.ckpt_window = ckpt_window;
    return from_hip(
        gdn::launch_prefill(d_k, d_v, io_dtype, o_dtype, a, static_cast<hipStream_t>(stream)));
}

int gdn_prefill_shared(const void *q, const void *k, const void *v, const float *log_alpha,
                       const float *beta, const int32_t *cu_seqlens, int n_seq, int n_tokens,
                       int H, int d_k, int d_v, int chunk, const float *conv_w, int qk_l2norm,
                       const float *init_state, const void *init_window, void *o,
                       float *final_state, void *final_window, int variant, int io_dtype,
                       int o_dtype, void *workspace, size_t ws_bytes, void *stream) {
    if (!final_state) return GDN_ERR_INVALID_ARG;
    return prefill_common(q, k, v, log_alpha, beta, cu_seqlens, nullptr, n_seq, n_seq, n_tokens,
                          H, d_k, d_v, chunk, conv_w, qk_l2norm, init_state, init_window, o,
                          final_state, final_window, variant, io_dtype, o_dtype, workspace,
                          ws_bytes, stream);
}

int gdn_prefill_checkpointed(const void *q, const void *k, const void *v, const float *log_alpha,
                             const float *beta, const int32_t *cu_seqlens, int n_seq,
                             int n_tokens, int H, int d_k, int d_v, int chunk,
                             const float *conv_w, int qk_l2norm, const float *init_state,
                             const void *init_window, void *o, float *final_state,
                             void *final_window, int ckpt_every, int ckpt_cap,
                             float *ckpt_state, void *ckpt_window, int variant, int io_dtype,
                             int o_dtype, void *workspace, size_t ws_bytes, void *stream) {
    if (!final_state) return GDN_ERR_INVALID_ARG;
    if (ckpt_every < 1 || ckpt_cap < 0 || (ckpt_cap > 0 && !ckpt_state))
        return GDN_ERR_INVALID_ARG;
    return prefill_common(q, k, v, log_alpha, beta, cu_seqlens, nullptr, n_seq, n_seq, n_tokens,
                          H, d_k, d_v, chunk, conv_w, qk_l2norm, init_state, init_window, o,
                          final_state, final_window, variant, io_dtype, o_dtype, workspace,
                          ws_bytes, stream, ckpt_every, ckpt_cap, ckpt_state, ckpt_window);
}
int gdn_fork_branches(const void *q, const void *k, const void *v, const float *log_alpha,
                      const float *beta, const int32_t *branch_cu, const int32_t *branch_parent,
                      int n_branch, int n_parent, int n_tokens, int H, int d_k, int d_v,
                      int chunk, const float *conv_w, int qk_l2norm, const float *parent_state,
                      const void *parent_window, void *o, float *branch_state,
                      void *branch_window, int variant, int io_dtype, int o_dtype,
                      void *workspace, size_t ws_bytes, void *stream) {
    if (!branch_parent || !parent_state || !o) return GDN_ERR_INVALID_ARG;
    return prefill_common(q, k, v, log_alpha, beta, branch_cu, branch_parent, n_branch,
                          n_parent, n_tokens, H, d_k, d_v, chunk, conv_w, qk_l2norm,
                          parent_state, parent_window, o, branch_state, branch_window, variant,
                          io_dtype, o_dtype, workspace, ws_bytes, stream);
}

size_t gdn_fork_attention_workspace_bytes(int n_req, int n_branch) {
    if (n_req < 0 || n_branch < 0) return 0;
    return gdn::attention_workspace_bytes(n_req, n_branch);
}

static int attention_common(const void *q, const void *k, const void *v,
                            const int32_t *cu_seqlens, int n_req, const int32_t *branch_cu,
                            const int32_t *branch_parent, int n_branch, int n_tokens, int H,
                            int H_kv, int d, float scale, int trunk_queries, void *o,
                            int io_dtype, int o_dtype) {
    if (!q || !k || !v || !o) return GDN_ERR_INVALID_ARG;
    if (n_req < 0 || n_branch < 0 || n_tokens < 0 || H < 1 || H_kv < 1 || H % H_kv != 0)
        return GDN_ERR_INVALID_ARG;
    if (!cu_seqlens || (n_branch > 0 && (!branch_cu || !branch_parent)))
        return GDN_ERR_INVALID_ARG;
    if (!dtype_ok(io_dtype) || !dtype_ok(o_dtype) || !std::isfinite(scale) || !(scale > 0.f))
        return GDN_ERR_INVALID_ARG;
    if (io_dtype != GDN_BF16 || (d != 64 && d != 128)) return GDN_ERR_UNSUPPORTED;
    // in-kernel row offsets are 32-bit
    if ((long long)n_tokens * H * d >= (1LL << 31)) return GDN_ERR_UNSUPPORTED;
    (void)trunk_queries;
    return GDN_OK;
}

static int attention_launch(const void *q, const void *k, const void *v,
                            const int32_t *cu_seqlens, int n_req, const int32_t *branch_cu,
                            const int32_t *branch_parent, int n_branch, int n_tokens, int H,
                            int H_kv, int d, float scale, int trunk_queries, void *o, int o_dtype,
                            void *workspace, void *stream) {
    gdn::AttnArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.cu = cu_seqlens;
    a.bcu = branch_cu;
    a.bparent = branch_parent;
    a.o = o;
    a.ws = workspace;
    a.n_req = n_req;
    a.n_branch = n_branch;
    a.n_tokens = n_tokens;
    a.H = H;
    a.Hkv = H_kv;
    a.scale = scale;
    a.trunk_queries = trunk_queries ? 1 : 0;
    return from_hip(gdn::launch_attention(d, o_dtype, a, static_cast<hipStream_t>(stream)));
}

int gdn_fork_attention(const void *q, const void *k, const void *v, const int32_t *cu_seqlens,
                       int n_req, const int32_t *branch_cu, const int32_t *branch_parent,
                       int n_branch, int n_tokens, int H, int H_kv, int d, float scale,
                       int trunk_queries, void *o, int io_dtype, int o_dtype, void *workspace,
                       size_t ws_bytes, void *stream) {
    const int st = attention_common(q, k, v, cu_seqlens, n_req, branch_cu, branch_parent,
                                    n_branch, n_tokens, H, H_kv, d, scale, trunk_queries, o,
                                    io_dtype, o_dtype);
    if (st != GDN_OK) return st;
    if (!workspace || ws_bytes < gdn::attention_workspace_bytes(n_req, n_branch))
        return GDN_ERR_WORKSPACE;
    return attention_launch(q, k, v, cu_seqlens, n_req, branch_cu, branch_parent, n_branch,
                            n_tokens, H, H_kv, d, scale, trunk_queries, o, o_dtype, workspace,
                            stream);
}

int gdn_fork_attention_noalloc(const void *q, const void *k, const void *v,
                               const int32_t *cu_seqlens, int n_req, const int32_t *branch_cu,
                               const int32_t *branch_parent, int n_branch, int n_tokens, int H,
                               int H_kv, int d, float scale, int trunk_queries, void *o,
                               int io_dtype, int o_dtype, void *stream) {
    const int st = attention_common(q, k, v, cu_seqlens, n_req, branch_cu, branch_parent,
                                    n_branch, n_tokens, H, H_kv, d, scale, trunk_queries, o,
                                    io_dtype, o_dtype);
    if (st != GDN_OK) return st;
    if ((long long)n_req + n_branch > gdn::kAttnScratchSegments) return GDN_ERR_WORKSPACE;
    // the tile table is the current device's copy of the file-scope array:
    // the stream must belong to that device
    int cur = 0;
    hipDevice_t sdev = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess) e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
    if (e != hipSuccess) return from_hip(e);
    if (sdev != cur) return GDN_ERR_INVALID_ARG;
    void *ws = nullptr;
    size_t ws_bytes = 0;
    e = gdn::attention_scratch(&ws, &ws_bytes);
    if (e != hipSuccess) return from_hip(e);
    if (ws_bytes < gdn::attention_workspace_bytes(n_req, n_branch)) return GDN_ERR_WORKSPACE;
    return attention_launch(q, k, v, cu_seqlens, n_req, branch_cu, branch_parent, n_branch,
                            n_tokens, H, H_kv, d, scale, trunk_queries, o, o_dtype, ws, stream);
}

int gdn_stream_probe(const void *src, void *dst, size_t n_bytes, int mode, void *stream) {
    if ((mode != 0 && mode != 1) || n_bytes % 16 != 0) return GDN_ERR_INVALID_ARG;
    if (n_bytes == 0) return GDN_OK;
    if (!src || !dst) return GDN_ERR_INVALID_ARG;
    return from_hip(gdn::launch_stream_probe(src, dst, n_bytes, mode,
                                             static_cast<hipStream_t>(stream)));
}

}  // extern "C"
