/*
 * gdn_mi355x.h -- C ABI of the MI355X (gfx950) Gated DeltaNet recurrence
 * library: shared-context prefill, forked branches, and decode steps
 * (eager, and deferred base + log).
 *
 * Sources, cited by page title and section:
 *  [FL] "같은 맥락에서 여러 판단을 빠르게 처리하는 Flide" (yozm.zip summary):
 *       glossary "ForkAttention" / "Gated DeltaNet"; section
 *       "연구방법을 단계별로" (method), steps 1-4.
 *  [DL] "DeltaLog: Deferred Materialization of Recurrent States for Linear
 *       Attention Decoding" (gist.science summary): sections
 *       "문제: 선형 어텐션 디코딩의 상태 업데이트 세금" (problem),
 *       "핵심 메커니즘: Base + Log" (base + log), "트래픽 모델" (traffic
 *       model), "커널 구현" (kernel implementation and operator list).
 *  [GD] Gated delta rule: S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T,
 *       o_t = S_t q_t (Yang, Kautz, Hatamizadeh, ICLR 2025).
 *
 * Conventions for every call
 *  - Every array argument is a caller-owned DEVICE pointer (HBM), dense
 *    row-major with the layout given, 16-byte aligned. The library never
 *    allocates, frees or keeps a caller's pointer. Its only global mutable
 *    state is a thread-local copy of the last HIP error code and, for
 *    gdn_fork_attention_noalloc, one file-scope device table per GPU (with
 *    a mutex-guarded cache of its per-device address).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream);
 *    calls return after enqueue without synchronising. Integer metadata
 *    (offsets, parents, slots, log lengths) lives in device memory, so a
 *    call can be captured in a HIP graph and replayed with new metadata.
 *  - State orientation: the math state S is d_v x d_k; storage is its
 *    transpose [.., d_k, d_v] ([DL] problem section), element [i][j] =
 *    key row i, value column j. State, base and log factors are fp32.
 *  - io_dtype (GDN_F32 | GDN_BF16) is the element type of q, k, v, of the
 *    conv windows and of the logged keys; o_dtype that of o. log_alpha
 *    (natural log of the decay, every entry <= 0) and beta are fp32.
 *  - variant: GDN_SCALAR (one decay per (token, head), delta rule),
 *    GDN_KDA (a decay per key, delta rule), GDN_RWKV6 (a decay per key,
 *    raw-value update u_t = v_t, beta unused and may be NULL) -- [DL]
 *    operator list.
 *  - d_k and d_v are each 32, 64 or 128, in any combination (d_k != d_v is
 *    allowed; any other width returns GDN_ERR_UNSUPPORTED).
 *  - Return value: GDN_OK or a negative status (below). Host-checkable
 *    arguments are validated before any HIP call; a failing call enqueues
 *    nothing. Device-side preconditions (offsets non-decreasing, parents
 *    and slots in range, distinct slots in one call) are documented per
 *    call; violating rows are skipped and their o rows set to NaN where
 *    noted, never read or written out of bounds.
 */
#ifndef GDN_MI355X_H
#define GDN_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARG = -1, /* NULL required pointer, negative size, bad enum,
                                 chunk not 16, 32 or 64 */
    GDN_ERR_UNSUPPORTED = -2, /* head width not 32/64/128, chunk 16 or 32 (not
                                 built), Mcap above the on-chip capacity */
    GDN_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
    GDN_ERR_HIP = -4          /* a HIP launch failed: see gdn_last_hip_error() */
};

enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 };

enum gdn_variant { GDN_SCALAR = 0, GDN_KDA = 1, GDN_RWKV6 = 2 };

/* Human-readable name of a status code (static storage). */
const char *gdn_status_string(int status);

/* hipError_t of the last failed launch on the calling thread (0 if none). */
int gdn_last_hip_error(void);

/* Largest log capacity (Mcap) the deferred kernels accept. */
int gdn_max_log_capacity(void);

/* ------------------------------------------------------------------ prefill
 * Workspace bytes gdn_prefill_shared / gdn_prefill_checkpointed /
 * gdn_fork_branches need for a stream of at most n_tokens tokens in n_seq
 * sequences with the given variant. The calls run in S segments, segment k
 * taking chunks [k n / S, (k + 1) n / S) of each sequence of n chunks, with
 * S the smallest count (at most one per chunk of an average sequence, at
 * most 64) whose records fit 512 MiB (the environment variable
 * GDN_PREFILL_SEGMENT_RECORD_BYTES replaces that bound when it holds a
 * positive integer; the calls read it as this function does, so set it
 * before sizing and leave it while the calls run). The workspace holds a
 * 256-byte-aligned int32 table of 3 n_seq + 4 entries, for S > 1 the state
 * carried between segments (n_seq * H * d_k * d_v fp32), and the records of
 * one segment: (n_tokens / 64 + n_seq) / S + n_seq chunk rows (rounded up;
 * n_tokens / 64 + n_seq for S = 1) of H records each, 25 KiB + 512 * d_k
 * bytes per record with GDN_SCALAR (89 KiB at d_k = 128) and 25 KiB +
 * 768 * d_k bytes with the per-key variants. The fork_prefill prefix
 * (65,536 tokens, 8 sequences, H = 16, d_k = d_v = 128) runs in 3 segments
 * with 0.49 KiB per token-head. Returns 0 for arguments the calls reject
 * (negative sizes, H < 1, widths not 32/64/128, bad variant).
 */
size_t gdn_prefill_workspace_bytes(int n_tokens, int n_seq, int H, int d_k,
                                   int d_v, int chunk, int variant);

/*
 * gdn_prefill_shared -- call 1 of the two-call fork ([FL] method step 2):
 * run every shared context of a flat token stream ([FL] step 1: tokens of
 * all requests packed into one stream, membership as device offsets) from
 * its initial state and return its outputs, final recurrent state and
 * final convolution window.
 *
 * Per sequence r (tokens [cu_seqlens[r], cu_seqlens[r+1])) and head h:
 *  1. short conv (if conv_w): y_t[c] = sum_{j<4} conv_w[c][j] x_{t-3+j}[c]
 *     over the channels [q | k | v] of all heads (q: h*d_k+i, k:
 *     H*d_k+h*d_k+i, v: 2*H*d_k+h*d_v+j; CC = H*(2d_k+d_v) channels),
 *     positions before the first token read init_window; no bias, no
 *     activation;
 *  2. if qk_l2norm: q, k <- y / sqrt(sum y^2 + 1e-6) per (token, head);
 *  3. the recurrence from init_state, o_t = S_t q_t, in chunks of `chunk`
 *     tokens: GDN_SCALAR S_t = S_{t-1} a_t (I - b_t k_t k_t^T) + b_t v_t k_t^T
 *     ([GD]); GDN_KDA the same delta rule with a per-key decay,
 *     S_t = S_{t-1} diag(a_t) (I - b_t k_t k_t^T) + b_t v_t k_t^T; GDN_RWKV6
 *     the raw value update S_t = S_{t-1} diag(a_t) + v_t k_t^T ([DL] "커널
 *     구현": the KDA and RWKV6 operators). a_t = exp(log_alpha).
 *     Any decay is allowed (log_alpha finite and <= 0; chunk sums of
 *     -1000 and single steps of -1000 are tested): every decay factor a
 *     chunk forms is e^{x} with x <= 0, except a per-key block factor up
 *     to e^80, beyond which the chunk takes the affected products from
 *     their definition.
 *
 *  q, k         [n_tokens, H, d_k]   io_dtype
 *  v            [n_tokens, H, d_v]   io_dtype
 *  log_alpha    [n_tokens, H] fp32 (GDN_SCALAR) or [n_tokens, H, d_k] fp32
 *               (GDN_KDA, GDN_RWKV6)
 *  beta         [n_tokens, H]        fp32 (NULL allowed for GDN_RWKV6)
 *  cu_seqlens   [n_seq + 1]          int32, device; cu[0] = 0, non-decreasing,
 *                                    cu[n_seq] <= n_tokens
 *  conv_w       [CC, 4] fp32 or NULL (no convolution)
 *  init_state   [n_seq, H, d_k, d_v] fp32 or NULL (zeros)
 *  init_window  [n_seq, 3, CC]       io_dtype or NULL (zeros); row 0 oldest
 *  o            [n_tokens, H, d_v]   o_dtype, or NULL (not written)
 *  final_state  [n_seq, H, d_k, d_v] fp32 (required)
 *  final_window [n_seq, 3, CC]       io_dtype or NULL: the last 3 raw
 *                                    inputs (from init_window when the
 *                                    sequence is shorter than 3)
 *  chunk        the chunk length of the chunked form: the interface takes
 *               16, 32 or 64 (the result does not depend on it beyond
 *               rounding); this build computes chunk = 64 only, so 16 and
 *               32 return GDN_ERR_UNSUPPORTED and any other value
 *               GDN_ERR_INVALID_ARG
 *  variant      GDN_SCALAR, GDN_KDA or GDN_RWKV6
 *  workspace    >= gdn_prefill_workspace_bytes(n_tokens, n_seq, ..., variant)
 *               bytes
 * Errors: INVALID_ARG (NULL required pointer, n_seq < 0, n_tokens < 0,
 * H < 1, bad dtype or variant, chunk not 16/32/64), UNSUPPORTED (d_k or
 * d_v not 32/64/128, chunk 16 or 32), WORKSPACE, HIP.
 */
int gdn_prefill_shared(const void *q, const void *k, const void *v,
                       const float *log_alpha, const float *beta,
                       const int32_t *cu_seqlens, int n_seq, int n_tokens,
                       int H, int d_k, int d_v, int chunk,
                       const float *conv_w, int qk_l2norm,
                       const float *init_state, const void *init_window,
                       void *o, float *final_state, void *final_window,
                       int variant, int io_dtype, int o_dtype, void *workspace,
                       size_t ws_bytes, void *stream);

/*
 * gdn_prefill_checkpointed -- gdn_prefill_shared that also keeps the state
 * and convolution window at internal positions of every sequence ([FL]
 * "연구방법을 단계별로": incremental checkpoints within a long history, so a
 * later request sharing a prefix of it resumes from the nearest one -- by
 * passing the checkpoint as init_state / init_window of a new call).
 * Checkpoint j (0 <= j < ckpt_cap) of sequence r is the state and window
 * after its first (j + 1) * ckpt_every * chunk tokens; it is written when
 * that position is inside the sequence or at its end, and left untouched
 * otherwise.
 *
 *  ckpt_every  chunks between checkpoints, >= 1
 *  ckpt_cap    checkpoints per sequence the buffers hold, >= 0
 *  ckpt_state  [n_seq, ckpt_cap, H, d_k, d_v] fp32 (required when ckpt_cap > 0)
 *  ckpt_window [n_seq, ckpt_cap, 3, CC] io_dtype, or NULL (not written)
 * Everything else as gdn_prefill_shared. Errors as gdn_prefill_shared, and
 * INVALID_ARG for ckpt_every < 1, ckpt_cap < 0 or a missing ckpt_state.
 */
int gdn_prefill_checkpointed(const void *q, const void *k, const void *v,
                             const float *log_alpha, const float *beta,
                             const int32_t *cu_seqlens, int n_seq, int n_tokens,
                             int H, int d_k, int d_v, int chunk,
                             const float *conv_w, int qk_l2norm,
                             const float *init_state, const void *init_window,
                             void *o, float *final_state, void *final_window,
                             int ckpt_every, int ckpt_cap, float *ckpt_state,
                             void *ckpt_window, int variant, int io_dtype,
                             int o_dtype, void *workspace, size_t ws_bytes,
                             void *stream);

/*
 * gdn_fork_branches -- call 2 of the two-call fork ([FL] method step 2;
 * glossary "ForkAttention": in GDN layers each branch forks exactly from
 * the shared state by a second call plus state indexing). Branch b
 * (tokens [branch_cu[b], branch_cu[b+1]) of its own stream) starts from
 * parent_state[branch_parent[b]] and parent_window[branch_parent[b]] and
 * runs steps 1-3 of gdn_prefill_shared. The parent arrays are read-only
 * and shared by all branches of a request.
 *
 *  q, k, v, log_alpha, beta : branch stream, layouts as above
 *  branch_cu     [n_branch + 1] int32 device
 *  branch_parent [n_branch]     int32 device, in [0, n_parent)
 *  parent_state  [n_parent, H, d_k, d_v] fp32
 *  parent_window [n_parent, 3, CC] io_dtype, or NULL (zeros)
 *  o             [n_tokens, H, d_v] o_dtype (required)
 *  branch_state  [n_branch, H, d_k, d_v] fp32 or NULL
 *  branch_window [n_branch, 3, CC] io_dtype or NULL
 * A branch whose parent is out of range is skipped and its o rows are set
 * to NaN. Errors as gdn_prefill_shared.
 * Branches of at most 64 tokens (the common case) run the chunk
 * preparation and the chunk step in one workgroup per (branch, head),
 * with no chunk record in the workspace (per-key variants pass it through
 * the (branch, head)'s own workspace slot); so do sequences of at most 64
 * tokens in gdn_prefill_shared. The results are bit for bit those of the
 * chunked path, which GDN_PREFILL_ONE_CHUNK=0 in the environment selects
 * (read at each call; for tests). Calls with checkpoints always take the
 * chunked path.
 */
int gdn_fork_branches(const void *q, const void *k, const void *v,
                      const float *log_alpha, const float *beta,
                      const int32_t *branch_cu, const int32_t *branch_parent,
                      int n_branch, int n_parent, int n_tokens, int H,
                      int d_k, int d_v, int chunk, const float *conv_w,
                      int qk_l2norm, const float *parent_state,
                      const void *parent_window, void *o, float *branch_state,
                      void *branch_window, int variant, int io_dtype,
                      int o_dtype, void *workspace, size_t ws_bytes,
                      void *stream);

/* ------------------------------------------------------------------ decode
 * gdn_decode_eager -- one decode step, materialised eagerly: the whole
 * [d_k, d_v] state of every (row, head) is read and rewritten in HBM
 * ([DL] problem section: the eager baseline). Per row b, head h, with
 * s = slot_idx ? slot_idx[b] : b and a_i = exp(log_alpha_i):
 *     y = S (a . k);  u = beta (v - y)  (RWKV6: u = v)
 *     S <- S diag(a) + u k^T;  o = S q
 *
 *  q, k      [B, H, d_k] io_dtype     v [B, H, d_v] io_dtype
 *  log_alpha [B, H] (GDN_SCALAR) or [B, H, d_k] (KDA, RWKV6) fp32
 *  beta      [B, H] fp32 (NULL allowed for RWKV6)
 *  state     [n_slots, H, d_k, d_v] fp32, in/out
 *  slot_idx  [B] int32 device, or NULL (row b uses slot b; needs B <= n_slots)
 *  o         [B, H, d_v] o_dtype
 * Slots must be distinct within a call; a row whose slot is outside
 * [0, n_slots) is skipped and its o row set to NaN.
 */
int gdn_decode_eager(const void *q, const void *k, const void *v,
                     const float *log_alpha, const float *beta, float *state,
                     const int32_t *slot_idx, void *o, int B, int H, int d_k,
                     int d_v, int n_slots, int variant, int io_dtype,
                     int o_dtype, void *stream);

/*
 * deltalog_append_decode -- one decode step under deferred materialisation
 * ([DL] "핵심 메커니즘: Base + Log": the state is a dense base plus a
 * bounded log of rank-1 factors with log-decay metadata; in the append
 * phase the base is left untouched and the step's factors are appended).
 * Per (row, head) with m = log_len[s][h] entries logged since the base was
 * written, and Lam the running log-decay since then (scalar or per key):
 *     Lam_t = Lam_{m} + log_alpha          (Lam_0 = 0)
 *     y = S_{t-1}(a . k) replayed from base and log;  u = beta (v - y)
 *     o = S_t q replayed from base, log and the step itself
 * then, if the step merges, base <- S_t and log_len <- 0 ([DL] merge
 * phase), else entry m <- (u, k, Lam_t) and log_len <- m + 1.
 * The step merges when merge_at > 0 and m + 1 >= merge_at, or when the
 * log is full (m >= Mcap). merge_at = 1 is the eager step.
 *
 *  base       [n_slots, H, d_k, d_v] fp32 (rewritten only on merging steps)
 *  log_u      [n_slots, H, Mcap, d_v] fp32
 *  log_k      [n_slots, H, Mcap, d_k] io_dtype (exact copies of k)
 *  log_lambda [n_slots, H, Mcap] (GDN_SCALAR) or [n_slots, H, Mcap, d_k] fp32
 *  log_len    [n_slots, H] int32 device, in/out; values outside [0, Mcap]
 *             are clamped into it
 *  Mcap       1 .. gdn_max_log_capacity() (16);  merge_at 0 .. Mcap
 *  other arguments as gdn_decode_eager.
 */
int deltalog_append_decode(const void *q, const void *k, const void *v,
                           const float *log_alpha, const float *beta,
                           float *base, float *log_u, void *log_k,
                           float *log_lambda, int32_t *log_len,
                           const int32_t *slot_idx, void *o, int B, int H,
                           int d_k, int d_v, int n_slots, int Mcap,
                           int merge_at, int variant, int io_dtype,
                           int o_dtype, void *stream);

/*
 * deltalog_merge -- the merge phase on its own ([DL] "핵심 메커니즘: Base +
 * Log": the accumulated logical state, base plus replayed log entries, is
 * written back as the new base and the log is cleared). For each listed
 * slot s (slot_idx[b] for b < B, or b itself when slot_idx is NULL) and
 * head h with m = log_len[s][h] >= max(min_len, 1):
 *     base[i][j] <- exp(Lam_m[i]) base[i][j]
 *                   + sum_{e<m} k_e[i] exp(Lam_m[i] - Lam_e[i]) u_e[j]
 *     log_len <- 0
 * Slot-heads with fewer entries are left bit-for-bit unchanged.
 * Arrays as deltalog_append_decode; variant selects scalar (GDN_SCALAR)
 * or per-key (KDA, RWKV6) log_lambda.
 */
int deltalog_merge(float *base, const float *log_u, const void *log_k,
                   const float *log_lambda, int32_t *log_len,
                   const int32_t *slot_idx, int B, int H, int d_k, int d_v,
                   int n_slots, int Mcap, int min_len, int variant,
                   int io_dtype, void *stream);

/* ---------------------------------------------------------- fork attention
 * Softmax attention over a flat token stream under the fork visibility rule
 * ([FL] "연구방법을 단계별로", method step 1, and glossary "ForkAttention":
 * requests and questions are GPU metadata over one flat stream; a token
 * reads only its own request's trunk and the current and earlier tokens of
 * its own branch -- other questions and other requests are invisible):
 *   trunk token at position p of request r: keys = trunk r, positions 0..p
 *   branch token at position p of branch b: keys = the whole trunk of
 *       request branch_parent[b], then positions 0..p of branch b
 *   o_i = sum_j softmax_j(scale <q_i, k_j>) v_j over those keys.
 * Positions are not applied here (rotary or other position encodings are
 * applied to q and k by the caller, with branch positions continuing after
 * the trunk as in an independent prompt).
 *
 * Workspace bytes gdn_fork_attention needs: (n_req + n_branch + 1) int32.
 */
size_t gdn_fork_attention_workspace_bytes(int n_req, int n_branch);

/*
 * gdn_fork_attention -- one call over the whole stream.
 *  q            [n_tokens, H, d] bf16
 *  k, v         [n_tokens, H_kv, d] bf16 (head h reads k/v head
 *               h / (H / H_kv); H_kv must divide H)
 *  cu_seqlens   [n_req + 1] int32 device: trunk r is tokens
 *               [cu_seqlens[r], cu_seqlens[r+1]) of the stream
 *  branch_cu    [n_branch + 1] int32 device: branch b is tokens
 *               [branch_cu[b], branch_cu[b+1]) (absolute, like cu_seqlens)
 *  branch_parent [n_branch] int32 device, request index of each branch
 *  scale        score scale, finite and > 0 (1/sqrt(d) is the usual choice)
 *  trunk_queries 1: trunk rows of o are computed too; 0: trunks only serve
 *               as keys/values (their o rows are left untouched) -- a round
 *               of new branches against trunks computed earlier
 *  o            [n_tokens, H, d] o_dtype (GDN_F32 or GDN_BF16); rows of
 *               tokens in no queried segment are left untouched
 *  d            64 or 128; io_dtype must be GDN_BF16
 * Segments must be disjoint ranges of the stream (trunks and branches in
 * any order) with non-decreasing offsets; offsets are clamped into
 * [0, n_tokens]. A branch whose parent is outside [0, n_req) gets NaN
 * outputs. Accumulation is fp32 with split-bf16 probabilities.
 * Errors: INVALID_ARG (NULL pointer, negative count, H_kv not dividing H,
 * scale not finite and positive, bad dtype code), UNSUPPORTED (d, fp32
 * q/k/v, or n_tokens * H * d >= 2^31), WORKSPACE, HIP.
 */
int gdn_fork_attention(const void *q, const void *k, const void *v,
                       const int32_t *cu_seqlens, int n_req,
                       const int32_t *branch_cu, const int32_t *branch_parent,
                       int n_branch, int n_tokens, int H, int H_kv, int d,
                       float scale, int trunk_queries, void *o, int io_dtype,
                       int o_dtype, void *workspace, size_t ws_bytes,
                       void *stream);

/*
 * gdn_fork_attention_noalloc -- gdn_fork_attention for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same computation and
 * arguments without a workspace. Its tile table lives in one file-scope
 * device array of the library, (GDN_FORK_ATTENTION_NOALLOC_MAX_SEGMENTS + 1)
 * int32 (256 KiB), which every GPU the library runs on holds from the
 * library's load until the process ends; its address on a device is looked
 * up on the first call with that device current. The call allocates and
 * frees nothing. Every call on one GPU shares that GPU's table, so calls
 * that overlap in time on one GPU (concurrent streams, or host threads
 * without ordering) race and must not be issued; calls ordered on one
 * stream are safe. Each call writes the whole part of the table it reads
 * before reading it, so nothing needs clearing between calls.
 *  n_req + n_branch  at most GDN_FORK_ATTENTION_NOALLOC_MAX_SEGMENTS
 *  stream            a stream of the calling thread's current device
 * Errors: as gdn_fork_attention; WORKSPACE when n_req + n_branch exceeds
 * the maximum; INVALID_ARG when the stream belongs to another device.
 */
#define GDN_FORK_ATTENTION_NOALLOC_MAX_SEGMENTS 65536
int gdn_fork_attention_noalloc(const void *q, const void *k, const void *v,
                               const int32_t *cu_seqlens, int n_req,
                               const int32_t *branch_cu,
                               const int32_t *branch_parent, int n_branch,
                               int n_tokens, int H, int H_kv, int d,
                               float scale, int trunk_queries, void *o,
                               int io_dtype, int o_dtype, void *stream);

/*
 * gdn_stream_probe -- a measurement aid, not part of the recurrence: streams
 * a device buffer with the access form the decode step uses for its state
 * (non-temporal 16-byte loads, and stores in copy mode), so the attainable
 * HBM rate is measured beside the kernels' own rates.
 *  src      n_bytes of device memory, read once
 *  dst      mode 0 (read): at least 4 bytes, normally left untouched (the
 *           loaded data is folded into a value that is stored only when it
 *           equals one NaN bit pattern); mode 1 (copy): n_bytes, receives a
 *           copy of src (the two buffers must not overlap)
 *  n_bytes  a multiple of 16 (0: nothing is enqueued, and src / dst may be
 *           NULL)
 * Errors: INVALID_ARG (NULL pointer with n_bytes > 0, n_bytes not a multiple
 * of 16, mode not 0 or 1), HIP.
 */
int gdn_stream_probe(const void *src, void *dst, size_t n_bytes, int mode, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_MI355X_H */
