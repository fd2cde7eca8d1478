/*
 * gdn_oracle.c -- plain fp64 CPU oracle for the Gated DeltaNet (GDN)
 * matrix-state recurrence and the three operations built on it
 * (shared-context prefill, forked branches, decode under a deferred
 * base + log schedule).
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * bench's CPU-baseline leg load this library. The product path (the HIP
 * library and its Python binding) never calls it, and the two share no
 * code: no headers, helpers, tables or constants. Every input arrives as
 * fp64 (bf16 / fp32 values widened exactly); every result is fp64.
 * Nothing here is blocked, fused or reordered beyond the definitions.
 *
 * Sources, cited by page title and section:
 *  [FL] "같은 맥락에서 여러 판단을 빠르게 처리하는 Flide" (yozm.zip summary of
 *       the Flide paper): glossary entries "ForkAttention" and "Gated
 *       DeltaNet" (the layer folds every past token into a fixed-size
 *       matrix state S_t; branches are forked from the shared state by two
 *       calls plus state indexing); section "연구방법을 단계별로" (method,
 *       step 2: the first call stores each request's final recurrent state
 *       and convolution window, the second runs every question from its own
 *       request's saved state; step 4: checkpoints hold state + conv window).
 *  [DL] "DeltaLog: Deferred Materialization of Recurrent States for Linear
 *       Attention Decoding" (gist.science summary): section
 *       "문제: 선형 어텐션 디코딩의 상태 업데이트 세금" (S_t is a dense d_k x d_v
 *       matrix per head, stored as [B,H,d_k,d_v]); "핵심 메커니즘: Base + Log"
 *       (dense base plus a bounded log of compressed factors and log-decay
 *       metadata; merge materialises base + replayed log); the operator list
 *       under "커널 구현" (GDN: scalar per-head decay with delta-rule
 *       correction; KDA: per-key decay with delta rule; RWKV6: per-key decay,
 *       raw-value update, no delta correction).
 *  [GD] The gated delta rule, S_t = a_t S_{t-1} (I - b_t k_t k_t^T)
 *       + b_t v_t k_t^T, o_t = S_t q_t (Yang, Kautz, Hatamizadeh, "Gated
 *       Delta Networks: Improving Mamba2 with Delta Rule", ICLR 2025).
 *
 * Orientation. The math state S is d_v x d_k. Storage follows [DL]'s
 * [.., d_k, d_v] layout, i.e. the stored matrix is Sig = S^T with
 * Sig[i][j] = S[j][i]; i indexes keys, j values.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - KDA decays before the delta correction:
 *      S_t = S_{t-1} diag(a_t) (I - b_t k_t k_t^T) + b_t v_t k_t^T;
 *    with equal entries of a_t this is exactly [GD].
 *  - RWKV6-style: S_t = S_{t-1} diag(a_t) + v_t k_t^T, o_t = S_t q_t
 *    (no beta, no bonus term).
 *  - Short convolution: depthwise, causal, width 4, over the concatenated
 *    channels [q | k | v] of all heads, no bias, no activation; positions
 *    before a sequence's first token come from the incoming 3-row window;
 *    the outgoing window is the last 3 raw inputs.
 *  - q and k are L2-normalised after the convolution:
 *      y <- y / sqrt(sum(y^2) + eps).
 *
 * parity: every function here is pinned by CPU tests (brute-force unrolled
 * products, closed forms, write-then-read, lookup table, linearity,
 * conv impulse/identity/split, fork == full run, replay == recurrence).
 */

#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_GDN 0
#define OR_KDA 1
#define OR_RWKV6 2

#define CONV_W 4 /* taps of the short convolution */
#define WIN (CONV_W - 1)

static int set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    return nthreads;
#else
    (void)nthreads;
    return 1;
#endif
}

int oracle_max_threads(void) { return set_threads(0); }

/*
 * One step of the recurrence on a stored state Sig (d_k x d_v, in place).
 *   a_i  = exp(log_alpha_i)          (scalar GDN: one value for every i)
 *   y    = S_{t-1} (a . k)           y_j = sum_i Sig[i][j] a_i k_i
 *   u    = b (v - y)                 (GDN, KDA; [GD] / [DL] delta rule)
 *        = v                         (RWKV6: raw-value update)
 *   S_t  = S_{t-1} diag(a) + u k^T   Sig[i][j] <- a_i Sig[i][j] + k_i u_j
 *   o    = S_t q                     o_j = sum_i Sig[i][j] q_i
 * For scalar a this is [GD]'s S_{t-1} a (I - b k k^T) + b v k^T with the
 * product distributed: a S - a b (S k) k^T + b v k^T = a S + b (v - a S k) k^T.
 * `y` is scratch of length d_v.
 */
static void recurrence_step(int dk, int dv, int variant, int per_key,
                            const double *q, const double *k, const double *v,
                            const double *log_alpha, double beta, double *Sig,
                            double *o, double *u_out, double *y, double *u) {
    for (int j = 0; j < dv; ++j) y[j] = 0.0;
    for (int i = 0; i < dk; ++i) {
        const double a = exp(per_key ? log_alpha[i] : log_alpha[0]);
        const double w = a * k[i];
        const double *row = Sig + (size_t)i * dv;
        for (int j = 0; j < dv; ++j) y[j] += row[j] * w;
    }
    for (int j = 0; j < dv; ++j)
        u[j] = (variant == OR_RWKV6) ? v[j] : beta * (v[j] - y[j]);
    for (int i = 0; i < dk; ++i) {
        const double a = exp(per_key ? log_alpha[i] : log_alpha[0]);
        double *row = Sig + (size_t)i * dv;
        for (int j = 0; j < dv; ++j) row[j] = a * row[j] + k[i] * u[j];
    }
    if (o) {
        for (int j = 0; j < dv; ++j) o[j] = 0.0;
        for (int i = 0; i < dk; ++i) {
            const double *row = Sig + (size_t)i * dv;
            for (int j = 0; j < dv; ++j) o[j] += row[j] * q[i];
        }
    }
    if (u_out)
        for (int j = 0; j < dv; ++j) u_out[j] = u[j];
}

/*
 * T steps of the recurrence for one (sequence, head), strided inputs:
 * element d of step t of q lives at q[t * qs + d] (same for the rest).
 * la_stride / beta_stride step the decay and beta arrays.
 */
static void run_unit(int T, int dk, int dv, int variant, int per_key,
                     const double *q, size_t qs, const double *k, size_t ks,
                     const double *v, size_t vs, const double *la,
                     size_t las, const double *beta, size_t bs, double *Sig,
                     double *o, size_t os, double *u, size_t us) {
    double *scratch = (double *)malloc(sizeof(double) * 2 * (size_t)dv);
    for (int t = 0; t < T; ++t) {
        const double b = (variant == OR_RWKV6 || !beta) ? 1.0 : beta[t * bs];
        recurrence_step(dk, dv, variant, per_key, q + t * qs, k + t * ks,
                        v + t * vs, la + t * las, b, Sig,
                        o ? o + t * os : NULL, u ? u + t * us : NULL, scratch,
                        scratch + dv);
    }
    free(scratch);
}

/*
 * O1 -- batched decode under the plain recurrence (eager semantics, which
 * is also what every deferred schedule must reproduce, [DL] "방법론").
 *   q, k  : [steps][B][H][dk]    v : [steps][B][H][dv]
 *   la    : [steps][B][H] (scalar) or [steps][B][H][dk] (per-key)
 *   beta  : [steps][B][H] (ignored for RWKV6; may be NULL then)
 *   state : [B][H][dk][dv] in/out (storage orientation)
 *   o     : [steps][B][H][dv] (may be NULL)
 *   u     : [steps][B][H][dv] (may be NULL) -- the rank-1 value factor
 *           u_t of each step, the quantity a deferred log records.
 */
void oracle_decode(int steps, int B, int H, int dk, int dv, int variant,
                   int per_key, const double *q, const double *k,
                   const double *v, const double *la, const double *beta,
                   double *state, double *o, double *u, int nthreads) {
    const int nt = set_threads(nthreads);
    const size_t BH = (size_t)B * H;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (long unit = 0; unit < (long)BH; ++unit) {
        const size_t ldk = per_key ? (size_t)dk : 1;
        run_unit(steps, dk, dv, variant, per_key, q + unit * dk, BH * dk,
                 k + unit * dk, BH * dk, v + unit * dv, BH * dv,
                 la + unit * ldk, BH * ldk, beta ? beta + unit : NULL, BH,
                 state + unit * (size_t)dk * dv, o ? o + unit * dv : NULL,
                 BH * dv, u ? u + unit * dv : NULL, BH * dv);
    }
}

/*
 * O2 -- short convolution + window for one head of one sequence, then the
 * q/k normalisation. Channel c of the concatenated stream:
 *   q channels  h*dk + i            (i < dk)
 *   k channels  H*dk + h*dk + i
 *   v channels  2*H*dk + h*dv + j   (j < dv)
 *   CC = H*(2*dk + dv) channels in all.
 * For token t of the sequence and tap r:
 *   y_t[c] = sum_{r=0..3} w[c][r] * x_{t-3+r}[c]
 * where x_p for p < 0 is row 3+p of the incoming window (rows are oldest
 * first). conv_w == NULL means no convolution (y = x).
 * The outgoing window row r holds x_{len-3+r} (window rows when that
 * position is before the sequence start).
 * Output buffers: yq [len][dk], yk [len][dk], yv [len][dv].
 */
static void conv_head(int len, int H, int h, int dk, int dv,
                      const double *q, const double *k, const double *v,
                      const double *win_in, const double *conv_w, int qk_norm,
                      double eps, double *yq, double *yk, double *yv,
                      double *win_out) {
    const size_t cc = (size_t)H * (2 * dk + dv);
    /* the three inputs as parts of one channel space: (pointer at this
     * head's first channel, token stride, first channel inside the
     * concatenation, width) */
    const double *src[3] = {q + (size_t)h * dk, k + (size_t)h * dk,
                            v + (size_t)h * dv};
    const size_t tok_stride[3] = {(size_t)H * dk, (size_t)H * dk,
                                  (size_t)H * dv};
    const size_t c0[3] = {(size_t)h * dk, (size_t)H * dk + (size_t)h * dk,
                          2 * (size_t)H * dk + (size_t)h * dv};
    const int width[3] = {dk, dk, dv};
    double *dst[3] = {yq, yk, yv};
    for (int part = 0; part < 3; ++part) {
        for (int ch = 0; ch < width[part]; ++ch) {
            const size_t c = c0[part] + ch;
            /* raw input of this channel at sequence position p (p < 0: the
             * incoming window, oldest row first; no window: zeros) */
#define RAW(p)                                                              \
    ((p) >= 0 ? src[part][(size_t)(p) * tok_stride[part] + ch]              \
              : (win_in ? win_in[(size_t)(WIN + (p)) * cc + c] : 0.0))
            for (int t = 0; t < len; ++t) {
                double y;
                if (conv_w) {
                    y = 0.0;
                    for (int r = 0; r < CONV_W; ++r)
                        y += conv_w[c * CONV_W + r] * RAW(t - WIN + r);
                } else {
                    y = RAW(t);
                }
                dst[part][(size_t)t * width[part] + ch] = y;
            }
            if (win_out)
                for (int r = 0; r < WIN; ++r)
                    win_out[(size_t)r * cc + c] = RAW(len - WIN + r);
#undef RAW
        }
    }
    if (qk_norm) {
        for (int part = 0; part < 2; ++part) {
            for (int t = 0; t < len; ++t) {
                double *row = dst[part] + (size_t)t * dk;
                double ss = 0.0;
                for (int i = 0; i < dk; ++i) ss += row[i] * row[i];
                const double inv = 1.0 / sqrt(ss + eps);
                for (int i = 0; i < dk; ++i) row[i] *= inv;
            }
        }
    }
}

/*
 * O2 (exported) -- the convolution + normalisation of one whole sequence,
 * every head: q, k [len][H][dk], v [len][H][dv] in; yq, yk [len][H][dk],
 * yv [len][H][dv] out; win_in / win_out [3][CC] (either may be NULL).
 */
void oracle_conv(int len, int H, int dk, int dv, const double *q,
                 const double *k, const double *v, const double *win_in,
                 const double *conv_w, int qk_norm, double eps, double *yq,
                 double *yk, double *yv, double *win_out) {
    double *tq = (double *)malloc(sizeof(double) * ((size_t)len * dk + 1));
    double *tk = (double *)malloc(sizeof(double) * ((size_t)len * dk + 1));
    double *tv = (double *)malloc(sizeof(double) * ((size_t)len * dv + 1));
    for (int h = 0; h < H; ++h) {
        conv_head(len, H, h, dk, dv, q, k, v, win_in, conv_w, qk_norm, eps, tq,
                  tk, tv, win_out);
        for (int t = 0; t < len; ++t) {
            memcpy(yq + ((size_t)t * H + h) * dk, tq + (size_t)t * dk,
                   sizeof(double) * dk);
            memcpy(yk + ((size_t)t * H + h) * dk, tk + (size_t)t * dk,
                   sizeof(double) * dk);
            memcpy(yv + ((size_t)t * H + h) * dv, tv + (size_t)t * dv,
                   sizeof(double) * dv);
        }
    }
    free(tq);
    free(tk);
    free(tv);
}

/*
 * O3 -- run a set of sequences of a flat token stream ([FL] method step 1:
 * tokens packed into one stream, membership given by offsets).
 * Sequence s covers tokens [cu[s], cu[s+1]) and starts from the state and
 * window of `src(s)` = parent ? parent[s] : s.
 *   q, k : [N][H][dk]   v : [N][H][dv]   la, beta : [N][H] (or [N][H][dk])
 *   state_in  : [*][H][dk][dv] or NULL (zeros)
 *   win_in    : [*][3][CC] or NULL (zeros)
 *   o         : [N][H][dv] or NULL
 *   state_out : [nseq][H][dk][dv] or NULL
 *   win_out   : [nseq][3][CC] or NULL
 * With parent == NULL this is the shared-context prefill (call 1 of [FL]
 * step 2); with a parent map it is the branch call (call 2).
 */
void oracle_sequences(int nseq, const int *cu, const int *parent, int H,
                      int dk, int dv, int variant, int per_key,
                      const double *q, const double *k, const double *v,
                      const double *la, const double *beta,
                      const double *conv_w, int qk_norm, double eps,
                      const double *state_in, const double *win_in, double *o,
                      double *state_out, double *win_out, int nthreads) {
    const int nt = set_threads(nthreads);
    const size_t cc = (size_t)H * (2 * dk + dv);
    const size_t ldk = per_key ? (size_t)dk : 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (long unit = 0; unit < (long)nseq * H; ++unit) {
        const int s = (int)(unit / H), h = (int)(unit % H);
        const int src = parent ? parent[s] : s;
        const int t0 = cu[s], len = cu[s + 1] - cu[s];
        double *yq = (double *)malloc(sizeof(double) * ((size_t)len * dk + 1));
        double *yk = (double *)malloc(sizeof(double) * ((size_t)len * dk + 1));
        double *yv = (double *)malloc(sizeof(double) * ((size_t)len * dv + 1));
        double *Sig = (double *)calloc((size_t)dk * dv, sizeof(double));
        const double *w_in = win_in ? win_in + (size_t)src * WIN * cc : NULL;
        double *w_out = win_out ? win_out + (size_t)s * WIN * cc : NULL;
        conv_head(len, H, h, dk, dv, q + (size_t)t0 * H * dk,
                  k + (size_t)t0 * H * dk, v + (size_t)t0 * H * dv, w_in,
                  conv_w, qk_norm, eps, yq, yk, yv, w_out);
        if (state_in)
            memcpy(Sig, state_in + ((size_t)src * H + h) * dk * dv,
                   sizeof(double) * (size_t)dk * dv);
        run_unit(len, dk, dv, variant, per_key, yq, dk, yk, dk, yv, dv,
                 la + ((size_t)t0 * H + h) * ldk, (size_t)H * ldk,
                 beta ? beta + (size_t)t0 * H + h : NULL, H, Sig,
                 o ? o + ((size_t)t0 * H + h) * dv : NULL, (size_t)H * dv,
                 NULL, 0);
        if (state_out)
            memcpy(state_out + ((size_t)s * H + h) * dk * dv, Sig,
                   sizeof(double) * (size_t)dk * dv);
        free(yq);
        free(yk);
        free(yv);
        free(Sig);
    }
}

/*
 * O4 -- materialise a deferred state ([DL] "핵심 메커니즘: Base + Log"): the
 * logical state is the dense base carried forward by the log's decay plus
 * every logged rank-1 update replayed with the decay accumulated since it
 * was logged. Entry e (0-based, e < m) holds u_e [dv], k_e [dk] and the
 * cumulative log-decay Lam_e since the base was written (scalar or [dk]).
 *   Sig[i][j] = exp(Lam_{m-1}[i]) base[i][j]
 *             + sum_{e<m} k_e[i] exp(Lam_{m-1}[i] - Lam_e[i]) u_e[j]
 * m == 0 returns the base unchanged.
 *   base  : [n][dk][dv]   log_u : [n][Mcap][dv]   log_k : [n][Mcap][dk]
 *   log_lam : [n][Mcap] or [n][Mcap][dk]   m : [n]   out : [n][dk][dv]
 */
void oracle_materialize(int n, int dk, int dv, int per_key, int Mcap,
                        const int *m, const double *base, const double *log_u,
                        const double *log_k, const double *log_lam,
                        double *out, int nthreads) {
    const int nt = set_threads(nthreads);
    const size_t ldk = per_key ? (size_t)dk : 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (long unit = 0; unit < (long)n; ++unit) {
        const int mu = m[unit];
        const double *B0 = base + (size_t)unit * dk * dv;
        const double *U = log_u + (size_t)unit * Mcap * dv;
        const double *K = log_k + (size_t)unit * Mcap * dk;
        const double *L = log_lam + (size_t)unit * Mcap * ldk;
        double *S = out + (size_t)unit * dk * dv;
        for (int i = 0; i < dk; ++i) {
            const double lam_last =
                mu > 0 ? L[(size_t)(mu - 1) * ldk + (per_key ? i : 0)] : 0.0;
            for (int j = 0; j < dv; ++j) {
                double acc = exp(lam_last) * B0[(size_t)i * dv + j];
                for (int e = 0; e < mu; ++e) {
                    const double lam_e = L[(size_t)e * ldk + (per_key ? i : 0)];
                    acc += K[(size_t)e * dk + i] * exp(lam_last - lam_e) *
                           U[(size_t)e * dv + j];
                }
                S[(size_t)i * dv + j] = acc;
            }
        }
    }
}
