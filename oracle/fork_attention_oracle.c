/*
 * fork_attention_oracle.c -- plain fp64 CPU oracle for softmax attention
 * over a flat token stream under the fork visibility rule.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the
 * bench's CPU-baseline leg load this code (it is linked into the same
 * liboracle.so as gdn_oracle.c). It shares nothing with the HIP library.
 * Every input arrives as fp64; every result is fp64. Nothing is blocked,
 * fused or reordered beyond the definition below.
 *
 * Source: "같은 맥락에서 여러 판단을 빠르게 처리하는 Flide" (yozm.zip summary
 * of the Flide paper), section "연구방법을 단계별로", method step 1, and the
 * glossary entry "ForkAttention": requests and questions are recorded as
 * GPU metadata over one flat token stream; a token reads only its own
 * request's shared trunk and the current and earlier tokens of its own
 * branch; other questions placed earlier in the stream and other requests
 * stay invisible. Softmax attention itself is the textbook definition:
 *     o_i = sum_j w_ij v_j,   w_ij = exp(s_ij) / sum_j' exp(s_ij'),
 *     s_ij = scale * <q_i, k_j>,   j, j' over the keys visible to i.
 *
 * Readings where the page is silent (each is listed in the design notes):
 *  - a trunk token at position p of its request sees the trunk tokens at
 *    positions 0..p of the same request (causal);
 *  - a branch token at position p of its branch sees its parent request's
 *    whole trunk and positions 0..p of its own branch;
 *  - grouped heads: head h reads key/value head h / (H / H_kv);
 *  - the exponent is taken relative to the largest visible score, which
 *    leaves every weight unchanged in exact arithmetic.
 *
 * parity: pinned by CPU tests (a library causal attention on each trunk,
 * fork == the same attention over trunk ++ branch as one sequence,
 * identical keys give the mean of the visible values, a dominant key
 * returns its value, invisible tokens have no effect, grouped heads equal
 * repeated heads).
 */

#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Attention of query row i (head h) over the visible key rows listed in
 * keys[0..n-1]; writes d values to out. */
static void attend_one(int n, const int *keys, const double *q, const double *k,
                       const double *v, int H, int Hkv, int d, int i, int h, double scale,
                       double *w, double *out) {
    const int hk = h / (H / Hkv);
    const double *qi = q + ((size_t)i * H + h) * d;
    double smax = -INFINITY;
    for (int t = 0; t < n; ++t) {
        const double *kj = k + ((size_t)keys[t] * Hkv + hk) * d;
        double s = 0.0;
        for (int c = 0; c < d; ++c) s += qi[c] * kj[c];
        w[t] = scale * s;
        if (w[t] > smax) smax = w[t];
    }
    double den = 0.0;
    for (int t = 0; t < n; ++t) {
        w[t] = exp(w[t] - smax);
        den += w[t];
    }
    for (int c = 0; c < d; ++c) out[c] = 0.0;
    for (int t = 0; t < n; ++t) {
        const double *vj = v + ((size_t)keys[t] * Hkv + hk) * d;
        for (int c = 0; c < d; ++c) out[c] += (w[t] / den) * vj[c];
    }
}

/*
 * q [n_tokens, H, d], k and v [n_tokens, H_kv, d]; cu [n_req + 1] trunk
 * offsets, bcu [n_branch + 1] branch offsets (both absolute token indices
 * into the stream), bparent [n_branch] the request of each branch.
 * o [n_tokens, H, d]: rows of trunk tokens (when trunk_queries) and of
 * branch tokens are written; every other row is left as it is.
 */
void oracle_fork_attention(int n_tokens, int H, int Hkv, int d, const double *q,
                           const double *k, const double *v, int n_req, const int *cu,
                           int n_branch, const int *bcu, const int *bparent, double scale,
                           int trunk_queries, double *o, int nthreads) {
    (void)n_tokens;
    const int n_seg = n_req + n_branch;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#else
    (void)nthreads;
#endif
    for (int sh = 0; sh < n_seg * H; ++sh) {
        const int seg = sh / H, h = sh % H;
        int t0, len, p0 = 0, plen = 0;
        if (seg < n_req) {
            if (!trunk_queries) continue;
            t0 = cu[seg];
            len = cu[seg + 1] - cu[seg];
        } else {
            const int b = seg - n_req, r = bparent[b];
            t0 = bcu[b];
            len = bcu[b + 1] - bcu[b];
            p0 = cu[r];
            plen = cu[r + 1] - cu[r];
        }
        if (len <= 0) continue;
        int *keys = malloc(sizeof(int) * (size_t)(plen + len));
        double *w = malloc(sizeof(double) * (size_t)(plen + len));
        for (int p = 0; p < len; ++p) {
            int n = 0;
            for (int j = 0; j < plen; ++j) keys[n++] = p0 + j; /* the parent's trunk */
            for (int j = 0; j <= p; ++j) keys[n++] = t0 + j;   /* own tokens 0..p */
            attend_one(n, keys, q, k, v, H, Hkv, d, t0 + p, h, scale, w,
                       o + ((size_t)(t0 + p) * H + h) * d);
        }
        free(keys);
        free(w);
    }
}
