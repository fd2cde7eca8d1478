// prefill.hip -- chunked prefill of the GDN recurrence over a flat token
// stream, used by both calls of the two-call fork: the shared contexts
// (call 1) and the branches, each started from its own request's saved
// state and conv window (call 2).
//
// Sources: "같은 맥락에서 여러 판단을 빠르게 처리하는 Flide" (yozm.zip summary)
// -- section "연구방법을 단계별로", step 1 (tokens of all requests packed in
// one flat stream, membership as GPU metadata), step 2 (call 1 stores the
// final recurrent state and conv window, call 2 runs every question from
// its own request's saved state); glossary "Gated DeltaNet" (fixed-size
// matrix state). The pages do not describe a prefill algorithm: the chunked
// form below is derived from the recurrence (gated delta rule, Yang et al.,
// ICLR 2025) and checked against the fp64 step-by-step oracle.
//
// Chunked form. In a chunk of L <= C tokens with incoming stored state
// Sig0 (= S0^T, [d_k][d_v]), g_r = running sum of log a inside the chunk,
// gamma_r = exp(g_r):
//   A[r][s] = beta_r exp(g_r - g_s) <k_r, k_s>            (s < r)
//   T = (I + A)^-1 (unit lower triangular),  T' = T diag(beta)
//   P[r][s] = exp(g_r - g_s) <q_r, k_s>                    (s <= r)
//   U = T' (V - diag(gamma) K Sig0)       the chunk's rank-1 factors u_r
//   O = diag(gamma) Q Sig0 + P U          o_r = S_r q_r
//   Sig_L = gamma_L Sig0 + sum_r exp(g_L - g_r) k_r u_r^T
// Column j of U, O, Sig depends only on column j of V and Sig0, so value
// tiles are independent.
//
// Kernels:
//   plan  -- one workgroup: per-sequence chunk offsets (prefix sum of
//            ceil(len/C)) into the workspace, from the device offsets.
//   prep  -- one workgroup per (chunk, head), all chunks in parallel: conv
//            + q/k norm of the chunk, then T' and P (key-side only) to the
//            workspace.
//   scan  -- one workgroup per (sequence, head, value tile of 32): walks the
//            sequence's chunks in order with the state tile resident in LDS,
//            recomputing the chunk's conv'd q/k/v and applying the chunk
//            form; writes o, the final state tile and (tile 0) the window.

#include <type_traits>

#include "gdn_device.hpp"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int C = 64;        // chunk length
constexpr int CP = C + 4;    // padded row of a transposed [d][C] tile
constexpr int TV = 32;       // value-tile width of the scan
constexpr float kNormEps = 1e-6f;

// ------------------------------------------------------------ workspace
struct WsLayout {
    size_t chunk_start_off;  // int32 [n_seq + 1]
    size_t rec_off;          // per (chunk, head) record
    size_t rec_floats;       // T'^T [C][C], P^T [C][C], g [C]
    size_t max_chunks;
    size_t total;
};

__host__ __device__ WsLayout ws_layout(int n_tokens, int n_seq, int H) {
    WsLayout w{};
    auto align = [](size_t x) { return (x + 255) & ~size_t(255); };
    w.max_chunks = (size_t)n_tokens / C + (size_t)n_seq;
    w.chunk_start_off = 0;
    w.rec_off = align(sizeof(int32_t) * ((size_t)n_seq + 1));
    w.rec_floats = 2 * (size_t)C * C + C;
    w.total = w.rec_off + sizeof(float) * w.rec_floats * w.max_chunks * (size_t)H;
    return w;
}

struct SeqSpan {
    int start, len;
};

__device__ __forceinline__ SeqSpan seq_span(const int32_t *cu, int s, int n_tokens) {
    const int a = min(max(cu[s], 0), n_tokens);
    const int b = min(max(cu[s + 1], a), n_tokens);
    return {a, b - a};
}

// ------------------------------------------------------------ plan
// chunk_start[s] = min(sum_{s' < s} ceil(len_s' / C), max_chunks): the
// first record of sequence s; sequence s owns chunk_start[s+1] -
// chunk_start[s] chunks. With valid offsets the cap never binds; with
// overlapping (invalid) offsets it keeps every record inside the workspace.
__global__ __launch_bounds__(kThreads) void plan_kernel(const int32_t *cu, int n_seq, int n_tokens,
                                                        long long max_chunks,
                                                        int32_t *chunk_start) {
    __shared__ long long s_part[kThreads];
    const int tid = threadIdx.x;
    const int per = (n_seq + kThreads - 1) / kThreads;
    const int lo = min(tid * per, n_seq), hi = min(lo + per, n_seq);
    long long sum = 0;
    for (int s = lo; s < hi; ++s) sum += (seq_span(cu, s, n_tokens).len + C - 1) / C;
    s_part[tid] = sum;
    __syncthreads();
    if (tid == 0) {
        long long run = 0;
        for (int i = 0; i < kThreads; ++i) {
            const long long x = s_part[i];
            s_part[i] = run;
            run += x;
        }
    }
    __syncthreads();
    long long run = s_part[tid];
    for (int s = lo; s < hi; ++s) {
        chunk_start[s] = (int32_t)min(run, max_chunks);
        run += (seq_span(cu, s, n_tokens).len + C - 1) / C;
    }
    if (tid == kThreads - 1) chunk_start[n_seq] = (int32_t)min(run, max_chunks);
}

// ------------------------------------------------------------ conv + norm
// Conv'd inputs of one part (q, k or v) of head h for the chunk rows
// l < L, columns [d_begin, d_begin + W) of the part (head size D), written
// to dst[d * ld + l] (transposed) or dst[l * ld + d]; rows l >= L are zero.
// Position p of the sequence reads x[(seq0 + p)] for p >= 0, else row 3+p
// of the incoming window (zeros without one).
template <typename TI, bool TRANSPOSED>
__device__ void conv_part(const TI *x, int H, int D, int h, int d_begin, int W, int seq0, int p0,
                          int L, const TI *win, int CC, int cbase, const float *w, float *dst,
                          int ld) {
    for (int idx = threadIdx.x; idx < C * W; idx += kThreads) {
        const int d = idx % W, l = idx / W;
        float y = 0.f;
        if (l < L) {
            const int c = cbase + h * D + d_begin + d;  // channel in [q | k | v]
            const size_t col = (size_t)h * D + d_begin + d;
            if (w) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int p = p0 + l - 3 + r;
                    float xv;
                    if (p >= 0)
                        xv = to_f32(x[(size_t)(seq0 + p) * H * D + col]);
                    else
                        xv = win ? to_f32(win[(size_t)(3 + p) * CC + c]) : 0.f;
                    y = fmaf(w[(size_t)c * 4 + r], xv, y);
                }
            } else {
                y = to_f32(x[(size_t)(seq0 + p0 + l) * H * D + col]);
            }
        }
        dst[TRANSPOSED ? d * ld + l : l * ld + d] = y;
    }
}

// L2-normalise the C rows of a transposed [D][ld] tile in place.
template <int D>
__device__ void norm_rows_transposed(float *t, int ld, float *s_inv) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    for (int l = wave; l < C; l += kWaves) {
        float ss = 0.f;
        for (int d = lane; d < D; d += kWave) ss = fmaf(t[d * ld + l], t[d * ld + l], ss);
        ss = wave_sum(ss);
        if (lane == 0) s_inv[l] = 1.0f / sqrtf(ss + kNormEps);
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < C * D; idx += kThreads) {
        const int d = idx / C, l = idx % C;
        t[d * ld + l] *= s_inv[l];
    }
    __syncthreads();
}

__device__ __forceinline__ int find_seq(const int32_t *chunk_start, int n_seq, int gc) {
    int lo = 0, hi = n_seq;  // last s in [0, n_seq) with chunk_start[s] <= gc
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (chunk_start[mid] <= gc) lo = mid;
        else hi = mid;
    }
    return lo;
}

// ------------------------------------------------------------ prep
template <int DK, int DV, typename TI>
__global__ __launch_bounds__(kThreads) void prep_kernel(PrefillArgs a) {
    __shared__ float s_qt[DK * CP], s_kt[DK * CP];
    __shared__ float s_A[C * (C + 1)];   // A, then T (row-major, padded)
    __shared__ float s_g[C], s_b[C], s_inv[C];

    const int32_t *chunk_start = static_cast<const int32_t *>(a.ws);
    const int gc = blockIdx.x, h = blockIdx.y;
    if (gc >= chunk_start[a.n_seq]) return;
    const int s = find_seq(chunk_start, a.n_seq, gc);
    const SeqSpan sp = seq_span(a.cu, s, a.n_tokens);
    const int c = gc - chunk_start[s];
    const int p0 = c * C;
    const int L = min(C, sp.len - p0);
    const int H = a.H;
    const int CC = H * (2 * DK + DV);
    const int src = a.parent ? a.parent[s] : s;
    const bool src_ok = src >= 0 && src < a.n_parent;
    const TI *win = (a.win_in && src_ok) ? static_cast<const TI *>(a.win_in) + (size_t)src * 3 * CC
                                         : nullptr;
    const int tid = threadIdx.x;

    conv_part<TI, true>(static_cast<const TI *>(a.q), H, DK, h, 0, DK, sp.start, p0, L, win, CC, 0,
                        a.conv_w, s_qt, CP);
    conv_part<TI, true>(static_cast<const TI *>(a.k), H, DK, h, 0, DK, sp.start, p0, L, win, CC,
                        H * DK, a.conv_w, s_kt, CP);
    if (tid == 0) {
        float g = 0.f;
        for (int r = 0; r < C; ++r) {
            if (r < L) g += a.log_alpha[(size_t)(sp.start + p0 + r) * H + h];
            s_g[r] = g;
            s_b[r] = r < L ? a.beta[(size_t)(sp.start + p0 + r) * H + h] : 0.f;
        }
    }
    __syncthreads();
    if (a.qk_norm) {
        norm_rows_transposed<DK>(s_qt, CP, s_inv);
        norm_rows_transposed<DK>(s_kt, CP, s_inv);
    }

    // A and P: 4x4 outputs per thread
    float *rec = reinterpret_cast<float *>(static_cast<char *>(a.ws) +
                                           ws_layout(a.n_tokens, a.n_seq, H).rec_off) +
                 ((size_t)gc * H + h) * (2 * C * C + C);
    float *Tt = rec;            // T'^T : Tt[s][r] = T[r][s] beta_s
    float *Pt = rec + C * C;    // P^T  : Pt[s][r] = P[r][s]
    float *G = rec + 2 * C * C; // g
    {
        const int r0 = (tid / 16) * 4, c0 = (tid % 16) * 4;
        float kk[4][4] = {}, qk[4][4] = {};
        for (int d = 0; d < DK; ++d) {
            const float4 kr = *reinterpret_cast<const float4 *>(s_kt + d * CP + r0);
            const float4 qr = *reinterpret_cast<const float4 *>(s_qt + d * CP + r0);
            const float4 kc = *reinterpret_cast<const float4 *>(s_kt + d * CP + c0);
            const float krv[4] = {kr.x, kr.y, kr.z, kr.w}, qrv[4] = {qr.x, qr.y, qr.z, qr.w};
            const float kcv[4] = {kc.x, kc.y, kc.z, kc.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    kk[i][j] = fmaf(krv[i], kcv[j], kk[i][j]);
                    qk[i][j] = fmaf(qrv[i], kcv[j], qk[i][j]);
                }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = r0 + i, sc = c0 + j;
                const bool live = r < L && sc < L;
                const float dec = live && sc <= r ? expf(s_g[r] - s_g[sc]) : 0.f;
                s_A[r * (C + 1) + sc] = (sc < r) ? s_b[r] * dec * kk[i][j] : 0.f;
                Pt[sc * C + r] = dec * qk[i][j];
            }
    }
    __syncthreads();

    // T = (I + A)^-1 by forward substitution, row by row; T overwrites A
    // (row r of A is read before row r of T is written; rows < r hold T).
    // Four lanes share one column s and split the sum over j.
    {
        const int sc = tid / 4, part = tid % 4;
        for (int r = 1; r < C; ++r) {
            float acc = 0.f;
            if (sc < r)
                for (int j = sc + part; j < r; j += 4)
                    acc = fmaf(s_A[r * (C + 1) + j], (j == sc) ? 1.f : s_A[j * (C + 1) + sc], acc);
            acc += __shfl_xor(acc, 1, kWave);
            acc += __shfl_xor(acc, 2, kWave);
            __syncthreads();
            if (sc < r && part == 0) s_A[r * (C + 1) + sc] = -acc;
            __syncthreads();
        }
    }
    for (int idx = tid; idx < C * C; idx += kThreads) {
        const int sc = idx / C, r = idx % C;  // Tt[sc][r] = T[r][sc] beta_sc
        const float t = r == sc ? 1.f : (sc < r ? s_A[r * (C + 1) + sc] : 0.f);
        Tt[idx] = t * s_b[sc];
    }
    if (tid < C) G[tid] = s_g[tid];
}

// ------------------------------------------------------------ scan
template <int DK, int DV, typename TI, typename TO>
__global__ __launch_bounds__(kThreads) void scan_kernel(PrefillArgs a) {
    __shared__ float s_S[DK * TV];     // state tile [DK][TV]
    __shared__ float s_qt[DK * CP];    // conv'd, normalised q, transposed
    __shared__ float s_kt[DK * CP];    // conv'd, normalised k, transposed
    __shared__ float s_v[C * TV];      // V, then R
    __shared__ float s_u[C * TV];      // U
    __shared__ float s_tt[C * C];      // T'^T
    __shared__ float s_pt[C * C];      // P^T
    __shared__ float s_g[C], s_inv[C];

    constexpr int NT = DV / TV;
    const int tile = blockIdx.x % NT;
    const int sh = blockIdx.x / NT;
    const int s = sh / a.H, h = sh % a.H;
    const int H = a.H;
    const int CC = H * (2 * DK + DV);
    const int j0 = tile * TV;
    const int tid = threadIdx.x;
    const int32_t *chunk_start = static_cast<const int32_t *>(a.ws);
    const WsLayout wl = ws_layout(a.n_tokens, a.n_seq, H);
    const SeqSpan sp = seq_span(a.cu, s, a.n_tokens);
    const int src = a.parent ? a.parent[s] : s;
    const bool src_ok = src >= 0 && src < a.n_parent;

    if (!src_ok) {  // a branch with an invalid parent: NaN outputs, nothing else
        if (a.o)
            for (int idx = tid; idx < sp.len * TV; idx += kThreads)
                static_cast<TO *>(a.o)[((size_t)(sp.start + idx / TV) * H + h) * DV + j0 + idx % TV] =
                    from_f32<TO>(quiet_nan());
        if (a.state_out)
            for (int idx = tid; idx < DK * TV; idx += kThreads)
                a.state_out[(((size_t)s * H + h) * DK + idx / TV) * DV + j0 + idx % TV] = quiet_nan();
        return;
    }
    const TI *win = a.win_in ? static_cast<const TI *>(a.win_in) + (size_t)src * 3 * CC : nullptr;

    for (int idx = tid; idx < DK * TV; idx += kThreads) {
        const int d = idx / TV, j = idx % TV;
        s_S[idx] = a.state_in ? a.state_in[(((size_t)src * H + h) * DK + d) * DV + j0 + j] : 0.f;
    }

    const int nchunks = chunk_start[s + 1] - chunk_start[s];  // <= ceil(len / C)
    for (int c = 0; c < nchunks; ++c) {
        const int p0 = c * C;
        const int L = min(C, sp.len - p0);
        const float *rec = reinterpret_cast<const float *>(static_cast<const char *>(a.ws) + wl.rec_off) +
                           ((size_t)(chunk_start[s] + c) * H + h) * wl.rec_floats;
        __syncthreads();  // previous chunk done with every buffer
        conv_part<TI, true>(static_cast<const TI *>(a.q), H, DK, h, 0, DK, sp.start, p0, L, win, CC,
                            0, a.conv_w, s_qt, CP);
        conv_part<TI, true>(static_cast<const TI *>(a.k), H, DK, h, 0, DK, sp.start, p0, L, win, CC,
                            H * DK, a.conv_w, s_kt, CP);
        conv_part<TI, false>(static_cast<const TI *>(a.v), H, DV, h, j0, TV, sp.start, p0, L, win,
                             CC, 2 * H * DK, a.conv_w, s_v, TV);
        for (int idx = tid; idx < C * C / 4; idx += kThreads) {
            reinterpret_cast<float4 *>(s_tt)[idx] = reinterpret_cast<const float4 *>(rec)[idx];
            reinterpret_cast<float4 *>(s_pt)[idx] = reinterpret_cast<const float4 *>(rec + C * C)[idx];
        }
        if (tid < C) s_g[tid] = rec[2 * C * C + tid];
        __syncthreads();
        if (a.qk_norm) {
            norm_rows_transposed<DK>(s_qt, CP, s_inv);
            norm_rows_transposed<DK>(s_kt, CP, s_inv);
        }

        // 4 rows x 2 columns of a [C][TV] output per thread
        const int l0 = (tid / 16) * 4, cj = (tid % 16) * 2;
        float gam[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) gam[i] = expf(s_g[l0 + i]);

        // R = V - diag(gamma) K Sig0
        {
            float acc[4][2] = {};
            for (int d = 0; d < DK; ++d) {
                const float4 kr = *reinterpret_cast<const float4 *>(s_kt + d * CP + l0);
                const float2 sv = *reinterpret_cast<const float2 *>(s_S + d * TV + cj);
                const float kv[4] = {kr.x, kr.y, kr.z, kr.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[i][0] = fmaf(kv[i], sv.x, acc[i][0]);
                    acc[i][1] = fmaf(kv[i], sv.y, acc[i][1]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    float *vv = s_v + (l0 + i) * TV + cj + j;
                    *vv = *vv - gam[i] * acc[i][j];
                }
        }
        __syncthreads();
        // U = T' R
        {
            float acc[4][2] = {};
            const int smax = min(l0 + 4, C);
            for (int sc = 0; sc < smax; ++sc) {
                const float4 tr = *reinterpret_cast<const float4 *>(s_tt + sc * C + l0);
                const float2 rv = *reinterpret_cast<const float2 *>(s_v + sc * TV + cj);
                const float tv[4] = {tr.x, tr.y, tr.z, tr.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[i][0] = fmaf(tv[i], rv.x, acc[i][0]);
                    acc[i][1] = fmaf(tv[i], rv.y, acc[i][1]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s_u[(l0 + i) * TV + cj] = acc[i][0];
                s_u[(l0 + i) * TV + cj + 1] = acc[i][1];
            }
        }
        __syncthreads();
        // O = diag(gamma) Q Sig0 + P U
        if (a.o) {
            float acc[4][2] = {}, pu[4][2] = {};
            for (int d = 0; d < DK; ++d) {
                const float4 qr = *reinterpret_cast<const float4 *>(s_qt + d * CP + l0);
                const float2 sv = *reinterpret_cast<const float2 *>(s_S + d * TV + cj);
                const float qv[4] = {qr.x, qr.y, qr.z, qr.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[i][0] = fmaf(qv[i], sv.x, acc[i][0]);
                    acc[i][1] = fmaf(qv[i], sv.y, acc[i][1]);
                }
            }
            const int smax = min(l0 + 4, C);
            for (int sc = 0; sc < smax; ++sc) {
                const float4 pr = *reinterpret_cast<const float4 *>(s_pt + sc * C + l0);
                const float2 uv = *reinterpret_cast<const float2 *>(s_u + sc * TV + cj);
                const float pv[4] = {pr.x, pr.y, pr.z, pr.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pu[i][0] = fmaf(pv[i], uv.x, pu[i][0]);
                    pu[i][1] = fmaf(pv[i], uv.y, pu[i][1]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int l = l0 + i;
                if (l < L) {
                    TO *orow = static_cast<TO *>(a.o) + ((size_t)(sp.start + p0 + l) * H + h) * DV + j0 + cj;
                    orow[0] = from_f32<TO>(fmaf(gam[i], acc[i][0], pu[i][0]));
                    orow[1] = from_f32<TO>(fmaf(gam[i], acc[i][1], pu[i][1]));
                }
            }
        }
        __syncthreads();  // O read the old state
        // Sig <- gamma_L Sig + K~^T U,  K~_l = exp(g_L - g_l) k_l
        {
            const float gL = s_g[C - 1];  // rows >= L add nothing to g
            const float gamL = expf(gL);
            for (int idx = tid; idx < C * TV; idx += kThreads) {
                const int l = idx / TV;
                s_u[idx] *= (l < L) ? expf(gL - s_g[l]) : 0.f;
            }
            __syncthreads();
            const int d0 = (tid / 8) * 4, c0 = (tid % 8) * 4;  // DK <= 128 rows
            float acc[4][4] = {};
            if (d0 < DK)
            for (int l = 0; l < L; ++l) {
                const float4 uv = *reinterpret_cast<const float4 *>(s_u + l * TV + c0);
                const float uu[4] = {uv.x, uv.y, uv.z, uv.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float kd = s_kt[(d0 + i) * CP + l];
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(kd, uu[j], acc[i][j]);
                }
            }
            if (d0 < DK)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float4 *sp4 = reinterpret_cast<float4 *>(s_S + (d0 + i) * TV + c0);
                const float4 old = *sp4;
                *sp4 = make_float4(fmaf(gamL, old.x, acc[i][0]), fmaf(gamL, old.y, acc[i][1]),
                                   fmaf(gamL, old.z, acc[i][2]), fmaf(gamL, old.w, acc[i][3]));
            }
        }
    }
    __syncthreads();
    if (a.state_out)
        for (int idx = tid; idx < DK * TV; idx += kThreads) {
            const int d = idx / TV, j = idx % TV;
            a.state_out[(((size_t)s * H + h) * DK + d) * DV + j0 + j] = s_S[idx];
        }
    // window out (tile 0): the last 3 raw inputs of the head's channels
    if (a.win_out && tile == 0) {
        TI *wo = static_cast<TI *>(a.win_out) + (size_t)s * 3 * CC;
        const int W = 2 * DK + DV;
        for (int idx = tid; idx < 3 * W; idx += kThreads) {
            const int r = idx / W, w = idx % W;
            const int p = sp.len - 3 + r;
            int cch;
            const TI *xs;
            size_t col, stride;
            if (w < DK) {
                cch = h * DK + w; xs = static_cast<const TI *>(a.q); col = (size_t)h * DK + w; stride = (size_t)H * DK;
            } else if (w < 2 * DK) {
                cch = H * DK + h * DK + (w - DK); xs = static_cast<const TI *>(a.k);
                col = (size_t)h * DK + (w - DK); stride = (size_t)H * DK;
            } else {
                cch = 2 * H * DK + h * DV + (w - 2 * DK); xs = static_cast<const TI *>(a.v);
                col = (size_t)h * DV + (w - 2 * DK); stride = (size_t)H * DV;
            }
            TI val;
            if (p >= 0) val = xs[(size_t)(sp.start + p) * stride + col];
            else if (win) val = win[(size_t)(3 + p) * CC + cch];
            else val = from_f32<TI>(0.f);
            wo[(size_t)r * CC + cch] = val;
        }
    }
}

template <int D, typename TI, typename TO>
hipError_t launch_typed(const PrefillArgs &a, hipStream_t stream) {
    if (a.n_seq == 0) return hipSuccess;
    const WsLayout wl = ws_layout(a.n_tokens, a.n_seq, a.H);
    int32_t *chunk_start = static_cast<int32_t *>(a.ws);
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kThreads), 0, stream, a.cu, a.n_seq, a.n_tokens,
                       (long long)wl.max_chunks, chunk_start);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (wl.max_chunks > 0) {
        hipLaunchKernelGGL((prep_kernel<D, D, TI>), dim3((unsigned)wl.max_chunks, a.H), dim3(kThreads),
                           0, stream, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const unsigned blocks = (unsigned)((size_t)a.n_seq * a.H * (D / TV));
    hipLaunchKernelGGL((scan_kernel<D, D, TI, TO>), dim3(blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

size_t prefill_workspace_bytes(int n_tokens, int n_seq, int H, int dk, int dv, int chunk) {
    (void)dk;
    (void)dv;
    (void)chunk;
    return ws_layout(n_tokens, n_seq, H).total;
}

hipError_t launch_prefill(int dk, int dv, int io, int out, const PrefillArgs &a,
                          hipStream_t stream) {
    (void)dv;
    auto go = [&](auto dtag) -> hipError_t {
        constexpr int D = decltype(dtag)::value;
        if (io == kBF16) {
            if (out == kBF16) return launch_typed<D, bf16, bf16>(a, stream);
            return launch_typed<D, bf16, float>(a, stream);
        }
        if (out == kBF16) return launch_typed<D, float, bf16>(a, stream);
        return launch_typed<D, float, float>(a, stream);
    };
    switch (dk) {
        case 32: return go(std::integral_constant<int, 32>{});
        case 64: return go(std::integral_constant<int, 64>{});
        default: return go(std::integral_constant<int, 128>{});
    }
}

}  // namespace gdn
