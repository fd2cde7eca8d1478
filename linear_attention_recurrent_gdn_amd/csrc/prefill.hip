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
//   T' = (I + A)^-1 diag(beta)
//   P[r][s] = exp(g_r - g_s) <q_r, k_s>                    (s <= r)
//   U = T' (V - diag(gamma) K Sig0)       the chunk's rank-1 factors u_r
//   O = diag(gamma) Q Sig0 + P U          o_r = S_r q_r
//   Sig_L = gamma_L Sig0 + sum_r exp(g_L - g_r) k_r u_r^T
// Column j of U, O, Sig depends only on column j of V and Sig0, so value
// tiles are independent.
//
// Every contraction runs on the gfx950 matrix cores (v_mfma_f32_16x16x32_bf16)
// with split-bf16 operands: x = hi + lo with hi = bf16(x), lo = bf16(x - hi),
// and a.b ~ hi.hi + hi.lo + lo.hi accumulated in fp32 -- about 2^-16
// relative per product, where a single bf16 product (2^-9) would not meet a
// 2e-3 end-to-end tolerance.
//
// Kernels:
//   plan  -- one workgroup: per-sequence chunk offsets (prefix sum of
//            ceil(len/C)) into the workspace, from the device offsets.
//   prep  -- one workgroup per (chunk, head), all chunks in parallel: conv
//            + q/k norm of the chunk rows, KK^T and QK^T on MFMA, then
//            T = (I + A)^-1 by per-column forward substitution; writes T'
//            and P to the workspace.
//   scan  -- one workgroup per (sequence, head, 32-wide value tile): walks
//            the sequence's chunks in order. Each of its 4 waves owns 16
//            chunk rows: it forms the conv'd, normalised K and Q rows
//            directly in MFMA operand registers, and the state tile Sig^T
//            [32][d_k] stays in LDS across chunks.

#include <type_traits>

#include "gdn_device.hpp"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int C = 64;        // chunk length
constexpr int TV = 32;       // value-tile width of the scan
constexpr int RB = 16;       // chunk rows per wave
constexpr float kNormEps = 1e-6f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------ split-bf16 MFMA
struct Split8 {
    bf16x8 hi, lo;
};

__device__ __forceinline__ Split8 split8(const float (&x)[8]) {
    Split8 s;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const __bf16 h = (__bf16)x[e];
        s.hi[e] = h;
        s.lo[e] = (__bf16)(x[e] - (float)h);
    }
    return s;
}

// c += a . b for 16x16 tiles with K = 32, fp32-faithful via three products
__device__ __forceinline__ f32x4v mma3(const Split8 &a, const Split8 &b, f32x4v c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, c, 0, 0, 0);
    return c;
}

__device__ __forceinline__ void lds_read8(const float *p, float (&x)[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// 8 consecutive io-dtype values as fp32 (16-byte aligned)
__device__ __forceinline__ void load8(const float *p, float (&x)[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void load8(const bf16 *p, float (&x)[8]) {
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

// ------------------------------------------------------------ workspace
struct WsLayout {
    size_t rec_off;     // per (chunk, head) record: T' [C][C], P [C][C] (row-major)
    size_t rec_floats;
    size_t max_chunks;
    size_t total;
};

__host__ __device__ WsLayout ws_layout(int n_tokens, int n_seq, int H) {
    WsLayout w{};
    w.max_chunks = (size_t)n_tokens / C + (size_t)n_seq;
    w.rec_off = ((sizeof(int32_t) * ((size_t)n_seq + 1)) + 255) & ~size_t(255);
    w.rec_floats = 2 * (size_t)C * C;
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

__device__ __forceinline__ int find_seq(const int32_t *chunk_start, int n_seq, int gc) {
    int lo = 0, hi = n_seq;  // last s in [0, n_seq) with chunk_start[s] <= gc
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (chunk_start[mid] <= gc) lo = mid;
        else hi = mid;
    }
    return lo;
}

// ------------------------------------------------------------ chunk inputs
// Where a chunk's tokens live: sequence start in the stream, position of the
// chunk's first token in the sequence, live rows, incoming window.
template <typename TI>
struct ChunkSrc {
    int seq0, p0, L;
    const TI *win;  // [3][CC] or null (zeros)
};

// Running sum of log a over the chunk rows, one row per lane (rows >= L add
// nothing): lane l returns g_l. A wave-wide inclusive scan, shared by the
// prep and scan kernels so both see identical g.
__device__ __forceinline__ float chunk_g(const float *log_alpha, int H, int h, int seq0, int p0,
                                         int L) {
    const int lane = threadIdx.x % kWave;
    float g = lane < L ? log_alpha[(size_t)(seq0 + p0 + lane) * H + h] : 0.f;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const float o = __shfl_up(g, off, kWave);
        if (lane >= off) g += o;
    }
    return g;
}

// Conv'd (and, for q / k, normalised) rows rb*16 .. rb*16+15 of the chunk in
// the A-operand layout of a 16x16x32 MFMA: lane l holds row rb*16 + l%16,
// columns ks*32 + (l/16)*8 + e for ks < D/32, e < 8. Rows >= L are zero.
// x is the [N][H][D] stream of this part; cbase its first channel in the
// [q | k | v] concatenation of CC channels.
template <int D, typename TI>
__device__ void rows_afrag(const TI *x, int H, int h, const ChunkSrc<TI> &cs, int rb, int CC,
                           int cbase, const float *w, bool norm, float (&out)[D / 32][8]) {
    const int lane = threadIdx.x % kWave;
    const int row = rb * RB + lane % 16;
    const int cq = (lane / 16) * 8;
    const bool live = row < cs.L;
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
        const int d0 = ks * 32 + cq;
        float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (live) {
            if (w) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int p = cs.p0 + row - 3 + r;
                    float xv[8];
                    if (p >= 0) {
                        load8(x + (size_t)(cs.seq0 + p) * H * D + (size_t)h * D + d0, xv);
                    } else if (cs.win) {
                        load8(cs.win + (size_t)(3 + p) * CC + cbase + h * D + d0, xv);
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) xv[e] = 0.f;
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        y[e] = fmaf(w[(size_t)(cbase + h * D + d0 + e) * 4 + r], xv[e], y[e]);
                }
            } else {
                load8(x + (size_t)(cs.seq0 + cs.p0 + row) * H * D + (size_t)h * D + d0, y);
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            out[ks][e] = y[e];
            ss = fmaf(y[e], y[e], ss);
        }
    }
    if (norm) {
        ss += __shfl_xor(ss, 16, kWave);
        ss += __shfl_xor(ss, 32, kWave);
        const float inv = 1.0f / sqrtf(ss + kNormEps);
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) out[ks][e] *= inv;
    }
}

// Conv'd value entries of one 16-row block in the C/D layout of a 16x16 MFMA:
// lane l holds rows rb*16 + (l/16)*4 + i (i < 4) of columns j0 + t*16 + l%16
// for the value tiles t < TV/16.
template <int DV, typename TI>
__device__ void rows_dfrag_v(const TI *v, int H, int h, const ChunkSrc<TI> &cs, int rb, int j0,
                             int CC, int cbase, const float *w, float (&out)[TV / 16][4]) {
    const int lane = threadIdx.x % kWave;
#pragma unroll
    for (int t = 0; t < TV / 16; ++t) {
        const int j = j0 + t * 16 + lane % 16;
        const int c = cbase + h * DV + j;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = rb * RB + (lane / 16) * 4 + i;
            float y = 0.f;
            if (row < cs.L) {
                if (w) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int p = cs.p0 + row - 3 + r;
                        float xv = 0.f;
                        if (p >= 0) xv = to_f32(v[(size_t)(cs.seq0 + p) * H * DV + (size_t)h * DV + j]);
                        else if (cs.win) xv = to_f32(cs.win[(size_t)(3 + p) * CC + c]);
                        y = fmaf(w[(size_t)c * 4 + r], xv, y);
                    }
                } else {
                    y = to_f32(v[(size_t)(cs.seq0 + cs.p0 + row) * H * DV + (size_t)h * DV + j]);
                }
            }
            out[t][i] = y;
        }
    }
}

// ------------------------------------------------------------ prep
template <int DK, int DV, typename TI>
__global__ __launch_bounds__(kThreads) void prep_kernel(PrefillArgs a) {
    constexpr int KP = DK + 4;           // padded row of the staged K rows
    // staged K rows [C][KP], then (reused) T' [C][C + 1]
    constexpr int SK = C * KP > C * (C + 1) ? C * KP : C * (C + 1);
    __shared__ __attribute__((aligned(16))) float s_k[SK];
    __shared__ __attribute__((aligned(16))) float s_A[C * (C + 1)];  // strictly lower A

    const int32_t *chunk_start = static_cast<const int32_t *>(a.ws);
    const int gc = blockIdx.x, h = blockIdx.y;
    if (gc >= chunk_start[a.n_seq]) return;
    const int s = find_seq(chunk_start, a.n_seq, gc);
    const SeqSpan sp = seq_span(a.cu, s, a.n_tokens);
    const int c = gc - chunk_start[s];
    const int H = a.H;
    const int CC = H * (2 * DK + DV);
    const int src = a.parent ? a.parent[s] : s;
    const bool src_ok = src >= 0 && src < a.n_parent;
    ChunkSrc<TI> cs{sp.start, c * C, min(C, sp.len - c * C),
                    (a.win_in && src_ok) ? static_cast<const TI *>(a.win_in) + (size_t)src * 3 * CC
                                         : nullptr};
    const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;

    float kf[DK / 32][8], qf[DK / 32][8];
    rows_afrag<DK, TI>(static_cast<const TI *>(a.k), H, h, cs, w, CC, H * DK, a.conv_w,
                       a.qk_norm != 0, kf);
    rows_afrag<DK, TI>(static_cast<const TI *>(a.q), H, h, cs, w, CC, 0, a.conv_w, a.qk_norm != 0,
                       qf);
    const float g = chunk_g(a.log_alpha, H, h, cs.seq0, cs.p0, cs.L);
    const float b_l = lane < cs.L ? a.beta[(size_t)(cs.seq0 + cs.p0 + lane) * H + h] : 0.f;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            s_k[(w * RB + lane % 16) * KP + ks * 32 + (lane / 16) * 8 + e] = kf[ks][e];
    __syncthreads();

    float *rec = reinterpret_cast<float *>(static_cast<char *>(a.ws) +
                                           ws_layout(a.n_tokens, a.n_seq, H).rec_off) +
                 ((size_t)gc * H + h) * (2 * C * C);
    float *Tg = rec;          // T' [C][C] row-major
    float *Pg = rec + C * C;  // P  [C][C] row-major

    // KK^T and QK^T tiles (w, ct), ct <= w, on MFMA; the rest of the rows are zero
    Split8 ka[DK / 32], qa[DK / 32];
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
        ka[ks] = split8(kf[ks]);
        qa[ks] = split8(qf[ks]);
    }
    for (int ct = 0; ct < C / RB; ++ct) {
        f32x4v kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
        if (ct <= w) {
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks) {
                float bx[8];
                lds_read8(s_k + (ct * RB + lane % 16) * KP + ks * 32 + (lane / 16) * 8, bx);
                const Split8 bs = split8(bx);
                kk = mma3(ka[ks], bs, kk);
                qk = mma3(qa[ks], bs, qk);
            }
        }
        // D layout: rows w*16 + (l/16)*4 + i, column ct*16 + l%16
        const int col = ct * RB + lane % 16;
        const float g_c = __shfl(g, col, kWave);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = w * RB + (lane / 16) * 4 + i;
            const float g_r = __shfl(g, row, kWave);
            const float b_r = __shfl(b_l, row, kWave);
            const bool live = row < cs.L && col < cs.L;
            const float dec = (live && col <= row) ? expf(g_r - g_c) : 0.f;
            s_A[row * (C + 1) + col] = col < row ? b_r * dec * kk[i] : 0.f;
            Pg[row * C + col] = dec * qk[i];
        }
    }
    __syncthreads();

    // T = (I + A)^-1, one column per group of 4 lanes (columns are
    // independent): lane (col, part) keeps T[j][col] for j = part (mod 4).
    {
        const int col = w * 16 + lane / 4, part = lane % 4;
        float t[C / 4];
#pragma unroll
        for (int q = 0; q < C / 4; ++q) t[q] = 0.f;
#pragma unroll
        for (int r = 0; r < C; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int q = 0; q < C / 4; ++q) {
                const int j = q * 4 + part;
                if (j < r) acc = fmaf(s_A[r * (C + 1) + j], t[q], acc);
            }
            acc += __shfl_xor(acc, 1, kWave);
            acc += __shfl_xor(acc, 2, kWave);
            const float val = (r == col) ? 1.f : (r > col ? -acc : 0.f);
            if (r % 4 == part) t[r / 4] = val;
        }
        __syncthreads();  // every lane is done with s_A; s_k is free as well
        // T'[j][col] = T[j][col] beta_col, staged through LDS for coalesced stores
        const float bcol = __shfl(b_l, col, kWave);
#pragma unroll
        for (int q = 0; q < C / 4; ++q) s_k[(q * 4 + part) * (C + 1) + col] = t[q] * bcol;
    }
    __syncthreads();
    for (int idx = tid; idx < C * C; idx += kThreads)
        Tg[idx] = s_k[(idx / C) * (C + 1) + idx % C];
}

// ------------------------------------------------------------ scan
template <int DK, int DV, typename TI, typename TO>
__global__ __launch_bounds__(kThreads) void scan_kernel(PrefillArgs a) {
    constexpr int KS = DK / 32;       // k-steps over d_k
    constexpr int SP = DK + 4;        // padded row of Sig^T
    constexpr int CPd = C + 4;        // padded row of K~^T, R^T, U^T
    constexpr int NVT = TV / 16;      // 16-wide value sub-tiles
    constexpr int NFT = NVT * (DK / 16);  // output tiles of the state update
    __shared__ __attribute__((aligned(16))) float s_St[TV * SP];   // Sig^T tile [TV][DK]
    __shared__ __attribute__((aligned(16))) float s_Kt[DK * CPd];  // K~^T [DK][C]
    __shared__ __attribute__((aligned(16))) float s_Rt[TV * CPd];  // R^T  [TV][C]
    __shared__ __attribute__((aligned(16))) float s_Ut[TV * CPd];  // U^T  [TV][C]

    constexpr int NT = DV / TV;
    const int tile = blockIdx.x % NT;
    const int shd = blockIdx.x / NT;
    const int s = shd / a.H, h = shd % a.H;
    const int H = a.H;
    const int CC = H * (2 * DK + DV);
    const int j0 = tile * TV;
    const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
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
        s_St[j * SP + d] =
            a.state_in ? a.state_in[(((size_t)src * H + h) * DK + d) * DV + j0 + j] : 0.f;
    }
    __syncthreads();

    const int nchunks = chunk_start[s + 1] - chunk_start[s];  // <= ceil(len / C)
    for (int c = 0; c < nchunks; ++c) {
        const ChunkSrc<TI> cs{sp.start, c * C, min(C, sp.len - c * C), win};
        const float *rec = reinterpret_cast<const float *>(static_cast<const char *>(a.ws) +
                                                           wl.rec_off) +
                           ((size_t)(chunk_start[s] + c) * H + h) * wl.rec_floats;
        const float *Tg = rec, *Pg = rec + C * C;

        // this wave's 16 rows: K, Q (A operands), V (C/D layout), g
        float kf[KS][8], qf[KS][8], vf[NVT][4];
        rows_afrag<DK, TI>(static_cast<const TI *>(a.k), H, h, cs, w, CC, H * DK, a.conv_w,
                           a.qk_norm != 0, kf);
        rows_afrag<DK, TI>(static_cast<const TI *>(a.q), H, h, cs, w, CC, 0, a.conv_w,
                           a.qk_norm != 0, qf);
        rows_dfrag_v<DV, TI>(static_cast<const TI *>(a.v), H, h, cs, w, j0, CC, 2 * H * DK,
                             a.conv_w, vf);
        const float g = chunk_g(a.log_alpha, H, h, cs.seq0, cs.p0, cs.L);
        const float gL = __shfl(g, C - 1, kWave);

        // K~^T[d][row] = exp(g_L - g_row) k_row[d] for the state update
        {
            const int row = w * RB + lane % 16;
            const float f = expf(gL - __shfl(g, row, kWave));
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    s_Kt[(ks * 32 + (lane / 16) * 8 + e) * CPd + row] = kf[ks][e] * f;
        }
        Split8 ka[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) ka[ks] = split8(kf[ks]);

        // R = V - diag(gamma) K Sig0 : rows w*16.., all value columns
        float gam[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) gam[i] = expf(__shfl(g, w * RB + (lane / 16) * 4 + i, kWave));
#pragma unroll
        for (int t = 0; t < NVT; ++t) {
            f32x4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                float bx[8];
                lds_read8(s_St + (t * 16 + lane % 16) * SP + ks * 32 + (lane / 16) * 8, bx);
                acc = mma3(ka[ks], split8(bx), acc);
            }
            float4 r4;
            r4.x = vf[t][0] - gam[0] * acc[0];
            r4.y = vf[t][1] - gam[1] * acc[1];
            r4.z = vf[t][2] - gam[2] * acc[2];
            r4.w = vf[t][3] - gam[3] * acc[3];
            *reinterpret_cast<float4 *>(s_Rt + (t * 16 + lane % 16) * CPd + w * RB + (lane / 16) * 4) = r4;
        }
        __syncthreads();

        // U = T' R (T' lower triangular: k-steps up to this wave's rows)
        const int kmax = (w * RB + RB - 1) / 32;
        Split8 ta[2];
#pragma unroll
        for (int kq = 0; kq < 2; ++kq) {
            if (kq <= kmax) {
                float tx[8];
                load8(Tg + (w * RB + lane % 16) * C + kq * 32 + (lane / 16) * 8, tx);
                ta[kq] = split8(tx);
            }
        }
#pragma unroll
        for (int t = 0; t < NVT; ++t) {
            f32x4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kq = 0; kq < 2; ++kq) {
                if (kq <= kmax) {
                    float bx[8];
                    lds_read8(s_Rt + (t * 16 + lane % 16) * CPd + kq * 32 + (lane / 16) * 8, bx);
                    acc = mma3(ta[kq], split8(bx), acc);
                }
            }
            *reinterpret_cast<float4 *>(s_Ut + (t * 16 + lane % 16) * CPd + w * RB + (lane / 16) * 4) =
                make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
        __syncthreads();

        // O = diag(gamma) Q Sig0 + P U
        if (a.o) {
            Split8 qa[KS], pa[2];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qa[ks] = split8(qf[ks]);
#pragma unroll
            for (int kq = 0; kq < 2; ++kq) {
                if (kq <= kmax) {
                    float px[8];
                    load8(Pg + (w * RB + lane % 16) * C + kq * 32 + (lane / 16) * 8, px);
                    pa[kq] = split8(px);
                }
            }
#pragma unroll
            for (int t = 0; t < NVT; ++t) {
                f32x4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    float bx[8];
                    lds_read8(s_St + (t * 16 + lane % 16) * SP + ks * 32 + (lane / 16) * 8, bx);
                    acc = mma3(qa[ks], split8(bx), acc);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] *= gam[i];
#pragma unroll
                for (int kq = 0; kq < 2; ++kq) {
                    if (kq <= kmax) {
                        float bx[8];
                        lds_read8(s_Ut + (t * 16 + lane % 16) * CPd + kq * 32 + (lane / 16) * 8, bx);
                        acc = mma3(pa[kq], split8(bx), acc);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = w * RB + (lane / 16) * 4 + i;
                    if (row < cs.L)
                        static_cast<TO *>(a.o)[((size_t)(cs.seq0 + cs.p0 + row) * H + h) * DV + j0 +
                                               t * 16 + lane % 16] = from_f32<TO>(acc[i]);
                }
            }
        }
        __syncthreads();  // Sig^T fully read before it is rewritten

        // Sig^T <- gamma_L Sig^T + U^T K~   (tiles: value sub-tile x 16 keys)
        const float gamL = expf(gL);
        for (int ft = w; ft < NFT; ft += kWaves) {
            const int t = ft % NVT, dt = ft / NVT;
            f32x4v acc;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i] = gamL * s_St[(t * 16 + (lane / 16) * 4 + i) * SP + dt * 16 + lane % 16];
#pragma unroll
            for (int kq = 0; kq < 2; ++kq) {
                float ax[8], bx[8];
                lds_read8(s_Ut + (t * 16 + lane % 16) * CPd + kq * 32 + (lane / 16) * 8, ax);
                lds_read8(s_Kt + (dt * 16 + lane % 16) * CPd + kq * 32 + (lane / 16) * 8, bx);
                acc = mma3(split8(ax), split8(bx), acc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                s_St[(t * 16 + (lane / 16) * 4 + i) * SP + dt * 16 + lane % 16] = acc[i];
        }
        __syncthreads();
    }

    if (a.state_out)
        for (int idx = tid; idx < DK * TV; idx += kThreads) {
            const int d = idx / TV, j = idx % TV;
            a.state_out[(((size_t)s * H + h) * DK + d) * DV + j0 + j] = s_St[j * SP + d];
        }
    // window out (tile 0): the last 3 raw inputs of the head's channels
    if (a.win_out && tile == 0) {
        TI *wo = static_cast<TI *>(a.win_out) + (size_t)s * 3 * CC;
        const int W = 2 * DK + DV;
        for (int idx = tid; idx < 3 * W; idx += kThreads) {
            const int r = idx / W, wc = idx % W;
            const int p = sp.len - 3 + r;
            int cch;
            const TI *xs;
            size_t col, stride;
            if (wc < DK) {
                cch = h * DK + wc; xs = static_cast<const TI *>(a.q);
                col = (size_t)h * DK + wc; stride = (size_t)H * DK;
            } else if (wc < 2 * DK) {
                cch = H * DK + h * DK + (wc - DK); xs = static_cast<const TI *>(a.k);
                col = (size_t)h * DK + (wc - DK); stride = (size_t)H * DK;
            } else {
                cch = 2 * H * DK + h * DV + (wc - 2 * DK); xs = static_cast<const TI *>(a.v);
                col = (size_t)h * DV + (wc - 2 * DK); stride = (size_t)H * DV;
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
        hipLaunchKernelGGL((prep_kernel<D, D, TI>), dim3((unsigned)wl.max_chunks, a.H),
                           dim3(kThreads), 0, stream, a);
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
