// prefill_kernels.hpp -- chunked prefill of the GDN recurrence over a flat token
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
// Every contraction runs on the gfx950 matrix cores. With bf16 I/O the
// operands are split bf16 (v_mfma_f32_16x16x32_bf16): x = hi + lo with
// hi = bf16(x), lo = bf16(x - hi), and a.b ~ hi.hi + hi.lo + lo.hi
// accumulated in fp32 -- about 2^-16 relative per product, where a single
// bf16 product (2^-9) would not meet a 2e-3 end-to-end tolerance. With fp32
// I/O they are the fp32 values (v_mfma_f32_16x16x4f32, eight per 16x16x32
// step), in the same 4 bytes per element (see Frag).
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

#pragma once

#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "gdn_device.hpp"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr long long kScanResident = 2 * 256;  // scan workgroups resident at once (2 per CU)
constexpr int C = 64;        // chunk length
constexpr int TV = 32;       // value-tile width of the scan
constexpr int RB = 16;       // chunk rows per wave
constexpr float kNormEps = 1e-6f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------ MFMA operands
// A lane's piece of a 16x16x32 MFMA operand: 8 values (A layout: row l % 16,
// k = 8 (l / 16) + e; B layout the same with column for row). Two forms,
// both 32 bytes, kept in two "planes" (hi, lo) of 16 bytes per 8 elements:
//  - F = false (bf16 I/O): x = hi + lo split into bf16 (round to nearest
//    even, then the residual rounded); products take three bf16 MFMAs
//    (hi hi + hi lo + lo hi), about 16 bits of each operand;
//  - F = true (fp32 I/O): the fp32 values themselves, elements 0..3 in the
//    hi plane's 16 bytes and 4..7 in the lo plane's; products take eight
//    fp32 MFMAs (16x16x4, k split by e: the e-th takes k = 8 g + e of the
//    four lane groups g), exact fp32 products.
template <bool F> struct Frag;
template <> struct Frag<false> {
    bf16x8 hi, lo;
};
template <> struct Frag<true> {
    f32x4v hi, lo;
};

// Two values rounded to bf16 (nearest even) as one 32-bit word, a in the
// low half (the element order of a bf16 vector in memory).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
// hi / lo split of two values as bf16 pair words: hi = bf16(x), lo =
// bf16(x - hi), with hi widened back from the packed word itself (the
// compiler's own widening converts each value again).
__device__ __forceinline__ void split_pair(float a, float b, uint32_t &hi, uint32_t &lo) {
    hi = bf16_pair(a, b);
    lo = bf16_pair(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

template <bool F>
__device__ __forceinline__ Frag<F> frag(const float (&x)[8]) {
    Frag<F> s;
    if constexpr (F) {
        s.hi = f32x4v{x[0], x[1], x[2], x[3]};
        s.lo = f32x4v{x[4], x[5], x[6], x[7]};
    } else {
        uint4 h, l;
        split_pair(x[0], x[1], h.x, l.x);
        split_pair(x[2], x[3], h.y, l.y);
        split_pair(x[4], x[5], h.z, l.z);
        split_pair(x[6], x[7], h.w, l.w);
        s.hi = __builtin_bit_cast(bf16x8, h);
        s.lo = __builtin_bit_cast(bf16x8, l);
    }
    return s;
}

// c += a . b for 16x16 tiles with K = 32
__device__ __forceinline__ f32x4v mma(const Frag<false> &a, const Frag<false> &b, f32x4v c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, c, 0, 0, 0);
    return c;
}
__device__ __forceinline__ f32x4v mma(const Frag<true> &a, const Frag<true> &b, f32x4v c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[e], b.hi[e], c, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[e], b.lo[e], c, 0, 0, 0);
    return c;
}

// The 8 elements at element offset o (a multiple of 8) of a plane pair
// (16-byte aligned): read, written.
template <bool F>
__device__ __forceinline__ Frag<F> read_frag(const __bf16 *hi, const __bf16 *lo) {
    Frag<F> s;
    s.hi = *reinterpret_cast<const decltype(s.hi) *>(hi);
    s.lo = *reinterpret_cast<const decltype(s.lo) *>(lo);
    return s;
}
template <bool F>
__device__ __forceinline__ void store_frag(__bf16 *hi, __bf16 *lo, const Frag<F> &s) {
    *reinterpret_cast<decltype(s.hi) *>(hi) = s.hi;
    *reinterpret_cast<decltype(s.lo) *>(lo) = s.lo;
}

// base + an unsigned 32-bit byte offset: with base wave-uniform, global
// accesses through it take the scalar-base form (no 64-bit lane math).
template <class T>
__device__ __forceinline__ T *byte_at(T *base, unsigned bytes) {
    return reinterpret_cast<T *>(reinterpret_cast<char *>(base) + bytes);
}
template <class T>
__device__ __forceinline__ const T *byte_at(const T *base, unsigned bytes) {
    return reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + bytes);
}

// One element at element offset o of a plane pair.
template <bool F>
__device__ __forceinline__ void put1(__bf16 *hi, __bf16 *lo, int o, float x) {
    if constexpr (F) {
        float *const p = reinterpret_cast<float *>(((o & 7) < 4 ? hi : lo) + (o & ~7));
        p[o & 3] = x;
    } else {
        const __bf16 h = (__bf16)x;
        hi[o] = h;
        lo[o] = (__bf16)(x - (float)h);
    }
}

// 4 consecutive elements at element offset o (a multiple of 4) of a plane
// pair: one 8-byte store per plane (bf16), one 16-byte store (fp32).
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
template <bool F>
__device__ __forceinline__ void put4(__bf16 *hi, __bf16 *lo, int o, f32x4v x) {
    if constexpr (F) {
        *reinterpret_cast<f32x4v *>(((o & 7) < 4 ? hi : lo) + (o & ~7)) = x;
    } else {
        uint2 h, l;
        split_pair(x[0], x[1], h.x, l.x);
        split_pair(x[2], x[3], h.y, l.y);
        *reinterpret_cast<uint2 *>(hi + o) = h;
        *reinterpret_cast<uint2 *>(lo + o) = l;
    }
}

// 16x16x16 products (the blocked triangular inverse): a lane's piece is 4
// values, k = 4 (l / 16) + e; split bf16 (three 16x16x16 bf16 MFMAs) or
// fp32 (four 16x16x4 fp32 MFMAs, k split by e as in Frag).
template <bool F> struct Frag4;
template <> struct Frag4<false> {
    bf16x4 hi, lo;
};
template <> struct Frag4<true> {
    f32x4v v;
};
template <bool F>
__device__ __forceinline__ Frag4<F> frag4(f32x4v x) {
    Frag4<F> s;
    if constexpr (F) {
        s.v = x;
    } else {
        uint2 h, l;
        split_pair(x[0], x[1], h.x, l.x);
        split_pair(x[2], x[3], h.y, l.y);
        s.hi = __builtin_bit_cast(bf16x4, h);
        s.lo = __builtin_bit_cast(bf16x4, l);
    }
    return s;
}
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4v mma16(const Frag4<false> &a, const Frag4<false> &b, f32x4v c) {
    const s16x4 ah = __builtin_bit_cast(s16x4, a.hi), al = __builtin_bit_cast(s16x4, a.lo);
    const s16x4 bh = __builtin_bit_cast(s16x4, b.hi), bl = __builtin_bit_cast(s16x4, b.lo);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bh, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bl, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, c, 0, 0, 0);
    return c;
}
__device__ __forceinline__ f32x4v mma16(const Frag4<true> &a, const Frag4<true> &b, f32x4v c) {
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
    return c;
}

__device__ __forceinline__ void lds_read8(const float *p, float (&x)[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// 8 consecutive fp32 values (16-byte aligned)
__device__ __forceinline__ void load8(const float *p, float (&x)[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// ------------------------------------------------------------ workspace
// Per (chunk, head) record written by the prep kernel for the scan, as
// hi / lo plane pairs of MFMA operands (split bf16, or fp32, see Frag):
//   T', P  [C][C] lower triangular, only their 16 x 32 blocks at or below
//          the diagonal, in the order the 16x16x32 MFMA reads an A operand
//          (tri_off)
//   fp32 slot of 4C floats: scalar decay -- per row r the factors the scan
//          applies to its MFMA rows, gamma_r (for K Sig0 and Q Sig0) and
//          e^{g_L - g_r} (for the state update), then gamma_L; per-key decay
//          -- e^{g_L} per key column
//   K, Q   [C][d_k] the conv'd, normalised chunk rows (per-key decay: the
//          decayed K^ = K . e^{g}, Q^ = Q . e^{g}), A operands in fragment
//          order (frag_off)
//   per-key decay only: K~^T [d_k][C] = (k_r . e^{g_L - g_r})^T (B operand
//          rows); with a scalar decay the scan forms K^T itself from K
// 89 KiB per chunk-head with a scalar decay at d_k = 128 (1.4 KiB per
// token-head), 105 KiB per key.
//
// Fragment order: the 16-row x 32-column block (w, ks) of a plane is 1 KiB
// contiguous, lane l's 8 values (row w*16 + l%16, columns ks*32 + (l/16)*8
// ..) at element frag_off(nks, w, ks, l), nks = columns / 32. A wave's
// operand load then covers 8 whole 128-byte lines instead of 16 half lines.
__host__ __device__ constexpr int frag_off(int nks, int w, int ks, int lane) {
    return ((w * nks + ks) * kWave + lane) * 8;
}

// Lower-triangular C x C planes keep the blocks (w, kq) with
// kq <= (16 w + 15) / 32: (0,0) (1,0) (2,0) (2,1) (3,0) (3,1).
constexpr int kTriBlocks = 6;
__host__ __device__ constexpr int tri_block(int w, int kq) { return w < 2 ? w : 2 * w - 2 + kq; }
__host__ __device__ constexpr int tri_off(int w, int kq, int lane) {
    return (tri_block(w, kq) * kWave + lane) * 8;
}
constexpr int kTriElems = kTriBlocks * kWave * 8;  // bf16 per plane
constexpr int kFacFloats = 4 * C;                 // the fp32 slot
static_assert(kFacFloats >= 128, "the slot holds e^{g_L} of every key");

struct RecLayout {
    size_t thi, tlo, phi, plo, fac, khi, klo, qhi, qlo, kthi, ktlo, elems;
};

__host__ __device__ constexpr RecLayout rec_layout(int dk, bool per_key) {
    const size_t t = kTriElems, k0 = 4 * t + 2 * (size_t)kFacFloats, cd = (size_t)C * dk;
    return RecLayout{0,      t,           2 * t,       3 * t,       4 * t,
                     k0,     k0 + cd,     k0 + 2 * cd, k0 + 3 * cd, k0 + 4 * cd,
                     k0 + 5 * cd, k0 + (per_key ? 6 : 4) * cd};
}

// Workspace: int32 header (chunk_start [n_seq + 1], the branch group table
// [n_seq + 3], each sequence's first chunk in the current segment [n_seq]),
// then, when the prefill runs in segments, the fp32 state carried from one
// segment to the next [n_seq][H][dk][dv], then the records of one segment.
// A prefill of nseg segments gives segment k of every sequence the chunks
// [k n / nseg, (k + 1) n / nseg) of its n chunks, so one segment needs at
// most all_chunks / nseg + n_seq records.
struct WsLayout {
    size_t grp_off;     // int32 index of the branch group table
    size_t win_off;     // int32 index of the per-sequence segment start chunks
    size_t carry_off;   // byte offset of the carried state (nseg > 1)
    size_t rec_off;     // byte offset of the records
    size_t rec_elems;   // bf16 elements per record
    size_t max_chunks;  // records of one segment
    size_t total;
};

__host__ __device__ WsLayout ws_layout(int n_tokens, int n_seq, int H, int dk, int dv, bool per_key,
                                       int nseg) {
    WsLayout w{};
    const size_t all = (size_t)n_tokens / C + (size_t)n_seq;
    w.max_chunks = nseg <= 1 ? all : (all + nseg - 1) / nseg + (size_t)n_seq;
    w.grp_off = (size_t)n_seq + 1;
    w.win_off = 2 * (size_t)n_seq + 4;
    w.carry_off = ((sizeof(int32_t) * (3 * (size_t)n_seq + 4)) + 255) & ~size_t(255);
    const size_t carry = nseg > 1 ? sizeof(float) * (size_t)n_seq * H * dk * dv : 0;
    w.rec_off = (w.carry_off + carry + 255) & ~size_t(255);
    w.rec_elems = rec_layout(dk, per_key).elems;
    w.total = w.rec_off + sizeof(__bf16) * w.rec_elems * w.max_chunks * (size_t)H;
    return w;
}

// Segments of a prefill: enough that one segment's records stay within
// kSegmentRecordBytes (512 MiB: the fork_prefill prefix, 1.5 GB of records
// in one segment, runs in 3 and needs 0.49 KiB of workspace per token-head),
// at most one per chunk of an average sequence and at most kMaxSegments.
// Each segment past the first costs about 25-45 us (launches, the scan's
// restart and the carried state). The environment variable
// GDN_PREFILL_SEGMENT_RECORD_BYTES overrides the bound (a smaller value
// forces segments on small inputs, for tests; a large one a single
// segment); the workspace size and the launcher read it alike.
constexpr size_t kSegmentRecordBytes = size_t(512) << 20;
constexpr int kMaxSegments = 64;
inline int prefill_segments(int n_tokens, int n_seq, int H, int dk, bool per_key) {
    size_t bound = kSegmentRecordBytes;
    if (const char *env = std::getenv("GDN_PREFILL_SEGMENT_RECORD_BYTES")) {
        const long long v = std::atoll(env);
        if (v > 0) bound = (size_t)v;
    }
    const size_t all = (size_t)n_tokens / C + (size_t)n_seq;
    const size_t rec = sizeof(__bf16) * rec_layout(dk, per_key).elems * (size_t)H;
    const long long want = (long long)((all * rec + bound - 1) / bound);
    const long long avg = n_seq > 0 ? (long long)n_tokens / ((long long)C * n_seq) : 1;
    return (int)std::max(1LL, std::min({want, avg, (long long)kMaxSegments}));
}

struct SeqSpan {
    int start, len;
};

__device__ __forceinline__ SeqSpan seq_span(const int32_t *cu, int s, int n_tokens) {
    const int a = min(max(cu[s], 0), n_tokens);
    const int b = min(max(cu[s + 1], a), n_tokens);
    return {a, b - a};
}

// Exclusive scan of x over the workgroup's threads in thread order under op
// (associative, with identity id); the value over all threads goes to
// *total when asked. Wave-wide shuffles, then the waves' totals through LDS.
// Every thread of the workgroup calls it.
template <typename T>
__device__ __forceinline__ T shfl_up_any(T x, int off) {
    if constexpr (sizeof(T) == 8) {
        const long long v = (long long)x;
        const int lo = __shfl_up((int)(v & 0xffffffffLL), off, kWave);
        const int hi = __shfl_up((int)(v >> 32), off, kWave);
        return (T)(((long long)hi << 32) | (unsigned)lo);
    } else {
        return __shfl_up(x, off, kWave);
    }
}
template <typename T, typename Op>
__device__ __forceinline__ T block_exclusive_scan(T x, T id, Op op, T *total = nullptr) {
    __shared__ T s_w[kWaves];
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    T inc = x;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const T o = shfl_up_any(inc, off);
        if (lane >= off) inc = op(o, inc);
    }
    const T prev = shfl_up_any(inc, 1);
    if (lane == kWave - 1) s_w[w] = inc;
    __syncthreads();
    T before = id, all = id;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        if (i < w) before = op(before, s_w[i]);
        all = op(all, s_w[i]);
    }
    __syncthreads();  // s_w is free for the next call
    if (total) *total = all;
    return op(before, lane == 0 ? id : prev);
}

// Branch groups for the scan: the maximal runs of consecutive branches with
// one parent, cut into pieces of at most G branches (a workgroup of the scan
// then runs a group's branches from one load of the parent state).
// groups[0] = the count, groups[1 + g] = the first branch of group g,
// groups[1 + count] = n_seq. One workgroup: per-thread slices of the
// branches, with the run start carried across slices by a max-scan (run
// starts grow with the branch index) and the group counts by a sum-scan.
__device__ __forceinline__ void plan_groups(const int32_t *parent, int n_seq, int G,
                                            int32_t *groups) {
    const int tid = threadIdx.x;
    const int per = (n_seq + kThreads - 1) / kThreads;
    const int lo = min(tid * per, n_seq), hi = min(lo + per, n_seq);
    const auto starts_run = [&](int b) { return b == 0 || parent[b] != parent[b - 1]; };
    int last = -1;
    for (int b = lo; b < hi; ++b)
        if (starts_run(b)) last = b;
    // the run start in effect where each slice begins
    const int rs0 = block_exclusive_scan(last, 0, [](int x, int y) { return max(x, y); });
    int rs = rs0, cnt = 0;
    for (int b = lo; b < hi; ++b) {
        if (starts_run(b)) rs = b;
        cnt += (b - rs) % G == 0;
    }
    int count = 0;
    int gi = block_exclusive_scan(cnt, 0, [](int x, int y) { return x + y; }, &count);
    if (tid == 0) {
        groups[0] = count;
        groups[1 + count] = n_seq;
    }
    rs = rs0;
    for (int b = lo; b < hi; ++b) {
        if (starts_run(b)) rs = b;
        if ((b - rs) % G == 0) groups[1 + gi++] = b;
    }
}

// ------------------------------------------------------------ plan
// Segment seg of nseg: sequence s of n = ceil(len / C) chunks takes its
// chunks [n seg / nseg, n (seg + 1) / nseg) (win0[s] = the first);
// chunk_start[s] = min(sum of the earlier sequences' counts, max_chunks) is
// its first record, and it owns chunk_start[s+1] - chunk_start[s]. With
// valid offsets the cap never binds; with overlapping (invalid) offsets it
// keeps every record inside the workspace. One workgroup; plan_kernel
// launches it alone, and the one-chunk kernel runs it for the first segment
// in an extra workgroup of its own grid.
__device__ __forceinline__ void plan_body(const int32_t *cu, int n_seq, int n_tokens,
                                          long long max_chunks, int32_t *chunk_start,
                                          const int32_t *parent, int G, int32_t *groups, int seg,
                                          int nseg, int32_t *win0, int fuse1) {
    const int tid = threadIdx.x;
    const int per = (n_seq + kThreads - 1) / kThreads;
    const int lo = min(tid * per, n_seq), hi = min(lo + per, n_seq);
    // sequence s's chunks in this segment: [first, first + count)
    // (none for a sequence the one-chunk kernel takes)
    const auto window = [&](int s, long long &first) {
        const int len = seq_span(cu, s, n_tokens).len;
        const long long n = (fuse1 && len <= C) ? 0 : (len + C - 1) / C;
        first = n * seg / nseg;
        return n * (seg + 1) / nseg - first;
    };
    long long sum = 0, first;
    for (int s = lo; s < hi; ++s) sum += window(s, first);
    long long run = block_exclusive_scan(sum, 0LL, [](long long x, long long y) { return x + y; });
    for (int s = lo; s < hi; ++s) {
        chunk_start[s] = (int32_t)min(run, max_chunks);
        run += window(s, first);
        win0[s] = (int32_t)first;
    }
    if (tid == kThreads - 1) chunk_start[n_seq] = (int32_t)min(run, max_chunks);
    if (groups) plan_groups(parent, n_seq, G, groups);  // branch calls
}

__global__ __launch_bounds__(kThreads) void plan_kernel(const int32_t *cu, int n_seq, int n_tokens,
                                                        long long max_chunks,
                                                        int32_t *chunk_start,
                                                        const int32_t *parent, int G,
                                                        int32_t *groups, int seg, int nseg,
                                                        int32_t *win0, int fuse1) {
    plan_body(cu, n_seq, n_tokens, max_chunks, chunk_start, parent, G, groups, seg, nseg, win0,
              fuse1);
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
    const int r = min(lane, L - 1);  // clamped: the load is unconditional
    float g = log_alpha[(size_t)(seq0 + p0 + r) * H + h];
    g = lane < L ? g : 0.f;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const float o = __shfl_up(g, off, kWave);
        if (lane >= off) g += o;
    }
    return g;
}

// Raw io-dtype words of 8 consecutive values: 4 words for bf16, 8 for fp32.
template <typename TI>
struct Raw8 {
    static constexpr int W = 8 * (int)sizeof(TI) / 4;
    uint32_t w[W];
};

template <typename TI>
__device__ __forceinline__ void raw_load(const TI *p, Raw8<TI> &r) {
#pragma unroll
    for (int i = 0; i < Raw8<TI>::W / 4; ++i) {
        const uint4 u = reinterpret_cast<const uint4 *>(p)[i];
        r.w[4 * i] = u.x;
        r.w[4 * i + 1] = u.y;
        r.w[4 * i + 2] = u.z;
        r.w[4 * i + 3] = u.w;
    }
}

__device__ __forceinline__ void raw_unpack(const Raw8<float> &r, float (&x)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = __uint_as_float(r.w[e]);
}
__device__ __forceinline__ void raw_unpack(const Raw8<bf16> &r, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(r.w[i] << 16);
        x[2 * i + 1] = __uint_as_float(r.w[i] & 0xffff0000u);
    }
}

// lane i <- lane (i - N) mod 16 of its 16-lane DPP row (row_ror:N)
template <int N>
__device__ __forceinline__ uint32_t ror16(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x120 + N, 0xf, 0xf, false);
}

// Conv'd (and, for q / k, normalised) rows rb*16 .. rb*16+15 of the chunk in
// the A-operand layout of a 16x16x32 MFMA: lane l holds row rb*16 + l%16,
// columns ks*32 + (l/16)*8 + e for ks < D/32, e < 8. Rows >= L are zero.
// x is the [N][H][D] stream of this part, cwin the part's first channel of
// head h in the [q | k | v] window rows, s_w the part's taps [D][4] in LDS
// (null: no convolution). Each lane loads only its own raw row; lanes 13-15
// also load the 3 rows before the block (from the stream or the incoming
// window). The three earlier taps of a row then come from the lanes 1-3 rows
// up through DPP row rotations, which match the 16-row layout exactly.
template <int D, typename TI>
struct RawRows {
    Raw8<TI> own[D / 32], halo[D / 32];
};

// rows_load issues the loads (two parts' loads can then be in flight
// together): every load is unconditional from a clamped, in-bounds address
// (validity is applied in rows_compute) and nothing is consumed here.
template <int D, typename TI>
__device__ __forceinline__ void rows_load(const TI *x, int H, int h, const ChunkSrc<TI> &cs,
                                          int rb, int CC, int cwin, bool conv,
                                          RawRows<D, TI> &rr, int ks0 = 0, int ks1 = D / 32) {
    constexpr int KS = D / 32;
    const int lane = threadIdx.x % kWave;
    const int i = lane % 16;
    const int cq = (lane / 16) * 8;
    const int row = rb * RB + i;
    const TI *own_p = x + (size_t)(cs.seq0 + cs.p0 + min(row, cs.L - 1)) * H * D + (size_t)h * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        if (ks >= ks0 && ks < ks1) raw_load(own_p + ks * 32 + cq, rr.own[ks]);
    if (conv) {
        // halo rows (lanes 13..15): stream position ph, or window row 3 + ph.
        // A block with no live row may put ph past the sequence: clamp it (a
        // block with a live row has its halo inside the sequence).
        const int ph = cs.p0 + rb * RB + i - RB;
        const TI *hp = own_p;
        if (i >= RB - 3) {
            if (ph >= 0)
                hp = x + (size_t)(cs.seq0 + min(ph, cs.p0 + cs.L - 1)) * H * D + (size_t)h * D;
            else if (cs.win)
                hp = cs.win + (size_t)(3 + max(ph, -3)) * CC + cwin;
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            if (ks >= ks0 && ks < ks1) raw_load(hp + ks * 32 + cq, rr.halo[ks]);
    }
}

// With norm the rows are scaled to unit length and, if inv is given, the
// scale 1 / sqrt(sum y^2 + eps) of this lane's row is returned there.
template <int D, typename TI>
__device__ __forceinline__ void rows_compute(RawRows<D, TI> &rr, const ChunkSrc<TI> &cs, int rb,
                                             const float *s_w, bool norm,
                                             float (&out)[D / 32][8], float *inv_out = nullptr) {
    constexpr int KS = D / 32;
    const int lane = threadIdx.x % kWave;
    const int i = lane % 16;
    const int cq = (lane / 16) * 8;
    const int row = rb * RB + i;
    const bool live = row < cs.L;
    const bool conv = s_w != nullptr;
    Raw8<TI>(&own)[KS] = rr.own;
    Raw8<TI>(&halo)[KS] = rr.halo;
    if (conv) {
        const int ph = cs.p0 + rb * RB + i - RB;
        const bool hvalid = i >= RB - 3 && (ph >= 0 || cs.win != nullptr);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int q = 0; q < Raw8<TI>::W; ++q) halo[ks].w[q] = hvalid ? halo[ks].w[q] : 0u;
    }
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int d0 = ks * 32 + cq;
        float y[8];
        raw_unpack(own[ks], y);
        if (conv) {
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] *= s_w[(d0 + e) * 4 + 3];
            // taps n = 1, 2, 3 rows up: source lane j = i - n (mod 16) offers
            // its own row if j <= 15 - n, else its halo row
#define GDN_TAP(N)                                                                       \
    {                                                                                    \
        Raw8<TI> t;                                                                      \
        _Pragma("unroll") for (int q = 0; q < Raw8<TI>::W; ++q)                          \
            t.w[q] = ror16<N>(i <= 15 - (N) ? own[ks].w[q] : halo[ks].w[q]);             \
        float xt[8];                                                                     \
        raw_unpack(t, xt);                                                               \
        _Pragma("unroll") for (int e = 0; e < 8; ++e)                                    \
            y[e] = fmaf(s_w[(d0 + e) * 4 + 3 - (N)], xt[e], y[e]);                       \
    }
            GDN_TAP(1)
            GDN_TAP(2)
            GDN_TAP(3)
#undef GDN_TAP
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            out[ks][e] = live ? y[e] : 0.f;
            ss = fmaf(out[ks][e], out[ks][e], ss);
        }
    }
    if (norm) {
        ss += __shfl_xor(ss, 16, kWave);
        ss += __shfl_xor(ss, 32, kWave);
        const float inv = 1.0f / sqrtf(ss + kNormEps);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) out[ks][e] *= inv;
        if (inv_out) *inv_out = inv;
    } else if (inv_out) {
        *inv_out = 1.f;
    }
}

// Stage the conv taps of `n` channels starting at channel c0 into LDS [n][4].
__device__ __forceinline__ void stage_taps(const float *conv_w, int c0, int n, float *s_w) {
    for (int idx = threadIdx.x; idx < n; idx += kThreads)
        reinterpret_cast<float4 *>(s_w)[idx] = reinterpret_cast<const float4 *>(conv_w)[c0 + idx];
}

// ------------------------------------------------------------ prep
// DPP row shift within each 16-lane row: lane i gets lane i - N of its row,
// lanes i < N get 0 (row_shr:N with bound_ctrl).
template <int N>
__device__ __forceinline__ float row_shr(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + N, 0xf, 0xf, true));
}

// e^x for the decay factors inside a chunk (|x| is at most the chunk's
// summed log decay): the hardware base-2 exponential of x log2(e), about
// 1e-6 relative here, in place of the library expf's longer range reduction
// (per key 128 of these per lane per chunk, 16 with a scalar decay).
__device__ __forceinline__ float exp_pk(float x) { return __expf(x); }

// Sum over each group of 4 lanes (DPP quad permutations: lane ^ 1, lane ^ 2).
__device__ __forceinline__ float quad_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, false));
    return x;
}

// Per-key running sums: log a of this lane's row (rows >= L add nothing)
// and keys ks * 32 + cq + e, scanned inclusively over the wave's 16 rows
// (DPP within 16-lane rows). g_add_earlier then adds the totals of the
// earlier waves' row blocks (s_gt [kWaves][DK]), giving g_r from the chunk
// start.
template <int DK>
__device__ __forceinline__ void g_scan_rows(const PrefillArgs &a, int h, int row0, int L, int row,
                                            int cq, float (&g)[DK / 32][8]) {
    const float *lap = a.log_alpha + ((size_t)(row0 + min(row, L - 1)) * a.H + h) * DK;
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) load8(lap + ks * 32 + cq, g[ks]);
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = row < L ? g[ks][e] : 0.f;
            x += row_shr<1>(x);
            x += row_shr<2>(x);
            x += row_shr<4>(x);
            x += row_shr<8>(x);
            g[ks][e] = x;
        }
}

template <int DK>
__device__ __forceinline__ void g_add_earlier(const float *s_gt, int w, int cq,
                                              float (&g)[DK / 32][8]) {
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int d = ks * 32 + cq + e;
            float before = 0.f;
#pragma unroll
            for (int ww = 0; ww < kWaves; ++ww) before += ww < w ? s_gt[ww * DK + d] : 0.f;
            g[ks][e] += before;
        }
}

// Largest exponent of the per-key join factor e^{g0[R] - g15[R]} (a row
// block's decay across its 16 rows) taken inside a factored product; past
// it the block's diagonal tile is evaluated from the definition
// (diag_direct). e^80 and the operands down to e^-80 stay normal in fp32.
constexpr float kJoinLimit = 80.f;

// Wave w's diagonal 16 x 16 tile of KK^T and QK^T under per-key decay,
// from the definition: entry (r, s), s <= r, is
// sum_d k_r[d] k_s[d] e^{g_r[d] - g_s[d]} (q_r in place of k_r for QK^T),
// every exponent <= 0. The lane's entries are those of the MFMA output
// layout: rows 16 w + 4 (lane / 16) + i, column 16 w + lane % 16. g holds
// this lane's sums (row 16 w + lane % 16, keys ks * 32 + cq + e); the Q and
// K rows are formed here (taps s_wq / s_wk, or null) and pass through
// s_work (kWaves * 3 * 16 rows of kDirectPitch floats) 32 keys at a time.
// Every thread of the block calls it (it synchronises).
constexpr int kDirectPitch = 36;  // staged row: 32 keys + 4 pad floats
constexpr int kDirectWork = kWaves * 3 * RB * kDirectPitch;

template <int DK, typename TI>
__device__ __forceinline__ void diag_direct(const PrefillArgs &a, const ChunkSrc<TI> &cs, int h,
                                            int CC, const float (&g)[DK / 32][8],
                                            const float *s_wq, const float *s_wk, float *s_work,
                                            f32x4v &kk, f32x4v &qk) {
    constexpr int KS = DK / 32, SP = kDirectPitch;
    const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
    const int cq = (lane / 16) * 8;
    const int H = a.H;
    const bool conv = a.conv_w != nullptr;
    float *const s_st = s_work + w * 3 * RB * SP;  // this wave's K | Q | g rows
    float qf[KS][8], kf[KS][8];
    {
        RawRows<DK, TI> rr;
        rows_load<DK, TI>(static_cast<const TI *>(a.q), H, h, cs, w, CC, h * DK, conv, rr);
        rows_compute<DK, TI>(rr, cs, w, s_wq, a.qk_norm != 0, qf);
    }
    {
        RawRows<DK, TI> rr;
        rows_load<DK, TI>(static_cast<const TI *>(a.k), H, h, cs, w, CC, H * DK + h * DK, conv,
                          rr);
        rows_compute<DK, TI>(rr, cs, w, s_wk, a.qk_norm != 0, kf);
    }
    kk = f32x4v{0.f, 0.f, 0.f, 0.f};
    qk = f32x4v{0.f, 0.f, 0.f, 0.f};
    const int sl = lane % 16, rl = 4 * (lane / 16);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        float *const p = s_st + (lane % 16) * SP + cq;
#pragma unroll
        for (int e = 0; e < 8; e += 4) {
            *reinterpret_cast<float4 *>(p + e) = make_float4(kf[ks][e], kf[ks][e + 1],
                                                             kf[ks][e + 2], kf[ks][e + 3]);
            *reinterpret_cast<float4 *>(p + RB * SP + e) =
                make_float4(qf[ks][e], qf[ks][e + 1], qf[ks][e + 2], qf[ks][e + 3]);
            *reinterpret_cast<float4 *>(p + 2 * RB * SP + e) =
                make_float4(g[ks][e], g[ks][e + 1], g[ks][e + 2], g[ks][e + 3]);
        }
        __syncthreads();
        const float *const sk = s_st, *const sq = s_st + RB * SP, *const sg = s_st + 2 * RB * SP;
#pragma unroll 1
        for (int d = 0; d < 32; d += 4) {
            const float4 kc = *reinterpret_cast<const float4 *>(sk + sl * SP + d);
            const float4 gc = *reinterpret_cast<const float4 *>(sg + sl * SP + d);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = rl + i;
                const float4 kr = *reinterpret_cast<const float4 *>(sk + r * SP + d);
                const float4 qr = *reinterpret_cast<const float4 *>(sq + r * SP + d);
                const float4 gv = *reinterpret_cast<const float4 *>(sg + r * SP + d);
                const bool in = sl <= r;
                const float f0 = in ? exp_pk(fminf(gv.x - gc.x, 0.f)) : 0.f;
                const float f1 = in ? exp_pk(fminf(gv.y - gc.y, 0.f)) : 0.f;
                const float f2 = in ? exp_pk(fminf(gv.z - gc.z, 0.f)) : 0.f;
                const float f3 = in ? exp_pk(fminf(gv.w - gc.w, 0.f)) : 0.f;
                const float t0 = kc.x * f0, t1 = kc.y * f1, t2 = kc.z * f2, t3 = kc.w * f3;
                kk[i] = fmaf(kr.x, t0, fmaf(kr.y, t1, fmaf(kr.z, t2, fmaf(kr.w, t3, kk[i]))));
                qk[i] = fmaf(qr.x, t0, fmaf(qr.y, t1, fmaf(qr.z, t2, fmaf(qr.w, t3, qk[i]))));
            }
        }
        __syncthreads();  // before the staging is written again
    }
}

// VAR: the decay / update rule. kScalar: log a [N, H], the gated delta rule.
// kKda: per-key log a [N, H, d_k], delta rule. kRwkv6: per-key log a, raw
// value update (u = v: no A, T' = I, no K Sig term, beta unused).
// Per-key chunk form (g_r[d] running sums per key, <= 0 and
// non-increasing): with K^ = K . e^{g}, Q^ = Q . e^{g},
//   A[r][s] = beta_r sum_d k_r[d] k_s[d] e^{g_r[d] - g_s[d]}   (s < r),
//   P[r][s] = sum_d q_r[d] k_s[d] e^{g_r[d] - g_s[d]}          (s <= r),
//   U = T' (V - K^ Sig0),  O = Q^ Sig0 + P U,
//   Sig_L = diag(e^{g_L}) Sig0 + sum_r (k_r . e^{g_L - g_r}) u_r^T,
// which the scan runs with gamma = 1 and a per-key state decay. Every
// factor the record holds is <= 1. A and P are products against 16-row
// block references (see prep_body), so no factor leaves fp32's range for
// any decay: e^{-g_s} alone would overflow once a chunk decays past e^-88.
// Rows x C matrix staged in LDS (rows padded to C + 1 floats) -> hi / lo
// bf16 planes of the record, 8 elements (16 bytes) per store: row-major
// [rows][C], or in A-fragment order (FRAG: a lower-triangular C x C matrix,
// T' or P, of which only the 16 x 32 blocks at or below the diagonal are
// kept, tri_off).
template <int ROWS, bool F, bool FRAG = false>
__device__ __forceinline__ void put_planes(const float *src, __bf16 *hi, __bf16 *lo) {
    constexpr int G = C / 8;  // 8-element groups per row
    for (int idx = threadIdx.x; idx < ROWS * G; idx += kThreads) {
        const int r = idx / G, c0 = (idx % G) * 8;
        if (FRAG && c0 / 32 > (r / 16 * 16 + 15) / 32) continue;
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = src[r * (C + 1) + c0 + e];
        const int off = FRAG ? tri_off(r / 16, c0 / 32, r % 16 + 16 * ((c0 % 32) / 8))
                             : r * C + c0;
        store_frag<F>(hi + off, lo + off, frag<F>(x));
    }
}

// The prep's two LDS buffers (floats): s_k holds the staged K rows
// [C][DK + 4], then K~^T [DK][C + 1], then P and T' [C][C + 1] side by side;
// s_A holds A [C][C + 4].
__host__ __device__ constexpr int prep_sk_floats(int dk) {
    return std::max({C * (dk + 4), dk * (C + 1), 2 * C * (C + 1)});
}
constexpr int kPrepAFloats = C * (C + 4);

// How prep_body finds its chunk and where its results go: kPrepGrid, the
// prep kernel (chunk and head from the block index, the record in the
// workspace); for the one-chunk kernel (chunk 0 of out->s, head out->h),
// kPrepOnChip (scalar decay: no record, the operands handed over in
// PrepOut) or kPrepToSlot (per-key decay: the record written to the
// workspace slot of the (sequence, head), read back by the same
// workgroup).
enum PrepMode { kPrepGrid = 0, kPrepOnChip = 1, kPrepToSlot = 2 };

// What the one-chunk kernel takes from the prep steps: the chunk's sequence
// and head (in), with kPrepOnChip the Q and K A operands of the lane's rows,
// g of row `lane` and g_L (out), and the prep's LDS: P and T' [C][C + 1] at
// lds_k and lds_k + C (C + 1) when it returns, free for reuse with lds_a
// and lds_tab (per key, [4 kWaves + 10] DK floats) once they are read.
template <int DK, typename TI>
struct PrepOut {
    int s, h;
    Frag<std::is_same<TI, float>::value> qa[DK / 32], ka[DK / 32];
    float g, gL;
    float *lds_k, *lds_a, *lds_tab;
};

template <int DK, typename TI, int VAR, int MODE = kPrepGrid>
__device__ __forceinline__ void prep_body(const PrefillArgs &a, PrepOut<DK, TI> *out = nullptr) {
    constexpr bool FUSED = MODE == kPrepOnChip;  // operands kept on chip, no record
    constexpr bool ONE = MODE != kPrepGrid;      // the one-chunk kernel's chunk
    static_assert(!FUSED || VAR == kScalar, "operands on chip with a scalar decay only");
    constexpr bool kPerKey = VAR != kScalar;
    constexpr bool kDelta = VAR != kRwkv6;
    constexpr bool F = std::is_same<TI, float>::value;  // fp32 operands (see Frag)
    constexpr int KS = DK / 32;
    constexpr int SK = prep_sk_floats(DK);
    __shared__ __attribute__((aligned(16))) float s_k[SK];
    // the split B operand rows of KK^T / QK^T [C][DK] hi / lo, in s_k's space
    static_assert(C * DK <= SK, "split K rows fit s_k");
    __bf16 *const s_bh = reinterpret_cast<__bf16 *>(s_k), *const s_bl = s_bh + C * DK;
    // A, strictly lower, rows of AP floats with each row's entries grouped by
    // j mod 4 (see a_idx), so the substitution reads them as float4
    constexpr int AP = C + 4;
    const auto a_idx = [](int r, int j) { return r * AP + (j % 4) * (C / 4) + j / 4; };
    __shared__ __attribute__((aligned(16))) float s_A[kPrepAFloats];
    // the q / k conv taps live in s_A's space until A is formed
    static_assert(2 * DK * 4 <= C * AP, "taps fit the A buffer");
    float *const s_wq = s_A, *const s_wk = s_A + DK * 4;
    __shared__ float s_gt[kPerKey ? kWaves * DK : 1];  // per-key: each wave's row-block sums
    __shared__ __attribute__((aligned(16))) float s_gl[kPerKey ? DK : 4];  // per-key: g_L
    // per key, [kWaves][DK] each: the row blocks' first- and last-row sums
    // g0 and g15, e^{g0}, e^{g_L - g15}; then the join factors
    // e^{g0[R] - g15[S]} (S <= R, pair R (R + 1) / 2 + S) [kPairs][DK];
    // s_slow: some block decays past e^{-kJoinLimit} in some key
    constexpr int kPairs = kWaves * (kWaves + 1) / 2;
    constexpr int TG0 = 0, TG15 = kWaves * DK, TEG0 = 2 * kWaves * DK, TEL = 3 * kWaves * DK,
                  TM = 4 * kWaves * DK;
    __shared__ __attribute__((aligned(16))) float s_tab[kPerKey ? TM + kPairs * DK : 4];
    __shared__ int s_slow;

    const int32_t *chunk_start = static_cast<const int32_t *>(a.ws);
    const int gc = ONE ? 0 : (int)blockIdx.x, h = ONE ? out->h : (int)blockIdx.y;
    if (!ONE && gc >= chunk_start[a.n_seq]) return;
    const int s = ONE ? out->s : find_seq(chunk_start, a.n_seq, gc);
    const SeqSpan sp = seq_span(a.cu, s, a.n_tokens);
    const WsLayout wl = ws_layout(a.n_tokens, a.n_seq, a.H, DK, a.dv, kPerKey, a.nseg);
    // the chunk's index in its sequence (the segment's window starts there)
    const int c = ONE ? 0 : gc - chunk_start[s] + chunk_start[wl.win_off + s];
    const int H = a.H;
    const int CC = H * (2 * DK + a.dv);
    const int src = a.parent ? a.parent[s] : s;
    const bool src_ok = src >= 0 && src < a.n_parent;
    ChunkSrc<TI> cs{sp.start, c * C, min(C, sp.len - c * C),
                    (a.win_in && src_ok) ? static_cast<const TI *>(a.win_in) + (size_t)src * 3 * CC
                                         : nullptr};
    const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
    constexpr RecLayout RL = rec_layout(DK, kPerKey);
    // the record: of chunk gc, or (kPrepToSlot) in slot s H + h
    __bf16 *rec = FUSED ? nullptr
                        : reinterpret_cast<__bf16 *>(static_cast<char *>(a.ws) + wl.rec_off) +
                              ((size_t)(ONE ? s : gc) * H + h) * wl.rec_elems;
    float *const fac = FUSED ? nullptr : reinterpret_cast<float *>(rec + RL.fac);

    const bool conv = a.conv_w != nullptr;
    if (conv) {
        stage_taps(a.conv_w, h * DK, DK, s_wq);
        stage_taps(a.conv_w, H * DK + h * DK, DK, s_wk);
    }
    if (kPerKey && tid == 0) s_slow = 0;
    __syncthreads();
    const int row = w * RB + lane % 16;  // this lane's row in the A layout
    const int cq = (lane / 16) * 8;
    // scalar decay: g of row `lane`; per key: g of this lane's row and
    // columns (A layout), the factors e^{g}, e^{-g}, e^{g_L - g} taken where
    // they are used (few registers stay live across the loads)
    float g = 0.f, gL = 0.f;
    float gr[KS][8];
    if constexpr (!kPerKey) {
        g = chunk_g(a.log_alpha, H, h, cs.seq0, cs.p0, cs.L);
        gL = __shfl(g, C - 1, kWave);
    } else {
        g_scan_rows<DK>(a, h, cs.seq0 + cs.p0, cs.L, row, cq, gr);
        if (lane % 16 == 15)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) s_gt[w * DK + ks * 32 + cq + e] = gr[ks][e];
        __syncthreads();
        g_add_earlier<DK>(s_gt, w, cq, gr);
        // the block's first- and last-row sums
        if (lane % 16 == 0 || lane % 16 == 15) {
            float *const dst = s_tab + (lane % 16 == 0 ? TG0 : TG15) + w * DK + cq;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) dst[ks * 32 + e] = gr[ks][e];
        }
        // g_L per key; e^{g_L} for the scan's state decay
        if (tid < DK) {
            float total = 0.f;
#pragma unroll
            for (int ww = 0; ww < kWaves; ++ww) total += s_gt[ww * DK + tid];
            s_gl[tid] = total;
            fac[tid] = expf(total);
        }
        __syncthreads();
        for (int idx = tid; idx < kWaves * DK; idx += kThreads) {
            s_tab[TEG0 + idx] = exp_pk(s_tab[TG0 + idx]);
            s_tab[TEL + idx] = exp_pk(s_gl[idx % DK] - s_tab[TG15 + idx]);
        }
        for (int idx = tid; idx < kPairs * DK; idx += kThreads) {
            const int pr = idx / DK, d = idx % DK;
            int R = 0;
            while ((R + 1) * (R + 2) / 2 <= pr) ++R;
            const int S = pr - R * (R + 1) / 2;
            const float x = s_tab[TG0 + R * DK + d] - s_tab[TG15 + S * DK + d];
            if (S == R && x > kJoinLimit) s_slow = 1;
            s_tab[TM + idx] = exp_pk(fminf(x, kJoinLimit));
        }
        __syncthreads();
    }
    // a block decays past e^{-kJoinLimit} in some key: its join factor is
    // clamped, and every wave takes its diagonal tile from the definition
    // instead (while s_k is still free and the taps are staged)
    f32x4v kk_diag = {0.f, 0.f, 0.f, 0.f}, qk_diag = {0.f, 0.f, 0.f, 0.f};
    bool slow = false;
    if constexpr (kPerKey) {
        slow = __builtin_amdgcn_readfirstlane(s_slow) != 0;
        static_assert(kDirectWork <= SK, "direct staging fits s_k");
        if (slow)
            diag_direct<DK, TI>(a, cs, h, CC, gr, conv ? s_wq : nullptr, conv ? s_wk : nullptr,
                                s_k, kk_diag, qk_diag);
    }
    float b_l = 1.f;
    if constexpr (kDelta) b_l = a.beta[(size_t)(cs.seq0 + cs.p0 + min(lane, cs.L - 1)) * H + h];
    b_l = lane < cs.L ? b_l : 0.f;

    // conv'd, normalised Q and K rows (per key: decayed); their split A
    // operands go to the record. With a scalar decay the raw Q and K rows
    // are requested together (the per-key form has no registers to spare).
    // Per key the matrix products take each row block against its own first
    // row, e1 = e^{g_r - g0} <= 1 (row operands Q. e1, K. e1), and each
    // column against its block's last row, e^{g15 - g_s} <= 1 (column
    // operand, kept in fp32 in s_b32); a tile (R, S) joins the two with the
    // per-key factor e^{g0[R] - g15[S]} (<= 1 off the diagonal). The record
    // keeps the forms from the chunk start, Q^ = Q. e^{g}, K^ = K. e^{g}.
    Frag<F> qa[DK / 32], ka[DK / 32];
    float *const s_b32 = s_k;  // per key: the column operands [C][DK], fragment order
    float e1[kPerKey ? DK / 32 : 1][8];
    if constexpr (kPerKey) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float g0v[8];
            lds_read8(s_tab + TG0 + w * DK + ks * 32 + cq, g0v);
#pragma unroll
            for (int e = 0; e < 8; ++e) e1[ks][e] = exp_pk(gr[ks][e] - g0v[e]);
        }
    }
    RawRows<DK, TI> rk;
    const auto load_k = [&] {
        rows_load<DK, TI>(static_cast<const TI *>(a.k), H, h, cs, w, CC, H * DK + h * DK, conv,
                          rk);
    };
    {
        RawRows<DK, TI> rq;
        rows_load<DK, TI>(static_cast<const TI *>(a.q), H, h, cs, w, CC, h * DK, conv, rq);
        if constexpr (!kPerKey) load_k();
        float qf[DK / 32][8];
        rows_compute<DK, TI>(rq, cs, w, conv ? s_wq : nullptr, a.qk_norm != 0, qf);
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks) {
            const int off = frag_off(KS, w, ks, lane);
            if constexpr (kPerKey) {
                float eg[8], qr[8];
                lds_read8(s_tab + TEG0 + w * DK + ks * 32 + cq, eg);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    qf[ks][e] *= e1[ks][e];
                    qr[e] = qf[ks][e] * eg[e];  // Q^
                }
                qa[ks] = frag<F>(qf[ks]);
                store_frag<F>(rec + RL.qhi + off, rec + RL.qlo + off, frag<F>(qr));
            } else {
                qa[ks] = frag<F>(qf[ks]);
                if constexpr (!FUSED) store_frag<F>(rec + RL.qhi + off, rec + RL.qlo + off, qa[ks]);
            }
        }
    }
    if constexpr (kPerKey) load_k();
    float kf[DK / 32][8];
    rows_compute<DK, TI>(rk, cs, w, conv ? s_wk : nullptr, a.qk_norm != 0, kf);
    if constexpr (!kPerKey && !FUSED) {
        // the scan's row factors: gamma_r, e^{g_L - g_r}, and gamma_L
        if (w == 0) {
            fac[lane] = expf(g);
            fac[C + lane] = expf(gL - g);
        }
        if (tid == 0) fac[2 * C] = expf(gL);
    }
#pragma unroll
    for (int ks = 0; ks < DK / 32; ++ks) {
        const int off = frag_off(KS, w, ks, lane);
        if constexpr (kPerKey) {
            // row operand K. e1; the record's K^ (the scan's K Sig term; zero
            // for the raw value update); the column operand K. e^{g15 - g}
            float g15v[8], eg[8], ak[8], kr[8], bk[8];
            lds_read8(s_tab + TG15 + w * DK + ks * 32 + cq, g15v);
            lds_read8(s_tab + TEG0 + w * DK + ks * 32 + cq, eg);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                ak[e] = kf[ks][e] * e1[ks][e];
                kr[e] = kDelta ? ak[e] * eg[e] : 0.f;
                bk[e] = kf[ks][e] * exp_pk(g15v[e] - gr[ks][e]);
            }
            ka[ks] = frag<F>(ak);
            store_frag<F>(rec + RL.khi + off, rec + RL.klo + off, frag<F>(kr));
            *reinterpret_cast<f32x4v *>(s_b32 + off) = f32x4v{bk[0], bk[1], bk[2], bk[3]};
            *reinterpret_cast<f32x4v *>(s_b32 + off + 4) = f32x4v{bk[4], bk[5], bk[6], bk[7]};
        } else {
            // A operand of KK^T and the scan's K Sig term: K; the B operand
            // rows of KK^T and QK^T, split once, in fragment order: the
            // reader of row block ct takes lane l's piece of wave ct
            ka[ks] = frag<F>(kf[ks]);
            if constexpr (!FUSED) store_frag<F>(rec + RL.khi + off, rec + RL.klo + off, ka[ks]);
            store_frag<F>(s_bh + off, s_bl + off, ka[ks]);
        }
    }
    __syncthreads();

    // KK^T and QK^T tiles (w, ct), ct <= w, on MFMA; A to LDS, P kept in
    // registers until s_k is free. g and beta of this lane's 4 rows are
    // taken once.
    float g_rr[4], b_rr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        g_rr[i] = __shfl(g, w * RB + (lane / 16) * 4 + i, kWave);
        b_rr[i] = __shfl(b_l, w * RB + (lane / 16) * 4 + i, kWave);
    }
    float pv[C / RB][4];
    // D layout: rows w*16 + (l/16)*4 + i, column ct*16 + l%16
    const auto put_tile = [&](int ct, const f32x4v &kk, const f32x4v &qk, float (&pvc)[4]) {
        const int col = ct * RB + lane % 16;
        const float g_c = __shfl(g, col, kWave);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = w * RB + (lane / 16) * 4 + i;
            const bool live = r < cs.L && col < cs.L;
            // the decay between rows: a factor here (scalar), inside the
            // products already (per key)
            const float dec = (live && col <= r) ? (kPerKey ? 1.f : exp_pk(g_rr[i] - g_c)) : 0.f;
            s_A[a_idx(r, col)] = (kDelta && col < r) ? b_rr[i] * dec * kk[i] : 0.f;
            pvc[i] = dec * qk[i];
        }
    };
#pragma unroll
    for (int ct = 0; ct < C / RB; ++ct) {
        f32x4v kk = {0.f, 0.f, 0.f, 0.f}, qk = {0.f, 0.f, 0.f, 0.f};
        if (ct <= w) {
#pragma unroll
            for (int ks = 0; ks < DK / 32; ++ks) {
                const int off = frag_off(KS, ct, ks, lane);
                Frag<F> bs;
                if constexpr (kPerKey) {
                    float bv[8], mv[8];
                    lds_read8(s_b32 + off, bv);
                    lds_read8(s_tab + TM + (w * (w + 1) / 2 + ct) * DK + ks * 32 + cq, mv);
#pragma unroll
                    for (int e = 0; e < 8; ++e) bv[e] *= mv[e];
                    bs = frag<F>(bv);
                } else {
                    bs = read_frag<F>(s_bh + off, s_bl + off);
                }
                if constexpr (kDelta) kk = mma(ka[ks], bs, kk);
                qk = mma(qa[ks], bs, qk);
            }
        }
        if (kPerKey && slow && ct == w) {
            kk = kk_diag;
            qk = qk_diag;
        }
        put_tile(ct, kk, qk, pv[ct]);
    }
    if constexpr (kPerKey) {
        // this row's K~ = K. e^{g_L - g} = (column operand) e^{g_L - g15},
        // read back before s_k is reused
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float bv[8], ev[8];
            lds_read8(s_b32 + frag_off(KS, w, ks, lane), bv);
            lds_read8(s_tab + TEL + w * DK + ks * 32 + cq, ev);
#pragma unroll
            for (int e = 0; e < 8; ++e) kf[ks][e] = bv[e] * ev[e];
        }
    }
    __syncthreads();  // s_A complete; the K rows in s_k are no longer needed

    if constexpr (kPerKey) {
        // K~^T[d][r] = k_r[d] e^{g_L - g_r}, staged transposed for coalesced stores
#pragma unroll
        for (int ks = 0; ks < DK / 32; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) s_k[(ks * 32 + cq + e) * (C + 1) + row] = kf[ks][e];
        __syncthreads();
        put_planes<DK, F>(s_k, rec + RL.kthi, rec + RL.ktlo);
    }

    // T = (I + A)^-1 by 16-row blocks (block row R = wave R), staged
    // unscaled in s_T (the blocks at or below the diagonal; the two blocks
    // above it that share a stored 16 x 32 block are zero):
    //  1. T_RR = (I + A_RR)^-1 by forward substitution, one column per group
    //     of 4 lanes: lane (cl, part) keeps T_RR[j][cl] for j = part (mod 4),
    //     from the identity column (rows r <= cl leave it unchanged);
    //  2. level by level (R - S = 1, 2, 3), T_RS = -T_RR sum_{S<=K<R} A_RK T_KS
    //     on MFMA (16 x 16 x 16 products; the sum's output layout is the B
    //     operand of the left product as it stands).
    // Then T' = T diag(beta) in place.
    if constexpr (kPerKey) __syncthreads();  // the K~^T copy-out has read s_k
    float *const s_P = s_k, *const s_T = s_k + C * (C + 1);
    static_assert(2 * C * (C + 1) <= SK, "P and T' staging fit s_k");
    constexpr int TP = C + 1;  // s_T row pitch
    {
        const int cl = lane / 4, part = lane % 4;
        float t[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) t[q] = (4 * q + part == cl) ? 1.f : 0.f;
        // A[16w + r][16w + 4q + part] = arow[r * AP + q] (a_idx groups j by j % 4)
        const float *arow = s_A + (w * RB) * AP + part * (C / 4) + 4 * w;
#pragma unroll
        for (int r = 1; r < RB; ++r) {
            const float4 av = *reinterpret_cast<const float4 *>(arow + r * AP);
            float acc = 0.f;
            if (part < r) acc = fmaf(av.x, t[0], acc);
            if (4 + part < r) acc = fmaf(av.y, t[1], acc);
            if (8 + part < r) acc = fmaf(av.z, t[2], acc);
            if (12 + part < r) acc = fmaf(av.w, t[3], acc);
            acc = quad_sum(acc);
            if (r > cl && r % 4 == part) t[r / 4] = -acc;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) s_T[(w * RB + 4 * q + part) * TP + w * RB + cl] = t[q];
        if (w % 2 == 0)  // the block above the diagonal in this row block's 16 x 32 pair
#pragma unroll
            for (int q = 0; q < 4; ++q) s_T[(w * RB + 4 * q + part) * TP + (w + 1) * RB + cl] = 0.f;
    }
    __syncthreads();
    {
        const int g = lane / 16, n = lane % 16;
#pragma unroll
        for (int level = 1; level < kWaves; ++level) {
            if (w >= level) {
                const int R = w, S = w - level;
                f32x4v x = {0.f, 0.f, 0.f, 0.f};
                for (int K = S; K < R; ++K) {
                    f32x4v av, bv;  // A_RK (row 16R + n, k = 16K + 4g + e); T_KS (col 16S + n)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        av[e] = s_A[(R * RB + n) * AP + e * (C / 4) + 4 * K + g];
                        bv[e] = s_T[(K * RB + 4 * g + e) * TP + S * RB + n];
                    }
                    x = mma16(frag4<F>(av), frag4<F>(bv), x);
                }
                f32x4v tv;  // T_RR (row 16R + n, k = 16R + 4g + e)
#pragma unroll
                for (int e = 0; e < 4; ++e) tv[e] = s_T[(R * RB + n) * TP + R * RB + 4 * g + e];
                const f32x4v y = mma16(frag4<F>(tv), frag4<F>(x), f32x4v{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int i = 0; i < 4; ++i) s_T[(R * RB + 4 * g + i) * TP + S * RB + n] = -y[i];
            }
            __syncthreads();
        }
    }
    // P (from registers) beside T, for coalesced stores; T' = T diag(beta):
    // a thread's column is its lane, whose beta it holds
#pragma unroll
    for (int ct = 0; ct < C / RB; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            s_P[(w * RB + (lane / 16) * 4 + i) * (C + 1) + ct * RB + lane % 16] = pv[ct][i];
    for (int idx = tid; idx < C * C; idx += kThreads) s_T[(idx / C) * TP + idx % C] *= b_l;
    __syncthreads();
    if constexpr (FUSED) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            out->qa[ks] = qa[ks];
            out->ka[ks] = ka[ks];
        }
        out->g = g;
        out->gL = gL;
        out->lds_k = s_k;
        out->lds_a = s_A;
    } else {
        put_planes<C, F, true>(s_P, rec + RL.phi, rec + RL.plo);
        put_planes<C, F, true>(s_T, rec + RL.thi, rec + RL.tlo);
        if constexpr (ONE) {
            out->lds_k = s_k;
            out->lds_a = s_A;
            out->lds_tab = s_tab;
        }
    }
}

template <int DK, typename TI>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void prep_kernel(PrefillArgs a) {
    prep_body<DK, TI, kScalar>(a);
}

// Per key the decay factors add registers; capped so two workgroups of the
// largest head size still share a compute unit (measured faster than one,
// while the scalar form runs best at its natural allocation).
template <int DK, typename TI, int VAR>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void prep_kernel_pk(
    PrefillArgs a) {
    prep_body<DK, TI, VAR>(a);
}

// ------------------------------------------------------------ scan
// Conv window after position `end` of the sequence starting at stream row
// seq0: its last 3 raw inputs (from the incoming window win where end < 3,
// zeros without one), head h's q, k and v channels, into wo [3][CC].
template <int DK, int DV, typename TI>
__device__ __forceinline__ void write_window(const PrefillArgs &a, int h, int seq0, const TI *win,
                                             TI *wo, int end) {
    const int H = a.H, CC = H * (2 * DK + DV), W = 2 * DK + DV;
    for (int idx = threadIdx.x; idx < 3 * W; idx += kThreads) {
        const int r = idx / W, wc = idx % W;
        const int p = end - 3 + r;
        const int part = wc < DK ? 0 : wc < 2 * DK ? 1 : 2;  // q, k or v
        const int i = wc - part * DK;
        const int cch = part == 2 ? 2 * H * DK + h * DV + i : part * H * DK + h * DK + i;
        TI val = from_f32<TI>(0.f);
        if (p >= 0) {
            const size_t row = (size_t)(seq0 + p);
            if (part == 0) val = static_cast<const TI *>(a.q)[row * H * DK + (size_t)h * DK + i];
            else if (part == 1) val = static_cast<const TI *>(a.k)[row * H * DK + (size_t)h * DK + i];
            else val = static_cast<const TI *>(a.v)[row * H * DV + (size_t)h * DV + i];
        } else if (win) {
            val = win[(size_t)(3 + p) * CC + cch];
        }
        wo[(size_t)r * CC + cch] = val;
    }
}

// Workgroup -> (sequence-head, value tile): the NT value tiles of one
// sequence-head get block indices congruent modulo 8, so they are dispatched
// to the same XCD and share its L2 for the chunk records they all read.
__device__ __forceinline__ void scan_unit(int b, int NT, int &sh, int &tile) {
    const int xcd = b % 8, local = b / 8;
    tile = local % NT;
    sh = (local / NT) * 8 + xcd;
}

// Offset (in bf16 elements) of 16-byte chunk `ch` of row `r` in an LDS
// plane of rows of C bf16 (128 bytes): the chunk index is XOR-swizzled by
// the row so that 16 lanes reading one chunk of 16 consecutive rows spread
// over all banks.
__device__ __forceinline__ int kt_swz(int r, int ch) { return r * C + ((ch ^ (r & 7)) << 3); }

// Registers a chunk step needs from memory, loaded ahead of use: only loads
// go in here (no arithmetic on the results), so the loads can stay in
// flight until the step consumes them.

// Two adjacent outputs (pair-aligned) in one store.
__device__ __forceinline__ void store_pair(float *p, float x, float y) {
    *reinterpret_cast<float2 *>(p) = make_float2(x, y);
}
__device__ __forceinline__ void store_pair(bf16 *p, float x, float y) {
    *reinterpret_cast<uint32_t *>(p) =
        (uint32_t)from_f32<bf16>(x).bits | ((uint32_t)from_f32<bf16>(y).bits << 16);
}

// 16-byte direct-to-LDS load (lane l lands at lds + 8 l elements). Kept out
// of the kernel templates: with the builtin inside a template the host pass
// drops the kernel's launch stub without a diagnostic.
__device__ __forceinline__ void lds_dma16(const __bf16 *g, __bf16 *lds) {
    __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
}

// Two adjacent io-dtype values in one load: the value columns 2n, 2n + 1 of
// a lane (see vcol).
template <typename TI> struct VPair;
template <> struct VPair<bf16> {
    typedef uint32_t type;
    static __device__ __forceinline__ float get(type x, int t) {
        return __uint_as_float(t == 0 ? x << 16 : x & 0xffff0000u);
    }
};
template <> struct VPair<float> {
    typedef float2 type;
    static __device__ __forceinline__ float get(type x, int t) { return t == 0 ? x.x : x.y; }
};

// Value columns of a scan tile: internal column c (sub-tile t = c / 16,
// MFMA column n = c % 16) is the tile's column 2n + t, so the two columns a
// lane holds are adjacent in memory (one load / store per row for both).
__device__ __forceinline__ int vcol(int c) { return 2 * (c % 16) + c / 16; }

// K^T [d_k][C] in LDS for the scalar-decay state update, formed from the
// K operands of the chunk record. Rows (key d) hold C = 64 bf16 (128 bytes:
// eight 16-byte pieces of 8 consecutive chunk rows); the piece index is
// XOR-swizzled by the key so that the writes (one bf16 per store from the
// A-operand layout: a lane's chunk row r, 8 keys, 8 apart across the 16-lane
// groups) and the 16-byte B-operand reads (a lane's key, 8 consecutive
// chunk rows; 16 consecutive keys per 16 lanes) spread over the banks.
__device__ __forceinline__ int kt_off(int d, int r) {
    const int sw = ((d >> 1) & 7) ^ (((d >> 4) & 1) << 1);
    return d * C + ((((r >> 3) ^ sw) & 7) << 3) + (r & 7);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The 8 values of a lane's A-operand piece (chunk row r, keys d0 .. d0 + 7,
// d0 a multiple of 8) into the K^T planes. Split bf16: one bf16 per store
// (the halves of each 32-bit word are written from the word itself); for
// such d0 the swizzle of key d0 + e is sw(d0) ^ (e >> 1), so the 8 stores
// of a plane use 4 base offsets and constant displacements. fp32: one
// element per store (put1).
__device__ __forceinline__ void put_kt(const Frag<true> &x, int d0, int r, __bf16 *kh, __bf16 *kl) {
#pragma unroll
    for (int e = 0; e < 8; ++e) put1<true>(kh, kl, kt_off(d0 + e, r), e < 4 ? x.hi[e] : x.lo[e - 4]);
}
__device__ __forceinline__ void put_kt(const Frag<false> &x, int d0, int r, __bf16 *kh, __bf16 *kl) {
    const u32x4 h = __builtin_bit_cast(u32x4, x.hi);
    const u32x4 l = __builtin_bit_cast(u32x4, x.lo);
    const int sw = ((d0 >> 1) & 7) ^ (((d0 >> 4) & 1) << 1);
    const int X = ((r >> 3) ^ sw) & 7, base = d0 * C + (r & 7);
    uint16_t *ph = reinterpret_cast<uint16_t *>(kh) + base;
    uint16_t *pl = reinterpret_cast<uint16_t *>(kl) + base;
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // keys d0 + 2q, d0 + 2q + 1: slot X ^ q
        const int o = ((X ^ q) << 3) + 2 * q * C;
        ph[o] = (uint16_t)(h[q] & 0xffffu);
        ph[o + C] = (uint16_t)(h[q] >> 16);
        pl[o] = (uint16_t)(l[q] & 0xffffu);
        pl[o + C] = (uint16_t)(l[q] >> 16);
    }
}

// The split state planes Sig^T [TV][d_k] (bf16 elements): row = value
// column, 16-byte pieces of 8 consecutive keys (the B operand of K Sig0 and
// Q Sig0: 16 lanes read one piece of 16 consecutive rows), written one bf16
// at a time from the state update's output layout (16 lanes write 16
// consecutive keys of a row); the piece index is XOR-swizzled by the row.
template <int DK>
__device__ __forceinline__ int st_off(int v, int key) {
    constexpr int P = DK / 8;                            // pieces per row
    constexpr int S = DK == 128 ? 0 : DK == 64 ? 1 : 2;  // log2(16 / P)
    return v * DK + ((((key >> 3) ^ (v >> S)) & (P - 1)) << 3) + (key & 7);
}

template <int KS, int NVT, typename TI>
struct ChunkRegs {
    static_assert(NVT == 2, "a lane holds one adjacent pair of value columns");
    Frag<std::is_same<TI, float>::value> ka[KS], qa[KS], ta[2], pa[2];
    typename VPair<TI>::type vraw[7];  // raw V rows r0-3 .. r0+3 of this lane's column pair
    f32x4v gam;       // scalar decay: gamma_r of this lane's 4 rows (C/D layout)
    f32x4v gu;        // scalar decay: e^{g_L - g_r} of the same rows
    float gaml;       // scalar decay: gamma_L
};

// PK: per-key decay (K and Q arrive decayed, gamma = 1; the state decays by
// e^{g_L} per key column, staged in LDS with the chunk's K~^T planes, which
// the record holds). Scalar decay: K^T is formed in LDS from the chunk's K
// operands and the update takes W = diag(e^{g_L - g}) U, since
// K~^T U = K^T W.
// CK: also write checkpoints (state and window every ckpt_every chunks);
// a separate instance so the plain scan keeps its register budget.
// GRP: branch groups (a.groups set); else one sequence per workgroup, so
// the sequence loop below runs once and compiles away.
// scan_body runs workgroup unit b (a sequence-head or branch group, and a
// value tile; see scan_unit) and returns false, having done nothing, when
// neither b nor any unit b + 8 k has work.
template <int DK, int DV, typename TI, typename TO, bool PK, bool CK, bool GRP>
__device__ __forceinline__ bool scan_body(const PrefillArgs &a, int b) {
    constexpr bool F = std::is_same<TI, float>::value;  // fp32 operands (see Frag)
    constexpr int KS = DK / 32;          // k-steps over d_k
    constexpr int CB = C + 8;            // padded row of the R^T / U^T / W^T planes
    constexpr int NVT = TV / 16;         // 16-wide value sub-tiles
    constexpr int NFT = NVT * (DK / 16); // output tiles of the state update
    constexpr int NEG = NFT / kWaves;    // state-update tiles per wave
    static_assert(NFT % kWaves == 0, "state-update tiles split evenly over the waves");
    static_assert(DK / 4 <= kWave, "e^{g_L} row fits one wave's 16-byte copies");
    constexpr RecLayout RL = rec_layout(DK, PK);
    // The fp32 state tile lives in registers: each wave owns NEG 16 x 16
    // output tiles of the state update (mst). LDS holds it split into hi /
    // lo bf16 planes Sig^T [TV][DK] (st_off), the B operand of K Sig0 and
    // Q Sig0; R^T, U^T (and, scalar decay, W^T) [TV][C] as hi / lo bf16
    // planes (split once when written; the same buffer stages state
    // write-outs); K~^T (per key: copied from the chunk record by direct-to-
    // LDS loads, swizzled rows) or K^T (scalar decay: formed from the K
    // operands, kt_off) [DK][C] hi / lo.
    constexpr int NPL = PK ? 4 : 6;  // R, U (, W) hi / lo planes
    __shared__ __attribute__((aligned(16))) __bf16 s_Sh[TV * DK], s_Sl[TV * DK];
    __shared__ __attribute__((aligned(16))) __bf16 s_pl[NPL * TV * CB];
    static_assert(DK * TV * 4 <= NPL * TV * CB * 2, "state staging fits the plane buffer");
    __bf16 *const s_Rh = s_pl, *const s_Rl = s_pl + TV * CB;
    __bf16 *const s_Uh = s_pl + 2 * TV * CB, *const s_Ul = s_pl + 3 * TV * CB;
    __bf16 *const s_Wh = s_pl + (PK ? 0 : 4) * TV * CB, *const s_Wl = s_pl + (PK ? 0 : 5) * TV * CB;
    float *const s_stage = reinterpret_cast<float *>(s_pl);  // [DK][TV] fp32
    __shared__ __attribute__((aligned(16))) __bf16 s_Kh[DK * C], s_Kl[DK * C];
    __shared__ __attribute__((aligned(16))) float s_wv[TV * 4];
    __shared__ __attribute__((aligned(16))) __bf16 s_eg[PK ? 2 * DK : 8];  // e^{g_L}, fp32 bits

    constexpr int NT = DV / TV;
    int shd, tile;
    scan_unit(b, NT, shd, tile);
    if (shd >= a.n_seq * a.H) return false;
    const int unit = shd / a.H, h = shd % a.H;
    // one segment and no chunk records: every sequence is the one-chunk
    // kernel's (a sequence past one chunk has records in the only segment)
    if (a.fuse1 && a.nseg == 1 && static_cast<const int32_t *>(a.ws)[a.n_seq] == 0) return false;
    // this workgroup's sequences: one, or (branch calls) a group of branches
    // of one parent, which run one after another from one load of the
    // parent's state while no branch changes it
    int s_first = unit, s_last = unit + 1;
    if constexpr (GRP) {
        if (unit >= a.groups[0]) return false;
        s_first = a.groups[1 + unit];
        s_last = a.groups[2 + unit];
    }
    const int H = a.H;
    const int CC = H * (2 * DK + DV);
    const int j0 = tile * TV;
    const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
    const int32_t *chunk_start = static_cast<const int32_t *>(a.ws);
    const WsLayout wl = ws_layout(a.n_tokens, a.n_seq, H, DK, DV, PK, a.nseg);
    // a prefill in segments carries each sequence's state through the
    // workspace from one segment to the next
    const bool carry_in = a.seg > 0, carry_out = a.seg + 1 < a.nseg;
    float *const carry = reinterpret_cast<float *>(static_cast<char *>(a.ws) + wl.carry_off);
    // the current sequence (set per sequence below; the helpers read them):
    // chunks c_beg .. c_end - 1 of it in this segment, chunk c's record at
    // cs0 + c
    int s = s_first, src = 0, cs0 = 0, nchunks = 0, c_beg = 0, c_end = 0;
    SeqSpan sp{0, 0};
    const TI *win = nullptr;

    const bool conv = a.conv_w != nullptr;
    if (conv) stage_taps(a.conv_w, 2 * H * DK + h * DV + j0, TV, s_wv);

    const bool want_o = a.o != nullptr;
    const int kmax = (w * RB + RB - 1) / 32;  // T', P lower triangular: k-steps to use
    // the v base pointer as a local that every V load indexes directly
    const TI *const vs = static_cast<const TI *>(a.v);
    const int cwin_v = 2 * H * DK + h * DV;

    // The state tiles of this wave: tile m is ft = w + 4 m, value sub-tile
    // t = ft % NVT, keys dt*16 .. dt*16 + 15 (dt = ft / NVT); the lane holds
    // the keys dt*16 + (l/16)*4 + i (i < 4) of the internal value column
    // t*16 + l%16 (the output layout of the update Sig = K^T W, rows = keys).
    float mst[NEG][4];
    // the split planes of the state from the registers: a lane's 4 keys are
    // consecutive in a plane row (one 8-byte store per plane and tile)
    auto put_split = [&](int lane) {
#pragma unroll
        for (int m = 0; m < NEG; ++m) {
            const int ft = w + m * kWaves, t = ft % NVT, key0 = (ft / NVT) * 16 + (lane / 16) * 4;
            put4<F>(s_Sh, s_Sl, st_off<DK>(t * 16 + lane % 16, key0),
                    f32x4v{mst[m][0], mst[m][1], mst[m][2], mst[m][3]});
        }
    };
    // the state tile [DK][TV] of this workgroup into a [DK][DV] state at
    // dst, through the staging buffer (4 consecutive tile columns per
    // 16-byte store); called between barriers, so the plane buffer is free
    auto put_state = [&](float *dst) {
        const int lane = __builtin_amdgcn_update_dpp(0, tid % kWave, 0xE4, 0xf, 0xf, false);
#pragma unroll
        for (int m = 0; m < NEG; ++m) {
            const int ft = w + m * kWaves, t = ft % NVT, key0 = (ft / NVT) * 16 + (lane / 16) * 4;
            const int col = vcol(t * 16 + lane % 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) s_stage[(key0 + i) * TV + col] = mst[m][i];
        }
        __syncthreads();
        for (int idx = tid; idx < DK * TV / 4; idx += kThreads) {
            const int d = idx / (TV / 4), j = 4 * (idx % (TV / 4));
            *reinterpret_cast<float4 *>(dst + (size_t)d * DV + j0 + j) =
                *reinterpret_cast<const float4 *>(s_stage + d * TV + j);
        }
        __syncthreads();
    };
    auto put_window = [&](TI *wo, int end) { write_window<DK, DV, TI>(a, h, sp.start, win, wo, end); };
    // checkpoint k of the sequence: the state and window after
    // (k + 1) * ckpt_every chunks; `ckpt_at(c)` says whether the boundary
    // before chunk c is one (k < ckpt_cap)
    auto ckpt_at = [&](int c) {
        return a.ckpt_state && a.ckpt_every > 0 && c > 0 && c % a.ckpt_every == 0 &&
               c / a.ckpt_every - 1 < a.ckpt_cap;
    };
    auto put_checkpoint = [&](int c) {
        const size_t k = (size_t)s * a.ckpt_cap + (c / a.ckpt_every - 1);
        put_state(a.ckpt_state + (k * H + h) * DK * DV);
        if (a.ckpt_window && tile == 0) put_window(static_cast<TI *>(a.ckpt_window) + k * 3 * CC, c * C);
    };

    auto record = [&](int c) {
        return reinterpret_cast<const __bf16 *>(static_cast<const char *>(a.ws) + wl.rec_off) +
               ((size_t)(cs0 + c) * H + h) * wl.rec_elems;
    };
    // loads only: every address is clamped in bounds, nothing is consumed here
    // Addresses: a wave-uniform base per chunk plus an unsigned 32-bit lane
    // offset (the scalar-base form of the global loads, no 64-bit lane math).
    auto load_regs = [&](int c, ChunkRegs<KS, NVT, TI> &r) {
        const __bf16 *rec = record(c);
        const int p0 = c * C, L = min(C, sp.len - p0);
        // lane-derived offsets formed at each call from an opaque copy of the
        // lane (hoisted, they would stay live across the sequence loop)
        const int lane = __builtin_amdgcn_update_dpp(0, tid % kWave, 0xE4, 0xf, 0xf, false);
        const int r0v = w * RB + (lane / 16) * 4;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const unsigned ob = 2u * frag_off(KS, w, ks, lane);  // bytes
            // Q and P unconditionally (a branch here would keep their
            // addresses out of the scalar-base form)
            r.ka[ks] = read_frag<F>(byte_at(rec + RL.khi, ob), byte_at(rec + RL.klo, ob));
            r.qa[ks] = read_frag<F>(byte_at(rec + RL.qhi, ob), byte_at(rec + RL.qlo, ob));
        }
#pragma unroll
        for (int kq = 0; kq < 2; ++kq)
            if (kq <= kmax) {
                const unsigned ob = 2u * tri_off(w, kq, lane);
                r.ta[kq] = read_frag<F>(byte_at(rec + RL.thi, ob), byte_at(rec + RL.tlo, ob));
                r.pa[kq] = read_frag<F>(byte_at(rec + RL.phi, ob), byte_at(rec + RL.plo, ob));
            }
        if (c == 0) {  // rows before the sequence come from the incoming window
            const int j = j0 + 2 * (lane % 16);  // columns j, j + 1 (even: pair-aligned)
#pragma unroll
            for (int q = 0; q < 7; ++q) {
                const int p = p0 + r0v - 3 + q;  // >= -3
                const TI *ptr = (p < 0 && win) ? win + (size_t)(3 + p) * CC + cwin_v + j
                                               : vs + (size_t)(sp.start + min(max(p, 0), p0 + L - 1)) *
                                                          H * DV + (size_t)h * DV + j;
                r.vraw[q] = *reinterpret_cast<const typename VPair<TI>::type *>(ptr);
            }
        } else {  // rows p0 - 3 .. p0 + L - 1 all lie inside the sequence
            const TI *base = vs + ((size_t)(sp.start + p0 - 3) * H + h) * DV + j0;
            const unsigned stride = (unsigned)H * DV;
#pragma unroll
            for (int q = 0; q < 7; ++q) {
                const unsigned row = (unsigned)min(r0v + q, L + 2);
                r.vraw[q] = *reinterpret_cast<const typename VPair<TI>::type *>(
                    byte_at(base, (row * stride + 2u * (lane % 16)) * (unsigned)sizeof(TI)));
            }
        }
        if constexpr (PK) {
            r.gam = f32x4v{1.f, 1.f, 1.f, 1.f};
            r.gu = r.gam;
            r.gaml = 1.f;
        } else {
            const float *fac = reinterpret_cast<const float *>(rec + RL.fac);
            r.gam = *reinterpret_cast<const f32x4v *>(byte_at(fac, 4u * r0v));
            r.gu = *reinterpret_cast<const f32x4v *>(byte_at(fac + C, 4u * r0v));
            r.gaml = fac[2 * C];
        }
    };
    // per key: K~^T hi / lo planes of chunk c into LDS (direct-to-LDS, 16 B
    // per lane; the LDS position of a lane's bytes is fixed, so the swizzle
    // is applied by choosing which global chunk each lane fetches)
    auto load_kt = [&](int c) {
        const __bf16 *rec = record(c);
        constexpr int PER_WAVE = DK * C * 2 / 16 / kThreads;  // 16-byte pieces per lane, per plane
#pragma unroll
        for (int q = 0; q < PER_WAVE; ++q) {
            const int piece = (q * kWaves + w) * kWave + lane;  // 16-byte piece of the plane
            const int r = piece / 8, chl = piece % 8;           // LDS row, LDS chunk slot
            const int chg = chl ^ (r & 7);                      // global chunk stored there
            const int lds0 = (q * kWaves + w) * kWave * 8;      // wave-uniform LDS element offset
            lds_dma16(rec + RL.kthi + r * C + chg * 8, s_Kh + lds0);
            lds_dma16(rec + RL.ktlo + r * C + chg * 8, s_Kl + lds0);
        }
        if constexpr (PK)  // DK floats: one 16-byte piece per lane of wave 0
            if (w == 0 && lane < DK / 4) lds_dma16(rec + RL.fac + lane * 8, s_eg);
    };

    bool have = false;  // the registers and planes hold the parent's state
    for (; s < s_last; ++s) {
    sp = seq_span(a.cu, s, a.n_tokens);
    if (a.fuse1 && sp.len <= C) continue;  // the one-chunk kernel's
    src = a.parent ? a.parent[s] : s;
    ChunkRegs<KS, NVT, TI> nxt;
    if (!(src >= 0 && src < a.n_parent)) {  // invalid parent: NaN outputs, nothing else
        if (a.o)
            for (int idx = tid; idx < sp.len * TV; idx += kThreads)
                static_cast<TO *>(a.o)[((size_t)(sp.start + idx / TV) * H + h) * DV + j0 + idx % TV] =
                    from_f32<TO>(quiet_nan());
        if (a.state_out)
            for (int idx = tid; idx < DK * TV; idx += kThreads)
                a.state_out[(((size_t)s * H + h) * DK + idx / TV) * DV + j0 + idx % TV] = quiet_nan();
        continue;
    }
    win = a.win_in ? static_cast<const TI *>(a.win_in) + (size_t)src * 3 * CC : nullptr;
    // read once: inside the loop the compiler could not prove these unchanged
    // across the o stores and would reload them behind a full wait
    c_beg = chunk_start[wl.win_off + s];
    nchunks = chunk_start[s + 1] - chunk_start[s];  // <= ceil(len / C)
    c_end = c_beg + nchunks;
    cs0 = chunk_start[s] - c_beg;

    // the first chunk's operands are requested before the incoming state
    // tile, so the two round trips overlap (a one-chunk branch pays one)
    if (nchunks > 0) load_regs(c_beg, nxt);
    if (!have) {
        const int lane = __builtin_amdgcn_update_dpp(0, tid % kWave, 0xE4, 0xf, 0xf, false);
        // the incoming state: the carried one past the first segment
        const float *sin = carry_in ? carry + (size_t)s * H * DK * DV
                                    : (a.state_in ? a.state_in + (size_t)src * H * DK * DV : nullptr);
#pragma unroll
        for (int m = 0; m < NEG; ++m) {
            const int ft = w + m * kWaves, t = ft % NVT, key0 = (ft / NVT) * 16 + (lane / 16) * 4;
            const int col = j0 + vcol(t * 16 + lane % 16);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                mst[m][i] = sin ? sin[((size_t)h * DK + key0 + i) * DV + col] : 0.f;
        }
        put_split(lane);
        __syncthreads();
        have = true;
    }
    // the state after the last chunk is needed only as an output (a branch
    // call may not ask for it): the last step then skips the state update
    const bool need_final = a.state_out != nullptr || CK || carry_out;
    for (int c = c_beg; c < c_end; ++c) {
        const bool upd = need_final || c + 1 < c_end;
        if constexpr (CK)
            if (ckpt_at(c)) put_checkpoint(c);  // the state after c chunks
        const ChunkSrc<TI> cs{sp.start, c * C, min(C, sp.len - c * C), win};
        const ChunkRegs<KS, NVT, TI> cur = nxt;
        // The step's lane-derived LDS offsets are formed inside the step from
        // an opaque copy of the lane index (an identity DPP move): hoisted
        // out of the loop, the compiler keeps them live and spills.
        const int lane = __builtin_amdgcn_update_dpp(0, tid % kWave, 0xE4, 0xf, 0xf, false);
        const int acol = (lane / 16) * 8, r0v = w * RB + (lane / 16) * 4;
        if (upd) {
            if constexpr (PK) {
                load_kt(c);
            } else {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    put_kt(cur.ka[ks], ks * 32 + acol, w * RB + lane % 16, s_Kh, s_Kl);
            }
        }

        // gamma_r = exp(g_r) of this lane's rows, from the chunk record (the
        // prep kernel's running sums; rows >= L add nothing)
        const f32x4v gam = cur.gam;

        // conv'd V entries of this lane (C/D layout), from the raw rows; a
        // full chunk past the first has every row inside the sequence, so it
        // takes the rows without validity masks
        float vf[NVT][4];
        const auto conv_v = [&](auto masked) {
#pragma unroll
            for (int t = 0; t < NVT; ++t) {
                const int jt = vcol(t * 16 + lane % 16);  // the tile column, for its taps
                float xr[7];
#pragma unroll
                for (int q = 0; q < 7; ++q) {
                    xr[q] = VPair<TI>::get(cur.vraw[q], t);
                    if constexpr (decltype(masked)::value) {
                        const int row = r0v - 3 + q, p = cs.p0 + row;
                        const bool ok = (conv || q >= 3) && ((row < cs.L && p >= 0) || (p < 0 && win));
                        xr[q] = ok ? xr[q] : 0.f;
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float y = xr[i + 3];
                    if (conv) {
                        y = 0.f;
#pragma unroll
                        for (int r = 0; r < 4; ++r) y = fmaf(s_wv[jt * 4 + r], xr[i + r], y);
                    }
                    if constexpr (decltype(masked)::value) y = r0v + i < cs.L ? y : 0.f;
                    vf[t][i] = y;
                }
            }
        };
        if (cs.p0 > 0 && cs.L == C) conv_v(std::false_type{});
        else conv_v(std::true_type{});

        // K Sig0 and Q Sig0 share the split Sig^T fragments;
        // R = V - diag(gamma) K Sig0 goes to LDS, Q Sig0 stays in registers
        f32x4v acc_o[NVT];
#pragma unroll
        for (int t = 0; t < NVT; ++t) {
            f32x4v acc = {0.f, 0.f, 0.f, 0.f};
            acc_o[t] = acc;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int so = st_off<DK>(t * 16 + lane % 16, ks * 32 + acol);
                const Frag<F> bs = read_frag<F>(s_Sh + so, s_Sl + so);
                acc = mma(cur.ka[ks], bs, acc);
                if (want_o) acc_o[t] = mma(cur.qa[ks], bs, acc_o[t]);
            }
            // the lane's 4 rows are consecutive in the R^T planes
            f32x4v rv;
#pragma unroll
            for (int i = 0; i < 4; ++i) rv[i] = vf[t][i] - gam[i] * acc[i];
            const int ro = (t * 16 + lane % 16) * CB + r0v;
            put4<F>(s_Rh, s_Rl, ro, rv);
        }
        // Per key, this wave's direct-to-LDS copies of K~^T are its only
        // vector memory operations in flight here: finish them before this
        // barrier (a workgroup fence would wait for them here anyway), so the
        // whole plane is visible to every wave after it and the state update
        // needs no barrier of its own. Sig^T is last read above (K Sig0,
        // Q Sig0), so it may be rewritten by the state update after the next
        // barrier.
        if constexpr (PK) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();

        // U = T' R
#pragma unroll
        for (int t = 0; t < NVT; ++t) {
            f32x4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kq = 0; kq < 2; ++kq)
                if (kq <= kmax) {
                    const int off = (t * 16 + lane % 16) * CB + kq * 32 + acol;
                    acc = mma(cur.ta[kq], read_frag<F>(s_Rh + off, s_Rl + off), acc);
                }
            const int uo = (t * 16 + lane % 16) * CB + r0v;
            put4<F>(s_Uh, s_Ul, uo, acc);
            if (!PK && upd) {  // W = diag(e^{g_L - g}) U for the state update
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] *= cur.gu[i];
                put4<F>(s_Wh, s_Wl, uo, acc);
            }
        }
        __syncthreads();

        // O = diag(gamma) Q Sig0 + P U (stored below, after the next chunk's
        // operands are requested)
        if (want_o) {
#pragma unroll
            for (int t = 0; t < NVT; ++t) {
#pragma unroll
                for (int i = 0; i < 4; ++i) acc_o[t][i] *= gam[i];
#pragma unroll
                for (int kq = 0; kq < 2; ++kq)
                    if (kq <= kmax) {
                        const int off = (t * 16 + lane % 16) * CB + kq * 32 + acol;
                        acc_o[t] = mma(cur.pa[kq], read_frag<F>(s_Uh + off, s_Ul + off), acc_o[t]);
                    }
            }
        }

        if (c + 1 < c_end) load_regs(c + 1, nxt);  // prefetch the next step
        if (want_o) {
            TO *const obase = static_cast<TO *>(a.o) + ((size_t)(cs.seq0 + cs.p0) * H + h) * DV + j0;
            const unsigned ostride = (unsigned)H * DV;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = r0v + i;
                if (r < cs.L)
                    store_pair(byte_at(obase, ((unsigned)r * ostride + 2u * (lane % 16)) *
                                                  (unsigned)sizeof(TO)),
                               acc_o[0][i], acc_o[1][i]);
            }
        }

        if (!upd) break;  // the last chunk, no final state wanted
        // Sig <- gamma_L Sig + K~^T U = gamma_L Sig + K^T W (scalar decay;
        // per key: diag(e^{g_L}) Sig + K~^T U)   (tiles: 16 keys x value
        // sub-tile; A = the key rows of K^T, B = the value rows of W^T)
        const float gamL = cur.gaml;
#pragma unroll
        for (int m = 0; m < NEG; ++m) {
            const int ft = w + m * kWaves;
            const int t = ft % NVT, dt = ft / NVT;
            // per key: e^{g_L} of this lane's keys dt*16 + (l/16)*4 + i
            f32x4v dec = {gamL, gamL, gamL, gamL};
            if constexpr (PK)
                dec = *reinterpret_cast<const f32x4v *>(reinterpret_cast<const float *>(s_eg) + dt * 16 +
                                                        (lane / 16) * 4);
            f32x4v acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = dec[i] * mst[m][i];
#pragma unroll
            for (int kq = 0; kq < 2; ++kq) {
                const int ou = (t * 16 + lane % 16) * CB + kq * 32 + acol;
                const int ok = PK ? kt_swz(dt * 16 + lane % 16, kq * 4 + lane / 16)
                                  : kt_off(dt * 16 + lane % 16, kq * 32 + acol);
                acc = PK ? mma(read_frag<F>(s_Kh + ok, s_Kl + ok), read_frag<F>(s_Uh + ou, s_Ul + ou), acc)
                         : mma(read_frag<F>(s_Kh + ok, s_Kl + ok), read_frag<F>(s_Wh + ou, s_Wl + ou), acc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) mst[m][i] = acc[i];
        }
        put_split(lane);
        __syncthreads();
    }
    if (carry_out) {
        put_state(carry + ((size_t)s * H + h) * DK * DV);
    } else {
        if (a.state_out) put_state(a.state_out + ((size_t)s * H + h) * DK * DV);
        if (a.win_out && tile == 0) put_window(static_cast<TI *>(a.win_out) + (size_t)s * 3 * CC, sp.len);
    }
    // a checkpoint at the end of the sequence (its length a multiple of the
    // checkpoint spacing)
    if constexpr (CK)
        if (ckpt_at(c_end) && c_end * C == sp.len) put_checkpoint(c_end);
    // a state update ran: the next branch of the group reloads the parent's
    if (nchunks > 1 || (need_final && nchunks > 0)) have = false;
    }
    return true;
}

// Branch groups (GRP): a grid of at most kScanResident workgroups (a
// multiple of 8), block b taking the units b, b + gridDim.x, ... (one XCD)
// while they have work, so that a branch call whose branches all take the
// one-chunk kernel, or that forms few groups, runs one round of
// workgroups. Otherwise one unit per workgroup.
template <int DK, int DV, typename TI, typename TO, bool PK, bool CK, bool GRP = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void scan_kernel(PrefillArgs a) {
    if constexpr (GRP) {
#pragma unroll 1
        for (int b = blockIdx.x; scan_body<DK, DV, TI, TO, PK, CK, GRP>(a, b); b += gridDim.x)
            __syncthreads();  // the LDS of one unit before the next
    } else {
        scan_body<DK, DV, TI, TO, PK, CK, GRP>(a, blockIdx.x);
    }
}

// ------------------------------------------------------------ one-chunk sequences
// Workgroup -> (sequence, head) of the one-chunk kernel: with a head count
// that is a multiple of 8, head h runs on XCD h mod 8 (block indices
// congruent mod 8) and consecutive sequences follow one another there, so
// the branches of one parent read its state tile through one L2.
__device__ __forceinline__ void one_chunk_unit(int b, int H, int &s, int &h) {
    if (H % 8 == 0) {
        const int hx = H / 8, k = b / 8;
        h = b % 8 + 8 * (k % hx);
        s = k / hx;
    } else {
        s = b / H;
        h = b % H;
    }
}

// A sequence of at most C tokens (a branch of the fork, typically) is one
// chunk: one workgroup per (sequence, head) runs the prep steps with their
// results kept on chip -- Q and K as A operands in registers, T' and P in
// LDS, then in registers -- and the chunk step against the incoming state
// for each value tile in turn. No chunk record goes through memory and
// nothing waits on a chain of chunk steps. The arithmetic is the prep's and
// the scan's in the same order, so the outputs are bit for bit those of the
// two-kernel path. ST: the sequence's final state is written (the state
// update runs; K^T is formed once in LDS).
// Per-key decay (VAR kKda / kRwkv6): the prep steps write the chunk record
// into the workspace slot of the (sequence, head) as the prep kernel would,
// and the workgroup reads its operands back from there (mostly from L2):
// Q^ and K^ into registers, with ST K~^T and e^{g_L} per key into LDS; the
// chunk step is the scan's per-key one (gamma = 1, the state decayed per
// key column).
// LDS: the prep's buffers, reused once T' and P are in registers (s_A: the
// split state planes; s_k: the R and U planes, or with ST the K^T planes),
// the value channels' conv taps, and with ST the R, U and W planes (per
// key: K~^T in the K buffer, then R and U in one pair of planes, U written
// over R behind a barrier, and e^{g_L} after them, behind K~^T where they
// fit (d_k <= 64), else in the prep's table buffer).
template <int DK, int DV, typename TI, typename TO, bool ST, int VAR = kScalar>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(ST || VAR != kScalar ? 2 : 3))) void one_chunk_kernel(
    PrefillArgs a) {
    constexpr bool PK = VAR != kScalar;
    constexpr bool RU1 = PK && ST;  // R and U share one pair of planes
    constexpr bool F = std::is_same<TI, float>::value;
    constexpr int KS = DK / 32;
    constexpr int CB = C + 8;            // padded row of the R^T / U^T / W^T planes
    constexpr int NVT = TV / 16;
    constexpr int NFT = NVT * (DK / 16);
    constexpr int NEG = NFT / kWaves;
    static_assert(NFT % kWaves == 0 && NVT == 2, "the scan's tiling");
    static_assert(2 * TV * DK * 2 <= kPrepAFloats * 4, "split state planes fit the prep's A buffer");
    static_assert(4 * TV * CB * 2 <= prep_sk_floats(DK) * 4, "R and U planes fit the prep's K buffer");
    static_assert(2 * DK * C * 2 <= prep_sk_floats(DK) * 4, "K^T planes fit the prep's K buffer");
    // per key with ST: the shared R / U planes and e^{g_L} after the K~^T
    // planes in the prep's K buffer where they fit, else in its table
    constexpr int kRUBytes = 2 * TV * CB * 2 + DK * 4;
    constexpr bool RU_IN_K = prep_sk_floats(DK) * 4 - 2 * DK * C * 2 >= kRUBytes;
    static_assert(!RU1 || RU_IN_K || kRUBytes <= (4 * kWaves + 10) * DK * 4,
                  "per key: R / U planes and e^{g_L} fit the prep's buffers");
    __shared__ __attribute__((aligned(16))) float s_wv[DV * 4];
    __shared__ __attribute__((aligned(16))) __bf16 s_pl_st[ST && !PK ? 6 * TV * CB : 8];

    if (blockIdx.x == gridDim.x - 1) {  // the extra workgroup: the first segment's plan
        const WsLayout wl = ws_layout(a.n_tokens, a.n_seq, a.H, DK, DV, PK, a.nseg);
        int32_t *const chunk_start = static_cast<int32_t *>(a.ws);
        plan_body(a.cu, a.n_seq, a.n_tokens, (long long)wl.max_chunks, chunk_start, a.parent,
                  a.group_size, const_cast<int32_t *>(a.groups), 0, a.nseg,
                  chunk_start + wl.win_off, a.fuse1);
        return;
    }
    int s, h;
    one_chunk_unit(blockIdx.x, a.H, s, h);
    if (s >= a.n_seq) return;
    const SeqSpan sp = seq_span(a.cu, s, a.n_tokens);
    if (!a.fuse1 || sp.len > C) return;  // the chunked kernels take it
    const int H = a.H, CC = H * (2 * DK + DV);
    const int tid = threadIdx.x;
    const int src = a.parent ? a.parent[s] : s;
    TO *const o = static_cast<TO *>(a.o);
    float *const st_out = ST ? a.state_out + ((size_t)s * H + h) * DK * DV : nullptr;
    if (!(src >= 0 && src < a.n_parent)) {  // invalid parent: NaN outputs, nothing else
        if (o)
            for (int idx = tid; idx < sp.len * DV; idx += kThreads)
                o[((size_t)(sp.start + idx / DV) * H + h) * DV + idx % DV] = from_f32<TO>(quiet_nan());
        if constexpr (ST)
            for (int idx = tid; idx < DK * DV; idx += kThreads) st_out[idx] = quiet_nan();
        return;
    }
    const TI *const win = a.win_in ? static_cast<const TI *>(a.win_in) + (size_t)src * 3 * CC : nullptr;
    const float *const sin = a.state_in ? a.state_in + ((size_t)src * H + h) * DK * DV : nullptr;
    if (a.win_out) write_window<DK, DV, TI>(a, h, sp.start, win, static_cast<TI *>(a.win_out) + (size_t)s * 3 * CC, sp.len);
    if (sp.len == 0) {  // no tokens: the final state is the incoming one
        if constexpr (ST)
            for (int idx = tid; idx < DK * DV; idx += kThreads) st_out[idx] = sin ? sin[idx] : 0.f;
        return;
    }
    const bool conv = a.conv_w != nullptr;
    if (conv) stage_taps(a.conv_w, 2 * H * DK + h * DV, DV, s_wv);  // visible after the prep's barriers

    PrepOut<DK, TI> po;
    po.s = s;
    po.h = h;
    prep_body<DK, TI, VAR, PK ? kPrepToSlot : kPrepOnChip>(a, &po);
    constexpr RecLayout RL = rec_layout(DK, PK);
    const __bf16 *const rec =
        PK ? reinterpret_cast<const __bf16 *>(static_cast<const char *>(a.ws) +
                                              ws_layout(a.n_tokens, a.n_seq, H, DK, DV, PK, a.nseg).rec_off) +
                 ((size_t)s * H + h) * RL.elems
           : nullptr;
    if constexpr (PK) __syncthreads();  // the record in the slot is complete

    const int lane = tid % kWave, w = tid / kWave;
    const int L = sp.len;
    const TI *const vs = static_cast<const TI *>(a.v);
    // A value tile's inputs, requested ahead of use (loads only): the
    // incoming state tile in this lane's update layout, and the raw V rows
    // r0v - 3 .. r0v + 3 of its column pair (rows before the sequence from
    // the incoming window). Addresses: wave-uniform bases plus unsigned
    // 32-bit lane offsets (the scalar-base form); offsets come from an
    // opaque copy of the lane.
    typedef typename VPair<TI>::type VRaw;
    const unsigned vstride = (unsigned)H * DV * (unsigned)sizeof(TI);  // one stream row of v
    const auto load_tile = [&](int j0, float (&m4)[NEG][4], VRaw (&vr)[7]) {
        const int lane = __builtin_amdgcn_update_dpp(0, tid % kWave, 0xE4, 0xf, 0xf, false);
        const int r0v = w * RB + (lane / 16) * 4;
        if (sin) {
            // tile m of the wave is keys 32 m further down (ft = w + 4 m, two
            // value sub-tiles): one lane offset, the rest in the uniform base
            static_assert(kWaves == 4 && NVT == 2, "key step of the wave's state tiles");
            const int key0 = (w / NVT) * 16 + (lane / 16) * 4;
            const unsigned off = 4u * (unsigned)(key0 * DV + j0 + vcol((w % NVT) * 16 + lane % 16));
#pragma unroll
            for (int m = 0; m < NEG; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) m4[m][i] = *byte_at(sin + (32 * m + i) * DV, off);
        } else {
#pragma unroll
            for (int m = 0; m < NEG; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) m4[m][i] = 0.f;
        }
        const TI *const vbase = vs + ((size_t)sp.start * H + h) * DV + j0;
        const unsigned col = 2u * (unsigned)(lane % 16) * (unsigned)sizeof(TI);
#pragma unroll
        for (int q = 0; q < 7; ++q) {
            const int p = r0v - 3 + q;
            vr[q] = *reinterpret_cast<const VRaw *>(byte_at(vbase, (unsigned)min(max(p, 0), L - 1) * vstride + col));
            if (q < 3 && win && p < 0)  // wave 0's first rows: the incoming window
                vr[q] = *reinterpret_cast<const VRaw *>(
                    win + (size_t)(3 + p) * CC + 2 * H * DK + h * DV + j0 + 2 * (lane % 16));
        }
    };
    float nm[NEG][4];
    VRaw nv[7];
    load_tile(0, nm, nv);
    const int kmax = (w * RB + RB - 1) / 32;  // T', P lower triangular: k-steps to use
    const int acol = (lane / 16) * 8;
    const int r0v = w * RB + (lane / 16) * 4;  // first of this lane's rows in the C/D layout
    // T' and P A operands of this wave's rows (the scan's record blocks)
    Frag<F> ta[2], pa[2];
    {
        const float *const s_P = po.lds_k, *const s_T = po.lds_k + C * (C + 1);
        const int row = w * RB + lane % 16;
#pragma unroll
        for (int kq = 0; kq < 2; ++kq)
            if (kq <= kmax) {
                float x[8], y[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    x[e] = s_T[row * (C + 1) + kq * 32 + acol + e];
                    y[e] = s_P[row * (C + 1) + kq * 32 + acol + e];
                }
                ta[kq] = frag<F>(x);
                pa[kq] = frag<F>(y);
            }
    }
    // the row factors gamma_r, e^{g_L - g_r} of this lane's rows, gamma_L
    // (per key: 1, the decay sits in the operands and e^{g_L})
    f32x4v gam = {1.f, 1.f, 1.f, 1.f}, gu = gam;
    float gamL = 1.f;
    if constexpr (!PK) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float gr = __shfl(po.g, r0v + i, kWave);
            gam[i] = expf(gr);
            gu[i] = expf(po.gL - gr);
        }
        gamL = expf(po.gL);
    } else {  // Q^, K^ from the record
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int off = frag_off(KS, w, ks, lane);
            po.ka[ks] = read_frag<F>(rec + RL.khi + off, rec + RL.klo + off);
            po.qa[ks] = read_frag<F>(rec + RL.qhi + off, rec + RL.qlo + off);
        }
    }
    __syncthreads();  // T' and P are read: the prep's LDS is free

    __bf16 *const s_Sh = reinterpret_cast<__bf16 *>(po.lds_a), *const s_Sl = s_Sh + TV * DK;
    __bf16 *const s_pl = RU1 ? (RU_IN_K ? reinterpret_cast<__bf16 *>(po.lds_k) + 2 * DK * C
                                        : reinterpret_cast<__bf16 *>(po.lds_tab))
                             : ST ? s_pl_st : reinterpret_cast<__bf16 *>(po.lds_k);
    __bf16 *const s_Rh = s_pl, *const s_Rl = s_pl + TV * CB;
    __bf16 *const s_Uh = RU1 ? s_Rh : s_pl + 2 * TV * CB, *const s_Ul = RU1 ? s_Rl : s_pl + 3 * TV * CB;
    __bf16 *const s_Wh = s_pl + 4 * TV * CB, *const s_Wl = s_pl + 5 * TV * CB;  // ST, scalar decay
    __bf16 *const s_Kh = reinterpret_cast<__bf16 *>(po.lds_k), *const s_Kl = s_Kh + DK * C;  // ST
    float *const s_eg = reinterpret_cast<float *>(s_pl + 2 * TV * CB);  // ST, per key: e^{g_L}
    if constexpr (ST) {
        if constexpr (PK) {
            // K~^T planes (swizzled rows, as the scan stages them) and e^{g_L}
            // from the record by direct-to-LDS copies, finished before the
            // first tile's barrier
            constexpr int PER_WAVE = DK * C * 2 / 16 / kThreads;
#pragma unroll
            for (int q = 0; q < PER_WAVE; ++q) {
                const int piece = (q * kWaves + w) * kWave + lane;
                const int r = piece / 8, chl = piece % 8, chg = chl ^ (r & 7);
                const int lds0 = (q * kWaves + w) * kWave * 8;
                lds_dma16(rec + RL.kthi + r * C + chg * 8, s_Kh + lds0);
                lds_dma16(rec + RL.ktlo + r * C + chg * 8, s_Kl + lds0);
            }
            if (w == 0 && lane < DK / 4)
                lds_dma16(rec + RL.fac + lane * 8, reinterpret_cast<__bf16 *>(s_eg));
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) put_kt(po.ka[ks], ks * 32 + acol, w * RB + lane % 16, s_Kh, s_Kl);
        }
    }

    const bool want_o = o != nullptr;
#pragma unroll 1
    for (int j0 = 0; j0 < DV; j0 += TV) {
        // lane-derived offsets formed per tile from an opaque copy of the
        // lane (hoisted out of the loop, they would stay live and spill)
        const int lane = __builtin_amdgcn_update_dpp(0, tid % kWave, 0xE4, 0xf, 0xf, false);
        const int acol = (lane / 16) * 8, r0v = w * RB + (lane / 16) * 4;
        // this tile's inputs (requested during the previous tile): the
        // state tile split into the planes (kept with ST for the update),
        // the V rows convolved
        float mst[NEG][4];
#pragma unroll
        for (int m = 0; m < NEG; ++m) {
            const int ft = w + m * kWaves, t = ft % NVT, key0 = (ft / NVT) * 16 + (lane / 16) * 4;
#pragma unroll
            for (int i = 0; i < 4; ++i) mst[m][i] = nm[m][i];
            put4<F>(s_Sh, s_Sl, st_off<DK>(t * 16 + lane % 16, key0),
                    f32x4v{mst[m][0], mst[m][1], mst[m][2], mst[m][3]});
        }
        float vf[NVT][4];
#pragma unroll
        for (int t = 0; t < NVT; ++t) {
            const int jt = j0 + vcol(t * 16 + lane % 16);
            float xr[7];
#pragma unroll
            for (int q = 0; q < 7; ++q) {
                // rows before the sequence: the incoming window's, else
                // zero; rows past its end feed only rows zeroed below
                const bool ok = q >= 3 || (conv && (r0v - 3 + q >= 0 || win));
                xr[q] = ok ? VPair<TI>::get(nv[q], t) : 0.f;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float y = xr[i + 3];
                if (conv) {
                    y = 0.f;
#pragma unroll
                    for (int r = 0; r < 4; ++r) y = fmaf(s_wv[jt * 4 + r], xr[i + r], y);
                }
                vf[t][i] = r0v + i < L ? y : 0.f;
            }
        }
        __syncthreads();  // the state planes

        // R = V - diag(gamma) K Sig0 -> planes; Q Sig0 in registers
        f32x4v acc_o[NVT];
#pragma unroll
        for (int t = 0; t < NVT; ++t) {
            f32x4v acc = {0.f, 0.f, 0.f, 0.f};
            acc_o[t] = acc;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int so = st_off<DK>(t * 16 + lane % 16, ks * 32 + acol);
                const Frag<F> bs = read_frag<F>(s_Sh + so, s_Sl + so);
                acc = mma(po.ka[ks], bs, acc);
                if (want_o) acc_o[t] = mma(po.qa[ks], bs, acc_o[t]);
            }
            f32x4v rv;
#pragma unroll
            for (int i = 0; i < 4; ++i) rv[i] = vf[t][i] - gam[i] * acc[i];
            put4<F>(s_Rh, s_Rl, (t * 16 + lane % 16) * CB + r0v, rv);
        }
        if (j0 + TV < DV) load_tile(j0 + TV, nm, nv);  // the next tile's inputs
        __syncthreads();

        // U = T' R (and W = diag(e^{g_L - g}) U for the scalar-decay update)
        f32x4v uacc[NVT];
#pragma unroll
        for (int t = 0; t < NVT; ++t) {
            f32x4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kq = 0; kq < 2; ++kq)
                if (kq <= kmax) {
                    const int off = (t * 16 + lane % 16) * CB + kq * 32 + acol;
                    acc = mma(ta[kq], read_frag<F>(s_Rh + off, s_Rl + off), acc);
                }
            uacc[t] = acc;
        }
        if constexpr (RU1) __syncthreads();  // R is read: U goes over it
#pragma unroll
        for (int t = 0; t < NVT; ++t) {
            f32x4v acc = uacc[t];
            const int uo = (t * 16 + lane % 16) * CB + r0v;
            put4<F>(s_Uh, s_Ul, uo, acc);
            if constexpr (ST && !PK) {
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] *= gu[i];
                put4<F>(s_Wh, s_Wl, uo, acc);
            }
        }
        __syncthreads();

        // O = diag(gamma) Q Sig0 + P U
        if (want_o) {
#pragma unroll
            for (int t = 0; t < NVT; ++t) {
#pragma unroll
                for (int i = 0; i < 4; ++i) acc_o[t][i] *= gam[i];
#pragma unroll
                for (int kq = 0; kq < 2; ++kq)
                    if (kq <= kmax) {
                        const int off = (t * 16 + lane % 16) * CB + kq * 32 + acol;
                        acc_o[t] = mma(pa[kq], read_frag<F>(s_Uh + off, s_Ul + off), acc_o[t]);
                    }
            }
            TO *const obase = o + ((size_t)sp.start * H + h) * DV + j0;
            const unsigned ostride = (unsigned)H * DV;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = r0v + i;
                if (r < L)
                    store_pair(byte_at(obase, ((unsigned)r * ostride + 2u * (lane % 16)) * (unsigned)sizeof(TO)),
                               acc_o[0][i], acc_o[1][i]);
            }
        }

        if constexpr (ST) {
            // Sig <- gamma_L Sig + K^T W (per key: diag(e^{g_L}) Sig +
            // K~^T U), each lane's 4 keys of its value column straight out
            // (the next tile rewrites no buffer this reads before its own
            // barriers)
#pragma unroll
            for (int m = 0; m < NEG; ++m) {
                const int ft = w + m * kWaves, t = ft % NVT, dt = ft / NVT;
                f32x4v dec = {gamL, gamL, gamL, gamL};
                if constexpr (PK) dec = *reinterpret_cast<const f32x4v *>(s_eg + dt * 16 + (lane / 16) * 4);
                f32x4v acc;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = dec[i] * mst[m][i];
#pragma unroll
                for (int kq = 0; kq < 2; ++kq) {
                    const int ou = (t * 16 + lane % 16) * CB + kq * 32 + acol;
                    if constexpr (PK) {
                        const int ok = kt_swz(dt * 16 + lane % 16, kq * 4 + lane / 16);
                        acc = mma(read_frag<F>(s_Kh + ok, s_Kl + ok), read_frag<F>(s_Uh + ou, s_Ul + ou), acc);
                    } else {
                        const int ok = kt_off(dt * 16 + lane % 16, kq * 32 + acol);
                        acc = mma(read_frag<F>(s_Kh + ok, s_Kl + ok), read_frag<F>(s_Wh + ou, s_Wl + ou), acc);
                    }
                }
                const unsigned off = 4u * (unsigned)((dt * 16 + (lane / 16) * 4) * DV + j0 + vcol(t * 16 + lane % 16));
#pragma unroll
                for (int i = 0; i < 4; ++i) *byte_at(st_out + i * DV, off) = acc[i];
            }
        }
    }
}

template <int DK, int DV, typename TI, typename TO>
hipError_t launch_typed(const PrefillArgs &a0, hipStream_t stream) {
    auto prep = [&](auto vtag) {
        constexpr int VAR = decltype(vtag)::value;
        if constexpr (VAR == kScalar) return prep_kernel<DK, TI>;
        else return prep_kernel_pk<DK, TI, VAR>;
    };
    if (a0.n_seq == 0) return hipSuccess;
    const bool pk = a0.variant != kScalar;
    const int nseg = prefill_segments(a0.n_tokens, a0.n_seq, a0.H, DK, pk);
    const WsLayout wl = ws_layout(a0.n_tokens, a0.n_seq, a0.H, DK, DV, pk, nseg);
    int32_t *chunk_start = static_cast<int32_t *>(a0.ws);
    // Branch calls in one segment: groups of up to G consecutive branches
    // of one parent per scan workgroup, G chosen so that about two
    // workgroups per compute unit have work (fewer, longer workgroups
    // amortise the parent-state load); the plan kernel forms them.
    PrefillArgs a = a0;
    a.nseg = nseg;
    int G = 1;
    if (a.parent && nseg == 1) {
        const long long units = (long long)a.H * (DV / TV);
        const long long target = std::max(1LL, (kScanResident + units - 1) / units);
        G = (int)std::max(1LL, ((long long)a.n_seq + target - 1) / target);
        if (G > 1) a.groups = chunk_start + wl.grp_off;
    }
    const size_t n_sh = (size_t)a.n_seq * a.H;
    const size_t sh_pad = (n_sh + 7) / 8 * 8;  // see scan_unit
    const bool ck = a.ckpt_state != nullptr && a.ckpt_every > 0 && a.ckpt_cap > 0;
    const dim3 scan_grid((unsigned)(sh_pad * (DV / TV)));
    const dim3 grp_grid((unsigned)std::min((long long)(sh_pad * (DV / TV)), kScanResident));
    // Sequences of at most one chunk (calls without checkpoints) run in
    // the one-chunk kernel; the plan gives them no records and the scan
    // skips them. GDN_PREFILL_ONE_CHUNK=0 sends them through the chunked
    // kernels instead (the same results bit for bit; for tests).
    const char *oc = std::getenv("GDN_PREFILL_ONE_CHUNK");
    a.fuse1 = !ck && !(oc && oc[0] == '0');
    a.group_size = G;
    if (a.fuse1) {  // with one more workgroup: the first segment's plan
        const dim3 g1((unsigned)(n_sh + 1));
        const auto go = [&](auto vtag) {
            constexpr int VAR = decltype(vtag)::value;
            if (a.state_out)
                hipLaunchKernelGGL((one_chunk_kernel<DK, DV, TI, TO, true, VAR>), g1, dim3(kThreads), 0,
                                   stream, a);
            else
                hipLaunchKernelGGL((one_chunk_kernel<DK, DV, TI, TO, false, VAR>), g1, dim3(kThreads), 0,
                                   stream, a);
        };
        if (a.variant == kKda) go(std::integral_constant<int, kKda>{});
        else if (a.variant == kRwkv6) go(std::integral_constant<int, kRwkv6>{});
        else go(std::integral_constant<int, kScalar>{});
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    for (int seg = 0; seg < nseg; ++seg) {
        a.seg = seg;
        hipError_t e = hipSuccess;
        if (seg > 0 || !a.fuse1) {
            hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kThreads), 0, stream, a.cu, a.n_seq,
                               a.n_tokens, (long long)wl.max_chunks, chunk_start, a.parent, G,
                               const_cast<int32_t *>(a.groups), seg, nseg, chunk_start + wl.win_off,
                               a.fuse1);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        if (wl.max_chunks > 0) {
            const dim3 grid((unsigned)wl.max_chunks, a.H);
            if (a.variant == kKda)
                hipLaunchKernelGGL(prep(std::integral_constant<int, kKda>{}), grid, dim3(kThreads),
                                   0, stream, a);
            else if (a.variant == kRwkv6)
                hipLaunchKernelGGL(prep(std::integral_constant<int, kRwkv6>{}), grid,
                                   dim3(kThreads), 0, stream, a);
            else
                hipLaunchKernelGGL(prep(std::integral_constant<int, kScalar>{}), grid,
                                   dim3(kThreads), 0, stream, a);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        if (a.groups) {  // branch calls never take checkpoints
            if (pk)
                hipLaunchKernelGGL((scan_kernel<DK, DV, TI, TO, true, false, true>), grp_grid,
                                   dim3(kThreads), 0, stream, a);
            else
                hipLaunchKernelGGL((scan_kernel<DK, DV, TI, TO, false, false, true>), grp_grid,
                                   dim3(kThreads), 0, stream, a);
        } else if (ck) {
            if (pk)
                hipLaunchKernelGGL((scan_kernel<DK, DV, TI, TO, true, true>), scan_grid,
                                   dim3(kThreads), 0, stream, a);
            else
                hipLaunchKernelGGL((scan_kernel<DK, DV, TI, TO, false, true>), scan_grid,
                                   dim3(kThreads), 0, stream, a);
        } else {
            if (pk)
                hipLaunchKernelGGL((scan_kernel<DK, DV, TI, TO, true, false>), scan_grid,
                                   dim3(kThreads), 0, stream, a);
            else
                hipLaunchKernelGGL((scan_kernel<DK, DV, TI, TO, false, false>), scan_grid,
                                   dim3(kThreads), 0, stream, a);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// every value width, io and output type for one key width (one translation
// unit per key width, so the instances compile in parallel)
template <int DK>
hipError_t launch_prefill_dk(int dv, int io, int out, const PrefillArgs &a, hipStream_t stream) {
    auto go = [&](auto vtag) -> hipError_t {
        constexpr int DV = decltype(vtag)::value;
        if (io == kBF16) {
            if (out == kBF16) return launch_typed<DK, DV, bf16, bf16>(a, stream);
            return launch_typed<DK, DV, bf16, float>(a, stream);
        }
        if (out == kBF16) return launch_typed<DK, DV, float, bf16>(a, stream);
        return launch_typed<DK, DV, float, float>(a, stream);
    };
    switch (dv) {
        case 32: return go(std::integral_constant<int, 32>{});
        case 64: return go(std::integral_constant<int, 64>{});
        default: return go(std::integral_constant<int, 128>{});
    }
}

}  // namespace
}  // namespace gdn
