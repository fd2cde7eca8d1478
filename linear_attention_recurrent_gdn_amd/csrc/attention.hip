// attention.hip -- ForkAttention: softmax attention over a flat token stream
// in which every token reads only its own request's shared trunk and the
// current and earlier tokens of its own branch.
//
// Source: "같은 맥락에서 여러 판단을 빠르게 처리하는 Flide" (yozm.zip summary
// of the Flide paper), section "연구방법을 단계별로", method step 1 (tokens of
// all requests and questions in one flat stream, membership as GPU metadata,
// question positions continuing after the shared context; other questions
// and other requests invisible), and the glossary entry "ForkAttention"
// (in standard attention the fork is a visibility rule).
//
// Visibility as a causal rule. A branch of length L whose request's trunk
// has P tokens sees exactly what its tokens would see in the independent
// prompt trunk ++ branch: its query at branch position p is the query at
// virtual position P + p of that prompt, and the keys it may read are the
// virtual positions 0 .. P + p, where virtual position x < P is trunk token
// x and x >= P is branch token x - P. A trunk token is the same rule with
// P = 0 over its own request. So every work item is a causal attention over
// a virtual key sequence, gathered from two ranges of the stream.
//
// Kernels:
//   plan -- one workgroup: query tiles per segment (branches first, then
//           trunks), exclusive prefix sums into the workspace, capped at
//           the grid's capacity.
//   attn -- one workgroup per (head, query tile of 64 rows): streams the
//           tile's virtual keys in blocks of 64 through LDS (K row-major,
//           V transposed, so both MFMA operands read contiguous keys) with
//           an online softmax. Each of the 4 waves owns 16 queries.
//
// Layout of the products (v_mfma_f32_16x16x32_bf16; A rows and B columns
// are indexed by lane % 16, the 8 reduction slots of a lane by lane / 16):
//   S^T = K Q^T   keys x queries; a lane ends up with 4 keys of 4 key tiles
//                 for one query (lane % 16), so the softmax statistics of a
//                 query live in the 4 lanes lane % 16 + {0, 16, 32, 48};
//   O^T = V^T P^T d x queries; the lane's own probabilities are its B
//                 operand as they stand (its 8 reduction slots are the keys
//                 of two adjacent key tiles), and V^T is read with the same
//                 key order; the result keeps one query per lane column, so
//                 the online-softmax rescale needs no data exchange.
// q, k, v are bf16 (their products are exact in the fp32 accumulators);
// the probabilities are split into bf16 hi + lo and both go through the
// matrix cores (P = P_hi + P_lo to about 2^-17), since one bf16 rounding
// of P (2^-9 relative) would not hold a 2e-3 end-to-end tolerance.

#include <mutex>

#include "attention_launch.hpp"
#include "gdn_device.hpp"

namespace gdn {
namespace {

constexpr int kAThreads = 256;
constexpr int BN = 64;   // keys per block
// queries per workgroup: 16 * QR per wave. Branches (typically short) use
// QR = 1; trunks QR = 2, where each K / V operand read from LDS feeds two
// query groups (half the LDS traffic per product).
constexpr int kQrBranch = 1, kQrTrunk = 2;
constexpr int kGroup = 16;  // consecutive work items that share an XCD (and its L2)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Seg {
    int t0, len;    // the segment's own tokens [t0, t0 + len)
    int p0, plen;   // the trunk a branch reads first (plen = 0 for a trunk)
    bool ok;        // false: a branch whose parent index is out of range
};

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return min(max(x, lo), hi); }

// Segment `seg` in work order: branches 0 .. n_branch-1, then trunks.
// Offsets are clamped into the stream, so bad metadata cannot address
// outside it.
__device__ __forceinline__ Seg segment(const AttnArgs &a, int seg) {
    const int N = a.n_tokens;
    Seg s{0, 0, 0, 0, true};
    if (seg < a.n_branch) {
        const int b0 = clampi(a.bcu[seg], 0, N), b1 = clampi(a.bcu[seg + 1], b0, N);
        s.t0 = b0;
        s.len = b1 - b0;
        const int r = a.bparent[seg];
        if (r < 0 || r >= a.n_req) {
            s.ok = false;
        } else {
            const int c0 = clampi(a.cu[r], 0, N), c1 = clampi(a.cu[r + 1], c0, N);
            s.p0 = c0;
            s.plen = c1 - c0;
        }
    } else {
        const int r = seg - a.n_branch;
        const int c0 = clampi(a.cu[r], 0, N), c1 = clampi(a.cu[r + 1], c0, N);
        s.t0 = c0;
        s.len = a.trunk_queries ? c1 - c0 : 0;
    }
    return s;
}

// Branches 2i and 2i + 1 share one tile of 128 queries (64 each, two query
// groups per wave like a trunk tile) when they hang off the same valid
// request and are at most 64 tokens long: both read the same trunk, each
// then its own tokens (a branch's keys are invisible to the other's
// queries).
__device__ __forceinline__ bool pair_first(const AttnArgs &a, int b) {
    if ((b & 1) || b + 1 >= a.n_branch) return false;
    const Seg x = segment(a, b), y = segment(a, b + 1);
    return x.ok && y.ok && a.bparent[b] == a.bparent[b + 1] && x.len <= 64 && y.len <= 64;
}

// query tiles of segment seg: trunks of 128 queries, branches of 64 or in
// pairs
__device__ __forceinline__ int seg_tiles(const AttnArgs &a, int seg) {
    if (seg >= a.n_branch) return (segment(a, seg).len + 64 * kQrTrunk - 1) / (64 * kQrTrunk);
    if (pair_first(a, seg)) return segment(a, seg).len + segment(a, seg + 1).len > 0 ? 1 : 0;
    if ((seg & 1) && pair_first(a, seg - 1)) return 0;
    return (segment(a, seg).len + 64 * kQrBranch - 1) / (64 * kQrBranch);
}

// ws[seg] = first tile of segment seg, ws[n_seg] = number of tiles, all
// capped at max_tiles (the grid's capacity; only overlapping segments,
// which the interface excludes, can reach it).
__global__ __launch_bounds__(kAThreads) void attn_plan_kernel(AttnArgs a, int max_tiles) {
    __shared__ int s_scan[kAThreads];
    int *ts = static_cast<int *>(a.ws);
    const int n_seg = a.n_branch + a.n_req, tid = threadIdx.x;
    int run = 0;
    for (int base = 0; base < n_seg; base += kAThreads) {
        const int seg = base + tid;
        int c = 0;
        if (seg < n_seg) c = seg_tiles(a, seg);
        s_scan[tid] = c;
        __syncthreads();
        for (int off = 1; off < kAThreads; off <<= 1) {
            const int x = tid >= off ? s_scan[tid - off] : 0;
            __syncthreads();
            s_scan[tid] += x;
            __syncthreads();
        }
        if (seg < n_seg) ts[seg] = min(run + s_scan[tid] - c, max_tiles);
        run += s_scan[kAThreads - 1];
        __syncthreads();
    }
    if (tid == 0) ts[n_seg] = min(run, max_tiles);
}

// One query tile of one segment and head: 16 * QR queries per wave. PAIR:
// a tile of two branches sg (rows 0..63) and sb (rows 64..127) of the same
// request; their virtual keys are the trunk, then sg's tokens, then sb's,
// and sb's queries skip sg's tokens.
template <int D, typename TO, int QR, bool PAIR>
__device__ __forceinline__ void attn_tile(const AttnArgs &a, const Seg &sg, const Seg &sb, int h,
                                          int tile, __bf16 *s_k, __bf16 *s_vt) {
    static_assert(!PAIR || QR == 2, "a branch pair fills two query groups per wave");
    constexpr int BM = 64 * QR;               // queries per workgroup
    constexpr int KSD = D / 32;               // reduction steps of S^T over d
    constexpr int NDT = D / 16;               // 16-row d tiles of O^T
    constexpr int KP = D + 8;                 // padded K row in LDS (bf16)
    constexpr int VP = BN + 4;                // padded V^T row (see attn_kernel)
    constexpr int CPR = D / 8;                // 16-byte pieces per key row
    constexpr int KPASS = BN * CPR / kAThreads;       // K pieces per thread
    constexpr int PPP = kAThreads / CPR;              // key pairs per V pass
    constexpr int VPASS = (BN / 2) / PPP;             // V passes (2 pieces each)
    static_assert(KPASS >= 1 && VPASS >= 1 && PPP >= 16, "block shape");

    const int q_first = PAIR ? 0 : tile * BM;
    const int L = PAIR ? BM : min(BM, sg.len - q_first);
    const int H = a.H;
    const int tid = threadIdx.x, lane = tid % kWave;
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
    TO *o = static_cast<TO *>(a.o);

    if (!PAIR && !sg.ok) {  // a branch with an invalid parent: NaN outputs
        for (int idx = tid; idx < L * D; idx += kAThreads)
            o[((size_t)(sg.t0 + q_first + idx / D) * H + h) * D + idx % D] =
                from_f32<TO>(quiet_nan());
        return;
    }

    const int hk = h / (H / a.Hkv);
    const int Hkv = a.Hkv;
    const int la = PAIR ? sg.len : 0;  // keys of the first branch of a pair
    // virtual keys the tile reads
    const int kv_len = PAIR ? sg.plen + sg.len + sb.len : sg.plen + q_first + L;
    const int nblk = (kv_len + BN - 1) / BN;
    const int g4 = (lane / 16) * 4, g8 = (lane / 16) * 8;
    // query group qg of this wave: tile row w*16*QR + qg*16 + lane % 16;
    // its stream token, virtual position, validity, and the virtual keys
    // [hlo, hhi) it skips (the other branch of a pair)
    int qtok[QR], qp[QR], hlo[QR], hhi[QR];
    bool qok[QR];
    bf16x8 qf[QR][KSD];  // Q^T operand: 8 consecutive d per reduction step
#pragma unroll
    for (int qg = 0; qg < QR; ++qg) {
        const int r = w * 16 * QR + qg * 16 + lane % 16;
        if constexpr (PAIR) {
            const bool second = w >= 2;  // rows 64..127: waves 2 and 3
            const int pos = r & 63, len = second ? sb.len : sg.len;
            const int posc = len > 0 ? min(pos, len - 1) : 0;  // clamped for rows past the end
            qok[qg] = pos < len;
            // an empty branch's rows read the other (non-empty) branch's token
            qtok[qg] = len > 0 ? (second ? sb.t0 : sg.t0) + posc : (second ? sg.t0 : sb.t0);
            qp[qg] = sg.plen + (second ? sg.len : 0) + posc;
            hlo[qg] = second ? sg.plen : 0;
            hhi[qg] = second ? sg.plen + sg.len : 0;
        } else {
            const int qrow = min(r, L - 1);  // clamped for rows past the tile end
            qok[qg] = r < L;
            qtok[qg] = sg.t0 + q_first + qrow;
            qp[qg] = sg.plen + q_first + qrow;
            hlo[qg] = hhi[qg] = 0;
        }
        const __bf16 *qsrc =
            static_cast<const __bf16 *>(a.q) + ((size_t)qtok[qg] * H + h) * D + g8;
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks)
            qf[qg][ks] = *reinterpret_cast<const bf16x8 *>(qsrc + ks * 32);
    }

    // k / v rows of the ranges a tile reads (the parent's trunk, the
    // segment itself, and for a pair the second branch); offsets inside a
    // range fit 32 bits (checked on the host)
    const uint32_t rs = (uint32_t)(Hkv * D);  // elements per stream row
    const __bf16 *kg = static_cast<const __bf16 *>(a.k) + hk * D;
    const __bf16 *vg = static_cast<const __bf16 *>(a.v) + hk * D;
    const int t_last = PAIR ? sb.t0 : sg.t0;  // the range after the first la own keys
    const __bf16 *k_tr = kg + (size_t)sg.p0 * rs, *k_own = kg + (size_t)sg.t0 * rs;
    const __bf16 *v_tr = vg + (size_t)sg.p0 * rs, *v_own = vg + (size_t)sg.t0 * rs;
    const __bf16 *k_last = kg + (size_t)t_last * rs, *v_last = vg + (size_t)t_last * rs;
    // row of virtual key x (clamped into the tile's keys)
    auto row = [&](const __bf16 *tr, const __bf16 *own, const __bf16 *last, int x) {
        x = min(x, kv_len - 1);
        if (x < sg.plen) return tr + (uint32_t)x * rs;
        if (PAIR && x < sg.plen + la) return own + (uint32_t)(x - sg.plen) * rs;
        return last + (uint32_t)(x - sg.plen - la) * rs;
    };
    bf16x8 kreg[KPASS];
    u32x4 vreg[VPASS][2];
    auto load_block = [&](int j) {
#pragma unroll
        for (int p = 0; p < KPASS; ++p) {
            const int piece = p * kAThreads + tid, r = piece / CPR, c = piece % CPR;
            kreg[p] =
                *reinterpret_cast<const bf16x8 *>(row(k_tr, k_own, k_last, j * BN + r) + c * 8);
        }
#pragma unroll
        for (int p = 0; p < VPASS; ++p) {
            const int c = tid / PPP, r = 2 * (p * PPP + tid % PPP);
#pragma unroll
            for (int u = 0; u < 2; ++u)
                vreg[p][u] = *reinterpret_cast<const u32x4 *>(
                    row(v_tr, v_own, v_last, j * BN + r + u) + c * 8);
        }
    };
    auto store_block = [&](int buf) {
        __bf16 *sk = s_k + buf * (BN * KP);
        __bf16 *sv = s_vt + buf * (D * VP);
#pragma unroll
        for (int p = 0; p < KPASS; ++p) {
            const int piece = p * kAThreads + tid, r = piece / CPR, c = piece % CPR;
            *reinterpret_cast<bf16x8 *>(sk + r * KP + c * 8) = kreg[p];
        }
#pragma unroll
        for (int p = 0; p < VPASS; ++p) {
            const int c = tid / PPP, r = 2 * (p * PPP + tid % PPP);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                // keys r and r + 1 of rows d = 8c + 2x (low halves) and
                // 8c + 2x + 1 (high halves), each pair as one 4-byte word
                const uint32_t a0 = vreg[p][0][x], a1 = vreg[p][1][x];
                *reinterpret_cast<uint32_t *>(sv + (c * 8 + 2 * x) * VP + r) =
                    (a0 & 0xffffu) | (a1 << 16);
                *reinterpret_cast<uint32_t *>(sv + (c * 8 + 2 * x + 1) * VP + r) =
                    (a0 >> 16) | (a1 & 0xffff0000u);
            }
        }
    };

    // Online softmax in log2 units with a lazily moved reference: the
    // exponent base m changes only when a block's maximum exceeds it by more
    // than kLazy, so most blocks skip the rescale of o and of the row sum;
    // the weights exp2(s - m) then stay below 2^kLazy (exact in fp32 either
    // way: the same m scales o and the row sum).
    constexpr float kLazy = 8.f;
    const float c2 = a.scale * 1.4426950408889634f;  // scale > 0 (checked on the host)
    const int qp_lo = sg.plen + q_first;              // first query of the tile
    float m[QR], lsum[QR];
    f32x4v acc[QR][NDT];
#pragma unroll
    for (int qg = 0; qg < QR; ++qg) {
        // finite: a pair's second branch over an empty trunk sees no key in
        // its first blocks, and exp2(-inf - m) must then give 0, not NaN
        m[qg] = -1e30f;
        lsum[qg] = 0.f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[qg][dt] = f32x4v{0.f, 0.f, 0.f, 0.f};
    }

    load_block(0);
    store_block(0);
    if (nblk > 1) load_block(1);
    __syncthreads();
    for (int j = 0; j < nblk; ++j) {
        const __bf16 *sk = s_k + (j & 1) * (BN * KP);
        const __bf16 *sv = s_vt + (j & 1) * (D * VP);

        // S^T: rows = keys kt*16 + g4 + i, column = the lane's query of group qg
        f32x4v st[QR][4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
            for (int qg = 0; qg < QR; ++qg) st[qg][kt] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KSD; ++ks) {
                const bf16x8 kf =
                    *reinterpret_cast<const bf16x8 *>(sk + (kt * 16 + lane % 16) * KP + ks * 32 + g8);
#pragma unroll
                for (int qg = 0; qg < QR; ++qg)
                    st[qg][kt] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qg][ks], st[qg][kt], 0, 0, 0);
            }
        }
        // keys after a query (and past the tile's keys) only in the last blocks
        if (j * BN + BN - 1 > qp_lo) {
#pragma unroll
            for (int qg = 0; qg < QR; ++qg)
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = j * BN + kt * 16 + g4 + i;
                        if (key > qp[qg] || (key >= hlo[qg] && key < hhi[qg]))
                            st[qg][kt][i] = -INFINITY;
                    }
        }
        u32x4 ph[QR][2];
        bf16x8 pl[QR][2];
#pragma unroll
        for (int qg = 0; qg < QR; ++qg) {
            // the reference is shared by a query's 4 lanes (their products
            // are summed by the matrix cores); lanes compare their own maxima
            // and only a move of the reference combines them
            float mloc = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) mloc = fmaxf(mloc, st[qg][kt][i]);
            mloc *= c2;
            if (__builtin_amdgcn_ballot_w64(mloc > m[qg] + kLazy) != 0) {
                mloc = fmaxf(mloc, __shfl_xor(mloc, 16, kWave));
                mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
                const float mn = fmaxf(m[qg], mloc);
                const float alpha = __builtin_amdgcn_exp2f(m[qg] - mn);
                m[qg] = mn;
                lsum[qg] *= alpha;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) acc[qg][dt] *= alpha;
            }
            // P^T operands: p = hi + lo with hi the upper half of p's bits
            // (exact split: lo = p - hi has at most 16 significant bits, of
            // which bf16 keeps 8 -- p to about 2^-16 relative)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(st[qg][kt][i], c2, -m[qg]));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(st[qg][kt][i + 1], c2, -m[qg]));
                    lsum[qg] += p0 + p1;
                    const uint32_t h0 = __float_as_uint(p0) & 0xffff0000u;
                    const uint32_t h1 = __float_as_uint(p1) & 0xffff0000u;
                    const int e = (kt % 2) * 4 + i;  // reduction slot of key kt*16 + g4 + i
                    ph[qg][kt / 2][e / 2] = (h0 >> 16) | h1;
                    pl[qg][kt / 2][e] = (__bf16)(p0 - __uint_as_float(h0));
                    pl[qg][kt / 2][e + 1] = (__bf16)(p1 - __uint_as_float(h1));
                }
        }
        // O^T += V^T P^T over the two 32-key halves of the block
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const __bf16 *vp = sv + (dt * 16 + lane % 16) * VP + c * 32 + g4;
                const bf16x4 v0 = *reinterpret_cast<const bf16x4 *>(vp);
                const bf16x4 v1 = *reinterpret_cast<const bf16x4 *>(vp + 16);
                const bf16x8 vf = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
                for (int qg = 0; qg < QR; ++qg) {
                    acc[qg][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        vf, __builtin_bit_cast(bf16x8, ph[qg][c]), acc[qg][dt], 0, 0, 0);
                    acc[qg][dt] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pl[qg][c], acc[qg][dt], 0, 0, 0);
                }
            }
        }
        // block j + 1 into the other buffer (its readers finished before the
        // previous barrier), then fetch block j + 2
        if (j + 1 < nblk) {
            store_block((j + 1) & 1);
            if (j + 2 < nblk) load_block(j + 2);
        }
        __syncthreads();
    }

#pragma unroll
    for (int qg = 0; qg < QR; ++qg) {
        // the row sum of a query is split over its 4 lanes
        float ltot = lsum[qg] + __shfl_xor(lsum[qg], 16, kWave);
        ltot += __shfl_xor(ltot, 32, kWave);
        if (qok[qg]) {
            TO *orow = o + ((size_t)qtok[qg] * H + h) * D;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    orow[dt * 16 + g4 + i] = from_f32<TO>(acc[qg][dt][i] / ltot);
        }
    }
}

template <int D, typename TO>
__global__ __launch_bounds__(kAThreads) __attribute__((amdgpu_waves_per_eu(2))) void attn_kernel(AttnArgs a) {
    constexpr int KP = D + 8;
    // V^T rows of BN keys padded to 34 words: the transposing stores (16
    // key pairs of one row per quarter-wave, rows 8 apart across quarter-
    // waves) and the operand reads (16 consecutive rows, same keys) both
    // spread over all 32 banks
    constexpr int VP = BN + 4;
    // two buffers: block j + 1 is written while block j is read
    __shared__ __attribute__((aligned(16))) __bf16 s_k[2 * BN * KP];
    __shared__ __attribute__((aligned(16))) __bf16 s_vt[2 * D * VP];

    const int *ts = static_cast<const int *>(a.ws);
    const int n_seg = a.n_branch + a.n_req;
    const int T = ts[n_seg];
    // block -> work item: groups of kGroup consecutive items per XCD
    // (blocks are dispatched to the 8 XCDs round-robin)
    const int b = blockIdx.x, xcd = b % 8, local = b / 8;
    const int wi = ((local / kGroup) * 8 + xcd) * kGroup + local % kGroup;
    if (wi >= a.H * T) return;
    const int h = wi / T, t = wi % T;
    int lo = 0, hi = n_seg;  // ts[lo] <= t < ts[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (ts[mid] <= t) lo = mid;
        else hi = mid;
    }
    const Seg sg = segment(a, lo);
    const int ntile = ts[lo + 1] - ts[lo];
    const int tile = ntile - 1 - (t - ts[lo]);  // the longest tiles of a segment first
    if (lo >= a.n_branch)
        attn_tile<D, TO, kQrTrunk, false>(a, sg, sg, h, tile, s_k, s_vt);
    else if (pair_first(a, lo))
        attn_tile<D, TO, 2, true>(a, sg, segment(a, lo + 1), h, 0, s_k, s_vt);
    else
        attn_tile<D, TO, kQrBranch, false>(a, sg, sg, h, tile, s_k, s_vt);
}

template <int D, typename TO>
hipError_t launch_typed(const AttnArgs &a, hipStream_t stream) {
    const int n_seg = a.n_branch + a.n_req;
    if (n_seg == 0) return hipSuccess;
    const long long max_tiles = (long long)(a.n_tokens + 63) / 64 + n_seg;  // tiles of >= 64
    const long long items = max_tiles * a.H;
    const long long per = 8LL * kGroup;
    const long long blocks = (items + per - 1) / per * per;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(attn_plan_kernel, dim3(1), dim3(kAThreads), 0, stream, a, (int)max_tiles);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_kernel<D, TO>), dim3((unsigned)blocks), dim3(kAThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

size_t attention_workspace_bytes(int n_req, int n_branch) {
    return sizeof(int32_t) * ((size_t)n_req + (size_t)n_branch + 1);
}

// Tile table of the allocation-free entry point: one file-scope device array
// that every GPU the library runs on holds from module load to process end.
// In host code `scratch` names a host-side stand-in, not device memory, so
// host code only ever uses the per-device address hipGetSymbolAddress
// returns for it (kept in g_scratch_ptr below).
static __device__ __align__(256) int32_t scratch[kAttnScratchSegments + 1];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // per device: the address of its copy of `scratch`
}  // namespace

hipError_t attention_scratch(void **ptr, size_t *bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        // once per device, with that device current: its copy's address
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    *bytes = sizeof(scratch);
    return hipSuccess;
}

hipError_t launch_attention(int d, int out, const AttnArgs &a, hipStream_t stream) {
    if (d == 128) return out == kBF16 ? launch_typed<128, bf16>(a, stream)
                                      : launch_typed<128, float>(a, stream);
    if (d == 64) return out == kBF16 ? launch_typed<64, bf16>(a, stream)
                                     : launch_typed<64, float>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace gdn
