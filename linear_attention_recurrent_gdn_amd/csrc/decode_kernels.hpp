// decode_kernels.hpp -- decode-step kernels for gfx950: the eager dense update, the
// deferred (base + log) append step with its merge, and a merge-only pass.
//
// Sources: "DeltaLog: Deferred Materialization of Recurrent States for
// Linear Attention Decoding" (gist.science summary) -- problem section (the
// eager update rewrites the whole [B,H,d_k,d_v] state every token), "핵심
// 메커니즘: Base + Log" (base + bounded log; append phase leaves the base
// untouched; merge phase writes base + replayed log back), "커널 구현"
// (value-tile parallelism; key-side factors and log-decay metadata shared
// by the value tiles; one shared ReplayPrep stage per slot-head followed by
// per-value-tile AppendDecode stages; GDN / KDA / RWKV6 operators).
//
// MI355X mapping. One workgroup of 256 threads (4 wave64s) owns one
// (row, head) for the whole step. The pages' two stages become two phases
// of that workgroup with LDS as the hand-off:
//   ReplayPrep  -- per slot-head, once: decayed key / query (k^, q^), the
//                  replay coefficients c_e = <k~_e, k>, d_e = <k~_e, q> of
//                  the logged entries (k~_e = k_e . exp(Lam_t - Lam_e)) and
//                  k.q, written to LDS where every value tile reads them.
//   AppendDecode -- the value tiles: each thread streams float4 columns of
//                  the base from HBM (16 x dwordx4 loads in flight per
//                  thread at d=128), reduces S^T k^ and S^T q^ over the key
//                  rows (wave64 shuffles, then LDS across the 4 waves), and
//                  the threads of column j finish x_j, u_j, o_j by replaying
//                  the logged u_e[j].
// On a merging step the base tile is still in registers, so the merge
// (base <- diag(exp Lam_t) base + sum_e k~_e u_e^T) costs one write and no
// second read. The eager step is the same code with an empty log that
// merges every step, so a deferred run with merge_at = 1 is bit-identical
// to the eager one.
//
// Math: storage Sig = S^T, [d_k][d_v]. With a = exp(Lam_t):
//   y = S_{t-1}(a . k) = Sig_base^T (a.k) + sum_e c_e u_e
//   u = beta (v - y)            (RWKV6: u = v)
//   o = S_t q = Sig_base^T (a.q) + sum_e d_e u_e + (k.q) u
// which follows from the recurrence S_t = S_{t-1} diag(a_t) + u_t k_t^T.

#pragma once

#include "gdn_device.hpp"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

enum Mode { kEager = 0, kAppend = 1, kMergeOnly = 2 };

// Entries a log may hold: the whole log of a slot-head is prefetched into
// registers with the base stream, so its capacity is a compile-time bound.
constexpr int kMaxLog = 16;

// Sum over aligned groups of SEG lanes (SEG a power of two <= 64); every
// lane of a group ends with the group total.
template <int SEG>
__device__ __forceinline__ float wave_sum_seg(float x) {
#pragma unroll
    for (int off = 1; off < SEG; off <<= 1) x += __shfl_xor(x, off, kWave);
    return x;
}

// Thread -> (row, float4 column) map of one [DK][DV] fp32 tile.
template <int DK, int DV>
struct TileMap {
    static constexpr int TPR = DV / 4;          // threads across a row
    static constexpr int RPP = kThreads / TPR;  // rows per pass
    static constexpr int P = DK / RPP;          // passes (float4 per thread)
    static_assert(TPR <= kWave && kWave % TPR == 0, "row must fit a wave");
    static_assert(P >= 1 && DK % RPP == 0, "tile must cover the rows");
};

// Row-gathered position of key row i: the thread owning rows r0 + p*RPP
// (p < P) finds them at r0*P .. r0*P + P - 1.
template <int DK, int DV>
__device__ __forceinline__ int row_gather(int i) {
    using Map = TileMap<DK, DV>;
    return (i % Map::RPP) * Map::P + i / Map::RPP;
}

// N consecutive floats from LDS (16-byte aligned when N >= 4).
template <int N>
__device__ __forceinline__ void lds_gather(const float *p, float (&x)[N]) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            const float4 v = reinterpret_cast<const float4 *>(p)[i];
            x[4 * i] = v.x;
            x[4 * i + 1] = v.y;
            x[4 * i + 2] = v.z;
            x[4 * i + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] = p[i];
    }
}

// Write-back of a materialised base row piece. The eager step rewrites every
// tile (a copy-like stream: non-temporal stores); the deferred steps write
// the few merging slots, whose lines are read again at the next step.
template <bool NT>
__device__ __forceinline__ void store_base(float *p, float4 x) {
    if (NT) store_stream(p, x);
    else *reinterpret_cast<float4 *>(p) = x;
}

template <int DK, int DV, int VAR, typename TI, typename TO, int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void decode_kernel(DecodeArgs a) {
    using Map = TileMap<DK, DV>;
    const auto rg = [](int i) { return row_gather<DK, DV>(i); };
    constexpr bool kPerKey = VAR != kScalar;
    constexpr bool kDelta = VAR != kRwkv6;
    constexpr int LS = kPerKey ? DK : 1;                 // log-decay values per log entry
    constexpr int ML = MODE == kEager ? 0 : kMaxLog;     // log entries held on chip
    constexpr int NKE = ML ? (ML * DK + kThreads - 1) / kThreads : 1;  // key-side elems/thread
    constexpr int NUE = ML ? (ML * DV + kThreads - 1) / kThreads : 1;  // value-side elems/thread
    constexpr int SEG = DK < kWave ? DK : kWave;         // lanes summing one key range
    constexpr int NSEG = DK / SEG;                       // partial sums per key vector

    // LDS. Per-row vectors of the key side are kept in "row-gathered" order
    // (rg(i): the P rows a thread owns are consecutive), so a thread fetches
    // its rows with P/4 float4 reads.
    __shared__ __attribute__((aligned(16))) float s_k[DK], s_q[DK], s_lam[DK];
    __shared__ __attribute__((aligned(16))) float s_khg[DK], s_qhg[DK], s_ag[DK];  // a.k, a.q, a
    __shared__ __attribute__((aligned(16))) float s_red[kWaves][2][DV];
    __shared__ __attribute__((aligned(16))) float s_cd[ML + 1][4];  // c_e, d_e partial sums
    __shared__ float s_dtpart[NSEG];
    __shared__ __attribute__((aligned(16))) float s_ktg[(ML + 1) * DK];  // k~_e / k_e, row-gathered
    __shared__ __attribute__((aligned(16))) float s_u[(ML + 1) * DV];    // u_e
    __shared__ float s_fac[ML + 1];  // scalar decay: exp(Lam_t - Lam_e)
    static_assert(NSEG <= 2, "two partial sums per key vector at most");

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int row = blockIdx.x;  // (b, h) of the batch, flattened
    const int b = row / a.H;
    const int h = row - b * a.H;
    const int slot = a.slot_idx ? a.slot_idx[b] : b;
    if (slot < 0 || slot >= a.n_slots) {
        if (MODE != kMergeOnly)
            for (int j = tid; j < DV; j += kThreads)
                static_cast<TO *>(a.o)[(size_t)row * DV + j] = from_f32<TO>(quiet_nan());
        return;
    }
    const size_t sh = (size_t)slot * a.H + h;  // slot-head
    float *S = a.state + sh * DK * DV;
    const int Mcap = a.Mcap;
    const float *lam_log = MODE != kEager ? a.log_lam + sh * Mcap * LS : nullptr;
    const TI *logk = MODE != kEager ? static_cast<const TI *>(a.log_k) + sh * Mcap * DK : nullptr;
    float *logu = MODE != kEager ? a.log_u + sh * Mcap * DV : nullptr;

    // ---- one round trip. The base stream is issued first; everything else
    // is a small branch-free load behind it (addresses clamped in bounds,
    // conversions deferred), so no wait can fall between the base loads. The
    // log length is uniform and comes through the scalar path, so the log
    // entries that depend on it are issued while the base is in flight.
    const int col = (tid % Map::TPR) * 4;
    const int r0 = tid / Map::TPR;
    // 32-bit element offsets from the uniform tile base keep the addresses
    // of the 16 loads and stores in single VGPRs (scalar base + vector offset)
    const auto tile_off = [&](int p) { return (uint32_t)((r0 + p * Map::RPP) * DV + col); };
    // The waves of a deferred-step workgroup issue all of its loads at
    // raised priority (back to normal before the first use), so a newly
    // started workgroup gets its requests out ahead of the arithmetic of the
    // others on the CU (measured 105 -> 102 us per deferred step on 256 x 32
    // slot-heads). The eager step, a copy-like stream with a store for every
    // load, measured slower with it (192 -> 203 us) and runs without.
    if constexpr (MODE != kEager) __builtin_amdgcn_s_setprio(1);
    float4 reg[Map::P];
#pragma unroll
    for (int p = 0; p < Map::P; ++p)
        reg[p] = load_stream(S + tile_off(p));

    int m_raw = 0;
    if (MODE != kEager) m_raw = a.log_len[sh];
    const int ik = min(tid, DK - 1), iv = min(tid, DV - 1);
    TI k_raw{}, q_raw{}, v_raw{};
    float lax = 0.f, bx = 1.f;
    if (MODE != kMergeOnly) {
        k_raw = static_cast<const TI *>(a.k)[(size_t)row * DK + ik];
        q_raw = static_cast<const TI *>(a.q)[(size_t)row * DK + ik];
        v_raw = static_cast<const TI *>(a.v)[(size_t)row * DV + iv];
        lax = a.log_alpha[(size_t)row * LS + (kPerKey ? ik : 0)];
        if (kDelta) bx = a.beta[row];
    }

    const int m = MODE == kEager ? 0 : min(max(m_raw, 0), Mcap);
    bool merge = true;
    if (MODE == kAppend) merge = (a.merge_at > 0 && m + 1 >= a.merge_at) || m >= Mcap;
    if (MODE == kMergeOnly) merge = m > 0 && m >= a.min_len;
    if (!merge && MODE == kMergeOnly) return;
    const int e_last = max(m - 1, 0);  // a valid entry index for clamped loads
    float lam_prev = 0.f, lam_e_s = 0.f;
    TI kl_raw[NKE];
    float ll[kPerKey ? NKE : 1], ul[NUE];
    if (MODE != kEager) {
        lam_prev = lam_log[e_last * LS + (kPerKey ? ik : 0)];
        if (!kPerKey) lam_e_s = lam_log[min(tid, e_last)];
#pragma unroll
        for (int r = 0; r < NKE; ++r) {
            const int idx = tid + r * kThreads, e = min(idx / DK, e_last), i = idx % DK;
            kl_raw[r] = logk[(size_t)e * DK + i];
            if (kPerKey) ll[r] = lam_log[e * LS + i];
        }
#pragma unroll
        for (int r = 0; r < NUE; ++r) {
            const int idx = tid + r * kThreads, e = min(idx / DV, e_last), j = idx % DV;
            ul[r] = logu[e * DV + j];
        }
    }
    if constexpr (MODE != kEager) __builtin_amdgcn_s_setprio(0);
    if (m == 0) lam_prev = 0.f;
    const float kx = to_f32(k_raw), qx = to_f32(q_raw), vx = to_f32(v_raw);

    // ---- ReplayPrep (key side, once per slot-head)
    if (tid < DK) {
        const float lam = MODE == kMergeOnly ? lam_prev : lam_prev + lax;
        const float ai = expf(lam);
        const int g = rg(tid);
        s_lam[tid] = lam;
        s_k[tid] = kx;
        s_q[tid] = qx;
        s_ag[g] = ai;
        s_khg[g] = ai * kx;
        s_qhg[g] = ai * qx;
    }
    if (!kPerKey && tid < m) s_fac[tid] = lam_e_s;  // Lam_e, turned into a factor below
    if (MODE != kMergeOnly) {  // k . q
        float p = wave_sum_seg<SEG>(kx * qx);
        if (tid < DK && lane % SEG == 0) s_dtpart[tid / SEG] = p;
    }
    __syncthreads();
    // No barrier closes this part: what it writes (s_fac, s_cd, s_ktg, s_u)
    // is read only after the reduction barrier or the merge barrier below.
    if (!kPerKey && tid < m) s_fac[tid] = expf(s_lam[0] - s_fac[tid]);  // exp(Lam_t - Lam_e)
    if (ML > 0) {
#pragma unroll
        for (int r = 0; r < NKE; ++r) {
            const int idx = tid + r * kThreads, e = idx / DK, i = idx % DK;
            float pc = 0.f, pd = 0.f;
            if (e < m) {
                // per-key: fold the decay ratio into k~ here (the hardware
                // base-2 exponential: the argument is <= 0 and at most the
                // log's summed decay, about 1e-6 relative); scalar: it
                // factors out of the sums and is applied per entry
                const float kl = to_f32(kl_raw[r]);
                const float kt = kPerKey ? kl * __expf(s_lam[i] - ll[r]) : kl;
                pc = kt * s_k[i];
                pd = kt * s_q[i];
                if (merge) s_ktg[e * DK + rg(i)] = kt;
            }
            if (MODE != kMergeOnly) {
                pc = wave_sum_seg<SEG>(pc);
                pd = wave_sum_seg<SEG>(pd);
                if (e < m && lane % SEG == 0) {
                    s_cd[e][i / SEG] = pc;
                    s_cd[e][2 + i / SEG] = pd;
                    if (NSEG == 1) {
                        s_cd[e][1] = 0.f;
                        s_cd[e][3] = 0.f;
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < NUE; ++r) {
            const int idx = tid + r * kThreads, e = idx / DV;
            if (e < m) s_u[idx] = ul[r];
        }
    }
    if (MODE != kMergeOnly && merge && tid < DK) s_ktg[m * DK + rg(tid)] = kx;

    // ---- AppendDecode: S^T k^ and S^T q^ over the key rows
    if (MODE != kMergeOnly) {
        float ax[4] = {0.f, 0.f, 0.f, 0.f}, ao[4] = {0.f, 0.f, 0.f, 0.f};
        constexpr int G = Map::P < 4 ? Map::P : 4;  // rows per LDS fetch
#pragma unroll
        for (int p0 = 0; p0 < Map::P; p0 += G) {
            float kh[G], qh[G];
            lds_gather<G>(s_khg + r0 * Map::P + p0, kh);
            lds_gather<G>(s_qhg + r0 * Map::P + p0, qh);
#pragma unroll
            for (int pp = 0; pp < G; ++pp) {
                const float4 xv = reg[p0 + pp];
                const float x4[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (kDelta) ax[c] = fmaf(x4[c], kh[pp], ax[c]);
                    ao[c] = fmaf(x4[c], qh[pp], ao[c]);
                }
            }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (kDelta) ax[c] = wave_sum_strided<Map::TPR>(ax[c]);
            ao[c] = wave_sum_strided<Map::TPR>(ao[c]);
        }
        if (lane < Map::TPR) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                s_red[wave][0][col + c] = kDelta ? ax[c] : 0.f;
                s_red[wave][1][col + c] = ao[c];
            }
        }
        __syncthreads();

        // the value columns: replay the log, form u, o; append or stage
        if (tid < DV) {
            const int j = tid;
            float x = 0.f, oo = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                x += s_red[w][0][j];
                oo += s_red[w][1][j];
            }
            // groups of 4 entries, unrolled and predicated (m is uniform), so
            // the LDS reads of a group are issued together
#pragma unroll
            for (int e0 = 0; e0 < ML; e0 += 4) {
                if (e0 >= m) break;
#pragma unroll
                for (int e = e0; e < e0 + 4; ++e) {
                if (e < m) {
                    const float4 cd = *reinterpret_cast<const float4 *>(&s_cd[e][0]);
                    float c = cd.x + cd.y, d = cd.z + cd.w;
                    if (!kPerKey) {
                        c *= s_fac[e];
                        d *= s_fac[e];
                    }
                    const float ue = s_u[e * DV + j];
                    x = fmaf(c, ue, x);
                    oo = fmaf(d, ue, oo);
                }
                }
            }
            float dt = 0.f;
#pragma unroll
            for (int g = 0; g < NSEG; ++g) dt += s_dtpart[g];
            const float u = kDelta ? bx * (vx - x) : vx;
            oo = fmaf(dt, u, oo);
            static_cast<TO *>(a.o)[(size_t)row * DV + j] = from_f32<TO>(oo);
            if (merge)
                s_u[m * DV + j] = u;
            else
                logu[m * DV + j] = u;
        }
        if (MODE == kAppend && !merge && tid < DK) {
            static_cast<TI *>(a.log_k)[(sh * Mcap + m) * DK + tid] = k_raw;
            if (kPerKey) a.log_lam[(sh * Mcap + m) * DK + tid] = s_lam[tid];
            else if (tid == 0) a.log_lam[sh * Mcap + m] = s_lam[0];
        }
    }
    if (MODE != kEager && tid == 0) a.log_len[sh] = merge ? 0 : m + 1;

    // ---- merge: base <- diag(exp Lam) base + sum_e k~_e u_e^T (base still in registers)
    if (merge) {
        __syncthreads();
        const int ne = MODE == kMergeOnly ? m : m + 1;
        constexpr int G = Map::P < 4 ? Map::P : 4;  // rows per LDS fetch
        // The thread's offset passes through an empty asm statement so the
        // store addresses are formed at the stores (scalar base + one vector
        // offset) instead of being kept live as 64-bit VGPR pairs from the loads.
        uint32_t off0 = tile_off(0);
        asm volatile("" : "+v"(off0));
        auto decay = [&](int p0) {  // rows p0 .. p0+G-1 of the thread
            float ar[G];
            lds_gather<G>(s_ag + r0 * Map::P + p0, ar);
#pragma unroll
            for (int pp = 0; pp < G; ++pp) {
                float4 &x = reg[p0 + pp];
                x.x *= ar[pp];
                x.y *= ar[pp];
                x.z *= ar[pp];
                x.w *= ar[pp];
            }
        };
        auto entry_u = [&](int e) {  // u_e, times the scalar decay factor of a logged entry
            float4 ue = *reinterpret_cast<const float4 *>(s_u + e * DV + col);
            if (!kPerKey && e < m) {
                const float f = s_fac[e];
                ue = make_float4(ue.x * f, ue.y * f, ue.z * f, ue.w * f);
            }
            return ue;
        };
        auto rank1 = [&](int e, float4 ue, int p0) {  // rows p0.. += k~_e[row] u_e
            float kt[G];
            lds_gather<G>(s_ktg + e * DK + r0 * Map::P + p0, kt);
#pragma unroll
            for (int pp = 0; pp < G; ++pp) {
                float4 &x = reg[p0 + pp];
                x.x = fmaf(kt[pp], ue.x, x.x);
                x.y = fmaf(kt[pp], ue.y, x.y);
                x.z = fmaf(kt[pp], ue.z, x.z);
                x.w = fmaf(kt[pp], ue.w, x.w);
            }
        };
        auto store = [&](int p) {
            store_base<MODE == kEager>(S + (off0 + (uint32_t)(p * Map::RPP * DV)), reg[p]);
        };
        if constexpr (MODE == kEager) {
            // every tile is written, a copy-like stream: each group of rows is
            // stored as soon as it is done, so the writes start early
#pragma unroll
            for (int p0 = 0; p0 < Map::P; p0 += G) {
                decay(p0);
                rank1(0, entry_u(0), p0);
#pragma unroll
                for (int pp = 0; pp < G; ++pp) store(p0 + pp);
            }
        } else {
            // few merging tiles: the whole update (entries in order, each u_e
            // read once), then the stores
#pragma unroll
            for (int p0 = 0; p0 < Map::P; p0 += G) decay(p0);
#pragma unroll
            for (int e = 0; e < ML + 1; ++e) {
                if (e < ne) {
                    const float4 ue = entry_u(e);
#pragma unroll
                    for (int p0 = 0; p0 < Map::P; p0 += G) rank1(e, ue, p0);
                }
            }
#pragma unroll
            for (int p = 0; p < Map::P; ++p) store(p);
        }
    }
}

template <int DK, int DV, int VAR, typename TI, typename TO, int MODE>
hipError_t launch_one(const DecodeArgs &a, hipStream_t stream) {
    const int blocks = a.B * a.H;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((decode_kernel<DK, DV, VAR, TI, TO, MODE>), dim3(blocks), dim3(kThreads), 0,
                       stream, a);
    return hipGetLastError();
}

template <int DK, int DV, int VAR, int MODE>
hipError_t dispatch_types(int io, int out, const DecodeArgs &a, hipStream_t s) {
    if (io == kBF16) {
        if (out == kBF16) return launch_one<DK, DV, VAR, bf16, bf16, MODE>(a, s);
        return launch_one<DK, DV, VAR, bf16, float, MODE>(a, s);
    }
    if (out == kBF16) return launch_one<DK, DV, VAR, float, bf16, MODE>(a, s);
    return launch_one<DK, DV, VAR, float, float, MODE>(a, s);
}

template <int DK, int DV, int MODE>
hipError_t dispatch_variant(int variant, int io, int out, const DecodeArgs &a, hipStream_t s) {
    switch (variant) {
        case kScalar: return dispatch_types<DK, DV, kScalar, MODE>(io, out, a, s);
        case kKda: return dispatch_types<DK, DV, kKda, MODE>(io, out, a, s);
        default: return dispatch_types<DK, DV, kRwkv6, MODE>(io, out, a, s);
    }
}

template <int DK, int DV>
hipError_t dispatch_mode(int mode, int variant, int io, int out, const DecodeArgs &a,
                         hipStream_t s) {
    if (mode == kEager) return dispatch_variant<DK, DV, kEager>(variant, io, out, a, s);
    if (mode == kAppend) return dispatch_variant<DK, DV, kAppend>(variant, io, out, a, s);
    // merge only: the output type is unused; KDA and RWKV6 merge alike.
    return dispatch_variant<DK, DV, kMergeOnly>(variant == kScalar ? kScalar : kKda, io, kF32, a,
                                                s);
}

// every value width for one key width (one translation unit per key width,
// so the instances compile in parallel)
template <int DK>
hipError_t dispatch_dv(int mode, int dv, int variant, int io, int out, const DecodeArgs &a,
                       hipStream_t s) {
    switch (dv) {
        case 32: return dispatch_mode<DK, 32>(mode, variant, io, out, a, s);
        case 64: return dispatch_mode<DK, 64>(mode, variant, io, out, a, s);
        default: return dispatch_mode<DK, 128>(mode, variant, io, out, a, s);
    }
}

}  // namespace
}  // namespace gdn
