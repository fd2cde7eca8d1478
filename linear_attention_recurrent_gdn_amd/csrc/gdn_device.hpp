// gdn_device.hpp -- device-side helpers shared by the gfx950 kernels:
// element loads/stores for the io dtypes, wave64 reductions, and the
// internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kWave = 64;

// bf16 is carried as its 16-bit pattern; widening is exact.
struct bf16 {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) {
    return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}

template <typename T>
__device__ __forceinline__ T from_f32(float x);

template <>
__device__ __forceinline__ float from_f32<float>(float x) {
    return x;
}

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return bf16{static_cast<uint16_t>((u >> 16) | 0x40u)};
    const uint32_t r = u + 0x7fffu + ((u >> 16) & 1u);
    return bf16{static_cast<uint16_t>(r >> 16)};
}

// Sum over the lanes of a wave whose lane index agrees modulo `stride`
// (stride a power of two, < 64): after the call every such lane holds the
// total of its class.
template <int STRIDE>
__device__ __forceinline__ float wave_sum_strided(float x) {
#pragma unroll
    for (int off = STRIDE; off < kWave; off <<= 1) x += __shfl_xor(x, off, kWave);
    return x;
}

__device__ __forceinline__ float wave_sum(float x) { return wave_sum_strided<1>(x); }

__device__ __forceinline__ float quiet_nan() { return __uint_as_float(0x7fc00000u); }

// Streaming (non-temporal) 16-byte load / store for data touched once per
// launch: the state tiles of the decode step. Keeps the caches for data that
// is re-read (logs, inputs).
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 load_stream(const float *p) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store_stream(float *p, float4 x) {
    f32x4 v = {x.x, x.y, x.z, x.w};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(p));
}

// ---------------------------------------------------------------- launch API
enum Variant { kScalar = 0, kKda = 1, kRwkv6 = 2 };
enum DType { kF32 = 0, kBF16 = 1 };

struct DecodeArgs {
    const void *q, *k, *v;
    const float *log_alpha, *beta;
    float *state;        // eager state, or deferred base
    float *log_u;        // [slots, H, Mcap, dv]
    void *log_k;         // [slots, H, Mcap, dk] io dtype
    float *log_lam;      // [slots, H, Mcap] or [slots, H, Mcap, dk]
    int32_t *log_len;    // [slots, H]
    const int32_t *slot_idx;
    void *o;
    int B, H, n_slots, Mcap, merge_at, min_len;
};

// mode: 0 eager step, 1 deferred append (with merge on the merging steps),
// 2 merge only.
hipError_t launch_decode(int mode, int dk, int dv, int variant, int io,
                         int out, const DecodeArgs &a, hipStream_t stream);

struct PrefillArgs {
    const void *q, *k, *v;
    const float *log_alpha, *beta;
    const int32_t *cu;      // [n_seq + 1]
    const int32_t *parent;  // [n_seq] or null (identity)
    const float *conv_w;    // [CC, 4] or null
    const float *state_in;  // [*, H, dk, dv] or null
    const void *win_in;     // [*, 3, CC] or null
    void *o;                // [N, H, dv] or null
    float *state_out;       // [n_seq, H, dk, dv] or null
    void *win_out;          // [n_seq, 3, CC] or null
    void *ws;
    size_t ws_bytes;
    int n_seq, n_parent, n_tokens, H, qk_norm, chunk;
    int dv;                 // value width (the key width is a template parameter)
    int variant;            // Variant: scalar log a [N, H], or per-key [N, H, dk]
    // checkpoints: state / window after every ckpt_every chunks, at most
    // ckpt_cap per sequence ([n_seq, ckpt_cap, H, dk, dv] / [n_seq, ckpt_cap, 3, CC])
    float *ckpt_state;      // or null
    void *ckpt_window;      // or null
    int ckpt_every, ckpt_cap;
    // set by the launcher: for branch calls [count, first branch of each
    // group..., n_seq] (groups of branches of one parent), or null; the
    // segment being run and the number of segments of the prefill
    const int32_t *groups;
    int seg, nseg;
    // set by the launcher: sequences of at most one chunk run in the
    // one-chunk kernel (the chunked kernels skip them); the branch group
    // size
    int fuse1, group_size;
};

size_t prefill_workspace_bytes(int n_tokens, int n_seq, int H, int dk, int dv,
                               int chunk, int variant);
hipError_t launch_prefill(int dk, int dv, int io, int out, const PrefillArgs &a,
                          hipStream_t stream);

// Streaming read (copy = 0) or copy (copy = 1) of n_bytes (a multiple of 16).
hipError_t launch_stream_probe(const void *src, void *dst, size_t n_bytes, int copy,
                               hipStream_t stream);

}  // namespace gdn
