// probe.hip -- a measurement aid beside the recurrence kernels: a plain
// streaming read or copy of a device buffer with the same access form the
// decode step uses for its state (non-temporal 16-byte loads and stores),
// so the attainable HBM rate of this GPU is measured next to the kernels'
// own figures instead of being taken from a library copy.

#include "gdn_device.hpp"

namespace gdn {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 16;                           // 16-byte loads per thread
constexpr int kProbeTile = kProbeThreads * kProbeUnroll;   // float4s per workgroup (64 KiB)

// One workgroup per 64 KiB tile, each thread with its 16 loads in flight at
// once -- the decode step's shape (one workgroup streams one 64 KiB state
// tile). Read mode folds the data into one value per thread that is stored
// only when it equals a bit pattern the caller never supplies (so the loads
// cannot be dropped and nothing is written in practice); copy mode writes
// every element to dst. Addresses past the end are clamped (loads) or
// skipped (stores).
template <bool COPY>
__global__ __launch_bounds__(kProbeThreads) void stream_probe_kernel(const float *src, float *dst,
                                                                     size_t n4) {
    const size_t base = (size_t)blockIdx.x * kProbeTile + threadIdx.x;
    float4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
        size_t i = base + (size_t)u * kProbeThreads;
        i = i < n4 ? i : n4 - 1;
        v[u] = load_stream(src + 4 * i);
    }
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
        const size_t i = base + (size_t)u * kProbeThreads;
        if (COPY) {
            if (i < n4) store_stream(dst + 4 * i, v[u]);
        } else {
            acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
        }
    }
    if (!COPY && __float_as_uint(acc) == 0x7fbadbadu) dst[0] = acc;
}

}  // namespace

hipError_t launch_stream_probe(const void *src, void *dst, size_t n_bytes, int copy,
                               hipStream_t stream) {
    const size_t n4 = n_bytes / 16;
    if (n4 == 0) return hipSuccess;
    const size_t blocks = (n4 + kProbeTile - 1) / kProbeTile;
    if (blocks > 0x7fffffffu) return hipErrorInvalidValue;
    const float *s = static_cast<const float *>(src);
    float *d = static_cast<float *>(dst);
    if (copy)
        hipLaunchKernelGGL(stream_probe_kernel<true>, dim3((unsigned)blocks), dim3(kProbeThreads), 0,
                           stream, s, d, n4);
    else
        hipLaunchKernelGGL(stream_probe_kernel<false>, dim3((unsigned)blocks),
                           dim3(kProbeThreads), 0, stream, s, d, n4);
    return hipGetLastError();
}

}  // namespace gdn
