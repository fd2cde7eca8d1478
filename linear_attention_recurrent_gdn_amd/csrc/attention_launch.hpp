// attention_launch.hpp -- internal launch interface of the fork-attention
// kernels (attention.hip) for the C ABI (api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

struct AttnArgs {
    const void *q;             // [n_tokens, H, d] bf16
    const void *k, *v;         // [n_tokens, H_kv, d] bf16
    const int32_t *cu;         // [n_req + 1] trunk offsets (absolute)
    const int32_t *bcu;        // [n_branch + 1] branch offsets (absolute)
    const int32_t *bparent;    // [n_branch] request of each branch
    void *o;                   // [n_tokens, H, d]
    void *ws;                  // int32 tile table [n_req + n_branch + 1]
    int n_req, n_branch, n_tokens, H, Hkv;
    float scale;
    int trunk_queries;         // 0: trunk rows give keys/values only
};

size_t attention_workspace_bytes(int n_req, int n_branch);

// Segments (n_req + n_branch) the allocation-free entry point's file-scope
// tile table holds.
constexpr int kAttnScratchSegments = 65536;

// The calling thread's current device's copy of that table (its address is
// looked up once per device, with the device current) and its size in bytes.
hipError_t attention_scratch(void **ptr, size_t *bytes);
hipError_t launch_attention(int d, int out, const AttnArgs &a, hipStream_t stream);

}  // namespace gdn
