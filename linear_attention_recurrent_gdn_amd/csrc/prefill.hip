// prefill.hip -- workspace size of the chunked prefill and dispatch of a
// launch to the translation unit that holds its key width (prefill_d32.hip,
// prefill_d64.hip, prefill_d128.hip; the kernels are in prefill_kernels.hpp).

#include "prefill_kernels.hpp"

namespace gdn {

hipError_t launch_prefill_dk32(int dv, int io, int out, const PrefillArgs &a,
                               hipStream_t stream);
hipError_t launch_prefill_dk64(int dv, int io, int out, const PrefillArgs &a,
                               hipStream_t stream);
hipError_t launch_prefill_dk128(int dv, int io, int out, const PrefillArgs &a,
                                hipStream_t stream);

size_t prefill_workspace_bytes(int n_tokens, int n_seq, int H, int dk, int dv, int chunk,
                               int variant) {
    (void)chunk;
    const bool pk = variant != kScalar;
    return ws_layout(n_tokens, n_seq, H, dk, dv, pk, prefill_segments(n_tokens, n_seq, H, dk, pk))
        .total;
}

hipError_t launch_prefill(int dk, int dv, int io, int out, const PrefillArgs &a,
                          hipStream_t stream) {
    switch (dk) {
        case 32: return launch_prefill_dk32(dv, io, out, a, stream);
        case 64: return launch_prefill_dk64(dv, io, out, a, stream);
        default: return launch_prefill_dk128(dv, io, out, a, stream);
    }
}

}  // namespace gdn
