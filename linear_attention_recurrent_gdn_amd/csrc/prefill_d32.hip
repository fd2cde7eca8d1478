// prefill_d32.hip -- the chunked-prefill kernel instances with d_k = 32
// (every d_v, variant, io and output type), one translation unit per key
// width.

#include "prefill_kernels.hpp"

namespace gdn {

hipError_t launch_prefill_dk32(int dv, int io, int out, const PrefillArgs &a,
                                hipStream_t stream) {
    return launch_prefill_dk<32>(dv, io, out, a, stream);
}

}  // namespace gdn
