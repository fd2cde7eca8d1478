// prefill_d64.hip -- the chunked-prefill kernel instances with d_k = 64
// (every d_v, variant, io and output type), one translation unit per key
// width.

#include "prefill_kernels.hpp"

namespace gdn {

hipError_t launch_prefill_dk64(int dv, int io, int out, const PrefillArgs &a,
                                hipStream_t stream) {
    return launch_prefill_dk<64>(dv, io, out, a, stream);
}

}  // namespace gdn
