// prefill_d128.hip -- the chunked-prefill kernel instances with d_k = 128
// (every d_v, variant, io and output type), one translation unit per key
// width.

#include "prefill_kernels.hpp"

namespace gdn {

hipError_t launch_prefill_dk128(int dv, int io, int out, const PrefillArgs &a,
                                hipStream_t stream) {
    return launch_prefill_dk<128>(dv, io, out, a, stream);
}

}  // namespace gdn
