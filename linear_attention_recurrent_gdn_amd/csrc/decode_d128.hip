// decode_d128.hip -- the decode-step kernel instances with d_k = 128 (every
// d_v, variant, io and output type), one translation unit per key width.

#include "decode_kernels.hpp"

namespace gdn {

hipError_t launch_decode_dk128(int mode, int dv, int variant, int io, int out,
                               const DecodeArgs &a, hipStream_t stream) {
    return dispatch_dv<128>(mode, dv, variant, io, out, a, stream);
}

}  // namespace gdn
