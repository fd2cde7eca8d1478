// decode.hip -- dispatch of a decode-step launch to the translation unit that
// holds its key width (decode_d32.hip, decode_d64.hip, decode_d128.hip; the
// kernels themselves are in decode_kernels.hpp).

#include "gdn_device.hpp"

namespace gdn {

hipError_t launch_decode_dk32(int mode, int dv, int variant, int io, int out,
                              const DecodeArgs &a, hipStream_t stream);
hipError_t launch_decode_dk64(int mode, int dv, int variant, int io, int out,
                              const DecodeArgs &a, hipStream_t stream);
hipError_t launch_decode_dk128(int mode, int dv, int variant, int io, int out,
                               const DecodeArgs &a, hipStream_t stream);

hipError_t launch_decode(int mode, int dk, int dv, int variant, int io, int out,
                         const DecodeArgs &a, hipStream_t stream) {
    switch (dk) {
        case 32: return launch_decode_dk32(mode, dv, variant, io, out, a, stream);
        case 64: return launch_decode_dk64(mode, dv, variant, io, out, a, stream);
        default: return launch_decode_dk128(mode, dv, variant, io, out, a, stream);
    }
}

}  // namespace gdn
