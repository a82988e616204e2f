// Placeholder until the matrix-core decode kernel lands.
#include "decode_common.h"

namespace sr {

hipError_t launch_decode_mfma(const sr_shape&, const DecodeArgs&, int, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace sr
