// Matrix-core decode kernel of libkvq (uniform formats, GQA groups).
#include <hip/hip_runtime.h>

#include "splitk.h"

namespace kvq {

bool mfma_supported(const DecodeArgs&) { return false; }

hipError_t launch_decode_mfma(const DecodeArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace kvq
