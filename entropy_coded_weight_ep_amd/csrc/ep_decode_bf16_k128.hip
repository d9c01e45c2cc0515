// Fused tile decoder instantiated for the bf16 container, two rANS states per lane (128 per
// tile; kernels in ep_decode.h).
#include "ep_decode.h"

namespace ep {
template hipError_t launch_decode<EP_BF16, 2>(const DecodeArgs&, int, bool, bool, bool, bool, bool,
                                          int, size_t, hipStream_t);
}  // namespace ep
