// Fused tile decoder instantiated for the fp8 e4m3fn container, two rANS states per lane (128 per
// tile; kernels in ep_decode.h).
#include "ep_decode.h"

namespace ep {
template hipError_t launch_decode<EP_FP8_E4M3FN, 2>(const DecodeArgs&, int, bool, bool, bool, bool, bool,
                                          int, size_t, hipStream_t);
}  // namespace ep
