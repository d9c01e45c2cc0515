// Fused tile decoder instantiated for the fp8 container (kernels in ep_decode.h).
#include "ep_decode.h"

namespace ep {
template hipError_t launch_decode<EP_FP8_E4M3FN>(const DecodeArgs&, int, bool, bool, bool, bool, bool,
                                              int, size_t, hipStream_t);
template hipError_t launch_patch<EP_FP8_E4M3FN>(const uint32_t*, const void*, uint32_t, const float*,
                                      uint32_t, uint32_t, void*, bool, uint32_t*, hipStream_t);
}  // namespace ep
