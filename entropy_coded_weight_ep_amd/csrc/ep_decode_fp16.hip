// Fused tile decoder instantiated for the fp16 container (kernels in ep_decode.h).
#include "ep_decode.h"

namespace ep {
template hipError_t launch_decode<EP_FP16>(const DecodeArgs&, int, bool, bool, bool, bool, bool,
                                              int, size_t, hipStream_t);
template hipError_t launch_patch<EP_FP16>(const uint32_t*, const void*, uint32_t, const float*,
                                      uint32_t, uint32_t, void*, bool, uint32_t*, hipStream_t);
}  // namespace ep
