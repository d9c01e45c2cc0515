// Fused tile decoder instantiated for the fp8 e4m3fn container, one rANS state per lane (64 per tile),
// with and without the saturation clamp (bounded blobs), and the escape patch launcher (kernels in
// ep_decode.h).
#include "ep_decode.h"

namespace ep {
template hipError_t launch_decode<EP_FP8_E4M3FN, 1>(const DecodeArgs&, int, bool, bool, bool, bool, bool,
                                          int, size_t, hipStream_t);
template hipError_t launch_decode<kFp8Bounded, 1>(const DecodeArgs&, int, bool, bool, bool, bool, bool,
                                        int, size_t, hipStream_t);
template hipError_t launch_patch<EP_FP8_E4M3FN>(const uint32_t*, const void*, uint32_t, const float*,
                                      uint32_t, uint32_t, void*, bool, uint32_t*, hipStream_t);
}  // namespace ep
