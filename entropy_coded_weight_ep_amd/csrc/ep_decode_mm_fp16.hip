// The tile decoder fused into its consumer product, instantiated for the fp16 container with one
// and two rANS states per lane (kernels in ep_decode.h).
#include "ep_decode.h"

namespace ep {
template hipError_t launch_decode_mm<EP_FP16, 1>(const DecodeArgs&, int, bool, bool, bool, int,
                                              size_t, hipStream_t);
template hipError_t launch_decode_mm<EP_FP16, 2>(const DecodeArgs&, int, bool, bool, bool, int,
                                              size_t, hipStream_t);
}  // namespace ep
