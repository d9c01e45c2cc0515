// The tile decoder with its per-phase clock trace, instantiated for the bf16 and fp8 containers with
// one and two rANS states per lane (kernels in ep_decode.h).
#include "ep_decode.h"

namespace ep {
template hipError_t launch_decode_trace<EP_BF16, 1>(const DecodeArgs&, int, bool, bool, int, size_t,
                                                   hipStream_t);
template hipError_t launch_decode_trace<EP_BF16, 2>(const DecodeArgs&, int, bool, bool, int, size_t,
                                                   hipStream_t);
template hipError_t launch_decode_trace<EP_FP8_E4M3FN, 1>(const DecodeArgs&, int, bool, bool, int,
                                                         size_t, hipStream_t);
template hipError_t launch_decode_trace<EP_FP8_E4M3FN, 2>(const DecodeArgs&, int, bool, bool, int,
                                                         size_t, hipStream_t);
}  // namespace ep
