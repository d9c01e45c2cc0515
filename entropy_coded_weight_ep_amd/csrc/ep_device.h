// Device-side helpers of the decoder and the other HIP translation units of libep.so: rANS
// constants and the conversions to a container (BF16, FP16, FP8 E4M3FN and INT8 containers, as
// the EntroPack abstract lists them, and FP32).  Conversions to a container round to nearest
// even; E4M3FN saturates at +-448, INT8 saturates at [-128, 127]; FP32 is stored as is.
// (Loading and widening containers, for the encoder kernels, is in ep_load.h.)
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ep.h"

namespace ep {

constexpr uint32_t kL = 1u << 16;         // rANS lower bound: states live in [2^16, 2^32)
constexpr uint32_t kM = 1u << EP_PRECISION;
constexpr uint32_t kMask = kM - 1u;

// ------------------------------------------------------------------------------------------
// Containers
// ------------------------------------------------------------------------------------------
// fp32 -> bf16 / fp16, round to nearest even (hardware conversions; fp16 overflow -> inf).
template <int DT>
__device__ __forceinline__ uint32_t narrow(float y) {
  static_assert(DT == EP_BF16 || DT == EP_FP16, "fp8 and int8 are converted in the decoder");
  if constexpr (DT == EP_BF16) return __builtin_bit_cast(uint16_t, (__bf16)y);
  else return __builtin_bit_cast(uint16_t, (_Float16)y);
}

// Two fp32 values -> packed pair (low half: a), round to nearest even: one packed conversion.
template <int DT>
__device__ __forceinline__ uint32_t narrow2(float a, float b) {
  static_assert(DT == EP_BF16 || DT == EP_FP16, "16-bit containers only");
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {a, b};
  if constexpr (DT == EP_BF16) {
    typedef __bf16 b16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b16x2));
  } else {
    typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h16x2));
  }
}

}  // namespace ep
