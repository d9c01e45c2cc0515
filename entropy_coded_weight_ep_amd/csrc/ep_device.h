// Device-side helpers shared by the HIP translation units of libep.so: rANS constants and the
// container conversions (BF16, FP16, FP8 E4M3FN and INT8 containers, as the EntroPack abstract
// lists them).  Conversions to a container round to nearest even; E4M3FN saturates at +-448,
// INT8 saturates at [-128, 127].
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
__device__ __forceinline__ float fp8e4m3_to_f32(uint32_t b) {
  uint32_t s = (b >> 7) & 1u, e = (b >> 3) & 15u, m = b & 7u;
  float v;
  if (e == 0) v = (float)m * 0.001953125f;                       // m * 2^-9, exact
  else if (e == 15 && m == 7) v = __builtin_nanf("");
  else v = __uint_as_float(((e + 120u) << 23) | (m << 20));       // rebias 7 -> 127
  return s ? -v : v;
}

template <int DT>
__device__ __forceinline__ float widen(uint32_t bits) {
  if constexpr (DT == EP_BF16) {
    return __uint_as_float(bits << 16);
  } else if constexpr (DT == EP_FP16) {
    _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)bits);
    return (float)h;
  } else if constexpr (DT == EP_FP8_E4M3FN) {
    return fp8e4m3_to_f32(bits);
  } else {
    return (float)(int8_t)(uint8_t)bits;
  }
}

// fp32 -> E4M3FN, round to nearest even, saturating at +-448 (NaN -> 0x7F).
__device__ __forceinline__ uint32_t f32_to_fp8e4m3(float y) {
  uint32_t u = __float_as_uint(y);
  uint32_t sign = (u >> 24) & 0x80u;
  float a = __builtin_fabsf(y);
  uint32_t code;
  if (a != a) {
    code = 0x7Fu;
  } else if (a >= 448.0f) {
    code = 0x7Eu;                                                  // saturate
  } else if (a < 0.015625f) {                                      // below 2^-6: subnormal step
    code = (uint32_t)__builtin_rintf(a * 512.0f);                  // 8 -> smallest normal
  } else {
    uint32_t ua = __float_as_uint(a);
    uint32_t r = ua + 0x7FFFFu + ((ua >> 20) & 1u);                // RNE to 3 mantissa bits
    code = (r >> 20) - (120u << 3);
  }
  return sign | code;
}

template <int DT>
__device__ __forceinline__ uint32_t narrow(float y) {
  if constexpr (DT == EP_BF16) {
    return __builtin_bit_cast(uint16_t, (__bf16)y);
  } else if constexpr (DT == EP_FP16) {
    return __builtin_bit_cast(uint16_t, (_Float16)y);
  } else if constexpr (DT == EP_FP8_E4M3FN) {
    return f32_to_fp8e4m3(y);
  } else {
    float r = __builtin_rintf(y);
    r = __builtin_fminf(__builtin_fmaxf(r, -128.0f), 127.0f);
    int32_t q = (y != y) ? 0 : (int32_t)r;
    return (uint32_t)(uint8_t)(int8_t)q;
  }
}

template <int DT>
struct Elem8;  // eight consecutive container elements
template <>
struct Elem8<EP_BF16> { using V = uint4; };
template <>
struct Elem8<EP_FP16> { using V = uint4; };
template <>
struct Elem8<EP_FP8_E4M3FN> { using V = uint2; };
template <>
struct Elem8<EP_INT8> { using V = uint2; };

template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float out[8]) {
  if constexpr (DT == EP_BF16 || DT == EP_FP16) {
    uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
    uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      out[2 * i] = widen<DT>(w[i] & 0xFFFFu);
      out[2 * i + 1] = widen<DT>(w[i] >> 16);
    }
  } else {
    uint2 q = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(base) + elem);
    uint32_t w[2] = {q.x, q.y};
#pragma unroll
    for (int i = 0; i < 8; i++) out[i] = widen<DT>((w[i >> 2] >> (8 * (i & 3))) & 0xFFu);
  }
}

}  // namespace ep
