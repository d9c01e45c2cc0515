// Container loads and widening for the encoder-side kernels of libep.so (row statistics, the
// E8 quantiser): one vector's 8 container values as loaded from memory, and their exact fp32
// values.  Widening is exact for every container (BF16, FP16, FP8 E4M3FN, INT8, FP32).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ep.h"

namespace ep {

template <int DT>
__device__ __forceinline__ float widen(uint32_t bits) {
  if constexpr (DT == EP_BF16) {
    return __uint_as_float(bits << 16);
  } else if constexpr (DT == EP_FP16) {
    _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)bits);
    return (float)h;
  } else if constexpr (DT == EP_FP8_E4M3FN) {
    // gfx950's conversion reads the OCP E4M3FN encoding (exact; S.1111.111 is NaN)
    return __builtin_amdgcn_cvt_f32_fp8((int)bits, 0);
  } else if constexpr (DT == EP_FP32) {
    return __uint_as_float(bits);
  } else {
    return (float)(int8_t)(uint8_t)bits;
  }
}

// The 8 container values of one vector as loaded from memory: 32 bytes (fp32), 16 bytes (bf16,
// fp16) or 8 bytes (fp8, int8).  A vector starts at element 8m of a row whose length is a
// multiple of 8, so its load is aligned whenever the tensor is 16-byte aligned.
struct U32x8 {
  uint4 a, b;
};

template <int DT>
struct RawVec {
  using T = typename std::conditional<
      DT == EP_FP32, U32x8,
      typename std::conditional<(DT == EP_BF16 || DT == EP_FP16), uint4, uint2>::type>::type;
};

template <int DT>
__device__ __forceinline__ typename RawVec<DT>::T raw_load(const void* base, int64_t vec) {
  return reinterpret_cast<const typename RawVec<DT>::T*>(base)[vec];
}

// One container element's bits.
template <int DT>
__device__ __forceinline__ uint32_t elem_bits(const void* base, int64_t i) {
  if constexpr (DT == EP_FP32) return static_cast<const uint32_t*>(base)[i];
  else if constexpr (DT == EP_BF16 || DT == EP_FP16) return static_cast<const uint16_t*>(base)[i];
  else return static_cast<const uint8_t*>(base)[i];
}

// Vector m of a row of `cols` elements starting at element e0, for a width that is not a multiple
// of 8: element loads, and zeros for the coordinates past the row's end.
template <int DT>
__device__ __forceinline__ typename RawVec<DT>::T raw_load_padded(const void* base, int64_t e0,
                                                                  int64_t m, int64_t cols) {
  uint32_t b[8];
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const int64_t c = 8 * m + k;
    b[k] = c < cols ? elem_bits<DT>(base, e0 + c) : 0u;
  }
  typename RawVec<DT>::T q;
  if constexpr (DT == EP_FP32) {
    q.a = make_uint4(b[0], b[1], b[2], b[3]);
    q.b = make_uint4(b[4], b[5], b[6], b[7]);
  } else if constexpr (DT == EP_BF16 || DT == EP_FP16) {
    q = make_uint4(b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16),
                   b[6] | (b[7] << 16));
  } else {
    q = make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24),
                   b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
  }
  return q;
}

template <int DT>
__device__ __forceinline__ typename RawVec<DT>::T raw_zero() {
  typename RawVec<DT>::T z;
  __builtin_memset(&z, 0, sizeof(z));
  return z;
}

template <int DT>
__device__ __forceinline__ void raw_widen(const typename RawVec<DT>::T& q, float out[8]) {
  if constexpr (DT == EP_FP32) {
    const uint32_t w[8] = {q.a.x, q.a.y, q.a.z, q.a.w, q.b.x, q.b.y, q.b.z, q.b.w};
#pragma unroll
    for (int i = 0; i < 8; i++) out[i] = __uint_as_float(w[i]);
  } else if constexpr (DT == EP_BF16 || DT == EP_FP16) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      out[2 * i] = widen<DT>(w[i] & 0xFFFFu);
      out[2 * i + 1] = widen<DT>(w[i] >> 16);
    }
  } else if constexpr (DT == EP_FP8_E4M3FN) {
    out[0] = __builtin_amdgcn_cvt_f32_fp8((int)q.x, 0);
    out[1] = __builtin_amdgcn_cvt_f32_fp8((int)q.x, 1);
    out[2] = __builtin_amdgcn_cvt_f32_fp8((int)q.x, 2);
    out[3] = __builtin_amdgcn_cvt_f32_fp8((int)q.x, 3);
    out[4] = __builtin_amdgcn_cvt_f32_fp8((int)q.y, 0);
    out[5] = __builtin_amdgcn_cvt_f32_fp8((int)q.y, 1);
    out[6] = __builtin_amdgcn_cvt_f32_fp8((int)q.y, 2);
    out[7] = __builtin_amdgcn_cvt_f32_fp8((int)q.y, 3);
  } else {
    const uint32_t w[2] = {q.x, q.y};
#pragma unroll
    for (int i = 0; i < 8; i++) out[i] = widen<DT>((w[i >> 2] >> (8 * (i & 3))) & 0xFFu);
  }
}

}  // namespace ep
