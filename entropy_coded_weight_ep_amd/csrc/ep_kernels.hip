// HIP kernels (gfx950) of the lattice-rANS weight codec and their C-ABI entry points.
//
// What is computed follows the EntroPack design page "EntroPack lattice compression"
// (sections "Lattice quantization and integer fields" and "Encoding and reconstruction") and the
// EntroPack abstract (fused GPU symbol decoding and weight reconstruction; BF16/FP16/FP8/INT8
// containers).  The kernels are written for CDNA4: wave64, LDS-staged tables and words,
// wavefront ballot/prefix renormalisation, 16-byte stores.
//
// Build: hipcc --offload-arch=gfx950 -O3 -ffp-contract=off (the E8 quantiser and the row sums
// must round every product and sum separately so that their results are reproducible).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "ep.h"
#include "ep_device.h"
#include "ep_load.h"
#include "ep_internal.h"

namespace ep {

// ------------------------------------------------------------------------------------------
// Row sums of squares: one lane per row, left-to-right fp64 accumulation (each square is exact
// in fp64 for every container, so the sum is reproducible).  The chain is serial per row, so a
// lane streams its own row: the next chunk of kRowChunk vectors is loaded (8- or 16-byte loads)
// while the current one is summed, which keeps the loads off the chain's critical path.
// ------------------------------------------------------------------------------------------
constexpr int kRowChunk = 8;                       // vectors per lane per prefetch stage

// PAD: a width that is not a multiple of 8; the zeros past the row's end add exactly nothing.
template <int DT, bool PAD>
__device__ __forceinline__ typename RawVec<DT>::T row_vec(const void* w, int64_t r, int64_t cols,
                                                          int64_t vpr, int64_t m) {
  if constexpr (PAD) return raw_load_padded<DT>(w, r * cols, m, cols);
  else return raw_load<DT>(w, r * vpr + m);
}

template <int DT, bool PAD>
__global__ __launch_bounds__(64) void k_row_sumsq(const void* __restrict__ w, int64_t rows,
                                                  int64_t cols, double* __restrict__ out) {
  using Raw = typename RawVec<DT>::T;
  const int64_t r = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (r >= rows) return;
  const int64_t vpr = (cols + 7) / 8;
  // loads past the row's end re-read its last vector (never summed): no branch around a load,
  // so the wait before a chunk covers only that chunk's loads, not the prefetch behind it
  auto vec = [&](int64_t m) { return row_vec<DT, PAD>(w, r, cols, vpr, m < vpr ? m : vpr - 1); };
  Raw cur[kRowChunk], nxt[kRowChunk];
#pragma unroll
  for (int k = 0; k < kRowChunk; k++) cur[k] = vec(k);
  double acc = 0.0;
  for (int64_t v0 = 0; v0 < vpr; v0 += kRowChunk) {
    const int64_t v1 = v0 + kRowChunk;
#pragma unroll
    for (int k = 0; k < kRowChunk; k++) nxt[k] = vec(v1 + k);
#pragma unroll
    for (int k = 0; k < kRowChunk; k++) {
      if (v0 + k < vpr) {
        float x[8];
        raw_widen<DT>(cur[k], x);
#pragma unroll
        for (int i = 0; i < 8; i++) {
          const double v = (double)x[i];
          acc = __dadd_rn(acc, __dmul_rn(v, v));
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kRowChunk; k++) cur[k] = nxt[k];
  }
  out[r] = acc;
}

// ------------------------------------------------------------------------------------------
// E8 nearest point (Conway & Sloane 1982 fast quantiser for D8 u (D8 + 1/2)): round each
// coordinate half-to-even; if the coordinate sum is odd, move the worst-rounded coordinate
// (lowest index among equals) one step towards x (upwards for a zero residual).  Candidates
// for x and for x - 1/2; the closer one wins, coset 0 on ties.  Every operation is a single
// IEEE fp32 op (no contraction), distances summed e0^2 + e1^2 + ... in index order.
// ------------------------------------------------------------------------------------------
// Branch-free: every lane computes the residuals and the worst coordinate, and the move is a
// select (an odd sum is about every other vector, so a branch would diverge in every wavefront).
// The worst coordinate is the first whose |residual| equals the largest one: one maximum over
// the eight magnitudes, one compare per coordinate, and the "first hit" kept in lane masks
// (scalar ops), instead of a running compare-and-select of (residual, index).
// The residual u - rint(u) is exact and never -0 (x - x rounds to +0), so copysign(1, r_k) is
// the step towards u, +1 for a zero residual.
// The coordinate sum is formed in fp32: the eight rounded values are integers of magnitude at
// most 65537 (|x| <= 65536 is checked before), so every partial sum is exact and one conversion
// gives the parity (the sign of a zero partial sum does not change it).
__device__ __forceinline__ void d8_round(const float u[8], float a[8]) {
  float r[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    a[i] = __builtin_rintf(u[i]);
    r[i] = __fsub_rn(u[i], a[i]);
  }
  float fsum = __fadd_rn(a[0], a[1]);
#pragma unroll
  for (int i = 2; i < 8; i++) fsum = __fadd_rn(fsum, a[i]);
  const bool odd = ((int32_t)fsum & 1) != 0;
  // the largest |r|: max(a, b) = med3(a, b, 1) since every |r| is at most 1/2 (one instruction
  // each, where fmaxf would add a canonicalisation of every operand)
  auto mx = [](float a, float b) { return __builtin_amdgcn_fmed3f(a, b, 1.0f); };
  const float m = mx(mx(mx(__builtin_fabsf(r[0]), __builtin_fabsf(r[1])),
                        mx(__builtin_fabsf(r[2]), __builtin_fabsf(r[3]))),
                     mx(mx(__builtin_fabsf(r[4]), __builtin_fabsf(r[5])),
                        mx(__builtin_fabsf(r[6]), __builtin_fabsf(r[7]))));
  bool done = !odd;                                // an even sum moves nothing
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const bool hit = !done && __builtin_fabsf(r[i]) == m;
    done = done || hit;
    a[i] = hit ? __fadd_rn(a[i], __builtin_copysignf(1.0f, r[i])) : a[i];
  }
}

__device__ __forceinline__ float sqdist8(const float x[8], const float p[8]) {
  float e = __fsub_rn(x[0], p[0]);
  float d = __fmul_rn(e, e);
#pragma unroll
  for (int i = 1; i < 8; i++) {
    e = __fsub_rn(x[i], p[i]);
    d = __fadd_rn(d, __fmul_rn(e, e));
  }
  return d;
}

// Returns the coset; z receives the D8 part (p - coset/2) as integer-valued floats.
__device__ __forceinline__ int e8_nearest(const float x[8], float z[8]) {
  float A[8], u[8], Bz[8], B[8];
  d8_round(x, A);
#pragma unroll
  for (int i = 0; i < 8; i++) u[i] = __fsub_rn(x[i], 0.5f);
  d8_round(u, Bz);
#pragma unroll
  for (int i = 0; i < 8; i++) B[i] = __fadd_rn(Bz[i], 0.5f);
  const float dA = sqdist8(x, A);
  const float dB = sqdist8(x, B);
  const int c = (dA <= dB) ? 0 : 1;
#pragma unroll
  for (int i = 0; i < 8; i++) z[i] = c ? Bz[i] : A[i];
  return c;
}

// Histogram privatisation window in LDS: values [-256, 255] of every table.  Tables are laid
// out 514 counters apart, which puts the coset-1 table of a field 16 banks away from the coset-0
// one: the most frequent bins of the two (values near 0) do not share an LDS bank.
constexpr int kHistWin = 512;
constexpr int kHistOff = 256;
constexpr int kHistStride = 514;
// The hottest bins: values [-16, 15] of the 16 field tables in four copies, copy = lane & 3, so
// that at most 16 lanes of a wavefront add to the same counter (the ds_add of many lanes to one
// address is serialised).  Tables 33 counters apart, copies 528 apart (16 banks).
constexpr int kNarrowWin = 32;
constexpr int kNarrowOff = 16;
constexpr int kNarrowStride = 33;
constexpr int kNarrowCopies = 4;
constexpr int kNarrowBins = kNarrowCopies * 16 * kNarrowStride;

// Clears n16 16-byte words, one store per thread (the histogram's 4.25 MiB in 1088 workgroups).
__global__ __launch_bounds__(256) void k_zero16(uint4* __restrict__ p, int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n16) p[i] = uint4{0u, 0u, 0u, 0u};
}

__global__ __launch_bounds__(256) void k_fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = v;
}

// Two 16-bit lanes added separately (a packed add: no carry from the low half into the high).
typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_add16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t,
                            __builtin_bit_cast(u16x2_t, a) + __builtin_bit_cast(u16x2_t, b));
}

// One vector's input, fetched one iteration ahead of its use: raw container bits, the row gain,
// and whether the row index was valid.
template <int DT>
struct QIn {
  typename RawVec<DT>::T raw;
  float g;
  bool ok;
};

// Where vector v lies: selected row i = v / vpr and vector m = v mod vpr within it.  The first
// position is divided out exactly (fp64 estimate, one correction); the grid stride then moves it
// by the constant quotient and remainder of stride / vpr, with one carry.
struct QPos {
  uint32_t i, m;
};

__device__ __forceinline__ QPos q_pos(uint32_t v, uint32_t vpr, double inv_vpr) {
  uint32_t i = (uint32_t)((double)v * inv_vpr);
  const int64_t rem = (int64_t)v - (int64_t)i * vpr;
  i = rem < 0 ? i - 1 : (rem >= (int64_t)vpr ? i + 1 : i);
  return QPos{i, v - i * vpr};
}

__device__ __forceinline__ QPos q_advance(QPos p, QPos step, uint32_t vpr) {
  p.i += step.i;
  p.m += step.m;                                   // < 2 vpr: both terms are below vpr
  const bool carry = p.m >= vpr;
  return QPos{carry ? p.i + 1 : p.i, carry ? p.m - vpr : p.m};
}

template <int DT, bool PAD>
__device__ __forceinline__ QIn<DT> q_fetch(const void* __restrict__ w, int64_t rows,
                                           int64_t cols, const float* __restrict__ gain,
                                           const int64_t* __restrict__ row_index, QPos p,
                                           uint32_t vpr) {
  QIn<DT> q;
  const uint32_t i = p.i, m = p.m;
  const int64_t r = row_index ? row_index[i] : (int64_t)i;
  q.ok = r >= 0 && r < rows;
  q.raw = raw_zero<DT>();
  q.g = 0.0f;
  if (q.ok) {
    q.raw = row_vec<DT, PAD>(w, r, cols, vpr, (int64_t)m);
    q.g = gain[r];
  }
  return q;
}

// E8 quantiser + fused per-(coset, field) histogram.  A workgroup of 16 wavefronts walks the
// vectors with a grid stride, fetching the next vector's input before quantising the current
// one.  The histogram is privatised per workgroup in LDS (values [-256, 255] of every table; the
// rest go straight to the global counts) and merged once at the end; the coset table's two
// counts are kept per lane and summed per wavefront at the end.  Few, large workgroups keep the
// merge short, and each workgroup starts its merge at a different bin so that they do not all
// hit the same global counters at once.
constexpr int kQThreads = 1024;

template <int DT, bool PAD>
__global__ __launch_bounds__(kQThreads) void k_quantize_e8(
    const void* __restrict__ w, int64_t rows, int64_t cols, const float* __restrict__ gain,
    const int64_t* __restrict__ row_index, uint32_t n_vec, uint32_t vpr, double inv_vpr,
    uint8_t* __restrict__ coset, int16_t* __restrict__ fields, uint32_t* __restrict__ hist,
    uint32_t* __restrict__ err) {
  __shared__ uint32_t sh[EP_NTABLES * kHistStride];
  __shared__ uint32_t sn[kNarrowBins];
  const bool do_hist = hist != nullptr;
  if (do_hist) {
    for (int i = threadIdx.x; i < EP_NTABLES * kHistStride; i += kQThreads) sh[i] = 0;
    for (int i = threadIdx.x; i < kNarrowBins; i += kQThreads) sn[i] = 0;
    __syncthreads();
  }
  bool bad = false, bad_row = false;
  uint32_t n_c0 = 0, n_c1 = 0;
  const uint32_t stride = gridDim.x * (uint32_t)kQThreads;
  uint32_t v = blockIdx.x * (uint32_t)kQThreads + threadIdx.x;
  const QPos step = q_pos(stride, vpr, inv_vpr);
  QPos pos = q_pos(v, vpr, inv_vpr);
  // The loads of the next vector are issued at the top of an iteration and the stores of the
  // previous one right after them, so that both complete during this iteration's arithmetic:
  // while loads and stores are both outstanding the compiler can only wait for all of them at
  // once, which it does before the next iteration.
  QIn<DT> nxt;
  if (v < n_vec) nxt = q_fetch<DT, PAD>(w, rows, cols, gain, row_index, pos, vpr);
  bool has_prev = false;
  uint32_t v_prev = 0, c_prev = 0;
  uint4 pk_prev = uint4{0u, 0u, 0u, 0u};
  for (; v < n_vec; v += stride) {
    const QIn<DT> cur = nxt;                       // fetched one iteration ago
    const bool more = v + stride < n_vec;         // (no overflow: n_vec + stride < 2^32)
    pos = q_advance(pos, step, vpr);               // the position of v + stride
    if (more) nxt = q_fetch<DT, PAD>(w, rows, cols, gain, row_index, pos, vpr);
    if (has_prev) {
      coset[v_prev] = (uint8_t)c_prev;
      reinterpret_cast<uint4*>(fields)[v_prev] = pk_prev;
    }
    has_prev = false;
    if (!cur.ok) {                                // a row index outside the tensor: skip, report
      bad_row = true;
    } else {
      float x[8];
      raw_widen<DT>(cur.raw, x);
      // !(|x| <= 65536) for all eight at once: the bit patterns without their sign compare
      // as unsigned integers in the order of |x|, with infinities and NaNs above every finite
      // value
      uint32_t mag = 0;
#pragma unroll
      for (int k = 0; k < 8; k++) {
        x[k] = __fmul_rn(x[k], cur.g);
        const uint32_t b = __float_as_uint(x[k]) << 1;
        mag = mag > b ? mag : b;
      }
      bool out_of_range = mag > (0x47800000u << 1);   // 65536.0f
      if (out_of_range) {
#pragma unroll
        for (int k = 0; k < 8; k++) x[k] = 0.0f;
      }
      float zf[8];
      int c = e8_nearest(x, zf);
      // a coordinate outside [-32767, 32767]: one maximum over the magnitudes (integers below
      // 2^17 here, so the fp32 compare is exact) instead of two integer compares per coordinate
      const float zmax = fmaxf(fmaxf(fmaxf(__builtin_fabsf(zf[0]), __builtin_fabsf(zf[1])),
                                     fmaxf(__builtin_fabsf(zf[2]), __builtin_fabsf(zf[3]))),
                               fmaxf(fmaxf(__builtin_fabsf(zf[4]), __builtin_fabsf(zf[5])),
                                     fmaxf(__builtin_fabsf(zf[6]), __builtin_fabsf(zf[7]))));
      out_of_range |= zmax > 32767.0f;
      int32_t z[8];
#pragma unroll
      for (int k = 0; k < 8; k++) z[k] = (int32_t)zf[k];
      bad |= out_of_range;
      int32_t f[8];
#pragma unroll
      for (int k = 0; k < 7; k++) f[k] = z[k];
      f[7] = z[7] >> 1;                           // arithmetic shift = floor(z7 / 2)
      uint4 pk;
      pk.x = (uint32_t)(f[0] & 0xFFFF) | ((uint32_t)f[1] << 16);
      pk.y = (uint32_t)(f[2] & 0xFFFF) | ((uint32_t)f[3] << 16);
      pk.z = (uint32_t)(f[4] & 0xFFFF) | ((uint32_t)f[5] << 16);
      pk.w = (uint32_t)(f[6] & 0xFFFF) | ((uint32_t)f[7] << 16);
      if (out_of_range) {                         // flagged: written as coset 0, fields 0, and
        c = 0;                                    // left out of the histogram
        pk = uint4{0u, 0u, 0u, 0u};
      }
      has_prev = true;                            // written in the next iteration
      v_prev = v;
      c_prev = (uint32_t)c;
      pk_prev = pk;
      if (do_hist && !out_of_range) {
        n_c1 += (uint32_t)c;
        n_c0 += 1u - (uint32_t)c;
        // bins of value 0 of this vector's coset tables (field k at + k * kHistStride)
        uint32_t* const hc = sh + (1 + 8 * c) * kHistStride + kHistOff;
        // window tests on the packed 16-bit fields (halfword adds, no carry between halves):
        // f + 16 in [0, 32) and f + 256 in [0, 512) for all eight
        static_assert(kNarrowOff == 16 && kNarrowWin == 32 && kHistOff == 256 && kHistWin == 512,
                      "the masks below encode these windows");
        const uint32_t orn = pk_add16(pk.x, 0x00100010u) | pk_add16(pk.y, 0x00100010u) |
                             pk_add16(pk.z, 0x00100010u) | pk_add16(pk.w, 0x00100010u);
        const uint32_t orr = pk_add16(pk.x, 0x01000100u) | pk_add16(pk.y, 0x01000100u) |
                             pk_add16(pk.z, 0x01000100u) | pk_add16(pk.w, 0x01000100u);
        // the hottest-bin copies take a wavefront's vectors only when every one of them fits
        // there: a mixed wavefront would run both paths, twice the LDS adds
        if (__ballot((orn & 0xFFE0FFE0u) != 0u) == 0ull) {   // every field among the hottest
          uint32_t* const hn =
              sn + ((threadIdx.x & (kNarrowCopies - 1)) * 16 + 8 * c) * kNarrowStride + kNarrowOff;
#pragma unroll
          for (int k = 0; k < 8; k++) atomicAdd(&hn[k * kNarrowStride + f[k]], 1u);
        } else if ((orr & 0xFE00FE00u) == 0u) {   // every field inside the window
#pragma unroll
          for (int k = 0; k < 8; k++) atomicAdd(&hc[k * kHistStride + f[k]], 1u);
        } else {
#pragma unroll
          for (int k = 0; k < 8; k++) {
            const int32_t val = f[k];
            if ((uint32_t)(val + kHistOff) < (uint32_t)kHistWin)
              atomicAdd(&hc[k * kHistStride + val], 1u);
            else
              atomicAdd(&hist[(int64_t)(1 + 8 * c + k) * EP_HIST_BINS + (val + 32768)], 1u);
          }
        }
      }
    }
  }
  if (has_prev) {
    coset[v_prev] = (uint8_t)c_prev;
    reinterpret_cast<uint4*>(fields)[v_prev] = pk_prev;
  }
  if (bad) atomicOr(err, 1u << EP_ERR_RANGE);
  if (bad_row) atomicOr(err, 1u << EP_ERR_ARG);
  if (do_hist) {
    // the coset counts summed over the wavefront first: one LDS add per wavefront (the adds of
    // all 1024 lanes to the same two counters are serialised, and took a quarter of the kernel)
    uint32_t s0 = n_c0, s1 = n_c1;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
      s0 += __shfl_xor(s0, d, 64);
      s1 += __shfl_xor(s1, d, 64);
    }
    if ((threadIdx.x & 63) == 0) {
      if (s0) atomicAdd(&sh[kHistOff + 0], s0);
      if (s1) atomicAdd(&sh[kHistOff + 1], s1);
    }
    __syncthreads();
    // fold the copies of the hottest bins into the window (one thread per bin)
    for (int i = threadIdx.x; i < 16 * kNarrowWin; i += kQThreads) {
      const int tf = i / kNarrowWin, b = i % kNarrowWin;
      uint32_t sum = 0;
#pragma unroll
      for (int cp = 0; cp < kNarrowCopies; cp++) sum += sn[(cp * 16 + tf) * kNarrowStride + b];
      sh[(1 + tf) * kHistStride + kHistOff + (b - kNarrowOff)] += sum;
    }
    __syncthreads();
    constexpr int kBins = EP_NTABLES * kHistStride;
    const int rot = (int)((blockIdx.x * 1031u) % (uint32_t)kBins);
    for (int j = threadIdx.x; j < kBins; j += kQThreads) {
      const int i = j + rot < kBins ? j + rot : j + rot - kBins;
      const uint32_t cnt = sh[i];
      if (cnt) {
        const int t = i / kHistStride;
        const int val = i % kHistStride - kHistOff;   // (the 2 padding counters stay 0)
        atomicAdd(&hist[(int64_t)t * EP_HIST_BINS + (val + 32768)], cnt);
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// Row statistics in any order, for the containers where that gives the left-to-right fp64 sums
// bit for bit.  An e4m3fn value is an integer multiple of 2^-9 below 2^18 of them (448 = 229376
// x 2^-9); an int8 value is an integer.  So each square w^2 and each product w p (p = h/2, |h| <
// 2^16) is an integer multiple of a fixed quantum (2^-18, 2^-10; 1, 1/2) of at most 36 bits, and
// every partial sum of a row of at most 2^17 elements stays below 2^53 quanta: exact in fp64,
// whatever the order (finite inputs; a NaN row sums to a NaN either way).  One 256-thread
// workgroup per row; each thread sums its strided vectors, then wavefront shuffles and the four
// wavefronts' partial sums.  kOrderFreeCols bounds the fp8 row width (int8 rows are exact at any
// width the library accepts).
// ------------------------------------------------------------------------------------------
constexpr int64_t kOrderFreeCols = (int64_t)1 << 17;
constexpr int kRowThreads = 256;

static inline bool order_free_host(int dt, int64_t cols) {
  return dt == EP_INT8 || (dt == EP_FP8_E4M3FN && cols <= kOrderFreeCols);
}

template <typename T>
__device__ __forceinline__ T row_reduce(T acc, T* part) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) acc += __shfl_xor(acc, d, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  return (part[0] + part[1]) + (part[2] + part[3]);
}

template <int DT, bool PAD>
__global__ __launch_bounds__(kRowThreads) void k_row_sumsq_any(const void* __restrict__ w,
                                                               int64_t rows, int64_t cols,
                                                               double* __restrict__ out) {
  static_assert(DT == EP_INT8 || DT == EP_FP8_E4M3FN, "order-free containers only");
  __shared__ double part[kRowThreads / 64];
  const int64_t r = blockIdx.x;
  const int64_t vpr = (cols + 7) / 8;
  double acc = 0.0;
  for (int64_t m = threadIdx.x; m < vpr; m += kRowThreads) {
    float x[8];
    raw_widen<DT>(row_vec<DT, PAD>(w, r, cols, vpr, m), x);   // padding widens to 0
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const double v = (double)x[i];
      acc = __dadd_rn(acc, __dmul_rn(v, v));
    }
  }
  const double sum = row_reduce(acc, part);
  if (threadIdx.x == 0) out[r] = sum;
}

template <int DT, bool PAD>
__global__ __launch_bounds__(kRowThreads) void k_row_lsq_any(
    const void* __restrict__ w, int64_t rows, int64_t cols, const uint8_t* __restrict__ coset,
    const int16_t* __restrict__ fields, double* __restrict__ num, int64_t* __restrict__ den4) {
  static_assert(DT == EP_INT8 || DT == EP_FP8_E4M3FN, "order-free containers only");
  __shared__ double part[kRowThreads / 64];
  __shared__ long long part4[kRowThreads / 64];
  const int64_t r = blockIdx.x;
  const int64_t vpr = (cols + 7) / 8, v_row = r * vpr;
  const uint4* fv = reinterpret_cast<const uint4*>(fields);
  double acc = 0.0;
  long long d4 = 0;
  for (int64_t m = threadIdx.x; m < vpr; m += kRowThreads) {
    float x[8];
    raw_widen<DT>(row_vec<DT, PAD>(w, r, cols, vpr, m), x);
    const uint4 fq = fv[v_row + m];
    const int32_t c = (int32_t)coset[v_row + m];
    const uint32_t q[4] = {fq.x, fq.y, fq.z, fq.w};
    int32_t f[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      f[2 * i] = (int32_t)(int16_t)(q[i] & 0xFFFFu);
      f[2 * i + 1] = (int32_t)q[i] >> 16;
    }
    int32_t par = 0;
#pragma unroll
    for (int i = 0; i < 7; i++) par ^= f[i];
    f[7] = 2 * f[7] + (par & 1);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      if (PAD && 8 * m + i >= cols) break;            // padding: not a weight
      const int64_t h = 2 * (int64_t)f[i] + c;
      acc = __dadd_rn(acc, __dmul_rn((double)x[i], (double)h * 0.5));
      d4 += h * h;
    }
  }
  const double sum = row_reduce(acc, part);
  const long long s4 = row_reduce(d4, part4);
  if (threadIdx.x == 0) {
    num[r] = sum;
    den4[r] = s4;
  }
}

// ------------------------------------------------------------------------------------------
// Row least-squares terms: one lane per row, streamed like the row sums (weights, fields and
// cosets of the next kRowChunk vectors loaded while the current ones are summed).
// num = sum w * p (fp64, left to right; each product exact), den4 = sum (2p)^2 (int64).
// ------------------------------------------------------------------------------------------
template <int DT, bool PAD>
__global__ __launch_bounds__(64) void k_row_lsq(const void* __restrict__ w, int64_t rows,
                                                int64_t cols, const uint8_t* __restrict__ coset,
                                                const int16_t* __restrict__ fields,
                                                double* __restrict__ num,
                                                int64_t* __restrict__ den4) {
  using Raw = typename RawVec<DT>::T;
  const int64_t r = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (r >= rows) return;
  const int64_t vpr = (cols + 7) / 8, v_row = r * vpr;
  const uint4* fv = reinterpret_cast<const uint4*>(fields);
  Raw cw[kRowChunk], nw[kRowChunk];
  uint4 cf[kRowChunk], nf[kRowChunk];
  uint32_t cc[kRowChunk], nc[kRowChunk];
  // loads past the row's end re-read its last vector (never summed): no branch around a load
  auto clampv = [&](int64_t m) { return m < vpr ? m : vpr - 1; };
#pragma unroll
  for (int k = 0; k < kRowChunk; k++) {
    const int64_t m = clampv(k);
    cw[k] = row_vec<DT, PAD>(w, r, cols, vpr, m);
    cf[k] = fv[v_row + m];
    cc[k] = coset[v_row + m];
  }
  double acc = 0.0;
  int64_t d4 = 0;
  for (int64_t v0 = 0; v0 < vpr; v0 += kRowChunk) {
    const int64_t v1 = v0 + kRowChunk;
#pragma unroll
    for (int k = 0; k < kRowChunk; k++) {
      const int64_t m = clampv(v1 + k);
      nw[k] = row_vec<DT, PAD>(w, r, cols, vpr, m);
      nf[k] = fv[v_row + m];
      nc[k] = coset[v_row + m];
    }
#pragma unroll
    for (int k = 0; k < kRowChunk; k++) {
      if (v0 + k < vpr) {
        float x[8];
        raw_widen<DT>(cw[k], x);
        const uint32_t q[4] = {cf[k].x, cf[k].y, cf[k].z, cf[k].w};
        int32_t f[8];
#pragma unroll
        for (int i = 0; i < 4; i++) {
          f[2 * i] = (int32_t)(int16_t)(q[i] & 0xFFFFu);
          f[2 * i + 1] = (int32_t)q[i] >> 16;
        }
        int32_t par = 0;
#pragma unroll
        for (int i = 0; i < 7; i++) par ^= f[i];
        f[7] = 2 * f[7] + (par & 1);
        const int32_t c = (int32_t)cc[k];
#pragma unroll
        for (int i = 0; i < 8; i++) {
          if (PAD && 8 * (v0 + k) + i >= cols) break;     // padding: not a weight
          const int64_t h = 2 * (int64_t)f[i] + c;
          const double p = (double)h * 0.5;
          acc = __dadd_rn(acc, __dmul_rn((double)x[i], p));
          d4 += h * h;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kRowChunk; k++) {
      cw[k] = nw[k];
      cf[k] = nf[k];
      cc[k] = nc[k];
    }
  }
  num[r] = acc;
  den4[r] = d4;
}

// ------------------------------------------------------------------------------------------
// Decode-table expansion (once per blob).  For each of the 16 field tables, slot s of [0, 2^P)
// belongs to the value v with cum(v) <= s < cum(v) + f(v) and gets
//   entry = f(v) | (s - cum(v)) << 13 | (v & 127) << 25        (u32)
//   value = v                                                   (i16, for wide alphabets)
// and a slot that no value covers gets 0 in both.  The 7-bit value in the entry is exact
// whenever every field value lies in [-64, 63].
// One 1024-lane workgroup per table, in three steps: a scan of the frequencies gives cum(v) and
// marks slot cum(v) of each value with f(v) > 0 (mark = slot + 1; the value's index and f(v)
// beside it); a running maximum of the marks hands every slot the first slot of its run; each
// lane then writes its 4 consecutive slots with one 16-byte and one 8-byte store.
// ------------------------------------------------------------------------------------------
constexpr int kExpandThreads = 1024;
static_assert(kExpandThreads * 4 == kM, "each lane expands 4 slots");

template <bool MAX>
__device__ __forceinline__ uint32_t expand_op(uint32_t a, uint32_t b) {
  return MAX ? (a > b ? a : b) : a + b;
}

// Scan (sum, or maximum when MAX) of one value per lane over the workgroup: returns the
// exclusive scan at this lane (0 at lane 0) and sets total to the workgroup's.  part: the wave
// totals; the call opens with a barrier, so consecutive calls may share it.
template <bool MAX>
__device__ __forceinline__ uint32_t expand_scan(uint32_t x, uint32_t* part, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(inc, d, 64);
    if (lane >= d) inc = expand_op<MAX>(inc, y);
  }
  uint32_t exc = __shfl_up(inc, 1, 64);
  if (lane == 0) exc = 0;
  __syncthreads();
  if (lane == 63) part[wave] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kExpandThreads / 64; w++) {
    const uint32_t p = part[w];
    if (w < wave) before = expand_op<MAX>(before, p);
    tot = expand_op<MAX>(tot, p);
  }
  total = tot;
  return expand_op<MAX>(before, exc);
}

__global__ __launch_bounds__(kExpandThreads) void k_expand_tables(const uint8_t* __restrict__ blob,
                                                                  TableArgs ta, DecTables dt) {
  __shared__ __align__(16) uint32_t mark[kM];  // slot + 1 where a value's run starts, else 0
  __shared__ uint32_t info[kM];                // at such a slot: value index | f(v) << 16
  __shared__ uint32_t part[kExpandThreads / 64];
  const int t = blockIdx.x;                    // field table 0..15 = blob table 1 + t
  const uint32_t n = ta.n[1 + t];
  const int32_t lo = ta.lo[1 + t];
  const uint16_t* freq = reinterpret_cast<const uint16_t*>(blob + ta.off[1 + t] + 8);
  reinterpret_cast<uint4*>(mark)[threadIdx.x] = make_uint4(0, 0, 0, 0);
  __syncthreads();
  uint32_t base = 0, total;                    // base: cum of the pass's first value
  for (uint32_t c0 = 0; c0 < n; c0 += kExpandThreads) {
    const uint32_t i = c0 + threadIdx.x;
    const uint32_t f = i < n ? freq[i] : 0u;
    const uint32_t cum = base + expand_scan<false>(f, part, total);
    if (f > 0 && cum < (uint32_t)kM) {
      mark[cum] = cum + 1;
      info[cum] = i | f << 16;
    }
    base += total;
  }
  __syncthreads();
  const uint4 mk = reinterpret_cast<const uint4*>(mark)[threadIdx.x];
  uint32_t run[4];
  run[0] = mk.x;
  run[1] = expand_op<true>(run[0], mk.y);
  run[2] = expand_op<true>(run[1], mk.z);
  run[3] = expand_op<true>(run[2], mk.w);
  const uint32_t before = expand_scan<true>(run[3], part, total);
  const uint32_t s0 = 4 * threadIdx.x;         // this lane's slots s0 .. s0 + 3
  uint32_t e[4];
  uint16_t v[4];
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const uint32_t m = expand_op<true>(before, run[k]);
    e[k] = 0;
    v[k] = 0;
    if (m > 0) {
      const uint32_t start = m - 1, inf = info[start], f = inf >> 16, q = s0 + k - start;
      if (q < f) {
        const int32_t val = lo + (int32_t)(inf & 0xffffu);
        e[k] = f | q << 13 | ((uint32_t)val & 127u) << 25;
        v[k] = (uint16_t)val;
      }
    }
  }
  reinterpret_cast<uint4*>(dt.ent + (size_t)t * kM)[threadIdx.x] =
      make_uint4(e[0], e[1], e[2], e[3]);
  reinterpret_cast<uint2*>(dt.val + (size_t)t * kM)[threadIdx.x] =
      make_uint2(v[0] | (uint32_t)v[1] << 16, v[2] | (uint32_t)v[3] << 16);
}

}  // namespace ep

// ==========================================================================================
// C-ABI entry points that launch kernels
// ==========================================================================================
using namespace ep;

static bool valid_dtype(int32_t dt) { return dt >= EP_BF16 && dt <= EP_FP32; }

extern "C" ep_status ep_row_sumsq(const void* d_w, int32_t dtype, int64_t rows, int64_t cols,
                                  double* d_out, void* stream) {
  ep::clear_pending_error();
  if (!d_w || !d_out) return EP_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(d_w) & 15u) return EP_ERR_ARG;
  if (!valid_dtype(dtype)) return EP_ERR_DTYPE;
  if (!shape_fits(rows, cols)) return EP_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool pad = cols % 8 != 0;
  if (rows > 0 && order_free_host(dtype, cols)) {      // one workgroup per row, any order
    const dim3 rgrid((unsigned)rows);
    if (dtype == EP_INT8)
      pad ? k_row_sumsq_any<EP_INT8, true><<<rgrid, kRowThreads, 0, s>>>(d_w, rows, cols, d_out)
          : k_row_sumsq_any<EP_INT8, false><<<rgrid, kRowThreads, 0, s>>>(d_w, rows, cols, d_out);
    else
      pad ? k_row_sumsq_any<EP_FP8_E4M3FN, true><<<rgrid, kRowThreads, 0, s>>>(d_w, rows, cols,
                                                                              d_out)
          : k_row_sumsq_any<EP_FP8_E4M3FN, false><<<rgrid, kRowThreads, 0, s>>>(d_w, rows, cols,
                                                                               d_out);
    return hipGetLastError() == hipSuccess ? EP_OK : EP_ERR_HIP;
  }
  const dim3 grid((unsigned)((rows + 63) / 64));
#define EP_S(DT)                                                                              \
  (pad ? k_row_sumsq<DT, true><<<grid, 64, 0, s>>>(d_w, rows, cols, d_out)                    \
       : k_row_sumsq<DT, false><<<grid, 64, 0, s>>>(d_w, rows, cols, d_out))
  switch (dtype) {
    case EP_BF16: EP_S(EP_BF16); break;
    case EP_FP16: EP_S(EP_FP16); break;
    case EP_FP8_E4M3FN: EP_S(EP_FP8_E4M3FN); break;
    case EP_FP32: EP_S(EP_FP32); break;
    default: EP_S(EP_INT8); break;
  }
#undef EP_S
  return hipGetLastError() == hipSuccess ? EP_OK : EP_ERR_HIP;
}

extern "C" ep_status ep_quantize_e8(const void* d_w, int32_t dtype, int64_t rows, int64_t cols,
                                    const float* d_row_gain, const int64_t* d_row_index,
                                    int64_t n_rows_sel, uint8_t* d_coset, int16_t* d_fields,
                                    ep_hist* d_hist, uint32_t* d_err, void* stream) {
  ep::clear_pending_error();
  if (!d_w || !d_row_gain || !d_coset || !d_fields || !d_err) return EP_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(d_w) & 15u) || (reinterpret_cast<uintptr_t>(d_fields) & 15u))
    return EP_ERR_ARG;
  if (!valid_dtype(dtype)) return EP_ERR_DTYPE;
  if (rows < 1 || cols < 1 || cols > ((int64_t)1 << 40)) return EP_ERR_SHAPE;
  const int64_t nsel = d_row_index ? n_rows_sel : rows;
  if (nsel < 0 || (d_row_index && nsel > (int64_t)1 << 31)) return EP_ERR_ARG;
  if (nsel > 0 && !shape_fits(nsel, cols)) return EP_ERR_SHAPE;
  const int64_t nvec = nsel * ((cols + 7) / 8);
  if (nvec >= ((int64_t)1 << 31)) return EP_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* hist = d_hist ? d_hist->counts : nullptr;
  if (hist) {
    constexpr int64_t n = (int64_t)EP_NTABLES * EP_HIST_BINS;
    if (reinterpret_cast<uintptr_t>(hist) & 15u)
      k_fill_u32<<<1024, 256, 0, s>>>(hist, n, 0u);
    else
      k_zero16<<<(unsigned)((n / 4 + 255) / 256), 256, 0, s>>>(reinterpret_cast<uint4*>(hist),
                                                              n / 4);
  }
  if (nvec == 0) return hipGetLastError() == hipSuccess ? EP_OK : EP_ERR_HIP;
  // two 16-wavefront workgroups per compute unit at most: enough waves in flight with the
  // one-ahead fetch, and few per-workgroup histogram merges
  int64_t blocks = (nvec + kQThreads - 1) / kQThreads;
  if (blocks > 2 * kCUs) blocks = 2 * kCUs;
  const dim3 grid((unsigned)blocks);
  const uint32_t nv = (uint32_t)nvec, vpr = (uint32_t)((cols + 7) / 8);
  const bool pad = cols % 8 != 0;
  const double inv_vpr = 1.0 / (double)vpr;
#define EP_Q1(DT, PAD)                                                                        \
  k_quantize_e8<DT, PAD><<<grid, kQThreads, 0, s>>>(d_w, rows, cols, d_row_gain, d_row_index, \
                                                    nv, vpr, inv_vpr, d_coset, d_fields, hist, \
                                                    d_err)
#define EP_Q(DT) (pad ? EP_Q1(DT, true) : EP_Q1(DT, false))
  switch (dtype) {
    case EP_BF16: EP_Q(EP_BF16); break;
    case EP_FP16: EP_Q(EP_FP16); break;
    case EP_FP8_E4M3FN: EP_Q(EP_FP8_E4M3FN); break;
    case EP_FP32: EP_Q(EP_FP32); break;
    default: EP_Q(EP_INT8); break;
  }
#undef EP_Q
#undef EP_Q1
  return hipGetLastError() == hipSuccess ? EP_OK : EP_ERR_HIP;
}

extern "C" ep_status ep_row_lsq(const void* d_w, int32_t dtype, int64_t rows, int64_t cols,
                                const uint8_t* d_coset, const int16_t* d_fields, double* d_num,
                                int64_t* d_den4, void* stream) {
  ep::clear_pending_error();
  if (!d_w || !d_coset || !d_fields || !d_num || !d_den4) return EP_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(d_w) & 15u) || (reinterpret_cast<uintptr_t>(d_fields) & 15u))
    return EP_ERR_ARG;
  if (!valid_dtype(dtype)) return EP_ERR_DTYPE;
  if (!shape_fits(rows, cols)) return EP_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool pad = cols % 8 != 0;
  if (rows > 0 && order_free_host(dtype, cols)) {      // one workgroup per row, any order
    const dim3 rgrid((unsigned)rows);
#define EP_LA(DT, PAD)                                                                        \
  k_row_lsq_any<DT, PAD><<<rgrid, kRowThreads, 0, s>>>(d_w, rows, cols, d_coset, d_fields,     \
                                                       d_num, d_den4)
    if (dtype == EP_INT8)
      pad ? EP_LA(EP_INT8, true) : EP_LA(EP_INT8, false);
    else
      pad ? EP_LA(EP_FP8_E4M3FN, true) : EP_LA(EP_FP8_E4M3FN, false);
#undef EP_LA
    return hipGetLastError() == hipSuccess ? EP_OK : EP_ERR_HIP;
  }
  const dim3 grid((unsigned)((rows + 63) / 64));
#define EP_L1(DT, PAD)                                                                        \
  k_row_lsq<DT, PAD><<<grid, 64, 0, s>>>(d_w, rows, cols, d_coset, d_fields, d_num, d_den4)
#define EP_L(DT) (pad ? EP_L1(DT, true) : EP_L1(DT, false))
  switch (dtype) {
    case EP_BF16: EP_L(EP_BF16); break;
    case EP_FP16: EP_L(EP_FP16); break;
    case EP_FP8_E4M3FN: EP_L(EP_FP8_E4M3FN); break;
    case EP_FP32: EP_L(EP_FP32); break;
    default: EP_L(EP_INT8); break;
  }
#undef EP_L
#undef EP_L1
  return hipGetLastError() == hipSuccess ? EP_OK : EP_ERR_HIP;
}

extern "C" ep_status ep_prepare_decode(const void* d_blob, const ep_blob_info* info,
                                       void* d_dec_tables, void* stream) {
  ep::clear_pending_error();
  if (!d_blob || !info || !d_dec_tables) return EP_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(d_dec_tables) & 15u) return EP_ERR_ARG;
  TableArgs ta;
  for (int t = 0; t < EP_NTABLES; t++) {
    ta.off[t] = info->table_off[t];
    ta.n[t] = info->n[t];
    ta.lo[t] = info->lo[t];
  }
  k_expand_tables<<<16, kExpandThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint8_t*>(d_blob), ta, dec_tables(d_dec_tables));
  return hipGetLastError() == hipSuccess ? EP_OK : EP_ERR_HIP;
}


// Decodes n blobs of one container and tile size: the full tiles of all of them in launches of up
// to kMaxBatch blobs, then the ragged last tiles (if any) the same way.
// stamps (one blob only): the traced decode, which records each tile's phase boundaries; it
// takes the linear words layout and the fused scaling, for bf16 and fp8 containers.
static ep_status decode_blobs(int n, const void* const* d_blobs, const ep_blob_info* infos,
                              const void* const* d_dec_tables, void* const* d_outs,
                              uint32_t* d_err, uint32_t flags, hipStream_t s,
                              unsigned long long* stamps = nullptr) {
  if (stamps) {
    if (n != 1 || flags) return EP_ERR_ARG;
    flags = EP_DECODE_LINEAR;
  }
  const uint32_t layout = flags & (EP_DECODE_LINEAR | EP_DECODE_RING | EP_DECODE_RING_MIN);
  if ((flags & ~layout) || (layout & (layout - 1u))) return EP_ERR_ARG;
  if (n < 1 || !d_blobs || !infos || !d_dec_tables || !d_outs || !d_err) return EP_ERR_ARG;
  const ep_blob_info& i0 = infos[0];
  if (!valid_dtype(i0.dtype)) return EP_ERR_DTYPE;
  const int J = i0.tile_fields / (8 * EP_LANES);
  if (i0.tile_fields % (8 * EP_LANES) || (J != 8 && J != 16 && J != 32)) return EP_ERR_VERSION;
  if (i0.lanes != EP_LANES && i0.lanes != 2 * EP_LANES) return EP_ERR_VERSION;
  const int S = i0.lanes / EP_LANES;                 // rANS states per lane
  // batch-wide choices: the largest tile, any wide alphabet, any tiny row scale
  uint32_t maxw = 0;
  bool big = false, slow = false, long_rows = true, bounded = true;
  int64_t total_tiles = 0;
  for (int i = 0; i < n; i++) {
    const ep_blob_info& in = infos[i];
    if (!d_blobs[i] || !d_dec_tables[i] || !d_outs[i]) return EP_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(d_blobs[i]) & 15u) ||
        (reinterpret_cast<uintptr_t>(d_outs[i]) & 15u))
      return EP_ERR_ARG;
    if (in.precision != EP_PRECISION || (in.lanes != EP_LANES && in.lanes != 2 * EP_LANES))
      return EP_ERR_VERSION;
    if (in.dtype != i0.dtype || in.tile_fields != i0.tile_fields || in.lanes != i0.lanes)
      return EP_ERR_ARG;
    // (the vector count is bounded before the product is formed: no overflow on any header)
    if (!shape_fits(in.rows, in.cols)) return EP_ERR_SHAPE;
    const int64_t nv_in = in.rows * ((in.cols + 7) / 8);
    if (nv_in >= ((int64_t)1 << 31) || in.tiles < 1 ||
        in.tiles != (nv_in + J * 64 - 1) / (J * 64))
      return EP_ERR_SHAPE;
    if (in.n_exceptions < 0 || in.n_exceptions > nv_in ||
        (in.n_exceptions > 0 &&
         (in.off_exceptions < 64 || (in.off_exceptions & 15) || (in.off_exception_fields & 15) ||
          in.off_exceptions + 4 * in.n_exceptions > in.off_exception_fields ||
          in.off_exception_fields + 16 * in.n_exceptions > in.bytes)))
      return EP_ERR_ARG;
    maxw = std::max(maxw, in.max_tile_words);
    long_rows &= (in.cols + 7) / 8 >= (int64_t)J * 64;   // a tile spans at most two rows
    big |= in.big_alphabet != 0;
    slow |= in.tiny_scale != 0;
    bounded &= in.bounded != 0;
    total_tiles += in.tiles;
  }
  // Words region per wave.  Linear: the aligned chunks of the largest tile plus one wave of
  // slack.  Ring: a power of two of at least 512 words and 2/7 of the largest tile (two field
  // phases' worth), refilled as the tile is decoded; used only when it keeps more tiles resident.
  // Half that ring is also offered (automatic choice only): a heavy phase then waits for its
  // refill, but when LDS is what limits the waves per CU (wide alphabets at high rates) the
  // extra resident tiles hide more of the rANS chains' latency.
  const uint32_t lin_stride = ((maxw + 7u + 7u) & ~7u) + 64u;
  uint32_t ring_stride = 512u;
  while (layout != EP_DECODE_RING_MIN && ring_stride < 8192u &&
         (uint64_t)ring_stride * 7u < 2ull * maxw)
    ring_stride <<= 1;
  const uint32_t ring_half = (layout == 0 && ring_stride >= 1024u) ? ring_stride / 2 : ring_stride;
  // LDS: slot tables (2 phases x 2 cosets x 4096 x 4 B, + 2 B values for wide alphabets), then
  // per wave 256 S bytes of states and the words region.  Waves per workgroup and layout: the
  // choice that keeps the most tiles resident at once; ties go to the linear layout, then to the
  // less crowded CU (the smaller workgroup, spread over more CUs, unless it would share CUs) of
  // at least 4 waves.
  // (a ring region also holds the copy of its first 64 words)
  auto lds_of = [&](int w, uint32_t stride, bool rg) -> size_t {
    return (size_t)(big ? kWideTop : kNarTop) +
           (size_t)w * ((size_t)256 * S + (size_t)stride * 2 + (rg ? kRingMirrorBytes : 0u));
  };
  // waves per SIMD the decoder's registers allow: 8, 4 and 4 for 8, 16 and 32 vectors per lane
  // (2 at 32 with wide alphabets, whose fields take 16 bits each, or 3 when every row holds a
  // tile's vectors twice over and two row scales per wave replace one per vector; 7 at 8 with
  // two states per lane and wide alphabets)
  const bool rows2 = J == 32 && long_rows && !stamps;
  if (stamps && ((i0.dtype != EP_BF16 && i0.dtype != EP_FP8_E4M3FN) || slow))
    return EP_ERR_VERSION;                           // not instantiated with the trace
  const int occ = J <= 8 ? ((S == 2 && big) ? 7 : 8) : (J <= 16 ? 4 : (big ? (rows2 ? 3 : 2) : 4));
  const int64_t waves_per_cu = 4 * occ;
  const int max_waves = occ >= 4 ? kDecWaves : (occ == 3 ? 12 : kDecWaves / 2);
  int waves = 0;
  bool ring = false;
  uint32_t stride = 0;
  int64_t best = -1, best_crowd = 0;
  // candidates: linear (ties go to it, and among its sizes to the smaller workgroup down to 4
  // waves, below which each wave would load a large share of the tables itself), then the full
  // ring and the half ring, each taken only when it keeps strictly more tiles resident.  The
  // count of resident tiles is capped at the tiles there are (a partly filled last workgroup
  // adds none).
  for (int lay = 0; lay < 3; lay++) {
    const bool rg = lay >= 1;
    if (layout == EP_DECODE_LINEAR && rg) continue;
    if ((layout == EP_DECODE_RING || layout == EP_DECODE_RING_MIN) && !rg) continue;
    if (lay == 2 && ring_half == ring_stride) continue;
    const uint32_t st = lay == 0 ? lin_stride : (lay == 1 ? ring_stride : ring_half);
    if (rg && layout == 0 && st >= lin_stride) continue;
    for (const int w : {16, 12, 8, 4, 2, 1}) {
      if (w > max_waves || (int64_t)lds_of(w, st, rg) > kLdsPerCU) continue;
      const int64_t per_cu =
          std::min<int64_t>(kLdsPerCU / (int64_t)lds_of(w, st, rg), waves_per_cu / w);
      const int64_t grid = (total_tiles + w - 1) / w;
      const int64_t resident = std::min(std::min(grid, kCUs * per_cu) * w, total_tiles);
      // the most waves one CU holds at once: a smaller workgroup that still ends up two to a CU
      // (its tables then loaded twice there) gains nothing over a larger one alone
      const int64_t crowd = std::min((grid + kCUs - 1) / kCUs, per_cu) * w;
      if (resident > best || (resident == best && !rg && w >= 4 && crowd < best_crowd)) {
        best = resident;
        best_crowd = crowd;
        waves = w;
        ring = rg;
        stride = st;
      }
    }
  }
  if (waves == 0) return EP_ERR_VERSION;             // one tile's words do not fit in LDS
  // 32 vectors per lane with byte fields: 4 waves per SIMD, bound by VALU issue, and a 16-wave
  // workgroup's waves reach its phase barriers far apart while their SIMDs idle.  Two 8-wave
  // workgroups per CU, which LDS holds only with the ring layout, let one workgroup decode
  // while the other waits at a barrier (measured at 8192 x 28672 fp8: 195 -> 188 us); taken
  // when they keep as many tiles resident.
  if (J == 32 && !big && S == 1 && layout == 0 && !stamps && waves == 16 && !ring) {
    const size_t l8 = lds_of(8, ring_stride, true);
    const int64_t per_cu = std::min<int64_t>(kLdsPerCU / (int64_t)l8, waves_per_cu / 8);
    const int64_t grid8 = (total_tiles + 7) / 8;
    const int64_t resident = std::min(std::min(grid8, kCUs * per_cu) * 8, total_tiles);
    if (per_cu >= 2 && resident >= best) {
      waves = 8;
      ring = true;
      stride = ring_stride;
    }
  }
  const size_t lds = lds_of(waves, stride, ring);
  const uint32_t V = (uint32_t)i0.tile_fields / 8;

  DecodeArgs a;
  a.err = d_err;
  a.words_stride = stride;
  a.stamps = stamps;
  auto flush = [&](bool ragged) -> ep_status {
    if (a.n == 0) return EP_OK;
    hipError_t e;
    if (stamps) {
      if (i0.dtype == EP_BF16)
        e = S == 2 ? launch_decode_trace<EP_BF16, 2>(a, J, big, ragged, waves, lds, s)
                   : launch_decode_trace<EP_BF16, 1>(a, J, big, ragged, waves, lds, s);
      else
        e = S == 2 ? launch_decode_trace<EP_FP8_E4M3FN, 2>(a, J, big, ragged, waves, lds, s)
                   : launch_decode_trace<EP_FP8_E4M3FN, 1>(a, J, big, ragged, waves, lds, s);
      a.n = 0;
      return e == hipSuccess ? EP_OK : EP_ERR_HIP;
    }
#define EP_LD(DT, SL)                                                                         \
  (S == 2 ? launch_decode<DT, 2>(a, J, big, ragged, SL, rows2, ring, waves, lds, s)            \
          : launch_decode<DT, 1>(a, J, big, ragged, SL, rows2, ring, waves, lds, s))
    switch (i0.dtype) {
      case EP_BF16: e = EP_LD(EP_BF16, slow); break;
      case EP_FP16: e = EP_LD(EP_FP16, false); break;
      case EP_FP8_E4M3FN:
        // a bounded batch needs no saturation clamp (instantiated with one state per lane)
        e = (bounded && S == 1) ? launch_decode<kFp8Bounded, 1>(a, J, big, ragged, false, rows2,
                                                                 ring, waves, lds, s)
                                : EP_LD(EP_FP8_E4M3FN, false);
        break;
      case EP_FP32: e = EP_LD(EP_FP32, slow); break;
      default: e = EP_LD(EP_INT8, false); break;
    }
#undef EP_LD
    a.n = 0;
    return e == hipSuccess ? EP_OK : EP_ERR_HIP;
  };
  // the fused scaling is exact for fp16, fp8 and int8 whatever the scales (a tiny scale's products
  // round to zero in those containers); bf16 and fp32 keep the subnormal range and need the exact
  // half
  for (int pass = 0; pass < 2; pass++) {             // full tiles, then ragged last tiles
    const bool ragged = pass == 1;
    a.n = 0;
    a.wg_begin[0] = 0;
    for (int i = 0; i < n; i++) {
      const ep_blob_info& in = infos[i];
      const int64_t nv = in.rows * ((in.cols + 7) / 8);
      const uint32_t tiles = (uint32_t)in.tiles;
      const bool last_ragged = (uint64_t)tiles * V != (uint64_t)nv;
      const uint32_t t0 = ragged ? tiles - 1 : 0;
      const uint32_t t1 = ragged ? tiles : (last_ragged ? tiles - 1 : tiles);
      if ((ragged && !last_ragged) || t1 <= t0) continue;
      DecodeBlob& b = a.b[a.n];
      const uint8_t* p = static_cast<const uint8_t*>(d_blobs[i]);
      b.alpha = reinterpret_cast<const float*>(p + in.off_alpha);
      b.word_off = reinterpret_cast<const uint32_t*>(p + in.off_word_off);
      b.states = reinterpret_cast<const uint32_t*>(p + in.off_states);
      b.words = reinterpret_cast<const uint16_t*>(p + in.off_words);
      {
        const DecTables dt = dec_tables(const_cast<void*>(d_dec_tables[i]));
        b.ent = dt.ent;
        b.val = reinterpret_cast<const uint16_t*>(dt.val);
      }
      b.out = d_outs[i];
      b.tile_begin = t0;
      b.tile_end = t1;
      b.n_vec = (uint32_t)nv;
      b.vpr = (uint32_t)((in.cols + 7) / 8);
      b.max_tile_words = in.max_tile_words;
      b.coset_f0 = in.coset_freq0;
      b.lo0 = in.lo[0];
      b.inv_vpr_f = 1.0f / (float)b.vpr;
      b.inv_vpr = 1.0 / (double)b.vpr;
      a.wg_begin[a.n + 1] = a.wg_begin[a.n] + (t1 - t0 + waves - 1) / waves;
      if (++a.n == kMaxBatch) {
        const ep_status st = flush(ragged);
        if (st != EP_OK) return st;
        a.wg_begin[0] = 0;
      }
    }
    const ep_status st = flush(ragged);
    if (st != EP_OK) return st;
  }
  // escaped vectors, rewritten once the tiles are decoded (stream order)
  for (int i = 0; i < n; i++) {
    const ep_blob_info& in = infos[i];
    if (in.n_exceptions == 0) continue;
    const uint8_t* p = static_cast<const uint8_t*>(d_blobs[i]);
    const uint32_t* idx = reinterpret_cast<const uint32_t*>(p + in.off_exceptions);
    const void* xf = p + in.off_exception_fields;
    const float* alpha = reinterpret_cast<const float*>(p + in.off_alpha);
    const uint32_t vpr = (uint32_t)((in.cols + 7) / 8);
    const uint32_t nvb = (uint32_t)(in.rows * (int64_t)vpr);
    const uint32_t m = (uint32_t)in.n_exceptions;
    const bool tiny = in.tiny_scale != 0;
    hipError_t e;
    switch (i0.dtype) {
      case EP_BF16: e = launch_patch<EP_BF16>(idx, xf, m, alpha, vpr, nvb, d_outs[i], tiny, d_err, s); break;
      case EP_FP16: e = launch_patch<EP_FP16>(idx, xf, m, alpha, vpr, nvb, d_outs[i], false, d_err, s); break;
      case EP_FP8_E4M3FN:
        e = launch_patch<EP_FP8_E4M3FN>(idx, xf, m, alpha, vpr, nvb, d_outs[i], false, d_err, s);
        break;
      case EP_FP32: e = launch_patch<EP_FP32>(idx, xf, m, alpha, vpr, nvb, d_outs[i], tiny, d_err, s); break;
      default: e = launch_patch<EP_INT8>(idx, xf, m, alpha, vpr, nvb, d_outs[i], false, d_err, s); break;
    }
    if (e != hipSuccess) return EP_ERR_HIP;
  }
  return EP_OK;
}

extern "C" ep_status ep_decompress(const void* d_blob, const ep_blob_info* info,
                                   const void* d_dec_tables, void* d_out, uint32_t* d_err,
                                   void* stream) {
  return ep_decompress_ex(d_blob, info, d_dec_tables, d_out, d_err, 0u, stream);
}

// ------------------------------------------------------------------------------------------
// The decode fused into its consumer product: Y = X W^T without W in global memory.  A
// workgroup takes 16 rows of W, decodes the tiles holding them (one wave per tile, the tile
// decoder's own code and LDS layout), stages the rows' container values in LDS and multiplies
// them with MFMA; the waves' shares of the columns are summed in wave order.
// ------------------------------------------------------------------------------------------
// The decode fused into its product for n blobs of one shape (n = 1: ep_decompress_matmul), in
// launches of up to kMaxBatch blobs: workgroups [wg_begin[i], wg_begin[i + 1]) take blob i's
// 16-row groups.
static ep_status matmul_blobs(int n, const void* const* d_blobs, const ep_blob_info* infos,
                              const void* const* d_tabs, const void* const* d_xs, int64_t m,
                              float* const* d_ys, uint32_t* d_err, hipStream_t s) {
  if (n < 1 || !d_blobs || !infos || !d_tabs || !d_xs || !d_ys || !d_err) return EP_ERR_ARG;
  const ep_blob_info& in = infos[0];
  if (!valid_dtype(in.dtype)) return EP_ERR_DTYPE;
  if (in.dtype != EP_BF16 && in.dtype != EP_FP16) return EP_ERR_DTYPE;
  if (m < 1 || m > EP_MM_MAX_M) return EP_ERR_ARG;
  if (in.precision != EP_PRECISION || (in.lanes != EP_LANES && in.lanes != 2 * EP_LANES))
    return EP_ERR_VERSION;
  const int J = in.tile_fields / (8 * EP_LANES);
  if (in.tile_fields % (8 * EP_LANES) || (J != 8 && J != 16)) return EP_ERR_SHAPE;
  if (in.cols < 8 || in.cols % 8 || in.cols > EP_MM_MAX_COLS || !shape_fits(in.rows, in.cols))
    return EP_ERR_SHAPE;
  const int64_t vpr = in.cols / 8, nv = in.rows * vpr;
  const int64_t V = (int64_t)J * 64;
  bool big = false, slow = false;
  uint32_t max_words = 0;
  for (int i = 0; i < n; i++) {
    const ep_blob_info& bi = infos[i];
    if (!d_blobs[i] || !d_tabs[i] || !d_xs[i] || !d_ys[i]) return EP_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(d_blobs[i]) & 15u) ||
        (reinterpret_cast<uintptr_t>(d_xs[i]) & 15u) || (reinterpret_cast<uintptr_t>(d_ys[i]) & 3u))
      return EP_ERR_ARG;
    if (i > 0 && (bi.dtype != in.dtype || bi.rows != in.rows || bi.cols != in.cols ||
                  bi.tile_fields != in.tile_fields || bi.lanes != in.lanes ||
                  bi.precision != in.precision))
      return EP_ERR_ARG;                             // one shape per call
    if (bi.tiles < 1 || bi.tiles != (nv + V - 1) / V || nv >= ((int64_t)1 << 31))
      return EP_ERR_SHAPE;
    if (bi.n_exceptions != 0) return EP_ERR_VERSION; // escaped vectors need the patch pass
    big |= bi.big_alphabet != 0;
    slow |= bi.tiny_scale != 0;
    max_words = std::max(max_words, bi.max_tile_words);
  }
  const int S = in.lanes / EP_LANES;
  // waves per workgroup: the tiles a group of 16 rows can touch (16 vpr vectors from any start
  // touch at most ceil(16 vpr / V) + 1 tiles; exactly 16 vpr / V when that divides)
  const int64_t gv = 16 * vpr;
  const int64_t wpg = gv % V == 0 ? gv / V : (gv + V - 1) / V + 1;
  const uint32_t kpad = (uint32_t)((in.cols + 31) / 32 * 32);
  const uint32_t pitch = 2u * kpad + 16u;            // +16 B: the 16 rows fall in distinct banks
  const uint32_t lin_stride = ((max_words + 7u + 7u) & ~7u) + 64u;
  const int64_t groups = (in.rows + 15) / 16;
  // LDS: the decoder's (tables, then per wave its states and words) while decoding, then the
  // staged rows (16 x pitch) and the waves' partial products (4 KiB each)
  auto lds_of = [&](int64_t w) -> size_t {
    const size_t dec = (size_t)(big ? kWideTop : kNarTop) +
                       (size_t)w * ((size_t)256 * S + (size_t)lin_stride * 2);
    return std::max(dec, std::max<size_t>((size_t)16 * pitch, (size_t)w * 4096));
  };
  const bool ragged = (int64_t)in.tiles * V != nv;
  for (int c0 = 0; c0 < n; c0 += kMaxBatch) {
    const int nb = std::min(n - c0, kMaxBatch);
    // one or two 16-row groups per workgroup: two when that keeps more tiles decoding at once
    // (registers allow 16 waves per CU; the LDS decides how many workgroups share one)
    int64_t ng = 0, best = -1;
    for (int64_t G = 1; G <= 2; G++) {
      const int64_t w = G * wpg;
      if (w > kDecWaves || (int64_t)lds_of(w) > kLdsPerCU) continue;
      const int64_t per_cu = std::min<int64_t>(kLdsPerCU / (int64_t)lds_of(w), kDecWaves / w);
      const int64_t wgs = nb * ((groups + G - 1) / G);
      const int64_t resident = std::min(wgs, kCUs * per_cu) * w;
      if (resident > best) {
        best = resident;
        ng = G;
      }
    }
    if (ng == 0) return EP_ERR_SHAPE;                // a tile's words do not fit beside the rest
    const int64_t waves = ng * wpg;
    const size_t lds = lds_of(waves);
    DecodeArgs a;
    a.err = d_err;
    a.words_stride = lin_stride;
    a.stamps = nullptr;
    a.n = (uint32_t)nb;
    a.wg_begin[0] = 0;
    for (int i = 0; i < nb; i++) {
      const ep_blob_info& bi = infos[c0 + i];
      a.wg_begin[i + 1] = a.wg_begin[i] + (uint32_t)((groups + ng - 1) / ng);
      DecodeBlob& b = a.b[i];
      const uint8_t* p = static_cast<const uint8_t*>(d_blobs[c0 + i]);
      b.alpha = reinterpret_cast<const float*>(p + bi.off_alpha);
      b.word_off = reinterpret_cast<const uint32_t*>(p + bi.off_word_off);
      b.states = reinterpret_cast<const uint32_t*>(p + bi.off_states);
      b.words = reinterpret_cast<const uint16_t*>(p + bi.off_words);
      {
        const DecTables dt = dec_tables(const_cast<void*>(d_tabs[c0 + i]));
        b.ent = dt.ent;
        b.val = reinterpret_cast<const uint16_t*>(dt.val);
      }
      b.out = nullptr;
      b.tile_begin = 0;
      b.tile_end = (uint32_t)bi.tiles;
      b.n_vec = (uint32_t)nv;
      b.vpr = (uint32_t)vpr;
      b.max_tile_words = bi.max_tile_words;
      b.coset_f0 = bi.coset_freq0;
      b.lo0 = bi.lo[0];
      b.inv_vpr_f = 1.0f / (float)b.vpr;
      b.inv_vpr = 1.0 / (double)b.vpr;
      a.mm_x[i] = d_xs[c0 + i];
      a.mm_y[i] = d_ys[c0 + i];
    }
    a.mm_m = (uint32_t)m;
    a.mm_cols = (uint32_t)in.cols;
    a.mm_rows = (uint32_t)in.rows;
    a.mm_kpad = kpad;
    a.mm_pitch = pitch;
    a.mm_groups = (uint32_t)ng;
    hipError_t e;
    if (in.dtype == EP_BF16)
      e = S == 2 ? launch_decode_mm<EP_BF16, 2>(a, J, big, ragged, slow, (int)waves, lds, s)
                 : launch_decode_mm<EP_BF16, 1>(a, J, big, ragged, slow, (int)waves, lds, s);
    else
      e = S == 2 ? launch_decode_mm<EP_FP16, 2>(a, J, big, ragged, false, (int)waves, lds, s)
                 : launch_decode_mm<EP_FP16, 1>(a, J, big, ragged, false, (int)waves, lds, s);
    if (e != hipSuccess) return EP_ERR_HIP;
  }
  return EP_OK;
}

extern "C" ep_status ep_decompress_matmul(const void* d_blob, const ep_blob_info* info,
                                          const void* d_dec_tables, const void* d_x, int64_t m,
                                          float* d_y, uint32_t* d_err, void* stream) {
  ep::clear_pending_error();
  if (!d_blob || !info || !d_dec_tables || !d_x || !d_y || !d_err) return EP_ERR_ARG;
  return matmul_blobs(1, &d_blob, info, &d_dec_tables, &d_x, m, &d_y, d_err,
                      static_cast<hipStream_t>(stream));
}

extern "C" ep_status ep_decompress_matmul_batch(int32_t n, const void* const* d_blobs,
                                                const ep_blob_info* infos,
                                                const void* const* d_dec_tables,
                                                const void* const* d_x, int64_t m,
                                                float* const* d_y, uint32_t* d_err,
                                                void* stream) {
  ep::clear_pending_error();
  if (n < 1 || n > (1 << 20)) return EP_ERR_ARG;
  return matmul_blobs(n, d_blobs, infos, d_dec_tables, d_x, m, d_y, d_err,
                      static_cast<hipStream_t>(stream));
}

// ------------------------------------------------------------------------------------------
// The decode without a caller-supplied table buffer and without any allocation: the expanded
// decode tables go to a file-scope device array, one per GPU, which lives until the process
// ends.  In host code `scratch` names only a host-side stand-in: its device address is taken
// once per device with hipGetSymbolAddress, and only that address is ever passed to a kernel.
// ------------------------------------------------------------------------------------------
namespace {
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[EP_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];                   // device address of `scratch`, per device

// The address of this device's `scratch` (looked up on the device's first call), or null.
void* device_scratch(int dev) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" ep_status ep_decompress_noalloc(const void* d_blob, const ep_blob_info* info,
                                           void* d_out, uint32_t* d_err, void* stream) {
  ep::clear_pending_error();
  if (!d_blob || !info || !d_out || !d_err) return EP_ERR_ARG;
  static_assert(EP_NOALLOC_SCRATCH_BYTES >= EP_DEC_TABLE_BYTES, "one blob's decode tables");
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return EP_ERR_HIP;
  if (dev >= kMaxDevices) return EP_ERR_ARG;
  void* tables = device_scratch(dev);
  if (!tables) return EP_ERR_HIP;
  const ep_status st = ep_prepare_decode(d_blob, info, tables, stream);
  if (st != EP_OK) return st;
  const void* const t = tables;
  return decode_blobs(1, &d_blob, info, &t, &d_out, d_err, 0u, static_cast<hipStream_t>(stream));
}

extern "C" ep_status ep_decompress_ex(const void* d_blob, const ep_blob_info* info,
                                      const void* d_dec_tables, void* d_out, uint32_t* d_err,
                                      uint32_t flags, void* stream) {
  ep::clear_pending_error();
  if (!d_blob || !info || !d_dec_tables || !d_out || !d_err) return EP_ERR_ARG;
  return decode_blobs(1, &d_blob, info, &d_dec_tables, &d_out, d_err, flags,
                      static_cast<hipStream_t>(stream));
}

extern "C" ep_status ep_decompress_traced(const void* d_blob, const ep_blob_info* info,
                                          const void* d_dec_tables, void* d_out, uint32_t* d_err,
                                          unsigned long long* d_stamps, void* stream) {
  ep::clear_pending_error();
  if (!d_blob || !info || !d_dec_tables || !d_out || !d_err || !d_stamps) return EP_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(d_stamps) & 7u) return EP_ERR_ARG;
  return decode_blobs(1, &d_blob, info, &d_dec_tables, &d_out, d_err, 0u,
                      static_cast<hipStream_t>(stream), d_stamps);
}

extern "C" ep_status ep_decompress_batch(int32_t n, const void* const* d_blobs,
                                         const ep_blob_info* infos,
                                         const void* const* d_dec_tables, void* const* d_outs,
                                         uint32_t* d_err, void* stream) {
  ep::clear_pending_error();
  return decode_blobs(n, d_blobs, infos, d_dec_tables, d_outs, d_err, 0u,
                      static_cast<hipStream_t>(stream));
}
