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
// The residual u - rint(u) is exact and never -0 (x - x rounds to +0), so copysign(1, r_k) is
// the step towards u, +1 for a zero residual.
// The coordinate sum is formed in fp32: the eight rounded values are integers of magnitude at
// most 65537 (|x| <= 65536 is checked before), so every partial sum is exact and one conversion
// gives the parity.
__device__ __forceinline__ void d8_round(const float u[8], float a[8]) {
  float fsum = 0.0f;
  float r[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    a[i] = __builtin_rintf(u[i]);
    fsum = __fadd_rn(fsum, a[i]);
    r[i] = __fsub_rn(u[i], a[i]);
  }
  const int32_t sum = (int32_t)fsum;
  int k = 0;
  float rk = r[0];                                 // residual of the worst coordinate so far
#pragma unroll
  for (int i = 1; i < 8; i++) {
    const bool worse = __builtin_fabsf(r[i]) > __builtin_fabsf(rk);
    rk = worse ? r[i] : rk;
    k = worse ? i : k;
  }
  k = (sum & 1) ? k : 8;                           // an even sum moves nothing
  const float step = __builtin_copysignf(1.0f, rk);
#pragma unroll
  for (int i = 0; i < 8; i++) a[i] = (i == k) ? __fadd_rn(a[i], step) : a[i];
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

// Returns the coset; z receives the D8 part (p - coset/2).
__device__ __forceinline__ int e8_nearest(const float x[8], int32_t z[8]) {
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
  for (int i = 0; i < 8; i++) z[i] = (int32_t)(c ? Bz[i] : A[i]);
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

__global__ __launch_bounds__(256) void k_fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = v;
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
// counts are kept per lane.  Few, large workgroups keep the merge short, and each workgroup
// starts its merge at a different bin so that they do not all hit the same global counters at
// once.
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
  QIn<DT> cur;
  if (v < n_vec) cur = q_fetch<DT, PAD>(w, rows, cols, gain, row_index, pos, vpr);
  for (; v < n_vec; v += stride) {
    QIn<DT> nxt;
    const bool more = v + stride < n_vec;         // (no overflow: n_vec + stride < 2^32)
    pos = q_advance(pos, step, vpr);               // the position of v + stride
    if (more) nxt = q_fetch<DT, PAD>(w, rows, cols, gain, row_index, pos, vpr);
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
      int32_t z[8];
      int c = e8_nearest(x, z);
#pragma unroll
      for (int k = 0; k < 8; k++) out_of_range |= (z[k] > 32767) | (z[k] < -32767);
      if (out_of_range) {                         // flagged; keep every field (and bin) in range
        c = 0;
#pragma unroll
        for (int k = 0; k < 8; k++) z[k] = 0;
      }
      bad |= out_of_range;
      int32_t f[8];
#pragma unroll
      for (int k = 0; k < 7; k++) f[k] = z[k];
      f[7] = z[7] >> 1;                           // arithmetic shift = floor(z7 / 2)
      coset[v] = (uint8_t)c;
      uint4 pk;
      pk.x = (uint32_t)(f[0] & 0xFFFF) | ((uint32_t)f[1] << 16);
      pk.y = (uint32_t)(f[2] & 0xFFFF) | ((uint32_t)f[3] << 16);
      pk.z = (uint32_t)(f[4] & 0xFFFF) | ((uint32_t)f[5] << 16);
      pk.w = (uint32_t)(f[6] & 0xFFFF) | ((uint32_t)f[7] << 16);
      reinterpret_cast<uint4*>(fields)[v] = pk;
      if (do_hist) {
        n_c1 += (uint32_t)c;
        n_c0 += 1u - (uint32_t)c;
        // bins of value 0 of this vector's coset tables (field k at + k * kHistStride)
        uint32_t* const hc = sh + (1 + 8 * c) * kHistStride + kHistOff;
        uint32_t orr = 0, orn = 0;
#pragma unroll
        for (int k = 0; k < 8; k++) {
          orr |= (uint32_t)(f[k] + kHistOff);
          orn |= (uint32_t)(f[k] + kNarrowOff);
        }
        if (orn < (uint32_t)kNarrowWin) {         // every field among the hottest values
          uint32_t* const hn =
              sn + ((threadIdx.x & (kNarrowCopies - 1)) * 16 + 8 * c) * kNarrowStride + kNarrowOff;
#pragma unroll
          for (int k = 0; k < 8; k++) atomicAdd(&hn[k * kNarrowStride + f[k]], 1u);
        } else if (orr < (uint32_t)kHistWin) {    // every field inside the window
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
    cur = nxt;
  }
  if (bad) atomicOr(err, 1u << EP_ERR_RANGE);
  if (bad_row) atomicOr(err, 1u << EP_ERR_ARG);
  if (do_hist) {
    if (n_c0) atomicAdd(&sh[kHistOff + 0], n_c0);
    if (n_c1) atomicAdd(&sh[kHistOff + 1], n_c1);
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
// The 7-bit value in the entry is exact whenever every field value lies in [-64, 63].
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_expand_tables(const uint8_t* __restrict__ blob,
                                                       TableArgs ta, uint32_t* __restrict__ ent,
                                                       int16_t* __restrict__ val) {
  __shared__ uint32_t scan[256];
  const int t = blockIdx.x;                    // field table 0..15 = blob table 1 + t
  const uint32_t n = ta.n[1 + t];
  const int32_t lo = ta.lo[1 + t];
  const uint16_t* freq = reinterpret_cast<const uint16_t*>(blob + ta.off[1 + t] + 8);
  uint32_t* E = ent + (size_t)t * kM;
  int16_t* S = val + (size_t)t * kM;
  for (uint32_t i = threadIdx.x; i < kM; i += 256) { E[i] = 0; S[i] = 0; }
  __syncthreads();
  uint32_t base = 0;
  for (uint32_t c0 = 0; c0 < n; c0 += 256) {
    const uint32_t s = c0 + threadIdx.x;
    const uint32_t f = (s < n) ? freq[s] : 0u;
    scan[threadIdx.x] = f;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
      uint32_t add = (threadIdx.x >= (unsigned)d) ? scan[threadIdx.x - d] : 0u;
      __syncthreads();
      scan[threadIdx.x] += add;
      __syncthreads();
    }
    const uint32_t cum = base + scan[threadIdx.x] - f;
    const int32_t v = lo + (int32_t)s;
    for (uint32_t q = 0; q < f; q++) {
      const uint32_t slot = cum + q;
      if (slot < kM) {
        E[slot] = f | (q << 13) | (((uint32_t)v & 127u) << 25);
        S[slot] = (int16_t)v;
      }
    }
    base += scan[255];
    __syncthreads();
  }
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
  if (rows < 1 || cols < 1) return EP_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)((rows + 63) / 64));
  const bool pad = cols % 8 != 0;
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
  if (rows < 1 || cols < 1) return EP_ERR_SHAPE;
  const int64_t nsel = d_row_index ? n_rows_sel : rows;
  if (nsel < 0 || (d_row_index && nsel > (int64_t)1 << 31)) return EP_ERR_ARG;
  const int64_t nvec = nsel * ((cols + 7) / 8);
  if (nvec >= ((int64_t)1 << 31)) return EP_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t* hist = d_hist ? d_hist->counts : nullptr;
  if (hist) {
    k_fill_u32<<<1024, 256, 0, s>>>(hist, (int64_t)EP_NTABLES * EP_HIST_BINS, 0u);
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
  if (rows < 1 || cols < 1) return EP_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)((rows + 63) / 64));
  const bool pad = cols % 8 != 0;
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
  TableArgs ta;
  for (int t = 0; t < EP_NTABLES; t++) {
    ta.off[t] = info->table_off[t];
    ta.n[t] = info->n[t];
    ta.lo[t] = info->lo[t];
  }
  uint32_t* ent = static_cast<uint32_t*>(d_dec_tables);
  int16_t* val = reinterpret_cast<int16_t*>(ent + 16 * kM);
  k_expand_tables<<<16, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint8_t*>(d_blob), ta, ent, val);
  return hipGetLastError() == hipSuccess ? EP_OK : EP_ERR_HIP;
}


// Decodes n blobs of one container and tile size: the full tiles of all of them in launches of up
// to kMaxBatch blobs, then the ragged last tiles (if any) the same way.
static ep_status decode_blobs(int n, const void* const* d_blobs, const ep_blob_info* infos,
                              const void* const* d_dec_tables, void* const* d_outs,
                              uint32_t* d_err, uint32_t flags, hipStream_t s) {
  const uint32_t layout = flags & (EP_DECODE_LINEAR | EP_DECODE_RING | EP_DECODE_RING_MIN);
  if ((flags & ~layout) || (layout & (layout - 1u))) return EP_ERR_ARG;
  if (n < 1 || !d_blobs || !infos || !d_dec_tables || !d_outs || !d_err) return EP_ERR_ARG;
  const ep_blob_info& i0 = infos[0];
  if (!valid_dtype(i0.dtype)) return EP_ERR_DTYPE;
  const int J = i0.tile_fields / (8 * EP_LANES);
  if (i0.tile_fields % (8 * EP_LANES) || (J != 8 && J != 16 && J != 32)) return EP_ERR_VERSION;
  // batch-wide choices: the largest tile, any wide alphabet, any tiny row scale
  uint32_t maxw = 0;
  bool big = false, slow = false, long_rows = true;
  int64_t total_tiles = 0;
  for (int i = 0; i < n; i++) {
    const ep_blob_info& in = infos[i];
    if (!d_blobs[i] || !d_dec_tables[i] || !d_outs[i]) return EP_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(d_blobs[i]) & 15u) ||
        (reinterpret_cast<uintptr_t>(d_outs[i]) & 15u))
      return EP_ERR_ARG;
    if (in.precision != EP_PRECISION || in.lanes != EP_LANES) return EP_ERR_VERSION;
    if (in.dtype != i0.dtype || in.tile_fields != i0.tile_fields) return EP_ERR_ARG;
    const int64_t nv_in = in.rows * ((in.cols + 7) / 8);
    if (in.rows < 1 || in.cols < 1 || nv_in >= ((int64_t)1 << 31) || in.tiles < 1 ||
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
  // per wave 256 B of states and the words region.  Waves per workgroup and layout: the choice
  // that keeps the most tiles resident at once; ties go to the linear layout, then to the smaller
  // workgroup (spread over more CUs) of at least 4 waves.
  const size_t lds_tables = (size_t)2 * 2 * kM * 4 + (big ? (size_t)2 * 2 * kM * 2 : 0);
  auto lds_of = [&](int w, uint32_t stride) {
    return lds_tables + (size_t)w * (256 + (size_t)stride * 2);
  };
  // waves per SIMD the decoder's registers allow: 8, 4 and 4 for 8, 16 and 32 vectors per lane
  // (2 at 32 with wide alphabets, whose fields take 16 bits each, or 3 when every row holds a
  // tile's vectors twice over and two row scales per wave replace one per vector)
  const bool rows2 = J == 32 && big && long_rows;
  const int occ = J <= 8 ? 8 : (J <= 16 ? 4 : (big ? (rows2 ? 3 : 2) : 4));
  const int64_t waves_per_cu = 4 * occ;
  const int max_waves = occ >= 4 ? kDecWaves : (occ == 3 ? 12 : kDecWaves / 2);
  int waves = 0;
  bool ring = false;
  uint32_t stride = 0;
  int64_t best = -1;
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
      if (w > max_waves || (int64_t)lds_of(w, st) > kLdsPerCU) continue;
      const int64_t per_cu =
          std::min<int64_t>(kLdsPerCU / (int64_t)lds_of(w, st), waves_per_cu / w);
      const int64_t grid = (total_tiles + w - 1) / w;
      const int64_t resident = std::min(std::min(grid, kCUs * per_cu) * w, total_tiles);
      if (resident > best || (resident == best && !rg && w >= 4)) {
        best = resident;
        waves = w;
        ring = rg;
        stride = st;
      }
    }
  }
  if (waves == 0) return EP_ERR_VERSION;             // one tile's words do not fit in LDS
  const size_t lds = lds_of(waves, stride);
  const uint32_t V = (uint32_t)i0.tile_fields / 8;

  DecodeArgs a;
  a.err = d_err;
  a.words_stride = stride;
  auto flush = [&](bool ragged) -> ep_status {
    if (a.n == 0) return EP_OK;
    hipError_t e;
    switch (i0.dtype) {
      case EP_BF16: e = launch_decode<EP_BF16>(a, J, big, ragged, slow, rows2, ring, waves, lds, s); break;
      case EP_FP16: e = launch_decode<EP_FP16>(a, J, big, ragged, false, rows2, ring, waves, lds, s); break;
      case EP_FP8_E4M3FN:
        e = launch_decode<EP_FP8_E4M3FN>(a, J, big, ragged, false, rows2, ring, waves, lds, s);
        break;
      case EP_FP32: e = launch_decode<EP_FP32>(a, J, big, ragged, slow, rows2, ring, waves, lds, s); break;
      default: e = launch_decode<EP_INT8>(a, J, big, ragged, false, rows2, ring, waves, lds, s); break;
    }
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
      b.ent = static_cast<const uint32_t*>(d_dec_tables[i]);
      b.val = reinterpret_cast<const int16_t*>(b.ent + 16 * kM);
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

extern "C" ep_status ep_decompress_ex(const void* d_blob, const ep_blob_info* info,
                                      const void* d_dec_tables, void* d_out, uint32_t* d_err,
                                      uint32_t flags, void* stream) {
  ep::clear_pending_error();
  if (!d_blob || !info || !d_dec_tables || !d_out || !d_err) return EP_ERR_ARG;
  return decode_blobs(1, &d_blob, info, &d_dec_tables, &d_out, d_err, flags,
                      static_cast<hipStream_t>(stream));
}

extern "C" ep_status ep_decompress_batch(int32_t n, const void* const* d_blobs,
                                         const ep_blob_info* infos,
                                         const void* const* d_dec_tables, void* const* d_outs,
                                         uint32_t* d_err, void* stream) {
  ep::clear_pending_error();
  return decode_blobs(n, d_blobs, infos, d_dec_tables, d_outs, d_err, 0u,
                      static_cast<hipStream_t>(stream));
}
