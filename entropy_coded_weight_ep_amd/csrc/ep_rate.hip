// Device side of the rate search (gfx950): the table normalisation of a device histogram and
// the coded-size sum of the sampled symbols, so that a scale candidate costs the host a few
// hundred bytes of transfer instead of the whole 17 x 65536 histogram.
//
// The design page ("Rate selection and refinement") picks the scale from sampled rows by
// estimating the coded field size plus the metadata for each candidate, without encoding the
// full stream.  Here the estimate's two data-heavy parts run on the device:
//   k_build_tables  one workgroup per table: the table's span [first, last] of seen values, then
//                   the same integer normalisation as the host table build (frequency 0 for an
//                   unseen value, else max(1, floor(count * 2^P / total)); a deficit goes to the
//                   most frequent value, an excess is taken from the largest frequencies, lowest
//                   index first on ties);
//   k_sum_bits      one workgroup: the products count * (P - log2 f) formed in parallel, then
//                   summed over tables, then values, by one lane in exactly the host's order,
//                   with every product and sum rounded on its own, so the result is the host's
//                   double bit for bit (P - log2 f comes from a table the host fills with its own
//                   log2).
// The host finishes the estimate (sampling factor and metadata bytes) from that sum and the
// tables' sizes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <array>
#include <cmath>

#include "ep.h"
#include "ep_internal.h"

namespace ep {

constexpr uint32_t kNormM = 1u << EP_PRECISION;
constexpr int kBT = 1024;                          // threads of a table-build workgroup
static_assert(EP_HIST_BINS % (4 * kBT) == 0, "whole 16-byte loads per thread");

// Largest (MAX) or total 64-bit value of a workgroup: every thread passes one and all get the
// result.  Shuffles within each wavefront, then the 16 wavefront results through LDS (s: at
// least kBT / 64 entries); it ends with a barrier, so s may be reused at once.
template <bool MAX>
__device__ uint64_t block_reduce_u64(uint64_t v, uint64_t* s) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, d, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), d, 64);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = MAX ? (o > v ? o : v) : v + o;
  }
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = v;
  __syncthreads();
  uint64_t r = s[0];
#pragma unroll
  for (int w = 1; w < kBT / 64; w++) r = MAX ? (s[w] > r ? s[w] : r) : r + s[w];
  __syncthreads();
  return r;
}
__device__ uint64_t block_max_u64(uint64_t v, uint64_t* s) { return block_reduce_u64<true>(v, s); }
__device__ uint64_t block_sum_u64(uint64_t v, uint64_t* s) { return block_reduce_u64<false>(v, s); }

// Table t = blockIdx.x of the histogram -> lo[t], n[t], freq[t][0..n) of the device ep_tables.
__global__ __launch_bounds__(kBT) void k_build_tables(const uint32_t* __restrict__ hist,
                                                     ep_tables* __restrict__ out,
                                                     uint32_t* __restrict__ err) {
  __shared__ uint64_t s[kBT / 64];
  const int t = blockIdx.x;
  const uint32_t* c = hist + (size_t)t * EP_HIST_BINS;
  uint16_t* f = out->freq + (size_t)t * EP_HIST_BINS;

  // span, total and number of distinct values.  Each thread visits its bins in increasing
  // order, so the last nonzero one it sees is its largest.  With 16-byte aligned counts all 16
  // of a thread's 16-byte loads are issued at once.
  uint32_t first = 0xFFFFFFFFu, last = 0, distinct = 0;
  uint64_t total = 0;
  auto visit = [&](uint32_t b, uint32_t v) {
    if (v) {
      first = b < first ? b : first;
      last = b;
      total += v;
      distinct++;
    }
  };
  if ((reinterpret_cast<uintptr_t>(c) & 15u) == 0) {
    const uint4* c4 = reinterpret_cast<const uint4*>(c);
    constexpr int kQ = EP_HIST_BINS / 4 / kBT;
    uint4 q[kQ];
#pragma unroll
    for (int k = 0; k < kQ; k++) q[k] = c4[threadIdx.x + kBT * k];
#pragma unroll
    for (int k = 0; k < kQ; k++) {
      const uint32_t b = 4u * (threadIdx.x + kBT * k);
      visit(b, q[k].x);
      visit(b + 1, q[k].y);
      visit(b + 2, q[k].z);
      visit(b + 3, q[k].w);
    }
  } else {
    for (uint32_t b = threadIdx.x; b < EP_HIST_BINS; b += kBT) visit(b, c[b]);
  }
  first = 0xFFFFFFFFu - (uint32_t)block_max_u64(0xFFFFFFFFu - first, s);
  last = (uint32_t)block_max_u64(distinct ? last : 0u, s);
  total = block_sum_u64(total, s);
  distinct = (uint32_t)block_sum_u64(distinct, s);
  if (distinct == 0) {
    if (threadIdx.x == 0) {
      out->lo[t] = 0;
      out->n[t] = 0;
    }
    return;
  }
  if (distinct > kNormM) {
    if (threadIdx.x == 0) atomicOr(err, 1u << EP_ERR_ALPHABET);
    return;
  }
  const uint32_t n = last - first + 1u;
  if (threadIdx.x == 0) {
    out->lo[t] = (int32_t)first - 32768;
    out->n[t] = n;
  }

  // first frequencies, their sum, and the most frequent value (lowest index on ties)
  uint64_t assigned = 0, top_cnt = 0;
  for (uint32_t i = threadIdx.x; i < n; i += kBT) {
    const uint32_t v = c[first + i];
    uint32_t q = 0;
    if (v) {
      q = (uint32_t)(((uint64_t)v * kNormM) / total);
      q = q < 1u ? 1u : q;
    }
    f[i] = (uint16_t)q;
    assigned += q;
    const uint64_t key = ((uint64_t)v << 32) | (0xFFFFFFFFu - i);
    top_cnt = key > top_cnt ? key : top_cnt;
  }
  assigned = block_sum_u64(assigned, s);
  top_cnt = block_max_u64(top_cnt, s);
  int64_t gap = (int64_t)kNormM - (int64_t)assigned;
  if (gap > 0) {
    if (threadIdx.x == 0) {
      const uint32_t i = 0xFFFFFFFFu - (uint32_t)top_cnt;
      f[i] = (uint16_t)(f[i] + gap);
    }
    return;
  }
  // excess: repeatedly the largest frequency above 1 (lowest index on ties) gives up what it can
  while (gap < 0) {
    uint64_t key = 0;
    for (uint32_t i = threadIdx.x; i < n; i += kBT) {
      const uint32_t q = f[i];
      const uint64_t k = q > 1u ? (((uint64_t)q << 32) | (0xFFFFFFFFu - i)) : 0u;
      key = k > key ? k : key;
    }
    key = block_max_u64(key, s);                  // (ends with a barrier: every f[] read done)
    if (key == 0) break;                          // (cannot happen: distinct <= 2^P)
    const uint32_t i = 0xFFFFFFFFu - (uint32_t)key;
    const int64_t q = (int64_t)(key >> 32);
    const int64_t take = -gap < q - 1 ? -gap : q - 1;
    if (threadIdx.x == 0) f[i] = (uint16_t)(q - take);
    gap += take;
    __syncthreads();                              // the update before the next scan
  }
}

// Sum over tables t, then values i < n[t] with a nonzero count, of count * cost[freq], left to
// right, each product and each sum rounded separately.  The entries of all tables are taken as
// one sequence, in chunks of kSumChunk: the workgroup forms the chunk's products in parallel
// and packs the nonzero ones into LDS in their order (a ballot rank within each wave, the
// counts of the waves before it), then one lane adds them to the running sum in that order.
// The addends are >= 0 and the sum starts at +0, so the entries skipped (count 0) would add
// exactly nothing: the result is the host's left-to-right sum bit for bit.
constexpr int kSumThreads = 1024;
constexpr int kSumChunk = 4 * kSumThreads;

__global__ __launch_bounds__(kSumThreads) void k_sum_bits(const uint32_t* __restrict__ hist,
                                                          const ep_tables* __restrict__ tab,
                                                          const double* __restrict__ cost,
                                                          const uint32_t* __restrict__ err,
                                                          double* __restrict__ bits) {
  __shared__ double s_p[kSumChunk];                 // the chunk's nonzero products, in order
  __shared__ uint32_t s_base[EP_NTABLES + 1];       // first entry of each table
  __shared__ int32_t s_lo[EP_NTABLES];
  __shared__ uint32_t s_wave[kSumThreads / 64];     // nonzero products per wave in a pass
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (*err & (1u << EP_ERR_ALPHABET)) {
    if (tid == 0) *bits = 0.0;
    return;
  }
  if (tid == 0) {
    uint32_t b = 0;
    for (int t = 0; t < EP_NTABLES; t++) {
      s_base[t] = b;
      s_lo[t] = tab->lo[t];
      b += tab->n[t];
    }
    s_base[EP_NTABLES] = b;
  }
  __syncthreads();
  const uint32_t total = s_base[EP_NTABLES];
  double acc = 0.0;                                 // lane 0 of wave 0 keeps the sum
  for (uint32_t c0 = 0; c0 < total; c0 += kSumChunk) {
    uint32_t packed = 0;                            // products packed so far in this chunk
    for (int pass = 0; pass < kSumChunk / kSumThreads; pass++) {
      const uint32_t e = c0 + (uint32_t)(pass * kSumThreads + tid);
      double p = 0.0;
      bool nz = false;
      if (e < total) {
        int t = 0;
        while (e >= s_base[t + 1]) t++;
        const uint32_t q = e - s_base[t];
        const uint32_t v = hist[(size_t)t * EP_HIST_BINS + (uint32_t)(s_lo[t] + 32768) + q];
        if (v) {
          p = __dmul_rn((double)v, cost[tab->freq[(size_t)t * EP_HIST_BINS + q]]);
          nz = true;
        }
      }
      const uint64_t m = __ballot(nz);
      const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      if (lane == 0) s_wave[wave] = (uint32_t)__popcll(m);
      __syncthreads();
      uint32_t before = packed, all = packed;
      for (int w = 0; w < kSumThreads / 64; w++) {
        const uint32_t c = s_wave[w];
        before += w < wave ? c : 0u;
        all += c;
      }
      if (nz) s_p[before + rank] = p;
      packed = all;
      __syncthreads();                              // s_wave is rewritten by the next pass
    }
    if (tid == 0) {
      uint32_t i = 0;
      for (; i + 8 <= packed; i += 8) {
        double v[8];
#pragma unroll
        for (int k = 0; k < 8; k++) v[k] = s_p[i + k];
#pragma unroll
        for (int k = 0; k < 8; k++) acc = __dadd_rn(acc, v[k]);
      }
      for (; i < packed; i++) acc = __dadd_rn(acc, s_p[i]);
    }
    __syncthreads();                                // s_p is rewritten by the next chunk
  }
  if (tid == 0) *bits = acc;
}

// Rate of row blockIdx.x in units of 2^-16 bit under the device tables: the sum over its vectors
// of cost[f] for the coset symbol (table 0) and the eight fields (tables 1 + 8c + k), where f is
// the value's frequency, or 0 (cost[0]) for a value outside its table.  One workgroup per row;
// the integer sum is exact, so the order of the additions does not matter.
constexpr int kRT = 256;

__global__ __launch_bounds__(kRT) void k_row_rates(const uint8_t* __restrict__ coset,
                                                   const int16_t* __restrict__ fields,
                                                   uint32_t vpr, const ep_tables* __restrict__ tab,
                                                   const uint32_t* __restrict__ cost,
                                                   int64_t* __restrict__ rate) {
  __shared__ int32_t s_lo[EP_NTABLES];
  __shared__ uint32_t s_n[EP_NTABLES];
  __shared__ uint64_t s_sum[kRT / 64];
  if (threadIdx.x < EP_NTABLES) {
    s_lo[threadIdx.x] = tab->lo[threadIdx.x];
    s_n[threadIdx.x] = tab->n[threadIdx.x];
  }
  __syncthreads();
  auto cost_of = [&](int t, int32_t value) -> uint64_t {
    const uint32_t i = (uint32_t)(value - s_lo[t]);
    const uint32_t f = i < s_n[t] ? tab->freq[(size_t)t * EP_HIST_BINS + i] : 0u;
    return cost[f];
  };
  const int64_t v0 = (int64_t)blockIdx.x * vpr;
  const uint4* fv = reinterpret_cast<const uint4*>(fields);
  uint64_t acc = 0;
  for (uint32_t m = threadIdx.x; m < vpr; m += kRT) {
    const uint32_t c = coset[v0 + m];
    acc += cost_of(0, (int32_t)c);
    const uint4 q = fv[v0 + m];
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    const int tb = 1 + 8 * (int)(c & 1u);
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const uint32_t h = w[k >> 1];
      const int32_t value = (k & 1) ? (int32_t)h >> 16 : (int32_t)(int16_t)(h & 0xFFFFu);
      acc += cost_of(tb + k, value);
    }
  }
  // wavefront sum, then the workgroup's
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)acc, d);
    const uint32_t hi = __shfl_xor((uint32_t)(acc >> 32), d);
    acc += ((uint64_t)hi << 32) | lo;
  }
  if ((threadIdx.x & 63) == 0) s_sum[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t t = 0;
    for (int i = 0; i < kRT / 64; i++) t += s_sum[i];
    rate[blockIdx.x] = (int64_t)t;
  }
}

// P - log2(f) for f = 1 .. 2^P (entry 0 unused), with the host's log2.
static const std::array<double, kNormM + 1>& cost_table() {
  static const std::array<double, kNormM + 1> tab = [] {
    std::array<double, kNormM + 1> a{};
    for (uint32_t f = 1; f <= kNormM; f++) a[f] = (double)EP_PRECISION - std::log2((double)f);
    return a;
  }();
  return tab;
}

// Workspace of the device estimate: tables, cost table, bit sum + error word.
struct RateWs {
  ep_tables* tables;
  double* cost;
  double* bits;
  uint32_t* err;
  size_t total;
};

static RateWs rate_carve(void* base) {
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  uint8_t* p = static_cast<uint8_t*>(base);
  size_t o = 0;
  RateWs w;
  w.tables = reinterpret_cast<ep_tables*>(p + o); o += up(sizeof(ep_tables));
  w.cost = reinterpret_cast<double*>(p + o); o += up(8 * (size_t)(kNormM + 1));
  w.bits = reinterpret_cast<double*>(p + o); o += up(8);
  w.err = reinterpret_cast<uint32_t*>(p + o); o += up(4);
  w.total = o;
  return w;
}

__global__ void k_zero_u32(uint32_t* p) { *p = 0u; }

}  // namespace ep

using namespace ep;

extern "C" ep_status ep_build_tables_gpu(const ep_hist* d_hist, ep_tables* d_out, uint32_t* d_err,
                                         void* stream) {
  ep::clear_pending_error();
  if (!d_hist || !d_out || !d_err) return EP_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  k_build_tables<<<EP_NTABLES, kBT, 0, s>>>(d_hist->counts, d_out, d_err);
  return hipGetLastError() == hipSuccess ? EP_OK : EP_ERR_HIP;
}

extern "C" size_t ep_estimate_workspace_bytes(void) { return rate_carve(nullptr).total; }

extern "C" ep_status ep_row_rates(const uint8_t* d_coset, const int16_t* d_fields, int64_t rows,
                                  int64_t cols, const ep_tables* d_tables, const uint32_t* d_cost,
                                  int64_t* d_rates, void* stream) {
  ep::clear_pending_error();
  if (!d_coset || !d_fields || !d_tables || !d_cost || !d_rates) return EP_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(d_fields) & 15u) return EP_ERR_ARG;
  if (!ep::shape_fits(rows, cols)) return EP_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  k_row_rates<<<(unsigned)rows, kRT, 0, s>>>(d_coset, d_fields, (uint32_t)((cols + 7) / 8), d_tables,
                                             d_cost, d_rates);
  return hipGetLastError() == hipSuccess ? EP_OK : EP_ERR_HIP;
}

// Internal: the device part of the estimate, enqueued on `s`; the sum of bits lands in
// h_bits and the table sizes in h_n after the stream synchronises.  Returns false on a HIP error.
namespace ep {
bool estimate_enqueue(const ep_hist* d_hist, void* d_workspace, bool upload_cost, hipStream_t s,
                      double* h_bits, uint32_t* h_err, uint32_t* h_n) {
  const RateWs w = rate_carve(d_workspace);
  bool ok = true;
  if (upload_cost)
    ok &= hipMemcpyAsync(w.cost, cost_table().data(), 8 * (size_t)(kNormM + 1),
                         hipMemcpyHostToDevice, s) == hipSuccess;
  k_zero_u32<<<1, 1, 0, s>>>(w.err);
  k_build_tables<<<EP_NTABLES, kBT, 0, s>>>(d_hist->counts, w.tables, w.err);
  k_sum_bits<<<1, kSumThreads, 0, s>>>(d_hist->counts, w.tables, w.cost, w.err, w.bits);
  ok &= hipGetLastError() == hipSuccess;
  ok &= hipMemcpyAsync(h_bits, w.bits, 8, hipMemcpyDeviceToHost, s) == hipSuccess;
  ok &= hipMemcpyAsync(h_err, w.err, 4, hipMemcpyDeviceToHost, s) == hipSuccess;
  ok &= hipMemcpyAsync(h_n, w.tables->n, 4 * EP_NTABLES, hipMemcpyDeviceToHost, s) == hipSuccess;
  return ok;
}

const ep_tables* estimate_tables(void* d_workspace) { return rate_carve(d_workspace).tables; }
}  // namespace ep
