// GPU tile encoder (gfx950): the interleaved 64-state rANS encoding of the coset and field
// symbols, tile by tile, producing the blob's tile offsets, final states and word stream.
//
// The fields are rANS-coded in tiles that each decode on their own (EntroPack design page,
// "Encoding and reconstruction"; rANS after Duda, "Asymmetric numeral systems", 2009; the
// interleaving after Giesen, "Interleaved entropy coders", 2014).  The word order is the
// decoder's: phases (coset, field 0..7), inside each the lane's vectors ascending, inside that the
// lanes ascending.  The encoder walks that order backwards, so every tile's stream is the reverse
// of the words in the order the encoder emits them.
//
// One wavefront encodes one tile, lane l owning the vectors l, l+64, ..., l+64(J-1).  With 64
// states per tile lane l holds state l; with 128 (S = 2 per lane) vector l + 64u belongs to state
// l + 64 (u mod 2), held by the lane as its state u mod 2.  Either way the symbols are visited in
// the same (phase, u, lane) order, so only the state a step updates changes.
// At each (phase, vector) step the lanes that must flush a word do so together; in the backward
// order lane 63 comes first, so a flushing lane's word goes after those of the flushing lanes
// above it.  The words go onto a per-tile stack in scratch memory in that order, with the tile's
// count and its 64 final states (the decoder's initial states); a scan turns the counts into
// offsets, and a copy writes every stack reversed into the blob's word stream.
//
// Per symbol: entry (f, cum) of value - lo in the table of this phase and coset; flush
// x & 0xFFFF when x >= f * 2^20; then x = (x / f) * 2^12 + x mod f + cum.  x / f: the fp32
// product of x and the hardware reciprocal of f, truncated, then corrected exactly by one step
// either way from the integer remainder.  After the flush x < f * 2^20, so the quotient is below
// 2^20; rounding x to fp32 (2^-24), the reciprocal (1 ulp, 2^-23) and the product (2^-24) put
// the estimate within 2^-22 relative, under 1/4 absolute, and the one-step correction is exact.
// The step has no branch: a lane without a vector divides by 2^12 and adds 0, which leaves its
// state as it was.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>
#include <vector>

#include "ep.h"
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

constexpr int kEncWaves = 4;                       // tiles (wavefronts) per workgroup
constexpr uint32_t kEncLdsEntries = 16384;         // table entries held in LDS (64 KiB)

// Where each table's entries start in the packed entry array, and its value range.
struct EncTabs {
  uint32_t off[EP_NTABLES];
  uint32_t n[EP_NTABLES];
  int32_t lo[EP_NTABLES];
};

// Field k (0..7) of a vector's packed fields: eight int16, two per word, or eight int8, four
// per word.
__device__ __forceinline__ int32_t field_of(const uint4& q, int k) {
  const uint32_t w = (k >> 1) == 0 ? q.x : (k >> 1) == 1 ? q.y : (k >> 1) == 2 ? q.z : q.w;
  return (k & 1) ? (int32_t)w >> 16 : (int32_t)(int16_t)(w & 0xFFFFu);
}
__device__ __forceinline__ int32_t field_of(const uint2& q, int k) {
  return __builtin_amdgcn_sbfe((int32_t)(k < 4 ? q.x : q.y), 8 * (k & 3), 8);
}

// BYTES: every field table lies within [-128, 127], so the lane's fields are held as bytes, two
// registers per vector instead of four (a field that does not fit a byte is an alphabet error,
// reported like any value outside its table).
// Waves per SIMD the registers are budgeted for (the compiler fits the kernel to 512 / waves).
template <int J, bool BYTES>
struct EncOcc {
  static constexpr int waves = J <= 8 ? 8 : (J <= 16 ? (BYTES ? 5 : 4) : (BYTES ? 3 : 2));
};

template <int J, int S, bool LDS_TAB, bool BYTES>
__global__ __launch_bounds__(64 * kEncWaves)
__attribute__((amdgpu_waves_per_eu(EncOcc<J, BYTES>::waves, EncOcc<J, BYTES>::waves)))
void k_encode_tiles(
    const uint8_t* __restrict__ coset, const int16_t* __restrict__ fields, uint32_t n_vec,
    uint32_t tiles, const uint32_t* __restrict__ ent, uint32_t n_ent, EncTabs ta,
    uint32_t* __restrict__ counts, uint32_t* __restrict__ states, uint16_t* __restrict__ stack,
    uint32_t* __restrict__ err) {
  extern __shared__ uint32_t s_ent[];
  if constexpr (LDS_TAB) {
    for (uint32_t i = threadIdx.x; i < n_ent; i += blockDim.x) s_ent[i] = ent[i];
    __syncthreads();
  }
  const int lane = threadIdx.x & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t t = blockIdx.x * kEncWaves + wave;
  if (t >= tiles) return;
  constexpr uint32_t V = 64u * J;
  const uint32_t tv = t * V;
  const uint32_t nvt = n_vec - tv < V ? n_vec - tv : V;

  // the lane's vectors (j < nj): packed fields and coset bits
  const uint32_t nj = nvt > (uint32_t)lane ? (nvt - (uint32_t)lane + 63u) >> 6 : 0u;
  using Packed = typename std::conditional<BYTES, uint2, uint4>::type;
  Packed fk[J];
  uint32_t cbits = 0;
  uint32_t bad = 0;                                 // a symbol outside its table
#pragma unroll
  for (int j = 0; j < J; j++) {
    uint4 q = make_uint4(0, 0, 0, 0);
    if ((uint32_t)j < nj) {
      const uint32_t u = (uint32_t)lane + 64u * j;
      q = reinterpret_cast<const uint4*>(fields)[tv + u];
      const uint32_t cb = coset[tv + u];
      bad |= cb > 1u ? 1u : 0u;
      cbits |= (cb & 1u) << j;
    }
    if constexpr (BYTES) {
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int k = 0; k < 8; k++) {
        const int32_t v = __builtin_amdgcn_sbfe((int32_t)w[k >> 1], 16 * (k & 1), 16);
        bad |= v == __builtin_amdgcn_sbfe(v, 0, 8) ? 0u : 1u;
      }
      // the low byte of each field: f0 f1 f2 f3 | f4 f5 f6 f7
      fk[j] = make_uint2(__builtin_amdgcn_perm(q.y, q.x, 0x06040200u),
                         __builtin_amdgcn_perm(q.w, q.z, 0x06040200u));
    } else {
      fk[j] = q;
    }
  }

  uint32_t xs[S];
#pragma unroll
  for (int i = 0; i < S; i++) xs[i] = kL;
  uint32_t sp = 0;                                  // words emitted so far (wave-uniform)
  uint16_t* const stk = stack + (size_t)t * 9u * V; // room for one word per symbol
#pragma unroll
  for (int phase = 8; phase >= 0; --phase) {
    // the two tables of this phase (coset 0 and coset 1; the coset phase has one), their
    // parameters read here (the index is hidden from the compiler, which would otherwise keep
    // all 17 tables' parameters in scalar registers across the whole unrolled loop)
    int t0 = phase == 0 ? 0 : phase;
    int t1 = phase == 0 ? 0 : 8 + phase;
    asm volatile("" : "+s"(t0), "+s"(t1));
    // a value's entry is at value + (off - lo) of its coset's table; coset 1's parameters are
    // copied to vector registers once per phase so that one bitfield insert picks them per lane
    const uint32_t lo0 = (uint32_t)ta.lo[t0], n0 = ta.n[t0], d0 = ta.off[t0] - lo0;
    uint32_t lo1 = (uint32_t)ta.lo[t1], n1 = ta.n[t1], d1 = ta.off[t1] - lo1;
    asm volatile("" : "+v"(lo1), "+v"(n1), "+v"(d1));
#pragma unroll
    for (int j = J - 1; j >= 0; --j) {
      // 0 or ~0, opaque so that the selects below stay bitfield inserts on vector registers
      // (left alone, the compiler keeps every vector's coset as a lane mask in scalar registers
      // across the unrolled loop and spills them)
      uint32_t cm = (uint32_t)__builtin_amdgcn_sbfe((int32_t)cbits, j, 1);
      asm volatile("" : "+v"(cm));
      int32_t value;
      if (phase == 0) value = (int32_t)(cm & 1u);
      else value = field_of(fk[j], phase - 1);     // (byte or half of the packed fields)
      const uint32_t lo = (lo1 & cm) | (lo0 & ~cm);
      const uint32_t nt = (n1 & cm) | (n0 & ~cm);
      const uint32_t d = (d1 & cm) | (d0 & ~cm);
      const bool in = (uint32_t)value - lo < nt;    // (an empty table has nt = 0)
      // an in-range index always (entry 0 of the packed array when the value is not in the table)
      const uint32_t idx = in ? (uint32_t)value + d : 0u;
      uint32_t e;
      if constexpr (LDS_TAB) e = s_ent[idx];
      else e = ent[idx];
      const uint32_t fr = e & 0x1FFFu;
      const bool valid = (uint32_t)j < nj;
      const bool use = valid && in && fr != 0u;
      bad |= (valid && !use) ? 1u : 0u;
      asm volatile("" : "+v"(bad));                 // or-ed in now, not kept as lane masks
      // lanes that encode nothing take f = 2^12 and cum = 0: they never flush (x >> 20 < 2^12),
      // and the update below gives back x itself, (x / 2^12) 2^12 + x mod 2^12
      const uint32_t f = use ? fr : 4096u;
      uint32_t cum = use ? e >> 13 : 0u;
      asm volatile("" : "+v"(cum));                 // chosen here: the mask dies before the flush
      uint32_t& x = xs[j % S];
      const bool flush = (x >> 20) >= f;            // x >= f 2^20
      const uint64_t m = __ballot(flush);
      if (flush) {
        // emission index: the flushing lanes above this one come first
        const uint32_t above =
            (uint32_t)__popcll(m) -
            __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                      __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) -
            1u;
        stk[sp + above] = (uint16_t)(x & 0xFFFFu);
      }
      sp += (uint32_t)__popcll(m);
      {
        const uint32_t xs = flush ? x >> 16 : x;
        // quotient estimate in fp32: xs < f 2^20, so xs / f < 2^20; the conversion of xs, the
        // hardware reciprocal (1 ulp) and the product err by at most ~2^-22 relative, i.e. by
        // less than 1/4 in absolute terms, and one integer step either way makes it exact
        uint32_t q = (uint32_t)(__fmul_rn((float)xs, __builtin_amdgcn_rcpf((float)f)));
        int32_t r = (int32_t)(xs - q * f);
        q = r < 0 ? q - 1u : (r >= (int32_t)f ? q + 1u : q);
        r = r < 0 ? r + (int32_t)f : (r >= (int32_t)f ? r - (int32_t)f : r);
        x = (q << EP_PRECISION) + (uint32_t)r + cum;
      }
    }
  }
  if (__ballot(bad != 0u) != 0ull && lane == 0) atomicOr(err, 1u << EP_ERR_ALPHABET);
#pragma unroll
  for (int i = 0; i < S; i++) states[(size_t)t * 64 * S + 64 * i + lane] = xs[i];
  if (lane == 0) counts[t] = sp;
}

// Exclusive scan of the tile word counts -> word_off[0..tiles] and the largest count; one
// workgroup, 1024 tiles per round.
__global__ __launch_bounds__(1024) void k_scan_offsets(const uint32_t* __restrict__ counts,
                                                       uint32_t tiles,
                                                       uint32_t* __restrict__ word_off,
                                                       uint32_t* __restrict__ max_count,
                                                       uint64_t words_cap,
                                                       uint32_t* __restrict__ err) {
  __shared__ uint32_t s[1024];
  __shared__ uint32_t s_max[1024];
  uint64_t carry = 0;
  uint32_t mx = 0;
  for (uint32_t b = 0; b < tiles; b += 1024) {
    const uint32_t i = b + threadIdx.x;
    const uint32_t v = i < tiles ? counts[i] : 0u;
    s[threadIdx.x] = v;
    mx = v > mx ? v : mx;
    __syncthreads();
    for (uint32_t d = 1; d < 1024; d <<= 1) {      // inclusive Hillis-Steele scan
      const uint32_t add = threadIdx.x >= d ? s[threadIdx.x - d] : 0u;
      __syncthreads();
      s[threadIdx.x] += add;
      __syncthreads();
    }
    const uint64_t incl = carry + s[threadIdx.x];
    if (i < tiles) {
      if (incl > 0xFFFFFFFFull) atomicOr(err, 1u << EP_ERR_CAPACITY);
      word_off[i + 1] = (uint32_t)incl;
    }
    carry += s[1023];
    __syncthreads();
  }
  s_max[threadIdx.x] = mx;
  __syncthreads();
  for (uint32_t d = 512; d > 0; d >>= 1) {
    if (threadIdx.x < d && s_max[threadIdx.x + d] > s_max[threadIdx.x])
      s_max[threadIdx.x] = s_max[threadIdx.x + d];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    word_off[0] = 0;
    *max_count = s_max[0];
    if (carry > words_cap) atomicOr(err, 1u << EP_ERR_CAPACITY);
  }
}

// Each tile's stack, reversed, into the word stream at word_off[t] (one workgroup per tile).
__global__ __launch_bounds__(256) void k_copy_words(const uint16_t* __restrict__ stack,
                                                    uint32_t stack_words,
                                                    const uint32_t* __restrict__ word_off,
                                                    uint16_t* __restrict__ words,
                                                    uint64_t words_cap) {
  const uint32_t t = blockIdx.x;
  const uint32_t b = word_off[t], cnt = word_off[t + 1] - b;
  if (cnt > stack_words) return;                   // (never: a tile has at most one word a symbol)
  const uint16_t* stk = stack + (size_t)t * stack_words;
  for (uint32_t i = threadIdx.x; i < cnt; i += 256) {
    if ((uint64_t)b + i < words_cap) words[(uint64_t)b + i] = stk[cnt - 1u - i];
  }
}

template <int J, bool LDS_TAB, bool BYTES>
static void launch_enc(dim3 grid, size_t lds, hipStream_t s, int S, const uint8_t* coset,
                       const int16_t* fields, uint32_t nv, uint32_t tiles, const uint32_t* ent,
                       uint32_t n_ent, const EncTabs& ta, uint32_t* counts, uint32_t* states,
                       uint16_t* stack, uint32_t* err) {
  if (S == 2)
    k_encode_tiles<J, 2, LDS_TAB, BYTES><<<grid, 64 * kEncWaves, lds, s>>>(
        coset, fields, nv, tiles, ent, n_ent, ta, counts, states, stack, err);
  else
    k_encode_tiles<J, 1, LDS_TAB, BYTES><<<grid, 64 * kEncWaves, lds, s>>>(
        coset, fields, nv, tiles, ent, n_ent, ta, counts, states, stack, err);
}

// Workspace layout: packed table entries, tile counts, per-tile word stacks (9V words each).
struct EncWs {
  uint32_t* ent;
  uint32_t* counts;
  uint16_t* stack;
  size_t total;
};

static EncWs enc_carve(void* base, int64_t n_vectors, uint32_t tile_fields) {
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  const int64_t V = tile_fields / 8;
  const int64_t tiles = (n_vectors + V - 1) / V;
  uint8_t* p = static_cast<uint8_t*>(base);
  size_t o = 0;
  EncWs w;
  w.ent = reinterpret_cast<uint32_t*>(p + o); o += up((size_t)4 * EP_NTABLES * EP_HIST_BINS);
  w.counts = reinterpret_cast<uint32_t*>(p + o); o += up((size_t)4 * tiles);
  w.stack = reinterpret_cast<uint16_t*>(p + o); o += up((size_t)2 * 9 * V * tiles);
  w.total = o;
  return w;
}

}  // namespace ep

using namespace ep;

extern "C" size_t ep_encode_workspace_bytes(int64_t n_vectors, uint32_t tile_fields) {
  if (n_vectors < 1 || tile_fields < 512 || tile_fields % 512) return 0;
  return enc_carve(nullptr, n_vectors, tile_fields).total;
}

namespace ep {

ep_status encode_tiles_dev(const uint8_t* d_coset, const int16_t* d_fields, int64_t n_vectors,
                           uint32_t tile_fields, uint32_t lanes, const ep_tables* h_tables,
                           bool substitute,
                           void* d_workspace, size_t workspace_bytes, uint32_t* d_word_off,
                           uint32_t* d_max_tile_words, uint32_t* d_states, uint16_t* d_words,
                           int64_t words_cap, uint32_t* d_err, hipStream_t s) {
  if (!d_coset || !d_fields || !h_tables || !d_workspace || !d_word_off || !d_max_tile_words ||
      !d_states || !d_words || !d_err || words_cap < 0)
    return EP_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(d_fields) & 15u) return EP_ERR_ARG;
  if (n_vectors < 1 || n_vectors >= ((int64_t)1 << 31)) return EP_ERR_SHAPE;
  const int J = (int)(tile_fields / (8 * EP_LANES));
  if (tile_fields % (8 * EP_LANES) || (J != 8 && J != 16 && J != 32)) return EP_ERR_ARG;
  if (lanes != EP_LANES && lanes != 2 * EP_LANES) return EP_ERR_ARG;
  const int S = (int)(lanes / EP_LANES);
  if (workspace_bytes < ep_encode_workspace_bytes(n_vectors, tile_fields)) return EP_ERR_CAPACITY;
  const uint32_t nv = (uint32_t)n_vectors;
  const uint32_t V = tile_fields / 8;
  const uint32_t tiles = (uint32_t)((n_vectors + V - 1) / V);
  const EncWs ws = enc_carve(d_workspace, n_vectors, tile_fields);

  // packed entries f | cum << 13 of every table, in table order
  EncTabs ta;
  std::vector<uint32_t> ent;
  for (int t = 0; t < EP_NTABLES; t++) {
    ta.off[t] = (uint32_t)ent.size();
    ta.n[t] = h_tables->n[t];
    ta.lo[t] = h_tables->lo[t];
    if (ta.n[t] > EP_HIST_BINS) return EP_ERR_ARG;
    uint32_t cum = 0;
    for (uint32_t i = 0; i < ta.n[t]; i++) {
      const uint32_t f = h_tables->freq[(size_t)t * EP_HIST_BINS + i];
      ent.push_back(f | (cum << 13));
      cum += f;
    }
    if (ta.n[t] && cum != (1u << EP_PRECISION)) return EP_ERR_ARG;
    if (substitute && t >= 1 && ta.n[t] > 0) {
      // widen the field table to every int16 value: a value it lacks takes the entry of its
      // substitute, the most probable value (the lowest on ties)
      const uint16_t* f = h_tables->freq + (size_t)t * EP_HIST_BINS;
      uint32_t best = 0;
      for (uint32_t i = 1; i < ta.n[t]; i++)
        if (f[i] > f[best]) best = i;
      std::vector<uint32_t> wide(EP_HIST_BINS, ent[ta.off[t] + best]);
      for (uint32_t i = 0; i < ta.n[t]; i++)
        if (f[i]) wide[(size_t)(ta.lo[t] + 32768) + i] = ent[ta.off[t] + i];
      ent.resize(ta.off[t]);
      ent.insert(ent.end(), wide.begin(), wide.end());
      ta.lo[t] = -32768;
      ta.n[t] = EP_HIST_BINS;
    }
  }
  if (ent.empty()) ent.push_back(0);
  const uint32_t n_ent = (uint32_t)ent.size();
  if (hipMemcpyAsync(ws.ent, ent.data(), 4 * (size_t)n_ent, hipMemcpyHostToDevice, s) !=
      hipSuccess)
    return EP_ERR_HIP;
  const dim3 grid((tiles + kEncWaves - 1) / kEncWaves);
  const bool lds_tab = n_ent <= kEncLdsEntries;
  const size_t lds = lds_tab ? 4 * (size_t)n_ent : 0;
  // every field table (1..16) within [-128, 127]: the kernel holds the fields as bytes
  bool bytes = true;
  for (int t = 1; t < EP_NTABLES; t++)
    if (ta.n[t] && (ta.lo[t] < -128 || (int64_t)ta.lo[t] + (int64_t)ta.n[t] - 1 > 127))
      bytes = false;
  auto go = [&](auto jc, auto lc) {
    if (bytes)
      launch_enc<decltype(jc)::value, decltype(lc)::value, true>(
          grid, lds, s, S, d_coset, d_fields, nv, tiles, ws.ent, n_ent, ta, ws.counts, d_states,
          ws.stack, d_err);
    else
      launch_enc<decltype(jc)::value, decltype(lc)::value, false>(
          grid, lds, s, S, d_coset, d_fields, nv, tiles, ws.ent, n_ent, ta, ws.counts, d_states,
          ws.stack, d_err);
  };
  using T8 = std::integral_constant<int, 8>;
  using T16 = std::integral_constant<int, 16>;
  using T32 = std::integral_constant<int, 32>;
  auto by_j = [&](auto lc) {
    if (J == 8) go(T8{}, lc);
    else if (J == 16) go(T16{}, lc);
    else go(T32{}, lc);
  };
  if (lds_tab) by_j(std::true_type{});
  else by_j(std::false_type{});
  k_scan_offsets<<<1, 1024, 0, s>>>(ws.counts, tiles, d_word_off, d_max_tile_words,
                                    (uint64_t)words_cap, d_err);
  k_copy_words<<<tiles, 256, 0, s>>>(ws.stack, 9 * V, d_word_off, d_words, (uint64_t)words_cap);
  return hipGetLastError() == hipSuccess ? EP_OK : EP_ERR_HIP;
}

// Exception list: whether vector v has a field its table lacks, from per-table bitmaps of the
// kept values (table 1 + t: 2048 words, bit value + 32768).
__device__ __forceinline__ bool has_escape(const uint8_t* __restrict__ coset,
                                           const uint4* __restrict__ fields,
                                           const uint32_t* __restrict__ keep, uint32_t v,
                                           uint32_t& c, uint4& q) {
  c = coset[v] & 1u;
  q = fields[v];
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  bool esc = false;
#pragma unroll
  for (int k = 0; k < 8; k++) {
    const uint32_t bin = ((k & 1) ? (w[k >> 1] >> 16) : w[k >> 1]) + 32768u;   // int16 + 32768
    const uint32_t b = bin & 0xFFFFu;
    const uint32_t word = keep[(8u * c + (uint32_t)k) * 2048u + (b >> 5)];
    esc |= ((word >> (b & 31u)) & 1u) == 0u;
  }
  return esc;
}

constexpr int kExcThreads = 256;

__global__ __launch_bounds__(kExcThreads) void k_exc_count(const uint8_t* __restrict__ coset,
                                                          const uint4* __restrict__ fields,
                                                          uint32_t nv,
                                                          const uint32_t* __restrict__ keep,
                                                          uint32_t* __restrict__ counts) {
  __shared__ uint32_t s_n[kExcThreads / 64];
  const uint32_t v = blockIdx.x * kExcThreads + threadIdx.x;
  uint32_t c;
  uint4 q;
  const bool esc = v < nv && has_escape(coset, fields, keep, v, c, q);
  const uint64_t m = __ballot(esc);
  if ((threadIdx.x & 63) == 0) s_n[threadIdx.x >> 6] = (uint32_t)__popcll(m);
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int i = 0; i < kExcThreads / 64; i++) t += s_n[i];
    counts[blockIdx.x] = t;
  }
}

// Writes the block's entries in vector order from its first position offsets[block].
__global__ __launch_bounds__(kExcThreads) void k_exc_write(const uint8_t* __restrict__ coset,
                                                          const uint4* __restrict__ fields,
                                                          uint32_t nv,
                                                          const uint32_t* __restrict__ keep,
                                                          const uint32_t* __restrict__ offsets,
                                                          uint32_t* __restrict__ idx,
                                                          uint4* __restrict__ xf) {
  __shared__ uint32_t s_n[kExcThreads / 64];
  const uint32_t v = blockIdx.x * kExcThreads + threadIdx.x;
  uint32_t c = 0;
  uint4 q;
  const bool esc = v < nv && has_escape(coset, fields, keep, v, c, q);
  const uint64_t m = __ballot(esc);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) s_n[wave] = (uint32_t)__popcll(m);
  __syncthreads();
  uint32_t pos = offsets[blockIdx.x];
  for (int i = 0; i < wave; i++) pos += s_n[i];
  pos += __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
  if (esc) {
    idx[pos] = v | (c << 31);
    xf[pos] = q;
  }
}

ep_status find_exceptions(const uint8_t* d_coset, const int16_t* d_fields, int64_t n_vectors,
                          uint32_t tile_fields, const ep_tables* h_tables, void* d_workspace,
                          size_t workspace_bytes, void* d_scratch, std::vector<uint32_t>& idx,
                          std::vector<uint8_t>& fields, hipStream_t s) {
  if (!d_coset || !d_fields || !h_tables || !d_workspace || !d_scratch) return EP_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(d_fields) & 15u) return EP_ERR_ARG;
  if (n_vectors < 1 || n_vectors >= ((int64_t)1 << 31)) return EP_ERR_SHAPE;
  if (workspace_bytes < ep_encode_workspace_bytes(n_vectors, tile_fields)) return EP_ERR_CAPACITY;
  const EncWs ws = enc_carve(d_workspace, n_vectors, tile_fields);
  const uint32_t nv = (uint32_t)n_vectors;
  const uint32_t blocks = (nv + kExcThreads - 1) / kExcThreads;
  // kept-value bitmaps in the entry region; the list's indices, then the block counts, in the
  // tile stacks' region (at least 18 bytes per vector); the fields in d_scratch
  std::vector<uint32_t> keep((size_t)16 * 2048, 0u);
  for (int t = 1; t < EP_NTABLES; t++) {
    const uint16_t* f = h_tables->freq + (size_t)t * EP_HIST_BINS;
    for (uint32_t i = 0; i < h_tables->n[t]; i++)
      if (f[i]) {
        const uint32_t b = (uint32_t)(h_tables->lo[t] + 32768) + i;
        keep[(size_t)(t - 1) * 2048 + (b >> 5)] |= 1u << (b & 31u);
      }
  }
  uint32_t* d_idx = reinterpret_cast<uint32_t*>(ws.stack);
  uint32_t* d_counts = d_idx + ((size_t)nv + 63) / 64 * 64;
  std::vector<uint32_t> counts(blocks);
  const uint4* f4 = reinterpret_cast<const uint4*>(d_fields);
  bool ok = hipMemcpyAsync(ws.ent, keep.data(), 4 * keep.size(), hipMemcpyHostToDevice, s) ==
            hipSuccess;
  k_exc_count<<<blocks, kExcThreads, 0, s>>>(d_coset, f4, nv, ws.ent, d_counts);
  ok &= hipMemcpyAsync(counts.data(), d_counts, 4 * (size_t)blocks, hipMemcpyDeviceToHost, s) ==
        hipSuccess;
  ok &= hipStreamSynchronize(s) == hipSuccess;
  if (!ok) return EP_ERR_HIP;
  uint32_t total = 0;
  for (uint32_t b = 0; b < blocks; b++) {
    const uint32_t c = counts[b];
    counts[b] = total;
    total += c;
  }
  idx.assign(total, 0u);
  fields.assign((size_t)16 * total, 0u);
  if (total == 0) return EP_OK;
  ok &= hipMemcpyAsync(d_counts, counts.data(), 4 * (size_t)blocks, hipMemcpyHostToDevice, s) ==
        hipSuccess;
  k_exc_write<<<blocks, kExcThreads, 0, s>>>(d_coset, f4, nv, ws.ent, d_counts, d_idx,
                                             static_cast<uint4*>(d_scratch));
  ok &= hipMemcpyAsync(idx.data(), d_idx, 4 * (size_t)total, hipMemcpyDeviceToHost, s) ==
        hipSuccess;
  ok &= hipMemcpyAsync(fields.data(), d_scratch, 16 * (size_t)total, hipMemcpyDeviceToHost, s) ==
        hipSuccess;
  ok &= hipStreamSynchronize(s) == hipSuccess;
  return ok && hipGetLastError() == hipSuccess ? EP_OK : EP_ERR_HIP;
}

}  // namespace ep

extern "C" ep_status ep_encode_tiles_gpu(const uint8_t* d_coset, const int16_t* d_fields,
                                         int64_t n_vectors, uint32_t tile_fields, uint32_t lanes,
                                         const ep_tables* h_tables, void* d_workspace,
                                         size_t workspace_bytes, uint32_t* d_word_off,
                                         uint32_t* d_max_tile_words, uint32_t* d_states,
                                         uint16_t* d_words, int64_t words_cap, uint32_t* d_err,
                                         void* stream) {
  ep::clear_pending_error();
  return ep::encode_tiles_dev(d_coset, d_fields, n_vectors, tile_fields, lanes, h_tables, false,
                              d_workspace, workspace_bytes, d_word_off, d_max_tile_words,
                              d_states, d_words, words_cap, d_err,
                              static_cast<hipStream_t>(stream));
}
