// Internal structures shared by the kernel launchers and the host driver of libep.so.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "ep.h"

namespace ep {

// Clears an error that an earlier HIP call outside the library left pending.  Every entry point
// that launches kernels calls it first: its launch checks (hipGetLastError after a launch) then
// report only its own launches.
inline void clear_pending_error() { (void)hipGetLastError(); }

// A shape whose vector count rows * ceil(cols / 8) stays below 2^31 (the library's limit),
// checked without forming the product, so that no caller-supplied size can overflow it.
inline bool shape_fits(int64_t rows, int64_t cols) {
  if (rows < 1 || cols < 1 || cols > ((int64_t)1 << 40)) return false;
  return rows <= (((int64_t)1 << 31) - 1) / ((cols + 7) / 8);
}

// Byte offsets (into the blob) and sizes of the 17 table records, for table expansion.
struct TableArgs {
  int64_t off[EP_NTABLES];
  uint32_t n[EP_NTABLES];
  int32_t lo[EP_NTABLES];
};

// Largest number of wavefronts (= tiles) per decoder workgroup: 16 where the registers allow 4
// or more waves per SIMD, 12 at 3 and 8 at 2.  The launcher picks 16, 12, 8, 4, 2 or 1 from LDS,
// registers and the tile count.
constexpr int kDecWaves = 16;
// Compute units of an MI355X and LDS bytes per CU, for the decoder's workgroup size choice.
constexpr int64_t kCUs = 256;
constexpr int64_t kLdsPerCU = 160 * 1024;
// The decoder's word ring is followed by a copy of its first 64 words (16-bit each).
constexpr uint32_t kRingMirrorBytes = 128;

// The decode tables of one blob (EP_DEC_TABLE_BYTES of device memory).
struct DecTables {
  uint32_t* ent;              // f | (slot - cum) << 13 | (value & 127) << 25: u32[16][4096]
  int16_t* val;               // value: i16[16][4096] (read for wide alphabets)
};
inline DecTables dec_tables(void* base) {
  constexpr size_t n = (size_t)16 * (1u << EP_PRECISION);
  uint8_t* p = static_cast<uint8_t*>(base);
  DecTables d;
  d.ent = reinterpret_cast<uint32_t*>(p);
  d.val = reinterpret_cast<int16_t*>(p + 4 * n);
  return d;
}

// LDS byte offsets of the decoder's slot tables (two phase buffers, two cosets): entries (u32)
// from 0, and for wide alphabets values (i16) from kWideV; the waves' regions follow the tables,
// at kNarTop (narrow alphabets) or kWideTop.
constexpr uint32_t kNarTop = 64 * 1024;
constexpr uint32_t kWideV = 64 * 1024;
constexpr uint32_t kWideTop = 96 * 1024;

// One blob's part of the fused tile decoder's arguments.
struct DecodeBlob {
  const float* alpha;         // f32[rows]
  const uint32_t* word_off;   // u32[tiles + 1]
  const uint32_t* states;     // u32[tiles][K]
  const uint16_t* words;      // u16[payload words], 16-byte aligned section
  const uint32_t* ent;        // slot entries f | (slot - cum) << 13 | value << 25: u32[16][4096]
  const uint16_t* val;        // field value per slot (bits of an i16): u16[16][4096]
  void* out;                  // container[rows][cols]
  uint32_t tile_begin, tile_end;  // tiles of this blob decoded by the launch
  uint32_t n_vec, vpr, max_tile_words, coset_f0;
  int32_t lo0;                // smallest coset value (table 0)
  float inv_vpr_f;
  double inv_vpr;             // 1 / vectors per row
};

// Kernel arguments of the fused tile decoder: up to kMaxBatch blobs per launch (same container,
// tile size and LDS layout).  Workgroups [wg_begin[i], wg_begin[i + 1]) decode blob i.
// 32 descriptors of 96 B (and the fused product's two pointers per blob) keep the arguments
// near 3.7 KiB, inside the 4 KiB kernel-argument space.  Fewer, larger launches also waste less on each launch's last, partly filled round of
// tiles (64 matrices of 3072^2: 589 us in four launches, 541 us in two).
constexpr int kMaxBatch = 32;
struct DecodeArgs {
  uint32_t* err;              // device error word
  uint32_t words_stride;      // words per wave region: the largest tile + slack, or the ring size
  uint32_t n;
  uint32_t wg_begin[kMaxBatch + 1];
  DecodeBlob b[kMaxBatch];
  // the fused product (ep_decompress_matmul[_batch]): Y[m][n] = sum_k X[m][k] W[n][k] per blob
  const void* mm_x[kMaxBatch];  // X: mm_m x mm_cols container values, row-major
  float* mm_y[kMaxBatch];       // Y: mm_m x mm_rows, row-major
  uint32_t mm_m, mm_cols, mm_rows;
  uint32_t mm_kpad;           // columns staged per row (zeros past the last): a multiple of 32
  uint32_t mm_pitch;          // bytes per staged row in LDS
  uint32_t mm_groups;         // 16-row groups per workgroup (1 or 2), taken one after the other
  unsigned long long* stamps; // the traced decode (one blob): per tile, the phase-boundary clocks
};
static_assert(sizeof(DecodeArgs) <= 4096, "kernel arguments");

// Decoder launchers, one translation unit per container dtype and states per lane S (K = 64 S per
// tile): ep_decode_<dtype>.hip (S = 1, with the patch launcher) and ep_decode_<dtype>_k128.hip.
// `slow`: scale without the fused multiply-add (needed for bf16 when some row scale is tiny).
// `rows2`: every blob has at least 64 J vectors per row (a tile spans at most two rows), so the
// kernel keeps two row scales per wave instead of one per vector (used with wide alphabets at
// J = 32, where it lets 3 waves per SIMD fit the registers).
// `ring`: stream each tile's words through an LDS ring of words_stride words (a power of two)
// instead of holding the whole tile.
// DT may also be kFp8Bounded: an fp8 e4m3fn container whose blob is `bounded` (every decoded
// value within +-448), converted without the saturation clamp (S = 1 only).
constexpr int kFp8Bounded = 0x100 | EP_FP8_E4M3FN;
template <int DT, int S>
hipError_t launch_decode(const DecodeArgs& a, int J, bool big, bool ragged, bool slow, bool rows2,
                         bool ring, int waves, size_t lds, hipStream_t s);
// The traced decode (bf16 and fp8 containers): the same kernel recording each tile's phase
// boundaries.  ep_decode_trace.hip.
template <int DT, int S>
hipError_t launch_decode_trace(const DecodeArgs& a, int J, bool big, bool ragged, int waves,
                               size_t lds, hipStream_t s);
// The decode fused into its product (bf16 and fp16 containers, 8 or 16 vectors per lane): one
// workgroup per 16 rows of the matrix, `waves` waves.  ep_decode_mm_<dtype>.hip.
template <int DT, int S>
hipError_t launch_decode_mm(const DecodeArgs& a, int J, bool big, bool ragged, bool slow,
                            int waves, size_t lds, hipStream_t s);

// Rewrites a blob's escaped vectors after its tiles are decoded (ep_decode_<dtype>.hip): idx and
// xf are the exception list on the device (n entries), alpha the blob's row scales.
template <int DT>
hipError_t launch_patch(const uint32_t* idx, const void* xf, uint32_t n, const float* alpha,
                        uint32_t vpr, uint32_t n_vec, void* out, bool slow, uint32_t* err,
                        hipStream_t s);

// Tile encoder (ep_encode.hip), lanes = 64 or 128 states per tile, with an option for tables built
// with escapes: `substitute` codes a
// field value that its table lacks as the table's substitute (its most probable value, the lowest
// on ties) instead of reporting an alphabet error.
ep_status encode_tiles_dev(const uint8_t* d_coset, const int16_t* d_fields, int64_t n_vectors,
                           uint32_t tile_fields, uint32_t lanes, const ep_tables* h_tables,
                           bool substitute,
                           void* d_workspace, size_t workspace_bytes, uint32_t* d_word_off,
                           uint32_t* d_max_tile_words, uint32_t* d_states, uint16_t* d_words,
                           int64_t words_cap, uint32_t* d_err, hipStream_t s);

// The exception list of quantised vectors under tables built with escapes (ep_encode.hip): every
// vector with a field its table lacks, in vector order, as idx = v | coset << 31 and its eight
// fields (16 bytes each).  Uses the encoder workspace and d_scratch (>= 16 bytes per vector) and
// synchronises `s`.
ep_status find_exceptions(const uint8_t* d_coset, const int16_t* d_fields, int64_t n_vectors,
                          uint32_t tile_fields, const ep_tables* h_tables, void* d_workspace,
                          size_t workspace_bytes, void* d_scratch, std::vector<uint32_t>& idx,
                          std::vector<uint8_t>& fields, hipStream_t s);

// Device part of the rate estimate (ep_rate.hip): enqueue on `s` the table build of d_hist and
// the coded-bit sum of its symbols into the rate workspace (the cost table is copied in when
// upload_cost), then copies of the sum, the error word and the 17 table sizes to the host
// pointers, which are valid once `s` has synchronised.  False on a HIP error.
bool estimate_enqueue(const ep_hist* d_hist, void* d_workspace, bool upload_cost, hipStream_t s,
                      double* h_bits, uint32_t* h_err, uint32_t* h_n);
// The device tables inside a rate workspace.
const ep_tables* estimate_tables(void* d_workspace);

}  // namespace ep
