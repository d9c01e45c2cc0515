// Internal structures shared by the kernel launchers and the host driver of libep.so.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ep.h"

namespace ep {

// Byte offsets (into the blob) and sizes of the 17 table records, for table expansion.
struct TableArgs {
  int64_t off[EP_NTABLES];
  uint32_t n[EP_NTABLES];
  int32_t lo[EP_NTABLES];
};

// Largest number of wavefronts (= tiles) per decoder workgroup; the launcher uses 8, 4, 2 or 1,
// the most whose LDS (tables + per-wave words) fits in a CU.
constexpr int kDecWaves = 8;

// Kernel arguments of the fused tile decoder.
struct DecodeArgs {
  const float* alpha;         // f32[rows]
  const uint32_t* word_off;   // u32[tiles + 1]
  const uint32_t* states;     // u32[tiles][64]
  const uint16_t* words;      // u16[payload words], 16-byte aligned section
  const uint32_t* ent;        // expanded field tables: u32[16][4096]
  const int16_t* val;         // field value per slot: i16[16][4096]
  void* out;                  // container[rows][cols]
  uint32_t* err;              // device error word
  uint32_t tile_begin, tile_end;  // tiles decoded by this launch
  uint32_t n_vec, vpr, max_tile_words, words_stride, coset_f0;
  double inv_vpr;
  int32_t lo[EP_NTABLES];
};

// Decoder launchers, one translation unit per container dtype (ep_decode_<dtype>.hip).
template <int DT>
hipError_t launch_decode(const DecodeArgs& a, int J, bool big, bool ragged, int waves,
                         size_t lds, hipStream_t s);

}  // namespace ep
