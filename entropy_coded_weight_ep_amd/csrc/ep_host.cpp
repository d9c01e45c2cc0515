// Host side of libep.so: table normalisation, the interleaved rANS tile encoder, the blob
// format, the sampled-row rate search and the compress driver.
//
// Sources: EntroPack design page "EntroPack lattice compression" -- "Lattice quantization and
// integer fields" (coset-conditioned model), "Rate selection and refinement" (sampled-row size
// estimate incl. metadata, per-row least squares), "Encoding and reconstruction" (rANS in
// independently decodable tiles; stored tables, row scales, tile metadata; actual_bpp).
// rANS: Duda, "Asymmetric numeral systems" (arXiv 0902.0271); several states sharing one word
// stream: Giesen, "Interleaved entropy coders" (arXiv 1402.3392).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "ep.h"
#include "ep_internal.h"

namespace {

constexpr uint32_t kM = 1u << EP_PRECISION;
constexpr uint32_t kL = 1u << 16;
constexpr int kK = EP_LANES;          // states per tile by default
constexpr int kMaxK = 2 * EP_LANES;   // the most the format allows (two per wavefront lane)

// A lane count the blob format takes for a tile of tile_fields fields: 64 or 128, dividing the
// tile's vector count.
inline bool lanes_ok(int64_t lanes, int64_t tile_fields) {
  return (lanes == kK || lanes == kMaxK) && (tile_fields / 8) % lanes == 0;
}
constexpr int kHeaderBytes = 64;

inline int64_t round16(int64_t b) { return (b + 15) / 16 * 16; }
inline int64_t record_bytes(uint32_t n) { return (8 + 2 * (int64_t)n + 3) / 4 * 4; }

int64_t tables_bytes(const uint32_t* n) {
  int64_t b = 0;
  for (int t = 0; t < EP_NTABLES; t++) b += record_bytes(n[t]);
  return round16(b);
}

struct Layout {
  int64_t tables, alpha, word_off, states, words, exc_idx, exc_fields, total;
};

// Sections in blob order; a blob with escapes (version 1.1) ends with its exception list: the
// indices u32[n_exc], then the fields i16[n_exc][8].
Layout layout(int64_t rows, int64_t tiles, int64_t lanes, int64_t table_bytes, int64_t words,
              int64_t n_exc = 0) {
  Layout L;
  L.tables = kHeaderBytes;
  L.alpha = L.tables + table_bytes;
  L.word_off = L.alpha + round16(4 * rows);
  L.states = L.word_off + round16(4 * (tiles + 1));
  L.words = L.states + round16(4 * lanes * tiles);
  L.exc_idx = L.words + round16(2 * words);
  L.exc_fields = L.exc_idx + round16(4 * n_exc);
  L.total = n_exc > 0 ? L.exc_fields + 16 * n_exc : L.exc_idx;
  return L;
}

// Frequencies summing to M for one table's counts (rule documented in ep.h, ep_build_tables).
ep_status normalise(const uint32_t* cnt, uint32_t n, uint16_t* out) {
  uint64_t total = 0;
  uint32_t distinct = 0;
  for (uint32_t i = 0; i < n; i++) {
    total += cnt[i];
    distinct += cnt[i] != 0;
  }
  if (distinct > kM) return EP_ERR_ALPHABET;
  std::vector<int64_t> f(n, 0);
  int64_t assigned = 0;
  for (uint32_t i = 0; i < n; i++) {
    if (!cnt[i]) continue;
    f[i] = std::max<int64_t>(1, (int64_t)(((uint64_t)cnt[i] * kM) / total));
    assigned += f[i];
  }
  int64_t gap = (int64_t)kM - assigned;
  if (gap > 0) {
    uint32_t top = 0;
    for (uint32_t i = 1; i < n; i++)
      if (cnt[i] > cnt[top]) top = i;
    f[top] += gap;
  }
  while (gap < 0) {
    int64_t top = -1;
    for (uint32_t i = 0; i < n; i++)
      if (f[i] > 1 && (top < 0 || f[i] > f[top])) top = i;
    const int64_t take = std::min(-gap, f[top] - 1);
    f[top] -= take;
    gap += take;
  }
  for (uint32_t i = 0; i < n; i++) out[i] = (uint16_t)f[i];
  return EP_OK;
}

// Per-table symbol lookups for the encoder.
struct EncTable {
  int32_t lo = 0;
  uint32_t n = 0;
  std::vector<uint32_t> freq, cum;
};

std::vector<EncTable> enc_tables(const ep_tables* T) {
  std::vector<EncTable> out(EP_NTABLES);
  for (int t = 0; t < EP_NTABLES; t++) {
    EncTable& e = out[t];
    e.lo = T->lo[t];
    e.n = T->n[t];
    e.freq.resize(e.n);
    e.cum.resize(e.n);
    uint32_t c = 0;
    for (uint32_t i = 0; i < e.n; i++) {
      e.freq[i] = T->freq[(size_t)t * EP_HIST_BINS + i];
      e.cum[i] = c;
      c += e.freq[i];
    }
  }
  return out;
}

// Encode one tile into `stream` (forward word order) and its K final states (state k owns the
// tile's vectors k, k + K, ...; J = vectors per state).
bool encode_tile(const uint8_t* cs, const int16_t* fs, int64_t v0, int64_t nvt, int J, int K,
                 const std::vector<EncTable>& tabs, uint32_t* states,
                 std::vector<uint16_t>& scratch, std::vector<uint16_t>& stream) {
  uint32_t x[kMaxK];
  std::fill(x, x + K, kL);
  scratch.clear();
  for (int phase = 8; phase >= 0; --phase) {
    for (int j = J - 1; j >= 0; --j) {
      for (int l = K - 1; l >= 0; --l) {
        const int64_t u = l + (int64_t)K * j;
        if (u >= nvt) continue;
        const int64_t v = v0 + u;
        const int c = cs[v];
        const EncTable& tb = (phase == 0) ? tabs[0] : tabs[1 + 8 * c + (phase - 1)];
        const int32_t value = (phase == 0) ? c : fs[8 * v + (phase - 1)];
        const int64_t s = (int64_t)value - tb.lo;
        if (s < 0 || s >= (int64_t)tb.n || tb.freq[s] == 0) return false;
        const uint32_t f = tb.freq[s];
        uint32_t xs = x[l];
        if ((uint64_t)xs >= ((uint64_t)f << (32 - EP_PRECISION))) {
          scratch.push_back((uint16_t)xs);
          xs >>= 16;
        }
        x[l] = (xs / f) * kM + (xs % f) + tb.cum[s];
      }
    }
  }
  stream.insert(stream.end(), scratch.rbegin(), scratch.rend());
  std::copy(x, x + K, states);
  return true;
}

struct Hip {
  hipError_t e = hipSuccess;
  bool ok() const { return e == hipSuccess; }
  void operator()(hipError_t r) {
    if (e == hipSuccess) e = r;
  }
};

}  // namespace

// ==========================================================================================
extern "C" const char* ep_status_string(ep_status st) {
  switch (st) {
    case EP_OK: return "ok";
    case EP_ERR_ARG: return "invalid argument";
    case EP_ERR_SHAPE: return "unsupported shape (cols must be a multiple of 8)";
    case EP_ERR_DTYPE: return "unsupported container dtype";
    case EP_ERR_NONFINITE: return "input holds NaN or infinity";
    case EP_ERR_RANGE: return "lattice coordinate outside the int16 field range";
    case EP_ERR_ALPHABET: return "more than 2^P distinct symbols in one table";
    case EP_ERR_CORRUPT: return "corrupt blob or tile";
    case EP_ERR_VERSION: return "unsupported blob version or parameters";
    case EP_ERR_HIP: return "HIP runtime error";
    case EP_ERR_CAPACITY: return "buffer too small";
  }
  return "unknown status";
}

extern "C" void ep_config_default(ep_config* cfg) {
  if (!cfg) return;
  cfg->target_bpp = 4.0;
  cfg->tile_fields = 8192;
  cfg->sample_rows = 256;
  cfg->search_iters = 40;
  cfg->lanes = kK;
  cfg->rate_check = 1;
  cfg->refine = 0;
  cfg->force_scale = 0.0;
}

namespace {
// Table t of h_out from its counts c (EP_HIST_BINS bins).
ep_status build_table(const uint32_t* c, int t, ep_tables* h_out) {
  {
    int first = -1, last = -1;
    for (int b = 0; b < EP_HIST_BINS; b++) {
      if (c[b]) {
        if (first < 0) first = b;
        last = b;
      }
    }
    uint16_t* f = h_out->freq + (size_t)t * EP_HIST_BINS;
    if (first < 0) {
      h_out->lo[t] = 0;
      h_out->n[t] = 0;
      return EP_OK;
    }
    h_out->lo[t] = first - 32768;
    h_out->n[t] = (uint32_t)(last - first + 1);
    return normalise(c + first, h_out->n[t], f);
  }
}

// Tables with escapes: a field table whose counts hold more than M distinct values keeps the M
// most frequent (larger count first, lower value on ties) and is built over those alone; its
// other values are escaped (coded as the table's substitute and listed as exceptions).
ep_status build_tables_escaped(const ep_hist* h_hist, ep_tables* h_out) {
  std::vector<uint32_t> kept(EP_HIST_BINS);
  std::vector<std::pair<uint32_t, int>> order;
  for (int t = 0; t < EP_NTABLES; t++) {
    const uint32_t* c = h_hist->counts + (size_t)t * EP_HIST_BINS;
    order.clear();
    for (int b = 0; b < EP_HIST_BINS; b++)
      if (c[b]) order.emplace_back(c[b], b);
    if (t >= 1 && order.size() > (size_t)kM) {
      std::sort(order.begin(), order.end(), [](const auto& x, const auto& y) {
        return x.first != y.first ? x.first > y.first : x.second < y.second;
      });
      std::fill(kept.begin(), kept.end(), 0u);
      for (uint32_t i = 0; i < kM; i++) kept[order[i].second] = order[i].first;
      c = kept.data();
    }
    const ep_status st = build_table(c, t, h_out);
    if (st != EP_OK) return st;
  }
  return EP_OK;
}
}  // namespace

extern "C" ep_status ep_build_tables(const ep_hist* h_hist, uint32_t precision_bits,
                                     ep_tables* h_out) {
  if (!h_hist || !h_out) return EP_ERR_ARG;
  if (precision_bits != EP_PRECISION) return EP_ERR_ARG;
  for (int t = 0; t < EP_NTABLES; t++) {
    const ep_status st = build_table(h_hist->counts + (size_t)t * EP_HIST_BINS, t, h_out);
    if (st != EP_OK) return st;
  }
  return EP_OK;
}

namespace {
// Bits per element from the sampled symbols' coded size `acc` (bits) and the table sizes:
// the sample scaled to all rows, plus every byte of the blob before the payload words.
double finish_estimate(double acc, const uint32_t* n, int64_t rows, int64_t cols,
                       int64_t n_sample_rows, uint32_t tile_fields, uint32_t lanes) {
  const double bits = acc * ((double)rows / (double)n_sample_rows);
  const int64_t nv = rows * ((cols + 7) / 8), V = tile_fields / 8, tiles = (nv + V - 1) / V;
  const Layout L = layout(rows, tiles, lanes, tables_bytes(n), 0);
  const double meta = (double)L.words;      // everything before the payload words
  return (bits + 8.0 * meta) / ((double)rows * (double)cols);
}
}  // namespace

extern "C" double ep_estimate_bpp(const ep_hist* h_hist, int64_t rows, int64_t cols,
                                  int64_t n_sample_rows, uint32_t tile_fields, uint32_t lanes) {
  if (!h_hist || !ep::shape_fits(rows, cols) || n_sample_rows < 1 || tile_fields < 8 ||
      !lanes_ok(lanes, tile_fields))
    return INFINITY;
  std::vector<ep_tables> tv(1);
  ep_tables& T = tv[0];
  if (ep_build_tables(h_hist, EP_PRECISION, &T) != EP_OK) return INFINITY;
  double acc = 0.0;
  for (int t = 0; t < EP_NTABLES; t++) {
    const uint32_t* c = h_hist->counts + (size_t)t * EP_HIST_BINS + (T.lo[t] + 32768);
    for (uint32_t i = 0; i < T.n[t]; i++) {
      if (!c[i]) continue;
      const double f = (double)T.freq[(size_t)t * EP_HIST_BINS + i];
      acc = acc + (double)c[i] * ((double)EP_PRECISION - std::log2(f));
    }
  }
  return finish_estimate(acc, T.n, rows, cols, n_sample_rows, tile_fields, lanes);
}

extern "C" double ep_estimate_bpp_gpu(const ep_hist* d_hist, int64_t rows, int64_t cols,
                                      int64_t n_sample_rows, uint32_t tile_fields, uint32_t lanes,
                                      void* d_workspace, size_t workspace_bytes, void* stream) {
  ep::clear_pending_error();
  if (!d_hist || !d_workspace || !ep::shape_fits(rows, cols) || n_sample_rows < 1 ||
      tile_fields < 8 || !lanes_ok(lanes, tile_fields))
    return INFINITY;
  if (workspace_bytes < ep_estimate_workspace_bytes()) return INFINITY;
  hipStream_t s = static_cast<hipStream_t>(stream);
  double bits = 0.0;
  uint32_t err = 0, n[EP_NTABLES];
  if (!ep::estimate_enqueue(d_hist, d_workspace, true, s, &bits, &err, n) ||
      hipStreamSynchronize(s) != hipSuccess)
    return NAN;
  if (err) return INFINITY;
  return finish_estimate(bits, n, rows, cols, n_sample_rows, tile_fields, lanes);
}

extern "C" void ep_rate_costs(uint32_t* h_cost) {
  if (!h_cost) return;
  h_cost[0] = (uint32_t)(EP_PRECISION + 1) * 65536u;
  for (uint32_t f = 1; f <= kM; f++)
    h_cost[f] = (uint32_t)std::llround(((double)EP_PRECISION - std::log2((double)f)) * 65536.0);
}

namespace {
// Total rate of the per-row choice minimising D + lambda * bits (first minimum in candidate
// order; candidates with D = +inf are not offered); the choice goes to sel.
int64_t pick_at(const double* D, const int64_t* Rq, int64_t rows, int nc, double lambda,
                int32_t* sel) {
  int64_t total = 0;
  for (int64_t r = 0; r < rows; r++) {
    int best = -1;
    double bj = 0.0;
    for (int k = 0; k < nc; k++) {
      const double d = D[r * nc + k];
      if (std::isinf(d)) continue;
      const double bits = (double)Rq[r * nc + k] / 65536.0;
      const double j = d + lambda * bits;
      if (best < 0 || j < bj) {
        best = k;
        bj = j;
      }
    }
    if (best < 0) best = 0;
    sel[r] = best;
    total += Rq[r * nc + best];
  }
  return total;
}
}  // namespace

extern "C" double ep_refine_select(const double* h_D, const int64_t* h_Rq, int64_t rows,
                                   int32_t nc, int64_t budget_q, int32_t* h_sel) {
  if (!h_D || !h_Rq || !h_sel || rows < 1 || nc < 1) return NAN;
  if (pick_at(h_D, h_Rq, rows, nc, 0.0, h_sel) <= budget_q) return 0.0;
  if (pick_at(h_D, h_Rq, rows, nc, std::exp2(60.0), h_sel) > budget_q) return std::exp2(60.0);
  double lo = -60.0, hi = 60.0;
  for (int it = 0; it < 60; it++) {
    const double mid = 0.5 * (lo + hi);
    if (pick_at(h_D, h_Rq, rows, nc, std::exp2(mid), h_sel) <= budget_q) hi = mid;
    else lo = mid;
  }
  pick_at(h_D, h_Rq, rows, nc, std::exp2(hi), h_sel);
  return std::exp2(hi);
}

extern "C" ep_status ep_encode_tiles(const uint8_t* h_coset, const int16_t* h_fields,
                                     int64_t n_vectors, uint32_t tile_fields, uint32_t lanes,
                                     const ep_tables* tables, uint32_t* h_word_off,
                                     uint32_t* h_states, uint16_t* h_words, int64_t words_cap) {
  if (!h_coset || !h_fields || !tables || !h_word_off || !h_states || !h_words) return EP_ERR_ARG;
  if (tile_fields < 512 || tile_fields % 512 || n_vectors < 1) return EP_ERR_ARG;
  if (!lanes_ok(lanes, tile_fields)) return EP_ERR_ARG;
  const int K = (int)lanes;
  const int64_t V = tile_fields / 8, tiles = (n_vectors + V - 1) / V;
  const int J = (int)(V / K);
  const std::vector<EncTable> tabs = enc_tables(tables);
  unsigned nth = std::max(1u, std::thread::hardware_concurrency());
  nth = (unsigned)std::min<int64_t>(nth, tiles);
  // each worker encodes a contiguous tile range into its own stream
  std::vector<std::vector<uint16_t>> streams(nth);
  std::vector<std::vector<uint32_t>> counts(nth);
  std::vector<int> ok(nth, 1);
  auto work = [&](unsigned w) {
    const int64_t t0 = tiles * w / nth, t1 = tiles * (w + 1) / nth;
    std::vector<uint16_t> scratch;
    scratch.reserve(9 * V);
    for (int64_t t = t0; t < t1; t++) {
      const size_t before = streams[w].size();
      const int64_t v0 = t * V, nvt = std::min<int64_t>(V, n_vectors - v0);
      if (!encode_tile(h_coset, h_fields, v0, nvt, J, K, tabs, h_states + t * K, scratch,
                       streams[w])) {
        ok[w] = 0;
        return;
      }
      counts[w].push_back((uint32_t)(streams[w].size() - before));
    }
  };
  std::vector<std::thread> pool;
  for (unsigned w = 1; w < nth; w++) pool.emplace_back(work, w);
  work(0);
  for (auto& th : pool) th.join();
  for (unsigned w = 0; w < nth; w++)
    if (!ok[w]) return EP_ERR_ARG;
  int64_t pos = 0, t = 0;
  for (unsigned w = 0; w < nth; w++) {
    if (pos + (int64_t)streams[w].size() > words_cap) return EP_ERR_CAPACITY;
    std::memcpy(h_words + pos, streams[w].data(), streams[w].size() * 2);
    for (uint32_t c : counts[w]) {
      h_word_off[t++] = (uint32_t)pos;
      pos += c;
    }
  }
  h_word_off[tiles] = (uint32_t)pos;
  return EP_OK;
}

extern "C" ep_status ep_compress_bound(int64_t rows, int64_t cols, uint32_t tile_fields,
                                       size_t* bytes) {
  if (!bytes) return EP_ERR_ARG;
  if (!ep::shape_fits(rows, cols)) return EP_ERR_SHAPE;
  if (tile_fields < 512 || tile_fields % 512) return EP_ERR_ARG;
  const int64_t nv = rows * ((cols + 7) / 8), V = tile_fields / 8, tiles = (nv + V - 1) / V;
  uint32_t nmax[EP_NTABLES];
  for (int t = 0; t < EP_NTABLES; t++) nmax[t] = 65535;
  *bytes = (size_t)layout(rows, tiles, kMaxK, tables_bytes(nmax), 9 * nv, nv).total;
  return EP_OK;
}

namespace {
struct Workspace {
  ep_hist* hist;
  double* sumsq;
  float* gains;
  int64_t* rows_sel;
  double* num;
  int64_t* den4;
  uint32_t* err;
  uint8_t* coset;
  int16_t* fields;
  void* rate;           // device rate estimate (tables, cost table, sums)
  void* enc;            // device tile encoder workspace
  size_t enc_bytes;
  uint32_t* word_off;   // encoder outputs: u32[tiles + 1], u32[1], u32[tiles * 64], u16[9 NV + 1]
  uint32_t* max_words;
  uint32_t* cost;       // refinement: fixed-point code lengths, u32[2^P + 1]
  int64_t* rates;       // refinement: per-row rates, i64[rows]
  uint32_t* states;
  uint16_t* words;
  size_t total;
};

// Tile sizes the device tile encoder (and the device decoder) handle: 8, 16 or 32 vectors a lane.
inline bool device_tile_size(uint32_t F) { return F == 4096 || F == 8192 || F == 16384; }

Workspace carve(void* base, int64_t rows, int64_t cols) {
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  uint8_t* p = static_cast<uint8_t*>(base);
  size_t o = 0;
  Workspace w;
  const int64_t nv = rows * ((cols + 7) / 8);
  w.hist = reinterpret_cast<ep_hist*>(p + o); o += up(sizeof(ep_hist));
  w.sumsq = reinterpret_cast<double*>(p + o); o += up(8 * rows);
  w.gains = reinterpret_cast<float*>(p + o); o += up(4 * rows);
  w.rows_sel = reinterpret_cast<int64_t*>(p + o); o += up(8 * (size_t)std::min<int64_t>(rows, 1 << 20));
  w.num = reinterpret_cast<double*>(p + o); o += up(8 * rows);
  w.den4 = reinterpret_cast<int64_t*>(p + o); o += up(8 * rows);
  w.err = reinterpret_cast<uint32_t*>(p + o); o += up(4);
  w.coset = p + o; o += up(nv);
  w.fields = reinterpret_cast<int16_t*>(p + o); o += up(2 * 8 * nv);
  w.rate = p + o; o += up(ep_estimate_workspace_bytes());
  // the device encoder's workspace and outputs, sized for the smallest tiles it takes (the
  // most tiles) and the largest (the most rounding of the last tile)
  w.enc_bytes = std::max({ep_encode_workspace_bytes(nv, 4096), ep_encode_workspace_bytes(nv, 8192),
                          ep_encode_workspace_bytes(nv, 16384)});
  const int64_t max_tiles = (nv + 511) / 512;
  w.enc = p + o; o += up(w.enc_bytes);
  w.word_off = reinterpret_cast<uint32_t*>(p + o); o += up(4 * (max_tiles + 1));
  w.max_words = reinterpret_cast<uint32_t*>(p + o); o += up(4);
  w.states = reinterpret_cast<uint32_t*>(p + o); o += up(4 * (size_t)kMaxK * max_tiles);
  w.words = reinterpret_cast<uint16_t*>(p + o); o += up(2 * (9 * (size_t)nv + 1));
  w.cost = reinterpret_cast<uint32_t*>(p + o); o += up(4 * (size_t)(kM + 1));
  w.rates = reinterpret_cast<int64_t*>(p + o); o += up(8 * (size_t)rows);
  w.total = o;
  return w;
}

inline float row_gain(double sumsq, int64_t cols, double s) {
  const double rms = std::sqrt(sumsq / (double)cols);
  if (rms == 0.0) return 0.0f;
  return (float)(1.0 / (rms * s));
}
}  // namespace

extern "C" size_t ep_compress_workspace_bytes(int64_t rows, int64_t cols) {
  if (!ep::shape_fits(rows, cols)) return 0;
  return carve(nullptr, rows, cols).total;
}

extern "C" ep_status ep_blob_parse(const void* h_blob, size_t bytes, ep_blob_info* out) {
  if (!h_blob || !out) return EP_ERR_ARG;
  const uint8_t* b = static_cast<const uint8_t*>(h_blob);
  if (bytes < (size_t)kHeaderBytes || std::memcmp(b, "EPK1", 4) != 0) return EP_ERR_CORRUPT;
  // version 1.0, or 1.1 for a blob that lists escaped vectors
  if (b[4] != 1 || b[5] > 1) return EP_ERR_VERSION;
  ep_blob_info I;
  std::memset(&I, 0, sizeof I);
  I.dtype = b[6];
  I.precision = b[7];
  uint64_t u64;
  uint32_t u32;
  std::memcpy(&u64, b + 8, 8); I.rows = (int64_t)u64;
  std::memcpy(&u64, b + 16, 8); I.cols = (int64_t)u64;
  std::memcpy(&u32, b + 24, 4); I.tile_fields = (int32_t)u32;
  std::memcpy(&u32, b + 28, 4); I.lanes = (int32_t)u32;
  std::memcpy(&u32, b + 32, 4); I.tiles = u32;
  uint32_t tb;
  std::memcpy(&tb, b + 36, 4);
  std::memcpy(&I.scale, b + 40, 8);
  std::memcpy(&u64, b + 48, 8); I.payload_words = (int64_t)u64;
  std::memcpy(&I.max_tile_words, b + 56, 4);
  if (I.dtype < EP_BF16 || I.dtype > EP_FP32) return EP_ERR_DTYPE;
  if (I.precision != EP_PRECISION || (I.lanes != kK && I.lanes != kMaxK)) return EP_ERR_VERSION;
  if (I.rows < 1 || I.cols < 1 || I.tile_fields < 512 || I.tile_fields % 512 ||
      !lanes_ok(I.lanes, I.tile_fields))
    return EP_ERR_CORRUPT;
  if (I.rows > ((int64_t)1 << 40) || I.cols > ((int64_t)1 << 40)) return EP_ERR_CORRUPT;
  // the vector count must stay below 2^31 (the limit of compress and decode); checked before the
  // product is formed, so a crafted header cannot overflow it
  const int64_t vpr = (I.cols + 7) / 8;
  if (I.rows > (((int64_t)1 << 31) - 1) / vpr) return EP_ERR_CORRUPT;
  const int64_t nv = I.rows * vpr, V = I.tile_fields / 8;
  if (I.tiles != (nv + V - 1) / V) return EP_ERR_CORRUPT;
  if (I.payload_words < 0 || I.payload_words > ((int64_t)1 << 32)) return EP_ERR_CORRUPT;
  uint32_t n_exc;
  std::memcpy(&n_exc, b + 60, 4);
  if ((b[5] == 0) != (n_exc == 0) || (int64_t)n_exc > nv) return EP_ERR_CORRUPT;
  const Layout L = layout(I.rows, I.tiles, I.lanes, tb, I.payload_words, n_exc);
  if ((int64_t)bytes != L.total) return EP_ERR_CORRUPT;
  // the exception list names vectors in increasing order, each inside the tensor
  for (uint32_t i = 0; i < n_exc; i++) {
    uint32_t e, prev = 0;
    std::memcpy(&e, b + L.exc_idx + 4 * (int64_t)i, 4);
    if (i > 0) std::memcpy(&prev, b + L.exc_idx + 4 * (int64_t)(i - 1), 4);
    const int64_t v = e & 0x7FFFFFFFu;
    if (v >= nv || (i > 0 && v <= (int64_t)(prev & 0x7FFFFFFFu))) return EP_ERR_CORRUPT;
  }
  int64_t p = L.tables;
  bool big = false;
  for (int t = 0; t < EP_NTABLES; t++) {
    if (p + 8 > L.alpha) return EP_ERR_CORRUPT;
    int32_t lo;
    uint32_t n;
    std::memcpy(&lo, b + p, 4);
    std::memcpy(&n, b + p + 4, 4);
    if (n > 65535 || p + record_bytes(n) > L.alpha) return EP_ERR_CORRUPT;
    uint32_t sum = 0;
    for (uint32_t i = 0; i < n; i++) {
      uint16_t f;
      std::memcpy(&f, b + p + 8 + 2 * i, 2);
      sum += f;
    }
    if (n && sum != kM) return EP_ERR_CORRUPT;
    if (t == 0) {
      // coset table: one or two symbols inside {0, 1}
      if (n < 1 || n > 2 || lo < 0 || lo + (int64_t)n > 2) return EP_ERR_CORRUPT;
      uint16_t f0;
      std::memcpy(&f0, b + p + 8, 2);
      if (f0 == 0) return EP_ERR_CORRUPT;
      I.coset_freq0 = f0;
    } else if (n > 0 && (lo < -64 || lo + (int64_t)n - 1 > 63)) {
      big = true;                 // field values do not all fit the 7-bit slot-entry value
    }
    I.table_off[t] = p;
    I.lo[t] = lo;
    I.n[t] = n;
    p += record_bytes(n);
  }
  if (round16(p - L.tables) != (int64_t)tb) return EP_ERR_CORRUPT;
  // row scales must be finite (the decoder's saturating conversions assume it); a nonzero scale
  // below 2^-125 in magnitude has an inexact half, which the decoder's fused scaling needs exact
  bool tiny = false;
  float max_alpha = 0.0f;
  for (int64_t r = 0; r < I.rows; r++) {
    float alpha;
    std::memcpy(&alpha, b + L.alpha + 4 * r, 4);
    if (!std::isfinite(alpha)) return EP_ERR_CORRUPT;
    tiny |= alpha != 0.0f && std::fabs(alpha) < 0x1p-125f;
    max_alpha = std::max(max_alpha, std::fabs(alpha));
  }
  // the largest |p| the tile decode can produce: a field of table 1 + 8c + k lies in
  // [lo, lo + n - 1]; z7 = 2 f7 + parity; p = z + c/2.  (Escaped vectors, rewritten by the patch
  // pass with its own conversion, are not bounded by this.)  Both products below are exact in
  // double: max_alpha has 24 significant bits, max_p at most 18.
  double max_p = 0.0;
  for (int t = 1; t < EP_NTABLES; t++) {
    if (I.n[t] == 0) continue;
    const int c = (t - 1) / 8, k = (t - 1) % 8;
    int64_t m = std::max(std::llabs((int64_t)I.lo[t]), std::llabs((int64_t)I.lo[t] + I.n[t] - 1));
    if (k == 7) m = 2 * m + 1;
    max_p = std::max(max_p, (double)m + 0.5 * c);
  }
  I.bounded = (double)max_alpha * max_p <= 448.0 ? 1u : 0u;
  const uint32_t* off = reinterpret_cast<const uint32_t*>(b + L.word_off);
  if (off[0] != 0 || (int64_t)off[I.tiles] != I.payload_words) return EP_ERR_CORRUPT;
  uint32_t maxw = 0;
  for (int64_t t = 0; t < I.tiles; t++) {
    if (off[t + 1] < off[t]) return EP_ERR_CORRUPT;
    maxw = std::max(maxw, off[t + 1] - off[t]);
  }
  if (maxw != I.max_tile_words) return EP_ERR_CORRUPT;
  I.big_alphabet = big ? 1u : 0u;
  I.tiny_scale = tiny ? 1u : 0u;
  I.bytes = (int64_t)bytes;
  I.actual_bpp = 8.0 * (double)bytes / ((double)I.rows * (double)I.cols);
  I.off_tables = L.tables;
  I.off_alpha = L.alpha;
  I.off_word_off = L.word_off;
  I.off_states = L.states;
  I.off_words = L.words;
  I.n_exceptions = n_exc;
  I.off_exceptions = n_exc > 0 ? L.exc_idx : 0;
  I.off_exception_fields = n_exc > 0 ? L.exc_fields : 0;
  *out = I;
  return EP_OK;
}

extern "C" ep_status ep_compress(const void* d_w, int32_t dtype, int64_t rows, int64_t cols,
                                 const ep_config* cfg, void* d_workspace, size_t workspace_bytes,
                                 void* h_blob, size_t cap, size_t* out_bytes, double* scale_out,
                                 void* stream) {
  ep::clear_pending_error();
  if (!d_w || !cfg || !d_workspace || !h_blob || !out_bytes) return EP_ERR_ARG;
  if (dtype < EP_BF16 || dtype > EP_FP32) return EP_ERR_DTYPE;
  if (rows < 1 || cols < 1) return EP_ERR_SHAPE;
  const uint32_t F = cfg->tile_fields;
  if (!device_tile_size(F)) return EP_ERR_ARG;        // the tile sizes the GPU decodes
  const uint32_t K = cfg->lanes;
  if (!lanes_ok(K, F)) return EP_ERR_ARG;
  const int nc = (int)cfg->refine;
  if (cfg->refine > 9 || (nc > 0 && nc % 2 == 0)) return EP_ERR_ARG;
  if (nc > 0 && !(std::isfinite(cfg->target_bpp) && cfg->target_bpp >= 0.001 &&
                  cfg->target_bpp <= 11.0))
    return EP_ERR_ARG;
  const bool forced = cfg->force_scale > 0.0;
  if (!forced && !(std::isfinite(cfg->target_bpp) && cfg->target_bpp >= 0.001 &&
                   cfg->target_bpp <= 11.0))
    return EP_ERR_ARG;
  if (!ep::shape_fits(rows, cols)) return EP_ERR_SHAPE;
  const int64_t nv = rows * ((cols + 7) / 8);
  if (workspace_bytes < ep_compress_workspace_bytes(rows, cols)) return EP_ERR_CAPACITY;
  const Workspace ws = carve(d_workspace, rows, cols);
  hipStream_t s = static_cast<hipStream_t>(stream);
  Hip hip;
  ep_status st;

  // 1. row RMS
  std::vector<double> sumsq(rows);
  if ((st = ep_row_sumsq(d_w, dtype, rows, cols, ws.sumsq, stream)) != EP_OK) return st;
  hip(hipMemcpyAsync(sumsq.data(), ws.sumsq, 8 * rows, hipMemcpyDeviceToHost, s));
  hip(hipStreamSynchronize(s));
  if (!hip.ok()) return EP_ERR_HIP;
  for (double v : sumsq)
    if (!std::isfinite(v)) return EP_ERR_NONFINITE;

  std::vector<float> gains(rows, 0.0f);
  uint32_t err_host = 0;
  const uint32_t zero = 0;

  // enqueue the quantisation of (a subset of) rows at scale sc, with its histogram
  auto quantise = [&](double sc, const int64_t* d_sel, int64_t nsel,
                      const std::vector<int64_t>& sel) -> ep_status {
    if (d_sel) {
      for (int64_t r : sel) gains[r] = row_gain(sumsq[r], cols, sc);
    } else {
      for (int64_t r = 0; r < rows; r++) gains[r] = row_gain(sumsq[r], cols, sc);
    }
    hip(hipMemcpyAsync(ws.gains, gains.data(), 4 * rows, hipMemcpyHostToDevice, s));
    hip(hipMemcpyAsync(ws.err, &zero, 4, hipMemcpyHostToDevice, s));
    return ep_quantize_e8(d_w, dtype, rows, cols, ws.gains, d_sel, nsel, ws.coset, ws.fields,
                          ws.hist, ws.err, stream);
  };

  // enqueue the quantisation of all rows with the given per-row gains (histogram optional)
  auto quantise_with = [&](const float* g, bool with_hist) -> ep_status {
    hip(hipMemcpyAsync(ws.gains, g, 4 * rows, hipMemcpyHostToDevice, s));
    hip(hipMemcpyAsync(ws.err, &zero, 4, hipMemcpyHostToDevice, s));
    return ep_quantize_e8(d_w, dtype, rows, cols, ws.gains, nullptr, rows, ws.coset, ws.fields,
                          with_hist ? ws.hist : nullptr, ws.err, stream);
  };

  // 2. rate search on sampled rows: per candidate the device quantises the sample, builds the
  // tables and sums the coded bits; the host gets the sum and the table sizes
  double sc;
  if (forced) {
    sc = cfg->force_scale;
  } else {
    const int64_t ns = std::min<int64_t>(std::min<int64_t>(rows, std::max<uint32_t>(1, cfg->sample_rows)),
                                         (int64_t)1 << 20);
    std::vector<int64_t> sel(ns);
    for (int64_t i = 0; i < ns; i++) sel[i] = (i * rows) / ns;
    hip(hipMemcpyAsync(ws.rows_sel, sel.data(), 8 * ns, hipMemcpyHostToDevice, s));
    bool cost_sent = false;
    auto est = [&](double scale) -> double {
      const ep_status q = quantise(scale, ws.rows_sel, ns, sel);
      if (q != EP_OK) return q == EP_ERR_HIP ? NAN : INFINITY;
      double bits = 0.0;
      uint32_t terr = 0, n[EP_NTABLES];
      if (!ep::estimate_enqueue(ws.hist, ws.rate, !cost_sent, s, &bits, &terr, n)) return NAN;
      cost_sent = true;
      hip(hipMemcpyAsync(&err_host, ws.err, 4, hipMemcpyDeviceToHost, s));
      hip(hipStreamSynchronize(s));
      if (!hip.ok()) return NAN;
      if (err_host || terr) return INFINITY;
      return finish_estimate(bits, n, rows, cols, ns, F, K);
    };
    double lo = -20.0, hi = 12.0;
    const double target = cfg->target_bpp;
    double e_hi = est(std::exp2(hi));
    if (std::isnan(e_hi)) return EP_ERR_HIP;
    if (e_hi > target) {
      sc = std::exp2(hi);
    } else {
      const double e_lo = est(std::exp2(lo));
      if (std::isnan(e_lo)) return EP_ERR_HIP;
      if (e_lo <= target) {
        sc = std::exp2(lo);
      } else {
        for (uint32_t it = 0; it < cfg->search_iters; it++) {
          const double mid = 0.5 * (lo + hi);
          const double e = est(std::exp2(mid));
          if (std::isnan(e)) return EP_ERR_HIP;
          if (e <= target) hi = mid;
          else lo = mid;
        }
        sc = std::exp2(hi);
      }
    }
    // 2a. whole-tensor check of the searched scale (ep_config.rate_check): the same estimate over
    // every row; if it misses the target, raise log2 s by 1/8, 1/4, 1/2, ... (to at most 12)
    // until it meets it, then ten bisection steps keep the meeting end
    if (cfg->rate_check) {
      auto full = [&](double e) -> double {
        const ep_status q = quantise(std::exp2(e), nullptr, rows, {});
        if (q != EP_OK) return q == EP_ERR_HIP ? NAN : INFINITY;
        double bits = 0.0;
        uint32_t terr = 0, n[EP_NTABLES];
        if (!ep::estimate_enqueue(ws.hist, ws.rate, !cost_sent, s, &bits, &terr, n)) return NAN;
        cost_sent = true;
        hip(hipMemcpyAsync(&err_host, ws.err, 4, hipMemcpyDeviceToHost, s));
        hip(hipStreamSynchronize(s));
        if (!hip.ok()) return NAN;
        if (err_host || terr) return INFINITY;
        return finish_estimate(bits, n, rows, cols, rows, F, K);
      };
      double lo = std::log2(sc);
      double e = full(lo);
      if (std::isnan(e)) return EP_ERR_HIP;
      if (e > target) {
        double hi = lo, step = 0.125;
        bool met = false;
        for (;;) {
          hi = lo + step;
          if (hi >= 12.0) {
            hi = 12.0;
            break;
          }
          e = full(hi);
          if (std::isnan(e)) return EP_ERR_HIP;
          if (e <= target) {
            met = true;
            break;
          }
          lo = hi;
          step *= 2.0;
        }
        if (!met) {
          e = full(hi);
          if (std::isnan(e)) return EP_ERR_HIP;
          met = e <= target;
        }
        if (met) {
          for (int it = 0; it < 10; it++) {
            const double mid = 0.5 * (lo + hi);
            e = full(mid);
            if (std::isnan(e)) return EP_ERR_HIP;
            if (e <= target) hi = mid;
            else lo = mid;
          }
        }
        sc = std::exp2(hi);
      }
    }
  }
  if (scale_out) *scale_out = sc;

  // 2b. optional per-row rate-distortion refinement: the per-row gains of the chosen resolutions
  std::vector<float> final_gains(rows);
  for (int64_t r = 0; r < rows; r++) final_gains[r] = row_gain(sumsq[r], cols, sc);
  if (nc > 0) {
    const int c = (nc - 1) / 2;
    const int64_t V = F / 8, tiles = (nv + V - 1) / V;
    std::vector<float> gk((size_t)rows * nc), gcol(rows);
    for (int k = 0; k < nc; k++) {
      const double sk = sc * std::exp2((double)(k - c) / 4.0);
      for (int64_t r = 0; r < rows; r++) gk[(size_t)r * nc + k] = row_gain(sumsq[r], cols, sk);
    }
    std::vector<uint32_t> cost(kM + 1);
    ep_rate_costs(cost.data());
    hip(hipMemcpyAsync(ws.cost, cost.data(), 4 * (size_t)(kM + 1), hipMemcpyHostToDevice, s));
    // distortions of every candidate (model-free): the rows' LS residuals
    std::vector<double> D((size_t)rows * nc), num(rows);
    std::vector<int64_t> Rq((size_t)rows * nc, 0), den4(rows), rate(rows);
    std::vector<int> offered(nc);
    for (int k = 0; k < nc; k++) {
      for (int64_t r = 0; r < rows; r++) gcol[r] = gk[(size_t)r * nc + k];
      if ((st = quantise_with(gcol.data(), false)) != EP_OK) return st;
      if ((st = ep_row_lsq(d_w, dtype, rows, cols, ws.coset, ws.fields, ws.num, ws.den4,
                           stream)) != EP_OK)
        return st;
      hip(hipMemcpyAsync(num.data(), ws.num, 8 * rows, hipMemcpyDeviceToHost, s));
      hip(hipMemcpyAsync(den4.data(), ws.den4, 8 * rows, hipMemcpyDeviceToHost, s));
      hip(hipMemcpyAsync(&err_host, ws.err, 4, hipMemcpyDeviceToHost, s));
      hip(hipStreamSynchronize(s));
      if (!hip.ok()) return EP_ERR_HIP;
      offered[k] = err_host == 0;
      if (!offered[k] && k == c) return (err_host & (1u << EP_ERR_RANGE)) ? EP_ERR_RANGE : EP_ERR_ARG;
      for (int64_t r = 0; r < rows; r++) {
        double d = INFINITY;
        if (offered[k]) {
          d = sumsq[r];
          if (den4[r] != 0) d = sumsq[r] - num[r] * num[r] / ((double)den4[r] / 4.0);
        }
        D[(size_t)r * nc + k] = d;
      }
    }
    std::vector<int32_t> sel(rows, c), next(rows);
    ep_tables* d_T = const_cast<ep_tables*>(ep::estimate_tables(ws.rate));
    for (int round = 0; round < 3; round++) {
      // the model of the current selection
      for (int64_t r = 0; r < rows; r++) gcol[r] = gk[(size_t)r * nc + sel[r]];
      if ((st = quantise_with(gcol.data(), true)) != EP_OK) return st;
      if ((st = ep_build_tables_gpu(ws.hist, d_T, ws.err, stream)) != EP_OK) return st;
      uint32_t n_tab[EP_NTABLES];
      hip(hipMemcpyAsync(n_tab, d_T->n, 4 * EP_NTABLES, hipMemcpyDeviceToHost, s));
      hip(hipMemcpyAsync(&err_host, ws.err, 4, hipMemcpyDeviceToHost, s));
      hip(hipStreamSynchronize(s));
      if (!hip.ok()) return EP_ERR_HIP;
      if (err_host & (1u << EP_ERR_RANGE)) return EP_ERR_RANGE;
      if (err_host & ~(1u << EP_ERR_ALPHABET)) return EP_ERR_ARG;
      if (err_host) break;                            // the model cannot be built: stop here
      const double budget = cfg->target_bpp * (double)rows * (double)cols -
                            8.0 * (double)layout(rows, tiles, K, tables_bytes(n_tab), 0).words;
      const int64_t budget_q = budget > 0.0 ? std::llround(budget * 65536.0) : 0;
      // the rates of every offered candidate under this model
      for (int k = 0; k < nc; k++) {
        if (!offered[k]) continue;
        for (int64_t r = 0; r < rows; r++) gcol[r] = gk[(size_t)r * nc + k];
        if ((st = quantise_with(gcol.data(), false)) != EP_OK) return st;
        if ((st = ep_row_rates(ws.coset, ws.fields, rows, cols, d_T, ws.cost, ws.rates,
                               stream)) != EP_OK)
          return st;
        hip(hipMemcpyAsync(rate.data(), ws.rates, 8 * rows, hipMemcpyDeviceToHost, s));
        hip(hipStreamSynchronize(s));
        if (!hip.ok()) return EP_ERR_HIP;
        for (int64_t r = 0; r < rows; r++) Rq[(size_t)r * nc + k] = rate[r];
      }
      ep_refine_select(D.data(), Rq.data(), rows, nc, budget_q, next.data());
      sel = next;
    }
    for (int64_t r = 0; r < rows; r++) final_gains[r] = gk[(size_t)r * nc + sel[r]];
  }

  // 3. full quantisation + histogram, 4. row least-squares scales, 5. tables (device)
  std::vector<double> num(rows);
  std::vector<int64_t> den4(rows);
  std::vector<ep_tables> tabv(1);
  ep_tables& T = tabv[0];
  bool escapes = false;
  {
    const ep_status q = quantise_with(final_gains.data(), true);
    if (q != EP_OK) return q == EP_ERR_HIP ? EP_ERR_HIP : EP_ERR_ARG;
    if ((st = ep_row_lsq(d_w, dtype, rows, cols, ws.coset, ws.fields, ws.num, ws.den4, stream)) !=
        EP_OK)
      return st;
    ep_tables* d_T = const_cast<ep_tables*>(ep::estimate_tables(ws.rate));
    if ((st = ep_build_tables_gpu(ws.hist, d_T, ws.err, stream)) != EP_OK) return st;
    hip(hipMemcpyAsync(num.data(), ws.num, 8 * rows, hipMemcpyDeviceToHost, s));
    hip(hipMemcpyAsync(den4.data(), ws.den4, 8 * rows, hipMemcpyDeviceToHost, s));
    hip(hipMemcpyAsync(&T, d_T, sizeof(ep_tables), hipMemcpyDeviceToHost, s));
    hip(hipMemcpyAsync(&err_host, ws.err, 4, hipMemcpyDeviceToHost, s));
    hip(hipStreamSynchronize(s));
    if (!hip.ok()) return EP_ERR_HIP;
    if (err_host & (1u << EP_ERR_RANGE)) return EP_ERR_RANGE;
    if (err_host & ~(1u << EP_ERR_ALPHABET)) return EP_ERR_ARG;
    if (err_host) {
      // some field table holds more than M distinct values: build the tables with escapes on
      // the host from the full histogram
      std::vector<ep_hist> hh(1);
      hip(hipMemcpyAsync(hh.data(), ws.hist, sizeof(ep_hist), hipMemcpyDeviceToHost, s));
      hip(hipStreamSynchronize(s));
      if (!hip.ok()) return EP_ERR_HIP;
      if ((st = build_tables_escaped(hh.data(), &T)) != EP_OK) return st;
      escapes = true;
    }
  }
  // the exception list: the vectors with a field their table lacks
  std::vector<uint32_t> x_idx;
  std::vector<uint8_t> x_fields;
  if (escapes &&
      (st = ep::find_exceptions(ws.coset, ws.fields, nv, F, &T, ws.enc, ws.enc_bytes, ws.words,
                                x_idx, x_fields, s)) != EP_OK)
    return st;
  const int64_t n_exc = (int64_t)x_idx.size();
  std::vector<float> alpha(rows);
  for (int64_t r = 0; r < rows; r++)
    alpha[r] = den4[r] == 0 ? 0.0f : (float)(num[r] / ((double)den4[r] / 4.0));

  // 6. tiles (device encoder), 7. blob
  const int64_t V = F / 8, tiles = (nv + V - 1) / V;
  const int64_t tb = tables_bytes(T.n);
  std::vector<uint32_t> word_off(tiles + 1);
  uint8_t* b = static_cast<uint8_t*>(h_blob);
  Layout L;
  int64_t W;
  {
    hip(hipMemcpyAsync(ws.err, &zero, 4, hipMemcpyHostToDevice, s));
    if ((st = ep::encode_tiles_dev(ws.coset, ws.fields, nv, F, K, &T, escapes, ws.enc,
                                   ws.enc_bytes, ws.word_off, ws.max_words, ws.states, ws.words,
                                   9 * nv + 1, ws.err, s)) != EP_OK)
      return st;
    hip(hipMemcpyAsync(word_off.data(), ws.word_off, 4 * (tiles + 1), hipMemcpyDeviceToHost, s));
    hip(hipMemcpyAsync(&err_host, ws.err, 4, hipMemcpyDeviceToHost, s));
    hip(hipStreamSynchronize(s));
    if (!hip.ok()) return EP_ERR_HIP;
    if (err_host) return EP_ERR_ARG;
    W = word_off[tiles];
    L = layout(rows, tiles, K, tb, W, n_exc);
    *out_bytes = (size_t)L.total;
    if ((size_t)L.total > cap) return EP_ERR_CAPACITY;
    // zero what the copies below do not write: every section before the states (their padding
    // included) and the words section's tail padding; the states fill their section exactly
    std::memset(b, 0, (size_t)L.states);
    std::memset(b + L.words + 2 * W, 0, (size_t)(L.total - L.words - 2 * W));
    hip(hipMemcpyAsync(b + L.states, ws.states, 4 * (size_t)K * tiles, hipMemcpyDeviceToHost, s));
    hip(hipMemcpyAsync(b + L.words, ws.words, 2 * W, hipMemcpyDeviceToHost, s));
    hip(hipStreamSynchronize(s));
    if (!hip.ok()) return EP_ERR_HIP;
  }

  std::memcpy(b, "EPK1", 4);
  b[4] = 1;                                           // version 1.0, or 1.1 with escapes
  b[5] = n_exc > 0 ? 1 : 0;
  b[6] = (uint8_t)dtype;
  b[7] = EP_PRECISION;
  const uint64_t r64 = (uint64_t)rows, c64 = (uint64_t)cols, w64 = (uint64_t)W;
  const uint32_t f32 = F, k32 = K, t32 = (uint32_t)tiles, tb32 = (uint32_t)tb;
  uint32_t maxw = 0;
  for (int64_t t = 0; t < tiles; t++) maxw = std::max(maxw, word_off[t + 1] - word_off[t]);
  std::memcpy(b + 8, &r64, 8);
  std::memcpy(b + 16, &c64, 8);
  std::memcpy(b + 24, &f32, 4);
  std::memcpy(b + 28, &k32, 4);
  std::memcpy(b + 32, &t32, 4);
  std::memcpy(b + 36, &tb32, 4);
  std::memcpy(b + 40, &sc, 8);
  std::memcpy(b + 48, &w64, 8);
  std::memcpy(b + 56, &maxw, 4);
  const uint32_t x32 = (uint32_t)n_exc;
  std::memcpy(b + 60, &x32, 4);
  if (n_exc > 0) {
    std::memcpy(b + L.exc_idx, x_idx.data(), 4 * (size_t)n_exc);
    std::memcpy(b + L.exc_fields, x_fields.data(), 16 * (size_t)n_exc);
  }
  int64_t p = L.tables;
  for (int t = 0; t < EP_NTABLES; t++) {
    std::memcpy(b + p, &T.lo[t], 4);
    std::memcpy(b + p + 4, &T.n[t], 4);
    std::memcpy(b + p + 8, T.freq + (size_t)t * EP_HIST_BINS, 2 * (size_t)T.n[t]);
    p += record_bytes(T.n[t]);
  }
  std::memcpy(b + L.alpha, alpha.data(), 4 * rows);
  std::memcpy(b + L.word_off, word_off.data(), 4 * (tiles + 1));
  return EP_OK;
}
