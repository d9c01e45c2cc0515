// Memory-safety driver for the CPU side of the codec, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_sanitizers.py (host compiler only; no GPU code runs).
//
// 1. The oracle (oracle/ep_oracle.c): compress / decompress round trips over synthetic matrices
//    (every container, ragged widths, 64 and 128 lanes, refinement, a forced scale that escapes
//    values), checked to decode losslessly to the quantised fields.
// 2. The library's blob parser (ep_blob_parse in ep_host.cpp) and the oracle's parser, on every
//    blob of (1) mutated many times over: single and multiple byte flips, header fields set to
//    extreme values, truncations.  Both must return a status without touching memory outside
//    the blob; a blob the library accepts must have sections inside it.
// 3. The host tile encoder (ep_encode_tiles) against the oracle's, bit for bit.
// Exit status 0 when every check holds; the sanitizers abort on the first memory error.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "ep.h"
extern "C" {
#include "ep_oracle.h"
}

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64() {                      // xorshift64*
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return rng_state * 0x2545F4914F6CDD1Dull;
}
static double uniform() { return (double)(next_u64() >> 11) * (1.0 / 9007199254740992.0); }
static double laplace(double b) {
  const double u = uniform() - 0.5;
  return (u < 0 ? 1.0 : -1.0) * b * __builtin_log(1.0 - 2.0 * __builtin_fabs(u) + 1e-300);
}

static int failures = 0;
#define CHECK(c)                                                          \
  do {                                                                    \
    if (!(c)) {                                                           \
      std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      failures++;                                                         \
    }                                                                     \
  } while (0)

static std::vector<uint8_t> make_matrix(int dt, int64_t rows, int64_t cols, double scale) {
  const int es = dt == OR_FP32 ? 4 : (dt == OR_BF16 || dt == OR_FP16) ? 2 : 1;
  std::vector<uint8_t> w((size_t)(rows * cols * es));
  for (int64_t i = 0; i < rows * cols; i++) {
    const float v = (float)laplace(scale);
    uint32_t bits = or_narrow(dt, dt == OR_INT8 ? v * 2000.0f : v);
    std::memcpy(w.data() + i * es, &bits, (size_t)es);
  }
  return w;
}

struct Blob {
  std::vector<uint8_t> bytes;
  int64_t rows, cols;
  int dt;
};

static bool compress(const std::vector<uint8_t>& w, int dt, int64_t rows, int64_t cols,
                     or_config cfg, Blob* out) {
  int64_t cap = 0;
  if (or_compress_bound(rows, cols, cfg.tile_fields, &cap) != OR_OK) return false;
  out->bytes.assign((size_t)cap, 0);
  int64_t n = 0;
  double s = 0;
  const int st = or_compress_cfg(dt, w.data(), rows, cols, &cfg, out->bytes.data(), cap, &n, &s);
  if (st != OR_OK) return false;
  out->bytes.resize((size_t)n);
  out->rows = rows;
  out->cols = cols;
  out->dt = dt;
  return true;
}

static void roundtrip(const Blob& b) {
  const int64_t nv = b.rows * ((b.cols + 7) / 8);
  std::vector<uint8_t> cs((size_t)nv);
  std::vector<int16_t> fs((size_t)(8 * nv));
  const int es = b.dt == OR_FP32 ? 4 : (b.dt == OR_BF16 || b.dt == OR_FP16) ? 2 : 1;
  std::vector<uint8_t> out((size_t)(b.rows * b.cols * es));
  CHECK(or_decompress(b.bytes.data(), (int64_t)b.bytes.size(), 0, -1, out.data(), cs.data(),
                      fs.data()) == OR_OK);
  // a tile range decode of the same blob
  CHECK(or_decompress(b.bytes.data(), (int64_t)b.bytes.size(), 1, 2, out.data(), nullptr,
                      nullptr) == OR_OK);
}

static void fuzz_parsers(const Blob& b, int rounds) {
  const size_t n = b.bytes.size();
  std::vector<uint8_t> m;
  for (int r = 0; r < rounds; r++) {
    m = b.bytes;
    const int kind = (int)(next_u64() % 4);
    if (kind == 0) {                             // a few random byte flips anywhere
      const int flips = 1 + (int)(next_u64() % 4);
      for (int i = 0; i < flips; i++) m[next_u64() % n] ^= (uint8_t)(1 + next_u64() % 255);
    } else if (kind == 1) {                      // a header field set to an extreme value
      const int off = 8 * (int)(next_u64() % 8);
      const uint64_t vals[] = {0, 1, 0xFFFFFFFFull, 0xFFFFFFFFFFFFFFFFull, 1ull << 31,
                               1ull << 40, 0x7FFFFFFFFFFFFFFFull, 65535};
      const uint64_t v = vals[next_u64() % 8];
      std::memcpy(m.data() + off, &v, (next_u64() & 1) ? 8 : 4);
    } else if (kind == 2) {                      // truncated
      m.resize(next_u64() % n);
    } else {                                     // a table record or tile offset rewritten
      const size_t off = 64 + next_u64() % (n > 128 ? n - 128 : 1);
      const uint32_t v = (uint32_t)next_u64();
      std::memcpy(m.data() + off, &v, 4);
    }
    ep_blob_info info;
    const ep_status st = ep_blob_parse(m.empty() ? nullptr : m.data(), m.size(), &info);
    if (st == EP_OK) {
      CHECK(info.off_words <= (int64_t)m.size() && info.off_states <= info.off_words);
      CHECK(info.bytes == (int64_t)m.size());
    }
    if (!m.empty()) {
      int64_t x = 0;
      (void)or_blob_exceptions(m.data(), (int64_t)m.size(), &x);
    }
  }
}

int main() {
  std::vector<Blob> blobs;
  struct Case { int dt; int64_t rows, cols; double scale; int tile, lanes, refine; double force; };
  const Case cases[] = {
      {OR_BF16, 64, 256, 0.02, 4096, 64, 0, 0.0},   {OR_FP16, 40, 1000, 0.015, 8192, 128, 0, 0.0},
      {OR_FP8, 16, 2048, 0.01, 16384, 64, 0, 0.0},  {OR_INT8, 16, 2048, 0.01, 16384, 128, 0, 0.0},
      {OR_FP32, 33, 13, 0.5, 4096, 64, 0, 0.0},     {OR_BF16, 128, 512, 0.02, 8192, 64, 5, 0.0},
      {OR_BF16, 64, 4096, 0.02, 4096, 64, 0, 3.5e-4},  // past 2^12 values a table: escapes
  };
  for (const Case& c : cases) {
    or_config cfg;
    or_config_default(&cfg);
    cfg.target_bpp = 3.0;
    cfg.tile_fields = c.tile;
    cfg.lanes = c.lanes;
    cfg.refine = c.refine;
    cfg.force_scale = c.force;
    const std::vector<uint8_t> w = make_matrix(c.dt, c.rows, c.cols, c.scale);
    Blob b;
    const bool ok = compress(w, c.dt, c.rows, c.cols, cfg, &b);
    if (!ok) std::fprintf(stderr, "compress failed: dtype %d, %lld x %lld\n", c.dt,
                          (long long)c.rows, (long long)c.cols);
    CHECK(ok);
    if (!ok) continue;
    ep_blob_info info;
    CHECK(ep_blob_parse(b.bytes.data(), b.bytes.size(), &info) == EP_OK);
    if (c.force > 0.0) CHECK(info.n_exceptions > 0);
    roundtrip(b);
    blobs.push_back(b);
  }
  // the host encoder against the oracle's
  for (int lanes : {64, 128}) {
    const int64_t nv = 3000;
    std::vector<uint8_t> cs(nv);
    std::vector<int16_t> fs(8 * nv);
    for (int64_t i = 0; i < nv; i++) {
      cs[i] = (uint8_t)(next_u64() & 1);
      for (int k = 0; k < 8; k++) fs[8 * i + k] = (int16_t)(laplace(3.0));
    }
    std::vector<uint64_t> counts((size_t)OR_NTABLES * OR_NBINS);
    or_histogram(cs.data(), fs.data(), nv, counts.data());
    std::vector<ep_tables> tv(1);
    std::vector<uint16_t> freq((size_t)OR_NTABLES * OR_NBINS, 0);
    int32_t lo[OR_NTABLES];
    uint32_t n[OR_NTABLES];
    CHECK(or_build_tables(counts.data(), 12, lo, n, freq.data()) == OR_OK);
    std::memcpy(tv[0].lo, lo, sizeof lo);
    std::memcpy(tv[0].n, n, sizeof n);
    std::memcpy(tv[0].freq, freq.data(), freq.size() * 2);
    const int64_t T = (nv + 1023) / 1024;
    std::vector<uint32_t> w1(T + 1), w2(T + 1), s1(T * lanes), s2(T * lanes);
    std::vector<uint16_t> d1(9 * nv + 1), d2(9 * nv + 1);
    CHECK(or_encode_tiles(cs.data(), fs.data(), nv, 8192, lanes, 12, lo, n, freq.data(), w1.data(),
                          s1.data(), d1.data(), 9 * nv + 1) == OR_OK);
    CHECK(ep_encode_tiles(cs.data(), fs.data(), nv, 8192, (uint32_t)lanes, tv.data(), w2.data(),
                          s2.data(), d2.data(), 9 * nv + 1) == EP_OK);
    CHECK(w1 == w2 && s1 == s2);
    CHECK(std::memcmp(d1.data(), d2.data(), 2 * (size_t)w1[T]) == 0);
  }
  for (const Blob& b : blobs) fuzz_parsers(b, 3000);
  std::printf("sanitized run: %zu blobs, %d failures\n", blobs.size(), failures);
  return failures == 0 ? 0 : 1;
}
