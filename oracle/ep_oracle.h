/*
 * CPU ORACLE for the lattice-rANS weight codec -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded C implementation of what the EntroPack design page
 * ("EntroPack lattice compression", sections "Lattice quantization and integer fields",
 * "Rate selection and refinement", "Encoding and reconstruction") describes, written step by
 * step in the page's order.  It shares no code with the HIP library and must never be linked
 * into it: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may load it.
 *
 * Every floating-point step runs in a pinned order with no FMA contraction (built with
 * -ffp-contract=off), so its results are reproducible bit for bit.
 *
 * Pins (see tests/test_oracle_*.py): converters vs torch/numpy casts; E8 quantiser vs brute force
 * and the 240-root certificate and the E8 second moment; field map bijection; table-rule worked
 * examples; rANS round trip and size bounds; LS scale closed forms; blob size closed form.
 * The rate search: the estimate (every row sampled) against the information an actual encode
 * stores (words plus each final state's excess over 2^16), the search against the bracket a
 * bisection on a monotone estimate must leave.
 * Escapes: the kept set against a brute-force ranking; a blob with escapes decodes to the
 * direct reconstruction of the quantised vectors (the coding is lossless whatever it escapes).
 */
#ifndef EP_ORACLE_H
#define EP_ORACLE_H
#include <stddef.h>
#include <stdint.h>

enum {
  OR_OK = 0, OR_ERR_ARG = 1, OR_ERR_SHAPE = 2, OR_ERR_DTYPE = 3, OR_ERR_NONFINITE = 4,
  OR_ERR_RANGE = 5, OR_ERR_ALPHABET = 6, OR_ERR_CORRUPT = 7, OR_ERR_VERSION = 8,
  OR_ERR_CAPACITY = 10
};
enum { OR_BF16 = 1, OR_FP16 = 2, OR_FP8 = 3, OR_INT8 = 4, OR_FP32 = 5 };

#define OR_NTABLES 17
#define OR_NBINS 65536 /* histogram bins per table: value + 32768 */

/* container <-> fp32 */
float or_widen(int dt, uint32_t bits);
uint32_t or_narrow(int dt, float y);
void or_widen_array(int dt, const void* src, int64_t n, float* dst);
void or_narrow_array(int dt, const float* src, int64_t n, void* dst);

/* row statistics */
void or_row_sumsq(int dt, const void* w, int64_t rows, int64_t cols, double* out);
float or_gain(double sumsq, int64_t cols, double s);

/* E8 */
int or_e8_nearest(const float x[8], int32_t z[8]);
int or_e8_brute(const float x[8], int32_t z[8], long double* dist);
long double or_e8_dist_exact(const float x[8], int coset, const int32_t z[8]);
int64_t or_e8_certificate(const float* x, int64_t nv, double rel_tol, int64_t* n_checked);
int64_t or_e8_vs_brute(const float* x, int64_t nv, double rel_tol);
double or_e8_mse(const float* x, int64_t nv);
void or_fields_from_point(int coset, const int32_t z[8], int32_t f[8]);
void or_point_from_fields(const int32_t f[8], int32_t z[8]);
int64_t or_field_bijection_box(int radius);

int or_quantize(int dt, const void* w, int64_t rows, int64_t cols, const float* gains,
                const int64_t* row_sel, int64_t n_sel, uint8_t* coset, int16_t* fields);

/* model */
void or_histogram(const uint8_t* coset, const int16_t* fields, int64_t nv, uint64_t* counts);
int or_normalize(const uint64_t* counts, int32_t n, int precision, uint16_t* freq);
int or_build_tables(const uint64_t* counts, int precision, int32_t* lo, uint32_t* n,
                    uint16_t* freq /* [17][65536] */);
/* escapes != 0: a field table with more than 2^P distinct values keeps the 2^P most frequent */
int or_build_tables_ex(const uint64_t* counts, int precision, int escapes, int32_t* lo,
                       uint32_t* n, uint16_t* freq);
void or_escape_keep(const uint64_t* counts /* one table */, int precision, uint8_t* kept);
int32_t or_substitute(int32_t lo, uint32_t n, const uint16_t* freq /* one table */);
int64_t or_exceptions(const uint8_t* coset, const int16_t* fields, int64_t nv, const int32_t* lo,
                      const uint32_t* n, const uint16_t* freq, uint32_t* idx, int16_t* xf);

/* row least squares */
void or_row_lsq(int dt, const void* w, int64_t rows, int64_t cols, const uint8_t* coset,
                const int16_t* fields, double* num, int64_t* den4);
float or_alpha(double num, int64_t den4);

/* rANS tiles */
int or_encode_tiles(const uint8_t* coset, const int16_t* fields, int64_t nv, int tile_fields,
                    int lanes, int precision, const int32_t* lo, const uint32_t* n,
                    const uint16_t* freq, uint32_t* word_off, uint32_t* states, uint16_t* words,
                    int64_t words_cap);
int or_encode_tiles_ex(const uint8_t* coset, const int16_t* fields, int64_t nv, int tile_fields,
                       int lanes, int precision, const int32_t* lo, const uint32_t* n,
                       const uint16_t* freq, int substitute, uint32_t* word_off, uint32_t* states,
                       uint16_t* words, int64_t words_cap);
int or_decode_tiles(const uint32_t* word_off, const uint32_t* states, const uint16_t* words,
                    int64_t nv, int tile_fields, int lanes, int precision, const int32_t* lo,
                    const uint32_t* n, const uint16_t* freq, int64_t t0, int64_t t1,
                    uint8_t* coset, int16_t* fields);

/* blob */
/* Compression settings (the page's LatticeRANSConfig: target rate, search and refinement
 * settings).  lanes: rANS states per tile, 64 or 128; sample_rows: rows of the rate search's
 * sample; search_iters: bisection steps on log2 s; refine: 0 or the odd number (<= 9) of
 * candidate resolutions per row; force_scale > 0 skips the search; rate_check: 1 (default)
 * checks the searched scale against the whole tensor's estimate (or_check_scale). */
typedef struct {
  double target_bpp;
  int tile_fields, lanes, sample_rows, search_iters, refine;
  double force_scale;
  int rate_check;
} or_config;
void or_config_default(or_config* cfg);
int or_compress_cfg(int dt, const void* w, int64_t rows, int64_t cols, const or_config* cfg,
                    uint8_t* blob, int64_t cap, int64_t* out_bytes, double* s_out);
int or_compress(int dt, const void* w, int64_t rows, int64_t cols, double target_bpp,
                int tile_fields, double force_s, int refine, uint8_t* blob, int64_t cap,
                int64_t* out_bytes, double* s_out);
int or_compress_bound(int64_t rows, int64_t cols, int tile_fields, int64_t* bytes);
int or_decompress(const uint8_t* blob, int64_t bytes, int64_t t0, int64_t t1, void* out,
                  uint8_t* coset_out, int16_t* fields_out);
int or_blob_fields(const uint8_t* blob, int64_t bytes, int64_t* rows, int64_t* cols, int* dt,
                   int* tile_fields, int64_t* tiles, double* s, int64_t* payload_words,
                   int64_t* table_bytes);
int or_blob_exceptions(const uint8_t* blob, int64_t bytes, int64_t* n_exc);
double or_estimate_bpp(int dt, const void* w, int64_t rows, int64_t cols, const double* sumsq,
                       int tile_fields, double s);
double or_search_scale(int dt, const void* w, int64_t rows, int64_t cols, const double* sumsq,
                       int tile_fields, double target_bpp);
double or_check_scale(int dt, const void* w, int64_t rows, int64_t cols, const double* sumsq,
                      int tile_fields, int lanes, double target_bpp, double s0);
double or_estimate_bpp_ex(int dt, const void* w, int64_t rows, int64_t cols, const double* sumsq,
                          int tile_fields, int lanes, int sample_rows, double s);
double or_search_scale_ex(int dt, const void* w, int64_t rows, int64_t cols, const double* sumsq,
                          int tile_fields, int lanes, int sample_rows, int search_iters,
                          double target_bpp);

/* per-row rate-distortion refinement (refine = number of candidate resolutions, odd, <= 9) */
void or_rate_costs(uint32_t* cost /* [2^P + 1]: [0] = a value absent from the model */);
void or_row_rates(const uint8_t* cs, const int16_t* fs, int64_t rows, int64_t cols,
                  const int32_t* lo, const uint32_t* n, const uint16_t* freq,
                  const uint32_t* cost, int64_t* rate);
double or_refine_select(const double* D, const int64_t* Rq, int64_t rows, int nc,
                        int64_t budget_q, int32_t* sel);

#endif
