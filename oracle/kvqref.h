/*
 * kvqref.h -- CPU oracle for low-bit KV-cache encode and decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load or call this code; the product
 * path (the HIP library) never does, and shares no source with it.
 *
 * What is computed follows the pages:
 *   PatternKV (arXiv 2510.05176v2): Eq 1 (asymmetric min-max quantizer),
 *   section 3.2 / Eq 6 (min-max distance, nearest pattern, residual, stored
 *   index), section 3.3 / Eq 7-10 (V threshold), section 3.1 Eq 4 (k-means
 *   pattern mining), Eq 5 (Chebyshev-centre pattern per G_pattern window).
 *   KVarN (arXiv 2606.03458, abstract): Hadamard rotation followed by a
 *   variance normalisation over both axes of the K and V matrices; NSNQuant
 *   (arXiv 2505.18231, abstract): token-wise normalisation with a Hadamard
 *   transform.
 * Where the pages are silent, the oracle takes the readings listed in
 * kvqref.c's header comment.
 *
 * Every floating-point step of the encode is an IEEE binary32 operation with
 * round-to-nearest-even (built with -ffp-contract=off, no fast-math), so that
 * codes, scales and indices are a deterministic function of the input.
 * Attention is evaluated in binary64.
 */
#ifndef KVQREF_H
#define KVQREF_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { KVQREF_PATTERN = 0, KVQREF_KVARN = 1, KVQREF_NSN = 2 };
enum { KVQREF_IN_F32 = 0, KVQREF_IN_BF16 = 1 };
enum { KVQREF_NONE = 0xFF };      /* stored pattern index meaning "raw" */
enum { KVQREF_KBLOCK = 128 };     /* tokens per K block with k_per_channel */

typedef struct {
  int32_t batch, n_q_heads, n_kv_heads, head_dim, max_tokens;
  int32_t bits, group, mode, max_patterns, pattern_window;
  double v_alpha;                 /* <= 0: V threshold disabled */
  int32_t in_dtype;
  int32_t shared_patterns;        /* PATTERN: 1 = one table and window per kv-head for the batch */
  int32_t k_per_channel;          /* PATTERN: 1 = K quantised per channel over 128-token blocks,
                                     the open block's residuals held in binary16 (R17) */
} kvqref_cfg;

typedef struct kvqref_cache kvqref_cache;

kvqref_cache* kvqref_new(const kvqref_cfg* cfg);
void kvqref_free(kvqref_cache* c);

/* Explicit pattern tables [B][Hkv][n][D] (PATTERN; [Hkv][n][D] with
 * shared_patterns), channel scales [B][Hkv][D] (KVARN, n ignored) or channel
 * centres [B][Hkv][D] (NSN, n ignored).  fp32 host arrays. */
int kvqref_set_patterns(kvqref_cache* c, const float* k_tab, const float* v_tab, int32_t n);

/* Prefill mining: per-unit k-means (PATTERN; per kv-head over the B
 * prefixes pooled batch-major with shared_patterns) or channel scales (KVARN)
 * over [B][Hkv][n_tok][D] inputs of the configured dtype. */
int kvqref_init_patterns(kvqref_cache* c, const void* k, const void* v, int32_t n_tok,
                         int32_t n_patterns);

/* Encode and append n_new tokens per unit; update != 0 marks decode appends
 * that feed the Chebyshev window. */
int kvqref_encode_append(kvqref_cache* c, const void* k, const void* v, int32_t n_new,
                         int32_t update);

/* fp32 reconstruction [B][Hkv][n][D] of tokens tok0..tok0+n-1. */
int kvqref_dequant(const kvqref_cache* c, int32_t which, int32_t tok0, int32_t n, float* out);

/* Single-query attention: q [B][Hq][D] (configured dtype), out fp32 [B][Hq][D]. */
int kvqref_attn_decode(const kvqref_cache* c, const void* q, float* out, double sm_scale);

/* Same attention over explicit fp32 K/V [B][Hkv][T][D] (no quantizer). */
int kvqref_attn_exact(const kvqref_cfg* cfg, const float* k, const float* v, int32_t T,
                      const float* q, float* out, double sm_scale);

/* State accessors.  which: 0 = K, 1 = V. */
int32_t kvqref_n_tokens(const kvqref_cache* c);
int32_t kvqref_n_patterns(const kvqref_cache* c);
int32_t kvqref_dropped(const kvqref_cache* c);
int32_t kvqref_win_count(const kvqref_cache* c);
/* Region pointers and their byte sizes (for whole-cache comparison). */
const void* kvqref_region(const kvqref_cache* c, const char* name, int64_t* bytes);

/* Scalar helpers exposed for pinning. */
double kvqref_norm_ppf(double p);
double kvqref_rho_star(int32_t d, double alpha);
float kvqref_rho_star_f32(int32_t d, double alpha);
uint16_t kvqref_f16_round(float x, int32_t mode);  /* -1 down, 0 nearest-even, +1 up */
float kvqref_f16_to_f32(uint16_t h);
void kvqref_fwht_f32(float* x, int32_t n);        /* unnormalised, in place */
/* Quantise one group of g residuals; returns codes, s16, z16, tie flags. */
void kvqref_quant_group(const float* r, int32_t g, int32_t bits, uint8_t* codes,
                        uint16_t* s16, uint16_t* z16, uint8_t* ties);
/* Nearest pattern under the min-max distance; returns index (NONE if n == 0)
 * and its distance in *e. */
int32_t kvqref_nearest(const float* x, const float* pats, int32_t n, int32_t d, float* e);
/* k-means on one unit's rows x [n][d]; centroids out [k][d]; returns iterations. */
int32_t kvqref_kmeans(const float* x, int32_t n, int32_t d, int32_t k, float* cent,
                      int32_t* assign_out);

#ifdef __cplusplus
}
#endif
#endif
