/*
 * kvqref.c -- plain, slow CPU oracle for low-bit KV-cache encode / decode.
 *
 * TEST INFRASTRUCTURE ONLY: it exists to check the HIP library.  Only the
 * tests, the package smoke check and the benchmark's CPU-baseline leg load it.
 * It shares no source, header, table or constant generator with the library.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC
 * (no FTZ/DAZ; x86-64 SSE arithmetic, so every float op below is one IEEE
 * binary32 operation rounded to nearest-even).
 *
 * Readings taken where the pages leave a step open (each is restated where it
 * is used):
 *  R1  Rounding in Eq 1 is round-half-to-even (rintf).  Exact .5 cases are
 *      recorded in a tie mask.
 *  R2  s and z are stored as binary16: z = fp16 rounded toward -inf of the
 *      group minimum, s = fp16 rounded toward +inf of (max - z)/(2^n - 1);
 *      codes are computed from the stored values, so |r - r^| <= s/2 holds
 *      with the stored s.  Zero results are stored as +0.
 *  R3  s == 0 (constant group) gives all-zero codes and no division.
 *  R4  (X - z)/s is evaluated as (X - z) * fl(1/s), one correctly rounded
 *      division per group.
 *  R5  Quantisation groups are G consecutive channels of each token vector,
 *      for K and V alike.
 *  R6  d_mm and the V threshold use the whole head_dim vector.
 *  R7  argmin ties go to the lowest pattern index.
 *  R8  alpha of the z-test is a parameter (0.05 by default); alpha <= 0 turns
 *      the V threshold off (V always uses its nearest pattern).  K has no
 *      threshold.  A rejected V vector stores index NONE (0xFF) and
 *      quantises the raw vector.
 *  R9  Pattern tables are per (batch, kv-head) unit, at most 255 patterns
 *      (per kv-head with shared_patterns, R16).
 *  R10 The Chebyshev window covers decode appends only; its centre
 *      fl(fl(lo + hi) * 0.5) is appended after the window's last token is
 *      encoded and serves later tokens; when the table is full the centre is
 *      dropped and counted.
 *  R11 KVarN encode: y = FWHT(x) (Sylvester order, stages h = 1, 2, 4, ...)
 *      times fp32(1/sqrt(D)); y~ = y * fl(1/c) with a per-channel scale c;
 *      t = sqrtf(fl(ss * (1/D))) with ss the halving-fold sum of y~^2
 *      (v[i] += v[i + D/2], then D/4, ..., 1); t stored as RNE binary16;
 *      u = y~ * fl(1/t) is quantised with the Eq 1 quantiser.
 *  R12 KVarN channel scale: c_j = sqrt(mean over prefix tokens of
 *      (y_j / rms(y))^2) in binary64, rounded to fp32; 0 is replaced by 1.
 *  R13 k-means (Eq 4): Euclidean Lloyd in binary64; centroid j starts at
 *      prefix row floor(j*T/k); iterate until no assignment changes (at most
 *      50 assignment passes); ties to the lowest index; an empty cluster
 *      keeps its centroid; result rounded to fp32.
 *  R14 Attention: softmax(sm_scale * q.k^) v^ over every cached token, q-head
 *      hq reading kv-head hq / (Hq/Hkv), evaluated in binary64 over the
 *      dequantised cache and rounded to fp32.
 *  R15 Code layout (the pages fix none): K and V codes alike, one record of
 *      D*n/8 bytes per token, tokens in order, channel d at bit n*d of the
 *      record (little-endian).  The GPU library keeps V in another order;
 *      the tests map its bytes to these records before comparing.
 *  R16 Batch-shared tables (shared_patterns, PATTERN mode): the pattern
 *      memory estimate of PatternKV's memory analysis carries no batch factor
 *      (its share of the KV memory falls as 1/B) and one decode pattern per
 *      G_pattern steps gives a 1/(B G_pattern) share, i.e. the table and the
 *      window belong to the kv-head.  k-means then runs per kv-head over the
 *      B prefixes pooled batch-major (row b*n_tok + t), the window's min / max
 *      run over every sequence's decode vectors of the window, and each
 *      closure appends one centre per kv-head; every (batch, kv-head) unit
 *      encodes and reconstructs against its kv-head's table.
 *  R17 K per channel (k_per_channel, PATTERN mode): PatternKV's experiments
 *      (section 4.1 quantization settings, appendix E) quantise K per channel
 *      and V per token as KIVI does, K in groups of 128 tokens with a 128-token
 *      residual that is cleared once its group is quantised.  A K vector
 *      takes its nearest pattern on arrival (Eq 6, current table, no
 *      threshold); its residual x - M_k* is rounded to binary16 (nearest-even)
 *      into the unit's residual buffer at slot t mod 128.  When a block of 128
 *      tokens is complete, each channel's 128 binary16 residuals (as binary32)
 *      go through the Eq 1 quantiser (R1-R4 along the token axis): one (s, z)
 *      per (block, channel), codes in the K layout of R15.  Tokens of the open
 *      block reconstruct as f32(residual) + M_k*.  Bulk and token-by-token
 *      appends are the same computation.  V, the Chebyshev window and the
 *      pattern tables are unchanged.
 *  R18 NSN scalar mode (NSNQuant, abstract: token-wise normalisation,
 *      channel-wise centring, token-wise normalisation, with a Hadamard
 *      transform; its vector-quantisation codebook is out of scope, so the
 *      normalised vector goes through the Eq 1 quantiser, at 1, 2 or 4 bits):
 *      n1 = sqrtf(fl(ss(x) * (1/D))) with ss the halving-fold sum of squares
 *      (as R11), stored as RNE binary16; a = x * fl(1/n1); b = a - mu with mu
 *      the unit's channel centre; n2 likewise from b, stored as RNE binary16;
 *      y = FWHT(b * fl(1/n2)) * fp32(1/sqrt(D)); Eq 1 on y.  A zero n1 or n2
 *      gives zero codes and scales from that point.  Reconstruction:
 *      w = FWHT(fmaf(q, s, z)) * fp32(1/sqrt(D)), x^ = fl(fl(fl(w * n2) + mu) * n1).
 *      mu = mean over the prefix tokens of x / rms(x) in binary64 (tokens with
 *      rms 0 skipped), rounded to fp32; 0 before any init.
 *
 * Pins of R12 and R13 (no printed numbers exist for them): the channel
 * scale equals a closed form on prefixes built in the rotated space (each
 * row a token magnitude times a channel profile times random signs), which
 * fixes the transform's order, the per-token normalisation and the RMS; the
 * k-means empty-cluster rule is fixed by a hand-traced Lloyd run in which a
 * strided start leaves a cluster empty.  The other readings are pinned by
 * the test suite against independent computations, closed forms and
 * hand-derived bytes.
 */
#include "kvqref.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#define MAX_D 1024
#define KM_MAX_ITERS 50

struct kvqref_cache {
  kvqref_cfg cfg;
  int32_t D, U, PU, NG, tcap, kbytes;   /* PU: pattern-table units */
  int32_t n_tokens, n_patterns, win_count, dropped;
  int32_t thr_on;
  float rho;
  uint8_t* codes[2];
  uint16_t* sz[2];
  uint8_t* idx[2];
  uint16_t* t16[2];   /* KVARN: token scale t; NSN: first norm n1 */
  uint16_t* t2[2];    /* NSN: second norm n2 */
  uint8_t* tie[2];
  float* pat[2];
  float* wlo[2];
  float* whi[2];
  float* cscale[2];
  int32_t nblk;       /* K blocks per unit (k_per_channel) */
  uint16_t* kbsz;     /* [U][nblk][D][s, z] binary16 */
  uint16_t* ktail;    /* [U][KBLOCK][D] binary16 residuals of the open block */
};

/* ------------------------------------------------------------ binary16 */

/* Round a binary32 value to binary16 by the definition of the three rounding
 * directions: scale by the binary16 spacing at x (exact in binary64), take
 * floor / ceil / nearest-even of the quotient, scale back. */
uint16_t kvqref_f16_round(float xf, int32_t mode) {
  double x = (double)xf;
  if (isnan(x)) return 0x7E00;
  uint16_t sgn = signbit(x) ? 0x8000 : 0;
  if (isinf(x)) return sgn | 0x7C00;
  double ax = fabs(x), ulp;
  if (ax < 0x1p-14) {
    ulp = 0x1p-24;
  } else {
    int e;
    frexp(ax, &e);            /* ax = f * 2^e, f in [0.5, 1) */
    ulp = ldexp(1.0, (e - 1) - 10);
  }
  double q = x / ulp, rq;
  if (mode < 0) rq = floor(q);
  else if (mode > 0) rq = ceil(q);
  else rq = rint(q);          /* default rounding mode: half to even */
  double v = rq * ulp;
  if (v > 65504.0) return mode < 0 ? 0x7BFF : 0x7C00;
  if (v < -65504.0) return mode > 0 ? 0xFBFF : 0xFC00;
  uint16_t s = signbit(v) ? 0x8000 : 0;
  double av = fabs(v);
  if (av == 0.0) return s;
  if (av < 0x1p-14) return s | (uint16_t)(av / 0x1p-24);
  int e;
  frexp(av, &e);
  int E = e - 1;
  uint16_t mant = (uint16_t)((av / ldexp(1.0, E) - 1.0) * 1024.0);
  return s | (uint16_t)((E + 15) << 10) | mant;
}

float kvqref_f16_to_f32(uint16_t h) {
  int sgn = h >> 15, E = (h >> 10) & 0x1F, m = h & 0x3FF;
  double v;
  if (E == 0) v = ldexp((double)m, -24);
  else if (E == 31) v = m ? NAN : INFINITY;
  else v = ldexp(1.0 + m / 1024.0, E - 15);
  return (float)(sgn ? -v : v);
}

static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* ------------------------------------------------------------ Eq 7-10 */

/* Inverse of the standard normal CDF by bisection on 0.5*erfc(-x/sqrt 2). */
double kvqref_norm_ppf(double p) {
  if (!(p > 0.0 && p < 1.0)) return NAN;
  double lo = -40.0, hi = 40.0;
  for (int i = 0; i < 400; ++i) {
    double mid = 0.5 * (lo + hi);
    if (mid == lo || mid == hi) break;
    double cdf = 0.5 * erfc(-mid / sqrt(2.0));
    if (cdf < p) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

/* rho_*(d, alpha): the root in (0, 1) of 1 - rho^2 = c sqrt(1 + rho^4),
 * c = 2 z_{1-alpha} / sqrt(5 d)  (Eq 10).  Squaring gives
 * a u^2 - 2u + a = 0 with u = rho^2, a = 1 - c^2; the smaller root is
 * u = a / (1 + sqrt(1 - a^2)). */
double kvqref_rho_star(int32_t d, double alpha) {
  if (!(alpha > 0.0 && alpha < 0.5) || d <= 0) return NAN;
  double z = kvqref_norm_ppf(1.0 - alpha);
  double c = 2.0 * z / sqrt(5.0 * d);
  double a = 1.0 - c * c;
  if (a <= 0.0) return 0.0;
  double u = a / (1.0 + sqrt(1.0 - a * a));
  return sqrt(u);
}

float kvqref_rho_star_f32(int32_t d, double alpha) { return (float)kvqref_rho_star(d, alpha); }

/* ------------------------------------------------------------ Eq 1 */

void kvqref_quant_group(const float* r, int32_t g, int32_t bits, uint8_t* codes,
                        uint16_t* s16, uint16_t* z16, uint8_t* ties) {
  float lo = r[0], hi = r[0];
  for (int i = 1; i < g; ++i) {
    if (r[i] < lo) lo = r[i];
    if (r[i] > hi) hi = r[i];
  }
  uint16_t zb = kvqref_f16_round(lo, -1);
  if ((zb & 0x7FFF) == 0) zb = 0;
  float zf = kvqref_f16_to_f32(zb);
  float qmax = (float)((1 << bits) - 1);
  float s32 = (hi - zf) / qmax;
  uint16_t sb = kvqref_f16_round(s32, +1);
  if ((sb & 0x7FFF) == 0) sb = 0;
  float sf = kvqref_f16_to_f32(sb);
  if (sf == 0.0f) {
    for (int i = 0; i < g; ++i) { codes[i] = 0; if (ties) ties[i] = 0; }
  } else {
    float inv = 1.0f / sf;
    for (int i = 0; i < g; ++i) {
      float v = (r[i] - zf) * inv;
      if (ties) ties[i] = (v - floorf(v) == 0.5f);
      float q = rintf(v);
      if (q < 0.0f) q = 0.0f;
      if (q > qmax) q = qmax;
      codes[i] = (uint8_t)q;
    }
  }
  *s16 = sb;
  *z16 = zb;
}

/* ------------------------------------------------------------ Eq 6 */

int32_t kvqref_nearest(const float* x, const float* pats, int32_t n, int32_t d, float* e_out) {
  int32_t best = KVQREF_NONE;
  float be = 0.0f;
  for (int32_t j = 0; j < n; ++j) {
    const float* m = pats + (int64_t)j * d;
    float mx = -INFINITY, mn = INFINITY;
    for (int32_t i = 0; i < d; ++i) {
      float diff = x[i] - m[i];
      if (diff > mx) mx = diff;
      if (diff < mn) mn = diff;
    }
    float e = mx - mn;
    if (best == KVQREF_NONE || e < be) { be = e; best = j; }
  }
  if (e_out) *e_out = be;
  return best;
}

/* ------------------------------------------------------------ Hadamard */

void kvqref_fwht_f32(float* x, int32_t n) {
  for (int32_t h = 1; h < n; h <<= 1)
    for (int32_t i = 0; i < n; i += 2 * h)
      for (int32_t j = i; j < i + h; ++j) {
        float a = x[j], b = x[j + h];
        x[j] = a + b;
        x[j + h] = a - b;
      }
}

static void fwht_f64(double* x, int32_t n) {
  for (int32_t h = 1; h < n; h <<= 1)
    for (int32_t i = 0; i < n; i += 2 * h)
      for (int32_t j = i; j < i + h; ++j) {
        double a = x[j], b = x[j + h];
        x[j] = a + b;
        x[j + h] = a - b;
      }
}

/* ------------------------------------------------------------ Eq 4 */

int32_t kvqref_kmeans(const float* x, int32_t n, int32_t d, int32_t k, float* cent,
                      int32_t* assign_out) {
  double* c = (double*)malloc(sizeof(double) * (size_t)k * d);
  double* sums = (double*)malloc(sizeof(double) * (size_t)k * d);
  int64_t* cnt = (int64_t*)malloc(sizeof(int64_t) * (size_t)k);
  int32_t* a = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
  int32_t* prev = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
  for (int32_t j = 0; j < k; ++j) {
    int64_t row = (int64_t)j * n / k;
    for (int32_t i = 0; i < d; ++i) c[(int64_t)j * d + i] = (double)x[row * d + i];
  }
  int have_prev = 0, it;
  for (it = 0; it < KM_MAX_ITERS; ++it) {
    for (int32_t t = 0; t < n; ++t) {
      int32_t best = 0;
      double bd = INFINITY;
      for (int32_t j = 0; j < k; ++j) {
        double dist = 0.0;
        for (int32_t i = 0; i < d; ++i) {
          double diff = (double)x[(int64_t)t * d + i] - c[(int64_t)j * d + i];
          dist += diff * diff;
        }
        if (dist < bd) { bd = dist; best = j; }
      }
      a[t] = best;
    }
    if (have_prev && memcmp(a, prev, sizeof(int32_t) * (size_t)n) == 0) break;
    memset(sums, 0, sizeof(double) * (size_t)k * d);
    memset(cnt, 0, sizeof(int64_t) * (size_t)k);
    for (int32_t t = 0; t < n; ++t) {
      cnt[a[t]]++;
      for (int32_t i = 0; i < d; ++i) sums[(int64_t)a[t] * d + i] += (double)x[(int64_t)t * d + i];
    }
    for (int32_t j = 0; j < k; ++j)
      if (cnt[j] > 0)
        for (int32_t i = 0; i < d; ++i) c[(int64_t)j * d + i] = sums[(int64_t)j * d + i] / (double)cnt[j];
    memcpy(prev, a, sizeof(int32_t) * (size_t)n);
    have_prev = 1;
  }
  for (int64_t i = 0; i < (int64_t)k * d; ++i) cent[i] = (float)c[i];
  if (assign_out) memcpy(assign_out, a, sizeof(int32_t) * (size_t)n);
  free(c); free(sums); free(cnt); free(a); free(prev);
  return it < KM_MAX_ITERS ? it + 1 : KM_MAX_ITERS;
}

/* ------------------------------------------------------------ cache */

static int valid_cfg(const kvqref_cfg* g) {
  if (!g) return 0;
  if (g->batch <= 0 || g->n_kv_heads <= 0 || g->n_q_heads <= 0) return 0;
  if (g->n_q_heads % g->n_kv_heads) return 0;
  if (g->head_dim <= 0 || g->head_dim > MAX_D || g->max_tokens <= 0) return 0;
  if (g->bits != 2 && g->bits != 4 && !(g->bits == 1 && g->mode == KVQREF_NSN)) return 0;
  if (g->group <= 0 || g->head_dim % g->group) return 0;
  if ((g->group * g->bits) % 8) return 0;
  if (g->mode != KVQREF_PATTERN && g->mode != KVQREF_KVARN && g->mode != KVQREF_NSN) return 0;
  if (g->mode != KVQREF_PATTERN && (g->head_dim & (g->head_dim - 1))) return 0;
  if (g->max_patterns < 0 || g->max_patterns > 255) return 0;
  if (g->pattern_window < 0) return 0;
  if (g->in_dtype != KVQREF_IN_F32 && g->in_dtype != KVQREF_IN_BF16) return 0;
  if (g->v_alpha >= 0.5) return 0;
  if (g->shared_patterns != 0 && g->shared_patterns != 1) return 0;
  if (g->shared_patterns && g->mode != KVQREF_PATTERN) return 0;
  if (g->k_per_channel != 0 && g->k_per_channel != 1) return 0;
  if (g->k_per_channel && g->mode != KVQREF_PATTERN) return 0;
  return 1;
}

/* pattern-table (and window) unit of (batch, kv-head) unit u */
static int64_t pu_of(const kvqref_cache* c, int64_t u) {
  return c->cfg.shared_patterns ? u % c->cfg.n_kv_heads : u;
}

static void reset_window(kvqref_cache* c) {
  for (int k = 0; k < 2; ++k)
    for (int64_t i = 0; i < (int64_t)c->PU * c->D; ++i) {
      c->wlo[k][i] = INFINITY;
      c->whi[k][i] = -INFINITY;
    }
  c->win_count = 0;
}

kvqref_cache* kvqref_new(const kvqref_cfg* cfg) {
  if (!valid_cfg(cfg)) return NULL;
  kvqref_cache* c = (kvqref_cache*)calloc(1, sizeof(kvqref_cache));
  c->cfg = *cfg;
  c->D = cfg->head_dim;
  c->U = cfg->batch * cfg->n_kv_heads;
  c->PU = cfg->shared_patterns ? cfg->n_kv_heads : c->U;
  c->NG = cfg->head_dim / cfg->group;
  c->tcap = cfg->max_tokens;
  c->kbytes = c->D * cfg->bits / 8;
  c->thr_on = cfg->v_alpha > 0.0;
  c->rho = c->thr_on ? kvqref_rho_star_f32(c->D, cfg->v_alpha) : 0.0f;
  int64_t U = c->U, T = c->tcap, D = c->D;
  for (int k = 0; k < 2; ++k) {
    c->codes[k] = (uint8_t*)calloc((size_t)(U * T * c->kbytes), 1);
    c->sz[k] = (uint16_t*)calloc((size_t)(U * T * c->NG * 2), 2);
    c->idx[k] = (uint8_t*)malloc((size_t)(U * T));
    memset(c->idx[k], KVQREF_NONE, (size_t)(U * T));
    c->t16[k] = (uint16_t*)calloc((size_t)(U * T), 2);
    c->t2[k] = (uint16_t*)calloc((size_t)(U * T), 2);
    c->tie[k] = (uint8_t*)calloc((size_t)(U * T * D), 1);
    c->pat[k] = (float*)calloc((size_t)(c->PU * (cfg->max_patterns ? cfg->max_patterns : 1) * D), 4);
    c->wlo[k] = (float*)malloc((size_t)(c->PU * D) * 4);
    c->whi[k] = (float*)malloc((size_t)(c->PU * D) * 4);
    c->cscale[k] = (float*)malloc((size_t)(U * D) * 4);
    for (int64_t i = 0; i < U * D; ++i) c->cscale[k][i] = cfg->mode == KVQREF_NSN ? 0.0f : 1.0f;
  }
  c->nblk = (c->tcap + KVQREF_KBLOCK - 1) / KVQREF_KBLOCK;
  c->kbsz = (uint16_t*)calloc((size_t)(U * c->nblk * D * 2), 2);
  c->ktail = (uint16_t*)calloc((size_t)(U * KVQREF_KBLOCK * D), 2);
  reset_window(c);
  return c;
}

void kvqref_free(kvqref_cache* c) {
  if (!c) return;
  for (int k = 0; k < 2; ++k) {
    free(c->codes[k]); free(c->sz[k]); free(c->idx[k]); free(c->t16[k]); free(c->t2[k]); free(c->tie[k]);
    free(c->pat[k]); free(c->wlo[k]); free(c->whi[k]); free(c->cscale[k]);
  }
  free(c->kbsz);
  free(c->ktail);
  free(c);
}

static int64_t code_byte(const kvqref_cache* c, int kind, int64_t u, int32_t t, int32_t d,
                         int* shift) {
  (void)kind;   /* K and V records share the layout (R15) */
  int64_t bit = (int64_t)d * c->cfg.bits;
  *shift = (int)(bit & 7);
  return (u * c->tcap + t) * c->kbytes + bit / 8;
}

static void put_code(kvqref_cache* c, int kind, int64_t u, int32_t t, int32_t d, unsigned q) {
  int sh;
  int64_t at = code_byte(c, kind, u, t, d, &sh);
  unsigned mask = ((1u << c->cfg.bits) - 1u) << sh;
  c->codes[kind][at] = (uint8_t)((c->codes[kind][at] & ~mask) | ((q << sh) & mask));
}

static unsigned get_code(const kvqref_cache* c, int kind, int64_t u, int32_t t, int32_t d) {
  int sh;
  int64_t at = code_byte(c, kind, u, t, d, &sh);
  return (c->codes[kind][at] >> sh) & ((1u << c->cfg.bits) - 1u);
}

static void load_vec(const kvqref_cache* c, const void* src, int64_t row, float* x) {
  int D = c->D;
  if (c->cfg.in_dtype == KVQREF_IN_F32) {
    memcpy(x, (const float*)src + row * D, sizeof(float) * D);
  } else {
    const uint16_t* b = (const uint16_t*)src + row * D;
    for (int i = 0; i < D; ++i) x[i] = bf16_to_f32(b[i]);
  }
}

/* Quantise a whole vector (groups of G channels) and store codes/scales. */
static void store_quantised(kvqref_cache* c, int kind, int64_t u, int32_t t, const float* r) {
  int D = c->D, G = c->cfg.group;
  uint8_t codes[MAX_D], ties[MAX_D];
  for (int g = 0; g < c->NG; ++g) {
    uint16_t s16, z16;
    kvqref_quant_group(r + g * G, G, c->cfg.bits, codes + g * G, &s16, &z16, ties + g * G);
    uint16_t* sz = c->sz[kind] + ((u * c->tcap + t) * c->NG + g) * 2;
    sz[0] = s16;
    sz[1] = z16;
  }
  for (int d = 0; d < D; ++d) {
    put_code(c, kind, u, t, d, codes[d]);
    c->tie[kind][(u * c->tcap + t) * D + d] = ties[d];
  }
}

/* K per channel (R17): quantise block blk of unit u, channel by channel, from
 * the binary16 residuals of its 128 tokens. */
static void quantise_k_block(kvqref_cache* c, int64_t u, int32_t blk) {
  int D = c->D;
  float col[KVQREF_KBLOCK];
  uint8_t codes[KVQREF_KBLOCK], ties[KVQREF_KBLOCK];
  const uint16_t* tail = c->ktail + u * KVQREF_KBLOCK * D;
  for (int d = 0; d < D; ++d) {
    for (int i = 0; i < KVQREF_KBLOCK; ++i) col[i] = kvqref_f16_to_f32(tail[i * D + d]);
    uint16_t s16, z16;
    kvqref_quant_group(col, KVQREF_KBLOCK, c->cfg.bits, codes, &s16, &z16, ties);
    uint16_t* sz = c->kbsz + ((u * c->nblk + blk) * D + d) * 2;
    sz[0] = s16;
    sz[1] = z16;
    for (int i = 0; i < KVQREF_KBLOCK; ++i) {
      int32_t t = blk * KVQREF_KBLOCK + i;
      put_code(c, 0, u, t, d, codes[i]);
      c->tie[0][(u * c->tcap + t) * D + d] = ties[i];
    }
  }
}

/* PatternKV encode of one vector: Eq 6 (nearest pattern, residual), the
 * section 3.3 V threshold, then Eq 1 on the residual (K per channel: the
 * residual waits in binary16 for its block, R17). */
static void encode_pattern_vec(kvqref_cache* c, int kind, int64_t u, int32_t t, const float* x) {
  int D = c->D;
  const float* pats = c->pat[kind] + pu_of(c, u) * (int64_t)c->cfg.max_patterns * D;
  float e = 0.0f;
  int32_t k = kvqref_nearest(x, pats, c->n_patterns, D, &e);
  if (kind == 1 && c->thr_on && k != KVQREF_NONE) {
    float mx = x[0], mn = x[0];
    for (int i = 1; i < D; ++i) {
      if (x[i] > mx) mx = x[i];
      if (x[i] < mn) mn = x[i];
    }
    float r_raw = mx - mn;
    float lim = c->rho * r_raw;
    if (!(e <= lim)) k = KVQREF_NONE;
  }
  float r[MAX_D];
  for (int i = 0; i < D; ++i) r[i] = (k == KVQREF_NONE) ? x[i] : x[i] - pats[(int64_t)k * D + i];
  c->idx[kind][u * c->tcap + t] = (uint8_t)k;
  if (kind == 0 && c->cfg.k_per_channel) {
    uint16_t* slot = c->ktail + (u * KVQREF_KBLOCK + t % KVQREF_KBLOCK) * D;
    for (int i = 0; i < D; ++i) slot[i] = kvqref_f16_round(r[i], 0);
    if (t % KVQREF_KBLOCK == KVQREF_KBLOCK - 1) quantise_k_block(c, u, t / KVQREF_KBLOCK);
    return;
  }
  store_quantised(c, kind, u, t, r);
}

/* KVarN-style encode of one vector (reading R11). */
static void encode_kvarn_vec(kvqref_cache* c, int kind, int64_t u, int32_t t, const float* x) {
  int D = c->D;
  const float* cs = c->cscale[kind] + u * D;
  float y[MAX_D], v[MAX_D];
  memcpy(y, x, sizeof(float) * D);
  kvqref_fwht_f32(y, D);
  const float isd = (float)(1.0 / sqrt((double)D));
  for (int i = 0; i < D; ++i) y[i] = y[i] * isd;
  for (int i = 0; i < D; ++i) {
    float ic = 1.0f / cs[i];
    y[i] = y[i] * ic;
  }
  for (int i = 0; i < D; ++i) v[i] = y[i] * y[i];
  for (int h = D / 2; h >= 1; h >>= 1)
    for (int i = 0; i < h; ++i) v[i] = v[i] + v[i + h];
  float tt = sqrtf(v[0] * (1.0f / (float)D));
  uint16_t tb = kvqref_f16_round(tt, 0);
  float tf = kvqref_f16_to_f32(tb);
  c->t16[kind][u * c->tcap + t] = tb;
  if (tf == 0.0f) {
    for (int i = 0; i < D; ++i) v[i] = 0.0f;
  } else {
    float it = 1.0f / tf;
    for (int i = 0; i < D; ++i) v[i] = y[i] * it;
  }
  store_quantised(c, kind, u, t, v);
}

/* Root mean square by the halving-fold sum of squares (R11): sqrtf(fl(ss * (1/D))). */
static float rms_fold(const float* x, int D) {
  float v[MAX_D];
  for (int i = 0; i < D; ++i) v[i] = x[i] * x[i];
  for (int h = D / 2; h >= 1; h >>= 1)
    for (int i = 0; i < h; ++i) v[i] = v[i] + v[i + h];
  return sqrtf(v[0] * (1.0f / (float)D));
}

/* NSN scalar encode of one vector (reading R18). */
static void encode_nsn_vec(kvqref_cache* c, int kind, int64_t u, int32_t t, const float* x) {
  int D = c->D;
  const float* mu = c->cscale[kind] + u * D;
  float y[MAX_D];
  uint16_t n1b = kvqref_f16_round(rms_fold(x, D), 0), n2b = 0;
  float n1 = kvqref_f16_to_f32(n1b);
  if (n1 != 0.0f) {
    float i1 = 1.0f / n1;
    for (int i = 0; i < D; ++i) y[i] = x[i] * i1 - mu[i];
    /* (two roundings: the product, then the difference; contraction is off) */
    n2b = kvqref_f16_round(rms_fold(y, D), 0);
  }
  float n2 = kvqref_f16_to_f32(n2b);
  c->t16[kind][u * c->tcap + t] = n1b;
  c->t2[kind][u * c->tcap + t] = n2b;
  if (n1 == 0.0f || n2 == 0.0f) {
    for (int i = 0; i < D; ++i) y[i] = 0.0f;
  } else {
    float i2 = 1.0f / n2;
    for (int i = 0; i < D; ++i) y[i] = y[i] * i2;
    kvqref_fwht_f32(y, D);
    const float isd = (float)(1.0 / sqrt((double)D));
    for (int i = 0; i < D; ++i) y[i] = y[i] * isd;
  }
  store_quantised(c, kind, u, t, y);
}

int kvqref_set_patterns(kvqref_cache* c, const float* k_tab, const float* v_tab, int32_t n) {
  if (!c) return -1;
  int64_t U = c->U, D = c->D;
  const float* tabs[2] = {k_tab, v_tab};
  if (c->cfg.mode != KVQREF_PATTERN) {
    for (int k = 0; k < 2; ++k) memcpy(c->cscale[k], tabs[k], sizeof(float) * (size_t)(U * D));
    return 0;
  }
  if (n < 0 || n > c->cfg.max_patterns) return -1;
  for (int k = 0; k < 2; ++k)
    for (int64_t p = 0; p < c->PU; ++p)
      memcpy(c->pat[k] + p * c->cfg.max_patterns * D, tabs[k] + p * n * D, sizeof(float) * (size_t)(n * D));
  c->n_patterns = n;
  reset_window(c);
  return 0;
}

int kvqref_init_patterns(kvqref_cache* c, const void* k, const void* v, int32_t n_tok,
                         int32_t n_pat) {
  if (!c || n_tok <= 0) return -1;
  int64_t U = c->U, D = c->D;
  const void* src[2] = {k, v};
  float* rows = (float*)malloc(sizeof(float) * (size_t)(n_tok * D));
  if (c->cfg.mode == KVQREF_NSN) {
    /* channel centre: mean over the prefix of x / rms(x), binary64 */
    double* acc = (double*)malloc(sizeof(double) * D);
    for (int kind = 0; kind < 2; ++kind)
      for (int64_t u = 0; u < U; ++u) {
        for (int64_t t = 0; t < n_tok; ++t) load_vec(c, src[kind], u * n_tok + t, rows + t * D);
        memset(acc, 0, sizeof(double) * D);
        int64_t cnt = 0;
        for (int64_t t = 0; t < n_tok; ++t) {
          double ss = 0.0;
          for (int i = 0; i < D; ++i) ss += (double)rows[t * D + i] * rows[t * D + i];
          double r = sqrt(ss / (double)D);
          if (!(r > 0.0)) continue;
          for (int i = 0; i < D; ++i) acc[i] += rows[t * D + i] / r;
          cnt++;
        }
        for (int i = 0; i < D; ++i) c->cscale[kind][u * D + i] = cnt ? (float)(acc[i] / (double)cnt) : 0.0f;
      }
    free(acc);
    free(rows);
    return 0;
  }
  if (c->cfg.mode == KVQREF_KVARN) {
    double* y = (double*)malloc(sizeof(double) * D);
    double* acc = (double*)malloc(sizeof(double) * D);
    for (int kind = 0; kind < 2; ++kind)
      for (int64_t u = 0; u < U; ++u) {
        for (int64_t t = 0; t < n_tok; ++t) load_vec(c, src[kind], u * n_tok + t, rows + t * D);
        memset(acc, 0, sizeof(double) * D);
        int64_t cnt = 0;
        for (int64_t t = 0; t < n_tok; ++t) {
          for (int i = 0; i < D; ++i) y[i] = rows[t * D + i];
          fwht_f64(y, (int32_t)D);
          double ss = 0.0;
          for (int i = 0; i < D; ++i) { y[i] /= sqrt((double)D); ss += y[i] * y[i]; }
          double r = sqrt(ss / (double)D);
          if (!(r > 0.0)) continue;
          for (int i = 0; i < D; ++i) acc[i] += (y[i] / r) * (y[i] / r);
          cnt++;
        }
        for (int i = 0; i < D; ++i) {
          float cj = cnt ? (float)sqrt(acc[i] / (double)cnt) : 1.0f;
          c->cscale[kind][u * D + i] = (cj == 0.0f) ? 1.0f : cj;
        }
      }
    free(y);
    free(acc);
    free(rows);
    return 0;
  }
  if (n_pat < 0 || n_pat > c->cfg.max_patterns) { free(rows); return -1; }
  /* k-means rows of pattern unit p: its own prefix, or (shared tables) the
   * prefixes of kv-head p in every sequence, batch-major */
  const int64_t H = c->cfg.n_kv_heads, nb = c->cfg.shared_patterns ? c->cfg.batch : 1;
  free(rows);
  rows = (float*)malloc(sizeof(float) * (size_t)(nb * n_tok * D));
  for (int kind = 0; kind < 2; ++kind)
    for (int64_t p = 0; p < c->PU; ++p) {
      for (int64_t b = 0; b < nb; ++b)
        for (int64_t t = 0; t < n_tok; ++t) {
          const int64_t u = c->cfg.shared_patterns ? b * H + p : p;
          load_vec(c, src[kind], u * n_tok + t, rows + (b * n_tok + t) * D);
        }
      if (n_pat > 0)
        kvqref_kmeans(rows, (int32_t)(nb * n_tok), (int32_t)D, n_pat,
                      c->pat[kind] + p * c->cfg.max_patterns * D, NULL);
    }
  free(rows);
  c->n_patterns = n_pat;
  reset_window(c);
  return 0;
}

int kvqref_encode_append(kvqref_cache* c, const void* k, const void* v, int32_t n_new,
                         int32_t update) {
  if (!c || n_new < 0) return -1;
  if ((int64_t)c->n_tokens + n_new > c->cfg.max_tokens) return -2;
  int64_t U = c->U, D = c->D;
  const void* src[2] = {k, v};
  float x[MAX_D];
  int window = c->cfg.mode == KVQREF_PATTERN && update && c->cfg.pattern_window > 0;
  for (int32_t j = 0; j < n_new; ++j) {
    int32_t t = c->n_tokens + j;
    for (int kind = 0; kind < 2; ++kind)
      for (int64_t u = 0; u < U; ++u) {
        load_vec(c, src[kind], u * n_new + j, x);
        if (c->cfg.mode == KVQREF_PATTERN) encode_pattern_vec(c, kind, u, t, x);
        else if (c->cfg.mode == KVQREF_NSN) encode_nsn_vec(c, kind, u, t, x);
        else encode_kvarn_vec(c, kind, u, t, x);
        if (window) {
          float* lo = c->wlo[kind] + pu_of(c, u) * D;
          float* hi = c->whi[kind] + pu_of(c, u) * D;
          for (int i = 0; i < D; ++i) {
            if (x[i] < lo[i]) lo[i] = x[i];
            if (x[i] > hi[i]) hi[i] = x[i];
          }
        }
      }
    if (window && ++c->win_count == c->cfg.pattern_window) {
      if (c->n_patterns < c->cfg.max_patterns) {
        for (int kind = 0; kind < 2; ++kind)
          for (int64_t p = 0; p < c->PU; ++p) {
            float* m = c->pat[kind] + (p * c->cfg.max_patterns + c->n_patterns) * D;
            for (int i = 0; i < D; ++i) {
              float s = c->wlo[kind][p * D + i] + c->whi[kind][p * D + i];
              m[i] = s * 0.5f;
            }
          }
        c->n_patterns++;
      } else {
        c->dropped++;
      }
      reset_window(c);
    }
  }
  c->n_tokens += n_new;
  return 0;
}

/* Reconstruct token t of unit u (Eq 1 inverse + pattern restore, or the
 * KVarN inverse of reading R11). */
static void dequant_vec(const kvqref_cache* c, int kind, int64_t u, int32_t t, float* out) {
  int D = c->D, G = c->cfg.group;
  const uint16_t* sz = c->sz[kind] + (u * c->tcap + t) * c->NG * 2;
  if (c->cfg.mode == KVQREF_PATTERN) {
    int k = c->idx[kind][u * c->tcap + t];
    const float* m = (k == KVQREF_NONE) ? NULL
                     : c->pat[kind] + (pu_of(c, u) * c->cfg.max_patterns + k) * (int64_t)D;
    if (kind == 0 && c->cfg.k_per_channel) {
      const int32_t blk = t / KVQREF_KBLOCK;
      const int closed = (int64_t)(blk + 1) * KVQREF_KBLOCK <= c->n_tokens;
      const uint16_t* bsz = c->kbsz + (u * c->nblk + blk) * (int64_t)D * 2;
      const uint16_t* res = c->ktail + (u * KVQREF_KBLOCK + t % KVQREF_KBLOCK) * (int64_t)D;
      for (int d = 0; d < D; ++d) {
        float r;
        if (closed) {
          float q = (float)get_code(c, kind, u, t, d);
          r = fmaf(q, kvqref_f16_to_f32(bsz[d * 2]), kvqref_f16_to_f32(bsz[d * 2 + 1]));
        } else {
          r = kvqref_f16_to_f32(res[d]);
        }
        out[d] = m ? r + m[d] : r;
      }
      return;
    }
    for (int d = 0; d < D; ++d) {
      float s = kvqref_f16_to_f32(sz[(d / G) * 2]);
      float z = kvqref_f16_to_f32(sz[(d / G) * 2 + 1]);
      float q = (float)get_code(c, kind, u, t, d);
      float r = fmaf(q, s, z);
      out[d] = m ? r + m[d] : r;
    }
    return;
  }
  const float* cs = c->cscale[kind] + u * D;
  if (c->cfg.mode == KVQREF_NSN) {
    for (int d = 0; d < D; ++d) {
      float s = kvqref_f16_to_f32(sz[(d / G) * 2]);
      float z = kvqref_f16_to_f32(sz[(d / G) * 2 + 1]);
      out[d] = fmaf((float)get_code(c, kind, u, t, d), s, z);
    }
    kvqref_fwht_f32(out, D);
    const float isd = (float)(1.0 / sqrt((double)D));
    const float n1 = kvqref_f16_to_f32(c->t16[kind][u * c->tcap + t]);
    const float n2 = kvqref_f16_to_f32(c->t2[kind][u * c->tcap + t]);
    for (int d = 0; d < D; ++d) out[d] = ((out[d] * isd) * n2 + cs[d]) * n1;
    return;
  }
  float tf = kvqref_f16_to_f32(c->t16[kind][u * c->tcap + t]);
  for (int d = 0; d < D; ++d) {
    float s = kvqref_f16_to_f32(sz[(d / G) * 2]);
    float z = kvqref_f16_to_f32(sz[(d / G) * 2 + 1]);
    float q = (float)get_code(c, kind, u, t, d);
    float w = fmaf(q, s, z);
    w = w * tf;
    out[d] = w * cs[d];
  }
  kvqref_fwht_f32(out, D);
  const float isd = (float)(1.0 / sqrt((double)D));
  for (int d = 0; d < D; ++d) out[d] = out[d] * isd;
}

int kvqref_dequant(const kvqref_cache* c, int32_t which, int32_t tok0, int32_t n, float* out) {
  if (!c || (which != 0 && which != 1) || tok0 < 0 || n < 0 || tok0 + n > c->n_tokens) return -1;
  for (int64_t u = 0; u < c->U; ++u)
    for (int32_t j = 0; j < n; ++j) dequant_vec(c, which, u, tok0 + j, out + (u * n + j) * c->D);
  return 0;
}

static void attn_unit(int D, int T, const float* K, const float* V, const double* q, double sm,
                      double* s, float* out) {
  double m = -INFINITY;
  for (int i = 0; i < T; ++i) {
    double acc = 0.0;
    for (int d = 0; d < D; ++d) acc += q[d] * (double)K[(int64_t)i * D + d];
    s[i] = sm * acc;
    if (s[i] > m) m = s[i];
  }
  double l = 0.0;
  for (int i = 0; i < T; ++i) { s[i] = exp(s[i] - m); l += s[i]; }
  for (int d = 0; d < D; ++d) {
    double acc = 0.0;
    for (int i = 0; i < T; ++i) acc += s[i] * (double)V[(int64_t)i * D + d];
    out[d] = (float)(acc / l);
  }
}

static void load_q(const kvqref_cfg* g, const void* q, int64_t row, double* out) {
  int D = g->head_dim;
  for (int d = 0; d < D; ++d)
    out[d] = g->in_dtype == KVQREF_IN_F32 ? (double)((const float*)q)[row * D + d]
                                          : (double)bf16_to_f32(((const uint16_t*)q)[row * D + d]);
}

int kvqref_attn_decode(const kvqref_cache* c, const void* q, float* out, double sm_scale) {
  if (!c) return -1;
  if (c->n_tokens == 0) return -3;
  int D = c->D, T = c->n_tokens;
  int Hq = c->cfg.n_q_heads, Hkv = c->cfg.n_kv_heads, rep = Hq / Hkv;
  if (!(sm_scale > 0.0)) sm_scale = 1.0 / sqrt((double)D);
  float* K = (float*)malloc(sizeof(float) * (size_t)T * D);
  float* V = (float*)malloc(sizeof(float) * (size_t)T * D);
  double* s = (double*)malloc(sizeof(double) * (size_t)T);
  double qd[MAX_D];
  for (int b = 0; b < c->cfg.batch; ++b)
    for (int h = 0; h < Hkv; ++h) {
      int64_t u = (int64_t)b * Hkv + h;
      for (int t = 0; t < T; ++t) {
        dequant_vec(c, 0, u, t, K + (int64_t)t * D);
        dequant_vec(c, 1, u, t, V + (int64_t)t * D);
      }
      for (int r = 0; r < rep; ++r) {
        int64_t row = (int64_t)b * Hq + h * rep + r;
        load_q(&c->cfg, q, row, qd);
        attn_unit(D, T, K, V, qd, sm_scale, s, out + row * D);
      }
    }
  free(K); free(V); free(s);
  return 0;
}

int kvqref_attn_exact(const kvqref_cfg* g, const float* k, const float* v, int32_t T,
                      const float* q, float* out, double sm_scale) {
  if (!g || T <= 0) return -1;
  int D = g->head_dim, Hq = g->n_q_heads, Hkv = g->n_kv_heads, rep = Hq / Hkv;
  if (!(sm_scale > 0.0)) sm_scale = 1.0 / sqrt((double)D);
  double* s = (double*)malloc(sizeof(double) * (size_t)T);
  double qd[MAX_D];
  for (int b = 0; b < g->batch; ++b)
    for (int h = 0; h < Hkv; ++h) {
      int64_t u = (int64_t)b * Hkv + h;
      for (int r = 0; r < rep; ++r) {
        int64_t row = (int64_t)b * Hq + h * rep + r;
        for (int d = 0; d < D; ++d) qd[d] = q[row * D + d];
        attn_unit(D, T, k + u * T * D, v + u * T * D, qd, sm_scale, s, out + row * D);
      }
    }
  free(s);
  return 0;
}

int32_t kvqref_n_tokens(const kvqref_cache* c) { return c->n_tokens; }
int32_t kvqref_n_patterns(const kvqref_cache* c) { return c->n_patterns; }
int32_t kvqref_dropped(const kvqref_cache* c) { return c->dropped; }
int32_t kvqref_win_count(const kvqref_cache* c) { return c->win_count; }

const void* kvqref_region(const kvqref_cache* c, const char* name, int64_t* bytes) {
  int64_t U = c->U, T = c->tcap, D = c->D, M = c->cfg.max_patterns;
  int kind = name[0] == 'v';
  const char* r = name + 2;
  if (!strcmp(r, "codes")) { *bytes = U * T * c->kbytes; return c->codes[kind]; }
  if (!strcmp(r, "sz")) { *bytes = U * T * c->NG * 4; return c->sz[kind]; }
  if (!strcmp(r, "idx")) { *bytes = U * T; return c->idx[kind]; }
  if (!strcmp(r, "t16")) { *bytes = U * T * 2; return c->t16[kind]; }
  if (!strcmp(r, "t2")) { *bytes = U * T * 2; return c->t2[kind]; }
  if (!strcmp(r, "tie")) { *bytes = U * T * D; return c->tie[kind]; }
  if (!strcmp(r, "pat")) { *bytes = c->PU * M * D * 4; return c->pat[kind]; }
  if (!strcmp(r, "wlo")) { *bytes = c->PU * D * 4; return c->wlo[kind]; }
  if (!strcmp(r, "whi")) { *bytes = c->PU * D * 4; return c->whi[kind]; }
  if (!strcmp(r, "scale")) { *bytes = U * D * 4; return c->cscale[kind]; }
  if (!strcmp(name, "k_bsz")) { *bytes = U * c->nblk * D * 4; return c->kbsz; }
  if (!strcmp(name, "k_tail")) { *bytes = U * KVQREF_KBLOCK * D * 2; return c->ktail; }
  *bytes = 0;
  return NULL;
}
