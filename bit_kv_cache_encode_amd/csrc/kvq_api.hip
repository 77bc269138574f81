// kvq_api.hip -- the C-ABI entry points of include/kvq.h: argument checks,
// cache layout, host-side state (token, pattern and window counters) and
// kernel launches.  Every check runs before the first launch of a call.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "kvq_internal.h"

using namespace kvq;

namespace {

thread_local int g_last_hip = 0;

constexpr int KM_GPU_MAX_PATTERNS = 64;
constexpr int ATTN_MIN_CHUNK = 64;
// In the one-launch step, split 0's block also encodes the new token in two
// of its eight waves, so its token range is this much shorter (measured: with
// 256 its loop ended ~2 us after the other splits' at the 32k context).
constexpr int FUSED_LEAD_TOKENS = 640;
constexpr int ATTN_TARGET_BLOCKS = 2048;

int dev_fail(hipError_t e) {
  g_last_hip = (int)e;
  return KVQ_EDEVICE;
}

uint64_t align256(uint64_t x) { return (x + 255) & ~(uint64_t)255; }

bool cfg_ok(const kvq_config* c) {
  if (!c) return false;
  if (c->batch <= 0 || c->n_kv_heads <= 0 || c->n_q_heads <= 0) return false;
  if (c->n_q_heads % c->n_kv_heads) return false;
  // up to MAX_GQ q-heads per kv-head on every path; up to 16 where the MFMA
  // attention serves the shape (q-head blocks)
  const int gq = c->n_q_heads / c->n_kv_heads;
  if (gq > MAX_GQ && !(gq <= 16 && mfma_attention_supported(c->bits, c->group, gq))) return false;
  if (c->head_dim != D) return false;
  if (c->max_tokens <= 0 || c->max_tokens > (1 << 28)) return false;
  // 1-bit codes in NSN mode (served by the VALU attention)
  if (c->bits != 2 && c->bits != 4 && !(c->bits == 1 && c->mode == KVQ_MODE_NSN)) return false;
  if (c->group < 8 || c->group > D || D % c->group) return false;
  if (c->mode != KVQ_MODE_PATTERN && c->mode != KVQ_MODE_KVARN && c->mode != KVQ_MODE_NSN) return false;
  if (c->group * c->bits % 8) return false;
  if (c->max_patterns < 0 || c->max_patterns > 255) return false;
  if (c->pattern_window < 0) return false;
  if (!(c->v_alpha < 0.5f) || isnan(c->v_alpha)) return false;
  if (c->in_dtype != KVQ_F32 && c->in_dtype != KVQ_BF16) return false;
  if (c->max_splits < 0) return false;
  if (c->shared_patterns != 0 && c->shared_patterns != 1) return false;
  if (c->shared_patterns && c->mode != KVQ_MODE_PATTERN) return false;
  if (c->k_per_channel != 0 && c->k_per_channel != 1) return false;
  if (c->k_per_channel && c->mode != KVQ_MODE_PATTERN) return false;
  return true;
}

// pattern-table (and window) units: one per kv-head when the batch shares them
int64_t pattern_units(const kvq_config& c) {
  return c.shared_patterns ? c.n_kv_heads : (int64_t)c.batch * c.n_kv_heads;
}

// Standard normal quantile: Acklam's rational approximation refined by two
// Halley steps on the CDF written with erfc.
double norm_quantile(double p) {
  static const double a[] = {-3.969683028665376e+01, 2.209460984245205e+02, -2.759285104469687e+02,
                             1.383577518672690e+02, -3.066479806614716e+01, 2.506628277459239e+00};
  static const double b[] = {-5.447609879822406e+01, 1.615858368580409e+02, -1.556989798598866e+02,
                             6.680131188771972e+01, -1.328068155288572e+01};
  static const double c[] = {-7.784894002430293e-03, -3.223964580411365e-01, -2.400758277161838e+00,
                             -2.549732539343734e+00, 4.374664141464968e+00, 2.938163982698783e+00};
  static const double d[] = {7.784695709041462e-03, 3.224671290700398e-01, 2.445134137142996e+00,
                             3.754408661907416e+00};
  double x;
  if (p < 0.02425) {
    double q = sqrt(-2 * log(p));
    x = (((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
        ((((d[0] * q + d[1]) * q + d[2]) * q + d[3]) * q + 1);
  } else if (p > 1 - 0.02425) {
    double q = sqrt(-2 * log(1 - p));
    x = -(((((c[0] * q + c[1]) * q + c[2]) * q + c[3]) * q + c[4]) * q + c[5]) /
        ((((d[0] * q + d[1]) * q + d[2]) * q + d[3]) * q + 1);
  } else {
    double q = p - 0.5, r = q * q;
    x = (((((a[0] * r + a[1]) * r + a[2]) * r + a[3]) * r + a[4]) * r + a[5]) * q /
        (((((b[0] * r + b[1]) * r + b[2]) * r + b[3]) * r + b[4]) * r + 1);
  }
  for (int i = 0; i < 2; ++i) {
    double e = 0.5 * erfc(-x / sqrt(2.0)) - p;
    double u = e * sqrt(2 * M_PI) * exp(x * x / 2);
    x = x - u / (1 + x * u / 2);
  }
  return x;
}

// rho*(d, alpha): where the Eq 10 criterion 1 - rho^2 >= c sqrt(1 + rho^4),
// c = 2 z_{1-alpha} / sqrt(5 d), turns from true to false on (0, 1); found by
// bisection on the criterion itself.
float rho_star(int d, float alpha) {
  double z = norm_quantile(1.0 - (double)alpha);
  double c = 2.0 * z / sqrt(5.0 * d);
  double lo = 0.0, hi = 1.0;
  for (int i = 0; i < 200; ++i) {
    double mid = 0.5 * (lo + hi);
    if (mid == lo || mid == hi) break;
    double f = (1.0 - mid * mid) - c * sqrt(1.0 + mid * mid * mid * mid);
    if (f >= 0.0) lo = mid; else hi = mid;
  }
  return (float)(0.5 * (lo + hi));
}

int max_splits_for(const kvq_config* c, int tcap) {
  if (c->max_splits > 0) return c->max_splits;
  int units = c->batch * c->n_kv_heads;
  int by_tokens = (tcap + ATTN_MIN_CHUNK - 1) / ATTN_MIN_CHUNK;
  int by_blocks = (2 * ATTN_TARGET_BLOCKS + units - 1) / units;
  return by_tokens < by_blocks ? by_tokens : by_blocks;
}

Regions regions_of(const kvq_cache* c, const kvq_layout& L) {
  Regions r;
  uint8_t* base = (uint8_t*)c->base;
  r.codes[0] = base + L.k_codes;
  r.codes[1] = base + L.v_codes;
  r.sz[0] = (uint32_t*)(base + L.k_sz);
  r.sz[1] = (uint32_t*)(base + L.v_sz);
  r.idx[0] = base + L.k_idx;
  r.idx[1] = base + L.v_idx;
  r.pat_h = c->cfg.shared_patterns ? c->cfg.n_kv_heads : 0;
  r.t16[0] = (uint16_t*)(base + L.k_t16);
  r.t16[1] = (uint16_t*)(base + L.v_t16);
  r.t2[0] = (uint16_t*)(base + L.k_t2);
  r.t2[1] = (uint16_t*)(base + L.v_t2);
  r.tab[0] = (float*)(base + L.k_tab);
  r.tab[1] = (float*)(base + L.v_tab);
  r.win[0] = (float*)(base + L.k_win);
  r.win[1] = (float*)(base + L.v_win);
  r.ws = (float*)(base + L.ws);
  r.cnt = (uint32_t*)(base + L.cnt);
  r.kch = c->cfg.k_per_channel;
  r.kbsz = (uint32_t*)(base + L.k_bsz);
  r.ktail = (uint16_t*)(base + L.k_tail);
  r.status = (uint32_t*)(base + L.status);
  return r;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// K per channel after an encode launch of tokens [a.t0, a.t0 + a.n_new): the
// blocks it completes, then the open block's residuals.
hipError_t kch_after(const EncodeArgs& a, int units, hipStream_t s) {
  KchArgs k;
  memset(&k, 0, sizeof(k));
  k.r = a.r;
  k.src = a.src[0];
  k.src_rows = a.src_rows;
  k.t0 = a.t0;
  k.n_new = a.n_new;
  k.blk0 = a.t0 / KBLOCK;
  k.blk1 = (a.t0 + a.n_new) / KBLOCK;
  k.tail0 = k.blk1 * KBLOCK > a.t0 ? k.blk1 * KBLOCK : a.t0;
  if (a.kch_tail_direct) k.tail0 = a.t0 + a.n_new;   // the encode wrote it
  k.tcap = a.tcap;
  k.bits = a.bits;
  k.bf16 = a.bf16;
  k.max_pat = a.max_pat;
  return launch_kch_append(k, units, s);
}

}  // namespace

extern "C" {

int kvq_layout_of(const kvq_config* cfg, kvq_layout* out) {
  if (!cfg_ok(cfg) || !out) return KVQ_EINVAL;
  kvq_layout L;
  memset(&L, 0, sizeof(L));
  const uint64_t U = (uint64_t)cfg->batch * cfg->n_kv_heads;
  const int tcap = (cfg->max_tokens + 63) / 64 * 64;
  const bool pattern = cfg->mode == KVQ_MODE_PATTERN;
  L.token_cap = tcap;
  L.n_groups = D / cfg->group;
  L.max_splits = max_splits_for(cfg, tcap);
  L.codes_bytes = U * tcap * (D * cfg->bits / 8);
  L.sz_bytes = U * tcap * L.n_groups * 4;
  L.idx_bytes = pattern ? U * tcap : 0;
  L.t16_bytes = pattern ? 0 : U * tcap * 2;
  const uint64_t PU = (uint64_t)pattern_units(*cfg);
  L.tab_bytes = pattern ? PU * (uint64_t)cfg->max_patterns * D * 4 : U * D * 4;
  L.win_bytes = pattern ? PU * 2 * D * 4 : 0;
  // split-K partials: o[D], (m, l) and the per-pattern mass w[max_patterns]
  uint64_t ws_attn = (uint64_t)cfg->batch * cfg->n_q_heads * L.max_splits *
                     (D + 2 + (uint64_t)cfg->max_patterns) * 4;
  uint64_t ws_init = 2 * U * (uint64_t)tcap;       // k-means assignments (one byte per token)
  L.ws_bytes = ws_attn > ws_init ? ws_attn : ws_init;
  L.record_bytes = (int)(D * cfg->bits / 8 + L.n_groups * 4 +
                         (pattern ? 1 : cfg->mode == KVQ_MODE_NSN ? 4 : 2));
  uint64_t off = 0;
  auto place = [&](uint64_t bytes) { uint64_t at = off; off = align256(off + bytes); return at; };
  L.k_codes = place(L.codes_bytes);
  L.v_codes = place(L.codes_bytes);
  L.k_sz = place(L.sz_bytes);
  L.v_sz = place(L.sz_bytes);
  L.k_idx = place(L.idx_bytes);
  L.v_idx = place(L.idx_bytes);
  L.k_t16 = place(L.t16_bytes);
  L.v_t16 = place(L.t16_bytes);
  L.k_tab = place(L.tab_bytes);
  L.v_tab = place(L.tab_bytes);
  L.k_win = place(L.win_bytes);
  L.v_win = place(L.win_bytes);
  L.ws = place(L.ws_bytes);
  L.cnt_bytes = (uint64_t)cfg->batch * cfg->n_q_heads * 4;   // one per (unit, q-head block) at most
  L.cnt = place(L.cnt_bytes);
  // K per channel: block scales and the open block's residuals (placed last,
  // so that the other offsets do not depend on the option)
  L.bsz_bytes = cfg->k_per_channel ? U * (uint64_t)kch_blocks(tcap) * D * 4 : 0;
  L.tail_bytes = cfg->k_per_channel ? U * (uint64_t)KBLOCK * D * 2 : 0;
  L.k_bsz = place(L.bsz_bytes);
  L.k_tail = place(L.tail_bytes);
  // NSN: the second norm (after every other region)
  L.t2_bytes = cfg->mode == KVQ_MODE_NSN ? U * tcap * 2 : 0;
  L.k_t2 = place(L.t2_bytes);
  L.v_t2 = place(L.t2_bytes);
  L.status = place(256);
  L.total = off;
  *out = L;
  return KVQ_OK;
}

int kvq_cache_init(kvq_cache* cache, const kvq_config* cfg, void* base, uint64_t bytes,
                   void* stream) {
  kvq_layout L;
  if (!cache || kvq_layout_of(cfg, &L) != KVQ_OK) return KVQ_EINVAL;
  if (!base || ((uintptr_t)base & 255) || bytes < L.total) return KVQ_EINVAL;
  memset(cache, 0, sizeof(*cache));
  cache->cfg = *cfg;
  cache->base = base;
  cache->rho = cfg->v_alpha > 0.0f ? rho_star(D, cfg->v_alpha) : -1.0f;
  // attention kernel and grid: read from the environment here, once per cache
  const char* kenv = getenv("KVQ_ATTN_KERNEL");
  cache->attn_kernel = (kenv && strcmp(kenv, "valu") == 0) ? KVQ_ATTN_VALU : KVQ_ATTN_AUTO;
  const char* benv = getenv("KVQ_ATTN_BLOCKS");
  cache->attn_blocks = benv && atoi(benv) > 0 ? atoi(benv) : 0;
  hipStream_t s = (hipStream_t)stream;
  Regions r = regions_of(cache, L);
  hipError_t ec = launch_fill((float*)r.cnt, 0.0f, (int64_t)(L.cnt_bytes / 4), s);
  if (ec == hipSuccess) ec = launch_fill((float*)r.status, 0.0f, 1, s);
  if (ec != hipSuccess) return dev_fail(ec);
  if (cfg->mode == KVQ_MODE_PATTERN) {
    hipError_t e = launch_window_reset(r.win[0], r.win[1], (int)pattern_units(*cfg),
                                       cfg->shared_patterns, s);
    if (e != hipSuccess) return dev_fail(e);
  } else {
    // KVARN channel scales start at 1, NSN channel centres at 0
    const float v0 = cfg->mode == KVQ_MODE_NSN ? 0.0f : 1.0f;
    hipError_t e = launch_fill(r.tab[0], v0, (int64_t)(L.tab_bytes / 4), s);
    if (e == hipSuccess) e = launch_fill(r.tab[1], v0, (int64_t)(L.tab_bytes / 4), s);
    if (e != hipSuccess) return dev_fail(e);
  }
  return KVQ_OK;
}

int kvq_set_patterns(kvq_cache* cache, const float* k_tab, const float* v_tab, int32_t n,
                     void* stream) {
  kvq_layout L;
  if (!cache || !cache->base || kvq_layout_of(&cache->cfg, &L) != KVQ_OK) return KVQ_EINVAL;
  if (!k_tab || !v_tab || !aligned16(k_tab) || !aligned16(v_tab)) return KVQ_EINVAL;
  const kvq_config& c = cache->cfg;
  const bool pattern = c.mode == KVQ_MODE_PATTERN;
  if (pattern && (n < 0 || n > c.max_patterns)) return KVQ_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  Regions r = regions_of(cache, L);
  const size_t units = (size_t)c.batch * c.n_kv_heads;
  const size_t tab_units = (size_t)pattern_units(c);
  const float* src[2] = {k_tab, v_tab};
  for (int k = 0; k < 2; ++k) {
    hipError_t e;
    if (pattern) {
      if (n == 0) continue;
      e = hipMemcpy2DAsync(r.tab[k], (size_t)c.max_patterns * D * 4, src[k], (size_t)n * D * 4,
                           (size_t)n * D * 4, tab_units, hipMemcpyDeviceToDevice, s);
    } else {
      e = hipMemcpyAsync(r.tab[k], src[k], units * D * 4, hipMemcpyDeviceToDevice, s);
    }
    if (e != hipSuccess) return dev_fail(e);
  }
  if (pattern) {
    hipError_t e = launch_window_reset(r.win[0], r.win[1], (int)tab_units, c.shared_patterns, s);
    if (e != hipSuccess) return dev_fail(e);
    cache->n_patterns = n;
    cache->win_count = 0;
  }
  return KVQ_OK;
}

int kvq_init_patterns(kvq_cache* cache, const void* k, const void* v, int32_t n_tok,
                      int32_t n_patterns, void* stream) {
  kvq_layout L;
  if (!cache || !cache->base || kvq_layout_of(&cache->cfg, &L) != KVQ_OK) return KVQ_EINVAL;
  const kvq_config& c = cache->cfg;
  if (!k || !v || n_tok < 1 || n_tok > L.token_cap) return KVQ_EINVAL;
  const bool pattern = c.mode == KVQ_MODE_PATTERN;
  if (pattern && (n_patterns < 0 || n_patterns > c.max_patterns ||
                  n_patterns > KM_GPU_MAX_PATTERNS))
    return KVQ_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  Regions r = regions_of(cache, L);
  const int units = c.batch * c.n_kv_heads;
  const int bf16 = c.in_dtype == KVQ_BF16;
  hipError_t e = launch_domain_check(k, v, (int64_t)units * n_tok * D, bf16, r.status, s);
  if (e != hipSuccess) return dev_fail(e);
  if (pattern) {
    if (n_patterns > 0) {
      // shared tables: per kv-head over its prefixes in every sequence,
      // pooled batch-major
      const int groups = c.shared_patterns ? c.batch : 1;
      e = launch_kmeans_pair(k, v, bf16, n_tok, groups, (int64_t)c.n_kv_heads * n_tok, n_patterns,
                             r.tab[0], r.tab[1], c.max_patterns, (int)pattern_units(c),
                             (uint8_t*)r.ws, s);
      if (e != hipSuccess) return dev_fail(e);
    }
    e = launch_window_reset(r.win[0], r.win[1], (int)pattern_units(c), c.shared_patterns, s);
    if (e != hipSuccess) return dev_fail(e);
    cache->n_patterns = n_patterns;
    cache->win_count = 0;
  } else if (c.mode == KVQ_MODE_NSN) {
    e = launch_chan_centre_pair(k, v, bf16, n_tok, r.tab[0], r.tab[1], units, s);
    if (e != hipSuccess) return dev_fail(e);
  } else {
    e = launch_chan_scale_pair(k, v, bf16, n_tok, r.tab[0], r.tab[1], units, s);
    if (e != hipSuccess) return dev_fail(e);
  }
  return KVQ_OK;
}

int kvq_encode_append(kvq_cache* cache, const void* k_new, const void* v_new, int32_t n_new,
                      int32_t update_patterns, void* stream) {
  kvq_layout L;
  if (!cache || !cache->base || kvq_layout_of(&cache->cfg, &L) != KVQ_OK) return KVQ_EINVAL;
  const kvq_config& c = cache->cfg;
  if (n_new < 0) return KVQ_EINVAL;
  if (n_new == 0) return KVQ_OK;
  if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)) return KVQ_EINVAL;
  if ((int64_t)cache->n_tokens + n_new > c.max_tokens) return KVQ_ECAPACITY;
  hipStream_t s = (hipStream_t)stream;
  const int units = c.batch * c.n_kv_heads;
  const int in_bytes = c.in_dtype == KVQ_BF16 ? 2 : 4;
  EncodeArgs a;
  memset(&a, 0, sizeof(a));
  a.r = regions_of(cache, L);
  a.tcap = L.token_cap;
  a.ngroups = L.n_groups;
  a.group = c.group;
  a.bits = c.bits;
  a.bf16 = c.in_dtype == KVQ_BF16;
  a.mode = c.mode;
  a.max_pat = c.max_patterns;
  a.rho = cache->rho;
  const bool window = c.mode == KVQ_MODE_PATTERN && update_patterns && c.pattern_window > 0;
  if (!window) {
    a.src[0] = k_new;
    a.src[1] = v_new;
    a.src_rows = n_new;
    a.n_new = n_new;
    a.t0 = cache->n_tokens;
    a.n_pat = cache->n_patterns;
    a.kch_tail_direct = c.k_per_channel && n_new == 1 && (a.t0 + 1) % KBLOCK != 0;
    const int tiles = (a.t0 + n_new - 1) / VT - a.t0 / VT + 1;
    // about 2048 blocks in all, so that each block's pattern-table copy
    // serves many tokens
    int tpb = (int)(((int64_t)tiles * units * 2 + 2047) / 2048);
    a.tiles_per_block = tpb < 1 ? 1 : tpb;
    hipError_t e = launch_encode(a, units, (tiles + a.tiles_per_block - 1) / a.tiles_per_block, s);
    if (e == hipSuccess && c.k_per_channel) e = kch_after(a, units, s);
    if (e != hipSuccess) return dev_fail(e);
    cache->n_tokens += n_new;
    return KVQ_OK;
  }
  // Decode-stage appends: split at Chebyshev window boundaries so that a
  // centre formed by one token serves every later token.  A chunk starting at
  // input row `done` reads rows done.. of every unit (row stride n_new).
  int done = 0;
  while (done < n_new) {
    const int room = c.pattern_window - cache->win_count;
    const int chunk = n_new - done < room ? n_new - done : room;
    a.src[0] = (const uint8_t*)k_new + (size_t)done * D * in_bytes;
    a.src[1] = (const uint8_t*)v_new + (size_t)done * D * in_bytes;
    a.src_rows = n_new;
    a.n_new = chunk;
    a.t0 = cache->n_tokens;
    a.n_pat = cache->n_patterns;
    a.win_update = 1;
    a.win_close = cache->win_count + chunk == c.pattern_window;
    a.close_slot = cache->n_patterns < c.max_patterns ? cache->n_patterns : -1;
    a.kch_tail_direct = c.k_per_channel && chunk == 1 && (a.t0 + 1) % KBLOCK != 0;
    const int tiles = (a.t0 + chunk - 1) / VT - a.t0 / VT + 1;
    a.tiles_per_block = tiles;
    hipError_t e = launch_encode(a, units, 1, s);
    if (e == hipSuccess && c.k_per_channel) e = kch_after(a, units, s);
    // a batch-shared window closes once every unit has folded its vectors in
    if (e == hipSuccess && a.win_close && c.shared_patterns)
      e = launch_window_close(a.r, (int)pattern_units(c), c.max_patterns, a.close_slot, s);
    if (e != hipSuccess) return dev_fail(e);
    cache->n_tokens += chunk;
    cache->win_count += chunk;
    if (a.win_close) {
      if (a.close_slot >= 0) cache->n_patterns += 1;
      else cache->dropped += 1;
      cache->win_count = 0;
    }
    done += chunk;
  }
  return KVQ_OK;
}

// Attention arguments over the cache's first T tokens and the kernel choice.
// `reserve` partial slots per (b, q-head) are kept free for a fused step.
// Kernel choice: the MFMA kernel covers groups of 32 / 64 channels with up
// to 16 q-heads per kv-head and is the default wherever it applies; the
// cache's attn_kernel field may select the VALU kernel (a cross-check) and
// attn_blocks the target grid size (both fixed at kvq_cache_init from the
// environment unless the caller changes them).
enum AttnKernel { ATTN_MFMA, ATTN_VALU };
static AttnKernel attn_setup(const kvq_cache* cache, const kvq_layout& L, const void* q, float* out,
                             float sm_scale, int T, int reserve, AttnArgs& a) {
  const kvq_config& c = cache->cfg;
  memset(&a, 0, sizeof(a));
  a.r = regions_of(cache, L);
  a.q = q;
  a.out = out;
  a.B = c.batch;
  a.Hq = c.n_q_heads;
  a.Hkv = c.n_kv_heads;
  a.gq = c.n_q_heads / c.n_kv_heads;
  a.T = T;
  a.tcap = L.token_cap;
  a.ngroups = L.n_groups;
  a.group = c.group;
  a.bits = c.bits;
  a.bf16 = c.in_dtype == KVQ_BF16;
  a.mode = c.mode;
  a.n_pat = cache->n_patterns;
  a.max_pat = c.max_patterns;
  a.kclosed = T / KBLOCK * KBLOCK;
  const float sm = sm_scale > 0.0f ? sm_scale : 1.0f / sqrtf((float)D);
  a.qscale = sm * 1.4426950408889634f;
  const int units = c.batch * c.n_kv_heads;
  const bool mfma_ok = mfma_attention_supported(c.bits, c.group, a.gq);
  // (the VALU kernel holds at most MAX_GQ q-heads per kv-head)
  const bool valu_ok = a.gq <= MAX_GQ;
  const AttnKernel k = (!mfma_ok || (valu_ok && cache->attn_kernel == KVQ_ATTN_VALU)) ? ATTN_VALU
                                                                                     : ATTN_MFMA;
  // one 8-wave MFMA block per compute unit; the MFMA kernel's blocks are
  // (unit, q-head block, split), so a unit with several q-head blocks takes
  // fewer splits (one round of blocks, fewer partials to combine)
  int target = k == ATTN_VALU ? ATTN_TARGET_BLOCKS : 256;
  if (cache->attn_blocks > 0) target = cache->attn_blocks;
  const int per_split = units * (k == ATTN_MFMA ? mfma_head_blocks(c.group, a.gq) : 1);
  int want = (target + per_split - 1) / per_split;
  if (want > L.max_splits - reserve) want = L.max_splits - reserve;
  if (want < 1) want = 1;
  // split 0 is `lead` tokens shorter (at least one chunk unit long)
  const int lead = reserve ? FUSED_LEAD_TOKENS : 0;
  int chunk = (a.T + lead + want - 1) / want;
  chunk = (chunk + ATTN_MIN_CHUNK - 1) / ATTN_MIN_CHUNK * ATTN_MIN_CHUNK;
  // K per channel: splits start on block boundaries (the MFMA kernel hands
  // out both tiles of a block to one wave)
  if (c.k_per_channel) chunk = (chunk + KBLOCK - 1) / KBLOCK * KBLOCK;
  int chunk0 = chunk - lead < ATTN_MIN_CHUNK ? ATTN_MIN_CHUNK : chunk - lead;
  a.chunk = chunk;
  a.chunk0 = chunk0;
  a.splits = a.T <= chunk0 ? 1 : 1 + (a.T - chunk0 + chunk - 1) / chunk;
  return k;
}

static int attn_launch(AttnKernel k, const AttnArgs& a, void* stream) {
  hipError_t e = k == ATTN_MFMA ? launch_attention_mfma(a, (hipStream_t)stream)
                                : launch_attention(a, (hipStream_t)stream);
  return e == hipSuccess ? KVQ_OK : dev_fail(e);
}

int kvq_attn_decode(kvq_cache* cache, const void* q, float* out, float sm_scale, void* stream) {
  kvq_layout L;
  if (!cache || !cache->base || kvq_layout_of(&cache->cfg, &L) != KVQ_OK) return KVQ_EINVAL;
  if (!q || !out || !aligned16(q) || !aligned16(out)) return KVQ_EINVAL;
  if (cache->n_tokens <= 0) return KVQ_ESTATE;
  AttnArgs a;
  const AttnKernel k = attn_setup(cache, L, q, out, sm_scale, cache->n_tokens, 0, a);
  return attn_launch(k, a, stream);
}

}  // extern "C"

// ---------------------------------------------------------------- no-allocation attention
// Split-K workspace of kvq_attn_decode_noalloc: arrival counters in the first
// KVQ_NOALLOC_COUNTER_BYTES, partials after them.  One copy per GPU, held
// until the process ends; every such call on a GPU shares it.  Host code
// never passes the array's name to a kernel: its device address comes from
// hipGetSymbolAddress, once per device, with that device current.
static __device__ __align__(256) unsigned char scratch[KVQ_NOALLOC_COUNTER_BYTES + KVQ_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[SCRATCH_MAX_DEVICES];

// The current device's scratch address; its first use on a device clears the
// counters (a fill kernel on `s`, so the call stays capturable).
int scratch_of_current_device(void** out, hipStream_t s) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return dev_fail(e);
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES) return KVQ_EINVAL;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return dev_fail(e != hipSuccess ? e : hipErrorInvalidSymbol);
    e = launch_fill((float*)p, 0.0f, (int64_t)(KVQ_NOALLOC_COUNTER_BYTES / 4), s);
    if (e != hipSuccess) return dev_fail(e);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KVQ_OK;
}
}  // namespace

extern "C" {

int kvq_attn_decode_noalloc(kvq_cache* cache, const void* q, float* out, float sm_scale,
                            void* stream) {
  kvq_layout L;
  if (!cache || !cache->base || kvq_layout_of(&cache->cfg, &L) != KVQ_OK) return KVQ_EINVAL;
  if (!q || !out || !aligned16(q) || !aligned16(out)) return KVQ_EINVAL;
  if (cache->n_tokens <= 0) return KVQ_ESTATE;
  AttnArgs a;
  const AttnKernel k = attn_setup(cache, L, q, out, sm_scale, cache->n_tokens, 0, a);
  const kvq_config& c = cache->cfg;
  // partials o[D] and (m, l) per (b, q-head, split); at most one arrival
  // counter per (b, q-head)
  const uint64_t ws_need = (uint64_t)c.batch * c.n_q_heads * a.splits * (D + 2) * 4;
  const uint64_t cnt_need = (uint64_t)c.batch * c.n_q_heads * 4;
  if (ws_need > KVQ_NOALLOC_SCRATCH_BYTES || cnt_need > KVQ_NOALLOC_COUNTER_BYTES) return KVQ_ESCRATCH;
  void* p = nullptr;
  const int st = scratch_of_current_device(&p, (hipStream_t)stream);
  if (st != KVQ_OK) return st;
  a.r.cnt = (uint32_t*)p;
  a.r.ws = (float*)((unsigned char*)p + KVQ_NOALLOC_COUNTER_BYTES);
  return attn_launch(k, a, stream);
}

int kvq_decode_step(kvq_cache* cache, const void* k_new, const void* v_new, const void* q,
                    float* out, float sm_scale, int32_t update_patterns, void* stream) {
  kvq_layout L;
  if (!cache || !cache->base || kvq_layout_of(&cache->cfg, &L) != KVQ_OK) return KVQ_EINVAL;
  if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)) return KVQ_EINVAL;
  if (!q || !out || !aligned16(q) || !aligned16(out)) return KVQ_EINVAL;
  const kvq_config& c = cache->cfg;
  if ((int64_t)cache->n_tokens + 1 > c.max_tokens) return KVQ_ECAPACITY;
  AttnArgs a;
  const AttnKernel k = cache->n_tokens > 0 && L.max_splits >= 2
                           ? attn_setup(cache, L, q, out, sm_scale, cache->n_tokens, 1, a)
                           : ATTN_VALU;
  // The fused launch covers the MFMA kernel (PatternKV and KVarN modes) with
  // a non-empty cache; anything else is the two calls in sequence.
  // K per channel: a token that completes its block needs the block kernel
  const bool kch_close = c.k_per_channel && (cache->n_tokens + 1) % KBLOCK == 0;
  if (k != ATTN_MFMA || kch_close || c.mode == KVQ_MODE_NSN) {
    int st = kvq_encode_append(cache, k_new, v_new, 1, update_patterns, stream);
    if (st != KVQ_OK) return st;
    return kvq_attn_decode(cache, q, out, sm_scale, stream);
  }
  EncodeArgs& e = a.enc;
  memset(&e, 0, sizeof(e));
  e.r = a.r;
  e.src[0] = k_new;
  e.src[1] = v_new;
  e.src_rows = 1;
  e.n_new = 1;
  e.t0 = cache->n_tokens;
  e.tcap = L.token_cap;
  e.ngroups = L.n_groups;
  e.group = c.group;
  e.bits = c.bits;
  e.bf16 = c.in_dtype == KVQ_BF16;
  e.mode = c.mode;
  e.n_pat = cache->n_patterns;
  e.max_pat = c.max_patterns;
  e.rho = cache->rho;
  e.tiles_per_block = 1;
  e.kch_tail_direct = c.k_per_channel;   // the token leaves its block open (checked above)
  const bool window = c.mode == KVQ_MODE_PATTERN && update_patterns && c.pattern_window > 0;
  if (window) {
    e.win_update = 1;
    e.win_close = cache->win_count + 1 == c.pattern_window;
    e.close_slot = cache->n_patterns < c.max_patterns ? cache->n_patterns : -1;
  }
  a.fuse = 1;
  const int st = attn_launch(k, a, stream);
  if (st != KVQ_OK) return st;
  if (window && e.win_close && c.shared_patterns) {
    // the new centre serves later tokens only, so it may follow the step
    hipError_t he = launch_window_close(a.r, (int)pattern_units(c), c.max_patterns, e.close_slot,
                                        (hipStream_t)stream);
    if (he != hipSuccess) return dev_fail(he);
  }
  cache->n_tokens += 1;
  if (window) {
    cache->win_count += 1;
    if (e.win_close) {
      if (e.close_slot >= 0) cache->n_patterns += 1;
      else cache->dropped += 1;
      cache->win_count = 0;
    }
  }
  return KVQ_OK;
}

int kvq_dequant(const kvq_cache* cache, int32_t which, int32_t tok0, int32_t n, float* out,
                void* stream) {
  kvq_layout L;
  if (!cache || !cache->base || kvq_layout_of(&cache->cfg, &L) != KVQ_OK) return KVQ_EINVAL;
  if (which != 0 && which != 1) return KVQ_EINVAL;
  if (tok0 < 0 || n < 0 || (int64_t)tok0 + n > cache->n_tokens) return KVQ_EINVAL;
  if (n == 0) return KVQ_OK;
  if (!out || !aligned16(out)) return KVQ_EINVAL;
  const kvq_config& c = cache->cfg;
  DequantArgs a;
  memset(&a, 0, sizeof(a));
  a.r = regions_of(cache, L);
  a.out = out;
  a.which = which;
  a.tok0 = tok0;
  a.n = n;
  a.tcap = L.token_cap;
  a.ngroups = L.n_groups;
  a.group = c.group;
  a.bits = c.bits;
  a.mode = c.mode;
  a.max_pat = c.max_patterns;
  a.n_closed = cache->n_tokens / KBLOCK * KBLOCK;
  hipError_t e = launch_dequant(a, c.batch * c.n_kv_heads, (hipStream_t)stream);
  if (e != hipSuccess) return dev_fail(e);
  return KVQ_OK;
}

int kvq_cache_status(kvq_cache* cache, uint32_t* flags, int32_t clear, void* stream) {
  kvq_layout L;
  if (!cache || !cache->base || !flags || kvq_layout_of(&cache->cfg, &L) != KVQ_OK) return KVQ_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  uint32_t* dev = (uint32_t*)((uint8_t*)cache->base + L.status);
  uint32_t h = 0;
  hipError_t e = hipMemcpyAsync(&h, dev, 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess && clear) e = launch_fill((float*)dev, 0.0f, 1, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return dev_fail(e);
  *flags = h;
  return KVQ_OK;
}

const char* kvq_strerror(int status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_EINVAL: return "invalid argument or unsupported configuration";
    case KVQ_ECAPACITY: return "append exceeds the cache's max_tokens";
    case KVQ_ESTATE: return "operation not valid in the cache's current state";
    case KVQ_EDEVICE: return "HIP launch or runtime call failed";
    case KVQ_ESCRATCH:
      return "split-K workspace exceeds the static scratch of kvq_attn_decode_noalloc "
             "(KVQ_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int kvq_last_device_error(void) { return g_last_hip; }

}  // extern "C"
