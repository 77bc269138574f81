/*
 * kvq.h -- low-bit (2/4-bit) KV-cache encode and single-query decode
 * attention over the packed cache, for AMD Instinct MI355X (gfx950).
 *
 * The method is PatternKV's pattern-aligned residual quantization
 * (arXiv 2510.05176v2, "PatternKV: Flattening KV Representation Expands
 * Quantization Headroom"), with a KVarN-style second encode mode (arXiv
 * 2606.03458, Hadamard rotation plus variance normalisation over both axes;
 * NSNQuant, arXiv 2505.18231, token-wise normalisation with a Hadamard
 * transform).
 *
 * Conventions shared by every call
 *  - Return 0 (KVQ_OK) or a negative status.  Every argument is validated on
 *    the host before anything is launched, so a call that fails leaves the
 *    cache and all outputs untouched.  No exception crosses this interface.
 *  - Tensor pointers are DEVICE pointers, 16-byte aligned, row-major and
 *    contiguous in the shapes stated.  Inputs are binary32 (KVQ_F32) or
 *    bfloat16 (KVQ_BF16) as the cache's in_dtype says; outputs are binary32.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *    work on it and never synchronise or copy device data to the host, with
 *    one exception: kvq_cache_status, which exists to read a device word.
 *  - A cache must not be used from two streams or two threads at once.
 *  - The library never allocates device memory: the caller owns one device
 *    buffer per cache (kvq_layout_of().total bytes, 256-byte aligned) and
 *    frees it.  The split-K workspace of the attention lives in that buffer.
 *  - Supported shapes: head_dim 128; bits 2 or 4 (also 1 in NSN mode); group
 *    divides 128 and is a multiple of 8; max_patterns <= 255; n_q_heads a
 *    multiple of n_kv_heads with at most 8 q-heads per kv-head, or at most 16
 *    where bits is 2 or 4 and group is 32 or 64 (served by the matrix-core
 *    attention).  shared_patterns and k_per_channel are PATTERN-mode options.
 *  - Domain: finite K/V inputs with |x| < KVQ_KV_LIMIT (4096: binary16
 *    scales of residuals stay below 2^13, which the attention's binary16
 *    p * s operands assume) and finite queries with |q| * sm_scale <
 *    KVQ_Q_LIMIT (2^96: scores stay finite in binary32).  Results computed
 *    from inputs outside it are unspecified; the kernels that read an input
 *    flag such elements in a sticky word in the cache buffer (no host sync),
 *    which kvq_cache_status reads.
 *
 * Stored format (per (batch, kv-head) "unit", for K and for V alike unless
 * noted; T = token capacity, max_tokens rounded up to a multiple of 64):
 *  - codes: T * 128 * bits / 8 bytes.  K is token-major: channel d of a token
 *    sits at bit bits*d of the token's record (little-endian).  V is stored
 *    in tiles of 32 tokens; a tile is made of 32-bit words, each holding
 *    32/bits consecutive tokens of one channel (token k of the word at bit
 *    bits*k), word w of channel d at byte (w*128 + d)*4 of the tile.
 *  - sz: per token and group, the binary16 scale s then the binary16 zero z
 *    (Eq 1: x^ = s*q + z).  z is the group minimum rounded toward -inf, s is
 *    (max - z)/(2^bits - 1) rounded toward +inf; codes are
 *    clamp(rint((r - z) * fl(1/s)), 0, 2^bits - 1), 0 when s == 0.
 *  - idx (PATTERN): one byte per token, the stored pattern index k* of
 *    section 3.2, 0xFF when the raw vector was quantized.
 *  - t16 (KVARN): one binary16 token scale per token; (NSN) the first norm n1.
 *  - t2 (NSN): the second norm n2, one binary16 per token.
 *  - NSN mode (a scalar reading of NSNQuant's double normalisation, arXiv
 *    2505.18231, abstract): n1 = rms(x), a = x * fl(1/n1) - mu (mu the
 *    unit's channel centre, the tables), n2 = rms(a), y = Hadamard(a *
 *    fl(1/n2)) / sqrt(D), Eq 1 on y with 1, 2 or 4 bits; rms is
 *    sqrtf(fl(ss * (1/D))) with ss the halving-fold sum of squares, n1 and
 *    n2 are stored as nearest-even binary16 (a zero one gives zero codes and
 *    scales).  x^ = fl(fl(fl(w * n2) + mu) * n1), w = Hadamard(fmaf(q, s, z))
 *    / sqrt(D).
 *  - k_per_channel (PATTERN): K is quantized per channel over blocks of
 *    KVQ_KBLOCK = 128 tokens instead of per token and group (PatternKV's
 *    experimental setting, section 4.1, after KIVI; appendix E: groups of 128
 *    with a 128-token residual cleared once its group is quantized).  A K
 *    vector takes its nearest pattern on arrival (idx as above); its residual
 *    x - M_k*, rounded to binary16 (nearest-even), waits in k_tail (slot
 *    t mod 128).  When a block is complete each channel's 128 residuals go
 *    through the Eq 1 quantizer along the token axis: k_bsz holds one packed
 *    (s | z << 16) word per block and channel, the codes keep the K layout
 *    above.  Tokens of the open block reconstruct as residual + M_k*.  The K
 *    sz region is unused; V is unchanged.
 */
#ifndef KVQ_H
#define KVQ_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_OK 0
#define KVQ_EINVAL (-1)     /* bad argument or configuration */
#define KVQ_ECAPACITY (-2)  /* append would exceed max_tokens */
#define KVQ_ESTATE (-3)     /* call not valid in the cache's state */
#define KVQ_EDEVICE (-4)    /* a HIP launch or runtime call failed */
#define KVQ_ESCRATCH (-5)   /* kvq_attn_decode_noalloc: workspace beyond its static scratch */

#define KVQ_MODE_PATTERN 0  /* PatternKV residual encode */
#define KVQ_MODE_KVARN 1    /* Hadamard + dual-axis normalisation encode */
#define KVQ_MODE_NSN 2      /* token norm, channel centre, token norm, Hadamard */
#define KVQ_F32 0
#define KVQ_BF16 1
#define KVQ_INDEX_NONE 0xFF
#define KVQ_VTILE 32
#define KVQ_KBLOCK 128      /* tokens per K block with k_per_channel */
#define KVQ_KV_LIMIT 4096.0f        /* K/V domain: |x| < KVQ_KV_LIMIT */
#define KVQ_Q_LIMIT 0x1p96f         /* query domain: |q| * sm_scale < KVQ_Q_LIMIT */
#define KVQ_DOMAIN_KV 1u    /* status bit: a K/V input element outside its domain */
#define KVQ_DOMAIN_Q 2u     /* status bit: a query element outside its domain */

typedef struct {
  int32_t batch;          /* B */
  int32_t n_q_heads;      /* Hq */
  int32_t n_kv_heads;     /* Hkv; q-head hq attends to kv-head hq / (Hq/Hkv) */
  int32_t head_dim;       /* D, must be 128 */
  int32_t max_tokens;     /* token capacity per unit */
  int32_t bits;           /* 2 or 4; also 1 in NSN mode */
  int32_t group;          /* channels per quantization group (Eq 1 scope) */
  int32_t mode;           /* KVQ_MODE_PATTERN, KVQ_MODE_KVARN or KVQ_MODE_NSN */
  int32_t max_patterns;   /* pattern table capacity per unit and kind, <= 255 */
  int32_t pattern_window; /* G_pattern of Eq 5 (0 = no decode-time patterns) */
  float v_alpha;          /* z-test level of section 3.3; <= 0 disables it */
  int32_t in_dtype;       /* KVQ_F32 or KVQ_BF16 for k, v and q inputs */
  int32_t max_splits;     /* split-K workspace capacity; 0 = derived */
  int32_t shared_patterns; /* PATTERN mode: 1 = one pattern table and one Chebyshev
                              window per kv-head, shared by the whole batch (the
                              batch-free pattern memory of PatternKV's memory
                              analysis); 0 = per (batch, kv-head) unit */
  int32_t k_per_channel;  /* PATTERN mode: 1 = K quantized per channel over 128-token
                             blocks with a binary16 residual for the open block
                             (see the stored format above); 0 = per token */
} kvq_config;

/* Byte offsets (from the cache base) and sizes of every region. */
typedef struct {
  uint64_t k_codes, v_codes, k_sz, v_sz, k_idx, v_idx, k_t16, v_t16;
  uint64_t k_tab, v_tab;  /* PATTERN: fp32 [PU][max_patterns][D]; KVARN: fp32 [U][D];
                             PU = Hkv with shared_patterns, else U = B * Hkv */
  uint64_t k_win, v_win;  /* PATTERN window state [PU][2][D] (min, max): fp32, or
                             with shared_patterns int32 order keys of the fp32
                             values (atomic min / max across the batch) */
  uint64_t ws;            /* split-K partials */
  uint64_t cnt;           /* split-K arrival counters, uint32 [U], zero between calls */
  uint64_t codes_bytes, sz_bytes, idx_bytes, t16_bytes, tab_bytes, win_bytes, ws_bytes;
  uint64_t cnt_bytes;
  uint64_t total;
  int32_t token_cap;      /* max_tokens rounded up to a multiple of 64 */
  int32_t n_groups;       /* head_dim / group */
  int32_t record_bytes;   /* stored bytes per token per unit and kind */
  int32_t max_splits;
  uint64_t k_bsz;         /* k_per_channel: packed (s | z << 16) [U][token_cap / 128][D] */
  uint64_t k_tail;        /* k_per_channel: binary16 residuals [U][128][D] of the open block */
  uint64_t bsz_bytes, tail_bytes;   /* 0 without k_per_channel */
  uint64_t k_t2, v_t2;    /* NSN: binary16 second norm n2 [U][token_cap] */
  uint64_t t2_bytes;      /* 0 outside NSN mode */
  uint64_t status;        /* uint32 domain flags (KVQ_DOMAIN_*), sticky; 256 bytes
                             reserved, after every other region */
} kvq_layout;

typedef struct {
  kvq_config cfg;
  void* base;             /* device buffer of layout.total bytes */
  int32_t n_tokens;       /* tokens stored per unit */
  int32_t n_patterns;     /* patterns in every unit's table */
  int32_t win_count;      /* decode appends in the open Chebyshev window */
  int32_t dropped;        /* window centres dropped because the table was full */
  float rho;              /* binary32 rho*(head_dim, v_alpha) of Eq 10 */
  int32_t attn_kernel;    /* attention kernel: KVQ_ATTN_AUTO (the matrix-core kernel
                             wherever it applies) or KVQ_ATTN_VALU (the vector
                             kernel, a cross-check, for at most 8 q-heads per
                             kv-head); kvq_cache_init sets it from the environment
                             variable KVQ_ATTN_KERNEL ("valu"), callers may change it */
  int32_t attn_blocks;    /* target grid size of the attention (0 = the default: one
                             8-wave block per compute unit, 256); kvq_cache_init sets
                             it from KVQ_ATTN_BLOCKS, callers may change it */
} kvq_cache;

#define KVQ_ATTN_AUTO 0
#define KVQ_ATTN_VALU 1

/* Layout of a cache for `cfg`.  Host only; touches no device.
 * KVQ_EINVAL if the configuration is not supported. */
int kvq_layout_of(const kvq_config* cfg, kvq_layout* out);

/* Bind `cache` to a caller-allocated device buffer of `bytes` bytes
 * (>= layout.total, 256-byte aligned) and reset it: no tokens, no patterns,
 * empty Chebyshev window (launches one fill kernel on `stream`).
 * KVQ_EINVAL on a bad config, size or alignment. */
int kvq_cache_init(kvq_cache* cache, const kvq_config* cfg, void* base, uint64_t bytes,
                   void* stream);

/* Prefill pattern mining (PatternKV section 3.1, Eq 4): for every unit and for
 * K and V separately, Euclidean k-means over the n_tok prefix vectors
 * (k: [B][Hkv][n_tok][D], v likewise) into n_patterns centroids.  With
 * shared_patterns the k-means of kv-head h runs over its B prefixes pooled
 * batch-major (row b*n_tok + t), so N = B*n_tok rows; otherwise N = n_tok.
 * Centroid j starts at row floor(j*N/n_patterns); Lloyd iterations run until
 * no assignment changes (at most 50), ties go to the lowest index, an empty
 * cluster keeps its centroid; binary64 arithmetic, stored as fp32.
 * KVARN mode instead sets each unit's per-channel scale c_j to the root mean
 * square over the prefix of (y_j / rms(y)) with y the orthonormal Hadamard
 * rotation of the token (0 becomes 1): the channel axis of KVarN's dual-axis
 * normalisation (arXiv 2606.03458, abstract).  NSN mode sets each unit's
 * channel centre mu to the mean over the prefix of x / rms(x) (binary64,
 * stored as fp32).  Resets the Chebyshev window.
 * KVQ_EINVAL if n_tok < 1 or n_patterns > max_patterns. */
int kvq_init_patterns(kvq_cache* cache, const void* k, const void* v, int32_t n_tok,
                      int32_t n_patterns, void* stream);

/* Upload pattern tables mined elsewhere: k_tab and v_tab are fp32 device
 * arrays [B][Hkv][n][D] (PATTERN, n <= max_patterns; [Hkv][n][D] with
 * shared_patterns), per-channel scales [B][Hkv][D] (KVARN, n ignored) or
 * channel centres [B][Hkv][D] (NSN, n ignored).
 * Resets the Chebyshev window.
 * KVQ_EINVAL on a bad n or null pointer. */
int kvq_set_patterns(kvq_cache* cache, const float* k_tab, const float* v_tab, int32_t n,
                     void* stream);

/* Encode n_new tokens per unit (k_new, v_new: [B][Hkv][n_new][D]) and append
 * them at position n_tokens.
 * PATTERN (section 3.2, Eq 6 and Eq 1): each vector takes its nearest pattern
 * under d_mm(x, m) = max_i(x_i - m_i) - min_j(x_j - m_j) (lowest index on
 * ties), subtracts it and quantizes the residual per group; a V vector keeps
 * its pattern only if R_flat <= rho* R_raw (section 3.3, Eq 10), else it
 * stores index 0xFF and quantizes the raw vector.  update_patterns != 0 marks
 * decode-stage appends: they feed the Chebyshev window (Eq 5) whose centre
 * fl(fl(min + max) * 0.5) joins the table after every pattern_window-th such
 * token and serves the tokens after it.  With shared_patterns the window of
 * kv-head h takes its min / max over every sequence's vectors, and each
 * closure adds one centre to h's table (a second, small launch).
 * KVARN: y = Hadamard(x)/sqrt(D), y~ = y / c, t = rms(y~) stored as binary16,
 * u = y~ / t quantized per group (update_patterns is ignored).
 * NSN: as described with the stored format above (update_patterns ignored).
 * k_per_channel: K residuals go to the open block's binary16 buffer, and every
 * block this append completes is quantized per channel (two more launches).
 * KVQ_ECAPACITY if n_tokens + n_new > max_tokens; KVQ_EINVAL on null inputs
 * or n_new < 0. */
int kvq_encode_append(kvq_cache* cache, const void* k_new, const void* v_new, int32_t n_new,
                      int32_t update_patterns, void* stream);

/* Single-query decode attention over all n_tokens cached tokens, reading the
 * packed cache directly (PatternKV section 3.4: pattern restore, dequant and
 * the QK product fused; dequant, pattern restore and the attention-weighted
 * sum over V fused).  q: [B][Hq][D] in in_dtype; out: fp32 [B][Hq][D];
 * out = softmax(sm_scale * q . k^) v^ with k^, v^ the dequantized cache
 * (sm_scale <= 0 means 1/sqrt(D)).  Split-K over tokens with a combine pass.
 * KVQ_ESTATE if the cache is empty; KVQ_EINVAL on null pointers. */
int kvq_attn_decode(kvq_cache* cache, const void* q, float* out, float sm_scale, void* stream);

/* kvq_attn_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same kernels and results, with the split-K partials and arrival
 * counters in a static device array of the library instead of the cache
 * buffer's workspace region (which it leaves untouched).  The array holds
 * KVQ_NOALLOC_SCRATCH_BYTES of partials (B * Hq * splits * (D + 2) * 4
 * bytes; splits is about 256 / (B * Hkv) with the default grid, and
 * attn_blocks raises it) and KVQ_NOALLOC_COUNTER_BYTES of counters
 * (B * Hq * 4 bytes).  Each GPU has its own copy, kept until the process
 * ends; the first call on a device (which must be the calling thread's
 * current device) looks up its address and clears its counters on `stream`.
 * Every call on a GPU shares that GPU's copy: calls that overlap on one GPU
 * (different streams, or different threads without ordering) race.  No call
 * to hipMalloc, hipFree or any allocating routine.
 * Errors as kvq_attn_decode, plus KVQ_ESCRATCH (nothing launched) when the
 * call's workspace exceeds the scratch. */
#define KVQ_NOALLOC_SCRATCH_BYTES (8u << 20)
#define KVQ_NOALLOC_COUNTER_BYTES (64u << 10)
int kvq_attn_decode_noalloc(kvq_cache* cache, const void* q, float* out, float sm_scale,
                            void* stream);

/* One decode step in one launch: append one token per unit (k_new, v_new:
 * [B][Hkv][1][D], encoded exactly as kvq_encode_append with n_new = 1) and
 * attend with q over all n_tokens + 1 tokens (as kvq_attn_decode after the
 * append).  The new token's own attention term is computed from its freshly
 * dequantized K and V by the block that encodes it (each q-head block of the
 * unit where one MFMA row block holds fewer q-heads than the unit has), while
 * the other blocks attend over the earlier tokens; the split-K combine merges
 * both (the decode-stage fusion of PatternKV section 3.4 extended to the
 * append).  Cache contents afterwards are identical to the two separate
 * calls; `out` agrees with them to floating-point rounding.  Falls back to
 * the two calls in sequence where the fused launch does not apply (an empty
 * cache, shapes served by the VALU kernel, NSN mode, a k_per_channel token
 * that completes its block).
 * Errors as kvq_encode_append (n_new = 1) and kvq_attn_decode; nothing is
 * written when a check fails. */
int kvq_decode_step(kvq_cache* cache, const void* k_new, const void* v_new, const void* q,
                    float* out, float sm_scale, int32_t update_patterns, void* stream);

/* Dequantize tokens tok0 .. tok0+n-1 of K (which = 0) or V (which = 1) into
 * fp32 out [B][Hkv][n][D]: PATTERN x^ = fl(fmaf(q, s, z) + M_k*) (the index
 * restore of section 3.2), or fmaf(q, s, z) alone for index 0xFF; KVARN
 * x^ = Hadamard(fl(fl(fmaf(q, s, z) * t) * c)) / sqrt(D); NSN as in the
 * stored format above; k_per_channel K
 * in the open block x^ = fl(residual + M_k*).
 * KVQ_EINVAL on a bad `which` or a span outside [0, n_tokens). */
int kvq_dequant(const kvq_cache* cache, int32_t which, int32_t tok0, int32_t n, float* out,
                void* stream);

/* Input-domain flags of the cache: *flags receives the KVQ_DOMAIN_* bits set
 * since kvq_cache_init or the last clearing read.  KVQ_DOMAIN_KV: an element
 * of k / v given to kvq_encode_append, kvq_decode_step or kvq_init_patterns
 * was not finite or had |x| >= KVQ_KV_LIMIT.  KVQ_DOMAIN_Q: an element of a
 * query given to an attention call was not finite or had |q| * sm_scale >=
 * KVQ_Q_LIMIT.  The flags are set by the kernels that read the inputs (an
 * atomic OR by each offending lane, nothing on the normal path), so work
 * enqueued before this call is covered.  clear != 0 resets the word after
 * the read.  This call synchronises `stream` (it copies the word to the
 * host) and therefore cannot be captured in a graph.  KVQ_EINVAL on a null
 * cache or flags. */
int kvq_cache_status(kvq_cache* cache, uint32_t* flags, int32_t clear, void* stream);

/* Message for a status code (static storage). */
const char* kvq_strerror(int status);

/* The HIP error code behind the most recent KVQ_EDEVICE on this thread. */
int kvq_last_device_error(void);

#ifdef __cplusplus
}
#endif
#endif
