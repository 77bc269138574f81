// kvq_internal.h -- device helpers and launch parameter blocks shared by the
// library's HIP sources (not installed; the public interface is include/kvq.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

constexpr int D = 128;        // head_dim supported by the kernels
constexpr int VT = KVQ_VTILE; // tokens per V code tile
constexpr int MAX_GQ = 8;     // q-heads per kv-head handled by one attention block

// ------------------------------------------------------------ binary16 bits
__device__ __forceinline__ uint16_t h2bits(_Float16 h) { return __builtin_bit_cast(uint16_t, h); }
__device__ __forceinline__ float bits2f(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// binary16 of x rounded toward -inf: convert to nearest-even, then step one
// binary16 value down if that overshot x.
__device__ __forceinline__ uint16_t f16_down(float x) {
  uint16_t b = h2bits((_Float16)x);
  if (bits2f(b) > x) b = (b & 0x8000u) ? (uint16_t)(b + 1) : (b == 0 ? (uint16_t)0x8001 : (uint16_t)(b - 1));
  if ((b & 0x7FFFu) == 0) b = 0;   // store zero as +0
  return b;
}

// binary16 of x rounded toward +inf.
__device__ __forceinline__ uint16_t f16_up(float x) {
  uint16_t b = h2bits((_Float16)x);
  if (bits2f(b) < x) b = (b & 0x8000u) ? (b == 0x8000u ? (uint16_t)1 : (uint16_t)(b - 1)) : (uint16_t)(b + 1);
  if ((b & 0x7FFFu) == 0) b = 0;
  return b;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Load channel d of row `row` of an input tensor (fp32 or bf16).
__device__ __forceinline__ float load_in(const void* p, int64_t idx, int bf16) {
  return bf16 ? bf16_to_f32(((const uint16_t*)p)[idx]) : ((const float*)p)[idx];
}

// ------------------------------------------------------------ wave reductions
template <int W>
__device__ __forceinline__ float wmax(float v) {
#pragma unroll
  for (int o = 1; o < W; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
template <int W>
__device__ __forceinline__ float wmin(float v) {
#pragma unroll
  for (int o = 1; o < W; o <<= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wmax_n(float v, int w) {
  for (int o = 1; o < w; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wmin_n(float v, int w) {
  for (int o = 1; o < w; o <<= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ uint32_t wor_n(uint32_t v, int w) {
  for (int o = 1; o < w; o <<= 1) v |= __shfl_xor(v, o, 64);
  return v;
}

// ------------------------------------------------------------ launch blocks
struct Regions {
  uint8_t* codes[2];
  uint32_t* sz[2];      // [U][tcap][NG] packed (s | z << 16)
  uint8_t* idx[2];
  uint16_t* t16[2];     // KVARN token scale; NSN first norm n1
  uint16_t* t2[2];      // NSN second norm n2
  float* tab[2];
  float* win[2];
  float* ws;
  uint32_t* cnt;        // [U] arrival counters of the fused split-K combine
  int pat_h;            // pattern tables and windows per kv-head (= Hkv) when
                        // shared by the batch; 0 = per (batch, kv-head) unit
  int kch;              // K quantized per channel over KVQ_KBLOCK-token blocks
  uint32_t* kbsz;       // kch: [U][tcap / KBLOCK][D] packed (s | z << 16)
  uint16_t* ktail;      // kch: [U][KBLOCK][D] binary16 residuals of the open block
  uint32_t* status;     // sticky input-domain flags (KVQ_DOMAIN_*)
};

// Input domain: a lane that holds an offending element ORs its flag into the
// cache's status word (a vector atomic, issued only on a violation).
__device__ __forceinline__ bool kv_out_of_domain(float x) { return !(fabsf(x) < KVQ_KV_LIMIT); }
__device__ __forceinline__ void flag_domain(uint32_t* status, bool bad, uint32_t bit) {
  if (bad) __hip_atomic_fetch_or(status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int KBLOCK = KVQ_KBLOCK;
// K blocks per unit (token capacity rounded up to whole blocks)
__host__ __device__ inline int kch_blocks(int tcap) { return (tcap + KBLOCK - 1) / KBLOCK; }

// Pattern-table (and Chebyshev-window) unit of (batch, kv-head) unit u.
__host__ __device__ inline int64_t pat_unit(const Regions& r, int64_t u) {
  return r.pat_h ? u % r.pat_h : u;
}

// Order-preserving integer key of a binary32 value and its inverse: integer
// min / max of keys = binary32 min / max (non-NaN).  Batch-shared windows hold
// keys so that every unit folds its vectors in with one atomic each.
__device__ __forceinline__ int f32_order_key(float f) {
  const int b = __builtin_bit_cast(int, f);
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float f32_from_order_key(int k) {
  return __builtin_bit_cast(float, k ^ ((k >> 31) & 0x7FFFFFFF));
}

struct EncodeArgs {
  Regions r;
  const void* src[2];   // [U][src_rows][D]; this launch reads rows 0..n_new-1
  int src_rows;
  int n_new, t0, tcap, ngroups, group, bits, bf16, mode;
  int n_pat, max_pat;
  float rho;            // V threshold constant; < 0 disables
  int tiles_per_block;  // V code tiles handled by one block
  int win_update;       // accumulate the Chebyshev window over these tokens
  int win_close;        // this call ends a window
  int close_slot;       // table slot for the new centre, -1 = dropped
  int kch_tail_direct;  // K per channel, one token that leaves its block open:
                        // the encode stores its binary16 residual itself
};

struct AttnArgs {
  Regions r;
  const void* q;        // [B][Hq][D]
  float* out;           // [B][Hq][D]
  int B, Hq, Hkv, gq, T, tcap, ngroups, group, bits, bf16, mode;
  int n_pat, max_pat;
  int splits, chunk;    // tokens per split (multiple of 64)
  int chunk0;           // tokens of split 0 (multiple of 64; = chunk unless the
                        // fused step shortens it to offset its encode)
  float qscale;         // sm_scale * log2(e)
  // Fused one-token decode step: the block of split 0 of each unit also
  // encodes and appends the new token (position T, described by `enc`) and
  // writes its one-token softmax partial into slot `splits` (so the combine
  // merges splits + 1 partials).  The splits cover tokens [0, T).
  int fuse;
  EncodeArgs enc;
  int kclosed;          // K per channel: tokens in complete blocks (multiple of KBLOCK)
};

struct DequantArgs {
  Regions r;
  float* out;           // [U][n][D]
  int which, tok0, n, tcap, ngroups, group, bits, mode, max_pat;
  int n_closed;         // kch: tokens in complete K blocks (a multiple of KBLOCK)
};

// K per channel after an append of tokens [t0, t0 + n_new) whose indices are
// stored: quantize the complete blocks [blk0, blk1) and write the residuals of
// tokens [tail0, t0 + n_new) of the open block.  Row t - t0 of unit u's input
// is at src + (u * src_rows + t - t0) * D; residuals of tokens before t0 come
// from the open-block buffer.
struct KchArgs {
  Regions r;
  const void* src;
  int src_rows, t0, n_new, blk0, blk1, tail0, tcap, bits, bf16, max_pat;
};

// Host launchers (each returns the hipError_t of its launch).
// K per channel: the complete blocks, then (a second launch, after the first
// has read the buffer) the open block's residuals.
hipError_t launch_kch_append(const KchArgs& a, int units, hipStream_t s);
hipError_t launch_fill(float* p, float value, int64_t n, hipStream_t s);
hipError_t launch_domain_check(const void* xk, const void* xv, int64_t n, int bf16, uint32_t* status,
                               hipStream_t s);
// (lo, hi) = (+inf, -inf) for `units` windows, as binary32 or (keys != 0) as
// order keys
hipError_t launch_window_reset(float* win_k, float* win_v, int units, int keys, hipStream_t s);
// Batch-shared windows: write each window's centre fl(fl(lo + hi) * 0.5) into
// table slot `slot` (none if slot < 0) and reset the window.
hipError_t launch_window_close(const Regions& r, int units, int max_pat, int slot, hipStream_t s);
hipError_t launch_encode(const EncodeArgs& a, int units, int n_blocks_x, hipStream_t s);
hipError_t launch_dequant(const DequantArgs& a, int units, hipStream_t s);
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);
hipError_t launch_attention_combine(const AttnArgs& a, hipStream_t s);
bool mfma_attention_supported(int bits, int group, int gq);
int mfma_head_blocks(int group, int gq);
hipError_t launch_attention_mfma(const AttnArgs& a, hipStream_t s);
// k-means per (unit, kind) over `groups` * n_tok rows: row i of unit u is
// input row (i / n_tok) * group_stride + u * n_tok + i % n_tok.
hipError_t launch_kmeans_pair(const void* xk, const void* xv, int bf16, int n_tok, int groups,
                              int64_t group_stride, int k, float* tab_k, float* tab_v, int max_pat,
                              int units, uint8_t* assign, hipStream_t s);
hipError_t launch_chan_scale_pair(const void* xk, const void* xv, int bf16, int n_tok, float* sk,
                                  float* sv, int units, hipStream_t s);
hipError_t launch_chan_centre_pair(const void* xk, const void* xv, int bf16, int n_tok, float* mk,
                                   float* mv, int units, hipStream_t s);

}  // namespace kvq
