// attn_mfma_common.h -- device helpers shared by the MFMA decode-attention
// kernels: operand layouts of v_mfma_f32_16x16x32_f16 for the QK and PV
// products over packed codes, the staged-tile shapes and LDS swizzles, DPP row
// reductions and the binary16 hi/lo operand split.
#pragma once

#include "kvq_internal.h"

namespace kvq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

constexpr int TILE = 64;         // tokens per wave iteration (4 QK column blocks, 2 V tiles)

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                __builtin_bit_cast(half8, b), c, 0, 0, 0);
}

// ---- K side: lane group j owns channels 32j..32j+31 of a token (8 or 16 B).
// MFMA element i = 2p + e of reduction chunk c maps to this channel:
template <int BITS>
__device__ __forceinline__ int qk_channel(int j, int c, int i) {
  const int p = i >> 1, e = i & 1;
  return BITS == 2 ? 32 * j + 16 * (c >> 1) + 4 * (c & 1) + 8 * e + p : 32 * j + 8 * c + p + 4 * e;
}
// Codes enter the MFMA as binary16 subnormals: a field masked in place at
// bit position b of a 16-bit half is code * 2^(b - 24).  log2 of the power the
// unpacked K code carries in element i:
template <int BITS>
__device__ __forceinline__ int code_shift(int i) {
  const int p = i >> 1;
  return BITS == 2 ? 2 * p : 4 * (p & 1);
}
template <int BITS>
__device__ __forceinline__ u32x4 unpack_k(const uint32_t* w, int c) {
  u32x4 r;
  if (BITS == 2) {
    const uint32_t x = w[c >> 1] >> (8 * (c & 1));
    r[0] = x & 0x00030003u; r[1] = x & 0x000C000Cu; r[2] = x & 0x00300030u; r[3] = x & 0x00C000C0u;
  } else {
    const uint32_t x = w[c], y = x >> 8;
    r[0] = x & 0x000F000Fu; r[1] = x & 0x00F000F0u; r[2] = y & 0x000F000Fu; r[3] = y & 0x00F000F0u;
  }
  return r;
}

// The f16 dot product lines the products of a group of 8 elements up on the
// sum of their exponent fields (a subnormal counts as 2^-14) and truncates
// about 24 bits below, so a code whose leading bit sits k bits under the top
// of the 10-bit mantissa keeps only ~24 - k bits, and the error is one-signed.
// On the K side that error moves scores by a tiny fraction of one code step.
// On the V side it biases sum_t p_t s_t c_t by up to ~2^-14 of itself when
// fields sit at the bottom.  In KVarN mode that sum nearly cancels against
// sum_t p_t z_t, so the bias shows up in full after the inverse rotation:
// there (PRECISE) V fields are rotated to bit 6 or 8 (2-bit) or 2 or 6
// (4-bit) before masking, at most 4 (2-bit) or 8 (4-bit) bits under the top,
// for one rotate more per word.  Otherwise 2-bit fields take the one shift
// the byte select needs anyway as a rotate to bits 2..8 (at most 8 bits
// under the top) and 4-bit fields stay in place.
__device__ __forceinline__ uint32_t rotr32(uint32_t x, int s) {
  return __builtin_amdgcn_alignbit(x, x, (uint32_t)s);
}

// ---- V side: lane group j, element i = 2p + e -> token slot of a 32-token tile
template <int BITS>
__device__ __forceinline__ int pv_token(int j, int i) {
  const int p = i >> 1, e = i & 1;
  return BITS == 2 ? 16 * (j >> 1) + 4 * (j & 1) + p + 8 * e : 8 * j + p + 4 * e;
}
// power of two the code of token slot tau carries (slot tau & 3 = p)
template <int BITS, bool PRECISE>
__device__ __forceinline__ int pv_shift(int tau) {
  if (BITS == 2) return PRECISE ? 6 + 2 * (tau & 1) : 2 + 2 * (tau & 3);
  return PRECISE ? 2 + 4 * (tau & 1) : 4 * (tau & 1);
}
// the p*s operand carries 2^(pv_ep - shift): at most 2^4
template <int BITS, bool PRECISE>
constexpr int pv_ep() { return 4 + (BITS == 2 ? (PRECISE ? 6 : 2) : (PRECISE ? 2 : 0)); }
template <int BITS, bool PRECISE>
__device__ __forceinline__ u32x4 unpack_v(uint32_t w, int j) {
  u32x4 r;
  const int sb = 8 * (j & 1);
  if (BITS == 2 && PRECISE) {
    // byte j & 1 of each half: fields 0, 1 to bits 6, 8 (rotate left 6),
    // fields 2, 3 likewise (rotate left 2)
    const uint32_t xa = rotr32(w, (26 + sb) & 31), xb = rotr32(w, (30 + sb) & 31);
    r[0] = xa & 0x00C000C0u; r[1] = xa & 0x03000300u; r[2] = xb & 0x00C000C0u; r[3] = xb & 0x03000300u;
  } else if (BITS == 2) {
    // byte j & 1 of each half to bits 2..9
    const uint32_t x = rotr32(w, (30 + sb) & 31);
    r[0] = x & 0x000C000Cu; r[1] = x & 0x00300030u; r[2] = x & 0x00C000C0u; r[3] = x & 0x03000300u;
  } else if (PRECISE) {
    // nibbles 0, 1 to bits 2, 6 (rotate left 2); nibbles 2, 3 likewise (right 6)
    const uint32_t xa = rotr32(w, 30), xb = rotr32(w, 6);
    r[0] = xa & 0x003C003Cu; r[1] = xa & 0x03C003C0u; r[2] = xb & 0x003C003Cu; r[3] = xb & 0x03C003C0u;
  } else {
    const uint32_t y = w >> 8;
    r[0] = w & 0x000F000Fu; r[1] = w & 0x00F000F0u; r[2] = y & 0x000F000Fu; r[3] = y & 0x00F000F0u;
  }
  return r;
}

// Per-wave LDS copy of one 64-token tile, byte offsets.  Every segment is
// contiguous in the cache and 16-byte aligned, so the copy is plain 16-byte
// loads per lane.
template <int BITS, int NG, bool KVARN, bool KCH = false, bool NSNM = false>
struct TileShape {
  static constexpr int KREC = D * BITS / 8;
  static constexpr int KC = TILE * KREC;            // K codes
  // K (s, z) words: per token and group, or (K per channel) the tile's block's
  // word for each channel
  static constexpr int KS = KCH ? D * 4 : TILE * NG * 4;
  static constexpr int VC = 2 * VT * D * BITS / 8;  // two V code tiles
  static constexpr int VS = TILE * NG * 4;          // V (s, z) words
  // K idx or t16 (NSN: t16 then t2); V likewise
  static constexpr int IX = KVARN ? 2 * TILE * (NSNM ? 2 : 1) : TILE;
  static constexpr int O_KC = 0, O_KS = KC, O_VC = O_KS + KS, O_VS = O_VC + VC;
  static constexpr int O_KI = O_VS + VS, O_VI = O_KI + IX;
  static constexpr int BYTES = O_VI + IX;
  static constexpr int R_KC = KC / 16 / 64, R_VC = VC / 16 / 64;   // pieces per lane
  static constexpr int P_KS = KS / 16, P_IX = IX / 16;              // pieces (<= 64)
};

// LDS bank layout.  A wave's p tables hold one 64-token row per head; row h
// starts at 64 h + o(h) words with o(h) = 16 h (4 heads) or
// 16 (h / 2) + 4 (h % 2) (8 heads), so that the 16-word write runs of the
// heads one instruction covers, and the 4-word reads of all heads of a lane
// group, fall on distinct banks.
template <int HB>
__host__ __device__ inline int prow(int h) {
  return 64 * h + (HB == 4 ? 16 * h : 16 * (h >> 1) + 4 * (h & 1));
}
template <int HB>
constexpr int ptab_words() { return HB == 4 ? 320 : 576; }   // >= prow<HB>(HB - 1) + 64
constexpr int VS_STRIDE = TILE + 16;   // binary16 per V-scale row: rows 40 words apart
// 16-byte pieces of the staged code tiles are stored XOR-swizzled: K piece P
// of a token record at P ^ ((P / 16) mod pieces-per-token), V piece P at
// P ^ ((P / 16) mod 2), which makes the per-lane reads of 16 consecutive
// tokens (K) or channel blocks (V) conflict-free.
template <int BITS>
__device__ __forceinline__ int kpiece(int P) {
  constexpr int PPT = D * BITS / 8 / 16;
  return P ^ ((P >> 4) & (PPT - 1));
}
__device__ __forceinline__ int vpiece(int P) { return P ^ ((P >> 4) & 1); }

__host__ __device__ inline int al16(int x) { return (x + 15) & ~15; }
__host__ __device__ inline int pad_pat(int n) { return n < 4 ? 4 : (n + 3) & ~3; }

// Reductions over the 16 lanes of a DPP row (lanes 16r .. 16r+15): swap
// neighbours, swap pairs, mirror halves, mirror the row.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                0xF, 0xF, false));
}
// Max over the 16 lanes of a DPP row on an integer key that orders like the
// binary32 values (non-NaN): integer max folds into the DPP move, a float max
// would not (its operands need canonicalising).
__device__ __forceinline__ int f32_key(float f) {
  const int b = __builtin_bit_cast(int, f);
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ float row_max16(float v) {
  int k = f32_key(v);
  k = max(k, dpp_i<0xB1>(k));    // quad_perm [1,0,3,2]
  k = max(k, dpp_i<0x4E>(k));    // quad_perm [2,3,0,1]
  k = max(k, dpp_i<0x141>(k));   // row_half_mirror
  k = max(k, dpp_i<0x140>(k));   // row_mirror
  return __builtin_bit_cast(float, k ^ ((k >> 31) & 0x7FFFFFFF));
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  return v + dpp_f<0x140>(v);
}

// Two fp32 values -> packed binary16 hi parts and lo residuals, both rounded
// to nearest even (one v_cvt_pk_f16_f32 each): hi + lo keeps ~22 significant
// bits and what is left over is unbiased.  (Truncation would leave a
// one-signed remainder; summed over many tokens whose p s sits in the
// binary16 subnormal range it becomes a bias, which the KVarN inverse
// Hadamard gathers into one output channel.)
// m1 is -1 and z is +0, passed in as values the compiler cannot fold, so that
// fma(binary16, m1, a) and fma(binary16, p, z) stay single v_fma_mix
// instructions that read the binary16 operand in place.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split2(float a, float b, float m1, uint32_t& hi, uint32_t& lo) {
  const f16x2 h = __builtin_convertvector(f32x2{a, b}, f16x2);
  hi = __builtin_bit_cast(uint32_t, h);
  // a - hi is exact
  const f16x2 l = __builtin_convertvector(
      f32x2{__builtin_fmaf((float)h[0], m1, a), __builtin_fmaf((float)h[1], m1, b)}, f16x2);
  lo = __builtin_bit_cast(uint32_t, l);
}
// p * s with s in binary16 and p >= 0 (exact product rounded once)
__device__ __forceinline__ float mul_h(float p, uint16_t s, float z) {
  return __builtin_fmaf((float)__builtin_bit_cast(_Float16, s), p, z);
}

}  // namespace kvq
