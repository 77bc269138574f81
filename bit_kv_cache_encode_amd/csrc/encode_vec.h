// encode_vec.h -- per-vector encode device code shared by the encode kernels
// and the fused one-token decode step of the attention kernel.
//
// PatternKV (arXiv 2510.05176v2): nearest pattern under the min-max distance
// and residual (section 3.2, Eq 6), V threshold (section 3.3, Eq 10),
// per-group asymmetric quantization (section 2.1, Eq 1), Chebyshev-centre
// window (section 3.1, Eq 5).  KVarN-style mode (arXiv 2606.03458, abstract):
// Hadamard rotation, channel scale, token RMS scale, then the same quantizer.
//
// One wave encodes one vector; lane l holds channels l and l + 64.
#pragma once
#include "kvq_internal.h"

namespace kvq {

constexpr int PAT_PASS = 64;       // patterns per distance pass (one per lane at S = 1)
constexpr int XS = D + 16;         // staged vector: S chunks of D/S (+4 pad) floats

// ---------------------------------------------------------------- DPP reductions
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_fl(float v) {
  return __builtin_bit_cast(float, dpp_u<CTRL>(__builtin_bit_cast(uint32_t, v)));
}
__device__ __forceinline__ float rlane(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ uint32_t rlane_u(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

// Every lane receives the min (MAX = false) or max over its aligned group of
// W lanes, W in {1, 2, 4, ..., 64}.  Exact: min / max do not round.
template <bool MAX>
__device__ __forceinline__ float fmm(float a, float b) { return MAX ? fmaxf(a, b) : fminf(a, b); }
template <bool MAX>
__device__ __forceinline__ float group_mm(float v, int W, int lane) {
  if (W >= 2) v = fmm<MAX>(v, dpp_fl<0xB1>(v));    // quad_perm [1,0,3,2]
  if (W >= 4) v = fmm<MAX>(v, dpp_fl<0x4E>(v));    // quad_perm [2,3,0,1]
  if (W >= 8) v = fmm<MAX>(v, dpp_fl<0x141>(v));   // row_half_mirror
  if (W >= 16) v = fmm<MAX>(v, dpp_fl<0x140>(v));  // row_mirror
  if (W >= 32) {
    const float lo = fmm<MAX>(rlane(v, 0), rlane(v, 16));
    const float hi = fmm<MAX>(rlane(v, 32), rlane(v, 48));
    v = W >= 64 ? fmm<MAX>(lo, hi) : ((lane & 32) ? hi : lo);
  }
  return v;
}
__device__ __forceinline__ uint32_t wave_min_u(uint32_t v) {
  v = min(v, dpp_u<0xB1>(v));
  v = min(v, dpp_u<0x4E>(v));
  v = min(v, dpp_u<0x141>(v));
  v = min(v, dpp_u<0x140>(v));
  return min(min(rlane_u(v, 0), rlane_u(v, 16)), min(rlane_u(v, 32), rlane_u(v, 48)));
}
// OR over aligned groups of W <= 32 lanes
__device__ __forceinline__ uint32_t group_or(uint32_t v, int W) {
  if (W >= 2) v |= dpp_u<0xB1>(v);
  if (W >= 4) v |= dpp_u<0x4E>(v);
  if (W >= 8) v |= dpp_u<0x141>(v);
  if (W >= 16) v |= dpp_u<0x140>(v);
  if (W >= 32) v |= (uint32_t)__shfl_xor((int)v, 16, 64);
  return v;
}

// Root mean square of the 128 channels a wave holds (lane l: channels l and
// l + 64) by the halving-fold sum of squares: v[i] += v[i + 64], then + 32,
// ..., + 1; sqrtf(fl(ss * (1/128))).  Every lane gets it.
__device__ __forceinline__ float rms_fold(float x0, float x1, int lane) {
  float v = x0 * x0;
  const float v1 = x1 * x1;
  v = v + v1;
#pragma unroll
  for (int h = 32; h >= 1; h >>= 1) {
    const float o = __shfl_down(v, h, 64);
    if (lane < h) v = v + o;
  }
  return sqrtf(__shfl(v, 0, 64) * (1.0f / 128.0f));
}

// ---------------------------------------------------------------- Eq 1 quantizer
// Quantize the two channels a lane holds (group of channel l and of l + 64);
// returns the codes and the packed (s | z << 16) words of the lane's groups.
__device__ __forceinline__ void quantize_pair(float r0, float r1, int lane, int group, int bits,
                                              uint32_t& c0, uint32_t& c1, uint32_t& w0,
                                              uint32_t& w1) {
  const float qmax = (float)((1 << bits) - 1);
  float lo0, hi0, lo1, hi1;
  if (group <= 64) {
    lo0 = group_mm<false>(r0, group, lane); hi0 = group_mm<true>(r0, group, lane);
    lo1 = group_mm<false>(r1, group, lane); hi1 = group_mm<true>(r1, group, lane);
  } else {  // group of 128: both halves together
    lo0 = lo1 = group_mm<false>(fminf(r0, r1), 64, lane);
    hi0 = hi1 = group_mm<true>(fmaxf(r0, r1), 64, lane);
  }
  uint16_t zb0 = f16_down(lo0), zb1 = f16_down(lo1);
  float z0 = bits2f(zb0), z1 = bits2f(zb1);
  float s0 = (hi0 - z0) / qmax, s1 = (hi1 - z1) / qmax;
  uint16_t sb0 = f16_up(s0), sb1 = f16_up(s1);
  float sf0 = bits2f(sb0), sf1 = bits2f(sb1);
  c0 = 0;
  c1 = 0;
  if (sf0 != 0.0f) {
    float inv = 1.0f / sf0;
    float v = rintf((r0 - z0) * inv);
    c0 = (uint32_t)fminf(fmaxf(v, 0.0f), qmax);
  }
  if (sf1 != 0.0f) {
    float inv = 1.0f / sf1;
    float v = rintf((r1 - z1) * inv);
    c1 = (uint32_t)fminf(fmaxf(v, 0.0f), qmax);
  }
  w0 = (uint32_t)sb0 | ((uint32_t)zb0 << 16);
  w1 = (uint32_t)sb1 | ((uint32_t)zb1 << 16);
}

// ---------------------------------------------------------------- Eq 6 distance
// Chunks per pattern for n patterns in one pass.
__host__ __device__ inline int dist_chunks(int n) { return n <= 16 ? 4 : (n <= 32 ? 2 : 1); }

// Staged vector (per wave): chunk s of D/S channels at s * (D/S + 4).
__device__ __forceinline__ void stage_x(float* sx, float x0, float x1, int lane, int S) {
  const int ch = D / S;
  sx[(lane / ch) * (ch + 4) + lane % ch] = x0;
  sx[((lane + 64) / ch) * (ch + 4) + (lane + 64) % ch] = x1;
}

// d_mm(x, M_j) for the pattern j = j0 + lane / S of this lane's pass, reading
// chunk s = lane % S; `row` is the start of that pattern chunk (LDS or global).
// FULL unrolls the chunk loop so that every load is in flight at once (the
// global table of the one-token kernel); the LDS table of the bulk kernel
// takes four chunks per step to keep registers for more waves.
template <int S, bool FULL>
__device__ __forceinline__ float dist_chunk(const float* sx, const float* row, int lane) {
  constexpr int ch = D / S;
  const int s = lane % S;
  const float* xs = sx + s * (ch + 4);
  float mx = -INFINITY, mn = INFINITY;
  constexpr int UNR = FULL ? ch / 4 : 4;
#pragma unroll UNR
  for (int i = 0; i < ch; i += 4) {
    const float4 xv = *(const float4*)(xs + i);
    const float4 mv = *(const float4*)(row + i);
    const float e0 = xv.x - mv.x, e1 = xv.y - mv.y, e2 = xv.z - mv.z, e3 = xv.w - mv.w;
    mx = fmaxf(mx, fmaxf(e0, e1)); mx = fmaxf(mx, fmaxf(e2, e3));
    mn = fminf(mn, fminf(e0, e1)); mn = fminf(mn, fminf(e2, e3));
  }
  // combine the S chunks of the pattern (adjacent lanes)
  if (S >= 2) { mx = fmaxf(mx, dpp_fl<0xB1>(mx)); mn = fminf(mn, dpp_fl<0xB1>(mn)); }
  if (S >= 4) { mx = fmaxf(mx, dpp_fl<0x4E>(mx)); mn = fminf(mn, dpp_fl<0x4E>(mn)); }
  return mx - mn;
}

// Nearest pattern (lowest index on ties) of the staged vector; `best` = its
// distance.  tab_lds: the unit's table in pass-0 row layout (row = lane, D/S
// + 4 floats), used when n_pat <= PAT_PASS; otherwise the global table.
template <int S, bool FULL>
__device__ __forceinline__ int nearest_pattern_s(const float* sx, const float* tab_lds,
                                                 const float* tab, int n_pat, int lane, float& best) {
  int kbest = KVQ_INDEX_NONE;
  best = INFINITY;
  constexpr int ch = D / S;
  for (int j0 = 0; j0 < n_pat; j0 += PAT_PASS / S) {
    // every lane runs the chunk loop (the DPP combines read neighbours);
    // lanes past the last pattern read pattern 0 (or a zero LDS row) and are
    // masked afterwards
    const int j = j0 + lane / S;
    const int jr = j < n_pat ? j : 0;
    const float* row = tab_lds ? tab_lds + lane * (ch + 4) : tab + (int64_t)jr * D + (lane % S) * ch;
    float e = dist_chunk<S, FULL>(sx, row, lane);
    if (j >= n_pat) e = INFINITY;
    const float emin = group_mm<false>(e, 64, lane);
    const uint32_t jmin = wave_min_u(e == emin && j < n_pat ? (uint32_t)j : 0xFFFFFFFFu);
    if (jmin != 0xFFFFFFFFu && (emin < best || kbest == KVQ_INDEX_NONE)) {
      best = emin;
      kbest = (int)jmin;
    }
  }
  return kbest;
}
template <bool FULL>
__device__ __forceinline__ int nearest_pattern(const float* sx, const float* tab_lds,
                                               const float* tab, int n_pat, int lane, float& best) {
  const int S = dist_chunks(n_pat);
  if (S == 4) return nearest_pattern_s<4, FULL>(sx, tab_lds, tab, n_pat, lane, best);
  if (S == 2) return nearest_pattern_s<2, FULL>(sx, tab_lds, tab, n_pat, lane, best);
  return nearest_pattern_s<1, FULL>(sx, tab_lds, tab, n_pat, lane, best);
}

// Four consecutive channels of an input row as fp32.
__device__ __forceinline__ float4 load4_in(const void* p, int64_t idx, int bf16) {
  if (bf16) {
    const uint2 w = *(const uint2*)((const uint16_t*)p + idx);
    return float4{bf16_to_f32((uint16_t)(w.x & 0xFFFFu)), bf16_to_f32((uint16_t)(w.x >> 16)),
                  bf16_to_f32((uint16_t)(w.y & 0xFFFFu)), bf16_to_f32((uint16_t)(w.y >> 16))};
  }
  return *(const float4*)((const float*)p + idx);
}

// Encode one vector (PATTERN or KVARN) held as x0 = x[lane], x1 = x[lane + 64];
// returns the codes and the lane's (s, z) words; `kidx` = pattern index and
// `t16` = token scale.  `sx` is this wave's staging area; `sres` (PATTERN)
// receives the chosen pattern row for the residual when tab_lds is null.
// FULL: fully unrolled distance loop (the one-token kernel).
template <bool FULL>
__device__ __forceinline__ void encode_vector(const EncodeArgs& a, int kind, int64_t u, float x0,
                                              float x1, int lane, float* sx, const float* tab_lds,
                                              int64_t row, uint32_t& c0, uint32_t& c1,
                                              uint32_t& w0, uint32_t& w1, int& kidx,
                                              uint32_t& t16) {
  const float* tab = a.r.tab[kind] + (a.mode == KVQ_MODE_PATTERN ? pat_unit(a.r, u) * a.max_pat * D : u * D);
  flag_domain(a.r.status, kv_out_of_domain(x0) || kv_out_of_domain(x1), KVQ_DOMAIN_KV);
  kidx = KVQ_INDEX_NONE;
  t16 = 0;
  if (a.mode == KVQ_MODE_PATTERN) {
    float r0 = x0, r1 = x1;
    if (a.n_pat > 0) {
      const int S = dist_chunks(a.n_pat);
      float best;
      int kbest;
      stage_x(sx, x0, x1, lane, S);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      kbest = nearest_pattern<FULL>(sx, tab_lds, tab, a.n_pat, lane, best);
      // section 3.3: V keeps its pattern iff R_flat <= rho* R_raw
      if (kind == 1 && a.rho >= 0.0f && kbest != KVQ_INDEX_NONE) {
        const float mx = group_mm<true>(fmaxf(x0, x1), 64, lane);
        const float mn = group_mm<false>(fminf(x0, x1), 64, lane);
        const float r_raw = mx - mn;
        const float lim = a.rho * r_raw;
        if (!(best <= lim)) kbest = KVQ_INDEX_NONE;
      }
      if (kbest != KVQ_INDEX_NONE) {
        float m0, m1;
        if (tab_lds) {
          const int ch = D / S;
          const float* base = tab_lds + (kbest * S) * (ch + 4);
          m0 = base[(lane / ch) * (ch + 4) + lane % ch];
          m1 = base[((lane + 64) / ch) * (ch + 4) + (lane + 64) % ch];
        } else {
          m0 = tab[(int64_t)kbest * D + lane];
          m1 = tab[(int64_t)kbest * D + lane + 64];
        }
        r0 = x0 - m0;
        r1 = x1 - m1;
      }
      kidx = kbest;
      // the staged vector is rewritten by the wave's next token
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if (kind == 0 && a.kch_tail_direct) {
      // K per channel: the residual waits in binary16 (nearest-even) for its block
      uint16_t* slot = a.r.ktail + (u * KBLOCK + a.t0 % KBLOCK) * D;
      slot[lane] = h2bits((_Float16)r0);
      slot[lane + 64] = h2bits((_Float16)r1);
    }
    quantize_pair(r0, r1, lane, a.group, a.bits, c0, c1, w0, w1);
  } else if (a.mode == KVQ_MODE_NSN) {
    // NSN reading: n1 = rms(x), b = x * fl(1/n1) - mu, n2 = rms(b),
    // y = FWHT(b * fl(1/n2)) * fp32(1/sqrt(D)), Eq 1 on y; t16 carries
    // n1 | n2 << 16 (binary16, nearest-even)
    const uint16_t n1b = h2bits((_Float16)rms_fold(x0, x1, lane));
    const float n1 = bits2f(n1b);
    float b0 = 0.0f, b1 = 0.0f;
    uint16_t n2b = 0;
    if (n1 != 0.0f) {
      const float i1 = 1.0f / n1;
      b0 = x0 * i1 - tab[lane];
      b1 = x1 * i1 - tab[lane + 64];
      n2b = h2bits((_Float16)rms_fold(b0, b1, lane));
    }
    const float n2 = bits2f(n2b);
    float y0 = 0.0f, y1 = 0.0f;
    if (n1 != 0.0f && n2 != 0.0f) {
      const float i2 = 1.0f / n2;
      y0 = b0 * i2;
      y1 = b1 * i2;
#pragma unroll
      for (int h = 1; h < 64; h <<= 1) {
        const float p0 = __shfl_xor(y0, h, 64), p1 = __shfl_xor(y1, h, 64);
        if (lane & h) { y0 = p0 - y0; y1 = p1 - y1; }
        else { y0 = y0 + p0; y1 = y1 + p1; }
      }
      const float a0 = y0 + y1, a1 = y0 - y1;   // stage h = 64 (in-lane)
      const float isd = (float)(1.0 / __builtin_sqrt(128.0));
      y0 = a0 * isd;
      y1 = a1 * isd;
    }
    t16 = (uint32_t)n1b | ((uint32_t)n2b << 16);
    quantize_pair(y0, y1, lane, a.group, a.bits, c0, c1, w0, w1);
  } else {
    // KVarN reading: FWHT (stages h = 1..64), 1/sqrt(D), channel scale,
    // token RMS (halving-fold sum), then Eq 1 on u = y~ / t.
#pragma unroll
    for (int h = 1; h < 64; h <<= 1) {
      float p0 = __shfl_xor(x0, h, 64), p1 = __shfl_xor(x1, h, 64);
      if (lane & h) { x0 = p0 - x0; x1 = p1 - x1; }
      else { x0 = x0 + p0; x1 = x1 + p1; }
    }
    {
      float a0 = x0 + x1, a1 = x0 - x1;   // stage h = 64 (in-lane)
      x0 = a0; x1 = a1;
    }
    const float isd = (float)(1.0 / __builtin_sqrt(128.0));   // fp32(1/sqrt(128))
    x0 = x0 * isd;
    x1 = x1 * isd;
    const float ic0 = 1.0f / tab[lane], ic1 = 1.0f / tab[lane + 64];
    x0 = x0 * ic0;
    x1 = x1 * ic1;
    float v = x0 * x0;
    float v1 = x1 * x1;
    v = v + v1;                                         // fold h = 64
#pragma unroll
    for (int h = 32; h >= 1; h >>= 1) {
      float o = __shfl_down(v, h, 64);
      if (lane < h) v = v + o;
    }
    float ss = __shfl(v, 0, 64);
    float tt = sqrtf(ss * (1.0f / 128.0f));
    uint16_t tb = h2bits((_Float16)tt);
    float tf = bits2f(tb);
    t16 = tb;
    float u0 = 0.0f, u1 = 0.0f;
    if (tf != 0.0f) {
      float it = 1.0f / tf;
      u0 = x0 * it;
      u1 = x1 * it;
    }
    quantize_pair(u0, u1, lane, a.group, a.bits, c0, c1, w0, w1);
  }
}

// Store a token's (s, z) words, index / token scale and (K) packed record.
__device__ __forceinline__ void store_token(const EncodeArgs& a, int kind, int64_t u, int t,
                                            int lane, uint32_t c0, uint32_t c1, uint32_t w0,
                                            uint32_t w1, int kidx, uint32_t t16) {
  if (lane == 0) {
    if (a.mode == KVQ_MODE_PATTERN) a.r.idx[kind][u * a.tcap + t] = (uint8_t)kidx;
    else a.r.t16[kind][u * a.tcap + t] = (uint16_t)t16;
    if (a.mode == KVQ_MODE_NSN) a.r.t2[kind][u * a.tcap + t] = (uint16_t)(t16 >> 16);
  }
  // K per channel keeps only the index here; its block quantizer runs later
  if (kind == 0 && a.r.kch) return;
  uint32_t* sz_tok = a.r.sz[kind] + ((u * a.tcap) + t) * a.ngroups;
  if (lane % a.group == 0) sz_tok[lane / a.group] = w0;
  if ((lane + 64) % a.group == 0 && a.group <= 64) sz_tok[(lane + 64) / a.group] = w1;
  if (kind == 0) {
    // token-major record: channel d's code at bit bits*d; lanes OR their
    // shifted codes into 32-bit words
    const int per = 32 / a.bits;
    const uint32_t s0 = group_or(c0 << (a.bits * (lane % per)), per);
    const uint32_t s1 = group_or(c1 << (a.bits * (lane % per)), per);
    if (lane % per == 0) {
      uint32_t* out = (uint32_t*)(a.r.codes[0] + (u * a.tcap + t) * (D * a.bits / 8));
      out[lane / per] = s0;
      out[(lane + 64) / per] = s1;
    }
  }
}

// Store one appended token (position t) of kind K (0) or V (1): record, (s, z)
// words and index, the V code words of its 32-token tile (written whole, later
// positions zero, at the tile's first token; OR-ed in afterwards), and the
// Chebyshev window update (Eq 5) with the window's (lo, hi) state as loaded.
// A batch-shared window is folded into with atomic min / max of order keys
// instead; its closure is a separate launch once every unit has folded in.
// own_window: this caller updates (and closes) the Chebyshev window; another
// caller appending the same token (identical record writes) leaves it alone
__device__ __forceinline__ void token_append(const EncodeArgs& a, int kind, int64_t u, int t,
                                             int lane, float x0, float x1, float wl0, float wl1,
                                             float wh0, float wh1, uint32_t c0, uint32_t c1,
                                             uint32_t w0, uint32_t w1, int kidx, uint32_t t16,
                                             bool own_window = true) {
  float* win = a.r.win[kind] + pat_unit(a.r, u) * 2 * D;
  store_token(a, kind, u, t, lane, c0, c1, w0, w1, kidx, t16);
  if (kind == 1) {
    // V word of channel d holding token t: whole tile written on its first
    // token (other positions zero), OR-ed in afterwards
    const int per = 32 / a.bits, tt = t % VT, wi = tt / per, bit = (tt % per) * a.bits;
    uint32_t* tile_out = (uint32_t*)(a.r.codes[1] + ((u * (a.tcap / VT)) + t / VT) * (VT * D * a.bits / 8));
    if (tt == 0) {
      for (int w = 0; w < a.bits; ++w) {
        tile_out[w * D + lane] = w == wi ? c0 << bit : 0u;
        tile_out[w * D + lane + 64] = w == wi ? c1 << bit : 0u;
      }
    } else {
      if (c0) atomicOr(&tile_out[wi * D + lane], c0 << bit);
      if (c1) atomicOr(&tile_out[wi * D + lane + 64], c1 << bit);
    }
  }
  if (a.win_update && own_window && a.r.pat_h) {
    int* wk = (int*)win;
    atomicMin(&wk[lane], f32_order_key(x0));
    atomicMin(&wk[lane + 64], f32_order_key(x1));
    atomicMax(&wk[D + lane], f32_order_key(x0));
    atomicMax(&wk[D + lane + 64], f32_order_key(x1));
  } else if (a.win_update && own_window) {
    // Chebyshev window (Eq 5) over this token
    const float lo0 = fminf(wl0, x0), lo1 = fminf(wl1, x1);
    const float hi0 = fmaxf(wh0, x0), hi1 = fmaxf(wh1, x1);
    if (a.win_close) {
      if (a.close_slot >= 0) {
        float* dst = a.r.tab[kind] + (pat_unit(a.r, u) * a.max_pat + a.close_slot) * D;
        const float s0 = lo0 + hi0, s1 = lo1 + hi1;
        dst[lane] = s0 * 0.5f;
        dst[lane + 64] = s1 * 0.5f;
      }
      win[lane] = INFINITY; win[lane + 64] = INFINITY;
      win[D + lane] = -INFINITY; win[D + lane + 64] = -INFINITY;
    } else {
      win[lane] = lo0; win[lane + 64] = lo1;
      win[D + lane] = hi0; win[D + lane + 64] = hi1;
    }
  }
}

}  // namespace kvq
