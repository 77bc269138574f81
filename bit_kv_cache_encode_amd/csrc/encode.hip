// encode.hip -- decode-time encode of new K/V vectors into the packed cache.
//
// PatternKV (arXiv 2510.05176v2): nearest pattern under the min-max distance
// and residual (section 3.2, Eq 6), V threshold (section 3.3, Eq 10),
// per-group asymmetric quantization (section 2.1, Eq 1), Chebyshev-centre
// window (section 3.1, Eq 5).  KVarN-style mode (arXiv 2606.03458, abstract):
// Hadamard rotation, channel scale, token RMS scale, then the same quantizer.
//
// Work split: one block per (V code tile of 32 tokens, unit, K|V).  Its four
// waves encode the tile's new tokens one vector per wave; lane l holds
// channels l and l+64.  Pattern distances use a lane-per-pattern mapping over
// an LDS copy of the table.  K records (token-major) are written directly;
// V codes are staged in LDS and written word by word once per tile, merging
// with the bits of tokens outside this call at the tile's edges.
#include "kvq_internal.h"

namespace kvq {

constexpr int ENC_WAVES = 4;
constexpr int ENC_THREADS = ENC_WAVES * 64;
constexpr int PAT_LDS = 64;   // patterns staged in LDS per pass

struct EncodeShared {
  float pat[D / 4][PAT_LDS][4];    // pattern block, [channel/4][pattern][4]
  float x[ENC_WAVES][D];           // the vector each wave encodes
  uint8_t vcode[VT][D];            // V codes of the tile, [token][channel]
  float wlo[ENC_WAVES][D];         // per-wave window partials
  float whi[ENC_WAVES][D];
};

// Quantize the two channels a lane holds (group of channel l and of l+64)
// with Eq 1 per group; returns codes and writes the packed (s, z) words.
__device__ __forceinline__ void quantize_pair(float r0, float r1, int lane, int group, int bits,
                                              uint32_t* sz_tok, uint32_t& c0, uint32_t& c1) {
  const float qmax = (float)((1 << bits) - 1);
  float lo0, hi0, lo1, hi1;
  if (group <= 64) {
    lo0 = wmin_n(r0, group); hi0 = wmax_n(r0, group);
    lo1 = wmin_n(r1, group); hi1 = wmax_n(r1, group);
  } else {  // group of 128: both halves together
    lo0 = lo1 = wmin<64>(fminf(r0, r1));
    hi0 = hi1 = wmax<64>(fmaxf(r0, r1));
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
  int ch0 = lane, ch1 = lane + 64;
  if (ch0 % group == 0) sz_tok[ch0 / group] = (uint32_t)sb0 | ((uint32_t)zb0 << 16);
  if (ch1 % group == 0) sz_tok[ch1 / group] = (uint32_t)sb1 | ((uint32_t)zb1 << 16);
}

// Write one token's K codes (token-major record): code of channel d at bit
// bits*d.  Lanes OR their shifted codes into 32-bit words.
__device__ __forceinline__ void store_k_record(uint8_t* rec, int lane, int bits, uint32_t c0,
                                               uint32_t c1) {
  const int per = 32 / bits;                 // channels per 32-bit word
  uint32_t w0 = c0 << (bits * (lane % per));
  uint32_t w1 = c1 << (bits * (lane % per));
  w0 = wor_n(w0, per);
  w1 = wor_n(w1, per);
  if (lane % per == 0) {
    uint32_t* out = (uint32_t*)rec;
    out[lane / per] = w0;
    out[(lane + 64) / per] = w1;
  }
}

__global__ void __launch_bounds__(ENC_THREADS) encode_kernel(EncodeArgs a) {
  __shared__ EncodeShared sh;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kind = blockIdx.z;
  const int64_t u = blockIdx.y;
  const int t_end = a.t0 + a.n_new;
  const int tile_first = a.t0 / VT + blockIdx.x * a.tiles_per_block;
  const int tile_last = min((t_end - 1) / VT, tile_first + a.tiles_per_block - 1);
  const float* tab = a.r.tab[kind] + (a.mode == KVQ_MODE_PATTERN ? u * a.max_pat * D : u * D);
  const int use_thr = (kind == 1) && (a.rho >= 0.0f);

  float wlo0 = INFINITY, wlo1 = INFINITY, whi0 = -INFINITY, whi1 = -INFINITY;
  // Pattern table resident in LDS when it fits in one pass.
  const bool one_pass = a.mode == KVQ_MODE_PATTERN && a.n_pat <= PAT_LDS;
  if (one_pass) {
    for (int i = threadIdx.x; i < a.n_pat * D; i += ENC_THREADS) {
      int j = i / D, d = i % D;
      sh.pat[d / 4][j][d % 4] = tab[(int64_t)j * D + d];
    }
    __syncthreads();
  }

  for (int tile = tile_first; tile <= tile_last; ++tile) {
    const int tt0 = max(tile * VT, a.t0), tt1 = min(tile * VT + VT, t_end);
    for (int t = tt0 + wave; t < tt1; t += ENC_WAVES) {
      const int64_t row = u * a.src_rows + (t - a.t0);
      float x0 = load_in(a.src[kind], row * D + lane, a.bf16);
      float x1 = load_in(a.src[kind], row * D + lane + 64, a.bf16);
      if (a.win_update) {
        wlo0 = fminf(wlo0, x0); wlo1 = fminf(wlo1, x1);
        whi0 = fmaxf(whi0, x0); whi1 = fmaxf(whi1, x1);
      }
      uint32_t* sz_tok = a.r.sz[kind] + ((u * a.tcap) + t) * a.ngroups;
      uint32_t c0, c1;
      if (a.mode == KVQ_MODE_PATTERN) {
        // ---- Eq 6: nearest pattern under d_mm, lane-per-pattern.
        sh.x[wave][lane] = x0;
        sh.x[wave][lane + 64] = x1;
        __builtin_amdgcn_wave_barrier();
        float best = INFINITY;
        int kbest = KVQ_INDEX_NONE;
        for (int j0 = 0; j0 < a.n_pat; j0 += 64) {
          const int j = j0 + lane;
          float e = INFINITY;
          if (j < a.n_pat) {
            float mx = -INFINITY, mn = INFINITY;
            if (one_pass) {
              for (int d4 = 0; d4 < D / 4; ++d4) {
                const float4 xv = *(const float4*)&sh.x[wave][d4 * 4];
                const float4 mv = *(const float4*)&sh.pat[d4][j][0];
                float e0 = xv.x - mv.x, e1 = xv.y - mv.y, e2 = xv.z - mv.z, e3 = xv.w - mv.w;
                mx = fmaxf(mx, fmaxf(e0, e1)); mx = fmaxf(mx, fmaxf(e2, e3));
                mn = fminf(mn, fminf(e0, e1)); mn = fminf(mn, fminf(e2, e3));
              }
            } else {
              const float* m = tab + (int64_t)j * D;
              for (int d4 = 0; d4 < D / 4; ++d4) {
                const float4 xv = *(const float4*)&sh.x[wave][d4 * 4];
                const float4 mv = *(const float4*)&m[d4 * 4];
                float e0 = xv.x - mv.x, e1 = xv.y - mv.y, e2 = xv.z - mv.z, e3 = xv.w - mv.w;
                mx = fmaxf(mx, fmaxf(e0, e1)); mx = fmaxf(mx, fmaxf(e2, e3));
                mn = fminf(mn, fminf(e0, e1)); mn = fminf(mn, fminf(e2, e3));
              }
            }
            e = mx - mn;
          }
          // argmin over lanes, lowest index on ties
          int jj = (j < a.n_pat) ? j : 0x7FFFFFFF;
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            float eo = __shfl_xor(e, o, 64);
            int jo = __shfl_xor(jj, o, 64);
            if (eo < e || (eo == e && jo < jj)) { e = eo; jj = jo; }
          }
          if (jj != 0x7FFFFFFF && (e < best || kbest == KVQ_INDEX_NONE)) { best = e; kbest = jj; }
        }
        __builtin_amdgcn_wave_barrier();
        // ---- section 3.3: V keeps its pattern iff R_flat <= rho* R_raw.
        if (use_thr && kbest != KVQ_INDEX_NONE) {
          float mx = wmax<64>(fmaxf(x0, x1)), mn = wmin<64>(fminf(x0, x1));
          float r_raw = mx - mn;
          float lim = a.rho * r_raw;
          if (!(best <= lim)) kbest = KVQ_INDEX_NONE;
        }
        float r0 = x0, r1 = x1;
        if (kbest != KVQ_INDEX_NONE) {
          const float* m = tab + (int64_t)kbest * D;
          r0 = x0 - m[lane];
          r1 = x1 - m[lane + 64];
        }
        if (lane == 0) a.r.idx[kind][u * a.tcap + t] = (uint8_t)kbest;
        quantize_pair(r0, r1, lane, a.group, a.bits, sz_tok, c0, c1);
      } else {
        // ---- KVarN reading: FWHT (stages h = 1..64), 1/sqrt(D), channel
        // scale, token RMS (halving-fold sum), then Eq 1 on u = y~ / t.
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
        if (lane == 0) a.r.t16[kind][u * a.tcap + t] = tb;
        float u0 = 0.0f, u1 = 0.0f;
        if (tf != 0.0f) {
          float it = 1.0f / tf;
          u0 = x0 * it;
          u1 = x1 * it;
        }
        quantize_pair(u0, u1, lane, a.group, a.bits, sz_tok, c0, c1);
      }
      if (kind == 0) {
        store_k_record(a.r.codes[0] + (u * a.tcap + t) * (D * a.bits / 8), lane, a.bits, c0, c1);
      } else {
        sh.vcode[t - tile * VT][lane] = (uint8_t)c0;
        sh.vcode[t - tile * VT][lane + 64] = (uint8_t)c1;
      }
    }
    if (kind == 1) {
      // Pack the V tile: 32-bit word (wi, d) holds tokens wi*per .. +per-1
      // of channel d and sits at word index wi*D + d of the tile.
      __syncthreads();
      const int per = 32 / a.bits;                    // tokens per word
      const int words = D * a.bits;                   // words per tile (VT*D*bits/32)
      uint32_t* tile_out = (uint32_t*)(a.r.codes[1] + ((u * (a.tcap / VT)) + tile) * (VT * D * a.bits / 8));
      for (int w = threadIdx.x; w < words; w += ENC_THREADS) {
        const int d = w % D, tok0 = (w / D) * per;
        uint32_t word = 0, keep = 0;
        for (int i = 0; i < per; ++i) {
          const int t = tile * VT + tok0 + i;
          const uint32_t m = ((1u << a.bits) - 1u) << (i * a.bits);
          if (t >= tt0 && t < tt1) word |= ((uint32_t)sh.vcode[tok0 + i][d] << (i * a.bits));
          else keep |= m;
        }
        if (keep) word |= tile_out[w] & keep;
        tile_out[w] = word;
      }
      __syncthreads();
    }
  }

  if (a.win_update) {
    // Chebyshev window (Eq 5): fold this block's min/max into the state; on
    // the window's last token append fl(fl(lo + hi) * 0.5) as a new pattern.
    sh.wlo[wave][lane] = wlo0; sh.wlo[wave][lane + 64] = wlo1;
    sh.whi[wave][lane] = whi0; sh.whi[wave][lane + 64] = whi1;
    __syncthreads();
    if (threadIdx.x < D) {
      const int d = threadIdx.x;
      float lo = sh.wlo[0][d], hi = sh.whi[0][d];
      for (int w = 1; w < ENC_WAVES; ++w) { lo = fminf(lo, sh.wlo[w][d]); hi = fmaxf(hi, sh.whi[w][d]); }
      float* win = a.r.win[kind] + u * 2 * D;
      lo = fminf(lo, win[d]);
      hi = fmaxf(hi, win[D + d]);
      if (a.win_close) {
        if (a.close_slot >= 0) {
          float s = lo + hi;
          a.r.tab[kind][(u * a.max_pat + a.close_slot) * D + d] = s * 0.5f;
        }
        win[d] = INFINITY;
        win[D + d] = -INFINITY;
      } else {
        win[d] = lo;
        win[D + d] = hi;
      }
    }
  }
}

hipError_t launch_encode(const EncodeArgs& a, int units, int n_blocks_x, hipStream_t s) {
  dim3 grid(n_blocks_x, units, 2);
  hipLaunchKernelGGL(encode_kernel, grid, dim3(ENC_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
