// encode.hip -- decode-time encode of new K/V vectors into the packed cache.
//
// PatternKV (arXiv 2510.05176v2): nearest pattern under the min-max distance
// and residual (section 3.2, Eq 6), V threshold (section 3.3, Eq 10),
// per-group asymmetric quantization (section 2.1, Eq 1), Chebyshev-centre
// window (section 3.1, Eq 5).  KVarN-style mode (arXiv 2606.03458, abstract):
// Hadamard rotation, channel scale, token RMS scale, then the same quantizer.
//
// One wave encodes one vector; lane l holds channels l and l + 64.  All
// reductions across lanes (group min / max, the distance argmin, the range
// used by the V threshold, the OR that packs K records) are DPP row
// operations plus readlane across rows, so a vector's chain has no LDS round
// trips except for staging the vector for the distance loop.  The distance
// to the patterns uses every lane: lane = (pattern p, channel chunk s) with S
// chunks per pattern, S = 4, 2 or 1 for up to 16, 32 or 64 patterns.
//
// The per-vector code lives in encode_vec.h; two kernels here use it (and
// the attention kernel's fused one-token decode step does too):
//  * encode_kernel: one block per (V code tile of 32 tokens, unit, K|V), four
//    waves taking the tile's tokens in turn, the pattern table staged in LDS;
//    V codes are staged and written as whole 32-bit words once per tile;
//  * encode_token_kernel: one wave per (unit, K|V) for a single appended
//    token (the decode step), every load issued up front, V codes OR-ed into
//    their words (a tile's words are written whole, later positions zero,
//    when its first token is appended).
#include "encode_vec.h"

namespace kvq {

constexpr int ENC_WAVES = 4;
constexpr int ENC_THREADS = ENC_WAVES * 64;

// ---------------------------------------------------------------- bulk kernel
struct EncodeShared {
  float x[ENC_WAVES][XS];          // the vector each wave encodes, in chunks
  uint8_t vcode[VT][D];            // V codes of the tile, [token][channel]
  float wlo[ENC_WAVES][D];         // per-wave window partials
  float whi[ENC_WAVES][D];
};

// Dynamic LDS: the pass-0 pattern table, row = lane (pattern, chunk) of
// D/S + 4 floats, when one pass covers the table (sized by the host).
__host__ __device__ inline int enc_tab_floats(int mode, int n_pat) {
  if (mode != KVQ_MODE_PATTERN || n_pat <= 0 || n_pat > PAT_PASS) return 0;
  return PAT_PASS * (D / dist_chunks(n_pat) + 4);
}

__global__ void __launch_bounds__(ENC_THREADS) encode_kernel(EncodeArgs a) {
  __shared__ EncodeShared sh;
  extern __shared__ __attribute__((aligned(16))) float s_tab[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kind = blockIdx.z;
  const int64_t u = blockIdx.y;
  const int t_end = a.t0 + a.n_new;
  const int tile_first = a.t0 / VT + blockIdx.x * a.tiles_per_block;
  const int tile_last = min((t_end - 1) / VT, tile_first + a.tiles_per_block - 1);

  float wlo0 = INFINITY, wlo1 = INFINITY, whi0 = -INFINITY, whi1 = -INFINITY;
  // The pattern table in the pass-0 row layout, when one pass covers it.
  const bool staged = a.mode == KVQ_MODE_PATTERN && a.n_pat > 0 && a.n_pat <= PAT_PASS;
  if (staged) {
    const float* tab = a.r.tab[kind] + pat_unit(a.r, u) * a.max_pat * D;
    const int S = dist_chunks(a.n_pat), ch = D / S;
    for (int i = threadIdx.x; i < PAT_PASS * ch; i += ENC_THREADS) {
      const int row = i / ch, c = i % ch, j = row / S, s = row % S;
      s_tab[row * (ch + 4) + c] = j < a.n_pat ? tab[(int64_t)j * D + s * ch + c] : 0.0f;
    }
    __syncthreads();
  }

  for (int tile = tile_first; tile <= tile_last; ++tile) {
    const int tt0 = max(tile * VT, a.t0), tt1 = min(tile * VT + VT, t_end);
    // the next token's vector is loaded while this one is encoded
    float nx0 = 0.0f, nx1 = 0.0f;
    if (tt0 + wave < tt1) {
      const int64_t row = u * a.src_rows + (tt0 + wave - a.t0);
      nx0 = load_in(a.src[kind], row * D + lane, a.bf16);
      nx1 = load_in(a.src[kind], row * D + lane + 64, a.bf16);
    }
    for (int t = tt0 + wave; t < tt1; t += ENC_WAVES) {
      const int64_t row = u * a.src_rows + (t - a.t0);
      const float x0 = nx0, x1 = nx1;
      if (t + ENC_WAVES < tt1) {
        nx0 = load_in(a.src[kind], (row + ENC_WAVES) * D + lane, a.bf16);
        nx1 = load_in(a.src[kind], (row + ENC_WAVES) * D + lane + 64, a.bf16);
      }
      if (a.win_update) {
        wlo0 = fminf(wlo0, x0); wlo1 = fminf(wlo1, x1);
        whi0 = fmaxf(whi0, x0); whi1 = fmaxf(whi1, x1);
      }
      uint32_t c0, c1, w0, w1;
      int kidx;
      uint32_t t16;
      encode_vector<false>(a, kind, u, x0, x1, lane, sh.x[wave], staged ? s_tab : nullptr, row,
                           c0, c1, w0, w1, kidx, t16);
      store_token(a, kind, u, t, lane, c0, c1, w0, w1, kidx, t16);
      if (kind == 1) {
        sh.vcode[t - tile * VT][lane] = (uint8_t)c0;
        sh.vcode[t - tile * VT][lane + 64] = (uint8_t)c1;
      }
    }
    if (kind == 1) {
      // Pack the V tile: 32-bit word (wi, d) holds tokens wi*per .. +per-1
      // of channel d and sits at word index wi*D + d of the tile.  Tokens
      // before this call keep their bits; positions after it are zero.
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
          else if (t < tt0) keep |= m;
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
      float* win = a.r.win[kind] + pat_unit(a.r, u) * 2 * D;
      if (a.r.pat_h) {
        // batch-shared window: fold in with order-key atomics; closed later
        atomicMin((int*)&win[d], f32_order_key(lo));
        atomicMax((int*)&win[D + d], f32_order_key(hi));
      } else if (a.win_close) {
        lo = fminf(lo, win[d]);
        hi = fmaxf(hi, win[D + d]);
        if (a.close_slot >= 0) {
          float s = lo + hi;
          a.r.tab[kind][(u * a.max_pat + a.close_slot) * D + d] = s * 0.5f;
        }
        win[d] = INFINITY;
        win[D + d] = -INFINITY;
      } else {
        win[d] = fminf(lo, win[d]);
        win[D + d] = fmaxf(hi, win[D + d]);
      }
    }
  }
}

// ---------------------------------------------------------------- bulk, lane per token
// PATTERN-mode bulk appends (no window): one lane encodes one token's vector
// (all 128 channels in registers), so the distance, argmin, group min/max and
// packing are in-lane sequences with no cross-lane reduction, and each
// instruction serves 64 tokens.  The pattern table sits in LDS with rows of
// D + 4 floats: the distance loop reads one element for all lanes
// (broadcast), the residual gathers the chosen row per lane.
// Work: a block of LANE_WAVES waves owns LANE_SPAN consecutive tokens
// (aligned, so that no V tile is shared with another block); each wave
// takes one 64-token chunk.  Short spans give 32k tokens of one kv-head
// 128 blocks per K/V, so a batch-1 prefill fills the chip; the register
// budget is capped for three waves per SIMD (latency of the LDS reads in the
// distance loop is what the extra wave hides).
constexpr int LANE_WAVES = 4;
constexpr int LANE_SPAN = 256;
constexpr int LROW = D + 4;          // LDS table row (floats)
constexpr int LANE_MAX_PAT = 64;

__host__ __device__ inline bool lane_encode_ok(const EncodeArgs& a) {
  return a.mode == KVQ_MODE_PATTERN && !a.win_update && a.n_pat <= LANE_MAX_PAT && a.n_new > 1 &&
         (a.group == 32 || a.group == 64);
}

template <int BITS, int G>
__global__ void __launch_bounds__(LANE_WAVES * 64) __attribute__((amdgpu_waves_per_eu(3, 3)))
encode_lane_kernel(EncodeArgs a) {
  constexpr int NGL = D / G;
  constexpr int RW = D * BITS / 32;           // words of a packed record
  extern __shared__ __attribute__((aligned(16))) float s_tab[];   // [n_pat][LROW]
  // V records of a chunk's 64 tokens (row padded by one word: the lanes'
  // stores fall on distinct banks)
  __shared__ uint32_t s_vr[LANE_WAVES][64][RW + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kind = blockIdx.z;
  const int64_t u = blockIdx.y;
  const int t_end = a.t0 + a.n_new;
  const int span0 = (a.t0 / LANE_SPAN + blockIdx.x) * LANE_SPAN;
  const int s_begin = max(span0, a.t0), s_end = min(span0 + LANE_SPAN, t_end);
  const int n_pat = a.n_pat;
  {
    const float* tab = a.r.tab[kind] + pat_unit(a.r, u) * a.max_pat * D;
    for (int i = threadIdx.x; i < n_pat * D; i += LANE_WAVES * 64)
      s_tab[(i / D) * LROW + i % D] = tab[i];
  }
  __syncthreads();
  constexpr float qmax = (float)((1 << BITS) - 1);
  constexpr int per = 32 / BITS;                     // codes per 32-bit word
  for (int c0 = (s_begin / 64) * 64 + 64 * wave; c0 < s_end; c0 += 64 * LANE_WAVES) {
    const int t = c0 + lane;
    const bool valid = t >= s_begin && t < s_end;
    float x[D];
    {
      const int64_t row = u * a.src_rows + (valid ? t - a.t0 : s_begin - a.t0);
#pragma unroll
      for (int i = 0; i < D; i += 4) {
        const float4 v = load4_in(a.src[kind], row * D + i, a.bf16);
        x[i] = v.x; x[i + 1] = v.y; x[i + 2] = v.z; x[i + 3] = v.w;
      }
    }
    {
      // input domain: the largest |x| bit pattern (NaN and inf included)
      uint32_t mb = 0;
#pragma unroll
      for (int i = 0; i < D; ++i) mb = max(mb, __builtin_bit_cast(uint32_t, x[i]) & 0x7FFFFFFFu);
      flag_domain(a.r.status, valid && mb >= __builtin_bit_cast(uint32_t, KVQ_KV_LIMIT), KVQ_DOMAIN_KV);
    }
    // nearest pattern under d_mm, lowest index on ties (Eq 6)
    int kbest = KVQ_INDEX_NONE;
    float best = INFINITY;
#pragma unroll 2
    for (int jp = 0; jp < n_pat; ++jp) {
      const float* m = s_tab + jp * LROW;
      // two max and two min chains, each step a three-operand max / min
      float mxa = -INFINITY, mxb = -INFINITY, mna = INFINITY, mnb = INFINITY;
#pragma unroll
      for (int i = 0; i < D; i += 4) {
        const float4 mv = *(const float4*)(m + i);
        const float e0 = x[i] - mv.x, e1 = x[i + 1] - mv.y, e2 = x[i + 2] - mv.z, e3 = x[i + 3] - mv.w;
        mxa = fmaxf(fmaxf(mxa, e0), e1); mxb = fmaxf(fmaxf(mxb, e2), e3);
        mna = fminf(fminf(mna, e0), e1); mnb = fminf(fminf(mnb, e2), e3);
      }
      const float e = fmaxf(mxa, mxb) - fminf(mna, mnb);
      if (e < best || kbest == KVQ_INDEX_NONE) { best = e; kbest = jp; }
    }
    // V threshold (Eq 10): keep the pattern iff R_flat <= rho* R_raw
    if (kind == 1 && a.rho >= 0.0f && kbest != KVQ_INDEX_NONE) {
      float mx = x[0], mn = x[0];
#pragma unroll
      for (int i = 1; i < D; ++i) { mx = fmaxf(mx, x[i]); mn = fminf(mn, x[i]); }
      const float r_raw = mx - mn;
      if (!(best <= a.rho * r_raw)) kbest = KVQ_INDEX_NONE;
    }
    if (kbest != KVQ_INDEX_NONE) {
      const float* m = s_tab + kbest * LROW;
#pragma unroll
      for (int i = 0; i < D; i += 4) {
        const float4 mv = *(const float4*)(m + i);
        x[i] -= mv.x; x[i + 1] -= mv.y; x[i + 2] -= mv.z; x[i + 3] -= mv.w;
      }
    }
    // Eq 1 per group; codes packed into the K record layout (channel d at
    // bit bits * d of the token's record), then stored or staged (V)
    uint32_t rec[D * BITS / 32];
    uint32_t szw[NGL];
#pragma unroll
    for (int w = 0; w < D * BITS / 32; ++w) rec[w] = 0u;
#pragma unroll
    for (int g = 0; g < NGL; ++g) {
      const int i0 = g * G;
      float lo = x[i0], hi = x[i0];
#pragma unroll
      for (int i = i0 + 1; i < i0 + G; ++i) { lo = fminf(lo, x[i]); hi = fmaxf(hi, x[i]); }
      const uint16_t zb = f16_down(lo);
      const float z = bits2f(zb);
      const float sv = (hi - z) / qmax;
      const uint16_t sb = f16_up(sv);
      const float sf = bits2f(sb);
      const float inv = sf != 0.0f ? 1.0f / sf : 0.0f;
#pragma unroll
      for (int i = i0; i < i0 + G; ++i) {
        uint32_t c = 0;
        if (sf != 0.0f) {
          const float v = rintf((x[i] - z) * inv);
          c = (uint32_t)fminf(fmaxf(v, 0.0f), qmax);
        }
        rec[i / per] |= c << (BITS * (i % per));
      }
      szw[g] = (uint32_t)sb | ((uint32_t)zb << 16);
    }
    if (valid) {
      a.r.idx[kind][u * a.tcap + t] = (uint8_t)kbest;
      // K per channel keeps only the index here (its block quantizer runs later)
      uint32_t* sz_tok = a.r.sz[kind] + ((u * a.tcap) + t) * a.ngroups;
      if (!(kind == 0 && a.r.kch))
#pragma unroll
        for (int g = 0; g < NGL; ++g) sz_tok[g] = szw[g];
      if (kind == 0 && !a.r.kch) {
        uint4* out = (uint4*)(a.r.codes[0] + (u * a.tcap + t) * (D * BITS / 8));
#pragma unroll
        for (int w = 0; w < D * BITS / 32; w += 4) out[w / 4] = make_uint4(rec[w], rec[w + 1], rec[w + 2], rec[w + 3]);
      }
    }
    if (kind == 1) {
      // V tiles of this chunk (two of 32 tokens): word (wi, d) holds tokens
      // wi*per .. of channel d.  Tokens before the append keep their bits;
      // positions after it are zero.
#pragma unroll
      for (int w = 0; w < RW; ++w) s_vr[wave][lane][w] = rec[w];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      constexpr int words = D * BITS;                 // words per 32-token tile
      for (int half = 0; half < 2; ++half) {
        const int tile = c0 / VT + half, tt0 = max(tile * VT, s_begin), tt1 = min(tile * VT + VT, s_end);
        if (tt0 >= tt1) continue;
        uint32_t* tile_out = (uint32_t*)(a.r.codes[1] + ((u * (a.tcap / VT)) + tile) * (VT * D * BITS / 8));
        for (int w = lane; w < words; w += 64) {
          const int d = w % D, tok0 = (w / D) * per;
          uint32_t word = 0, keep = 0;
          for (int i = 0; i < per; ++i) {
            const int tk = tile * VT + tok0 + i;
            const uint32_t msk = ((1u << BITS) - 1u) << (i * BITS);
            if (tk >= tt0 && tk < tt1)
              word |= ((s_vr[wave][half * VT + tok0 + i][d / per] >> (BITS * (d % per))) & ((1u << BITS) - 1u))
                      << (i * BITS);
            else if (tk < tt0) keep |= msk;
          }
          if (keep) word |= tile_out[w] & keep;
          tile_out[w] = word;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

// ---------------------------------------------------------------- one token
// One wave per (unit, K|V): the token at position t0 (row 0 of the input).
// The vector, the window state and the pattern table (coalesced, up to
// PAT_PASS patterns) are loaded before anything waits; the table is then
// written to LDS in the distance loop's row layout.
constexpr int TOK_TAB4 = PAT_PASS * D / 4 / 64;   // float4 per lane for a full pass
__global__ void __launch_bounds__(64) encode_token_kernel(EncodeArgs a) {
  __shared__ float sx[XS];
  __shared__ __attribute__((aligned(16))) float stab[PAT_PASS * (D + 4)];
  const int lane = threadIdx.x;
  const int64_t u = blockIdx.x;
  const int kind = blockIdx.y;
  const int t = a.t0;
  const int64_t row = u * a.src_rows;
  const float x0 = load_in(a.src[kind], row * D + lane, a.bf16);
  const float x1 = load_in(a.src[kind], row * D + lane + 64, a.bf16);
  float* win = a.r.win[kind] + pat_unit(a.r, u) * 2 * D;
  float wl0 = 0.0f, wl1 = 0.0f, wh0 = 0.0f, wh1 = 0.0f;
  if (a.win_update && !a.r.pat_h) {
    wl0 = win[lane]; wl1 = win[lane + 64];
    wh0 = win[D + lane]; wh1 = win[D + lane + 64];
  }
  const bool staged = a.mode == KVQ_MODE_PATTERN && a.n_pat > 0 && a.n_pat <= PAT_PASS;
  if (staged) {
    const float4* tab4 = (const float4*)(a.r.tab[kind] + pat_unit(a.r, u) * a.max_pat * D);
    const int n4 = a.n_pat * D / 4;
    float4 tr[TOK_TAB4];
#pragma unroll
    for (int r = 0; r < TOK_TAB4; ++r) {
      const int f = lane + 64 * r;
      tr[r] = f < n4 ? tab4[f] : float4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const int S = dist_chunks(a.n_pat), ch = D / S;
#pragma unroll
    for (int r = 0; r < TOK_TAB4; ++r) {
      const int f = lane + 64 * r, j = f / (D / 4), c = 4 * (f % (D / 4));
      if (j < PAT_PASS / S) *(float4*)(stab + (j * S + c / ch) * (ch + 4) + c % ch) = tr[r];
    }
    // (rows of the pass past the last pattern receive the zero pieces above)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  uint32_t c0, c1, w0, w1;
  int kidx;
  uint32_t t16;
  encode_vector<true>(a, kind, u, x0, x1, lane, sx, staged ? stab : nullptr, row, c0, c1, w0, w1,
                      kidx, t16);
  token_append(a, kind, u, t, lane, x0, x1, wl0, wl1, wh0, wh1, c0, c1, w0, w1, kidx, t16);
}

hipError_t launch_encode(const EncodeArgs& a, int units, int n_blocks_x, hipStream_t s) {
  if (a.n_new == 1) {
    hipLaunchKernelGGL(encode_token_kernel, dim3(units, 2), dim3(64), 0, s, a);
    return hipGetLastError();
  }
  if (lane_encode_ok(a)) {
    const int spans = (a.t0 + a.n_new - 1) / LANE_SPAN - a.t0 / LANE_SPAN + 1;
    const dim3 grid(spans, units, 2), block(LANE_WAVES * 64);
    const size_t lds = (size_t)a.n_pat * LROW * 4;
    if (a.bits == 2 && a.group == 32) hipLaunchKernelGGL((encode_lane_kernel<2, 32>), grid, block, lds, s, a);
    else if (a.bits == 2) hipLaunchKernelGGL((encode_lane_kernel<2, 64>), grid, block, lds, s, a);
    else if (a.group == 32) hipLaunchKernelGGL((encode_lane_kernel<4, 32>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((encode_lane_kernel<4, 64>), grid, block, lds, s, a);
    return hipGetLastError();
  }
  dim3 grid(n_blocks_x, units, 2);
  const size_t lds = (size_t)enc_tab_floats(a.mode, a.n_pat) * 4;
  hipLaunchKernelGGL(encode_kernel, grid, dim3(ENC_THREADS), lds, s, a);
  return hipGetLastError();
}

}  // namespace kvq
