// attn_mfma.hip -- decode attention over the packed cache on the CDNA4 matrix
// cores (v_mfma_f32_16x16x32_f16), with the split-K combine fused into the
// last block of each (batch, kv-head) unit.
//
// Same algebra as attn.hip (PatternKV, arXiv 2510.05176v2, section 3.4:
// index restore + dequant + QK fused; dequant + index restore + weighted sum
// over V fused), arranged for the MFMA tiles:
//
//  QK:  rows = (head, group) pairs, columns = 16 tokens, reduction = channels.
//       A row (h, g) holds q_h on the channels of group g and 0 elsewhere, so
//       one 16x16 output gives every per-group partial dot q_g . c_g at once;
//       the VALU then applies s_g, z_g and the pattern term (q . M^K)[k*].
//  PV:  rows = (head, group), columns = 16 channels, reduction = 32 tokens of
//       one V code tile.  Row (h, g) carries p_h * s_g per token; a column
//       only keeps the row of its own group.  z and pattern terms are summed
//       on the side (sum p z per group; a per-head histogram of p over k*).
//
// Codes enter the MFMA as binary16 subnormals: a 2-bit (4-bit) field masked
// in place inside a 32-bit word is the integer code times 2^-24 times a power
// of 4 (16) that depends only on the field's position; the other operand
// carries the inverse power, so unpacking a pair of codes is one AND.  q and
// p*s are split into binary16 hi + lo parts (two MFMAs), so products keep
// about 22 bits; accumulation is fp32.
#include "kvq_internal.h"

namespace kvq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int MF_WAVES = 4;
constexpr int MF_THREADS = MF_WAVES * 64;
constexpr int TILE = 64;         // tokens per wave iteration (4 QK column blocks, 2 V tiles)
constexpr int EQ = 10;           // q operand carries 2^EQ
constexpr int EP = 4;            // p*s operand carries 2^EP
constexpr int MAXP = 256;

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                __builtin_bit_cast(half8, b), c, 0, 0, 0);
}

__device__ __forceinline__ void split_pack(const float* v, u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    _Float16 h0 = (_Float16)v[2 * p], h1 = (_Float16)v[2 * p + 1];
    _Float16 l0 = (_Float16)(v[2 * p] - (float)h0), l1 = (_Float16)(v[2 * p + 1] - (float)h1);
    hi[p] = (uint32_t)h2bits(h0) | ((uint32_t)h2bits(h1) << 16);
    lo[p] = (uint32_t)h2bits(l0) | ((uint32_t)h2bits(l1) << 16);
  }
}

// ---- K side: lane group j owns channels 32j..32j+31 of a token (8 or 16 B).
// MFMA element i = 2p + e of reduction chunk c maps to this channel:
template <int BITS>
__device__ __forceinline__ int qk_channel(int j, int c, int i) {
  const int p = i >> 1, e = i & 1;
  return BITS == 2 ? 32 * j + 16 * (c >> 1) + 4 * (c & 1) + 8 * e + p : 32 * j + 8 * c + p + 4 * e;
}
// log2 of the power the unpacked code carries in element i
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

// ---- V side: lane group j, element i = 2p + e -> token slot of a 32-token tile
template <int BITS>
__device__ __forceinline__ int pv_token(int j, int i) {
  const int p = i >> 1, e = i & 1;
  return BITS == 2 ? 16 * (j >> 1) + 4 * (j & 1) + p + 8 * e : 8 * j + p + 4 * e;
}
// power of two the code of token slot tau carries (slot tau & 3 = p)
template <int BITS>
__device__ __forceinline__ int pv_shift(int tau) {
  return BITS == 2 ? 2 * (tau & 3) : 4 * (tau & 1);
}
template <int BITS>
__device__ __forceinline__ u32x4 unpack_v(uint32_t w, int j) {
  u32x4 r;
  if (BITS == 2) {
    const uint32_t x = w >> (8 * (j & 1));
    r[0] = x & 0x00030003u; r[1] = x & 0x000C000Cu; r[2] = x & 0x00300030u; r[3] = x & 0x00C000C0u;
  } else {
    const uint32_t y = w >> 8;
    r[0] = w & 0x000F000Fu; r[1] = w & 0x00F000F0u; r[2] = y & 0x000F000Fu; r[3] = y & 0x00F000F0u;
  }
  return r;
}

template <int NG>
struct MfShared {
  static constexpr int HB = 16 / NG;
  float q[HB][D];                 // q' = q * sm_scale * log2(e) (KVarN: rotated, * c_K)
  float qm[HB][MAXP];             // q' . M^K_j
  float ps[MF_WAVES][HB][TILE];   // p * 2^(EP - code power) (* t_V) per wave
  _Float16 vs[MF_WAVES][NG][TILE];// V group scales s per wave
  float w[MF_WAVES][HB][MAXP];    // V pattern mass per wave
  float alpha[MF_WAVES][HB];
  float m[MF_WAVES][HB];
  float o[HB][D];                 // merged o
  float z[HB][NG];                // merged sum p z
  float l[HB];
  float wsum[HB][MAXP];
  float M[HB];
  int last;
};

template <int BITS, int NG, bool KVARN>
__global__ void __launch_bounds__(MF_THREADS) attn_mfma_kernel(AttnArgs a) {
  constexpr int G = D / NG;            // channels per group
  constexpr int HB = 16 / NG;          // heads per row block
  constexpr int CPG = 16 / NG;         // PV columns per group
  constexpr int SPL = 4 / NG;          // heads per lane in the 16x16 output
  constexpr int KREC = D * BITS / 8;   // K record bytes
  constexpr int KW = BITS;             // dwords of a lane's 32-channel K slice
  constexpr int VTB = VT * D * BITS / 8;
  extern __shared__ unsigned char mf_raw[];
  MfShared<NG>& sh = *reinterpret_cast<MfShared<NG>*>(mf_raw);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane >> 4, n16 = lane & 15;
  const int U = a.B * a.Hkv;
  const int u = blockIdx.x % U, split = blockIdx.x / U;
  const int b = u / a.Hkv, hk = u % a.Hkv, hq0 = hk * a.gq;
  const int t_begin = split * a.chunk, t_end = min(a.T, t_begin + a.chunk);
  const int T = a.T;
  const int n_pat = KVARN ? 0 : a.n_pat;

  // ---------------------------------------------------------------- prologue
  for (int i = tid; i < HB * D; i += MF_THREADS) {
    const int h = i / D, d = i % D;
    sh.q[h][d] = h < a.gq ? load_in(a.q, ((int64_t)b * a.Hq + hq0 + h) * D + d, a.bf16) : 0.0f;
    sh.o[h][d] = 0.0f;
  }
  for (int i = tid; i < MF_WAVES * HB * MAXP; i += MF_THREADS) (&sh.w[0][0][0])[i] = 0.0f;
  for (int i = tid; i < HB * MAXP; i += MF_THREADS) {
    (&sh.wsum[0][0])[i] = 0.0f;
    (&sh.qm[0][0])[i] = 0.0f;
  }
  if (tid < HB * NG) (&sh.z[0][0])[tid] = 0.0f;
  if (tid < HB) sh.l[tid] = 0.0f;
  __syncthreads();
  if (KVARN) {
    for (int hs = 1; hs < D; hs <<= 1) {
      float v[HB * D / MF_THREADS];
#pragma unroll
      for (int k = 0; k < HB * D / MF_THREADS; ++k) {
        const int i = tid + k * MF_THREADS, h = i / D, d = i % D;
        const float mine = sh.q[h][d], other = sh.q[h][d ^ hs];
        v[k] = (d & hs) ? other - mine : mine + other;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < HB * D / MF_THREADS; ++k) {
        const int i = tid + k * MF_THREADS;
        sh.q[i / D][i % D] = v[k];
      }
      __syncthreads();
    }
  }
  {
    const float isd = (float)(1.0 / __builtin_sqrt(128.0));
    const float* ck = a.r.tab[0] + (int64_t)u * D;
    for (int i = tid; i < HB * D; i += MF_THREADS) {
      const int d = i % D;
      float v = (&sh.q[0][0])[i];
      if (KVARN) v = v * isd * ck[d];
      (&sh.q[0][0])[i] = v * a.qscale;
    }
  }
  __syncthreads();
  if (!KVARN) {
    const float* mk = a.r.tab[0] + (int64_t)u * a.max_pat * D;
    for (int i = tid; i < a.gq * n_pat; i += MF_THREADS) {
      const int h = i / n_pat, jj = i % n_pat;
      float s = 0.0f;
      for (int d = 0; d < D; ++d) s = __builtin_fmaf(sh.q[h][d], mk[(int64_t)jj * D + d], s);
      sh.qm[h][jj] = s;
    }
  }
  __syncthreads();

  // QK A operands: row m = n16 -> (h, g); element i of chunk c -> channel.
  u32x4 aq_hi[4], aq_lo[4];
  {
    const int h = n16 / NG, g = n16 % NG;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ch = qk_channel<BITS>(j, c, i);
        v[i] = (ch / G == g) ? ldexpf(sh.q[h][ch], EQ - code_shift<BITS>(i)) : 0.0f;
      }
      split_pack(v, aq_hi[c], aq_lo[c]);
    }
  }
  // Per-lane constants of the QK output layout: register r <-> row
  // 4j + r = (head hq_r, group r % NG).
  float qsum[4];
  int head_r[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * j + r, h = m / NG, g = m % NG;
    head_r[r] = h;
    float s = 0.0f;
    for (int d = g * G; d < (g + 1) * G; ++d) s += sh.q[h][d];
    qsum[r] = s;
  }

  // running state per head slot (SPL heads per lane)
  float m_run[SPL], l_run[SPL], zacc[4];
#pragma unroll
  for (int s = 0; s < SPL; ++s) { m_run[s] = -INFINITY; l_run[s] = 0.0f; }
#pragma unroll
  for (int r = 0; r < 4; ++r) zacc[r] = 0.0f;
  f32x4 oacc[8];
#pragma unroll
  for (int bb = 0; bb < 8; ++bb) oacc[bb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const uint8_t* kcodes = a.r.codes[0] + (int64_t)u * a.tcap * KREC;
  const uint8_t* vcodes = a.r.codes[1] + (int64_t)u * a.tcap * KREC;
  const uint32_t* ksz = a.r.sz[0] + (int64_t)u * a.tcap * NG;
  const uint32_t* vsz = a.r.sz[1] + (int64_t)u * a.tcap * NG;
  const uint8_t* kidx = a.r.idx[0] + (int64_t)u * a.tcap;
  const uint8_t* vidx = a.r.idx[1] + (int64_t)u * a.tcap;
  const uint16_t* kt16 = a.r.t16[0] + (int64_t)u * a.tcap;
  const uint16_t* vt16 = a.r.t16[1] + (int64_t)u * a.tcap;
  float* wrow = &sh.w[wave][0][0];

  // ---------------------------------------------------------------- tiles
  for (int tile = t_begin + TILE * wave; tile < t_end; tile += TILE * MF_WAVES) {
    // ---- loads (token indices clamped into the stored range)
    uint32_t kw[4][KW];
    uint32_t kszw[4][NG], vszw[4][NG];
    int kix[4], vix[4];
    float tk[4], tv[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int tc = min(tile + 16 * nb + n16, T - 1);
      const uint32_t* kp = (const uint32_t*)(kcodes + (int64_t)tc * KREC) + j * KW;
#pragma unroll
      for (int w = 0; w < KW; ++w) kw[nb][w] = kp[w];
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        kszw[nb][g] = ksz[(int64_t)tc * NG + g];
        vszw[nb][g] = vsz[(int64_t)tc * NG + g];
      }
      if (KVARN) {
        tk[nb] = bits2f(kt16[tc]);
        tv[nb] = bits2f(vt16[tc]);
        kix[nb] = vix[nb] = KVQ_INDEX_NONE;
      } else {
        kix[nb] = kidx[tc];
        vix[nb] = vidx[tc];
        tk[nb] = tv[nb] = 1.0f;
      }
    }
    uint32_t vw[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint8_t* vt = vcodes + (int64_t)((tile >> 5) + kb) * VTB;
#pragma unroll
      for (int bb = 0; bb < 8; ++bb) {
        const int ch = G * (n16 / CPG) + CPG * bb + (n16 % CPG);
        vw[kb][bb] = BITS == 2 ? *(const uint32_t*)(vt + ch * 8 + 4 * (j >> 1))
                               : *(const uint32_t*)(vt + ch * 16 + 4 * j);
      }
    }

    // ---- QK scores: sc[nb][s] for head slot s of this lane
    float sc[4][SPL];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      f32x4 C = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x4 B = unpack_k<BITS>(kw[nb], c);
        C = mfma16(aq_hi[c], B, C);
        C = mfma16(aq_lo[c], B, C);
      }
      const bool valid = tile + 16 * nb + n16 < t_end;
#pragma unroll
      for (int s = 0; s < SPL; ++s) {
        float dot = 0.0f, zt = 0.0f;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const int r = s * NG + g;
          const uint32_t w = kszw[nb][g];
          dot = __builtin_fmaf(bits2f((uint16_t)(w & 0xFFFFu)), C[r], dot);
          zt = __builtin_fmaf(bits2f((uint16_t)(w >> 16)), qsum[r], zt);
        }
        float v = __builtin_fmaf(dot, (float)(1 << (24 - EQ)), zt);
        if (!KVARN) {
          if (kix[nb] != KVQ_INDEX_NONE) v += sh.qm[head_r[s * NG]][kix[nb]];
        } else {
          v *= tk[nb];
        }
        sc[nb][s] = valid ? v : -INFINITY;
      }
    }

    // ---- online softmax (log2 domain); rescale only when a max grows
    float mnew[SPL];
    bool grow = false;
#pragma unroll
    for (int s = 0; s < SPL; ++s) {
      float mt = fmaxf(fmaxf(sc[0][s], sc[1][s]), fmaxf(sc[2][s], sc[3][s]));
      mt = wmax<16>(mt);
      mnew[s] = fmaxf(m_run[s], mt);
      grow |= mnew[s] > m_run[s];
    }
    if (__any(grow)) {
      float al[SPL];
#pragma unroll
      for (int s = 0; s < SPL; ++s) {
        al[s] = exp2f(m_run[s] - mnew[s]);
        l_run[s] *= al[s];
        m_run[s] = mnew[s];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) zacc[r] *= al[r / NG];
#pragma unroll
      for (int bb = 0; bb < 8; ++bb)
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[bb][r] *= al[r / NG];
      if (!KVARN && n_pat > 0) {
        if (n16 == 0)
#pragma unroll
          for (int s = 0; s < SPL; ++s) sh.alpha[wave][head_r[s * NG]] = al[s];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        for (int e = lane; e < a.gq * n_pat; e += 64) {
          const int h = e / n_pat;
          wrow[h * MAXP + (e % n_pat)] *= sh.alpha[wave][h];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int t64 = 16 * nb + n16;
#pragma unroll
      for (int s = 0; s < SPL; ++s) {
        const float p = exp2f(sc[nb][s] - m_run[s]);
        l_run[s] += p;
        const int h = head_r[s * NG];
        const float pt = p * tv[nb];          // KVarN: v^ carries the token scale t
#pragma unroll
        for (int g = 0; g < NG; ++g)
          zacc[s * NG + g] = __builtin_fmaf(pt, bits2f((uint16_t)(vszw[nb][g] >> 16)), zacc[s * NG + g]);
        if (!KVARN && vix[nb] != KVQ_INDEX_NONE && p != 0.0f && h < a.gq)
          atomicAdd(&wrow[h * MAXP + vix[nb]], p);
        sh.ps[wave][h][t64] = ldexpf(pt, EP - pv_shift<BITS>(t64 & 31));
      }
      if (j < NG) sh.vs[wave][j][t64] = __builtin_bit_cast(_Float16, (uint16_t)(vszw[nb][j] & 0xFFFFu));
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- PV over the two 32-token V tiles of this iteration
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      u32x4 ahi, alo;
      {
        const int h = n16 / NG, g = n16 % NG;
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int t64 = 32 * kb + pv_token<BITS>(j, i);
          v[i] = h < a.gq ? sh.ps[wave][h][t64] * (float)sh.vs[wave][g][t64] : 0.0f;
        }
        split_pack(v, ahi, alo);
      }
#pragma unroll
      for (int bb = 0; bb < 8; ++bb) {
        const u32x4 B = unpack_v<BITS>(vw[kb][bb], j);
        oacc[bb] = mfma16(ahi, B, oacc[bb]);
        oacc[bb] = mfma16(alo, B, oacc[bb]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---------------------------------------------------------------- merge waves
#pragma unroll
  for (int s = 0; s < SPL; ++s) {
    l_run[s] = l_run[s] + __shfl_xor(l_run[s], 1, 64);
    l_run[s] = l_run[s] + __shfl_xor(l_run[s], 2, 64);
    l_run[s] = l_run[s] + __shfl_xor(l_run[s], 4, 64);
    l_run[s] = l_run[s] + __shfl_xor(l_run[s], 8, 64);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) zacc[r] += __shfl_xor(zacc[r], o, 64);
  if (n16 == 0)
#pragma unroll
    for (int s = 0; s < SPL; ++s) sh.m[wave][head_r[s * NG]] = m_run[s];
  __syncthreads();
  if (tid < HB) {
    float M = -INFINITY;
    for (int w = 0; w < MF_WAVES; ++w) M = fmaxf(M, sh.m[w][tid]);
    sh.M[tid] = M;
  }
  __syncthreads();
  float f[SPL];
#pragma unroll
  for (int s = 0; s < SPL; ++s) {
    const int h = head_r[s * NG];
    f[s] = (m_run[s] == -INFINITY) ? 0.0f : exp2f(m_run[s] - sh.M[h]);
  }
  if (n16 == 0) {
#pragma unroll
    for (int s = 0; s < SPL; ++s) {
      const int h = head_r[s * NG];
      atomicAdd(&sh.l[h], f[s] * l_run[s]);
#pragma unroll
      for (int g = 0; g < NG; ++g) atomicAdd(&sh.z[h][g], f[s] * zacc[s * NG + g]);
    }
  }
  {
    const float oscale = (float)(1 << (24 - EP));
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) {
      const int ch = G * (n16 / CPG) + CPG * bb + (n16 % CPG);
      const int gcol = n16 / CPG;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r % NG != gcol) continue;
        const int s = r / NG, h = head_r[r];
        if (h < a.gq) atomicAdd(&sh.o[h][ch], oacc[bb][r] * oscale * f[s]);
      }
    }
  }
  if (!KVARN && n_pat > 0) {
    // per-wave pattern mass scaled by that wave's factor for each head
    if (n16 == 0)
#pragma unroll
      for (int s = 0; s < SPL; ++s) sh.alpha[wave][head_r[s * NG]] = f[s];
    __syncthreads();
    for (int e = tid; e < a.gq * n_pat; e += MF_THREADS) {
      const int h = e / n_pat, jj = e % n_pat;
      float acc = 0.0f;
      for (int w = 0; w < MF_WAVES; ++w) acc = __builtin_fmaf(sh.alpha[w][h], sh.w[w][h][jj], acc);
      sh.wsum[h][jj] = acc;
    }
  }
  __syncthreads();

  // ---------------------------------------------------------------- partial out
  const int S = a.splits;
  float* ml = a.r.ws + (int64_t)a.B * a.Hq * S * D;
  const float* mv = a.r.tab[1] + (int64_t)u * a.max_pat * D;
  for (int i = tid; i < a.gq * D; i += MF_THREADS) {
    const int h = i / D, d = i % D;
    float o = sh.o[h][d] + sh.z[h][d / G];
    if (!KVARN)
      for (int jj = 0; jj < n_pat; ++jj) o = __builtin_fmaf(sh.wsum[h][jj], mv[(int64_t)jj * D + d], o);
    const int64_t row = ((int64_t)b * a.Hq + hq0 + h) * S + split;
    a.r.ws[row * D + d] = o;
    if (d == 0) {
      ml[row * 2] = sh.M[h];
      ml[row * 2 + 1] = sh.l[h];
    }
  }
  // ---------------------------------------------------------------- fused combine
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&a.r.cnt[u], 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    sh.last = prev == (uint32_t)(S - 1);
  }
  __syncthreads();
  if (!sh.last) return;
  __threadfence();
  for (int i = tid; i < a.gq * D; i += MF_THREADS) {
    const int h = i / D, d = i % D;
    const int64_t row0 = ((int64_t)b * a.Hq + hq0 + h) * S;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, ml[(row0 + s) * 2]);
    float L = 0.0f, o = 0.0f;
    for (int s = 0; s < S; ++s) {
      const float fs = exp2f(ml[(row0 + s) * 2] - M);
      L = __builtin_fmaf(ml[(row0 + s) * 2 + 1], fs, L);
      o = __builtin_fmaf(a.r.ws[(row0 + s) * D + d], fs, o);
    }
    const float r = o / L;
    if (!KVARN) a.out[((int64_t)b * a.Hq + hq0 + h) * D + d] = r;
    else sh.o[h][d] = r * a.r.tab[1][(int64_t)u * D + d];
  }
  if (KVARN) {
    __syncthreads();
    for (int hs = 1; hs < D; hs <<= 1) {
      float v[HB * D / MF_THREADS];
#pragma unroll
      for (int k = 0; k < HB * D / MF_THREADS; ++k) {
        const int i = tid + k * MF_THREADS, h = i / D, d = i % D;
        const float mine = sh.o[h][d], other = sh.o[h][d ^ hs];
        v[k] = (d & hs) ? other - mine : mine + other;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < HB * D / MF_THREADS; ++k) {
        const int i = tid + k * MF_THREADS;
        sh.o[i / D][i % D] = v[k];
      }
      __syncthreads();
    }
    const float isd = (float)(1.0 / __builtin_sqrt(128.0));
    for (int i = tid; i < a.gq * D; i += MF_THREADS) {
      const int h = i / D, d = i % D;
      a.out[((int64_t)b * a.Hq + hq0 + h) * D + d] = sh.o[h][d] * isd;
    }
  }
  if (tid == 0) a.r.cnt[u] = 0;   // ready for the next call (stream-ordered)
}

template <int BITS, int NG, bool KVARN>
static hipError_t launch_one(const AttnArgs& a, hipStream_t s) {
  const size_t lds = sizeof(MfShared<NG>);
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_mfma_kernel<BITS, NG, KVARN>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL((attn_mfma_kernel<BITS, NG, KVARN>), dim3(a.B * a.Hkv * a.splits),
                     dim3(MF_THREADS), lds, s, a);
  return hipGetLastError();
}

bool mfma_attention_supported(int bits, int group, int gq) {
  if (bits != 2 && bits != 4) return false;
  if (group == 32) return gq <= 4;
  if (group == 64) return gq <= 8;
  return false;
}

hipError_t launch_attention_mfma(const AttnArgs& a, hipStream_t s) {
  const bool kv = a.mode == KVQ_MODE_KVARN;
  if (a.group == 32) {
    if (a.bits == 2) return kv ? launch_one<2, 4, true>(a, s) : launch_one<2, 4, false>(a, s);
    return kv ? launch_one<4, 4, true>(a, s) : launch_one<4, 4, false>(a, s);
  }
  if (a.bits == 2) return kv ? launch_one<2, 2, true>(a, s) : launch_one<2, 2, false>(a, s);
  return kv ? launch_one<4, 2, true>(a, s) : launch_one<4, 2, false>(a, s);
}

}  // namespace kvq
