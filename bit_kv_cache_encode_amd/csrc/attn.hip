// attn.hip -- single-query decode attention that reads the packed cache.
//
// PatternKV (arXiv 2510.05176v2) section 3.4 fuses, for K, pattern-index
// restore + dequant + the QK product, and for V, dequant + pattern restore +
// the attention-weighted sum.  Here both are folded algebraically:
//   q . k^_i = sum_g s_ig (q_g . c_ig) + z_ig sum(q_g) + (q . M^K)[k*_i]
//   sum_i p_i v^_i = sum_i p_i (s_i c_i + z_i) + sum_j w_j M^V_j,
//   w_j = sum of p_i over tokens with k*_i = j,
// so the pattern tables are touched once per block, not once per token.
// KVarN-style caches use q' = Hadamard(q)/sqrt(D) * c_K and a per-token t:
//   q . k^_i = t_i (q' . u^_i),  sum_i p_i v^_i = Hadamard(c_V * sum_i p_i t_i u^_i)/sqrt(D).
//
// Split-K over tokens: block (split, unit) handles `chunk` tokens for all the
// q-heads that share the unit's kv-head and writes an unnormalised partial
// (running max m in log2 units, sum l, o[D]); attn_combine merges them.
#include "kvq_internal.h"

namespace kvq {

constexpr int AT_THREADS = 256;
constexpr int AT_TILE = 64;
constexpr int MAX_NG = 16;
constexpr int MAX_PAT = 256;

struct AttnShared {
  float q[MAX_GQ][D];
  float qsum[MAX_GQ][MAX_NG];
  float qm[MAX_GQ][MAX_PAT];
  float w[MAX_GQ][MAX_PAT];
  float p[MAX_GQ][AT_TILE];
  float alpha[MAX_GQ];
  float m[MAX_GQ];
  float l[MAX_GQ];
  uint32_t vsz[AT_TILE][MAX_NG];
  float tv[AT_TILE];
  uint8_t vidx[AT_TILE];
  // NSN: sm_scale * log2(e) * (q . mu_K) per head, the sums sum_t p_t n1_t,
  // each V token's n1 and the rotated V centre Hadamard(mu_V) / sqrt(D)
  float qmu[MAX_GQ];
  float s1[MAX_GQ];
  float tn1[AT_TILE];
  float muv[D];
};

__device__ __forceinline__ uint32_t code_at(const uint32_t* words, int d, int bits) {
  int bit = d * bits;
  return (words[bit >> 5] >> (bit & 31)) & ((1u << bits) - 1u);
}

__global__ void __launch_bounds__(AT_THREADS) attn_split_kernel(AttnArgs a) {
  __shared__ AttnShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x;
  const int64_t u = blockIdx.y;
  const int b = (int)(u / a.Hkv), hk = (int)(u % a.Hkv);
  const int hq0 = hk * a.gq;
  const int t_begin = split * a.chunk, t_end = min(a.T, t_begin + a.chunk);
  const bool pattern = a.mode == KVQ_MODE_PATTERN;
  const bool nsn = a.mode == KVQ_MODE_NSN;
  const int G = a.group, NG = a.ngroups, bits = a.bits;
  const int rec_words = D * bits / 32;

  // ---- prologue: scaled queries, per-group sums, q . M^K table
  for (int i = tid; i < a.gq * D; i += AT_THREADS) {
    int h = i / D, d = i % D;
    const float qv = load_in(a.q, ((int64_t)b * a.Hq + hq0 + h) * D + d, a.bf16);
    flag_domain(a.r.status, !(fabsf(qv) * a.qscale < KVQ_Q_LIMIT * 1.4426950408889634f), KVQ_DOMAIN_Q);
    sh.q[h][d] = qv;
  }
  __syncthreads();
  if (nsn) {
    // q . mu_K in the original space (the rotation is orthonormal), and the
    // V centre rotated like the V partials
    const float* muk = a.r.tab[0] + u * D;
    for (int h = tid; h < a.gq; h += AT_THREADS) {
      float s = 0.0f;
      for (int dd = 0; dd < D; ++dd) s = __builtin_fmaf(sh.q[h][dd], muk[dd], s);
      sh.qmu[h] = s * a.qscale;
    }
    if (tid < D) sh.muv[tid] = a.r.tab[1][u * D + tid];
    __syncthreads();
    for (int hstep = 1; hstep < D; hstep <<= 1) {
      float v = 0.0f;
      if (tid < D) v = (tid & hstep) ? sh.muv[tid ^ hstep] - sh.muv[tid] : sh.muv[tid] + sh.muv[tid ^ hstep];
      __syncthreads();
      if (tid < D) sh.muv[tid] = v;
      __syncthreads();
    }
    if (tid < D) sh.muv[tid] *= (float)(1.0 / __builtin_sqrt(128.0));
    __syncthreads();
  }
  if (!pattern) {
    // q' = Hadamard(q) / sqrt(D) * c_K (NSN: no channel scale)
    for (int hstep = 1; hstep < D; hstep <<= 1) {
      float v[MAX_GQ * D / AT_THREADS];
      int n = 0;
      for (int i = tid; i < a.gq * D; i += AT_THREADS, ++n) {
        int h = i / D, d = i % D;
        float mine = sh.q[h][d], other = sh.q[h][d ^ hstep];
        v[n] = (d & hstep) ? other - mine : mine + other;
      }
      __syncthreads();
      n = 0;
      for (int i = tid; i < a.gq * D; i += AT_THREADS, ++n) sh.q[i / D][i % D] = v[n];
      __syncthreads();
    }
    const float* ck = a.r.tab[0] + u * D;
    const float isd = (float)(1.0 / __builtin_sqrt(128.0));
    for (int i = tid; i < a.gq * D; i += AT_THREADS) sh.q[i / D][i % D] *= nsn ? isd : isd * ck[i % D];
    __syncthreads();
  }
  for (int i = tid; i < a.gq * D; i += AT_THREADS) sh.q[i / D][i % D] *= a.qscale;
  __syncthreads();
  for (int i = tid; i < a.gq * NG; i += AT_THREADS) {
    int h = i / NG, g = i % NG;
    float s = 0.0f;
    for (int d = g * G; d < (g + 1) * G; ++d) s += sh.q[h][d];
    sh.qsum[h][g] = s;
  }
  if (pattern) {
    const float* mk = a.r.tab[0] + pat_unit(a.r, u) * a.max_pat * D;
    for (int i = tid; i < a.gq * a.n_pat; i += AT_THREADS) {
      int h = i / a.n_pat, j = i % a.n_pat;
      float s = 0.0f;
      for (int d = 0; d < D; ++d) s = __builtin_fmaf(sh.q[h][d], mk[(int64_t)j * D + d], s);
      sh.qm[h][j] = s;
      sh.w[h][j] = 0.0f;
    }
  }
  if (tid < MAX_GQ) {
    sh.m[tid] = -INFINITY;
    sh.l[tid] = 0.0f;
    sh.s1[tid] = 0.0f;
  }
  __syncthreads();

  const int d = tid % D, hh = tid / D;      // PV: channel d, heads hh, hh+2, ...
  float acc[MAX_GQ / 2];
#pragma unroll
  for (int i = 0; i < MAX_GQ / 2; ++i) acc[i] = 0.0f;

  const uint8_t* kcodes = a.r.codes[0] + (u * a.tcap) * (D * bits / 8);
  const uint32_t* ksz = a.r.sz[0] + u * a.tcap * NG;
  const uint32_t* vsz = a.r.sz[1] + u * a.tcap * NG;

  for (int tok0 = t_begin; tok0 < t_end; tok0 += AT_TILE) {
    const int nvalid = min(AT_TILE, t_end - tok0);
    // ---- phase A: scores for (head, token) items
    for (int i = tid; i < a.gq * AT_TILE; i += AT_THREADS) {
      const int h = i / AT_TILE, j = i % AT_TILE, t = tok0 + j;
      float sc = -INFINITY;
      if (j < nvalid) {
        uint32_t rec[16];
        const uint32_t* src = (const uint32_t*)(kcodes + (int64_t)t * (D * bits / 8));
        for (int w = 0; w < rec_words; ++w) rec[w] = src[w];
        float tot = 0.0f;
        if (a.r.kch) {
          // K per channel: (s, z) of the token's block for each channel, or
          // the open block's binary16 residual
          if (t < a.kclosed) {
            const uint32_t* bsz = a.r.kbsz + (u * kch_blocks(a.tcap) + t / KBLOCK) * D;
            for (int dd = 0; dd < D; ++dd) {
              const uint32_t p = bsz[dd];
              const float kv = __builtin_fmaf((float)code_at(rec, dd, bits), bits2f((uint16_t)(p & 0xFFFF)),
                                              bits2f((uint16_t)(p >> 16)));
              tot = __builtin_fmaf(sh.q[h][dd], kv, tot);
            }
          } else {
            const uint16_t* res = a.r.ktail + (u * KBLOCK + t % KBLOCK) * D;
            for (int dd = 0; dd < D; ++dd) tot = __builtin_fmaf(sh.q[h][dd], bits2f(res[dd]), tot);
          }
        } else {
          for (int g = 0; g < NG; ++g) {
            float dot = 0.0f;
            for (int dd = g * G; dd < (g + 1) * G; ++dd)
              dot = __builtin_fmaf(sh.q[h][dd], (float)code_at(rec, dd, bits), dot);
            uint32_t p = ksz[(int64_t)t * NG + g];
            float s = bits2f((uint16_t)(p & 0xFFFF)), z = bits2f((uint16_t)(p >> 16));
            tot = __builtin_fmaf(s, dot, tot);
            tot = __builtin_fmaf(z, sh.qsum[h][g], tot);
          }
        }
        if (pattern) {
          int k = a.r.idx[0][u * a.tcap + t];
          if (k != KVQ_INDEX_NONE) tot += sh.qm[h][k];
        } else if (nsn) {
          // k^ rotated = n1 n2 (s c + z) + n1 Hadamard(mu_K) / sqrt(D)
          const float n1 = bits2f(a.r.t16[0][u * a.tcap + t]), n2 = bits2f(a.r.t2[0][u * a.tcap + t]);
          tot = __builtin_fmaf(tot, n1 * n2, n1 * sh.qmu[h]);
        } else {
          tot *= bits2f(a.r.t16[0][u * a.tcap + t]);
        }
        sc = tot;
      }
      sh.p[h][j] = sc;
    }
    if (tid < AT_TILE) {
      const int t = tok0 + tid;
      if (tid < nvalid) {
        for (int g = 0; g < NG; ++g) sh.vsz[tid][g] = vsz[(int64_t)t * NG + g];
        sh.vidx[tid] = pattern ? a.r.idx[1][u * a.tcap + t] : (uint8_t)KVQ_INDEX_NONE;
        const float t1 = pattern ? 1.0f : bits2f(a.r.t16[1][u * a.tcap + t]);
        sh.tv[tid] = nsn ? t1 * bits2f(a.r.t2[1][u * a.tcap + t]) : t1;
        sh.tn1[tid] = nsn ? t1 : 0.0f;
      } else {
        sh.tn1[tid] = 0.0f;
      }
    }
    __syncthreads();
    // ---- phase B: online softmax (log2 domain), one wave per head
    for (int h = wave; h < a.gq; h += AT_THREADS / 64) {
      float s = sh.p[h][lane];
      float mt = wmax<64>(s);
      float mold = sh.m[h];
      float mnew = fmaxf(mold, mt);
      float alpha = exp2f(mold - mnew);
      float p = exp2f(s - mnew);
      float ps = p;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) ps += __shfl_xor(ps, o, 64);
      sh.p[h][lane] = p;
      if (nsn) {
        // sum_t p_t n1_t, rescaled like l
        float p1 = p * sh.tn1[lane];
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) p1 += __shfl_xor(p1, o, 64);
        if (lane == 0) sh.s1[h] = sh.s1[h] * alpha + p1;
      }
      if (pattern) {
        for (int j = lane; j < a.n_pat; j += 64) sh.w[h][j] *= alpha;
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        if (lane < nvalid && sh.vidx[lane] != KVQ_INDEX_NONE) atomicAdd(&sh.w[h][sh.vidx[lane]], p);
      }
      if (lane == 0) {
        sh.alpha[h] = alpha;
        sh.m[h] = mnew;
        sh.l[h] = sh.l[h] * alpha + ps;
      }
    }
    __syncthreads();
    // ---- phase C: V side, thread = (channel d, head set hh)
    {
      for (int i = 0; i < MAX_GQ / 2; ++i) {
        int h = hh + 2 * i;
        if (h < a.gq) acc[i] *= sh.alpha[h];
      }
      const int g = d / G;
      for (int j = 0; j < nvalid; ++j) {
        const int t = tok0 + j;
        const int per = 32 / bits, i = t % VT;
        const uint32_t* vt = (const uint32_t*)(a.r.codes[1] + ((u * (a.tcap / VT)) + t / VT) *
                                                                  (VT * D * bits / 8));
        const uint32_t c = (vt[(i / per) * D + d] >> ((i % per) * bits)) & ((1u << bits) - 1u);
        const uint32_t p = sh.vsz[j][g];
        float vv = __builtin_fmaf((float)c, bits2f((uint16_t)(p & 0xFFFF)), bits2f((uint16_t)(p >> 16)));
        vv *= sh.tv[j];
        for (int i = 0; i < MAX_GQ / 2; ++i) {
          int h = hh + 2 * i;
          if (h < a.gq) acc[i] = __builtin_fmaf(sh.p[h][j], vv, acc[i]);
        }
      }
    }
    __syncthreads();
  }

  // ---- epilogue: V pattern term, write the partial
  const float* mv = a.r.tab[1] + pat_unit(a.r, u) * a.max_pat * D;
  for (int i = 0; i < MAX_GQ / 2; ++i) {
    int h = hh + 2 * i;
    if (h >= a.gq) continue;
    float o = acc[i];
    if (pattern)
      for (int j = 0; j < a.n_pat; ++j) o = __builtin_fmaf(sh.w[h][j], mv[(int64_t)j * D + d], o);
    if (nsn) o = __builtin_fmaf(sh.s1[h], sh.muv[d], o);
    const int64_t row = ((int64_t)b * a.Hq + hq0 + h) * a.splits + split;
    a.r.ws[row * D + d] = o;
    if (d == 0) {
      float* ml = a.r.ws + (int64_t)a.B * a.Hq * a.splits * D;
      ml[row * 2] = sh.m[h];
      ml[row * 2 + 1] = sh.l[h];
    }
  }
}

// Merge split partials: m = max m_s, l = sum l_s 2^(m_s - m),
// o = sum o_s 2^(m_s - m) / l.  KVarN-style caches then apply c_V and the
// inverse rotation.
__global__ void __launch_bounds__(D) attn_combine_kernel(AttnArgs a) {
  __shared__ float buf[D];
  const int row0 = blockIdx.x;           // b * Hq + hq
  const int d = threadIdx.x;
  const float* ml = a.r.ws + (int64_t)a.B * a.Hq * a.splits * D;
  float M = -INFINITY;
  for (int s = 0; s < a.splits; ++s) M = fmaxf(M, ml[((int64_t)row0 * a.splits + s) * 2]);
  float L = 0.0f, o = 0.0f;
  for (int s = 0; s < a.splits; ++s) {
    const int64_t row = (int64_t)row0 * a.splits + s;
    float f = exp2f(ml[row * 2] - M);
    L = __builtin_fmaf(ml[row * 2 + 1], f, L);
    o = __builtin_fmaf(a.r.ws[row * D + d], f, o);
  }
  float r = o / L;
  if (a.mode == KVQ_MODE_PATTERN) {
    a.out[(int64_t)row0 * D + d] = r;
    return;
  }
  const int b = row0 / a.Hq, hq = row0 % a.Hq;
  const int64_t u = (int64_t)b * a.Hkv + hq / a.gq;
  buf[d] = a.mode == KVQ_MODE_NSN ? r : r * a.r.tab[1][u * D + d];
  __syncthreads();
  for (int h = 1; h < D; h <<= 1) {
    float mine = buf[d], other = buf[d ^ h];
    __syncthreads();
    buf[d] = (d & h) ? other - mine : mine + other;
    __syncthreads();
  }
  a.out[(int64_t)row0 * D + d] = buf[d] * (float)(1.0 / __builtin_sqrt(128.0));
}

hipError_t launch_attention_combine(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(attn_combine_kernel, dim3(a.B * a.Hq), dim3(D), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(attn_split_kernel, dim3(a.splits, a.B * a.Hkv), dim3(AT_THREADS), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attention_combine(a, s);
}

}  // namespace kvq
