// misc.hip -- dequant readback, state fills and the prefill init kernels.
//
// Dequant: PatternKV section 3.2 (index restore after the Eq 1 inverse);
// KVarN-style inverse (channel and token scale, inverse Hadamard rotation).
// Init: PatternKV section 3.1 Eq 4 (per-head k-means over the prefill) and
// the channel axis of KVarN's dual-axis normalisation.
#include "kvq_internal.h"

namespace kvq {

// ------------------------------------------------------------ fills
__global__ void fill_kernel(float* p, float v, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill(float* p, float value, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t want = (n + 255) / 256;
  int blocks = (int)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(fill_kernel, dim3(blocks), dim3(256), 0, s, p, value, n);
  return hipGetLastError();
}

// Window state [U][2][D]: min row = +inf, max row = -inf.
__global__ void window_reset_kernel(float* wk, float* wv, int units, int keys) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= units * 2 * D) return;
  const float v = ((i / D) & 1) ? -INFINITY : INFINITY;
  const float w = keys ? __builtin_bit_cast(float, f32_order_key(v)) : v;
  wk[i] = w;
  wv[i] = w;
}

hipError_t launch_window_reset(float* wk, float* wv, int units, int keys, hipStream_t s) {
  int n = units * 2 * D;
  hipLaunchKernelGGL(window_reset_kernel, dim3((n + 255) / 256), dim3(256), 0, s, wk, wv, units,
                     keys);
  return hipGetLastError();
}

// Batch-shared Chebyshev windows (Eq 5): every unit of a kv-head has folded
// its vectors into the window's order keys; the centre of the closed window
// goes to table slot `slot` and the window starts again.  One block of D
// threads per (pattern unit, kind).
__global__ void window_close_kernel(Regions r, int max_pat, int slot) {
  const int d = threadIdx.x;
  const int64_t p = blockIdx.x;
  const int kind = blockIdx.y;
  int* win = (int*)(r.win[kind] + p * 2 * D);
  const float lo = f32_from_order_key(win[d]), hi = f32_from_order_key(win[D + d]);
  if (slot >= 0) {
    const float s = lo + hi;
    r.tab[kind][(p * max_pat + slot) * D + d] = s * 0.5f;
  }
  win[d] = f32_order_key(INFINITY);
  win[D + d] = f32_order_key(-INFINITY);
}

hipError_t launch_window_close(const Regions& r, int units, int max_pat, int slot, hipStream_t s) {
  hipLaunchKernelGGL(window_close_kernel, dim3(units, 2), dim3(D), 0, s, r, max_pat, slot);
  return hipGetLastError();
}

// ------------------------------------------------------------ dequant
__device__ __forceinline__ uint32_t read_code(const uint8_t* codes, int which, int64_t u, int t,
                                              int d, int tcap, int bits) {
  int64_t byte;
  int sh;
  if (which == 0) {
    int64_t bit = (int64_t)d * bits;
    byte = (u * tcap + t) * (D * bits / 8) + bit / 8;
    sh = (int)(bit & 7);
  } else {
    const int per = 32 / bits, i = t % VT;
    const int64_t bit = (int64_t)(i % per) * bits;
    byte = (u * (tcap / VT) + t / VT) * (VT * D * bits / 8) + ((int64_t)(i / per) * D + d) * 4 + bit / 8;
    sh = (int)(bit & 7);
  }
  return (codes[byte] >> sh) & ((1u << bits) - 1u);
}

// One wave per (token, unit); lane l holds channels l and l+64.
__global__ void __launch_bounds__(64) dequant_kernel(DequantArgs a) {
  const int lane = threadIdx.x;
  const int j = blockIdx.x, t = a.tok0 + j;
  const int64_t u = blockIdx.y;
  const int w = a.which;
  const uint32_t* sz = a.r.sz[w] + (u * a.tcap + t) * a.ngroups;
  float v[2];
  if (w == 0 && a.r.kch) {
    // K per channel: a complete block's (s, z) of the channel, or the open
    // block's binary16 residual
    const uint32_t* bsz = a.r.kbsz + (u * kch_blocks(a.tcap) + t / KBLOCK) * D;
    const uint16_t* res = a.r.ktail + (u * KBLOCK + t % KBLOCK) * D;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int d = lane + 64 * k;
      if (t < a.n_closed) {
        const uint32_t p = bsz[d];
        const float s = bits2f((uint16_t)(p & 0xFFFF)), z = bits2f((uint16_t)(p >> 16));
        v[k] = __builtin_fmaf((float)read_code(a.r.codes[0], 0, u, t, d, a.tcap, a.bits), s, z);
      } else {
        v[k] = bits2f(res[d]);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      int d = lane + 64 * k;
      uint32_t p = sz[d / a.group];
      float s = bits2f((uint16_t)(p & 0xFFFF)), z = bits2f((uint16_t)(p >> 16));
      float q = (float)read_code(a.r.codes[w], w, u, t, d, a.tcap, a.bits);
      v[k] = __builtin_fmaf(q, s, z);
    }
  }
  float* out = a.out + (u * a.n + j) * D;
  if (a.mode == KVQ_MODE_PATTERN) {
    int k = a.r.idx[w][u * a.tcap + t];
    if (k != KVQ_INDEX_NONE) {
      const float* m = a.r.tab[w] + (pat_unit(a.r, u) * a.max_pat + k) * D;
      v[0] = v[0] + m[lane];
      v[1] = v[1] + m[lane + 64];
    }
    out[lane] = v[0];
    out[lane + 64] = v[1];
    return;
  }
  if (a.mode == KVQ_MODE_NSN) {
    // NSN inverse: y = FWHT(fmaf(q, s, z)) * fp32(1/sqrt(D));
    // x^ = fl(fl(fl(y * n2) + mu) * n1)
    float x0 = v[0], x1 = v[1];
#pragma unroll
    for (int h = 1; h < 64; h <<= 1) {
      float p0 = __shfl_xor(x0, h, 64), p1 = __shfl_xor(x1, h, 64);
      if (lane & h) { x0 = p0 - x0; x1 = p1 - x1; }
      else { x0 = x0 + p0; x1 = x1 + p1; }
    }
    const float a0 = x0 + x1, a1 = x0 - x1;
    const float isd = (float)(1.0 / __builtin_sqrt(128.0));
    const float n1 = bits2f(a.r.t16[w][u * a.tcap + t]), n2 = bits2f(a.r.t2[w][u * a.tcap + t]);
    const float* mu = a.r.tab[w] + u * D;
    out[lane] = ((a0 * isd) * n2 + mu[lane]) * n1;
    out[lane + 64] = ((a1 * isd) * n2 + mu[lane + 64]) * n1;
    return;
  }
  // KVarN inverse: y^ = fl(fl(w * t) * c); x^ = FWHT(y^) * fp32(1/sqrt(D)).
  const float tf = bits2f(a.r.t16[w][u * a.tcap + t]);
  const float* c = a.r.tab[w] + u * D;
  float x0 = v[0] * tf, x1 = v[1] * tf;
  x0 = x0 * c[lane];
  x1 = x1 * c[lane + 64];
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
    float p0 = __shfl_xor(x0, h, 64), p1 = __shfl_xor(x1, h, 64);
    if (lane & h) { x0 = p0 - x0; x1 = p1 - x1; }
    else { x0 = x0 + p0; x1 = x1 + p1; }
  }
  float a0 = x0 + x1, a1 = x0 - x1;
  const float isd = (float)(1.0 / __builtin_sqrt(128.0));
  out[lane] = a0 * isd;
  out[lane + 64] = a1 * isd;
}

hipError_t launch_dequant(const DequantArgs& a, int units, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(dequant_kernel, dim3(a.n, units), dim3(64), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ K per channel
// Binary16 residual (nearest-even) of token t >= a.t0 of unit u, channel d:
// x - M_k* with the index the encode stored, or x for index NONE.
__device__ __forceinline__ uint16_t kch_residual(const KchArgs& a, int64_t u, int t, int d) {
  const float x = load_in(a.src, (u * a.src_rows + (t - a.t0)) * D + d, a.bf16);
  const int k = a.r.idx[0][u * a.tcap + t];
  if (k == KVQ_INDEX_NONE) return h2bits((_Float16)x);
  const float m = a.r.tab[0][(pat_unit(a.r, u) * a.max_pat + k) * D + d];
  return h2bits((_Float16)(x - m));
}

// OR of this lane's value and the N lanes before it within its 16-lane DPP
// row (row_shr with zeros shifted in)
template <int N>
__device__ __forceinline__ uint32_t or_shr(uint32_t v) {
  return v | (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x110 + N, 0xF, 0xF, true);
}

// One block per (unit, complete block): thread d gathers channel d's 128
// residuals (the open-block buffer before this append, recomputed from the
// input after), runs the Eq 1 quantizer down the channel (z rounded down, s
// rounded up, codes from the stored values), and for each token the 32/bits
// channels of one record word (consecutive lanes of a DPP row) OR their
// shifted codes together; the row's last lane of each word stores it.
__global__ void __launch_bounds__(KBLOCK) kch_block_kernel(KchArgs a) {
  __shared__ uint16_t s_r[KBLOCK][D];
  __shared__ int s_k[KBLOCK];              // pattern index of each token
  const int d = threadIdx.x;
  const int64_t u = blockIdx.x;
  const int blk = a.blk0 + blockIdx.y, tb = blk * KBLOCK;
  s_k[d] = a.r.idx[0][u * a.tcap + tb + d];
  __syncthreads();
  // residuals, 8 tokens' loads in flight at a time
  const float* tab = a.r.tab[0] + pat_unit(a.r, u) * a.max_pat * D + d;
  for (int i0 = 0; i0 < KBLOCK; i0 += 8) {
    float x[8], m[8];
    uint16_t old[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = tb + i0 + e, k = s_k[i0 + e];
      if (t < a.t0) {
        old[e] = a.r.ktail[(u * KBLOCK + i0 + e) * D + d];
      } else {
        x[e] = load_in(a.src, (u * a.src_rows + (t - a.t0)) * D + d, a.bf16);
        m[e] = k == KVQ_INDEX_NONE ? 0.0f : tab[(int64_t)k * D];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = tb + i0 + e, k = s_k[i0 + e];
      // x - M_k* (x alone for index NONE), binary16 nearest-even
      s_r[i0 + e][d] = t < a.t0 ? old[e] : h2bits((_Float16)(k == KVQ_INDEX_NONE ? x[e] : x[e] - m[e]));
    }
  }
  float lo = bits2f(s_r[0][d]), hi = lo;
  for (int i = 1; i < KBLOCK; ++i) {
    const float v = bits2f(s_r[i][d]);
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
  const float qmax = (float)((1 << a.bits) - 1);
  const uint16_t zb = f16_down(lo);
  const float z = bits2f(zb);
  const uint16_t sb = f16_up((hi - z) / qmax);
  const float sf = bits2f(sb);
  const float inv = sf != 0.0f ? 1.0f / sf : 0.0f;
  a.r.kbsz[(u * kch_blocks(a.tcap) + blk) * D + d] = (uint32_t)sb | ((uint32_t)zb << 16);
  const int per = 32 / a.bits;             // channels per record word: 16 or 8
  const int sh = a.bits * (d % per);
  uint32_t* rec = (uint32_t*)(a.r.codes[0] + (u * a.tcap + tb) * (D * a.bits / 8)) + d / per;
  const int rec_words = D * a.bits / 32;
  for (int i = 0; i < KBLOCK; ++i) {
    uint32_t c = 0;
    if (sf != 0.0f) {
      const float v = rintf((bits2f(s_r[i][d]) - z) * inv);
      c = (uint32_t)fminf(fmaxf(v, 0.0f), qmax);
    }
    uint32_t w = or_shr<4>(or_shr<2>(or_shr<1>(c << sh)));
    if (per == 16) w = or_shr<8>(w);
    if (d % per == per - 1) rec[i * rec_words] = w;
  }
}

// Residuals of this append's tokens in the open block, one thread per channel.
__global__ void __launch_bounds__(D) kch_tail_kernel(KchArgs a) {
  const int d = threadIdx.x;
  const int64_t u = blockIdx.x;
  for (int t = a.tail0; t < a.t0 + a.n_new; ++t)
    a.r.ktail[(u * KBLOCK + t % KBLOCK) * D + d] = kch_residual(a, u, t, d);
}

hipError_t launch_kch_append(const KchArgs& a, int units, hipStream_t s) {
  if (a.blk1 > a.blk0) {
    hipLaunchKernelGGL(kch_block_kernel, dim3(units, a.blk1 - a.blk0), dim3(KBLOCK), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.tail0 < a.t0 + a.n_new) hipLaunchKernelGGL(kch_tail_kernel, dim3(units), dim3(D), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ k-means (Eq 4)
// One block per (unit, kind).  Arithmetic mirrors the definition step by step
// in binary64: distance = sum over channels, in channel order, of diff*diff;
// strict '<' keeps the lowest index; centroid = member sum in token order
// divided by the member count; empty clusters keep their centroid.
constexpr int KM_THREADS = 256;
constexpr int KM_MAXK = 64;
constexpr int KM_ITERS = 50;

// Input row of row i of unit u's k-means rows: the unit's own prefix
// (groups = 1), or the prefixes of its kv-head in every sequence pooled
// batch-major (group stride Hkv * n_tok).
__device__ __forceinline__ int64_t km_row(int64_t u, int i, int n_tok, int64_t gstride) {
  const int g = i / n_tok;
  return g * gstride + u * n_tok + (i - g * n_tok);
}

struct KmShared {
  double cent[KM_MAXK][D];
  double sums[KM_MAXK][D];
  int cnt[KM_MAXK];
  int changed;
};

__global__ void __launch_bounds__(KM_THREADS) kmeans_kernel(const void* xk, const void* xv,
                                                             int bf16, int n_tok, int groups,
                                                             int64_t gstride, int k, float* tab_k,
                                                             float* tab_v, int max_pat,
                                                             uint8_t* assign) {
  extern __shared__ unsigned char km_raw[];
  KmShared& sh = *reinterpret_cast<KmShared*>(km_raw);
  const int kind = blockIdx.y;
  const int64_t u = blockIdx.x;
  const void* x = kind ? xv : xk;
  float* tab = (kind ? tab_v : tab_k) + u * max_pat * D;
  const int n = groups * n_tok;
  uint8_t* a = assign + ((int64_t)kind * gridDim.x + u) * n;

  for (int i = threadIdx.x; i < k * D; i += KM_THREADS) {
    int j = i / D, d = i % D;
    int64_t row = (int64_t)j * n / k;
    sh.cent[j][d] = (double)load_in(x, km_row(u, (int)row, n_tok, gstride) * D + d, bf16);
  }
  __syncthreads();
  for (int it = 0; it < KM_ITERS; ++it) {
    if (threadIdx.x == 0) sh.changed = 0;
    __syncthreads();
    int changed = 0;
    for (int t = threadIdx.x; t < n; t += KM_THREADS) {
      float xr[D];
      const int64_t xr0 = km_row(u, t, n_tok, gstride) * D;
      for (int d = 0; d < D; ++d) xr[d] = load_in(x, xr0 + d, bf16);
      int best = 0;
      double bd = INFINITY;
      for (int j = 0; j < k; ++j) {
        double dist = 0.0;
        for (int d = 0; d < D; ++d) {
          double diff = (double)xr[d] - sh.cent[j][d];
          dist = dist + diff * diff;
        }
        if (dist < bd) { bd = dist; best = j; }
      }
      if (it == 0 || a[t] != (uint8_t)best) changed = 1;
      a[t] = (uint8_t)best;
    }
    if (changed) atomicOr(&sh.changed, 1);
    __threadfence_block();
    __syncthreads();
    if (it > 0 && sh.changed == 0) break;
    // update: thread d owns column d of the sums; tokens in order
    for (int i = threadIdx.x; i < k * D; i += KM_THREADS) sh.sums[i / D][i % D] = 0.0;
    if (threadIdx.x < KM_MAXK) sh.cnt[threadIdx.x] = 0;
    __syncthreads();
    if (threadIdx.x < D) {
      const int d = threadIdx.x;
      for (int t = 0; t < n; ++t) {
        int j = a[t];
        sh.sums[j][d] = sh.sums[j][d] + (double)load_in(x, km_row(u, t, n_tok, gstride) * D + d, bf16);
        if (d == 0) sh.cnt[j] += 1;
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < k * D; i += KM_THREADS) {
      int j = i / D, d = i % D;
      if (sh.cnt[j] > 0) sh.cent[j][d] = sh.sums[j][d] / (double)sh.cnt[j];
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < k * D; i += KM_THREADS) tab[i] = (float)sh.cent[i / D][i % D];
}

// The same iteration, arithmetic and operation order with the work spread
// over a 1024-thread block, for prefixes of up to KF_MAXN tokens:
// * assignment: lane = token, 16 distance chains at a time (each still summed
//   in channel order); the centroid reads are LDS broadcasts;
// * update: members of each cluster listed in token order (per 64-token
//   chunk: ballot counts and ranks, then prefixes over chunks), then one
//   thread per (pattern, channel) sums its members in that order.
constexpr int KF_THREADS = 1024;
constexpr int KF_MAXN = 65535;          // rows (uint16 member lists)
constexpr int KF_LDS_MAX = 160 * 1024;  // a compute unit's LDS
constexpr int KF_PC = 8;    // patterns per distance pass

// 16 consecutive channels of an input row (16-byte aligned) as fp32
__device__ __forceinline__ void km_load16(const void* x, int64_t idx, int bf16, float (&o)[16]) {
  if (bf16) {
    const uint4* p = (const uint4*)((const uint16_t*)x + idx);
    const uint4 w0 = p[0], w1 = p[1];
    const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      o[2 * i] = bf16_to_f32((uint16_t)(w[i] & 0xFFFFu));
      o[2 * i + 1] = bf16_to_f32((uint16_t)(w[i] >> 16));
    }
  } else {
    const float4* p = (const float4*)((const float*)x + idx);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 f = p[i];
      o[4 * i] = f.x; o[4 * i + 1] = f.y; o[4 * i + 2] = f.z; o[4 * i + 3] = f.w;
    }
  }
}

// LDS layout of the block-parallel k-means for n rows and k patterns (bytes):
// centroids [k rounded up to KF_PC][D] binary64, then per row its assignment
// and its rank in its chunk (one byte each), the member lists (uint16), per
// chunk counts / prefixes [n/64][k] (uint16) and the cluster offsets and
// counts.  It serves any (n, k) whose total fits a compute unit's LDS.
struct KfLds { int cent, a, rank, mem, pre, off, cnt, changed, total; };
__host__ __device__ inline KfLds kf_lds(int n, int k) {
  KfLds L;
  const int kr = (k + KF_PC - 1) / KF_PC * KF_PC, nch = (n + 63) / 64;
  int o = 0;
  L.cent = o; o += kr * D * 8;
  L.a = o; o += (n + 15) / 16 * 16;
  L.rank = o; o += (n + 15) / 16 * 16;
  L.mem = o; o += (2 * n + 15) / 16 * 16;
  L.pre = o; o += (2 * nch * k + 15) / 16 * 16;
  L.off = o; o += 4 * KM_MAXK;
  L.cnt = o; o += 4 * KM_MAXK;
  L.changed = o; o += 16;
  L.total = o;
  return L;
}

__global__ void __launch_bounds__(KF_THREADS) kmeans_fast_kernel(const void* xk, const void* xv,
                                                                  int bf16, int n_tok, int groups,
                                                                  int64_t gstride, int k,
                                                                  float* tab_k, float* tab_v,
                                                                  int max_pat) {
  extern __shared__ __attribute__((aligned(16))) unsigned char km_raw[];
  const int kind = blockIdx.y;
  const int64_t u = blockIdx.x;
  const void* x = kind ? xv : xk;
  float* tab = (kind ? tab_v : tab_k) + u * max_pat * D;
  const int n = groups * n_tok;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = (n + 63) / 64;
  const int kr = (k + KF_PC - 1) / KF_PC * KF_PC;
  const KfLds Lo = kf_lds(n, k);
  double (*cent)[D] = (double (*)[D])(km_raw + Lo.cent);   // [kr][D]
  uint8_t* s_a = km_raw + Lo.a;                              // [n]
  uint8_t* s_rank = km_raw + Lo.rank;                        // [n]
  uint16_t* s_mem = (uint16_t*)(km_raw + Lo.mem);            // [n]
  uint16_t* s_pre = (uint16_t*)(km_raw + Lo.pre);            // [nch][k]
  int* s_off = (int*)(km_raw + Lo.off);
  int* s_cnt = (int*)(km_raw + Lo.cnt);
  int* s_changed = (int*)(km_raw + Lo.changed);

  for (int i = tid; i < kr * D; i += KF_THREADS) {
    const int j = i / D, d = i % D;
    cent[j][d] = j < k ? (double)load_in(x, km_row(u, (int)((int64_t)j * n / k), n_tok, gstride) * D + d, bf16)
                       : 0.0;
  }
  __syncthreads();
  for (int it = 0; it < KM_ITERS; ++it) {
    if (tid == 0) *s_changed = 0;
    __syncthreads();
    int changed = 0;
    for (int t = tid; t < n; t += KF_THREADS) {
      const int64_t row = km_row(u, t, n_tok, gstride) * D;
      int best = 0;
      double bd = INFINITY;
      for (int p0 = 0; p0 < k; p0 += KF_PC) {
        double dist[KF_PC];
#pragma unroll
        for (int q = 0; q < KF_PC; ++q) dist[q] = 0.0;
        // channels in blocks of 16; the next block's loads are in flight
        // while this one is used
        float xb[16], xn[16];
        km_load16(x, row, bf16, xb);
        for (int d0 = 0; d0 < D; d0 += 16) {
          if (d0 + 16 < D) km_load16(x, row + d0 + 16, bf16, xn);
#pragma unroll
          for (int dd = 0; dd < 16; ++dd) {
            const double xd = (double)xb[dd];
#pragma unroll
            for (int q = 0; q < KF_PC; ++q) {
              const double diff = xd - cent[p0 + q][d0 + dd];
              dist[q] = dist[q] + diff * diff;
            }
          }
#pragma unroll
          for (int dd = 0; dd < 16; ++dd) xb[dd] = xn[dd];
        }
        // strict '<' in pattern order keeps the lowest index
#pragma unroll
        for (int q = 0; q < KF_PC; ++q)
          if (p0 + q < k && dist[q] < bd) { bd = dist[q]; best = p0 + q; }
      }
      if (it == 0 || s_a[t] != (uint8_t)best) changed = 1;
      s_a[t] = (uint8_t)best;
    }
    if (changed) atomicOr(s_changed, 1);
    __syncthreads();
    if (it > 0 && *s_changed == 0) break;
    // per chunk: member counts per cluster and each token's rank among them
    for (int c = wave; c < nch; c += KF_THREADS / 64) {
      const int t = c * 64 + lane;
      const int at = t < n ? s_a[t] : -1;
      int rank = 0;
      for (int j = 0; j < k; ++j) {
        const uint64_t m = __ballot(at == j);
        if (at == j) rank = __popcll(m & ((1ull << lane) - 1ull));
        if (lane == 0) s_pre[c * k + j] = (uint16_t)__popcll(m);
      }
      if (t < n) s_rank[t] = (uint8_t)rank;
    }
    __syncthreads();
    if (tid < k) {
      int acc = 0;
      for (int c = 0; c < nch; ++c) {
        const int v = s_pre[c * k + tid];
        s_pre[c * k + tid] = (uint16_t)acc;
        acc += v;
      }
      s_cnt[tid] = acc;
    }
    __syncthreads();
    if (tid == 0) {
      int o = 0;
      for (int j = 0; j < k; ++j) { s_off[j] = o; o += s_cnt[j]; }
    }
    __syncthreads();
    for (int t = tid; t < n; t += KF_THREADS) {
      const int j = s_a[t];
      s_mem[s_off[j] + s_pre[(t >> 6) * k + j] + s_rank[t]] = (uint16_t)t;
    }
    __syncthreads();
    // centroid = member sum in token order / member count; empty keeps its centroid
    for (int i = tid; i < k * D; i += KF_THREADS) {
      const int j = i / D, d = i % D, c = s_cnt[j];
      if (c == 0) continue;
      const uint16_t* m = s_mem + s_off[j];
      // members in blocks of 8 (their loads issued together), summed in order
      double acc = 0.0;
      int e = 0;
      for (; e + 8 <= c; e += 8) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = load_in(x, km_row(u, m[e + i], n_tok, gstride) * D + d, bf16);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = acc + (double)v[i];
      }
      for (; e < c; ++e) acc = acc + (double)load_in(x, km_row(u, m[e], n_tok, gstride) * D + d, bf16);
      cent[j][d] = acc / (double)c;
    }
    __syncthreads();
  }
  for (int i = tid; i < k * D; i += KF_THREADS) tab[i] = (float)cent[i / D][i % D];
}

hipError_t launch_kmeans_pair(const void* xk, const void* xv, int bf16, int n_tok, int groups,
                              int64_t gstride, int k, float* tab_k, float* tab_v, int max_pat,
                              int units, uint8_t* assign, hipStream_t s) {
  const int64_t n = (int64_t)groups * n_tok;
  if (n <= KF_MAXN && k <= KM_MAXK && kf_lds((int)n, k).total <= KF_LDS_MAX) {
    const int lds = kf_lds((int)n, k).total;
    static int fast_attr = 0;
    if (lds > fast_attr) {
      hipError_t e = hipFuncSetAttribute((const void*)kmeans_fast_kernel,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      if (e != hipSuccess) return e;
      fast_attr = lds;
    }
    hipLaunchKernelGGL(kmeans_fast_kernel, dim3(units, 2), dim3(KF_THREADS), lds, s, xk, xv, bf16,
                       n_tok, groups, gstride, k, tab_k, tab_v, max_pat);
    return hipGetLastError();
  }
  size_t lds = sizeof(KmShared);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kmeans_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kmeans_kernel, dim3(units, 2), dim3(KM_THREADS), lds, s, xk, xv, bf16,
                     n_tok, groups, gstride, k, tab_k, tab_v, max_pat, assign);
  return hipGetLastError();
}

// ------------------------------------------------------------ KVarN channel scale
// c_j = sqrt(mean over prefix tokens of (y_j / rms(y))^2), y = FWHT(x)/sqrt(D),
// in binary64; 0 becomes 1.  One block of 128 threads per (unit, kind).
__global__ void __launch_bounds__(D) chan_scale_kernel(const void* xk, const void* xv, int bf16,
                                                       int n, float* sk, float* sv) {
  __shared__ double buf[D];
  __shared__ double red[D];
  const int kind = blockIdx.y, d = threadIdx.x;
  const int64_t u = blockIdx.x;
  const void* x = kind ? xv : xk;
  double acc = 0.0;
  int cnt = 0;
  for (int t = 0; t < n; ++t) {
    buf[d] = (double)load_in(x, (u * n + t) * D + d, bf16);
    __syncthreads();
    for (int h = 1; h < D; h <<= 1) {
      double mine = buf[d], other = buf[d ^ h];
      __syncthreads();
      buf[d] = (d & h) ? other - mine : mine + other;
      __syncthreads();
    }
    double y = buf[d] / sqrt((double)D);
    red[d] = y * y;
    __syncthreads();
    for (int h = D / 2; h >= 1; h >>= 1) {
      if (d < h) red[d] += red[d + h];
      __syncthreads();
    }
    double r = sqrt(red[0] / (double)D);
    __syncthreads();
    if (r > 0.0) {
      acc += (y / r) * (y / r);
      cnt++;
    }
  }
  float c = cnt ? (float)sqrt(acc / (double)cnt) : 1.0f;
  (kind ? sv : sk)[u * D + d] = (c == 0.0f) ? 1.0f : c;
}

hipError_t launch_chan_scale_pair(const void* xk, const void* xv, int bf16, int n_tok, float* sk,
                                  float* sv, int units, hipStream_t s) {
  hipLaunchKernelGGL(chan_scale_kernel, dim3(units, 2), dim3(D), 0, s, xk, xv, bf16, n_tok, sk, sv);
  return hipGetLastError();
}

// NSN channel centre: mu_j = mean over prefix tokens of x_j / rms(x) (tokens
// with rms 0 skipped; no tokens: 0), binary64.  One block of 128 threads per
// (unit, kind).
__global__ void __launch_bounds__(D) chan_centre_kernel(const void* xk, const void* xv, int bf16,
                                                        int n, float* mk, float* mv) {
  __shared__ double red[D];
  const int kind = blockIdx.y, d = threadIdx.x;
  const int64_t u = blockIdx.x;
  const void* x = kind ? xv : xk;
  double acc = 0.0;
  int cnt = 0;
  for (int t = 0; t < n; ++t) {
    const double v = (double)load_in(x, (u * n + t) * D + d, bf16);
    red[d] = v * v;
    __syncthreads();
    for (int h = D / 2; h >= 1; h >>= 1) {
      if (d < h) red[d] += red[d + h];
      __syncthreads();
    }
    const double r = sqrt(red[0] / (double)D);
    __syncthreads();
    if (r > 0.0) {
      acc += v / r;
      cnt++;
    }
  }
  (kind ? mv : mk)[u * D + d] = cnt ? (float)(acc / (double)cnt) : 0.0f;
}

hipError_t launch_chan_centre_pair(const void* xk, const void* xv, int bf16, int n_tok, float* mk,
                                   float* mv, int units, hipStream_t s) {
  hipLaunchKernelGGL(chan_centre_kernel, dim3(units, 2), dim3(D), 0, s, xk, xv, bf16, n_tok, mk, mv);
  return hipGetLastError();
}

}  // namespace kvq
