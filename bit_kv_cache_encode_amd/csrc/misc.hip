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

// Input-domain check of a pair of inputs (k and v, n elements each) for the
// init calls, whose mining kernels read them several times: any element
// outside |x| < KVQ_KV_LIMIT (or not finite) sets KVQ_DOMAIN_KV.
__global__ void domain_check_kernel(const void* xk, const void* xv, int64_t n, int bf16,
                                    uint32_t* status) {
  bool bad = false;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    bad |= kv_out_of_domain(load_in(xk, i, bf16)) || kv_out_of_domain(load_in(xv, i, bf16));
  flag_domain(status, bad, KVQ_DOMAIN_KV);
}

hipError_t launch_domain_check(const void* xk, const void* xv, int64_t n, int bf16, uint32_t* status,
                               hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t want = (n + 255) / 256;
  int blocks = (int)(want < 2048 ? want : 2048);
  hipLaunchKernelGGL(domain_check_kernel, dim3(blocks), dim3(256), 0, s, xk, xv, n, bf16, status);
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
__device__ __forceinline__ int64_t km_row(int64_t u, int i, int n_tok, int64_t gstride, int groups) {
  if (groups == 1) return u * n_tok + i;
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
    sh.cent[j][d] = (double)load_in(x, km_row(u, (int)row, n_tok, gstride, groups) * D + d, bf16);
  }
  __syncthreads();
  for (int it = 0; it < KM_ITERS; ++it) {
    if (threadIdx.x == 0) sh.changed = 0;
    __syncthreads();
    int changed = 0;
    for (int t = threadIdx.x; t < n; t += KM_THREADS) {
      float xr[D];
      const int64_t xr0 = km_row(u, t, n_tok, gstride, groups) * D;
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
        sh.sums[j][d] = sh.sums[j][d] + (double)load_in(x, km_row(u, t, n_tok, gstride, groups) * D + d, bf16);
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
// centroids [k rounded up to KF_PC][D] binary64; their binary32 copies for
// the matrix cores [k rounded up to 16][KF_CSTRIDE] with binary64 squared
// norms and binary32 norms; then per row its assignment and its rank in its
// chunk (one byte each), the member lists (uint16), per chunk counts /
// prefixes [n/64][k] (uint16) and the cluster offsets and counts.  The list
// of rows whose nearest centroid the matrix-core distances leave open
// (uint16) shares the rank and member-list bytes, which serve only the
// update.  It serves any (n, k) whose total fits a compute unit's LDS.
constexpr int KF_CSTRIDE = D + 4;   // floats per binary32 centroid row (bank shift)
// bfloat16 input: two bfloat16 parts of each binary32 centroid, [2][k16][KB_STRIDE]
// (a 16-byte shift per row keeps the 16-byte operand reads conflict-free)
constexpr int KB_STRIDE = D + 8;
constexpr int KF_CBYTES = (2 * KB_STRIDE * 2 > KF_CSTRIDE * 4) ? 2 * KB_STRIDE * 2 : KF_CSTRIDE * 4;
struct KfLds { int cent, c32, cc, cn, a, rank, mem, pre, off, cnt, changed, namb, total; };
__host__ __device__ inline KfLds kf_lds(int n, int k) {
  KfLds L;
  const int kr = (k + KF_PC - 1) / KF_PC * KF_PC, k16 = (k + 15) / 16 * 16, nch = (n + 63) / 64;
  int o = 0;
  L.cent = o; o += kr * D * 8;
  L.c32 = o; o += k16 * KF_CBYTES;
  L.cc = o; o += k16 * 8;
  L.cn = o; o += (k16 * 4 + 15) / 16 * 16;
  L.a = o; o += (n + 15) / 16 * 16;
  L.rank = o; o += (n + 15) / 16 * 16;
  L.mem = o; o += (2 * n + 15) / 16 * 16;
  L.pre = o; o += (2 * nch * k + 15) / 16 * 16;
  L.off = o; o += 4 * KM_MAXK;
  L.cnt = o; o += 4 * KM_MAXK;
  L.changed = o; o += 16;
  L.namb = o; o += 16;
  L.total = o;
  return L;
}

// 32 consecutive channels of an input row (16-byte aligned) as fp32
__device__ __forceinline__ void km_load32(const void* x, int64_t idx, int bf16, float (&o)[32]) {
  float a[16], b[16];
  km_load16(x, idx, bf16, a);
  km_load16(x, idx + 16, bf16, b);
#pragma unroll
  for (int i = 0; i < 16; ++i) { o[i] = a[i]; o[16 + i] = b[i]; }
}

// minimum over the 16 lanes of a DPP row (lanes 16r .. 16r+15) on an
// integer key that orders like the binary32 values (no NaN): swap
// neighbours, swap pairs, mirror halves, mirror the row
__device__ __forceinline__ float km_rowmin16(float v) {
  const int b = __builtin_bit_cast(int, v);
  int key = b ^ ((b >> 31) & 0x7FFFFFFF);
  key = min(key, __builtin_amdgcn_update_dpp(key, key, 0xB1, 0xF, 0xF, true));
  key = min(key, __builtin_amdgcn_update_dpp(key, key, 0x4E, 0xF, 0xF, true));
  key = min(key, __builtin_amdgcn_update_dpp(key, key, 0x141, 0xF, 0xF, true));
  key = min(key, __builtin_amdgcn_update_dpp(key, key, 0x140, 0xF, 0xF, true));
  return __builtin_bit_cast(float, key ^ ((key >> 31) & 0x7FFFFFFF));
}

typedef float km_f32x4 __attribute__((ext_vector_type(4)));

// binary32 -> bfloat16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t km_bf16_rne(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

typedef __bf16 km_bf16x8 __attribute__((ext_vector_type(8)));

// NCB: column blocks of 16 patterns in the matrix-core distances (k <= 16 NCB)
// BF: bfloat16 input rows, whose products with the centroids run on the
// bfloat16 matrix cores (see the assignment)
template <int NCB, bool BF>
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
  float* s_c32 = (float*)(km_raw + Lo.c32);                  // [k16][KF_CSTRIDE]
  double* s_cc = (double*)(km_raw + Lo.cc);                  // [k16] |c|^2
  float* s_cn = (float*)(km_raw + Lo.cn);                    // [k16] |c| rounded up
  int* s_namb = (int*)(km_raw + Lo.namb);
  uint8_t* s_a = km_raw + Lo.a;                              // [n]
  uint8_t* s_rank = km_raw + Lo.rank;                        // [n]
  uint16_t* s_mem = (uint16_t*)(km_raw + Lo.mem);            // [n]
  uint16_t* s_pre = (uint16_t*)(km_raw + Lo.pre);            // [nch][k]
  int* s_off = (int*)(km_raw + Lo.off);
  int* s_cnt = (int*)(km_raw + Lo.cnt);
  int* s_changed = (int*)(km_raw + Lo.changed);
  uint16_t* s_amb = (uint16_t*)(km_raw + Lo.rank);           // [n], assignment only
  const int k16 = (k + 15) / 16 * 16;

  for (int i = tid; i < kr * D; i += KF_THREADS) {
    const int j = i / D, d = i % D;
    cent[j][d] = j < k ? (double)load_in(x, km_row(u, (int)((int64_t)j * n / k), n_tok, gstride, groups) * D + d, bf16)
                       : 0.0;
  }
  // bfloat16 rows: are binary64 member sums exact in any order?  Every value
  // is an integer multiple of 2^(e_min - 7), e_min the smallest exponent of
  // a nonzero value (subnormals count as -126), and a sum of at most n
  // values is below n 2^(e_max + 1).  With e_max - e_min + ceil(log2 n) <=
  // 45 every partial sum, in whatever order, is a multiple of 2^(e_min - 7)
  // below 2^(e_min + 46): exactly representable in binary64, so every
  // addition is exact and any order gives the exact sum, which the
  // token-order sum also is.  The update then spreads a cluster's members
  // over several threads.
  bool exact_sums = false;
  if constexpr (BF) {
    int* s_fr = s_namb + 1;   // [min, max] exponent field of the nonzero values
    if (tid == 0) { s_fr[0] = 255; s_fr[1] = 0; }
    __syncthreads();
    int fmn = 255, fmx = 0;
    for (int i = tid; i < n * (D / 8); i += KF_THREADS) {
      const int r = i / (D / 8), c8 = i % (D / 8);
      const uint4 w = *(const uint4*)((const uint16_t*)x + km_row(u, r, n_tok, gstride, groups) * D + 8 * c8);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        const uint32_t a = (ws[h >> 1] >> (16 * (h & 1))) & 0x7FFFu;
        const int f = (int)(a >> 7);
        if (a) { fmn = min(fmn, max(f, 1)); fmx = max(fmx, f); }
      }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      fmn = min(fmn, __shfl_xor(fmn, o, 64));
      fmx = max(fmx, __shfl_xor(fmx, o, 64));
    }
    if (lane == 0) { atomicMin(&s_fr[0], fmn); atomicMax(&s_fr[1], fmx); }
    __syncthreads();
    int lg = 0;
    while ((1 << lg) < n) ++lg;
    exact_sums = s_fr[1] < 255 && (s_fr[1] == 0 || s_fr[1] - s_fr[0] + lg <= 45);
  }
  __syncthreads();
  for (int it = 0; it < KM_ITERS; ++it) {
    // ---- assignment (Eq 4's nearest centroid, Euclidean).  The matrix cores
    // give every row's binary32 dot products with binary32 copies of the
    // centroids, so each distance |x|^2 + |c|^2 - 2 x.c (binary64) is known
    // to within E = 2 (D + 3) 2^-24 |x| |c| (the dot over D channels in
    // binary32 from the rounded centroid) plus a small binary64 term.  A row
    // whose intervals leave one centroid below every other takes it: the
    // binary64 distances of the other centroids exceed its own, so a plain
    // binary64 nearest-centroid scan picks it too.  Any other row is listed
    // and its distances are recomputed in binary64 in channel order.
    if constexpr (BF) {
      // c = (binary32) centroid = c1 + c2 + r: c1 = bf16(c), c2 = bf16(c - c1)
      // (c - c1 is exact: the two are within a factor of two), |r| <= 2^-18 |c|
      uint16_t* s_cb = (uint16_t*)s_c32;
      for (int i = tid; i < k16 * D; i += KF_THREADS) {
        const int j = i / D, d = i % D;
        const float c = j < k ? (float)cent[j][d] : 0.0f;
        const uint32_t h1 = km_bf16_rne(c);
        const uint32_t h2 = km_bf16_rne(c - __builtin_bit_cast(float, h1 << 16));
        s_cb[j * KB_STRIDE + d] = (uint16_t)h1;
        s_cb[(k16 + j) * KB_STRIDE + d] = (uint16_t)h2;
      }
    } else {
      for (int i = tid; i < k16 * D; i += KF_THREADS) {
        const int j = i / D, d = i % D;
        s_c32[j * KF_CSTRIDE + d] = j < k ? (float)cent[j][d] : 0.0f;
      }
    }
    if (tid < k16) {
      double acc = 0.0;
      if (tid < k)
        for (int d = 0; d < D; ++d) acc = __builtin_fma(cent[tid][d], cent[tid][d], acc);
      s_cc[tid] = acc;
      s_cn[tid] = (float)(__builtin_sqrt(acc) * (1.0 + 0x1p-40));   // |c| rounded up
    }
    if (tid == 0) { *s_changed = 0; *s_namb = 0; }
    __syncthreads();
    int changed = 0;
    if constexpr (BF) {
      // bfloat16 rows are exact operands.  Products x . c1 and x . c2 are
      // exact in the matrix cores; their sums over 2 x 128 channels carry at
      // most a few binary32 roundings (or truncations below the largest
      // product) of partial sums bounded by sum |x_d| |c_d| <= |x| |c|: the
      // bound takes 2^-13 |x| |c|, far above that, plus 2^-18 |x| |c| for
      // the part r the two bfloat16 parts leave out and 2^-24 |x| |c| for
      // the binary32 centroid.  The distance |x|^2 + |c|^2 - 2 x.c is then
      // formed in binary32 (|x|^2 of a bfloat16 row summed in binary32 to
      // within 2^-17, |c|^2 rounded once, two operations): 2^-16 (|x|^2 +
      // |c|^2 + 2 |x| |c|) covers those roundings and the binary64 scan's own.
      // As above, a row whose intervals single out one centroid takes it;
      // the others are recomputed in binary64.
      const int li = lane & 15, lk = lane >> 4;
      const uint16_t* s_cb = (const uint16_t*)s_c32;
      const float e1f = 0x1p-13f + 0x1p-18f + 0x1p-24f, e2f = 0x1p-16f;
      // A: row 16 rb + li; chunk c holds channels 32 c + 8 lk .. + 7 (B the same)
      const int nrb = (n + 15) / 16;
      // per centroid 16 cb + li: |c|^2 rounded to binary32 and the bound's
      // centroid terms (e1 + 2 e2) |c| and e2 |c|^2
      float ccf[NCB], ca[NCB], cbv[NCB];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        const int j = min(16 * cb + li, k16 - 1);
        ccf[cb] = (float)s_cc[j];
        ca[cb] = (e1f + 2.0f * e2f) * s_cn[j];
        cbv[cb] = e2f * ccf[cb];
      }
      uint4 xn[4];
      auto load_row = [&](int rb) {
        const uint4* p = (const uint4*)((const uint16_t*)x +
                                        km_row(u, min(16 * rb + li, n - 1), n_tok, gstride, groups) * D + 8 * lk);
#pragma unroll
        for (int c = 0; c < 4; ++c) xn[c] = p[4 * c];
      };
      if (wave < nrb) load_row(wave);
      for (int rb = wave; rb < nrb; rb += KF_THREADS / 64) {
        uint4 xa[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) xa[c] = xn[c];
        if (rb + KF_THREADS / 64 < nrb) load_row(rb + KF_THREADS / 64);
        km_f32x4 acc[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[cb] = km_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int part = 0; part < 2; ++part)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
              const uint4 bw = *(const uint4*)(s_cb + ((part * k16 + 16 * cb + li) * KB_STRIDE + 32 * c + 8 * lk));
              acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(km_bf16x8, xa[c]),
                                                                __builtin_bit_cast(km_bf16x8, bw), acc[cb], 0, 0, 0);
            }
        // |x|^2 of row li in binary32: this lane's 32 channels, then the
        // four lanes holding the row
        float xx = 0.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t w[4] = {xa[c].x, xa[c].y, xa[c].z, xa[c].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float lo = __builtin_bit_cast(float, w[i] << 16), hi = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
            xx = __builtin_fmaf(lo, lo, xx);
            xx = __builtin_fmaf(hi, hi, xx);
          }
        }
        xx += __shfl_xor(xx, 16, 64);
        xx += __shfl_xor(xx, 32, 64);
        // output slot r of this lane: row 16 rb + 4 lk + r, centroid 16 cb + li
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * rb + 4 * lk + r;
          const float xr = __shfl(xx, 4 * lk + r, 64);
          const float xnr = __builtin_sqrtf(xr) * (1.0f + 0x1p-19f);   // |x| rounded up
          float lo[NCB], hi[NCB];
          float U = INFINITY;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            const int j = 16 * cb + li;
            lo[cb] = hi[cb] = INFINITY;
            if (j < k) {
              // e1 |x| |c| + e2 (|x|^2 + |c|^2 + 2 |x| |c|), widened for its
              // own roundings
              const float ap = __builtin_fmaf(-2.0f, acc[cb][r], xr + ccf[cb]);
              const float E = __builtin_fmaf(xnr, ca[cb], cbv[cb] + e2f * xr) * (1.0f + 0x1p-19f)
                              + __builtin_fmaf(fabsf(ap), 0x1p-22f, 0x1p-100f);
              lo[cb] = ap - E;
              hi[cb] = ap + E;
            }
            U = fminf(U, hi[cb]);
          }
          U = km_rowmin16(U);
          int count = 0, first = -1;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            const uint64_t bal = __ballot(lo[cb] <= U);
            const uint32_t bits = (uint32_t)(bal >> (16 * lk)) & 0xFFFFu;
            count += __popc(bits);
            if (first < 0 && bits) first = 16 * cb + __ffs(bits) - 1;
          }
          if (li == 0 && row < n) {
            if (count == 1) {
              if (it == 0 || s_a[row] != (uint8_t)first) changed = 1;
              s_a[row] = (uint8_t)first;
            } else {
              s_amb[atomicAdd(s_namb, 1)] = (uint16_t)row;
            }
          }
        }
      }
    } else {
      const int li = lane & 15, lk = lane >> 4;
      // E = e1 |x| |c| + e2 (|x|^2 + |c|^2 + 2 |x| |c|): the binary32 dot over D
      // channels from the rounded centroid, and (e2) the binary64 roundings
      const float e1f = 2.0f * (D + 3) * 0x1p-24f * (1.0f + 0x1p-20f), e2f = 0x1p-40f;
      // A: row 16 rb + li; half h of the channels, 16 per lane: channels
      // 64 h + 16 lk .. + 15 (B uses the same order).  The next half (of this
      // row block or the next) is loaded while one is used.
      const int nrb = (n + 15) / 16;
      float xn[16];
      auto load_half = [&](int rb, int h) {
        km_load16(x, km_row(u, min(16 * rb + li, n - 1), n_tok, gstride, groups) * D + 64 * h + 16 * lk, bf16, xn);
      };
      if (wave < nrb) load_half(wave, 0);
      for (int rb = wave; rb < nrb; rb += KF_THREADS / 64) {
        km_f32x4 acc[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[cb] = km_f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        double xx = 0.0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float xa[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) xa[i] = xn[i];
          if (h == 0) load_half(rb, 1);
          else if (rb + KF_THREADS / 64 < nrb) load_half(rb + KF_THREADS / 64, 0);
#pragma unroll
          for (int i = 0; i < 16; ++i) xx = __builtin_fma((double)xa[i], (double)xa[i], xx);
          // the pattern blocks' accumulation chains interleaved
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4) {
            float4 cv[NCB];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
              cv[cb] = *(const float4*)(s_c32 + (16 * cb + li) * KF_CSTRIDE + 64 * h + 16 * lk + 4 * s4);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
              acc[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[4 * s4], cv[cb].x, acc[cb], 0, 0, 0);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
              acc[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[4 * s4 + 1], cv[cb].y, acc[cb], 0, 0, 0);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
              acc[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[4 * s4 + 2], cv[cb].z, acc[cb], 0, 0, 0);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
              acc[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[4 * s4 + 3], cv[cb].w, acc[cb], 0, 0, 0);
          }
        }
        // |x|^2 of row li: the four lanes holding it add their parts
        xx += __shfl_xor(xx, 16, 64);
        xx += __shfl_xor(xx, 32, 64);
        // output slot r of this lane: row 16 rb + 4 lk + r, centroid 16 cb + li
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * rb + 4 * lk + r;
          const double xr = __shfl(xx, 4 * lk + r, 64);
          // |x| rounded up (binary32 sqrt of the rounded square, widened)
          const float xrf = (float)xr;
          const float xn = __builtin_sqrtf(xrf) * (1.0f + 0x1p-19f);
          float lo[NCB], hi[NCB];
          float U = INFINITY;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            const int j = 16 * cb + li;
            lo[cb] = hi[cb] = INFINITY;
            if (j < k) {
              const double ap = (xr + s_cc[j]) - 2.0 * (double)acc[cb][r];
              // the bound in binary32, widened by 2^-19 for its own roundings
              const float cn = s_cn[j], apf = (float)ap;
              const float E = (e1f * xn * cn + e2f * (xrf + (float)s_cc[j] + 2.0f * xn * cn)) * (1.0f + 0x1p-19f)
                              + fabsf(apf) * 0x1p-22f + 0x1p-100f;
              lo[cb] = apf - E;
              hi[cb] = apf + E;
            }
            U = fminf(U, hi[cb]);
          }
          U = km_rowmin16(U);
          int count = 0, first = -1;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            const uint64_t bal = __ballot(lo[cb] <= U);
            const uint32_t bits = (uint32_t)(bal >> (16 * lk)) & 0xFFFFu;
            count += __popc(bits);
            if (first < 0 && bits) first = 16 * cb + __ffs(bits) - 1;
          }
          if (li == 0 && row < n) {
            if (count == 1) {
              if (it == 0 || s_a[row] != (uint8_t)first) changed = 1;
              s_a[row] = (uint8_t)first;
            } else {
              s_amb[atomicAdd(s_namb, 1)] = (uint16_t)row;
            }
          }
        }
      }
    }
    __syncthreads();
    // the listed rows: one wave per row, lane j sums centroid j's squared
    // differences in channel order (binary64); the smallest distance, lowest
    // index on ties, is the pattern a scan with strict '<' in pattern order
    // keeps
    const int namb = *s_namb;
    for (int i = wave; i < namb; i += KF_THREADS / 64) {
      const int t = s_amb[i];
      const int64_t row = km_row(u, t, n_tok, gstride, groups) * D;
      double dist[KM_MAXK / 64 + 1];
      int best = 0;
      double bd = INFINITY;
#pragma unroll
      for (int h = 0; h * 64 < KM_MAXK; ++h) {
        const int j = h * 64 + lane;
        double acc = 0.0;
        if (j < k) {
          float xb[16];
          for (int d0 = 0; d0 < D; d0 += 16) {
            km_load16(x, row + d0, bf16, xb);
#pragma unroll
            for (int dd = 0; dd < 16; ++dd) {
              const double diff = (double)xb[dd] - cent[j][d0 + dd];
              acc = acc + diff * diff;
            }
          }
        }
        dist[h] = j < k ? acc : INFINITY;
      }
      // lexicographic minimum of (distance, index) over the wave
#pragma unroll
      for (int h = 0; h * 64 < KM_MAXK; ++h) {
        double dv = dist[h];
        int jv = h * 64 + lane;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const double od = __shfl_xor(dv, o, 64);
          const int oj = __shfl_xor(jv, o, 64);
          if (od < dv || (od == dv && oj < jv)) { dv = od; jv = oj; }
        }
        if (dv < bd) { bd = dv; best = jv; }
      }
      if (lane == 0) {
        if (it == 0 || s_a[t] != (uint8_t)best) changed = 1;
        s_a[t] = (uint8_t)best;
      }
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
    // centroid = member sum in token order / member count; empty keeps its
    // centroid.
    if (BF && exact_sums) {
      // Exact sums (see above): the member list, grouped by cluster, is cut
      // into 32 equal segments; thread (segment, q) sums channels 4 q .. 4 q
      // + 3 over its segment's run of each cluster and adds the run's sum to
      // the cluster's row of `cent` (zeroed first) with an LDS atomic add,
      // every addition exact.  Then each row is divided by its count.
      for (int i = tid; i < k * D; i += KF_THREADS)
        if (s_cnt[i / D] > 0) cent[i / D][i % D] = 0.0;
      __syncthreads();
      const int q = tid & 31, seg = tid >> 5;
      const int e0 = (int)((int64_t)seg * n / (KF_THREADS / 32));
      const int e1 = (int)((int64_t)(seg + 1) * n / (KF_THREADS / 32));
      double acc[4] = {0.0, 0.0, 0.0, 0.0};
      int cj = -1;
      constexpr int MF = 16;
      for (int e = e0; e < e1; e += MF) {
        uint2 w[MF];
        int jm[MF];
#pragma unroll
        for (int i2 = 0; i2 < MF; ++i2) {
          const int t = s_mem[min(e + i2, e1 - 1)];
          jm[i2] = s_a[t];
          w[i2] = *(const uint2*)((const uint16_t*)x + km_row(u, t, n_tok, gstride, groups) * D + 4 * q);
        }
#pragma unroll
        for (int i2 = 0; i2 < MF; ++i2)
          if (e + i2 < e1) {
            if (jm[i2] != cj) {
              if (cj >= 0)
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) atomicAdd(&cent[cj][4 * q + qq], acc[qq]);
              cj = jm[i2];
#pragma unroll
              for (int qq = 0; qq < 4; ++qq) acc[qq] = 0.0;
            }
            acc[0] = acc[0] + (double)bf16_to_f32((uint16_t)(w[i2].x & 0xFFFFu));
            acc[1] = acc[1] + (double)bf16_to_f32((uint16_t)(w[i2].x >> 16));
            acc[2] = acc[2] + (double)bf16_to_f32((uint16_t)(w[i2].y & 0xFFFFu));
            acc[3] = acc[3] + (double)bf16_to_f32((uint16_t)(w[i2].y >> 16));
          }
      }
      if (cj >= 0)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) atomicAdd(&cent[cj][4 * q + qq], acc[qq]);
      __syncthreads();
      for (int i = tid; i < k * D; i += KF_THREADS) {
        const int j = i / D, c = s_cnt[j];
        if (c > 0) cent[j][i % D] = cent[j][i % D] / (double)c;
      }
      __syncthreads();
      continue;
    }
    // Thread (j, q) sums channels 4 q .. 4 q + 3 of cluster j's members in
    // token order (one accumulator per channel), with the loads of several
    // members in flight; the threads of a cluster read whole rows.
    for (int i = tid; i < k * (D / 4); i += KF_THREADS) {
      const int j = i / (D / 4), d0 = 4 * (i % (D / 4)), c = s_cnt[j];
      if (c == 0) continue;
      const uint16_t* m = s_mem + s_off[j];
      double acc[4] = {0.0, 0.0, 0.0, 0.0};
      if constexpr (BF) {
        // raw bfloat16 words of 16 members in flight
        constexpr int MF = 16;
        for (int e = 0; e < c; e += MF) {
          uint2 w[MF];
#pragma unroll
          for (int i2 = 0; i2 < MF; ++i2)
            w[i2] = *(const uint2*)((const uint16_t*)x + km_row(u, m[min(e + i2, c - 1)], n_tok, gstride, groups) * D + d0);
#pragma unroll
          for (int i2 = 0; i2 < MF; ++i2)
            if (e + i2 < c) {
              acc[0] = acc[0] + (double)bf16_to_f32((uint16_t)(w[i2].x & 0xFFFFu));
              acc[1] = acc[1] + (double)bf16_to_f32((uint16_t)(w[i2].x >> 16));
              acc[2] = acc[2] + (double)bf16_to_f32((uint16_t)(w[i2].y & 0xFFFFu));
              acc[3] = acc[3] + (double)bf16_to_f32((uint16_t)(w[i2].y >> 16));
            }
        }
      } else {
        for (int e = 0; e < c; e += 8) {
          float4 f[8];
#pragma unroll
          for (int i2 = 0; i2 < 8; ++i2)
            f[i2] = *(const float4*)((const float*)x + km_row(u, m[min(e + i2, c - 1)], n_tok, gstride, groups) * D + d0);
#pragma unroll
          for (int i2 = 0; i2 < 8; ++i2)
            if (e + i2 < c) {
              acc[0] = acc[0] + (double)f[i2].x;
              acc[1] = acc[1] + (double)f[i2].y;
              acc[2] = acc[2] + (double)f[i2].z;
              acc[3] = acc[3] + (double)f[i2].w;
            }
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) cent[j][d0 + q] = acc[q] / (double)c;
    }
    __syncthreads();
  }
  for (int i = tid; i < k * D; i += KF_THREADS) tab[i] = (float)cent[i / D][i % D];
}

template <int NCB, bool BF>
static hipError_t launch_kmeans_fast(const void* xk, const void* xv, int bf16, int n_tok, int groups,
                                     int64_t gstride, int k, float* tab_k, float* tab_v, int max_pat,
                                     int units, int lds, hipStream_t s) {
  static int attr = 0;
  if (lds > attr) {
    hipError_t e = hipFuncSetAttribute((const void*)kmeans_fast_kernel<NCB, BF>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    attr = lds;
  }
  hipLaunchKernelGGL((kmeans_fast_kernel<NCB, BF>), dim3(units, 2), dim3(KF_THREADS), lds, s, xk, xv, bf16,
                     n_tok, groups, gstride, k, tab_k, tab_v, max_pat);
  return hipGetLastError();
}

template <bool BF>
static hipError_t launch_kmeans_ncb(int ncb, const void* xk, const void* xv, int bf16, int n_tok, int groups,
                                    int64_t gstride, int k, float* tab_k, float* tab_v, int max_pat,
                                    int units, int lds, hipStream_t s) {
  if (ncb <= 1) return launch_kmeans_fast<1, BF>(xk, xv, bf16, n_tok, groups, gstride, k, tab_k, tab_v, max_pat, units, lds, s);
  if (ncb == 2) return launch_kmeans_fast<2, BF>(xk, xv, bf16, n_tok, groups, gstride, k, tab_k, tab_v, max_pat, units, lds, s);
  if (ncb == 3) return launch_kmeans_fast<3, BF>(xk, xv, bf16, n_tok, groups, gstride, k, tab_k, tab_v, max_pat, units, lds, s);
  return launch_kmeans_fast<4, BF>(xk, xv, bf16, n_tok, groups, gstride, k, tab_k, tab_v, max_pat, units, lds, s);
}

hipError_t launch_kmeans_pair(const void* xk, const void* xv, int bf16, int n_tok, int groups,
                              int64_t gstride, int k, float* tab_k, float* tab_v, int max_pat,
                              int units, uint8_t* assign, hipStream_t s) {
  const int64_t n = (int64_t)groups * n_tok;
  if (n <= KF_MAXN && k <= KM_MAXK && kf_lds((int)n, k).total <= KF_LDS_MAX) {
    const int lds = kf_lds((int)n, k).total;
    const int ncb = (k + 15) / 16;
    return bf16 ? launch_kmeans_ncb<true>(ncb, xk, xv, bf16, n_tok, groups, gstride, k, tab_k, tab_v, max_pat, units, lds, s)
                : launch_kmeans_ncb<false>(ncb, xk, xv, bf16, n_tok, groups, gstride, k, tab_k, tab_v, max_pat, units, lds, s);
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
