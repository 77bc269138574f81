// attn_pp.hip -- decode attention over the packed cache with paired score and
// value waves (the default MFMA path).
//
// Same algebra and MFMA operand layouts as attn_mfma.hip (PatternKV, arXiv
// 2510.05176v2, section 3.4: index restore + dequant + QK fused; dequant +
// index restore + weighted sum over V fused), split by role so that each wave
// holds only half of the state:
//
//  * the first PP_PAIRS waves (score waves) stage the K half of their 64-token
//    tile, run the QK products, the score epilogue and the online softmax,
//    and leave p (as p * 2^(pv_ep - shift) for the PV operand and as binary16
//    hi/lo for the pattern mass) plus the rescale factor of the tile in a slot;
//  * the other PP_PAIRS waves (value waves) stage the V half of the same tile
//    one step later and run the PV products, the pattern-mass product and the
//    z sums from the slot their partner filled in the previous step.
//
// Slots are double-buffered per pair and every step ends with one block
// barrier, so a slot is never written while its reader may still use it.
// The split-K combine is fused into the last block of each unit as in
// attn_mfma.hip.
#include <type_traits>

#include "attn_mfma_common.h"

namespace kvq {

constexpr int PP_PAIRS = 2;   // score/value wave pairs per block
constexpr int PP_THREADS = 2 * PP_PAIRS * 64;

// The K and V halves of a staged 64-token tile (bytes).
template <int BITS, int NG, bool KVARN>
struct PpShape {
  static constexpr int KREC = D * BITS / 8;
  static constexpr int KC = TILE * KREC;              // K codes
  static constexpr int SZ = TILE * NG * 4;            // (s, z) words of one kind
  static constexpr int VC = 2 * VT * D * BITS / 8;    // two V code tiles
  static constexpr int IX = KVARN ? 2 * TILE : TILE;  // idx or t16 of one kind
  static constexpr int K_SZ = KC, K_IX = KC + SZ, K_BYTES = KC + SZ + IX;
  static constexpr int V_SZ = VC, V_IX = VC + SZ, V_BYTES = VC + SZ + IX;
  static constexpr int R_KC = KC / 1024, R_VC = VC / 1024;   // 16-byte pieces per lane
  static constexpr int P_SZ = SZ / 16, P_IX = IX / 16;       // pieces (<= 64)
};

struct PpLds {
  int q, qsum, qm, kst, vst, svs, ps, ph, al, w, m, f, lz, z, l, wsum, M, last, total;
};
template <int BITS, int NG, bool KVARN>
__host__ __device__ inline PpLds pp_lds(int npat, bool hist_mfma) {
  using PS = PpShape<BITS, NG, KVARN>;
  constexpr int HB = 16 / NG, PW = ptab_words<16 / NG>();
  PpLds L;
  int o = 0;
  L.q = o; o = al16(o + HB * D * 4);
  L.qsum = o; o = al16(o + HB * NG * 4);
  L.qm = o; o = al16(o + HB * 256 * 4);
  // staging, reused after the loop for the per-pair partial o[HB][D]
  const int st = PP_PAIRS * (PS::K_BYTES + PS::V_BYTES);
  const int part = PP_PAIRS * HB * D * 4;
  L.kst = o;
  L.vst = o + PP_PAIRS * PS::K_BYTES;
  o = al16(o + (st > part ? st : part));
  L.svs = o; o = al16(o + PP_PAIRS * NG * VS_STRIDE * 2);
  L.ps = o; o = al16(o + PP_PAIRS * 2 * PW * 4);
  L.ph = o; o = al16(o + (hist_mfma ? PP_PAIRS * 2 * PW * 4 : 0));
  L.al = o; o = al16(o + PP_PAIRS * 2 * HB * 4);
  L.w = o; o = al16(o + PP_PAIRS * HB * npat * 4);
  L.m = o; o = al16(o + PP_PAIRS * HB * 4);
  L.f = o; o = al16(o + PP_PAIRS * HB * 4);
  L.lz = o; o = al16(o + PP_PAIRS * HB * (1 + NG) * 4);
  L.z = o; o = al16(o + HB * NG * 4);
  L.l = o; o = al16(o + HB * 4);
  L.wsum = o; o = al16(o + HB * npat * 4);
  L.M = o; o = al16(o + HB * 4);
  L.last = o; o = al16(o + 16);
  L.total = o;
  return L;
}

template <int BITS, int NG, bool KVARN, int NPB>
__global__ void __launch_bounds__(PP_THREADS)
__attribute__((amdgpu_waves_per_eu(BITS == 2 && NG == 4 && !KVARN ? 3 : 2,
                                    BITS == 2 && NG == 4 && !KVARN ? 3 : 2)))
attn_pp_kernel(AttnArgs a) {
  static_assert(!(KVARN && NPB), "KVarN has no pattern term");
  using PS = PpShape<BITS, NG, KVARN>;
  constexpr int G = D / NG;            // channels per group
  constexpr int HB = 16 / NG;          // heads per row block
  constexpr int CPG = 16 / NG;         // PV columns per group
  constexpr int SPL = 4 / NG;          // heads per lane in a 16x16 output
  constexpr int KW = BITS;             // dwords of a lane's 32-channel K slice
  constexpr int VTB = VT * D * BITS / 8;
  constexpr int PW = ptab_words<HB>();
  extern __shared__ __attribute__((aligned(16))) unsigned char pp_raw[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pair = wave & (PP_PAIRS - 1);
  const bool score = wave < PP_PAIRS;
  const int j = lane >> 4, n16 = lane & 15;
  const int head0 = (4 * j) / NG;     // head of output register slot s is head0 + s
  const int U = a.B * a.Hkv;
  const int u = blockIdx.x % U, split = blockIdx.x / U;
  const int b = u / a.Hkv, hk = u % a.Hkv, hq0 = hk * a.gq;
  const int t_begin = split * a.chunk, t_end = min(a.T, t_begin + a.chunk);
  const int n_pat = KVARN ? 0 : a.n_pat;
  const int npat = pad_pat(n_pat);
  const PpLds Lo = pp_lds<BITS, NG, KVARN>(npat, NPB > 0);
  float* s_q = (float*)(pp_raw + Lo.q);            // [HB][D]
  float* s_qsum = (float*)(pp_raw + Lo.qsum);      // [HB][NG]
  float* s_qm = (float*)(pp_raw + Lo.qm);          // [HB][256]; entry 0xFF (no pattern) is 0
  unsigned char* kt = pp_raw + Lo.kst + pair * PS::K_BYTES;   // this pair's K half
  unsigned char* vt = pp_raw + Lo.vst + pair * PS::V_BYTES;   // this pair's V half
  _Float16* s_vs = (_Float16*)(pp_raw + Lo.svs) + pair * NG * VS_STRIDE;   // V scales [g][t]
  float* s_ps = (float*)(pp_raw + Lo.ps) + pair * 2 * PW;        // [slot][PW]
  uint32_t* s_ph = (uint32_t*)(pp_raw + Lo.ph) + pair * 2 * PW;  // [slot][PW]
  float* s_al = (float*)(pp_raw + Lo.al) + pair * 2 * HB;        // [slot][HB]
  float* s_w = (float*)(pp_raw + Lo.w);            // [PAIRS][HB][npat]
  float* wrow = s_w + pair * HB * npat;
  float* s_m = (float*)(pp_raw + Lo.m);            // [PAIRS][HB]
  float* s_f = (float*)(pp_raw + Lo.f);            // [PAIRS][HB]
  float* s_lz = (float*)(pp_raw + Lo.lz);          // [PAIRS][HB][1 + NG]
  float* s_z = (float*)(pp_raw + Lo.z);            // [HB][NG]
  float* s_l = (float*)(pp_raw + Lo.l);            // [HB]
  float* s_wsum = (float*)(pp_raw + Lo.wsum);      // [HB][npat]
  float* s_M = (float*)(pp_raw + Lo.M);            // [HB]
  int* s_last = (int*)(pp_raw + Lo.last);

  const uint8_t* kcodes = a.r.codes[0] + (int64_t)u * a.tcap * PS::KREC;
  const uint8_t* vcodes = a.r.codes[1] + (int64_t)u * a.tcap * PS::KREC;
  const uint8_t* ksz = (const uint8_t*)(a.r.sz[0] + (int64_t)u * a.tcap * NG);
  const uint8_t* vsz = (const uint8_t*)(a.r.sz[1] + (int64_t)u * a.tcap * NG);
  const uint8_t* kix_src = KVARN ? (const uint8_t*)(a.r.t16[0] + (int64_t)u * a.tcap)
                                 : a.r.idx[0] + (int64_t)u * a.tcap;
  const uint8_t* vix_src = KVARN ? (const uint8_t*)(a.r.t16[1] + (int64_t)u * a.tcap)
                                 : a.r.idx[1] + (int64_t)u * a.tcap;
  const int ix_bytes = KVARN ? 2 : 1;

  // ---------------------------------------------------------------- tile halves
  // Each role keeps the next tile's half in registers (one 16-byte piece per
  // lane and segment) while it computes the current one.
  constexpr int R_C = PS::R_KC > PS::R_VC ? PS::R_KC : PS::R_VC;
  u32x4 rc[R_C], rsz, rix;
  auto issue = [&](int tile) {
    if (score) {
      const u32x4* src = (const u32x4*)(kcodes + (int64_t)tile * PS::KREC);
#pragma unroll
      for (int r = 0; r < PS::R_KC; ++r) rc[r] = src[lane + 64 * r];
      if (lane < PS::P_SZ) rsz = ((const u32x4*)(ksz + (int64_t)tile * NG * 4))[lane];
      if (lane < PS::P_IX) rix = ((const u32x4*)(kix_src + (int64_t)tile * ix_bytes))[lane];
    } else {
      const u32x4* src = (const u32x4*)(vcodes + (int64_t)(tile >> 5) * VTB);
#pragma unroll
      for (int r = 0; r < PS::R_VC; ++r) rc[r] = src[lane + 64 * r];
      if (lane < PS::P_SZ) rsz = ((const u32x4*)(vsz + (int64_t)tile * NG * 4))[lane];
      if (lane < PS::P_IX) rix = ((const u32x4*)(vix_src + (int64_t)tile * ix_bytes))[lane];
    }
  };
  auto commit = [&](int tile) {
    if (score) {
      u32x4* t4 = (u32x4*)kt;
#pragma unroll
      for (int r = 0; r < PS::R_KC; ++r) t4[kpiece<BITS>(lane + 64 * r)] = rc[r];
      if (lane < PS::P_SZ) t4[PS::K_SZ / 16 + lane] = rsz;
      if (lane < PS::P_IX) t4[PS::K_IX / 16 + lane] = rix;
    } else {
      u32x4* t4 = (u32x4*)vt;
#pragma unroll
      for (int r = 0; r < PS::R_VC; ++r) t4[vpiece(lane + 64 * r)] = rc[r];
      if (lane < PS::P_SZ) {
        t4[PS::V_SZ / 16 + lane] = rsz;
        // V scales, transposed to [group][token] for the PV operand (0 past
        // the end, so that stale bytes there cannot reach the products)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int w = 4 * lane + i, t = w / NG, g = w % NG;
          const uint16_t sv = tile + t < t_end ? (uint16_t)(rsz[i] & 0xFFFFu) : (uint16_t)0;
          s_vs[g * VS_STRIDE + t] = __builtin_bit_cast(_Float16, sv);
        }
      }
      if (lane < PS::P_IX) t4[PS::V_IX / 16 + lane] = rix;
    }
  };

  const int tile0 = t_begin + TILE * pair;
  if (tile0 < t_end) issue(tile0);

  // ---------------------------------------------------------------- prologue
  // This thread's 32-channel slice of pattern row tid / 4 of M^K is loaded
  // with q, before anything waits.
  const int qm_j = tid >> 2, qm_part = tid & 3;
  const float* mk = a.r.tab[0] + pat_unit(a.r, u) * a.max_pat * D;
  float4 mkr[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) mkr[k] = float4{0.0f, 0.0f, 0.0f, 0.0f};
  if (!KVARN && qm_j < n_pat) {
    const float4* m4 = (const float4*)(mk + (int64_t)qm_j * D + qm_part * 32);
#pragma unroll
    for (int k = 0; k < 8; ++k) mkr[k] = m4[k];
  }
  for (int i = tid; i < HB * D; i += PP_THREADS) {
    const int h = i / D, d = i % D;
    s_q[i] = h < a.gq ? load_in(a.q, ((int64_t)b * a.Hq + hq0 + h) * D + d, a.bf16) : 0.0f;
  }
  for (int i = tid; i < PP_PAIRS * HB * npat; i += PP_THREADS) s_w[i] = 0.0f;
  for (int i = tid; i < HB * 256; i += PP_THREADS) s_qm[i] = 0.0f;
  __syncthreads();
  if (KVARN) {
    for (int hs = 1; hs < D; hs <<= 1) {
      float v[HB * D / PP_THREADS];
#pragma unroll
      for (int k = 0; k < HB * D / PP_THREADS; ++k) {
        const int i = tid + k * PP_THREADS, d = i % D;
        const float mine = s_q[i], other = s_q[i ^ hs];
        v[k] = (d & hs) ? other - mine : mine + other;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < HB * D / PP_THREADS; ++k) s_q[tid + k * PP_THREADS] = v[k];
      __syncthreads();
    }
  }
  {
    const float isd = (float)(1.0 / __builtin_sqrt(128.0));
    const float* ck = a.r.tab[0] + (int64_t)u * D;
    for (int i = tid; i < HB * D; i += PP_THREADS) {
      float v = s_q[i];
      if (KVARN) v = v * isd * ck[i % D];
      s_q[i] = v * a.qscale;
    }
  }
  __syncthreads();
  // per-group sums of q': thread (h = tid/32) adds 4 channels, then the G/4
  // lanes of a group reduce
  if (tid < HB * 32) {
    const int h = tid >> 5, c0 = (tid & 31) * 4;
    float s = (s_q[h * D + c0] + s_q[h * D + c0 + 1]) + (s_q[h * D + c0 + 2] + s_q[h * D + c0 + 3]);
#pragma unroll
    for (int o = 1; o < G / 4; o <<= 1) s += __shfl_xor(s, o, 64);
    if (((tid & 31) % (G / 4)) == 0) s_qsum[h * NG + c0 / G] = s;
  }
  // q' . M^K_j: four threads per pattern (32 channels each); patterns beyond
  // the first PP_THREADS / 4 take further passes
  if (!KVARN && n_pat > 0) {
    for (int j0 = 0; j0 < n_pat; j0 += PP_THREADS / 4) {
      const int jj = j0 + qm_j;
      if (j0 > 0) {
#pragma unroll
        for (int k = 0; k < 8; ++k) mkr[k] = float4{0.0f, 0.0f, 0.0f, 0.0f};
        if (jj < n_pat) {
          const float4* m4 = (const float4*)(mk + (int64_t)jj * D + qm_part * 32);
#pragma unroll
          for (int k = 0; k < 8; ++k) mkr[k] = m4[k];
        }
      }
#pragma unroll
      for (int h = 0; h < HB; ++h) {
        if (h >= a.gq) break;
        const float* qh = s_q + h * D + qm_part * 32;
        float sdot = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          sdot = __builtin_fmaf(qh[4 * k], mkr[k].x, sdot);
          sdot = __builtin_fmaf(qh[4 * k + 1], mkr[k].y, sdot);
          sdot = __builtin_fmaf(qh[4 * k + 2], mkr[k].z, sdot);
          sdot = __builtin_fmaf(qh[4 * k + 3], mkr[k].w, sdot);
        }
        sdot += __shfl_xor(sdot, 1, 64);
        sdot += __shfl_xor(sdot, 2, 64);
        if (qm_part == 0 && jj < n_pat) s_qm[h * 256 + jj] = sdot;
      }
    }
  }
  __syncthreads();

  // -1 and +0 the compiler cannot fold (qscale is finite)
  const float k_m1 = __builtin_fmaf(a.qscale, 0.0f, -1.0f);
  const float k_z = a.qscale * 0.0f;

  // ---------------------------------------------------------------- main loop
  // Step k: score waves take tile k of their pair, value waves tile k - 1.
  const int n_steps = t_end > t_begin ? (t_end - t_begin + PP_PAIRS * TILE - 1) / (PP_PAIRS * TILE) + 1 : 0;
  // The V pattern rows of this thread's output channel d = tid % D are loaded
  // at loop exit, so that they arrive while the pairs merge.
  const float* mv = a.r.tab[1] + pat_unit(a.r, u) * a.max_pat * D;
  constexpr int MVR = NPB > 0 ? 16 * NPB : 1;
  float mvr[MVR];
  // per-pair partial o[HB][D], over the staging
  float* s_ow = (float*)(pp_raw + Lo.kst);
  // Each role runs its own loop with the same number of block barriers (one
  // per step, four in the merge), so the two loops' barriers meet in order.
  if (score) {
    // ---- score-wave state: QK A operands (row m = n16 -> (h, g); element i of
    // chunk c -> channel), per-row group sums, running max and sum
    u32x4 aq_hi[4], aq_lo[4];
    float qsum[4];
    float m_run[SPL], l_run[SPL];
  #pragma unroll
    for (int s = 0; s < SPL; ++s) { m_run[s] = -INFINITY; l_run[s] = 0.0f; }
    {
      const int h = n16 / NG, g = n16 % NG;
  #pragma unroll
      for (int c = 0; c < 4; ++c) {
  #pragma unroll
        for (int p = 0; p < 4; ++p) {
          float v2[2];
  #pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int i = 2 * p + e, ch = qk_channel<BITS>(j, c, i);
            v2[e] = (ch / G == g) ? ldexpf(s_q[h * D + ch], EQ - code_shift<BITS>(i)) : 0.0f;
          }
          uint32_t hi, lo;
          split2(v2[0], v2[1], k_m1, hi, lo);
          aq_hi[c][p] = hi;
          aq_lo[c][p] = lo;
        }
      }
  #pragma unroll
      for (int r = 0; r < 4; ++r) qsum[r] = s_qsum[((4 * j + r) / NG) * NG + r % NG];
    }
    for (int k = 0; k < n_steps; ++k) {
      const int slot = k & 1;
        const int tile = tile0 + PP_PAIRS * TILE * k;
        if (tile < t_end) {
          __builtin_amdgcn_wave_barrier();
          commit(tile);
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          if (tile + PP_PAIRS * TILE < t_end) issue(tile + PP_PAIRS * TILE);
          const int nvalid = t_end - tile;
          float* ps = s_ps + slot * PW;
          uint32_t* ph = s_ph + slot * PW;
          auto score_body = [&](auto full_tag) {
            constexpr bool FULL = decltype(full_tag)::value;
            // ---- QK: four independent accumulators, one per 16-token column block
            f32x4 C[4];
            {
              uint32_t kw[4][KW];
  #pragma unroll
              for (int nb = 0; nb < 4; ++nb) {
                const int t64 = 16 * nb + n16;
                if (KW == 2) {
                  const uint2 w = *(const uint2*)(kt + kpiece<BITS>(2 * t64 + (j >> 1)) * 16 + (j & 1) * 8);
                  kw[nb][0] = w.x; kw[nb][1 % KW] = w.y;
                } else {
                  const u32x4 w = *(const u32x4*)(kt + kpiece<BITS>(4 * t64 + j) * 16);
  #pragma unroll
                  for (int q = 0; q < KW; ++q) kw[nb][q] = w[q];
                }
                C[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
              }
  #pragma unroll
              for (int c = 0; c < 4; ++c)
  #pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                  const u32x4 B = unpack_k<BITS>(kw[nb], c);
                  C[nb] = mfma16(aq_hi[c], B, C[nb]);
                  C[nb] = mfma16(aq_lo[c], B, C[nb]);
                }
            }
            float sc[4][SPL];
  #pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
              const int t64 = 16 * nb + n16;
              const bool valid = FULL || t64 < nvalid;
              uint32_t kszw[NG];
              {
                const uint32_t* kszp = (const uint32_t*)(kt + PS::K_SZ) + t64 * NG;
                if (NG == 4) {
                  const u32x4 k4 = *(const u32x4*)kszp;
  #pragma unroll
                  for (int g = 0; g < NG; ++g) kszw[g] = k4[g];
                } else {
                  const uint2 k2 = *(const uint2*)kszp;
                  kszw[0] = k2.x; kszw[1 % NG] = k2.y;
                }
              }
              float tk = 1.0f;
              int kix = KVQ_INDEX_NONE;
              if (KVARN) tk = bits2f(((const uint16_t*)(kt + PS::K_IX))[t64]);
              else kix = kt[PS::K_IX + t64];   // 0xFF (no pattern) reads a 0 entry
  #pragma unroll
              for (int s = 0; s < SPL; ++s) {
                float dot = 0.0f, zt = 0.0f;
  #pragma unroll
                for (int g = 0; g < NG; ++g) {
                  const int r = s * NG + g;
                  dot = __builtin_fmaf(bits2f((uint16_t)(kszw[g] & 0xFFFFu)), C[nb][r], dot);
                  zt = __builtin_fmaf(bits2f((uint16_t)(kszw[g] >> 16)), qsum[r], zt);
                }
                float v = __builtin_fmaf(dot, (float)(1 << (24 - EQ)), zt);
                if (!KVARN) v += s_qm[(head0 + s) * 256 + kix];
                else v *= tk;
                sc[nb][s] = valid ? v : -INFINITY;
              }
            }
            // ---- online softmax (log2 domain): the tile's rescale factor goes
            // to the slot for the value wave
  #pragma unroll
            for (int s = 0; s < SPL; ++s) {
              float mt = fmaxf(fmaxf(sc[0][s], sc[1][s]), fmaxf(sc[2][s], sc[3][s]));
              mt = row_max16(mt);
              const float mnew = fmaxf(m_run[s], mt);
              const float al = __builtin_amdgcn_exp2f(m_run[s] - mnew);
              m_run[s] = mnew;
              l_run[s] *= al;
              if (n16 == 0) s_al[slot * HB + head0 + s] = al;
            }
  #pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
              const int t64 = 16 * nb + n16;
  #pragma unroll
              for (int s = 0; s < SPL; ++s) {
                const float p = __builtin_amdgcn_exp2f(sc[nb][s] - m_run[s]);
                l_run[s] += p;
                ps[prow<HB>(head0 + s) + t64] = ldexpf(p, pv_ep<BITS, KVARN>() - pv_shift<BITS, KVARN>(t64 & 31));
                if constexpr (NPB > 0) {
                  // p * 2^15 <= 2^15 as binary16 hi + lo (round to nearest even)
                  const float x = p * 32768.0f;
                  const _Float16 hi = (_Float16)x;
                  const _Float16 lo = (_Float16)__builtin_fmaf((float)hi, k_m1, x);
                  ph[prow<HB>(head0 + s) + t64] = (uint32_t)h2bits(hi) | ((uint32_t)h2bits(lo) << 16);
                }
              }
            }
          };
          if (nvalid >= TILE) score_body(std::true_type{});
          else score_body(std::false_type{});
        }
      __syncthreads();
    }
#pragma unroll
    for (int jj = 0; jj < MVR; ++jj)
      mvr[jj] = (NPB > 0 && jj < n_pat) ? mv[(int64_t)jj * D + tid % D] : 0.0f;
    // ---- merge, score side: running max and sum of each pair
#pragma unroll
    for (int s = 0; s < SPL; ++s) {
      l_run[s] = row_sum16(l_run[s]);
      if (n16 == 0) s_m[pair * HB + head0 + s] = m_run[s];
    }
    __syncthreads();
    if (tid < HB) {
      float M = -INFINITY;
      for (int w = 0; w < PP_PAIRS; ++w) M = fmaxf(M, s_m[w * HB + tid]);
      s_M[tid] = M;
    }
    __syncthreads();
    // pair factors f = 2^(m_pair - M), and l relative to M
    if (n16 == 0) {
#pragma unroll
      for (int s = 0; s < SPL; ++s) {
        const int h = head0 + s;
        const float f = (m_run[s] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run[s] - s_M[h]);
        s_f[pair * HB + h] = f;
        s_lz[(pair * HB + h) * (1 + NG)] = f * l_run[s];
      }
    }
    __syncthreads();
    __syncthreads();
  } else {
    // ---- value-wave state: PV, z and pattern-mass accumulators
    f32x4 oacc[8];
  #pragma unroll
    for (int bb = 0; bb < 8; ++bb) oacc[bb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float zacc[4];
  #pragma unroll
    for (int r = 0; r < 4; ++r) zacc[r] = 0.0f;
    f32x4 hacc[NPB > 0 ? NPB : 1];
  #pragma unroll
    for (int cb = 0; cb < (NPB > 0 ? NPB : 1); ++cb) hacc[cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // hist A: row (head n16 / NG, part n16 % NG) takes the low (part 0) or high
    // (part 1) binary16 of each packed word; other rows are 0
    const uint32_t hsel = (n16 / NG >= a.gq || n16 % NG > 1) ? 0x0C0C0C0Cu
                          : (n16 % NG == 0 ? 0x05040100u : 0x07060302u);
    // p of this lane's column token t64 = 16 nb + n16 from the PV operand value
    // p * 2^(pv_ep - shift(t64)); the shift depends on n16 only
    const float unshift = ldexpf(1.0f, pv_shift<BITS, KVARN>(n16) - pv_ep<BITS, KVARN>());
    for (int k = 0; k < n_steps; ++k) {
      const int slot = k & 1;
        const int tile = tile0 + PP_PAIRS * TILE * (k - 1);
        if (k >= 1 && tile < t_end) {
          __builtin_amdgcn_wave_barrier();
          commit(tile);
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          if (tile + PP_PAIRS * TILE < t_end) issue(tile + PP_PAIRS * TILE);
          const int nvalid = t_end - tile;
          const float* ps = s_ps + (slot ^ 1) * PW;
          const uint32_t* ph = s_ph + (slot ^ 1) * PW;
          // ---- rescale when the partner's running max grew on this tile
          {
            float al[SPL];
            bool grow = false;
  #pragma unroll
            for (int s = 0; s < SPL; ++s) {
              al[s] = s_al[(slot ^ 1) * HB + head0 + s];
              grow |= al[s] != 1.0f;
            }
            if (__any(grow)) {
  #pragma unroll
              for (int r = 0; r < 4; ++r) zacc[r] *= al[r / NG];
  #pragma unroll
              for (int bb = 0; bb < 8; ++bb)
  #pragma unroll
                for (int r = 0; r < 4; ++r) oacc[bb][r] *= al[r / NG];
              if constexpr (NPB > 0) {
  #pragma unroll
                for (int cb = 0; cb < NPB; ++cb)
  #pragma unroll
                  for (int r = 0; r < 4; ++r) hacc[cb][r] *= al[r / NG];
              } else if (!KVARN && n_pat > 0) {
                for (int e = lane; e < a.gq * npat; e += 64) wrow[e] *= s_al[(slot ^ 1) * HB + e / npat];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
              }
            }
          }
          // ---- z sums (and the pattern mass by LDS atomics past 64 patterns)
  #pragma unroll
          for (int nb = 0; nb < 4; ++nb) {
            const int t64 = 16 * nb + n16;
            const bool valid = nvalid >= TILE || t64 < nvalid;
            uint32_t vszz[NG];
            {
              const uint32_t* vszp = (const uint32_t*)(vt + PS::V_SZ) + t64 * NG;
              if (NG == 4) {
                const u32x4 v4 = *(const u32x4*)vszp;
  #pragma unroll
                for (int g = 0; g < NG; ++g) vszz[g] = valid ? v4[g] : 0u;
              } else {
                const uint2 v2 = *(const uint2*)vszp;
                vszz[0] = valid ? v2.x : 0u;
                vszz[1 % NG] = valid ? v2.y : 0u;
              }
            }
            float tv = 1.0f;
            if (KVARN) {
              const float t = bits2f(((const uint16_t*)(vt + PS::V_IX))[t64]);
              tv = valid ? t : 0.0f;
            }
  #pragma unroll
            for (int s = 0; s < SPL; ++s) {
              // p is 0 on tokens past the end, whatever the staged bytes hold
              const float p = valid ? ps[prow<HB>(head0 + s) + t64] * unshift : 0.0f;
              const float pt = p * tv;   // KVarN: v^ carries the token scale t
  #pragma unroll
              for (int g = 0; g < NG; ++g)
                zacc[s * NG + g] = __builtin_fmaf(pt, bits2f((uint16_t)(vszz[g] >> 16)), zacc[s * NG + g]);
              if (!KVARN && NPB == 0 && n_pat > 0) {
                const int vix = vt[PS::V_IX + t64];
                if (valid && vix != KVQ_INDEX_NONE && head0 + s < a.gq)
                  atomicAdd(&wrow[(head0 + s) * npat + vix], p);
              }
            }
          }
          // ---- PV over the two 32-token V tiles (+ the pattern mass)
  #pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            u32x4 ahi, alo;
            {
              // rows of heads >= gq hold finite values that are never stored
              const int h = n16 / NG, g = n16 % NG;
              const int base = 32 * kb + pv_token<BITS>(j, 0), off = pv_token<BITS>(j, 1) - pv_token<BITS>(j, 0);
              const float4 p0 = *(const float4*)(ps + prow<HB>(h) + base);
              const float4 p1 = *(const float4*)(ps + prow<HB>(h) + base + off);
              const uint2 v0 = *(const uint2*)(s_vs + g * VS_STRIDE + base);
              const uint2 v1 = *(const uint2*)(s_vs + g * VS_STRIDE + base + off);
              float pa[4] = {p0.x, p0.y, p0.z, p0.w}, pb[4] = {p1.x, p1.y, p1.z, p1.w};
              if (KVARN) {
                const uint16_t* t16 = (const uint16_t*)(vt + PS::V_IX);
  #pragma unroll
                for (int p = 0; p < 4; ++p) {
                  const float ta = bits2f(t16[base + p]), tb2 = bits2f(t16[base + off + p]);
                  pa[p] *= (base + p < nvalid) ? ta : 0.0f;
                  pb[p] *= (base + off + p < nvalid) ? tb2 : 0.0f;
                }
              }
              const uint32_t va[2] = {v0.x, v0.y}, vb[2] = {v1.x, v1.y};
  #pragma unroll
              for (int p = 0; p < 4; ++p) {
                const float x0 = mul_h(pa[p], (uint16_t)(va[p >> 1] >> (16 * (p & 1))), k_z);
                const float x1 = mul_h(pb[p], (uint16_t)(vb[p >> 1] >> (16 * (p & 1))), k_z);
                uint32_t hi, lo;
                split2(x0, x1, k_m1, hi, lo);
                ahi[p] = hi;
                alo[p] = lo;
              }
            }
            if constexpr (NPB > 0) {
              // element i = 2p + e of lane group j <-> token 32 kb + 8 j + i
              const u32x4 h0 = *(const u32x4*)(ph + prow<HB>(n16 / NG) + 32 * kb + 8 * j);
              const u32x4 h1 = *(const u32x4*)(ph + prow<HB>(n16 / NG) + 32 * kb + 8 * j + 4);
              u32x4 ah;
              ah[0] = __builtin_amdgcn_perm(h0[1], h0[0], hsel);
              ah[1] = __builtin_amdgcn_perm(h0[3], h0[2], hsel);
              ah[2] = __builtin_amdgcn_perm(h1[1], h1[0], hsel);
              ah[3] = __builtin_amdgcn_perm(h1[3], h1[2], hsel);
              // pattern indices of tokens 2p, 2p + 1 in the high bytes of the two halves
              const uint2 vw = *(const uint2*)(vt + PS::V_IX + 32 * kb + 8 * j);
              uint32_t pr[4];
              pr[0] = __builtin_amdgcn_perm(0u, vw.x, 0x010C000Cu);
              pr[1] = __builtin_amdgcn_perm(0u, vw.x, 0x030C020Cu);
              pr[2] = __builtin_amdgcn_perm(0u, vw.y, 0x010C000Cu);
              pr[3] = __builtin_amdgcn_perm(0u, vw.y, 0x030C020Cu);
  #pragma unroll
              for (int cb = 0; cb < NPB; ++cb) {
                // B = 2^-16 (binary16 0x0100: the top of the mantissa, where
                // the dot product's alignment keeps it whole) where the index
                // equals this column's pattern, else 0
                const u16x2 tgt = u16x2{(uint16_t)((16 * cb + n16) << 8), (uint16_t)((16 * cb + n16) << 8)};
                u32x4 Bh;
  #pragma unroll
                for (int q = 0; q < 4; ++q) {
                  const u16x2 d = __builtin_bit_cast(u16x2, pr[q]) ^ tgt;
                  Bh[q] = __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(u16x2{0x100, 0x100}, d));
                }
                hacc[cb] = mfma16(ah, Bh, hacc[cb]);
              }
            }
            // this lane's word of channels 8*n16 .. 8*n16+7 (word-major V tile);
            // pieces 2 n16 and 2 n16 + 1, stored swapped for n16 >= 8
            const int word = BITS == 2 ? (j >> 1) : j;
            const u32x4* vp = (const u32x4*)(vt + kb * VTB) + word * (D / 4) + 2 * n16;
            const int vk = (n16 >> 3) & 1;
            const u32x4 w0 = vp[vk], w1 = vp[vk ^ 1];
  #pragma unroll
            for (int bb = 0; bb < 8; ++bb) {
              const u32x4 B = unpack_v<BITS, KVARN>(bb < 4 ? w0[bb] : w1[bb - 4], j);
              oacc[bb] = mfma16(ahi, B, oacc[bb]);
              oacc[bb] = mfma16(alo, B, oacc[bb]);
            }
          }
        }
      __syncthreads();
    }
#pragma unroll
    for (int jj = 0; jj < MVR; ++jj)
      mvr[jj] = (NPB > 0 && jj < n_pat) ? mv[(int64_t)jj * D + tid % D] : 0.0f;
    // ---- merge, value side: o, z and the pattern mass relative to M
#pragma unroll
    for (int r = 0; r < 4; ++r) zacc[r] = row_sum16(zacc[r]);
    __syncthreads();
    __syncthreads();
    __syncthreads();
    float f[SPL];
#pragma unroll
    for (int s = 0; s < SPL; ++s) f[s] = s_f[pair * HB + head0 + s];
    const float oscale = (float)(1 << (24 - pv_ep<BITS, KVARN>()));
    const int gcol = n16 / CPG;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r % NG != gcol) continue;
      const int s = r / NG;
      const float sc = oscale * f[s];
      float* dst = s_ow + (pair * HB + head0 + s) * D + 8 * n16;
      *(float4*)dst = float4{oacc[0][r] * sc, oacc[1][r] * sc, oacc[2][r] * sc, oacc[3][r] * sc};
      *(float4*)(dst + 4) = float4{oacc[4][r] * sc, oacc[5][r] * sc, oacc[6][r] * sc, oacc[7][r] * sc};
    }
    if (n16 == 0)
#pragma unroll
      for (int s = 0; s < SPL; ++s)
#pragma unroll
        for (int g = 0; g < NG; ++g)
          s_lz[(pair * HB + head0 + s) * (1 + NG) + 1 + g] = f[s] * zacc[s * NG + g];
    if constexpr (NPB > 0) {
      // w = (hi + lo rows) * 2^-15 / 2^-16, relative to the block max
#pragma unroll
      for (int cb = 0; cb < NPB; ++cb) {
        const int pat = 16 * cb + n16;
#pragma unroll
        for (int s = 0; s < SPL; ++s)
          if (pat < npat)
            wrow[(head0 + s) * npat + pat] = (hacc[cb][s * NG] + hacc[cb][s * NG + 1]) * (2.0f * f[s]);
      }
    }
    __syncthreads();
  }
  // block totals: pattern masses w[h][j], l[h], z[h][g]
  if (!KVARN && n_pat > 0)
    for (int e = tid; e < a.gq * npat; e += PP_THREADS) {
      const int h = e / npat;
      float acc = 0.0f;
#pragma unroll
      for (int w = 0; w < PP_PAIRS; ++w) {
        const float x = s_w[(w * HB) * npat + e];
        acc = NPB > 0 ? acc + x : __builtin_fmaf(s_f[w * HB + h], x, acc);
      }
      s_wsum[e] = acc;
    }
  if (tid < HB * (1 + NG)) {
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < PP_PAIRS; ++w) acc += s_lz[w * HB * (1 + NG) + tid];
    const int h = tid / (1 + NG), kk = tid % (1 + NG);
    if (kk == 0) s_l[h] = acc;
    else s_z[h * NG + kk - 1] = acc;
  }
  __syncthreads();

  // ---------------------------------------------------------------- partial out
  // Row (b, head, split): o + z + sum_j w_j M^V_j and (M, l), relative to this
  // split's max M; agent-scope stores, coherent across the XCDs' L2s.
  const int S = a.splits;
  float* ml = a.r.ws + (int64_t)a.B * a.Hq * S * D;
  for (int i = tid; i < a.gq * D; i += PP_THREADS) {
    const int h = i / D, d = i % D;
    const int64_t row = ((int64_t)b * a.Hq + hq0 + h) * S + split;
    float o = s_z[h * NG + d / G];
#pragma unroll
    for (int w = 0; w < PP_PAIRS; ++w) o += s_ow[(w * HB + h) * D + d];
    if constexpr (NPB > 0) {
#pragma unroll
      for (int jj = 0; jj < MVR; ++jj)
        if (jj < n_pat) o = __builtin_fmaf(s_wsum[h * npat + jj], mvr[jj], o);
    } else if (!KVARN) {
#pragma unroll 8
      for (int jj = 0; jj < n_pat; ++jj) o = __builtin_fmaf(s_wsum[h * npat + jj], mv[(int64_t)jj * D + d], o);
    }
    __hip_atomic_store(&a.r.ws[row * D + d], o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == 0) {
      __hip_atomic_store(&ml[row * 2], s_M[h], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&ml[row * 2 + 1], s_l[h], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // ---------------------------------------------------------------- fused combine
  // Each thread waits until its partial stores have completed at agent scope;
  // after the barrier thread 0 counts this split in, and the block that
  // arrives last (it observes S - 1 earlier increments, each made after that
  // split's stores completed) merges all splits of the unit with agent-scope
  // loads.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&a.r.cnt[u], 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    *s_last = prev == (uint32_t)(S - 1);
  }
  __syncthreads();
  if (!*s_last) return;
  // out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s, running max over
  // chunks of 8 splits so that each chunk's loads are issued together
  constexpr int OPT = HB * D / PP_THREADS;   // outputs per thread
  float r_out[OPT];
#pragma unroll
  for (int kk = 0; kk < OPT; ++kk) {
    const int i = tid + kk * PP_THREADS, h = i / D, d = i % D;
    r_out[kk] = 0.0f;
    if (h >= a.gq) continue;
    const int64_t row0 = ((int64_t)b * a.Hq + hq0 + h) * S;
    float M = -INFINITY, L = 0.0f, O = 0.0f;
    for (int c0 = 0; c0 < S; c0 += 8) {
      float mm[8], ll[8], oo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sp = c0 + e < S ? c0 + e : c0;
        mm[e] = __hip_atomic_load(&ml[(row0 + sp) * 2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ll[e] = __hip_atomic_load(&ml[(row0 + sp) * 2 + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        oo[e] = __hip_atomic_load(&a.r.ws[(row0 + sp) * D + d], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      float cm = M;
#pragma unroll
      for (int e = 0; e < 8; ++e) cm = (c0 + e < S) ? fmaxf(cm, mm[e]) : cm;
      const float rs = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - cm);
      L *= rs;
      O *= rs;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float fs = (c0 + e < S && mm[e] != -INFINITY) ? __builtin_amdgcn_exp2f(mm[e] - cm) : 0.0f;
        L = __builtin_fmaf(ll[e], fs, L);
        O = __builtin_fmaf(oo[e], fs, O);
      }
      M = cm;
    }
    r_out[kk] = O / L;
  }
  if (!KVARN) {
#pragma unroll
    for (int kk = 0; kk < OPT; ++kk) {
      const int i = tid + kk * PP_THREADS, h = i / D;
      if (h < a.gq) a.out[((int64_t)b * a.Hq + hq0) * D + i] = r_out[kk];
    }
  } else {
    // undo the channel scale c_V, then the rotation: v = H (c_V * v^) / sqrt(D)
    float* s_o = s_ow;
#pragma unroll
    for (int kk = 0; kk < OPT; ++kk) {
      const int i = tid + kk * PP_THREADS;
      s_o[i] = r_out[kk] * a.r.tab[1][(int64_t)u * D + i % D];
    }
    __syncthreads();
    for (int hs = 1; hs < D; hs <<= 1) {
      float v[OPT];
#pragma unroll
      for (int kk = 0; kk < OPT; ++kk) {
        const int i = tid + kk * PP_THREADS, d = i % D;
        const float mine = s_o[i], other = s_o[i ^ hs];
        v[kk] = (d & hs) ? other - mine : mine + other;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < OPT; ++kk) s_o[tid + kk * PP_THREADS] = v[kk];
      __syncthreads();
    }
    const float isd = (float)(1.0 / __builtin_sqrt(128.0));
    for (int i = tid; i < a.gq * D; i += PP_THREADS)
      a.out[((int64_t)b * a.Hq + hq0) * D + i] = s_o[i] * isd;
  }
  // ready for the next call (stream-ordered)
  if (tid == 0) __hip_atomic_store(&a.r.cnt[u], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int BITS, int NG, bool KVARN, int NPB>
static hipError_t launch_pp_one(const AttnArgs& a, hipStream_t s) {
  const int npat = pad_pat(KVARN ? 0 : a.n_pat);
  const PpLds L = pp_lds<BITS, NG, KVARN>(npat, NPB > 0);
  static int attr = 0;
  if (L.total > attr) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_pp_kernel<BITS, NG, KVARN, NPB>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, L.total);
    if (e != hipSuccess) return e;
    attr = L.total;
  }
  hipLaunchKernelGGL((attn_pp_kernel<BITS, NG, KVARN, NPB>), dim3(a.B * a.Hkv * a.splits),
                     dim3(PP_THREADS), L.total, s, a);
  return hipGetLastError();
}

template <int BITS, int NG>
static hipError_t launch_pp_bits_group(const AttnArgs& a, hipStream_t s) {
  if (a.mode == KVQ_MODE_KVARN) return launch_pp_one<BITS, NG, true, 0>(a, s);
  if (a.n_pat <= 0) return launch_pp_one<BITS, NG, false, 0>(a, s);
  if (a.n_pat <= 16) return launch_pp_one<BITS, NG, false, 1>(a, s);
  if (a.n_pat <= 32) return launch_pp_one<BITS, NG, false, 2>(a, s);
  if (a.n_pat <= 64) return launch_pp_one<BITS, NG, false, 4>(a, s);
  return launch_pp_one<BITS, NG, false, 0>(a, s);
}

hipError_t launch_attention_pp(const AttnArgs& a, hipStream_t s) {
  if (a.group == 32) return a.bits == 2 ? launch_pp_bits_group<2, 4>(a, s) : launch_pp_bits_group<4, 4>(a, s);
  return a.bits == 2 ? launch_pp_bits_group<2, 2>(a, s) : launch_pp_bits_group<4, 2>(a, s);
}

}  // namespace kvq
