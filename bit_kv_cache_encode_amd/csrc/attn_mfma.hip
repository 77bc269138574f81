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
//       only keeps the row of its own group.  z is summed on the side
//       (sum p z per group).
//  V pattern mass  w_j = sum_t p_t [k*_t = j]  is a third product: rows =
//       (head, part) with part 0/1 = binary16 hi/lo of p, columns = 16
//       patterns, reduction = 32 tokens, B = the one-hot matrix of the
//       tokens' pattern indices.  For more than 80 patterns it falls back to
//       LDS atomics.
//
// Codes enter the MFMA as binary16 subnormals: a 2-bit (4-bit) field masked
// in place (K) or rotated near the top of the mantissa first (V) is the
// integer code times 2^-24 times a power of two fixed by its position; the
// other operand carries the inverse power, so unpacking a pair of codes is
// one AND (plus a rotate per V word).  p*s is one binary16 operand in
// PatternKV mode and binary16 hi + lo parts (two MFMAs, about 22 bits) in the
// rotated modes, where the V sums cancel against the zero-point sums; q is one
// binary16 operand when it comes in bfloat16 (exact, see the exponent choice)
// and hi + lo otherwise; accumulation is fp32.
#include <type_traits>

#include "attn_mfma_common.h"
#include "encode_vec.h"

namespace kvq {

constexpr int MF_WAVES = 8;
constexpr int MF_THREADS = MF_WAVES * 64;

// A 16-byte tile load, non-temporal (the line is not kept for reuse) or not
template <bool NT>
__device__ __forceinline__ u32x4 tile_ld(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// Dynamic LDS layout of a block (bytes); npat = padded pattern count.
struct MfLds {
  int q, qsum, qe, next, qm, qa, ps, ph, vs, vz, w, alpha, m, o, z, l, wsum, M, last, tiles,
      nsn, mv, mv_rows, total;
};
// binary16 per row of the p hi / lo tables of the pattern-mass product
constexpr int PH_STRIDE = 72;
// hist_mfma: the pattern masses are a one-hot MFMA product (p hi / lo rows,
// V zero points staged per group)
// kch: K per channel, which keeps the per-lane q operands of the QK product
// (64 lanes x 32 fp32, quad-major) for the per-tile q * s operand
// nsn: NSN mode, which keeps q . mu_K and sum p n1 per head and the rotated
// V centre
__host__ __device__ inline MfLds mf_lds(int HB, int NG, int npat, int tile_bytes, bool hist_mfma,
                                        int mv_rows, bool kch = false, bool nsn = false) {
  MfLds L;
  int o = 0;
  L.q = o; o = al16(o + HB * D * 4);
  L.qsum = o; o = al16(o + HB * NG * 4);
  L.qe = o; o = al16(o + HB * 4);
  L.next = o; o = al16(o + 4);
  L.qm = o; o = al16(o + HB * 256 * 4);
  L.qa = o; o = al16(o + (kch ? 64 * 32 * 4 : 0));
  const int pw = HB == 4 ? ptab_words<4>() : ptab_words<8>();
  L.ps = o; o = al16(o + MF_WAVES * pw * 4);
  // one shared zero row, then per wave HB rows of p hi and HB rows of p lo
  L.ph = o; o = al16(o + (hist_mfma ? (1 + MF_WAVES * 2 * HB) * PH_STRIDE * 2 : 0));
  L.vs = o; o = al16(o + MF_WAVES * NG * VS_STRIDE * 2);
  L.vz = o; o = al16(o + (hist_mfma ? MF_WAVES * NG * VS_STRIDE * 2 : 0));
  L.w = o; o = al16(o + MF_WAVES * HB * npat * 4);
  L.alpha = o; o = al16(o + MF_WAVES * HB * 4);
  L.m = o; o = al16(o + MF_WAVES * HB * 4);
  L.o = o; o = al16(o + HB * D * 4);
  L.z = o; o = al16(o + HB * NG * 4);
  L.l = o; o = al16(o + HB * 4);
  L.wsum = o; o = al16(o + HB * npat * 4);
  L.M = o; o = al16(o + HB * 4);
  L.last = o; o = al16(o + 16);
  L.nsn = o; o = al16(o + (nsn ? (2 * HB + D) * 4 : 0));
  // the tile buffers, reused after the loop for per-wave o[HB][D] and (l, z[NG]
  // and with NSN sum p n1)
  const int part_bytes = MF_WAVES * HB * (D + 1 + NG + (nsn ? 1 : 0)) * 4;
  L.tiles = o; o = al16(o + (MF_WAVES * tile_bytes > part_bytes ? MF_WAVES * tile_bytes : part_bytes));
  // rows of M^V for the pattern term (one-hot path), where they fit the
  // 160 KiB of a compute unit
  L.mv = o;
  L.mv_rows = (hist_mfma && o + mv_rows * D * 4 <= 160 * 1024) ? mv_rows : 0;
  o = al16(o + L.mv_rows * D * 4);
  L.total = o;
  return L;
}

// Pattern-mass path: NPB > 0 -> one-hot MFMA over NPB blocks of 16 patterns;
// NPB == 0 -> LDS atomics (or no pattern term at all for KVarN).
// QLO: q needs a binary16 lo part (binary32 queries, or the KVarN rotation);
// a bfloat16 query is a single binary16 operand (see the exponent choice).
// NGS: quantization groups stored per token.  NG = NGS normally; NG = 2 NGS
// splits each stored group into two virtual groups that share its (s, z)
// word (s (q_a . c_a + q_b . c_b) = s q_a . c_a + s q_b . c_b, and likewise
// for z and for p s, p z on the V side), which fills the 16 MFMA rows with
// 4 q-heads at G = 64 instead of leaving half of an 8-head row block idle.
// NTL: the tile copy takes non-temporal loads (chosen per launch).
template <int BITS, int NG, int NGS, bool KVARN, int NPB, bool QLO, bool KCH, bool NSNM, bool NTL>
__global__ void __launch_bounds__(MF_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_mfma_kernel(AttnArgs a) {
  static_assert(!(KVARN && NPB), "KVarN has no pattern term");
  static_assert(NG == NGS || NG == 2 * NGS, "a stored group spans one or two virtual groups");
  static_assert(!KCH || (!KVARN && QLO), "K per channel: PatternKV mode, q * s needs a lo part");
  static_assert(!NSNM || KVARN, "NSN is a rotated mode");
  using TS = TileShape<BITS, NGS, KVARN, KCH, NSNM>;
  // per-wave (l, z[NG]) partial rows, with NSN also sum p n1
  constexpr int LZ = 1 + NG + (NSNM ? 1 : 0);
  constexpr int VPS = NG / NGS;        // virtual groups per stored group
  constexpr int G = D / NG;            // channels per (virtual) group
  constexpr int HB = 16 / NG;          // heads per row block
  constexpr int CPG = 16 / NG;         // PV columns per group
  constexpr int SPL = 4 / NG;          // heads per lane in a 16x16 output
  constexpr int KW = BITS;             // dwords of a lane's 32-channel K slice
  // p * s as binary16 hi + lo (two PV products) in the rotated modes, whose
  // V sums cancel against the zero-point sums; one binary16 operand (an
  // fp16 P.V product with fp32 accumulation) otherwise
  constexpr bool PLO = KVARN;
  constexpr int VTB = VT * D * BITS / 8;
  extern __shared__ __attribute__((aligned(16))) unsigned char mf_raw[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = tid >> 6;
  const int j = lane >> 4, n16 = lane & 15;
  const int U = a.B * a.Hkv;
  // blocks: (unit, q-head block of HB heads, split); unit fastest so that all
  // blocks of a unit share an XCD
  const int n_hb = (a.gq + HB - 1) / HB;
  const int u = blockIdx.x % U, hb = (blockIdx.x / U) % n_hb, split = blockIdx.x / U / n_hb;
  const int b = u / a.Hkv, hk = u % a.Hkv, hq0 = hk * a.gq + hb * HB;
  const int gq = min(HB, a.gq - hb * HB);   // q-heads of this block
  const int cu = u * n_hb + hb;              // arrival counter of (unit, head block)
  const int t_begin = split == 0 ? 0 : a.chunk0 + (split - 1) * a.chunk;
  const int t_end = min(a.T, split == 0 ? a.chunk0 : t_begin + a.chunk);
  // fused decode step: split 0 also appends the new token and writes its
  // one-token partial into slot a.splits
  const bool fuse_here = a.fuse && split == 0;
  const int S_tot = a.splits + a.fuse;
  const int n_pat = KVARN ? 0 : a.n_pat;
  const int npat = pad_pat(n_pat);
  const MfLds Lo = mf_lds(HB, NG, npat, TS::BYTES, NPB > 0, 16 * NPB, KCH, NSNM);
  float* s_q = (float*)(mf_raw + Lo.q);            // [HB][D]
  float* s_qsum = (float*)(mf_raw + Lo.qsum);      // [HB][NG]
  int* s_qe = (int*)(mf_raw + Lo.qe);              // [HB]: max |q| bits, then the exponent
  int* s_next = (int*)(mf_raw + Lo.next);          // next unclaimed tile of the block
  float* s_qm = (float*)(mf_raw + Lo.qm);          // [HB][256]; entry 0xFF (no pattern) is 0
  float4* s_qa = (float4*)(mf_raw + Lo.qa);        // K per channel: [8 quads][64 lanes]
  float* s_qmu = (float*)(mf_raw + Lo.nsn);        // NSN: [HB] qscale (q . mu_K)
  float* s_s1 = s_qmu + HB;                        // NSN: [HB] block sum p n1
  float* s_muv = s_s1 + HB;                        // NSN: [D] Hadamard(mu_V) / sqrt(D)
  float* s_ps = (float*)(mf_raw + Lo.ps) + wave * ptab_words<HB>();
  // pattern-mass operand rows: p 2^15 as binary16 hi [HB][PH_STRIDE], then lo
  _Float16* s_phh = (_Float16*)(mf_raw + Lo.ph) + (1 + wave * 2 * HB) * PH_STRIDE;
  _Float16* s_phl = s_phh + HB * PH_STRIDE;
  _Float16* s_vs = (_Float16*)(mf_raw + Lo.vs) + wave * NG * VS_STRIDE;   // V scales [g][token]
  _Float16* s_vz = (_Float16*)(mf_raw + Lo.vz) + wave * NG * VS_STRIDE;   // V zero points [g][token]
  float* s_w = (float*)(mf_raw + Lo.w);            // [WAVES][HB][npat]
  float* s_alpha = (float*)(mf_raw + Lo.alpha);    // [WAVES][HB]
  float* s_m = (float*)(mf_raw + Lo.m);            // [WAVES][HB]
  float* s_o = (float*)(mf_raw + Lo.o);            // [HB][D]
  float* s_z = (float*)(mf_raw + Lo.z);            // [HB][NG]
  float* s_l = (float*)(mf_raw + Lo.l);            // [HB]
  float* s_wsum = (float*)(mf_raw + Lo.wsum);      // [HB][npat]
  float* s_M = (float*)(mf_raw + Lo.M);            // [HB]
  int* s_last = (int*)(mf_raw + Lo.last);
  unsigned char* tb = mf_raw + Lo.tiles + wave * TS::BYTES;
  float* wrow = s_w + wave * HB * npat;

  const uint8_t* kcodes = a.r.codes[0] + (int64_t)u * a.tcap * TS::KREC;
  const uint8_t* vcodes = a.r.codes[1] + (int64_t)u * a.tcap * TS::KREC;
  const uint8_t* ksz = (const uint8_t*)(a.r.sz[0] + (int64_t)u * a.tcap * NGS);
  const uint8_t* vsz = (const uint8_t*)(a.r.sz[1] + (int64_t)u * a.tcap * NGS);
  const uint8_t* kix_src = KVARN ? (const uint8_t*)(a.r.t16[0] + (int64_t)u * a.tcap)
                                 : a.r.idx[0] + (int64_t)u * a.tcap;
  const uint8_t* vix_src = KVARN ? (const uint8_t*)(a.r.t16[1] + (int64_t)u * a.tcap)
                                 : a.r.idx[1] + (int64_t)u * a.tcap;
  // NSN: the second norms follow the first in the tile's index section
  const uint8_t* kt2_src = (const uint8_t*)(a.r.t2[0] + (int64_t)u * a.tcap);
  const uint8_t* vt2_src = (const uint8_t*)(a.r.t2[1] + (int64_t)u * a.tcap);

  // ---------------------------------------------------------------- tile copy
  // K and V (s, z) words of a tile take 16-byte pieces P_KS and P_VS; where
  // both fit one 64-lane pass (groups of 64 channels) they share registers
  constexpr int P_VS = TILE * NGS * 4 / 16;
  constexpr bool SZ_PAIR = !KCH && TS::P_KS + P_VS <= 64;
  u32x4 rkc[TS::R_KC], rvc[TS::R_VC], rks, rvs, rix;
  // The tile words are read once: non-temporal loads where the launch asks
  // for them (see launch_one)
  constexpr bool NT = NTL;
  auto issue = [&](int tile) {
    const u32x4* kc = (const u32x4*)(kcodes + (int64_t)tile * TS::KREC);
    const u32x4* vc = (const u32x4*)(vcodes + (int64_t)(tile >> 5) * VTB);
#pragma unroll
    for (int r = 0; r < TS::R_KC; ++r) rkc[r] = tile_ld<NT>(&kc[lane + 64 * r]);
#pragma unroll
    for (int r = 0; r < TS::R_VC; ++r) rvc[r] = tile_ld<NT>(&vc[lane + 64 * r]);
    if constexpr (SZ_PAIR) {
      // K scales in lanes [0, P_KS), V scales in the lanes after them
      if (lane < TS::P_KS) rks = tile_ld<NT>(&((const u32x4*)(ksz + (int64_t)tile * NGS * 4))[lane]);
      else if (lane < TS::P_KS + P_VS) rks = tile_ld<NT>(&((const u32x4*)(vsz + (int64_t)tile * NGS * 4))[lane - TS::P_KS]);
    } else {
      if (lane < TS::P_KS) {
        // K per channel: the words of the tile's block (a tile never straddles
        // a block); those of an open block are not read
        const u32x4* ks = KCH ? (const u32x4*)(a.r.kbsz + ((int64_t)u * kch_blocks(a.tcap) + tile / KBLOCK) * D)
                              : (const u32x4*)(ksz + (int64_t)tile * NGS * 4);
        // (non-temporal in the pattern modes only: the rotated modes ran
        // 2.5% slower with these words so loaded)
        rks = tile_ld<NT && !KVARN>(&ks[lane]);
      }
      if (lane < P_VS) rvs = tile_ld<NT>(&((const u32x4*)(vsz + (int64_t)tile * NGS * 4))[lane]);
    }
    const int ix_bytes = KVARN ? 2 : 1;
    if (NSNM) {
      // [K t16 | K t2 | V t16 | V t2], 8 pieces each (one fixed source per
      // lane range: a select over the four would become a private table)
      constexpr int Q = TS::P_IX / 2;
      const int64_t o = (int64_t)tile * ix_bytes;
      if (lane < Q) rix = tile_ld<NT>(&((const u32x4*)(kix_src + o))[lane]);
      else if (lane < 2 * Q) rix = tile_ld<NT>(&((const u32x4*)(kt2_src + o))[lane - Q]);
      else if (lane < 3 * Q) rix = tile_ld<NT>(&((const u32x4*)(vix_src + o))[lane - 2 * Q]);
      else if (lane < 4 * Q) rix = tile_ld<NT>(&((const u32x4*)(vt2_src + o))[lane - 3 * Q]);
    } else if (lane < TS::P_IX) {
      rix = tile_ld<NT>(&((const u32x4*)(kix_src + (int64_t)tile * ix_bytes))[lane]);
    } else if (lane < 2 * TS::P_IX) {
      rix = tile_ld<NT>(&((const u32x4*)(vix_src + (int64_t)tile * ix_bytes))[lane - TS::P_IX]);
    }
  };
  auto commit = [&]() {
    u32x4* t4 = (u32x4*)tb;
#pragma unroll
    for (int r = 0; r < TS::R_KC; ++r) t4[TS::O_KC / 16 + kpiece<BITS>(lane + 64 * r)] = rkc[r];
#pragma unroll
    for (int r = 0; r < TS::R_VC; ++r) t4[TS::O_VC / 16 + vpiece(lane + 64 * r)] = rvc[r];
    if constexpr (SZ_PAIR) {
      if (lane < TS::P_KS) t4[TS::O_KS / 16 + lane] = rks;
      else if (lane < TS::P_KS + P_VS) t4[TS::O_VS / 16 + lane - TS::P_KS] = rks;
    } else {
      if (lane < TS::P_KS) t4[TS::O_KS / 16 + lane] = rks;
      if (lane < P_VS) t4[TS::O_VS / 16 + lane] = rvs;
    }
    if (lane < 2 * TS::P_IX) t4[TS::O_KI / 16 + lane] = rix;
  };

  // Prologue loads, oldest first: a wave waits for a load with a count of the
  // loads issued after it, so each can be used without waiting for the later
  // ones: q (one or two elements per thread), this thread's 32-channel slice
  // of pattern row tid / 4 of M^K (for q' . M^K), then the first tile.
  // q is read as one aligned dword for either input type and converted where
  // it is used
  constexpr int QPT = HB * D / MF_THREADS;
  uint32_t qraw[QPT];
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int i = tid + k * MF_THREADS, h = min(i / D, gq - 1), d = i % D;
    const int64_t e = ((int64_t)b * a.Hq + hq0 + h) * D + d;
    const uint32_t* qw = (const uint32_t*)a.q + (a.bf16 ? e >> 1 : e);
    qraw[k] = *qw;
  }
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
  // q goes to LDS before the first tile is issued: a wait for it then counts
  // only the loads after it (with the tile's loads behind a branch, the
  // count would fall back to waiting for every load)
  bool q_bad = false;   // an element outside the query domain
#pragma unroll
  for (int k = 0; k < QPT; ++k) {
    const int i = tid + k * MF_THREADS;
    const uint32_t bits = !a.bf16 ? qraw[k] : (i & 1) ? (qraw[k] & 0xFFFF0000u) : (qraw[k] << 16);
    const float qv = __builtin_bit_cast(float, bits);
    q_bad |= !(fabsf(qv) * a.qscale < KVQ_Q_LIMIT * 1.4426950408889634f);
    s_q[i] = i / D < gq ? qv : 0.0f;
    s_o[i] = 0.0f;
  }
  flag_domain(a.r.status, q_bad, KVQ_DOMAIN_Q);
  const int n_tiles = (t_end - t_begin + TILE - 1) / TILE;
  // in the fused step waves 0 and 1 of split 0 encode the new token first and
  // take their tiles from the counter afterwards
  // K per channel: a wave takes both tiles of a 128-token block (splits start
  // on block boundaries), so the q * s operand serves two tiles
  const int first = !fuse_here ? (KCH ? 2 * wave : wave)
                                : (wave < 2 ? n_tiles : (KCH ? 2 * (wave - 2) : wave - 2));
  if (first < n_tiles) issue(t_begin + TILE * first);
  // M^V rows for the pattern term go to LDS before the loop, so that the
  // merge after it reads no global memory.  They are loaded after the first
  // tile: the prologue's first round trip then carries only q and M^K.
  constexpr int MVL = NPB > 0 ? 16 * NPB * D / 4 / MF_THREADS : 1;   // float4 per thread
  float4 mvl[MVL];
  const bool stage_mv = NPB > 0 && Lo.mv_rows > 0;
  if (stage_mv) {
    const float4* mv4 = (const float4*)(a.r.tab[1] + pat_unit(a.r, u) * a.max_pat * D);
#pragma unroll
    for (int k = 0; k < MVL; ++k) {
      const int c = tid + k * MF_THREADS;    // float4 index over rows < 16 NPB
      mvl[k] = c < n_pat * (D / 4) ? mv4[c] : float4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }

  // ---------------------------------------------------------------- prologue
  for (int i = tid; i < MF_WAVES * HB * npat; i += MF_THREADS) s_w[i] = 0.0f;
  for (int i = tid; i < HB * npat; i += MF_THREADS) s_wsum[i] = 0.0f;
  for (int i = tid; i < HB * 256; i += MF_THREADS) s_qm[i] = 0.0f;
  if (tid < HB * NG) s_z[tid] = 0.0f;
  if (NPB > 0 && tid < PH_STRIDE) ((_Float16*)(mf_raw + Lo.ph))[tid] = (_Float16)0.0f;
  if (tid < HB) { s_l[tid] = 0.0f; s_qe[tid] = 0; }
  if (tid == 0) *s_next = fuse_here ? MF_WAVES - 2 : MF_WAVES;
  __syncthreads();
  if constexpr (NSNM) {
    // q . mu_K in the original space (the rotation is orthonormal): wave h
    // < HB reduces head h; the V centre is rotated like the V partials
    if (wave < HB) {
      const float* muk = a.r.tab[0] + (int64_t)u * D;
      float pq = __builtin_fmaf(s_q[wave * D + lane], muk[lane], s_q[wave * D + lane + 64] * muk[lane + 64]);
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) pq += __shfl_xor(pq, o, 64);
      if (lane == 0) s_qmu[wave] = pq * a.qscale;
    }
    if (tid < D) s_muv[tid] = a.r.tab[1][(int64_t)u * D + tid];
    __syncthreads();
    for (int hs = 1; hs < D; hs <<= 1) {
      float v = 0.0f;
      if (tid < D) v = (tid & hs) ? s_muv[tid ^ hs] - s_muv[tid] : s_muv[tid] + s_muv[tid ^ hs];
      __syncthreads();
      if (tid < D) s_muv[tid] = v;
      __syncthreads();
    }
    if (tid < D) s_muv[tid] *= (float)(1.0 / __builtin_sqrt(128.0));
  }
  if (KVARN) {
    for (int hs = 1; hs < D; hs <<= 1) {
      float v[HB * D / MF_THREADS];
#pragma unroll
      for (int k = 0; k < HB * D / MF_THREADS; ++k) {
        const int i = tid + k * MF_THREADS, d = i % D;
        const float mine = s_q[i], other = s_q[i ^ hs];
        v[k] = (d & hs) ? other - mine : mine + other;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < HB * D / MF_THREADS; ++k) s_q[tid + k * MF_THREADS] = v[k];
      __syncthreads();
    }
  }
  if constexpr (KVARN) {
    const float isd = (float)(1.0 / __builtin_sqrt(128.0));
    const float* ck = a.r.tab[0] + (int64_t)u * D;
    for (int i = tid; i < HB * D; i += MF_THREADS) {
      const float v = s_q[i];
      s_q[i] = NSNM ? v * isd : v * isd * ck[i % D];
    }
    __syncthreads();
  }
  // Per-head binary exponent e_h that puts max_d |q_hd| 2^e_h in [2^14, 2^15).
  // The QK A operand is q 2^(e_h - shift) in binary16 (shift <= 6): a
  // bfloat16 q (8 significant bits) is exact there except for elements below
  // the binary16 subnormal step 2^-24, whose error is then under 2^-24, i.e.
  // under 2^-38 of the largest operand.  Other queries add a lo part.  The
  // softmax scale is applied after the products.
  {
    // max |q_h| as binary32 bits (ordered like the values for x >= 0):
    // lanes of one head reduce, then one LDS max per wave and head
    constexpr int VPT = HB * D / MF_THREADS, TPH = D / VPT, RED = TPH < 64 ? TPH : 64;
    const int h = tid / TPH;
    float mx = 0.0f;
#pragma unroll
    for (int k = 0; k < VPT; ++k) mx = fmaxf(mx, fabsf(s_q[tid * VPT + k]));
#pragma unroll
    for (int o = 1; o < RED; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if (tid % RED == 0) atomicMax(&s_qe[h], __builtin_bit_cast(int, mx));
  }
  __syncthreads();
  if (tid < HB) {
    const int bits = s_qe[tid];
    const int ex = ((bits >> 23) & 0xFF) - 127;
    s_qe[tid] = bits > 0 ? min(14 - ex, 120) : 0;
  }
  // per-group sums of q': thread (h = tid/32) adds 4 channels, then lanes of a
  // group reduce (G/4 lanes per group)
  {
    const int h = tid >> 5, c0 = (tid & 31) * 4;
    float s = 0.0f;
    if (h < HB) s = (s_q[h * D + c0] + s_q[h * D + c0 + 1]) + (s_q[h * D + c0 + 2] + s_q[h * D + c0 + 3]);
    // sum over the G / 4 (8 or 16) aligned lanes of a group: DPP quad swaps,
    // then the half-row and row mirrors
    static_assert(G / 4 == 8 || G / 4 == 16, "groups of 32 or 64 channels");
    s += dpp_f<0xB1>(s);
    s += dpp_f<0x4E>(s);
    s += dpp_f<0x141>(s);
    if (G / 4 == 16) s += dpp_f<0x140>(s);
    if (h < HB && ((tid & 31) % (G / 4)) == 0) s_qsum[h * NG + c0 / G] = s * a.qscale;
  }
  // q' . M^K_j: four threads per pattern j (32 channels each), all heads;
  // patterns beyond the first MF_THREADS / 4 take further passes
  if (!KVARN && n_pat > 0) {
    // with the one-hot path (at most 80 patterns) one pass covers the table
    const int passes = NPB > 0 ? 1 : (n_pat + MF_THREADS / 4 - 1) / (MF_THREADS / 4);
    for (int pass = 0; pass < passes; ++pass) {
      const int j0 = pass * (MF_THREADS / 4);
      const int jj = j0 + qm_j;
      if (NPB == 0 && j0 > 0) {
#pragma unroll
        for (int k = 0; k < 8; ++k) mkr[k] = float4{0.0f, 0.0f, 0.0f, 0.0f};
        if (jj < n_pat) {
          const float4* m4 = (const float4*)(mk + (int64_t)jj * D + qm_part * 32);
#pragma unroll
          for (int k = 0; k < 8; ++k) mkr[k] = m4[k];
        }
      }
      // a wave holds patterns j0 + 16 wave .. + 15: waves past the table skip
      // the pass (a wave64 FMA takes its SIMD four cycles, live rows or not).
      // Every head row (rows of heads >= gq are zero and not stored), so the
      // heads' LDS reads and FMAs interleave; two FMA chains per dot, then
      // the four threads of a pattern sum with DPP quad swaps
      if (j0 + 16 * wave >= n_pat) continue;
#pragma unroll
      for (int h = 0; h < HB; ++h) {
        const float4* qh = (const float4*)(s_q + h * D + qm_part * 32);
        float sd[2] = {0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float4 qv = qh[k];
          float& acc = sd[k & 1];
          acc = __builtin_fmaf(qv.x, mkr[k].x, acc);
          acc = __builtin_fmaf(qv.y, mkr[k].y, acc);
          acc = __builtin_fmaf(qv.z, mkr[k].z, acc);
          acc = __builtin_fmaf(qv.w, mkr[k].w, acc);
        }
        float sdot = sd[0] + sd[1];
        sdot += dpp_f<0xB1>(sdot);
        sdot += dpp_f<0x4E>(sdot);
        if (qm_part == 0 && jj < n_pat) s_qm[h * 256 + jj] = sdot * a.qscale;
      }
    }
  }
  __syncthreads();

  // -1 and +0 the compiler cannot fold (qscale is finite)
  const float k_m1 = __builtin_fmaf(a.qscale, 0.0f, -1.0f);
  const float k_z = a.qscale * 0.0f;
  // QK A operands: row m = n16 -> (h, g); element i of chunk c -> channel.
  // K per channel: the operand is q * s with s the channel's scale in the
  // tile's block, so it is rebuilt per tile from this lane's q values, kept
  // in LDS with the power 2^(e_h - shift - KCH_E) (s < 2^13 in the input
  // domain, so q * s stays under 2^15).
  constexpr int KCH_E = 13;
  u32x4 aq_hi[4], aq_lo[QLO ? 4 : 1];
  if constexpr (KCH) {
    if (tid < 64) {
      const int h = n16 / NG, g = n16 % NG;
      const int eh = s_qe[h];
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int pq = 0; pq < 2; ++pq) {
          float v[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int i = 2 * (2 * pq + (k >> 1)) + (k & 1), ch = qk_channel<BITS>(j, c, i);
            v[k] = (ch / G == g) ? ldexpf(s_q[h * D + ch], eh - code_shift<BITS>(i) - KCH_E) : 0.0f;
          }
          s_qa[(2 * c + pq) * 64 + lane] = float4{v[0], v[1], v[2], v[3]};
        }
    }
    __syncthreads();
  } else {
    const int h = n16 / NG, g = n16 % NG;
    const int eh = s_qe[h];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        float v2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          // unconditional read and a select (no branch around the LDS read)
          const int i = 2 * p + e, ch = qk_channel<BITS>(j, c, i);
          const float qv = ldexpf(s_q[h * D + ch], eh - code_shift<BITS>(i));
          v2[e] = (ch / G == g) ? qv : 0.0f;
        }
        uint32_t hi, lo;
        split2(v2[0], v2[1], k_m1, hi, lo);
        aq_hi[c][p] = hi;
        if (QLO) aq_lo[QLO ? c : 0][p] = lo;
      }
    }
  }
  // QK output register r <-> row 4j + r = (head 4j/NG + r/NG, group r % NG)
  float qsum[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) qsum[r] = s_qsum[((4 * j + r) / NG) * NG + r % NG];
  const int head0 = (4 * j) / NG;   // head of register slot s is head0 + s
  // scale of the binary16 partial dots: 2^(24 - e_h) (code and q operand
  // powers) times the softmax scale
  float dsc[SPL];
#pragma unroll
  for (int s = 0; s < SPL; ++s) dsc[s] = a.qscale * ldexpf(1.0f, 24 + (KCH ? KCH_E : 0) - s_qe[head0 + s]);

  float m_run[SPL], l_run[SPL], zacc[4];
  // NSN: running sum_t p_t n1_t per head, and qscale (q . mu_K) per head
  float s1_run[SPL], qmu_r[SPL];
#pragma unroll
  for (int s = 0; s < SPL; ++s) { s1_run[s] = 0.0f; qmu_r[s] = NSNM ? s_qmu[head0 + s] : 0.0f; }
#pragma unroll
  for (int s = 0; s < SPL; ++s) { m_run[s] = -INFINITY; l_run[s] = 0.0f; }
#pragma unroll
  for (int r = 0; r < 4; ++r) zacc[r] = 0.0f;
  f32x4 oacc[8];
#pragma unroll
  for (int bb = 0; bb < 8; ++bb) oacc[bb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // pattern-mass accumulators: row 4j + r = (head head0 + r / NG, part r % NG)
  f32x4 hacc[NPB > 0 ? NPB : 1];
#pragma unroll
  for (int cb = 0; cb < (NPB > 0 ? NPB : 1); ++cb) hacc[cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // with the one-hot path the V zero-point sums sum_t p_t z_tg are a product
  // of the same p operand and a B of binary16 zero points: rows as hacc,
  // column g = group (columns >= NG repeat a group and are not read)
  f32x4 zm = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // hist A: this lane's row (head n16 / NG, part n16 % NG) reads the hi
  // (part 0) or lo (part 1) table of its head; other rows read the zero row
  const _Float16* ph_row = (n16 / NG >= gq || n16 % NG > 1)
                               ? (const _Float16*)(mf_raw + Lo.ph)
                               : (n16 % NG == 0 ? s_phh : s_phl) + (n16 / NG) * PH_STRIDE;

  // Tiles are handed out dynamically: each wave starts with tile `wave` and
  // claims its next one from the block counter while the current one is
  // computed, so the waves of the block finish together whatever their
  // issue priority.
  // (the wait for these rows falls with the wait for the first tile)
  if (stage_mv)
#pragma unroll
    for (int k = 0; k < MVL; ++k) ((float4*)(mf_raw + Lo.mv))[tid + k * MF_THREADS] = mvl[k];
  int cur = first;
  // K per channel: block whose q * s operand and z sums are in registers
  int kch_built = -1;
  float zq[SPL];
  if (fuse_here && wave < 2) {
    // ---- the new token (position a.enc.t0): wave 0 encodes K, wave 1 V,
    // with the one-token encode of the append path; then its dequantised
    // vector gives this token's own partial (m = its score, l = 1, o = v^).
    // KVarN stays in the rotated space of the tiles: score t * (q' . u^)
    // with q' the prologue's rotated, channel-scaled query and u^ = c s + z,
    // partial o = t u^ (the combine scales by c_V and rotates back).
    const EncodeArgs& e = a.enc;
    const int kind = wave;
    const int64_t uu = u;
    const float x0 = load_in(e.src[kind], uu * D + lane, e.bf16);
    const float x1 = load_in(e.src[kind], uu * D + lane + 64, e.bf16);
    float wl0 = 0.0f, wl1 = 0.0f, wh0 = 0.0f, wh1 = 0.0f;
    if (e.win_update && !e.r.pat_h && hb == 0) {
      const float* win = e.r.win[kind] + uu * 2 * D;
      wl0 = win[lane]; wl1 = win[lane + 64];
      wh0 = win[D + lane]; wh1 = win[D + lane + 64];
    }
    uint32_t c0, c1, w0, w1;
    int kidx;
    uint32_t t16;
    float* sx = (float*)tb;   // this wave's tile buffer is idle until its first tile
    encode_vector<true>(e, kind, uu, x0, x1, lane, sx, nullptr, uu, c0, c1, w0, w1, kidx, t16);
    // with several q-head blocks per unit, each block of split 0 appends the
    // token (the same bytes) for its own heads' partials; the first owns the
    // window's read-modify-write and closure
    token_append(e, kind, uu, e.t0, lane, x0, x1, wl0, wl1, wh0, wh1, c0, c1, w0, w1, kidx, t16,
                 hb == 0);
    float m0 = 0.0f, m1 = 0.0f;
    if (kidx != KVQ_INDEX_NONE) {
      const float* mrow = e.r.tab[kind] + (pat_unit(e.r, uu) * e.max_pat + kidx) * D;
      m0 = mrow[lane];
      m1 = mrow[lane + 64];
    }
    float xh0 = __builtin_fmaf((float)c0, bits2f((uint16_t)(w0 & 0xFFFFu)), bits2f((uint16_t)(w0 >> 16))) + m0;
    float xh1 = __builtin_fmaf((float)c1, bits2f((uint16_t)(w1 & 0xFFFFu)), bits2f((uint16_t)(w1 >> 16))) + m1;
    if (KCH && kind == 0) {
      // K per channel: the token stays in its open block as the binary16
      // residual this lane just stored, plus its pattern
      const uint16_t* slot = e.r.ktail + (uu * KBLOCK + e.t0 % KBLOCK) * D;
      xh0 = bits2f(slot[lane]) + m0;
      xh1 = bits2f(slot[lane + 64]) + m1;
    }
    if (KVARN) {
      const float tf = bits2f((uint16_t)t16);
      xh0 *= tf;
      xh1 *= tf;
    }
    float* mlp = a.r.ws + (int64_t)a.B * a.Hq * S_tot * D;
    for (int h = 0; h < gq; ++h) {
      const int64_t qrow = (int64_t)b * a.Hq + hq0 + h, row = qrow * S_tot + a.splits;
      if (kind == 0) {
        const float q0 = KVARN ? s_q[h * D + lane] : load_in(a.q, qrow * D + lane, a.bf16);
        const float q1 = KVARN ? s_q[h * D + lane + 64] : load_in(a.q, qrow * D + lane + 64, a.bf16);
        float dot = __builtin_fmaf(q0, xh0, q1 * xh1);
        dot = row_sum16(dot);
        dot = (rlane(dot, 0) + rlane(dot, 16)) + (rlane(dot, 32) + rlane(dot, 48));
        if (lane == 0) {
          __hip_atomic_store(&mlp[row * 2], dot * a.qscale, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(&mlp[row * 2 + 1], 1.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      } else {
        __hip_atomic_store(&a.r.ws[row * D + lane], xh0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&a.r.ws[row * D + lane + 64], xh1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    int nx = 0;
    if (lane == 0) nx = atomicAdd(s_next, 1);
    cur = __builtin_amdgcn_readfirstlane(nx) * (KCH ? 2 : 1);
    if (cur < n_tiles) issue(t_begin + TILE * cur);
  }
  for (; cur < n_tiles;) {
    const int tile = t_begin + TILE * cur;
    __builtin_amdgcn_wave_barrier();
    commit();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    int nxt = 0;
    if (KCH && (cur & 1) == 0 && cur + 1 < n_tiles) {
      nxt = cur + 1;
    } else {
      if (lane == 0) nxt = atomicAdd(s_next, 1);
      nxt = __builtin_amdgcn_readfirstlane(nxt);
      if (KCH) nxt *= 2;
    }
    if (nxt < n_tiles) issue(t_begin + TILE * nxt);
    cur = nxt;
    const int nvalid = t_end - tile;
    auto tile_body = [&](auto full_tag) {
      constexpr bool FULL = decltype(full_tag)::value;

    // ---- K per channel: a tile of a complete block rebuilds the operand
    // q * s (hi + lo) and its heads' sum_d q_d z_d; a tile of the open block
    // scores against the binary16 residuals instead (below).
    bool open_tile = false;
    if constexpr (KCH) {
      open_tile = tile >= a.kclosed;
      if (!open_tile && tile / KBLOCK != kch_built) {
        kch_built = tile / KBLOCK;
        const uint32_t* bw = (const uint32_t*)(tb + TS::O_KS);   // [D] (s | z << 16)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          // channels of elements (p, e): qk_channel(j, c, 2p + e), runs of 4 in p
          const u32x4 w0 = *(const u32x4*)(bw + qk_channel<BITS>(j, c, 0));
          const u32x4 w1 = *(const u32x4*)(bw + qk_channel<BITS>(j, c, 1));
          const float4 qa0 = s_qa[(2 * c) * 64 + lane], qa1 = s_qa[(2 * c + 1) * 64 + lane];
          const float qv[8] = {qa0.x, qa0.y, qa0.z, qa0.w, qa1.x, qa1.y, qa1.z, qa1.w};
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const float x0 = mul_h(qv[2 * p], (uint16_t)(w0[p] & 0xFFFFu), k_z);
            const float x1 = mul_h(qv[2 * p + 1], (uint16_t)(w1[p] & 0xFFFFu), k_z);
            uint32_t hi, lo;
            split2(x0, x1, k_m1, hi, lo);
            aq_hi[c][p] = hi;
            aq_lo[QLO ? c : 0][p] = lo;
          }
        }
        // sum_d q_hd z_d: channels 8 n16 .. 8 n16 + 7 per lane, summed over the row
        const u32x4 z0 = *(const u32x4*)(bw + 8 * n16), z1 = *(const u32x4*)(bw + 8 * n16 + 4);
#pragma unroll
        for (int s = 0; s < SPL; ++s) {
          const float4 q0 = *(const float4*)(s_q + (head0 + s) * D + 8 * n16);
          const float4 q1 = *(const float4*)(s_q + (head0 + s) * D + 8 * n16 + 4);
          float acc = mul_h(q0.x, (uint16_t)(z0[0] >> 16), k_z);
          acc = __builtin_fmaf(q0.y, bits2f((uint16_t)(z0[1] >> 16)), acc);
          acc = __builtin_fmaf(q0.z, bits2f((uint16_t)(z0[2] >> 16)), acc);
          acc = __builtin_fmaf(q0.w, bits2f((uint16_t)(z0[3] >> 16)), acc);
          acc = __builtin_fmaf(q1.x, bits2f((uint16_t)(z1[0] >> 16)), acc);
          acc = __builtin_fmaf(q1.y, bits2f((uint16_t)(z1[1] >> 16)), acc);
          acc = __builtin_fmaf(q1.z, bits2f((uint16_t)(z1[2] >> 16)), acc);
          acc = __builtin_fmaf(q1.w, bits2f((uint16_t)(z1[3] >> 16)), acc);
          zq[s] = row_sum16(acc) * a.qscale;
        }
      }
    }
    // ---- QK: four independent accumulators (one per 16-token column block)
    // so consecutive MFMAs never wait on each other.
    f32x4 C[4] = {};
    if (!open_tile) {
      // this lane's K words of column block nb: 32 channels of token 16 nb + n16
      auto load_kw = [&](int nb, uint32_t* kw) {
        const int t64 = 16 * nb + n16;
        if (KW == 2) {
          const uint2 w = *(const uint2*)(tb + TS::O_KC + kpiece<BITS>(2 * t64 + (j >> 1)) * 16 + (j & 1) * 8);
          kw[0] = w.x; kw[1 % KW] = w.y;
        } else {
          const u32x4 w = *(const u32x4*)(tb + TS::O_KC + kpiece<BITS>(4 * t64 + j) * 16);
#pragma unroll
          for (int q = 0; q < KW; ++q) kw[q] = w[q];
        }
      };
      // two column blocks at a time: their K words (2 KW dwords) are live
      // through the chunk loop, and the two accumulator chains alternate
#pragma unroll
      for (int np = 0; np < 4; np += 2) {
        uint32_t kw[2][KW];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          load_kw(np + e, kw[e]);
          C[np + e] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const u32x4 B = unpack_k<BITS>(kw[e], c);
            C[np + e] = mfma16(aq_hi[c], B, C[np + e]);
            if constexpr (QLO) C[np + e] = mfma16(aq_lo[QLO ? c : 0], B, C[np + e]);
          }
      }
    }
    float sc[4][SPL];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int t64 = 16 * nb + n16;
      const bool valid = FULL || t64 < nvalid;
      if constexpr (KCH) {
        const int kix = tb[TS::O_KI + t64];   // 0xFF (no pattern) reads a 0 entry
#pragma unroll
        for (int s = 0; s < SPL; ++s) {
          const float qm = s_qm[(head0 + s) * 256 + kix];
          float v;
          if (!open_tile) {
            float dot = 0.0f;
#pragma unroll
            for (int g = 0; g < NG; ++g) dot += C[nb][s * NG + g];
            v = __builtin_fmaf(dot, dsc[s], zq[s] + qm);
          } else {
            // open block: q . residual over the whole vector (a rare tile)
            const uint4* res = (const uint4*)(a.r.ktail + ((int64_t)u * KBLOCK + (tile + t64) % KBLOCK) * D);
            const float* qh = s_q + (head0 + s) * D;
            float acc = 0.0f;
            for (int d8 = 0; d8 < D / 8; ++d8) {
              const uint4 r8 = res[d8];
              const uint32_t rw[4] = {r8.x, r8.y, r8.z, r8.w};
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                acc = __builtin_fmaf(qh[8 * d8 + 2 * k], bits2f((uint16_t)(rw[k] & 0xFFFFu)), acc);
                acc = __builtin_fmaf(qh[8 * d8 + 2 * k + 1], bits2f((uint16_t)(rw[k] >> 16)), acc);
              }
            }
            v = __builtin_fmaf(acc, a.qscale, qm);
          }
          sc[nb][s] = valid ? v : -INFINITY;
        }
        continue;
      }
      uint32_t kszw[NG];   // (s, z) word of each virtual group
      {
        const uint32_t* kszp = (const uint32_t*)(tb + TS::O_KS) + t64 * NGS;
        if (NGS == 4) {
          const u32x4 k4 = *(const u32x4*)kszp;
#pragma unroll
          for (int g = 0; g < NG; ++g) kszw[g] = k4[g];
        } else {
          const uint2 k2 = *(const uint2*)kszp;
#pragma unroll
          for (int g = 0; g < NG; ++g) kszw[g] = g / VPS == 0 ? k2.x : k2.y;
        }
      }
      float tk = 1.0f, tk1 = 0.0f;
      int kix = KVQ_INDEX_NONE;
      if (KVARN) {
        tk = bits2f(((const uint16_t*)(tb + TS::O_KI))[t64]);
        if (NSNM) {
          // NSN: k^ rotated = n1 n2 (s c + z) + n1 Hadamard(mu_K) / sqrt(D)
          tk1 = tk;
          tk *= bits2f(((const uint16_t*)(tb + TS::O_KI + 2 * TILE))[t64]);
        }
      } else {
        kix = tb[TS::O_KI + t64];   // 0xFF (no pattern) reads a 0 entry
      }
#pragma unroll
      for (int s = 0; s < SPL; ++s) {
        // the pattern term (q . M^K)[k*] starts the zero-point sum
        float dot = 0.0f, zt = KVARN ? 0.0f : s_qm[(head0 + s) * 256 + kix];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const int r = s * NG + g;
          dot = __builtin_fmaf(bits2f((uint16_t)(kszw[g] & 0xFFFFu)), C[nb][r], dot);
          zt = __builtin_fmaf(bits2f((uint16_t)(kszw[g] >> 16)), qsum[r], zt);
        }
        float v = __builtin_fmaf(dot, dsc[s], zt);
        if (KVARN) v = NSNM ? __builtin_fmaf(v, tk, tk1 * qmu_r[s]) : v * tk;
        sc[nb][s] = valid ? v : -INFINITY;
      }
    }

    // ---- online softmax (log2 domain); rescale only when a max grows.  A
    // max grows exactly when one of its lanes holds a larger score, so a
    // vote over the lanes' own maxima decides, and the row maxima are
    // reduced across lanes only then
    float lmax[SPL];
    bool grow = false;
#pragma unroll
    for (int s = 0; s < SPL; ++s) {
      lmax[s] = fmaxf(fmaxf(sc[0][s], sc[1][s]), fmaxf(sc[2][s], sc[3][s]));
      grow |= lmax[s] > m_run[s];
    }
    if (__any(grow)) {
      float al[SPL];
#pragma unroll
      for (int s = 0; s < SPL; ++s) {
        const float mnew = fmaxf(m_run[s], row_max16(lmax[s]));
        al[s] = __builtin_amdgcn_exp2f(m_run[s] - mnew);
        l_run[s] *= al[s];
        if constexpr (NSNM) s1_run[s] *= al[s];
        m_run[s] = mnew;
      }
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
#pragma unroll
        for (int r = 0; r < 4; ++r) zm[r] *= al[r / NG];
      } else if (!KVARN && n_pat > 0) {
        if (n16 == 0)
#pragma unroll
          for (int s = 0; s < SPL; ++s) s_alpha[wave * HB + head0 + s] = al[s];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        for (int e = lane; e < gq * npat; e += 64) wrow[e] *= s_alpha[wave * HB + e / npat];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
    float pk[4][SPL];
    int vk[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int t64 = 16 * nb + n16;
      const bool valid = FULL || t64 < nvalid;
      uint32_t vszz[NG];
      if constexpr (NPB == 0) {
        const uint32_t* vszp = (const uint32_t*)(tb + TS::O_VS) + t64 * NGS;
        if (NGS == 4) {
          const u32x4 v4 = *(const u32x4*)vszp;
#pragma unroll
          for (int g = 0; g < NG; ++g) vszz[g] = valid ? v4[g] : 0u;
        } else {
          const uint2 v2 = *(const uint2*)vszp;
#pragma unroll
          for (int g = 0; g < NG; ++g) vszz[g] = valid ? (g / VPS == 0 ? v2.x : v2.y) : 0u;
        }
      }
      float tv = 1.0f, tn1 = 0.0f;
      int vix = KVQ_INDEX_NONE;
      if (KVARN) {
        const float t = bits2f(((const uint16_t*)(tb + TS::O_VI))[t64]);
        tv = valid ? t : 0.0f;
        if (NSNM) {
          // NSN: v^ rotated = n1 n2 (s c + z) + n1 Hadamard(mu_V) / sqrt(D)
          tn1 = tv;
          tv *= bits2f(((const uint16_t*)(tb + TS::O_VI + 2 * TILE))[t64]);
        }
      } else {
        const int vi = tb[TS::O_VI + t64];
        vix = valid ? vi : KVQ_INDEX_NONE;
      }
#pragma unroll
      for (int s = 0; s < SPL; ++s) {
        const float p = __builtin_amdgcn_exp2f(sc[nb][s] - m_run[s]);
        l_run[s] += p;
        if constexpr (NSNM) s1_run[s] = __builtin_fmaf(p, tn1, s1_run[s]);
        const float pt = p * tv;              // KVarN: v^ carries the token scale t
        if constexpr (NPB == 0)
#pragma unroll
          for (int g = 0; g < NG; ++g)
            zacc[s * NG + g] = __builtin_fmaf(pt, bits2f((uint16_t)(vszz[g] >> 16)), zacc[s * NG + g]);
        pk[nb][s] = p;
        s_ps[prow<HB>(head0 + s) + t64] = ldexpf(pt, pv_ep<BITS, KVARN>() - pv_shift<BITS, KVARN>(t64 & 31));
        if constexpr (NPB > 0) {
          // p * 2^15 <= 2^15 as binary16 hi + lo (round to nearest even)
          const float x = p * 32768.0f;
          const _Float16 hi = (_Float16)x;
          const _Float16 lo = (_Float16)__builtin_fmaf((float)hi, k_m1, x);
          s_phh[(head0 + s) * PH_STRIDE + t64] = hi;
          s_phl[(head0 + s) * PH_STRIDE + t64] = lo;
        }
      }
      vk[nb] = vix;
      // V group scale of this token for group j (lanes j < NG)
      if (j < NG) {
        const uint32_t sw = ((const uint32_t*)(tb + TS::O_VS))[t64 * NGS + j / VPS];
        s_vs[j * VS_STRIDE + t64] = __builtin_bit_cast(_Float16, (uint16_t)(valid ? sw & 0xFFFFu : 0u));
        if constexpr (NPB > 0)
          s_vz[j * VS_STRIDE + t64] = __builtin_bit_cast(_Float16, (uint16_t)(valid ? sw >> 16 : 0u));
      }
    }
    // V pattern mass: the tile's LDS adds are issued back to back so their
    // latencies overlap (nothing reads LDS between them)
    if (!KVARN && NPB == 0 && n_pat > 0) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int s = 0; s < SPL; ++s)
          if (vk[nb] != KVQ_INDEX_NONE && head0 + s < gq)
            atomicAdd(&wrow[(head0 + s) * npat + vk[nb]], pk[nb][s]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- PV over the two 32-token V tiles
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      u32x4 ahi, alo = {};
      {
        // rows of heads >= gq hold finite values that are never stored
        const int h = n16 / NG, g = n16 % NG;
        // element (p, e) of this lane reads token base + p + e*off: two runs of
        // four consecutive tokens
        const int base = 32 * kb + pv_token<BITS>(j, 0), off = pv_token<BITS>(j, 1) - pv_token<BITS>(j, 0);
        const float4 p0 = *(const float4*)(s_ps + prow<HB>(h) + base);
        const float4 p1 = *(const float4*)(s_ps + prow<HB>(h) + base + off);
        const uint2 v0 = *(const uint2*)(s_vs + g * VS_STRIDE + base);
        const uint2 v1 = *(const uint2*)(s_vs + g * VS_STRIDE + base + off);
        const float pa[4] = {p0.x, p0.y, p0.z, p0.w}, pb[4] = {p1.x, p1.y, p1.z, p1.w};
        const uint32_t va[2] = {v0.x, v0.y}, vb[2] = {v1.x, v1.y};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float x0 = mul_h(pa[p], (uint16_t)(va[p >> 1] >> (16 * (p & 1))), k_z);
          const float x1 = mul_h(pb[p], (uint16_t)(vb[p >> 1] >> (16 * (p & 1))), k_z);
          if constexpr (PLO) {
            uint32_t hi, lo;
            split2(x0, x1, k_m1, hi, lo);
            ahi[p] = hi;
            alo[p] = lo;
          } else {
            ahi[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x0, x1}, f16x2));
          }
        }
      }
      if constexpr (NPB > 0) {
        // element i = 2p + e of lane group j <-> token 32 kb + 8 j + i
        const u32x4 ah = *(const u32x4*)(ph_row + 32 * kb + 8 * j);
        // pattern indices of tokens 2p, 2p + 1 in the high bytes of the two halves
        const uint2 vw = *(const uint2*)(tb + TS::O_VI + 32 * kb + 8 * j);
        uint32_t pr[4];
        pr[0] = __builtin_amdgcn_perm(0u, vw.x, 0x010C000Cu);
        pr[1] = __builtin_amdgcn_perm(0u, vw.x, 0x030C020Cu);
        pr[2] = __builtin_amdgcn_perm(0u, vw.y, 0x010C000Cu);
        pr[3] = __builtin_amdgcn_perm(0u, vw.y, 0x030C020Cu);
#pragma unroll
        for (int cb = 0; cb < NPB; ++cb) {
          // B = 2^-16 (binary16 0x0100: the top of the mantissa, where the
          // dot product's alignment keeps it whole) where the index equals
          // this column's pattern, else 0
          const u16x2 tgt = u16x2{(uint16_t)((16 * cb + n16) << 8), (uint16_t)((16 * cb + n16) << 8)};
          u32x4 B;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u16x2 d = __builtin_bit_cast(u16x2, pr[q]) ^ tgt;
            B[q] = __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(u16x2{0x100, 0x100}, d));
          }
          hacc[cb] = mfma16(ah, B, hacc[cb]);
        }
        // B = zero points z_tg (binary16) of the same tokens for group
        // n16 % NG, staged per group like the scales (0 past the end)
        const u32x4 bz = *(const u32x4*)(s_vz + (n16 % NG) * VS_STRIDE + 32 * kb + 8 * j);
        zm = mfma16(ah, bz, zm);
      }
      // this lane's word of channels 8*n16 .. 8*n16+7 (word-major V tile)
      const int word = BITS == 2 ? (j >> 1) : j;
      // pieces 2 n16 and 2 n16 + 1 of this word's block, stored swapped for n16 >= 8
      const u32x4* vp = (const u32x4*)(tb + TS::O_VC + kb * VTB) + word * (D / 4) + 2 * n16;
      const int vk = (n16 >> 3) & 1;
      const u32x4 w0 = vp[vk], w1 = vp[vk ^ 1];
#pragma unroll
      for (int bb = 0; bb < 8; ++bb) {
        const u32x4 B = unpack_v<BITS, KVARN>(bb < 4 ? w0[bb] : w1[bb - 4], j);
        oacc[bb] = mfma16(ahi, B, oacc[bb]);
        if constexpr (PLO) oacc[bb] = mfma16(alo, B, oacc[bb]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      };
    if (nvalid >= TILE) tile_body(std::true_type{});
    else tile_body(std::false_type{});
  }

  // ---------------------------------------------------------------- merge waves
  // Without staged M^V rows: the M^V column of this thread's first output row
  // (the pattern term), read from global memory now so that the loads overlap
  // the merge below.
  const float* mv = a.r.tab[1] + pat_unit(a.r, u) * a.max_pat * D;
  constexpr int MVR = NPB > 0 ? 16 * NPB : 1;
  float mvr[MVR];
  const float* s_mv = (const float*)(mf_raw + Lo.mv);   // [16 NPB][D] when staged
  if constexpr (NPB > 0) {
    if (!stage_mv)
#pragma unroll
      for (int jj = 0; jj < MVR; ++jj) mvr[jj] = jj < n_pat ? mv[(int64_t)jj * D + tid % D] : 0.0f;
  }
#pragma unroll
  for (int s = 0; s < SPL; ++s) l_run[s] = row_sum16(l_run[s]);
  if constexpr (NSNM)
#pragma unroll
    for (int s = 0; s < SPL; ++s) s1_run[s] = row_sum16(s1_run[s]);
  if constexpr (NPB == 0)
#pragma unroll
    for (int r = 0; r < 4; ++r) zacc[r] = row_sum16(zacc[r]);
  if (n16 == 0)
#pragma unroll
    for (int s = 0; s < SPL; ++s) s_m[wave * HB + head0 + s] = m_run[s];
  __syncthreads();
  if (tid < HB) {
    float M = -INFINITY;
    for (int w = 0; w < MF_WAVES; ++w) M = fmaxf(M, s_m[w * HB + tid]);
    s_M[tid] = M;
  }
  __syncthreads();
  float f[SPL];
#pragma unroll
  for (int s = 0; s < SPL; ++s)
    f[s] = (m_run[s] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run[s] - s_M[head0 + s]);
  // Per-wave partials, relative to the block max, with plain LDS stores into
  // the tile region (free now): o [WAVES][HB][D], then (l, z[NG]) per row.
  float* s_ow = (float*)(mf_raw + Lo.tiles);
  float* s_lz = s_ow + MF_WAVES * HB * D;
  {
    const float oscale = (float)(1 << (24 - pv_ep<BITS, KVARN>()));
    const int gcol = n16 / CPG;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r % NG != gcol) continue;
      const int s = r / NG;
      const float sc = oscale * f[s];
      float* dst = s_ow + (wave * HB + head0 + s) * D + 8 * n16;
      *(float4*)dst = float4{oacc[0][r] * sc, oacc[1][r] * sc, oacc[2][r] * sc, oacc[3][r] * sc};
      *(float4*)(dst + 4) = float4{oacc[4][r] * sc, oacc[5][r] * sc, oacc[6][r] * sc, oacc[7][r] * sc};
    }
#pragma unroll
    for (int s = 0; s < SPL; ++s) {
      float* lz = s_lz + (wave * HB + head0 + s) * LZ;
      if (n16 == 0) {
        lz[0] = f[s] * l_run[s];
        if constexpr (NSNM) lz[1 + NG] = f[s] * s1_run[s];
        if constexpr (NPB == 0)
#pragma unroll
          for (int g = 0; g < NG; ++g) lz[1 + g] = f[s] * zacc[s * NG + g];
      }
      // zm rows (head, hi | lo) carry p 2^15
      if constexpr (NPB > 0)
        if (n16 < NG) lz[1 + n16] = (zm[s * NG] + zm[s * NG + 1]) * (f[s] * (1.0f / 32768.0f));
    }
  }
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
  } else if (!KVARN && n_pat > 0) {
    if (n16 == 0)
#pragma unroll
      for (int s = 0; s < SPL; ++s) s_alpha[wave * HB + head0 + s] = f[s];
  }
  __syncthreads();
  // block totals: pattern masses w[h][j], l[h], z[h][g]
  if (!KVARN && n_pat > 0)
    for (int e = tid; e < gq * npat; e += MF_THREADS) {
      const int h = e / npat;
      float acc = 0.0f;
#pragma unroll
      for (int w = 0; w < MF_WAVES; ++w) {
        const float x = s_w[(w * HB) * npat + e];
        acc = NPB > 0 ? acc + x : __builtin_fmaf(s_alpha[w * HB + h], x, acc);
      }
      s_wsum[e] = acc;
    }
  if (tid < HB * LZ) {
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < MF_WAVES; ++w) acc += s_lz[w * HB * LZ + tid];
    const int h = tid / LZ, k = tid % LZ;
    if (k == 0) s_l[h] = acc;
    else if (k <= NG) s_z[h * NG + k - 1] = acc;
    else s_s1[h] = acc;
  }
  __syncthreads();

  // ---------------------------------------------------------------- partial out
  // Row (b, head, split): o + z + sum_j w_j M^V_j and (M, l), all relative
  // to this split's max M.  Stores are agent-scope atomics (coherent across
  // the XCDs' L2s), so publishing them needs only their completion.
  const int S = S_tot;
  float* ml = a.r.ws + (int64_t)a.B * a.Hq * S * D;
  for (int i = tid; i < gq * D; i += MF_THREADS) {
    const int h = i / D, d = i % D;
    const int64_t row = ((int64_t)b * a.Hq + hq0 + h) * S + split;
    float o = s_z[h * NG + d / G];
    // NSN: the centre term sum_t p_t n1_t Hadamard(mu_V) / sqrt(D)
    if constexpr (NSNM) o = __builtin_fmaf(s_s1[h], s_muv[d], o);
#pragma unroll
    for (int w = 0; w < MF_WAVES; ++w) o += s_ow[(w * HB + h) * D + d];
    if constexpr (NPB > 0) {
      // staged rows in LDS; else the first output row of this thread uses
      // the registers loaded above (separate loops keep each one's loads in
      // a single address space).  Both hold zeros in the rows from n_pat up
      // to 16 NPB, so these loops run to 16 NPB without a test per row (a
      // branch per row would make each LDS read wait for the previous one);
      // past the padded pattern count the weight index is clamped, and the
      // finite weight times the zero row adds +-0.
      if (stage_mv) {
#pragma unroll
        for (int jj = 0; jj < MVR; ++jj)
          o = __builtin_fmaf(s_wsum[h * npat + min(jj, npat - 1)], s_mv[jj * D + d], o);
      } else if (i == tid) {
#pragma unroll
        for (int jj = 0; jj < MVR; ++jj)
          o = __builtin_fmaf(s_wsum[h * npat + min(jj, npat - 1)], mvr[jj], o);
      } else {
#pragma unroll
        for (int jj = 0; jj < MVR; ++jj)
          if (jj < n_pat) o = __builtin_fmaf(s_wsum[h * npat + jj], mv[(int64_t)jj * D + d], o);
      }
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
  // arrives last (it observes splits - 1 earlier increments, each made after
  // that split's stores completed) merges all partials of the unit (the
  // splits', and in the fused step the new token's, written by split 0
  // before it counted itself in) with agent-scope loads.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&a.r.cnt[cu], 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    *s_last = prev == (uint32_t)(a.splits - 1);
  }
  __syncthreads();
  if (!*s_last) return;
  // out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s, with a running max
  // over chunks of CC splits.  The partials of other blocks are read with
  // agent-scope loads, each a long round trip, so a chunk issues all of its
  // loads before it uses any: one round trip per chunk.  (m, l) is one
  // 64-bit load; the lanes of a wave share its address (one head per wave).
  constexpr int OPT = HB * D / MF_THREADS;   // outputs per thread
  constexpr int CC = 32 / OPT;               // splits per chunk
  float Mr[OPT], Lr[OPT], Or[OPT];
#pragma unroll
  for (int k = 0; k < OPT; ++k) { Mr[k] = -INFINITY; Lr[k] = 0.0f; Or[k] = 0.0f; }
  for (int c0 = 0; c0 < S; c0 += CC) {
    const int n = min(CC, S - c0);
    uint64_t mlw[OPT][CC];
    float oo[OPT][CC];
#pragma unroll
    for (int k = 0; k < OPT; ++k) {
      // rows of heads >= gq repeat head gq - 1 and are not stored
      const int i = tid + k * MF_THREADS, h = min(i / D, gq - 1), d = i % D;
      const int64_t row0 = ((int64_t)b * a.Hq + hq0 + h) * S + c0;
#pragma unroll
      for (int e = 0; e < CC; ++e) {
        mlw[k][e] = 0xFF800000u;   // (m, l) = (-inf, 0) past the last split
        oo[k][e] = 0.0f;
        if (e < n) {
          mlw[k][e] = __hip_atomic_load((const uint64_t*)(ml + (row0 + e) * 2), __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
          oo[k][e] = __hip_atomic_load(&a.r.ws[(row0 + e) * D + d], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < OPT; ++k) {
      float cm = Mr[k];
#pragma unroll
      for (int e = 0; e < CC; ++e) cm = fmaxf(cm, __builtin_bit_cast(float, (uint32_t)mlw[k][e]));
      const float rs = Mr[k] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(Mr[k] - cm);
      Lr[k] *= rs;
      Or[k] *= rs;
#pragma unroll
      for (int e = 0; e < CC; ++e) {
        const float mm = __builtin_bit_cast(float, (uint32_t)mlw[k][e]);
        const float ll = __builtin_bit_cast(float, (uint32_t)(mlw[k][e] >> 32));
        const float fs = mm == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mm - cm);
        Lr[k] = __builtin_fmaf(ll, fs, Lr[k]);
        Or[k] = __builtin_fmaf(oo[k][e], fs, Or[k]);
      }
      Mr[k] = cm;
    }
  }
  float r_out[OPT];
#pragma unroll
  for (int k = 0; k < OPT; ++k) r_out[k] = Or[k] / Lr[k];
  if (!KVARN) {
#pragma unroll
    for (int k = 0; k < OPT; ++k) {
      const int i = tid + k * MF_THREADS, h = i / D;
      if (h < gq) a.out[((int64_t)b * a.Hq + hq0) * D + i] = r_out[k];
    }
  } else {
    // undo the channel scale c_V, then the rotation: v = H (c_V * v^) / sqrt(D)
#pragma unroll
    for (int k = 0; k < OPT; ++k) {
      const int i = tid + k * MF_THREADS;
      s_o[i] = NSNM ? r_out[k] : r_out[k] * a.r.tab[1][(int64_t)u * D + i % D];
    }
    __syncthreads();
    for (int hs = 1; hs < D; hs <<= 1) {
      float v[HB * D / MF_THREADS];
#pragma unroll
      for (int k = 0; k < HB * D / MF_THREADS; ++k) {
        const int i = tid + k * MF_THREADS, d = i % D;
        const float mine = s_o[i], other = s_o[i ^ hs];
        v[k] = (d & hs) ? other - mine : mine + other;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < HB * D / MF_THREADS; ++k) s_o[tid + k * MF_THREADS] = v[k];
      __syncthreads();
    }
    const float isd = (float)(1.0 / __builtin_sqrt(128.0));
    for (int i = tid; i < gq * D; i += MF_THREADS)
      a.out[((int64_t)b * a.Hq + hq0) * D + i] = s_o[i] * isd;
  }
  // ready for the next call (stream-ordered)
  if (tid == 0) __hip_atomic_store(&a.r.cnt[cu], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int BITS, int NG, int NGS, bool KVARN, int NPB, bool QLO, bool KCH, bool NSNM, bool NTL>
static hipError_t launch_impl(const AttnArgs& a, hipStream_t s) {
  using K = void (*)(AttnArgs);
  const K fn = attn_mfma_kernel<BITS, NG, NGS, KVARN, NPB, QLO, KCH, NSNM, NTL>;
  constexpr int HB = 16 / NG;
  const int npat = pad_pat(KVARN ? 0 : a.n_pat);
  const MfLds L = mf_lds(HB, NG, npat, TileShape<BITS, NGS, KVARN, KCH, NSNM>::BYTES, NPB > 0, 16 * NPB, KCH, NSNM);
  static int attr = 0;
  if (L.total > attr) {
    hipError_t e = hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, L.total);
    if (e != hipSuccess) return e;
    attr = L.total;
  }
  const int n_hb = (a.gq + HB - 1) / HB;
  hipLaunchKernelGGL(fn, dim3(a.B * a.Hkv * a.splits * n_hb), dim3(MF_THREADS), L.total, s, a);
  return hipGetLastError();
}

// Non-temporal tile loads where they measured faster: 2-bit codes with K per
// token (4-6% per call).  The 4-bit and K-per-channel variants keep ordinary
// loads, which time faster there, and so do units with several q-head blocks,
// whose blocks after the first read the unit's tiles from L2 (non-temporal
// lines leave it early: 1.18x the algorithmic HBM bytes at 7 q-heads per
// kv-head, against 1.0035x with ordinary loads).
template <int BITS, int NG, int NGS, bool KVARN, int NPB, bool QLO, bool KCH = false, bool NSNM = false>
static hipError_t launch_one(const AttnArgs& a, hipStream_t s) {
  if constexpr (BITS == 2 && !KCH) {
    if (a.gq <= 16 / NG) return launch_impl<BITS, NG, NGS, KVARN, NPB, QLO, KCH, NSNM, true>(a, s);
  }
  return launch_impl<BITS, NG, NGS, KVARN, NPB, QLO, KCH, NSNM, false>(a, s);
}

template <int BITS, int NG, int NGS, bool QLO>
static hipError_t launch_pattern(const AttnArgs& a, hipStream_t s) {
  if (a.n_pat <= 0) return launch_one<BITS, NG, NGS, false, 0, QLO>(a, s);
  if (a.n_pat <= 16) return launch_one<BITS, NG, NGS, false, 1, QLO>(a, s);
  if (a.n_pat <= 32) return launch_one<BITS, NG, NGS, false, 2, QLO>(a, s);
  if (a.n_pat <= 64) return launch_one<BITS, NG, NGS, false, 4, QLO>(a, s);
  // 64 prefill patterns plus up to 16 Chebyshev-window centres
  if (a.n_pat <= 80) return launch_one<BITS, NG, NGS, false, 5, QLO>(a, s);
  return launch_one<BITS, NG, NGS, false, 0, QLO>(a, s);
}

// K per channel: the q * s operand always has a lo part
template <int BITS, int NG, int NGS>
static hipError_t launch_kch(const AttnArgs& a, hipStream_t s) {
  if (a.n_pat <= 0) return launch_one<BITS, NG, NGS, false, 0, true, true>(a, s);
  if (a.n_pat <= 16) return launch_one<BITS, NG, NGS, false, 1, true, true>(a, s);
  if (a.n_pat <= 32) return launch_one<BITS, NG, NGS, false, 2, true, true>(a, s);
  if (a.n_pat <= 64) return launch_one<BITS, NG, NGS, false, 4, true, true>(a, s);
  if (a.n_pat <= 80) return launch_one<BITS, NG, NGS, false, 5, true, true>(a, s);
  return launch_one<BITS, NG, NGS, false, 0, true, true>(a, s);
}

template <int BITS, int NG, int NGS>
static hipError_t launch_bits_group(const AttnArgs& a, hipStream_t s) {
  if (a.mode == KVQ_MODE_KVARN) return launch_one<BITS, NG, NGS, true, 0, true>(a, s);
  if (a.mode == KVQ_MODE_NSN) return launch_one<BITS, NG, NGS, true, 0, true, false, true>(a, s);
  if (a.r.kch) return launch_kch<BITS, NG, NGS>(a, s);
  return a.bf16 ? launch_pattern<BITS, NG, NGS, false>(a, s) : launch_pattern<BITS, NG, NGS, true>(a, s);
}

// q-head blocks per unit: 4 heads per row block, 8 at G = 64 beyond 4 q-heads
// per kv-head (the row layouts the launch below picks)
int mfma_head_blocks(int group, int gq) {
  const int hb = (group == 64 && gq > 4) ? 8 : 4;
  return (gq + hb - 1) / hb;
}

bool mfma_attention_supported(int bits, int group, int gq) {
  if (bits != 2 && bits != 4) return false;
  // q-heads beyond one row block (4 at G = 32, 8 at G = 64) take further
  // blocks that re-read the unit's cache
  if (group == 32 || group == 64) return gq >= 1 && gq <= 16;
  return false;
}

// Row blocks: 4 q-heads x 4 groups at G = 32; at G = 64, 4 q-heads x 4 virtual
// half-groups when a unit has at most 4 q-heads, else 8 q-heads x 2 groups.
hipError_t launch_attention_mfma(const AttnArgs& a, hipStream_t s) {
  if (a.group == 32) return a.bits == 2 ? launch_bits_group<2, 4, 4>(a, s) : launch_bits_group<4, 4, 4>(a, s);
  if (a.gq <= 4) return a.bits == 2 ? launch_bits_group<2, 4, 2>(a, s) : launch_bits_group<4, 4, 2>(a, s);
  return a.bits == 2 ? launch_bits_group<2, 2, 2>(a, s) : launch_bits_group<4, 2, 2>(a, s);
}

}  // namespace kvq
