// Top-K block-sparse decode on gfx950 (bound by HBM bandwidth).
//
// SpotAttention (arXiv 2606.22874), Figure 2 caption: score every past block, keep a sink
// prefix, a recency window and the top-scoring blocks, then attend over the gathered K/V of
// that index set.  The learned scorer is replaced by a training-free block representative
// (SALE, arXiv 2505.24179, "The reading": coarse block-representative schemes), the block's
// mean key, and grouped query heads are combined with max (KVpop, arXiv 2607.05061,
// referee minor comment 4).
//
// Kernels:
//   dec_block_summary  kbar[b, J, g, :] = mean of the block's cached keys (exact fp64 sum ->
//                      fp32 -> bf16), all KV heads of a block per workgroup, coalesced
//   dec_summary_q4     4-bit summaries: codes and one bf16 scale per 32 dims
//   dec_score_rows     score[b, g, J] = max over the group's heads of c * q_h . kbar_J, one
//                      coalesced summary row per 16-lane group, DPP reductions
//   dec_score_q4_mfma  the same from 4-bit summaries on bf16 MFMA (heads as MFMA columns)
//   dec_summary_fp4    FP4 (MXFP4) summaries: E2M1 codes and one E8M0 exponent per 32 dims
//   dec_score_fp4_mfma the same from FP4 summaries (codes to bf16 by the fp4 convert)
//   dec_select_radix   forced blocks + top (K - |F|) others by (score desc, block asc): radix
//                      select of the K-th key (11 bits per pass, LDS histograms), ascending
//                      output list; or a top-p budget of others by the same passes over
//                      histograms of fixed-point softmax weight
//   dec_splitk_mfma    64-key blocks: per (b, g, split), each wave takes whole blocks; the G
//                      heads are the 32-wide row dimension of S^T = K Q^T and O^T = V^T P^T
//                      on bf16 MFMA, K in registers, V -> LDS by direct loads; one partial per
//                      split
//   dec_splitk         other block sizes: 16-lane groups stream the split's selected keys
//                      (one 16-byte K and V slice per lane), online softmax for the G packed
//                      heads, merged in-wave then across waves into one partial (m, l, acc)
//   dec_combine        LSE merge of the partials -> O (bf16) and LSE
#include "sa_common.h"
#include "sa_internal.h"

#define NEG_INF (-__builtin_huge_valf())

// ---------------------------------------------------------------------------------------
// kbar[b, J, g, :] for every KV head of one block: 256 threads cover the (g, d) elements of a
// token row four at a time (8-byte loads, consecutive threads on consecutive elements), and
// sum the block's tokens in fp64 -- exact, hence independent of the summation order, while
// the block's values of one element span less than about 2^39 in magnitude (8-bit bf16
// significands, at most 2^6 terms, 53-bit sum) -- then divide, round to fp32, then to bf16.
template <int D>
__global__ __launch_bounds__(256) void dec_block_summary(DecArgs a) {
  const int J = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lb = min(max(a.cache_len[b], 0), a.L);
  if (J == 0 && tid == 0)
    SA_DCHECK(a.dbg, a.cache_len[b] >= 0 && a.cache_len[b] <= a.L, SA_DBG_CACHE_LEN);
  const int t0 = J * a.bk, t1 = min(lb, t0 + a.bk);
  for (int base = 0; base < a.Hkv * D; base += 1024) {
    const int idx = base + tid * 4;
    if (idx >= a.Hkv * D) break;
    const int g = idx / D, d = idx % D;
    uint16_t* out = (uint16_t*)a.ksum + (((int64_t)b * a.nKB + J) * a.Hkv + g) * D + d;
    if (t0 >= lb) {
      *(u32x2*)out = (u32x2){0u, 0u};
      continue;
    }
    const uint16_t* kp = a.kc + b * a.ks0 + g * a.ks2 + d;
    double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
    auto add = [&](u32x2 u) {
      s0 += bf16_bits_to_double((unsigned short)(u.x & 0xFFFFu));
      s1 += bf16_bits_to_double((unsigned short)(u.x >> 16));
      s2 += bf16_bits_to_double((unsigned short)(u.y & 0xFFFFu));
      s3 += bf16_bits_to_double((unsigned short)(u.y >> 16));
    };
    int t = t0;
    for (; t + 8 <= t1; t += 8) {                    // eight independent loads in flight
      u32x2 u[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) u[e] = *(const u32x2*)(kp + (int64_t)(t + e) * a.ks1);
#pragma unroll
      for (int e = 0; e < 8; ++e) add(u[e]);
    }
    for (; t < t1; ++t) add(*(const u32x2*)(kp + (int64_t)t * a.ks1));
    const double n = (double)(t1 - t0);             // divided, as the mean is defined
    const unsigned int lo = float_to_bf16_bits((float)(s0 / n)) |
                            ((unsigned int)float_to_bf16_bits((float)(s1 / n)) << 16);
    const unsigned int hi = float_to_bf16_bits((float)(s2 / n)) |
                            ((unsigned int)float_to_bf16_bits((float)(s3 / n)) << 16);
    *(u32x2*)out = (u32x2){lo, hi};
  }
}

// ---------------------------------------------------------------------------------------
// Sum of a value over each 16-lane row of the wave with DPP (the result in every lane).
SA_DEV float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));   // lane ^ 1
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));   // lane ^ 2
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));  // half mirror
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));  // mirror
  return v;
}

// score[b, g, J] = c * max over the G heads of q_h . kbar[b, J, g].  A 16-lane group reads one
// summary row (d bf16 values) with one load per lane and reduces the per-head dot products
// over the group with DPP; each workgroup covers 128 blocks (8 per group, loaded up front).
template <int D, int G>
__global__ __launch_bounds__(256) void dec_score_rows(DecArgs a) {
  constexpr int DPL = D / 16;              // dims per lane (8 or 4)
  constexpr int RPG = 8;                   // rows per group
  // the KV head varies fastest over the grid: the workgroups of all heads of a block range
  // run together and read each row group [b, J, 0..Hkv) of the summaries as a whole
  const int g = blockIdx.x, b = blockIdx.z;
  const int tid = threadIdx.x, sub = tid & 15, grp = tid >> 4;
  const int nb = (min(max(a.cache_len[b], 0), a.L) + a.bk - 1) / a.bk;
  float qv[G][DPL];
#pragma unroll
  for (int hg = 0; hg < G; ++hg) {
    const uint16_t* qp = a.q + b * a.qs0 + a.qh[g * G + hg] * a.qs2 + sub * DPL;
    if (DPL == 8) {
      const u16x8 u = *(const u16x8*)qp;
#pragma unroll
      for (int e = 0; e < DPL; ++e) qv[hg][e] = bf16_bits_to_float(u[e]);
    } else {
#pragma unroll
      for (int e = 0; e < DPL; ++e) qv[hg][e] = bf16_bits_to_float(qp[e]);
    }
  }
  const int J0 = blockIdx.y * 16 * RPG + grp;
  float kx[RPG][DPL];
#pragma unroll
  for (int r = 0; r < RPG; ++r) {
    const int J = min(J0 + 16 * r, a.nKB - 1);
    const uint16_t* kp = a.ksum + (((int64_t)b * a.nKB + J) * a.Hkv + g) * D + sub * DPL;
    if (DPL == 8) {
      const u16x8 u = *(const u16x8*)kp;
#pragma unroll
      for (int e = 0; e < DPL; ++e) kx[r][e] = bf16_bits_to_float(u[e]);
    } else {
#pragma unroll
      for (int e = 0; e < DPL; ++e) kx[r][e] = bf16_bits_to_float(kp[e]);
    }
  }
#pragma unroll
  for (int r = 0; r < RPG; ++r) {
    const int J = J0 + 16 * r;
    float mx = NEG_INF;
#pragma unroll
    for (int hg = 0; hg < G; ++hg) {
      float p = 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) p = fmaf(qv[hg][e], kx[r][e], p);
      mx = fmaxf(mx, row16_sum(p));
    }
    if (sub == 0 && J < a.nKB)
      a.scores[((int64_t)b * a.Hkv + g) * a.nKB + J] = J < nb ? mx * a.c : NEG_INF;
  }
}

// ---------------------------------------------------------------------------------------
// 4-bit block summaries (SpotAttention "Key findings": an INT4 / FP4 selector key cache,
// 3.5x smaller at no accuracy cost).  One thread per group of 32 dims of a bf16 summary row:
// a = max |x|; scale = bf16(fp32(a / 7)); code = clamp(rint_even(fp32(x * fp32(7 / a))), -7, 7)
// (all zero when a = 0).  Stored as offset-binary nibbles u = code + 8, 8 dims per 32-bit
// word with dim 2j in nibble j and dim 2j+1 in nibble j+4: (word >> 4j) & 0x000F000F then
// holds the pair (2j, 2j+1) in the two 16-bit halves, and OR-ing 0x4300 into each half
// makes the bf16 values 128 + u = 136 + code exactly.
__global__ __launch_bounds__(256) void dec_summary_q4(const uint16_t* ksum, uint8_t* codes,
                                                      uint16_t* scales, int64_t n_groups) {
  const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gi >= n_groups) return;
  const uint16_t* x = ksum + gi * 32;
  float v[32];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u16x8 u = *(const u16x8*)(x + 8 * j);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[8 * j + e] = bf16_bits_to_float(u[e]);
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(v[e]));
  const float inv = amax > 0.f ? __fdiv_rn(7.0f, amax) : 0.f;
  unsigned int w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const float r = fminf(fmaxf(rintf(__fmul_rn(v[e], inv)), -7.f), 7.f);
    const int d = e & 7;                               // dim 2j -> nibble j, 2j+1 -> nibble j+4
    const int nib = (d >> 1) + ((d & 1) << 2);
    w[e >> 3] |= (unsigned int)((int)r + 8) << (4 * nib);
  }
  *(u32x4*)(codes + gi * 16) = (u32x4){w[0], w[1], w[2], w[3]};
  scales[gi] = amax > 0.f ? float_to_bf16_bits(__fdiv_rn(amax, 7.0f)) : (uint16_t)0;
}

// score[b, g, J] from 4-bit summaries on bf16 MFMA: S = Q Kbar'^T with the G query heads as
// the 32-row dimension (zero beyond G) and 32 blocks as the columns, Kbar' holding the
// summaries as bf16 values 136 + code.  Lane l then owns block J0 + l % 32 and heads
// (l / 32) * 4 + 8 (r / 4) + r % 4 of its 16 accumulator entries, so for G <= 8 the group's
// heads sit in entries r < 4 of the lane and of lane l ^ 32.  Per 32-dim group gi the
// accumulator is sum q (136 + code); subtracting 136 sum q (per head and group) and
// multiplying by the block's group scale gives sum q * scale * code (fp32, well inside the
// selection's ambiguity band).  Each wave scores DEC_Q4_TILES consecutive 32-block tiles,
// all of whose codes and scales are loaded up front.  Two tiles per wave keeps 4096 waves
// in flight at 2048 blocks x 8 KV heads x batch 16 while one tile's loads still overlap
// the other's MFMA work (measured: one tile 14.0 us, two 12.6 us, four 13.2 us).
constexpr int DEC_Q4_TILES = 2;
template <int D>
__global__ __launch_bounds__(256) void dec_score_q4_mfma(DecArgs a) {
  constexpr int KS = D / 16, NGR = D / 32, TILES = DEC_Q4_TILES;
  const int g = blockIdx.x, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = tid >> 6;
  const int Jw = (blockIdx.y * 4 + wave) * (32 * TILES);   // this wave's first block
  if (Jw >= a.nKB) return;
  const int nb = (min(max(a.cache_len[b], 0), a.L) + a.bk - 1) / a.bk;
  const int64_t row0 = ((int64_t)b * a.nKB) * a.Hkv + g;   // row of block J: row0 + J * Hkv
  // loads of one tile: the lane's code words (B operand: block J0 + l % 32, dims 16 ks +
  // 8 half .. +8) and that block's group scales
  auto load = [&](int J0, unsigned int* w, u32x2& sc) {
    const int64_t rowi = row0 + (int64_t)min(J0 + l32, a.nKB - 1) * a.Hkv;
    const uint8_t* crow = a.ksum_q4 + rowi * (D / 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) w[ks] = *(const unsigned int*)(crow + (2 * ks + half) * 4);
    if (NGR == 4) sc = *(const u32x2*)(a.ksum_scale + rowi * NGR);
    else sc = (u32x2){*(const unsigned int*)(a.ksum_scale + rowi * NGR), 0u};
  };
  // every tile's loads are issued up front (10 registers a tile)
  unsigned int wt[TILES][KS];
  u32x2 st[TILES];
#pragma unroll
  for (int tt = 0; tt < TILES; ++tt) load(Jw + 32 * tt, wt[tt], st[tt]);
  // Q (A operand): lane l holds head l % 32 of the group (zero beyond G), dims 16 ks + 8 half
  bf16x8 qf[KS];
  float qs_l[NGR];                       // 136 * sum of head l % 32's dims in group gi
  {
    const int hc = min(l32, a.G - 1);
    const uint16_t* qp = a.q + b * a.qs0 + a.qh[g * a.G + hc] * a.qs2 + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = *(const bf16x8*)(qp + ks * 16);
      if (l32 >= a.G) qf[ks] = (bf16x8){};
    }
#pragma unroll
    for (int gi = 0; gi < NGR; ++gi) {
      float t = 0.f;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int e = 0; e < 8; ++e) t += (float)qf[2 * gi + k2][e];
      qs_l[gi] = 136.0f * half_pair_sum(t);
    }
  }
  // the corrections of the heads in this lane's entries r = 0..3: heads 4 half + r
  float qcor[4][NGR];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int gi = 0; gi < NGR; ++gi) {
      const float v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(qs_l[gi]), r));
      const float v1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(qs_l[gi]), 4 + r));
      qcor[r][gi] = half ? v1 : v0;
    }
  const int nh = min(a.G - 4 * half, 4);            // valid heads among this lane's r = 0..3
  float* out = a.scores + ((int64_t)b * a.Hkv + g) * a.nKB;
#pragma unroll
  for (int tt = 0; tt < TILES; ++tt) {
    const int J0 = Jw + 32 * tt;
    const unsigned int* w = wt[tt];
    const u32x2 sc = st[tt];
    f32x16 acc[NGR];
#pragma unroll
    for (int gi = 0; gi < NGR; ++gi) acc[gi] = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 pr;
#pragma unroll
      for (int j = 0; j < 4; ++j) pr[j] = ((w[ks] >> (4 * j)) & 0x000F000Fu) | 0x43004300u;
      bf16x8 kf;
      __builtin_memcpy(&kf, &pr, 16);
      acc[ks / 2] = mfma_bf16(qf[ks], kf, acc[ks / 2]);
    }
    const unsigned int sw[2] = {sc.x, sc.y};
    float sg[NGR];
#pragma unroll
    for (int gi = 0; gi < NGR; ++gi)
      sg[gi] = bf16_bits_to_float((unsigned short)((sw[gi >> 1] >> (16 * (gi & 1))) & 0xFFFFu));
    float mx = NEG_INF;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = 0.f;
#pragma unroll
      for (int gi = 0; gi < NGR; ++gi) v += sg[gi] * (acc[gi][r] - qcor[r][gi]);
      if (r < nh) mx = fmaxf(mx, v);
    }
    mx = half_pair_max(mx) * a.c;                      // heads 4..7 live in lane ^ 32
    const int J = J0 + l32;
    if (half == 0 && J < a.nKB) out[J] = J < nb ? mx : NEG_INF;
  }
}

// ---------------------------------------------------------------------------------------
// FP4 block summaries (SpotAttention "Key findings": the INT4 / FP4 microscale selector key
// cache), in the OCP Microscaling v1.0 MXFP4 format, per group of 32 dims of a bf16 summary
// row: shared exponent e = floor(log2 max|x|) - 2 clamped to [-127, 127], stored as the E8M0
// byte e + 127; codes E2M1 of |x| * 2^-e (an exact scaling) with the sign bit of x (negative
// zero included) in bit 3; dim 2k in the low and dim 2k + 1 in the high nibble of byte k.
// 4.25 bits per dim.  One thread per group.
__global__ __launch_bounds__(256) void dec_summary_fp4(const uint16_t* ksum, uint8_t* codes,
                                                       uint8_t* exps, int64_t n_groups) {
  const int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gi >= n_groups) return;
  const uint16_t* x = ksum + gi * 32;
  unsigned short bits[32];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u16x8 u = *(const u16x8*)(x + 8 * j);
#pragma unroll
    for (int e = 0; e < 8; ++e) bits[8 * j + e] = u[e];
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(bf16_bits_to_float(bits[e])));
  // floor(log2 amax) is the unbiased exponent field of a normal float; subnormals clamp to -127
  int ex = -127;
  if (amax > 0.f) ex = max((int)((__float_as_uint(amax) >> 23) & 0xFF) - 129, -127);
  unsigned int w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const unsigned int code = e2m1_code(ldexpf(fabsf(bf16_bits_to_float(bits[e])), -ex)) |
                              ((unsigned int)(bits[e] >> 15) << 3);
    w[e >> 3] |= code << (4 * (e & 7));
  }
  *(u32x4*)(codes + gi * 16) = (u32x4){w[0], w[1], w[2], w[3]};
  exps[gi] = (uint8_t)(ex + 127);
}

// score[b, g, J] from FP4 summaries on bf16 MFMA, laid out as dec_score_q4_mfma (G heads as
// the MFMA rows, 32 blocks as the columns, DEC_Q4_TILES tiles per wave).  The codes become
// bf16 with v_cvt_scalef32_pk_bf16_fp4 at scale 1 (every E2M1 value is exact in bf16, two
// dims per instruction, low nibble first); each 32-dim group accumulates on its own and is
// scaled by its 2^e afterwards (exact), so the score is sum over groups of 2^e * q . code.
template <int D>
__global__ __launch_bounds__(256) void dec_score_fp4_mfma(DecArgs a) {
  constexpr int KS = D / 16, NGR = D / 32, TILES = DEC_Q4_TILES;
  const int g = blockIdx.x, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = tid >> 6;
  const int Jw = (blockIdx.y * 4 + wave) * (32 * TILES);   // this wave's first block
  if (Jw >= a.nKB) return;
  const int nb = (min(max(a.cache_len[b], 0), a.L) + a.bk - 1) / a.bk;
  const int64_t row0 = ((int64_t)b * a.nKB) * a.Hkv + g;   // row of block J: row0 + J * Hkv
  // loads of one tile: the lane's code words (B operand: block J0 + l % 32, dims 16 ks +
  // 8 half .. +8) and that block's group exponents
  auto load = [&](int J0, unsigned int* w, unsigned int& ev) {
    const int64_t rowi = row0 + (int64_t)min(J0 + l32, a.nKB - 1) * a.Hkv;
    const uint8_t* crow = a.ksum_q4 + rowi * (D / 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) w[ks] = *(const unsigned int*)(crow + (2 * ks + half) * 4);
    if (NGR == 4) ev = *(const unsigned int*)(a.ksum_exp + rowi * 4);
    else ev = *(const unsigned short*)(a.ksum_exp + rowi * 2);
  };
  unsigned int wt[TILES][KS], et[TILES];
#pragma unroll
  for (int tt = 0; tt < TILES; ++tt) load(Jw + 32 * tt, wt[tt], et[tt]);
  // Q (A operand): lane l holds head l % 32 of the group (zero beyond G), dims 16 ks + 8 half
  bf16x8 qf[KS];
  {
    const int hc = min(l32, a.G - 1);
    const uint16_t* qp = a.q + b * a.qs0 + a.qh[g * a.G + hc] * a.qs2 + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = *(const bf16x8*)(qp + ks * 16);
      if (l32 >= a.G) qf[ks] = (bf16x8){};
    }
  }
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const int nh = min(a.G - 4 * half, 4);            // valid heads among this lane's r = 0..3
  float* out = a.scores + ((int64_t)b * a.Hkv + g) * a.nKB;
#pragma unroll
  for (int tt = 0; tt < TILES; ++tt) {
    const int J0 = Jw + 32 * tt;
    const unsigned int* w = wt[tt];
    f32x16 acc[NGR];
#pragma unroll
    for (int gi = 0; gi < NGR; ++gi) acc[gi] = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x2 p[4] = {__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[ks], 1.0f, 0),
                           __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[ks], 1.0f, 1),
                           __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[ks], 1.0f, 2),
                           __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[ks], 1.0f, 3)};
      bf16x8 kf;
      __builtin_memcpy(&kf, p, 16);
      acc[ks / 2] = mfma_bf16(qf[ks], kf, acc[ks / 2]);
    }
    int eg[NGR];
#pragma unroll
    for (int gi = 0; gi < NGR; ++gi) eg[gi] = (int)((et[tt] >> (8 * gi)) & 0xFFu) - 127;
    float mx = NEG_INF;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float v = 0.f;
#pragma unroll
      for (int gi = 0; gi < NGR; ++gi) v += ldexpf(acc[gi][r], eg[gi]);
      if (r < nh) mx = fmaxf(mx, v);
    }
    mx = half_pair_max(mx) * a.c;                      // heads 4..7 live in lane ^ 32
    const int J = J0 + l32;
    if (half == 0 && J < a.nKB) out[J] = J < nb ? mx : NEG_INF;
  }
}

// ---------------------------------------------------------------------------------------
// Exclusive sum over the 256 threads of a workgroup (4 waves) of a non-negative count, in
// thread order (reverse = true: over the threads after this one).  Two barriers.
SA_DEV int block_excl_sum(int v, bool reverse, int* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int t = reverse ? __shfl_down(incl, o) : __shfl_up(incl, o);
    if (reverse ? lane + o < 64 : lane >= o) incl += t;
  }
  __syncthreads();                                   // wsum free
  if (reverse ? lane == 0 : lane == 63) wsum[wave] = incl;
  __syncthreads();
  int ex = incl - v;
  for (int w = 0; w < 4; ++w)
    if (reverse ? w > wave : w < wave) ex += wsum[w];
  return ex;
}

// The same over 64-bit values.
SA_DEV unsigned long long block_excl_sum_u64(unsigned long long v, bool reverse,
                                             unsigned long long* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  unsigned long long incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long t = reverse ? __shfl_down(incl, o) : __shfl_up(incl, o);
    if (reverse ? lane + o < 64 : lane >= o) incl += t;
  }
  __syncthreads();
  if (reverse ? lane == 0 : lane == 63) wsum[wave] = incl;
  __syncthreads();
  unsigned long long ex = incl - v;
  for (int w = 0; w < 4; ++w)
    if (reverse ? w > wave : w < wave) ex += wsum[w];
  return ex;
}

// Top-K by radix select.  One workgroup (256 threads) per (b, g).  Each candidate block
// j < nb gets the order-preserving 32-bit key of its score (forced blocks: the maximum key);
// the K-th largest key is found 11 bits at a time (3 passes at most; it stops early once the
// bin it falls in is taken whole), then the
// output takes every key above the threshold T and, among keys equal to T on the resolved
// bits, the smallest block ids -- the order (key desc, block asc) -- in ascending block order.
//
// With top_p > 0 the number of content (non-forced) blocks is the top-p budget: each block
// weighs w_j = exp(score_j - max score), held in fixed point (2^40 units, so every sum is an
// exact integer and independent of the order of the additions); the same radix passes, with
// histograms of weight besides counts, find the key at which the forced weight plus the
// weight of the content keys above it first reaches top_p * sum w.  Keys equal on all 32 bits
// have equal scores and weights, so the last r of them follow from one division.  When the
// budget exceeds K - |forced| the fixed-K selection is made instead.
__global__ __launch_bounds__(256) void dec_select_radix(DecArgs a) {
  constexpr int BINS = 2048;
  constexpr unsigned int FORCED = 0xFFFFFFFFu;
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  extern __shared__ unsigned int skey[];             // [nKB] keys, then [nKB] scores
  float* ssc = (float*)(skey + a.nKB);
  __shared__ unsigned int hist[BINS];
  __shared__ unsigned long long hmass[BINS];
  __shared__ unsigned int s_dig, s_need, s_cab;
  __shared__ int wsum[4];
  __shared__ unsigned long long wsum64[4];
  __shared__ unsigned long long s_z, s_f, s_wq;
  __shared__ double s_needm;
  __shared__ float s_max[4];
  __shared__ int s_nf;
  const int lb = min(max(a.cache_len[b], 0), a.L);
  if (g == 0 && tid == 0)
    SA_DCHECK(a.dbg, a.cache_len[b] >= 0 && a.cache_len[b] <= a.L, SA_DBG_CACHE_LEN);
  const int nb = (lb + a.bk - 1) / a.bk;
  const float* sc = a.scores + ((int64_t)b * a.Hkv + g) * a.nKB;
  // Thread t owns blocks t, t + 256, ... in every loop over the blocks below.  Its scores are
  // loaded eight at a time, all in flight together: one load per iteration would wait out
  // the memory latency once per 256 blocks.
  int nf_local = 0;
  for (int j0 = tid; j0 < nb; j0 += 256 * 8) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = sc[min(j0 + 256 * e, nb - 1)];
    // every value is taken here, so no load sinks into the conditional stores below
#pragma unroll
    for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(v[e]));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = j0 + 256 * e;
      if (j < nb) {
        const bool forced = (j * a.bk < a.sink) || ((j + 1) * a.bk - 1 >= lb - a.local);
        skey[j] = forced ? FORCED : float_order_key(v[e]);
        ssc[j] = v[e];
        nf_local += forced;
      }
    }
  }
  const int kk = min(a.top_k, nb);
  unsigned int T = 0, mask = 0;                      // threshold on the resolved bits
  unsigned int need = (unsigned int)kk;
  bool all = kk >= nb;                               // every block is selected
  int total = kk;                                    // blocks selected
  bool done = false;

  if (a.top_p > 0.f) {
    // max score, then the fixed-point weights and their sums (all, forced)
    float mloc = NEG_INF;
    for (int j = tid; j < nb; j += 256) mloc = fmaxf(mloc, ssc[j]);
    for (int o = 32; o > 0; o >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o));
    if (tid == 0) { s_z = 0; s_f = 0; s_nf = 0; }
    if ((tid & 63) == 0) s_max[tid >> 6] = mloc;
    __syncthreads();
    const float M = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    auto wfix = [&](int j) -> unsigned long long {
      return (unsigned long long)(expf(ssc[j] - M) * 0x1p40f);
    };
    unsigned long long zl = 0, fl = 0;
    for (int j = tid; j < nb; j += 256) {
      const unsigned long long w = wfix(j);
      zl += w;
      if (skey[j] == FORCED) fl += w;
    }
    atomicAdd(&s_z, zl);
    atomicAdd(&s_f, fl);
    atomicAdd(&s_nf, nf_local);
    __syncthreads();
    const int nF = s_nf;
    double needm = (double)a.top_p * (double)s_z - (double)s_f;
    int n_content = 0;
    unsigned int Tp = FORCED, maskp = FORCED, needp = (unsigned int)nF;
    if (needm > 0.0) {
      const int shifts[3] = {21, 10, 0};
      unsigned int cab = 0;                          // content keys above the resolved prefix
      Tp = 0;
      maskp = 0;
      for (int p = 0; p < 3; ++p) {
        const int shift = shifts[p];
        const unsigned int dmask = p == 2 ? 1023u : 2047u;
        for (int e = tid; e < BINS; e += 256) {
          hist[e] = 0;
          hmass[e] = 0;
        }
        __syncthreads();
        for (int j = tid; j < nb; j += 256) {
          const unsigned int k = skey[j];
          if (k != FORCED && (k & maskp) == Tp) {
            const unsigned int dg = (k >> shift) & dmask;
            atomicAdd(&hist[dg], 1u);
            atomicAdd(&hmass[dg], wfix(j));
          }
        }
        __syncthreads();
        unsigned int c[8], totc = 0;
        unsigned long long m[8], totm = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          c[e] = hist[8 * tid + e];
          m[e] = hmass[8 * tid + e];
          totc += c[e];
          totm += m[e];
        }
        unsigned int runc = (unsigned int)block_excl_sum((int)totc, true, wsum);
        unsigned long long runm = block_excl_sum_u64(totm, true, wsum64);
#pragma unroll
        for (int e = 7; e >= 0; --e) {
          if ((double)runm < needm && (double)(runm + m[e]) >= needm) {   // crossing digit
            s_dig = (unsigned int)(8 * tid + e);
            s_needm = needm - (double)runm;
            s_cab = runc;
            s_wq = m[e] / c[e];                      // one weight per key on the last pass
          }
          runm += m[e];
          runc += c[e];
        }
        __syncthreads();
        needm = s_needm;
        cab += s_cab;
        Tp |= s_dig << shift;
        maskp |= dmask << shift;
      }
      // every content key equal to Tp weighs s_wq: the first r of them complete the share
      const unsigned int r = (unsigned int)max(1.0, ceil(needm / (double)s_wq));
      n_content = (int)(cab + r);
      needp = r;
    }
    if (n_content <= max(0, a.top_k - nF)) {
      T = Tp;
      mask = maskp;
      need = needp;
      all = false;
      total = nF + n_content;
      done = true;
    }
  }

  if (!done && kk < nb) {
    const int shifts[3] = {21, 10, 0};
    for (int p = 0; p < 3; ++p) {
      const int shift = shifts[p];
      const unsigned int dmask = p == 2 ? 1023u : 2047u;
      for (int e = tid; e < BINS; e += 256) hist[e] = 0;
      __syncthreads();                                 // also: skey written
      for (int j = tid; j < nb; j += 256) {
        const unsigned int k = skey[j];
        if ((k & mask) == T) atomicAdd(&hist[(k >> shift) & dmask], 1u);
      }
      __syncthreads();
      // thread t owns the digits 8t .. 8t+7; counts of larger digits come from later threads
      unsigned int c[8], tot = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 8 * tid + e;
        c[e] = hist[d];
        tot += c[e];
      }
      unsigned int run = (unsigned int)block_excl_sum((int)tot, true, wsum);
#pragma unroll
      for (int e = 7; e >= 0; --e) {
        if (run < need && run + c[e] >= need) {        // the K-th key has digit 8t+e
          s_dig = (unsigned int)(8 * tid + e) | ((need - run == c[e]) ? 0x80000000u : 0u);
          s_need = need - run;
        }
        run += c[e];
      }
      __syncthreads();
      const unsigned int dg = s_dig;
      need = s_need;
      T |= (dg & 0x7FFFFFFFu) << shift;
      mask |= dmask << shift;
      if (dg & 0x80000000u) break;                     // every key in that bin is taken
    }
  }
  // flags: resolved key > T, or == T among the first `need` equal keys by block id
  constexpr int MAXPER = 32;                           // nKB <= 8192 = 256 * 32
  const int per = (nb + 255) / 256;
  const int j0 = tid * per;
  int eq = 0;
  if (!all)
    for (int e = 0; e < per && j0 + e < nb; ++e) eq += (skey[j0 + e] & mask) == T;
  int eq_before = block_excl_sum(eq, false, wsum);
  unsigned int sel_bits = 0;                           // bit e: block j0 + e selected
  int cnt = 0;
  for (int e = 0; e < per && e < MAXPER && j0 + e < nb; ++e) {
    const unsigned int k = skey[j0 + e] & mask;
    bool take;
    if (all || k > T) {
      take = true;
    } else if (k == T) {
      take = (unsigned int)eq_before < need;
      ++eq_before;
    } else {
      take = false;
    }
    if (take) {
      sel_bits |= 1u << e;
      ++cnt;
    }
  }
  int pos = block_excl_sum(cnt, false, wsum);
  int32_t* out = a.selected + ((int64_t)b * a.Hkv + g) * a.top_k;
  for (int e = 0; e < per && e < MAXPER; ++e)
    if (sel_bits & (1u << e)) out[pos++] = j0 + e;
  for (int p = total + tid; p < a.top_k; p += 256) out[p] = -1;
  if (tid == 0) a.sel_count[b * a.Hkv + g] = total;
}

// ---------------------------------------------------------------------------------------
// Split-K attention of one query per (b, head) over the selected blocks.  Workgroup =
// 16 groups of 16 lanes; a group handles every 16th key of the split, each lane a
// D/16-wide slice of the head dimension.  Four keys per group are loaded ahead.
template <int D, int G>
__global__ __launch_bounds__(256) void dec_splitk(DecArgs a) {
  constexpr int DPL = D / 16;              // dims per lane (8 or 4)
  constexpr int UNR = 4;
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = tid & 15, grp = tid >> 4;
  const int lb = min(max(a.cache_len[b], 0), a.L);
  const int nb = (lb + a.bk - 1) / a.bk;
  const int nsel = a.sel_count[b * a.Hkv + g];
  const int bps = (nsel + a.n_splits - 1) / a.n_splits;
  const int blk0 = s * bps, blk1 = min(nsel, blk0 + bps);
  const int nkeys = max(0, blk1 - blk0) * a.bk;
  const int32_t* sel = a.selected + ((int64_t)b * a.Hkv + g) * a.top_k;
  const float sl2 = a.c * 1.4426950408889634f;

  float qv[G][DPL];
#pragma unroll
  for (int hg = 0; hg < G; ++hg) {
    const uint16_t* qp = a.q + b * a.qs0 + a.qh[g * G + hg] * a.qs2 + sub * DPL;
#pragma unroll
    for (int e = 0; e < DPL; ++e) qv[hg][e] = bf16_bits_to_float(qp[e]) * sl2;
  }
  float m[G], l[G], acc[G][DPL];
#pragma unroll
  for (int hg = 0; hg < G; ++hg) {
    m[hg] = -1e30f;
    l[hg] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[hg][e] = 0.f;
  }
  const uint16_t* kb = a.kc + b * a.ks0 + g * a.ks2 + sub * DPL;
  const uint16_t* vb = a.vc + b * a.vs0 + g * a.vs2 + sub * DPL;

  for (int e0 = grp; e0 < nkeys; e0 += 16 * UNR) {
    float kf[UNR][DPL], vf[UNR][DPL];
    bool ok[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int e = e0 + u * 16;
      int tok = 0;
      ok[u] = false;
      if (e < nkeys) {
        tok = sel[blk0 + e / a.bk] * a.bk + e % a.bk;
        ok[u] = tok < lb;
      }
      const int tc = ok[u] ? tok : 0;
      if (DPL == 8) {
        const u16x8 kx = *(const u16x8*)(kb + (int64_t)tc * a.ks1);
        const u16x8 vx = *(const u16x8*)(vb + (int64_t)tc * a.vs1);
#pragma unroll
        for (int j = 0; j < DPL; ++j) {
          kf[u][j] = bf16_bits_to_float(kx[j]);
          vf[u][j] = bf16_bits_to_float(vx[j]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < DPL; ++j) {
          kf[u][j] = bf16_bits_to_float(kb[(int64_t)tc * a.ks1 + j]);
          vf[u][j] = bf16_bits_to_float(vb[(int64_t)tc * a.vs1 + j]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float z[G];
#pragma unroll
      for (int hg = 0; hg < G; ++hg) {
        float p = 0.f;
#pragma unroll
        for (int j = 0; j < DPL; ++j) p = fmaf(qv[hg][j], kf[u][j], p);
        p += __shfl_xor(p, 1);
        p += __shfl_xor(p, 2);
        p += __shfl_xor(p, 4);
        p += __shfl_xor(p, 8);
        z[hg] = p;
      }
      if (ok[u]) {
#pragma unroll
        for (int hg = 0; hg < G; ++hg) {
          const float mn = fmaxf(m[hg], z[hg]);
          const float al = __builtin_amdgcn_exp2f(m[hg] - mn);
          const float p = __builtin_amdgcn_exp2f(z[hg] - mn);
          m[hg] = mn;
          l[hg] = fmaf(l[hg], al, p);
#pragma unroll
          for (int j = 0; j < DPL; ++j) acc[hg][j] = fmaf(acc[hg][j], al, p * vf[u][j]);
        }
      }
    }
  }
  // merge the 4 groups of a wave (xor 16, xor 32)
#pragma unroll
  for (int o = 16; o <= 32; o <<= 1) {
#pragma unroll
    for (int hg = 0; hg < G; ++hg) {
      const float mo = __shfl_xor(m[hg], o);
      const float lo = __shfl_xor(l[hg], o);
      const float mn = fmaxf(m[hg], mo);
      const float sa = __builtin_amdgcn_exp2f(m[hg] - mn), sb = __builtin_amdgcn_exp2f(mo - mn);
      l[hg] = l[hg] * sa + lo * sb;
#pragma unroll
      for (int j = 0; j < DPL; ++j) {
        const float ao = __shfl_xor(acc[hg][j], o);
        acc[hg][j] = acc[hg][j] * sa + ao * sb;
      }
      m[hg] = mn;
    }
  }
  // merge the 4 waves through LDS
  __shared__ float sm[4][G], sl[4][G], sacc[4][G][D];
  if (lane < 16) {
#pragma unroll
    for (int hg = 0; hg < G; ++hg) {
      if (lane == 0) {
        sm[wave][hg] = m[hg];
        sl[wave][hg] = l[hg];
      }
#pragma unroll
      for (int j = 0; j < DPL; ++j) sacc[wave][hg][sub * DPL + j] = acc[hg][j];
    }
  }
  __syncthreads();
  for (int p = tid; p < G * D; p += 256) {
    const int hg = p / D, d = p % D;
    float mx = sm[0][hg];
    for (int w = 1; w < 4; ++w) mx = fmaxf(mx, sm[w][hg]);
    float lt = 0.f, at = 0.f;
    for (int w = 0; w < 4; ++w) {
      const float f = __builtin_amdgcn_exp2f(sm[w][hg] - mx);
      lt += sl[w][hg] * f;
      at += sacc[w][hg][d] * f;
    }
    float* part = a.partial + (((int64_t)b * a.Hq + g * G + hg) * a.n_splits + s) * (D + 2);
    part[d] = at;
    if (d == 0) {
      part[D] = mx;
      part[D + 1] = lt;
    }
  }
}

// ---------------------------------------------------------------------------------------
// Split-K attention for 64-key blocks on MFMA.  The G query heads of a KV head play the role
// of the query rows of the prefill kernel: S^T = K Q^T with Q^T's 32 columns holding the G
// heads (zero beyond G), so each lane owns one head and 16 keys of each 32-key half and the
// softmax statistics stay in-lane (plus one exchange with lane ^ 32); P^T stays in registers
// as the B operand of O^T += V^T P^T.  About one workgroup per CU: each wave streams its
// share of the split's blocks (w, w + 4, ...) with the next block in flight -- its K rows go
// straight into registers in the A-operand layout, its V rows HBM -> LDS by direct loads
// (320-byte rows for d = 128, two buffers per wave) -- while the current block is computed;
// V^T is read with transposing LDS reads.  The four waves' (m, l, O) are merged through LDS
// into one partial per (b, head, split).  MFMA work is 8x the useful work for G = 4 and still
// far below the time the K/V bytes take to arrive.
template <int D>
__global__ __launch_bounds__(256, 1) void dec_splitk_mfma(DecArgs a) {
  // The host pass only needs this kernel's signature (for its launch stub).
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int KS = D / 16, DM = D / 32, ROWB = D * 2;
  constexpr int VPITCH = D == 128 ? 320 : 192;
  constexpr int VREG = 64 * VPITCH;
  constexpr int VWIN = VREG / 1024;
  constexpr int LOADS = 2 * KS + VWIN;             // vector-memory ops per block
  static_assert(VREG % 1024 == 0, "DMA windows must tile the region");
  static_assert(4 * VREG >= (2 * 4 * 32 + 4 * 32 * D) * 4, "merge buffers must fit the regions");
  static_assert(LOADS < 64, "one block's loads must fit the vmcnt counter");
  // two V buffers per wave, as distinct objects so the compiler can tell a load into one
  // from reads of the other
  __shared__ __attribute__((aligned(1024))) unsigned char vb0[4 * VREG];
  __shared__ __attribute__((aligned(1024))) unsigned char vb1[4 * VREG];

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = wave_uniform(tid >> 6);
  unsigned char* reg0 = vb0 + wave * VREG;
  unsigned char* reg1 = vb1 + wave * VREG;
  const int lb = min(max(a.cache_len[b], 0), a.L);
  const int nb = (lb + 63) / 64;
  const int nsel = ((const __attribute__((address_space(4))) int32_t*)a.sel_count)[b * a.Hkv + g];
  const int bps = (nsel + a.n_splits - 1) / a.n_splits;
  const int blk0 = s * bps, blk1 = min(nsel, blk0 + bps);
  const int nw = max(0, (blk1 - blk0 - wave + 3) / 4);   // this wave's blocks
  const __attribute__((address_space(4))) int32_t* sel =
      (const __attribute__((address_space(4))) int32_t*)(a.selected + ((int64_t)b * a.Hkv + g) * a.top_k);
  const float sl2 = a.c * 1.4426950408889634f;

  // Q^T as the B operand: lane l holds head l % 32 of the group (zero beyond G)
  bf16x8 qf[KS];
  {
    const int hc = min(l32, a.G - 1);
    const uint16_t* qp = a.q + b * a.qs0 + a.qh[g * a.G + hc] * a.qs2 + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = *(const bf16x8*)(qp + ks * 16);
      if (l32 >= a.G) qf[ks] = (bf16x8){};
    }
  }
  const uint16_t* kbase = a.kc + b * a.ks0 + g * a.ks2 + half * 8;
  const uint16_t* vbase = a.vc + b * a.vs0 + g * a.vs2;
  const int grp = lane >> 4, jj = lane & 15;
  const int v_rd = (4 * (grp >> 1) + (jj >> 2)) * VPITCH + (16 * (grp & 1) + 4 * (jj & 3)) * 2;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones2 = {(__bf16)1.0f, (__bf16)1.0f};

  f32x16 oacc[DM];
#pragma unroll
  for (int dm = 0; dm < DM; ++dm) oacc[dm] = (f32x16){};
  float m_run = -1e30f, l_run = 0.f;

  // issue the loads of this wave's i-th block: K rows into kf in the A-operand layout (lane l:
  // key 32 mt + l % 32, dims 16 ks + 8 (l / 32)), V rows into the LDS region; rows past the
  // cache end re-read the last cached row (their scores are masked)
  auto load = [&](int i, bf16x8 (*kf)[KS], unsigned char* reg) {
    const int t0 = sel[blk0 + wave + 4 * i] * 64;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int tok = min(t0 + mt * 32 + l32, lb - 1);
      const uint16_t* kp = kbase + (int64_t)tok * a.ks1;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[mt][ks] = *(const bf16x8*)(kp + ks * 16);
    }
#pragma unroll
    for (int w = 0; w < VWIN; ++w) {
      const int o = w * 1024 + lane * 16;
      const int r = o / VPITCH, cb = o % VPITCH;
      const int tok = min(t0 + r, lb - 1);
      __builtin_amdgcn_global_load_lds(vbase + (int64_t)tok * a.vs1 + (cb < ROWB ? cb / 2 : 0),
                                       LDS_PTR(void, reg + w * 1024), 16, 0, 0);
    }
  };
  // attention over the i-th block; `more`: the next block's loads are in flight behind it
  auto compute = [&](int i, bf16x8 (*kf)[KS], const unsigned char* reg, bool more) {
    const int t0 = sel[blk0 + wave + 4 * i] * 64;
    f32x16 sacc[2] = {(f32x16){}, (f32x16){}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) sacc[mt] = mfma_bf16(kf[mt][ks], qf[ks], sacc[mt]);
    if (t0 + 63 >= lb) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int tok = t0 + mt * 32 + half * 4 + 8 * (r >> 2) + (r & 3);
          if (tok >= lb) sacc[mt][r] = NEG_INF;
        }
    }
    // online softmax over the block (log2 domain)
    float v = NEG_INF;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) v = fmaxf(v, sacc[mt][r]);
    const float mnew = fmaxf(m_run, half_pair_max(v) * sl2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
    m_run = mnew;
#pragma unroll
    for (int dm = 0; dm < DM; ++dm) oacc[dm] *= alpha;
    float ls = l_run * alpha;
    bf16x8 pf[4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        f32x8 tt;
#pragma unroll
        for (int e = 0; e < 8; ++e) tt[e] = __builtin_amdgcn_exp2f(fmaf(sacc[mt][8 * s2 + e], sl2, -mnew));
        const bf16x8 pb = __builtin_convertvector(tt, bf16x8);
        pf[mt * 2 + s2] = pb;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 pr = {pb[e], pb[e + 1]};
          ls = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2, ls, false);
        }
      }
    l_run = ls;
    // this block's V rows have landed once only the next block's loads may be outstanding
    if (more)
      __builtin_amdgcn_s_waitcnt(VMCNT_IMM(LOADS));
    else
      __builtin_amdgcn_s_waitcnt(VMCNT_IMM(0));
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) {
        const unsigned char* vp = reg + v_rd + 16 * s4 * VPITCH + dm * 64;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4i16, vp));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4i16, vp + 8 * VPITCH));
        const v4i16 both[2] = {lo, hi};
        bf16x8 vf;
        __builtin_memcpy(&vf, both, 16);
        oacc[dm] = mfma_bf16(vf, pf[s4], oacc[dm]);
      }
    // every LDS read of the region has returned before a later block's loads overwrite it
    __builtin_amdgcn_s_waitcnt(LGKM0_IMM);
  };

  bf16x8 ka[2][KS], kb[2][KS];
  if (nw > 0) load(0, ka, reg0);
  for (int i = 0; i < nw; i += 2) {
    if (i + 1 < nw) load(i + 1, kb, reg1);
    compute(i, ka, reg0, i + 1 < nw);
    if (i + 1 < nw) {
      if (i + 2 < nw) load(i + 2, ka, reg0);
      compute(i + 1, kb, reg1, i + 2 < nw);
    }
  }

  // ---- merge the four waves through LDS (the regions are free once every wave is here) ----
  __syncthreads();
  float* mo = (float*)vb0;                     // [4][32] running max per wave and head
  float* lo = mo + 4 * 32;                     // [4][32] row sum
  float* ao = lo + 4 * 32;                     // [4][32][D] O per wave and head
  const float lt = half_pair_sum(l_run);
  if (l32 < a.G) {
    if (half == 0) {
      mo[wave * 32 + l32] = m_run;
      lo[wave * 32 + l32] = lt;
    }
#pragma unroll
    for (int dm = 0; dm < DM; ++dm)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        ao[(wave * 32 + l32) * D + dm * 32 + half * 4 + 8 * (r >> 2) + (r & 3)] = oacc[dm][r];
  }
  __syncthreads();
  for (int p = tid; p < a.G * D; p += 256) {
    const int hg = p / D, d = p % D;
    float mx = mo[hg];
    for (int w = 1; w < 4; ++w) mx = fmaxf(mx, mo[w * 32 + hg]);
    float ltot = 0.f, at = 0.f;
    for (int w = 0; w < 4; ++w) {
      const float f = __builtin_amdgcn_exp2f(mo[w * 32 + hg] - mx);
      ltot += lo[w * 32 + hg] * f;
      at += ao[(w * 32 + hg) * D + d] * f;
    }
    float* part = a.partial + (((int64_t)b * a.Hq + g * a.G + hg) * a.n_splits + s) * (D + 2);
    part[d] = at;
    if (d == 0) {
      part[D] = mx;
      part[D + 1] = ltot;
    }
  }

#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------------------------
// One workgroup per (b, head), one thread per dimension.  The (m, l) of every split are read
// up front (independent loads, chunks of 16), so the merge waits for memory about twice rather
// than once per split.
template <int D>
__global__ __launch_bounds__(D) void dec_combine(DecArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const float* part = a.partial + ((int64_t)b * a.Hq + h) * a.n_splits * (D + 2);
  constexpr int CH = 16;
  float mx = -1e30f;
  for (int s0 = 0; s0 < a.n_splits; s0 += CH) {
    float ms[CH], ls[CH];
#pragma unroll
    for (int e = 0; e < CH; ++e) {
      const int sp = min(s0 + e, a.n_splits - 1);
      ms[e] = part[sp * (D + 2) + D];
      ls[e] = part[sp * (D + 2) + D + 1];
    }
#pragma unroll
    for (int e = 0; e < CH; ++e)
      if (ls[e] > 0.f) mx = fmaxf(mx, ms[e]);
  }
  float lt = 0.f, at = 0.f;
  for (int s0 = 0; s0 < a.n_splits; s0 += CH) {
    float ms[CH], ls[CH], vs[CH];
#pragma unroll
    for (int e = 0; e < CH; ++e) {
      const int sp = min(s0 + e, a.n_splits - 1);
      ms[e] = part[sp * (D + 2) + D];
      ls[e] = s0 + e < a.n_splits ? part[sp * (D + 2) + D + 1] : 0.f;
      vs[e] = part[sp * (D + 2) + d];
    }
#pragma unroll
    for (int e = 0; e < CH; ++e)
      if (ls[e] > 0.f) {
        const float f = __builtin_amdgcn_exp2f(ms[e] - mx);
        lt += ls[e] * f;
        at += vs[e] * f;
      }
  }
  const float o = lt > 0.f ? at / lt : 0.f;
  const int hq = a.qh[h];                         // partials are kept per packed head
  ((uint16_t*)a.o)[b * a.os0 + hq * a.os2 + d] = float_to_bf16_bits(o);
  if (a.lse && d == 0)
    a.lse[(int64_t)b * a.Hq + hq] = lt > 0.f ? (mx + __log2f(lt)) * 0.69314718055994531f : NEG_INF;
}

// ---------------------------------------------------------------------------------------
hipError_t launch_block_summary(const DecArgs& a, hipStream_t s) {
  if (a.D == 64)
    hipLaunchKernelGGL(dec_block_summary<64>, dim3(a.nKB, a.B), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(dec_block_summary<128>, dim3(a.nKB, a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_decode_d(const DecArgs& a, hipStream_t s) {
  const dim3 sgrid(a.Hkv, (a.nKB + 127) / 128, a.B);
  if (a.ksum_q4 && a.ksum_exp) {
    hipLaunchKernelGGL(dec_score_fp4_mfma<D>, dim3(a.Hkv, (a.nKB + 128 * DEC_Q4_TILES - 1) / (128 * DEC_Q4_TILES), a.B),
                       dim3(256), 0, s, a);
  } else if (a.ksum_q4) {
    hipLaunchKernelGGL(dec_score_q4_mfma<D>, dim3(a.Hkv, (a.nKB + 128 * DEC_Q4_TILES - 1) / (128 * DEC_Q4_TILES), a.B),
                       dim3(256), 0, s, a);
  } else {
    switch (a.G) {
      case 1: hipLaunchKernelGGL((dec_score_rows<D, 1>), sgrid, dim3(256), 0, s, a); break;
      case 2: hipLaunchKernelGGL((dec_score_rows<D, 2>), sgrid, dim3(256), 0, s, a); break;
      case 4: hipLaunchKernelGGL((dec_score_rows<D, 4>), sgrid, dim3(256), 0, s, a); break;
      default: hipLaunchKernelGGL((dec_score_rows<D, 8>), sgrid, dim3(256), 0, s, a); break;
    }
  }
  hipLaunchKernelGGL(dec_select_radix, dim3(a.Hkv, a.B), dim3(256), a.nKB * 2 * sizeof(unsigned int), s, a);
  const dim3 grid(a.n_splits, a.Hkv, a.B);
  if (a.bk == 64) {
    hipLaunchKernelGGL(dec_splitk_mfma<D>, grid, dim3(256), 0, s, a);
  } else {
    switch (a.G) {
      case 1: hipLaunchKernelGGL((dec_splitk<D, 1>), grid, dim3(256), 0, s, a); break;
      case 2: hipLaunchKernelGGL((dec_splitk<D, 2>), grid, dim3(256), 0, s, a); break;
      case 4: hipLaunchKernelGGL((dec_splitk<D, 4>), grid, dim3(256), 0, s, a); break;
      default: hipLaunchKernelGGL((dec_splitk<D, 8>), grid, dim3(256), 0, s, a); break;
    }
  }
  hipLaunchKernelGGL(dec_combine<D>, dim3(a.Hq, a.B), dim3(D), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_summary_q4(const uint16_t* ksum, uint8_t* codes, uint16_t* scales, int64_t n_groups,
                             hipStream_t s) {
  if (n_groups == 0) return hipSuccess;
  hipLaunchKernelGGL(dec_summary_q4, dim3((unsigned)((n_groups + 255) / 256)), dim3(256), 0, s, ksum,
                     codes, scales, n_groups);
  return hipGetLastError();
}

hipError_t launch_summary_fp4(const uint16_t* ksum, uint8_t* codes, uint8_t* exps, int64_t n_groups,
                              hipStream_t s) {
  if (n_groups == 0) return hipSuccess;
  hipLaunchKernelGGL(dec_summary_fp4, dim3((unsigned)((n_groups + 255) / 256)), dim3(256), 0, s, ksum,
                     codes, exps, n_groups);
  return hipGetLastError();
}

hipError_t launch_decode(const DecArgs& a, hipStream_t s) {
  if (a.D == 64) return launch_decode_d<64>(a, s);
  return launch_decode_d<128>(a, s);
}
