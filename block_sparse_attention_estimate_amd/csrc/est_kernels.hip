// Estimation pass for anchor-based block/stripe-sparse prefill on gfx950.
//
// AnchorAttention (arXiv 2505.23520) Eq. (1): anchor = max score over the initial and
// local key regions, read from the row-max buffer (referee major comment 1); Eq. (2): keep
// where avgpool(x_a) - avgpool(Q) K^T / sqrt(d) <= theta; Eq. (3): per-query-block index
// set I.  SALE (arXiv 2505.24179), "What carries the argument": the estimate uses
// quantised Q and K and the decision is one log-domain comparison.  KVpop (arXiv
// 2607.05061), referee minor comment 4: grouped heads are combined with max.
//
// Kernels, in launch order:
//   est_quant_k       one workgroup per (b, g, key tile): int8 keys + one scale per tile
//   est_anchor_pool   one workgroup per (b, g, query block): the block's sink + local key rows
//                     staged once in LDS (direct loads) for all G heads, anchor max on bf16
//                     MFMA, block mean, pooled query (fp64 sum), int8 pooled query
//                     (est_anchor_pool_gl: the same with global key reads, for large windows)
//   est_score_block   int8 MFMA of key tiles against pooled queries, block max, margin,
//                     max over the group's heads -> one keep bit per (query block, key block)
//   est_score_stripe  same per key column (no block max)
//   est_step_or       (step > 1) keep bits OR-ed over groups of `step` query blocks
//   est_compact       bits | forced, causal -> ascending index lists + counts
// With the relative-score estimator (SALE) est_anchor_pool and est_score_block are replaced
// by est_quant_q_rows (int8 query rows) and est_score_rel (element-wise estimate, LSE of the
// sink-local keys, block max of S~ - LSE + theta, max over the group); with MXFP4 operands by
// est_quant_rows_fp4 (Q and K rows) and est_score_rel_fp4 (block-scaled fp4 MFMA).
//
// Floating-point steps that decide an integer (int8 codes, keep bits) use explicit
// round-to-nearest operations (__fmul_rn, __fdiv_rn, rintf) in the order the oracle uses.
#include <type_traits>

#include "sa_common.h"
#include "sa_internal.h"

#define NEG_INF (-__builtin_huge_valf())

// ---------------------------------------------------------------------------------------
// int8 key blocks: a = max |K| over the block's keys (block_k = 64, or each 32-key half of the
// 64-key tile when block_k = 32), scale = a / 127, code = rint(K * (127 / a)).
// One workgroup per 64-key tile.
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void est_quant_k(EstArgs a) {
  constexpr int CH = D / 8;              // 16-byte chunks per key row
  constexpr int PER = 64 * CH / 256;     // chunks per thread (tile of 64 keys)
  const int J = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  // chunk c of this thread holds key J*64 + tid / CH + c * (256 / CH): the first half of the
  // chunks lies in keys 0..31 of the tile, the second half in keys 32..63
  u16x8 v[PER];
  float amax[2] = {0.f, 0.f};
#pragma unroll
  for (int c = 0; c < PER; ++c) {
    const int ch = tid + c * 256;
    const int key = J * 64 + ch / CH;
    const int dc = (ch % CH) * 8;
    if (key < a.N) {
      v[c] = *(const u16x8*)(a.k + b * a.ks0 + (int64_t)key * a.ks1 + g * a.ks2 + dc);
    } else {
      v[c] = (u16x8)(0);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      amax[c / (PER / 2)] = fmaxf(amax[c / (PER / 2)], fabsf(bf16_bits_to_float(v[c][e])));
  }
  __shared__ float red[2][4];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const float m = wave_max(amax[hf]);
    if ((tid & 63) == 0) red[hf][tid >> 6] = m;
  }
  __syncthreads();
  const bool split = a.bk == 32;
  float inv[2], scale[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const float m0 = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
    const float m1 = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
    const float am = split ? (hf == 0 ? m0 : m1) : fmaxf(m0, m1);
    inv[hf] = 0.f;
    scale[hf] = 1.f;
    if (am > 0.f) {
      inv[hf] = __fdiv_rn(127.0f, am);
      scale[hf] = __fdiv_rn(am, 127.0f);
    }
  }
  int8_t* dst = a.kq + ((int64_t)(b * a.Hkv + g) * a.nKT * 64) * D;
#pragma unroll
  for (int c = 0; c < PER; ++c) {
    const int ch = tid + c * 256;
    const int key = J * 64 + ch / CH;
    const int dc = (ch % CH) * 8;
    const float iv = inv[c / (PER / 2)];
    unsigned int w[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float r = rintf(__fmul_rn(bf16_bits_to_float(v[c][e]), iv));
      r = fminf(fmaxf(r, -127.f), 127.f);
      const int qi = (int)r;
      w[e >> 2] |= ((unsigned int)(qi & 0xFF)) << (8 * (e & 3));
    }
    *(u32x2*)(dst + (int64_t)key * D + dc) = (u32x2){w[0], w[1]};
  }
  if (tid == 0) {
    float* sk = a.sk + (int64_t)(b * a.Hkv + g) * a.nKB;
    if (split) {
      sk[2 * J] = scale[0];
      if (2 * J + 1 < a.nKB) sk[2 * J + 1] = scale[1];
    } else {
      sk[J] = scale[0];
    }
  }
}

// ---------------------------------------------------------------------------------------
// Anchor (Eq. 1), block mean of the anchor and pooled, quantised query (Eq. 2).
// S^T = K_region Q^T on 32x32x16 bf16 MFMA: a lane owns one query row (column n) and
// sees 16 of the 32 keys of each tile, so the row max is in-lane plus one half swap.
// ---------------------------------------------------------------------------------------
#define EST_AP_WAVES 16
template <int D>
__global__ __launch_bounds__(64 * EST_AP_WAVES) void est_anchor_pool(EstArgs a) {
  constexpr int NW = EST_AP_WAVES;                 // waves: one 32-row tile each (G = 4, bq = 128)
  constexpr int KS = D / 16;
  constexpr int ROWB = D * 2;                       // bytes of one key row
  constexpr int KPITCH = D == 128 ? 272 : 144;      // padded LDS row (conflict-free A reads)
  // keys one query block can need: a 32-key sink tile block plus the causal window rounded
  // out to 32-key tiles: sink tiles + (local + bq) rows + 32 of alignment
  constexpr int MAXROWS = 512;
  // work item (b, g, i): workgroups are dealt to the 8 XCDs round-robin, and XCD x takes a
  // contiguous range of items, so the query blocks it runs together are neighbours whose key
  // windows overlap in its L2
  int item;
  {
    const int total = a.nQB * a.Hkv * a.B;
    const int x = blockIdx.x % 8, k = blockIdx.x / 8;
    int start = 0;
    for (int y = 0; y < x; ++y) start += (total - y + 7) / 8;   // workgroups XCD y receives
    item = start + k;
  }
  const int i = item % a.nQB, g = (item / a.nQB) % a.Hkv, b = item / (a.nQB * a.Hkv);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int G = a.G;
  const int r0 = i * a.bq;
  const int r1 = min(a.N, r0 + a.bq);
  const int nrows = r1 - r0;
  const int ntph = (a.bq + 31) / 32;
  __shared__ float xa_s[8][128];
  __shared__ float qbar_s[8][128];
  __shared__ __attribute__((aligned(1024))) unsigned char kw[MAXROWS * KPITCH];

  if (a.xa_ready) {
    // anchors computed by the anchor-state pass (same MFMA sequence, same values)
    for (int p = tid; p < G * nrows; p += 64 * NW) {
      const int hg = p / nrows, rr = p % nrows;
      xa_s[hg][rr] = a.xa[((int64_t)b * a.Hq + g * G + hg) * a.N + r0 + rr];
    }
  } else {
    // ---- the key rows this query block needs, staged once in LDS for all G heads ----
    // tiles of 32 keys: the sink tiles [0, ceil(min(sink, r1) / 32)), then the window tiles
    // from the tile holding max(0, r0 - local + 1) (not below the sink tiles) through r1 - 1
    const int hi_blk = r1 - 1;
    const int sink_end = min(a.sink, r1);
    const int n_sink_t = (sink_end + 31) / 32;
    const int lo_blk = max(0, r0 - a.local + 1);
    const int win_start = max((lo_blk / 32) * 32, n_sink_t * 32);
    const int n_win_t = win_start <= hi_blk ? (hi_blk - win_start) / 32 + 1 : 0;
    const int n_rows = (n_sink_t + n_win_t) * 32;     // <= MAXROWS for local <= 352, bq <= 128
    auto tile_start = [&](int t) { return t < n_sink_t ? t * 32 : win_start + (t - n_sink_t) * 32; };
    // Q fragments of this wave's n-tiles (32 rows of one head each), the next one loaded while
    // the current one's MFMAs run; the first goes out before the keys are staged
    auto load_q = [&](int nt, bf16x8* qf) {
      const int hg = nt / ntph, tr = nt % ntph;
      const int rowc = min(r0 + tr * 32 + l32, a.N - 1);
      const uint16_t* qp = a.q + b * a.qs0 + (int64_t)rowc * a.qs1 + a.qh[g * G + hg] * a.qs2 + half * 8;
  #pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const bf16x8*)(qp + ks * 16);
    };
    bf16x8 qn[KS];
    if (wave < G * ntph) load_q(wave, qn);
    {
      const uint16_t* kb = a.k + b * a.ks0 + g * a.ks2;
      const int nwin = (n_rows * KPITCH + 1023) / 1024;
      for (int w = wave; w < nwin; w += NW) {
        const int o = w * 1024 + lane * 16;
        const int r = min(o / KPITCH, n_rows - 1), cb = o % KPITCH;
        const int key = min(tile_start(r / 32) + (r % 32), a.N - 1);
        __builtin_amdgcn_global_load_lds(kb + (int64_t)key * a.ks1 + (cb < ROWB ? cb / 2 : 0),
                                         LDS_PTR(void, kw + w * 1024), 16, 0, 0);
      }
      __builtin_amdgcn_s_waitcnt(VMCNT_IMM(0));
      __syncthreads();
    }
    const int k_rd = l32 * KPITCH + half * 16;

    for (int nt = wave; nt < G * ntph; nt += NW) {
      const int hg = nt / ntph, tr = nt % ntph;
      const int ra = r0 + tr * 32;
      bf16x8 qf[KS];
  #pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = qn[ks];
      if (nt + NW < G * ntph) load_q(nt + NW, qn);
      if (ra >= r1) continue;
      const int row = ra + l32;
      float mx = NEG_INF;
      const int hi = min(ra + 31, a.N - 1);
      const int lo = max(0, ra - a.local + 1);
      // this n-tile's tiles: the sink tiles visible to it, then the window tiles from lo to hi
      for (int t = 0; t < n_sink_t + n_win_t; ++t) {
        const int ts = tile_start(t);
        if (ts > hi) break;                              // tiles ascend; later ones are causal-masked
        if (t >= n_sink_t && ts + 31 < lo) continue;     // window tile entirely before this window
        f32x16 acc = {};
  #pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 kf = *(const bf16x8*)(kw + k_rd + t * 32 * KPITCH + ks * 32);
          acc = mfma_bf16(kf, qf[ks], acc);
        }
        // a tile whose 32 keys are visible to all 32 rows of this n-tile needs no mask
        const bool all_sink = ts + 31 < a.sink && ts + 31 <= ra;
        const bool all_win = ts >= ra + 31 - a.local + 1 && ts + 31 <= ra;
        if (all_sink || all_win) {
  #pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[r]);
        } else {
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = ts + half * 4 + 8 * (r >> 2) + (r & 3);
            const bool ok = key <= row && (key < a.sink || key >= row - a.local + 1);
            if (ok) mx = fmaxf(mx, acc[r]);
          }
        }
      }
      mx = fmaxf(mx, swap_halves(mx));
      if (half == 0 && row < r1) xa_s[hg][row - r0] = __fmul_rn(mx, a.c);
    }
  }

  // Pooled query: fp64 sum over the block's rows, one rounding to fp32, fp32 division.
  // Thread t sums 8 dims (one 16-byte load per row) of every NW-th row; the NW row groups'
  // fp64 partials meet in LDS (the key window is no longer needed).  Sums of bf16 values are
  // exact in fp64 here, so neither split changes the result.
  __syncthreads();
  double* part = (double*)kw;                       // [NW][G * D]
  {
    const int ncg = G * D / 8;                      // 8-dim column groups of the G heads
    for (int c = tid % 64; c < ncg; c += 64) {
      const int rg = tid / 64;                      // row group = wave
      const int hg = c / (D / 8), d8 = (c % (D / 8)) * 8;
      const uint16_t* qp = a.q + b * a.qs0 + (int64_t)r0 * a.qs1 + a.qh[g * G + hg] * a.qs2 + d8;
      double acc[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
      int r = rg;
      for (; r + 7 * NW < nrows; r += 8 * NW) {     // eight rows of this group in flight
        u16x8 u[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) u[j] = *(const u16x8*)(qp + (int64_t)(r + NW * j) * a.qs1);
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += bf16_bits_to_double(u[j][e]);
      }
      for (; r < nrows; r += NW) {
        const u16x8 u = *(const u16x8*)(qp + (int64_t)r * a.qs1);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += bf16_bits_to_double(u[e]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) part[rg * G * D + hg * D + d8 + e] = acc[e];
    }
  }
  __syncthreads();
  for (int p = tid; p < G * D; p += 64 * NW) {
    double t = 0.0;
    for (int w = 0; w < NW; ++w) t += part[w * G * D + p];
    qbar_s[p / D][p % D] = __fdiv_rn((float)t, (float)nrows);
  }
  __syncthreads();

  for (int hg = wave; hg < G; hg += NW) {
    // block mean of the anchor (fp64 accumulation)
    double s = 0.0;
    for (int r = lane; r < nrows; r += 64) s += (double)xa_s[hg][r];
    s = wave_sum_d(s);
    float amax = 0.f;
    for (int dd = lane; dd < D; dd += 64) amax = fmaxf(amax, fabsf(qbar_s[hg][dd]));
    amax = wave_max(amax);
    float inv = 0.f, scale = 1.f;
    if (amax > 0.f) {
      inv = __fdiv_rn(127.0f, amax);
      scale = __fdiv_rn(amax, 127.0f);
    }
    const int64_t rowid = ((int64_t)(b * a.Hkv + g) * a.nQB + i) * G + hg;
    int8_t* dst = a.qq + rowid * D;
    for (int dd = lane; dd < D; dd += 64) {
      float r = rintf(__fmul_rn(qbar_s[hg][dd], inv));
      r = fminf(fmaxf(r, -127.f), 127.f);
      dst[dd] = (int8_t)(int)r;
    }
    if (lane == 0) {
      a.sq[rowid] = scale;
      a.abar[rowid] = (float)(s / (double)nrows);
    }
  }
}

// The same pass for windows too large to stage in LDS (sink or local beyond the sizes the
// staged kernel is built for): key tiles are read from global memory per row tile.
template <int D>
__global__ __launch_bounds__(256) void est_anchor_pool_gl(EstArgs a) {
  constexpr int KS = D / 16;
  const int i = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int G = a.G;
  const int r0 = i * a.bq;
  const int r1 = min(a.N, r0 + a.bq);
  const int nrows = r1 - r0;
  const int ntph = (a.bq + 31) / 32;
  __shared__ float xa_s[8][128];
  __shared__ float qbar_s[8][128];

  if (a.xa_ready) {
    // anchors computed by the anchor-state pass (same MFMA sequence, same values)
    for (int p = tid; p < G * nrows; p += 256) {
      const int hg = p / nrows, rr = p % nrows;
      xa_s[hg][rr] = a.xa[((int64_t)b * a.Hq + g * G + hg) * a.N + r0 + rr];
    }
  } else {
    for (int nt = wave; nt < G * ntph; nt += 4) {
      const int hg = nt / ntph, tr = nt % ntph;
      const int h = g * G + hg;
      const int ra = r0 + tr * 32;
      if (ra >= r1) continue;
      const int row = ra + l32;
      const int rowc = min(row, a.N - 1);
      bf16x8 qf[KS];
      const uint16_t* qp = a.q + b * a.qs0 + (int64_t)rowc * a.qs1 + a.qh[h] * a.qs2 + half * 8;
  #pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const bf16x8*)(qp + ks * 16);
      float mx = NEG_INF;
      const int hi = min(ra + 31, a.N - 1);
      const int sink_end = min(a.sink, hi + 1);
      const int sink_tiles_end = ((sink_end + 31) / 32) * 32;
      const int lo = max(0, ra - a.local + 1);
      const int win_start = max((lo / 32) * 32, sink_tiles_end);
      const uint16_t* kb = a.k + b * a.ks0 + g * a.ks2 + half * 8;
      // key tiles: the sink tiles, then the window tiles; fragments of the next tile are
      // loaded before the current tile's MFMAs
      const int n_sink_t = sink_tiles_end / 32;
      const int n_win_t = win_start <= hi ? (hi - win_start) / 32 + 1 : 0;
      const int n_t = n_sink_t + n_win_t;
      auto tile_start = [&](int t) { return t < n_sink_t ? t * 32 : win_start + (t - n_sink_t) * 32; };
      bf16x8 kf[KS], kn[KS];
      if (n_t > 0) {
        const uint16_t* kp = kb + (int64_t)min(tile_start(0) + l32, a.N - 1) * a.ks1;
  #pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[ks] = *(const bf16x8*)(kp + ks * 16);
      }
      for (int t = 0; t < n_t; ++t) {
        const int ts = tile_start(t);
        if (t + 1 < n_t) {
          const uint16_t* kp = kb + (int64_t)min(tile_start(t + 1) + l32, a.N - 1) * a.ks1;
  #pragma unroll
          for (int ks = 0; ks < KS; ++ks) kn[ks] = *(const bf16x8*)(kp + ks * 16);
        }
        f32x16 acc = {};
  #pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = mfma_bf16(kf[ks], qf[ks], acc);
        // a tile whose 32 keys are visible to all 32 rows of this n-tile needs no mask
        const bool all_sink = ts + 31 < a.sink && ts + 31 <= ra;
        const bool all_win = ts >= ra + 31 - a.local + 1 && ts + 31 <= ra;
        if (all_sink || all_win) {
  #pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[r]);
        } else {
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = ts + half * 4 + 8 * (r >> 2) + (r & 3);
            const bool ok = key <= row && (key < a.sink || key >= row - a.local + 1);
            if (ok) mx = fmaxf(mx, acc[r]);
          }
        }
  #pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[ks] = kn[ks];
      }
      mx = fmaxf(mx, swap_halves(mx));
      if (half == 0 && row < r1) xa_s[hg][row - r0] = __fmul_rn(mx, a.c);
    }
  }

  // Pooled query: fp64 sum over the block's rows, one rounding to fp32, fp32 division.
  // Each thread owns two adjacent dims of one head (one 4-byte load per row); four
  // independent fp64 partial sums keep several loads in flight.  Sums of bf16 values are
  // exact in fp64 here, so the split does not change the result.
  for (int p = tid; p < G * D / 2; p += 256) {
    const int hg = p / (D / 2), d2 = (p % (D / 2)) * 2;
    const int h = g * G + hg;
    const uint16_t* qp = a.q + b * a.qs0 + (int64_t)r0 * a.qs1 + a.qh[h] * a.qs2 + d2;
    double s0[4] = {0.0, 0.0, 0.0, 0.0}, s1[4] = {0.0, 0.0, 0.0, 0.0};
    int r = 0;
    for (; r + 8 <= nrows; r += 8) {
      unsigned int u[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) u[j] = *(const unsigned int*)(qp + (int64_t)(r + j) * a.qs1);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        s0[j & 3] += bf16_bits_to_double((unsigned short)(u[j] & 0xFFFFu));
        s1[j & 3] += bf16_bits_to_double((unsigned short)(u[j] >> 16));
      }
    }
    for (; r < nrows; ++r) {
      const unsigned int u = *(const unsigned int*)(qp + (int64_t)r * a.qs1);
      s0[0] += bf16_bits_to_double((unsigned short)(u & 0xFFFFu));
      s1[0] += bf16_bits_to_double((unsigned short)(u >> 16));
    }
    const double t0 = (s0[0] + s0[1]) + (s0[2] + s0[3]);
    const double t1 = (s1[0] + s1[1]) + (s1[2] + s1[3]);
    qbar_s[hg][d2] = __fdiv_rn((float)t0, (float)nrows);
    qbar_s[hg][d2 + 1] = __fdiv_rn((float)t1, (float)nrows);
  }
  __syncthreads();

  for (int hg = wave; hg < G; hg += 4) {
    // block mean of the anchor (fp64 accumulation)
    double s = 0.0;
    for (int r = lane; r < nrows; r += 64) s += (double)xa_s[hg][r];
    s = wave_sum_d(s);
    float amax = 0.f;
    for (int dd = lane; dd < D; dd += 64) amax = fmaxf(amax, fabsf(qbar_s[hg][dd]));
    amax = wave_max(amax);
    float inv = 0.f, scale = 1.f;
    if (amax > 0.f) {
      inv = __fdiv_rn(127.0f, amax);
      scale = __fdiv_rn(amax, 127.0f);
    }
    const int64_t rowid = ((int64_t)(b * a.Hkv + g) * a.nQB + i) * G + hg;
    int8_t* dst = a.qq + rowid * D;
    for (int dd = lane; dd < D; dd += 64) {
      float r = rintf(__fmul_rn(qbar_s[hg][dd], inv));
      r = fminf(fmaxf(r, -127.f), 127.f);
      dst[dd] = (int8_t)(int)r;
    }
    if (lane == 0) {
      a.sq[rowid] = scale;
      a.abar[rowid] = (float)(s / (double)nrows);
    }
  }
}

// ---------------------------------------------------------------------------------------
// Block scores.  D^T[key][row] = K_q . qbar_q^T on 32x32x32 int8 MFMA (exact int32); a lane
// owns one (query block, head) row and 16 keys of each 32-key half of a 64-key tile, so a
// block's max is in-lane plus one half swap.  Workgroup = 4 waves x 64 rows (256 rows), 32
// key tiles of 64 keys (32 key blocks of 64, or 64 key blocks of 32: block_k = 32 takes each
// half of a tile as its own block, with its own key scale).
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void est_score_block(EstArgs a, int n_rt, int n_jc) {
  // The host pass only needs this kernel's signature (for its launch stub).
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int KS = D / 32;
  constexpr int NT = 2;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  // blockIdx.x = (bg * n_rt + rt) * n_jc + jc, J-chunks of one row tile adjacent
  const int lin = blockIdx.x;
  const int jc = lin % n_jc;
  const int rt = (lin / n_jc) % n_rt;
  const int bg = lin / (n_jc * n_rt);
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.G;
  const int rows_total = a.nQB * G;
  const int R_last = min(rt * 256 + 255, rows_total - 1);
  const int e_last = min(a.N, (R_last / G + 1) * a.bq) - 1;
  const int J0 = jc * 32;                             // first 64-key tile of the chunk
  if (J0 * 64 > e_last) return;
  const int J_end = min(J0 + 32, e_last / 64 + 1);
  const bool bk32 = a.bk == 32;                      // key blocks of 32: two per tile

  int rowR[NT], e_i[NT], jmax[NT];
  float thr[NT], sqv[NT];
  i32x4 qf[NT][KS];
  const int64_t row_base = (int64_t)bg * rows_total;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int R = rt * 256 + wave * 64 + nt * 32 + l32;
    rowR[nt] = R;
    const int Rc = min(R, rows_total - 1);
    const int iq = Rc / G, hg = Rc % G;
    e_i[nt] = min(a.N, (iq + 1) * a.bq) - 1;
    jmax[nt] = R < rows_total ? e_i[nt] / a.bk : -1;     // last causal key block
    thr[nt] = a.abar[row_base + Rc] - a.theta[g * G + hg];
    sqv[nt] = a.sq[row_base + Rc];
    const int8_t* qp = a.qq + (row_base + Rc) * D + half * 16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[nt][ks] = *(const i32x4*)(qp + ks * 32);
  }
  const int e_min = min(a.N, ((rt * 256 + wave * 64) / G + 1) * a.bq) - 1;
  // K tiles go HBM -> LDS with direct loads into four stages shared by the four waves (rows
  // padded to D + 16 bytes: the 16 rows one quarter-wave reads land on distinct banks)
  constexpr int KP = D + 16;
  constexpr int WIN = (64 * KP + 1023) / 1024;       // 1 KB windows per tile
  constexpr int SL = (WIN + 3) / 4;                   // windows per wave
  __shared__ __attribute__((aligned(1024))) unsigned char ks0[WIN * 1024];
  __shared__ __attribute__((aligned(1024))) unsigned char ks1[WIN * 1024];
  __shared__ __attribute__((aligned(1024))) unsigned char ks2[WIN * 1024];
  __shared__ __attribute__((aligned(1024))) unsigned char ks3[WIN * 1024];
  __shared__ __attribute__((aligned(1024))) unsigned char kspare[1024];
  const int8_t* kbase = a.kq + ((int64_t)bg * a.nKT * 64) * D;
  int s_off[SL];                                      // byte offset in a tile of this lane's 16 bytes
#pragma unroll
  for (int k = 0; k < SL; ++k) {
    const int o = min(wave + 4 * k, WIN - 1) * 1024 + lane * 16;
    const int r = min(o / KP, 63), c = o % KP;
    s_off[k] = r * D + (c < D ? c : 0);               // pads and the tail get a harmless copy
  }
  auto issue = [&](unsigned char* st, int J) {
    const int8_t* tb = kbase + (int64_t)J * 64 * D;
#pragma unroll
    for (int k = 0; k < SL; ++k) {
      const int wdw = wave + 4 * k;
      __builtin_amdgcn_global_load_lds(tb + s_off[k], LDS_PTR(void, wdw < WIN ? st + wdw * 1024 : kspare), 16, 0, 0);
    }
  };
  const int k_rd = l32 * KP + half * 16;
  unsigned long long bits[NT] = {0ull, 0ull};   // bit (block - first block of the chunk)

  // one key tile: D^T on int8 MFMA, block max, margin, max over the group, keep bit
  auto tile = [&](const unsigned char* st, int J) {
    i32x16 acc[2][NT];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = (i32x16){};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const i32x4 kf = *(const i32x4*)(st + k_rd + mt * 32 * KP + ks * 32);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma_i8(kf, qf[nt][ks], acc[mt][nt]);
      }
    // key-block scales of the tile's blocks (block_k = 32: one per half)
    const float* skb = a.sk + (int64_t)bg * a.nKB;
    const float skv0 = load_uniform(skb + (bk32 ? 2 * J : J));
    const float skv1 = bk32 ? load_uniform(skb + min(2 * J + 1, a.nKB - 1)) : skv0;
    const bool need_mask = (J * 64 + 63 > e_min) || (J * 64 + 63 >= a.N);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      // max of the int32 dots over the block's causal keys: the whole tile (block_k = 64) or
      // each half (block_k = 32)
      int m[2] = {INT32_MIN, INT32_MIN};
      if (!need_mask) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) m[mt] = max(m[mt], acc[mt][nt][r]);
      } else {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = J * 64 + mt * 32 + half * 4 + 8 * (r >> 2) + (r & 3);
            if (key <= e_i[nt] && key < a.N) m[mt] = max(m[mt], acc[mt][nt][r]);
          }
      }
      if (!bk32) m[0] = max(m[0], m[1]);
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        if (hb == 1 && !bk32) break;
        const int Jb = bk32 ? 2 * J + hb : J;            // key block
        int mm = max(m[hb], swap_halves_i(m[hb]));
        const bool cand = Jb <= jmax[nt];
        float margin = NEG_INF;
        if (cand && mm != INT32_MIN) {
          const float skv = hb == 0 ? skv0 : skv1;
          const float mult = __fmul_rn(__fmul_rn(sqv[nt], skv), a.c);
          const float s_hat = __fmul_rn((float)mm, mult);
          margin = s_hat - thr[nt];
        }
        for (int o = 1; o < G; o <<= 1) margin = fmaxf(margin, __shfl_xor(margin, o));
        if (margin >= 0.f) bits[nt] |= 1ull << (bk32 ? 2 * (J - J0) + hb : J - J0);
        if (a.margins && cand && half == 0 && (rowR[nt] % G) == 0) {
          const int iq = rowR[nt] / G;
          a.margins[((int64_t)bg * a.nQB + iq) * a.nKB + Jb] = margin;
        }
      }
    }
  };

  // Tile J0 + j is in stage j % 4; tiles j+1 and j+2 are loaded or in flight.  Step j
  // computes tile j, issues tile j+3 (clamped to the last tile, so every wave issues SL loads
  // per step) into the stage of tile j-1 and waits until tile j+1 has landed.
  const int nt_ = J_end - J0;
  issue(ks0, J0);
  issue(ks1, J0 + min(1, nt_ - 1));
  issue(ks2, J0 + min(2, nt_ - 1));
  DMA_BARRIER(2 * SL);
  auto step = [&](const unsigned char* sc, unsigned char* sd, int j) {
    tile(sc, J0 + j);
    issue(sd, J0 + min(j + 3, nt_ - 1));
    DMA_BARRIER(2 * SL);
  };
  int j = 0;
  for (; j + 4 <= nt_; j += 4) {
    step(ks0, ks3, j);
    step(ks1, ks0, j + 1);
    step(ks2, ks1, j + 2);
    step(ks3, ks2, j + 3);
  }
  if (j < nt_) step(ks0, ks3, j);
  if (j + 1 < nt_) step(ks1, ks0, j + 1);
  if (j + 2 < nt_) step(ks2, ks1, j + 2);
  // no DMA may still be writing this workgroup's LDS when it exits
  __builtin_amdgcn_s_waitcnt(VMCNT_IMM(0));
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (half == 0 && rowR[nt] < rows_total && (rowR[nt] % G) == 0) {
      const int iq = rowR[nt] / G;
      uint32_t* wrow = a.bits + ((int64_t)bg * a.nQB + iq) * a.W;
      if (bk32) {
        wrow[2 * jc] = (unsigned int)bits[nt];
        if (2 * jc + 1 < a.W) wrow[2 * jc + 1] = (unsigned int)(bits[nt] >> 32);
      } else {
        wrow[jc] = (unsigned int)bits[nt];
      }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------------------------
// The 2*KS int8 key fragments of a tile (B operand: key row nt*32 + lane%32, bytes ks*32 +
// (lane/32)*16, rows KP bytes apart) read from LDS in one block that also waits for them.  The
// compiler sees no LDS read here, so it does not order the reads after the direct loads in
// flight into other stages; the explicit waits and barriers around the tiles order them.
template <int KS, int KP>
SA_DEV void read_key_fragments(unsigned int addr, i32x4 (&kf)[2][KS]);
template <>
SA_DEV void read_key_fragments<4, 144>(unsigned int addr, i32x4 (&kf)[2][4]) {
  asm volatile(
      "ds_read_b128 %0, %8 offset:0\n\t"
      "ds_read_b128 %1, %8 offset:32\n\t"
      "ds_read_b128 %2, %8 offset:64\n\t"
      "ds_read_b128 %3, %8 offset:96\n\t"
      "ds_read_b128 %4, %8 offset:4608\n\t"
      "ds_read_b128 %5, %8 offset:4640\n\t"
      "ds_read_b128 %6, %8 offset:4672\n\t"
      "ds_read_b128 %7, %8 offset:4704\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(kf[0][0]), "=&v"(kf[0][1]), "=&v"(kf[0][2]), "=&v"(kf[0][3]),
        "=&v"(kf[1][0]), "=&v"(kf[1][1]), "=&v"(kf[1][2]), "=&v"(kf[1][3])
      : "v"(addr));
}
template <>
SA_DEV void read_key_fragments<2, 80>(unsigned int addr, i32x4 (&kf)[2][2]) {
  asm volatile(
      "ds_read_b128 %0, %4 offset:0\n\t"
      "ds_read_b128 %1, %4 offset:32\n\t"
      "ds_read_b128 %2, %4 offset:2560\n\t"
      "ds_read_b128 %3, %4 offset:2592\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(kf[0][0]), "=&v"(kf[0][1]), "=&v"(kf[1][0]), "=&v"(kf[1][1])
      : "v"(addr));
}

// Stripe scores.  D[row][key] = qbar_q . K_q^T: rows are the A operand, keys the B operand,
// so a lane owns one key column and 16 rows; one compare per element becomes a wave
// ballot that holds, per row pair, the keep bits of 32 consecutive columns.
// Workgroup = 4 waves x 64 rows, 32 key tiles of 64 columns.
// ---------------------------------------------------------------------------------------
template <int D, int G, bool MARGINS>
__global__ __launch_bounds__(256, 4) void est_score_stripe(EstArgs a, int n_rt, int n_jc) {
  // The host pass only needs this kernel's signature (for its launch stub).
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int KS = D / 32;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = wave_uniform(tid >> 6);
  const int lin = blockIdx.x;
  const int jc = lin % n_jc;
  const int rt = (lin / n_jc) % n_rt;
  const int bg = lin / (n_jc * n_rt);
  const int g = bg % a.Hkv;
  const int rows_total = a.nQB * G;                    // G: query heads per KV head (1, 2, 4, 8)
  const int R_last = min(rt * 128 + 127, rows_total - 1);
  const int e_last = min(a.N, (R_last / G + 1) * a.bq) - 1;
  const int J0 = jc * 32;
  if (J0 * 64 > e_last) return;
  const int J_end = min(J0 + 32, e_last / 64 + 1);
  const int64_t row_base = (int64_t)bg * a.nQB * G;
  const int Rw = rt * 128 + wave * 32;                  // first row of this wave
  const bool wave_live = Rw < rows_total;               // waves past the rows only stage keys

  // A operand: pooled query rows Rw + l32
  i32x4 qf[KS];
  {
    const int Rc = min(Rw + l32, rows_total - 1);
    const int8_t* qp = a.qq + (row_base + Rc) * D + half * 16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const i32x4*)(qp + ks * 32);
  }
  // Per-register row data: register r holds row Rw + half*4 + 8(r/4) + r%4; rows past the end
  // never pass (threshold +inf)
  float thr[16], sqv[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int R = Rw + half * 4 + 8 * (r >> 2) + (r & 3);
    const int Rc = min(R, rows_total - 1);
    thr[r] = R < rows_total ? a.abar[row_base + Rc] - a.theta[g * G + Rc % G] : __builtin_huge_valf();
    sqv[r] = a.sq[row_base + Rc];
  }
  // last causal key of row R's query block (-1 past the rows), per register
  auto erow = [&](int R) { return R < rows_total ? min(a.N, (R / G + 1) * a.bq) - 1 : -1; };
  int erw[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) erw[r] = erow(Rw + half * 4 + 8 * (r >> 2) + (r & 3));
  // The keep test fp32(D * sq * sk * c) >= thr, rewritten per row as D * sk >= u with
  // u = thr / (sq * c) (a zero threshold stays zero, so 0 >= 0 keeps when a scale is zero):
  // per tile one product u * (1 / sk) per row, then per element one conversion and one
  // compare.  The decision can differ from the fp32 product only where the margin is within a
  // few ulps of zero (far inside the ambiguity band of the lists).
  float uthr[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) uthr[r] = thr[r] == 0.f ? 0.f : thr[r] / (sqv[r] * a.c);
  // the first row of the wave sees the fewest keys: tiles up to its last key need no causal test
  const int e_first = erow(Rw);

  // K tiles go HBM -> LDS with direct loads into three stages shared by the four waves (rows
  // padded to D + 16 bytes, so the 16 rows one quarter-wave reads land on distinct banks).
  // A step is short here (8 MFMAs) and latency-bound, so the stages are few and four
  // workgroups share a CU (16 waves) rather than keeping many tiles in flight per workgroup:
  // at 64K this is 1.4x faster than six stages at two workgroups per CU.  The stages are one
  // array indexed at run time, so the loop body (and the kernel's code) exists once.
  constexpr int KP = D + 16;
  constexpr int WIN = (64 * KP + 1023) / 1024;       // 1 KB windows per tile
  constexpr int SL = (WIN + 3) / 4;                   // windows per wave
  constexpr int NST = 3;
  __shared__ __attribute__((aligned(1024))) unsigned char kst[NST * WIN * 1024];
  __shared__ __attribute__((aligned(1024))) unsigned char kspare[1024];
  auto stage = [&](int j) { return kst + (j % NST) * (WIN * 1024); };
  const int8_t* kbase = a.kq + ((int64_t)bg * a.nKT * 64) * D;
  int s_off[SL];                                      // byte offset in a tile of this lane's 16 bytes
#pragma unroll
  for (int k = 0; k < SL; ++k) {
    const int o = min(wave + 4 * k, WIN - 1) * 1024 + lane * 16;
    const int r = min(o / KP, 63), c = o % KP;
    s_off[k] = r * D + (c < D ? c : 0);               // pads and the tail get a harmless copy
  }
  auto issue = [&](unsigned char* st, int J) {
    const int8_t* tb = kbase + (int64_t)J * 64 * D;
#pragma unroll
    for (int k = 0; k < SL; ++k) {
      const int wdw = wave + 4 * k;
      __builtin_amdgcn_global_load_lds(tb + s_off[k], LDS_PTR(void, wdw < WIN ? st + wdw * 1024 : kspare), 16, 0, 0);
    }
  };
  const int k_rd = l32 * KP + half * 16;
  // The workgroup's keep-bit words ([query block of its 128 rows][64 words of its 32 key
  // tiles]) collect in LDS and go out in one coalesced copy at the end: global stores inside
  // the loop would count in vmcnt and hold up the direct-load waits.
  constexpr int QBW = 128 / G;                        // query blocks per workgroup
  __shared__ unsigned int sbits[QBW * 64];
  const int R0 = rt * 128;                            // first row of the workgroup

  // one key tile: D = qbar K^T on int8 MFMA (a lane owns one key column and 16 rows), then one
  // compare per element, turned into keep-bit words by wave ballots
  auto tile = [&](const unsigned char* st, int J) {
    i32x4 kf[2][KS];
    read_key_fragments<KS, KP>((unsigned int)(uintptr_t)LDS_PTR(const unsigned char, st + k_rd), kf);
    i32x16 acc[2] = {(i32x16){}, (i32x16){}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[nt] = mfma_i8(qf[ks], kf[nt][ks], acc[nt]);
    const float skv = load_uniform(a.sk + (int64_t)bg * a.nKB + J);
    // keep <=> fp32(fp32(D) * m) - (abar - theta) >= 0 <=> fp32(fp32(D) * m) >= (abar - theta)
    float mult[16], tk[16];
    if (MARGINS) {
#pragma unroll
      for (int r = 0; r < 16; ++r) mult[r] = __fmul_rn(__fmul_rn(sqv[r], skv), a.c);
    } else {
      // D >= u / sk (1 / sk clamped to a finite value: a zero tile has D = 0, kept iff u <= 0)
      const float isk = fminf(1.0f / skv, 1e30f);
#pragma unroll
      for (int r = 0; r < 16; ++r) tk[r] = uthr[r] * isk;
    }
    // the keep bits and margins of the tile; CAUSAL: some key may lie past a row's last key
    auto epilogue = [&](auto causal_tag) {
    constexpr bool CAUSAL = decltype(causal_tag)::value;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int key = J * 64 + nt * 32 + l32;
      const int wi = J * 2 + nt;                         // bit word of columns [key - l32, +32)
      // register r = 4*ag + bb is row Rw + half*4 + 8*ag + bb
#pragma unroll
      for (int ag = 0; ag < 4; ++ag) {
        unsigned long long bal[4];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int r = 4 * ag + bb;
          if (MARGINS) {
            const float y = __fmul_rn((float)acc[nt][r], mult[r]);
            bal[bb] = __ballot(y >= thr[r] && key <= erw[r]);
          } else if (!CAUSAL) {
            bal[bb] = __ballot((float)acc[nt][r] >= tk[r]);
          } else {
            bal[bb] = __ballot((float)acc[nt][r] >= tk[r] && key <= erw[r]);
          }
        }
        const int Rg = Rw + 8 * ag;                      // first row of this 8-row group
        if (lane == 0) {
          if (G <= 4) {
            // G consecutive rows (same half) form one query block: OR their ballots
            unsigned long long word = 0ull;
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
              word |= bal[bb];
              if (((bb + 1) % G) == 0) {
                const int R_lo = Rg + bb + 1 - G, R_hi = R_lo + 4;
                sbits[((R_lo - R0) / G) * 64 + wi - 2 * J0] = (unsigned int)word;
                sbits[((R_hi - R0) / G) * 64 + wi - 2 * J0] = (unsigned int)(word >> 32);
                word = 0ull;
              }
            }
          } else {
            // G == 8: rows Rg .. Rg+7 (both halves) are one query block
            const unsigned long long word = bal[0] | bal[1] | bal[2] | bal[3];
            sbits[((Rg - R0) / G) * 64 + wi - 2 * J0] = (unsigned int)word | (unsigned int)(word >> 32);
          }
        }
        if (MARGINS) {
          // diagnostic output: max over the group's heads of score - (anchor - theta)
          float mv[4];
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            const int r = 4 * ag + bb;
            float m = __fmul_rn((float)acc[nt][r], mult[r]) - thr[r];
            if (key > erw[r] || erw[r] < 0) m = NEG_INF;
            mv[bb] = m;
          }
          if (G <= 4) {
            float mg = NEG_INF;
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
              mg = fmaxf(mg, mv[bb]);
              if (((bb + 1) % G) == 0) {
                const int b0 = bb + 1 - G;
                const int R = Rg + half * 4 + b0;
                if (R < rows_total && key <= erw[4 * ag + b0])
                  a.margins[((int64_t)bg * a.nQB + R / G) * a.N + key] = mg;
                mg = NEG_INF;
              }
            }
          } else {
            float mg = fmaxf(fmaxf(mv[0], mv[1]), fmaxf(mv[2], mv[3]));
            mg = fmaxf(mg, swap_halves(mg));
            if (half == 0 && Rg < rows_total && key <= erw[4 * ag])
              a.margins[((int64_t)bg * a.nQB + Rg / G) * a.N + key] = mg;
          }
        }
      }
    }
    };
    // one branch per tile: tiles wholly before the wave's first row's last key skip the test
    if (MARGINS || J * 64 + 63 > e_first)
      epilogue(std::integral_constant<bool, true>{});
    else
      epilogue(std::integral_constant<bool, false>{});
  };

  // Tile J0 + j is in stage j % NST; tiles j+1 .. j+NST-2 are loaded or in flight.  Step j
  // computes tile j, issues tile j+NST-1 (clamped to the last tile, so every wave issues SL
  // loads per step) into the stage of tile j-1 and waits until tile j+1 has landed.
  const int nt_ = J_end - J0;
#pragma unroll
  for (int p = 0; p < NST - 1; ++p) issue(stage(p), J0 + min(p, nt_ - 1));
  DMA_BARRIER((NST - 2) * SL);
  for (int j = 0; j < nt_; ++j) {
    if (wave_live) tile(stage(j), J0 + j);
    issue(stage(j + NST - 1), J0 + min(j + NST - 1, nt_ - 1));
    DMA_BARRIER((NST - 2) * SL);
  }
  // no DMA may still be writing this workgroup's LDS when it exits
  __builtin_amdgcn_s_waitcnt(VMCNT_IMM(0));
  __syncthreads();
  // the words of the tiles this workgroup computed, for its query blocks that exist
  const int qb0 = R0 / G;
  const int nwords = 2 * nt_;
  for (int p = tid; p < QBW * 64; p += 256) {
    const int qb = p / 64, wd = p % 64;
    if (wd < nwords && qb0 + qb < a.nQB)
      a.bits[(row_base / G + qb0 + qb) * a.W + 2 * J0 + wd] = sbits[p];
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------------------------
// Relative-score estimate (SALE, "What carries the argument"; the log form of the test as
// corrected in referee major comment 1).
//
// est_quant_q_rows: int8 query rows, the rule of the key tiles applied per (b, h, row):
// a = max |q_r|, scale = a / 127, code = rint(q * (127 / a)).  16 lanes per row.
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void est_quant_q_rows(EstArgs a) {
  constexpr int EPL = D / 16;                        // elements per lane (8 or 4)
  const int tid = threadIdx.x, sub = tid & 15;
  const int64_t nrows = (int64_t)a.B * a.N * a.Hq;
  const int64_t R = (int64_t)blockIdx.x * 16 + (tid >> 4);   // rows in (b, token, head) order
  const bool valid = R < nrows;
  const int64_t Rc = valid ? R : nrows - 1;
  const int h = (int)(Rc % a.Hq);
  const int r = (int)((Rc / a.Hq) % a.N);
  const int b = (int)(Rc / ((int64_t)a.Hq * a.N));
  const uint16_t* qp = a.q + b * a.qs0 + (int64_t)r * a.qs1 + a.qh[h] * a.qs2 + sub * EPL;
  float v[EPL];
  if (EPL == 8) {
    const u16x8 u = *(const u16x8*)qp;
#pragma unroll
    for (int e = 0; e < EPL; ++e) v[e] = bf16_bits_to_float(u[e]);
  } else {
    const u32x2 u = *(const u32x2*)qp;
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      v[e] = bf16_bits_to_float((unsigned short)(((e < 2 ? u.x : u.y) >> (16 * (e & 1))) & 0xFFFFu));
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(v[e]));
  for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));   // the 16 lanes
  float inv = 0.f, scale = 1.f;
  if (amax > 0.f) {
    inv = __fdiv_rn(127.0f, amax);
    scale = __fdiv_rn(amax, 127.0f);
  }
  unsigned int w[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    float x = rintf(__fmul_rn(v[e], inv));
    x = fminf(fmaxf(x, -127.f), 127.f);
    w[e >> 2] |= ((unsigned int)((int)x & 0xFF)) << (8 * (e & 3));
  }
  if (!valid) return;
  const int64_t orow = ((int64_t)b * a.Hq + h) * a.N + r;
  int8_t* dst = a.qr + orow * D + sub * EPL;
  if (EPL == 8)
    *(u32x2*)dst = (u32x2){w[0], w[1]};
  else
    *(unsigned int*)dst = w[0];
  if (sub == 0) a.sr[orow] = scale;
}

// est_score_rel: one workgroup per (b, g, query block), longest blocks first.  The block's
// rows of every head of the group are cut into units of 64 rows of one head; each wave takes
// two units at a time, keeps their int8 rows as the B operand of D^T = K_q Q_q^T (32x32x32
// int8 MFMA, exact int32), and
//  1. over the row's sink and local keys (their tiles only) forms LSE_r of the estimated
//     logits S~ = fp32(D) * fp32(fp32(s_q s_K) c) -- a lane owns one row and 16 of the keys
//     of each 32-key subtile, the other 16 sit in lane ^ 32;
//  2. over every causal key tile J takes the row's max of D (S~ is increasing in D for a
//     row and tile, so the max of S~ is S~ of the max), S~ - LSE_r + theta_h, the max over
//     the wave's rows and units, and folds it into the block's margin for J with an LDS
//     atomic max on order-preserving keys.
// The margins of all units (heads and row ranges) then give one keep bit per key block.
template <int D>
__global__ __launch_bounds__(256, 2) void est_score_rel(EstArgs a) {
  // The host pass only needs this kernel's signature (for its launch stub).
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int KS = D / 32;
  extern __shared__ unsigned int mkey[];             // [nKB] best margin key per key block
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = wave_uniform(tid >> 6);
  const int BG = a.B * a.Hkv;
  const int bg = blockIdx.x % BG;
  const int I = a.nQB - 1 - blockIdx.x / BG;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int r0 = I * a.bq;
  const int e = min(a.N, r0 + a.bq) - 1;
  const bool bk32 = a.bk == 32;                      // key blocks of 32: two per 64-key tile
  const int ncand = e / a.bk + 1;                    // causal key blocks
  for (int j = tid; j < ncand; j += 256) mkey[j] = 0u;
  __syncthreads();
  const int SUBS = a.bq / 64;
  const int U = a.G * SUBS;
  const int8_t* kbase = a.kq + ((int64_t)bg * a.nKT * 64) * D + half * 16;
  const float* skb = a.sk + (int64_t)bg * a.nKB;
  const int sink_last = a.sink > 0 ? (min(a.sink, a.N) - 1) / 64 : -1;

  auto load_k = [&](int J, i32x4 (*kf)[KS]) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[mt][ks] = *(const i32x4*)(kbase + (int64_t)(J * 64 + mt * 32 + l32) * D + ks * 32);
  };

  // main-loop key tiles go HBM -> LDS with direct loads into four stages shared by the four
  // waves (rows padded to D + 16 bytes: the 16 rows one quarter-wave reads land on distinct
  // banks)
  constexpr int KP = D + 16;
  constexpr int WIN = (64 * KP + 1023) / 1024;
  constexpr int SL = (WIN + 3) / 4;
  // the four stages are one array indexed at run time, so the main loop's body exists once
  // (its key fragments are read by read_key_fragments, which the compiler does not order
  // behind the loads in flight)
  __shared__ __attribute__((aligned(1024))) unsigned char kst[4 * WIN * 1024];
  __shared__ __attribute__((aligned(1024))) unsigned char kspare[1024];
  auto stage = [&](int j) { return kst + (j & 3) * (WIN * 1024); };
  const int8_t* ktile0 = a.kq + ((int64_t)bg * a.nKT * 64) * D;
  int s_off[SL];
#pragma unroll
  for (int k = 0; k < SL; ++k) {
    const int o = min(wave + 4 * k, WIN - 1) * 1024 + lane * 16;
    const int r = min(o / KP, 63), c = o % KP;
    s_off[k] = r * D + (c < D ? c : 0);               // pads and the tail get a harmless copy
  }
  auto issue = [&](unsigned char* st, int J) {
    const int8_t* tb = ktile0 + (int64_t)J * 64 * D;
#pragma unroll
    for (int k = 0; k < SL; ++k) {
      const int wdw = wave + 4 * k;
      __builtin_amdgcn_global_load_lds(tb + s_off[k], LDS_PTR(void, wdw < WIN ? st + wdw * 1024 : kspare), 16, 0, 0);
    }
  };
  const int k_rd = l32 * KP + half * 16;
  const int Jn = e / 64 + 1;                           // causal 64-key tiles of the block

  for (int u0 = 0; u0 < U; u0 += 8) {
    const int ua = u0 + 2 * wave;
    const int nu = max(0, min(2, U - ua));            // 0: this wave only loads and waits
    i32x4 qf[2][2][KS];
    float sqv[2][2], lse[2][2], thv[2];
    int rowv[2][2], rmin[2], rmax[2];
#pragma unroll
    for (int uu = 0; uu < 2; ++uu) {
      const int u = min(ua + uu, U - 1);
      const int hg = u / SUBS, sb = u % SUBS;
      const int h = g * a.G + hg;
      thv[uu] = a.theta[h];
      rmin[uu] = r0 + sb * 64;
      rmax[uu] = min(rmin[uu] + 63, a.N - 1);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int row = rmin[uu] + nt * 32 + l32;
        rowv[uu][nt] = row;
        const int64_t orow = ((int64_t)b * a.Hq + h) * a.N + min(row, a.N - 1);
        const int8_t* qp = a.qr + orow * D + half * 16;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[uu][nt][ks] = *(const i32x4*)(qp + ks * 32);
        sqv[uu][nt] = a.sr[orow];
      }
    }
    const bool two = nu == 2;
    // D^T of one unit against the key tile in kf
    auto dots = [&](int uu, i32x4 (*kf)[KS], i32x16 (*acc)[2]) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = (i32x16){};
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mfma_i8(kf[mt][ks], qf[uu][nt][ks], acc[mt][nt]);
    };

    // 1. LSE over each row's sink and local keys, from the tiles that hold them
    float mr[2][2], sr_[2][2];
#pragma unroll
    for (int uu = 0; uu < 2; ++uu)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        mr[uu][nt] = NEG_INF;
        sr_[uu][nt] = 0.f;
      }
    const int wlo = max(0, min(rmin[0], two ? rmin[1] : rmin[0]) - a.local + 1) / 64;
    const int whi = nu > 0 ? max(rmax[0], two ? rmax[1] : rmax[0]) / 64 : -1;
    for (int J = 0; J <= whi; ++J) {
      if (J > sink_last && J < wlo) J = wlo;           // skip the tiles between the areas
      i32x4 kf[2][KS];
      load_k(J, kf);
      const float skv0 = load_uniform(skb + (bk32 ? 2 * J : J));
      const float skv1 = bk32 ? load_uniform(skb + min(2 * J + 1, a.nKB - 1)) : skv0;
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        if (uu == 1 && !two) break;
        if (J * 64 > rmax[uu]) continue;
        i32x16 acc[2][2];
        dots(uu, kf, acc);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int row = rowv[uu][nt];
          const float mult0 = __fmul_rn(__fmul_rn(sqv[uu][nt], skv0), a.c);
          const float mult1 = __fmul_rn(__fmul_rn(sqv[uu][nt], skv1), a.c);
          // online log-sum-exp over the lane's keys of the row's area
          float m_ = mr[uu][nt], s_ = sr_[uu][nt];
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = J * 64 + mt * 32 + half * 4 + 8 * (r >> 2) + (r & 3);
              const bool in = key <= row && key < a.N && (key < a.sink || key >= row - a.local + 1);
              if (in) {
                const float v = __fmul_rn((float)acc[mt][nt][r], mt == 0 ? mult0 : mult1);
                const float mn = fmaxf(m_, v);
                s_ = s_ * __expf(m_ - mn) + __expf(v - mn);
                m_ = mn;
              }
            }
          mr[uu][nt] = m_;
          sr_[uu][nt] = s_;
        }
      }
    }
#pragma unroll
    for (int uu = 0; uu < 2; ++uu)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float mo = swap_halves(mr[uu][nt]), so = swap_halves(sr_[uu][nt]);
        const float mt_ = fmaxf(mr[uu][nt], mo);
        float st = 0.f;
        if (mr[uu][nt] > NEG_INF) st += sr_[uu][nt] * __expf(mr[uu][nt] - mt_);
        if (mo > NEG_INF) st += so * __expf(mo - mt_);
        // rows past the end of the sequence take no part
        lse[uu][nt] = (rowv[uu][nt] < a.N && mt_ > NEG_INF) ? mt_ + logf(st) : __builtin_huge_valf();
      }

    // 2. every causal key tile: best (S~ - LSE + theta) over the wave's rows and units
    auto tile = [&](const unsigned char* st, int J) {
      const float skv0 = load_uniform(skb + (bk32 ? 2 * J : J));
      const float skv1 = bk32 ? load_uniform(skb + min(2 * J + 1, a.nKB - 1)) : skv0;
      float best[2] = {NEG_INF, NEG_INF};                // per key block of the tile
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        if (uu == 1 && !two) break;
        if (J * 64 > rmax[uu]) continue;
        i32x16 acc[2][2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = (i32x16){};
        i32x4 kf[2][KS];
        read_key_fragments<KS, KP>((unsigned int)(uintptr_t)LDS_PTR(const unsigned char, st + k_rd), kf);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mfma_i8(kf[mt][ks], qf[uu][nt][ks], acc[mt][nt]);
        const bool need_mask = J * 64 + 63 > rmin[uu] || J * 64 + 63 >= a.N;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int row = rowv[uu][nt];
          int m[2] = {INT32_MIN, INT32_MIN};
          if (!need_mask) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
              for (int r = 0; r < 16; ++r) m[mt] = max(m[mt], acc[mt][nt][r]);
          } else {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int key = J * 64 + mt * 32 + half * 4 + 8 * (r >> 2) + (r & 3);
                if (key <= row && key < a.N) m[mt] = max(m[mt], acc[mt][nt][r]);
              }
          }
          if (!bk32) m[0] = max(m[0], m[1]);
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            if (hb == 1 && !bk32) break;
            const int mm = max(m[hb], swap_halves_i(m[hb]));
            if (mm != INT32_MIN && row < a.N) {
              const float mult = __fmul_rn(__fmul_rn(sqv[uu][nt], hb == 0 ? skv0 : skv1), a.c);
              const float rel = __fmul_rn((float)mm, mult) - lse[uu][nt];
              best[hb] = fmaxf(best[hb], rel + thv[uu]);
            }
          }
        }
      }
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        if (hb == 1 && !bk32) break;
        const float bw = wave_max(best[hb]);
        if (lane == 0 && bw > NEG_INF) lds_max_u32(&mkey[bk32 ? 2 * J + hb : J], float_order_key(bw));
      }
    };
    // Tile j is in stage j % 4; tiles j+1 and j+2 are loaded or in flight.  Step j computes
    // tile j (waves with units), issues tile j+3 (clamped to the last tile, so every wave
    // issues SL loads per step) into the stage of tile j-1 and waits until tile j+1 landed.
    issue(stage(0), 0);
    issue(stage(1), min(1, Jn - 1));
    issue(stage(2), min(2, Jn - 1));
    DMA_BARRIER(2 * SL);
    for (int J = 0; J < Jn; ++J) {
      if (nu > 0) tile(stage(J), J);
      issue(stage(J + 3), min(J + 3, Jn - 1));
      DMA_BARRIER(2 * SL);
    }
    // the stages are reused by the next pass: every load has landed and every wave is done
    __builtin_amdgcn_s_waitcnt(VMCNT_IMM(0));
    __syncthreads();
  }
  __syncthreads();
  // keep bits (forced blocks are added by the compaction) and the optional margins
  const int64_t brow = (int64_t)bg * a.nQB + I;
  for (int J0 = wave * 64; J0 < a.W * 32; J0 += 256) {
    const int J = J0 + lane;
    float margin = NEG_INF;
    if (J < ncand && mkey[J] != 0u) {
      const unsigned int k = mkey[J];
      margin = __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
    }
    const unsigned long long bal = __ballot(J < ncand && margin >= 0.f);
    if (lane == 0) {
      const int w = J0 / 32;
      a.bits[brow * a.W + w] = (unsigned int)bal;
      if (w + 1 < a.W) a.bits[brow * a.W + w + 1] = (unsigned int)(bal >> 32);
    }
    if (a.margins && J < ncand) a.margins[brow * a.nKB + J] = margin;
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------------------------
// MXFP4 relative estimate (the pages' estimate is 4-bit; here the OCP Microscaling v1.0
// MXFP4 format that the gfx950 block-scaled fp4 MFMA consumes).
//
// est_quant_rows_fp4: one thread per 32 head dims of a Q row (which = 0) or a K row (which =
// 1, rows up to the padded key count; rows past the sequence become zeros).  Shared exponent
// e = floor(log2 max|x|) - 2 clamped to [-127, 127] (stored as the E8M0 byte e + 127), codes
// E2M1 of |x| * 2^-e (exact scaling) rounded to nearest with ties to the even code, saturating
// at 6, sign in bit 3; 32 codes in 16 bytes, dim j of the block in nibble j (low nibble first).
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void est_quant_rows_fp4(EstArgs a, int which) {
  constexpr int NC = D / 32;                         // blocks per row
  const int64_t rows = which == 0 ? (int64_t)a.B * a.N * a.Hq : (int64_t)a.B * a.Hkv * a.nKT * 64;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= rows * NC) return;
  const int c = (int)(t % NC);
  const int64_t row = t / NC;
  const uint16_t* src = nullptr;
  uint8_t* codes;
  uint8_t* scales;
  if (which == 0) {                                  // row = (b, token, head): out [B, Hq, N]
    const int h = (int)(row % a.Hq);
    const int r = (int)((row / a.Hq) % a.N);
    const int b = (int)(row / ((int64_t)a.Hq * a.N));
    src = a.q + b * a.qs0 + (int64_t)r * a.qs1 + a.qh[h] * a.qs2 + c * 32;
    const int64_t orow = ((int64_t)b * a.Hq + h) * a.N + r;
    codes = (uint8_t*)a.qr + orow * (D / 2) + c * 16;
    scales = (uint8_t*)a.sr + orow * NC + c;
  } else {                                           // row = (b, g, token of the padded tiles)
    const int r = (int)(row % ((int64_t)a.nKT * 64));
    const int bg = (int)(row / ((int64_t)a.nKT * 64));
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    if (r < a.N) src = a.k + b * a.ks0 + (int64_t)r * a.ks1 + g * a.ks2 + c * 32;
    codes = a.k4 + row * (D / 2) + c * 16;
    scales = a.k4s + row * NC + c;
  }
  float v[32];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    u16x8 u = (u16x8)(0);
    if (src) u = *(const u16x8*)(src + 8 * j);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[8 * j + e] = bf16_bits_to_float(u[e]);
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(v[e]));
  int ex = -127;
  if (amax > 0.f) ex = max((int)((__float_as_uint(amax) >> 23) & 0xFF) - 129, -127);
  unsigned int w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    unsigned int code = e2m1_code(ldexpf(fabsf(v[e]), -ex));
    if (v[e] < 0.f) code |= 8u;
    w[e >> 3] |= code << (4 * (e & 7));
  }
  *(u32x4*)codes = (u32x4){w[0], w[1], w[2], w[3]};
  *scales = (uint8_t)(ex + 127);
}

// est_score_rel_fp4: est_score_rel with the dot products on v_mfma_scale_f32_32x32x64
// (fp4 x fp4, one E8M0 scale per lane = per 32 dims of its row): a lane holds 32 dims (16
// bytes) of its key row (A) or query row (B) per 64-dim k-step, lane halves taking the two
// 32-dim blocks, and the MFMA returns the real dot product; S~ = fp32(dot) * c.
typedef int v8i_ __attribute__((ext_vector_type(8)));
SA_DEV f32x16 mfma_fp4(i32x4 a, i32x4 b, f32x16 c, int sa, int sb) {
  const v8i_ av = {a.x, a.y, a.z, a.w, 0, 0, 0, 0};
  const v8i_ bv = {b.x, b.y, b.z, b.w, 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, 0, sa, 0, sb);
}

template <int D>
__global__ __launch_bounds__(256, 2) void est_score_rel_fp4(EstArgs a) {
  // The host pass only needs this kernel's signature (for its launch stub).
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int S = D / 64;                          // 64-dim k-steps
  constexpr int CB = D / 2, SB = D / 32;             // code / scale bytes per row
  extern __shared__ unsigned int mkey[];             // [nKB] best margin key per key block
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = wave_uniform(tid >> 6);
  const int BG = a.B * a.Hkv;
  const int bg = blockIdx.x % BG;
  const int I = a.nQB - 1 - blockIdx.x / BG;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int r0 = I * a.bq;
  const int e = min(a.N, r0 + a.bq) - 1;
  const bool bk32 = a.bk == 32;                      // key blocks of 32: two per 64-key tile
  const int ncand = e / a.bk + 1;                    // causal key blocks
  for (int j = tid; j < ncand; j += 256) mkey[j] = 0u;
  __syncthreads();
  const int SUBS = a.bq / 64;
  const int U = a.G * SUBS;
  const uint8_t* kc0 = a.k4 + ((int64_t)bg * a.nKT * 64) * CB;
  const uint8_t* ksc0 = a.k4s + ((int64_t)bg * a.nKT * 64) * SB;
  const int sink_last = a.sink > 0 ? (min(a.sink, a.N) - 1) / 64 : -1;

  // key tiles in LDS: 64 code rows (pitch CB + 16: the 16 rows one quarter-wave reads land on
  // distinct banks), then the 64 rows' scale bytes
  constexpr int KP = CB + 16;
  constexpr int CODEB = 64 * KP, TILEB = CODEB + 64 * SB;
  constexpr int WIN = (TILEB + 1023) / 1024;
  constexpr int SL = (WIN + 3) / 4;
  __shared__ __attribute__((aligned(1024))) unsigned char ks0[WIN * 1024];
  __shared__ __attribute__((aligned(1024))) unsigned char ks1[WIN * 1024];
  __shared__ __attribute__((aligned(1024))) unsigned char ks2[WIN * 1024];
  __shared__ __attribute__((aligned(1024))) unsigned char ks3[WIN * 1024];
  __shared__ __attribute__((aligned(1024))) unsigned char kspare[1024];
  int s_off[SL];
  bool s_sc[SL];                                     // wave-uniform: slot copies scale bytes
#pragma unroll
  for (int k = 0; k < SL; ++k) {
    const int o = min(wave + 4 * k, WIN - 1) * 1024 + lane * 16;
    if (o < CODEB) {
      const int r = o / KP, c = o % KP;
      s_off[k] = r * CB + (c < CB ? c : 0);         // pads get a harmless copy
      s_sc[k] = false;
    } else {
      const int so = o - CODEB;
      s_off[k] = so < 64 * SB ? so : 0;
      s_sc[k] = true;
    }
  }
  auto issue = [&](unsigned char* st, int J) {
    const uint8_t* ct = kc0 + (int64_t)J * 64 * CB;
    const uint8_t* stl = ksc0 + (int64_t)J * 64 * SB;
#pragma unroll
    for (int k = 0; k < SL; ++k) {
      const int wdw = wave + 4 * k;
      __builtin_amdgcn_global_load_lds((s_sc[k] ? stl : ct) + s_off[k],
                                       LDS_PTR(void, wdw < WIN ? st + wdw * 1024 : kspare), 16, 0, 0);
    }
  };
  const int Jn = e / 64 + 1;                         // causal 64-key tiles

  for (int u0 = 0; u0 < U; u0 += 8) {
    const int ua = u0 + 2 * wave;
    const int nu = max(0, min(2, U - ua));            // 0: this wave only loads and waits
    i32x4 qf[2][2][S];
    int qs[2][2][S];
    float lse[2][2], thv[2];
    int rowv[2][2], rmin[2], rmax[2];
#pragma unroll
    for (int uu = 0; uu < 2; ++uu) {
      const int u = min(ua + uu, U - 1);
      const int hg = u / SUBS, sb = u % SUBS;
      const int h = g * a.G + hg;
      thv[uu] = a.theta[h];
      rmin[uu] = r0 + sb * 64;
      rmax[uu] = min(rmin[uu] + 63, a.N - 1);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int row = rmin[uu] + nt * 32 + l32;
        rowv[uu][nt] = row;
        const int64_t orow = ((int64_t)b * a.Hq + h) * a.N + min(row, a.N - 1);
        const uint8_t* qp = (const uint8_t*)a.qr + orow * CB + half * 16;
        const uint8_t* sp = (const uint8_t*)a.sr + orow * SB + half;
#pragma unroll
        for (int s2 = 0; s2 < S; ++s2) {
          qf[uu][nt][s2] = *(const i32x4*)(qp + s2 * 32);
          qs[uu][nt][s2] = sp[s2 * 2];
        }
      }
    }
    const bool two = nu == 2;
    // real dot products of one unit's rows with key rows from `kc` (codes) / `ksc` (scales)
    auto dots = [&](int uu, const uint8_t* kc, int kpitch, const uint8_t* ksc, f32x16 (*acc)[2]) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = (f32x16){};
#pragma unroll
      for (int s2 = 0; s2 < S; ++s2)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const i32x4 kf = *(const i32x4*)(kc + (mt * 32 + l32) * kpitch + (2 * s2 + half) * 16);
          const int ksv = ksc[(mt * 32 + l32) * SB + 2 * s2 + half];
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            acc[mt][nt] = mfma_fp4(kf, qf[uu][nt][s2], acc[mt][nt], ksv, qs[uu][nt][s2]);
        }
    };

    // 1. LSE over each row's sink and local keys (their tiles, read from global memory)
    float mr[2][2], sr_[2][2];
#pragma unroll
    for (int uu = 0; uu < 2; ++uu)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        mr[uu][nt] = NEG_INF;
        sr_[uu][nt] = 0.f;
      }
    const int wlo = max(0, min(rmin[0], two ? rmin[1] : rmin[0]) - a.local + 1) / 64;
    const int whi = nu > 0 ? max(rmax[0], two ? rmax[1] : rmax[0]) / 64 : -1;
    for (int J = 0; J <= whi; ++J) {
      if (J > sink_last && J < wlo) J = wlo;           // skip the tiles between the areas
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        if (uu == 1 && !two) break;
        if (J * 64 > rmax[uu]) continue;
        f32x16 acc[2][2];
        dots(uu, kc0 + (int64_t)J * 64 * CB, CB, ksc0 + (int64_t)J * 64 * SB, acc);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int row = rowv[uu][nt];
          float m_ = mr[uu][nt], s_ = sr_[uu][nt];
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = J * 64 + mt * 32 + half * 4 + 8 * (r >> 2) + (r & 3);
              const bool in = key <= row && key < a.N && (key < a.sink || key >= row - a.local + 1);
              if (in) {
                const float v = __fmul_rn(acc[mt][nt][r], a.c);
                const float mn = fmaxf(m_, v);
                s_ = s_ * __expf(m_ - mn) + __expf(v - mn);
                m_ = mn;
              }
            }
          mr[uu][nt] = m_;
          sr_[uu][nt] = s_;
        }
      }
    }
#pragma unroll
    for (int uu = 0; uu < 2; ++uu)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float mo = swap_halves(mr[uu][nt]), so = swap_halves(sr_[uu][nt]);
        const float mt_ = fmaxf(mr[uu][nt], mo);
        float st = 0.f;
        if (mr[uu][nt] > NEG_INF) st += sr_[uu][nt] * __expf(mr[uu][nt] - mt_);
        if (mo > NEG_INF) st += so * __expf(mo - mt_);
        lse[uu][nt] = (rowv[uu][nt] < a.N && mt_ > NEG_INF) ? mt_ + logf(st) : __builtin_huge_valf();
      }

    // 2. every causal key tile: best (S~ - LSE + theta) over the wave's rows and units
    auto tile = [&](const unsigned char* st, int J) {
      float best[2] = {NEG_INF, NEG_INF};                // per key block of the tile
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        if (uu == 1 && !two) break;
        if (J * 64 > rmax[uu]) continue;
        f32x16 acc[2][2];
        dots(uu, st, KP, st + CODEB, acc);
        const bool need_mask = J * 64 + 63 > rmin[uu] || J * 64 + 63 >= a.N;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int row = rowv[uu][nt];
          float m[2] = {NEG_INF, NEG_INF};
          if (!need_mask) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
              for (int r = 0; r < 16; ++r) m[mt] = fmaxf(m[mt], acc[mt][nt][r]);
          } else {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int key = J * 64 + mt * 32 + half * 4 + 8 * (r >> 2) + (r & 3);
                if (key <= row && key < a.N) m[mt] = fmaxf(m[mt], acc[mt][nt][r]);
              }
          }
          if (!bk32) m[0] = fmaxf(m[0], m[1]);
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            if (hb == 1 && !bk32) break;
            const float mm = fmaxf(m[hb], swap_halves(m[hb]));
            if (mm > NEG_INF && row < a.N)
              best[hb] = fmaxf(best[hb], __fmul_rn(mm, a.c) - lse[uu][nt] + thv[uu]);
          }
        }
      }
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        if (hb == 1 && !bk32) break;
        const float bw = wave_max(best[hb]);
        if (lane == 0 && bw > NEG_INF) lds_max_u32(&mkey[bk32 ? 2 * J + hb : J], float_order_key(bw));
      }
    };
    issue(ks0, 0);
    issue(ks1, min(1, Jn - 1));
    issue(ks2, min(2, Jn - 1));
    DMA_BARRIER(2 * SL);
    auto step = [&](const unsigned char* sc, unsigned char* sd, int J) {
      if (nu > 0) tile(sc, J);
      issue(sd, min(J + 3, Jn - 1));
      DMA_BARRIER(2 * SL);
    };
    int J = 0;
    for (; J + 4 <= Jn; J += 4) {
      step(ks0, ks3, J);
      step(ks1, ks0, J + 1);
      step(ks2, ks1, J + 2);
      step(ks3, ks2, J + 3);
    }
    if (J < Jn) step(ks0, ks3, J);
    if (J + 1 < Jn) step(ks1, ks0, J + 1);
    if (J + 2 < Jn) step(ks2, ks1, J + 2);
    __builtin_amdgcn_s_waitcnt(VMCNT_IMM(0));
    __syncthreads();
  }
  // keep bits (forced blocks are added by the compaction) and the optional margins
  const int64_t brow = (int64_t)bg * a.nQB + I;
  for (int J0 = wave * 64; J0 < a.W * 32; J0 += 256) {
    const int J = J0 + lane;
    float margin = NEG_INF;
    if (J < ncand && mkey[J] != 0u) {
      const unsigned int k = mkey[J];
      margin = __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
    }
    const unsigned long long bal = __ballot(J < ncand && margin >= 0.f);
    if (lane == 0) {
      const int w = J0 / 32;
      a.bits[brow * a.W + w] = (unsigned int)bal;
      if (w + 1 < a.W) a.bits[brow * a.W + w + 1] = (unsigned int)(bal >> 32);
    }
    if (a.margins && J < ncand) a.margins[brow * a.nKB + J] = margin;
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------------------------
// Grouped identification (AnchorAttention's step): the keep bits of every query block of a
// group of `step` become the OR over the group; the compaction then adds each block's forced
// entries and keeps its causal candidates only.  One workgroup per (b, g, group).
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void est_step_or(EstArgs a) {
  const int n_groups = (a.nQB + a.step - 1) / a.step;
  const int gi = blockIdx.x % n_groups;
  const int bg = blockIdx.x / n_groups;
  const int i0 = gi * a.step, i1 = min(a.nQB, i0 + a.step);
  uint32_t* rows = a.bits + ((int64_t)bg * a.nQB) * a.W;
  for (int w = threadIdx.x; w < a.W; w += 256) {
    unsigned int acc = 0u;
    for (int i = i0; i < i1; ++i) acc |= rows[(int64_t)i * a.W + w];
    for (int i = i0; i < i1; ++i) rows[(int64_t)i * a.W + w] = acc;
  }
}

// ---------------------------------------------------------------------------------------
// Compaction: per (b, g, i) row, keep = (bits | forced) & causal candidates, written as
// ascending indices; `unit` = block_k (block lists) or 1 (stripe lists).
// ---------------------------------------------------------------------------------------
static __device__ __forceinline__ unsigned int range_bits(int w, int lo, int hi) {
  // bits of x in [lo, hi] within word w (x = w*32 + bit)
  const int base = w * 32;
  const int a = max(lo - base, 0);
  const int b = min(hi - base, 31);
  if (a > b) return 0u;
  const unsigned int upper = (b == 31) ? 0xFFFFFFFFu : ((1u << (b + 1)) - 1u);
  const unsigned int lower = (1u << a) - 1u;
  return upper & ~lower;
}

__global__ __launch_bounds__(256) void est_compact(EstArgs a, int unit) {
  const int row = blockIdx.x;
  const int iq = row % a.nQB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = iq * a.bq;
  const int e = min(a.N, r0 + a.bq) - 1;
  const int lo = max(0, r0 - a.local + 1);
  const int ncand = e / unit + 1;
  const int nwords = (ncand + 31) / 32;
  const int sink_last = (a.sink + unit - 1) / unit - 1;      // forced sink candidates [0, sink_last]
  const int win_lo = lo / unit, win_hi = e / unit;
  const uint32_t* wrow = a.bits + (int64_t)row * a.W;
  const int per = (nwords + 255) / 256;
  const int w0 = tid * per, w1 = min(w0 + per, nwords);
  int cnt = 0;
  for (int w = w0; w < w1; ++w) {
    unsigned int word = wrow[w] | range_bits(w, 0, sink_last) | range_bits(w, win_lo, win_hi);
    word &= range_bits(w, 0, ncand - 1);
    cnt += __popc(word);
  }
  // block-wide exclusive scan of cnt
  __shared__ int wsum[4];
  int incl = cnt;
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = incl - cnt;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  const int total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  int32_t* out = a.idx + (int64_t)row * a.stride;
  int pos = base;
  for (int w = w0; w < w1; ++w) {
    unsigned int word = wrow[w] | range_bits(w, 0, sink_last) | range_bits(w, win_lo, win_hi);
    word &= range_bits(w, 0, ncand - 1);
    while (word) {
      const int bit = __builtin_ctz(word);
      word &= word - 1u;
      if (pos < a.stride) out[pos] = w * 32 + bit;
      ++pos;
    }
  }
  if (tid == 0) a.counts[row] = total;
}

// ---------------------------------------------------------------------------------------
static void launch_step_or(const EstArgs& a, hipStream_t s) {
  if (a.step <= 1 || a.nQB <= 1) return;
  const int n_groups = (a.nQB + a.step - 1) / a.step;
  hipLaunchKernelGGL(est_step_or, dim3(a.B * a.Hkv * n_groups), dim3(256), 0, s, a);
}

template <int D>
static hipError_t launch_estimate_d(const EstArgs& a, int granularity, hipStream_t s) {
  if (a.estimator == SA_EST_RELATIVE_MXFP4) {
    const int64_t qchunks = (int64_t)a.B * a.N * a.Hq * (D / 32);
    const int64_t kchunks = (int64_t)a.B * a.Hkv * a.nKT * 64 * (D / 32);
    hipLaunchKernelGGL(est_quant_rows_fp4<D>, dim3((unsigned int)((qchunks + 255) / 256)), dim3(256), 0, s, a, 0);
    hipLaunchKernelGGL(est_quant_rows_fp4<D>, dim3((unsigned int)((kchunks + 255) / 256)), dim3(256), 0, s, a, 1);
    hipLaunchKernelGGL(est_score_rel_fp4<D>, dim3(a.B * a.Hkv * a.nQB), dim3(256),
                       (size_t)a.nKB * sizeof(unsigned int), s, a);
    launch_step_or(a, s);
    hipLaunchKernelGGL(est_compact, dim3(a.B * a.Hkv * a.nQB), dim3(256), 0, s, a, a.bk);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(est_quant_k<D>, dim3(a.nKT, a.Hkv, a.B), dim3(256), 0, s, a);
  if (a.estimator == SA_EST_RELATIVE) {
    const int64_t rows = (int64_t)a.B * a.N * a.Hq;
    hipLaunchKernelGGL(est_quant_q_rows<D>, dim3((unsigned int)((rows + 15) / 16)), dim3(256), 0, s, a);
    hipLaunchKernelGGL(est_score_rel<D>, dim3(a.B * a.Hkv * a.nQB), dim3(256),
                       (size_t)a.nKB * sizeof(unsigned int), s, a);
    launch_step_or(a, s);
    hipLaunchKernelGGL(est_compact, dim3(a.B * a.Hkv * a.nQB), dim3(256), 0, s, a, a.bk);
    return hipGetLastError();
  }
  // rows of the staged key window: sink tiles + window tiles of the largest query block
  const int sink_rows = ((min(a.sink, a.N) + 31) / 32) * 32;
  const int win_rows = ((a.local - 1 + a.bq - 1) / 32 + 2) * 32;
  if (sink_rows + win_rows <= 512)
    hipLaunchKernelGGL(est_anchor_pool<D>, dim3(a.nQB * a.Hkv * a.B), dim3(64 * EST_AP_WAVES), 0, s, a);
  else
    hipLaunchKernelGGL(est_anchor_pool_gl<D>, dim3(a.nQB, a.Hkv, a.B), dim3(256), 0, s, a);
  const int rows_total = a.nQB * a.G;
  const int n_rt = (rows_total + 255) / 256;
  const int n_jc = (a.nKT + 31) / 32;                // chunks of 32 key tiles of 64
  const int grid = a.B * a.Hkv * n_rt * n_jc;
  if (granularity == SA_STRIPE) {
    const int n_rt_s = (rows_total + 127) / 128;
    // the instance without the diagnostic margins output keeps its registers for the hot loop
    const dim3 sgrid(a.B * a.Hkv * n_rt_s * n_jc);
#define SA_STRIPE_LAUNCH(GG)                                                                  \
  if (a.margins)                                                                              \
    hipLaunchKernelGGL((est_score_stripe<D, GG, true>), sgrid, dim3(256), 0, s, a, n_rt_s, n_jc); \
  else                                                                                        \
    hipLaunchKernelGGL((est_score_stripe<D, GG, false>), sgrid, dim3(256), 0, s, a, n_rt_s, n_jc);
    if (a.G == 1) {
      SA_STRIPE_LAUNCH(1)
    } else if (a.G == 2) {
      SA_STRIPE_LAUNCH(2)
    } else if (a.G == 4) {
      SA_STRIPE_LAUNCH(4)
    } else {
      SA_STRIPE_LAUNCH(8)
    }
#undef SA_STRIPE_LAUNCH
    launch_step_or(a, s);
    hipLaunchKernelGGL(est_compact, dim3(a.B * a.Hkv * a.nQB), dim3(256), 0, s, a, 1);
  } else {
    hipLaunchKernelGGL(est_score_block<D>, dim3(grid), dim3(256), 0, s, a, n_rt, n_jc);
    launch_step_or(a, s);
    hipLaunchKernelGGL(est_compact, dim3(a.B * a.Hkv * a.nQB), dim3(256), 0, s, a, a.bk);
  }
  return hipGetLastError();
}

hipError_t launch_estimate(const EstArgs& a, int granularity, hipStream_t s) {
  if (a.D == 64) return launch_estimate_d<64>(a, granularity, s);
  return launch_estimate_d<128>(a, granularity, s);
}
