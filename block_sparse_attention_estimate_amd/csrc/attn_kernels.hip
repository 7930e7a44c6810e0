// Block- and stripe-sparse attention (the computation pass) on gfx950.
//
// SALE (arXiv 2505.24179), "What carries the argument": attention is computed only on the
// blocks the estimate keeps.  AnchorAttention (arXiv 2505.23520), "Core claim": stripe
// granularity loads only the selected key/value rows (discrete K/V loading).  The online
// softmax keeps a running row max and sum (the M and Acc buffers of AnchorAttention's
// kernel, referee major comment 1).
//
// attn_block (one workgroup = HPW query heads of one KV head x 64 query rows, 2 waves per head):
//  * the K tile (64 keys) and V tile are staged once in LDS and shared by the HPW packed query
//    heads (GQA packing), four stages filled by direct loads (below);
//  * S^T = K Q^T on 32x32x16 bf16 MFMA: each lane owns one query row and 16 keys of each
//    32-key half, so the row statistics are in-lane plus one exchange with lane ^ 32;
//  * O^T += V^T P^T: P^T is the S^T accumulator converted to bf16 in place (no LDS round
//    trip), V^T is read with transposing LDS reads;
//  * software pipeline: S(t+1) is computed while tile t's exponentials run;
//  * the running max moves only when a tile's probabilities would exceed 2^16, so O is rarely
//    rescaled;
//  * work items are ordered longest-first (last query blocks first), the two 64-row halves of
//    a 128-row query block (same list, same K/V) land on the same XCD, and the KV group
//    rotates every 16 query blocks;
//  * instances: block lists, column lists (gathered rows), and resuming from an anchor state.
#include <stdlib.h>

#include "sa_common.h"
#include "sa_internal.h"

#define NEG_INF (-__builtin_huge_valf())

// ---------------------------------------------------------------------------------------
// K/V tiles go HBM -> LDS with direct loads (global_load_lds_dwordx4), no staging registers.
// Four LDS stages: tile t is consumed while tiles t+1..t+3 are in flight.  Block lists load
// 64 consecutive key rows per tile; column lists (STRIPE) gather the 64 listed rows of a tile,
// each lane addressing the row its 16 bytes belong to (discrete K/V loading).
//  * K rows keep head_dim order with a 16-byte pad per row (pitch 272 B for d = 128), so the
//    A-operand reads of S^T = K Q^T (16 rows x 16 B per lane group) hit distinct banks.
//  * V rows are stored as they are (pitch 320 B for d = 128); the A operand of O^T += V^T P^T
//    is read with ds_read_b64_tr_b16: within a 16-lane group, lane j addresses the 4 dims
//    [d0 + 4(j%4), +4) of key row k0 + j/4, and the read returns to lane i the 4 keys
//    k0..k0+3 of dim d0 + i -- exactly the 4 keys the P^T register layout pairs with that lane.
// ---------------------------------------------------------------------------------------

template <int D, int HPW, bool RESUME, bool STRIPE>
__global__ __launch_bounds__(128 * HPW) void attn_block(AttnArgs a) {
  // The host pass only needs this kernel's signature (for its launch stub).
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NWV = 2 * HPW;             // waves: 2 slices of 32 rows per head
  constexpr int KS = D / 16;               // k-steps of S^T
  constexpr int DM = D / 32;               // d tiles of O^T
  constexpr int ROWB = D * 2;              // bytes of one K/V row
  constexpr int KPITCH = D == 128 ? 272 : 144;
  constexpr int VPITCH = D == 128 ? 320 : 192;
  constexpr int KREG = 64 * KPITCH, VREG = 64 * VPITCH;
  constexpr int KWIN = KREG / 1024, VWIN = VREG / 1024, NWIN = KWIN + VWIN;
  constexpr int STAGE = KREG + VREG;
  // DMA: the first half of the waves loads the K windows of a stage, the second half the V
  // windows; every wave issues SLOTS loads per tile (surplus slots go to `spare`)
  constexpr int HW = NWV / 2;
  constexpr int SLOTS = (KWIN + HW - 1) / HW > (VWIN + HW - 1) / HW ? (KWIN + HW - 1) / HW
                                                                      : (VWIN + HW - 1) / HW;
  static_assert(KREG % 1024 == 0 && VREG % 1024 == 0, "DMA windows must tile the stage");
  // four stages as distinct objects, so the compiler can tell a load into one stage from
  // reads of another; windows past NWIN (to give every wave the same count) go to `spare`
  __shared__ __attribute__((aligned(1024))) unsigned char st0[STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st1[STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st2[STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char st3[STAGE];
  __shared__ __attribute__((aligned(1024))) unsigned char spare[1024];

  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = wave_uniform(tid >> 6);

  // ---- work item (longest first; both halves of a query block on one XCD) ----
  int w = blockIdx.x;
  if (a.tpb == 2) {
    const int full = (a.total / 16) * 16;
    if (w < full) w = (w / 16) * 16 + (w % 8) * 2 + ((w / 8) & 1);
  }
  const int tsub = w % a.tpb;
  int rest = w / a.tpb;
  const int hp = rest % a.n_hp;
  rest /= a.n_hp;
  const int BG = a.B * a.Hkv;
  const int i_rev = rest / BG;
  // the KV group rotates every 16 query blocks: the ~16 work items an XCD runs at a time share
  // one group's K/V in that XCD's L2, while over the launch every XCD sees every group
  const int gb = (rest % BG + i_rev / 16) % BG;
  const int g = gb % a.Hkv;
  const int b = gb / a.Hkv;
  const int iq = a.nQB - 1 - i_rev;
  const int r0 = iq * a.bq + tsub * 64;
  if (iq < 0 || r0 >= a.N) return;
  const int r_last = min(r0 + 63, a.N - 1);
  const int h = g * a.G + hp * HPW + (wave >> 1);
  const int rw = r0 + (wave & 1) * 32;
  const int row = rw + l32;

  // the lists are read-only here: read them through the constant address space (scalar loads)
  const int64_t lrow = (int64_t)(b * a.Hkv + g) * a.nQB + iq;
  const __attribute__((address_space(4))) int32_t* list =
      (const __attribute__((address_space(4))) int32_t*)(a.idx + lrow * a.stride);
  int n = min(((const __attribute__((address_space(4))) int32_t*)a.counts)[lrow], a.stride);
  // the same list through a plain pointer, for per-lane reads of gathered column ids
  const int32_t* list_g = a.idx + lrow * a.stride;
  int ntile, n_main;
  if (STRIPE) {
    // column lists: the entries this work item can see (<= r_last, ascending); tiles of 64
    // gathered columns; tiles from n_main on need a mask (a column past the first row's
    // diagonal or the end, or entries past the list's end)
    int lo = 0, hi = n;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (list[mid] <= r_last) lo = mid + 1; else hi = mid;
    }
    n = lo;
    ntile = (n + 63) / 64;
    n_main = ntile;
    while (n_main > 0 && (list[min(n_main * 64, n) - 1] > r0 || n_main * 64 > n)) --n_main;
  } else {
    // Tiles past `cut` hold no key this work item needs: causally masked for every row, or (when
    // resuming) causally masked or inside every row's local window, which the anchor state holds.
    const int cut = RESUME ? r_last - a.local + 1 : r_last + 1;
    while (n > 0 && list[n - 1] * 64 >= cut) --n;
    if (RESUME) {
      // leading tiles entirely inside the sink tokens are in every row's anchor region too
      int first = 0;
      while (first < n && list[first] * 64 + 63 < a.sink) ++first;
      list += first;
      n -= first;
    }
    // Tiles from n_main on need a mask: they reach past the first row's diagonal (or, resuming,
    // into the first row's local window) or past the end of the sequence.
    const int mlim = RESUME ? r0 - a.local + 1 : r0 + 1;
    ntile = n;
    n_main = n;
    while (n_main > 0 && (list[n_main - 1] * 64 + 63 >= mlim || list[n_main - 1] * 64 + 63 >= a.N)) --n_main;
  }

  bf16x8 qf[KS];
  {
    const int rowc = min(row, a.N - 1);
    const uint16_t* qp = a.q + b * a.qs0 + (int64_t)rowc * a.qs1 + h * a.qs2 + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const bf16x8*)(qp + ks * 16);
  }

  // ---- DMA slots of this wave ----
  const bool dma_v = wave >= HW;                       // this wave loads V windows
  const int wbase = (dma_v ? wave - HW : wave) * SLOTS;  // first window of this wave
  const int nwin = dma_v ? VWIN : KWIN;
  const int pitch_b = dma_v ? VPITCH : KPITCH;
  const int64_t tstride = dma_v ? a.vs1 : a.ks1;       // elements between key rows
  const uint16_t* gbase = dma_v ? a.v + b * a.vs0 + g * a.vs2 : a.k + b * a.ks0 + g * a.ks2;
  const int region = dma_v ? KREG : 0;
  int s_off[SLOTS];                                    // element offset in a full tile
  int s_row[STRIPE ? SLOTS : 1];                       // (gathered tiles) row of this lane's bytes
#pragma unroll
  for (int k = 0; k < SLOTS; ++k) {
    const int o = min(wbase + k, nwin - 1) * 1024 + lane * 16;
    const int r = o / pitch_b, cb = o % pitch_b;
    if (STRIPE) {
      s_row[k] = r;
      s_off[k] = (cb < ROWB ? cb / 16 : 0) * 8;       // column offset within the row
    } else {
      s_off[k] = r * (int)tstride + (cb < ROWB ? cb / 16 : 0) * 8;   // pads get a harmless copy
    }
  }
  // What the DMA of tile t needs, read one step ahead of the issue: the key block id (block
  // lists; a scalar load), or this lane's column id per slot (column lists; vector loads, rows
  // past the list's end repeat its last entry).
  struct Src {
    int v[STRIPE ? SLOTS : 1];
  };
  auto fetch = [&](int t) -> Src {
    Src sv;
    if constexpr (STRIPE) {
      const int tt = min(t, ntile - 1);
#pragma unroll
      for (int k = 0; k < SLOTS; ++k) sv.v[k] = list_g[min(tt * 64 + s_row[k], n - 1)];
    } else {
      sv.v[0] = list[min(t, ntile - 1)];
    }
    return sv;
  };
  // Issue the DMA of tile t (clamped to the list) into the stage at stb.  Every wave issues exactly
  // SLOTS loads per call, so the vmcnt waits below are compile-time constants.
  auto issue = [&](unsigned char* stb, const Src& sv) {
    if constexpr (STRIPE) {
#pragma unroll
      for (int k = 0; k < SLOTS; ++k) {
        const int tok = min(max(sv.v[k], 0), a.N - 1);
        const uint16_t* src = gbase + (int64_t)tok * tstride + s_off[k];
        if (wbase + k < nwin)
          __builtin_amdgcn_global_load_lds(src, LDS_PTR(void, stb + region + (wbase + k) * 1024), 16, 0, 0);
        else
          __builtin_amdgcn_global_load_lds(src, LDS_PTR(void, spare), 16, 0, 0);
      }
      return;
    }
    const int jb = sv.v[0];
    const int t0 = jb * 64;
    if (t0 + 63 < a.N) {
      const uint16_t* tb = gbase + (int64_t)t0 * tstride;
#pragma unroll
      for (int k = 0; k < SLOTS; ++k) {
        if (wbase + k < nwin)
          __builtin_amdgcn_global_load_lds(tb + s_off[k], LDS_PTR(void, stb + region + (wbase + k) * 1024), 16, 0, 0);
        else
          __builtin_amdgcn_global_load_lds(tb + s_off[k], LDS_PTR(void, spare), 16, 0, 0);
      }
    } else {
      // ragged last block: rows past the end read the last row
#pragma unroll
      for (int k = 0; k < SLOTS; ++k) {
        const int o = min(wbase + k, nwin - 1) * 1024 + lane * 16;
        const int r = o / pitch_b;
        const int tok = min(t0 + r, a.N - 1);
        const uint16_t* src = gbase + (int64_t)tok * tstride + (s_off[k] - r * (int)tstride);
        if (wbase + k < nwin)
          __builtin_amdgcn_global_load_lds(src, LDS_PTR(void, stb + region + (wbase + k) * 1024), 16, 0, 0);
        else
          __builtin_amdgcn_global_load_lds(src, LDS_PTR(void, spare), 16, 0, 0);
      }
    }
  };

  // per-lane LDS read offsets within a stage
  const int k_rd = l32 * KPITCH + half * 16;
  const int grp = lane >> 4, jj = lane & 15;
  const int v_rd = KREG + (4 * (grp >> 1) + (jj >> 2)) * VPITCH + (16 * (grp & 1) + 4 * (jj & 3)) * 2;

  f32x16 oacc[DM];
#pragma unroll
  for (int dm = 0; dm < DM; ++dm) oacc[dm] = (f32x16){};
  float m_run = -1e30f, l_run = 0.f;
  const float sl2 = a.scale_log2;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones2 = {(__bf16)1.0f, (__bf16)1.0f};
  if (RESUME) {
    // Start from the anchor state: with its log-sum-exp as the reference point the state is
    // (m = LSE_A in the log2 domain, l = 1, O^T = O_A); l lives in the half-0 lane of the row.
    const int rowc = min(row, a.N - 1);
    const uint16_t* sp = a.st_o + (((int64_t)b * a.N + rowc) * a.Hq + h) * D + half * 4;
#pragma unroll
    for (int dm = 0; dm < DM; ++dm)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const u32x2 w2 = *(const u32x2*)(sp + dm * 32 + 8 * q4);
        oacc[dm][4 * q4 + 0] = __uint_as_float(w2[0] << 16);
        oacc[dm][4 * q4 + 1] = __uint_as_float(w2[0] & 0xFFFF0000u);
        oacc[dm][4 * q4 + 2] = __uint_as_float(w2[1] << 16);
        oacc[dm][4 * q4 + 3] = __uint_as_float(w2[1] & 0xFFFF0000u);
      }
    m_run = a.st_lse[((int64_t)b * a.Hq + h) * a.N + rowc] * 1.4426950408889634f;
    l_run = half == 0 ? 1.f : 0.f;
  }

  // ---- the phases of a tile ----
  // S^T = K Q^T from the stage at sb
  auto qk = [&](const unsigned char* sb, f32x16* sacc) {
    sacc[0] = (f32x16){};
    sacc[1] = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x8 kf = *(const bf16x8*)(sb + k_rd + mt * 32 * KPITCH + ks * 32);
        sacc[mt] = mfma_bf16(kf, qf[ks], sacc[mt]);
      }
  };
  // entries of tile t past the diagonal or the end of the sequence (resuming: also those in
  // the row's anchor region, which the state already holds; the window includes the diagonal)
  auto mask = [&](int t, f32x16* sacc) {
    if constexpr (STRIPE) {
      // the tile's 64 column ids, lane i holding entry 64 t + i (past the list's end: none)
      const int e = t * 64 + lane;
      const int mine = e < n ? list_g[e] : 0x7FFFFFFF;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int tok = __shfl(mine, mt * 32 + half * 4 + 8 * (r >> 2) + (r & 3));
          if (tok > row || tok >= a.N) sacc[mt][r] = NEG_INF;
        }
      return;
    }
    const int Jb = list[t];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tok = Jb * 64 + mt * 32 + half * 4 + 8 * (r >> 2) + (r & 3);
        const bool drop = RESUME ? (tok < a.sink || tok >= row - a.local + 1 || tok >= a.N)
                                 : (tok > row || tok >= a.N);
        if (drop) sacc[mt][r] = NEG_INF;
      }
  };
  // P^T of key half mt = exp2(S^T scale - m) in bf16 (pf[2 mt], pf[2 mt + 1]); returns this
  // lane's sum of the rounded values
  auto expo = [&](const f32x16* sacc, int mt, bf16x8* pf) -> float {
    const float mneg = -m_run;
    float ls = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      f32x8 tt;
#pragma unroll
      for (int e = 0; e < 8; ++e) tt[e] = __builtin_amdgcn_exp2f(fmaf(sacc[mt][8 * s2 + e], sl2, mneg));
      const bf16x8 pb = __builtin_convertvector(tt, bf16x8);
      pf[mt * 2 + s2] = pb;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const bf16x2 pr = {pb[e], pb[e + 1]};
        ls = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2, ls, false);
      }
    }
    return ls;
  };
  // The running max m stays fixed while every P value of a key half is at most 2^16 (checked
  // on the lane's partial row sum, which bounds each value).  A half that breaks the bound
  // (scores more than 16 above m in the log2 domain, or the first tile, while m is still
  // -1e30) moves m to the half's row max, rescales O and l -- which may already hold the other
  // half's P V at the old m -- and recomputes its P.  No per-tile row max is taken.
  auto settle = [&](const f32x16* sacc, int mt, bf16x8* pf, float ts) {
    if (__any(!(ts <= 65536.0f))) {
      float v = NEG_INF;
#pragma unroll
      for (int r = 0; r < 16; ++r) v = fmaxf(v, sacc[mt][r]);
      const float mnew = fmaxf(m_run, half_pair_max(v) * sl2);
      const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
      m_run = mnew;
      l_run *= alpha;
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) oacc[dm] *= alpha;
      ts = expo(sacc, mt, pf);
    }
    l_run += ts;
  };
  // O^T += V^T P^T over the 16-key groups of key half mt, with transposing V reads from the
  // stage at sb
  auto pv = [&](const unsigned char* sb, int mt, const bf16x8* pf) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) {
        const int s4 = 2 * mt + s2;
        const unsigned char* vp = sb + v_rd + 16 * s4 * VPITCH + dm * 64;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4i16, vp));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4i16, vp + 8 * VPITCH));
        const v4i16 both[2] = {lo, hi};
        bf16x8 vf;
        __builtin_memcpy(&vf, both, 16);
        oacc[dm] = mfma_bf16(vf, pf[s4], oacc[dm]);
      }
  };

  // Software pipeline over the list.  On entry to step t, S(t) is in `cur` (masked) and tiles
  // t+1 and t+2 are in LDS.  Step t computes P(t)'s first key half while the MFMAs of S(t+1)
  // run, P(t)'s second half while P V of the first half runs, and P V of the second half,
  // then issues the DMA of tile t+3 into the stage of tile t-1 and waits for tile t+2, so at
  // every barrier only the newest tile is in flight.
  if (ntile > 0) {
    issue(st0, fetch(0));
    issue(st1, fetch(1));
    issue(st2, fetch(2));
    DMA_BARRIER(SLOTS);
    f32x16 sa[2], sbb[2];
    qk(st0, sa);
    if (n_main == 0 || (RESUME && list[0] * 64 < a.sink)) mask(0, sa);
    auto step = [&](unsigned char* sc, unsigned char* sn, unsigned char* sd, int t,
                    f32x16* cur, f32x16* nxt, bool may_mask) {
      const Src jd = fetch(t + 3);
      bf16x8 pf[4];
      const float t0s = expo(cur, 0, pf);
      qk(sn, nxt);
      settle(cur, 0, pf, t0s);
      const float t1s = expo(cur, 1, pf);
      pv(sc, 0, pf);
      settle(cur, 1, pf, t1s);
      pv(sc, 1, pf);
      if (may_mask && t + 1 >= n_main) mask(t + 1, nxt);
      issue(sd, jd);
      DMA_BARRIER(SLOTS);
    };
    auto last = [&](unsigned char* sc, f32x16* cur) {
      bf16x8 pf[4];
      const float t0s = expo(cur, 0, pf);
      settle(cur, 0, pf, t0s);
      const float t1s = expo(cur, 1, pf);
      pv(sc, 0, pf);
      settle(cur, 1, pf, t1s);
      pv(sc, 1, pf);
    };
    int t = 0;
    for (; t + 4 < n_main; t += 4) {          // the next tile of every step needs no mask
      step(st0, st1, st3, t, sa, sbb, false);
      step(st1, st2, st0, t + 1, sbb, sa, false);
      step(st2, st3, st1, t + 2, sa, sbb, false);
      step(st3, st0, st2, t + 3, sbb, sa, false);
    }
    for (; t + 4 < ntile; t += 4) {
      step(st0, st1, st3, t, sa, sbb, true);
      step(st1, st2, st0, t + 1, sbb, sa, true);
      step(st2, st3, st1, t + 2, sa, sbb, true);
      step(st3, st0, st2, t + 3, sbb, sa, true);
    }
    // steps t .. n-2 (at most three) and the last tile n-1 <= t+3
    if (t + 1 >= ntile) {
      last(st0, sa);
    } else {
      step(st0, st1, st3, t, sa, sbb, true);
      if (t + 2 >= ntile) {
        last(st1, sbb);
      } else {
        step(st1, st2, st0, t + 1, sbb, sa, true);
        if (t + 3 >= ntile) {
          last(st2, sa);
        } else {
          step(st2, st3, st1, t + 2, sa, sbb, true);
          last(st3, sbb);
        }
      }
    }
    // no DMA may still be writing this workgroup's LDS when it exits
    __builtin_amdgcn_s_waitcnt(VMCNT_IMM(0));
  }

  const float lt = half_pair_sum(l_run);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (row < a.N) {
    uint16_t* op = a.o + b * a.os0 + (int64_t)row * a.os1 + h * a.os2 + half * 4;
#pragma unroll
    for (int dm = 0; dm < DM; ++dm)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const unsigned int lo = float_to_bf16_bits(oacc[dm][4 * q4 + 0] * inv) |
                                ((unsigned int)float_to_bf16_bits(oacc[dm][4 * q4 + 1] * inv) << 16);
        const unsigned int hi = float_to_bf16_bits(oacc[dm][4 * q4 + 2] * inv) |
                                ((unsigned int)float_to_bf16_bits(oacc[dm][4 * q4 + 3] * inv) << 16);
        *(u32x2*)(op + dm * 32 + 8 * q4) = (u32x2){lo, hi};
      }
    if (a.lse && half == 0)
      a.lse[((int64_t)b * a.Hq + h) * a.N + row] =
          lt > 0.f ? (m_run + __log2f(lt)) * 0.69314718055994531f : NEG_INF;
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------------------------
template <int D, int HPW>
static hipError_t launch_block(const AttnArgs& a0, hipStream_t s) {
  AttnArgs a = a0;
  a.n_hp = a.G / HPW;
  a.total = a.B * a.Hkv * a.n_hp * a.nQB * a.tpb;
  if (a.total == 0) return hipSuccess;
  if (a.st_o)
    hipLaunchKernelGGL((attn_block<D, HPW, true, false>), dim3(a.total), dim3(128 * HPW), 0, s, a);
  else if (a.stripe)
    hipLaunchKernelGGL((attn_block<D, HPW, false, true>), dim3(a.total), dim3(128 * HPW), 0, s, a);
  else
    hipLaunchKernelGGL((attn_block<D, HPW, false, false>), dim3(a.total), dim3(128 * HPW), 0, s, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const AttnArgs& a, hipStream_t s) {
  if (a.G >= 4) return launch_block<D, 4>(a, s);
  if (a.G == 2) return launch_block<D, 2>(a, s);
  return launch_block<D, 1>(a, s);
}

// Block and column lists both run attn_block; a.stripe (set from the granularity) selects the
// instance that gathers listed rows.
hipError_t launch_prefill(const AttnArgs& a, int D, int granularity, hipStream_t s) {
  (void)granularity;
  return D == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s);
}
