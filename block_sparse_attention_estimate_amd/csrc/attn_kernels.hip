// Block- and stripe-sparse attention (the computation pass) on gfx950.
//
// SALE (arXiv 2505.24179), "What carries the argument": attention is computed only on the
// blocks the estimate keeps.  AnchorAttention (arXiv 2505.23520), "Core claim": stripe
// granularity loads only the selected key/value rows (discrete K/V loading).  The online
// softmax keeps a running row max and sum (the M and Acc buffers of AnchorAttention's
// kernel, referee major comment 1).
//
// Design (one workgroup = HPW query heads of one KV head x 64 query rows, 2 waves per head):
//  * the K tile (64 keys) and V tile are staged once in LDS and shared by the HPW packed
//    query heads (GQA packing); three LDS buffers: tile t is consumed (P V), tile t+1's
//    S = K Q^T is computed while tile t's softmax runs (software pipeline, so the MFMA unit
//    has independent work during the exponentials), tile t+2 is written from registers
//    and tile t+3 is in flight from HBM;
//  * S^T = K Q^T on 32x32x16 bf16 MFMA: each lane owns one query row and 16 keys of each
//    32-key tile, so the row max / sum are in-lane plus one exchange with lane ^ 32;
//  * O^T += V^T P^T: P^T is the S^T accumulator converted to bf16 in place (no LDS round
//    trip); V is written to LDS transposed, with the key order permuted so each lane reads
//    its 8 keys of a k-step as one 16-byte load;
//  * stripe lists gather 64 listed key rows per tile (discrete loading), same inner loop;
//  * work items are ordered longest-first (last query blocks first) and the two 64-row
//    halves of a 128-row query block (same list, same K/V) land on the same XCD.
#include <stdlib.h>

#include "sa_common.h"
#include "sa_internal.h"

#define NEG_INF (-__builtin_huge_valf())

template <int D, int HPW, bool STRIPE>
__global__ __launch_bounds__(128 * HPW) void attn_sparse(AttnArgs a) {
  constexpr int NWV = 2 * HPW;             // waves per workgroup: 2 slices of 32 rows per head
  constexpr int T = 64 * NWV;              // threads
  constexpr int KS = D / 16;               // k-steps of S^T
  constexpr int DM = D / 32;               // d tiles of O^T
  constexpr int CPR = D / 8;               // 16-byte chunks per key row
  constexpr int KCH = 64 * CPR;            // K chunks per tile
  constexpr int VU = 16 * CPR;             // V units (4 keys x 8 dims) per tile
  constexpr int KP = D + 8;                // K row pitch in LDS (elements)
  constexpr int VP = 64 + 8;               // V^T row pitch in LDS (elements)
  constexpr int NB = 3;                    // LDS buffers
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[NB][64 * KP];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[NB][D * VP];
  __shared__ int kid_lds[STRIPE ? NB : 1][64];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, l32 = lane & 31;

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
  // rest = i_rev * (B * Hkv) + r2; rotating (b, g) with i_rev spreads every KV head (and so
  // every threshold) over all XCDs instead of pinning one head to one XCD
  const int BG = a.B * a.Hkv;
  const int i_rev = rest / BG;
  const int gb = (rest % BG + i_rev) % BG;
  const int g = gb % a.Hkv;
  const int b = gb / a.Hkv;
  const int iq = a.nQB - 1 - i_rev;
  const int r0 = iq * a.bq + tsub * 64;
  if (iq < 0 || r0 >= a.N) return;
  const int r_last = min(r0 + 63, a.N - 1);
  const int h = g * a.G + hp * HPW + (wave >> 1);
  const int rw = r0 + (wave & 1) * 32;     // first query row of this wave
  const int row = rw + l32;                // this lane's query row

  // ---- list of this (b, g, query block), trimmed to entries this tile can see ----
  const int64_t lrow = (int64_t)(b * a.Hkv + g) * a.nQB + iq;
  const int32_t* list = a.idx + lrow * a.stride;
  int n = min(a.counts[lrow], a.stride);
  if (!STRIPE) {
    while (n > 0 && list[n - 1] * 64 > r_last) --n;
  } else {
    int lo = 0, hi = n;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (list[mid] <= r_last) lo = mid + 1; else hi = mid;
    }
    n = lo;
  }
  const int n_tiles = STRIPE ? (n + 63) / 64 : n;
  // Tiles that need the causal / ragged / padding mask form a suffix of the (ascending)
  // list; every workgroup row sees all keys of the tiles before it.
  int n_main = n_tiles;
  if (!STRIPE) {
    while (n_main > 0 && (list[n_main - 1] * 64 + 63 > r0 || list[n_main - 1] * 64 + 63 >= a.N)) --n_main;
  } else {
    while (n_main > 0 && (list[min(n_main * 64, n) - 1] > r0 || n_main * 64 > n)) --n_main;
  }
  const int n_steady = max(0, min(n_main, n_tiles - 3));

  // ---- Q fragments (B operand of S^T = K Q^T) ----
  bf16x8 qf[KS];
  {
    const int rowc = min(row, a.N - 1);
    const uint16_t* qp = a.q + b * a.qs0 + (int64_t)rowc * a.qs1 + h * a.qs2 + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const bf16x8*)(qp + ks * 16);
  }

  const uint16_t* kg = a.k + b * a.ks0 + g * a.ks2;
  const uint16_t* vg = a.v + b * a.vs0 + g * a.vs2;
  // Staging roles.  With SPLIT (more threads than V units), threads tid < VU each stage one
  // V unit (4 keys x 8 dims) and the others stage K chunks; both use the same 4 registers.
  // V unit layout: 16 lanes share one dim chunk and cover the 16 key quads of the tile in
  // LDS position order, so a 16-lane group's transposed LDS writes fill one contiguous
  // 128-byte row segment (no bank conflicts); quad position p holds key quad {0,2,1,3}[p%4].
  constexpr bool SPLIT = T > VU;
  constexpr int KT = SPLIT ? T - VU : T;                  // threads staging K
  constexpr int PKS = (KCH + KT - 1) / KT;                // K chunks per K thread
  constexpr int PVS = SPLIT ? 1 : (VU + T - 1) / T;      // V units per V thread
  constexpr int NST = SPLIT ? (PKS > 4 ? PKS : 4) : PKS + 4 * PVS;
  const bool is_v = SPLIT ? tid < VU : true;
  const bool is_k = SPLIT ? tid >= VU : true;
  const int ktid = SPLIT ? tid - VU : tid;
  u32x4 stg[NST];
  int kidv = 0;
  int v_row[PVS], v_pos[PVS], v_dc[PVS];
#pragma unroll
  for (int u = 0; u < PVS; ++u) {
    const int un = u * T + tid;
    const int pq = un & 15;
    const int q = (pq & ~3) | ((pq & 1) << 1) | ((pq >> 1) & 1);
    v_row[u] = q * 4;
    v_pos[u] = pq * 4;
    v_dc[u] = (un >> 4) * 8;
  }
  // element offsets within a contiguous 64-key tile (fast path)
  int k_off[PKS], v_off[PVS][4];
#pragma unroll
  for (int c = 0; c < PKS; ++c) {
    const int ch = c * KT + ktid;
    k_off[c] = (ch / CPR) * (int)a.ks1 + (ch % CPR) * 8;
  }
#pragma unroll
  for (int u = 0; u < PVS; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) v_off[u][j] = (v_row[u] + j) * (int)a.vs1 + v_dc[u];
  auto kslot = [&](int c) -> u32x4& { return stg[c]; };
  auto vslot = [&](int u, int j) -> u32x4& { return stg[SPLIT ? j : PKS + 4 * u + j]; };

  auto load_tile = [&](int it) {
    if (!STRIPE) {
      const int t0 = list[it] * 64;
      if (t0 >= 0 && t0 + 63 < a.N) {
        const uint16_t* kt = kg + (int64_t)t0 * a.ks1;
        const uint16_t* vt = vg + (int64_t)t0 * a.vs1;
        if (is_k) {
#pragma unroll
          for (int c = 0; c < PKS; ++c)
            if (c * KT + ktid < KCH) kslot(c) = *(const u32x4*)(kt + k_off[c]);
        }
        if (is_v) {
#pragma unroll
          for (int u = 0; u < PVS; ++u)
            if (u * T + tid < VU) {
#pragma unroll
              for (int j = 0; j < 4; ++j) vslot(u, j) = *(const u32x4*)(vt + v_off[u][j]);
            }
        }
        return;
      }
    }
    // ragged last block or gathered (stripe) rows: per-row token ids, clamped in range
    auto tok_of = [&](int kk) -> int {
      if (STRIPE) {
        const int e = it * 64 + kk;
        return e < n ? min(max(list[e], 0), a.N - 1) : 0;
      }
      return min(max(list[it] * 64 + kk, 0), a.N - 1);
    };
    if (is_k) {
#pragma unroll
      for (int c = 0; c < PKS; ++c) {
        const int ch = c * KT + ktid;
        if (ch < KCH) kslot(c) = *(const u32x4*)(kg + (int64_t)tok_of(ch / CPR) * a.ks1 + (ch % CPR) * 8);
      }
    }
    if (is_v) {
#pragma unroll
      for (int u = 0; u < PVS; ++u)
        if (u * T + tid < VU) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            vslot(u, j) = *(const u32x4*)(vg + (int64_t)tok_of(v_row[u] + j) * a.vs1 + v_dc[u]);
        }
    }
    if (STRIPE && tid < 64) {
      const int e = it * 64 + tid;
      kidv = e < n ? list[e] : 0x7FFFFFFF;
    }
  };

  auto store_tile = [&](int buf) {
    if (is_k) {
#pragma unroll
      for (int c = 0; c < PKS; ++c) {
        const int ch = c * KT + ktid;
        if (ch < KCH) *(u32x4*)&k_lds[buf][(ch / CPR) * KP + (ch % CPR) * 8] = kslot(c);
      }
    }
    if (is_v) {
#pragma unroll
      for (int u = 0; u < PVS; ++u) {
        if (u * T + tid < VU) {
          const int pos = v_pos[u], dc = v_dc[u];
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            // dims dc + 2*e2 (low halves) and dc + 2*e2 + 1 (high halves) of the 4 keys
            const unsigned int w0 = vslot(u, 0)[e2], w1 = vslot(u, 1)[e2];
            const unsigned int w2 = vslot(u, 2)[e2], w3 = vslot(u, 3)[e2];
            const unsigned int lo01 = __builtin_amdgcn_perm(w1, w0, 0x05040100u);
            const unsigned int lo23 = __builtin_amdgcn_perm(w3, w2, 0x05040100u);
            const unsigned int hi01 = __builtin_amdgcn_perm(w1, w0, 0x07060302u);
            const unsigned int hi23 = __builtin_amdgcn_perm(w3, w2, 0x07060302u);
            *(u32x2*)&v_lds[buf][(dc + 2 * e2) * VP + pos] = (u32x2){lo01, lo23};
            *(u32x2*)&v_lds[buf][(dc + 2 * e2 + 1) * VP + pos] = (u32x2){hi01, hi23};
          }
        }
      }
    }
    if (STRIPE && tid < 64) kid_lds[STRIPE ? buf : 0][tid] = kidv;
  };

  // S^T tile for the K buffer `buf`: 2 x 32 keys against this lane's query row
  auto qk = [&](int buf, f32x16* sacc) {
    sacc[0] = (f32x16){};
    sacc[1] = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x8 kf = *(const bf16x8*)&k_lds[buf][(mt * 32 + l32) * KP + ks * 16 + half * 8];
        sacc[mt] = mfma_bf16(kf, qf[ks], sacc[mt]);
      }
    }
  };

  f32x16 oacc[DM];
#pragma unroll
  for (int dm = 0; dm < DM; ++dm) oacc[dm] = (f32x16){};
  float m_run = -1e30f, l_run = 0.f;
  const float sl2 = a.scale_log2;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones2 = {(__bf16)1.0f, (__bf16)1.0f};

  // ---- prologue: tiles 0 and 1 in LDS, tile 2 in registers, S of tile 0 ----
  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  if (n_tiles > 1) {
    load_tile(1);
    store_tile(1);
  }
  __syncthreads();
  if (n_tiles > 2) load_tile(2);
  f32x16 scur[2], snext[2];
  qk(0, scur);

  // online softmax (log2 domain) of the current S tile, then O^T += V^T P^T.  The running
  // max moves only when a row's new max exceeds it by more than 8 (a factor 256), so O is
  // rescaled rarely; otherwise probabilities use the stale max (<= 2^8, exact in the ratio).
  auto softmax_max = [&](const f32x16* sc) {
    float v = NEG_INF;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) v = fmaxf(v, sc[mt][r]);
    v = half_pair_max(v) * sl2;
    if (__any(v > m_run + 8.0f)) {
      const float mnew = fmaxf(m_run, v);
      const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
      m_run = mnew;
      l_run *= alpha;
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) oacc[dm] *= alpha;
    }
  };
  auto softmax_p = [&](const f32x16* sc, bf16x8* pf) {
    const float mneg = -m_run;
    float ls = l_run;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        f32x8 t;
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = __builtin_amdgcn_exp2f(fmaf(sc[mt][8 * s2 + e], sl2, mneg));
        const bf16x8 pb = __builtin_convertvector(t, bf16x8);
        pf[mt * 2 + s2] = pb;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 pr = {pb[e], pb[e + 1]};
          ls = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2, ls, false);
        }
      }
    l_run = ls;
  };
  auto pv = [&](int buf, const bf16x8* pf) {
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) {
        const bf16x8 vf = *(const bf16x8*)&v_lds[buf][(dm * 32 + l32) * VP + s4 * 16 + half * 8];
        oacc[dm] = mfma_bf16(vf, pf[s4], oacc[dm]);
      }
    }
  };

  // ---- steady state: unmasked tiles with three tiles ahead (two per trip, so the two
  // S register sets swap roles instead of being copied) ----
  int bc = 0;                               // buffer of tile it
  int it = 0;
  auto steady = [&](const f32x16* sc, f32x16* sn) {
    const int bn = bc == 2 ? 0 : bc + 1;
    const int bs = bn == 2 ? 0 : bn + 1;
    softmax_max(sc);
    bf16x8 pf[4];
    softmax_p(sc, pf);
#ifdef SA_EXP_SETPRIO
    __builtin_amdgcn_s_setprio(1);
#endif
    qk(bn, sn);
    pv(bc, pf);
#ifdef SA_EXP_SETPRIO
    __builtin_amdgcn_s_setprio(0);
#endif
    store_tile(bs);
    load_tile(it + 3);
    __syncthreads();
    bc = bn;
    ++it;
  };
  while (it + 1 < n_steady) {
    steady(scur, snext);
    steady(snext, scur);
  }
  if (it < n_steady) {
    steady(scur, snext);
    scur[0] = snext[0];
    scur[1] = snext[1];
  }
  // ---- tail: masked tiles and the last ones ----
  for (; it < n_tiles; ++it) {
    const int bn = bc == 2 ? 0 : bc + 1;
    const int bs = bn == 2 ? 0 : bn + 1;
    if (it >= n_main) {
      int Jb = 0;
      if (!STRIPE) Jb = list[it];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = mt * 32 + half * 4 + 8 * (r >> 2) + (r & 3);
          const int tok = STRIPE ? kid_lds[STRIPE ? bc : 0][kk] : Jb * 64 + kk;
          if (tok > row || tok >= a.N) scur[mt][r] = NEG_INF;
        }
    }
    softmax_max(scur);
    bf16x8 pf[4];
    softmax_p(scur, pf);
    if (it + 1 < n_tiles) qk(bn, snext);
    pv(bc, pf);
    if (it + 2 < n_tiles) store_tile(bs);
    if (it + 3 < n_tiles) load_tile(it + 3);
    __syncthreads();
    scur[0] = snext[0];
    scur[1] = snext[1];
    bc = bn;
  }

  // ---- epilogue: O = O^T / l, LSE = (m + log2 l) ln 2 ----
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
}

// ---------------------------------------------------------------------------------------
// Block lists: K/V tiles go HBM -> LDS with direct loads (global_load_lds_dwordx4), no
// staging registers.  Four LDS stages: tile t is consumed while tiles t+1..t+3 are in flight.
//  * K rows keep head_dim order with a 16-byte pad per row (pitch 272 B for d = 128), so the
//    A-operand reads of S^T = K Q^T (16 rows x 16 B per lane group) hit distinct banks.
//  * V rows are stored as they are (pitch 320 B for d = 128); the A operand of O^T += V^T P^T
//    is read with ds_read_b64_tr_b16: within a 16-lane group, lane j addresses the 4 dims
//    [d0 + 4(j%4), +4) of key row k0 + j/4, and the read returns to lane i the 4 keys
//    k0..k0+3 of dim d0 + i -- exactly the 4 keys the P^T register layout pairs with that lane.
// ---------------------------------------------------------------------------------------

template <int D, int HPW, bool RESUME>
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
  int n_main = n;
  while (n_main > 0 && (list[n_main - 1] * 64 + 63 >= mlim || list[n_main - 1] * 64 + 63 >= a.N)) --n_main;

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
#pragma unroll
  for (int k = 0; k < SLOTS; ++k) {
    const int o = min(wbase + k, nwin - 1) * 1024 + lane * 16;
    const int r = o / pitch_b, cb = o % pitch_b;
    s_off[k] = r * (int)tstride + (cb < ROWB ? cb / 16 : 0) * 8;   // pads get a harmless copy
  }
  // Issue the DMA of tile t (clamped to the list) into the stage at stb.  Every wave issues exactly
  // SLOTS loads per call, so the vmcnt waits below are compile-time constants.
  auto issue = [&](unsigned char* stb, int jb) {
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
  if (n > 0) {
    issue(st0, list[0]);
    issue(st1, list[min(1, n - 1)]);
    issue(st2, list[min(2, n - 1)]);
    DMA_BARRIER(SLOTS);
    f32x16 sa[2], sbb[2];
    qk(st0, sa);
    if (n_main == 0 || (RESUME && list[0] * 64 < a.sink)) mask(0, sa);
    auto step = [&](unsigned char* sc, unsigned char* sn, unsigned char* sd, int t,
                    f32x16* cur, f32x16* nxt, bool may_mask) {
      const int jd = list[min(t + 3, n - 1)];
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
    for (; t + 4 < n; t += 4) {
      step(st0, st1, st3, t, sa, sbb, true);
      step(st1, st2, st0, t + 1, sbb, sa, true);
      step(st2, st3, st1, t + 2, sa, sbb, true);
      step(st3, st0, st2, t + 3, sbb, sa, true);
    }
    // steps t .. n-2 (at most three) and the last tile n-1 <= t+3
    if (t + 1 >= n) {
      last(st0, sa);
    } else {
      step(st0, st1, st3, t, sa, sbb, true);
      if (t + 2 >= n) {
        last(st1, sbb);
      } else {
        step(st1, st2, st0, t + 1, sbb, sa, true);
        if (t + 3 >= n) {
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
template <int D, int HPW, bool STRIPE>
static hipError_t launch_one(const AttnArgs& a0, hipStream_t s) {
  AttnArgs a = a0;
  a.n_hp = a.G / HPW;
  a.total = a.B * a.Hkv * a.n_hp * a.nQB * a.tpb;
  if (a.total == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_sparse<D, HPW, STRIPE>), dim3(a.total), dim3(128 * HPW), 0, s, a);
  return hipGetLastError();
}

template <int D, int HPW>
static hipError_t launch_block(const AttnArgs& a0, hipStream_t s) {
  AttnArgs a = a0;
  a.n_hp = a.G / HPW;
  a.total = a.B * a.Hkv * a.n_hp * a.nQB * a.tpb;
  if (a.total == 0) return hipSuccess;
  if (a.st_o)
    hipLaunchKernelGGL((attn_block<D, HPW, true>), dim3(a.total), dim3(128 * HPW), 0, s, a);
  else
    hipLaunchKernelGGL((attn_block<D, HPW, false>), dim3(a.total), dim3(128 * HPW), 0, s, a);
  return hipGetLastError();
}

template <int D, bool STRIPE>
static hipError_t launch_d(const AttnArgs& a, hipStream_t s) {
  if (!STRIPE) {
    if (a.G >= 4) return launch_block<D, 4>(a, s);
    if (a.G == 2) return launch_block<D, 2>(a, s);
    return launch_block<D, 1>(a, s);
  }
  if (a.G >= 4) return launch_one<D, 4, STRIPE>(a, s);
  if (a.G == 2) return launch_one<D, 2, STRIPE>(a, s);
  return launch_one<D, 1, STRIPE>(a, s);
}

hipError_t launch_prefill(const AttnArgs& a, int D, int granularity, hipStream_t s) {
  const bool stripe = granularity == SA_STRIPE;
  if (D == 64) return stripe ? launch_d<64, true>(a, s) : launch_d<64, false>(a, s);
  return stripe ? launch_d<128, true>(a, s) : launch_d<128, false>(a, s);
}
