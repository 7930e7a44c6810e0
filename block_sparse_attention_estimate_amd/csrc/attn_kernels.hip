// Block- and stripe-sparse attention (the computation pass) on gfx950.
//
// SALE (arXiv 2505.24179), "What carries the argument": attention is computed only on the
// blocks the estimate keeps.  AnchorAttention (arXiv 2505.23520), "Core claim": stripe
// granularity loads only the selected key/value rows (discrete K/V loading).  The online
// softmax keeps a running row max and sum (the M and Acc buffers of AnchorAttention's
// kernel, referee major comment 1).
//
// Design (one workgroup = HPW query heads of one KV head x 64 query rows):
//  * the K tile (64 keys) and V tile are staged once in LDS and shared by the HPW packed
//    query heads (GQA packing); double-buffered, global loads for tile t+1 overlap tile t;
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

template <int D, int NT, int HPW, bool STRIPE>
__global__ __launch_bounds__(64 * HPW * 2 / NT) void attn_sparse(AttnArgs a) {
  constexpr int NWV = HPW * 2 / NT;        // waves per workgroup
  constexpr int T = 64 * NWV;              // threads
  constexpr int KS = D / 16;               // k-steps of S^T
  constexpr int DM = D / 32;               // d tiles of O^T
  constexpr int CPR = D / 8;               // 16-byte chunks per key row
  constexpr int KCH = 64 * CPR;            // K chunks per tile
  constexpr int VU = 16 * CPR;             // V units (4 keys x 8 dims) per tile
  constexpr int PK = (KCH + T - 1) / T;
  constexpr int PV = (VU + T - 1) / T;
  constexpr int KP = D + 8;                // K row pitch in LDS (elements)
  constexpr int VP = 64 + 8;               // V^T row pitch in LDS (elements)
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][64 * KP];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][D * VP];
  __shared__ int kid_lds[STRIPE ? 2 : 1][64];

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
  rest = i_rev;
  const int iq = a.nQB - 1 - rest;
  const int r0 = iq * a.bq + tsub * 64;
  if (iq < 0 || r0 >= a.N) return;
  const int r_last = min(r0 + 63, a.N - 1);
  const int hw = wave / (2 / NT);
  const int rs = wave % (2 / NT);
  const int h = g * a.G + hp * HPW + hw;
  const int rw = r0 + rs * 32 * NT;        // first query row of this wave

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

  // ---- Q fragments (B operand of S^T = K Q^T) ----
  bf16x8 qf[NT][KS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int rowc = min(rw + nt * 32 + l32, a.N - 1);
    const uint16_t* qp = a.q + b * a.qs0 + (int64_t)rowc * a.qs1 + h * a.qs2 + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[nt][ks] = *(const bf16x8*)(qp + ks * 16);
  }

  const uint16_t* kg = a.k + b * a.ks0 + g * a.ks2;
  const uint16_t* vg = a.v + b * a.vs0 + g * a.vs2;
  u32x4 kreg[PK];
  u32x4 vreg[PV][4];
  int kidv = 0;
  // per-thread staging coordinates (fixed for the whole loop)
  int k_row[PK], k_dc[PK], v_row[PV], v_dc[PV];
#pragma unroll
  for (int c = 0; c < PK; ++c) {
    const int ch = c * T + tid;
    k_row[c] = ch / CPR;
    k_dc[c] = (ch % CPR) * 8;
  }
#pragma unroll
  for (int u = 0; u < PV; ++u) {
    const int un = u * T + tid;
    v_row[u] = (un / CPR) * 4;
    v_dc[u] = (un % CPR) * 8;
  }

  auto load_tile = [&](int it) {
    if (!STRIPE) {
      const int t0 = list[it] * 64;
      if (t0 >= 0 && t0 + 63 < a.N) {
        const uint16_t* kt = kg + (int64_t)t0 * a.ks1;
        const uint16_t* vt = vg + (int64_t)t0 * a.vs1;
#pragma unroll
        for (int c = 0; c < PK; ++c)
          if (c * T + tid < KCH) kreg[c] = *(const u32x4*)(kt + (int64_t)k_row[c] * a.ks1 + k_dc[c]);
#pragma unroll
        for (int u = 0; u < PV; ++u)
          if (u * T + tid < VU) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              vreg[u][j] = *(const u32x4*)(vt + (int64_t)(v_row[u] + j) * a.vs1 + v_dc[u]);
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
#pragma unroll
    for (int c = 0; c < PK; ++c)
      if (c * T + tid < KCH)
        kreg[c] = *(const u32x4*)(kg + (int64_t)tok_of(k_row[c]) * a.ks1 + k_dc[c]);
#pragma unroll
    for (int u = 0; u < PV; ++u)
      if (u * T + tid < VU) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          vreg[u][j] = *(const u32x4*)(vg + (int64_t)tok_of(v_row[u] + j) * a.vs1 + v_dc[u]);
      }
    if (STRIPE && tid < 64) {
      const int e = it * 64 + tid;
      kidv = e < n ? list[e] : 0x7FFFFFFF;
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int c = 0; c < PK; ++c)
      if (c * T + tid < KCH) *(u32x4*)&k_lds[buf][k_row[c] * KP + k_dc[c]] = kreg[c];
#pragma unroll
    for (int u = 0; u < PV; ++u) {
      if (u * T + tid < VU) {
        const int kq = v_row[u], dc = v_dc[u];
        // 4-key chunk c of a 16-key group moves to chunk {0, 2, 1, 3}[c]
        const int cq = (kq & 15) >> 2;
        const int pos = (kq & ~15) + (((cq & 1) << 1) | (cq >> 1)) * 4;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          // dims dc + 2*e2 (low halves) and dc + 2*e2 + 1 (high halves) of the 4 keys
          const unsigned int w0 = vreg[u][0][e2], w1 = vreg[u][1][e2];
          const unsigned int w2 = vreg[u][2][e2], w3 = vreg[u][3][e2];
          const unsigned int lo01 = __builtin_amdgcn_perm(w1, w0, 0x05040100u);
          const unsigned int lo23 = __builtin_amdgcn_perm(w3, w2, 0x05040100u);
          const unsigned int hi01 = __builtin_amdgcn_perm(w1, w0, 0x07060302u);
          const unsigned int hi23 = __builtin_amdgcn_perm(w3, w2, 0x07060302u);
          *(u32x2*)&v_lds[buf][(dc + 2 * e2) * VP + pos] = (u32x2){lo01, lo23};
          *(u32x2*)&v_lds[buf][(dc + 2 * e2 + 1) * VP + pos] = (u32x2){hi01, hi23};
        }
      }
    }
    if (STRIPE && tid < 64) kid_lds[STRIPE ? buf : 0][tid] = kidv;
  };

  f32x16 oacc[DM][NT];
#pragma unroll
  for (int dm = 0; dm < DM; ++dm)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) oacc[dm][nt] = (f32x16){};
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = -1e30f;
    l_run[nt] = 0.f;
  }
  const float sl2 = a.scale_log2;
  // bf16 pair (1.0, 1.0) for row sums with v_dot2
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones2 = {(__bf16)1.0f, (__bf16)1.0f};

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int it = 0; it < n_tiles; ++it) {
    const int buf = it & 1;
    if (it + 1 < n_tiles) load_tile(it + 1);

    // S^T = K Q^T
    f32x16 sacc[2][NT];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sacc[mt][nt] = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x8 kf = *(const bf16x8*)&k_lds[buf][(mt * 32 + l32) * KP + ks * 16 + half * 8];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sacc[mt][nt] = mfma_bf16(kf, qf[nt][ks], sacc[mt][nt]);
      }
    }

    // causal / ragged / padding mask, only on tiles that need it
    bool need;
    int Jb = 0;
    if (!STRIPE) {
      Jb = list[it];
      need = (Jb * 64 + 63 > rw) || (Jb * 64 + 63 >= a.N);
    } else {
      const int last = list[min(it * 64 + 63, n - 1)];
      need = (last > rw) || (it * 64 + 64 > n);
    }
    if (need) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int row = rw + nt * 32 + l32;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = mt * 32 + half * 4 + 8 * (r >> 2) + (r & 3);
            const int tok = STRIPE ? kid_lds[STRIPE ? buf : 0][kk] : Jb * 64 + kk;
            if (tok > row || tok >= a.N) sacc[mt][nt][r] = NEG_INF;
          }
        }
    }

    // online softmax in the log2 domain.  The running max moves only when a row's new max
    // exceeds it by more than 8 (a factor 256), so O is rescaled rarely; otherwise the
    // probabilities are taken against the stale max (<= 2^8, exact in the final ratio).
    float mx[NT];
    bool grow = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float v = NEG_INF;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) v = fmaxf(v, sacc[mt][nt][r]);
      v = fmaxf(v, swap_halves(v)) * sl2;
      mx[nt] = v;
      grow |= v > m_run[nt] + 8.0f;
    }
    if (__any(grow)) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float mnew = fmaxf(m_run[nt], mx[nt]);
        const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - mnew);
        m_run[nt] = mnew;
        l_run[nt] *= alpha;
#pragma unroll
        for (int dm = 0; dm < DM; ++dm) oacc[dm][nt] *= alpha;
      }
    }
    bf16x8 pf[NT][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float mneg = -m_run[nt];
      float ls = l_run[nt];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          f32x8 t;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            t[e] = __builtin_amdgcn_exp2f(fmaf(sacc[mt][nt][8 * s2 + e], sl2, mneg));
          const bf16x8 pb = __builtin_convertvector(t, bf16x8);
          pf[nt][mt * 2 + s2] = pb;
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const bf16x2 pr = {pb[e], pb[e + 1]};
            ls = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2, ls, false);
          }
        }
      l_run[nt] = ls;
    }

    // O^T += V^T P^T
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
      for (int dm = 0; dm < DM; ++dm) {
        const bf16x8 vf = *(const bf16x8*)&v_lds[buf][(dm * 32 + l32) * VP + s4 * 16 + half * 8];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) oacc[dm][nt] = mfma_bf16(vf, pf[nt][s4], oacc[dm][nt]);
      }
    }

    if (it + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, LSE = (m + log2 l) ln 2 ----
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float lt = l_run[nt] + swap_halves(l_run[nt]);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const int row = rw + nt * 32 + l32;
    if (row < a.N) {
      uint16_t* op = a.o + b * a.os0 + (int64_t)row * a.os1 + h * a.os2 + half * 4;
#pragma unroll
      for (int dm = 0; dm < DM; ++dm)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const unsigned int lo = float_to_bf16_bits(oacc[dm][nt][4 * q4 + 0] * inv) |
                                  ((unsigned int)float_to_bf16_bits(oacc[dm][nt][4 * q4 + 1] * inv) << 16);
          const unsigned int hi = float_to_bf16_bits(oacc[dm][nt][4 * q4 + 2] * inv) |
                                  ((unsigned int)float_to_bf16_bits(oacc[dm][nt][4 * q4 + 3] * inv) << 16);
          *(u32x2*)(op + dm * 32 + 8 * q4) = (u32x2){lo, hi};
        }
      if (a.lse && half == 0)
        a.lse[((int64_t)b * a.Hq + h) * a.N + row] =
            lt > 0.f ? (m_run[nt] + __log2f(lt)) * 0.69314718055994531f : NEG_INF;
    }
  }
}

// ---------------------------------------------------------------------------------------
template <int D, int NT, int HPW, bool STRIPE>
static hipError_t launch_one(const AttnArgs& a0, hipStream_t s) {
  AttnArgs a = a0;
  a.n_hp = a.G / HPW;
  a.total = a.B * a.Hkv * a.n_hp * a.nQB * a.tpb;
  if (a.total == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_sparse<D, NT, HPW, STRIPE>), dim3(a.total), dim3(64 * HPW * 2 / NT), 0, s, a);
  return hipGetLastError();
}

template <int D, bool STRIPE>
static hipError_t launch_d(const AttnArgs& a, hipStream_t s) {
  static const int nt_pref = [] {
    const char* e = getenv("SA_ATTN_NT");
    return (e && atoi(e) == 2) ? 2 : 1;
  }();
  if (a.G >= 4) {
    if (nt_pref == 1) return launch_one<D, 1, 4, STRIPE>(a, s);
    return launch_one<D, 2, 4, STRIPE>(a, s);
  }
  if (a.G == 2) return launch_one<D, 1, 2, STRIPE>(a, s);
  return launch_one<D, 1, 1, STRIPE>(a, s);
}

hipError_t launch_prefill(const AttnArgs& a, int D, int granularity, hipStream_t s) {
  const bool stripe = granularity == SA_STRIPE;
  if (D == 64) return stripe ? launch_d<64, true>(a, s) : launch_d<64, false>(a, s);
  return stripe ? launch_d<128, true>(a, s) : launch_d<128, false>(a, s);
}
