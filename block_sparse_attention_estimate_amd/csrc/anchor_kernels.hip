// Anchor pass with a reusable attention state (anchor-state reuse) on gfx950.
//
// AnchorAttention (arXiv 2505.23520): "What carries the argument" -- the kernel keeps what
// the anchor computation produced and the sparse computation starts from it; referee major
// comment 1 -- the anchor kernel holds, per query row, the running max (M) and the p.V
// accumulator (Acc) of an online softmax; referee minor comment 2 -- the sparse loop starts
// past the initial key block, which the anchor computation has covered.
//
// est_anchor_state: one workgroup per (b, g, query block).  For every query row r of the
// block and every query head of the group it computes, over the anchor region
// A(r) = {j <= r : j < sink or j >= r - local + 1} (Eq. 1's token set):
//   * the anchor x_a[r] = c * max_j q_r . k_j, with the dot products on the same 32x32x16 bf16
//     MFMA sequence as the estimator's anchor kernel, so the value is bit-identical to it;
//   * the online-softmax state, stored as the normalised partial output O_A (bf16) and its
//     log-sum-exp LSE_A (natural log), from which the sparse pass resumes.
// The region's keys and values (32-key tiles: the sink tiles, then the window tiles) go
// HBM -> LDS by direct loads in chunks of 256 rows; each wave owns one 32-row slice of one
// head per round (S^T = K Q^T puts a query row in each lane, so the row statistics are in-lane
// plus one exchange with lane ^ 32), and P^T stays in registers for O^T += V^T P^T with
// transposing V reads, as in the attention kernel.
#include "sa_common.h"
#include "sa_internal.h"

#define NEG_INF (-__builtin_huge_valf())

#define AS_WAVES 8

template <int D>
__global__ __launch_bounds__(64 * AS_WAVES) void est_anchor_state(EstArgs a) {
  // The host pass only needs this kernel's signature (for its launch stub).
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NW = AS_WAVES;
  constexpr int KS = D / 16;                        // k-steps of S^T
  constexpr int DM = D / 32;                        // d tiles of O^T
  constexpr int ROWB = D * 2;                       // bytes of one key / value row
  constexpr int KPITCH = D == 128 ? 272 : 144;      // padded K row (conflict-free A reads)
  constexpr int VPITCH = D == 128 ? 320 : 192;      // padded V row (transposing reads)
  constexpr int CH = 256;                           // region rows per staged chunk
  constexpr int TPC = CH / 32;                      // 32-key tiles per chunk
  constexpr int KREG = CH * KPITCH, VREG = CH * VPITCH;
  static_assert(KREG % 1024 == 0 && VREG % 1024 == 0, "DMA windows must tile the regions");
  __shared__ __attribute__((aligned(1024))) unsigned char kv[KREG + VREG];

  // work item (b, g, i), dealt so that each XCD runs a contiguous range of query blocks
  int item;
  {
    const int total = a.nQB * a.Hkv * a.B;
    const int x = blockIdx.x % 8, k = blockIdx.x / 8;
    int start = 0;
    for (int y = 0; y < x; ++y) start += (total - y + 7) / 8;
    item = start + k;
  }
  const int i = item % a.nQB, g = (item / a.nQB) % a.Hkv, b = item / (a.nQB * a.Hkv);
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5, l32 = lane & 31;
  const int wave = wave_uniform(tid >> 6);
  const int G = a.G;
  const int r0 = i * a.bq;
  const int r1 = min(a.N, r0 + a.bq);
  const int ntph = (a.bq + 31) / 32;

  // the region's 32-key tiles: the sink tiles, then the window tiles from the tile holding
  // max(0, r0 - local + 1) (not below the sink tiles) through r1 - 1
  const int hi_blk = r1 - 1;
  const int sink_end = min(a.sink, r1);
  const int n_sink_t = (sink_end + 31) / 32;
  const int lo_blk = max(0, r0 - a.local + 1);
  const int win_start = max((lo_blk / 32) * 32, n_sink_t * 32);
  const int n_win_t = win_start <= hi_blk ? (hi_blk - win_start) / 32 + 1 : 0;
  const int n_t = n_sink_t + n_win_t;
  const int n_chunks = (n_t + TPC - 1) / TPC;
  auto tile_start = [&](int t) { return t < n_sink_t ? t * 32 : win_start + (t - n_sink_t) * 32; };

  const uint16_t* kb = a.k + b * a.ks0 + g * a.ks2;
  const uint16_t* vb = a.v + b * a.vs0 + g * a.vs2;
  const int k_rd = l32 * KPITCH + half * 16;
  const int grp = lane >> 4, jj = lane & 15;
  const int v_rd = KREG + (4 * (grp >> 1) + (jj >> 2)) * VPITCH + (16 * (grp & 1) + 4 * (jj & 3)) * 2;
  const float sl2 = a.c * 1.4426950408889634f;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones2 = {(__bf16)1.0f, (__bf16)1.0f};

  for (int nt0 = 0; nt0 < G * ntph; nt0 += NW) {
    const int nt = nt0 + wave;
    const int hg = nt / ntph, tr = nt % ntph;
    const int ra = r0 + tr * 32;
    const bool active = nt < G * ntph && ra < r1;   // uniform per wave
    const int h = g * G + hg;          // packed head (index of the anchors handed to the estimate)
    const int hq = a.qh[h];            // its query head (index of Q and of the state)
    const int row = ra + l32;
    bf16x8 qf[KS];
    if (active) {
      const int rowc = min(row, a.N - 1);
      const uint16_t* qp = a.q + b * a.qs0 + (int64_t)rowc * a.qs1 + hq * a.qs2 + half * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const bf16x8*)(qp + ks * 16);
    }
    const int hi = min(ra + 31, a.N - 1);
    const int lo = max(0, ra - a.local + 1);
    f32x16 oacc[DM];
#pragma unroll
    for (int dm = 0; dm < DM; ++dm) oacc[dm] = (f32x16){};
    float m_run = NEG_INF, l_run = 0.f, mx = NEG_INF;

    for (int c = 0; c < n_chunks; ++c) {
      const int crow = min(n_t - c * TPC, TPC) * 32;  // rows of this chunk
      __syncthreads();                                 // every wave is done with the last chunk
      {
        const int nwk = (crow * KPITCH + 1023) / 1024, nwv = (crow * VPITCH + 1023) / 1024;
        for (int w = wave; w < nwk + nwv; w += NW) {
          const bool isv = w >= nwk;
          const int pitch = isv ? VPITCH : KPITCH;
          const int o = (isv ? w - nwk : w) * 1024 + lane * 16;
          const int r = min(o / pitch, crow - 1), cb = o % pitch;
          const int key = min(tile_start(c * TPC + r / 32) + (r % 32), a.N - 1);
          const uint16_t* src = isv ? vb + (int64_t)key * a.vs1 : kb + (int64_t)key * a.ks1;
          unsigned char* dst = kv + (isv ? KREG + (w - nwk) * 1024 : w * 1024);
          __builtin_amdgcn_global_load_lds(src + (cb < ROWB ? cb / 2 : 0), LDS_PTR(void, dst), 16, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(VMCNT_IMM(0));
        __syncthreads();
      }
      if (!active) continue;
      for (int tt = 0; tt < crow / 32; ++tt) {
        const int t = c * TPC + tt;
        const int ts = tile_start(t);
        if (ts > hi) break;                            // tiles ascend; later ones are causal-masked
        if (t >= n_sink_t && ts + 31 < lo) continue;   // window tile entirely before this window
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 kf = *(const bf16x8*)(kv + k_rd + tt * 32 * KPITCH + ks * 32);
          acc = mfma_bf16(kf, qf[ks], acc);
        }
        // a tile whose 32 keys are visible to all 32 rows of the slice needs no mask (a
        // wave-uniform branch: most window tiles)
        const bool all_sink = ts + 31 < a.sink && ts + 31 <= ra;
        const bool all_win = ts >= ra + 31 - a.local + 1 && ts + 31 <= ra;
        float s[16];
        float tm = NEG_INF;
        if (all_sink || all_win) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            mx = fmaxf(mx, acc[r]);
            s[r] = acc[r] * sl2;
            tm = fmaxf(tm, s[r]);
          }
        } else {
          const int w_lo = row - a.local + 1;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = ts + half * 4 + 8 * (r >> 2) + (r & 3);
            const bool ok = key <= row && (key < a.sink || key >= w_lo);
            if (ok) mx = fmaxf(mx, acc[r]);
            s[r] = ok ? acc[r] * sl2 : NEG_INF;
            tm = fmaxf(tm, s[r]);
          }
        }
        tm = half_pair_max(tm);
        // The running max (log2 domain) moves only when a tile's scores exceed it by more than
        // 8, so P stays <= 2^8 and O is rescaled rarely (the result is exact in the ratio).
        if (__any(tm > m_run + 8.0f)) {
          const float mnew = fmaxf(m_run, tm);
          const float alpha = m_run == NEG_INF ? 0.f : __builtin_amdgcn_exp2f(m_run - mnew);
          l_run *= alpha;
#pragma unroll
          for (int dm = 0; dm < DM; ++dm) oacc[dm] *= alpha;
          m_run = mnew;
        }
        const float msub = m_run == NEG_INF ? 0.f : m_run;
        bf16x8 pf[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          f32x8 pt;
#pragma unroll
          for (int e = 0; e < 8; ++e) pt[e] = __builtin_amdgcn_exp2f(s[8 * s2 + e] - msub);
          pf[s2] = __builtin_convertvector(pt, bf16x8);
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const bf16x2 pr = {pf[s2][e], pf[s2][e + 1]};
            l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2, l_run, false);
          }
        }
        // O^T += V^T P^T over the tile's two 16-key groups
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int dm = 0; dm < DM; ++dm) {
            const unsigned char* vp = kv + v_rd + (tt * 32 + 16 * s2) * VPITCH + dm * 64;
            const v4i16 vlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4i16, vp));
            const v4i16 vhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4i16, vp + 8 * VPITCH));
            const v4i16 both[2] = {vlo, vhi};
            bf16x8 vf;
            __builtin_memcpy(&vf, both, 16);
            oacc[dm] = mfma_bf16(vf, pf[s2], oacc[dm]);
          }
      }
    }
    if (!active) continue;
    mx = fmaxf(mx, swap_halves(mx));
    const float lt = half_pair_sum(l_run);
    if (row < r1) {
      // every row's region holds its diagonal key, so lt >= 1 and m_run is finite
      const float inv = 1.0f / lt;
      uint16_t* op = a.st_o + (((int64_t)b * a.N + row) * a.Hq + hq) * D + half * 4;
#pragma unroll
      for (int dm = 0; dm < DM; ++dm)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const unsigned int w0 = float_to_bf16_bits(oacc[dm][4 * q4 + 0] * inv) |
                                  ((unsigned int)float_to_bf16_bits(oacc[dm][4 * q4 + 1] * inv) << 16);
          const unsigned int w1 = float_to_bf16_bits(oacc[dm][4 * q4 + 2] * inv) |
                                  ((unsigned int)float_to_bf16_bits(oacc[dm][4 * q4 + 3] * inv) << 16);
          *(u32x2*)(op + dm * 32 + 8 * q4) = (u32x2){w0, w1};
        }
      if (half == 0) {
        a.st_lse[((int64_t)b * a.Hq + hq) * a.N + row] = (m_run + __log2f(lt)) * 0.69314718055994531f;
        a.xa[((int64_t)b * a.Hq + h) * a.N + row] = __fmul_rn(mx, a.c);
      }
    }
  }
  // no direct load may still be writing this workgroup's LDS when it exits
  __builtin_amdgcn_s_waitcnt(VMCNT_IMM(0));
#endif  // __HIP_DEVICE_COMPILE__
}

hipError_t launch_anchor_state(const EstArgs& a, hipStream_t s) {
  const int grid = a.nQB * a.Hkv * a.B;
  if (a.D == 64)
    hipLaunchKernelGGL(est_anchor_state<64>, dim3(grid), dim3(64 * AS_WAVES), 0, s, a);
  else
    hipLaunchKernelGGL(est_anchor_state<128>, dim3(grid), dim3(64 * AS_WAVES), 0, s, a);
  return hipGetLastError();
}
