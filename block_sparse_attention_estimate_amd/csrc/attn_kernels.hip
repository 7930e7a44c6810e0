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
//  * O is written through LDS, so every store instruction writes whole rows;
//  * the running max moves only when a tile's probabilities would exceed 2^16, so O is rarely
//    rescaled;
//  * work items are ordered longest-first (last query blocks first), the two 64-row halves of
//    a 128-row query block (same list, same K/V) land on the same XCD, and the KV group
//    rotates every 16 query blocks;
//  * instances: block lists, column lists (gathered rows), 32-key block lists, and resuming
//    from an anchor state (block or column lists).
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

// MODE: 0 = lists of 64-key blocks; 1 = lists of key columns (stripes); 2 = lists of 32-key
// blocks (two listed blocks per 64-key tile, gathered like columns)
template <int D, int HPW, bool RESUME, int MODE>
__global__ __launch_bounds__(128 * HPW) void attn_block(AttnArgs a) {
  constexpr bool STRIPE = MODE == 1, BK32 = MODE == 2, GATHER = MODE != 0;
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
  // query head of this wave (packed head g * G + j of the workgroup's KV head)
  const int h = a.qh[g * a.G + hp * HPW + (wave >> 1)];
  const int rw = r0 + (wave & 1) * 32;
  const int row = rw + l32;

  // the lists are read-only here: read them through the constant address space (scalar loads)
  const int64_t lrow = (int64_t)(b * a.Hkv + g) * a.nQB + iq;
  const __attribute__((address_space(4))) int32_t* list =
      (const __attribute__((address_space(4))) int32_t*)(a.idx + lrow * a.stride);
  int n = min(((const __attribute__((address_space(4))) int32_t*)a.counts)[lrow], a.stride);
  // the same list through a plain pointer, for per-lane reads of gathered column ids
  const int32_t* list_g = a.idx + lrow * a.stride;
#ifdef SA_DEBUG
  if (wave == 0 && tsub == 0) {
    // caller-built lists: a count in [0, stride], entries inside the sequence, ascending
    const int cnt = ((const __attribute__((address_space(4))) int32_t*)a.counts)[lrow];
    SA_DCHECK(a.dbg, cnt >= 0 && cnt <= a.stride, SA_DBG_COUNT);
    const int lim = STRIPE ? a.N : BK32 ? (a.N + 31) >> 5 : (a.N + 63) >> 6;
    for (int e = lane; e < n; e += 64) {
      const int v = list_g[e];
      SA_DCHECK(a.dbg, v >= 0 && v < lim, SA_DBG_RANGE);
      if (e > 0) SA_DCHECK(a.dbg, list_g[e - 1] < v, SA_DBG_ORDER);
    }
  }
#endif
  int ntile, n_main;
  if (STRIPE) {
    // column lists: the entries this work item can see (<= r_last, ascending); tiles of 64
    // gathered columns; tiles from n_main on need a mask (a column past the first row's
    // diagonal or the end, or entries past the list's end).  The entries <= a limit are a
    // prefix of the list, counted by a 64-way search: each round every lane reads one entry
    // (vector loads, one round trip per round) and the wave's ballot narrows the range to one
    // lane's stride.
    auto count_le = [&](int limit) -> int {
      int lo = 0, len = n;                       // the count lies in [lo, lo + len]
      while (len > 0) {
        const int step = (len + 63) >> 6;
        const int idx = lo + min((lane + 1) * step, len) - 1;
        const int c = __popcll(__ballot(list_g[idx] <= limit));
        const int a0 = min(c * step, len);       // entries known to pass
        const int a1 = min((c + 1) * step, len) - 1;  // the entry at a1 fails (when c < 64)
        lo += a0;
        len = c >= 64 ? 0 : a1 - a0;
      }
      return lo;
    };
    if constexpr (RESUME) {
      // Resuming from the anchor state: row r needs the listed columns in [sink, r - local]
      // (the state holds its sink and window tokens), so the item needs the entries in
      // [sink, r_last - local], and those <= r0 - local are needed by every row (no mask).
      const int first = a.sink > 0 ? count_le(a.sink - 1) : 0;
      const int n_need = count_le(r_last - a.local);
      const int n_all = count_le(r0 - a.local);
      list += first;
      list_g += first;
      n = max(n_need - first, 0);
      ntile = (n + 63) / 64;
      n_main = max(n_all - first, 0) / 64;
    } else {
      const int n0 = count_le(r0);               // entries visible to every row of the item
      n = count_le(r_last);
      ntile = (n + 63) / 64;
      n_main = n0 / 64;                          // full tiles of entries <= r0
    }
  } else if (BK32) {
    // 32-key block lists: two listed blocks per tile; blocks from `r_last + 1` on hold no key
    // of this work item; the tiles from n_main on need a mask (a block past the first row's
    // diagonal or the end, or the empty second half of the last tile)
    while (n > 0 && list[n - 1] * 32 >= r_last + 1) --n;
    ntile = (n + 1) / 2;
    n_main = ntile;
    while (n_main > 0 && (2 * n_main > n || list[2 * n_main - 1] * 32 + 31 >= r0 + 1 ||
                          list[2 * n_main - 1] * 32 + 31 >= a.N))
      --n_main;
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
  const int nkb = (a.N + 63) >> 6;                     // key blocks of the sequence
  // Block lists: byte offset of this lane's 16 bytes within a tile (row r of the window's
  // bytes, column cb; pads get a harmless copy of the row start), added to the tile's
  // wave-uniform base address, so the loads take a scalar base and one 32-bit offset.
  // Column lists: the row of this lane's bytes and their element offset within the row.
  uint32_t s_voff[SLOTS];
  int s_off[GATHER ? SLOTS : 1];
  int s_row[GATHER ? SLOTS : 1];
#pragma unroll
  for (int k = 0; k < SLOTS; ++k) {
    const int o = min(wbase + k, nwin - 1) * 1024 + lane * 16;
    const int r = o / pitch_b, cb = o % pitch_b;
    const int cbytes = cb < ROWB ? cb : 0;
    if (GATHER) {
      s_row[k] = r;
      s_off[k] = cbytes / 2;
    }
    s_voff[k] = (uint32_t)((int64_t)r * tstride * 2 + cbytes);
  }
  // LDS window of slot k in the stage at stb (windows past NWIN go to `spare`)
  auto dst = [&](unsigned char* stb, int k) -> unsigned char* {
    return wbase + k < nwin ? stb + region + (wbase + k) * 1024 : spare;
  };
  // What the DMA of tile t needs, read ahead of the issue: the key block id (block lists; a
  // scalar load, clamped to the sequence's blocks so a bad entry cannot address memory
  // outside K and V), or this lane's column id per slot (column lists; vector loads, rows
  // past the list's end repeat its last entry).
  struct Src {
    int v[STRIPE ? SLOTS : (BK32 ? 2 : 1)];
  };
  auto fetch = [&](int t) -> Src {
    Src sv;
    if constexpr (STRIPE) {
      const int tt = min(t, ntile - 1);
#pragma unroll
      for (int k = 0; k < SLOTS; ++k) sv.v[k] = list_g[min(tt * 64 + s_row[k], n - 1)];
    } else if constexpr (BK32) {
      // the tile's two 32-key blocks (the second -1 when the list ends in the first); ids
      // clamped to the sequence's blocks
      const int tt = min(t, ntile - 1);
      const int nb32 = (a.N + 31) >> 5;
      sv.v[0] = min(max(list[2 * tt], 0), nb32 - 1);
      sv.v[1] = 2 * tt + 1 < n ? min(max(list[2 * tt + 1], 0), nb32 - 1) : -1;
    } else {
      sv.v[0] = min(max(list[min(t, ntile - 1)], 0), nkb - 1);
    }
    return sv;
  };
  // Issue the DMA of a tile into the stage at stb.  Every wave issues exactly SLOTS loads per
  // call, so the vmcnt waits below are compile-time constants.
  auto issue = [&](unsigned char* stb, const Src& sv) {
    if constexpr (GATHER) {
#pragma unroll
      for (int k = 0; k < SLOTS; ++k) {
        int tok;
        if constexpr (STRIPE) {
          tok = sv.v[k];
        } else {
          // row r of the tile: row r % 32 of the tile's first or second block (an empty
          // second half reads the first block's rows: a harmless copy, masked)
          const int blk = s_row[k] < 32 || sv.v[1] < 0 ? sv.v[0] : sv.v[1];
          tok = blk * 32 + (s_row[k] & 31);
        }
        tok = min(max(tok, 0), a.N - 1);
        const uint16_t* src = gbase + (int64_t)tok * tstride + s_off[k];
        __builtin_amdgcn_global_load_lds(src, LDS_PTR(void, dst(stb, k)), 16, 0, 0);
      }
      return;
    }
    // block lists: one buffer resource per tile (base = the tile's first row, in scalar
    // registers), the lane's 32-bit offset within the tile, the range = the tile's rows
    const int t0 = sv.v[0] * 64;
    const int last = min(63, a.N - 1 - t0);             // last row of the tile in the sequence
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(gbase + (int64_t)t0 * tstride), 0, (int)((int64_t)last * tstride * 2 + ROWB),
        0x00020000);
    if (last == 63) {
#pragma unroll
      for (int k = 0; k < SLOTS; ++k)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDS_PTR(void, dst(stb, k)), 16, (int)s_voff[k], 0, 0, 0);
    } else {
      // ragged last block: rows past the end read the last row
#pragma unroll
      for (int k = 0; k < SLOTS; ++k) {
        const int o = min(wbase + k, nwin - 1) * 1024 + lane * 16;
        const int r = dma_v ? o / VPITCH : o / KPITCH;
        const int back = (int)((int64_t)max(r - last, 0) * tstride * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDS_PTR(void, dst(stb, k)), 16, (int)s_voff[k] - back, 0, 0, 0);
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
  typedef float f32x2 __attribute__((ext_vector_type(2)));
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
  // K fragment i of S^T = K Q^T (key half i & 1, k-step i >> 1) from the stage at sb
  auto kread = [&](const unsigned char* sb, int i) -> bf16x8 {
    return *(const bf16x8*)(sb + k_rd + (i & 1) * 32 * KPITCH + (i >> 1) * 32);
  };
  // V^T fragment i of key half mt (16-key group 2 mt + i / DM, d tile i % DM), read with two
  // transposing LDS reads
  auto vread = [&](const unsigned char* sb, int mt, int i) -> bf16x8 {
    const int s4 = 2 * mt + i / DM, dm = i % DM;
    const unsigned char* vp = sb + v_rd + 16 * s4 * VPITCH + dm * 64;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4i16, vp));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(v4i16, vp + 8 * VPITCH));
    const v4i16 both[2] = {lo, hi};
    bf16x8 vf;
    __builtin_memcpy(&vf, both, 16);
    return vf;
  };
  // P^T is kept as packed bf16 pairs: pw[8 mt + 4 s2 + k] holds entries 8 s2 + 2k and
  // 8 s2 + 2k + 1 of key half mt of the lane's S^T column; B operand of 16-key group s4
  auto pfrag = [&](const uint32_t* pw, int s4) -> bf16x8 {
    const u32x4 w4 = {pw[4 * s4], pw[4 * s4 + 1], pw[4 * s4 + 2], pw[4 * s4 + 3]};
    bf16x8 f;
    __builtin_memcpy(&f, &w4, 16);
    return f;
  };
  // P entry e of key half mt: exp2(S scale - m); at odd e the pair is rounded to bf16, stored
  // and added to the lane's partial row sum (the sum of the values P V uses)
  auto exp_elem = [&](const f32x16* sacc, int mt, int e, float mneg, float* xs, uint32_t* pw,
                      float& ls) {
    xs[e] = __builtin_amdgcn_exp2f(fmaf(sacc[mt][e], sl2, mneg));
    if (e & 1) {
      const f32x2 x2 = {xs[e - 1], xs[e]};
      const bf16x2 pr = __builtin_convertvector(x2, bf16x2);
      pw[8 * mt + e / 2] = __builtin_bit_cast(uint32_t, pr);
      ls = __builtin_amdgcn_fdot2_f32_bf16(pr, ones2, ls, false);
    }
  };
  // P^T of key half mt in one go; returns this lane's sum of the rounded values
  auto expo = [&](const f32x16* sacc, int mt, uint32_t* pw) -> float {
    const float mneg = -m_run;
    float xs[16], ls = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) exp_elem(sacc, mt, e, mneg, xs, pw, ls);
    return ls;
  };
  // S^T = K Q^T from the stage at sb (no other work: the first tile)
  auto qk = [&](const unsigned char* sb, f32x16* sacc) {
    sacc[0] = (f32x16){};
    sacc[1] = (f32x16){};
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) sacc[i & 1] = mfma_bf16(kread(sb, i), qf[i >> 1], sacc[i & 1]);
  };
  // The phases of a step are written in issue order and fenced (sched_barrier), so that every
  // LDS read is issued several MFMAs ahead of its use and the softmax VALU work is spread
  // between the MFMAs of the same wave.
  // S(t+1) = K(t+1) Q^T from the stage at sb, with P(t)'s first key half: four K fragments in
  // flight, then per MFMA the next fragment's read and the exponentials of the next MFMA's share.
  auto qk_exp = [&](const unsigned char* sb, f32x16* nxt, const f32x16* cur, uint32_t* pw) -> float {
    constexpr int NF = 2 * KS, AH = 4, EPM = 16 / NF;
    const float mneg = -m_run;
    float xs[16], ls = 0.f;
    bf16x8 kf[AH];
#pragma unroll
    for (int i = 0; i < AH; ++i) kf[i] = kread(sb, i);
#pragma unroll
    for (int j = 0; j < EPM; ++j) exp_elem(cur, 0, j, mneg, xs, pw, ls);
    nxt[0] = (f32x16){};
    nxt[1] = (f32x16){};
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      nxt[i & 1] = mfma_bf16(kf[i % AH], qf[i >> 1], nxt[i & 1]);
      if (i + AH < NF) kf[i % AH] = kread(sb, i + AH);
      if (i + 1 < NF) {
#pragma unroll
        for (int j = 0; j < EPM; ++j) exp_elem(cur, 0, (i + 1) * EPM + j, mneg, xs, pw, ls);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return ls;
  };
  // O^T += V^T P^T over key half mt from the stage at sb: three V fragments in flight, then per
  // MFMA the next fragment's reads and (with_exp) the exponentials of P(t)'s second half.
  auto pv_exp = [&](const unsigned char* sb, int mt, uint32_t* pw, const f32x16* cur,
                    bool with_exp, auto&& extra) -> float {
    constexpr int NF = 2 * DM, AH = 3, EPM = 16 / NF;
    const float mneg = -m_run;
    float xs[16], ls = 0.f;
    bf16x8 vf[AH];
#pragma unroll
    for (int i = 0; i < AH; ++i) vf[i] = vread(sb, mt, i);
    if (with_exp) {
#pragma unroll
      for (int j = 0; j < EPM; ++j) exp_elem(cur, 1, j, mneg, xs, pw, ls);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      oacc[i % DM] = mfma_bf16(vf[i % AH], pfrag(pw, 2 * mt + i / DM), oacc[i % DM]);
      if (i + AH < NF) vf[i % AH] = vread(sb, mt, i + AH);
      if (with_exp && i + 1 < NF) {
#pragma unroll
        for (int j = 0; j < EPM; ++j) exp_elem(cur, 1, (i + 1) * EPM + j, mneg, xs, pw, ls);
      }
      extra(i, NF);
      __builtin_amdgcn_sched_barrier(0);
    }
    return ls;
  };
  auto no_extra = [](int, int) {};
  // entries of tile t past the diagonal or the end of the sequence (resuming: also those in
  // the row's anchor region, which the state already holds; the window includes the diagonal)
  // token of entry (mt, r) of a block-list tile with source ids js (-1: no token)
  auto tile_tok = [&](const Src& js, int mt, int r) -> int {
    const int key = mt * 32 + half * 4 + 8 * (r >> 2) + (r & 3);
    if constexpr (BK32) {
      const int blk = mt == 0 ? js.v[0] : js.v[1];
      return blk < 0 ? -1 : blk * 32 + (key & 31);
    } else {
      return js.v[0] * 64 + key;
    }
  };
  auto mask = [&](int t, const Src& js, f32x16* sacc) {
    if constexpr (STRIPE) {
      // the tile's 64 column ids, lane i holding entry 64 t + i (past the list's end: none)
      const int e = t * 64 + lane;
      const int mine = e < n ? list_g[e] : 0x7FFFFFFF;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int tok = __shfl(mine, mt * 32 + half * 4 + 8 * (r >> 2) + (r & 3));
          const bool drop = RESUME ? (tok < a.sink || tok >= row - a.local + 1 || tok >= a.N)
                                   : (tok > row || tok >= a.N);
          if (drop) sacc[mt][r] = NEG_INF;
        }
      return;
    }
    (void)t;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tok = tile_tok(js, mt, r);
        const bool drop = RESUME ? (tok < a.sink || tok >= row - a.local + 1 || tok >= a.N)
                                 : (tok < 0 || tok > row || tok >= a.N);
        if (drop) sacc[mt][r] = NEG_INF;
      }
  };
  // The running max m stays fixed while every P value of a key half is at most 2^16 (checked
  // on the lane's partial row sum, which bounds each value).  A half that breaks the bound
  // (scores more than 16 above m in the log2 domain, or the first tile, while m is still
  // -1e30) moves m to the half's row max, rescales O and l -- which may already hold the other
  // half's P V at the old m -- and recomputes its P.  No per-tile row max is taken.
  auto settle = [&](const f32x16* sacc, int mt, uint32_t* pw, float ts) {
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
      ts = expo(sacc, mt, pw);
    }
    l_run += ts;
  };

  // Software pipeline over the list.  On entry to step t, S(t) is in `cur` (masked), tiles t
  // and t+1 are in LDS, tile t+2 is in flight and the stage of tile t-1 is free.  Step t issues
  // the DMA of tile t+3 into that stage, computes P(t)'s first key half while the MFMAs of
  // S(t+1) run, P(t)'s second half while P V of the first half runs, and P V of the second
  // half, then waits for tile t+2: each tile has about two steps to arrive.  The list entries
  // a step needs were read one step earlier (the scalar loads return under the barrier).
  if (ntile > 0) {
    const Src j0 = fetch(0), j1 = fetch(1), j2 = fetch(2);
    issue(st0, j0);
    issue(st1, j1);
    issue(st2, j2);
    Src jc = fetch(3);                 // DMA source of tile t+3
    Src ja = j1, jb2 = j2;             // sources of tiles t+1 and t+2 (their masks)
    DMA_BARRIER(SLOTS);
    f32x16 sa[2], sbb[2];
    qk(st0, sa);
    if (n_main == 0 || (RESUME && !STRIPE && j0.v[0] * 64 < a.sink)) mask(0, j0, sa);
    auto step = [&](unsigned char* sc, unsigned char* sn, unsigned char* sd, int t,
                    f32x16* cur, f32x16* nxt, bool may_mask) {
      issue(sd, jc);
      const Src jd = fetch(t + 4);
      uint32_t pw[16];
      const float t0s = qk_exp(sn, nxt, cur, pw);
      settle(cur, 0, pw, t0s);
      const float t1s = pv_exp(sc, 0, pw, cur, true, no_extra);
      settle(cur, 1, pw, t1s);
      pv_exp(sc, 1, pw, cur, false, no_extra);
      if (may_mask && t + 1 >= n_main) mask(t + 1, ja, nxt);
      ja = jb2;
      jb2 = jc;
      jc = jd;
      DMA_BARRIER(SLOTS);
    };
    auto last = [&](unsigned char* sc, f32x16* cur) {
      uint32_t pw[16];
      const float t0s = expo(cur, 0, pw);
      settle(cur, 0, pw, t0s);
      const float t1s = pv_exp(sc, 0, pw, cur, true, no_extra);
      settle(cur, 1, pw, t1s);
      pv_exp(sc, 1, pw, cur, false, no_extra);
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
  // O leaves through LDS: each wave writes its 32 x D tile (bf16) into a region of the stages
  // of its own, then stores whole rows, 16 bytes per lane, so that a store instruction writes
  // complete rows instead of 16 bytes of each of 32 rows.
  constexpr int OPITCH = ROWB + 16;
  static_assert(2 * 32 * OPITCH <= STAGE, "two waves' output tiles must fit in a stage");
  __syncthreads();                   // no wave still reads a stage and no load still fills one
  {
    const int sel = wave >> 1;
    unsigned char* ob = (sel == 0 ? st0 : sel == 1 ? st1 : sel == 2 ? st2 : st3) + (wave & 1) * 32 * OPITCH;
#pragma unroll
    for (int dm = 0; dm < DM; ++dm)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const unsigned int lo = float_to_bf16_bits(oacc[dm][4 * q4 + 0] * inv) |
                                ((unsigned int)float_to_bf16_bits(oacc[dm][4 * q4 + 1] * inv) << 16);
        const unsigned int hi = float_to_bf16_bits(oacc[dm][4 * q4 + 2] * inv) |
                                ((unsigned int)float_to_bf16_bits(oacc[dm][4 * q4 + 3] * inv) << 16);
        *(u32x2*)(ob + l32 * OPITCH + (dm * 32 + 8 * q4 + half * 4) * 2) = (u32x2){lo, hi};
      }
    constexpr int CPR = ROWB / 16;   // 16-byte chunks of a row
    constexpr int RPI = 64 / CPR;    // rows per store instruction
    const int c = lane % CPR, rr = lane / CPR;
    uint16_t* obase = a.o + b * a.os0 + h * a.os2 + c * 8;
#pragma unroll
    for (int k = 0; k < 32 / RPI; ++k) {
      const int lr = rr + k * RPI;
      const u32x4 v = *(const u32x4*)(ob + lr * OPITCH + c * 16);
      if (rw + lr < a.N) *(u32x4*)(obase + (int64_t)(rw + lr) * a.os1) = v;
    }
  }
  if (a.lse && half == 0 && row < a.N)
    a.lse[((int64_t)b * a.Hq + h) * a.N + row] =
        lt > 0.f ? (m_run + __log2f(lt)) * 0.69314718055994531f : NEG_INF;
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------------------------
template <int D, int HPW>
static hipError_t launch_block(const AttnArgs& a0, hipStream_t s) {
  AttnArgs a = a0;
  a.n_hp = a.G / HPW;
  a.total = a.B * a.Hkv * a.n_hp * a.nQB * a.tpb;
  if (a.total == 0) return hipSuccess;
  if (a.st_o && a.stripe)
    hipLaunchKernelGGL((attn_block<D, HPW, true, 1>), dim3(a.total), dim3(128 * HPW), 0, s, a);
  else if (a.st_o)
    hipLaunchKernelGGL((attn_block<D, HPW, true, 0>), dim3(a.total), dim3(128 * HPW), 0, s, a);
  else if (a.stripe)
    hipLaunchKernelGGL((attn_block<D, HPW, false, 1>), dim3(a.total), dim3(128 * HPW), 0, s, a);
  else if (a.bk32)
    hipLaunchKernelGGL((attn_block<D, HPW, false, 2>), dim3(a.total), dim3(128 * HPW), 0, s, a);
  else
    hipLaunchKernelGGL((attn_block<D, HPW, false, 0>), dim3(a.total), dim3(128 * HPW), 0, s, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const AttnArgs& a, hipStream_t s) {
  if (a.G >= 4) return launch_block<D, 4>(a, s);
  if (a.G == 2) return launch_block<D, 2>(a, s);
  return launch_block<D, 1>(a, s);
}

// Block and column lists both run attn_block; a.stripe (set from the granularity) and a.bk32
// (32-key block lists) select the instances that gather listed rows.
hipError_t launch_prefill(const AttnArgs& a, int D, int granularity, hipStream_t s) {
  (void)granularity;
  return D == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s);
}
