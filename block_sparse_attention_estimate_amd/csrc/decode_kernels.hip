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
//   dec_block_summary  kbar[b, J, g, :] = mean of the block's cached keys (fp64 -> fp32 -> bf16)
//   dec_score          score[b, g, J] = max over the group's heads of c * q_h . kbar_J
//   dec_select         forced blocks + top (K - |F|) others by (score desc, block asc),
//                      bitonic sort of 64-bit keys in LDS, ascending output list
//   dec_splitk         per (b, g, split): 16-lane groups stream the split's selected keys
//                      (one 16-byte K and V slice per lane), online softmax for the G packed
//                      heads, merged in-wave then across waves into one partial (m, l, acc)
//   dec_combine        LSE merge of the partials -> O (bf16) and LSE
#include "sa_common.h"
#include "sa_internal.h"

#define NEG_INF (-__builtin_huge_valf())

// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(D) void dec_block_summary(DecArgs a) {
  const int J = blockIdx.x, g = blockIdx.y, b = blockIdx.z, d = threadIdx.x;
  const int lb = min(max(a.cache_len[b], 0), a.L);
  uint16_t* out = (uint16_t*)a.ksum + (((int64_t)b * a.nKB + J) * a.Hkv + g) * D + d;
  const int t0 = J * a.bk;
  if (t0 >= lb) {
    *out = 0;
    return;
  }
  const int t1 = min(lb, t0 + a.bk);
  const uint16_t* kp = a.kc + b * a.ks0 + g * a.ks2 + d;
  double s = 0.0;
  for (int t = t0; t < t1; ++t) s += bf16_bits_to_double(kp[(int64_t)t * a.ks1]);
  const double mean = s / (double)(t1 - t0);
  *out = float_to_bf16_bits((float)mean);
}

// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void dec_score(DecArgs a) {
  const int g = blockIdx.y, b = blockIdx.z;
  const int J = blockIdx.x * 256 + threadIdx.x;
  __shared__ float qs[8][D];
  for (int p = threadIdx.x; p < a.G * D; p += 256) {
    const int hg = p / D, d = p % D;
    qs[hg][d] = bf16_bits_to_float(a.q[b * a.qs0 + (g * a.G + hg) * a.qs2 + d]);
  }
  __syncthreads();
  if (J >= a.nKB) return;
  const int nb = (min(max(a.cache_len[b], 0), a.L) + a.bk - 1) / a.bk;
  float score = NEG_INF;
  if (J < nb) {
    const uint16_t* kp = a.ksum + (((int64_t)b * a.nKB + J) * a.Hkv + g) * D;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int d0 = 0; d0 < D; d0 += 8) {
      const u16x8 kv = *(const u16x8*)(kp + d0);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = bf16_bits_to_float(kv[e]);
#pragma unroll
        for (int hg = 0; hg < 8; ++hg)
          if (hg < a.G) acc[hg] = fmaf(qs[hg][d0 + e], x, acc[hg]);
      }
    }
    float mx = acc[0];
#pragma unroll
    for (int hg = 1; hg < 8; ++hg)
      if (hg < a.G) mx = fmaxf(mx, acc[hg]);
    score = mx * a.c;
  }
  a.scores[((int64_t)b * a.Hkv + g) * a.nKB + J] = score;
}

// ---------------------------------------------------------------------------------------
// NP = power of two >= nKB (<= 8192).  One workgroup of 1024 threads per (b, g).
template <int NP>
__global__ __launch_bounds__(1024) void dec_select(DecArgs a) {
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  __shared__ unsigned long long keys[NP];
  __shared__ unsigned char flag[NP];
  __shared__ int wsum[16];
  const int lb = min(max(a.cache_len[b], 0), a.L);
  const int nb = (lb + a.bk - 1) / a.bk;
  const float* sc = a.scores + ((int64_t)b * a.Hkv + g) * a.nKB;
  for (int j = tid; j < NP; j += 1024) {
    unsigned long long key = 0ull;
    if (j < nb) {
      const bool forced = (j * a.bk < a.sink) || ((j + 1) * a.bk - 1 >= lb - a.local);
      const unsigned int hi = forced ? 0xFFFFFFFFu : float_order_key(sc[j]);
      key = ((unsigned long long)hi << 32) | (unsigned long long)(0xFFFFFFFFu - (unsigned int)j);
    }
    keys[j] = key;
    flag[j] = 0;
  }
  __syncthreads();
  // bitonic sort, descending
  for (int k = 2; k <= NP; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < NP; i += 1024) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const unsigned long long x = keys[i], y = keys[ixj];
          const bool desc = (i & k) == 0;
          if (desc ? (x < y) : (x > y)) {
            keys[i] = y;
            keys[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  const int kk = min(a.top_k, nb);
  for (int p = tid; p < kk; p += 1024) {
    const unsigned int j = 0xFFFFFFFFu - (unsigned int)(keys[p] & 0xFFFFFFFFull);
    flag[j] = 1;
  }
  __syncthreads();
  // ascending compaction of the flags
  constexpr int PER = NP / 1024 > 0 ? NP / 1024 : 1;
  const int j0 = tid * PER;
  int cnt = 0;
  for (int j = j0; j < j0 + PER && j < NP; ++j) cnt += flag[j];
  const int lane = tid & 63, wave = tid >> 6;
  int incl = cnt;
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int pos = incl - cnt;
  for (int w = 0; w < wave; ++w) pos += wsum[w];
  int32_t* out = a.selected + ((int64_t)b * a.Hkv + g) * a.top_k;
  for (int j = j0; j < j0 + PER && j < NP; ++j)
    if (flag[j]) out[pos++] = j;
  for (int p = kk + tid; p < a.top_k; p += 1024) out[p] = -1;
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
  const int nsel = min(a.top_k, nb);
  const int bps = (nsel + a.n_splits - 1) / a.n_splits;
  const int blk0 = s * bps, blk1 = min(nsel, blk0 + bps);
  const int nkeys = max(0, blk1 - blk0) * a.bk;
  const int32_t* sel = a.selected + ((int64_t)b * a.Hkv + g) * a.top_k;
  const float sl2 = a.c * 1.4426950408889634f;

  float qv[G][DPL];
#pragma unroll
  for (int hg = 0; hg < G; ++hg) {
    const uint16_t* qp = a.q + b * a.qs0 + (g * G + hg) * a.qs2 + sub * DPL;
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
template <int D>
__global__ __launch_bounds__(D) void dec_combine(DecArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const float* part = a.partial + ((int64_t)b * a.Hq + h) * a.n_splits * (D + 2);
  float mx = -1e30f;
  for (int s = 0; s < a.n_splits; ++s)
    if (part[s * (D + 2) + D + 1] > 0.f) mx = fmaxf(mx, part[s * (D + 2) + D]);
  float lt = 0.f, at = 0.f;
  for (int s = 0; s < a.n_splits; ++s) {
    const float ls = part[s * (D + 2) + D + 1];
    if (ls > 0.f) {
      const float f = __builtin_amdgcn_exp2f(part[s * (D + 2) + D] - mx);
      lt += ls * f;
      at += part[s * (D + 2) + d] * f;
    }
  }
  const float o = lt > 0.f ? at / lt : 0.f;
  ((uint16_t*)a.o)[b * a.os0 + h * a.os2 + d] = float_to_bf16_bits(o);
  if (a.lse && d == 0)
    a.lse[(int64_t)b * a.Hq + h] = lt > 0.f ? (mx + __log2f(lt)) * 0.69314718055994531f : NEG_INF;
}

// ---------------------------------------------------------------------------------------
hipError_t launch_block_summary(const DecArgs& a, hipStream_t s) {
  if (a.D == 64)
    hipLaunchKernelGGL(dec_block_summary<64>, dim3(a.nKB, a.Hkv, a.B), dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL(dec_block_summary<128>, dim3(a.nKB, a.Hkv, a.B), dim3(128), 0, s, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_decode_d(const DecArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(dec_score<D>, dim3((a.nKB + 255) / 256, a.Hkv, a.B), dim3(256), 0, s, a);
  const int nkb = a.nKB;
  if (nkb <= 1024)
    hipLaunchKernelGGL(dec_select<1024>, dim3(a.Hkv, a.B), dim3(1024), 0, s, a);
  else if (nkb <= 2048)
    hipLaunchKernelGGL(dec_select<2048>, dim3(a.Hkv, a.B), dim3(1024), 0, s, a);
  else if (nkb <= 4096)
    hipLaunchKernelGGL(dec_select<4096>, dim3(a.Hkv, a.B), dim3(1024), 0, s, a);
  else
    hipLaunchKernelGGL(dec_select<8192>, dim3(a.Hkv, a.B), dim3(1024), 0, s, a);
  const dim3 grid(a.n_splits, a.Hkv, a.B);
  switch (a.G) {
    case 1: hipLaunchKernelGGL((dec_splitk<D, 1>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((dec_splitk<D, 2>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((dec_splitk<D, 4>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((dec_splitk<D, 8>), grid, dim3(256), 0, s, a); break;
  }
  hipLaunchKernelGGL(dec_combine<D>, dim3(a.Hq, a.B), dim3(D), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecArgs& a, hipStream_t s) {
  if (a.D == 64) return launch_decode_d<64>(a, s);
  return launch_decode_d<128>(a, s);
}
