// Per-head L1 output error for the theta calibration loop on gfx950.
//
// SALE (arXiv 2505.24179), "Assumptions & free parameters": the per-head threshold tau starts
// at 0.008 and is halved until the L1 output error Err(tau) = ||O - O~||_1 / N against full
// attention meets a user-chosen bound.  This kernel computes the numerator for every query
// head at once: the sum over batch, rows and head dimensions of |O - O~|.
#include "sa_common.h"
#include "sa_internal.h"

// Zero the per-head accumulators (a kernel rather than a memset, so the sequence could be
// captured in a graph).
__global__ void cal_zero(double* err, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) err[i] = 0.0;
}

// One workgroup per (32-row chunk, batch).  Both outputs are contiguous [B, N, Hq, D] bf16;
// thread t reads 8 consecutive elements (one 16-byte load) at offsets 8 t + 2048 i of a row,
// which all belong to head (8 t + 2048 i) / D.  Element differences are exact in fp32; sums
// are fp64 (per thread, then per workgroup in LDS, then one global atomic per head).
template <int D>
__global__ __launch_bounds__(256) void cal_head_l1(const uint16_t* o_ref, const uint16_t* o_sp,
                                                   int N, int Hq, double* err) {
  constexpr int ROWS = 32, MAXI = SA_MAX_Q_HEADS * D / 2048;
  __shared__ double red[SA_MAX_Q_HEADS];
  const int tid = threadIdx.x, b = blockIdx.y;
  const int r0 = blockIdx.x * ROWS, r1 = min(N, r0 + ROWS);
  const int row_elems = Hq * D;
  for (int h = tid; h < Hq; h += 256) red[h] = 0.0;
  double acc[MAXI];
#pragma unroll
  for (int i = 0; i < MAXI; ++i) acc[i] = 0.0;
  for (int r = r0; r < r1; ++r) {
    const int64_t base = ((int64_t)b * N + r) * row_elems;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int e = tid * 8 + 2048 * i;
      if (e < row_elems) {
        const u16x8 x = *(const u16x8*)(o_ref + base + e);
        const u16x8 y = *(const u16x8*)(o_sp + base + e);
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) s += fabsf(bf16_bits_to_float(x[j]) - bf16_bits_to_float(y[j]));
        acc[i] += (double)s;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    const int e = tid * 8 + 2048 * i;
    if (e < row_elems) atomicAdd(&red[e / D], acc[i]);
  }
  __syncthreads();
  for (int h = tid; h < Hq; h += 256) atomicAdd(err + h, red[h]);
}

hipError_t launch_head_l1(const uint16_t* o_ref, const uint16_t* o_sp, int B, int N, int Hq, int D,
                          double* err, hipStream_t s) {
  hipLaunchKernelGGL(cal_zero, dim3((Hq + 255) / 256), dim3(256), 0, s, err, Hq);
  const dim3 grid((N + 31) / 32, B);
  if (D == 64)
    hipLaunchKernelGGL(cal_head_l1<64>, grid, dim3(256), 0, s, o_ref, o_sp, N, Hq, err);
  else
    hipLaunchKernelGGL(cal_head_l1<128>, grid, dim3(256), 0, s, o_ref, o_sp, N, Hq, err);
  return hipGetLastError();
}
