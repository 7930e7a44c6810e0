// Shared device types and small helpers for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

// generic pointer -> LDS (address space 3) pointer, for the LDS-only builtins
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
// wait for vmcnt <= n only (expcnt and lgkmcnt at their maxima)
#define VMCNT_IMM(n) ((((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8)))
// wait for vmcnt <= n and lgkmcnt = 0 (every LDS read and scalar load of this wave returned)
#define VMCNT_LGKM0_IMM(n) ((((n) & 15) | (((n) >> 4) << 14) | (7 << 4)))
// wait for lgkmcnt = 0 only
#define LGKM0_IMM (15 | (3 << 14) | (7 << 4))

#define SA_DEV static __device__ __forceinline__

// Debug builds (-DSA_DEBUG, libsa_debug.so): kernels check the caller data that the release
// kernels clamp -- list counts and entries, cache lengths -- and set bits of a device word
// that the host reads after the call.  The release build compiles no check.
#define SA_DBG_COUNT 1u       // a list count outside [0, stride]
#define SA_DBG_RANGE 2u       // a list entry outside the sequence's key blocks (or columns)
#define SA_DBG_ORDER 4u       // list entries not strictly ascending
#define SA_DBG_CACHE_LEN 8u   // a cache length outside [0, seq_k]
#ifdef SA_DEBUG
#define SA_DCHECK(word, cond, bit)       \
  do {                                   \
    if (!(cond)) atomicOr((word), (bit)); \
  } while (0)
#else
#define SA_DCHECK(word, cond, bit) \
  do {                             \
  } while (0)
#endif

// 32x32x16 bf16 MFMA: A lane l holds A[l%32][(l/32)*8 .. +8]; B lane l holds
// B[(l/32)*8 .. +8][l%32]; C lane l holds C[(l/32)*4 + 8*(r/4) + r%4][l%32], r = 0..15.
SA_DEV f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 32x32x32 int8 MFMA, same lane pattern with 16 int8 (4 dwords) per lane along k.
SA_DEV i32x16 mfma_i8(i32x4 a, i32x4 b, i32x16 c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

SA_DEV float bf16_bits_to_float(unsigned short u) {
  return __uint_as_float(((unsigned int)u) << 16);
}

SA_DEV double bf16_bits_to_double(unsigned short u) {
  return (double)__uint_as_float(((unsigned int)u) << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
SA_DEV unsigned short float_to_bf16_bits(float f) {
  unsigned int u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

SA_DEV float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

SA_DEV double wave_sum_d(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

SA_DEV int wave_sum_i(int v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Exchange a value with lane ^ 32 (the other half of a wave64).
SA_DEV float swap_halves(float v) {
  return __shfl_xor(v, 32);
}

// max / sum of a value and its copy in lane ^ 32, with v_permlane32_swap (no LDS traffic).
// The swap leaves lanes 0-31 of the first result and lanes 32-63 of the second untouched and
// exchanges the others, so for every lane the pair holds {v[l], v[l ^ 32]} in some order.
SA_DEV float half_pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

SA_DEV float half_pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

SA_DEV int swap_halves_i(int v) {
  return __shfl_xor(v, 32);
}

// Wave-uniform copy of a value that is uniform across the wave (lets the compiler keep it in
// scalar registers and branch on it without exec-mask handling).
SA_DEV int wave_uniform(int v) {
  return __builtin_amdgcn_readfirstlane(v);
}

// Workgroup barrier for the DMA pipeline.  __syncthreads() carries a workgroup release fence,
// and since the direct-to-LDS loads write LDS the fence makes the compiler wait for every one
// of them (vmcnt(0)) -- including the prefetch just issued.  Here the wait is explicit: this
// wave's DMAs older than the newest n are complete and its LDS reads have returned; after the
// barrier the same holds for every wave.  The empty asm statements keep the compiler from
// moving memory operations across the barrier.
#define DMA_BARRIER(n)                                   \
  do {                                                   \
    __builtin_amdgcn_s_waitcnt(VMCNT_LGKM0_IMM(n));      \
    asm volatile("" ::: "memory");                       \
    __builtin_amdgcn_s_barrier();                        \
    asm volatile("" ::: "memory");                       \
  } while (0)

// A wave-uniform value of data the kernel only reads, loaded through the constant address
// space: a scalar load, which the compiler waits for with lgkmcnt.  A vector load would be
// waited for with vmcnt, and so behind every direct-to-LDS load in flight.
template <typename T>
SA_DEV T load_uniform(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// LDS atomic max without a returned value, as one instruction the compiler does not order
// against the direct-to-LDS loads in flight (it cannot tell the target from their stages).
// Completion is the caller's: an lgkmcnt(0) wait (DMA_BARRIER has one) before the value is
// read by any wave.
SA_DEV void lds_max_u32(unsigned int* p, unsigned int v) {
  asm volatile("ds_max_u32 %0, %1" : : "v"((unsigned int)(uintptr_t)LDS_PTR(unsigned int, p)), "v"(v));
}

// Order-preserving map of fp32 to uint32 (larger float -> larger unsigned).
SA_DEV unsigned int float_order_key(float f) {
  unsigned int u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// E2M1 magnitude code (OCP Microscaling v1.0 FP4) of y >= 0: the grid 0, 0.5, 1, 1.5, 2, 3, 4, 6
// is codes 0..7, round to nearest with the midpoints 0.25 0.75 1.25 1.75 2.5 3.5 5 going to
// the even code, saturating at 6.
SA_DEV unsigned int e2m1_code(float y) {
  if (y <= 0.25f) return 0u;
  if (y < 0.75f) return 1u;
  if (y <= 1.25f) return 2u;
  if (y < 1.75f) return 3u;
  if (y <= 2.5f) return 4u;
  if (y < 3.5f) return 5u;
  if (y <= 5.0f) return 6u;
  return 7u;
}
