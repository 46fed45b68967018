// common.h — helpers shared by the gfx950 kernels of libclsa.
//
// Wave64 primitives, bfloat16 handling and the order-preserving float key
// used by the radix top-k. Everything here is device code or launch
// plumbing; the C ABI lives in api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "clsa.h"

namespace clsa {

constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// ---------------------------------------------------------------------------
// bfloat16
// ---------------------------------------------------------------------------

// bf16 pair in one dword -> two floats (low half is the first element).
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// ---------------------------------------------------------------------------
// Order-preserving key of a float score: larger float <=> larger key, and
// -0.0 maps to the same key as +0.0.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// Wave64 reductions and scans (lane = threadIdx.x % 64)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return __lane_id(); }

template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    T n = __shfl_up(v, off, kWave);
    if (lane >= off) v += n;
  }
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Exclusive scan of one int per thread over the whole block (blockDim.x a
// multiple of 64, at most 1024). `tmp` is __shared__ int[16 + 1]. Returns the
// thread's exclusive prefix; *total receives the block total. Contains
// barriers: every thread of the block must call it.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = lane_id();
  const int wid = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  int inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) tmp[wid] = inc;
  __syncthreads();
  if (wid == 0) {
    int x = lane < nw ? tmp[lane] : 0;
    int xi = wave_inclusive_scan(x);
    if (lane < nw) tmp[lane] = xi - x;
    if (lane == nw - 1) tmp[16] = xi;
  }
  __syncthreads();
  int res = tmp[wid] + inc - v;
  *total = tmp[16];
  __syncthreads();
  return res;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

// Thread-local error message setter (defined in api.cpp).
int set_error(int status, const char* fmt, ...);

inline int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(CLSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return CLSA_OK;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Zero n 32-bit words on `stream` with a kernel (kept as a kernel so the
// sequence stays capturable in a HIP graph).
int zero_words(uint32_t* p, size_t n, hipStream_t stream);

}  // namespace clsa
