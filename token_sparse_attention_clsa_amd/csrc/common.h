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

// Inclusive scan of an int over the 64 lanes of a wave with DPP moves: row_shr
// 1, 2, 4, 8 scan each row of 16 lanes (a lane whose source lies outside its
// row adds 0), then row_bcast 15 adds row 0's total into row 1 and row 2's
// into row 3, and row_bcast 31 adds lane 31's running total into rows 2
// and 3 (rows outside the row mask keep their value).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Exclusive scan of one int per thread over the whole block of NT threads
// (the launch's block size: a multiple of 64, at most 1024; a compile-time
// constant, since reading blockDim.x costs a load from the dispatch's hidden
// arguments). `tmp` is __shared__ int[16 + 1] (the first NT / 64 entries are
// used). Returns the thread's exclusive prefix; *total receives the block
// total. Contains barriers: every thread of the block must call it, with the
// whole wave active.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp, int* total) {
  static_assert(NT % kWave == 0 && NT <= 1024, "block size");
  const int lane = lane_id();
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  constexpr int nw = NT / kWave;
  const int inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) tmp[wid] = inc;
  __syncthreads();
  // Every wave scans the wave totals itself, so no second publishing step.
  const int x = lane < nw ? tmp[lane] : 0;
  const int xi = wave_inclusive_scan(x);
  const int before = __builtin_amdgcn_readlane(xi - x, wid);
  *total = __builtin_amdgcn_readlane(xi, nw - 1);
  __syncthreads();  // the totals are read before tmp can be rewritten
  return before + inc - v;
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
