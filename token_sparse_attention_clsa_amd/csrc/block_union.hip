// block_union.hip — block-union KV tables for the chunked-prefill comparator.
//
// CompactAttention summary, "Méthodologie", selection step: for a chunk of
// queries, the KV blocks selected by any query block (and any head of a KV
// group) are merged into one minimal, coverage-preserving table per
// (batch, KV group), handed to a dense paged kernel as kv_indptr /
// kv_indices. Here the per-query selections are the token index rows, so a
// block is selected when one of the chunk's queries picked a visible
// position inside it; one index serves every head, so every KV group of a
// batch element gets the same table.
//
// Two launches: mark (one thread per index entry sets its block's flag) and
// compact (one workgroup writes, per batch element, the flagged block ids in
// ascending order, once per KV group, and the offsets).
#include "kernels.h"

namespace clsa {

int launch_block_attn_mfma(const void* q, const void* kc, const void* vc,
                           const int32_t* kv_indptr, const int32_t* kv_indices, int block,
                           void* out, float* lse, int B, int T, int Hq, int Hkv, int D, int kv_len,
                           int L_cap, float scale, bool head_major, hipStream_t stream);

namespace {

constexpr int kCompactThreads = 1024;

__global__ __launch_bounds__(256) void union_mark(const int32_t* __restrict__ idx,
                                                  uint32_t* __restrict__ flags, int B, int T,
                                                  int k, int kv_len, int block, int nblk) {
  const size_t n = (size_t)B * T * k;
  for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n;
       e += (size_t)gridDim.x * blockDim.x) {
    const int b = (int)(e / ((size_t)T * k));
    const int t = (int)((e / k) % T);
    const int s = idx[e];
    const int vis = kv_len - T + t + 1;
    if (s >= 0 && s < vis) flags[(size_t)b * nblk + s / block] = 1u;
  }
}

__global__ __launch_bounds__(kCompactThreads) void union_compact(const uint32_t* __restrict__ flags,
                                                                 int32_t* __restrict__ indptr,
                                                                 int32_t* __restrict__ indices,
                                                                 int B, int Hkv, int nblk) {
  __shared__ int tmp[17];
  int base = 0;
  for (int b = 0; b < B; b++) {
    const uint32_t* f = flags + (size_t)b * nblk;
    // Pass 1: number of flagged blocks of this batch element.
    int cnt = 0;
    for (int i = threadIdx.x; i < nblk; i += kCompactThreads) cnt += f[i] != 0u;
    int nb;
    block_exclusive_scan<kCompactThreads>(cnt, tmp, &nb);
    // Pass 2: ordered write, once per KV group.
    int run = 0;
    for (int t0 = 0; t0 < nblk; t0 += kCompactThreads) {
      const int i = t0 + threadIdx.x;
      const int flag = (i < nblk && f[i] != 0u) ? 1 : 0;
      int tot;
      const int off = run + block_exclusive_scan<kCompactThreads>(flag, tmp, &tot);
      if (flag)
        for (int g = 0; g < Hkv; g++) indices[base + g * nb + off] = i;
      run += tot;
    }
    if ((int)threadIdx.x < Hkv) indptr[b * Hkv + threadIdx.x] = base + (int)threadIdx.x * nb;
    base += Hkv * nb;
  }
  if (threadIdx.x == 0) indptr[B * Hkv] = base;
}

}  // namespace

size_t block_union_ws_bytes(int B, int kv_len, int block) {
  const size_t nblk = ((size_t)kv_len + block - 1) / block;
  return align_up((size_t)B * nblk * 4, 256);
}

int launch_block_union(const int32_t* idx, int B, int T, int k, int kv_len, int block, int Hkv,
                       int32_t* kv_indptr, int32_t* kv_indices, void* ws, hipStream_t stream) {
  const int nblk = (kv_len + block - 1) / block;
  uint32_t* flags = static_cast<uint32_t*>(ws);
  int rc;
  if ((rc = zero_words(flags, (size_t)B * nblk, stream))) return rc;
  const size_t n = (size_t)B * T * k;
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(union_mark, dim3((unsigned)blocks), dim3(256), 0, stream, idx, flags, B, T, k,
                     kv_len, block, nblk);
  if ((rc = check_launch("union_mark"))) return rc;
  hipLaunchKernelGGL(union_compact, dim3(1), dim3(kCompactThreads), 0, stream, flags, kv_indptr,
                     kv_indices, B, Hkv, nblk);
  return check_launch("union_compact");
}

bool block_paged_attn_supported(int dtype, int Hq, int Hkv, int D, int block) {
  return dtype == CLSA_BF16 && D == 128 && block >= 1 && Hkv >= 1 && Hq % Hkv == 0 &&
         (Hq / Hkv == 1 || Hq / Hkv == 2 || Hq / Hkv == 4 || Hq / Hkv == 8);
}

int launch_block_paged_attn(const void* q, const void* kc, const void* vc, int dtype,
                            const int32_t* kv_indptr, const int32_t* kv_indices, int block,
                            void* out, float* lse, int B, int T, int Hq, int Hkv, int D,
                            int kv_len, int L_cap, float scale, bool head_major,
                            hipStream_t stream) {
  (void)dtype;  // bf16 only (checked by the caller)
  return launch_block_attn_mfma(q, kc, vc, kv_indptr, kv_indices, block, out, lse, B, T, Hq, Hkv, D,
                                kv_len, L_cap, scale, head_major, stream);
}

}  // namespace clsa
