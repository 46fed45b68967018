// topk.hip — deterministic per-query top-k over indexer scores.
//
// Keeps, for each query row, the k visible positions with the largest score
// (CLSA article, "Comment CLSA fonctionne"; IndexCache summary,
// "1. Problématique"), ties to the lower position, output ascending, -1
// padding when fewer than k positions are visible.
//
// Scores become order-preserving 32-bit keys (-0 folded onto +0) and the
// k-th largest key theta is found by radix selection on three digits:
// bits 31..20, 19..8 and 7..0. Three launches:
//   1. topk_hist  (chunks x rows): per-row histogram of the top digit. Each
//      workgroup counts one 4096-element chunk in LDS and adds its non-zero
//      bins to the row histogram with global atomics (integer counts, so the
//      result does not depend on arrival order).
//   2. topk_part  (chunks x rows): every workgroup finds the threshold bin
//      b0 from the row histogram and writes, in position order, the
//      positions of its chunk whose top digit is >= b0 (a superset of the
//      answer, typically k plus one bin's worth) into the chunk's segment of
//      a candidate list, plus the segment's length.
//   3. topk_final (rows): one 1024-thread workgroup per row gathers the
//      candidate segments (in chunk order, hence position order) into LDS,
//      resolves the two low digits by LDS histograms, and emits the k
//      positions with one ordered scan: keys above theta always, keys equal
//      to theta for the first `quota` of them in position order. It then
//      clears the row histogram, leaving the workspace ready for the next
//      call.
// Rows whose visible count is <= k skip the selection: every visible
// position is a candidate and is emitted in order.
#include "kernels.h"

namespace clsa {
namespace {

constexpr int kBins0 = kTopkBins;       // top digit: 12 bits
constexpr int kChunk = kTopkChunk;      // elements per chunk
constexpr int kPartThreads = 256;       // 16 consecutive elements per thread
constexpr int kFinalThreads = 1024;
constexpr int kMaxChunks = kTopkMaxChunks;  // kv_len <= 4M
constexpr int kLdsCap = 12288;          // candidates gathered into LDS

// Finds the bin b (scanning bins from high to low) where the running count
// first reaches `need`; res[0] = b, res[1] = count in bins above b.
// Every thread of the block must call it; need must be in [1, total].
__device__ void find_bin(const uint32_t* h, int nbins, int need, int* res, int* tmp) {
  const int per = (nbins + blockDim.x - 1) / blockDim.x;
  const int hi = nbins - 1 - (int)threadIdx.x * per;
  int sum = 0;
  for (int j = 0; j < per; j++)
    if (hi - j >= 0) sum += h[hi - j];
  int total;
  const int before = block_exclusive_scan(sum, tmp, &total);
  if (before < need && need <= before + sum) {
    int acc = before;
    for (int j = 0; j < per; j++) {
      const int c = h[hi - j];
      if (acc + c >= need) {
        res[0] = hi - j;
        res[1] = acc;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void fill_zero(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// grid (nchunks, rows), block 256.
__global__ __launch_bounds__(kPartThreads) void topk_hist(const float* __restrict__ scores,
                                                          uint32_t* __restrict__ ghist, int T,
                                                          int kv_len) {
  __shared__ uint32_t h[kBins0];
  const int row = blockIdx.y;
  const int vis = kv_len - T + (row % T) + 1;
  const int c0 = blockIdx.x * kChunk;
  if (c0 >= vis) return;
  for (int i = threadIdx.x; i < kBins0; i += blockDim.x) h[i] = 0u;
  __syncthreads();
  const float* sr = scores + (size_t)row * kv_len;
  const int c1 = min(c0 + kChunk, vis);
  for (int s = c0 + threadIdx.x; s < c1; s += blockDim.x) atomicAdd(&h[score_key(sr[s]) >> 20], 1u);
  __syncthreads();
  uint32_t* gh = ghist + (size_t)row * kBins0;
  for (int i = threadIdx.x; i < kBins0; i += blockDim.x)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

// grid (nchunks, rows), block 256.
__global__ __launch_bounds__(kPartThreads) void topk_part(const float* __restrict__ scores,
                                                          const uint32_t* __restrict__ ghist,
                                                          uint32_t* __restrict__ counts,
                                                          int32_t* __restrict__ cand, int T,
                                                          int kv_len, int k, int nchunks) {
  __shared__ uint32_t h[kBins0];
  __shared__ int tmp[17];
  __shared__ int res[2];
  const int row = blockIdx.y;
  const int vis = kv_len - T + (row % T) + 1;
  const int c0 = blockIdx.x * kChunk;
  if (c0 >= vis) {
    if (threadIdx.x == 0) counts[(size_t)row * nchunks + blockIdx.x] = 0u;
    return;
  }
  uint32_t b0 = 0;  // every visible element qualifies when vis <= k
  if (vis > k) {
    const uint32_t* gh = ghist + (size_t)row * kBins0;
    for (int i = threadIdx.x; i < kBins0; i += blockDim.x) h[i] = gh[i];
    __syncthreads();
    find_bin(h, kBins0, k, res, tmp);
    b0 = (uint32_t)res[0];
  }
  const float* sr = scores + (size_t)row * kv_len;
  const int e0 = c0 + threadIdx.x * 16;
  uint32_t flags = 0;
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < 16; j++) {
    const int s = e0 + j;
    if (s < vis && (score_key(sr[s]) >> 20) >= b0) {
      flags |= 1u << j;
      cnt++;
    }
  }
  int total;
  int off = block_exclusive_scan(cnt, tmp, &total);
  int32_t* seg = cand + ((size_t)row * nchunks + blockIdx.x) * kChunk;
#pragma unroll
  for (int j = 0; j < 16; j++)
    if (flags >> j & 1u) seg[off++] = e0 + j;
  if (threadIdx.x == 0) counts[(size_t)row * nchunks + blockIdx.x] = (uint32_t)total;
}

// Candidate accessors for topk_final: LDS copy, or the segmented global list.
struct LdsCand {
  const int32_t* pos;
  const uint32_t* key;
  __device__ int p(int i) const { return pos[i]; }
  __device__ uint32_t k(int i) const { return key[i]; }
};
struct GlobalCand {
  const int32_t* seg;     // row's segments, kChunk entries each
  const int* chunk_off;   // LDS, nchunks + 1 exclusive offsets
  int nchunks;
  const float* srow;
  __device__ int p(int i) const {
    int lo = 0, hi = nchunks;  // largest c with chunk_off[c] <= i
    while (hi - lo > 1) {
      const int mid = (lo + hi) / 2;
      if (chunk_off[mid] <= i) lo = mid; else hi = mid;
    }
    return seg[(size_t)lo * kChunk + (i - chunk_off[lo])];
  }
  __device__ uint32_t k(int i) const { return score_key(srow[p(i)]); }
};

// Resolves theta among the candidates and emits the row's selection.
template <class Acc>
__device__ void select_and_emit(const Acc& acc, int n, int need0, uint32_t b0, uint32_t* h,
                                int* res, int* tmp, int32_t* out) {
  // Digit 1 (bits 19..8) among candidates whose top digit is b0.
  for (int i = threadIdx.x; i < kBins0; i += blockDim.x) h[i] = 0u;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const uint32_t key = acc.k(i);
    if ((key >> 20) == b0) atomicAdd(&h[(key >> 8) & 0xfffu], 1u);
  }
  __syncthreads();
  find_bin(h, kBins0, need0, res, tmp);
  const uint32_t b1 = (uint32_t)res[0];
  const int need1 = need0 - res[1];
  const uint32_t pre = (b0 << 12) | b1;
  // Digit 2 (bits 7..0) among candidates matching the top 24 bits.
  for (int i = threadIdx.x; i < 256; i += blockDim.x) h[i] = 0u;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const uint32_t key = acc.k(i);
    if ((key >> 8) == pre) atomicAdd(&h[key & 0xffu], 1u);
  }
  __syncthreads();
  find_bin(h, 256, need1, res, tmp);
  const uint32_t theta = (pre << 8) | (uint32_t)res[0];
  const int quota = need1 - res[1];  // how many keys equal to theta are taken
  // Ordered emission: 4 consecutive candidates per thread per tile.
  int gt_base = 0, eq_base = 0;
  for (int t0 = 0; t0 < n; t0 += 4 * blockDim.x) {
    const int i0 = t0 + threadIdx.x * 4;
    int gt = 0, eq = 0;
    for (int e = 0; e < 4; e++) {
      if (i0 + e < n) {
        const uint32_t key = acc.k(i0 + e);
        gt += key > theta;
        eq += key == theta;
      }
    }
    int tot;
    const int pre_cnt = block_exclusive_scan((eq << 16) | gt, tmp, &tot);
    int g = gt_base + (pre_cnt & 0xffff);
    int q = eq_base + (pre_cnt >> 16);
    for (int e = 0; e < 4; e++) {
      if (i0 + e < n) {
        const uint32_t key = acc.k(i0 + e);
        if (key > theta) {
          out[g + min(q, quota)] = acc.p(i0 + e);
          g++;
        } else if (key == theta) {
          if (q < quota) out[g + q] = acc.p(i0 + e);
          q++;
        }
      }
    }
    gt_base += tot & 0xffff;
    eq_base += tot >> 16;
  }
}

// grid (rows), block 1024.
__global__ __launch_bounds__(kFinalThreads) void topk_final(const float* __restrict__ scores,
                                                            uint32_t* __restrict__ ghist,
                                                            const uint32_t* __restrict__ counts,
                                                            const int32_t* __restrict__ cand,
                                                            int32_t* __restrict__ idx, int T,
                                                            int kv_len, int k, int nchunks) {
  __shared__ uint32_t h[kBins0];
  __shared__ int chunk_off[kMaxChunks + 1];
  __shared__ int32_t lpos[kLdsCap];
  __shared__ uint32_t lkey[kLdsCap];
  __shared__ int tmp[17];
  __shared__ int res[2];
  const int row = blockIdx.x;
  const int vis = kv_len - T + (row % T) + 1;
  const float* srow = scores + (size_t)row * kv_len;
  uint32_t* gh = ghist + (size_t)row * kBins0;
  int32_t* out = idx + (size_t)row * k;

  // Offsets of the candidate segments (chunk order = position order).
  int total;
  {
    const int c = threadIdx.x;
    const int v = c < nchunks ? (int)counts[(size_t)row * nchunks + c] : 0;
    const int off = block_exclusive_scan(v, tmp, &total);
    if (c < nchunks) chunk_off[c] = off;
    if (c == 0) chunk_off[nchunks] = total;
  }
  __syncthreads();
  const int n = total;
  GlobalCand gacc{cand + (size_t)row * nchunks * kChunk, chunk_off, nchunks, srow};

  if (vis <= k) {
    // Every visible position is selected, in order.
    for (int i = threadIdx.x; i < k; i += blockDim.x) out[i] = i < n ? gacc.p(i) : -1;
  } else {
    for (int i = threadIdx.x; i < kBins0; i += blockDim.x) h[i] = gh[i];
    __syncthreads();
    find_bin(h, kBins0, k, res, tmp);
    const uint32_t b0 = (uint32_t)res[0];
    const int need0 = k - res[1];
    if (n <= kLdsCap) {
      for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int p = gacc.p(i);
        lpos[i] = p;
        lkey[i] = score_key(srow[p]);
      }
      __syncthreads();
      select_and_emit(LdsCand{lpos, lkey}, n, need0, b0, h, res, tmp, out);
    } else {
      select_and_emit(gacc, n, need0, b0, h, res, tmp, out);
    }
  }
  // Leave the row histogram cleared for the next call.
  for (int i = threadIdx.x; i < kBins0; i += blockDim.x) gh[i] = 0u;
}

}  // namespace

int zero_words(uint32_t* p, size_t n, hipStream_t stream) {
  if (n == 0) return CLSA_OK;
  size_t blocks = (n + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(fill_zero, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return check_launch("fill_zero");
}

int launch_topk(const float* scores, int B, int T, int kv_len, int k, int32_t* idx,
                uint32_t* hist, uint32_t* counts, int32_t* cand, hipStream_t stream) {
  const int rows = B * T;
  const int nchunks = topk_nchunks(kv_len);
  if (nchunks > kMaxChunks)
    return set_error(CLSA_ERR_UNSUPPORTED, "topk: kv_len=%d above %d", kv_len, kMaxChunks * kChunk);
  int rc;
  hipLaunchKernelGGL(topk_hist, dim3(nchunks, rows), dim3(kPartThreads), 0, stream, scores, hist,
                     T, kv_len);
  if ((rc = check_launch("topk_hist"))) return rc;
  hipLaunchKernelGGL(topk_part, dim3(nchunks, rows), dim3(kPartThreads), 0, stream, scores, hist,
                     counts, cand, T, kv_len, k, nchunks);
  if ((rc = check_launch("topk_part"))) return rc;
  hipLaunchKernelGGL(topk_final, dim3(rows), dim3(kFinalThreads), 0, stream, scores, hist, counts,
                     cand, idx, T, kv_len, k, nchunks);
  return check_launch("topk_final");
}

}  // namespace clsa
