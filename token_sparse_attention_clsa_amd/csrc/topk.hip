// topk.hip — deterministic per-query top-k over indexer scores.
//
// Keeps, for each query row, the k visible positions with the largest score
// (CLSA article, "Comment CLSA fonctionne"; IndexCache summary,
// "1. Problématique"), ties to the lower position, output ascending, -1
// padding when fewer than k positions are visible.
//
// Scores become order-preserving 32-bit keys (-0 folded onto +0); selection
// is radix selection on digits of at most 12 bits. Short rows take one
// launch (topk_lds, below: the row is read into LDS once); longer rows two:
//   1. topk_filter (chunks x rows, 256 threads): every workgroup of a row
//      takes the same deterministic sample of the row (128 runs of 16
//      consecutive elements, evenly spaced, so the sample costs 128 cache
//      lines rather than 2048), histograms the sample's keys over their own
//      range in LDS and picks the bin where the sample's count from the top
//      reaches about twice the rank k would have in the sample; the bin's
//      lower bound is the threshold key. It then writes, in position order,
//      the (position, key) pairs of its 4096-element chunk at or above the
//      threshold (at most kTopkSegCap of them) and their count. With a
//      2048-element sample the chance that this keeps fewer than k
//      positions, or more than the cap in a chunk, is negligible for any
//      smooth score distribution, and the next kernel checks both anyway.
//   2. topk_select (rows, 1024 threads): gathers the candidate segments (in
//      chunk order, hence position order) into LDS and resolves the k-th key
//      theta exactly with LDS histograms over the candidates' own key range
//      (key - min, 12 bits per pass; a last bin of at most 64 keys is ranked
//      by one wave), then emits, in one ordered scan, keys above theta and
//      the first `quota` keys equal to theta. If the candidates number fewer
//      than k or a chunk overflowed its segment, it redoes the row on its own
//      (LDS histogram of the full row's top 12 bits, ordered candidate pass),
//      so the result is exact whatever the sample did.
// Few long rows (decode) take both steps in one launch (topk_fused, below),
// where the filter also builds each row's candidate histogram and the row's
// last workgroup selects.
// Rows whose visible count is <= k take every visible position. With a
// per-row count k_rows[row] (clamped to [0, k]), a row keeps its k_rows[row]
// best positions and the rest of its k slots hold -1.
// Ordered skipping (CoSA summary, the paragraphs on its proxy and its
// kernel): with a finite margin, the selection read in priority order (score
// descending, position ascending) stops at the first entry whose score is
// below thr = (row maximum) - margin, thr formed in float32. The kept
// entries are exactly the selected keys >= key(thr): when key(thr) is above
// theta, theta becomes key(thr) and every key equal to it is taken; the rest
// of the row is -1.
#include <climits>
#include <mutex>
#include <stdlib.h>

#include "kernels.h"

namespace clsa {
namespace {

constexpr int kBins0 = kTopkBins;  // bins of a 12-bit digit
constexpr int kThreads = 1024;     // topk_select
constexpr int kWaves = kThreads / kWave;
constexpr int kFilterThreads = 256;
constexpr int kChunk = kTopkChunk; // topk_filter: 16 consecutive elements per thread
constexpr int kSample = 2048;      // sample for the threshold estimate
constexpr int kSampleRun = 16;     // ... taken as kSample / kSampleRun evenly spaced runs
constexpr int kTile = 16384;       // fallback tile: 16 waves x 1024 consecutive elements
constexpr int kLdsCap = 12288;     // candidates kept in LDS
constexpr int kHistCopies = 2;     // fallback histogram copies
constexpr int kLdsRow = 16384;     // rows up to this length: one launch, row in LDS
constexpr int kArrStride = 32 + kTopkBins;  // topk_fused: u32 words per row (arrival word, row histogram)
static_assert(kThreads * 4 == kBins0, "the selection holds the row histogram as 4 bins per thread");
constexpr int kFusedMaxRows = 64;    // topk_fused: at most this many rows ...
constexpr int kFusedMaxChunks = 64;  // ... of at most this many 4096-element chunks

// Finds the bin b (scanning bins from high to low) where the running count
// first reaches `need`; res[0] = b, res[1] = count in bins above b. Thread t
// takes the `per` consecutive bins below nbins - per * t (consecutive
// threads, consecutive bins: no LDS bank conflicts); a wave scan, the wave
// totals through tmp and one barrier give each thread the count above its
// bins, and the thread where `need` falls walks them; res[2] = the count in
// bin b. Every thread of the block must call it; need must be in [1, total];
// tmp is int[16]; NT = the block size.
template <int NT>
__device__ __forceinline__ void find_bin(const uint32_t* h, int nbins, int need, int* res, int* tmp) {
  const int per = (nbins + NT - 1) / NT;
  const int hi = nbins - 1 - (int)threadIdx.x * per;
  int sum = 0;
  for (int j = 0; j < per; j++)
    if (hi - j >= 0) sum += h[hi - j];
  const int lane = threadIdx.x % kWave;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  constexpr int nw = NT / kWave;
  const int inc = wave_inclusive_scan(sum);
  if (lane == kWave - 1) tmp[wid] = inc;
  __syncthreads();
  const int x = lane < nw ? tmp[lane] : 0;
  const int before = __builtin_amdgcn_readlane(wave_inclusive_scan(x) - x, wid) + inc - sum;
  if (before < need && need <= before + sum) {
    int acc = before;
    for (int j = 0; j < per && hi - j >= 0; j++) {
      const int c = h[hi - j];
      if (acc + c >= need) {
        res[0] = hi - j;
        res[1] = acc;
        res[2] = c;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x111, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x112, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x114, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x118, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x142, 0xa, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, kWave - 1);
}

__global__ __launch_bounds__(256) void fill_zero(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// The score whose key is `key` (inverse of score_key; -0 comes back as +0).
__device__ __forceinline__ float key_score(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}
// Key of the ordered-skipping threshold (row maximum key mx) - margin, or 0
// (every key passes) when the margin is +inf or the threshold is NaN.
__device__ __forceinline__ uint32_t margin_key(uint32_t mx, float margin) {
  if (!(margin < INFINITY)) return 0u;
  const float thr = key_score(mx) - margin;
  return thr == thr ? score_key(thr) : 0u;
}

// Candidates: the first kLdsCap in LDS, the rest in the workspace (their
// keys are read back from the scores).
struct Cand {
  const int32_t* lpos;
  const uint32_t* lkey;
  const int32_t* gpos;
  const float* srow;
  __device__ int p(int i) const { return i < kLdsCap ? lpos[i] : gpos[i]; }
  __device__ uint32_t k(int i) const { return i < kLdsCap ? lkey[i] : score_key(srow[gpos[i]]); }
};

// Candidates still in the filter's chunk segments: candidate i lives in the
// chunk c with off[c] <= i < off[c + 1].
struct SegCand {
  const int2* seg;  // the row's segments, kTopkSegCap (position, key) pairs each
  const int* off;   // LDS, nchunks + 1 exclusive offsets
  int nchunks;
  __device__ int2 e(int i) const {
    int lo = 0, hi = nchunks;
    while (hi - lo > 1) {
      const int mid = (lo + hi) / 2;
      if (off[mid] <= i) lo = mid; else hi = mid;
    }
    return seg[(size_t)lo * kTopkSegCap + (i - off[lo])];
  }
  __device__ int p(int i) const { return e(i).x; }
  __device__ uint32_t k(int i) const { return (uint32_t)e(i).y; }
};

// One wave ranks the cnt <= 64 keys in few[] (keys strictly above and
// equal to each): res[0] = the need-th largest (theta), res[1] = how many
// keys equal to theta are still to take. Every thread calls it; the first
// wave works. need must be in [1, cnt].
__device__ __forceinline__ void rank_few(const uint32_t* few, int cnt, int need, int* res) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const uint32_t v = lane < cnt ? few[lane] : 0u;
    int gt = 0, eq = 0;
    for (int j = 0; j < cnt; j++) {  // uniform
      const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)v, j);
      gt += o > v;
      eq += o == v;
    }
    const unsigned long long hit = __ballot(lane < cnt && gt < need && need <= gt + eq);
    if (lane == __builtin_ctzll(hit)) {
      res[0] = (int)v;     // theta
      res[1] = need - gt;  // keys equal to theta still to take
    }
  }
}

template <class Acc>
__device__ void emit_selection(const Acc& acc, int n, uint32_t theta, int quota, int* tmp, int32_t* out,
                               int k, int32_t* kept);

// Resolves theta, the need-th largest key among the candidates, all of
// which in play lie in [lo, lo + R) (R a power of two <= 2^32), by radix
// passes of at most 12 bits on key - lo, then emits the row's selection:
// its k best keys, or with mkey above theta (ordered skipping) only the keys
// >= mkey, the rest of the k slots -1. kept (or NULL) receives the count.
template <class Acc>
__device__ void select_and_emit(const Acc& acc, int n, int need, uint32_t lo, uint64_t R,
                                uint32_t* h, int* res, int* tmp, int32_t* out, int k,
                                uint32_t mkey, int32_t* kept) {
  __shared__ uint32_t few[kWave];
  __shared__ int nfew;
  while (R > 1) {  // uniform over the workgroup
    const int bits = 63 - __clzll(R);
    const int s = bits > 12 ? bits - 12 : 0;
    const int nb = (int)(R >> s);
    for (int i = threadIdx.x; i < nb; i += kThreads) h[i] = 0u;
    if (threadIdx.x == 0) nfew = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kThreads) {
      const uint32_t key = acc.k(i);
      if (key >= lo && (uint64_t)(key - lo) < R) atomicAdd(&h[(key - lo) >> s], 1u);
    }
    __syncthreads();
    find_bin<kThreads>(h, nb, need, res, tmp);
    // Every thread reads res here, before the next pass's first barrier;
    // it is rewritten only after that pass's third one.
    lo += (uint32_t)res[0] << s;
    need -= res[1];
    R = 1ull << s;
    if (R > 1 && res[2] <= kWave) {
      // At most 64 keys left in [lo, lo + R): one wave ranks them (keys
      // strictly above and equal to each) instead of further passes.
      const int cnt = res[2];
      for (int i = threadIdx.x; i < n; i += kThreads) {
        const uint32_t key = acc.k(i);
        if (key >= lo && (uint64_t)(key - lo) < R) few[atomicAdd(&nfew, 1)] = key;
      }
      __syncthreads();
      rank_few(few, cnt, need, res);
      __syncthreads();
      lo = (uint32_t)res[0];
      need = res[1];
      R = 1;
    }
  }
  uint32_t theta = lo;
  int quota = need;  // how many keys equal to theta are taken
  if (mkey > theta) {  // uniform: reading stops before theta
    theta = mkey;
    quota = INT_MAX;
  }
  emit_selection(acc, n, theta, quota, tmp, out, k, kept);
}

// Ordered emission of a row's selection: keys above theta always, keys equal
// to theta for the first `quota` of them in candidate (position) order; the
// slots past the kept count hold -1 and kept (or NULL) receives the count.
// Thread t owns the run [t0 + t * run, t0 + (t + 1) * run) of the tile
// (run <= 16), so up to 16 * kThreads candidates take one block scan and no
// barrier waits behind the output stores.
template <class Acc>
__device__ void emit_selection(const Acc& acc, int n, uint32_t theta, int quota, int* tmp, int32_t* out,
                               int k, int32_t* kept) {
  const int run = min(16, max(1, (n + kThreads - 1) / kThreads));
  int gt_base = 0, eq_base = 0;
  for (int t0 = 0; t0 < n; t0 += run * kThreads) {  // uniform over the workgroup
    const int i0 = t0 + threadIdx.x * run;
    int gt = 0, eq = 0;
    for (int e = 0; e < run; e++) {
      if (i0 + e < n) {
        const uint32_t key = acc.k(i0 + e);
        gt += key > theta;
        eq += key == theta;
      }
    }
    int tot;  // per tile both counts stay below 2^16
    const int pre_cnt = block_exclusive_scan<kThreads>((eq << 16) | gt, tmp, &tot);
    int g = gt_base + (pre_cnt & 0xffff);
    int q = eq_base + (pre_cnt >> 16);
    for (int e = 0; e < run; e++) {
      if (i0 + e < n) {
        const uint32_t key = acc.k(i0 + e);
        if (key > theta) {
          const int o = g + min(q, quota);
          if (o < k) out[o] = acc.p(i0 + e);
          g++;
        } else if (key == theta) {
          if (q < quota && g + q < k) out[g + q] = acc.p(i0 + e);
          q++;
        }
      }
    }
    gt_base += tot & 0xffff;
    eq_base += tot >> 16;
  }
  const int nk = min(k, gt_base + min(eq_base, quota));  // k unless mkey cut the row
  for (int i = nk + threadIdx.x; i < k; i += kThreads) out[i] = -1;
  if (kept && threadIdx.x == 0) *kept = nk;
}

// Selection of the k largest among n >= k candidates whose keys lie in
// [mn, mx]. The radix passes run on key - mn over the candidates' own key
// range, so the first pass spreads them over its bins even when they share
// the top bits of their keys; a range of at most 2^24 keys takes two passes,
// or one when the bin it leaves holds at most 64 keys.
template <class Acc>
__device__ void select_top(const Acc& acc, int n, int k, uint32_t mn, uint32_t mx, uint32_t* h,
                           int* res, int* tmp, int32_t* out, uint32_t mkey, int32_t* kept) {
  const uint64_t span = (uint64_t)(mx - mn) + 1;  // n >= k >= 1, so mx >= mn
  const uint64_t R = span == 1 ? 1 : 1ull << (64 - __clzll(span - 1));
  select_and_emit(acc, n, k, mn, R, h, res, tmp, out, k, mkey, kept);
}

// Block-wide min and max of the threads' (mn, mx); ends with a barrier
// (the writes before it, e.g. an LDS gather, are visible after it).
__device__ __forceinline__ void block_minmax(uint32_t& mn, uint32_t& mx, uint32_t (*mm)[kWaves]) {
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  const int wave = threadIdx.x / kWave;
  constexpr int nw = kWaves;
  if (threadIdx.x % kWave == 0) {
    mm[0][wave] = mn;
    mm[1][wave] = mx;
  }
  __syncthreads();
  for (int w = 0; w < nw; w++) {
    mn = min(mn, mm[0][w]);
    mx = max(mx, mm[1][w]);
  }
}

template <bool VEC>
__device__ __forceinline__ void load4(const float* srow, int e, int vis, float* x) {
  if (VEC && e + 3 < vis) {
    const float4 v = *reinterpret_cast<const float4*>(srow + e);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  } else {
#pragma unroll
    for (int j = 0; j < 4; j++) x[j] = e + j < vis ? srow[e + j] : 0.f;
  }
}

// Pass 1 and pass 2 over one row (see the file comment).
template <bool VEC>
__device__ int histogram_and_candidates(const float* srow, int vis, int k, uint32_t* h,
                                        int32_t* lpos, uint32_t* lkey, int32_t* gpos,
                                        int* wtot, int* tmp, int* res, uint32_t* b0_out,
                                        int* above_out) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  // kHistCopies histograms side by side (scores cluster in a few bins; spreading
  // the waves over copies cuts same-address atomic serialisation), summed into h.
  uint32_t* hc = h + kBins0 * (1 + wave % kHistCopies);
  for (int i = threadIdx.x; i < kBins0 * (1 + kHistCopies); i += kThreads) h[i] = 0u;
  __syncthreads();
  constexpr int kBatch = 8;  // float4 loads in flight per thread
  for (int e0 = 4 * threadIdx.x; e0 < vis; e0 += 4 * kThreads * kBatch) {
    float x[kBatch][4];
#pragma unroll
    for (int u = 0; u < kBatch; u++) load4<VEC>(srow, e0 + u * 4 * kThreads, vis, x[u]);
#pragma unroll
    for (int u = 0; u < kBatch; u++)
#pragma unroll
      for (int j = 0; j < 4; j++)
        if (e0 + u * 4 * kThreads + j < vis) atomicAdd(&hc[score_key(x[u][j]) >> 20], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kBins0; i += kThreads) {
    uint32_t c = 0;
#pragma unroll
    for (int r = 1; r <= kHistCopies; r++) c += h[kBins0 * r + i];
    h[i] = c;
  }
  __syncthreads();
  find_bin<kThreads>(h, kBins0, k, res, tmp);
  const uint32_t b0 = (uint32_t)res[0];
  *b0_out = b0;
  *above_out = res[1];

  int total = 0;
  for (int t0 = 0; t0 < vis; t0 += kTile) {  // uniform over the workgroup
    // wave w owns [seg, seg + 1024) in 4 steps of 256; lane l owns 4 consecutive elements per step
    const int seg = t0 + wave * 1024;
    uint32_t flags[4];
    uint32_t keys[4][4];
    int step_off[4], step_tot[4];
    int wave_total = 0;
    float xs[4][4];
#pragma unroll
    for (int st = 0; st < 4; st++) load4<VEC>(srow, seg + st * 256 + 4 * lane, vis, xs[st]);
#pragma unroll
    for (int st = 0; st < 4; st++) {
      const int e = seg + st * 256 + 4 * lane;
      const float* x = xs[st];
      flags[st] = 0;
      int c = 0;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        keys[st][j] = score_key(x[j]);
        if (e + j < vis && (keys[st][j] >> 20) >= b0) {
          flags[st] |= 1u << j;
          c++;
        }
      }
      const int inc = wave_inclusive_scan(c);
      step_off[st] = wave_total + inc - c;
      step_tot[st] = __shfl(inc, kWave - 1, kWave);
      wave_total += step_tot[st];
    }
    if (lane == 0) wtot[wave] = wave_total;
    __syncthreads();
    if (wave == 0) {
      const int v = lane < kWaves ? wtot[lane] : 0;
      const int inc = wave_inclusive_scan(v);
      if (lane < kWaves) wtot[lane] = inc - v;  // exclusive base of each wave
      if (lane == kWaves - 1) wtot[kWaves] = inc;
    }
    __syncthreads();
    const int base = total + wtot[wave];
#pragma unroll
    for (int st = 0; st < 4; st++) {
      int o = base + step_off[st];
      const int e = seg + st * 256 + 4 * lane;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        if (flags[st] >> j & 1u) {
          if (o < kLdsCap) {
            lpos[o] = e + j;
            lkey[o] = keys[st][j];
          } else {
            gpos[o] = e + j;
          }
          o++;
        }
      }
    }
    total += wtot[kWaves];
    __syncthreads();  // wtot is rewritten by the next tile
  }
  return total;
}

// This thread's 16 consecutive elements of the chunk at c0 as keys (0 past vis).
__device__ __forceinline__ void load_chunk_keys(const float* srow, int c0, int vis, uint32_t (&key)[16]) {
  const int e0 = c0 + threadIdx.x * 16;
  if (e0 + 15 < vis && (reinterpret_cast<uintptr_t>(srow + e0) & 15) == 0) {
    const float4* p4 = reinterpret_cast<const float4*>(srow + e0);
    float4 v[4] = {p4[0], p4[1], p4[2], p4[3]};
    const float* x = reinterpret_cast<const float*>(v);
#pragma unroll
    for (int j = 0; j < 16; j++) key[j] = score_key(x[j]);
  } else {
#pragma unroll
    for (int j = 0; j < 16; j++) key[j] = e0 + j < vis ? score_key(srow[e0 + j]) : 0u;
  }
}

// grid (ceil(nchunks / cpw), rows), block 256: a workgroup takes cpw
// consecutive chunks of its row (one threshold for all of them).
__global__ __launch_bounds__(kFilterThreads) void topk_filter(const float* __restrict__ scores,
                                                              uint32_t* __restrict__ counts,
                                                              int2* __restrict__ cand, int T,
                                                              int kv_len, int k,
                                                              const int32_t* __restrict__ k_rows,
                                                              int nchunks, int cstride, int cpw) {
  __shared__ __attribute__((aligned(16))) uint32_t h[kBins0];
  __shared__ int tmp[17];
  __shared__ int res[3];
  __shared__ uint32_t fmm[2][kFilterThreads / kWave];
  const int row = blockIdx.y;
  const int vis = kv_len - T + (row % T) + 1;
  const int ci0 = blockIdx.x * cpw, ci1 = min(nchunks, ci0 + cpw);
  uint32_t* cnt = counts + (size_t)row * cstride;
  if (k_rows) k = min(max(k_rows[row], 0), k);
  if (vis <= k || ci0 * kChunk >= vis || k == 0) {
    for (int ci = ci0 + threadIdx.x; ci < ci1; ci += kFilterThreads) cnt[ci] = 0u;
    return;
  }
  const float* srow = scores + (size_t)row * kv_len;
  // The first chunk's elements are loaded first, so that their memory
  // latency overlaps the sample's.
  uint32_t key[16];
  load_chunk_keys(srow, ci0 * kChunk, vis, key);
  // Threshold from the row's sample (identical in every workgroup): the
  // whole row when it is short, else kSample / kSampleRun runs of kSampleRun
  // consecutive elements, the first at 0 and the last ending at vis - 1. The
  // sample's keys are binned over their own range (key - min, at most 4096
  // bins), so the threshold stays close to the target rank however narrow
  // the score distribution is.
  const int m = min(kSample, vis);
  constexpr int kRuns = kSample / kSampleRun;
  constexpr int kPer = kSample / kFilterThreads;  // sample elements per thread, all loaded at once
  float sv[kPer];
#pragma unroll
  for (int j = 0; j < kPer; j++) {
    const int i = threadIdx.x + j * kFilterThreads;
    const int pos = vis <= kSample
                        ? i
                        : (int)((long)(i / kSampleRun) * (vis - kSampleRun) / (kRuns - 1)) + i % kSampleRun;
    sv[j] = i < m ? srow[pos] : 0.f;
  }
  uint32_t sk[kPer];
  uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int j = 0; j < kPer; j++) {
    sk[j] = score_key(sv[j]);
    if ((int)threadIdx.x + j * kFilterThreads < m) {
      mn = min(mn, sk[j]);
      mx = max(mx, sk[j]);
    }
  }
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  const int wave = threadIdx.x / kWave;
  if (threadIdx.x % kWave == 0) {
    fmm[0][wave] = mn;
    fmm[1][wave] = mx;
  }
  for (int i = threadIdx.x; i < kBins0; i += kFilterThreads) h[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kFilterThreads / kWave; w++) {
    mn = min(mn, fmm[0][w]);
    mx = max(mx, fmm[1][w]);
  }
  const uint64_t span = (uint64_t)(mx - mn) + 1;
  const int bits = span == 1 ? 0 : 64 - __clzll(span - 1);  // range 2^bits covers the sample
  const int sh = bits > 12 ? bits - 12 : 0;
  const int nb = 1 << (bits - sh);
#pragma unroll
  for (int j = 0; j < kPer; j++)
    if ((int)threadIdx.x + j * kFilterThreads < m) atomicAdd(&h[(sk[j] - mn) >> sh], 1u);
  __syncthreads();
  const long expect = ((long)k * m + vis - 1) / vis;  // rank of the k-th key in the sample
  const int r = (int)min((long)m, 2 * expect + 8);
  find_bin<kFilterThreads>(h, nb, r, res, tmp);
  const uint32_t thr = mn + ((uint32_t)res[0] << sh);
  // Ordered compaction of each chunk's positions whose key is >= thr.
  for (int ci = ci0; ci < ci1; ci++) {  // uniform over the workgroup
    const int c0 = ci * kChunk;
    if (c0 >= vis) {
      if (threadIdx.x == 0) cnt[ci] = 0u;
      continue;
    }
    if (ci != ci0) load_chunk_keys(srow, c0, vis, key);
    const int e0 = c0 + threadIdx.x * 16;
    uint32_t flags = 0;
    int c = 0;
#pragma unroll
    for (int j = 0; j < 16; j++) {
      if (e0 + j < vis && key[j] >= thr) {
        flags |= 1u << j;
        c++;
      }
    }
    int total;
    int o = block_exclusive_scan<kFilterThreads>(c, tmp, &total);
    int2* seg = cand + ((size_t)row * nchunks + ci) * kTopkSegCap;
#pragma unroll
    for (int j = 0; j < 16; j++)
      if (flags >> j & 1u) {
        if (o < kTopkSegCap) seg[o] = make_int2(e0 + j, (int)key[j]);
        o++;
      }
    if (threadIdx.x == 0) cnt[ci] = (uint32_t)total;  // above kTopkSegCap: the row is redone
  }
}

// Row set-up shared by the select kernels: applies the row's own count
// (k_rows: slots past it hold -1; k becomes the count) and handles rows that
// keep every visible position (vis <= k: all of them in order, or with a
// finite margin those scoring at least the row maximum minus the margin).
// Returns true when the row is done (out and kept written). Uniform over the
// workgroup; every thread must call it.
__device__ bool row_prologue(const float* srow, int vis, int& k, const int32_t* k_rows, int row,
                             float margin, int32_t* out, int32_t* kept_row,
                             uint32_t (*mm)[kWaves], int* tmp) {
  if (k_rows) {  // this row keeps kr positions; slots kr .. k-1 hold -1
    const int kr = min(max(k_rows[row], 0), k);
    for (int i = kr + threadIdx.x; i < k; i += kThreads) out[i] = -1;
    k = kr;
    if (k == 0) {
      if (kept_row && threadIdx.x == 0) *kept_row = 0;
      return true;
    }
  }
  if (vis > k) return false;
  if (!(margin < INFINITY)) {  // every visible position, in order
    for (int i = threadIdx.x; i < k; i += kThreads) out[i] = i < vis ? i : -1;
    if (kept_row && threadIdx.x == 0) *kept_row = vis;
    return true;
  }
  // ... those at or above the threshold: row maximum, then an ordered
  // compaction of the visible positions.
  uint32_t mn = 0xffffffffu, mx = 0u;
  for (int i = threadIdx.x; i < vis; i += kThreads) mx = max(mx, score_key(srow[i]));
  block_minmax(mn, mx, mm);
  const uint32_t mkey = margin_key(mx, margin);
  int base = 0;
  for (int t0 = 0; t0 < vis; t0 += kThreads) {  // uniform
    const int i = t0 + threadIdx.x;
    const int f = i < vis && score_key(srow[i]) >= mkey;
    int tot;
    const int pre = block_exclusive_scan<kThreads>(f, tmp, &tot);
    if (f) out[base + pre] = i;
    base += tot;
  }
  for (int i = base + threadIdx.x; i < k; i += kThreads) out[i] = -1;
  if (kept_row && threadIdx.x == 0) *kept_row = base;
  return true;
}

// LDS of the selection (one 1024-thread workgroup per row).
struct SelectLds {
  uint32_t h[kBins0 * (1 + kHistCopies)];
  uint32_t few[kWave];  // keys of the k-th key's bin (row-histogram path)
  int nfew;
  int32_t lpos[kLdsCap];
  uint32_t lkey[kLdsCap];
  int off[kTopkMaxChunks + 1];
  uint32_t mm[2][kWaves];
  int wtot[kWaves + 1];
  int tmp[17];
  int res[3];
};

// Selection of row `row` from the filter's candidate segments (counts at
// counts[row * cstride + c]); every thread of the 1024-thread workgroup
// calls it. trust_segments false: redo the row from its scores alone.
// ghist (or NULL): the row's histogram of its candidates, gnb bins of 2^gs
// keys from key gthr, the last bin also holding every key above them (built
// by the one-launch filter). With it, the bin of the k-th key comes straight
// from the histogram, and the selection resolves the k-th key inside that
// bin only: up to 64 keys are collected while the candidates are gathered
// and ranked by one wave, more take radix passes over the bin's key range.
// The general path (the candidates' key range, radix passes over it) takes
// over when that bin is the open last one or the row is cut by a margin
// (which needs the row maximum).
__device__ __forceinline__ void select_row(int row, const float* __restrict__ scores, const uint32_t* __restrict__ counts,
                           int cstride, const int2* __restrict__ cand, int32_t* __restrict__ spill,
                           int32_t* __restrict__ idx, int T, int kv_len, int k,
                           const int32_t* __restrict__ k_rows, int nchunks, float margin,
                           int32_t* __restrict__ kept, bool trust_segments, const uint32_t* ghist,
                           uint32_t gthr, int gs, int gnb, SelectLds& L) {
  uint32_t* h = L.h;
  int32_t* lpos = L.lpos;
  uint32_t* lkey = L.lkey;
  int* off = L.off;
  uint32_t (*mm)[kWaves] = L.mm;
  int* wtot = L.wtot;
  int* tmp = L.tmp;
  int* res = L.res;
  const int vis = kv_len - T + (row % T) + 1;
  int32_t* out = idx + (size_t)row * k;  // k slots
  int32_t* kept_row = kept ? kept + row : nullptr;
  const float* srow = scores + (size_t)row * kv_len;
  if (row_prologue(srow, vis, k, k_rows, row, margin, out, kept_row, mm, tmp)) return;
  const bool skip = margin < INFINITY;  // ordered skipping (uniform)
  const bool use_hist = ghist != nullptr && !skip && gnb > 1;  // uniform
  // Thread t holds bins 4 (1023 - t) .. 4 (1023 - t) + 3 (kThreads * 4 =
  // kBins0), so the threads in order run from the highest bins down.
  // The counts and the histogram are loaded first: the scan below waits
  // only for them, while the speculative gather loads are still arriving.
  const int v = (int)threadIdx.x < nchunks ? (int)counts[(size_t)row * cstride + threadIdx.x] : 0;
  uint4 gh = make_uint4(0u, 0u, 0u, 0u);
  if (use_hist) gh = reinterpret_cast<const uint4*>(ghist)[kThreads - 1 - threadIdx.x];
  // Chunk owned by this thread for the gather: tpc threads per chunk, thread
  // j0 of a chunk takes entries j0, j0 + tpc, ... Its first kSpec entries are
  // loaded now, before the counts are known (the slots exist whatever the
  // count), so the usual gather costs one memory round trip.
  const int2* segs = cand + (size_t)row * nchunks * kTopkSegCap;
  const int tpc = kThreads / nchunks;  // nchunks <= kThreads
  const int gc = threadIdx.x / tpc, j0 = threadIdx.x % tpc;
  const int2* sg = segs + (size_t)min(gc, nchunks - 1) * kTopkSegCap;
  constexpr int kSpec = 8;
  int2 pre[kSpec];
#pragma unroll
  for (int u = 0; u < kSpec; u++)  // unconditional (clamped) loads: all in flight together
    pre[u] = sg[min(j0 + u * tpc, kTopkSegCap - 1)];  // used only where j0 + u * tpc < count <= kTopkSegCap
  if (use_hist && threadIdx.x == 0) L.nfew = 0;  // published by the barriers below
  // Offsets of the candidate segments, whether a segment overflowed, and
  // (with the row histogram) the bin of the k-th key: one block scan of the
  // counts and of the bin sums together.
  int n;
  bool overflow;
  int fb = -1, hab = 0, cb = 0;  // bin of the k-th key, keys above it, keys in it (fb < 0: none)
  {
    const int c = threadIdx.x;
    const int lane = c % kWave;
    const int wid = __builtin_amdgcn_readfirstlane(c / kWave);
    const int hs = (int)(gh.x + gh.y + gh.z + gh.w);
    const int inc = wave_inclusive_scan(v), hinc = wave_inclusive_scan(hs);
    const bool wave_ovf = __ballot(v > kTopkSegCap) != 0;
    if (lane == kWave - 1) {
      tmp[wid] = inc;
      wtot[wid] = hinc;
      mm[0][wid] = wave_ovf;
    }
    __syncthreads();
    const int x = lane < kWaves ? tmp[lane] : 0, hx = lane < kWaves ? wtot[lane] : 0;
    const int xs = wave_inclusive_scan(x), hxs = wave_inclusive_scan(hx);
    overflow = __ballot(lane < kWaves && mm[0][lane] != 0u) != 0;
    n = __builtin_amdgcn_readlane(xs, kWaves - 1);
    if (c < nchunks) off[c] = __builtin_amdgcn_readlane(xs - x, wid) + inc - v;
    if (c == 0) off[nchunks] = n;
    const int htot = __builtin_amdgcn_readlane(hxs, kWaves - 1);  // n, when the segments are trusted
    const bool hit = use_hist && k > 0 && htot >= k;             // uniform
    if (hit) {
      int acc = __builtin_amdgcn_readlane(hxs - hx, wid) + hinc - hs;  // keys in the bins above this thread's
      if (acc < k && k <= acc + hs) {  // the k-th key is in one of this thread's bins
        const int b3 = 4 * (kThreads - 1 - c) + 3;
        const uint32_t cnt[4] = {gh.w, gh.z, gh.y, gh.x};
        for (int j = 0; j < 4; j++) {
          if (acc + (int)cnt[j] >= k) {
            res[0] = b3 - j;
            res[1] = acc;
            res[2] = (int)cnt[j];
            break;
          }
          acc += (int)cnt[j];
        }
      }
    }
    __syncthreads();  // publishes off and res
    if (hit) {
      fb = res[0];
      hab = res[1];
      cb = res[2];
      if (fb >= gnb - 1) fb = -1;  // the open last bin: general path (uniform)
    }
  }
  if (n >= k && !overflow && trust_segments) {
    uint32_t mn = 0xffffffffu, mx = 0u;  // key range of the candidates
    if (n <= kLdsCap) {
      if (fb >= 0) {
        // The k-th key lies in [blo, bhi), with hab candidates above it.
        // Up to 64 keys there are collected during the gather and ranked by
        // one wave; more take radix passes over that range only.
        const uint64_t blo = (uint64_t)gthr + ((uint64_t)fb << gs), bhi = blo + (1ull << gs);
        const uint64_t flo = cb <= kWave ? blo : bhi;  // collect nothing past 64 keys
        if (gc < nchunks) {
          const int o = off[gc], cnt = off[gc + 1] - off[gc];
#pragma unroll
          for (int u = 0; u < kSpec; u++) {
            const int j = j0 + u * tpc;
            if (j < cnt) {
              const uint32_t key = (uint32_t)pre[u].y;
              lpos[o + j] = pre[u].x;
              lkey[o + j] = key;
              if (key >= flo && key < bhi) {
                const int f = atomicAdd(&L.nfew, 1);
                if (f < kWave) L.few[f] = key;  // cb <= kWave of them
              }
            }
          }
          for (int j = j0 + kSpec * tpc; j < cnt; j += tpc) {
            const int2 e = sg[j];
            const uint32_t key = (uint32_t)e.y;
            lpos[o + j] = e.x;
            lkey[o + j] = key;
            if (key >= flo && key < bhi) {
              const int f = atomicAdd(&L.nfew, 1);
              if (f < kWave) L.few[f] = key;
            }
          }
        }
        __syncthreads();  // the candidates (and the bin's keys) are in LDS
        const Cand acc{lpos, lkey, nullptr, srow};
        if (cb <= kWave) {
          rank_few(L.few, cb, k - hab, res);
          __syncthreads();
          emit_selection(acc, n, (uint32_t)res[0], res[1], tmp, out, k, kept_row);
        } else {
          select_and_emit(acc, n, k - hab, (uint32_t)blo, 1ull << gs, h, res, tmp, out, k, 0u, kept_row);
        }
        return;
      }
      if (gc < nchunks) {
        const int o = off[gc], cnt = off[gc + 1] - off[gc];
#pragma unroll
        for (int u = 0; u < kSpec; u++) {
          const int j = j0 + u * tpc;
          if (j < cnt) {
            lpos[o + j] = pre[u].x;
            lkey[o + j] = (uint32_t)pre[u].y;
            mn = min(mn, (uint32_t)pre[u].y);
            mx = max(mx, (uint32_t)pre[u].y);
          }
        }
        for (int j = j0 + kSpec * tpc; j < cnt; j += tpc) {
          const int2 e = sg[j];
          lpos[o + j] = e.x;
          lkey[o + j] = (uint32_t)e.y;
          mn = min(mn, (uint32_t)e.y);
          mx = max(mx, (uint32_t)e.y);
        }
      }
      block_minmax(mn, mx, mm);  // its barrier also publishes the gather
      select_top(Cand{lpos, lkey, nullptr, srow}, n, k, mn, mx, h, res, tmp, out,
                 margin_key(mx, margin), kept_row);
    } else {
      const SegCand acc{segs, off, nchunks};
      for (int i = threadIdx.x; i < n; i += kThreads) {
        const uint32_t key = acc.k(i);
        mn = min(mn, key);
        mx = max(mx, key);
      }
      block_minmax(mn, mx, mm);
      select_top(acc, n, k, mn, mx, h, res, tmp, out, margin_key(mx, margin), kept_row);
    }
    return;
  }
  // The sample overshot (or a chunk overflowed): redo this row from its
  // scores alone.
  int32_t* gpos = spill + (size_t)row * kv_len;
  uint32_t b0;
  int above;
  if ((reinterpret_cast<uintptr_t>(srow) & 15) == 0)
    n = histogram_and_candidates<true>(srow, vis, k, h, lpos, lkey, gpos, wtot, tmp, res, &b0, &above);
  else
    n = histogram_and_candidates<false>(srow, vis, k, h, lpos, lkey, gpos, wtot, tmp, res, &b0, &above);
  const Cand acc{lpos, lkey, gpos, srow};
  uint32_t mkey = 0u;
  if (skip) {  // the row maximum is among the candidates (the top bins)
    uint32_t mn = 0xffffffffu, mx = 0u;
    for (int i = threadIdx.x; i < n; i += kThreads) mx = max(mx, acc.k(i));
    block_minmax(mn, mx, mm);
    mkey = margin_key(mx, margin);
  }
  select_and_emit(acc, n, k - above, b0 << 20, 1ull << 20, h, res, tmp, out, k, mkey, kept_row);
}

// grid (rows), block 1024.
__global__ __launch_bounds__(kThreads) void topk_select(const float* __restrict__ scores,
                                                        const uint32_t* __restrict__ counts,
                                                        const int2* __restrict__ cand,
                                                        int32_t* __restrict__ spill,
                                                        int32_t* __restrict__ idx, int T,
                                                        int kv_len, int k,
                                                        const int32_t* __restrict__ k_rows,
                                                        int nchunks, int cstride, float margin,
                                                        int32_t* __restrict__ kept) {
  __shared__ __attribute__((aligned(16))) SelectLds L;
  select_row(blockIdx.x, scores, counts, cstride, cand, spill, idx, T, kv_len, k, k_rows, nchunks, margin,
             kept, true, nullptr, 0u, 0, 0, L);
}


// ---------------------------------------------------------------------------
// One-launch form for few rows (decode): grid = rows x filter workgroups,
// 1024 threads each. A workgroup takes cpw consecutive 4096-element chunks
// of its row, computes the row's sample threshold as topk_filter does and
// writes the chunks' candidate segments and counts, and adds its candidates
// to the row's candidate histogram (bins from the same sample); it then
// waits until its stores are done and counts itself in the row's arrival
// word. The
// workgroup that arrives last selects the row (topk_select's work) from the
// segments. Segments and counts are plain stores into the L2 of the
// writer's XCD; the selecting workgroup reads them through its own L2, so
// all of a row's workgroups must run on one XCD. The grid is laid out for
// that (workgroups go to the XCDs in turn, XCD = workgroup id mod n_xcd, and
// row r's workgroups all get ids = r mod n_xcd), and the arrival word checks
// it: each arrival adds 1, its XCD number x (register XCC_ID) and x^2 to
// three fields; the sums equal (n x, n x^2) only when all n arrivals ran on
// XCD x. Otherwise the last arrival redoes the row from its scores alone
// (the select's full-row path), which reads nothing the filter wrote.
// Arrival region: per row kArrStride u32 words, the 64-bit arrival word
// first (count bits 0..15, sum of x bits 16..31, sum of x^2 bits 32..63),
// then from word 32 the row's candidate histogram (4096 u32). The whole
// region is zero before every launch (the caller clears it; the last
// arrival also resets its word).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t xcc_id() {
  return __builtin_amdgcn_s_getreg((3 << 11) | 20);  // HW_REG_XCC_ID, bits [3:0]
}

constexpr int kFusedPer = kChunk / kThreads;  // elements of a chunk per thread (4)

__global__ __launch_bounds__(kThreads) void topk_fused(const float* __restrict__ scores,
                                                       uint32_t* __restrict__ counts, int2* __restrict__ cand,
                                                       int32_t* __restrict__ spill, int32_t* __restrict__ idx,
                                                       int T, int kv_len, int k,
                                                       const int32_t* __restrict__ k_rows, int nchunks,
                                                       int cstride, int cpw, int wpr, int rows, int n_xcd,
                                                       float margin, int32_t* __restrict__ kept,
                                                       uint32_t* __restrict__ arrivals, int force_redo) {
  __shared__ __attribute__((aligned(16))) SelectLds L;
  __shared__ int s_flag;
  const int x = blockIdx.x % n_xcd, slot = blockIdx.x / n_xcd;
  const int row = x + n_xcd * (slot / wpr);
  if (row >= rows) return;  // no row for this workgroup (uniform)
  uint32_t* ghist = arrivals + (size_t)row * kArrStride + 32;  // the row's candidate histogram
  uint32_t gthr = 0u;  // its bins: gnb bins of 2^gs keys from gthr (gnb = 0: not computed here)
  int gs = 0, gnb = 0;
  const int ci0 = (slot % wpr) * cpw, ci1 = min(nchunks, ci0 + cpw);
  const int vis = kv_len - T + (row % T) + 1;
  const float* srow = scores + (size_t)row * kv_len;
  uint32_t* cnt = counts + (size_t)row * cstride;
  int kr = k_rows ? min(max(k_rows[row], 0), k) : k;
  uint32_t* h = L.h;
  int* tmp = L.tmp;
  int* res = L.res;
  if (vis <= kr || ci0 * kChunk >= vis || kr == 0) {
    for (int ci = ci0 + threadIdx.x; ci < ci1; ci += kThreads) cnt[ci] = 0u;
  } else {
    // This thread's 4 consecutive elements of the first chunk, then the
    // row's sample (2 elements per thread), both in flight together.
    const bool a16 = (reinterpret_cast<uintptr_t>(srow) & 15) == 0;
    float xs[kFusedPer];
    if (a16)
      load4<true>(srow, ci0 * kChunk + threadIdx.x * kFusedPer, vis, xs);
    else
      load4<false>(srow, ci0 * kChunk + threadIdx.x * kFusedPer, vis, xs);
    const int m = min(kSample, vis);
    constexpr int kRuns = kSample / kSampleRun;
    constexpr int kPer = kSample / kThreads;
    float sv[kPer];
#pragma unroll
    for (int j = 0; j < kPer; j++) {
      const int i = threadIdx.x + j * kThreads;
      const int pos = vis <= kSample
                          ? i
                          : (int)((long)(i / kSampleRun) * (vis - kSampleRun) / (kRuns - 1)) + i % kSampleRun;
      sv[j] = i < m ? srow[pos] : 0.f;
    }
    uint32_t sk[kPer];
    uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int j = 0; j < kPer; j++) {
      sk[j] = score_key(sv[j]);
      if ((int)threadIdx.x + j * kThreads < m) {
        mn = min(mn, sk[j]);
        mx = max(mx, sk[j]);
      }
    }
    for (int i = threadIdx.x; i < kBins0; i += kThreads) h[i] = 0u;
    block_minmax(mn, mx, L.mm);  // its barrier also orders the clear before the counts
    const uint64_t span = (uint64_t)(mx - mn) + 1;
    const int bits = span == 1 ? 0 : 64 - __clzll(span - 1);
    const int sh = bits > 12 ? bits - 12 : 0;
    const int nb = 1 << (bits - sh);
#pragma unroll
    for (int j = 0; j < kPer; j++)
      if ((int)threadIdx.x + j * kThreads < m) atomicAdd(&h[(sk[j] - mn) >> sh], 1u);
    __syncthreads();
    const long expect = ((long)kr * m + vis - 1) / vis;  // rank of the k-th key in the sample
    find_bin<kThreads>(h, nb, (int)min((long)m, 2 * expect + 8), res, tmp);
    const uint32_t thr = mn + ((uint32_t)res[0] << sh);
    // The row's candidate histogram: at most 4096 bins of 2^gs keys from
    // thr, reaching the sample's largest key; keys above go to the last bin.
    // Every workgroup of the row derives the same bins from the same sample.
    // Each workgroup bins its own candidates in LDS first (the sample's
    // histogram is no longer read) and adds only its non-zero bins to the
    // row's, so no bin takes more than one global atomic per workgroup.
    {
      const uint64_t gspan = (uint64_t)(mx - thr) + 1;  // thr <= mx: its bin holds a sample key
      const int gbits = gspan == 1 ? 0 : 64 - __clzll(gspan - 1);
      gs = gbits > 12 ? gbits - 12 : 0;
      gnb = 1 << (gbits - gs);
      gthr = thr;
    }
    for (int i = threadIdx.x; i < kBins0; i += kThreads) h[i] = 0u;  // ordered before the adds by the scan's barriers
    for (int ci = ci0; ci < ci1; ci++) {  // uniform over the workgroup
      const int c0 = ci * kChunk;
      if (c0 >= vis) {
        if (threadIdx.x == 0) cnt[ci] = 0u;
        continue;
      }
      const int e = c0 + threadIdx.x * kFusedPer;
      if (ci != ci0) {
        if (a16)
          load4<true>(srow, e, vis, xs);
        else
          load4<false>(srow, e, vis, xs);
      }
      uint32_t key[kFusedPer];
      uint32_t flags = 0;
      int c = 0;
#pragma unroll
      for (int j = 0; j < kFusedPer; j++) {
        key[j] = score_key(xs[j]);
        if (e + j < vis && key[j] >= thr) {
          flags |= 1u << j;
          c++;
        }
      }
      int total;
      int o = block_exclusive_scan<kThreads>(c, tmp, &total);
      int2* seg = cand + ((size_t)row * nchunks + ci) * kTopkSegCap;
#pragma unroll
      for (int j = 0; j < kFusedPer; j++)
        if (flags >> j & 1u) {
          if (o < kTopkSegCap) seg[o] = make_int2(e + j, (int)key[j]);
          o++;
          atomicAdd(&h[min((key[j] - thr) >> gs, (uint32_t)gnb - 1u)], 1u);
        }
      if (threadIdx.x == 0) cnt[ci] = (uint32_t)total;  // above kTopkSegCap: the row is redone
    }
    __syncthreads();  // the workgroup's bins are complete
    for (int b = threadIdx.x; b < gnb; b += kThreads) {
      const uint32_t c = h[b];
      if (c) atomicAdd(&ghist[b], c);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // this thread's segment, count and histogram writes are done (in this XCD's L2)
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint64_t xi = xcc_id() & 15u;
    const uint64_t mine = 1ull | (xi << 16) | ((xi * xi) << 32);
    uint64_t* word = reinterpret_cast<uint64_t*>(arrivals + (size_t)row * kArrStride);
    const uint64_t now = __hip_atomic_fetch_add(word, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + mine;
    int flag = 0;
    if ((now & 0xffffu) == (uint64_t)wpr) {  // every workgroup of the row has arrived
      __hip_atomic_exchange(word, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const bool one_xcd =
          ((now >> 16) & 0xffffu) == (uint64_t)wpr * xi && (now >> 32) == (uint64_t)wpr * xi * xi;
      flag = one_xcd && !force_redo ? 1 : 2;
    }
    s_flag = flag;
  }
  __syncthreads();
  if (s_flag == 0) return;
  select_row(row, scores, counts, cstride, cand, spill, idx, T, kv_len, k, k_rows, nchunks, margin, kept,
             s_flag == 1, gnb ? ghist : nullptr, gthr, gs, gnb, L);
}

// A whole row held in LDS as keys.
struct RowCand {
  const uint32_t* key;
  __device__ int p(int i) const { return i; }
  __device__ uint32_t k(int i) const { return key[i]; }
};

// Loads the visible part of a row into LDS as keys; returns this thread's
// min and max key through mn, mx. Thread t takes elements t, t + 1024, ...
// (coalesced); every load is issued unconditionally from a clamped address
// and masked at use, so all of them are in flight together (conditional
// loads make the compiler wait for each one before the next).
__device__ void load_row_keys(const float* srow, int vis, uint32_t* key, uint32_t& mn, uint32_t& mx) {
  constexpr int kB = kLdsRow / kThreads;
  float x[kB];
#pragma unroll
  for (int u = 0; u < kB; u++) x[u] = srow[min((int)threadIdx.x + u * kThreads, vis - 1)];
#pragma unroll
  for (int u = 0; u < kB; u++) {
    const int e = threadIdx.x + u * kThreads;
    if (e < vis) {
      const uint32_t kk = score_key(x[u]);
      key[e] = kk;
      mn = min(mn, kk);
      mx = max(mx, kk);
    }
  }
}

// Short rows (at most kLdsRow positions), in one launch (grid (rows), block
// 1024): the row is read once into LDS as keys; a threshold from kSample
// evenly spaced keys of it, binned over the sample's own range like the
// filter's, is checked to leave at least k keys at or above it and then
// bounds the radix selection from below, so its passes histogram only those
// keys; the ordered emission scans the row in LDS. Same results as
// topk_filter + topk_select.
__global__ __launch_bounds__(kThreads) void topk_lds(const float* __restrict__ scores,
                                                     int32_t* __restrict__ idx, int T, int kv_len,
                                                     int k, const int32_t* __restrict__ k_rows,
                                                     float margin, int32_t* __restrict__ kept) {
  __shared__ __attribute__((aligned(16))) uint32_t key[kLdsRow];
  __shared__ uint32_t h[kBins0];
  __shared__ uint32_t mm[2][kWaves];
  __shared__ uint32_t smm[2][kWaves];
  __shared__ int tmp[17];
  __shared__ int res[3];
  const int row = blockIdx.x;
  const int vis = kv_len - T + (row % T) + 1;
  int32_t* out = idx + (size_t)row * k;
  int32_t* kept_row = kept ? kept + row : nullptr;
  const float* srow = scores + (size_t)row * kv_len;
  if (row_prologue(srow, vis, k, k_rows, row, margin, out, kept_row, mm, tmp)) return;
  uint32_t mn = 0xffffffffu, mx = 0u;
  load_row_keys(srow, vis, key, mn, mx);
  block_minmax(mn, mx, mm);  // its barrier also publishes the keys
  // Sample: kSample keys at evenly spaced positions (vis > k >= 1 here).
  const int m = min(kSample, vis);
  constexpr int kPer = kSample / kThreads;
  uint32_t sk[kPer];
  uint32_t smn = 0xffffffffu, smx = 0u;
#pragma unroll
  for (int j = 0; j < kPer; j++) {
    const int i = threadIdx.x + j * kThreads;
    sk[j] = i < m ? key[(int)((long)i * vis / m)] : 0u;
    if (i < m) {
      smn = min(smn, sk[j]);
      smx = max(smx, sk[j]);
    }
  }
  for (int i = threadIdx.x; i < kBins0; i += kThreads) h[i] = 0u;
  block_minmax(smn, smx, smm);  // its barrier also orders the clear before the counts
  const uint64_t sspan = (uint64_t)(smx - smn) + 1;
  const int bits = sspan == 1 ? 0 : 64 - __clzll(sspan - 1);
  const int sh = bits > 12 ? bits - 12 : 0;
  const int nb = 1 << (bits - sh);
#pragma unroll
  for (int j = 0; j < kPer; j++)
    if ((int)threadIdx.x + j * kThreads < m) atomicAdd(&h[(sk[j] - smn) >> sh], 1u);
  __syncthreads();
  const long expect = ((long)k * m + vis - 1) / vis;  // rank of the k-th key in the sample
  find_bin<kThreads>(h, nb, (int)min((long)m, 2 * expect + 8), res, tmp);
  uint32_t lo = smn + ((uint32_t)res[0] << sh);
  // Keep the threshold only if at least k keys reach it (else the whole range).
  int c = 0;
  for (int e = threadIdx.x; e < vis; e += kThreads) c += key[e] >= lo;
  int total;
  block_exclusive_scan<kThreads>(c, tmp, &total);
  if (total < k) lo = mn;
  const uint64_t span = (uint64_t)(mx - lo) + 1;  // mx >= lo: the k-th key is at or above lo
  const uint64_t R = span == 1 ? 1 : 1ull << (64 - __clzll(span - 1));
  select_and_emit(RowCand{key}, vis, k, lo, R, h, res, tmp, out, k,
                  margin < INFINITY ? margin_key(mx, margin) : 0u, kept_row);
}

}  // namespace

int zero_words(uint32_t* p, size_t n, hipStream_t stream) {
  if (n == 0) return CLSA_OK;
  size_t blocks = (n + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(fill_zero, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return check_launch("fill_zero");
}

TopkBuffers topk_buffers(int rows, int kv_len) {
  TopkBuffers b;
  b.nchunks = (kv_len + kChunk - 1) / kChunk;
  b.cstride = (b.nchunks + 31) / 32 * 32;  // a row's counts start on their own 128-byte line
  b.counts_words = (size_t)rows * b.cstride;
  b.cand_words = (size_t)rows * b.nchunks * kTopkSegCap * 2;
  b.spill_words = (size_t)rows * kv_len;
  // per row of the one-launch form (only for few rows): arrival word, row histogram
  b.arrival_words = rows <= kFusedMaxRows ? (size_t)rows * kArrStride : 0;
  return b;
}

bool topk_uses_arrivals(int rows, int kv_len, int k) {
  const int nchunks = (kv_len + kChunk - 1) / kChunk;
  const bool lds = kv_len <= kLdsRow / 2 || (kv_len <= kLdsRow && 8L * k >= kv_len);
  return !lds && rows <= kFusedMaxRows && nchunks <= kFusedMaxChunks;
}

namespace {
// XCDs of the current device (gfx950: 32 CUs each); workgroup i runs on XCD
// i % n_xcd. Used for placement only: topk_fused checks where it ran.
int device_xcds() {
  static std::mutex mu;
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
  std::lock_guard<std::mutex> lock(mu);
  if (!cached[dev]) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
    cached[dev] = (cus >= 32 && cus % 32 == 0) ? std::min(cus / 32, 16) : 1;
  }
  return cached[dev];
}
// CLSA_TOPK_FORCE_REDO=1: the one-launch top-k redoes every row from its
// scores (tests of that path).
int force_redo() {
  static const int v = [] {
    const char* e = getenv("CLSA_TOPK_FORCE_REDO");
    return e && e[0] == '1' ? 1 : 0;
  }();
  return v;
}
}  // namespace

int launch_topk(const float* scores, int B, int T, int kv_len, int k, const int32_t* k_rows,
                float margin, int32_t* idx, int32_t* kept, uint32_t* counts, int32_t* cand,
                int32_t* spill, uint32_t* arrivals, hipStream_t stream) {
  const int rows = B * T;
  const TopkBuffers tb = topk_buffers(rows, kv_len);
  if (tb.nchunks > kTopkMaxChunks)
    return set_error(CLSA_ERR_UNSUPPORTED, "topk: kv_len=%d above %d", kv_len, kTopkMaxChunks * kChunk);
  // One launch with the row in LDS for short rows: one CU reads a whole row,
  // which pays off up to 8K positions (4096: 10.0 against 12.9 us for the
  // two launches; 64 rows of 8192: 12.6 against 15.7 us), and up to 16K when
  // k is at least 1/8 of the row (the filter's segments then overflow into
  // the full-row redo: 2 rows of 12000, k = 2048: 13.9 against 22.5 us),
  // but not for 16K rows with few candidates (4 rows, k = 1024: 19.1
  // against 16.2 us) nor for longer rows (8 x 32768: 31.6 against 17.6 us).
  if (kv_len <= kLdsRow / 2 || (kv_len <= kLdsRow && 8L * k >= kv_len)) {
    hipLaunchKernelGGL(topk_lds, dim3(rows), dim3(kThreads), 0, stream, scores, idx, T, kv_len, k,
                       k_rows, margin, kept);
    return check_launch("topk_lds");
  }
  int2* segs = reinterpret_cast<int2*>(cand);
  if (topk_uses_arrivals(rows, kv_len, k)) {
    // Few rows: one launch, the selection done by each row's last workgroup.
    const int n_xcd = device_xcds();
    const int wpr = tb.nchunks;  // one 4096-element chunk per workgroup
    const int rpx = (rows + n_xcd - 1) / n_xcd;
    hipLaunchKernelGGL(topk_fused, dim3((unsigned)(n_xcd * rpx * wpr)), dim3(kThreads), 0, stream, scores,
                       counts, segs, spill, idx, T, kv_len, k, k_rows, tb.nchunks, tb.cstride, 1, wpr,
                       rows, n_xcd, margin, kept, arrivals, force_redo());
    return check_launch("topk_fused");
  }
  // Chunks per filter workgroup: one while the grid stays small (decode),
  // more when rows are many (a chunk's queries), so the row's threshold is
  // computed once per cpw chunks; about 8192 workgroups at most.
  const long total_chunks = (long)rows * tb.nchunks;
  int cpw = (int)min((long)tb.nchunks, max(1L, total_chunks / 8192));
  hipLaunchKernelGGL(topk_filter, dim3((tb.nchunks + cpw - 1) / cpw, rows), dim3(kFilterThreads), 0,
                     stream, scores, counts, segs, T, kv_len, k, k_rows, tb.nchunks, tb.cstride, cpw);
  int rc = check_launch("topk_filter");
  if (rc) return rc;
  hipLaunchKernelGGL(topk_select, dim3(rows), dim3(kThreads), 0, stream, scores, counts, segs, spill,
                     idx, T, kv_len, k, k_rows, tb.nchunks, tb.cstride, margin, kept);
  return check_launch("topk_select");
}

}  // namespace clsa
