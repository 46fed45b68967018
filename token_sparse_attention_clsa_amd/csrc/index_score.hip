// index_score.hip — indexer scores on gfx950 matrix cores.
//
// Computes, for every query (b, t) and visible cache position s,
//   score = sum_h w[h] * max(0, q_idx[h, :] . k_idx[s, :])
// (IndexCache summary, "1. Problématique": the lightning indexer scores every
// previous token; CLSA article, "Comment CLSA fonctionne": the shared indexer
// scores once). Positions a query does not see get -inf.
//
// Decode shape: per query the work is a [H_I x D_I] x [D_I x L] product whose
// operand A (the query's indexer heads) is tiny and read once, while B (one
// indexer key per cached token) streams from HBM exactly once. The kernel
// keeps A in registers for the whole launch, feeds B straight from global
// memory into MFMA operands (each key row is used by exactly one wave, so
// staging it through LDS would only add a round trip), and folds the ReLU,
// head weights and head sum into the epilogue so per-head scores never leave
// registers.
//
// MFMA (v_mfma_f32_16x16x32_bf16 / _fp8_fp8, wave64): lane l supplies row
// l%16 of A and column l%16 of B for the k-slice picked by l/16, and the
// 16x16 result element (i, j) lands in lane j + 16*(i/4), slot i%4. The sum
// runs over every k of the instruction, so the d-index carried by (lane
// group, slot) is free as long as A and B agree: lane group g, k-step s,
// slot e carries d = g*(D_I/4) + 8*s + e, which makes each lane's share of a
// key row one contiguous run of D_I/4 elements.
#include <algorithm>

#include "kernels.h"

namespace clsa {
namespace {

constexpr int kIdxThreads = 256;  // 4 waves

// This workgroup's share of clearing n words at p: workgroup g of the 2-D
// grid clears words g * nt + t, g * nt + t + G * nt, ... (G workgroups of nt
// threads), so no workgroup carries the whole clear.
__device__ __forceinline__ void zero_share(uint32_t* p, int n, int nt) {
  const int G = gridDim.x * gridDim.y, g = blockIdx.y * gridDim.x + blockIdx.x;
  for (int i = g * nt + (int)threadIdx.x; i < n; i += G * nt) p[i] = 0u;
}
constexpr int kKeysPerWaveIter = 64;  // 4 MFMA tiles of 16 keys

// max(x, 0) on the bit pattern: a non-negative float's bits are a
// non-negative int and a negative one's (-0 included) a negative int, so the
// signed integer max with 0 is ReLU for every non-NaN input in one
// v_max_i32 (fmaxf in IEEE mode also quiets its operand first).
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

template <int DT>
struct IdxElem;
template <>
struct IdxElem<CLSA_BF16> {
  static constexpr int bytes = 2;
  typedef bf16x8 frag;  // 8 elements per lane per k-step
  static __device__ __forceinline__ frag load(const uint8_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
  }
  static __device__ __forceinline__ f32x4 mfma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct IdxElem<CLSA_FP8_E4M3FN> {
  static constexpr int bytes = 1;
  typedef long frag;
  static __device__ __forceinline__ frag load(const uint8_t* p) {
    return *reinterpret_cast<const long*>(p);
  }
  static __device__ __forceinline__ f32x4 mfma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
  }
};

// With D_I = 128 the four 32-deep fp8 k-steps of a lane are one contiguous
// 32-byte run of the row (lane group g holds d = 32 g .. 32 g + 31), which
// is exactly the operand of gfx950's 128-deep fp8 MFMA: one
// v_mfma_scale_f32_16x16x128_f8f6f4 (A and B in E4M3, scale exponents 127,
// i.e. 1.0) replaces four v_mfma_f32_16x16x32_fp8_fp8. Measured on MI355X:
// the 32-deep fp8 instruction runs at about the bf16 rate (1.9 PFLOP/s), the
// 128-deep one at 4.8 PFLOP/s with the epilogue's VALU mostly hidden.
typedef __attribute__((ext_vector_type(8))) int i32x8;
__device__ __forceinline__ i32x8 cat4(long a, long b, long c, long d) {
  return i32x8{(int)a, (int)(a >> 32), (int)b, (int)(b >> 32), (int)c, (int)(c >> 32), (int)d, (int)(d >> 32)};
}
__device__ __forceinline__ f32x4 mfma_fp8_k128(const i32x8& a, const i32x8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
template <int DT, int DI>
constexpr bool kUseK128 = DT == CLSA_FP8_E4M3FN && DI == 128;

// grid: (ceil(kv_len / keys_per_wg), B*T), block: 256.
template <int DT, int DI, int HI>
__global__ __launch_bounds__(kIdxThreads) void idx_score_mfma(
    const uint8_t* __restrict__ q_idx, const uint8_t* __restrict__ k_idx,
    const float* __restrict__ w, float* __restrict__ scores, int T, int kv_len, int L_cap,
    int keys_per_wg, uint32_t* __restrict__ zero_p, int zero_n) {
  using E = IdxElem<DT>;
  // Words the step's next kernel needs zero (the one-launch top-k's arrival
  // region): cleared here, a share per workgroup, so that kernel needs no
  // launch of its own for it.
  if (zero_n) zero_share(zero_p, zero_n, kIdxThreads);
  constexpr int NS = DI / 32;          // k-steps per key row
  constexpr int NH = HI / 16;          // head tiles
  constexpr int SPAN = DI / 4 * E::bytes;  // bytes of a key row per lane

  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int col = lane % 16;   // A row / B column
  const int grp = lane / 16;   // k-slice group
  const int bt = blockIdx.y;
  const int b = bt / T, t = bt % T;
  const int vis = kv_len - T + t + 1;

  // A fragments: this query's indexer heads, resident for the whole launch.
  typename E::frag a[NH][NS];
  const uint8_t* qrow = q_idx + (size_t)bt * HI * DI * E::bytes;
#pragma unroll
  for (int ht = 0; ht < NH; ht++)
#pragma unroll
    for (int s = 0; s < NS; s++)
      a[ht][s] = E::load(qrow + ((size_t)(ht * 16 + col) * DI + grp * (DI / 4) + 8 * s) * E::bytes);
  // Head weights for the 4 result slots this lane holds in each head tile.
  float wv[NH][4];
#pragma unroll
  for (int ht = 0; ht < NH; ht++)
#pragma unroll
    for (int r = 0; r < 4; r++) wv[ht][r] = w[(size_t)bt * HI + ht * 16 + 4 * grp + r];

  const uint8_t* kbase = k_idx + (size_t)b * L_cap * DI * E::bytes + grp * SPAN;
  float* srow = scores + (size_t)bt * kv_len;
  const int k0 = blockIdx.x * keys_per_wg;
  const int k1 = min(k0 + keys_per_wg, kv_len);

  for (int base = k0 + wave * kKeysPerWaveIter; base < k1; base += 4 * kKeysPerWaveIter) {
    const int key_out = base + grp * 16 + col;  // key whose score this lane stores
    if (base >= vis) {  // whole group past this query's visible range (wave-uniform)
      if (key_out < k1) srow[key_out] = -INFINITY;
      continue;
    }
    // B fragments for 4 tiles of 16 keys; rows past the visible range are
    // clamped to a visible row and their results discarded.
    typename E::frag bf[4][NS];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int key = min(base + j * 16 + col, vis - 1);
      const uint8_t* p = kbase + (size_t)key * DI * E::bytes;
#pragma unroll
      for (int s = 0; s < NS; s++) bf[j][s] = E::load(p + 8 * s * E::bytes);
    }
    float res = 0.f;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      f32x4 acc[NH];
#pragma unroll
      for (int ht = 0; ht < NH; ht++) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (kUseK128<DT, DI>) {
        const i32x8 b8 = cat4(bf[j][0], bf[j][1], bf[j][2], bf[j][3]);
#pragma unroll
        for (int ht = 0; ht < NH; ht++)
          acc[ht] = mfma_fp8_k128(cat4(a[ht][0], a[ht][1], a[ht][2], a[ht][3]), b8, acc[ht]);
      } else {
#pragma unroll
        for (int s = 0; s < NS; s++)
#pragma unroll
          for (int ht = 0; ht < NH; ht++) acc[ht] = E::mfma(a[ht][s], bf[j][s], acc[ht]);
      }
      float v = 0.f;
#pragma unroll
      for (int ht = 0; ht < NH; ht++)
#pragma unroll
        for (int r = 0; r < 4; r++) v += wv[ht][r] * relu(acc[ht][r]);
      v += __shfl_xor(v, 16, kWave);
      v += __shfl_xor(v, 32, kWave);
      if (grp == j) res = v;
    }
    if (key_out < k1) srow[key_out] = key_out < vis ? res : -INFINITY;
  }
}

// Multi-query form (chunked prefill): a workgroup of kQB waves takes kQB
// consecutive queries of one batch element (wave w = query t0 + w, its heads
// in VGPRs as above) and a range of keys. Key tiles of kKT keys move from
// global memory straight into LDS (global_load_lds, 16 bytes per lane, no
// staging registers), double-buffered in two separate LDS objects so the
// compiler's wait analysis keeps a transfer into one buffer apart from reads
// of the other; every wave runs its MFMAs on the shared tile, so each key row
// leaves L2 once per kQB queries instead of once per query. Within the rows
// of each 256-byte span the 16-byte chunks are XOR-swizzled by row, so the 16
// rows one B-fragment read touches fall in distinct banks. A tile's scores
// are stored at the top of the next iteration, after its transfer is issued,
// so the per-tile wait for the transfer rarely waits on a store.
// grid (key_splits, B * ceil(T / kQB)), block kQB * 64.
constexpr int kQB = 8;
// Keys per LDS tile: 16 KiB tiles, 64 keys of 256-byte rows (bf16 x 128) or
// 128 keys of rows up to 128 bytes (fp8, or D_I = 64): each tile waits once
// for its transfer and once at a barrier, so shorter rows take longer tiles.
__host__ __device__ constexpr int key_tile(int rowb) { return rowb <= 128 ? 128 : 64; }
typedef __attribute__((address_space(3))) void lds_void;

// Lane group g (lanes 16 g .. 16 g + 15) receives v_g summed over the four
// lane groups (lanes l, l^16, l^32, l^48, added in that pairing order): a
// 4 x 4 transpose-reduce in three lane swaps and three adds.
__device__ __forceinline__ float group4_transpose_sum(float v0, float v1, float v2, float v3) {
  // Upper half receives the lower half's v2 / v3, lower half the upper's v0 / v1.
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v0), __float_as_uint(v2), false, false);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v1), __float_as_uint(v3), false, false);
  const float x02 = __uint_as_float(p[0]) + __uint_as_float(p[1]);  // lower: v0 sum, upper: v2 sum
  const float x13 = __uint_as_float(q[0]) + __uint_as_float(q[1]);  // lower: v1 sum, upper: v3 sum
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x02), __float_as_uint(x13), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int DT, int DI, int HI>
__global__ __launch_bounds__(kQB * kWave) void idx_score_multi(
    const uint8_t* __restrict__ q_idx, const uint8_t* __restrict__ k_idx,
    const float* __restrict__ w, float* __restrict__ scores, int T, int kv_len, int L_cap,
    int keys_per_split, uint32_t* __restrict__ zero_p, int zero_n) {
  using E = IdxElem<DT>;
  if (zero_n) zero_share(zero_p, zero_n, kQB * kWave);
  constexpr int NS = DI / 32;
  constexpr int NH = HI / 16;
  constexpr int ROWB = DI * E::bytes;          // bytes of one key row: 64, 128 or 256
  constexpr int CHUNKS = ROWB / 16;            // 16-byte chunks per row
  constexpr int RPS = 256 / ROWB;              // rows per 256-byte span
  constexpr int kKT = key_tile(ROWB);          // keys per tile
  constexpr int NR = kKT / 64;                 // results per lane per tile
  constexpr int NI = kKT * ROWB / 1024;        // 1 KiB transfers per tile
  static_assert(ROWB >= 64 && ROWB <= 256 && NI >= 1, "row size");
  __shared__ __attribute__((aligned(16))) uint8_t tile0[kKT * ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t tile1[kKT * ROWB];

  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int col = lane % 16, grp = lane / 16;
  const int groups_per_b = (T + kQB - 1) / kQB;
  const int b = blockIdx.y / groups_per_b;
  const int t = (blockIdx.y % groups_per_b) * kQB + wave;
  const bool active = t < T;
  const int tt = active ? t : T - 1;  // inactive waves mirror a valid query, store nothing
  const int bt = b * T + tt;
  const int vis = kv_len - T + tt + 1;
  const int vis_max = kv_len - T + min(T - 1, (blockIdx.y % groups_per_b) * kQB + kQB - 1) + 1;

  typename E::frag a[NH][NS];
  const uint8_t* qrow = q_idx + (size_t)bt * HI * DI * E::bytes;
#pragma unroll
  for (int ht = 0; ht < NH; ht++)
#pragma unroll
    for (int s = 0; s < NS; s++)
      a[ht][s] = E::load(qrow + ((size_t)(ht * 16 + col) * DI + grp * (DI / 4) + 8 * s) * E::bytes);
  float wv[NH][4];
#pragma unroll
  for (int ht = 0; ht < NH; ht++)
#pragma unroll
    for (int r = 0; r < 4; r++) wv[ht][r] = w[(size_t)bt * HI + ht * 16 + 4 * grp + r];
  i32x8 a8[kUseK128<DT, DI> ? NH : 1];  // the 128-deep fp8 operands (the same bytes as a)
  if constexpr (kUseK128<DT, DI>)
#pragma unroll
    for (int ht = 0; ht < NH; ht++) a8[ht] = cat4(a[ht][0], a[ht][1], a[ht][2], a[ht][3]);

  const uint8_t* kbase = k_idx + (size_t)b * L_cap * ROWB;
  float* srow = scores + (size_t)bt * kv_len;
  const int k0 = blockIdx.x * keys_per_split;
  const int k1 = min(k0 + keys_per_split, kv_len);
  const int kend = min(k1, vis_max);  // keys any query of the group sees

  // Keys past the group's visible range are written as -inf without compute.
  for (int key = max(k0, kend) + lane; key < k1; key += kWave)
    if (active) srow[key] = -INFINITY;
  if (k0 >= kend) return;  // uniform over the workgroup

  // LDS byte offset of logical 16-byte chunk c of tile row r.
#define CLSA_CHUNK_AT(r, c) ((r) * ROWB + 16 * ((c) ^ (((r) / RPS) & (CHUNKS - 1))))
  // Tile of keys key0 .. key0 + kKT - 1 into buffer BUF: transfer m carries
  // tile bytes [1024 m, 1024 m + 1024), lane L the 16 bytes at 1024 m + 16 L,
  // i.e. row (1024 m + 16 L) / ROWB, physical chunk L % CHUNKS, which holds
  // the row's logical chunk (L % CHUNKS) ^ swizzle(row). Keys past kv_len
  // read the last key (their scores are not stored).
#define CLSA_ISSUE(key0, BUF)                                                                         \
  for (int m = wave; m < NI; m += kQB) {                                                              \
    const int r = (1024 * m + 16 * lane) / ROWB;                                                      \
    const int c = (lane % CHUNKS) ^ ((r / RPS) & (CHUNKS - 1));                                       \
    const uint8_t* src = kbase + (size_t)min((key0) + r, kv_len - 1) * ROWB + 16 * c;                \
    __builtin_amdgcn_global_load_lds(src, (lds_void*)((BUF) + 1024 * m), 16, 0, 0);                  \
  }
  // Tile at key `base` from buffer CUR, after the transfer of the next tile
  // into NXT is issued and the previous tile's scores are stored. The wait +
  // barrier make this tile's transfers (every wave's) visible and guarantee
  // every wave is done with NXT, which held the previous tile.
#define CLSA_TILE(base, CUR, NXT)                                                                     \
  {                                                                                                   \
    __builtin_amdgcn_s_waitcnt(0x0070); /* vmcnt(0) lgkmcnt(0) */                                    \
    asm volatile("s_barrier" ::: "memory");                                                           \
    if ((base) + kKT < kend) { CLSA_ISSUE((base) + kKT, NXT) }                                        \
    _Pragma("unroll") for (int r = 0; r < NR; r++)                                                    \
      if (active && prev_key[r] < k1) srow[prev_key[r]] = prev_key[r] < vis ? prev_res[r] : -INFINITY; \
    float vs[kKT / 16];                                                                               \
    _Pragma("unroll") for (int j = 0; j < kKT / 16; j++) {                                            \
      f32x4 acc[NH];                                                                                  \
      _Pragma("unroll") for (int ht = 0; ht < NH; ht++) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};          \
      const int r = j * 16 + col;                                                                     \
      if constexpr (kUseK128<DT, DI>) {                                                               \
        typename E::frag bf[NS];                                                                      \
        _Pragma("unroll") for (int s = 0; s < NS; s++) {                                              \
          const int off = grp * (ROWB / 4) + 8 * s * E::bytes;                                        \
          bf[s] = E::load((CUR) + CLSA_CHUNK_AT(r, off / 16) + off % 16);                             \
        }                                                                                             \
        const i32x8 b8 = cat4(bf[0], bf[1], bf[2], bf[3]);                                            \
        _Pragma("unroll") for (int ht = 0; ht < NH; ht++) acc[ht] = mfma_fp8_k128(a8[ht], b8, acc[ht]); \
      } else {                                                                                        \
        _Pragma("unroll") for (int s = 0; s < NS; s++) {                                              \
          const int off = grp * (ROWB / 4) + 8 * s * E::bytes;                                        \
          const typename E::frag bf = E::load((CUR) + CLSA_CHUNK_AT(r, off / 16) + off % 16);         \
          _Pragma("unroll") for (int ht = 0; ht < NH; ht++) acc[ht] = E::mfma(a[ht][s], bf, acc[ht]); \
        }                                                                                             \
      }                                                                                               \
      float v = 0.f;                                                                                  \
      _Pragma("unroll") for (int ht = 0; ht < NH; ht++)                                               \
        _Pragma("unroll") for (int q = 0; q < 4; q++) v += wv[ht][q] * relu(acc[ht][q]);              \
      vs[j] = v;                                                                                      \
    }                                                                                                 \
    _Pragma("unroll") for (int r = 0; r < NR; r++) {                                                  \
      prev_res[r] = group4_transpose_sum(vs[4 * r], vs[4 * r + 1], vs[4 * r + 2], vs[4 * r + 3]);     \
      prev_key[r] = (base) + 64 * r + grp * 16 + col;                                                 \
    }                                                                                                 \
  }

  int prev_key[NR];  // the previous tile's results, stored during the next tile
  float prev_res[NR];
#pragma unroll
  for (int r = 0; r < NR; r++) {
    prev_key[r] = k1;  // nothing to store before the first tile
    prev_res[r] = 0.f;
  }
  CLSA_ISSUE(k0, tile0)
  for (int base = k0; base < kend; base += 2 * kKT) {  // uniform over the workgroup
    CLSA_TILE(base, tile0, tile1)
    if (base + kKT >= kend) break;
    CLSA_TILE(base + kKT, tile1, tile0)
  }
#pragma unroll
  for (int r = 0; r < NR; r++)
    if (active && prev_key[r] < k1) srow[prev_key[r]] = prev_key[r] < vis ? prev_res[r] : -INFINITY;
#undef CLSA_TILE
#undef CLSA_ISSUE
#undef CLSA_CHUNK_AT
}

// Float32 indexer (small head counts): one thread per key, the query's heads
// and weights staged in LDS. grid: (ceil(kv_len/256), B*T), block 256,
// dynamic LDS (H*D + H) floats.
constexpr int kF32Threads = 256;
__global__ __launch_bounds__(kF32Threads) void idx_score_f32(const float* __restrict__ q_idx,
                                                     const float* __restrict__ k_idx,
                                                     const float* __restrict__ w,
                                                     float* __restrict__ scores, int T, int H,
                                                     int D, int kv_len, int L_cap,
                                                     uint32_t* __restrict__ zero_p, int zero_n) {
  extern __shared__ float sh[];
  if (zero_n) zero_share(zero_p, zero_n, kF32Threads);
  const int bt = blockIdx.y;
  const int b = bt / T, t = bt % T;
  const int vis = kv_len - T + t + 1;
  for (int i = threadIdx.x; i < H * D; i += kF32Threads) sh[i] = q_idx[(size_t)bt * H * D + i];
  for (int i = threadIdx.x; i < H; i += kF32Threads) sh[H * D + i] = w[(size_t)bt * H + i];
  __syncthreads();
  const int s = blockIdx.x * kF32Threads + threadIdx.x;
  if (s >= kv_len) return;
  float* out = scores + (size_t)bt * kv_len + s;
  if (s >= vis) {
    *out = -INFINITY;
    return;
  }
  const float* kr = k_idx + ((size_t)b * L_cap + s) * D;
  float total = 0.f;
  for (int h = 0; h < H; h++) {
    float dot = 0.f;
    for (int d = 0; d < D; d++) dot = fmaf(sh[h * D + d], kr[d], dot);
    total = fmaf(sh[H * D + h], fmaxf(dot, 0.f), total);
  }
  *out = total;
}

template <int DT, int DI, int HI>
int launch_mfma(const void* q, const void* k, const float* w, float* scores, int B, int T,
                int kv_len, int L_cap, const ZeroJob& z, hipStream_t stream) {
  if (T >= kQB) {
    // Split the keys so that about 4096 workgroups run (16 per CU; at least 8
    // key tiles each). Measured on 2048 queries x 133120 keys: 3.09 ms against
    // 3.12 / 3.14 / 3.40 ms for 2048 / 512 / 256 workgroups and 3.16 ms for
    // 16384; on 2 x 2048 queries x 65536 keys 3.02 ms (8192) against 3.29 (512).
    const int groups = B * ((T + kQB - 1) / kQB);
    int splits = (4096 + groups - 1) / groups;
    constexpr int kKT = key_tile(DI * IdxElem<DT>::bytes);
    const int max_splits = (kv_len + kKT * 8 - 1) / (kKT * 8);  // at least 8 tiles per split
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
    int keys = (kv_len + splits - 1) / splits;
    keys = (keys + kKT - 1) / kKT * kKT;
    splits = (kv_len + keys - 1) / keys;
    dim3 grid(splits, groups);
    hipLaunchKernelGGL((idx_score_multi<DT, DI, HI>), grid, dim3(kQB * kWave), 0, stream,
                       static_cast<const uint8_t*>(q), static_cast<const uint8_t*>(k), w, scores, T,
                       kv_len, L_cap, keys, z.p, z.n);
    return check_launch("idx_score_multi");
  }
  // About one workgroup per CU (256 in all) measured best at every decode
  // shape: B=4 x 131072 keys 24.6 us at 2048 keys per workgroup (26.1 at
  // 1024, 35.0 at 4096); B=8 x 32768 13.9 us at 1024 (15.6 at 512, 19.9 at
  // 2048); B=16 x 65536 46.8 us at 4096 (50.8 at 1024).
  const long total = (long)B * T * kv_len;
  int keys_per_wg = (int)((total / 256 + kKeysPerWaveIter - 1) / kKeysPerWaveIter * kKeysPerWaveIter);
  keys_per_wg = std::max(keys_per_wg, 4 * kKeysPerWaveIter);
  dim3 grid((kv_len + keys_per_wg - 1) / keys_per_wg, B * T);
  hipLaunchKernelGGL((idx_score_mfma<DT, DI, HI>), grid, dim3(kIdxThreads), 0, stream,
                     static_cast<const uint8_t*>(q), static_cast<const uint8_t*>(k), w, scores, T,
                     kv_len, L_cap, keys_per_wg, z.p, z.n);
  return check_launch("idx_score_mfma");
}

template <int DT, int DI>
int dispatch_heads(int H_I, const void* q, const void* k, const float* w, float* scores, int B,
                   int T, int kv_len, int L_cap, const ZeroJob& z, hipStream_t stream) {
  switch (H_I) {
    case 16: return launch_mfma<DT, DI, 16>(q, k, w, scores, B, T, kv_len, L_cap, z, stream);
    case 32: return launch_mfma<DT, DI, 32>(q, k, w, scores, B, T, kv_len, L_cap, z, stream);
    case 48: return launch_mfma<DT, DI, 48>(q, k, w, scores, B, T, kv_len, L_cap, z, stream);
    case 64: return launch_mfma<DT, DI, 64>(q, k, w, scores, B, T, kv_len, L_cap, z, stream);
  }
  return set_error(CLSA_ERR_UNSUPPORTED, "index_score: H_I=%d", H_I);
}

template <int DT>
int dispatch_dim(int H_I, int D_I, const void* q, const void* k, const float* w, float* scores,
                 int B, int T, int kv_len, int L_cap, const ZeroJob& z, hipStream_t stream) {
  if (D_I == 64) return dispatch_heads<DT, 64>(H_I, q, k, w, scores, B, T, kv_len, L_cap, z, stream);
  if (D_I == 128) return dispatch_heads<DT, 128>(H_I, q, k, w, scores, B, T, kv_len, L_cap, z, stream);
  return set_error(CLSA_ERR_UNSUPPORTED, "index_score: D_I=%d", D_I);
}

}  // namespace

bool index_score_supported(int idx_dtype, int H_I, int D_I) {
  if (idx_dtype == CLSA_F32) return H_I >= 1 && D_I >= 1 && H_I * D_I <= 8192;
  if (idx_dtype == CLSA_BF16 || idx_dtype == CLSA_FP8_E4M3FN)
    return (H_I == 16 || H_I == 32 || H_I == 48 || H_I == 64) && (D_I == 64 || D_I == 128);
  return false;
}

int launch_index_score(const void* q_idx, const void* k_idx, int idx_dtype, const float* w,
                       float* scores, int B, int T, int H_I, int D_I, int kv_len, int L_cap,
                       const ZeroJob& z, hipStream_t stream) {
  if (idx_dtype == CLSA_F32) {
    dim3 grid((kv_len + kF32Threads - 1) / kF32Threads, B * T);
    size_t lds = sizeof(float) * ((size_t)H_I * D_I + H_I);
    hipLaunchKernelGGL(idx_score_f32, grid, dim3(kF32Threads), lds, stream,
                       static_cast<const float*>(q_idx), static_cast<const float*>(k_idx), w,
                       scores, T, H_I, D_I, kv_len, L_cap, z.p, z.n);
    return check_launch("idx_score_f32");
  }
  if (idx_dtype == CLSA_BF16)
    return dispatch_dim<CLSA_BF16>(H_I, D_I, q_idx, k_idx, w, scores, B, T, kv_len, L_cap, z, stream);
  return dispatch_dim<CLSA_FP8_E4M3FN>(H_I, D_I, q_idx, k_idx, w, scores, B, T, kv_len, L_cap, z,
                                       stream);
}

}  // namespace clsa
