// block_attn.hip — dense attention over the blocks of a block-union table,
// on gfx950 matrix cores (CompactAttention summary, "Méthodologie",
// execution step: the per-group block table is handed to a dense kernel as
// kv_indptr / kv_indices and the blocks are read in place).
//
// Query (b, t), head h of KV group g attends, with causal masking, to every
// position s < kv_len - T + t + 1 of the blocks listed for (b, g).
//
// One workgroup = (tile of 256 / G queries x the G heads of KV group g, i.e.
// 256 query rows; g; b), 8 waves of 32 rows (two 16-row MFMA column tiles,
// so every K and V fragment read from LDS feeds two products). The KV
// positions of the table are consumed in tiles of 64 positions (any block
// size; a tile can span blocks). K and V rows go from memory straight to LDS
// (global_load_lds, 16 bytes per lane, no registers), three tiles in flight;
// within a 256-byte row the 16-byte chunks are XOR-swizzled by row so that
// the operand reads below touch distinct banks.
//
// MFMA v_mfma_f32_16x16x32_bf16 operand layout (wave64): lane l supplies row
// l%16 of A and column l%16 of B for the k-slice l/16 (8 slots), and result
// (i, j) lands in lane j + 16*(i/4), slot i%4. The k-index carried by a
// (lane group, slot) pair is free as long as A and B agree.
//   S^T[key, row] = K[key, :] . Q[row, :]: A = K (16 keys x 32 d; lane reads 16
//     contiguous bytes of a key row), B = Q^T (query row l%16 of column tile
//     c, held in VGPRs). Lane l ends up with row l%16 of tile c and keys
//     4*(l/16) + r + 16*nt.
//   O^T[d, row] += V^T[d, keys] . P^T[keys, row]: B = P straight from the
//     lane's own S^T values (row l%16, its 16 keys; slot e of k-step ks is key
//     4*(l/16) + e%4 + 16*(2*ks + e/4)); A = V^T, read from the row-major V
//     tile with the LDS transpose read ds_read_b64_tr_b16: within each 16
//     lanes, lane i names the 4 elements V[key_{i/4}][d0 + 4*(i%4) + 0..3] and
//     lane 4a+b receives element b of lanes a, a+4, a+8, a+12, i.e. the 4
//     keys at d = d0 + 4a + b.
// So each lane owns one query row per column tile throughout: the row max and
// sum need only the 4 lanes l%16 + {0,16,32,48}, and the rescale of O is a
// per-lane scalar. Softmax in the log2 domain, fp32; P is rounded to bf16 for
// the PV product.
#include "kernels.h"

namespace clsa {
namespace {

constexpr int kD = 128;
constexpr int kWaves = 8;
constexpr int kRowsW = 32;              // query rows per wave (two MFMA column tiles)
constexpr int kRows = kWaves * kRowsW;  // query rows per workgroup
constexpr int kKT = 64;                 // KV positions per tile
constexpr int kRowB = kD * 2;           // bytes per K or V row (unpadded, swizzled)
constexpr int kTileB = kKT * kRowB;     // 16 KiB per K or V tile
constexpr int kBufs = 3;                // tiles in flight
constexpr float kLog2e = 1.4426950408889634f;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
constexpr float kLn2 = 0.6931471805599453f;

// Two floats to bf16 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// Byte offset of logical 16-byte chunk c of tile row r (chunks XOR-swizzled
// by row: K by r % 8, V by 2 * (r % 4), which keeps chunk pairs together).
__device__ __forceinline__ int k_chunk_at(int r, int c) { return r * kRowB + 16 * (c ^ (r & 7)); }
__device__ __forceinline__ int v_chunk_at(int r, int c) { return r * kRowB + 16 * (c ^ (2 * (r & 3))); }

// Online softmax of one column tile's 16 scores per lane (4 key tiles x 4),
// the row spread over the 4 lanes that hold it: updates the running max m
// and this lane's share l of the row sum, writes P as bf16 pairs in the slot
// order of the PV k-steps and returns the rescale factor of the
// accumulators. MASK: positions kp (this lane's 16 keys) outside [0, vis)
// count as -inf. Without it (every key valid and visible; kp unused) the max
// runs on the raw scores (the scale is positive) and exp2 takes
// fma(s, scale, -max).
template <bool MASK>
__device__ __forceinline__ float tile_softmax(f32x4 (&sc)[4], const int (&kp)[4][4], int vis,
                                              float c_log2, float& m, float& l, uint32_t (&pp)[8]) {
  float mt_max = -INFINITY;
#pragma unroll
  for (int nt = 0; nt < 4; nt++)
#pragma unroll
    for (int r = 0; r < 4; r++) {
      if constexpr (MASK) {
        const int p = kp[nt][r];
        sc[nt][r] = (p >= 0 && p < vis) ? sc[nt][r] * c_log2 : -INFINITY;
      }
      mt_max = fmaxf(mt_max, sc[nt][r]);
    }
  if constexpr (!MASK) mt_max *= c_log2;
  {  // max over the row's 4 lanes (l, l^16, l^32, l^48) by lane swaps
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt_max), __float_as_uint(mt_max), false, false);
    mt_max = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(mt_max), __float_as_uint(mt_max), false, false);
    mt_max = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
  }
  const float mn = fmaxf(m, mt_max);
  const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - mn);
  m = mn;
  float psum = 0.f;
#pragma unroll
  for (int nt = 0; nt < 4; nt++) {
    float p4[4];
#pragma unroll
    for (int r = 0; r < 4; r++) {
      if constexpr (MASK)
        p4[r] = sc[nt][r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[nt][r] - mn);
      else
        p4[r] = __builtin_amdgcn_exp2f(fmaf(sc[nt][r], c_log2, -mn));
      psum += p4[r];
    }
    pp[2 * nt] = pack_bf16(p4[0], p4[1]);
    pp[2 * nt + 1] = pack_bf16(p4[2], p4[3]);
  }
  l = l * alpha + psum;
  return alpha;
}

// grid (ceil(T / (kRows / G)), Hkv, B), block 512.
template <int G>
__global__ __launch_bounds__(kWaves * kWave) void block_attn_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ kv_indptr, const int32_t* __restrict__ kv_indices, int block,
    uint16_t* __restrict__ out, float* __restrict__ lse, int T, int Hkv, int kv_len, int L_cap,
    float c_log2, int head_major) {
  // Three tile buffers as separate LDS objects: the compiler then knows a
  // read of one buffer does not depend on the transfers into the others.
  __shared__ __attribute__((aligned(16))) uint8_t kt0[kTileB], kt1[kTileB], kt2[kTileB];
  __shared__ __attribute__((aligned(16))) uint8_t vt0[kTileB], vt1[kTileB], vt2[kTileB];
  __shared__ __attribute__((aligned(16))) int sp0[kKT], sp1[kKT], sp2[kKT];

  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int col = lane % 16, grp = lane / 16;
  const int g = blockIdx.y, b = blockIdx.z;
  const int Hq = Hkv * G;
  const int t0 = blockIdx.x * (kRows / G);
  const int vis_max = kv_len - T + min(T - 1, t0 + kRows / G - 1) + 1;

  // This lane's two query rows (column tiles c = 0, 1): row r of the
  // workgroup is query t0 + r / G, head g*G + r % G.
  int vis[2];
  bool active[2];
  size_t row[2];
  bf16x8 qf[2][4];
#pragma unroll
  for (int c = 0; c < 2; c++) {
    const int r = wave * kRowsW + 16 * c + col;
    const int t = t0 + r / G;
    const int h = g * G + r % G;
    active[c] = t < T;
    const int tq = active[c] ? t : T - 1;
    vis[c] = kv_len - T + tq + 1;
    row[c] = ((size_t)b * T + tq) * Hq + h;
#pragma unroll
    for (int ks = 0; ks < 4; ks++)
      qf[c][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(q + row[c] * kD + 8 * grp + 32 * ks));
  }

  // Smallest visible length over the wave's rows (inactive rows see every
  // key), uniform over the wave.
  int vis_min = min(vis[0], vis[1]);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) vis_min = min(vis_min, __shfl_xor(vis_min, off, kWave));
  vis_min = __builtin_amdgcn_readfirstlane(vis_min);

  f32x4 o[2][8];  // O^T tiles: lane holds d = 16*mt + 4*grp + r of its row in tile c
#pragma unroll
  for (int c = 0; c < 2; c++)
#pragma unroll
    for (int mt = 0; mt < 8; mt++) o[c][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};  // l: this lane's share of the row sum

  const int tab = b * Hkv + g;
  const int32_t* list = kv_indices + kv_indptr[tab];
  const int npos = (kv_indptr[tab + 1] - kv_indptr[tab]) * block;
  // Token-major [B, L_cap, Hkv, D]: a token's rows of the Hkv heads are
  // adjacent. Head-major [B, Hkv, L_cap, D]: each (b, g) is one contiguous
  // [L_cap, D] slab, so a block of positions is one contiguous piece.
  const size_t head0 = head_major ? ((size_t)b * Hkv + g) * L_cap * kD : ((size_t)b * L_cap * Hkv + g) * kD;
  const uint16_t* kbase = kc + head0;
  const uint16_t* vbase = vc + head0;
  const size_t tok = head_major ? (size_t)kD : (size_t)Hkv * kD;
  // Table index i -> cache position, or -1 past the table or past kv_len
  // (shift and mask when the block size is a power of two).
  const int bshift = (block & (block - 1)) == 0 ? __builtin_ctz(block) : -1;
  // Blocks of >= 64 positions (a power of two): the 64 rows of a tile lie in
  // one block, whose id is read with a scalar load (outside the vector-memory
  // counter that tracks the tile transfers).
  const bool tile_in_block = bshift >= 6;
  auto table_pos = [&](int tile, int r) -> int {
    const int i = tile * kKT + r;
    if (i >= npos) return -1;
    int p;
    if (tile_in_block) {
      const int blk = __builtin_amdgcn_readfirstlane((tile * kKT) >> bshift);
      p = (list[blk] << bshift) + (i & (block - 1));
    } else {
      p = bshift >= 0 ? (list[i >> bshift] << bshift) + (i & (block - 1)) : list[i / block] * block + i % block;
    }
    return p < kv_len ? p : -1;
  };

  int end = npos;
  {  // positions come in ascending order: stop at the first tile past every row
    int lo = 0, hi = npos;  // first table index whose position is >= vis_max
    while (lo < hi) {
      const int mid = (lo + hi) / 2;
      if (list[mid / block] * block + mid % block < vis_max) lo = mid + 1; else hi = mid;
    }
    end = lo;
  }
  const int ntiles = (end + kKT - 1) / kKT;

  // Tile `tile` into buffer `buf`: wave w moves rows 8w .. 8w+7 of K and V
  // (two 4-row, 1 KiB pieces each); lane L of a piece carries row L/16,
  // physical chunk L%16, i.e. logical chunk (L%16) ^ swizzle(row).
  // Tile `tile` into the buffers KT/VT/SP: wave w moves rows 8w .. 8w+7 of
  // K and V (two 4-row, 1 KiB pieces each); lane L of a piece carries row
  // L/16, physical chunk L%16, i.e. logical chunk (L%16) ^ swizzle(row). The
  // buffers are named directly (separate LDS objects), so the compiler knows
  // a transfer into one buffer does not feed reads of another.
#define CLSA_ISSUE(tile, KT, VT, SP)                                                                   \
  _Pragma("unroll") for (int j = 0; j < 2; j++) {                                                     \
    const int r = 8 * wave + 4 * j + lane / 16;                                                        \
    const int pos = table_pos(tile, r);                                                                \
    const size_t src = (size_t)max(pos, 0) * tok;                                                      \
    const int ck = (lane % 16) ^ (r & 7), cv = (lane % 16) ^ (2 * (r & 3));                            \
    __builtin_amdgcn_global_load_lds(kbase + src + 8 * ck, (lds_void*)((KT) + (8 * wave + 4 * j) * kRowB), 16, 0, 0); \
    __builtin_amdgcn_global_load_lds(vbase + src + 8 * cv, (lds_void*)((VT) + (8 * wave + 4 * j) * kRowB), 16, 0, 0); \
    if (lane % 16 == 0) (SP)[r] = pos;                                                                 \
  }
  // Tile `it` from buffers KB/VB/SP, after issuing tile it+2 into KN/VN/SPN.
  // First wait until this wave's transfers of tile `it` have landed (the next
  // tile's 4 may still be in flight) and its position writes are done; the
  // barrier then makes every wave's visible and guarantees every wave is done
  // with the buffer the issue overwrites.
#define CLSA_TILE(it, KB, VB, SP, KN, VN, SPN)                                                           \
  {                                                                                                      \
    if ((it) + 1 < ntiles) __builtin_amdgcn_s_waitcnt(0x0074); /* vmcnt(4) lgkmcnt(0) */                \
    else __builtin_amdgcn_s_waitcnt(0x0070);                   /* vmcnt(0) lgkmcnt(0) */                \
    asm volatile("s_barrier" ::: "memory");                                                              \
    if ((it) + kBufs - 1 < ntiles) { CLSA_ISSUE((it) + kBufs - 1, KN, VN, SPN) }                         \
    /* S^T for 4 tiles of 16 keys and both column tiles. */                                                    \
    f32x4 s[2][4];                                                                                             \
_Pragma("unroll")                                                                                              \
    for (int nt = 0; nt < 4; nt++) {                                                                           \
      s[0][nt] = f32x4{0.f, 0.f, 0.f, 0.f};                                                                    \
      s[1][nt] = f32x4{0.f, 0.f, 0.f, 0.f};                                                                    \
_Pragma("unroll")                                                                                              \
      for (int ks = 0; ks < 4; ks++) {                                                                         \
        const bf16x8 kf = __builtin_bit_cast(                                                                  \
            bf16x8, *reinterpret_cast<const uint4*>((KB) + k_chunk_at(16 * nt + col, grp + 4 * ks)));          \
        s[0][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[0][ks], s[0][nt], 0, 0, 0);                  \
        s[1][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[1][ks], s[1][nt], 0, 0, 0);                  \
      }                                                                                                        \
    }                                                                                                          \
    bf16x8 pf[2][2];  /* P^T operands per column tile and k-step */                                            \
    int kp[4][4];     /* positions of this lane's 16 keys */                                                   \
_Pragma("unroll")                                                                                              \
    for (int nt = 0; nt < 4; nt++) {                                                                           \
      const int4 v4 = *reinterpret_cast<const int4*>(&(SP)[16 * nt + 4 * grp]);                                \
      kp[nt][0] = v4.x; kp[nt][1] = v4.y; kp[nt][2] = v4.z; kp[nt][3] = v4.w;                                  \
    }                                                                                                          \
    /* A tile whose positions are all valid and visible to every row of the wave (its positions               \
       ascend, so its first and last decide) takes the unmasked softmax. */                                   \
    const int p_first = __builtin_amdgcn_readfirstlane((SP)[0]);                                              \
    const int p_last = __builtin_amdgcn_readfirstlane((SP)[kKT - 1]);                                         \
_Pragma("unroll")                                                                                             \
    for (int c = 0; c < 2; c++) {                                                                             \
      uint32_t pp[8];  /* P as bf16 pairs, slot order of the PV k-steps */                                    \
      float alpha;                                                                                            \
      if (p_first >= 0 && p_last >= 0 && p_last < vis_min)                                                    \
        alpha = tile_softmax<false>(s[c], kp, vis[c], c_log2, m[c], l[c], pp);                                \
      else                                                                                                    \
        alpha = tile_softmax<true>(s[c], kp, vis[c], c_log2, m[c], l[c], pp);                                 \
      if (__ballot(alpha != 1.f) != 0) {  /* some row's max moved: rescale */                                 \
_Pragma("unroll")                                                                                             \
        for (int mt = 0; mt < 8; mt++) o[c][mt] *= alpha;                                                     \
      }                                                                                                       \
_Pragma("unroll")                                                                                             \
      for (int ks = 0; ks < 2; ks++)                                                                          \
        pf[c][ks] = __builtin_bit_cast(bf16x8, uint4{pp[4 * ks], pp[4 * ks + 1], pp[4 * ks + 2], pp[4 * ks + 3]});\
    }                                                                                                         \
    /* O^T += V^T P^T over 2 k-steps of 32 keys, both column tiles per V^T */                                  \
    /* fragment. Lane (grp, i) names V[4*grp + i/4 + 32*ks + 16*h][16*mt + 4*(i%4)]. */                        \
    const int vkey = 4 * grp + col / 4, vd4 = 4 * (col % 4);                                                   \
_Pragma("unroll")                                                                                              \
    for (int ks = 0; ks < 2; ks++) {                                                                           \
_Pragma("unroll")                                                                                              \
      for (int mt = 0; mt < 8; mt++) {                                                                         \
        const int d = 16 * mt + vd4;                                                                           \
        const int r0 = vkey + 32 * ks, r1 = r0 + 16;                                                           \
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(                                              \
            (__attribute__((address_space(3))) v4i16*)((VB) + v_chunk_at(r0, d / 8) + 2 * (d % 8)));           \
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(                                              \
            (__attribute__((address_space(3))) v4i16*)((VB) + v_chunk_at(r1, d / 8) + 2 * (d % 8)));           \
        const uint2 lo2 = __builtin_bit_cast(uint2, lo), hi2 = __builtin_bit_cast(uint2, hi);                  \
        const bf16x8 vf = __builtin_bit_cast(bf16x8, uint4{lo2.x, lo2.y, hi2.x, hi2.y});                       \
        o[0][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[0][ks], o[0][mt], 0, 0, 0);                  \
        o[1][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[1][ks], o[1][mt], 0, 0, 0);                  \
      }                                                                                                        \
    }                                                                                                          \
  }
  if (ntiles > 0) { CLSA_ISSUE(0, kt0, vt0, sp0) }
  if (ntiles > 1) { CLSA_ISSUE(1, kt1, vt1, sp1) }
  for (int it = 0; it < ntiles; it += kBufs) {  // uniform over the workgroup; buffers it % 3
    CLSA_TILE(it, kt0, vt0, sp0, kt2, vt2, sp2)
    if (it + 1 >= ntiles) break;
    CLSA_TILE(it + 1, kt1, vt1, sp1, kt0, vt0, sp0)
    if (it + 2 >= ntiles) break;
    CLSA_TILE(it + 2, kt2, vt2, sp2, kt1, vt1, sp1)
  }
#undef CLSA_TILE
#undef CLSA_ISSUE
  // Row sums over each row's 4 lanes, then normalise and store.
#pragma unroll
  for (int c = 0; c < 2; c++) {
    float lc = l[c];
    lc += __shfl_xor(lc, 16, kWave);
    lc += __shfl_xor(lc, 32, kWave);
    if (!active[c]) continue;
    const float inv = lc > 0.f ? 1.f / lc : 0.f;
    uint16_t* orow = out + row[c] * kD;
#pragma unroll
    for (int mt = 0; mt < 8; mt++) {
      uint2 v;
      v.x = pack_bf16(o[c][mt][0] * inv, o[c][mt][1] * inv);
      v.y = pack_bf16(o[c][mt][2] * inv, o[c][mt][3] * inv);
      *reinterpret_cast<uint2*>(orow + 16 * mt + 4 * grp) = v;
    }
    if (grp == 0 && lse) lse[row[c]] = lc > 0.f ? (m[c] + log2f(lc)) * kLn2 : -INFINITY;
  }
}

template <int G>
int launch_g(const void* q, const void* kc, const void* vc, const int32_t* indptr,
             const int32_t* indices, int block, void* out, float* lse, int B, int T, int Hkv,
             int kv_len, int L_cap, float c_log2, bool head_major, hipStream_t stream) {
  dim3 grid((T + kRows / G - 1) / (kRows / G), Hkv, B);
  hipLaunchKernelGGL((block_attn_mfma<G>), grid, dim3(kWaves * kWave), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
                     static_cast<const uint16_t*>(vc), indptr, indices, block,
                     static_cast<uint16_t*>(out), lse, T, Hkv, kv_len, L_cap, c_log2, head_major ? 1 : 0);
  return check_launch("block_attn_mfma");
}

}  // namespace

int launch_block_attn_mfma(const void* q, const void* kc, const void* vc,
                           const int32_t* kv_indptr, const int32_t* kv_indices, int block,
                           void* out, float* lse, int B, int T, int Hq, int Hkv, int D, int kv_len,
                           int L_cap, float scale, bool head_major, hipStream_t stream) {
  const float c_log2 = (scale > 0.f ? scale : 1.f / sqrtf((float)D)) * kLog2e;
  switch (Hq / Hkv) {
    case 1: return launch_g<1>(q, kc, vc, kv_indptr, kv_indices, block, out, lse, B, T, Hkv, kv_len, L_cap, c_log2, head_major, stream);
    case 2: return launch_g<2>(q, kc, vc, kv_indptr, kv_indices, block, out, lse, B, T, Hkv, kv_len, L_cap, c_log2, head_major, stream);
    case 4: return launch_g<4>(q, kc, vc, kv_indptr, kv_indices, block, out, lse, B, T, Hkv, kv_len, L_cap, c_log2, head_major, stream);
    case 8: return launch_g<8>(q, kc, vc, kv_indptr, kv_indices, block, out, lse, B, T, Hkv, kv_len, L_cap, c_log2, head_major, stream);
  }
  return set_error(CLSA_ERR_UNSUPPORTED, "block_paged_attn: Hq/Hkv=%d", Hq / Hkv);
}

}  // namespace clsa
