// block_attn.hip — dense attention over the blocks of a block-union table,
// on gfx950 matrix cores (CompactAttention summary, "Méthodologie",
// execution step: the per-group block table is handed to a dense kernel as
// kv_indptr / kv_indices and the blocks are read in place).
//
// Query (b, t), head h of KV group g attends, with causal masking, to every
// position s < kv_len - T + t + 1 of the blocks listed for (b, g).
//
// One workgroup = (tile of 128 / G queries x the G heads of KV group g, i.e.
// 128 query rows; g; b), 8 waves of 16 rows. The KV positions of the table are
// consumed in tiles of 64 positions (any block size; a tile can span blocks).
// Per tile, K rows go to LDS as they are in memory and V goes to LDS
// transposed (d-major); the next tile's rows are already in registers while
// the current one is computed.
//
// MFMA v_mfma_f32_16x16x32_bf16 operand layout (wave64): lane l supplies row
// l%16 of A and column l%16 of B for the k-slice l/16 (8 slots), and result
// (i, j) lands in lane j + 16*(i/4), slot i%4. The k-index carried by a
// (lane group, slot) pair is free as long as A and B agree.
//   S^T[key, row] = K[key, :] . Q[row, :]: A = K (16 keys x 32 d; lane reads 16
//     contiguous bytes of a key row), B = Q^T (query row l%16, held in VGPRs).
//     Lane l ends up with query row l%16 and keys 4*(l/16) + r + 16*nt.
//   O^T[d, row] += V^T[d, keys] . P^T[keys, row]: B = P straight from the
//     lane's own S^T values (row l%16, its 16 keys; slot e of k-step ks is key
//     4*(l/16) + e%4 + 16*(2*ks + e/4)); A = V^T (d row l%16 + 16*mt, the same
//     key slots: two 8-byte reads of the transposed tile).
// So each lane owns one query row throughout: the row max and sum need only
// the 4 lanes l%16 + {0,16,32,48}, and the rescale of O is a per-lane scalar.
// Softmax in the log2 domain, fp32; P is rounded to bf16 for the PV product.
#include "kernels.h"

namespace clsa {
namespace {

constexpr int kD = 128;
constexpr int kWaves = 8;
constexpr int kRows = kWaves * 16;      // query rows per workgroup
constexpr int kKT = 64;                 // KV positions per tile
constexpr int kKPitch = kD * 2 + 16;    // K tile row, bytes (padded)
constexpr int kVPitch = kKT * 2 + 8;    // V^T tile row (one d), bytes (padded)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// grid (ceil(T / (kRows / G)), Hkv, B), block 512.
template <int G>
__global__ __launch_bounds__(kWaves * kWave) void block_attn_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ kv_indptr, const int32_t* __restrict__ kv_indices, int block,
    uint16_t* __restrict__ out, float* __restrict__ lse, int T, int Hkv, int kv_len, int L_cap,
    float c_log2, int head_major) {
  constexpr int QPW = 16 / G;            // queries per wave
  __shared__ __attribute__((aligned(16))) uint8_t kt[kKT * kKPitch];
  __shared__ __attribute__((aligned(16))) uint8_t vt[kD * kVPitch];
  __shared__ int s_pos[kKT];

  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int col = lane % 16, grp = lane / 16;
  const int g = blockIdx.y, b = blockIdx.z;
  const int Hq = Hkv * G;
  const int t0 = blockIdx.x * (kRows / G);
  // This lane's query row: query t, head h.
  const int t = t0 + wave * QPW + col / G;
  const int h = g * G + col % G;
  const bool active = t < T;
  const int tq = active ? t : T - 1;
  const int vis = kv_len - T + tq + 1;
  const int vis_max = kv_len - T + min(T - 1, t0 + kRows / G - 1) + 1;
  const size_t row = ((size_t)b * T + tq) * Hq + h;

  // Q^T fragments (B operand of S^T): row col, d = 8*grp + e + 32*ks.
  bf16x8 qf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ks++)
    qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(q + row * kD + 8 * grp + 32 * ks));

  f32x4 o[8];  // O^T tiles: lane holds d = 16*mt + 4*grp + r of row col
#pragma unroll
  for (int mt = 0; mt < 8; mt++) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;  // l: this lane's share of the row sum

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

  // Staging: 64 rows x 16 chunks of 16 bytes for K and for V; thread c moves
  // chunks c and c + 512 of each (row = chunk / 16, d0 = 8 * (chunk % 16)).
  uint4 sk0, sk1, sv0, sv1;
  int sp0, sp1;
  // Table index i -> cache position, or -1 past the table or past kv_len.
#define CLSA_POS(i)                                                                      \
  ((i) >= npos ? -1                                                                      \
               : (list[(i) / block] * block + (i) % block < kv_len                       \
                      ? list[(i) / block] * block + (i) % block                          \
                      : -1))
#define CLSA_FETCH1(base, c, sk, sv, sp)                                                 \
  {                                                                                      \
    sp = CLSA_POS((base) + (c) / 16);                                                    \
    const size_t off = (size_t)max(sp, 0) * tok + 8 * ((c) % 16);                        \
    sk = *reinterpret_cast<const uint4*>(kbase + off);                                   \
    sv = *reinterpret_cast<const uint4*>(vbase + off);                                   \
  }
#define CLSA_COMMIT1(c, sk, sv, sp)                                                      \
  {                                                                                      \
    const int r = (c) / 16, d0 = 8 * ((c) % 16);                                         \
    *reinterpret_cast<uint4*>(&kt[r * kKPitch + d0 * 2]) = sk;                           \
    const uint32_t w4[4] = {sv.x, sv.y, sv.z, sv.w};                                     \
    _Pragma("unroll") for (int e = 0; e < 4; e++) {                                      \
      *reinterpret_cast<uint16_t*>(&vt[(d0 + 2 * e) * kVPitch + r * 2]) =                \
          (uint16_t)(w4[e] & 0xffffu);                                                   \
      *reinterpret_cast<uint16_t*>(&vt[(d0 + 2 * e + 1) * kVPitch + r * 2]) =            \
          (uint16_t)(w4[e] >> 16);                                                       \
    }                                                                                    \
    if ((c) % 16 == 0) s_pos[r] = sp;                                                    \
  }
  const int ca = threadIdx.x, cb = threadIdx.x + kWaves * kWave;
#define CLSA_FETCH(base)                      \
  CLSA_FETCH1(base, ca, sk0, sv0, sp0)        \
  CLSA_FETCH1(base, cb, sk1, sv1, sp1)
#define CLSA_COMMIT()                         \
  CLSA_COMMIT1(ca, sk0, sv0, sp0)             \
  CLSA_COMMIT1(cb, sk1, sv1, sp1)

  int end = npos;
  {  // positions come in ascending order: stop at the first tile past every row
    int lo = 0, hi = npos;  // first table index whose position is >= vis_max
    while (lo < hi) {
      const int mid = (lo + hi) / 2;
      if (list[mid / block] * block + mid % block < vis_max) lo = mid + 1; else hi = mid;
    }
    end = lo;
  }
  if (end > 0) {
    CLSA_FETCH(0)
  }
  for (int base = 0; base < end; base += kKT) {  // uniform over the workgroup
    __syncthreads();  // previous tile fully consumed
    CLSA_COMMIT()
    __syncthreads();
    if (base + kKT < end) {
      CLSA_FETCH(base + kKT)  // in flight during this tile's math
    }
    // S^T for 4 tiles of 16 keys.
    f32x4 s[4];
#pragma unroll
    for (int nt = 0; nt < 4; nt++) {
      s[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ks++) {
        const bf16x8 kf = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(&kt[(16 * nt + col) * kKPitch + (8 * grp + 32 * ks) * 2]));
        s[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], s[nt], 0, 0, 0);
      }
    }
    // Mask, scale, running max over this lane's 16 keys, then the row's 4 lanes.
    float mt_max = -INFINITY;
#pragma unroll
    for (int nt = 0; nt < 4; nt++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int p = s_pos[16 * nt + 4 * grp + r];
        const float x = (p >= 0 && p < vis) ? s[nt][r] * c_log2 : -INFINITY;
        s[nt][r] = x;
        mt_max = fmaxf(mt_max, x);
      }
    mt_max = fmaxf(mt_max, __shfl_xor(mt_max, 16, kWave));
    mt_max = fmaxf(mt_max, __shfl_xor(mt_max, 32, kWave));
    const float mn = fmaxf(m, mt_max);
    const float alpha = mn == -INFINITY ? 1.f : exp2f(m - mn);
    m = mn;
    float psum = 0.f;
    uint32_t pp[8];  // P as bf16 pairs, slot order of the PV k-steps
#pragma unroll
    for (int nt = 0; nt < 4; nt++) {
      float p4[4];
#pragma unroll
      for (int r = 0; r < 4; r++) {
        p4[r] = s[nt][r] == -INFINITY ? 0.f : exp2f(s[nt][r] - mn);
        psum += p4[r];
      }
      pp[2 * nt] = pack_bf16(p4[0], p4[1]);
      pp[2 * nt + 1] = pack_bf16(p4[2], p4[3]);
    }
    l = l * alpha + psum;
#pragma unroll
    for (int mt = 0; mt < 8; mt++)
#pragma unroll
      for (int r = 0; r < 4; r++) o[mt][r] *= alpha;
    // O^T += V^T P^T over 2 k-steps of 32 keys.
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
      const bf16x8 pf = __builtin_bit_cast(
          bf16x8, uint4{pp[4 * ks], pp[4 * ks + 1], pp[4 * ks + 2], pp[4 * ks + 3]});
#pragma unroll
      for (int mt = 0; mt < 8; mt++) {
        const uint8_t* vrow = &vt[(16 * mt + col) * kVPitch];
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow + (4 * grp + 16 * (2 * ks)) * 2);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + (4 * grp + 16 * (2 * ks + 1)) * 2);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, uint4{lo.x, lo.y, hi.x, hi.y});
        o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, o[mt], 0, 0, 0);
      }
    }
  }
#undef CLSA_POS
#undef CLSA_FETCH1
#undef CLSA_COMMIT1
#undef CLSA_FETCH
#undef CLSA_COMMIT
  // Row sum over the row's 4 lanes, then normalise and store.
  l += __shfl_xor(l, 16, kWave);
  l += __shfl_xor(l, 32, kWave);
  if (!active) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  uint16_t* orow = out + row * kD;
#pragma unroll
  for (int mt = 0; mt < 8; mt++) {
    uint2 v;
    v.x = pack_bf16(o[mt][0] * inv, o[mt][1] * inv);
    v.y = pack_bf16(o[mt][2] * inv, o[mt][3] * inv);
    *reinterpret_cast<uint2*>(orow + 16 * mt + 4 * grp) = v;
  }
  if (grp == 0 && lse) lse[row] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
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
