// sparse_attn.hip — softmax attention over the k selected cache rows.
//
// For query (b, t), head h and its KV head g = h / G:
//   out = sum_j softmax_j(scale * q . K[idx_j, g]) V[idx_j, g]
// over the entries of idx[b, t, :] that lie in the query's visible range
// (IndexCache summary, "1. Problématique": main attention runs over the k
// selected tokens; CLSA article, "Comment CLSA fonctionne": every layer
// reuses the one index).
//
// Work split: one workgroup per (query, KV head, split of the k entries).
// The G query heads of a KV head share every gathered row, so each row is
// read from HBM once per layer. A row of one KV head is D contiguous
// elements (token-major cache), gathered by 16 lanes with one 16-byte load
// each (bf16), four rows per wave instruction. Scores use v_dot2_f32_bf16
// on bf16 pairs and a 16-lane butterfly; softmax runs online in the log2
// domain, in float32, one rescale per 4-row step. Lane groups and waves are
// merged through shuffles and LDS; the splits of a (query, KV head) are
// merged by whichever workgroup finishes last (an atomic ticket), reading
// the partial states in split order so the result does not depend on
// scheduling. The ticket is returned to zero by that workgroup.
#include "kernels.h"

namespace clsa {
namespace {

constexpr int kAttnThreads = 256;  // 4 waves
constexpr int kD = 128;
constexpr int kRowsPerStep = 64;   // 4 waves x 4 lane groups x 4 rows
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

template <int DT>
struct AttnElem;
template <>
struct AttnElem<CLSA_BF16> {
  static constexpr int bytes = 2;
  struct Frag {
    uint4 u;  // 8 bf16
  };
  static __device__ __forceinline__ Frag load(const char* p) {
    return Frag{*reinterpret_cast<const uint4*>(p)};
  }
  static __device__ __forceinline__ float dot(const Frag& q, const Frag& k) {
    float s = 0.f;
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.u.x),
                                        __builtin_bit_cast(bf16x2, k.u.x), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.u.y),
                                        __builtin_bit_cast(bf16x2, k.u.y), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.u.z),
                                        __builtin_bit_cast(bf16x2, k.u.z), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.u.w),
                                        __builtin_bit_cast(bf16x2, k.u.w), s, false);
    return s;
  }
  static __device__ __forceinline__ void to_f32(const Frag& v, float* f) {
    f[0] = bf16_lo(v.u.x); f[1] = bf16_hi(v.u.x);
    f[2] = bf16_lo(v.u.y); f[3] = bf16_hi(v.u.y);
    f[4] = bf16_lo(v.u.z); f[5] = bf16_hi(v.u.z);
    f[6] = bf16_lo(v.u.w); f[7] = bf16_hi(v.u.w);
  }
  static __device__ __forceinline__ void store(void* out, size_t i, float x) {
    static_cast<uint16_t*>(out)[i] = (uint16_t)f32_to_bf16_rne(x);
  }
};
template <>
struct AttnElem<CLSA_F32> {
  static constexpr int bytes = 4;
  struct Frag {
    float4 a, b;  // 8 floats
  };
  static __device__ __forceinline__ Frag load(const char* p) {
    const float4* f = reinterpret_cast<const float4*>(p);
    return Frag{f[0], f[1]};
  }
  static __device__ __forceinline__ float dot(const Frag& q, const Frag& k) {
    float s = q.a.x * k.a.x;
    s = fmaf(q.a.y, k.a.y, s); s = fmaf(q.a.z, k.a.z, s); s = fmaf(q.a.w, k.a.w, s);
    s = fmaf(q.b.x, k.b.x, s); s = fmaf(q.b.y, k.b.y, s); s = fmaf(q.b.z, k.b.z, s);
    s = fmaf(q.b.w, k.b.w, s);
    return s;
  }
  static __device__ __forceinline__ void to_f32(const Frag& v, float* f) {
    f[0] = v.a.x; f[1] = v.a.y; f[2] = v.a.z; f[3] = v.a.w;
    f[4] = v.b.x; f[5] = v.b.y; f[6] = v.b.z; f[7] = v.b.w;
  }
  static __device__ __forceinline__ void store(void* out, size_t i, float x) {
    static_cast<float*>(out)[i] = x;
  }
};

__device__ __forceinline__ float sum16(float v) {
  v += __shfl_xor(v, 1, kWave);
  v += __shfl_xor(v, 2, kWave);
  v += __shfl_xor(v, 4, kWave);
  v += __shfl_xor(v, 8, kWave);
  return v;
}

// exp2(a - b) with exp2(-inf - -inf) taken as 1 (both states empty).
__device__ __forceinline__ float rescale(float a, float b) {
  return b == -INFINITY ? 1.f : exp2f(a - b);
}

// Where the attended positions come from.
// IdxSrc: the k entries of the query's index row.
struct IdxSrc {
  const int32_t* idx;
  int k;
  const int32_t* row;
  __device__ void bind(int bt, int g) { row = idx + (size_t)bt * k; }
  __device__ int count() const { return k; }
  __device__ int pos(int r) const { return row[r]; }
};
// BlockSrc: every position of the blocks listed for (b, g) in a block table
// (kv_indptr / kv_indices), in table order.
struct BlockSrc {
  const int32_t* indptr;
  const int32_t* indices;
  int block, T, Hkv;
  const int32_t* list;
  int n;
  __device__ void bind(int bt, int g) {
    const int u = (bt / T) * Hkv + g;
    list = indices + indptr[u];
    n = (indptr[u + 1] - indptr[u]) * block;
  }
  __device__ int count() const { return n; }
  __device__ int pos(int r) const { return list[r / block] * block + r % block; }
};

// grid (S, Hkv, B*T), block 256.
template <int DT, int G, class Src>
__global__ __launch_bounds__(kAttnThreads) void sparse_attn_kernel(
    const char* __restrict__ q, const char* __restrict__ kc, const char* __restrict__ vc,
    Src src, void* __restrict__ out, float* __restrict__ lse,
    int T, int Hkv, int kv_len, int L_cap, float c_log2, int rows_per_split,
    uint32_t* __restrict__ counters, float* __restrict__ partials) {
  using E = AttnElem<DT>;
  constexpr int ROW = kD * E::bytes;  // bytes of one KV head of one token
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int sub = lane % 16;   // element slice [8*sub, 8*sub + 8)
  const int rg = lane / 16;    // row group within the wave
  const int split = blockIdx.x, S = gridDim.x;
  const int g = blockIdx.y;
  const int bt = blockIdx.z;
  const int b = bt / T, t = bt % T;
  const int vis = kv_len - T + t + 1;
  const int Hq = Hkv * G;

  // This lane's slice of the G query heads.
  typename E::Frag qf[G];
#pragma unroll
  for (int h = 0; h < G; h++)
    qf[h] = E::load(q + (((size_t)bt * Hq + g * G + h) * kD + 8 * sub) * E::bytes);

  float m[G], l[G], o[G][8];
#pragma unroll
  for (int h = 0; h < G; h++) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e++) o[h][e] = 0.f;
  }

  src.bind(bt, g);
  const char* kb = kc + ((size_t)b * L_cap * Hkv + g) * ROW + 8 * sub * E::bytes;
  const char* vb = vc + ((size_t)b * L_cap * Hkv + g) * ROW + 8 * sub * E::bytes;
  const size_t tok = (size_t)Hkv * ROW;  // bytes between consecutive tokens
  const int r0 = split * rows_per_split;
  const int r1 = min(src.count(), r0 + rows_per_split);

  // wb is wave-uniform; lane group rg takes rows wb + 4*rg .. wb + 4*rg + 3.
  for (int wb = r0 + wave * 16; wb < r1; wb += kRowsPerStep) {
    const int base = wb + rg * 4;
    int pos[4];
    bool valid[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int r = base + i;
      const int p = r < r1 ? src.pos(r) : -1;
      valid[i] = p >= 0 && p < vis;
      pos[i] = valid[i] ? p : 0;
    }
    typename E::Frag kf[4], vf[4];
#pragma unroll
    for (int i = 0; i < 4; i++) kf[i] = E::load(kb + (size_t)pos[i] * tok);
#pragma unroll
    for (int i = 0; i < 4; i++) vf[i] = E::load(vb + (size_t)pos[i] * tok);
    float u[4][G];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int h = 0; h < G; h++) {
        const float s = sum16(E::dot(qf[h], kf[i]));
        u[i][h] = valid[i] ? s * c_log2 : -INFINITY;
      }
    float v[4][8];
#pragma unroll
    for (int i = 0; i < 4; i++) E::to_f32(vf[i], v[i]);
#pragma unroll
    for (int h = 0; h < G; h++) {
      const float mc = fmaxf(fmaxf(u[0][h], u[1][h]), fmaxf(u[2][h], u[3][h]));
      const float mn = fmaxf(m[h], mc);
      const float a = rescale(m[h], mn);
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; i++) p[i] = valid[i] ? exp2f(u[i][h] - mn) : 0.f;
      l[h] = l[h] * a + (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
      for (int e = 0; e < 8; e++) {
        float x = o[h][e] * a;
#pragma unroll
        for (int i = 0; i < 4; i++) x = fmaf(p[i], v[i][e], x);
        o[h][e] = x;
      }
      m[h] = mn;
    }
  }

  // Merge the 4 row groups of the wave (lanes sub, sub+16, sub+32, sub+48).
#pragma unroll
  for (int x = 16; x <= 32; x <<= 1) {
#pragma unroll
    for (int h = 0; h < G; h++) {
      const float m2 = __shfl_xor(m[h], x, kWave);
      const float l2 = __shfl_xor(l[h], x, kWave);
      const float mn = fmaxf(m[h], m2);
      const float a1 = rescale(m[h], mn), a2 = rescale(m2, mn);
      l[h] = l[h] * a1 + l2 * a2;
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const float o2 = __shfl_xor(o[h][e], x, kWave);
        o[h][e] = o[h][e] * a1 + o2 * a2;
      }
      m[h] = mn;
    }
  }

  // Merge the 4 waves through LDS: st[wave][h] = {m, l, o[128]}.
  __shared__ float st[4][G][kD + 2];
  __shared__ int s_last;
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < G; h++) {
#pragma unroll
      for (int e = 0; e < 8; e++) st[wave][h][2 + 8 * sub + e] = o[h][e];
      if (sub == 0) {
        st[wave][h][0] = m[h];
        st[wave][h][1] = l[h];
      }
    }
  }
  __syncthreads();

  const size_t unit = (size_t)bt * Hkv + g;  // (query, KV head)
  float* part = partials + (unit * S + split) * (G * (kD + 2));
  for (int item = threadIdx.x; item < G * kD; item += blockDim.x) {
    const int h = item / kD, d = item % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; w++) M = fmaxf(M, st[w][h][0]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < 4; w++) {
      const float a = rescale(st[w][h][0], M);
      L += st[w][h][1] * a;
      O += st[w][h][2 + d] * a;
    }
    if (S == 1) {
      const size_t oi = ((size_t)bt * Hq + g * G + h) * kD + d;
      E::store(out, oi, L > 0.f ? O / L : 0.f);
      if (d == 0 && lse) lse[(size_t)bt * Hq + g * G + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
    } else {
      part[h * (kD + 2) + 2 + d] = O;
      if (d == 0) {
        part[h * (kD + 2)] = M;
        part[h * (kD + 2) + 1] = L;
      }
    }
  }
  if (S == 1) return;

  // Split combine by the last workgroup to finish this (query, KV head).
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = atomicAdd(&counters[unit], 1u) == (uint32_t)(S - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const float* pu = partials + unit * S * (G * (kD + 2));
  for (int item = threadIdx.x; item < G * kD; item += blockDim.x) {
    const int h = item / kD, d = item % kD;
    float M = -INFINITY;
    for (int s = 0; s < S; s++) M = fmaxf(M, pu[(size_t)s * G * (kD + 2) + h * (kD + 2)]);
    float L = 0.f, O = 0.f;
    for (int s = 0; s < S; s++) {
      const float* ps = pu + (size_t)s * G * (kD + 2) + h * (kD + 2);
      const float a = rescale(ps[0], M);
      L += ps[1] * a;
      O += ps[2 + d] * a;
    }
    const size_t oi = ((size_t)bt * Hq + g * G + h) * kD + d;
    E::store(out, oi, L > 0.f ? O / L : 0.f);
    if (d == 0 && lse) lse[(size_t)bt * Hq + g * G + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
  }
  if (threadIdx.x == 0) counters[unit] = 0u;
}

template <int DT, int G, class Src>
int launch_g(const void* q, const void* kc, const void* vc, Src src, void* out, float* lse,
             int B, int T, int Hkv, int kv_len, int L_cap, float c_log2, int splits,
             int rows_per_split, uint32_t* counters, float* partials, hipStream_t stream) {
  dim3 grid(splits, Hkv, B * T);
  hipLaunchKernelGGL((sparse_attn_kernel<DT, G, Src>), grid, dim3(kAttnThreads), 0, stream,
                     static_cast<const char*>(q), static_cast<const char*>(kc),
                     static_cast<const char*>(vc), src, out, lse, T, Hkv, kv_len, L_cap, c_log2,
                     rows_per_split, counters, partials);
  return check_launch("sparse_attn");
}

template <int DT, class Src>
int launch_dt(int G, const void* q, const void* kc, const void* vc, Src src, void* out,
              float* lse, int B, int T, int Hkv, int kv_len, int L_cap, float c_log2, int splits,
              int rows, uint32_t* cnt, float* part, hipStream_t stream) {
  switch (G) {
    case 1: return launch_g<DT, 1>(q, kc, vc, src, out, lse, B, T, Hkv, kv_len, L_cap, c_log2, splits, rows, cnt, part, stream);
    case 2: return launch_g<DT, 2>(q, kc, vc, src, out, lse, B, T, Hkv, kv_len, L_cap, c_log2, splits, rows, cnt, part, stream);
    case 4: return launch_g<DT, 4>(q, kc, vc, src, out, lse, B, T, Hkv, kv_len, L_cap, c_log2, splits, rows, cnt, part, stream);
    case 8: return launch_g<DT, 8>(q, kc, vc, src, out, lse, B, T, Hkv, kv_len, L_cap, c_log2, splits, rows, cnt, part, stream);
  }
  return set_error(CLSA_ERR_UNSUPPORTED, "attention: Hq/Hkv=%d", G);
}

}  // namespace

bool sparse_attn_supported(int dtype, int Hq, int Hkv, int D) {
  if (dtype != CLSA_BF16 && dtype != CLSA_F32) return false;
  if (D != kD || Hkv < 1 || Hq % Hkv) return false;
  const int G = Hq / Hkv;
  return G == 1 || G == 2 || G == 4 || G == 8;
}

AttnSplit attn_split(int B, int T, int Hkv, int k) {
  AttnSplit L;
  const long units = (long)B * T * Hkv;
  const int max_splits = (k + kRowsPerStep - 1) / kRowsPerStep;
  long s = (1024 + units - 1) / units;
  if (s > max_splits) s = max_splits;
  if (s < 1) s = 1;
  int rows = (int)((k + s - 1) / s);
  rows = (rows + kRowsPerStep - 1) / kRowsPerStep * kRowsPerStep;
  L.rows_per_split = rows;
  L.splits = (k + rows - 1) / rows;
  return L;
}

int launch_sparse_attn(const void* q, const void* kc, const void* vc, int dtype, const int32_t* idx,
                       int k, void* out, float* lse, int B, int T, int Hq, int Hkv, int D,
                       int kv_len, int L_cap, float scale, uint32_t* counters, float* partials,
                       hipStream_t stream) {
  const AttnSplit Lo = attn_split(B, T, Hkv, k);
  const float c_log2 = (scale > 0.f ? scale : 1.f / sqrtf((float)D)) * kLog2e;
  const int G = Hq / Hkv;
  IdxSrc src{idx, k, nullptr};
  if (dtype == CLSA_BF16)
    return launch_dt<CLSA_BF16>(G, q, kc, vc, src, out, lse, B, T, Hkv, kv_len, L_cap, c_log2,
                                Lo.splits, Lo.rows_per_split, counters, partials, stream);
  return launch_dt<CLSA_F32>(G, q, kc, vc, src, out, lse, B, T, Hkv, kv_len, L_cap, c_log2,
                             Lo.splits, Lo.rows_per_split, counters, partials, stream);
}

// Dense attention over block-table positions, one workgroup per (query, KV
// head), no split. Positions past the query's visible range are skipped.
int launch_block_attn_gather(const void* q, const void* kc, const void* vc, int dtype,
                             const int32_t* kv_indptr, const int32_t* kv_indices, int block,
                             void* out, float* lse, int B, int T, int Hq, int Hkv, int D,
                             int kv_len, int L_cap, float scale, hipStream_t stream) {
  const float c_log2 = (scale > 0.f ? scale : 1.f / sqrtf((float)D)) * kLog2e;
  const int G = Hq / Hkv;
  BlockSrc src{kv_indptr, kv_indices, block, T, Hkv, nullptr, 0};
  const int rows = 1 << 30;  // one split covers the whole table
  if (dtype == CLSA_BF16)
    return launch_dt<CLSA_BF16>(G, q, kc, vc, src, out, lse, B, T, Hkv, kv_len, L_cap, c_log2, 1,
                                rows, nullptr, nullptr, stream);
  return launch_dt<CLSA_F32>(G, q, kc, vc, src, out, lse, B, T, Hkv, kv_len, L_cap, c_log2, 1,
                             rows, nullptr, nullptr, stream);
}

}  // namespace clsa
