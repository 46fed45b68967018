// sparse_attn.hip — softmax attention over the k selected cache rows.
//
// For query (b, t), head h and its KV head g = h / G:
//   out = sum_j softmax_j(scale * q . K[idx_j, g]) V[idx_j, g]
// over the entries of idx[b, t, :] that lie in the query's visible range
// (IndexCache summary, "1. Problématique": main attention runs over the k
// selected tokens; CLSA article, "Comment CLSA fonctionne": every layer
// reuses the one index).
//
// Work split (index path): one workgroup per (query, split of the k
// entries, block of KV heads), W waves per KV head (W = 1, 2 or 4: see
// attn_split). With one wave per head the waves of a workgroup read the same
// tokens' K/V rows (contiguous across KV heads in the token-major cache) at
// about the same time; in every plan each row leaves HBM once per layer for
// all G query heads of its KV head. With per-row entry counts (row_len) a
// row's entries past its count are neither read nor gathered.
//  - bf16 (attn_split_mfma): q.K and P.V on matrix cores, 32 entries per
//    step; described above the kernel.
//  - fp32 (attn_split_kernel): the split's entries are staged in LDS; a row
//    of one KV head is gathered by 16 lanes with one 16-byte load each, four
//    rows per wave instruction; scores are fp32 dot products with a 16-lane
//    DPP butterfly; softmax runs online in the log2 domain with one rescale
//    per 8-row step.
// With several splits, each split writes its (max, sum, unnormalised
// output) state and a second small kernel merges the states of a head in
// split order (deterministic). Merging inside the first kernel would need an
// agent-scope release per workgroup, which on this GPU writes back the whole
// L2 and costs more than the extra launch.
#include "kernels.h"

namespace clsa {
namespace {

constexpr int kD = 128;
constexpr int kTileRows = 512;        // index entries staged in LDS per tile
constexpr int kMaxWaves = 8;          // KV heads per workgroup
constexpr int kPart = kD + 4;         // split state record: m, l, pad, pad, o[128]
constexpr int kMaxSplits = 2 * kD;    // the combine kernel reads <= 2 states per thread
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

template <int DT>
struct AttnElem;
template <>
struct AttnElem<CLSA_BF16> {  // output stores of the combine kernel
  static __device__ __forceinline__ void store(void* out, size_t i, float x) {
    static_cast<uint16_t*>(out)[i] = (uint16_t)f32_to_bf16_rne(x);
  }
};
template <>
struct AttnElem<CLSA_F32> {
  static constexpr int bytes = 4;
  static constexpr int rows_per_step = 4;
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
  static __device__ __forceinline__ void store8(void* out, size_t i, const float* x) {
    float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + i);
    o[0] = make_float4(x[0], x[1], x[2], x[3]);
    o[1] = make_float4(x[4], x[5], x[6], x[7]);
  }
};

// Sum over each row of 16 lanes, result in all 16 lanes (DPP butterfly:
// swap neighbours, swap pairs, mirror within 8, mirror within 16). Every
// source lane exists for these patterns, so bound_ctrl changes nothing; it
// lets the compiler fold each step into one v_add_f32_dpp.
__device__ __forceinline__ float dpp_sum16(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true));
  return v;
}

// exp2(a - b) with exp2(-inf - -inf) taken as 1 (both states empty).
__device__ __forceinline__ float rescale(float a, float b) {
  return b == -INFINITY ? 1.f : exp2f(a - b);
}

// Per-lane online-softmax state for the G query heads of one KV head, over
// the 8-element slice of D this lane owns.
template <int G>
struct HeadState {
  float m[G], l[G], o[G][8];
  __device__ void init() {
#pragma unroll
    for (int h = 0; h < G; h++) {
      m[h] = -INFINITY;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e++) o[h][e] = 0.f;
    }
  }
  // Fold in R rows: u[i][h] are log2-domain logits (-inf for skipped rows),
  // v[i] the rows' value slices.
  template <int R>
  __device__ void update(const float (&u)[R][G], const float (&v)[R][8]) {
#pragma unroll
    for (int h = 0; h < G; h++) {
      float mc = u[0][h];
#pragma unroll
      for (int i = 1; i < R; i++) mc = fmaxf(mc, u[i][h]);
      const float mn = fmaxf(m[h], mc);
      const float a = rescale(m[h], mn);
      float p[R];
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < R; i++) {
        p[i] = u[i][h] == -INFINITY ? 0.f : exp2f(u[i][h] - mn);
        ps += p[i];
      }
      l[h] = l[h] * a + ps;
#pragma unroll
      for (int e = 0; e < 8; e++) {
        float x = o[h][e] * a;
#pragma unroll
        for (int i = 0; i < R; i++) x = fmaf(p[i], v[i][e], x);
        o[h][e] = x;
      }
      m[h] = mn;
    }
  }
  // Merge with the state held by lane (lane ^ x).
  __device__ void merge_xor(int x) {
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
};

// Entries of index row bt that can hold a position: k, or with per-row counts
// (rows whose entries past their count are all -1) row_len[bt] clamped to
// [0, k], so the -1 tail is neither read nor gathered.
__device__ __forceinline__ int row_count(const int32_t* row_len, int bt, int k) {
  return row_len ? min(max(row_len[bt], 0), k) : k;
}

// Split kernel of the index path.
// grid (S, B*T, Hkv / NW), block 64 * NW; wave w handles KV head
// g = blockIdx.z * NW + w over entries [split*rows, split*rows + rows) of the
// query's index row. With S == 1 it writes out/lse, otherwise one state
// record per (query, head, split).
template <int DT, int G>
__global__ __launch_bounds__(kWave * kMaxWaves) void attn_split_kernel(
    const char* __restrict__ q, const char* __restrict__ kc, const char* __restrict__ vc,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ row_len, int k,
    void* __restrict__ out, float* __restrict__ lse, int T, int Hkv, int kv_len, int L_cap,
    float c_log2, int rows_per_split, float* __restrict__ partials, int nw) {
  // nw: waves (KV heads) per workgroup, passed rather than read from blockDim.x.
  using E = AttnElem<DT>;
  constexpr int RPI = G <= 4 ? E::rows_per_step : 4;  // fewer rows in flight for 8 heads
  constexpr int ROW = kD * E::bytes;
  __shared__ int s_pos[kTileRows];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int sub = lane % 16;  // element slice [8*sub, 8*sub + 8)
  const int rg = lane / 16;   // lane group: its own rows
  const int split = blockIdx.x, S = gridDim.x;
  const int bt = blockIdx.y;
  const int g = blockIdx.z * nw + wave;
  const int b = bt / T, t = bt % T;
  const int vis = kv_len - T + t + 1;
  const int Hq = Hkv * G;
  const int r0 = split * rows_per_split;
  const int r1 = min(row_count(row_len, bt, k), r0 + rows_per_split);
  const int32_t* irow = idx + (size_t)bt * k;

  typename E::Frag qf[G];
#pragma unroll
  for (int h = 0; h < G; h++)
    qf[h] = E::load(q + (((size_t)bt * Hq + g * G + h) * kD + 8 * sub) * E::bytes);
  HeadState<G> st;
  st.init();

  const char* kb = kc + ((size_t)b * L_cap * Hkv + g) * ROW + 8 * sub * E::bytes;
  const char* vb = vc + ((size_t)b * L_cap * Hkv + g) * ROW + 8 * sub * E::bytes;
  const size_t tok = (size_t)Hkv * ROW;  // bytes between consecutive tokens

  for (int t0 = r0; t0 < r1; t0 += kTileRows) {  // uniform over the workgroup
    const int n = min(kTileRows, r1 - t0);
    __syncthreads();  // the previous tile's positions are no longer read
    for (int i = threadIdx.x; i < n; i += nw * kWave) {
      const int p = irow[t0 + i];
      s_pos[i] = (p >= 0 && p < vis) ? p : -1;
    }
    __syncthreads();
    for (int base = 0; base < n; base += 4 * RPI) {  // uniform over the wave
      int pos[RPI];
#pragma unroll
      for (int i = 0; i < RPI; i++) {
        const int r = base + rg * RPI + i;
        pos[i] = r < n ? s_pos[r] : -1;
      }
      typename E::Frag kf[RPI], vf[RPI];
#pragma unroll
      for (int i = 0; i < RPI; i++) kf[i] = E::load(kb + (size_t)max(pos[i], 0) * tok);
#pragma unroll
      for (int i = 0; i < RPI; i++) vf[i] = E::load(vb + (size_t)max(pos[i], 0) * tok);
      float u[RPI][G];
#pragma unroll
      for (int i = 0; i < RPI; i++)
#pragma unroll
        for (int h = 0; h < G; h++) {
          const float sc = dpp_sum16(E::dot(qf[h], kf[i]));
          u[i][h] = pos[i] >= 0 ? sc * c_log2 : -INFINITY;
        }
      float v[RPI][8];
#pragma unroll
      for (int i = 0; i < RPI; i++) E::to_f32(vf[i], v[i]);
      st.update(u, v);
    }
  }
  // Merge the 4 lane groups: lanes sub, sub+16, sub+32, sub+48.
  st.merge_xor(16);
  st.merge_xor(32);
  if (rg != 0) return;
#pragma unroll
  for (int h = 0; h < G; h++) {
    const size_t head = (size_t)bt * Hq + g * G + h;
    if (S == 1) {
      float x[8];
      const float inv = st.l[h] > 0.f ? 1.f / st.l[h] : 0.f;
#pragma unroll
      for (int e = 0; e < 8; e++) x[e] = st.o[h][e] * inv;
      E::store8(out, head * kD + 8 * sub, x);
      if (sub == 0 && lse)
        lse[head] = st.l[h] > 0.f ? (st.m[h] + log2f(st.l[h])) * kLn2 : -INFINITY;
    } else {
      float* rec = partials + (head * S + split) * kPart;
      float4* o4 = reinterpret_cast<float4*>(rec + 4 + 8 * sub);
      o4[0] = make_float4(st.o[h][0], st.o[h][1], st.o[h][2], st.o[h][3]);
      o4[1] = make_float4(st.o[h][4], st.o[h][5], st.o[h][6], st.o[h][7]);
      if (sub == 0) {
        rec[0] = st.m[h];
        rec[1] = st.l[h];
      }
    }
  }
}

// bf16 split kernel on matrix cores (same outputs as attn_split_kernel).
// W waves (1, 2 or 4; see attn_split) per (query, split, KV head g); each
// wave takes 32-entry steps, as two tiles of 16 keys, reading the positions
// it needs straight from the query's index row. Lane l = 16 * grp + col.
//  - Scores: S^T[key, h] = K[key, :] . q[h, :] with v_mfma_f32_16x16x32_bf16.
//    A = 16 gathered K rows (lane: key col, d = 8 * grp + 32 * ks + 0..7),
//    B = the G query heads (lane: head col; columns >= G repeat head G - 1, unused). Lane
//    (grp, col) receives head col for keys 4 * grp + r of each tile.
//  - Softmax: one running max per head shared by the four lane groups (a
//    cross-group max through v_permlane16/32_swap), so the per-group partial
//    sums add without rescaling; each exp is taken once.
//  - Output: O^T[d, h] += V^T[d, key] . P^T[key, h], P split into bf16 hi
//    and bf16 lo parts (two products). The lane's 8 probabilities are
//    already the B operand (k slot x = 4 * tile +
//    r of lane group grp is key 16 * tile + 4 * grp + r). V^T goes through a
//    per-wave LDS tile: each lane gathers 16-byte V row pieces (same keys as
//    its probabilities, d = 8 * col + 0..7) and writes them transposed; the
//    A fragments are read back as two 8-byte pieces. Rows and 8-byte chunks of
//    the tile are XOR-swizzled so that both the writes (16 lanes: one key
//    group, 16 d-slices) and the reads (16 lanes: 16 consecutive d) touch 16
//    distinct 8-byte bank slots.
//  Lane (grp, col) ends with O^T[16 * j + 4 * grp + s][col], j = 0..7, s = 0..3.
constexpr int kVtBytes = kD * 64;  // per-wave V^T tile: 128 d-rows x 32 keys x bf16

// Byte offset of the 8-byte chunk c8 (keys 4 * c8 .. 4 * c8 + 3) of d-row d.
__host__ __device__ constexpr int vt_addr(int d, int c8) {
  const int row = d ^ ((d >> 4) & 1);
  const int h = (((d >> 1) ^ (d >> 5)) & 1) | ((((d >> 2) ^ (d >> 6)) & 1) << 1) | (((d >> 3) & 1) << 2);
  return row * 64 + 8 * (c8 ^ h);
}

__device__ __forceinline__ float xgroup_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xgroup_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// Low or high bf16 halves of four words packed as 4 x bf16 (8 bytes).
__device__ __forceinline__ uint2 pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d, bool hi) {
  const uint32_t sel = hi ? 0x07060302u : 0x05040100u;
  return make_uint2(__builtin_amdgcn_perm(b, a, sel), __builtin_amdgcn_perm(d, c, sel));
}
// Two floats to bf16 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// One 32-entry step of a wave: gathered K (MFMA A layout) and V (row
// pieces) fragments and the positions that mask them.
struct KvStep {
  bf16x8 kf[2][4];
  uint4 vf[2][4];
  uint32_t valid;  // bit 4 * tile + r: key 16 * tile + 4 * grp + r is visible
};

// This lane's raw index entries of one 32-entry step (entries e0 .. e0 + 31
// of the query's row): the K row entry of each 16-key tile and the 4 V row
// entries of its lane group in each tile. Every load is unconditional
// (entries past `end` read entry max(end - 1, 0)) and the values are masked
// only when the step is issued.
struct IdxStep {
  int k[2];
  int v[2][4];
};
__device__ __forceinline__ void idx_fetch(IdxStep& x, const int32_t* irow, int e0, int end, int col,
                                          int grp) {
  const int last = max(end - 1, 0);
#pragma unroll
  for (int tt = 0; tt < 2; tt++) {
    x.k[tt] = irow[min(e0 + 16 * tt + col, last)];
#pragma unroll
    for (int r = 0; r < 4; r++) x.v[tt][r] = irow[min(e0 + 16 * tt + 4 * grp + r, last)];
  }
}
// Entry e with raw position p: the position if e is before `end` and p is
// visible, else -1 (masked; its loads read cache row 0).
__device__ __forceinline__ int vis_pos(int p, int e, int end, int vis) {
  return (e < end && p >= 0 && p < vis) ? p : -1;
}

// Issues the K/V loads of the step at entries [e0, e0 + 32) from its index
// entries x (masked entries read cache row 0).
__device__ __forceinline__ void kv_issue(KvStep& f, const IdxStep& x, int e0, int end, int vis,
                                         int col, int grp, const char* kb, const char* vb,
                                         size_t tok) {
  int kp[2], vp[2][4];
#pragma unroll
  for (int tt = 0; tt < 2; tt++) {
    kp[tt] = vis_pos(x.k[tt], e0 + 16 * tt + col, end, vis);
#pragma unroll
    for (int r = 0; r < 4; r++) vp[tt][r] = vis_pos(x.v[tt][r], e0 + 16 * tt + 4 * grp + r, end, vis);
  }
  f.valid = 0u;
#pragma unroll
  for (int tt = 0; tt < 2; tt++)
#pragma unroll
    for (int r = 0; r < 4; r++) f.valid |= (vp[tt][r] >= 0 ? 1u : 0u) << (4 * tt + r);
#pragma unroll
  for (int tt = 0; tt < 2; tt++)
#pragma unroll
    for (int ks = 0; ks < 4; ks++)
      f.kf[tt][ks] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(kb + (size_t)max(kp[tt], 0) * tok + 64 * ks));
#pragma unroll
  for (int tt = 0; tt < 2; tt++)
#pragma unroll
    for (int r = 0; r < 4; r++)
      f.vf[tt][r] = *reinterpret_cast<const uint4*>(vb + (size_t)max(vp[tt][r], 0) * tok);
}

// Running state of one wave: O^T accumulators, max and sum of head col.
struct MfmaState {
  f32x4 o[8];
  float m, l;
};

__device__ __forceinline__ void kv_consume(const KvStep& f, MfmaState& st, const bf16x8 (&qf)[4],
                                           char* vt, int wbase, int rbase, float c_log2) {
  f32x4 sc[2];
#pragma unroll
  for (int tt = 0; tt < 2; tt++) {
    sc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ks++) sc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.kf[tt][ks], qf[ks], sc[tt], 0, 0, 0);
  }
  // Stage V^T while the scores are in flight.
#pragma unroll
  for (int tt = 0; tt < 2; tt++) {
    const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&f.vf[tt][0]);
    const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&f.vf[tt][1]);
    const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&f.vf[tt][2]);
    const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&f.vf[tt][3]);
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const int off = wbase ^ (vt_addr(e, 4 * tt) ^ vt_addr(0, 0));
      *reinterpret_cast<uint2*>(vt + off) = pack4(w0[e / 2], w1[e / 2], w2[e / 2], w3[e / 2], e & 1);
    }
  }
  // Online softmax of head col over the 32 keys.
  float u[2][4];
  float mc = -INFINITY;
#pragma unroll
  for (int tt = 0; tt < 2; tt++)
#pragma unroll
    for (int r = 0; r < 4; r++) {
      u[tt][r] = (f.valid >> (4 * tt + r) & 1u) ? sc[tt][r] * c_log2 : -INFINITY;
      mc = fmaxf(mc, u[tt][r]);
    }
  const float mn = fmaxf(st.m, xgroup_max(mc));
  const float alpha = rescale(st.m, mn);
  float pr[2][4];
  float ps = 0.f;
#pragma unroll
  for (int tt = 0; tt < 2; tt++)
#pragma unroll
    for (int r = 0; r < 4; r++) {
      pr[tt][r] = u[tt][r] == -INFINITY ? 0.f : exp2f(u[tt][r] - mn);
      ps += pr[tt][r];
    }
  st.l = st.l * alpha + ps;
  st.m = mn;
  if (__builtin_amdgcn_read_exec() & __ballot(alpha != 1.f)) {
#pragma unroll
    for (int j = 0; j < 8; j++) st.o[j] *= alpha;
  }
  // P enters the matrix cores as bf16 hi + bf16 lo: hi = bf16(p), lo =
  // bf16(p - hi) (p - hi is exact in float32), so P carries about 16
  // significant bits instead of 8; two products accumulate into O.
  const uint4 pb = make_uint4(pack_bf16(pr[0][0], pr[0][1]), pack_bf16(pr[0][2], pr[0][3]),
                              pack_bf16(pr[1][0], pr[1][1]), pack_bf16(pr[1][2], pr[1][3]));
  const uint32_t pw[4] = {pb.x, pb.y, pb.z, pb.w};
  uint32_t lw[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const float* pi = &pr[i / 2][2 * (i % 2)];
    lw[i] = pack_bf16(pi[0] - __uint_as_float(pw[i] << 16), pi[1] - __uint_as_float(pw[i] & 0xffff0000u));
  }
  const bf16x8 pf = __builtin_bit_cast(bf16x8, pb);
  const bf16x8 pl = __builtin_bit_cast(bf16x8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
  // The tile is private to the wave; the fences keep the compiler from
  // moving its accesses across the write/read phases.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint2 lo[8], hi[8];
#pragma unroll
  for (int j = 0; j < 8; j++) {
    lo[j] = *reinterpret_cast<const uint2*>(vt + (rbase ^ (vt_addr(16 * j, 0) ^ vt_addr(0, 0))));
    hi[j] = *reinterpret_cast<const uint2*>(vt + (rbase ^ (vt_addr(16 * j, 4) ^ vt_addr(0, 0))));
  }
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const bf16x8 af = __builtin_bit_cast(bf16x8, make_uint4(lo[j].x, lo[j].y, hi[j].x, hi[j].y));
    st.o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, pf, st.o[j], 0, 0, 0);
    st.o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, pl, st.o[j], 0, 0, 0);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// W waves share one KV head's split: wave w of the head takes the 32-entry
// steps w, w + W, ... and the W states are merged through LDS before the
// split's single state is written (W > 1 keeps many waves in flight with
// few splits, so fewer states go through memory).
template <int G, int W>
__global__ __launch_bounds__(kWave * kMaxWaves) void attn_split_mfma(
    const char* __restrict__ q, const char* __restrict__ kc, const char* __restrict__ vc,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ row_len, int k,
    void* __restrict__ out, float* __restrict__ lse, int T, int Hkv, int kv_len, int L_cap,
    float c_log2, int rows_per_split, float* __restrict__ partials, int gpw) {
  // gpw: KV heads per workgroup (blockDim.x = 64 * W * gpw). It is an argument
  // rather than derived from blockDim.x, whose read from the dispatch's hidden
  // arguments is a vector load the whole prologue would wait for.
  constexpr int ROW = kD * 2;
  __shared__ __attribute__((aligned(16))) char s_vt[kMaxWaves * kVtBytes];
  __shared__ float s_ml[kMaxWaves][16][2];
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int col = lane % 16;
  const int grp = lane / 16;
  const int split = blockIdx.x, S = gridDim.x;
  const int bt = blockIdx.y;
  const int w = wave % W;
  const int g = blockIdx.z * gpw + wave / W;
  const int b = bt / T, t = bt % T;
  const int vis = kv_len - T + t + 1;
  const int Hq = Hkv * G;
  const int r0 = split * rows_per_split;
  const int r1 = min(row_count(row_len, bt, k), r0 + rows_per_split);
  const int32_t* irow = idx + (size_t)bt * k;
  char* vt = s_vt + wave * kVtBytes;

  IdxStep xi;  // the wave's first step, requested first: the gather waits on it
  idx_fetch(xi, irow, r0 + 32 * w, r1, col, grp);
  bf16x8 qf[4];
  // B columns col >= G hold no head: they load head G - 1 again (their
  // scores, softmax and outputs stay in their own columns and are never
  // stored). An unconditional load keeps the q loads in flight with the
  // index loads that follow instead of waiting for them first.
  const int qh = g * G + min(col, G - 1);
#pragma unroll
  for (int ks = 0; ks < 4; ks++)
    qf[ks] = __builtin_bit_cast(
        bf16x8, *reinterpret_cast<const uint4*>(q + (((size_t)bt * Hq + qh) * kD + 8 * grp + 32 * ks) * 2));
  MfmaState st;
#pragma unroll
  for (int j = 0; j < 8; j++) st.o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;  // head col; shared by the four lane groups
  st.l = 0.f;        // this lane group's keys only

  // LDS offsets: the write addresses depend on the lane and on (e, tile)
  // only through XOR with a constant, likewise the reads on (j, tile).
  const int wbase = vt_addr(8 * col, grp);
  const int rbase = vt_addr(col, grp);

  const char* kb = kc + ((size_t)b * L_cap * Hkv + g) * ROW + (8 * grp) * 2;
  const char* vb = vc + ((size_t)b * L_cap * Hkv + g) * ROW + 16 * col;
  const size_t tok = (size_t)Hkv * ROW;

  // One 32-entry step at a time: at the usual split sizes a wave has one
  // or two steps, and the other waves of the SIMD cover its load latency.
  // The first step's index entries were requested before the q loads; each
  // later step's are requested once the previous step is consumed
  // (prefetching them a step ahead measured slower on the 2K-query prefill,
  // where a wave runs 128 steps).
  for (int e0 = r0 + 32 * w; e0 < r1; e0 += 32 * W) {  // uniform over the wave
    KvStep f;
    kv_issue(f, xi, e0, r1, vis, col, grp, kb, vb, tok);
    kv_consume(f, st, qf, vt, wbase, rbase, c_log2);
    idx_fetch(xi, irow, e0 + 32 * W, r1, col, grp);
  }
  float l = xgroup_sum(st.l);
  float m = st.m;
  if constexpr (W > 1) {
    // Each wave parks (m, l) per head and its accumulators ([j][lane] float4,
    // conflict-free) in its own V^T tile; wave 0 of the head merges.
    __syncthreads();  // every wave is done with its V^T tile
    float4* park = reinterpret_cast<float4*>(vt);
    if (grp == 0) {
      s_ml[wave][col][0] = m;
      s_ml[wave][col][1] = l;
    }
    if (w != 0) {
#pragma unroll
      for (int j = 0; j < 8; j++) park[j * kWave + lane] = make_float4(st.o[j][0], st.o[j][1], st.o[j][2], st.o[j][3]);
    }
    __syncthreads();
    if (w != 0) return;
    float mw[W], aw[W];
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < W; v++) {
      mw[v] = s_ml[wave + v][col][0];
      M = fmaxf(M, mw[v]);
    }
    l = 0.f;
#pragma unroll
    for (int v = 0; v < W; v++) {
      aw[v] = rescale(mw[v], M);
      l += s_ml[wave + v][col][1] * aw[v];
    }
#pragma unroll
    for (int j = 0; j < 8; j++) st.o[j] *= aw[0];
#pragma unroll
    for (int v = 1; v < W; v++) {
      const float4* pv = reinterpret_cast<const float4*>(s_vt + (wave + v) * kVtBytes);
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const float4 x = pv[j * kWave + lane];
        st.o[j][0] += aw[v] * x.x;
        st.o[j][1] += aw[v] * x.y;
        st.o[j][2] += aw[v] * x.z;
        st.o[j][3] += aw[v] * x.w;
      }
    }
    m = M;
  }
  if (col >= G) return;
  const size_t head = (size_t)bt * Hq + g * G + col;
  if (S == 1) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t* orow = static_cast<uint16_t*>(out) + head * kD + 4 * grp;
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const uint2 w = make_uint2(pack_bf16(st.o[j][0] * inv, st.o[j][1] * inv),
                                 pack_bf16(st.o[j][2] * inv, st.o[j][3] * inv));
      *reinterpret_cast<uint2*>(orow + 16 * j) = w;
    }
    if (grp == 0 && lse) lse[head] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  } else {
    float* rec = partials + (head * S + split) * kPart;
#pragma unroll
    for (int j = 0; j < 8; j++)
      *reinterpret_cast<float4*>(rec + 4 + 16 * j + 4 * grp) =
          make_float4(st.o[j][0], st.o[j][1], st.o[j][2], st.o[j][3]);
    if (grp == 0) {
      rec[0] = m;
      rec[1] = l;
    }
  }
}

// Merges the S split states of each (query, head), S <= kMaxSplits.
// grid (B*T*Hq), block D. The split weights exp2(m_s - M) go to LDS first so
// the S loads of each output element are independent of one another.
template <int DT>
__global__ __launch_bounds__(kD) void attn_combine_kernel(const float* __restrict__ partials,
                                                          void* __restrict__ out,
                                                          float* __restrict__ lse, int S) {
  using E = AttnElem<DT>;
  __shared__ float wgt[kMaxSplits];
  __shared__ float red[2];
  const size_t head = blockIdx.x;
  const int d = threadIdx.x;
  const int wave = d / kWave;
  const float* rec = partials + head * S * kPart;
  float mv[2], lv[2];
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int s = d + j * kD;
    mv[j] = s < S ? rec[(size_t)s * kPart] : -INFINITY;
    lv[j] = s < S ? rec[(size_t)s * kPart + 1] : 0.f;
  }
  float M = fmaxf(mv[0], mv[1]);
  for (int off = kWave / 2; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, kWave));
  if (d % kWave == 0) red[wave] = M;
  __syncthreads();
  M = fmaxf(red[0], red[1]);
  float Ls = 0.f;
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int s = d + j * kD;
    const float a = rescale(mv[j], M);
    if (s < S) wgt[s] = a;
    Ls += lv[j] * a;
  }
  for (int off = kWave / 2; off > 0; off >>= 1) Ls += __shfl_xor(Ls, off, kWave);
  __syncthreads();  // red[] reads of M done; wgt[] written
  if (d % kWave == 0) red[wave] = Ls;
  __syncthreads();
  const float L = red[0] + red[1];
  float O = 0.f;
#pragma unroll 16
  for (int s = 0; s < S; s++) O += rec[(size_t)s * kPart + 4 + d] * wgt[s];
  E::store(out, head * kD + d, L > 0.f ? O / L : 0.f);
  if (d == 0 && lse) lse[head] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

// KV heads per workgroup. One wave per head (W = 1): the largest divisor of
// Hkv up to kMaxWaves, so a workgroup reads whole token rows. W waves per
// head: the largest divisor with at most 4 waves per workgroup, since the
// merge barrier makes each wave wait for the slowest wave of its workgroup
// (measured on the 128K decode, W = 4: 10.94 us per call with one head per
// workgroup vs 11.2 us with two; W = 2: 11.5 us with two heads vs 13.6 us
// with one).
int heads_per_block(int Hkv, int W) {
  const int cap = W == 1 ? kMaxWaves : (W < 4 ? 4 / W : 1);
  for (int h = cap; h > 1; h--)
    if (Hkv % h == 0) return h;
  return 1;
}

template <int DT, int G>
int launch_index_path(const void* q, const void* kc, const void* vc, const int32_t* idx,
                      const int32_t* row_len, int k,
                      void* out, float* lse, int B, int T, int Hkv, int kv_len, int L_cap,
                      float c_log2, const AttnSplit& sp, float* partials, hipStream_t stream) {
  const int gpw = heads_per_block(Hkv, sp.waves_per_head);
  dim3 grid(sp.splits, B * T, Hkv / gpw);
  const dim3 block(kWave * gpw * sp.waves_per_head);
  if constexpr (DT == CLSA_BF16) {
#define CLSA_SPLIT_MFMA(W)                                                                   \
  hipLaunchKernelGGL((attn_split_mfma<G, W>), grid, block, 0, stream,                        \
                     static_cast<const char*>(q), static_cast<const char*>(kc),              \
                     static_cast<const char*>(vc), idx, row_len, k, out, lse, T, Hkv, kv_len, \
                     L_cap, c_log2, sp.rows_per_split, partials, gpw)
    if (sp.waves_per_head == 4) CLSA_SPLIT_MFMA(4);
    else if (sp.waves_per_head == 2) CLSA_SPLIT_MFMA(2);
    else CLSA_SPLIT_MFMA(1);
#undef CLSA_SPLIT_MFMA
  } else {
    hipLaunchKernelGGL((attn_split_kernel<DT, G>), grid, block, 0, stream,
                       static_cast<const char*>(q), static_cast<const char*>(kc),
                       static_cast<const char*>(vc), idx, row_len, k, out, lse, T, Hkv, kv_len,
                       L_cap, c_log2, sp.rows_per_split, partials, gpw);
  }
  int rc = check_launch("attn_split");
  if (rc || sp.splits == 1) return rc;
  hipLaunchKernelGGL((attn_combine_kernel<DT>), dim3(B * T * Hkv * G), dim3(kD), 0, stream,
                     partials, out, lse, sp.splits);
  return check_launch("attn_combine");
}

template <int DT>
int dispatch_index_path(int G, const void* q, const void* kc, const void* vc, const int32_t* idx,
                        const int32_t* row_len, int k, void* out, float* lse, int B, int T, int Hkv, int kv_len, int L_cap,
                        float c_log2, const AttnSplit& sp, float* part, hipStream_t s) {
  switch (G) {
    case 1: return launch_index_path<DT, 1>(q, kc, vc, idx, row_len, k, out, lse, B, T, Hkv, kv_len, L_cap, c_log2, sp, part, s);
    case 2: return launch_index_path<DT, 2>(q, kc, vc, idx, row_len, k, out, lse, B, T, Hkv, kv_len, L_cap, c_log2, sp, part, s);
    case 4: return launch_index_path<DT, 4>(q, kc, vc, idx, row_len, k, out, lse, B, T, Hkv, kv_len, L_cap, c_log2, sp, part, s);
    case 8: return launch_index_path<DT, 8>(q, kc, vc, idx, row_len, k, out, lse, B, T, Hkv, kv_len, L_cap, c_log2, sp, part, s);
  }
  return set_error(CLSA_ERR_UNSUPPORTED, "sparse_attn: Hq/Hkv=%d", G);
}

}  // namespace

bool sparse_attn_supported(int dtype, int Hq, int Hkv, int D) {
  if (dtype != CLSA_BF16 && dtype != CLSA_F32) return false;
  if (D != kD || Hkv < 1 || Hq % Hkv) return false;
  const int G = Hq / Hkv;
  return G == 1 || G == 2 || G == 4 || G == 8;
}

// Splits of the k entries: about one workgroup per CU (256), each wave
// taking a multiple of 32 entries (one 8-row step of its 4 lane groups), at
// most kMaxSplits splits. Measured on MI355X: one 8-wave workgroup per CU
// beat both fewer, longer splits and two workgroups per CU at B = 4, 8, 16.
// Work plan: about 2048 waves (8 per CU) over B*T*Hkv (query, KV head)
// units of ceil(k/32) steps each. With matrix cores and one step per wave,
// 4 (or 2) of a unit's waves share one split and merge in LDS, so 4x fewer
// split states go through memory (measured on the 128K decode: 11.1 us per
// call vs 12.2 us). With several steps per wave, one wave per split and a
// workgroup of 8 KV heads (reading whole token rows together) measured
// faster (B = 8: 16.5 vs 19.1 us; B = 16: 25.3 vs 27.0 us).
AttnSplit attn_split(int B, int T, int Hkv, int k, bool mfma) {
  constexpr long kTargetWaves = 2048;
  const int step = 32;
  AttnSplit L;
  const long units = (long)B * T * Hkv;
  const long steps = (k + step - 1) / step;
  long waves = (kTargetWaves + units - 1) / units;  // per unit
  if (waves > steps) waves = steps;
  if (waves < 1) waves = 1;
  int W = 1;
  if (mfma && waves == steps) W = waves % 4 == 0 ? 4 : (waves % 2 == 0 ? 2 : 1);
  long s = (waves + W - 1) / W;
  if (s > kMaxSplits) s = kMaxSplits;
  int rows = (int)((k + s - 1) / s);
  rows = (rows + step * W - 1) / (step * W) * (step * W);
  L.waves_per_head = W;
  L.rows_per_split = rows;
  L.splits = (k + rows - 1) / rows;
  return L;
}
size_t attn_partial_floats(int B, int T, int Hq, int Hkv, int k) {
  size_t n = 0;
  for (int mfma = 0; mfma < 2; mfma++) {  // either kernel family may run
    const AttnSplit s = attn_split(B, T, Hkv, k, mfma != 0);
    if (s.splits > 1) n = std::max(n, (size_t)B * T * Hq * s.splits * kPart);
  }
  return n;
}

int launch_sparse_attn(const void* q, const void* kc, const void* vc, int dtype, const int32_t* idx,
                       int k, void* out, float* lse, int B, int T, int Hq, int Hkv, int D,
                       int kv_len, int L_cap, float scale, float* partials,
                       const int32_t* row_len, hipStream_t stream) {
  const AttnSplit sp = attn_split(B, T, Hkv, k, dtype == CLSA_BF16);
  const float c_log2 = (scale > 0.f ? scale : 1.f / sqrtf((float)D)) * kLog2e;
  const int G = Hq / Hkv;
  if (dtype == CLSA_BF16)
    return dispatch_index_path<CLSA_BF16>(G, q, kc, vc, idx, row_len, k, out, lse, B, T, Hkv, kv_len, L_cap,
                                          c_log2, sp, partials, stream);
  return dispatch_index_path<CLSA_F32>(G, q, kc, vc, idx, row_len, k, out, lse, B, T, Hkv, kv_len, L_cap,
                                       c_log2, sp, partials, stream);
}

}  // namespace clsa
