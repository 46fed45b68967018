// api.cpp — the C ABI of libclsa (declared in include/clsa.h).
//
// Every entry point validates all of its arguments before it enqueues
// anything, carves the caller's workspace, and enqueues the kernels of
// cache_append.hip, index_score.hip, topk.hip, sparse_attn.hip,
// block_union.hip and block_attn.hip on the caller's stream. Nothing here
// allocates device memory or synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include "kernels.h"

namespace clsa {

static thread_local char g_err[512] = "";

int set_error(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

namespace {

constexpr int kMaxRowsPerGrid = 65535;  // B*T lands in grid.y / grid.z

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Workspace regions, each 256-byte aligned, in the order they are added.
struct Carver {
  size_t off = 0;
  size_t add(size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  }
};

struct TopkWs {
  size_t arrivals, arrival_words, counts, cand, spill, total;
};
TopkWs topk_ws(int rows, int kv_len) {
  const TopkBuffers tb = topk_buffers(rows, kv_len);
  Carver c;
  TopkWs w;
  w.arrival_words = tb.arrival_words;
  w.arrivals = c.add(tb.arrival_words * 4);
  w.counts = c.add(tb.counts_words * 4);
  w.cand = c.add(tb.cand_words * 4);
  w.spill = c.add(tb.spill_words * 4);
  w.total = c.off;
  return w;
}

struct AttnWs {
  size_t partials, total;
};
AttnWs attn_ws(int B, int T, int Hq, int Hkv, int k) {
  Carver c;
  AttnWs w;
  w.partials = c.add(attn_partial_floats(B, T, Hq, Hkv, k) * 4);
  w.total = c.off;
  return w;
}

// Decode step workspace: top-k buffers, attention split states, indexer
// scores.
struct StepWs {
  TopkWs topk;
  size_t partials, scores, kept, total;
};
StepWs step_ws(int B, int T, int Hq, int Hkv, int kv_len, int k) {
  StepWs w;
  w.topk = topk_ws(B * T, kv_len);
  Carver c;
  c.off = w.topk.total;
  w.partials = c.add(attn_partial_floats(B, T, Hq, Hkv, k) * 4);
  w.scores = c.add((size_t)B * T * kv_len * 4);
  w.kept = c.add((size_t)B * T * 4);
  w.total = c.off;
  return w;
}

int check_shape(int B, int T, int kv_len, int L_cap) {
  if (B < 1 || T < 1) return set_error(CLSA_ERR_INVALID_ARG, "B=%d and T=%d must be >= 1", B, T);
  if (kv_len < T) return set_error(CLSA_ERR_INVALID_ARG, "kv_len=%d must be >= T=%d", kv_len, T);
  if (L_cap < kv_len)
    return set_error(CLSA_ERR_INVALID_ARG, "L_cap=%d must be >= kv_len=%d", L_cap, kv_len);
  if ((long)B * T > kMaxRowsPerGrid)
    return set_error(CLSA_ERR_UNSUPPORTED, "B*T=%ld above %d", (long)B * T, kMaxRowsPerGrid);
  return CLSA_OK;
}

int check_index_args(const void* q_idx, const void* k_idx, int idx_dtype, const float* w,
                     const float* scores, int B, int T, int H_I, int D_I, int kv_len, int L_cap) {
  if (!q_idx || !k_idx || !w || !scores)
    return set_error(CLSA_ERR_INVALID_ARG, "index_score: null pointer");
  int rc = check_shape(B, T, kv_len, L_cap);
  if (rc) return rc;
  if (H_I < 1 || D_I < 1)
    return set_error(CLSA_ERR_INVALID_ARG, "index_score: H_I=%d, D_I=%d must be >= 1", H_I, D_I);
  if (idx_dtype != CLSA_F32 && idx_dtype != CLSA_BF16 && idx_dtype != CLSA_FP8_E4M3FN)
    return set_error(CLSA_ERR_INVALID_ARG, "index_score: unknown dtype %d", idx_dtype);
  if (!index_score_supported(idx_dtype, H_I, D_I))
    return set_error(CLSA_ERR_UNSUPPORTED, "index_score: dtype %d with H_I=%d, D_I=%d", idx_dtype,
                     H_I, D_I);
  if (!aligned(q_idx, 16) || !aligned(k_idx, 16) || !aligned(w, 4) || !aligned(scores, 4))
    return set_error(CLSA_ERR_INVALID_ARG, "index_score: misaligned pointer");
  return CLSA_OK;
}

int check_topk_args(const float* scores, int B, int T, int kv_len, int k, const int32_t* idx) {
  if (!scores || !idx) return set_error(CLSA_ERR_INVALID_ARG, "topk: null pointer");
  int rc = check_shape(B, T, kv_len, kv_len);
  if (rc) return rc;
  if (k < 1) return set_error(CLSA_ERR_INVALID_ARG, "topk: k=%d must be >= 1", k);
  if (topk_buffers(1, kv_len).nchunks > kTopkMaxChunks)
    return set_error(CLSA_ERR_UNSUPPORTED, "topk: kv_len=%d above %d", kv_len,
                     kTopkMaxChunks * kTopkChunk);
  if (!aligned(scores, 4) || !aligned(idx, 4))
    return set_error(CLSA_ERR_INVALID_ARG, "topk: misaligned pointer");
  return CLSA_OK;
}

int check_attn_args(const void* q, const void* kc, const void* vc, int dtype, const int32_t* idx,
                    int k, const void* out, const float* lse, int B, int T, int Hq, int Hkv, int D,
                    int kv_len, int L_cap) {
  if (!q || !kc || !vc || !idx || !out)
    return set_error(CLSA_ERR_INVALID_ARG, "sparse_attn: null pointer");
  int rc = check_shape(B, T, kv_len, L_cap);
  if (rc) return rc;
  if (k < 1) return set_error(CLSA_ERR_INVALID_ARG, "sparse_attn: k=%d must be >= 1", k);
  if (Hq < 1 || Hkv < 1 || D < 1 || Hq % Hkv)
    return set_error(CLSA_ERR_INVALID_ARG, "sparse_attn: Hq=%d, Hkv=%d, D=%d", Hq, Hkv, D);
  if (dtype != CLSA_F32 && dtype != CLSA_BF16 && dtype != CLSA_FP8_E4M3FN)
    return set_error(CLSA_ERR_INVALID_ARG, "sparse_attn: unknown dtype %d", dtype);
  if (!sparse_attn_supported(dtype, Hq, Hkv, D))
    return set_error(CLSA_ERR_UNSUPPORTED, "sparse_attn: dtype %d, Hq=%d, Hkv=%d, D=%d", dtype, Hq,
                     Hkv, D);
  if (!aligned(q, 16) || !aligned(kc, 16) || !aligned(vc, 16) || !aligned(out, 16) ||
      !aligned(idx, 4) || (lse && !aligned(lse, 4)))
    return set_error(CLSA_ERR_INVALID_ARG, "sparse_attn: misaligned pointer");
  return CLSA_OK;
}

int record(void* const* events, int i, hipStream_t s) {
  if (!events) return CLSA_OK;
  hipError_t e = hipEventRecord(static_cast<hipEvent_t>(events[i]), s);
  if (e != hipSuccess) return set_error(CLSA_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
  return CLSA_OK;
}

}  // namespace
}  // namespace clsa

using namespace clsa;

extern "C" {

int clsa_abi_version(void) { return CLSA_ABI_VERSION; }

const char* clsa_status_string(int status) {
  switch (status) {
    case CLSA_OK: return "ok";
    case CLSA_ERR_INVALID_ARG: return "invalid argument";
    case CLSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case CLSA_ERR_WORKSPACE: return "workspace missing or too small";
    case CLSA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* clsa_last_error(void) { return g_err; }

size_t clsa_workspace_bytes(int op, int B, int T, int Hq, int Hkv, int D, int kv_len, int k,
                            int block) {
  if (B < 1 || T < 1) return 0;
  switch (op) {
    case CLSA_OP_TOPK:
      if (kv_len < T || k < 1) return 0;
      return topk_ws(B * T, kv_len).total;
    case CLSA_OP_SPARSE_ATTN:
      if (Hq < 1 || Hkv < 1 || D < 1 || k < 1 || Hq % Hkv) return 0;
      return attn_ws(B, T, Hq, Hkv, k).total;
    case CLSA_OP_BLOCK_UNION:
      if (kv_len < 1 || block < 1) return 0;
      return block_union_ws_bytes(B, kv_len, block);
  }
  return 0;
}

int clsa_index_score(const void* q_idx, const void* k_idx, int idx_dtype, const float* w,
                     float* scores, int B, int T, int H_I, int D_I, int kv_len, int L_cap,
                     void* stream) {
  int rc = check_index_args(q_idx, k_idx, idx_dtype, w, scores, B, T, H_I, D_I, kv_len, L_cap);
  if (rc) return rc;
  return launch_index_score(q_idx, k_idx, idx_dtype, w, scores, B, T, H_I, D_I, kv_len, L_cap,
                            ZeroJob{}, static_cast<hipStream_t>(stream));
}

int clsa_topk_margin(const float* scores, int B, int T, int kv_len, int k,
                     const int32_t* k_per_query, float margin, int32_t* idx, int32_t* kept, void* ws,
                     size_t ws_bytes, void* stream) {
  int rc = check_topk_args(scores, B, T, kv_len, k, idx);
  if (rc) return rc;
  if (k_per_query && !aligned(k_per_query, 4))
    return set_error(CLSA_ERR_INVALID_ARG, "topk: misaligned k_per_query");
  if (kept && !aligned(kept, 4)) return set_error(CLSA_ERR_INVALID_ARG, "topk: misaligned kept");
  if (!(margin >= 0.f)) return set_error(CLSA_ERR_INVALID_ARG, "topk: margin must be >= 0 (or +inf)");
  const TopkWs L = topk_ws(B * T, kv_len);
  if (!ws || ws_bytes < L.total || !aligned(ws, 256))
    return set_error(CLSA_ERR_WORKSPACE, "topk: workspace of %zu bytes (256-aligned) required, got %zu",
                     L.total, ws ? ws_bytes : (size_t)0);
  char* base = static_cast<char*>(ws);
  uint32_t* arrivals = reinterpret_cast<uint32_t*>(base + L.arrivals);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (topk_uses_arrivals(B * T, kv_len, k) && (rc = zero_words(arrivals, L.arrival_words, s))) return rc;
  return launch_topk(scores, B, T, kv_len, k, k_per_query, margin, idx, kept,
                     reinterpret_cast<uint32_t*>(base + L.counts),
                     reinterpret_cast<int32_t*>(base + L.cand),
                     reinterpret_cast<int32_t*>(base + L.spill), arrivals, s);
}

int clsa_topk_vark(const float* scores, int B, int T, int kv_len, int k, const int32_t* k_per_query,
                   int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  return clsa_topk_margin(scores, B, T, kv_len, k, k_per_query, INFINITY, idx, nullptr, ws, ws_bytes,
                          stream);
}

int clsa_topk(const float* scores, int B, int T, int kv_len, int k, int32_t* idx, void* ws,
              size_t ws_bytes, void* stream) {
  return clsa_topk_margin(scores, B, T, kv_len, k, nullptr, INFINITY, idx, nullptr, ws, ws_bytes,
                          stream);
}

int clsa_sparse_attn(const void* q, const void* k_cache, const void* v_cache, int dtype,
                     const int32_t* idx, int k, void* out, float* lse, int B, int T, int Hq,
                     int Hkv, int D, int kv_len, int L_cap, float scale, void* ws, size_t ws_bytes,
                     void* stream) {
  int rc = check_attn_args(q, k_cache, v_cache, dtype, idx, k, out, lse, B, T, Hq, Hkv, D, kv_len,
                           L_cap);
  if (rc) return rc;
  if (!(scale == scale) || isinf(scale))
    return set_error(CLSA_ERR_INVALID_ARG, "sparse_attn: scale must be finite");
  const AttnWs L = attn_ws(B, T, Hq, Hkv, k);
  if (!ws || ws_bytes < L.total || !aligned(ws, 256))
    return set_error(CLSA_ERR_WORKSPACE,
                     "sparse_attn: workspace of %zu bytes (256-aligned) required, got %zu", L.total,
                     ws ? ws_bytes : (size_t)0);
  char* base = static_cast<char*>(ws);
  return launch_sparse_attn(q, k_cache, v_cache, dtype, idx, k, out, lse, B, T, Hq, Hkv, D, kv_len,
                            L_cap, scale, reinterpret_cast<float*>(base + L.partials), nullptr,
                            static_cast<hipStream_t>(stream));
}

static int check_step(const clsa_step_desc* d) {
  if (!d) return set_error(CLSA_ERR_INVALID_ARG, "decode_step: null descriptor");
  const int n = d->n_layers;
  if (n < 1 || !d->layer_src || !d->q || !d->k_cache || !d->v_cache || !d->out || !d->idx_out)
    return set_error(CLSA_ERR_INVALID_ARG, "decode_step: n_layers < 1 or null array");
  if (d->layer_src[0] != 0)
    return set_error(CLSA_ERR_INVALID_ARG, "decode_step: layer 0 must be a full (indexer) layer");
  int last_f = -1;
  for (int l = 0; l < n; l++) {
    if (d->layer_src[l] == l) last_f = l;
    if (d->layer_src[l] != last_f)
      return set_error(CLSA_ERR_INVALID_ARG,
                       "decode_step: layer_src[%d]=%d is not the nearest full layer (%d)", l,
                       d->layer_src[l], last_f);
    const bool full = d->layer_src[l] == l;
    if (full && (!d->q_idx || !d->k_idx || !d->w))
      return set_error(CLSA_ERR_INVALID_ARG, "decode_step: indexer arrays required");
    const float* lse = d->lse ? d->lse[l] : nullptr;
    int rc = check_attn_args(d->q[l], d->k_cache[l], d->v_cache[l], d->dtype, d->idx_out, d->k,
                             d->out[l], lse, d->B, d->T, d->Hq, d->Hkv, d->D, d->kv_len, d->L_cap);
    if (rc) return rc;
    if (full) {
      // scores are carved from the workspace; pass a dummy aligned pointer for the check
      rc = check_index_args(d->q_idx[l], d->k_idx[l], d->idx_dtype, d->w[l],
                            reinterpret_cast<const float*>(d->idx_out), d->B, d->T, d->H_I, d->D_I,
                            d->kv_len, d->L_cap);
      if (rc) return rc;
    }
    if (d->events)
      for (int e = 0; e < 4; e++)
        if (!d->events[4 * l + e])
          return set_error(CLSA_ERR_INVALID_ARG, "decode_step: null event %d", 4 * l + e);
  }
  int rc = check_topk_args(reinterpret_cast<const float*>(d->idx_out), d->B, d->T, d->kv_len, d->k,
                           d->idx_out);
  if (rc) return rc;
  if (!(d->scale == d->scale) || isinf(d->scale))
    return set_error(CLSA_ERR_INVALID_ARG, "decode_step: scale must be finite");
  if (d->k_per_query && !aligned(d->k_per_query, 4))
    return set_error(CLSA_ERR_INVALID_ARG, "decode_step: misaligned k_per_query");
  if (d->skip_margin && !(*d->skip_margin >= 0.f))
    return set_error(CLSA_ERR_INVALID_ARG, "decode_step: skip_margin must be >= 0 (or +inf)");
  return CLSA_OK;
}

size_t clsa_decode_step_workspace_bytes(const clsa_step_desc* d) {
  if (check_step(d)) return 0;
  return step_ws(d->B, d->T, d->Hq, d->Hkv, d->kv_len, d->k).total;
}

int clsa_decode_step(const clsa_step_desc* d, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_step(d);
  if (rc) return rc;
  const StepWs L = step_ws(d->B, d->T, d->Hq, d->Hkv, d->kv_len, d->k);
  if (!ws || ws_bytes < L.total || !aligned(ws, 256))
    return set_error(CLSA_ERR_WORKSPACE,
                     "decode_step: workspace of %zu bytes (256-aligned) required, got %zu", L.total,
                     ws ? ws_bytes : (size_t)0);
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  uint32_t* arrivals = reinterpret_cast<uint32_t*>(base + L.topk.arrivals);
  uint32_t* counts = reinterpret_cast<uint32_t*>(base + L.topk.counts);
  int32_t* cand = reinterpret_cast<int32_t*>(base + L.topk.cand);
  int32_t* spill = reinterpret_cast<int32_t*>(base + L.topk.spill);
  float* partials = reinterpret_cast<float*>(base + L.partials);
  float* scores = reinterpret_cast<float*>(base + L.scores);
  const float margin = d->skip_margin ? *d->skip_margin : INFINITY;
  // Per-query counts or a finite margin leave -1 tails in the index rows:
  // the top-k then writes each row's count and attention reads only that
  // many entries (the counts stay with the index for the S layers).
  int32_t* kept = d->k_per_query != nullptr || margin < INFINITY
                      ? reinterpret_cast<int32_t*>(base + L.kept)
                      : nullptr;
  // The one-launch top-k needs its arrival region (arrival words and row
  // histograms) zero: each F layer's indexer kernel clears it before the
  // top-k that follows it runs.
  ZeroJob zj;
  if (topk_uses_arrivals(d->B * d->T, d->kv_len, d->k)) zj = ZeroJob{arrivals, (int)L.topk.arrival_words};
  for (int l = 0; l < d->n_layers; l++) {
    if ((rc = record(d->events, 4 * l, s))) return rc;
    if (d->layer_src[l] == l) {
      rc = launch_index_score(d->q_idx[l], d->k_idx[l], d->idx_dtype, d->w[l], scores, d->B, d->T,
                              d->H_I, d->D_I, d->kv_len, d->L_cap, zj, s);
      if (rc) return rc;
      if ((rc = record(d->events, 4 * l + 1, s))) return rc;
      rc = launch_topk(scores, d->B, d->T, d->kv_len, d->k, d->k_per_query, margin, d->idx_out,
                       kept, counts, cand, spill, arrivals, s);
      if (rc) return rc;
    } else if ((rc = record(d->events, 4 * l + 1, s))) {
      return rc;
    }
    if ((rc = record(d->events, 4 * l + 2, s))) return rc;
    rc = launch_sparse_attn(d->q[l], d->k_cache[l], d->v_cache[l], d->dtype, d->idx_out, d->k,
                            d->out[l], d->lse ? d->lse[l] : nullptr, d->B, d->T, d->Hq, d->Hkv,
                            d->D, d->kv_len, d->L_cap, d->scale, partials, kept, s);
    if (rc) return rc;
    if ((rc = record(d->events, 4 * l + 3, s))) return rc;
  }
  return CLSA_OK;
}

int clsa_block_union_build(const int32_t* idx, int B, int T, int k, int kv_len, int block, int Hkv,
                           int32_t* kv_indptr, int32_t* kv_indices, void* ws, size_t ws_bytes,
                           void* stream) {
  if (!idx || !kv_indptr || !kv_indices)
    return set_error(CLSA_ERR_INVALID_ARG, "block_union_build: null pointer");
  int rc = check_shape(B, T, kv_len, kv_len);
  if (rc) return rc;
  if (k < 1 || block < 1 || Hkv < 1)
    return set_error(CLSA_ERR_INVALID_ARG, "block_union_build: k=%d, block=%d, Hkv=%d", k, block,
                     Hkv);
  if (!aligned(idx, 4) || !aligned(kv_indptr, 4) || !aligned(kv_indices, 4))
    return set_error(CLSA_ERR_INVALID_ARG, "block_union_build: misaligned pointer");
  const size_t need = block_union_ws_bytes(B, kv_len, block);
  if (!ws || ws_bytes < need || !aligned(ws, 256))
    return set_error(CLSA_ERR_WORKSPACE, "block_union_build: workspace of %zu bytes required", need);
  return launch_block_union(idx, B, T, k, kv_len, block, Hkv, kv_indptr, kv_indices, ws,
                            static_cast<hipStream_t>(stream));
}

static int block_paged_attn(const void* q, const void* k_cache, const void* v_cache, int dtype,
                          const int32_t* kv_indptr, const int32_t* kv_indices, int block, void* out,
                          float* lse, int B, int T, int Hq, int Hkv, int D, int kv_len, int L_cap,
                          float scale, bool head_major, void* stream) {
  if (!q || !k_cache || !v_cache || !kv_indptr || !kv_indices || !out)
    return set_error(CLSA_ERR_INVALID_ARG, "block_paged_attn: null pointer");
  int rc = check_shape(B, T, kv_len, L_cap);
  if (rc) return rc;
  if (Hq < 1 || Hkv < 1 || D < 1 || Hq % Hkv || block < 1)
    return set_error(CLSA_ERR_INVALID_ARG, "block_paged_attn: Hq=%d, Hkv=%d, D=%d, block=%d", Hq,
                     Hkv, D, block);
  if (!block_paged_attn_supported(dtype, Hq, Hkv, D, block))
    return set_error(CLSA_ERR_UNSUPPORTED, "block_paged_attn: dtype %d, Hq=%d, Hkv=%d, D=%d", dtype,
                     Hq, Hkv, D);
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(kv_indptr, 4) || !aligned(kv_indices, 4) || (lse && !aligned(lse, 4)))
    return set_error(CLSA_ERR_INVALID_ARG, "block_paged_attn: misaligned pointer");
  if (!(scale == scale) || isinf(scale))
    return set_error(CLSA_ERR_INVALID_ARG, "block_paged_attn: scale must be finite");
  return launch_block_paged_attn(q, k_cache, v_cache, dtype, kv_indptr, kv_indices, block, out, lse,
                                 B, T, Hq, Hkv, D, kv_len, L_cap, scale, head_major,
                                 static_cast<hipStream_t>(stream));
}

int clsa_block_paged_attn(const void* q, const void* k_cache, const void* v_cache, int dtype,
                          const int32_t* kv_indptr, const int32_t* kv_indices, int block, void* out,
                          float* lse, int B, int T, int Hq, int Hkv, int D, int kv_len, int L_cap,
                          float scale, void* stream) {
  return block_paged_attn(q, k_cache, v_cache, dtype, kv_indptr, kv_indices, block, out, lse, B, T, Hq,
                          Hkv, D, kv_len, L_cap, scale, false, stream);
}

int clsa_block_paged_attn_hm(const void* q, const void* k_cache, const void* v_cache, int dtype,
                             const int32_t* kv_indptr, const int32_t* kv_indices, int block,
                             void* out, float* lse, int B, int T, int Hq, int Hkv, int D, int kv_len,
                             int L_cap, float scale, void* stream) {
  return block_paged_attn(q, k_cache, v_cache, dtype, kv_indptr, kv_indices, block, out, lse, B, T, Hq,
                          Hkv, D, kv_len, L_cap, scale, true, stream);
}

int clsa_cache_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache, int dtype,
                      const void* kidx_new, void* k_idx, int idx_dtype, int B, int T, int Hkv, int D,
                      int D_I, int pos, int L_cap, void* stream) {
  if (!k_new || !v_new || !k_cache || !v_cache)
    return set_error(CLSA_ERR_INVALID_ARG, "cache_append: null pointer");
  if ((kidx_new == nullptr) != (k_idx == nullptr))
    return set_error(CLSA_ERR_INVALID_ARG, "cache_append: kidx_new and k_idx must both be set or both NULL");
  if (B < 1 || T < 1 || Hkv < 1 || D < 1 || (k_idx && D_I < 1))
    return set_error(CLSA_ERR_INVALID_ARG, "cache_append: B=%d T=%d Hkv=%d D=%d D_I=%d", B, T, Hkv, D, D_I);
  if (pos < 0 || (long)pos + T > L_cap)
    return set_error(CLSA_ERR_INVALID_ARG, "cache_append: rows [%d, %ld) outside L_cap=%d", pos,
                     (long)pos + T, L_cap);
  if ((long)B * T > 0x7fffffffL)
    return set_error(CLSA_ERR_UNSUPPORTED, "cache_append: B*T=%ld", (long)B * T);
  if (dtype != CLSA_F32 && dtype != CLSA_BF16)
    return set_error(CLSA_ERR_INVALID_ARG, "cache_append: unknown dtype %d", dtype);
  if (k_idx && idx_dtype != CLSA_F32 && idx_dtype != CLSA_BF16 && idx_dtype != CLSA_FP8_E4M3FN)
    return set_error(CLSA_ERR_INVALID_ARG, "cache_append: unknown indexer dtype %d", idx_dtype);
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      (k_idx && (!aligned(kidx_new, 16) || !aligned(k_idx, 16))))
    return set_error(CLSA_ERR_INVALID_ARG, "cache_append: misaligned pointer");
  const size_t kv_row = (size_t)Hkv * D * (dtype == CLSA_F32 ? 4 : 2);
  const size_t ki_row = k_idx ? (size_t)D_I * (idx_dtype == CLSA_F32 ? 4 : idx_dtype == CLSA_BF16 ? 2 : 1) : 0;
  AppendJob jobs[3] = {{static_cast<const char*>(k_new), static_cast<char*>(k_cache), kv_row},
                       {static_cast<const char*>(v_new), static_cast<char*>(v_cache), kv_row},
                       {static_cast<const char*>(kidx_new), static_cast<char*>(k_idx), ki_row}};
  const int n_jobs = k_idx ? 3 : 2;
  const size_t rows = (size_t)B * T;
  for (int i = 0; i < n_jobs; i++) {
    const size_t src_bytes = rows * jobs[i].row_bytes;
    for (int o = 0; o < n_jobs; o++) {
      const char* s0 = jobs[i].src;
      const char* d0 = jobs[o].dst;
      const size_t d_bytes = (size_t)B * L_cap * jobs[o].row_bytes;
      if (s0 < d0 + d_bytes && d0 < s0 + src_bytes)
        return set_error(CLSA_ERR_INVALID_ARG, "cache_append: a source overlaps a destination");
    }
  }
  return launch_cache_append(jobs, n_jobs, B, T, pos, L_cap, static_cast<hipStream_t>(stream));
}

}  // extern "C"
