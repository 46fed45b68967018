// kernels.h — internal launchers of libclsa (not part of the C ABI).
// Every launcher assumes its arguments were validated by api.cpp and returns
// a clsa_status.
#pragma once

#include "common.h"

namespace clsa {

// ---- cache append ------------------------------------------------------------
// One tensor to append: B*T rows of row_bytes from src (row r = b*T + t) to
// dst row b*L_cap + pos + t.
struct AppendJob {
  const char* src;
  char* dst;
  size_t row_bytes;
};
int launch_cache_append(const AppendJob* jobs, int n_jobs, int B, int T, int pos, int L_cap,
                        hipStream_t stream);

// ---- indexer score ---------------------------------------------------------
// Words a launch clears besides its own work (n = 0: none).
struct ZeroJob {
  uint32_t* p = nullptr;
  int n = 0;
};
int launch_index_score(const void* q_idx, const void* k_idx, int idx_dtype, const float* w,
                       float* scores, int B, int T, int H_I, int D_I, int kv_len, int L_cap,
                       const ZeroJob& z, hipStream_t stream);
bool index_score_supported(int idx_dtype, int H_I, int D_I);

// ---- top-k -----------------------------------------------------------------
// Buffers: counts [rows * nchunks] u32, cand [rows * nchunks * kTopkSegCap]
// (position, key) pairs of i32, spill [rows * kv_len] i32 (used only when a
// row is redone in full).
constexpr int kTopkBins = 4096;
constexpr int kTopkChunk = 4096;
constexpr int kTopkSegCap = 1024;     // candidates kept per chunk
constexpr int kTopkMaxChunks = 1024;  // kv_len <= 4M
struct TopkBuffers {
  int nchunks, cstride;  // chunks per row; counts words per row
  size_t counts_words, cand_words, spill_words, arrival_words;
};
TopkBuffers topk_buffers(int rows, int kv_len);
// Whether launch_topk takes the one-launch path, whose arrival region
// (arrival_words u32: per row an arrival word and a candidate histogram)
// must be zero before every launch.
bool topk_uses_arrivals(int rows, int kv_len, int k);
// k_rows: NULL, or a device int32 [B*T] of per-row counts (clamped to [0, k]).
// margin: +inf, or the ordered-skipping margin (>= 0): each row keeps only the
// selected positions scoring at least (row maximum - margin). kept: NULL, or
// a device int32 [B*T] receiving each row's count of kept positions.
int launch_topk(const float* scores, int B, int T, int kv_len, int k, const int32_t* k_rows,
                float margin, int32_t* idx, int32_t* kept, uint32_t* counts, int32_t* cand,
                int32_t* spill, uint32_t* arrivals, hipStream_t stream);

// ---- sparse attention --------------------------------------------------------
// Buffer: partials [attn_partial_floats(...)] f32 (split states; unused when
// the k entries are not split).
struct AttnSplit {
  int splits, rows_per_split;
  int waves_per_head;  // waves sharing one split of one KV head
};
AttnSplit attn_split(int B, int T, int Hkv, int k, bool mfma);
size_t attn_partial_floats(int B, int T, int Hq, int Hkv, int k);
bool sparse_attn_supported(int dtype, int Hq, int Hkv, int D);
// row_len: NULL, or a device int32 [B*T] of per-row entry counts for index
// rows whose entries past their count are all -1 (as the top-k writes them
// with per-query counts or a margin); only the first row_len[row] entries
// (clamped to [0, k]) are read.
int launch_sparse_attn(const void* q, const void* kc, const void* vc, int dtype, const int32_t* idx,
                       int k, void* out, float* lse, int B, int T, int Hq, int Hkv, int D,
                       int kv_len, int L_cap, float scale, float* partials,
                       const int32_t* row_len, hipStream_t stream);

// ---- block union comparator ----------------------------------------------------
size_t block_union_ws_bytes(int B, int kv_len, int block);
int launch_block_union(const int32_t* idx, int B, int T, int k, int kv_len, int block, int Hkv,
                       int32_t* kv_indptr, int32_t* kv_indices, void* ws, hipStream_t stream);
// head_major: caches are [B, Hkv, L_cap, D] instead of [B, L_cap, Hkv, D].
int launch_block_paged_attn(const void* q, const void* kc, const void* vc, int dtype,
                            const int32_t* kv_indptr, const int32_t* kv_indices, int block,
                            void* out, float* lse, int B, int T, int Hq, int Hkv, int D,
                            int kv_len, int L_cap, float scale, bool head_major,
                            hipStream_t stream);
bool block_paged_attn_supported(int dtype, int Hq, int Hkv, int D, int block);

}  // namespace clsa
