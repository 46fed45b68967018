/*
 * clsa.h — C ABI of libclsa.so: token-level sparse attention with one
 * routing index shared across layers, for AMD Instinct MI355X (gfx950).
 *
 * The method (sources are the pages this library is built from):
 *  - "CLSA: You Only Index Once", as reported by the SeventNews article
 *    "Le routage partagé entre couches accélère l'attention sparse de 7x sans
 *    perte de qualité", section "Comment CLSA fonctionne": in a model whose
 *    cross-decoder layers share one KV cache (YOCO family), one indexer layer
 *    scores the cache once, keeps the top-k tokens, and every following layer
 *    attends to exactly those tokens, so routing is paid once per step
 *    instead of once per layer.
 *  - "IndexCache: Accelerating Sparse Attention via Cross-Layer Index Reuse"
 *    (gist.science summary), section "2. Méthodologie : IndexCache": layers
 *    are either F (run their own indexer, overwrite the cached top-k indices)
 *    or S (run no indexer, reuse the indices of the nearest F layer above
 *    them); section "1. Problématique": the DSA lightning indexer scores all
 *    previous tokens and main attention then runs over the k selected ones.
 *  - "CompactAttention: Accelerating Chunked Prefill with Block-Union KV
 *    Selection" (gist.science summary), section "Méthodologie", selection and
 *    execution steps: per KV group, the union of selected KV blocks over all
 *    query blocks of a chunk and over the heads of the group, handed to a
 *    dense paged kernel as kv_indptr / kv_indices and read in place.
 *
 * Conventions shared by every entry point
 *  - Tensors are dense, row-major device buffers (hipMalloc'd or torch CUDA
 *    tensors). Shapes are written outermost-first.
 *  - B batch, T queries per call (1 for decode), kv_len cached tokens visible
 *    to the last query of the call, L_cap >= kv_len allocated cache rows,
 *    H_I / D_I indexer heads / dim, Hq / Hkv / D attention heads / dim.
 *  - Causality: query t (0-based) of a call sees cache positions
 *    [0, kv_len - T + t]; for decode (T = 1) that is the whole [0, kv_len).
 *  - GQA: query head h reads KV head g = h / (Hq / Hkv).
 *  - Ownership: the caller allocates and frees every buffer, including the
 *    workspace. The library allocates no device memory and keeps no device
 *    state between calls (one exception: the scratch array behind
 *    clsa_decode_step_static, which the library holds on each GPU). Host
 *    arrays are only read during the call.
 *  - Asynchrony: every call enqueues its kernels on `stream` (a hipStream_t;
 *    NULL means the default stream) and returns without synchronising.
 *  - Errors: all arguments are validated before the first launch, so a call
 *    that returns an error has enqueued nothing. CLSA_ERR_HIP reports a
 *    failed launch; launches already enqueued by that call stay enqueued.
 *    clsa_last_error() returns a thread-local message for the last failure.
 *  - Thread safety: calls are re-entrant. Calls that may run concurrently
 *    (different streams, or different threads) need separate workspaces.
 */
#ifndef CLSA_H
#define CLSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CLSA_ABI_VERSION 3

/* Status codes returned by every entry point. */
enum clsa_status {
  CLSA_OK = 0,
  CLSA_ERR_INVALID_ARG = -1, /* null pointer, bad size, inconsistent shapes */
  CLSA_ERR_UNSUPPORTED = -2, /* valid request outside what the kernels cover */
  CLSA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  CLSA_ERR_HIP = -4          /* a HIP runtime call or launch failed */
};

/* Element types. FP8 is the OCP E4M3FN format (bias 7, no infinities),
 * the native fp8 format of gfx950 matrix cores. */
enum clsa_dtype { CLSA_F32 = 0, CLSA_BF16 = 1, CLSA_FP8_E4M3FN = 2 };

/* Operation ids for clsa_workspace_bytes. */
enum clsa_op { CLSA_OP_TOPK = 0, CLSA_OP_SPARSE_ATTN = 1, CLSA_OP_BLOCK_UNION = 2 };

/* Library ABI version (CLSA_ABI_VERSION at build time). */
int clsa_abi_version(void);

/* Static description of a status code. Never NULL. */
const char* clsa_status_string(int status);

/* Thread-local message describing the last failing call on this thread
 * ("" if none). Valid until the next failing call on the same thread. */
const char* clsa_last_error(void);

/*
 * Workspace size, in bytes, for one call of operation `op` with the given
 * sizes (unused sizes are ignored; pass 0). Returns 0 for invalid sizes.
 *   CLSA_OP_TOPK:        uses B, T, kv_len, k
 *   CLSA_OP_SPARSE_ATTN: uses B, T, Hq, Hkv, D, k
 *   CLSA_OP_BLOCK_UNION: uses B, kv_len, block
 */
size_t clsa_workspace_bytes(int op, int B, int T, int Hq, int Hkv, int D,
                            int kv_len, int k, int block);

/*
 * Indexer scores (IndexCache summary, "1. Problématique": the lightning
 * indexer scores every previous token; CLSA article, "Comment CLSA
 * fonctionne": the shared indexer layer computes those scores once).
 * The pages give no formula; the score used here is
 *   scores[b,t,s] = sum_h w[b,t,h] * max(0, sum_d q_idx[b,t,h,d] * k_idx[b,s,d])
 * for every position s that query t sees, and -inf for s it does not see.
 *
 *   q_idx  [B, T, H_I, D_I]  idx_dtype (F32, BF16 or FP8_E4M3FN)
 *   k_idx  [B, L_cap, D_I]   idx_dtype, one indexer key per cached token
 *   w      [B, T, H_I]       float32 head weights
 *   scores [B, T, kv_len]    float32 output
 * Accumulation is float32. BF16 and FP8 run on matrix cores and need
 * H_I in {16, 32, 48, 64} and D_I in {64, 128}; F32 takes any H_I, D_I
 * with H_I * D_I <= 8192. Other shapes return CLSA_ERR_UNSUPPORTED.
 * Pointers must be 16-byte aligned.
 */
int clsa_index_score(const void* q_idx, const void* k_idx, int idx_dtype,
                     const float* w, float* scores, int B, int T, int H_I,
                     int D_I, int kv_len, int L_cap, void* stream);

/*
 * Per-query top-k over indexer scores (CLSA article, "Comment CLSA
 * fonctionne": the indexer keeps the top-k tokens; IndexCache summary,
 * "1. Problématique": DSA keeps the k most relevant tokens per query).
 *   scores [B, T, kv_len] float32 (entries past query t's visible range are
 *                          ignored, whatever they hold)
 *   idx    [B, T, k]      int32 output
 * Selection order is (score descending, position ascending): among equal
 * scores the lower position wins; -0.0 and +0.0 are equal. The k chosen
 * positions are written in ascending order; when query t sees fewer than k
 * positions, all of them are written and the rest of the row is -1.
 * Scores must not be NaN. k >= 1.
 * Workspace: clsa_workspace_bytes(CLSA_OP_TOPK, B, T, 0, 0, 0, kv_len, k, 0).
 */
int clsa_topk(const float* scores, int B, int T, int kv_len, int k,
              int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/*
 * clsa_topk with a per-query count: query (b, t) keeps its
 * k_per_query[b, t] best positions (clamped to [0, k]) and the remaining
 * slots of its k-wide row hold -1. The pages keep k fixed and name a k
 * chosen by the indexer layer as the open extension (CLSA article, "Le
 * coût : limites de compatibilité"; "Ce que cela signifie pour
 * l'inférence sur longs contextes"); the rule that picks each count is the
 * caller's. k_per_query: device int32 [B, T], or
 * NULL for k everywhere. Same workspace, ordering and errors as clsa_topk.
 */
int clsa_topk_vark(const float* scores, int B, int T, int kv_len, int k,
                   const int32_t* k_per_query, int32_t* idx, void* ws,
                   size_t ws_bytes, void* stream);

/*
 * Ordered skipping (CoSA summary, the paragraphs on the Kernel-Aware Proxy
 * and the Ordered-Skipping Kernel: the proxy hands the kernel a priority
 * list, the kernel reads the most important entries first and skips the
 * rest). The page gives no stopping rule; the one taken here: each query's
 * selection (as clsa_topk_vark) is read in priority order, score descending
 * then position ascending, and reading stops at the first entry whose score
 * is below thr = (the query's best score) - margin, thr computed in float32
 * (round to nearest). The positions read are written ascending and the rest
 * of the k-wide row is -1. Since the kept set is decided before attention,
 * attention visits it in position order; the result equals reading it in
 * priority order up to float32 summation order.
 *   margin  >= 0; +INFINITY keeps the whole selection (clsa_topk_vark).
 *           Negative or NaN: CLSA_ERR_INVALID_ARG.
 *   kept    device int32 [B, T] output (positions kept per query), or NULL.
 * If thr is NaN (best score +inf with margin +inf) nothing is skipped.
 * Same workspace, ordering, scores and other errors as clsa_topk.
 */
int clsa_topk_margin(const float* scores, int B, int T, int kv_len, int k,
                     const int32_t* k_per_query, float margin, int32_t* idx,
                     int32_t* kept, void* ws, size_t ws_bytes, void* stream);

/*
 * Gathered sparse attention over the selected tokens (IndexCache summary,
 * "1. Problématique": main attention over the k selected tokens, O(Lk);
 * CLSA article, "Comment CLSA fonctionne": every layer after the indexer
 * attends to the same index). For query head h with KV head g:
 *   z_j = scale * q[b,t,h,:] . k_cache[b, idx[b,t,j], g, :]
 *   out[b,t,h,:] = sum_j softmax(z)_j * v_cache[b, idx[b,t,j], g, :]
 *   lse[b,t,h]   = log sum_j exp(z_j)
 * over the entries j whose position lies in query t's visible range;
 * other entries (such as -1 padding) are skipped, repeated positions count
 * once per occurrence. A query with no valid entry gets out = 0, lse = -inf.
 *   q       [B, T, Hq, D]         dtype (F32 or BF16)
 *   k_cache [B, L_cap, Hkv, D]    dtype, token-major
 *   v_cache [B, L_cap, Hkv, D]    dtype
 *   idx     [B, T, k]             int32
 *   out     [B, T, Hq, D]         dtype output (BF16 rounded once, to nearest even)
 *   lse     [B, T, Hq]            float32 output, or NULL
 * scale <= 0 selects 1/sqrt(D). Softmax and accumulation are float32; with
 * BF16 the probabilities enter the matrix-core P.V product as a bf16 pair
 * (hi = bf16(p), lo = bf16(p - hi): about 16 significant bits), F32 keeps
 * them in float32.
 * Supported: D = 128, Hq / Hkv in {1, 2, 4, 8}.
 * Workspace: clsa_workspace_bytes(CLSA_OP_SPARSE_ATTN, B, T, Hq, Hkv, D, 0, k, 0).
 */
int clsa_sparse_attn(const void* q, const void* k_cache, const void* v_cache,
                     int dtype, const int32_t* idx, int k, void* out,
                     float* lse, int B, int T, int Hq, int Hkv, int D,
                     int kv_len, int L_cap, float scale, void* ws,
                     size_t ws_bytes, void* stream);

/*
 * One decode (or chunk) step over n_layers attention layers that share
 * routing (CLSA article, "Comment CLSA fonctionne"; IndexCache summary,
 * "2. Méthodologie : IndexCache").
 * layer_src[l] names the F layer whose index layer l uses. Layer l is an F
 * layer iff layer_src[l] == l; it then runs clsa_index_score and clsa_topk on
 * its own indexer inputs and overwrites idx_out. Every layer then runs
 * clsa_sparse_attn with idx_out. Constraints: layer_src[0] == 0 and
 * layer_src[l] is the nearest F layer at or before l (the cached index is
 * overwritten by each new F layer). CLSA's single shared indexer is the
 * pattern {0, 0, ..., 0}; IndexCache's 1-in-4 pattern is {0,0,0,0,4,4,...}.
 * Per-layer K/V pointers may alias (one YOCO cache) or differ.
 */
typedef struct clsa_step_desc {
  int n_layers;
  const int32_t* layer_src;     /* host [n_layers] */
  /* Host arrays of n_layers device pointers each. */
  const void* const* q;         /* [B, T, Hq, D] dtype */
  const void* const* k_cache;   /* [B, L_cap, Hkv, D] dtype */
  const void* const* v_cache;   /* [B, L_cap, Hkv, D] dtype */
  void* const* out;             /* [B, T, Hq, D] dtype */
  float* const* lse;            /* [B, T, Hq] float32; array or entries may be NULL */
  const void* const* q_idx;     /* F layers: [B, T, H_I, D_I] idx_dtype; S: ignored */
  const void* const* k_idx;     /* F layers: [B, L_cap, D_I] idx_dtype; S: ignored */
  const float* const* w;        /* F layers: [B, T, H_I] float32; S: ignored */
  int32_t* idx_out;             /* device [B, T, k]: the index cache, left holding
                                   the last F layer's index */
  int dtype, idx_dtype;
  int B, T, Hq, Hkv, D, H_I, D_I, kv_len, L_cap, k;
  float scale;                  /* <= 0: 1/sqrt(D) */
  /* Optional timing hooks: NULL, or a host array of 4 * n_layers hipEvent_t
   * handles created by the caller. For layer l the call records
   * events[4l] before the indexer, events[4l+1] between indexer and top-k,
   * events[4l+2] before attention and events[4l+3] after it (S layers record
   * the first three back to back). */
  void* const* events;
  /* Optional per-query counts: NULL (every query keeps k positions), or a
   * device int32 [B, T]; query (b, t) keeps its k_per_query[b, t] best
   * positions (clamped to [0, k]) as in clsa_topk_vark. */
  const int32_t* k_per_query;
  /* Optional ordered skipping: NULL (off), or a host pointer to the margin
   * (>= 0) that F layers' top-k apply as in clsa_topk_margin; read during
   * the call only. With per-query counts or a finite margin, the top-k keeps
   * each query's count in the workspace and attention reads only that many
   * entries of its index row. */
  const float* skip_margin;
} clsa_step_desc;

/* Workspace bytes needed by clsa_decode_step for this descriptor (0 if the
 * descriptor's sizes are invalid). */
size_t clsa_decode_step_workspace_bytes(const clsa_step_desc* d);

int clsa_decode_step(const clsa_step_desc* d, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * clsa_decode_step without a workspace argument, for callers that cannot
 * allocate device memory: work recorded under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation. The step's scratch (the
 * bytes clsa_decode_step_workspace_bytes(d) reports) lives in a device array
 * of CLSA_STATIC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends; the call allocates nothing. A step needing more
 * returns CLSA_ERR_WORKSPACE before launching anything (at the 128K-context
 * decode, B = 4, it needs about 6 MiB; a 2048-query chunk's scores alone are
 * about 1 GiB and do not fit). Every call on one GPU uses that GPU's array:
 * calls that overlap in time on one GPU (several streams or threads) race on
 * it and must be serialised by the caller. Results, errors and the
 * descriptor are as for clsa_decode_step on the current device.
 */
#define CLSA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int clsa_decode_step_static(const clsa_step_desc* d, void* stream);

/*
 * Block-union KV table (CompactAttention summary, "Méthodologie", selection
 * step): for each (b, KV group g), the ascending list of block ids
 * floor(s / block) over every valid position s in idx[b, :, :] (union over
 * all T queries of the chunk and, because one index serves every head,
 * trivially over the heads of the group). A position is valid when it lies
 * in its query's visible range.
 *   idx        [B, T, k] int32
 *   kv_indptr  [B * Hkv + 1] int32 output: table (b, g) is
 *              kv_indices[kv_indptr[b*Hkv+g] .. kv_indptr[b*Hkv+g+1])
 *   kv_indices [B * Hkv * ceil(kv_len / block)] int32 output (capacity)
 * Workspace: clsa_workspace_bytes(CLSA_OP_BLOCK_UNION, B, 0, 0, 0, 0, kv_len, 0, block).
 */
int clsa_block_union_build(const int32_t* idx, int B, int T, int k,
                           int kv_len, int block, int Hkv, int32_t* kv_indptr,
                           int32_t* kv_indices, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * Dense attention over the blocks of a block table, read in place from the
 * token-major cache (CompactAttention summary, "Méthodologie", execution
 * step). Query t of head h (group g) attends, with causal masking, to every
 * position s < kv_len - T + t + 1 inside the blocks listed for (b, g).
 * Shapes and dtype as clsa_sparse_attn (BF16 only), plus the table from
 * clsa_block_union_build. Supported: D = 128, Hq / Hkv in {1, 2, 4, 8}.
 */
int clsa_block_paged_attn(const void* q, const void* k_cache,
                          const void* v_cache, int dtype,
                          const int32_t* kv_indptr, const int32_t* kv_indices,
                          int block, void* out, float* lse, int B, int T,
                          int Hq, int Hkv, int D, int kv_len, int L_cap,
                          float scale, void* stream);

/*
 * clsa_block_paged_attn over head-major caches: k_cache and v_cache are
 * [B, Hkv, L_cap, D], so every (batch, KV head, block) is one contiguous
 * piece of memory, the layout CompactAttention's execution step reads in
 * place (CompactAttention summary, "Méthodologie", execution step:
 * zero-copy paged attention over the block table). Everything else as
 * clsa_block_paged_attn.
 */
int clsa_block_paged_attn_hm(const void* q, const void* k_cache,
                             const void* v_cache, int dtype,
                             const int32_t* kv_indptr,
                             const int32_t* kv_indices, int block, void* out,
                             float* lse, int B, int T, int Hq, int Hkv, int D,
                             int kv_len, int L_cap, float scale, void* stream);

/*
 * Appends T new tokens per batch element to the caches: every extra token of
 * context adds a K and a V row (CLSA article, opening section), written once
 * into the cache that all cross-decoder layers share (CLSA article,
 * "Comment CLSA fonctionne"), together with the token's indexer key.
 *   k_new, v_new  [B, T, Hkv, D]  dtype (F32 or BF16)  ->  k_cache, v_cache
 *                 [B, L_cap, Hkv, D], rows pos .. pos + T - 1
 *   kidx_new      [B, T, D_I]     idx_dtype            ->  k_idx [B, L_cap, D_I]
 * kidx_new and k_idx are both NULL (no indexer keys) or both set. Bytes are
 * copied unchanged; rows outside [pos, pos + T) are not touched. Needs
 * pos >= 0 and pos + T <= L_cap; sources must not overlap destinations. The
 * caller owns every buffer; one launch on `stream`, no workspace. Pointers
 * must be 16-byte aligned.
 */
int clsa_cache_append(const void* k_new, const void* v_new, void* k_cache,
                      void* v_cache, int dtype, const void* kidx_new,
                      void* k_idx, int idx_dtype, int B, int T, int Hkv,
                      int D, int D_I, int pos, int L_cap, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CLSA_H */
