/*
 * clsa_oracle.c — plain CPU oracle for token-level sparse attention with a
 * cross-layer shared index.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the reference that the HIP library
 * is checked against. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load it; the product path never does. It shares no
 * code, header, table or helper with the HIP library.
 *
 * Style: single-threaded, scalar, obviously correct. Every sum is taken in
 * double, in the natural loop order, with no blocking, fusion or reordering.
 * Element decoding (bfloat16, OCP fp8 E4M3FN) is written out from the format
 * definitions below. Library primitives used as steps: qsort (ordering),
 * exp and log from libm.
 *
 * Sources (pages; section names as they appear there):
 *  [CLSA]  SeventNews article on "CLSA: You Only Index Once", its opening
 *          section and section "Comment CLSA fonctionne".
 *  [IC]    gist.science summary of "IndexCache: Accelerating Sparse Attention
 *          via Cross-Layer Index Reuse", sections "1. Problématique" and
 *          "2. Méthodologie : IndexCache".
 *  [CA]    gist.science summary of "CompactAttention: Accelerating Chunked
 *          Prefill with Block-Union KV Selection", section "Méthodologie".
 *  [CoSA]  gist.science summary of "CoSA: Accelerating Long-Context Inference
 *          via Proxy-Kernel Co-Designed Sparse Attention" (no section titles;
 *          cited by the paragraphs on its proxy and its kernel).
 *
 * Readings of points the pages leave open (each is listed with its reason
 * in the design notes of the repository):
 *  - Indexer score: sum over indexer heads of w_h * ReLU(q_h . k_s), one
 *    indexer key per token. The pages name the lightning indexer but give
 *    no formula.
 *  - Causality: query t of a T-query call sees positions [0, kv_len - T + t].
 *  - Top-k order: score descending, then position ascending (lower position
 *    wins ties); chosen positions are returned ascending, padded with -1.
 *  - Ordered skipping: the priority list is the top-k in that order; reading
 *    stops at the first entry more than a fixed margin below the first one.
 *  - Attention uses one index per (b, t), shared by every head; softmax
 *    scale defaults to 1/sqrt(D); GQA groups are contiguous.
 *
 * Parity status of each function is stated in its comment; every function
 * here is pinned by the CPU tests (tests/test_oracle_*.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8_E4M3FN = 2 };

/* ------------------------------------------------------------------------ */
/* Element decoding                                                          */
/* ------------------------------------------------------------------------ */

/* IEEE-754 binary32: 1 sign bit, 8 exponent bits (bias 127), 23 fraction
 * bits. Decoded from its fields. */
static double orc_decode_f32_bits(uint32_t u) {
  int sign = (u >> 31) & 1;
  int e = (u >> 23) & 0xff;
  uint32_t f = u & 0x7fffff;
  double v;
  if (e == 0xff) {
    v = f ? NAN : INFINITY;
  } else if (e == 0) {
    v = ldexp((double)f, -126 - 23); /* subnormal */
  } else {
    v = ldexp((double)(f | 0x800000u), e - 127 - 23);
  }
  return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of a binary32 (1 sign, 8 exponent with bias
 * 127, 7 fraction bits). */
static double orc_decode_bf16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 7) & 0xff;
  uint32_t f = h & 0x7f;
  double v;
  if (e == 0xff) {
    v = f ? NAN : INFINITY;
  } else if (e == 0) {
    v = ldexp((double)f, -126 - 7);
  } else {
    v = ldexp((double)(f | 0x80u), e - 127 - 7);
  }
  return sign ? -v : v;
}

/* OCP 8-bit E4M3FN: 1 sign, 4 exponent bits (bias 7), 3 fraction bits; no
 * infinities; exponent and fraction all ones is NaN; largest finite 448. */
static double orc_decode_e4m3fn(uint8_t b) {
  int sign = (b >> 7) & 1;
  int e = (b >> 3) & 0xf;
  uint32_t f = b & 0x7;
  double v;
  if (e == 0xf && f == 0x7) {
    v = NAN;
  } else if (e == 0) {
    v = ldexp((double)f, 1 - 7 - 3); /* subnormal: f/8 * 2^(1-7) */
  } else {
    v = ldexp((double)(f | 0x8u), e - 7 - 3);
  }
  return sign ? -v : v;
}

/* Value tables of the two 16-/8-bit formats, filled once from the field
 * decoders above (the oracle is single-threaded; tables are filled on the
 * first call of each entry point). */
static double orc_bf16_table[65536];
static double orc_e4m3fn_table[256];
static int orc_tables_ready = 0;

static void orc_init_tables(void) {
  if (orc_tables_ready) return;
  for (uint32_t h = 0; h < 65536; h++) orc_bf16_table[h] = orc_decode_bf16((uint16_t)h);
  for (uint32_t b = 0; b < 256; b++) orc_e4m3fn_table[b] = orc_decode_e4m3fn((uint8_t)b);
  orc_tables_ready = 1;
}

/* Element i of a buffer of the given type. */
static double orc_elem(const void* base, size_t i, int dtype) {
  if (dtype == ORC_F32) {
    uint32_t u;
    memcpy(&u, (const unsigned char*)base + 4 * i, 4);
    return orc_decode_f32_bits(u);
  }
  if (dtype == ORC_BF16) {
    uint16_t h;
    memcpy(&h, (const unsigned char*)base + 2 * i, 2);
    return orc_bf16_table[h];
  }
  return orc_e4m3fn_table[((const uint8_t*)base)[i]];
}

/* Decode n elements into doubles (exported so tests can pin the decoders
 * against independent conversions). */
void orc_decode(const void* src, int dtype, long n, double* dst) {
  orc_init_tables();
  for (long i = 0; i < n; i++) dst[i] = orc_elem(src, (size_t)i, dtype);
}

/* Decode the n elements starting at element `first` (one row). */
static void orc_row(const void* base, size_t first, int n, int dtype, double* dst) {
  for (int i = 0; i < n; i++) dst[i] = orc_elem(base, first + (size_t)i, dtype);
}

/* Number of cache positions query t of a T-query call sees. */
static long orc_visible(int kv_len, int T, int t) {
  return (long)kv_len - T + t + 1;
}

/* ------------------------------------------------------------------------ */
/* Step 1: indexer score  [CLSA]; [IC] "1. Problématique"                    */
/* ------------------------------------------------------------------------ */

/*
 * scores[b,t,s] = sum_h w[b,t,h] * max(0, sum_d q[b,t,h,d] * k[b,s,d])
 * for s < visible(t); -inf for visible(t) <= s < kv_len.
 * q [B,T,H,D], k [B,L_cap,D] of `dtype`; w [B,T,H] float32;
 * scores [B,T,kv_len] double.
 * Also writes, when bound != NULL, the magnitude
 *   bound[b,t,s] = sum_h |w| * sum_d |q * k|
 * that scales the rounding error of any float32 evaluation of the score.
 */
int orc_index_score(const void* q, const void* k, int dtype, const float* w,
                    double* scores, double* bound, int B, int T, int H, int D,
                    int kv_len, int L_cap) {
  if (B < 1 || T < 1 || H < 1 || D < 1 || kv_len < T || L_cap < kv_len) return -1;
  orc_init_tables();
  double* qd = (double*)malloc(sizeof(double) * (size_t)H * D);
  double* kd = (double*)malloc(sizeof(double) * (size_t)D);
  if (!qd || !kd) {
    free(qd);
    free(kd);
    return -2;
  }
  for (int b = 0; b < B; b++) {
    for (int t = 0; t < T; t++) {
      long vis = orc_visible(kv_len, T, t);
      orc_row(q, ((size_t)b * T + t) * H * D, H * D, dtype, qd);
      const float* wr = w + ((size_t)b * T + t) * H;
      for (long s = 0; s < kv_len; s++) {
        size_t o = ((size_t)b * T + t) * kv_len + s;
        if (s >= vis) {
          scores[o] = -INFINITY;
          if (bound) bound[o] = 0.0;
          continue;
        }
        orc_row(k, ((size_t)b * L_cap + s) * D, D, dtype, kd);
        double total = 0.0, mag = 0.0;
        for (int h = 0; h < H; h++) {
          double dot = 0.0, adot = 0.0;
          for (int d = 0; d < D; d++) {
            dot += qd[h * D + d] * kd[d];
            adot += fabs(qd[h * D + d] * kd[d]);
          }
          double wh = (double)wr[h];
          total += wh * (dot > 0.0 ? dot : 0.0);
          mag += fabs(wh) * adot;
        }
        scores[o] = total;
        if (bound) bound[o] = mag;
      }
    }
  }
  free(qd);
  free(kd);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Step 2: top-k selection  [CLSA]; [IC] "1. Problématique"                 */
/* ------------------------------------------------------------------------ */

typedef struct {
  double score;
  long pos;
} orc_cand;

/* Order: higher score first; equal scores (with -0 == +0) lower position first. */
static int orc_cmp_rank(const void* a, const void* b) {
  const orc_cand* x = (const orc_cand*)a;
  const orc_cand* y = (const orc_cand*)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->pos > y->pos) - (x->pos < y->pos);
}

static int orc_cmp_long(const void* a, const void* b) {
  long x = *(const long*)a, y = *(const long*)b;
  return (x > y) - (x < y);
}

/*
 * For each (b,t): sort the visible positions by (score desc, position asc),
 * keep the first min(k_bt, visible), return them in ascending position
 * order, pad with -1 to k.  scores [B,T,kv_len] double, idx [B,T,k] int32.
 * k_bt = k, or with k_rows [B,T] (the per-query count of the query-dependent
 * k reading; [CLSA] "Le coût : limites de compatibilité") k_rows[b,t]
 * clamped to [0, k].
 *
 * Ordered skipping ([CoSA] summary, the paragraphs on the Kernel-Aware Proxy
 * and the Ordered-Skipping Kernel: the proxy hands over a priority list, the
 * kernel reads the most important entries first and skips the rest). With
 * margin != NULL the list above, in priority order, is read from its first
 * entry and reading stops at the first entry whose score is below
 * thr = s_first - *margin; only the entries read are kept. The pages give
 * no stopping rule; this fixed-margin rule is the reading taken here. thr
 * is formed in float (the scores are float values), and when it is NaN
 * (s_first = +inf with margin = +inf) nothing is skipped. kept [B,T] (may
 * be NULL) receives the number of positions kept per query.
 */
int orc_topk_margin(const double* scores, int B, int T, int kv_len, int k, const int32_t* k_rows,
                    const float* margin, int32_t* idx, int32_t* kept) {
  if (B < 1 || T < 1 || kv_len < T || k < 1) return -1;
  if (margin && !(*margin >= 0.0f)) return -1;
  orc_cand* c = (orc_cand*)malloc(sizeof(orc_cand) * (size_t)kv_len);
  long* chosen = (long*)malloc(sizeof(long) * (size_t)k);
  if (!c || !chosen) {
    free(c);
    free(chosen);
    return -2;
  }
  for (int b = 0; b < B; b++) {
    for (int t = 0; t < T; t++) {
      long vis = orc_visible(kv_len, T, t);
      const double* row = scores + ((size_t)b * T + t) * kv_len;
      for (long s = 0; s < vis; s++) {
        c[s].score = row[s];
        c[s].pos = s;
      }
      qsort(c, (size_t)vis, sizeof(orc_cand), orc_cmp_rank);
      long kb = k;
      if (k_rows) {
        kb = k_rows[(size_t)b * T + t];
        if (kb < 0) kb = 0;
        if (kb > k) kb = k;
      }
      long n = vis < kb ? vis : kb;
      if (margin && n > 0) {
        const float thr = (float)c[0].score - *margin;
        if (thr == thr) { /* not NaN */
          long r = 0;
          while (r < n && c[r].score >= (double)thr) r++;
          n = r;
        }
      }
      for (long j = 0; j < n; j++) chosen[j] = c[j].pos;
      qsort(chosen, (size_t)n, sizeof(long), orc_cmp_long);
      int32_t* out = idx + ((size_t)b * T + t) * k;
      for (long j = 0; j < k; j++) out[j] = j < n ? (int32_t)chosen[j] : -1;
      if (kept) kept[(size_t)b * T + t] = (int32_t)n;
    }
  }
  free(c);
  free(chosen);
  return 0;
}

int orc_topk(const double* scores, int B, int T, int kv_len, int k, const int32_t* k_rows,
             int32_t* idx) {
  return orc_topk_margin(scores, B, T, kv_len, k, k_rows, NULL, idx, NULL);
}

/* ------------------------------------------------------------------------ */
/* Step 4: gathered sparse attention  [IC] "1. Problématique"; [CA] GQA     */
/* ------------------------------------------------------------------------ */

/*
 * For each (b,t,h), g = h / (Hq/Hkv), over the entries j of idx[b,t,:] whose
 * position lies in [0, visible(t)):
 *   z_j = scale * sum_d q[b,t,h,d] * K[b,idx_j,g,d]
 *   m = max_j z_j, p_j = exp(z_j - m), l = sum_j p_j
 *   out[b,t,h,:] = sum_j p_j V[b,idx_j,g,:] / l,   lse = m + log(l)
 * With no valid entry: out = 0, lse = -inf.
 * q [B,T,Hq,D], K/V [B,L_cap,Hkv,D] of `dtype`; idx [B,T,k] int32;
 * out [B,T,Hq,D] double; lse [B,T,Hq] double. scale <= 0 means 1/sqrt(D).
 */
int orc_sparse_attn(const void* q, const void* kc, const void* vc, int dtype,
                    const int32_t* idx, int k, double* out, double* lse, int B,
                    int T, int Hq, int Hkv, int D, int kv_len, int L_cap,
                    double scale) {
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || D < 1 || k < 1 ||
      kv_len < T || L_cap < kv_len)
    return -1;
  orc_init_tables();
  if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
  int G = Hq / Hkv;
  double* z = (double*)malloc(sizeof(double) * (size_t)k);
  double* qd = (double*)malloc(sizeof(double) * (size_t)D);
  double* row = (double*)malloc(sizeof(double) * (size_t)D);
  if (!z || !qd || !row) {
    free(z);
    free(qd);
    free(row);
    return -2;
  }
  for (int b = 0; b < B; b++) {
    for (int t = 0; t < T; t++) {
      long vis = orc_visible(kv_len, T, t);
      const int32_t* sel = idx + ((size_t)b * T + t) * k;
      for (int h = 0; h < Hq; h++) {
        int g = h / G;
        orc_row(q, (((size_t)b * T + t) * Hq + h) * D, D, dtype, qd);
        double* o = out + (((size_t)b * T + t) * Hq + h) * D;
        for (int d = 0; d < D; d++) o[d] = 0.0;
        double m = -INFINITY;
        int nvalid = 0;
        for (int j = 0; j < k; j++) {
          long s = sel[j];
          if (s < 0 || s >= vis) continue;
          orc_row(kc, (((size_t)b * L_cap + s) * Hkv + g) * D, D, dtype, row);
          double dot = 0.0;
          for (int d = 0; d < D; d++) dot += qd[d] * row[d];
          z[j] = scale * dot;
          if (z[j] > m) m = z[j];
          nvalid++;
        }
        double* l_out = lse + ((size_t)b * T + t) * Hq + h;
        if (nvalid == 0) {
          *l_out = -INFINITY;
          continue;
        }
        double l = 0.0;
        for (int j = 0; j < k; j++) {
          long s = sel[j];
          if (s < 0 || s >= vis) continue;
          double p = exp(z[j] - m);
          l += p;
          orc_row(vc, (((size_t)b * L_cap + s) * Hkv + g) * D, D, dtype, row);
          for (int d = 0; d < D; d++) o[d] += p * row[d];
        }
        for (int d = 0; d < D; d++) o[d] /= l;
        *l_out = m + log(l);
      }
    }
  }
  free(z);
  free(qd);
  free(row);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Step 3: layer map  [CLSA]; [IC] "2. Méthodologie : IndexCache"           */
/* ------------------------------------------------------------------------ */

/*
 * One decode/chunk step over n_layers layers. layer_src[l] == l marks an F
 * layer: it scores its own indexer inputs and overwrites the single index
 * buffer idx_out [B,T,k]. Every layer l then attends with the buffer as the
 * nearest F layer at or before l left it.
 * Per-layer arrays hold host pointers to host buffers (F-layer indexer
 * inputs may be NULL for S layers). k_rows (may be NULL) gives each query
 * its own count, and skip_margin (may be NULL) the ordered-skipping margin,
 * as in orc_topk_margin. out[l] [B,T,Hq,D] double, lse[l]
 * [B,T,Hq] double. n_indexer_calls (may be NULL) receives how many times
 * the indexer ran. Returns -1 for an invalid layer map.
 */
int orc_decode_step(int n_layers, const int32_t* layer_src,
                    const void* const* q, const void* const* kc,
                    const void* const* vc, int dtype,
                    const void* const* q_idx, const void* const* k_idx,
                    const float* const* w, int idx_dtype, int32_t* idx_out,
                    double* const* out, double* const* lse, int B, int T,
                    int Hq, int Hkv, int D, int H_I, int D_I, int kv_len,
                    int L_cap, int k, const int32_t* k_rows, const float* skip_margin,
                    double scale, int* n_indexer_calls) {
  if (n_layers < 1 || layer_src[0] != 0) return -1;
  int last_f = -1;
  for (int l = 0; l < n_layers; l++) {
    if (layer_src[l] == l) last_f = l;
    if (layer_src[l] != last_f) return -1; /* must be the nearest F at or before l */
  }
  double* scores = (double*)malloc(sizeof(double) * (size_t)B * T * kv_len);
  if (!scores) return -2;
  int calls = 0;
  for (int l = 0; l < n_layers; l++) {
    if (layer_src[l] == l) {
      int rc = orc_index_score(q_idx[l], k_idx[l], idx_dtype, w[l], scores, NULL,
                               B, T, H_I, D_I, kv_len, L_cap);
      if (rc == 0) rc = orc_topk_margin(scores, B, T, kv_len, k, k_rows, skip_margin, idx_out, NULL);
      if (rc) {
        free(scores);
        return rc;
      }
      calls++;
    }
    int rc = orc_sparse_attn(q[l], kc[l], vc[l], dtype, idx_out, k, out[l], lse[l],
                             B, T, Hq, Hkv, D, kv_len, L_cap, scale);
    if (rc) {
      free(scores);
      return rc;
    }
  }
  free(scores);
  if (n_indexer_calls) *n_indexer_calls = calls;
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Step 5: block-union table and dense attention over it  [CA] "Méthodologie" */
/* ------------------------------------------------------------------------ */

/*
 * Per (b, g): ascending block ids floor(s / block) over every valid position
 * s in idx[b, :, :] (valid: inside its query's visible range). The index is
 * shared by all heads, so every group g of batch b gets the same table (the
 * union over the heads of a group changes nothing). kv_indptr [B*Hkv+1],
 * kv_indices capacity B*Hkv*ceil(kv_len/block).
 */
int orc_block_union(const int32_t* idx, int B, int T, int k, int kv_len, int block,
                    int Hkv, int32_t* kv_indptr, int32_t* kv_indices) {
  if (B < 1 || T < 1 || k < 1 || kv_len < T || block < 1 || Hkv < 1) return -1;
  long nblk = (kv_len + block - 1) / block;
  unsigned char* hit = (unsigned char*)malloc((size_t)nblk);
  if (!hit) return -2;
  int32_t pos = 0;
  kv_indptr[0] = 0;
  for (int b = 0; b < B; b++) {
    memset(hit, 0, (size_t)nblk);
    for (int t = 0; t < T; t++) {
      long vis = orc_visible(kv_len, T, t);
      for (int j = 0; j < k; j++) {
        long s = idx[((size_t)b * T + t) * k + j];
        if (s >= 0 && s < vis) hit[s / block] = 1;
      }
    }
    for (int g = 0; g < Hkv; g++) {
      for (long i = 0; i < nblk; i++)
        if (hit[i]) kv_indices[pos++] = (int32_t)i;
      kv_indptr[b * Hkv + g + 1] = pos;
    }
  }
  free(hit);
  return 0;
}

/*
 * Dense softmax attention of query (b,t,h) over every position s inside the
 * blocks of table (b, g) with s < visible(t) (causal within the chunk).
 * Same arithmetic and output convention as orc_sparse_attn. Caches are
 * token-major [B, L_cap, Hkv, D], or with head_major [B, Hkv, L_cap, D]
 * ([CA] "Méthodologie": head-major layout read in place).
 */
static size_t orc_kv_at(int head_major, int b, long s, int g, int d, int Hkv, int L_cap, int D) {
  return head_major ? (((size_t)b * Hkv + g) * L_cap + s) * D + d
                    : (((size_t)b * L_cap + s) * Hkv + g) * D + d;
}

int orc_block_attn(const void* q, const void* kc, const void* vc, int dtype,
                   const int32_t* kv_indptr, const int32_t* kv_indices, int block,
                   double* out, double* lse, int B, int T, int Hq, int Hkv, int D,
                   int kv_len, int L_cap, double scale, int head_major) {
  if (B < 1 || T < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || D < 1 || block < 1 ||
      kv_len < T || L_cap < kv_len)
    return -1;
  orc_init_tables();
  if (scale <= 0.0) scale = 1.0 / sqrt((double)D);
  int G = Hq / Hkv;
  double* z = (double*)malloc(sizeof(double) * (size_t)kv_len);
  long* sel = (long*)malloc(sizeof(long) * (size_t)kv_len);
  if (!z || !sel) {
    free(z);
    free(sel);
    return -2;
  }
  for (int b = 0; b < B; b++) {
    for (int t = 0; t < T; t++) {
      long vis = orc_visible(kv_len, T, t);
      for (int h = 0; h < Hq; h++) {
        int g = h / G;
        int tab = b * Hkv + g;
        long n = 0;
        for (int i = kv_indptr[tab]; i < kv_indptr[tab + 1]; i++)
          for (long s = (long)kv_indices[i] * block; s < (long)(kv_indices[i] + 1) * block; s++)
            if (s < vis) sel[n++] = s;
        double* o = out + (((size_t)b * T + t) * Hq + h) * D;
        for (int d = 0; d < D; d++) o[d] = 0.0;
        double* l_out = lse + ((size_t)b * T + t) * Hq + h;
        if (n == 0) {
          *l_out = -INFINITY;
          continue;
        }
        double m = -INFINITY;
        for (long j = 0; j < n; j++) {
          double dot = 0.0;
          for (int d = 0; d < D; d++)
            dot += orc_elem(q, (((size_t)b * T + t) * Hq + h) * D + d, dtype) *
                   orc_elem(kc, orc_kv_at(head_major, b, sel[j], g, d, Hkv, L_cap, D), dtype);
          z[j] = scale * dot;
          if (z[j] > m) m = z[j];
        }
        double l = 0.0;
        for (long j = 0; j < n; j++) {
          double p = exp(z[j] - m);
          l += p;
          for (int d = 0; d < D; d++)
            o[d] += p * orc_elem(vc, orc_kv_at(head_major, b, sel[j], g, d, Hkv, L_cap, D), dtype);
        }
        for (int d = 0; d < D; d++) o[d] /= l;
        *l_out = m + log(l);
      }
    }
  }
  free(z);
  free(sel);
  return 0;
}

/*
 * Cache append: row t of every batch element of src [B, T, row_bytes] is
 * copied byte for byte to row pos + t of dst [B, L_cap, row_bytes]; every
 * other row of dst is left as it is. One call per cache tensor (K, V,
 * indexer keys). Each new token of context adds its keys and values to the
 * stored cache ([CLSA] opening section), a cache written once and shared by
 * the cross-decoder layers ([CLSA] "Comment CLSA fonctionne").
 * Pinned by: appending T rows at once equals T single-row appends; rows
 * outside [pos, pos + T) unchanged; a decode step over a cache rebuilt by
 * appending its last rows equals the step over the original cache.
 */
int orc_cache_append(const unsigned char* src, unsigned char* dst, int B, int T,
                     long row_bytes, int pos, int L_cap) {
  if (B < 1 || T < 1 || row_bytes < 1 || pos < 0 || (long)pos + T > L_cap) return -1;
  for (int b = 0; b < B; b++)
    for (int t = 0; t < T; t++)
      for (long i = 0; i < row_bytes; i++)
        dst[((size_t)b * L_cap + pos + t) * (size_t)row_bytes + i] =
            src[((size_t)b * T + t) * (size_t)row_bytes + i];
  return 0;
}
