/*
 * oracle.c - plain, slow CPU oracle of the lightning-indexer decode step.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link or call this
 * file; only the tests, the smoke check and the benchmark's CPU-baseline leg do.
 * It shares no source with the HIP library.
 *
 * Every function works on ONE sequence, in fp64, with plain loops in index
 * order and the C library's qsort/exp/log as the only library steps. Build it
 * without FP contraction (-ffp-contract=off): each product that is not exact in
 * fp64 is rounded before it is added, which is part of the definitions below.
 *
 * Pages followed (title, part of the page):
 *   [ARCH] ai-muninn.com, "284B 塞得進 128GB、長 context 還跑得動:DeepSeek-V4-Flash
 *          打的是 KV cache,不是參數量" (Part 6): "(A) 壓縮你存的" (512-wide
 *          attn_comp_kv rows, layer table), "(B) 只讀你需要的" (128-dim index keys,
 *          top-512 / 1024, the comp_allowed mask and row ids, the SWA window of 128),
 *          "為什麼你沒辦法靠量化 KV 再省記憶體" (E4M3 in groups of 64 with a
 *          power-of-two scale for the non-RoPE dims, BF16 RoPE dims).
 *   [FMEN] ai-muninn.com, "FlashMemory can't improve DeepSeek-V4-Flash's own
 *          lightning indexer - I retrained it on my exact Q2 and it still lost"
 *          (Part 7): "The setup" (the gate restricts the native candidate set),
 *          "Act 1" / "Act 3" (overlap of two 512-sets; golden = unmasked dense softmax).
 *   [LSA]  zhichai.net, "FlashMemory-DeepSeek-V4 深度解读：用预言家替代记忆海绵":
 *          2.2 (sigmoid gate, keep at 0.5), 3.2 (softmax -> top-p 0.6 -> >=3 of 21
 *          layers vote), 4.1 (gate layers OR-ed), second reply (gated score equation).
 *
 * Parity status of each function is stated in its comment; the pins live in
 * tests/test_oracle_*.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1
#define OR_FP8 2

#define IDX_DIM 128
#define KV_DIM 512
#define FP8_DIMS 448
#define FP8_GROUP 64
#define SCALE_STRIDE 8

/* ---- element decoding ---------------------------------------------------- */

/* BF16 is the top half of an IEEE binary32; widening is exact. */
static double bf16_to_f64(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double elem(const void* base, int dtype, int64_t i) {
  if (dtype == OR_F32) return (double)((const float*)base)[i];
  return bf16_to_f64(((const uint16_t*)base)[i]);
}

/* OCP 8-bit floating point, E4M3FN variant ([ARCH] KV precision names E4M3):
 * 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 is
 * subnormal (m/8 * 2^-6); S.1111.111 is NaN; there is no infinity, so the
 * largest finite value is 1.75 * 2^8 = 448. Written from that definition. */
double or_fp8_e4m3(uint8_t byte) {
  int sign = (byte >> 7) & 1;
  int e = (byte >> 3) & 15;
  int m = byte & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

/* E8M0 scale byte: the power of two 2^(byte-127); 255 encodes NaN. */
double or_e8m0(uint8_t byte) {
  if (byte == 255) return NAN;
  return ldexp(1.0, (int)byte - 127);
}

/* One element of a compressed latent row ([ARCH] (A): 512 wide; KV precision:
 * dims 0..447 E4M3 times the group's power-of-two scale, dims 448..511 BF16). */
static double kv_elem(int dtype, const void* data, const void* rope, const uint8_t* scale,
                      int64_t n, int d) {
  if (dtype == OR_F32 || dtype == OR_BF16) return elem(data, dtype, n * KV_DIM + d);
  if (d < FP8_DIMS) {
    uint8_t code = ((const uint8_t*)data)[n * FP8_DIMS + d];
    uint8_t sc = scale[n * SCALE_STRIDE + d / FP8_GROUP];
    return or_fp8_e4m3(code) * or_e8m0(sc);
  }
  return bf16_to_f64(((const uint16_t*)rope)[n * (KV_DIM - FP8_DIMS) + (d - FP8_DIMS)]);
}

/* Dequantise a whole row set once: out[N][512] fp64. */
void or_kv_dequant(int dtype, const void* data, const void* rope, const uint8_t* scale,
                   int N, double* out) {
  for (int64_t n = 0; n < N; n++)
    for (int d = 0; d < KV_DIM; d++) out[n * KV_DIM + d] = kv_elem(dtype, data, rope, scale, n, d);
}

/* ---- a1: indexer score ------------------------------------------------------
 * [ARCH] (B): each compressed entry n is scored with its own 128-dim index key;
 * the score form is the "native ReLU-MQA" of the [LSA] reply equation without
 * its sigmoid:  s_n = sum_h w_h * max(0, q_h . k_n).
 * fp64, d ascending inside a head, then h ascending. q and k are BF16 or FP32,
 * so q*k is exact in fp64; w (fp32) * relu(acc) is rounded, then added.
 * Entries with allowed[n] == 0 score -inf (the gated candidate set, [FMEN]
 * "The setup"). allowed may be NULL. */
void or_idx_score(const void* q, const float* w, const void* k, int dtype, int H, int N,
                  const uint8_t* allowed, double* out) {
  for (int64_t n = 0; n < N; n++) {
    if (allowed && !allowed[n]) {
      out[n] = -INFINITY;
      continue;
    }
    double s = 0.0;
    for (int h = 0; h < H; h++) {
      double acc = 0.0;
      for (int d = 0; d < IDX_DIM; d++)
        acc += elem(q, dtype, (int64_t)h * IDX_DIM + d) * elem(k, dtype, n * IDX_DIM + d);
      double r = acc > 0.0 ? acc : 0.0;
      double prod = (double)w[h] * r;
      s += prod;
    }
    out[n] = s;
  }
}

/* ---- a2: top-k selection ----------------------------------------------------
 * [ARCH] (B): keep the k highest-scoring entries (n_indexer_top_k) and hand
 * them on as a bool mask and a list of row ids. Ties: the lower index wins.
 * -inf and NaN scores are never selected. Returns count = min(k, #selectable);
 * ids[0..count) ascending, ids[count..k) = -1; mask may be NULL. */
typedef struct {
  double s;
  int32_t n;
} scored;

static int by_score_desc_index_asc(const void* a, const void* b) {
  const scored* x = (const scored*)a;
  const scored* y = (const scored*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->n > y->n) - (x->n < y->n);
}

int or_topk(const double* s, int N, int k, int32_t* ids, uint8_t* mask) {
  scored* v = (scored*)malloc(sizeof(scored) * (size_t)(N > 0 ? N : 1));
  int m = 0;
  for (int n = 0; n < N; n++)
    if (!isnan(s[n]) && s[n] != -INFINITY) {
      v[m].s = s[n];
      v[m].n = n;
      m++;
    }
  qsort(v, (size_t)m, sizeof(scored), by_score_desc_index_asc);
  int count = m < k ? m : k;
  uint8_t* sel = (uint8_t*)calloc((size_t)(N > 0 ? N : 1), 1);
  for (int i = 0; i < count; i++) sel[v[i].n] = 1;
  int j = 0;
  for (int n = 0; n < N; n++)
    if (sel[n]) ids[j++] = n;
  for (; j < k; j++) ids[j] = -1;
  if (mask) memcpy(mask, sel, (size_t)N);
  free(sel);
  free(v);
  return count;
}

/* ---- a3/a4/a5: sparse MQA attention -----------------------------------------
 * [ARCH] (B): attention reads only the selected compressed rows plus the SWA
 * window of the most recent entries; HCA layers read every row ([ARCH] (A)).
 * [ARCH] (A): a row is the 512-wide attn_comp_kv latent, used as key and value
 * by every query head (MQA). R = ids[0..count) U {N-window..N-1}, each row once
 * (ids == NULL means every row). Per head, fp64:
 *   x_r = scale * (q_h . kv_r);  m = max_r x_r;  e_r = exp(x_r - m);
 *   Z = sum_r e_r;  out_h = (sum_r e_r * kv_r) / Z;  lse_h = m + log(Z).
 * Rows are visited in ascending index. Empty R: out = 0, lse = -inf. */
void or_attend(const void* q, int q_dtype, int Hq, int kv_dtype, const void* data,
               const void* rope, const uint8_t* scale_bytes, int N, const int32_t* ids,
               int count, int window, double scale, double* out, double* lse) {
  uint8_t* in_r = (uint8_t*)calloc((size_t)(N > 0 ? N : 1), 1);
  if (ids == NULL) {
    for (int n = 0; n < N; n++) in_r[n] = 1;
  } else {
    for (int i = 0; i < count; i++) in_r[ids[i]] = 1;
    int w = window < N ? window : N;
    for (int n = N - w; n < N; n++) in_r[n] = 1;
  }
  int R = 0;
  for (int n = 0; n < N; n++) R += in_r[n];
  int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * (size_t)(R > 0 ? R : 1));
  for (int n = 0, j = 0; n < N; n++)
    if (in_r[n]) rows[j++] = n;
  double* kvr = (double*)malloc(sizeof(double) * (size_t)(R > 0 ? R : 1) * KV_DIM);
  for (int j = 0; j < R; j++)
    for (int d = 0; d < KV_DIM; d++)
      kvr[(int64_t)j * KV_DIM + d] = kv_elem(kv_dtype, data, rope, scale_bytes, rows[j], d);
  double* x = (double*)malloc(sizeof(double) * (size_t)(R > 0 ? R : 1));
  for (int h = 0; h < Hq; h++) {
    double* o = out + (int64_t)h * KV_DIM;
    for (int d = 0; d < KV_DIM; d++) o[d] = 0.0;
    if (R == 0) {
      if (lse) lse[h] = -INFINITY;
      continue;
    }
    double m = -INFINITY;
    for (int j = 0; j < R; j++) {
      double dot = 0.0;
      for (int d = 0; d < KV_DIM; d++)
        dot += elem(q, q_dtype, (int64_t)h * KV_DIM + d) * kvr[(int64_t)j * KV_DIM + d];
      x[j] = scale * dot;
      if (x[j] > m) m = x[j];
    }
    double Z = 0.0;
    for (int j = 0; j < R; j++) {
      double e = exp(x[j] - m);
      Z += e;
      for (int d = 0; d < KV_DIM; d++) o[d] += e * kvr[(int64_t)j * KV_DIM + d];
    }
    for (int d = 0; d < KV_DIM; d++) o[d] /= Z;
    if (lse) lse[h] = m + log(Z);
  }
  free(x);
  free(kvr);
  free(rows);
  free(in_r);
}

/* ---- a6: dense golden top-k ---------------------------------------------------
 * [FMEN] "Act 3": the golden set is what the model attends to under an
 * unmasked softmax over all chunks; its top-k is compared with a selector's.
 * Head-averaged probabilities: P_h = softmax_n(scale * q_h . kv_n) over all N,
 * pbar_n = (sum_h P_h,n) / Hq, G = top-k of pbar (ties: lower index).
 * fp64; n ascending for the softmax sums, h ascending for the head sum.
 * pbar may be NULL. Returns |G|. */
int or_golden(const void* q, int q_dtype, int Hq, int kv_dtype, const void* data,
              const void* rope, const uint8_t* scale_bytes, int N, double scale, int k,
              double* pbar, int32_t* ids, uint8_t* mask) {
  double* kvd = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1) * KV_DIM);
  or_kv_dequant(kv_dtype, data, rope, scale_bytes, N, kvd);
  double* acc = (double*)calloc((size_t)(N > 0 ? N : 1), sizeof(double));
  double* x = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
  for (int h = 0; h < Hq; h++) {
    double m = -INFINITY;
    for (int64_t n = 0; n < N; n++) {
      double dot = 0.0;
      for (int d = 0; d < KV_DIM; d++)
        dot += elem(q, q_dtype, (int64_t)h * KV_DIM + d) * kvd[n * KV_DIM + d];
      x[n] = scale * dot;
      if (x[n] > m) m = x[n];
    }
    double Z = 0.0;
    for (int n = 0; n < N; n++) Z += exp(x[n] - m);
    for (int n = 0; n < N; n++) acc[n] += exp(x[n] - m) / Z;
  }
  double* pb = pbar ? pbar : (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
  for (int n = 0; n < N; n++) pb[n] = acc[n] / (double)Hq;
  int c = or_topk(pb, N, k, ids, mask);
  if (!pbar) free(pb);
  free(x);
  free(acc);
  free(kvd);
  return c;
}

/* ---- a7: recall ----------------------------------------------------------------
 * [FMEN] "Act 1" / "Act 3": overlap of two selections of the same entries. */
void or_recall(const uint8_t* a, const uint8_t* m, int N, int32_t* inter, int32_t* ca,
               int32_t* cb) {
  int32_t i = 0, x = 0, y = 0;
  for (int n = 0; n < N; n++) {
    x += a[n] != 0;
    y += m[n] != 0;
    i += (a[n] != 0) && (m[n] != 0);
  }
  *inter = i;
  *ca = x;
  *cb = y;
}

/* ---- a8: LSA sigmoid gate, one layer --------------------------------------------
 * [LSA] 2.2: a memory indexer scores every compressed chunk with a sigmoid and
 * keeps the chunk when the sigmoid reaches the threshold (0.5); 3.1 / [FMEN]
 * "Act 2": the query comes from three small projections of the hidden state
 * (wq_a, wq_b, weights_proj) and the keys are the frozen index keys; the second
 * reply's equation gives the score form sigma(sum_h w_h * ReLU(q_h . k)).
 *   u = wq_a . h (rank),  q = wq_b . u (as [H][128]),  w = w_proj . h (H)
 *   z_n = sum_h w_h * max(0, q_h . k_n)
 *   keep_n = sigmoid(z_n) >= threshold, i.e. z_n >= thr_logit where
 *   thr_logit = log(threshold / (1 - threshold)) (0 for 0.5).
 * fp64, each sum in ascending index order; a product that is not exact in
 * fp64 (bf16 times fp64) is rounded before it is added. z_out may be NULL. */
void or_gate_layer(const float* hvec, const uint16_t* wq_a, const uint16_t* wq_b,
                   const uint16_t* w_proj, const uint16_t* k, int H, int d_model, int rank,
                   int N, double thr_logit, double* z_out, uint8_t* keep) {
  double* u = (double*)malloc(sizeof(double) * (size_t)rank);
  double* qv = (double*)malloc(sizeof(double) * (size_t)H * IDX_DIM);
  double* wv = (double*)malloc(sizeof(double) * (size_t)H);
  for (int r = 0; r < rank; r++) {
    double a = 0.0;
    for (int i = 0; i < d_model; i++) {
      double p = bf16_to_f64(wq_a[(int64_t)r * d_model + i]) * (double)hvec[i];
      a += p;
    }
    u[r] = a;
  }
  for (int j = 0; j < H * IDX_DIM; j++) {
    double a = 0.0;
    for (int r = 0; r < rank; r++) {
      double p = bf16_to_f64(wq_b[(int64_t)j * rank + r]) * u[r];
      a += p;
    }
    qv[j] = a;
  }
  for (int h = 0; h < H; h++) {
    double a = 0.0;
    for (int i = 0; i < d_model; i++) {
      double p = bf16_to_f64(w_proj[(int64_t)h * d_model + i]) * (double)hvec[i];
      a += p;
    }
    wv[h] = a;
  }
  for (int64_t n = 0; n < N; n++) {
    double z = 0.0;
    for (int h = 0; h < H; h++) {
      double acc = 0.0;
      for (int d = 0; d < IDX_DIM; d++) {
        double p = qv[h * IDX_DIM + d] * bf16_to_f64(k[n * IDX_DIM + d]);
        acc += p;
      }
      double r = acc > 0.0 ? acc : 0.0;
      double p = wv[h] * r;
      z += p;
    }
    if (z_out) z_out[n] = z;
    keep[n] = z >= thr_logit;
  }
  free(wv);
  free(qv);
  free(u);
}

/* ---- a9: top-p per layer and the cross-layer vote --------------------------------
 * [LSA] 3.2: step 1 turns a layer's indexer logits into probabilities with a
 * softmax; step 2 keeps the smallest set of entries whose cumulative
 * probability reaches p = 0.6; step 3 marks an entry when at least 3 of the
 * 21 CSA layers kept it. x is [L][N] for one sequence; is_logits selects
 * whether the softmax is applied. Order: p descending, index ascending; the
 * running sum is added in that order and the entry that reaches top_p is kept.
 * If rounding keeps the total below top_p, every entry is kept.
 * Returns |gold|; votes may be NULL. */
int or_topp_vote(const double* x, int is_logits, int L, int N, double top_p, int min_votes,
                 uint8_t* gold, int32_t* votes) {
  int32_t* v = (int32_t*)calloc((size_t)(N > 0 ? N : 1), sizeof(int32_t));
  double* p = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
  scored* o = (scored*)malloc(sizeof(scored) * (size_t)(N > 0 ? N : 1));
  for (int l = 0; l < L; l++) {
    const double* xl = x + (int64_t)l * N;
    if (is_logits) {
      double m = -INFINITY;
      for (int n = 0; n < N; n++)
        if (xl[n] > m) m = xl[n];
      double Z = 0.0;
      for (int n = 0; n < N; n++) Z += exp(xl[n] - m);
      for (int n = 0; n < N; n++) p[n] = exp(xl[n] - m) / Z;
    } else {
      for (int n = 0; n < N; n++) p[n] = xl[n];
    }
    for (int n = 0; n < N; n++) {
      o[n].s = p[n];
      o[n].n = n;
    }
    qsort(o, (size_t)N, sizeof(scored), by_score_desc_index_asc);
    double run = 0.0;
    for (int i = 0; i < N; i++) {
      v[o[i].n] += 1;
      run += o[i].s;
      if (run >= top_p) break;
    }
  }
  int g = 0;
  for (int n = 0; n < N; n++) {
    gold[n] = v[n] >= min_votes;
    g += gold[n];
    if (votes) votes[n] = v[n];
  }
  free(o);
  free(p);
  free(v);
  return g;
}

/* ---- the timed path for one query (score -> select -> attend) ------------------
 * Used by the benchmark's CPU baseline: the same three steps as above, chained,
 * for one sequence of one layer. Returns the selection count. */
int or_decode_query(const void* q_idx, const float* w, const void* k_idx, int idx_dtype, int H,
                    int N, int k, const void* q, int q_dtype, int Hq, int kv_dtype,
                    const void* data, const void* rope, const uint8_t* scale_bytes, int window,
                    double scale, int32_t* ids, double* out, double* lse) {
  double* s = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
  or_idx_score(q_idx, w, k_idx, idx_dtype, H, N, NULL, s);
  int c = or_topk(s, N, k, ids, NULL);
  or_attend(q, q_dtype, Hq, kv_dtype, data, rope, scale_bytes, N, ids, c, window, scale, out,
            lse);
  free(s);
  return c;
}
