/*
 * lit.h - C ABI of the lightning-indexer decode step for MI355X (gfx950).
 *
 * One decode step of a Compressed Sparse Attention (CSA) layer, as the pages
 * below describe it, split into the calls a caller strings together:
 *
 *   lit_idx_score        score every compressed entry with the 128-dim index keys
 *   lit_topk_select      keep the k best entries (lower index wins ties)
 *   lit_sparse_attn_decode  MQA attention over the kept rows plus the SWA window
 *   lit_sparse_attn_decode_noalloc  the same without a workspace argument
 *   lit_golden_topk      dense "golden" attention and its top-k (measurement)
 *   lit_golden_topp_vote top-p 0.6 per layer, then a cross-layer vote (labels)
 *   lit_lookahead_golden the golden sets of the next T steps and their union
 *   lit_recall           set overlap of two selections
 *   lit_lsa_gate         sigmoid chunk gate of FlashMemory/LSA (candidate set)
 *   lit_pool_plan / lit_pool_gather / lit_pool_remap_ids
 *                        the LSA cold-pool fetch: gated entries into a compact pool
 *   lit_idx_score_mq / lit_topk_select_mq
 *                        the indexer for several queries per sequence (MTP, prefill)
 *
 * Pages cited (title, then the part of the page):
 *   [ARCH]  ai-muninn.com, "284B 塞得進 128GB、長 context 還跑得動:DeepSeek-V4-Flash
 *           打的是 KV cache,不是參數量" (series Part 6, the V4-Flash architecture post).
 *           Sections "(A) 壓縮你存的" (storage, layer table), "(B) 只讀你需要的"
 *           (lightning indexer), "為什麼你沒辦法靠量化 KV 再省記憶體" (KV precision).
 *   [FMEN]  ai-muninn.com, "FlashMemory can't improve DeepSeek-V4-Flash's own lightning
 *           indexer - I retrained it on my exact Q2 and it still lost" (series Part 7,
 *           English). Sections "The setup", "Act 1", "Act 3".
 *   [LSA]   zhichai.net, "FlashMemory-DeepSeek-V4 深度解读：用预言家替代记忆海绵".
 *           Sections 2.2 (the gate), 3.2 (labels), 4.1 (gate layers), and the
 *           gated-score equation quoted in the second reply.
 *
 * Conventions shared by every call
 *   - Every pointer is a DEVICE pointer unless its comment says "host".
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null stream).
 *   - Arguments are validated on the host before anything is enqueued. On a
 *     validation failure the call returns a non-zero lit_status, enqueues
 *     nothing, and lit_last_error() describes the failure. The library never
 *     exits or aborts the process.
 *   - A failed kernel launch returns LIT_ERR_LAUNCH. Faults inside a kernel
 *     surface at the caller's next synchronisation of `stream`.
 *   - The caller owns every buffer. The library allocates no device memory;
 *     scratch space comes from a caller-provided workspace whose size is given
 *     by the matching *_workspace_bytes() query. Workspace contents need no
 *     initialisation and are not meaningful after a call. The one exception is
 *     lit_sparse_attn_decode_noalloc, whose scratch is a fixed device array the
 *     library holds on each GPU (see that call).
 *   - Results are deterministic: the same inputs give bit-identical outputs.
 *   - Calls that overlap on one stream are ordered; calls on different streams
 *     that share an output or a workspace race.
 *   - Indices are int32 (N < 2^31). Dense arrays are C-contiguous, in the
 *     shapes given, with no padding between rows.
 */
#ifndef LIT_H
#define LIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LIT_ABI_VERSION 2

/* Width of an index key ([ARCH] (B): each compressed entry has its own 128-dim key). */
#define LIT_IDX_DIM 128
/* Width of a compressed latent row ([ARCH] (A): attn_comp_kv rows are 512 wide). */
#define LIT_KV_DIM 512
/* FP8 rows ([ARCH] KV precision): the first 448 dims are E4M3 in groups of 64,
 * the last 64 (RoPE) dims are BF16. */
#define LIT_KV_FP8_DIMS 448
#define LIT_KV_ROPE_DIMS 64
#define LIT_KV_FP8_GROUP 64
#define LIT_KV_SCALE_STRIDE 8 /* bytes per row of E8M0 scales: 7 used, 1 pad */
/* Entries per chunk of the key-norm part of lit_idx_score's hints. */
#define LIT_KNORM_CHUNK 256
/* Entries per group of the score-maximum part of lit_idx_score's hints. */
#define LIT_HINT_GROUP 16
/* Floats at the end of each sequence's hints holding the query-side bound sums. */
#define LIT_HINT_QBOUND 4
/* Limits. */
#define LIT_MAX_IDX_HEADS 64
#define LIT_MAX_Q_HEADS 64
#define LIT_MAX_WINDOW 8192
#define LIT_MAX_QUERIES 65536 /* queries per sequence of the multi-query calls */
#define LIT_MAX_HORIZON 1024  /* decode steps of a lookahead golden */

typedef enum {
  LIT_OK = 0,
  LIT_ERR_NULL = 1,      /* a required pointer is NULL */
  LIT_ERR_SHAPE = 2,     /* a size is out of range or sizes disagree */
  LIT_ERR_ALIGN = 3,     /* a pointer is not aligned as required */
  LIT_ERR_DTYPE = 4,     /* unsupported dtype or dtype combination */
  LIT_ERR_WORKSPACE = 5, /* workspace missing or smaller than required */
  LIT_ERR_LAUNCH = 6,    /* the HIP runtime refused a launch or query */
  LIT_ERR_MEMORY = 7     /* host memory the device must read is not page-locked */
} lit_status;

typedef enum {
  LIT_F32 = 0,
  LIT_BF16 = 1,
  /* [ARCH] KV precision: dims 0..447 are OCP E4M3FN bytes, one E8M0 power-of-two
   * scale byte per 64-dim group (value 2^(byte-127)); dims 448..511 are BF16. */
  LIT_FP8E4M3_G64_ROPE_BF16 = 2,
  /* Not a dtype: spans the enum over every int32 value, so that a value a C
   * caller passes outside the list above reaches the library as an ordinary
   * value (refused with LIT_ERR_DTYPE) rather than one C++ may assume away. */
  LIT_DTYPE_INT32_RANGE_ = 0x7fffffff
} lit_dtype;

/* Inputs of the lightning indexer ([ARCH] (B); score form from [LSA] reply
 * equation without the sigmoid, "native ReLU-MQA"). Host struct, read during
 * the call only.
 *   q : [B][H][128] index queries, dtype `dtype` (LIT_F32 or LIT_BF16), 16-B aligned
 *   w : [B][H] fp32 head weights
 *   k : [B][N][128] index keys (index_comp_kv), same dtype as q, 16-B aligned */
typedef struct {
  const void* q;
  const float* w;
  const void* k;
  lit_dtype dtype;
  int32_t H; /* 1..64 */
} lit_idx_in;

/* Compressed latent KV (attn_comp_kv, [ARCH] (A)); used as both K and V by the
 * MQA attention. Host struct, read during the call only.
 *   LIT_F32 / LIT_BF16: data = [B][N][512], 16-B aligned; rope, scale unused.
 *   LIT_FP8E4M3_G64_ROPE_BF16: data = [B][N][448] E4M3 bytes (16-B aligned),
 *     rope = [B][N][64] BF16 (16-B aligned), scale = [B][N][8] E8M0 bytes (byte 7
 *     unused; 4-B aligned).
 * Strides: row n of sequence b of an array X starts X_seq_stride * b +
 * X_row_stride * n bytes past X, so that a cache whose sequences hold more rows
 * than N, or whose rows sit inside wider records, is read in place. A row
 * stride of 0 takes the dense layout's: 2048 B (F32), 1024 B (BF16) or 448 B
 * (FP8 data), 128 B (rope), 8 B (scale); a sequence stride of 0 is N times the
 * array's row stride. Strides
 * are non-negative multiples of 16 B (data, rope) and of 4 B (scale): anything
 * else is refused with LIT_ERR_ALIGN, a negative one with LIT_ERR_SHAPE. */
typedef struct {
  lit_dtype dtype;
  int32_t n_rows; /* N */
  const void* data;
  const void* rope;
  const uint8_t* scale;
  int64_t seq_stride, row_stride;             /* of data, bytes (0 = dense) */
  int64_t rope_seq_stride, rope_row_stride;   /* of rope, bytes (0 = dense) */
  int64_t scale_seq_stride, scale_row_stride; /* of scale, bytes (0 = dense) */
} lit_kv;

/* Inputs of one FlashMemory/LSA gate layer ([LSA] 2.2, 4.1; projections named in
 * [FMEN] "Act 2": wq_a, wq_b, weights_proj). Host struct.
 *   h      : [B][d_model] fp32 hidden state at this layer
 *   wq_a   : [rank][d_model] BF16   (u = wq_a . h)
 *   wq_b   : [H*128][rank]  BF16    (q = wq_b . u, read as [H][128])
 *   w_proj : [H][d_model]   BF16    (w = w_proj . h, signed head weights)
 *   k      : [B][N][128]    BF16    frozen index keys of this layer, 16-B aligned */
typedef struct {
  const float* h;
  const void* wq_a;
  const void* wq_b;
  const void* w_proj;
  const void* k;
} lit_gate_layer;

int lit_abi_version(void);
/* Thread-local text describing the last failure on the calling thread (host string). */
const char* lit_last_error(void);

/* ---- a1: indexer scores ------------------------------------------------------
 * [ARCH] (B): a light indexer scores every compressed entry with its own 128-dim
 * key. For each sequence b and entry n:
 *     scores[b][n] = sum_h w[b][h] * max(0, sum_d q[b][h][d] * k[b][n][d])
 * computed with fp32 accumulation (bf16 products are exact in fp32).
 * allowed : [B][N] u8 or NULL. Where allowed[b][n] == 0 the score is -inf
 *           (the candidate set restricted by the gate, [FMEN] "The setup").
 * scores  : [B][N] fp32 output.
 * hints   : [B][lit_idx_hints_len(N)] fp32 output or NULL; the side output
 *           lit_topk_select reads. hints[b][c] for c < ceil(N/LIT_KNORM_CHUNK)
 *           is an upper bound of the largest Euclidean key norm among entries
 *           c*LIT_KNORM_CHUNK ... +LIT_KNORM_CHUNK-1; hints[b][ceil(N/LIT_KNORM_CHUNK) + j]
 *           is the largest of the scores written for entries LIT_HINT_GROUP*j ...
 *           +LIT_HINT_GROUP-1 (-inf when none is allowed); the last
 *           LIT_HINT_QBOUND floats hold two fp64 values as little-endian word
 *           pairs: sum_h |w[b][h]| * ||q[b][h]|| and sum_h |w[b][h]| (each
 *           within a relative 2^-40 of the exact sum), which scale the
 *           rounding bound of the exact selection. */
int32_t lit_idx_hints_len(int32_t N);
lit_status lit_idx_score(const lit_idx_in* in, const uint8_t* allowed, int32_t B, int32_t N,
                         float* scores, float* hints, void* stream);

/* ---- a2: top-k selection -----------------------------------------------------
 * [ARCH] (B): keep the n_indexer_top_k (512; 1024 for the Pro variant) best
 * entries and turn them into a comp_allowed mask and a list of row ids.
 * Order: score descending, then index ascending (the lower index wins a tie).
 * Entries whose score is -inf or NaN are never selected. count[b] =
 * min(k, number of selectable entries).
 * exact == NULL : the order is that of the fp32 `scores` as given.
 * exact != NULL : the order is that of the exact scores, i.e. the definition of
 *   lit_idx_score evaluated in fp64 in canonical order (d ascending within a head,
 *   then h ascending, each w*relu product rounded before it is added). `exact`
 *   must be the same inputs that produced `scores`, and `hints` its side output;
 *   entries whose fp32 score lies within a proven error bound of the k-th score
 *   are rescored in fp64 so the selection equals the fp64 one bit for bit.
 * hints : the side output of lit_idx_score for these scores, or NULL (then
 *   every score is scanned, which is slower; exact mode requires hints).
 *   With hints the call reads only the groups of entries that can reach the
 *   top k (a lower bound on the k-th score comes from the group maxima).
 * ids   : [B][k] int32 output, selected indices ascending, tail filled with -1.
 * count : [B] int32 output (-1 would signal that the proven rounding bound was
 *         violated; the call then selects nothing rather than guess).
 * mask  : [B][N] u8 output (1 = selected) or NULL.
 * Workspace: lit_topk_workspace_bytes(B, N, k) bytes. */
size_t lit_topk_workspace_bytes(int32_t B, int32_t N, int32_t k);
lit_status lit_topk_select(const float* scores, int32_t B, int32_t N, int32_t k,
                           const lit_idx_in* exact, const float* hints,
                           int32_t* ids, int32_t* count, uint8_t* mask,
                           void* ws, size_t ws_bytes, void* stream);

/* ---- a3/a4/a5: sparse MQA attention decode ------------------------------------
 * [ARCH] (B): attention reads only the selected compressed rows plus the
 * sliding window of the last `window` entries; [ARCH] (A): rows are the 512-wide
 * attn_comp_kv, shared by all query heads as key and value (MQA); HCA layers
 * read every row (ids == NULL). For each sequence b and head h:
 *     R      = { ids[b][0..count[b]) } U { N-window .. N-1 }   (each row once)
 *     x_r    = scale * (q[b][h] . kv[b][r])
 *     out[b][h] = sum_{r in R} softmax(x)_r * kv[b][r]
 *     lse[b][h] = log(sum_{r in R} exp(x_r))            (natural log)
 * q      : [B][Hq][512], dtype q_dtype (LIT_F32 with LIT_F32 kv, else LIT_BF16)
 * kv     : rows, see lit_kv. FP8 rows are dequantised exactly (E4M3 value times
 *          2^(scale-127)) before use ([ARCH] KV precision).
 * ids    : [B][k_cap] ascending ids (tail -1) with count[b] valid, or NULL for
 *          every row (then count and window are ignored). count[b] is taken
 *          up to min(k_cap, N); a negative count[b] (lit_topk_select's sign of a
 *          failed exact selection) makes out[b] and lse[b] NaN, so that the
 *          failure cannot pass for an answer.
 * window : 0..LIT_MAX_WINDOW, clamped to N.
 * out    : [B][Hq][512] fp32 output (16-byte aligned); lse: [B][Hq] fp32 output or NULL.
 * q, kv->data and kv->rope must be 16-byte aligned, kv->scale 4-byte. Errors: LIT_ERR_NULL,
 * LIT_ERR_SHAPE (B, Hq outside 1..64, window), LIT_ERR_DTYPE (unsupported row
 * or query dtype), LIT_ERR_ALIGN, LIT_ERR_WORKSPACE.
 * An empty R (count 0 and window 0) gives out = 0 and lse = -inf.
 * Workspace: lit_attn_workspace_bytes(B, Hq, N) bytes, 16-byte aligned; it
 * covers every k_cap and window on these shapes. A workspace given off a 16-byte
 * boundary is refused (LIT_ERR_ALIGN) whether or not the call would use it. */
size_t lit_attn_workspace_bytes(int32_t B, int32_t Hq, int32_t N);
lit_status lit_sparse_attn_decode(const void* q, lit_dtype q_dtype, int32_t Hq, const lit_kv* kv,
                                  int32_t B, const int32_t* ids, const int32_t* count,
                                  int32_t k_cap, int32_t window, float scale,
                                  float* out, float* lse, void* ws, size_t ws_bytes,
                                  void* stream);

/* ---- allocation-free attention ------------------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same call
 * as lit_sparse_attn_decode (same arguments, same results bit for bit) without
 * the workspace: the partial results of its row slices go to a scratch array the
 * library holds on each GPU it runs on, LIT_ATTN_SCRATCH_BYTES bytes, kept until
 * the process ends. The call itself allocates nothing. A call whose plan needs
 * more partial results than the array holds returns LIT_ERR_WORKSPACE and
 * enqueues nothing (lit_attn_workspace_bytes(B, Hq, N) bounds the need; plans of
 * at most 64 sequence-slices of 64 heads always fit). Every call on one GPU
 * shares that GPU's array, which keeps the last call's contents (nothing in it
 * needs to start at zero): calls on one stream are ordered, calls that overlap
 * on one GPU (other streams, other threads) race. LIT_ERR_LAUNCH when no device
 * is current or the array cannot be found on it. */
#define LIT_ATTN_SCRATCH_BYTES (16u << 20)
lit_status lit_sparse_attn_decode_noalloc(const void* q, lit_dtype q_dtype, int32_t Hq, const lit_kv* kv,
                                          int32_t B, const int32_t* ids, const int32_t* count, int32_t k_cap,
                                          int32_t window, float scale, float* out, float* lse, void* stream);

/* ---- a6: dense golden top-k ---------------------------------------------------
 * [FMEN] "Act 3": golden = what the model attends to under an unmasked softmax
 * over all chunks. In fp64, for each sequence b:
 *     P[h][n] = softmax_n(scale * (q[b][h] . kv[b][n]))     over all N rows
 *     pbar[n] = (sum_h P[h][n]) / Hq                          (head average)
 *     G       = top-k of pbar, pbar descending then index ascending.
 * ids   : [B][k] ascending (tail -1); count: [B]; mask: [B][N] u8 or NULL;
 * pbar  : [B][N] fp64 output or NULL.
 * q and the rows 16-byte aligned (FP8 row bytes 8-byte), else LIT_ERR_ALIGN. The
 * logits are fp64 sums on the matrix cores, whose order is not sequential: pbar
 * matches a sequential fp64 evaluation to a relative ~1e-15, and G can differ
 * from it only where pbar ties the k-th value within that margin.
 * Workspace: lit_golden_workspace_bytes(B, Hq, N, k) bytes. */
size_t lit_golden_workspace_bytes(int32_t B, int32_t Hq, int32_t N, int32_t k);
lit_status lit_golden_topk(const void* q, lit_dtype q_dtype, int32_t Hq, const lit_kv* kv,
                           int32_t B, float scale, int32_t k,
                           int32_t* ids, int32_t* count, uint8_t* mask, double* pbar,
                           void* ws, size_t ws_bytes, void* stream);

/* ---- NEXT: the lookahead golden -------------------------------------------------
 * [FMEN] "The one caveat I didn't test: lookahead" and [LSA] 2.2: the gate is
 * meant to predict what the next tau = 64 decode steps will attend to, not what
 * the current step does, and the golden for that target needs the dense
 * attention of every step of the horizon. For sequence b and each step t of the
 * horizon (query q[b][t], the same N rows), G[b][t] is the a6 golden set:
 *     P[h][n] = softmax_n(scale * (q[b][t][h] . kv[b][n])),  pbar[n] = (sum_h P[h][n]) / Hq,
 *     G[b][t] = top-k of pbar (descending, then index ascending)       (fp64)
 * and the lookahead golden is what the horizon needs:
 *     hits[b][n] = #{t : n in G[b][t]},  union_mask[b][n] = hits[b][n] > 0,
 *     union_count[b] = #{n : hits[b][n] > 0}.
 * The logits are fp64 sums of exact products (matrix cores; the order of the
 * fp64 additions is not sequential, so pbar matches a sequential fp64 sum to a
 * relative 1e-12, not bit for bit).
 * q         : [B][T][Hq][512] (the T queries of the horizon), dtype as for a6.
 * step_ids  : [B][T][k] int32 output (each step's golden ids ascending, tail -1) or NULL.
 * hits      : [B][N] int32 output or NULL;  union_mask : [B][N] u8 output or NULL;
 * union_count : [B] int32 output;  pbar : [B][T][N] fp64 output or NULL.
 * Workspace: lit_lookahead_workspace_bytes(B, T, Hq, N, k) bytes (it holds the
 * fp64 logits, B*T*Hq*N*8 bytes: 4.3 GB at B = 8, T = Hq = 64, N = 16384). */
size_t lit_lookahead_workspace_bytes(int32_t B, int32_t T, int32_t Hq, int32_t N, int32_t k);
lit_status lit_lookahead_golden(const void* q, lit_dtype q_dtype, int32_t T, int32_t Hq,
                                const lit_kv* kv, int32_t B, float scale, int32_t k,
                                int32_t* step_ids, int32_t* hits, uint8_t* union_mask,
                                int32_t* union_count, double* pbar, void* ws, size_t ws_bytes,
                                void* stream);

/* ---- a9: top-p per layer, then a cross-layer vote -----------------------------
 * [LSA] 3.2: per layer, turn the scores into probabilities with a softmax, keep
 * the smallest set whose cumulative probability reaches top_p (0.6), then mark
 * an entry golden when at least min_votes (3) of the L layers kept it.
 * For every layer l and sequence b (fp64):
 *     p    = x[l][b]            if is_logits == 0 (x already holds probabilities)
 *          = softmax_n(x[l][b]) if is_logits != 0
 *     order entries by p descending, index ascending; T = the shortest prefix
 *     whose running sum (added in that order) is >= top_p.
 *     votes[b][n] = number of layers whose T holds n;  gold = votes >= min_votes.
 * x     : [L][B][N] fp64
 * gold  : [B][N] u8 output; gold_count: [B] int32 output;
 * votes : [B][N] int32 output or NULL.
 * Workspace: lit_topp_workspace_bytes(L, B, N) bytes. */
size_t lit_topp_workspace_bytes(int32_t L, int32_t B, int32_t N);
lit_status lit_golden_topp_vote(const double* x, int32_t is_logits, int32_t L, int32_t B,
                                int32_t N, double top_p, int32_t min_votes,
                                uint8_t* gold, int32_t* gold_count, int32_t* votes,
                                void* ws, size_t ws_bytes, void* stream);

/* ---- exact indexer scores (label pipeline helper) ------------------------------
 * The lit_idx_score definition evaluated in fp64 in canonical order for every
 * entry (the order lit_topk_select's exact mode matches). Slow; for labels.
 * scores64 : [B][N] fp64 output (-inf where allowed[b][n] == 0). */
lit_status lit_idx_score_exact(const lit_idx_in* in, const uint8_t* allowed, int32_t B,
                               int32_t N, double* scores64, void* stream);

/* ---- a7: recall -----------------------------------------------------------------
 * [FMEN] "Act 1", "Act 3": overlap of two selections over the same entries.
 * inter[b] = #{n : a[b][n] != 0 and m[b][n] != 0}; count_a, count_b the set
 * sizes (any of the three outputs may be NULL). Recall = inter / |golden|. */
lit_status lit_recall(const uint8_t* a, const uint8_t* m, int32_t B, int32_t N,
                      int32_t* inter, int32_t* count_a, int32_t* count_b, void* stream);

/* ---- a8: FlashMemory / LSA sigmoid chunk gate ------------------------------------
 * [LSA] 2.2: every tau = 64 decode steps a memory indexer scores each compressed
 * chunk with a sigmoid and keeps those at or above the threshold; [LSA] 4.1: the
 * indexers sit at layers 10, 12 and 20 and their kept sets are OR-ed; the
 * score form is the second reply's gated equation. For each layer l, sequence b:
 *     u = wq_a . h ;  q = wq_b . u  (as [H][128]) ;  w = w_proj . h     (fp64)
 *     z[n] = sum_h w[h] * max(0, q[h] . k[b][n])
 *     keep[n] = sigmoid(z[n]) >= threshold  <=>  z[n] >= log(threshold/(1-threshold))
 * gate[b][n] = OR over layers of keep; gate_count[b] = number kept.
 * The decision is exact: the fp64 value of z in canonical order (h, then d
 * ascending; each product rounded before it is added) decides it.
 * layers : host array of n_layers (1..8) structs; threshold in (0,1);
 *          d_model and rank multiples of 64, at most 4096; the projection
 *          matrices and keys 16-byte aligned.
 * Workspace: lit_gate_workspace_bytes(n_layers, B, H, rank, N) bytes. */
size_t lit_gate_workspace_bytes(int32_t n_layers, int32_t B, int32_t H, int32_t rank, int32_t N);
lit_status lit_lsa_gate(const lit_gate_layer* layers, int32_t n_layers, int32_t B, int32_t N,
                        int32_t H, int32_t d_model, int32_t rank, double threshold,
                        uint8_t* gate, int32_t* gate_count, void* ws, size_t ws_bytes,
                        void* stream);

/* ---- NEXT: the LSA cold-pool fetch -------------------------------------------------
 * [LSA] 2.2: every tau = 64 decode steps the gate's kept blocks are moved from a
 * CPU "cold pool" to the GPU and the steps in between attend only inside the
 * moved set, so that GPU memory follows the gate, not the context length; the
 * later section of the same page notes that the swap engine was not published.
 * The three calls below form one: plan the compact pool from the gate, gather
 * each per-entry array (index keys, latent rows, their FP8 parts) into it, run
 * lit_idx_score / lit_topk_select / lit_sparse_attn_decode on the compact pool
 * (N = C, allowed = allowed_c, the same window), then map the selected ids back.
 * The compact pool keeps the original order of the entries, so the selection and
 * the attention output equal those of the same calls on the resident arrays
 * with allowed = gate.
 *
 * lit_pool_plan: for sequence b the kept entries are
 *     K_b = {n : gate[b][n] != 0}  union  {N - W' .. N - 1},  W' = min(window, N)
 * in ascending order, right-aligned in C slots so that the window stays in the
 * last W' slots:  map[b][C - |K_b| + i] = the i-th entry of K_b,  map[b][j] = -1
 * before that;  allowed_c[b][j] = 1 where map[b][j] is a gated entry (window
 * entries outside the gate get 0; allowed_c may be NULL);  count[b] = |K_b|.
 * When |K_b| > C the pool is too small: map[b] is all -1, allowed_c[b] all 0, and
 * count[b] = |K_b| tells the caller by how much.
 * gate : [B][N] u8;  map : [B][C] int32 output;  count : [B] int32 output;
 * allowed_c : [B][C] u8 output or NULL. */
lit_status lit_pool_plan(const uint8_t* gate, int32_t B, int32_t N, int32_t window, int32_t C,
                         int32_t* map, int32_t* count, uint8_t* allowed_c, void* stream);

/* lit_pool_gather: dst[b][j][:] = src[b][map[b][j]][:] (row_bytes bytes), and zeros
 * where map[b][j] is -1 or not below src_rows.
 * src : [B][src_rows][row_bytes] bytes, either device memory or page-locked
 *       (pinned) HOST memory, which the kernel reads in place over the host link;
 *       pageable host memory returns LIT_ERR_MEMORY.
 * map : [B][C] int32 (from lit_pool_plan);  dst : [B][C][row_bytes] device output.
 * row_bytes is a multiple of 4 (1 MiB at most); src, dst and map 4-byte aligned. */
lit_status lit_pool_gather(const void* src, int32_t src_rows, int64_t row_bytes, int32_t B,
                           const int32_t* map, int32_t C, void* dst, void* stream);

/* lit_pool_remap_ids: ids[b][j] = map[b][ids_c[b][j]] for j < count[b], -1 after
 * (ids_c and count as lit_topk_select wrote them on the compact pool). Ascending
 * compact ids give ascending original ids.
 * ids_c, ids : [B][k] int32;  count : [B] int32;  map : [B][C] int32. */
lit_status lit_pool_remap_ids(const int32_t* ids_c, const int32_t* count, int32_t B, int32_t k,
                              const int32_t* map, int32_t C, int32_t* ids, void* stream);

/* ---- NEXT: the multi-query indexer ----------------------------------------------
 * Several queries of one sequence scored against that sequence's compressed
 * entries in one call: the draft token of depth-1 MTP speculative decoding
 * ([ARCH], the series list at its end: Part 5) is verified together with the
 * current token (Q = 2), and a prefill chunk ([ARCH] (A), the resident prefill
 * cache) scores each of its tokens (Q = the chunk length). The keys are read
 * once per group of queries, so the scoring turns from a key stream into a
 * matrix product on the matrix cores.
 *
 * lit_idx_score_mq: for sequence b, query j (row r = b*Q + j) and entry n:
 *     scores[r][n] = sum_h w[r][h] * max(0, sum_d q[r][h][d] * k[b][n][d])
 * for n < lengths[r] (and allowed[b][n] != 0); -inf otherwise. A query sees
 * the entries that existed when its token was decoded: lengths[r] (NULL: all N
 * for every query); values above N act as N, values below 1 hide every entry.
 * in      : q [B][Q][H][128], w [B][Q][H], k [B][N][128] (the lit_idx_in layout
 *           with Q queries per sequence), LIT_BF16 or LIT_F32.
 * lengths : [B][Q] int32 or NULL;  allowed : [B][N] u8 or NULL (shared by the
 *           Q queries of a sequence).
 * scores  : [B][Q][N] fp32 output;  hints : [B][Q][lit_idx_hints_len(N)] fp32
 *           output or NULL, row r as lit_idx_score writes for one sequence.
 * Q == 1 with lengths == NULL gives lit_idx_score's results bit for bit. */
lit_status lit_idx_score_mq(const lit_idx_in* in, int32_t Q, const int32_t* lengths,
                            const uint8_t* allowed, int32_t B, int32_t N, float* scores,
                            float* hints, void* stream);

/* lit_topk_select_mq: lit_topk_select on the B*Q rows of lit_idx_score_mq's
 * scores (each row its own top k, ids [B*Q][k], count [B*Q], mask [B*Q][N]);
 * in exact mode row r is rescored with query r and the keys of sequence r / Q.
 * Workspace: lit_topk_workspace_bytes(B*Q, N, k) bytes. */
lit_status lit_topk_select_mq(const float* scores, int32_t B, int32_t Q, int32_t N, int32_t k,
                              const lit_idx_in* exact, const float* hints, int32_t* ids,
                              int32_t* count, uint8_t* mask, void* ws, size_t ws_bytes,
                              void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LIT_H */
