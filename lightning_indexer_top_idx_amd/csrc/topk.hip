// topk.hip - a2: top-k selection of the indexer scores, exact to the fp64 order.
//
// [ARCH] ai-muninn.com, "284B 塞得進 128GB、長 context 還跑得動:DeepSeek-V4-Flash 打的是
// KV cache,不是參數量", section "(B) 只讀你需要的": the indexer keeps the
// n_indexer_top_k = 512 highest-scoring compressed entries (1024 in the Pro
// variant), turns them into a bool mask (comp_allowed) and hands the selected row
// ids to the attention kernel. The pages build that mask on the host; here it
// never leaves the device. Ties go to the lower index.
//
// One workgroup (1024 threads) per sequence:
//   1. fp32 scores -> order-preserving u32 keys (in LDS when N <= 16384);
//   2. MSB-first radix select (4 passes of 8 bits) finds the k-th largest key T;
//   3. exact mode: every fp32 score is within Delta of its fp64 canonical value,
//      where Delta bounds the fp32 MFMA/FMA rounding through the key norms
//      (chunk maxima from lit_idx_score) and sum_h |w_h| |q_h|. Entries above
//      T + 2 Delta are in for sure, entries below T - 2 Delta out for sure; the
//      few in between are rescored in fp64 in canonical order and the best
//      k - (#sure) of them are taken by (score desc, index asc);
//   4. one ordered compaction pass writes ascending ids, the mask and the count.
#include <algorithm>
#include <math.h>

#include "exact.h"
#include "lit_common.h"
#include "select.h"

namespace lit {
lit_status check_idx_inputs(const lit_idx_in* in, int32_t B, int32_t N, const char* who);

namespace {

constexpr int TK_THREADS = 1024;
constexpr int LDS_KEYS = 16384;                                // keys held per LDS chunk
constexpr int LDS_KEY_WORDS = LDS_KEYS + (LDS_KEYS >> 5);      // one pad word per 32 keys
constexpr int BAND_LDS = 2048;                                  // band entries kept in LDS
// Safety factor on the rounding bound (2 already covers truncating adds).
constexpr double ERR_SAFETY = 4.0;

__device__ __forceinline__ int padi(int i) { return i + (i >> 5); }

struct TopkParams {
  const float* scores;
  int N, k;
  int exact;
  const void* q;
  const float* w;
  const void* kidx;
  int dtype, H;
  const float* kmax;
  int nchunks;
  int32_t* ids;
  int32_t* count;
  uint8_t* mask;
  double* ws_band_s;    // [B][N]
  int32_t* ws_band_n;   // [B][N]
  uint8_t* ws_band_sel; // [B][N]
};

struct TopkLds {
  SelectScratch sc;
  int imisc[8];
  double dmisc[4];
  float qT[LIT_IDX_DIM * 64];
  float krow[TK_THREADS / 64][LIT_IDX_DIM];
  double band_s[BAND_LDS];
  int32_t band_n[BAND_LDS];
  uint8_t band_sel[BAND_LDS];
  uint32_t keys[LDS_KEY_WORDS];
};

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float load_idx(const void* p, int dtype, size_t off) {
  return dtype == LIT_F32 ? ((const float*)p)[off] : bf16_to_f32(((const uint16_t*)p)[off]);
}

__global__ __launch_bounds__(TK_THREADS) void topk_kernel(TopkParams P) {
  extern __shared__ __align__(16) uint8_t smem[];
  TopkLds& L = *reinterpret_cast<TopkLds*>(smem);
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int N = P.N, k = P.k;
  const float* sb = P.scores + (size_t)b * N;
  const bool in_lds = N <= LDS_KEYS;
  int32_t* ids = P.ids + (size_t)b * k;
  uint8_t* mask = P.mask ? P.mask + (size_t)b * N : nullptr;
  double* g_band_s = P.ws_band_s + (size_t)b * N;
  int32_t* g_band_n = P.ws_band_n + (size_t)b * N;
  uint8_t* g_band_sel = P.ws_band_sel + (size_t)b * N;

  // 1. keys
  int nsel = 0;
  for (int i = tid; i < N; i += TK_THREADS) {
    const uint32_t kk = score_key(sb[i]);
    if (in_lds) L.keys[padi(i)] = kk;
    nsel += kk != 0u;
  }
  int total_sel;
  block_excl_scan(nsel, L.sc.scan, &total_sel);
  auto key = [&](int i) -> uint32_t { return in_lds ? L.keys[padi(i)] : score_key(sb[i]); };

  // Selection rule: key > def_key, or band_lo <= key <= band_hi and chosen.
  uint32_t def_key = 0u, band_lo = 1u, band_hi = 0u;  // empty band
  int r_eq = 0;
  bool exact_band = false;
  if (total_sel > k) {
    const uint32_t T = radix_select<uint32_t>(key, N, k, &L.sc, &r_eq);
    if (!P.exact) {
      def_key = T;
      band_lo = band_hi = T;
    } else {
      // 3. rounding bound
      if (wid == 0) {
        double wq = 0.0, wa = 0.0;
        if (lane < P.H) {
          const size_t qo = ((size_t)b * P.H + lane) * LIT_IDX_DIM;
          double n2 = 0.0;
          for (int d = 0; d < LIT_IDX_DIM; d++) {
            const double x = (double)load_idx(P.q, P.dtype, qo + d);
            n2 += x * x;
          }
          wa = fabs((double)P.w[(size_t)b * P.H + lane]);
          wq = wa * sqrt(n2);
        }
        wq = wave_sum_f64(wq);
        wa = wave_sum_f64(wa);
        if (lane == 0) {
          L.dmisc[0] = wq;
          L.dmisc[1] = wa;
        }
      }
      float km = 0.f;
      for (int j = tid; j < P.nchunks; j += TK_THREADS) km = fmaxf(km, P.kmax[(size_t)b * P.nchunks + j]);
      km = wave_max(km);
      if (lane == 0) L.krow[0][wid] = km;
      __syncthreads();
      if (tid == 0) {
        float m = 0.f;
        for (int i = 0; i < TK_THREADS / 64; i++) m = fmaxf(m, L.krow[0][i]);
        const double terms = (double)(LIT_IDX_DIM + P.H + 2);
        const double delta = (ERR_SAFETY * 0x1p-24 * terms * L.dmisc[0] * (double)m +
                              ERR_SAFETY * terms * 0x1p-126 * L.dmisc[1]) * (1.0 + 0x1p-20);
        const double t = (double)key_score(T);
        L.dmisc[2] = t - 2.0 * delta;
        L.dmisc[3] = t + 2.0 * delta;
      }
      __syncthreads();
      const uint32_t lo = score_key(__double2float_rd(L.dmisc[2]));
      band_lo = lo > 1u ? lo : 1u;
      band_hi = score_key(__double2float_ru(L.dmisc[3]));
      def_key = band_hi;
      exact_band = true;
    }
  }

  // Walk the entries chunk by chunk (one chunk when the keys live in LDS).
  const int CH = in_lds ? N : LDS_KEYS;
  auto stage = [&](int c0, int len) {
    if (!in_lds) {
      __syncthreads();
      for (int i = tid; i < len; i += TK_THREADS) L.keys[padi(i)] = score_key(sb[c0 + i]);
      __syncthreads();
    }
  };

  int M = 0;
  if (exact_band) {
    // gather the band in index order, count the sure ones
    int A = 0;
    for (int c0 = 0; c0 < N; c0 += CH) {
      const int len = min(CH, N - c0);
      stage(c0, len);
      const int seg = (len + TK_THREADS - 1) / TK_THREADS;
      const int a = min(len, tid * seg), e = min(len, a + seg);
      int nd = 0, nb = 0;
      for (int i = a; i < e; i++) {
        const uint32_t kk = L.keys[padi(i)];
        nd += kk > band_hi;
        nb += (kk >= band_lo) && (kk <= band_hi);
      }
      int tot;
      int pos = block_excl_scan((nd << 16) | nb, L.sc.scan, &tot);
      pos &= 0xffff;
      for (int i = a; i < e; i++) {
        const uint32_t kk = L.keys[padi(i)];
        if ((kk >= band_lo) && (kk <= band_hi)) g_band_n[M + pos++] = c0 + i;
      }
      A += tot >> 16;
      M += tot & 0xffff;
    }
    const int r = k - A;
    if (r < 1 || r > M) {
      // The rounding bound was violated: report instead of guessing.
      for (int j = tid; j < k; j += TK_THREADS) ids[j] = -1;
      if (mask)
        for (int i = tid; i < N; i += TK_THREADS) mask[i] = 0;
      if (tid == 0) P.count[b] = -1;
      return;
    }
    __syncthreads();
    const bool band_in_lds = M <= BAND_LDS;
    if (band_in_lds)
      for (int i = tid; i < M; i += TK_THREADS) L.band_n[i] = g_band_n[i];
    // rescore in fp64, canonical order
    for (int idx = tid; idx < LIT_IDX_DIM * 64; idx += TK_THREADS) {
      const int d = idx >> 6, h = idx & 63;
      L.qT[idx] = h < P.H ? load_idx(P.q, P.dtype, ((size_t)b * P.H + h) * LIT_IDX_DIM + d) : 0.f;
    }
    __syncthreads();
    const float w_h = lane < P.H ? P.w[(size_t)b * P.H + lane] : 0.f;
    for (int i = wid; i < M; i += TK_THREADS / 64) {
      const int n = band_in_lds ? L.band_n[i] : g_band_n[i];
      const size_t row = ((size_t)b * N + n) * LIT_IDX_DIM;
      for (int d = lane; d < LIT_IDX_DIM; d += 64) L.krow[wid][d] = load_idx(P.kidx, P.dtype, row + d);
      wave_sync();
      const double s = exact_score_wave(L.qT, L.krow[wid], w_h, P.H);
      if (lane == 0) {
        if (band_in_lds)
          L.band_s[i] = s;
        else
          g_band_s[i] = s;
      }
      wave_sync();
    }
    __syncthreads();
    // choose the best r of the band: (score desc, index asc); the band is in index order
    if (band_in_lds) {
      for (int i = tid; i < M; i += TK_THREADS) {
        const double si = L.band_s[i];
        int rank = 0;
        for (int j = 0; j < M; j++) {
          const double sj = L.band_s[j];
          rank += (sj > si) || (sj == si && j < i);
        }
        L.band_sel[i] = rank < r;
      }
    } else {
      auto bkey = [&](int i) -> uint64_t { return score_key64(g_band_s[i]); };
      int req;
      const uint64_t T64 = radix_select<uint64_t>(bkey, M, r, &L.sc, &req);
      mark_top<uint64_t>(bkey, M, T64, req, g_band_sel, &L.sc);
    }
    __syncthreads();
  }

  // 4. ordered compaction: ids ascending, mask, count
  const bool band_in_lds = M <= BAND_LDS;
  auto chosen = [&](int pos) -> bool {
    if (!exact_band) return pos < r_eq;
    return band_in_lds ? L.band_sel[pos] != 0 : g_band_sel[pos] != 0;
  };
  int out_base = 0, band_base = 0;
  for (int c0 = 0; c0 < N; c0 += CH) {
    const int len = min(CH, N - c0);
    stage(c0, len);
    const int seg = (len + TK_THREADS - 1) / TK_THREADS;
    const int a = min(len, tid * seg), e = min(len, a + seg);
    int nb = 0;
    for (int i = a; i < e; i++) {
      const uint32_t kk = L.keys[padi(i)];
      nb += (kk >= band_lo) && (kk <= band_hi);
    }
    int tb;
    int bpos = band_base + block_excl_scan(nb, L.sc.scan, &tb);
    int ns = 0;
    {
      int bp = bpos;
      for (int i = a; i < e; i++) {
        const uint32_t kk = L.keys[padi(i)];
        if (kk > def_key) {
          ns++;
        } else if ((kk >= band_lo) && (kk <= band_hi)) {
          ns += chosen(bp);
          bp++;
        }
      }
    }
    int ts;
    int opos = out_base + block_excl_scan(ns, L.sc.scan, &ts);
    for (int i = a; i < e; i++) {
      const uint32_t kk = L.keys[padi(i)];
      bool s = false;
      if (kk > def_key) {
        s = true;
      } else if ((kk >= band_lo) && (kk <= band_hi)) {
        s = chosen(bpos);
        bpos++;
      }
      if (s) ids[opos++] = c0 + i;
      if (mask) mask[c0 + i] = s;
    }
    out_base += ts;
    band_base += tb;
  }
  for (int j = out_base + tid; j < k; j += TK_THREADS) ids[j] = -1;
  if (tid == 0) P.count[b] = out_base;
}

}  // namespace
}  // namespace lit

using namespace lit;

extern "C" size_t lit_topk_workspace_bytes(int32_t B, int32_t N, int32_t k) {
  (void)k;
  if (B < 1 || N < 1) return 0;
  const size_t per = (size_t)B * (size_t)N;
  return round_up(per * sizeof(double), 256) + round_up(per * sizeof(int32_t), 256) + round_up(per, 256);
}

extern "C" lit_status lit_topk_select(const float* scores, int32_t B, int32_t N, int32_t k, const lit_idx_in* exact,
                                      const float* kmax, int32_t* ids, int32_t* count, uint8_t* mask, void* ws,
                                      size_t ws_bytes, void* stream) {
  clear_error();
  if (!scores || !ids || !count) return fail(LIT_ERR_NULL, "lit_topk_select: scores, ids and count must be non-NULL");
  if (B < 1 || N < 1 || k < 1) return fail(LIT_ERR_SHAPE, "lit_topk_select: B=%d N=%d k=%d must be >= 1", B, N, k);
  if (N > (1 << 24)) return fail(LIT_ERR_SHAPE, "lit_topk_select: N=%d above 2^24", N);
  if (!aligned(scores, 4) || !aligned(ids, 4) || !aligned(count, 4))
    return fail(LIT_ERR_ALIGN, "lit_topk_select: scores, ids and count must be 4-byte aligned");
  if (exact) {
    lit_status st = check_idx_inputs(exact, B, N, "lit_topk_select(exact)");
    if (st != LIT_OK) return st;
    if (!kmax) return fail(LIT_ERR_NULL, "lit_topk_select: exact mode needs the kmax side output of lit_idx_score");
  }
  const size_t need = lit_topk_workspace_bytes(B, N, k);
  if (!ws || ws_bytes < need)
    return fail(LIT_ERR_WORKSPACE, "lit_topk_select: workspace of %zu bytes given, %zu needed", ws_bytes, need);
  if (!aligned(ws, 256)) return fail(LIT_ERR_ALIGN, "lit_topk_select: workspace must be 256-byte aligned");
  const size_t per = (size_t)B * (size_t)N;
  uint8_t* w8 = (uint8_t*)ws;
  TopkParams P;
  P.scores = scores;
  P.N = N;
  P.k = k;
  P.exact = exact != nullptr;
  P.q = exact ? exact->q : nullptr;
  P.w = exact ? exact->w : nullptr;
  P.kidx = exact ? exact->k : nullptr;
  P.dtype = exact ? (int)exact->dtype : 0;
  P.H = exact ? exact->H : 0;
  P.kmax = kmax;
  P.nchunks = (int)cdiv(N, LIT_KNORM_CHUNK);
  P.ids = ids;
  P.count = count;
  P.mask = mask;
  P.ws_band_s = (double*)w8;
  P.ws_band_n = (int32_t*)(w8 + round_up(per * sizeof(double), 256));
  P.ws_band_sel = w8 + round_up(per * sizeof(double), 256) + round_up(per * sizeof(int32_t), 256);
  const size_t lds = sizeof(TopkLds);
  lit_status st = allow_lds((const void*)topk_kernel, lds, "lit_topk_select");
  if (st != LIT_OK) return st;
  topk_kernel<<<dim3((unsigned)B), dim3(TK_THREADS), lds, (hipStream_t)stream>>>(P);
  LIT_CHECK_LAUNCH("lit_topk_select");
  return LIT_OK;
}
