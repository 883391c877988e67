// topk.hip - a2: top-k selection of the indexer scores, exact to the fp64 order.
//
// [ARCH] ai-muninn.com, "284B 塞得進 128GB、長 context 還跑得動:DeepSeek-V4-Flash 打的是
// KV cache,不是參數量", section "(B) 只讀你需要的": the indexer keeps the
// n_indexer_top_k = 512 highest-scoring compressed entries (1024 in the Pro
// variant), turns them into a bool mask (comp_allowed) and hands the selected row
// ids to the attention kernel. The pages build that mask on the host; here it
// never leaves the device. Ties go to the lower index.
//
// Up to 16384 entries per row, one workgroup (1024 threads) per row keeps every
// score in registers (the small path below). Longer rows with the hints of
// lit_idx_score (N <= 131072) take two kernels (the wide path below):
//   1. the k-th largest of the per-16-entry score maxima is a lower bound L of
//      the k-th largest score (it is the k-th largest of a subset of the scores);
//   2. only groups whose maximum reaches L - 2 Delta can hold top-k entries (or
//      band members): many workgroups per row list their slices' entries above
//      that bound, in index order (~k groups are read, not N), and rescore in
//      fp64 those near L;
//   3. one workgroup per row takes the k-th score T over those candidates;
//   4. exact mode: every fp32 score is within Delta of its fp64 canonical value
//      (Delta bounds the fp32 MFMA/FMA rounding through the key-norm hints and
//      sum_h |w_h| |q_h|). Entries above T + 2 Delta are in for sure, entries below
//      T - 2 Delta out; those in between are ranked by their fp64 canonical
//      scores, and the best taken by (score desc, index asc);
//   5. the selection is compacted into ascending ids (and the mask).
// Anything that does not fit (no hints, larger N, too many candidates after ties)
// falls back to scanning every score with the same steps.
#include <algorithm>
#include <math.h>

#include "exact.h"
#include "lit_common.h"
#include "select.h"

namespace lit {
lit_status check_idx_inputs(const lit_idx_in* in, int32_t B, int32_t N, const char* who);

namespace {

constexpr int TK_THREADS = 1024;
constexpr int NWAVES = TK_THREADS / 64;
// full-scan path
constexpr int LDS_KEYS = 16384;                            // keys held per LDS chunk
constexpr int LDS_KEY_WORDS = LDS_KEYS + (LDS_KEYS >> 5);  // one pad word per 32 keys
constexpr int BAND_LDS = 2048;                             // band entries kept in LDS
// fast path
constexpr int GROUP = LIT_HINT_GROUP;
constexpr int GM_CAP = 8192;                   // group maxima in LDS: N <= 131072
constexpr int CAND_CAP = 2048;                 // candidates >= L in LDS
constexpr int FBAND_CAP = 1024;                // exact band in LDS

// Bound delta on |fp32 score - fp64 canonical score| for an entry whose key
// norm is at most kmax. On the way to a score, every fp32 operation of
// lit_idx_score is an add or multiply rounded at least faithfully (relative
// error below 2^-23, truncation included): per head 128 adds of the dot product
// (bf16 products are exact in fp32; fp32 products add one rounding each, 128
// more), one multiply by w_h, then H - 1 adds over the heads. Each rounded
// quantity is bounded by |w_h| ||q_h|| ||k|| (Cauchy-Schwarz), so the error is
// below 2^-23 * nr * sum_h |w_h| ||q_h|| * kmax with nr >= the roundings on
// any path. Flushed subnormals lose less than 2^-126 each: 128 per head scaled
// by |w_h|, at most 2H - 1 unscaled. The factor 1 + 2^-10 covers the
// second-order terms and the rounding of the fp64 canonical value itself.
__device__ __forceinline__ double score_err_bound(bool bf16_in, int H, double Q, double kmax, double Wa) {
  const double nr = (double)((bf16_in ? 1 : 2) * LIT_IDX_DIM + H + 2);
  return (0x1p-23 * nr * Q * kmax + 0x1p-126 * (nr * Wa + 2.0 * H + 2.0)) * (1.0 + 0x1p-10);
}

__device__ __forceinline__ int padi(int i) { return i + (i >> 5); }

struct TopkParams {
  const float* scores;
  int N, k;
  int exact;
  const void* q;
  const float* w;
  const void* kidx;
  int kq;  // rows per key batch: row b reads the keys of sequence b / kq
  int dtype, H;
  const float* hints;
  int hints_len, nchunks;
  int32_t* ids;
  int32_t* count;
  uint8_t* mask;
  double* ws_band_s;     // [B][N] (wide path: exact scores of the rescored candidates)
  int32_t* ws_band_n;    // [B][N] (wide path: candidate indices)
  uint32_t* ws_ckey;     // [B][N] wide path: candidate keys
  uint8_t* ws_band_sel;  // [B][N]
  int32_t* ws_wide;      // [B][WIDE_STRIDE] wide path: header and slice counts per row
  int rows;              // B (rows of scores)
  int wide_slices;       // slices per row of the wide path
};

struct FullLds {
  SelectScratch sc;
  int imisc[8];
  double dmisc[4];
  float qT[LIT_IDX_DIM * 64];
  float krow[NWAVES][LIT_IDX_DIM];
  double band_s[BAND_LDS];
  int32_t band_n[BAND_LDS];
  uint8_t band_sel[BAND_LDS];
  uint32_t keys[LDS_KEY_WORDS];
};

constexpr int QP_STRIDE = LIT_IDX_DIM + 4;  // fp32 q row stride in LDS (spreads banks)

constexpr int BW = 4;        // band entries per wave and round of the broadcast rescoring
constexpr int PSUM_LD = 66;  // fp64 row stride of the head terms (rows on distinct banks)

struct FastLds {  // the wide path's kernel B
  SelectScratch sc;
  union {
    float qP[64 * QP_STRIDE];  // the fallback's band rescoring
    double cexact[CAND_CAP];   // exact scores kernel A took, by candidate position
  };
  double psum[NWAVES][BW][PSUM_LD];  // head terms of the rescoring waves
  double band_s[FBAND_CAP];
  int32_t band_n[FBAND_CAP];
  uint8_t cflag[CAND_CAP];
  union {  // never live at the same time
    uint32_t hist2k[2048];
    uint16_t binpos[CAND_CAP];
  };
  uint32_t sel[CAND_CAP / 32];  // bit i: candidate i selected
  uint32_t ckey[CAND_CAP];
  int32_t cidx[CAND_CAP];
};

static_assert(sizeof(FastLds) <= 160 * 1024 && sizeof(FullLds) <= 160 * 1024, "LDS budget of a gfx950 CU");

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float load_idx(const void* p, int dtype, size_t off) {
  return dtype == LIT_F32 ? ((const float*)p)[off] : bf16_to_f32(((const uint16_t*)p)[off]);
}

// Exact-mode band edges around the k-th fp32 score `tkey`: keys outside
// [*lo, *hi] are provably on the same side of the fp64 k-th score as their fp32
// value says. Block-wide; uses krow[0][0..NWAVES) and dmisc as scratch.
__device__ void exact_band(const TopkParams& P, int b, uint32_t tkey, float (*krow)[LIT_IDX_DIM], double* dmisc,
                           uint32_t* lo, uint32_t* hi) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (wid == 0) {
    double wq = 0.0, wa = 0.0;
    if (lane < P.H) {
      const size_t qo = ((size_t)b * P.H + lane) * LIT_IDX_DIM;
      double n2 = 0.0;
#pragma unroll 8
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
      dmisc[0] = wq;
      dmisc[1] = wa;
    }
  }
  float km = 0.f;
  for (int j = tid; j < P.nchunks; j += TK_THREADS) km = fmaxf(km, P.hints[(size_t)b * P.hints_len + j]);
  km = wave_max(km);
  if (lane == 0) krow[0][wid] = km;
  __syncthreads();
  if (tid == 0) {
    float m = 0.f;
    for (int i = 0; i < NWAVES; i++) m = fmaxf(m, krow[0][i]);
    const double delta = score_err_bound(P.dtype == LIT_BF16, P.H, dmisc[0], (double)m, dmisc[1]);
    const double t = (double)key_score(tkey);
    dmisc[2] = t - 2.0 * delta;
    dmisc[3] = t + 2.0 * delta;
  }
  __syncthreads();
  const uint32_t l = score_key(__double2float_rd(dmisc[2]));
  *lo = l > 1u ? l : 1u;
  *hi = score_key(__double2float_ru(dmisc[3]));
  __syncthreads();
}

// Stages q transposed (qT[d*64 + h], zero for h >= H) for the fp64 rescoring.
__device__ void stage_qT(const TopkParams& P, int b, float* qT) {
  for (int idx = threadIdx.x; idx < LIT_IDX_DIM * 64; idx += TK_THREADS) {
    const int d = idx >> 6, h = idx & 63;
    qT[idx] = h < P.H ? load_idx(P.q, P.dtype, ((size_t)b * P.H + h) * LIT_IDX_DIM + d) : 0.f;
  }
  __syncthreads();
}

// fp64 canonical score of entry n, one wave.
__device__ __forceinline__ double rescore(const TopkParams& P, int b, int n, const float* qT, float* krow,
                                          float w_h) {
  const int lane = threadIdx.x & 63;
  const size_t row = ((size_t)(b / P.kq) * P.N + n) * LIT_IDX_DIM;
  for (int d = lane; d < LIT_IDX_DIM; d += 64) krow[d] = load_idx(P.kidx, P.dtype, row + d);
  wave_sync();
  const double s = exact_score_wave(qT, krow, w_h, P.H);
  wave_sync();
  return s;
}

__device__ void report_violation(const TopkParams& P, int b, int32_t* ids, uint8_t* mask) {
  for (int j = threadIdx.x; j < P.k; j += TK_THREADS) ids[j] = -1;
  if (mask)
    for (int i = threadIdx.x; i < P.N; i += TK_THREADS) mask[i] = 0;
  if (threadIdx.x == 0) P.count[b] = -1;
}

// acc[j] += KA[j] of lane N of this lane's 16-lane row (DPP row_newbcast) * QA,
// then acc[j] += KB[j] (same lane) * QB, for the wave's BW entries: v_fmac_f64
// rounds once, and the product of two values upcast from fp32/bf16 is exact,
// so each step is the oracle's add. s_nop 1 first: two wait states between a
// VALU write of a K register and its DPP read. Volatile: the blocks keep their
// place between the surrounding memory operations and exec-mask updates.
#define LIT_FMAC_LINE(I, KI, QI, N) \
  "v_fmac_f64_dpp %" #I ", %" #KI ", %" #QI " row_newbcast:" #N " row_mask:0xf bank_mask:0xf\n\t"
#define LIT_FMAC_BCAST(N, A, KA, KB, QA, QB)                                                              \
  asm volatile("s_nop 1\n\t" LIT_FMAC_LINE(0, 4, 12, N) LIT_FMAC_LINE(1, 5, 12, N) LIT_FMAC_LINE(2, 6, 12, N) \
                   LIT_FMAC_LINE(3, 7, 12, N) LIT_FMAC_LINE(0, 8, 13, N) LIT_FMAC_LINE(1, 9, 13, N)              \
                       LIT_FMAC_LINE(2, 10, 13, N) LIT_FMAC_LINE(3, 11, 13, N)                                   \
               : "+v"(A[0]), "+v"(A[1]), "+v"(A[2]), "+v"(A[3])                                                  \
               : "v"(KA[0]), "v"(KA[1]), "v"(KA[2]), "v"(KA[3]), "v"(KB[0]), "v"(KB[1]), "v"(KB[2]), "v"(KB[3]), \
                 "v"(QA), "v"(QB))

// One dim pair (32c + 2N, 32c + 2N + 1) of the running dot products: lane N of
// each row holds those two key values of every entry (kA, kB).
#define LIT_BAND_STEP(N)                                                 \
  {                                                                      \
    const double q0 = (double)qv[((N) >> 1) & 1][2 * ((N)&1)];           \
    const double q1 = (double)qv[((N) >> 1) & 1][2 * ((N)&1) + 1];       \
    LIT_FMAC_BCAST(N, acc, kA, kB, q0, q1);                              \
  }
// the q values of dims 32c + 8u .. +7 (quarter u of block c) were loaded into
// qn; they move to qv and the next quarter's are requested
#define LIT_BAND_QUARTER(U, S0, S1, S2, S3)                                             \
  {                                                                                     \
    qv[0] = qn[0];                                                                      \
    qv[1] = qn[1];                                                                      \
    if (32 * c + 8 * (U) + 8 < LIT_IDX_DIM) {                                           \
      qn[0] = *(const f32x4*)(qr + 32 * c + 8 * (U) + 8);                               \
      qn[1] = *(const f32x4*)(qr + 32 * c + 8 * (U) + 12);                              \
    }                                                                                   \
    LIT_BAND_STEP(S0) LIT_BAND_STEP(S1) LIT_BAND_STEP(S2) LIT_BAND_STEP(S3)             \
  }

// fp64 canonical scores of up to BW band entries by one wave: entry j is
// band_n[e0 + es * j] (entries at or past M, M >= 1, are computed on the row
// of entry 0 and dropped). Lane h owns head h: its q row is read from qP, and the key values
// come to it by DPP broadcast from the lanes of its row, each of which loaded
// one dim pair per 32-dim block. Every dot product runs in dim order, the head
// terms w_h * max(acc, 0) go through psum, and lane j adds entry j's terms in
// head order (lanes h >= H post +0.0, which leaves a sum that starts at +0.0
// unchanged).
template <bool BF16>
__device__ __forceinline__ void band_scores_bcast(const TopkParams& P, int b, const float* qP, float w_h,
                                                  const int32_t* band_n, int M, int e0, int es,
                                                  double (*psum)[PSUM_LD], double* band_s) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63, nl = lane & 15;
  const float* qr = qP + lane * QP_STRIDE;
  // the sequence's keys (a wave-uniform base) and 32-bit element offsets in it
  // (N * 128 < 2^32 on the paths that call this)
  const size_t kbase = (size_t)(b / P.kq) * P.N * LIT_IDX_DIM;
  uint32_t roff[BW];
#pragma unroll
  for (int j = 0; j < BW; j++) {
    const int e = e0 + es * j;
    roff[j] = (uint32_t)band_n[e < M ? e : 0] * LIT_IDX_DIM + 2 * nl;  // M >= 1; band_n[>= M] is unset
  }
  const uint16_t* kb16 = (const uint16_t*)P.kidx + kbase;
  const float* kb32 = (const float*)P.kidx + kbase;
  uint32_t kr[BW];  // bf16 key pairs of the next block (one dword per block)
  if constexpr (BF16) {
#pragma unroll
    for (int j = 0; j < BW; j++) kr[j] = *(const uint32_t*)(kb16 + roff[j]);
  }
  double acc[BW];
#pragma unroll
  for (int j = 0; j < BW; j++) acc[j] = 0.0;
  f32x4 qv[2], qn[2];
  qn[0] = *(const f32x4*)qr;
  qn[1] = *(const f32x4*)(qr + 4);
#pragma unroll
  for (int c = 0; c < 4; c++) {
    double kA[BW], kB[BW];
#pragma unroll
    for (int j = 0; j < BW; j++) {
      float2 kp;
      if constexpr (BF16) {
        kp = make_float2(bf16_lo(kr[j]), bf16_hi(kr[j]));
        if (c + 1 < 4) kr[j] = *(const uint32_t*)(kb16 + roff[j] + 32 * (c + 1));
      } else {
        kp = *(const float2*)(kb32 + roff[j] + 32 * c);
      }
      kA[j] = (double)kp.x;
      kB[j] = (double)kp.y;
    }
    LIT_BAND_QUARTER(0, 0, 1, 2, 3)
    LIT_BAND_QUARTER(1, 4, 5, 6, 7)
    LIT_BAND_QUARTER(2, 8, 9, 10, 11)
    LIT_BAND_QUARTER(3, 12, 13, 14, 15)
  }
#pragma unroll
  for (int j = 0; j < BW; j++) {
    const double a = acc[j] > 0.0 ? acc[j] : 0.0;
    psum[j][lane] = lane < P.H ? (double)w_h * a : 0.0;
  }
  wave_sync();
  {
    const double* pr = psum[lane & (BW - 1)];
    double s = 0.0;
#pragma unroll 16
    for (int h = 0; h < 64; h++) s = s + pr[h];
    const int e = e0 + es * lane;
    if (lane < BW && e < M) band_s[e] = s;
  }
  wave_sync();  // psum is refilled by the next round
}

// The same fp64 canonical scores with one entry per wave and round: entry
// band_n[w + nw * j] in round j of wave w (w < nw), so that no wave computes a
// padding slot and a short band spreads over all nw waves (fp64 issue runs at
// one instruction per ~8 cycles for a lone wave on its SIMD, ~4.5 with four).
// For M <= nw * BW. The key dwords of every round are requested first, in one
// round trip; the rounds' head terms go to psum[j], and lane j adds round j's
// in head order at the end.
#define LIT_FMAC1(N, A, KA, KB, QA, QB)                                                   \
  asm volatile("s_nop 1\n\t" LIT_FMAC_LINE(0, 1, 3, N) LIT_FMAC_LINE(0, 2, 4, N)          \
               : "+v"(A)                                                                  \
               : "v"(KA), "v"(KB), "v"(QA), "v"(QB))
#define LIT_ROUND_STEP(N)                                               \
  {                                                                     \
    const double q0 = (double)qv[((N) >> 1) & 1][2 * ((N)&1)];          \
    const double q1 = (double)qv[((N) >> 1) & 1][2 * ((N)&1) + 1];      \
    LIT_FMAC1(N, acc, kA, kB, q0, q1);                                  \
  }
#define LIT_ROUND_QUARTER(U, S0, S1, S2, S3)                                            \
  {                                                                                     \
    qv[0] = qn[0];                                                                      \
    qv[1] = qn[1];                                                                      \
    if (32 * c + 8 * (U) + 8 < LIT_IDX_DIM) {                                           \
      qn[0] = *(const f32x4*)(qr + 32 * c + 8 * (U) + 8);                               \
      qn[1] = *(const f32x4*)(qr + 32 * c + 8 * (U) + 12);                              \
    }                                                                                   \
    LIT_ROUND_STEP(S0) LIT_ROUND_STEP(S1) LIT_ROUND_STEP(S2) LIT_ROUND_STEP(S3)         \
  }
template <bool BF16>
__device__ __forceinline__ void band_scores_rounds(const TopkParams& P, int b, const float* qP, float w_h,
                                                   const int32_t* band_n, int M, int nw,
                                                   double (*psum)[PSUM_LD], double* band_s) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nl = lane & 15;
  const int R = wid < nw && wid < M ? (M - wid + nw - 1) / nw : 0;  // rounds of this wave (<= BW)
  if (R == 0) return;
  const float* qr = qP + lane * QP_STRIDE;
  const size_t kbase = (size_t)(b / P.kq) * P.N * LIT_IDX_DIM;
  // the key values of every round (rounds past R repeat round 0's entry and
  // are not computed): lane nl of each row holds dims 32c + 2nl, +1
  float2 kp[BW][4];
#pragma unroll
  for (int j = 0; j < BW; j++) {
    const uint32_t roff = (uint32_t)band_n[wid + nw * (j < R ? j : 0)] * LIT_IDX_DIM + 2 * nl;
#pragma unroll
    for (int c = 0; c < 4; c++) {
      if constexpr (BF16) {
        const uint32_t kr = *(const uint32_t*)((const uint16_t*)P.kidx + kbase + roff + 32 * c);
        kp[j][c] = make_float2(bf16_lo(kr), bf16_hi(kr));
      } else {
        kp[j][c] = *(const float2*)((const float*)P.kidx + kbase + roff + 32 * c);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < BW; j++) {
    if (j < R) {
      double acc = 0.0;
      f32x4 qv[2], qn[2];
      qn[0] = *(const f32x4*)qr;
      qn[1] = *(const f32x4*)(qr + 4);
#pragma unroll
      for (int c = 0; c < 4; c++) {
        const double kA = (double)kp[j][c].x, kB = (double)kp[j][c].y;
        LIT_ROUND_QUARTER(0, 0, 1, 2, 3)
        LIT_ROUND_QUARTER(1, 4, 5, 6, 7)
        LIT_ROUND_QUARTER(2, 8, 9, 10, 11)
        LIT_ROUND_QUARTER(3, 12, 13, 14, 15)
      }
      const double a = acc > 0.0 ? acc : 0.0;
      psum[j][lane] = lane < P.H ? (double)w_h * a : 0.0;
    }
  }
  wave_sync();
  if (lane < R) {
    const double* pr = psum[lane];
    double s = 0.0;
#pragma unroll 16
    for (int h = 0; h < 64; h++) s = s + pr[h];
    band_s[wid + nw * lane] = s;
  }
}
#undef LIT_ROUND_QUARTER
#undef LIT_ROUND_STEP
#undef LIT_FMAC1
#undef LIT_BAND_QUARTER
#undef LIT_BAND_STEP
#undef LIT_FMAC_BCAST
#undef LIT_FMAC_LINE

// ---------------------------------------------------------------- fast path

// Block-wide reduction of (sum, min, max) over all threads; uses sc->scan.
// (fresh: nothing has read sc in this workgroup yet, so the barrier that keeps
// its earlier readers from being overwritten is not needed.)
__device__ __forceinline__ void block_sum_min_max(int& s, uint32_t& mn, uint32_t& mx, float& fm,
                                                  SelectScratch* sc, bool fresh = false) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    s += __shfl_xor(s, o);
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
    fm = fmaxf(fm, __shfl_xor(fm, o));
  }
  if (!fresh) lds_barrier();
  if (lane == 0) {
    sc->scan[wid] = s;
    sc->hist[wid] = mn;
    sc->hist[16 + wid] = mx;
    sc->hist[32 + wid] = __float_as_uint(fm);
  }
  lds_barrier();
  s = 0;
  mn = 0xffffffffu;
  mx = 0u;
  fm = 0.f;
  for (int i = 0; i < NWAVES; i++) {
    s += sc->scan[i];
    mn = min(mn, sc->hist[i]);
    mx = max(mx, sc->hist[16 + i]);
    fm = fmaxf(fm, __uint_as_float(sc->hist[32 + i]));
  }
  lds_barrier();
}

// One 2048-bin histogram pass over the non-zero keys in [kmin, kmax] (the bins
// span the bits below the keys' common prefix). Finds the bin holding the r-th
// largest key. Returns the bin's lower edge; *above = keys in higher bins,
// *in_bin = keys in the bin; *binfn receives (prefix, shift) for bin numbers.
template <typename KeyFn>
__device__ uint32_t hist_kth(KeyFn key, int M, int r, uint32_t kmin, uint32_t kmax, uint32_t* hist2k,
                             SelectScratch* sc, int* above, int* in_bin, uint32_t* prefix_out, int* shift_out) {
  const int tid = threadIdx.x;
  const uint32_t diff = kmin ^ kmax;
  const int hb = diff ? 31 - __clz((int)diff) : 0;
  const int shift = hb > 10 ? hb - 10 : 0;
  const uint32_t prefix = kmax & ~((2u << hb) - 1u);
  for (int i = tid; i < 2048; i += TK_THREADS) hist2k[i] = 0u;
  lds_barrier();
  for (int i = tid; i < M; i += TK_THREADS) {
    const uint32_t kk = key(i);
    if (kk != 0u) atomicAdd(&hist2k[(kk - prefix) >> shift], 1u);
  }
  lds_barrier();
  // cumulative counts from the top bin down: thread t owns bins 2047-2t, 2046-2t
  const int c0 = (int)hist2k[2047 - 2 * tid], c1 = (int)hist2k[2046 - 2 * tid];
  int tot;
  const int ab = block_excl_scan(c0 + c1, sc->scan, &tot);
  if (ab < r && r <= ab + c0) {
    sc->misc[0] = 2047 - 2 * tid;
    sc->misc[1] = ab;
    sc->misc[2] = c0;
  } else if (ab + c0 < r && r <= ab + c0 + c1) {
    sc->misc[0] = 2046 - 2 * tid;
    sc->misc[1] = ab + c0;
    sc->misc[2] = c1;
  }
  lds_barrier();
  const int bin = sc->misc[0];
  *above = sc->misc[1];
  *in_bin = sc->misc[2];
  *prefix_out = prefix;
  *shift_out = shift;
  lds_barrier();
  return prefix + ((uint32_t)bin << shift);
}

// The row's q (fp32, exact mode) to LDS for the rescoring, one 8-dim piece
// per thread (q and w are per row).
__device__ void stage_q_rows(const TopkParams& P, float* qP, int b) {
  const int tid = threadIdx.x;
  const int h = tid >> 4, d8 = tid & 15;
  float x[8];
  if (h < P.H) {
    const size_t off = ((size_t)b * P.H + h) * LIT_IDX_DIM + 8 * d8;
    if (P.dtype == LIT_BF16) {
      const u32x4 v = *(const u32x4*)((const uint16_t*)P.q + off);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        x[2 * i] = bf16_lo(v[i]);
        x[2 * i + 1] = bf16_hi(v[i]);
      }
    } else {
      const f32x4 v0 = *(const f32x4*)((const float*)P.q + off), v1 = *(const f32x4*)((const float*)P.q + off + 4);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        x[i] = v0[i];
        x[4 + i] = v1[i];
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; i++) x[i] = 0.f;
  }
  *(f32x4*)&qP[h * QP_STRIDE + 8 * d8] = f32x4{x[0], x[1], x[2], x[3]};
  *(f32x4*)&qP[h * QP_STRIDE + 8 * d8 + 4] = f32x4{x[4], x[5], x[6], x[7]};
}

// Wide path: for long rows one workgroup per row leaves most CUs idle while it
// reads the group maxima, gathers candidates and rescores the band, so the
// work is split over two kernels.
//   A (S workgroups per row, slice s = groups s*GS .. +GS-1): every workgroup
//     builds the histogram of all the row's group maxima and reads off L, the
//     lower edge of the bin of the k-th largest (at least k entries reach it,
//     so the k-th score T >= L), and H, the upper edge of the bin of the
//     (k - WIDE_MARGIN)-th largest. In exact mode lo = L - 2 Delta and
//     hx = H + 2 Delta (Delta from the hints). It lists its slice's entries
//     with key >= lo (key, index), in index order, at the slice's own place in
//     the workspace, rescores in fp64 those with key <= hx, and clears its
//     slice of the mask.
//   B (one workgroup per row): the lists concatenated are the candidates, in
//     index order. Every entry of the exact top k is one: its fp32 score is at
//     least T - 2 Delta >= lo. When fewer than k candidates lie above
//     hx - 2 Delta, T <= hx - 2 Delta, so every candidate above hx has an exact
//     score above the k-th exact score and is selected; the other k - (those)
//     are the best rescored candidates by (exact score desc, index asc). When
//     that test fails (or a list overflowed) B finds T itself and rescores its
//     band; without exact mode it finds the k-th fp32 key.
constexpr int WIDE_SLICES_MAX = 64;  // slices per row
constexpr int WIDE_HDR = 8;          // header words per row before its slice counts
constexpr int WIDE_STRIDE = WIDE_HDR + WIDE_SLICES_MAX;
constexpr int WIDE_MARGIN = 64;      // ranks between the group maxima that give L and H
constexpr int WIDE_RCAP = 256;       // entries one slice rescores
constexpr int WIDE_RWAVES = 8;       // waves that rescore in kernel A
constexpr uint32_t WIDE_OVERFLOW = 1u << 30;  // in a slice count: more than WIDE_RCAP to rescore
// header words: 0 L, 1 lo, 2 selectable groups, 3 largest key-norm bound (bits),
// 4-5 Delta, 6 hx, 7 the key of hx - 2 Delta (rounded down)

// Kernel A's workgroup -> (row, slice). When the rows are a multiple of 8,
// every slice of row b has a workgroup id equal to b modulo 8 (XCD b % 8, where
// kernel B's workgroup b reads the lists); otherwise the slices of a row are
// consecutive workgroups, spread over every XCD.
__device__ __forceinline__ void wide_unit(int x, int rows, int S, int* b, int* s) {
  if (rows % 8 == 0) {
    *s = (x >> 3) % S;
    *b = ((x >> 3) / S) * 8 + (x & 7);
  } else {
    *b = x / S;
    *s = x % S;
  }
}

struct WideLds {  // kernel A
  SelectScratch sc;
  float qP[64 * QP_STRIDE];
  union {
    struct {
      uint32_t hist2k[2048];
      uint32_t gkey[GM_CAP];
    };
    double psum[WIDE_RWAVES][BW][PSUM_LD];  // once the group keys are dead
  };
  int32_t rl_n[WIDE_RCAP];     // entries to rescore
  int32_t rl_slot[WIDE_RCAP];  // their places in the slice's list
  double rl_s[WIDE_RCAP];      // their exact scores
};

__device__ void wide_candidates(const TopkParams& P, WideLds& L) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int S = P.wide_slices;
  int b, s;
  wide_unit((int)blockIdx.x, P.rows, S, &b, &s);
  const int N = P.N, k = P.k;
  const int G = (N + GROUP - 1) / GROUP;
  const float* sb = P.scores + (size_t)b * N;
  const float* hb = P.hints + (size_t)b * P.hints_len;
  const float* gmx = hb + P.nchunks;

  // 1. group keys (+ the largest key-norm bound, q and w in exact mode). The
  //    group maxima (at most GM_CAP / TK_THREADS per thread, at clamped
  //    addresses) are requested before anything waits, so that they and the
  //    exact mode's reads come back in one round trip instead of one per
  //    thousand groups
  constexpr int GPT = GM_CAP / TK_THREADS;
  static_assert(GPT * TK_THREADS == GM_CAP && GM_CAP * GROUP / LIT_KNORM_CHUNK <= TK_THREADS, "one pass of loads");
  float gv[GPT];
#pragma unroll
  for (int j = 0; j < GPT; j++) gv[j] = gmx[min(tid + TK_THREADS * j, G - 1)];
  float knorm = 0.f, w_h = 0.f;
  if (P.exact) {
    const float kn = hb[min(tid, P.nchunks - 1)];  // at most TK_THREADS chunks on this path
    knorm = tid < P.nchunks ? kn : 0.f;
    w_h = lane < P.H ? P.w[(size_t)b * P.H + lane] : 0.f;
    stage_q_rows(P, L.qP, b);
  }
  int ns = 0;
  uint32_t kmin = 0xffffffffu, kmx = 0u;
  uint32_t gk[GPT];  // this thread's group keys (0 past G), kept for the histogram
#pragma unroll
  for (int j = 0; j < GPT; j++) {
    const int g = tid + TK_THREADS * j;
    gk[j] = g < G ? score_key(gv[j]) : 0u;
    if (g < G) L.gkey[g] = gk[j];
    if (gk[j]) {
      ns++;
      kmin = min(kmin, gk[j]);
      kmx = max(kmx, gk[j]);
    }
  }
  // (cleared here: the reduction's barriers order it before the histogram)
  for (int i = tid; i < 2048; i += TK_THREADS) L.hist2k[i] = 0u;
  block_sum_min_max(ns, kmin, kmx, knorm, &L.sc, true);

  // 2. L and H from one histogram of the group keys (the bins span the bits
  //    below the common prefix of the smallest and largest)
  uint32_t lkey = 1u, hkey = kmx;
  if (ns >= k) {
    const uint32_t diff = kmin ^ kmx;
    const int hbit = diff ? 31 - __clz((int)diff) : 0;
    const int shift = hbit > 10 ? hbit - 10 : 0;
    const uint32_t prefix = kmx & ~((2u << hbit) - 1u);
#pragma unroll
    for (int j = 0; j < GPT; j++)
      if (gk[j] != 0u) atomicAdd(&L.hist2k[(gk[j] - prefix) >> shift], 1u);
    lds_barrier();
    // cumulative counts from the top bin down: thread t owns bins 2047-2t, 2046-2t
    const int c0 = (int)L.hist2k[2047 - 2 * tid], c1 = (int)L.hist2k[2046 - 2 * tid];
    int tot;
    const int ab = block_excl_scan1<NWAVES>(c0 + c1, L.sc.scan, &tot);
    const int r1 = k, r2 = max(1, k - WIDE_MARGIN);
    if (ab < r1 && r1 <= ab + c0) L.sc.misc[0] = 2047 - 2 * tid;
    if (ab + c0 < r1 && r1 <= ab + c0 + c1) L.sc.misc[0] = 2046 - 2 * tid;
    if (ab < r2 && r2 <= ab + c0) L.sc.misc[1] = 2047 - 2 * tid;
    if (ab + c0 < r2 && r2 <= ab + c0 + c1) L.sc.misc[1] = 2046 - 2 * tid;
    lds_barrier();
    lkey = prefix + ((uint32_t)L.sc.misc[0] << shift);
    hkey = min(kmx, prefix + ((uint32_t)(L.sc.misc[1] + 1) << shift) - 1u);
  }
  uint32_t lo = lkey, hx = 0u, c2 = 0u;
  double delta = 0.0;
  if (P.exact) {
    const uint32_t* qb = reinterpret_cast<const uint32_t*>(hb + P.hints_len) - LIT_HINT_QBOUND;
    const double Q = __longlong_as_double((long long)(((uint64_t)qb[1] << 32) | qb[0]));
    const double Wa = __longlong_as_double((long long)(((uint64_t)qb[3] << 32) | qb[2]));
    delta = score_err_bound(P.dtype == LIT_BF16, P.H, Q, (double)knorm, Wa);
    if (lkey > 1u) {
      const uint32_t l0 = score_key(__double2float_rd((double)key_score(lkey) - 2.0 * delta));
      lo = l0 > 1u ? l0 : 1u;
    }
    const uint32_t h0 = score_key(__double2float_ru((double)key_score(hkey) + 2.0 * delta));
    hx = h0 ? h0 : 0xff800000u;  // past the largest finite key: +inf's
    c2 = score_key(__double2float_rd((double)key_score(hx) - 2.0 * delta));
  }

  // 3. this slice's entries >= lo, one group per thread, in index order; in
  //    exact mode those <= hx are also listed for the rescoring
  const int GS = (G + S - 1) / S;
  const int g0 = min(G, s * GS), g1 = min(G, g0 + GS);
  const int g = g0 + tid;
  const bool live = g < g1 && L.gkey[g] >= lo;
  uint32_t kv[GROUP];
  int c = 0, r = 0;
  if (live) {
    const int e0 = GROUP * g;
    if ((reinterpret_cast<uintptr_t>(sb) & 15u) == 0 && e0 + GROUP <= N) {
#pragma unroll
      for (int q = 0; q < GROUP / 4; q++) {
        const f32x4 x = *(const f32x4*)(sb + e0 + 4 * q);
#pragma unroll
        for (int i = 0; i < 4; i++) kv[4 * q + i] = score_key(x[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < GROUP; i++) kv[i] = e0 + i < N ? score_key(sb[e0 + i]) : 0u;
    }
#pragma unroll
    for (int i = 0; i < GROUP; i++) {
      c += kv[i] >= lo;  // lo >= 1: key 0 is never listed
      r += kv[i] >= lo && kv[i] <= hx;
    }
  }
  int tot;
  int pos = block_excl_scan1<NWAVES>((c << 16) | r, L.sc.scan, &tot);
  int rpos = pos & 0xffff;
  pos >>= 16;
  const int ctot = tot >> 16, rtot = tot & 0xffff;
  const size_t base = (size_t)b * N + GROUP * g0;
  uint32_t* ck = P.ws_ckey + base;
  int32_t* ci = P.ws_band_n + base;
  if (live) {
#pragma unroll
    for (int i = 0; i < GROUP; i++)
      if (kv[i] >= lo) {
        ck[pos] = kv[i];
        ci[pos] = GROUP * g + i;
        if (kv[i] <= hx && rpos < WIDE_RCAP) {
          L.rl_n[rpos] = GROUP * g + i;
          L.rl_slot[rpos] = pos;
        }
        rpos += kv[i] <= hx;
        pos++;
      }
  }
  int32_t* hdr = P.ws_wide + (size_t)b * WIDE_STRIDE;
  if (tid == 0) {
    hdr[WIDE_HDR + s] = ctot | (rtot > WIDE_RCAP ? (int)WIDE_OVERFLOW : 0);
    if (s == 0) {
      const uint64_t db = (uint64_t)__double_as_longlong(delta);
      hdr[0] = (int32_t)lkey;
      hdr[1] = (int32_t)lo;
      hdr[2] = ns;
      hdr[3] = __float_as_int(knorm);
      hdr[4] = (int32_t)(uint32_t)db;
      hdr[5] = (int32_t)(uint32_t)(db >> 32);
      hdr[6] = (int32_t)hx;
      hdr[7] = (int32_t)c2;
    }
  }
  if (P.mask) {
    uint8_t* mb = P.mask + (size_t)b * N;
    const int m1 = min(N, GROUP * g1);
    for (int n = GROUP * g0 + tid; n < m1; n += TK_THREADS) mb[n] = 0;
  }

  // 4. exact mode: the listed entries rescored in fp64 (the group keys are dead:
  //    psum takes their place), their scores stored beside their list places
  if (P.exact && rtot > 0 && rtot <= WIDE_RCAP) {
    lds_barrier();  // the list, q and the last reads of the group keys
    const int M = rtot;
    if (M <= WIDE_RWAVES * BW) {
      if (wid < WIDE_RWAVES) {
        if (P.dtype == LIT_BF16)
          band_scores_rounds<true>(P, b, L.qP, w_h, L.rl_n, M, WIDE_RWAVES, L.psum[wid], L.rl_s);
        else
          band_scores_rounds<false>(P, b, L.qP, w_h, L.rl_n, M, WIDE_RWAVES, L.psum[wid], L.rl_s);
      }
    } else {
      const int nwr = WIDE_RWAVES;
      for (int e = 0; e + wid < M && wid < nwr; e += nwr * BW) {
        if (P.dtype == LIT_BF16)
          band_scores_bcast<true>(P, b, L.qP, w_h, L.rl_n, M, e + wid, nwr, L.psum[wid], L.rl_s);
        else
          band_scores_bcast<false>(P, b, L.qP, w_h, L.rl_n, M, e + wid, nwr, L.psum[wid], L.rl_s);
      }
    }
    lds_barrier();
    double* cs = P.ws_band_s + base;
    for (int i = tid; i < M; i += TK_THREADS) cs[L.rl_slot[i]] = L.rl_s[i];
  }
}

// Kernel B's steps over the candidates in L.ckey / L.cidx (index order, M1 of
// them: every entry with key >= lo, lo <= L, where L bounds the k-th key from
// below). The selection is kept as one bit per candidate position and written
// out by a scan over the candidates. Returns false, having written nothing,
// when a capacity is exceeded or the band reaches below lo (the caller then
// scans every score). The mask was cleared by kernel A: only selected entries
// are set.
__device__ bool finish_candidates(const TopkParams& P, FastLds& L, int b, int M1, uint32_t lo, double delta) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int N = P.N, k = P.k;
  int32_t* ids = P.ids + (size_t)b * k;
  uint8_t* mask = P.mask ? P.mask + (size_t)b * N : nullptr;
  uint32_t* sel = L.sel;  // bit i: candidate i selected
  const int SW = (M1 + 31) / 32;
  for (int w = tid; w < SW; w += TK_THREADS) sel[w] = M1 <= k ? ~0u : 0u;  // M1 <= k: every candidate
  if (M1 > k) {
    // 4. the k-th candidate: histogram bin, then exact ranks inside the bin
    uint32_t cmin = 0xffffffffu, cmx = 0u;
    int dummy = 0;
    float fd = 0.f;
    for (int i = tid; i < M1; i += TK_THREADS) {
      cmin = min(cmin, L.ckey[i]);
      cmx = max(cmx, L.ckey[i]);
    }
    block_sum_min_max(dummy, cmin, cmx, fd, &L.sc);
    int above, inb, shift;
    uint32_t prefix;
    const uint32_t bin_lo = hist_kth([&](int i) -> uint32_t { return L.ckey[i]; }, M1, k, cmin, cmx, L.hist2k,
                                     &L.sc, &above, &inb, &prefix, &shift);
    const uint32_t bin_id = (bin_lo - prefix) >> shift;
    const int r = k - above;  // members of the bin that are selected
    // rank inside the bin by (key desc, index asc); the r-th gives T. The bin's
    // members are listed first (candidate positions, index order) so the ranking
    // only compares members with each other.
    {
      const int cs = (M1 + TK_THREADS - 1) / TK_THREADS;
      const int c0 = min(M1, tid * cs), c1 = min(M1, c0 + cs);
      int nin = 0;
      for (int i = c0; i < c1; i++) nin += ((L.ckey[i] - prefix) >> shift) == bin_id;
      int m;
      int bp = block_excl_scan(nin, L.sc.scan, &m);
      for (int i = c0; i < c1; i++) {
        L.cflag[i] = 0;
        if (((L.ckey[i] - prefix) >> shift) == bin_id) L.binpos[bp++] = (uint16_t)i;
      }
      lds_barrier();
      for (int t = tid; t < m; t += TK_THREADS) {
        const int i = L.binpos[t];
        const uint32_t ki = L.ckey[i];
        const int ni = L.cidx[i];
        int rank = 0;
        for (int j0 = 0; j0 < m; j0 += 8) {  // reads 8 at a time (clamped in range)
          uint32_t kj[8];
          int nj[8];
#pragma unroll
          for (int u = 0; u < 8; u++) {
            const int pj = L.binpos[min(j0 + u, m - 1)];
            kj[u] = L.ckey[pj];
            nj[u] = L.cidx[pj];
          }
#pragma unroll
          for (int u = 0; u < 8; u++) rank += j0 + u < m && ((kj[u] > ki) || (kj[u] == ki && nj[u] < ni));
        }
        L.cflag[i] = rank < r;
        if (rank == r - 1) L.sc.misc[4] = (int)ki;
      }
    }
    lds_barrier();
    const uint32_t T = (uint32_t)L.sc.misc[4];
    if (!P.exact) {
      for (int i = tid; i < M1; i += TK_THREADS) {
        const uint32_t bi = (L.ckey[i] - prefix) >> shift;
        if (bi > bin_id || (bi == bin_id && L.cflag[i])) atomicOr(&sel[i >> 5], 1u << (i & 31));
      }
    } else {
      // 5. exact band around T: [T - 2 Delta, T + 2 Delta] (Delta as kernel A took it)
      const double t = (double)key_score(T);
      const uint32_t blo0 = score_key(__double2float_rd(t - 2.0 * delta));
      const uint32_t blo = blo0 > 1u ? blo0 : 1u;
      const uint32_t hi = score_key(__double2float_ru(t + 2.0 * delta));
      if (blo < lo) return false;  // entries below lo were not listed
      // band members among the candidates (index order) and the sure ones
      const int cseg = (M1 + TK_THREADS - 1) / TK_THREADS;
      const int ca = min(M1, tid * cseg), ce = min(M1, ca + cseg);
      int nd = 0, nb = 0;
      for (int i = ca; i < ce; i++) {
        const uint32_t kk = L.ckey[i];
        nd += kk > hi;
        nb += (kk >= blo) && (kk <= hi);
      }
      int tot;
      int bpos = block_excl_scan((nd << 16) | nb, L.sc.scan, &tot);
      bpos &= 0xffff;
      const int A = tot >> 16;
      const int M = tot & 0xffff;
      if (M > FBAND_CAP) return false;
      for (int i = ca; i < ce; i++) {
        const uint32_t kk = L.ckey[i];
        if (kk > hi) atomicOr(&sel[i >> 5], 1u << (i & 31));
        if ((kk >= blo) && (kk <= hi)) {
          L.band_n[bpos] = L.cidx[i];
          L.binpos[bpos] = (uint16_t)i;  // the member's candidate position
          bpos++;
        }
      }
      lds_barrier();
      const int rr = k - A;
      if (rr < 1 || rr > M) {
        report_violation(P, b, ids, mask);
        return true;
      }
      // fp64 rescoring: BW entries per wave and round, key values broadcast
      // across each row; as many waves as the band needs, a multiple of four
      // (one more per SIMD), at least eight
      const float w_h = lane < P.H ? P.w[(size_t)b * P.H + lane] : 0.f;
      const int nwr = min(NWAVES, max(8, ((M + BW - 1) / BW + 3) & ~3));  // 8, 12 or 16 waves
      for (int base = 0; base + wid < M && wid < nwr; base += nwr * BW) {
        if (P.dtype == LIT_BF16)
          band_scores_bcast<true>(P, b, L.qP, w_h, L.band_n, M, base + wid, nwr, L.psum[wid], L.band_s);
        else
          band_scores_bcast<false>(P, b, L.qP, w_h, L.band_n, M, base + wid, nwr, L.psum[wid], L.band_s);
      }
      lds_barrier();
      for (int i = tid; i < M; i += TK_THREADS) {
        const double si = L.band_s[i];
        const int ni = L.band_n[i];
        int rank = 0;
        for (int j0 = 0; j0 < M; j0 += 8) {  // reads 8 at a time (clamped in range)
          double sj[8];
          int nj[8];
#pragma unroll
          for (int u = 0; u < 8; u++) {
            sj[u] = L.band_s[min(j0 + u, M - 1)];
            nj[u] = L.band_n[min(j0 + u, M - 1)];
          }
#pragma unroll
          for (int u = 0; u < 8; u++) rank += j0 + u < M && ((sj[u] > si) || (sj[u] == si && nj[u] < ni));
        }
        if (rank < rr) {
          const int pos = L.binpos[i];
          atomicOr(&sel[pos >> 5], 1u << (pos & 31));
        }
      }
    }
  }
  lds_barrier();

  // 6. selected candidates -> ascending ids (candidates are in index order), mask, count
  const int cseg = (M1 + TK_THREADS - 1) / TK_THREADS;
  const int ca = min(M1, tid * cseg), ce = min(M1, ca + cseg);
  int c = 0;
  for (int i = ca; i < ce; i++) c += (sel[i >> 5] >> (i & 31)) & 1u;
  int total;
  int opos = block_excl_scan(c, L.sc.scan, &total);
  for (int i = ca; i < ce; i++)
    if ((sel[i >> 5] >> (i & 31)) & 1u) {
      const int n = L.cidx[i];
      if (opos < k) ids[opos] = n;
      opos++;
      if (mask) mask[n] = 1;
    }
  total = min(total, k);
  for (int j = total + tid; j < k; j += TK_THREADS) ids[j] = -1;
  if (tid == 0) P.count[b] = total;
  return true;
}

// Kernel B's fast case (exact mode; the candidates, their keys and kernel A's
// exact scores in LDS): selects the candidates above hx and the best
// k - (those) of the rescored ones. Returns false, having written nothing,
// when the test on hx fails (T may lie above hx - 2 Delta).
__device__ bool finish_rescored(const TopkParams& P, FastLds& L, int b, int M1, uint32_t lo, uint32_t hx,
                                uint32_t c2) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int N = P.N, k = P.k;
  const int cseg = (M1 + TK_THREADS - 1) / TK_THREADS;
  const int ca = min(M1, tid * cseg), ce = min(M1, ca + cseg);
  int sure = 0, resc = 0, above2 = 0;
  for (int i = ca; i < ce; i++) {
    const uint32_t kk = L.ckey[i];
    sure += kk > hx;
    resc += kk <= hx;  // every candidate is >= lo
    above2 += kk > c2;
  }
  above2 = wave_sum(above2);
  if (tid == 0) L.sc.misc[5] = 0;
  for (int w = tid; w < CAND_CAP / 32; w += TK_THREADS) L.sel[w] = 0u;
  int tot;
  int rpos = block_excl_scan1<NWAVES>((sure << 16) | resc, L.sc.scan, &tot);  // (its barrier orders misc[5] = 0)
  rpos &= 0xffff;
  if (lane == 0) atomicAdd(&L.sc.misc[5], above2);
  const int A = tot >> 16, R = tot & 0xffff;
  for (int i = ca; i < ce; i++) {
    const uint32_t kk = L.ckey[i];
    if (kk > hx) atomicOr(&L.sel[i >> 5], 1u << (i & 31));
    if (kk <= hx && rpos < FBAND_CAP) {
      L.band_n[rpos] = L.cidx[i];
      L.band_s[rpos] = L.cexact[i];
      L.binpos[rpos] = (uint16_t)i;
      rpos++;
    }
  }
  lds_barrier();
  const int need = k - A;
  if (L.sc.misc[5] >= k || R > FBAND_CAP || need < 1 || need > R) return false;
  // the best `need` rescored candidates by (exact score desc, index asc): lane
  // i of the block ranks entry i against every entry, each read by all lanes
  // at once (one broadcast per entry; the list is in index order)
  for (int i = tid; i - lane < R; i += TK_THREADS) {
    const double si = i < R ? L.band_s[i] : 0.0;
    int rank = 0;
    for (int j = 0; j < R; j++) {
      const double sj = L.band_s[j];
      rank += sj > si || (sj == si && j < i);
    }
    if (i < R && rank < need) {
      const int ps = L.binpos[i];
      atomicOr(&L.sel[ps >> 5], 1u << (ps & 31));
    }
  }
  lds_barrier();
  // selected candidates -> ascending ids, mask, count
  int32_t* ids = P.ids + (size_t)b * k;
  uint8_t* mask = P.mask ? P.mask + (size_t)b * N : nullptr;
  int c = 0;
  for (int i = ca; i < ce; i++) c += (L.sel[i >> 5] >> (i & 31)) & 1u;
  int total;
  int opos = block_excl_scan1<NWAVES>(c, L.sc.scan, &total);
  for (int i = ca; i < ce; i++)
    if ((L.sel[i >> 5] >> (i & 31)) & 1u) {
      const int n = L.cidx[i];
      ids[opos++] = n;
      if (mask) mask[n] = 1;
    }
  for (int j = total + tid; j < k; j += TK_THREADS) ids[j] = -1;
  if (tid == 0) P.count[b] = total;
  return true;
}

// Kernel B for row b. Returns false, having written nothing, when the row does
// not fit (the caller scans every score instead).
__device__ bool wide_finish(const TopkParams& P, FastLds& L, int b) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int S = P.wide_slices;
  const int N = P.N;
  const int G = (N + GROUP - 1) / GROUP;
  const int GS = (G + S - 1) / S;
  const int32_t* hdr = P.ws_wide + (size_t)b * WIDE_STRIDE;
  // every load in one round trip: the slice counts, the header, and the first
  // 64 entries of each list (wave w holds slices w, w + 16, ...; entries past
  // a list's capacity read its last slot and are dropped below)
  const int cword = tid < S ? hdr[WIDE_HDR + tid] : 0;
  const uint32_t lo = (uint32_t)hdr[1];
  const int ns = hdr[2];
  const double delta =
      __longlong_as_double((long long)(((uint64_t)(uint32_t)hdr[5] << 32) | (uint32_t)hdr[4]));
  const uint32_t hx = (uint32_t)hdr[6], c2 = (uint32_t)hdr[7];
  constexpr int SPW = WIDE_SLICES_MAX / NWAVES;  // slices per wave
  uint32_t sk[SPW];
  int32_t si[SPW];
  double sx[SPW];
#pragma unroll
  for (int u = 0; u < SPW; u++) {
    const int s = wid + NWAVES * u;
    const int e0 = GROUP * min(G, s * GS), cap = min(N, GROUP * min(G, s * GS + GS)) - e0;
    const size_t src = (size_t)b * N + e0 + (size_t)min(lane, max(cap - 1, 0));
    sk[u] = s < S ? P.ws_ckey[src] : 0u;
    si[u] = s < S ? P.ws_band_n[src] : 0;
    sx[u] = s < S && P.exact ? P.ws_band_s[src] : 0.0;  // set only where kernel A rescored
  }
  const int cnt = cword & ~(int)WIDE_OVERFLOW;
  int M1;
  const int off = block_excl_scan1<NWAVES>(cnt, L.sc.scan, &M1);
  const bool overflow = __syncthreads_or((cword & (int)WIDE_OVERFLOW) != 0);
  if (ns == 0) {  // nothing selectable (the mask is already clear)
    int32_t* ids = P.ids + (size_t)b * P.k;
    for (int j = tid; j < P.k; j += TK_THREADS) ids[j] = -1;
    if (tid == 0) P.count[b] = 0;
    return true;
  }
  // more candidates than LDS holds, or fewer than k although k group maxima
  // reach L (hints that are not these scores')
  if (M1 > CAND_CAP || (ns >= P.k && M1 < P.k)) return false;
  if (tid < S) {
    L.sc.hist[tid] = (uint32_t)off;
    L.sc.hist[WIDE_SLICES_MAX + tid] = (uint32_t)cnt;
  }
  lds_barrier();
#pragma unroll
  for (int u = 0; u < SPW; u++) {
    const int s = wid + NWAVES * u;
    if (s < S) {
      const int o = (int)L.sc.hist[s], n = (int)L.sc.hist[WIDE_SLICES_MAX + s];
      if (lane < n) {
        L.ckey[o + lane] = sk[u];
        L.cidx[o + lane] = si[u];
        L.cexact[o + lane] = sx[u];
      }
      if (n > 64) {  // the rest of a long list
        const size_t src = (size_t)b * N + GROUP * min(G, s * GS);
        for (int j = 64 + lane; j < n; j += 64) {
          L.ckey[o + j] = P.ws_ckey[src + j];
          L.cidx[o + j] = P.ws_band_n[src + j];
          L.cexact[o + j] = P.exact ? P.ws_band_s[src + j] : 0.0;
        }
      }
    }
  }
  lds_barrier();
  if (P.exact && !overflow && M1 > P.k) {
    if (finish_rescored(P, L, b, M1, lo, hx, c2)) return true;
    lds_barrier();
  }
  // T taken here, the band rescored here (q staged for it)
  if (P.exact) {
    stage_q_rows(P, L.qP, b);  // (the exact scores are no longer read)
    lds_barrier();
  }
  return finish_candidates(P, L, b, M1, lo, delta);
}

// ---------------------------------------------------------------- small path

// N <= 16 * 1024 has a kernel of its own (its own register budget): thread t
// keeps the scores of entries 16t .. 16t+15 in registers. With four waves per
// SIMD the workgroup's time goes to issuing per-entry vector instructions and
// to the barriers between its steps, so the entries are swept twice only, and
// the steps are few:
//   1. the range of the histogram comes from the hints alone (largest and
//      smallest of the per-16-entry score maxima; each group holds an entry
//      that large, so with k <= N/16 groups the k-th score is at least the
//      smallest), reduced while the scores are still in flight; without
//      usable hints, from the keys;
//   2. a histogram of the keys in that range, over the bits below the common
//      prefix of its ends, finds the bin of the k-th score;
//   3. each entry is then "above" (selected for sure) or in the band (decided
//      by rank) or out: the band is the bin itself (ranked by key and index),
//      or in exact mode the bin widened by 2 delta both ways, whose entries
//      are rescored in fp64; one scan gives every thread the number of above
//      and band entries before its own;
//   4. the output offset of a thread is the above entries before it plus the
//      chosen band entries before its first band slot, so each thread writes
//      its selected ids in index order with no further scan.
// Reductions and scans run on DPP lane moves; each step costs one barrier.
constexpr int SBIN_CAP = 2048;  // members of the k-th score's histogram bin (non-exact band)

struct SmallRescore {
  float qP[64 * QP_STRIDE];
  double psum[NWAVES][BW][PSUM_LD];  // head terms of the rescoring waves
};
struct SmallBand {
  double band_s[FBAND_CAP];
  int32_t band_n[SBIN_CAP];
};

struct SmallLds {
  SmallRescore rs;
  union {  // the histogram is dead once the k-th score's bin is known
    uint32_t hist2k[2048];
    SmallBand bd;
  };
  uint32_t bkey[SBIN_CAP];            // keys of the band (non-exact)
  uint32_t chosen[SBIN_CAP / 32];     // band slots selected
  int part[4][NWAVES];                // one per block scan
  uint32_t red_u[6][NWAVES];
  int misc[4];
};

static_assert(sizeof(SmallLds) <= 160 * 1024, "LDS budget of a gfx950 CU");

// the per-wave values red[0..15] reduced across a row of lanes (every lane
// gets the result): min when MIN, else max
template <bool MIN>
__device__ __forceinline__ uint32_t row_reduce16(const uint32_t* red) {
  const uint32_t id = MIN ? ~0u : 0u;
  uint32_t v = red[threadIdx.x & 15];
  v = MIN ? min(v, dpp_u32<0x111>(id, v)) : max(v, dpp_u32<0x111>(id, v));
  v = MIN ? min(v, dpp_u32<0x112>(id, v)) : max(v, dpp_u32<0x112>(id, v));
  v = MIN ? min(v, dpp_u32<0x114>(id, v)) : max(v, dpp_u32<0x114>(id, v));
  v = MIN ? min(v, dpp_u32<0x118>(id, v)) : max(v, dpp_u32<0x118>(id, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
}

// Returns false, having written nothing, when a capacity is exceeded (or the
// hints do not belong to these scores). BF16: the index q and keys are bf16
// (else fp32; unused without exact mode).
template <bool BF16>
__device__ bool small_path(const TopkParams& P, SmallLds& L, int b) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  // every kernel argument this path reads, in SGPRs at once: their scalar
  // loads then go out together instead of one round trip per use
  asm volatile("" ::"s"(P.scores), "s"(P.hints), "s"(P.q), "s"(P.w), "s"(P.ids), "s"(P.mask), "s"(P.N), "s"(P.k),
               "s"(P.exact), "s"(P.H), "s"(P.hints_len), "s"(P.nchunks));
  const int N = P.N, k = P.k;
  const float* sb = P.scores + (size_t)b * N;
  int32_t* ids = P.ids + (size_t)b * k;
  uint8_t* mask = P.mask ? P.mask + (size_t)b * N : nullptr;
  const int e0 = GROUP * tid;
  const int G = (N + GROUP - 1) / GROUP;  // score groups, one maximum each in the hints
  const bool full = e0 + GROUP <= N;

  // 0. every global read up front, the group maximum first (its reduction
  //    runs while the scores are in flight); in exact mode the key-norm
  //    bounds, w and this thread's 8-dim piece of q (head tid/16). Loads go to
  //    clamped addresses and are masked afterwards, and none sits in a branch:
  //    the compiler places a load's wait where the branch joins, which would
  //    hold every load issued after it
  const bool gm_ok = P.hints != nullptr;
  const float* gmp = gm_ok ? P.hints + (size_t)b * P.hints_len + P.nchunks : sb;
  const float gmax = gmp[min(tid, G - 1)];
  f32x4 sv[GROUP / 4];
  if (full && (reinterpret_cast<uintptr_t>(sb) & 15u) == 0) {
    // (plain loads: the scores were just written and sit in L2, which
    // non-temporal loads would pass by)
#pragma unroll
    for (int c = 0; c < GROUP / 4; c++) sv[c] = *(const f32x4*)(sb + e0 + 4 * c);
  } else {
#pragma unroll
    for (int c = 0; c < GROUP / 4; c++)
#pragma unroll
      for (int i = 0; i < 4; i++) sv[c][i] = sb[min(e0 + 4 * c + i, N - 1)];
  }
  const int qh = tid >> 4, d8 = tid & 15;
  float knorm = 0.f, w_h = 0.f;
  u32x4 qraw[2];
  u32x4 qbw = {0u, 0u, 0u, 0u};  // sum_h |w_h| ||q_h|| and sum_h |w_h| (fp64 word pairs) from the hints
  if (P.exact) {
    const int H = P.H;
    knorm = P.hints[(size_t)b * P.hints_len + min(tid, P.nchunks - 1)];
    const uint32_t* qb = reinterpret_cast<const uint32_t*>(P.hints + (size_t)b * P.hints_len + P.hints_len) - LIT_HINT_QBOUND;
#pragma unroll
    for (int i = 0; i < 4; i++) qbw[i] = qb[i];
    w_h = P.w[(size_t)b * H + min(lane, H - 1)];
    const size_t off = ((size_t)b * H + min(qh, H - 1)) * LIT_IDX_DIM + 8 * d8;
    if (BF16) {
      qraw[0] = *(const u32x4*)((const uint16_t*)P.q + off);
    } else {
      qraw[0] = *(const u32x4*)((const float*)P.q + off);
      qraw[1] = *(const u32x4*)((const float*)P.q + off + 4);
    }
  }
  for (int i = tid; i < 2048; i += TK_THREADS) L.hist2k[i] = 0u;
  if (tid < SBIN_CAP / 32) L.chosen[tid] = 0u;
  if (tid == 0) L.misc[3] = 0;

  // 1. largest and smallest group-maximum key; wave 0 (which holds the chunk
  //    bounds: at most 64 chunks here) takes the largest key norm
  {
    const uint32_t gk = score_key(gmax);
    const uint32_t mx_w = wave_max_dpp(tid < G ? gk : 0u), mn_w = wave_min_dpp(tid < G ? gk : ~0u);
    if (lane == 0) {
      L.red_u[0][wid] = mx_w;
      L.red_u[1][wid] = mn_w;
    }
    if (P.exact && wid == 0) {
      const uint32_t kn_w = wave_max_dpp(__float_as_uint(tid < P.nchunks ? knorm : 0.f));  // non-negative floats order as integers
      if (lane == 0) L.red_u[2][0] = kn_w;
    }
  }
  uint32_t kv[GROUP];
  if (full) {
#pragma unroll
    for (int i = 0; i < GROUP; i++) kv[i] = score_key(sv[i / 4][i % 4]);
  } else {
#pragma unroll
    for (int i = 0; i < GROUP; i++) kv[i] = e0 + i < N ? score_key(sv[i / 4][i % 4]) : 0u;
  }
  if (P.exact) {
    // q to LDS for the rescoring: its loads landed with the scores just used,
    // and the barrier below publishes it
    if (lane >= P.H) w_h = 0.f;
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      if (BF16) {
        x[2 * i] = bf16_lo(qraw[0][i]);
        x[2 * i + 1] = bf16_hi(qraw[0][i]);
      } else {
        x[i] = __uint_as_float(qraw[0][i]);
        x[4 + i] = __uint_as_float(qraw[1][i]);
      }
    }
    if (qh >= P.H) {
#pragma unroll
      for (int i = 0; i < 8; i++) x[i] = 0.f;
    }
    *(f32x4*)&L.rs.qP[qh * QP_STRIDE + 8 * d8] = f32x4{x[0], x[1], x[2], x[3]};
    *(f32x4*)&L.rs.qP[qh * QP_STRIDE + 8 * d8 + 4] = f32x4{x[4], x[5], x[6], x[7]};
  }
  lds_barrier();
  uint32_t kmx = row_reduce16<false>(L.red_u[0]);
  const uint32_t glo = row_reduce16<true>(L.red_u[1]);
  const uint32_t kn_u = P.exact ? L.red_u[2][0] : 0u;
  // the group bound holds when every group has a selectable entry and k <= G
  const bool useL = gm_ok && k <= G && glo > 0u;
  uint32_t Lb;
  if (useL) {
    Lb = glo;
  } else {
    // the smallest selectable key (key - 1 taken modulo 2^32, so that the
    // never-selected key 0 comes last) and the largest, from the keys
    uint32_t kx = 0u, kn1 = ~0u;
#pragma unroll
    for (int i = 0; i < GROUP; i++) {
      kx = max(kx, kv[i]);
      kn1 = min(kn1, kv[i] - 1u);
    }
    kx = wave_max_dpp(kx);
    kn1 = wave_min_dpp(kn1);
    if (lane == 0) {
      L.red_u[3][wid] = kx;
      L.red_u[4][wid] = kn1;
    }
    lds_barrier();
    kmx = row_reduce16<false>(L.red_u[3]);
    Lb = row_reduce16<true>(L.red_u[4]) + 1u;  // 0 when nothing is selectable
    Lb = Lb > 1u ? Lb : 1u;
  }
  double delta = 0.0;
  if (P.exact) {
    const double Q = __longlong_as_double((long long)(((uint64_t)qbw[1] << 32) | qbw[0]));
    const double Wa = __longlong_as_double((long long)(((uint64_t)qbw[3] << 32) | qbw[2]));
    // fp32 scores are within delta of their fp64 canonical values
    delta = score_err_bound(BF16, P.H, Q, (double)__uint_as_float(kn_u), Wa);
  }

  // 2. histogram of the keys in Lb .. kmx over the bits below the common
  //    prefix of the two (a key above the hints' largest means hints of other
  //    scores: no histogram then, and the path gives up)
  const uint32_t diff = Lb ^ kmx;
  const int hb = diff ? 31 - __clz((int)diff) : 0;
  const int shift = hb > 10 ? hb - 10 : 0;
  const uint32_t prefix = kmx & ~((2u << hb) - 1u);
  {
    uint32_t kr = kv[0];
#pragma unroll
    for (int i = 1; i < GROUP; i++) kr = max(kr, kv[i]);
    if (kr > kmx) {
      L.misc[3] = 1;
    } else {
#pragma unroll
      for (int i = 0; i < GROUP; i++)
        if (kv[i] >= Lb) atomicAdd(&L.hist2k[(kv[i] - prefix) >> shift], 1u);
    }
  }
  lds_barrier();
  if (L.misc[3]) return false;
  const int c0 = (int)L.hist2k[2047 - 2 * tid], c1 = (int)L.hist2k[2046 - 2 * tid];
  int tot;
  const int ab = block_excl_scan1<NWAVES>(c0 + c1, L.part[0], &tot);
  if (useL && tot < k) return false;  // hints of other scores
  // every histogrammed entry is selected (exact mode with the group bound
  // still ranks: entries below the bound may rank above in fp64)
  const bool all = tot <= k && !(P.exact && useL);
  if (!all) {
    if (ab < k && k <= ab + c0) {
      L.misc[0] = 2047 - 2 * tid;
      L.misc[1] = ab;
    } else if (ab + c0 < k && k <= ab + c0 + c1) {
      L.misc[0] = 2046 - 2 * tid;
      L.misc[1] = ab + c0;
    }
  }
  lds_barrier();

  // 3. above (key > hi_sel) and band (blo <= key <= hi_sel) entries
  uint32_t hi_sel = Lb - 1u, blo = Lb;  // all: every histogrammed key is above, no band
  int r = 0;
  if (!all) {
    // the k-th key's bin holds keys mlo .. blast (the histogrammed ones); r of
    // them are selected
    const uint32_t bin_t = (uint32_t)L.misc[0];
    r = k - L.misc[1];
    const uint32_t binlo = prefix + (bin_t << shift);
    const uint32_t blast = binlo + ((1u << shift) - 1u);
    const uint32_t mlo = max(binlo, Lb);
    hi_sel = blast;
    blo = mlo;
    if (P.exact) {
      // the k-th fp32 key T lies in mlo .. blast and the k-th fp64 score is
      // within delta of T: entries above blast + 2 delta are in, entries below
      // mlo - 2 delta out, and the band between (which holds T - 2 delta ..
      // T + 2 delta and the rest of the bin) is rescored
      const double s_lo = (double)key_score(max(mlo, 0x00800000u));
      const double s_hi = (double)key_score(min(blast, 0xff800000u));
      const uint32_t l0 = score_key(__double2float_rd(s_lo - 2.0 * delta));
      blo = l0 > 1u ? l0 : 1u;
      hi_sel = score_key(__double2float_ru(s_hi + 2.0 * delta));
    }
  }
  uint32_t am = 0u, bm = 0u;
#pragma unroll
  for (int i = 0; i < GROUP; i++) am |= (uint32_t)(kv[i] > hi_sel) << i;
  if (!all) {
    const uint32_t bw = hi_sel - blo;
#pragma unroll
    for (int i = 0; i < GROUP; i++) bm |= (uint32_t)(kv[i] - blo <= bw) << i;
  }
  // exact mode: the key rows of my first two band entries are requested now
  // (a dword from each of their first two 128-byte lines), so that the
  // rescoring finds them in L2 rather than waiting on HBM; the values only
  // feed an empty asm at the end (and so are not waited for before it)
  uint32_t touch[4] = {0u, 0u, 0u, 0u};
  if (P.exact && bm) {
    constexpr int RW = LIT_IDX_DIM * (BF16 ? 2 : 4) / 4;  // dwords per key row
    const uint32_t* kb = reinterpret_cast<const uint32_t*>(P.kidx) + (size_t)(b / P.kq) * N * RW;
    const uint32_t bm2 = bm & (bm - 1u);
    const int ea = e0 + __ffs(bm) - 1, eb = bm2 ? e0 + __ffs(bm2) - 1 : ea;
    touch[0] = kb[(size_t)ea * RW];
    touch[1] = kb[(size_t)ea * RW + 32];
    touch[2] = kb[(size_t)eb * RW];
    touch[3] = kb[(size_t)eb * RW + 32];
  }
  int tab;
  const int pab = block_excl_scan1<NWAVES>((__popc(am) << 16) | __popc(bm), L.part[1], &tab);
  const int A = tab >> 16, M = tab & 0xffff;     // above and band totals
  const int apos = pab >> 16, bpos = pab & 0xffff;  // mine before me
  if (M > (P.exact ? FBAND_CAP : SBIN_CAP)) return false;
  if (bm) {
    int p = bpos;
#pragma unroll
    for (int i = 0; i < GROUP; i++)
      if ((bm >> i) & 1u) {
        L.bd.band_n[p] = e0 + i;
        if (!P.exact) L.bkey[p] = kv[i];
        p++;
      }
  }
  int nsel = 0;  // band entries selected
  if (!all && P.exact) {
    lds_barrier();  // the band list is complete
    nsel = k - A;
    if (nsel < 1 || nsel > M) {
      report_violation(P, b, ids, mask);
      return true;
    }
    // exact scores of the band, BW entries per wave and round (each wave
    // reads its q rows once per round): as many waves as the band needs, a
    // multiple of four (one more per SIMD), at least eight. (One entry per
    // wave over all sixteen waves measured slower here, 15.6 against 14.2 us
    // for bands of ~20: it converts and reads each q value once per entry
    // instead of once per four.)
    const int nwr = min(NWAVES, max(8, ((M + BW - 1) / BW + 3) & ~3));  // 8, 12 or 16 waves
    for (int base = 0; base + wid < M && wid < nwr; base += nwr * BW)
      band_scores_bcast<BF16>(P, b, L.rs.qP, w_h, L.bd.band_n, M, base + wid, nwr, L.rs.psum[wid], L.bd.band_s);
    lds_barrier();
    // the nsel best of the band by (score desc, index asc): the rank of slot i
    // counted by ballots over 64 slots at a time, one wave per slot
    for (int i = wid; i < M; i += NWAVES) {
      const double si = L.bd.band_s[i];
      int rank = 0;
      for (int j0 = 0; j0 < M; j0 += 64) {
        const int j = j0 + lane;
        const double sj = j < M ? L.bd.band_s[j] : 0.0;
        rank += __popcll(__ballot(j < M && (sj > si || (sj == si && j < i))));  // the band is in index order
      }
      if (lane == 0 && rank < nsel) atomicOr(&L.chosen[i >> 5], 1u << (i & 31));
    }
    lds_barrier();
  } else if (!all) {
    lds_barrier();
    // the r best members of the bin by (key desc, index asc), as above
    nsel = r;
    for (int i = wid; i < M; i += NWAVES) {
      const uint32_t ki = L.bkey[i];
      int rank = 0;
      for (int j0 = 0; j0 < M; j0 += 64) {
        const int j = j0 + lane;
        const uint32_t kj = j < M ? L.bkey[j] : 0u;
        rank += __popcll(__ballot(j < M && (kj > ki || (kj == ki && j < i))));
      }
      if (lane == 0 && rank < nsel) atomicOr(&L.chosen[i >> 5], 1u << (i & 31));
    }
    lds_barrier();
  }

  // 4. output in index order: my offset is the above entries before me plus
  //    the chosen band slots before my first one
  uint32_t sm = am;
  int opos = apos;
  if (!all) {
    for (int w = 0; w < (bpos >> 5); w++) opos += __popc(L.chosen[w]);
    if (bpos & 31) opos += __popc(L.chosen[bpos >> 5] & ((1u << (bpos & 31)) - 1u));
    uint32_t rest = bm;
    int p = bpos;
    while (rest) {
      const int i = __ffs(rest) - 1;
      if ((L.chosen[p >> 5] >> (p & 31)) & 1u) sm |= 1u << i;
      p++;
      rest &= rest - 1u;
    }
  }
  {
    uint32_t rest = sm;
    while (rest) {
      const int i = __ffs(rest) - 1;
      if (opos < k) ids[opos] = e0 + i;
      opos++;
      rest &= rest - 1u;
    }
  }
  if (mask && e0 < N) {
    if (full && (reinterpret_cast<uintptr_t>(mask) & 15u) == 0) {
      u32x4 mv;
#pragma unroll
      for (int w = 0; w < 4; w++)
        mv[w] = ((sm >> (4 * w)) & 1u) | (((sm >> (4 * w + 1)) & 1u) << 8) | (((sm >> (4 * w + 2)) & 1u) << 16) |
                (((sm >> (4 * w + 3)) & 1u) << 24);
      *(u32x4*)(mask + e0) = mv;
    } else {
      for (int i = 0; i < GROUP && e0 + i < N; i++) mask[e0 + i] = (sm >> i) & 1u;
    }
  }
  const int total = min(A + nsel, k);
  for (int j = total + tid; j < k; j += TK_THREADS) ids[j] = -1;
  if (tid == 0) P.count[b] = total;
  asm volatile("" ::"v"(touch[0]), "v"(touch[1]), "v"(touch[2]), "v"(touch[3]));
  return true;
}

// ---------------------------------------------------------------- full scan

__device__ void full_path(const TopkParams& P, FullLds& L, int b) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int N = P.N, k = P.k;
  const float* sb = P.scores + (size_t)b * N;
  const bool in_lds = N <= LDS_KEYS;
  int32_t* ids = P.ids + (size_t)b * k;
  uint8_t* mask = P.mask ? P.mask + (size_t)b * N : nullptr;
  double* g_band_s = P.ws_band_s + (size_t)b * N;
  int32_t* g_band_n = P.ws_band_n + (size_t)b * N;
  uint8_t* g_band_sel = P.ws_band_sel + (size_t)b * N;

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
  bool exact_band_on = false;
  if (total_sel > k) {
    const uint32_t T = radix_select<uint32_t>(key, N, k, &L.sc, &r_eq);
    if (!P.exact) {
      def_key = T;
      band_lo = band_hi = T;
    } else {
      exact_band(P, b, T, L.krow, L.dmisc, &band_lo, &band_hi);
      def_key = band_hi;
      exact_band_on = true;
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
  if (exact_band_on) {
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
      report_violation(P, b, ids, mask);
      return;
    }
    __threadfence();
    __syncthreads();
    const bool band_in_lds = M <= BAND_LDS;
    if (band_in_lds)
      for (int i = tid; i < M; i += TK_THREADS) L.band_n[i] = g_band_n[i];
    stage_qT(P, b, L.qT);
    const float w_h = lane < P.H ? P.w[(size_t)b * P.H + lane] : 0.f;
    for (int i = wid; i < M; i += NWAVES) {
      const int n = band_in_lds ? L.band_n[i] : g_band_n[i];
      const double s = rescore(P, b, n, L.qT, L.krow[wid], w_h);
      if (lane == 0) {
        if (band_in_lds)
          L.band_s[i] = s;
        else
          g_band_s[i] = s;
      }
    }
    __threadfence();
    __syncthreads();
    // the band is in index order: position order is index order
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
    __threadfence();
    __syncthreads();
  }

  // ordered compaction: ids ascending, mask, count
  const bool band_in_lds = M <= BAND_LDS;
  auto chosen = [&](int pos) -> bool {
    if (!exact_band_on) return pos < r_eq;
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

// Workgroup -> score row. Rows kq*s .. kq*s + kq-1 belong to sequence s; when
// the sequences are a multiple of 8, every row of sequence s runs on XCD s % 8
// (workgroup id mod 8). The scoring call writes a sequence's rows there when
// one of its units covers all the sequence's queries (one query, or the two of
// a draft step), so the selection finds them in that XCD's L2. With kq = 1 this
// is the identity.
__device__ __forceinline__ int block_row(const TopkParams& P) {
  const int x = blockIdx.x;
  if ((gridDim.x / P.kq) % 8 != 0) return x;
  const int t = x >> 3;
  return ((t / P.kq) * 8 + (x & 7)) * P.kq + t % P.kq;
}

__global__ __launch_bounds__(TK_THREADS) void topk_kernel(TopkParams P) {
  extern __shared__ __align__(16) uint8_t smem[];
  full_path(P, *reinterpret_cast<FullLds*>(smem), block_row(P));
}

// Wide path, kernel A: candidate lists of the slices (grid: rows x slices).
__global__ __launch_bounds__(TK_THREADS) void topk_cand_kernel(TopkParams P) {
  __shared__ WideLds L;
  wide_candidates(P, L);
}

// Wide path, kernel B: one workgroup per row (workgroup b on XCD b % 8, as its
// lists), which scans every score when the row does not fit.
__global__ __launch_bounds__(TK_THREADS) void topk_finish_kernel(TopkParams P) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int b = (int)blockIdx.x;
  if (wide_finish(P, *reinterpret_cast<FastLds*>(smem), b)) return;
  __syncthreads();
  full_path(P, *reinterpret_cast<FullLds*>(smem), b);
}

// The small kernel's fallback, out of line so that its registers do not weigh
// on the small path.
__device__ __noinline__ void full_path_call(TopkParams P, int b) {
  extern __shared__ __align__(16) uint8_t smem[];
  full_path(P, *reinterpret_cast<FullLds*>(smem), b);
}

template <bool BF16>
__global__ __launch_bounds__(TK_THREADS) void topk_small_kernel(TopkParams P) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int b = block_row(P);
  if (small_path<BF16>(P, *reinterpret_cast<SmallLds*>(smem), b)) return;
  __syncthreads();
  full_path_call(P, b);
}

}  // namespace
}  // namespace lit

using namespace lit;

extern "C" size_t lit_topk_workspace_bytes(int32_t B, int32_t N, int32_t k) {
  (void)k;
  if (B < 1 || N < 1) return 0;
  const size_t per = (size_t)B * (size_t)N;
  return round_up(per * sizeof(double), 256) + round_up(per * sizeof(int32_t), 256) + round_up(per, 256) +
         round_up((size_t)B * WIDE_STRIDE * sizeof(int32_t), 256) + round_up(per * sizeof(uint32_t), 256);
}

// B rows of scores; rows kq*s .. kq*s + kq-1 share the keys of sequence s.
static lit_status topk_rows(const float* scores, int32_t B, int32_t kq, int32_t N, int32_t k, const lit_idx_in* exact,
                            const float* hints, int32_t* ids, int32_t* count, uint8_t* mask, void* ws,
                            size_t ws_bytes, void* stream, const char* who) {
  if (!scores || !ids || !count) return fail(LIT_ERR_NULL, "%s: scores, ids and count must be non-NULL", who);
  if (B < 1 || N < 1 || k < 1) return fail(LIT_ERR_SHAPE, "%s: rows=%d N=%d k=%d must be >= 1", who, B, N, k);
  if (B > (1 << 30) / 2) return fail(LIT_ERR_SHAPE, "%s: %d rows above 2^29", who, B);
  if (N > (1 << 24)) return fail(LIT_ERR_SHAPE, "%s: N=%d above 2^24", who, N);
  if (!aligned(scores, 4) || !aligned(ids, 4) || !aligned(count, 4) || (hints && !aligned(hints, 4)))
    return fail(LIT_ERR_ALIGN, "%s: scores, hints, ids and count must be 4-byte aligned", who);
  if (exact) {
    lit_status st = check_idx_inputs(exact, B / kq, N, who);
    if (st != LIT_OK) return st;
    if (!hints) return fail(LIT_ERR_NULL, "%s: exact mode needs the hints side output of the scoring call", who);
  }
  const size_t need = lit_topk_workspace_bytes(B, N, k);
  if (!ws || ws_bytes < need)
    return fail(LIT_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", who, ws_bytes, need);
  if (!aligned(ws, 256)) return fail(LIT_ERR_ALIGN, "%s: workspace must be 256-byte aligned", who);
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
  P.kq = kq;
  P.dtype = exact ? (int)exact->dtype : 0;
  P.H = exact ? exact->H : 0;
  P.hints = hints;
  P.hints_len = lit_idx_hints_len(N);
  P.nchunks = (int)cdiv(N, LIT_KNORM_CHUNK);
  P.ids = ids;
  P.count = count;
  P.mask = mask;
  P.ws_band_s = (double*)w8;
  P.ws_band_n = (int32_t*)(w8 + round_up(per * sizeof(double), 256));
  P.ws_band_sel = w8 + round_up(per * sizeof(double), 256) + round_up(per * sizeof(int32_t), 256);
  P.ws_wide = (int32_t*)(w8 + round_up(per * sizeof(double), 256) + round_up(per * sizeof(int32_t), 256) +
                         round_up(per, 256));
  P.ws_ckey = (uint32_t*)((uint8_t*)P.ws_wide + round_up((size_t)B * WIDE_STRIDE * sizeof(int32_t), 256));
  P.rows = B;
  P.wide_slices = 1;
  if (N <= TK_THREADS * GROUP) {
    const size_t lds = std::max(sizeof(FullLds), sizeof(SmallLds));
    const bool bf16 = P.exact && P.dtype == LIT_BF16;
    const void* kern = bf16 ? (const void*)topk_small_kernel<true> : (const void*)topk_small_kernel<false>;
    lit_status st = allow_lds(kern, lds, who);
    if (st != LIT_OK) return st;
    if (bf16)
      topk_small_kernel<true><<<dim3((unsigned)B), dim3(TK_THREADS), lds, (hipStream_t)stream>>>(P);
    else
      topk_small_kernel<false><<<dim3((unsigned)B), dim3(TK_THREADS), lds, (hipStream_t)stream>>>(P);
    LIT_CHECK_LAUNCH(who);
    return LIT_OK;
  }
  const size_t lds = std::max(sizeof(FullLds), sizeof(FastLds));
  hipStream_t hs = (hipStream_t)stream;
  if (hints && N <= GM_CAP * GROUP) {
    // wide path: about 512 candidate workgroups in all, at least enough
    // slices that one slice's groups fit one workgroup
    const int G = (int)cdiv(N, GROUP);
    const int s_min = (int)cdiv(G, TK_THREADS);
    P.wide_slices = std::min(WIDE_SLICES_MAX, std::max(s_min, (int)cdiv(512, B)));
    const int64_t ga = (int64_t)B * P.wide_slices;
    if (ga > INT32_MAX) return fail(LIT_ERR_SHAPE, "%s: %d rows too many for the candidate grid", who, B);
    lit_status st = allow_lds((const void*)topk_finish_kernel, lds, who);
    if (st != LIT_OK) return st;
    topk_cand_kernel<<<dim3((unsigned)ga), dim3(TK_THREADS), 0, hs>>>(P);
    LIT_CHECK_LAUNCH(who);
    topk_finish_kernel<<<dim3((unsigned)B), dim3(TK_THREADS), lds, hs>>>(P);
    LIT_CHECK_LAUNCH(who);
    return LIT_OK;
  }
  lit_status st = allow_lds((const void*)topk_kernel, sizeof(FullLds), who);
  if (st != LIT_OK) return st;
  topk_kernel<<<dim3((unsigned)B), dim3(TK_THREADS), sizeof(FullLds), hs>>>(P);
  LIT_CHECK_LAUNCH(who);
  return LIT_OK;
}

extern "C" lit_status lit_topk_select(const float* scores, int32_t B, int32_t N, int32_t k, const lit_idx_in* exact,
                                      const float* hints, int32_t* ids, int32_t* count, uint8_t* mask, void* ws,
                                      size_t ws_bytes, void* stream) {
  clear_error();
  return topk_rows(scores, B, 1, N, k, exact, hints, ids, count, mask, ws, ws_bytes, stream, "lit_topk_select");
}

extern "C" lit_status lit_topk_select_mq(const float* scores, int32_t B, int32_t Q, int32_t N, int32_t k,
                                         const lit_idx_in* exact, const float* hints, int32_t* ids, int32_t* count,
                                         uint8_t* mask, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  if (Q < 1 || Q > LIT_MAX_QUERIES || B < 1)
    return fail(LIT_ERR_SHAPE, "lit_topk_select_mq: B=%d, Q=%d (1..%d)", B, Q, LIT_MAX_QUERIES);
  if ((int64_t)B * Q > (1 << 29)) return fail(LIT_ERR_SHAPE, "lit_topk_select_mq: B x Q above 2^29");
  return topk_rows(scores, B * Q, Q, N, k, exact, hints, ids, count, mask, ws, ws_bytes, stream,
                   "lit_topk_select_mq");
}
