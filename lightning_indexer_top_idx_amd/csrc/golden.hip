// golden.hip - a6: dense "golden" attention top-k; a9: top-p per layer + vote.
//
// a6, ai-muninn.com, "FlashMemory can't improve DeepSeek-V4-Flash's own lightning indexer",
// section "Act 3": the ground truth a selector is scored against is the dense
// attention, an unmasked softmax over every chunk; its top-k is the golden set.
// The head-averaged form (average the per-head probabilities) is how the tiny
// workload states it. Everything is fp64: the logits are canonical sums (exact
// products, d ascending), so they are bit-identical to a sequential CPU sum; the
// softmax denominators are parallel tree sums.
//
// a9, zhichai.net, "FlashMemory-DeepSeek-V4 深度解读", section 3.2: labels come from a
// softmax of each layer's indexer logits, a top-p cut at p = 0.6 (the smallest
// set of entries whose cumulative probability reaches p), and a vote that keeps
// entries chosen by at least 3 of the 21 CSA layers. The running sum is added
// sequentially in sorted order (probability descending, index ascending), so the
// cut matches a sequential CPU walk.
#include <algorithm>
#include <math.h>

#include "lit_common.h"
#include "select.h"

namespace lit {
namespace {

// The KV arrays of a call (data, rope, scale rows), passed by value to kernels.
struct KvRows {
  KvArr d, r, s;
};

// pbar[b][n] = (sum_h exp(X - m_h) / Z_h) / Hq, h ascending.
__global__ __launch_bounds__(256) void golden_pbar_kernel(const double* __restrict__ X, const double* __restrict__ stats,
                                                          int Hq, int N, double* __restrict__ pbar) {
  const int b = blockIdx.y, n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  double acc = 0.0;
  for (int h = 0; h < Hq; h++) {
    const size_t bh = (size_t)b * Hq + h;
    acc += exp(X[bh * N + n] - stats[2 * bh]) / stats[2 * bh + 1];
  }
  pbar[(size_t)b * N + n] = acc / (double)Hq;
}

// Top-k of one sequence's fp64 values (value desc, index asc).
__global__ __launch_bounds__(1024) void topk_f64_kernel(const double* __restrict__ v, int N, int k, uint8_t* sel_ws,
                                                        int32_t* ids, int32_t* count, uint8_t* mask) {
  __shared__ SelectScratch sc;
  const int b = blockIdx.x;
  const double* vb = v + (size_t)b * N;
  uint8_t* sel = sel_ws + (size_t)b * N;
  auto key = [&](int i) -> uint64_t { return score_key64(vb[i]); };
  int nsel = 0;
  for (int i = threadIdx.x; i < N; i += blockDim.x) nsel += key(i) != 0ull;
  int total;
  block_excl_scan(nsel, sc.scan, &total);
  if (total <= k) {
    const int seg = (N + blockDim.x - 1) / blockDim.x;
    const int a = min(N, (int)threadIdx.x * seg), e = min(N, a + seg);
    for (int i = a; i < e; i++) sel[i] = key(i) != 0ull;
  } else {
    int r_eq;
    const uint64_t T = radix_select<uint64_t>(key, N, k, &sc, &r_eq);
    mark_top<uint64_t>(key, N, T, r_eq, sel, &sc);
  }
  emit_selection(sel, N, k, ids + (size_t)b * k, count + b, mask ? mask + (size_t)b * N : nullptr, &sc);
}

// ---- top-p + vote --------------------------------------------------------------

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* p, size_t n, int32_t v) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = v;
}

// One workgroup per (layer, sequence): probabilities, sort, sequential cut, votes.
__global__ __launch_bounds__(1024) void topp_kernel(const double* __restrict__ x, int is_logits, int B, int N,
                                                    int Np2, double top_p, double* __restrict__ prob_ws,
                                                    uint64_t* __restrict__ key_ws, int32_t* __restrict__ idx_ws,
                                                    int32_t* __restrict__ votes) {
  __shared__ double red[16];
  __shared__ double dshare[2];
  __shared__ double pchunk[1024];
  __shared__ int ishare[2];
  const int lb = blockIdx.x, b = lb % B;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const double* xr = x + (size_t)lb * N;
  double* pr = prob_ws + (size_t)lb * N;
  uint64_t* kr = key_ws + (size_t)lb * Np2;
  int32_t* ir = idx_ws + (size_t)lb * Np2;
  // probabilities
  if (is_logits) {
    double m = -INFINITY;
    for (int n = tid; n < N; n += 1024) m = fmax(m, xr[n]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmax(m, __shfl_xor(m, o));
    if (lane == 0) red[wid] = m;
    __syncthreads();
    if (tid == 0) {
      double mm = red[0];
      for (int i = 1; i < 16; i++) mm = fmax(mm, red[i]);
      dshare[0] = mm;
    }
    __syncthreads();
    m = dshare[0];
    for (int n = tid; n < N; n += 1024) pr[n] = exp(xr[n] - m);
    __threadfence();
    __syncthreads();
    if (tid == 0) {  // Z in index order, as a sequential CPU sum would add it
      double z = 0.0;
      for (int n = 0; n < N; n++) z += pr[n];
      dshare[1] = z;
    }
    __syncthreads();
    const double z = dshare[1];
    for (int n = tid; n < N; n += 1024) pr[n] = pr[n] / z;
  } else {
    for (int n = tid; n < N; n += 1024) pr[n] = xr[n];
  }
  __threadfence();
  __syncthreads();
  // sort ascending by (inverted key, index) == probability descending, index ascending
  for (int i = tid; i < Np2; i += 1024) {
    if (i < N) {
      kr[i] = ~score_key64(pr[i]);
      ir[i] = i;
    } else {
      kr[i] = ~0ull;
      ir[i] = 0x7fffffff;
    }
  }
  __threadfence();
  __syncthreads();
  for (int k2 = 2; k2 <= Np2; k2 <<= 1) {
    for (int j = k2 >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < Np2; i += 1024) {
        const int p = i ^ j;
        if (p > i) {
          const uint64_t ka = kr[i], kb = kr[p];
          const int ia = ir[i], ib = ir[p];
          const bool a_gt_b = (ka > kb) || (ka == kb && ia > ib);
          const bool up = (i & k2) == 0;
          if (a_gt_b == up) {
            kr[i] = kb;
            kr[p] = ka;
            ir[i] = ib;
            ir[p] = ia;
          }
        }
      }
      __threadfence();
      __syncthreads();
    }
  }
  // sequential cut: running sum in sorted order until it reaches top_p
  if (tid == 0) {
    ishare[0] = N;
    dshare[0] = 0.0;
  }
  __syncthreads();
  for (int c0 = 0; c0 < N; c0 += 1024) {
    if (c0 + tid < N) pchunk[tid] = pr[ir[c0 + tid]];
    __syncthreads();
    if (tid == 0 && ishare[0] == N) {
      double run = dshare[0];
      const int len = min(1024, N - c0);
      for (int i = 0; i < len; i++) {
        run += pchunk[i];
        if (run >= top_p) {
          ishare[0] = c0 + i + 1;
          break;
        }
      }
      dshare[0] = run;
    }
    __syncthreads();
    if (ishare[0] != N) break;
  }
  const int cut = ishare[0];
  int32_t* vb = votes + (size_t)b * N;
  for (int i = tid; i < cut; i += 1024) atomicAdd(&vb[ir[i]], 1);
}

__global__ __launch_bounds__(256) void vote_kernel(const int32_t* __restrict__ votes, int N, int min_votes,
                                                   uint8_t* __restrict__ gold, int32_t* __restrict__ gold_count,
                                                   int32_t* __restrict__ votes_out) {
  __shared__ int red[4];
  const int b = blockIdx.x, tid = threadIdx.x;
  int c = 0;
  for (int n = tid; n < N; n += 256) {
    const int v = votes[(size_t)b * N + n];
    const uint8_t gsel = v >= min_votes;
    gold[(size_t)b * N + n] = gsel;
    c += gsel;
    if (votes_out) votes_out[(size_t)b * N + n] = v;
  }
  c = wave_sum(c);
  if ((tid & 63) == 0) red[tid >> 6] = c;
  __syncthreads();
  if (tid == 0) gold_count[b] = red[0] + red[1] + red[2] + red[3];
}

// ---- lookahead golden ------------------------------------------------------------
//
// Logits of T queries x Hq heads against every row of a sequence: a [T*Hq x 512]
// x [512 x N] product, computed on the fp64 matrix cores (v_mfma_f64_16x16x4f64:
// lane l holds A[l%16][l/16] and B[l/16][l%16] of a 16x4 / 4x16 step, and its
// result register r holds D[l/16 + 4r][l%16] -- rows interleaved by four,
// unlike the fp32 16x16 forms, as measured on gfx950). Products of the bf16 / fp32 / decoded FP8
// inputs are exact in fp64, so the logits differ from a sequential fp64 sum only
// by the order of the fp64 additions. A workgroup computes a 64 x 64 tile (four
// waves of 32 x 32, i.e. 2 x 2 blocks of 16 x 16), staging 32 dims of both
// operands in LDS at a time, converted to fp64 once.
typedef double f64x4 __attribute__((__vector_size__(4 * sizeof(double))));
constexpr int LA_TILE = 64;
constexpr int LA_KC = 32;

// Raw bits of 8 consecutive dims of one row (one thread's share of a stage):
// fp32 in two 16-byte words, bf16 in one, FP8 bytes in the first half of one
// (RoPE dims as bf16), and the row's E8M0 scale byte of those dims.
struct Raw8 {
  u32x4 w[2];
  uint32_t sb;
};

__device__ __forceinline__ Raw8 load_q8(int q_dtype, const void* q, size_t off, bool live) {
  Raw8 r{};
  if (live) {
    if (q_dtype == LIT_F32) {
      r.w[0] = *(const u32x4*)((const float*)q + off);
      r.w[1] = *(const u32x4*)((const float*)q + off + 4);
    } else {
      r.w[0] = *(const u32x4*)((const uint16_t*)q + off);
    }
  }
  return r;
}

__device__ __forceinline__ Raw8 load_kv8(int kv_dtype, const KvRows& kv, int b, int n, int d, bool live) {
  Raw8 r{};
  if (!live) return r;
  if (kv_dtype == LIT_F32) {
    const float* row = (const float*)kv.d.at(b, n);
    r.w[0] = *(const u32x4*)(row + d);
    r.w[1] = *(const u32x4*)(row + d + 4);
  } else if (kv_dtype == LIT_BF16) {
    r.w[0] = *(const u32x4*)((const uint16_t*)kv.d.at(b, n) + d);
  } else if (d >= LIT_KV_FP8_DIMS) {
    r.w[0] = *(const u32x4*)((const uint16_t*)kv.r.at(b, n) + d - LIT_KV_FP8_DIMS);
  } else {
    const u32x2 v = *(const u32x2*)(kv.d.at(b, n) + d);
    r.w[0][0] = v[0];
    r.w[0][1] = v[1];
    r.sb = kv.s.at(b, n)[d / LIT_KV_FP8_GROUP];
  }
  return r;
}

// OCP E4M3FN byte and E8M0 scale byte to fp32 (the format's definition: E4M3FN with
// 0x7F / 0xFF NaN, E8M0 2^(byte-127) with 255 NaN).
__device__ __forceinline__ float fp8_e4m3_f32(uint32_t byte) {
  const uint32_t e = (byte >> 3) & 15u, m = byte & 7u;
  float v;
  if (e == 15u && m == 7u)
    v = __uint_as_float(0x7fc00000u);
  else if (e == 0u)
    v = (float)m * 0x1p-9f;
  else
    v = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return __uint_as_float(__float_as_uint(v) | ((byte & 0x80u) << 24));
}

__device__ __forceinline__ float e8m0_f32(uint32_t sb) {
  return sb == 255u ? __uint_as_float(0x7fc00000u) : (sb == 0u ? 0x1p-127f : __uint_as_float(sb << 23));
}

// The 8 values of a Raw8 as fp64 (the value the fp32 decode gives, widened).
__device__ __forceinline__ void widen8(int dtype, bool fp8_part, const Raw8& r, double (&x)[8]) {
  if (dtype == LIT_F32) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      x[i] = (double)__uint_as_float(r.w[0][i]);
      x[4 + i] = (double)__uint_as_float(r.w[1][i]);
    }
  } else if (!fp8_part) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      x[2 * i] = (double)bf16_lo(r.w[0][i]);
      x[2 * i + 1] = (double)bf16_hi(r.w[0][i]);
    }
  } else {
    const float sc = e8m0_f32(r.sb);
#pragma unroll
    for (int i = 0; i < 8; i++) x[i] = (double)(fp8_e4m3_f32((r.w[0][i >> 2] >> (8 * (i & 3))) & 255u) * sc);
  }
}

// part (when given): for every row and 32-entry block of the row, the block's
// maximum logit m and sum of exp(x - m), so that the softmax statistics need
// no further pass over the logits.
__global__ __launch_bounds__(256) void lookahead_logits_kernel(const void* q, int q_dtype, int M, int kv_dtype,
                                                               KvRows kv, int N, double sc, double* __restrict__ X,
                                                               double* __restrict__ part) {
  __shared__ double As[LA_KC][LA_TILE + 1];  // [dim][row]
  __shared__ double Bs[LA_KC][LA_TILE + 1];  // [dim][entry]
  const int b = blockIdx.z, m0 = blockIdx.y * LA_TILE, n0 = blockIdx.x * LA_TILE;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = (wid >> 1) * 32, wn = (wid & 1) * 32;
  const int r16 = lane & 15, k4 = lane >> 4;
  // staging: thread tid takes dims d0 .. d0+7 of row rr of both operands
  const int rr = tid >> 2, d0 = (tid & 3) * 8;
  const int m = m0 + rr, n = n0 + rr;
  const size_t qoff = ((size_t)b * M + m) * LIT_KV_DIM + d0;
  const bool fp8 = kv_dtype == LIT_FP8E4M3_G64_ROPE_BF16;
  f64x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
  // the next stage's raw operands are loaded while this stage multiplies
  Raw8 ra = load_q8(q_dtype, q, qoff, m < M);
  Raw8 rb = load_kv8(kv_dtype, kv, b, n, d0, n < N);
  for (int k0 = 0; k0 < LIT_KV_DIM; k0 += LA_KC) {
    double xa[8], xb[8];
    widen8(q_dtype, false, ra, xa);
    widen8(kv_dtype, fp8 && k0 + d0 < LIT_KV_FP8_DIMS, rb, xb);
    __syncthreads();  // the previous stage's reads are done
#pragma unroll
    for (int i = 0; i < 8; i++) {
      As[d0 + i][rr] = xa[i];
      Bs[d0 + i][rr] = xb[i];
    }
    __syncthreads();
    if (k0 + LA_KC < LIT_KV_DIM) {
      ra = load_q8(q_dtype, q, qoff + k0 + LA_KC, m < M);
      rb = load_kv8(kv_dtype, kv, b, n, k0 + LA_KC + d0, n < N);
    }
#pragma unroll
    for (int kk = 0; kk < LA_KC; kk += 4) {
      double a[2], bb[2];
#pragma unroll
      for (int i = 0; i < 2; i++) a[i] = As[kk + k4][wm + 16 * i + r16];
#pragma unroll
      for (int j = 0; j < 2; j++) bb[j] = Bs[kk + k4][wn + 16 * j + r16];
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], bb[j], acc[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int nn = n0 + wn + 16 * j + r16;
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int mm = m0 + wm + 16 * i + k4 + 4 * r;
        if (mm < M && nn < N) X[((size_t)b * M + mm) * N + nn] = sc * acc[i][j][r];
      }
    }
  if (part) {
    // this wave holds 32 entries (j, r16) of each of its rows: the sixteen
    // lanes of a row group (same k4) reduce them
    const int nb = (N + 31) / 32, blk = (n0 + wn) / 32;
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int mm = m0 + wm + 16 * i + k4 + 4 * r;
        const int nn0 = n0 + wn + r16, nn1 = nn0 + 16;
        const double v0 = nn0 < N ? sc * acc[i][0][r] : -INFINITY;
        const double v1 = nn1 < N ? sc * acc[i][1][r] : -INFINITY;
        double mx = fmax(v0, v1);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) mx = fmax(mx, __shfl_xor(mx, o));
        double sm = mx == -INFINITY ? 0.0 : exp(v0 - mx) + exp(v1 - mx);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) sm += __shfl_xor(sm, o);
        if (r16 == 0 && mm < M && blk < nb) {
          double* pp = part + (((size_t)b * M + mm) * nb + blk) * 2;
          pp[0] = mx;
          pp[1] = sm;
        }
      }
  }
}

// Softmax statistics of each row from its blocks' (maximum, sum): one wave per
// row, m = the largest block maximum, Z = sum of the blocks' sums scaled by
// exp(m_block - m).
__global__ __launch_bounds__(256) void golden_stats_parts_kernel(const double* __restrict__ part, int nb, int rows,
                                                                 double* __restrict__ stats) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (row >= rows) return;  // (the whole wave)
  const double* p = part + (size_t)row * nb * 2;
  double m = -INFINITY;
  for (int i = lane; i < nb; i += 64) m = fmax(m, p[2 * i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmax(m, __shfl_xor(m, o));
  double z = 0.0;
  for (int i = lane; i < nb; i += 64) {
    const double mi = p[2 * i];
    if (mi != -INFINITY) z += p[2 * i + 1] * exp(mi - m);
  }
  z = wave_sum_f64(z);
  if (lane == 0) {
    stats[2 * row] = m;
    stats[2 * row + 1] = z;
  }
}

// hits[b][n] = number of the T steps whose golden set holds n (t ascending);
// umask = hits > 0. One thread per entry.
__global__ __launch_bounds__(256) void lookahead_union_kernel(const uint8_t* __restrict__ step_mask, int T, int N,
                                                              int32_t* __restrict__ hits, uint8_t* __restrict__ umask) {
  const int b = blockIdx.y, n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  int h = 0;
  for (int t = 0; t < T; t++) h += step_mask[((size_t)b * T + t) * N + n];
  if (hits) hits[(size_t)b * N + n] = h;
  umask[(size_t)b * N + n] = h > 0;
}

// ucount[b] = number of set bytes of umask[b].
__global__ __launch_bounds__(256) void count_u8_kernel(const uint8_t* __restrict__ umask, int N,
                                                       int32_t* __restrict__ ucount) {
  __shared__ int red[4];
  const int b = blockIdx.x, tid = threadIdx.x;
  int c = 0;
  for (int n = tid; n < N; n += 256) c += umask[(size_t)b * N + n] != 0;
  c = wave_sum(c);
  if ((tid & 63) == 0) red[tid >> 6] = c;
  __syncthreads();
  if (tid == 0) ucount[b] = red[0] + red[1] + red[2] + red[3];
}

struct GoldenWs {
  double* X;
  double* part;  // per row and 32-entry block: maximum logit and its sum of exponentials
  double* stats;
  double* pbar;
  uint8_t* sel;
  size_t bytes;
};

// Byte `off` of a workspace, or NULL when only its size is being measured
// (base NULL: no pointer is formed from it).
uint8_t* ws_at(void* base, size_t off) { return base ? (uint8_t*)base + off : nullptr; }

GoldenWs golden_ws(void* base, int B, int Hq, int N) {
  GoldenWs w;
  size_t off = 0;
  w.X = (double*)ws_at(base, off);
  off += round_up((size_t)B * Hq * N * sizeof(double), 256);
  w.part = (double*)ws_at(base, off);
  off += round_up((size_t)B * Hq * ((N + 31) / 32) * 2 * sizeof(double), 256);
  w.stats = (double*)ws_at(base, off);
  off += round_up((size_t)B * Hq * 2 * sizeof(double), 256);
  w.pbar = (double*)ws_at(base, off);
  off += round_up((size_t)B * N * sizeof(double), 256);
  w.sel = ws_at(base, off);
  off += round_up((size_t)B * N, 256);
  w.bytes = off;
  return w;
}

int next_pow2(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

}  // namespace
}  // namespace lit

using namespace lit;

extern "C" size_t lit_golden_workspace_bytes(int32_t B, int32_t Hq, int32_t N, int32_t k) {
  (void)k;
  if (B < 1 || Hq < 1 || N < 1) return 0;
  return golden_ws(nullptr, B, Hq, N).bytes;
}

extern "C" lit_status lit_golden_topk(const void* q, lit_dtype q_dtype, int32_t Hq, const lit_kv* kv, int32_t B,
                                      float scale, int32_t k, int32_t* ids, int32_t* count, uint8_t* mask,
                                      double* pbar, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  const char* who = "lit_golden_topk";
  if (!q || !kv || !kv->data || !ids || !count) return fail(LIT_ERR_NULL, "%s: q, kv, ids and count are required", who);
  if (B < 1 || Hq < 1 || Hq > LIT_MAX_Q_HEADS || kv->n_rows < 1 || k < 1)
    return fail(LIT_ERR_SHAPE, "%s: B=%d Hq=%d N=%d k=%d", who, B, Hq, kv->n_rows, k);
  if (kv->dtype == LIT_F32 ? q_dtype != LIT_F32 : q_dtype != LIT_BF16)
    return fail(LIT_ERR_DTYPE, "%s: query dtype %d does not match rows dtype %d", who, (int)q_dtype, (int)kv->dtype);
  if (kv->dtype != LIT_F32 && kv->dtype != LIT_BF16 && kv->dtype != LIT_FP8E4M3_G64_ROPE_BF16)
    return fail(LIT_ERR_DTYPE, "%s: kv dtype %d unsupported", who, (int)kv->dtype);
  if (kv->dtype == LIT_FP8E4M3_G64_ROPE_BF16 && (!kv->rope || !kv->scale))
    return fail(LIT_ERR_NULL, "%s: FP8 rows need rope and scale arrays", who);
  if (!aligned(q, 16) || !aligned(kv->data, kv->dtype == LIT_FP8E4M3_G64_ROPE_BF16 ? 8 : 16) ||
      (kv->rope && !aligned(kv->rope, 16)))
    return fail(LIT_ERR_ALIGN, "%s: q and the rows must be 16-byte aligned (FP8 row bytes 8-byte)", who);
  KvRows kvr;
  const lit_status kst = kv_arrays(kv, &kvr.d, &kvr.r, &kvr.s, who);
  if (kst != LIT_OK) return kst;
  const int N = kv->n_rows;
  GoldenWs W = golden_ws(ws, B, Hq, N);
  if (!ws || ws_bytes < W.bytes)
    return fail(LIT_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", who, ws_bytes, W.bytes);
  if (!aligned(ws, 256) || (pbar && !aligned(pbar, 8)))
    return fail(LIT_ERR_ALIGN, "%s: workspace must be 256-byte aligned, pbar 8-byte aligned", who);
  hipStream_t st = (hipStream_t)stream;
  double* pb = pbar ? pbar : W.pbar;
  // the logits on the fp64 matrix cores (the one-step case of the lookahead's
  // kernel: Hq query rows per sequence), the softmax statistics from its blocks
  dim3 g1((unsigned)cdiv(N, LA_TILE), (unsigned)cdiv(Hq, LA_TILE), (unsigned)B);
  lookahead_logits_kernel<<<g1, 256, 0, st>>>(q, (int)q_dtype, Hq, (int)kv->dtype, kvr, N, (double)scale, W.X, W.part);
  LIT_CHECK_LAUNCH(who);
  golden_stats_parts_kernel<<<dim3((unsigned)cdiv(B * Hq, 4)), 256, 0, st>>>(W.part, (N + 31) / 32, B * Hq, W.stats);
  LIT_CHECK_LAUNCH(who);
  golden_pbar_kernel<<<dim3((unsigned)cdiv(N, 256), (unsigned)B), 256, 0, st>>>(W.X, W.stats, Hq, N, pb);
  LIT_CHECK_LAUNCH(who);
  topk_f64_kernel<<<dim3((unsigned)B), 1024, 0, st>>>(pb, N, k, W.sel, ids, count, mask);
  LIT_CHECK_LAUNCH(who);
  return LIT_OK;
}

extern "C" size_t lit_topp_workspace_bytes(int32_t L, int32_t B, int32_t N) {
  if (L < 1 || B < 1 || N < 1) return 0;
  const size_t rows = (size_t)L * B;
  const size_t np2 = (size_t)next_pow2(N);
  return round_up(rows * N * sizeof(double), 256) + round_up(rows * np2 * sizeof(uint64_t), 256) +
         round_up(rows * np2 * sizeof(int32_t), 256) + round_up((size_t)B * N * sizeof(int32_t), 256);
}

extern "C" lit_status lit_golden_topp_vote(const double* x, int32_t is_logits, int32_t L, int32_t B, int32_t N,
                                           double top_p, int32_t min_votes, uint8_t* gold, int32_t* gold_count,
                                           int32_t* votes, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  const char* who = "lit_golden_topp_vote";
  if (!x || !gold || !gold_count) return fail(LIT_ERR_NULL, "%s: x, gold and gold_count are required", who);
  if (L < 1 || B < 1 || N < 1 || N > (1 << 24)) return fail(LIT_ERR_SHAPE, "%s: L=%d B=%d N=%d", who, L, B, N);
  if (!(top_p > 0.0 && top_p <= 1.0)) return fail(LIT_ERR_SHAPE, "%s: top_p=%g outside (0,1]", who, top_p);
  const size_t need = lit_topp_workspace_bytes(L, B, N);
  if (!ws || ws_bytes < need)
    return fail(LIT_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", who, ws_bytes, need);
  if (!aligned(ws, 256) || !aligned(x, 8)) return fail(LIT_ERR_ALIGN, "%s: misaligned x or workspace", who);
  const size_t rows = (size_t)L * B;
  const int np2 = next_pow2(N);
  uint8_t* p = (uint8_t*)ws;
  double* prob = (double*)p;
  p += round_up(rows * N * sizeof(double), 256);
  uint64_t* keys = (uint64_t*)p;
  p += round_up(rows * np2 * sizeof(uint64_t), 256);
  int32_t* idx = (int32_t*)p;
  p += round_up(rows * np2 * sizeof(int32_t), 256);
  int32_t* vacc = (int32_t*)p;
  hipStream_t st = (hipStream_t)stream;
  const size_t nv = (size_t)B * N;
  fill_i32_kernel<<<dim3((unsigned)std::min<size_t>(cdiv(nv, 256), 4096)), 256, 0, st>>>(vacc, nv, 0);
  LIT_CHECK_LAUNCH(who);
  topp_kernel<<<dim3((unsigned)rows), 1024, 0, st>>>(x, is_logits, B, N, np2, top_p, prob, keys, idx, vacc);
  LIT_CHECK_LAUNCH(who);
  vote_kernel<<<dim3((unsigned)B), 256, 0, st>>>(vacc, N, min_votes, gold, gold_count, votes);
  LIT_CHECK_LAUNCH(who);
  return LIT_OK;
}

// ---- lookahead golden --------------------------------------------------------------

namespace {
struct LookaheadWs {
  GoldenWs g;  // logits / statistics / pbar / selection scratch of the B*T (sequence, step) rows
  int32_t* ids;
  int32_t* cnt;
  uint8_t* mask;
  uint8_t* umask;
  size_t bytes;
};

LookaheadWs lookahead_ws(void* base, int B, int T, int Hq, int N, int k) {
  LookaheadWs w;
  w.g = golden_ws(base, B * T, Hq, N);
  size_t off = w.g.bytes;
  w.ids = (int32_t*)ws_at(base, off);
  off += round_up((size_t)B * T * k * sizeof(int32_t), 256);
  w.cnt = (int32_t*)ws_at(base, off);
  off += round_up((size_t)B * T * sizeof(int32_t), 256);
  w.mask = ws_at(base, off);
  off += round_up((size_t)B * T * N, 256);
  w.umask = ws_at(base, off);
  off += round_up((size_t)B * N, 256);
  w.bytes = off;
  return w;
}
}  // namespace

extern "C" size_t lit_lookahead_workspace_bytes(int32_t B, int32_t T, int32_t Hq, int32_t N, int32_t k) {
  if (B < 1 || T < 1 || Hq < 1 || N < 1 || k < 1) return 0;
  return lookahead_ws(nullptr, B, T, Hq, N, k).bytes;
}

extern "C" lit_status lit_lookahead_golden(const void* q, lit_dtype q_dtype, int32_t T, int32_t Hq, const lit_kv* kv,
                                           int32_t B, float scale, int32_t k, int32_t* step_ids, int32_t* hits,
                                           uint8_t* union_mask, int32_t* union_count, double* pbar, void* ws,
                                           size_t ws_bytes, void* stream) {
  clear_error();
  const char* who = "lit_lookahead_golden";
  if (!q || !kv || !kv->data || !union_count)
    return fail(LIT_ERR_NULL, "%s: q, kv and union_count are required", who);
  if (B < 1 || T < 1 || T > LIT_MAX_HORIZON || Hq < 1 || Hq > LIT_MAX_Q_HEADS || kv->n_rows < 1 || k < 1)
    return fail(LIT_ERR_SHAPE, "%s: B=%d T=%d (1..%d) Hq=%d N=%d k=%d", who, B, T, LIT_MAX_HORIZON, Hq, kv->n_rows, k);
  if ((int64_t)B * T > 65535) return fail(LIT_ERR_SHAPE, "%s: B x T = %lld above 65535", who, (long long)B * T);
  if (kv->dtype == LIT_F32 ? q_dtype != LIT_F32 : q_dtype != LIT_BF16)
    return fail(LIT_ERR_DTYPE, "%s: query dtype %d does not match rows dtype %d", who, (int)q_dtype, (int)kv->dtype);
  if (kv->dtype != LIT_F32 && kv->dtype != LIT_BF16 && kv->dtype != LIT_FP8E4M3_G64_ROPE_BF16)
    return fail(LIT_ERR_DTYPE, "%s: kv dtype %d unsupported", who, (int)kv->dtype);
  if (kv->dtype == LIT_FP8E4M3_G64_ROPE_BF16 && (!kv->rope || !kv->scale))
    return fail(LIT_ERR_NULL, "%s: FP8 rows need rope and scale arrays", who);
  if (!aligned(q, 16) || !aligned(kv->data, kv->dtype == LIT_FP8E4M3_G64_ROPE_BF16 ? 8 : 16) ||
      (kv->rope && !aligned(kv->rope, 16)))
    return fail(LIT_ERR_ALIGN, "%s: q and the rows must be 16-byte aligned (FP8 row bytes 8-byte)", who);
  KvRows kvr;
  const lit_status kst = kv_arrays(kv, &kvr.d, &kvr.r, &kvr.s, who);
  if (kst != LIT_OK) return kst;
  const int N = kv->n_rows;
  LookaheadWs W = lookahead_ws(ws, B, T, Hq, N, k);
  if (!ws || ws_bytes < W.bytes)
    return fail(LIT_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", who, ws_bytes, W.bytes);
  if (!aligned(ws, 256) || (pbar && !aligned(pbar, 8)) || (step_ids && !aligned(step_ids, 4)) ||
      (hits && !aligned(hits, 4)) || !aligned(union_count, 4))
    return fail(LIT_ERR_ALIGN, "%s: workspace 256-byte, pbar 8-byte, integer outputs 4-byte aligned", who);
  hipStream_t st = (hipStream_t)stream;
  const int BT = B * T, M = T * Hq;
  double* pb = pbar ? pbar : W.g.pbar;
  int32_t* ids = step_ids ? step_ids : W.ids;
  dim3 g1((unsigned)cdiv(N, LA_TILE), (unsigned)cdiv(M, LA_TILE), (unsigned)B);
  lookahead_logits_kernel<<<g1, 256, 0, st>>>(q, (int)q_dtype, M, (int)kv->dtype, kvr, N, (double)scale, W.g.X,
                                              W.g.part);
  LIT_CHECK_LAUNCH(who);
  // each (sequence, step) row is one a6 golden: softmax per head, head average, top-k
  golden_stats_parts_kernel<<<dim3((unsigned)cdiv(BT * Hq, 4)), 256, 0, st>>>(W.g.part, (N + 31) / 32, BT * Hq,
                                                                              W.g.stats);
  LIT_CHECK_LAUNCH(who);
  golden_pbar_kernel<<<dim3((unsigned)cdiv(N, 256), (unsigned)BT), 256, 0, st>>>(W.g.X, W.g.stats, Hq, N, pb);
  LIT_CHECK_LAUNCH(who);
  topk_f64_kernel<<<dim3((unsigned)BT), 1024, 0, st>>>(pb, N, k, W.g.sel, ids, W.cnt, W.mask);
  LIT_CHECK_LAUNCH(who);
  uint8_t* um = union_mask ? union_mask : W.umask;
  lookahead_union_kernel<<<dim3((unsigned)cdiv(N, 256), (unsigned)B), 256, 0, st>>>(W.mask, T, N, hits, um);
  LIT_CHECK_LAUNCH(who);
  count_u8_kernel<<<dim3((unsigned)B), 256, 0, st>>>(um, N, union_count);
  LIT_CHECK_LAUNCH(who);
  return LIT_OK;
}
