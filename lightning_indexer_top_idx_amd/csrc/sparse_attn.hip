// sparse_attn.hip - a3/a4/a5: MQA decode attention over the selected rows.
//
// [ARCH] ai-muninn.com, "284B 塞得進 128GB、長 context 還跑得動:DeepSeek-V4-Flash 打的是
// KV cache,不是參數量": section "(B) 只讀你需要的" - the attention of a CSA layer
// reads only the top-k compressed rows picked by the indexer plus the sliding
// window of 128 recent entries, so a decode step touches a few hundred rows;
// section "(A) 壓縮你存的" - rows are the 512-wide attn_comp_kv latent (shared by
// every query head as key and value) and HCA layers read all of their rows;
// section "為什麼你沒辦法靠量化 KV 再省記憶體" - the non-RoPE dims are stored as
// E4M3 in groups of 64 with a power-of-two scale, the RoPE dims as BF16.
//
// Layout of the work: a workgroup owns one sequence and a contiguous slice of
// the row list (ids first, then the window rows not already selected). Per tile
// of 32 rows it gathers the rows into LDS (1 KiB coalesced loads; FP8 rows are
// dequantised exactly to BF16 on the way), then each wave (16 query heads)
// computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = rows from LDS, B = the
// wave's queries held in registers), updates an online softmax in fp32, and
// accumulates O += P V with the same instruction (A = P straight from the S^T
// accumulators, no transpose; B = V read from LDS). Slices of one sequence are
// merged by a log-sum-exp combine.
#include <algorithm>
#include <math.h>

#include "lit_common.h"

namespace lit {
namespace {

constexpr int TILE = 32;
constexpr int ROW_STRIDE = 520;  // bf16 per LDS row: 512 + 8 pad (spreads banks)
constexpr int PART = 516;        // floats per partial: O[512], m, l, 2 pad
constexpr int TARGET_WGS = 512;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

struct AttnParams {
  const uint16_t* q;  // [B][Hq][512] bf16
  int Hq;
  int kv_dtype;
  const uint8_t* data;
  const uint16_t* rope;
  const uint8_t* scale;
  int N;
  const int32_t* ids;
  const int32_t* count;
  int k_cap, window;  // window already clamped to N
  float scale_log2;   // scale * log2(e)
  int splits, rows_per_split;
  float* out;
  float* lse;
  float* part;  // [B][splits][Hq][PART] when splits > 1
};

// Exact E4M3FN -> BF16 with a power-of-two scale; the product has at most four
// significant bits, so dropping the low half of the fp32 is exact.
__device__ __forceinline__ uint32_t e4m3_bf16(uint32_t byte, float sc) {
  const uint32_t e = (byte >> 3) & 15u, m = byte & 7u;
  float v;
  if (e == 15u && m == 7u)
    v = __uint_as_float(0x7fc00000u);
  else if (e == 0u)
    v = (float)m * 0x1p-9f;
  else
    v = __uint_as_float(((e + 120u) << 23) | (m << 20));
  v = __uint_as_float(__float_as_uint(v) | ((byte & 0x80u) << 24)) * sc;
  return __float_as_uint(v) >> 16;
}

__device__ __forceinline__ float e8m0_f32(uint32_t b) {
  if (b == 255u) return __uint_as_float(0x7fc00000u);
  if (b == 0u) return 0x1p-127f;
  return __uint_as_float(b << 23);
}

// Row index of list position p for sequence b; -1 = skip (window row that is
// already among the ids, or past the end).
struct RowList {
  const int32_t* ids;
  int c, N, Wc, total;
  bool dense;
  const uint32_t* dup;  // LDS bitmap over the window rows
  __device__ __forceinline__ int row(int p) const {
    if (p >= total) return -1;
    if (dense) return p;
    if (p < c) {
      const int r = ids[p];
      return (r >= 0 && r < N) ? r : -1;  // ids outside the rows are skipped
    }
    const int j = p - c;
    if ((dup[j >> 5] >> (j & 31)) & 1u) return -1;
    return N - Wc + j;
  }
};

template <int NW>
__global__ __launch_bounds__(NW * 64) void attn_mfma_kernel(AttnParams P) {
  __shared__ __align__(16) uint16_t tile[TILE * ROW_STRIDE];
  __shared__ int rows[TILE];
  __shared__ uint32_t dup[LIT_MAX_WINDOW / 32];
  constexpr int NT = NW * 64;
  const int b = blockIdx.x / P.splits, s = blockIdx.x % P.splits;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int Hq = P.Hq;

  RowList RL;
  RL.dense = P.ids == nullptr;
  RL.N = P.N;
  RL.dup = dup;
  if (RL.dense) {
    RL.ids = nullptr;
    RL.c = 0;
    RL.Wc = 0;
    RL.total = P.N;
  } else {
    RL.ids = P.ids + (size_t)b * P.k_cap;
    int c = P.count[b];
    c = c < 0 ? 0 : (c > P.k_cap ? P.k_cap : c);
    RL.c = c;
    RL.Wc = P.window;
    RL.total = c + P.window;
  }
  const int p0 = s * P.rows_per_split;
  const int p1 = min(RL.total, p0 + P.rows_per_split);
  if (!RL.dense && p1 > RL.c && RL.Wc > 0) {
    for (int i = tid; i < (RL.Wc + 31) / 32; i += NT) dup[i] = 0u;
    __syncthreads();
    const int lo = P.N - RL.Wc;
    for (int j = tid; j < RL.c; j += NT) {
      const int id = RL.ids[j];
      if (id >= lo && id < P.N) atomicOr(&dup[(id - lo) >> 5], 1u << ((id - lo) & 31));
    }
  }
  __syncthreads();

  // This wave's 16 heads as B operands: K-step j, lane (c16 + 16 g) holds dims 8g + 32j .. +7.
  const int head = wid * 16 + c16;
  u32x4 qreg[16];
  {
    const uint16_t* qh = P.q + ((size_t)b * Hq + head) * LIT_KV_DIM;
#pragma unroll
    for (int j = 0; j < 16; j++) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (head < Hq) v = *(const u32x4*)(qh + 8 * g + 32 * j);
      qreg[j] = v;
    }
  }
  f32x4 o[32];
#pragma unroll
  for (int nt = 0; nt < 32; nt++) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const size_t seq_rows = (size_t)b * P.N;
#pragma unroll 1
  for (int t0 = p0; t0 < p1; t0 += TILE) {
    if (tid < TILE) rows[tid] = (t0 + tid < p1) ? RL.row(t0 + tid) : -1;
    __syncthreads();
    // gather
    if (P.kv_dtype == LIT_BF16) {
      const uint16_t* base = (const uint16_t*)P.data;
      for (int u = tid; u < TILE * 64; u += NT) {
        const int r = u >> 6, ch = u & 63;
        const int row = rows[r];
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row >= 0) v = *(const u32x4*)(base + (seq_rows + row) * LIT_KV_DIM + ch * 8);
        *(u32x4*)(tile + r * ROW_STRIDE + ch * 8) = v;
      }
    } else {
      // FP8: 28 chunks of 16 E4M3 bytes + 8 chunks of 8 BF16 RoPE dims per row
      for (int u = tid; u < TILE * 36; u += NT) {
        const int r = u / 36, ch = u % 36;
        const int row = rows[r];
        if (ch < 28) {
          u32x4 out0 = {0u, 0u, 0u, 0u}, out1 = {0u, 0u, 0u, 0u};
          if (row >= 0) {
            const size_t rr = seq_rows + row;
            const u32x4 v = *(const u32x4*)(P.data + rr * LIT_KV_FP8_DIMS + ch * 16);
            const float sc = e8m0_f32(P.scale[rr * LIT_KV_SCALE_STRIDE + (ch >> 2)]);
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const uint32_t wv = v[i];
              const uint32_t h0 = e4m3_bf16(wv & 255u, sc), h1 = e4m3_bf16((wv >> 8) & 255u, sc);
              const uint32_t h2 = e4m3_bf16((wv >> 16) & 255u, sc), h3 = e4m3_bf16(wv >> 24, sc);
              if (i < 2) {
                out0[2 * i] = h0 | (h1 << 16);
                out0[2 * i + 1] = h2 | (h3 << 16);
              } else {
                out1[2 * (i - 2)] = h0 | (h1 << 16);
                out1[2 * (i - 2) + 1] = h2 | (h3 << 16);
              }
            }
          }
          *(u32x4*)(tile + r * ROW_STRIDE + ch * 16) = out0;
          *(u32x4*)(tile + r * ROW_STRIDE + ch * 16 + 8) = out1;
        } else {
          const int rc = ch - 28;
          u32x4 v = {0u, 0u, 0u, 0u};
          if (row >= 0)
            v = *(const u32x4*)(P.rope + (seq_rows + row) * LIT_KV_ROPE_DIMS + rc * 8);
          *(u32x4*)(tile + r * ROW_STRIDE + LIT_KV_FP8_DIMS + rc * 8) = v;
        }
      }
    }
    __syncthreads();

    // S^T = K Q^T : acc[t] holds rows 16t + 4g + i for head c16
    f32x4 acc[2];
#pragma unroll
    for (int t = 0; t < 2; t++) {
      acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* krow = tile + (16 * t + c16) * ROW_STRIDE + 8 * g;
#pragma unroll
      for (int j = 0; j < 16; j++) {
        const u32x4 a = *(const u32x4*)(krow + 32 * j);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                         __builtin_bit_cast(bf16x8, qreg[j]), acc[t], 0, 0, 0);
      }
    }
    // online softmax (log2 domain)
    float x[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const bool valid = rows[16 * t + 4 * g + i] >= 0;
        const float v = valid ? acc[t][i] * P.scale_log2 : -INFINITY;
        x[4 * t + i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);  // m_run = -inf gives 0
    float psum = 0.f;
    uint32_t pk[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float p0v = exp2f(x[i] - m_use), p1v = exp2f(x[4 + i] - m_use);
      psum += p0v + p1v;
      x[i] = p0v;
      x[4 + i] = p1v;
    }
    // pack P as the A operand: element kk -> row kk<4 ? 4g+kk : 16+4g+kk-4
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint32_t lo = __float_as_uint(x[2 * i]), hi = __float_as_uint(x[2 * i + 1]);
      // round to nearest even into bf16
      const uint32_t lo16 = (lo + 0x7fffu + ((lo >> 16) & 1u)) >> 16;
      const uint32_t hi16 = (hi + 0x7fffu + ((hi >> 16) & 1u)) >> 16;
      pk[i] = lo16 | (hi16 << 16);
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // rescale O: O rows are heads 4g+i; their alpha lives in lane 4g+i
    float al[4];
#pragma unroll
    for (int i = 0; i < 4; i++) al[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
    for (int nt = 0; nt < 32; nt++)
#pragma unroll
      for (int i = 0; i < 4; i++) o[nt][i] *= al[i];
    const u32x4 pa = {pk[0], pk[1], pk[2], pk[3]};
    const bf16x8 pa8 = __builtin_bit_cast(bf16x8, pa);
    // O += P V : B operand lane (c16 + 16g) = V[rows 4g..4g+3, 16+4g..16+4g+3][16 nt + c16]
    const uint16_t* v0 = tile + (4 * g) * ROW_STRIDE + c16;
    const uint16_t* v1 = tile + (16 + 4 * g) * ROW_STRIDE + c16;
#pragma unroll
    for (int nt = 0; nt < 32; nt++) {
      const int d = 16 * nt;
      u32x4 vb;
      vb[0] = (uint32_t)v0[d] | ((uint32_t)v0[ROW_STRIDE + d] << 16);
      vb[1] = (uint32_t)v0[2 * ROW_STRIDE + d] | ((uint32_t)v0[3 * ROW_STRIDE + d] << 16);
      vb[2] = (uint32_t)v1[d] | ((uint32_t)v1[ROW_STRIDE + d] << 16);
      vb[3] = (uint32_t)v1[2 * ROW_STRIDE + d] | ((uint32_t)v1[3 * ROW_STRIDE + d] << 16);
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa8, __builtin_bit_cast(bf16x8, vb), o[nt], 0, 0, 0);
    }
    __syncthreads();
  }

  // finish: l per head (column c16) summed over the four row groups
  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16);
  l_tot += __shfl_xor(l_tot, 32);
  float lh[4], mh[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    lh[i] = __shfl(l_tot, 4 * g + i);
    mh[i] = __shfl(m_run, 4 * g + i);
  }
  if (P.splits == 1) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int h = wid * 16 + 4 * g + i;
      if (h >= Hq) continue;
      float* oh = P.out + ((size_t)b * Hq + h) * LIT_KV_DIM;
      const float inv = lh[i] > 0.f ? 1.f / lh[i] : 0.f;
#pragma unroll
      for (int nt = 0; nt < 32; nt++) oh[16 * nt + c16] = o[nt][i] * inv;
      if (P.lse && c16 == 0) P.lse[(size_t)b * Hq + h] = lh[i] > 0.f ? mh[i] * LN2 + logf(lh[i]) : -INFINITY;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int h = wid * 16 + 4 * g + i;
      if (h >= Hq) continue;
      float* ph = P.part + (((size_t)b * P.splits + s) * Hq + h) * PART;
#pragma unroll
      for (int nt = 0; nt < 32; nt++) ph[16 * nt + c16] = o[nt][i];
      if (c16 == 0) {
        ph[512] = mh[i];
        ph[513] = lh[i];
      }
    }
  }
}

// Log-sum-exp merge of the row slices of one (sequence, head).
__global__ __launch_bounds__(512) void attn_combine_kernel(const float* __restrict__ part, int splits, int Hq,
                                                           float* __restrict__ out, float* __restrict__ lse) {
  const int b = blockIdx.x / Hq, h = blockIdx.x % Hq, d = threadIdx.x;
  const float* base = part + ((size_t)b * splits * Hq + h) * PART;
  const size_t stride = (size_t)Hq * PART;
  float M = -INFINITY;
  for (int s = 0; s < splits; s++) M = fmaxf(M, base[s * stride + 512]);
  float L = 0.f, acc = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < splits; s++) {
      const float* ps = base + s * stride;
      const float wgt = exp2f(ps[512] - M);  // empty slices have m = -inf -> 0
      L += wgt * ps[513];
      acc += wgt * ps[d];
    }
  }
  out[((size_t)b * Hq + h) * LIT_KV_DIM + d] = L > 0.f ? acc / L : 0.f;
  if (lse && d == 0) lse[(size_t)b * Hq + h] = L > 0.f ? M * LN2 + logf(L) : -INFINITY;
}

// FP32 rows and queries: one workgroup per (sequence, head), fp32 VALU with an
// online softmax over chunks of 1024 list positions.
__global__ __launch_bounds__(256) void attn_f32_kernel(const float* __restrict__ q, int Hq, const float* __restrict__ kv,
                                                       int N, const int32_t* __restrict__ ids,
                                                       const int32_t* __restrict__ count, int k_cap, int window,
                                                       float scale, float* __restrict__ out, float* __restrict__ lse) {
  __shared__ float xs[1024];
  __shared__ int rs[1024];
  __shared__ uint32_t dup[LIT_MAX_WINDOW / 32];
  __shared__ float red[8];
  const int b = blockIdx.x / Hq, h = blockIdx.x % Hq;
  const int tid = threadIdx.x;
  RowList RL;
  RL.dense = ids == nullptr;
  RL.N = N;
  RL.dup = dup;
  if (RL.dense) {
    RL.ids = nullptr;
    RL.c = 0;
    RL.Wc = 0;
    RL.total = N;
  } else {
    RL.ids = ids + (size_t)b * k_cap;
    int c = count[b];
    c = c < 0 ? 0 : (c > k_cap ? k_cap : c);
    RL.c = c;
    RL.Wc = window;
    RL.total = c + window;
    for (int i = tid; i < (window + 31) / 32; i += 256) dup[i] = 0u;
    __syncthreads();
    for (int j = tid; j < c; j += 256) {
      const int id = RL.ids[j];
      if (id >= N - window && id < N) atomicOr(&dup[(id - (N - window)) >> 5], 1u << ((id - (N - window)) & 31));
    }
  }
  __syncthreads();
  const float* qh = q + ((size_t)b * Hq + h) * LIT_KV_DIM;
  const float* kvb = kv + (size_t)b * N * LIT_KV_DIM;
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int c0 = 0; c0 < RL.total; c0 += 1024) {
    const int len = min(1024, RL.total - c0);
    float cmax = -INFINITY;
    for (int p = tid; p < len; p += 256) {
      const int r = RL.row(c0 + p);
      float xv = -INFINITY;
      if (r >= 0) {
        const float* kr = kvb + (size_t)r * LIT_KV_DIM;
        float dot = 0.f;
        for (int d = 0; d < LIT_KV_DIM; d++) dot = fmaf(qh[d], kr[d], dot);
        xv = dot * scale;
      }
      xs[p] = xv;
      rs[p] = r;
      cmax = fmaxf(cmax, xv);
    }
    cmax = wave_max(cmax);
    if ((tid & 63) == 0) red[tid >> 6] = cmax;
    __syncthreads();
    cmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float m_new = fmaxf(m, cmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = expf(m - m_use);
    float ls = 0.f;
    float a0 = 0.f, a1 = 0.f;
    for (int p = 0; p < len; p++) {
      const int r = rs[p];
      if (r < 0) continue;
      const float e = expf(xs[p] - m_use);
      ls += e;
      const float* kr = kvb + (size_t)r * LIT_KV_DIM;
      a0 = fmaf(e, kr[tid], a0);
      a1 = fmaf(e, kr[tid + 256], a1);
    }
    l = l * alpha + ls;
    o0 = o0 * alpha + a0;
    o1 = o1 * alpha + a1;
    m = m_new;
    __syncthreads();
  }
  float* oh = out + ((size_t)b * Hq + h) * LIT_KV_DIM;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  oh[tid] = o0 * inv;
  oh[tid + 256] = o1 * inv;
  if (lse && tid == 0) lse[(size_t)b * Hq + h] = l > 0.f ? m + logf(l) : -INFINITY;
}

void plan_splits(int B, int rows_max, int* splits, int* rows_per_split) {
  const int tiles = std::max(1, (rows_max + TILE - 1) / TILE);
  const int want = std::max(1, (TARGET_WGS + B - 1) / B);
  int s = std::min(tiles, want);
  const int tiles_per = (tiles + s - 1) / s;
  s = (tiles + tiles_per - 1) / tiles_per;
  *splits = s;
  *rows_per_split = tiles_per * TILE;
}

}  // namespace
}  // namespace lit

using namespace lit;

extern "C" size_t lit_attn_workspace_bytes(int32_t B, int32_t Hq, int32_t N) {
  if (B < 1 || Hq < 1 || N < 1) return 0;
  int s, rps;
  plan_splits(B, N + LIT_MAX_WINDOW, &s, &rps);
  if (s <= 1) return 256;
  return round_up((size_t)B * s * Hq * PART * sizeof(float), 256);
}

extern "C" lit_status lit_sparse_attn_decode(const void* q, lit_dtype q_dtype, int32_t Hq, const lit_kv* kv, int32_t B,
                                             const int32_t* ids, const int32_t* count, int32_t k_cap, int32_t window,
                                             float scale, float* out, float* lse, void* ws, size_t ws_bytes,
                                             void* stream) {
  clear_error();
  const char* who = "lit_sparse_attn_decode";
  if (!q || !kv || !out || !kv->data) return fail(LIT_ERR_NULL, "%s: q, kv, kv->data and out must be non-NULL", who);
  if (B < 1 || Hq < 1 || Hq > LIT_MAX_Q_HEADS || kv->n_rows < 1)
    return fail(LIT_ERR_SHAPE, "%s: B=%d Hq=%d (1..%d) N=%d", who, B, Hq, LIT_MAX_Q_HEADS, kv->n_rows);
  const int N = kv->n_rows;
  if (ids) {
    if (!count) return fail(LIT_ERR_NULL, "%s: ids given without count", who);
    if (k_cap < 1) return fail(LIT_ERR_SHAPE, "%s: k_cap=%d must be >= 1", who, k_cap);
    if (window < 0 || window > LIT_MAX_WINDOW)
      return fail(LIT_ERR_SHAPE, "%s: window=%d outside 0..%d", who, window, LIT_MAX_WINDOW);
    if (!aligned(ids, 4) || !aligned(count, 4)) return fail(LIT_ERR_ALIGN, "%s: ids/count misaligned", who);
  }
  const int Wc = ids ? std::min(window, N) : 0;
  if (kv->dtype == LIT_F32) {
    if (q_dtype != LIT_F32) return fail(LIT_ERR_DTYPE, "%s: F32 rows need F32 queries", who);
  } else if (kv->dtype == LIT_BF16 || kv->dtype == LIT_FP8E4M3_G64_ROPE_BF16) {
    if (q_dtype != LIT_BF16) return fail(LIT_ERR_DTYPE, "%s: BF16/FP8 rows need BF16 queries", who);
    if (kv->dtype == LIT_FP8E4M3_G64_ROPE_BF16 && (!kv->rope || !kv->scale))
      return fail(LIT_ERR_NULL, "%s: FP8 rows need rope and scale arrays", who);
  } else {
    return fail(LIT_ERR_DTYPE, "%s: kv dtype %d unsupported", who, (int)kv->dtype);
  }
  if (!aligned(q, 16) || !aligned(kv->data, 16) || (kv->rope && !aligned(kv->rope, 16)) || !aligned(out, 4))
    return fail(LIT_ERR_ALIGN, "%s: q, kv->data and kv->rope must be 16-byte aligned", who);
  hipStream_t st = (hipStream_t)stream;
  if (kv->dtype == LIT_F32) {
    attn_f32_kernel<<<dim3((unsigned)(B * Hq)), dim3(256), 0, st>>>((const float*)q, Hq, (const float*)kv->data, N,
                                                                     ids, count, k_cap, Wc, scale, out, lse);
    LIT_CHECK_LAUNCH(who);
    return LIT_OK;
  }
  const int rows_max = ids ? (k_cap + Wc) : N;
  AttnParams P;
  plan_splits(B, rows_max, &P.splits, &P.rows_per_split);
  if (P.splits > 1) {
    const size_t need = round_up((size_t)B * P.splits * Hq * PART * sizeof(float), 256);
    if (!ws || ws_bytes < need)
      return fail(LIT_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", who, ws_bytes, need);
    if (!aligned(ws, 16)) return fail(LIT_ERR_ALIGN, "%s: workspace must be 16-byte aligned", who);
  }
  P.q = (const uint16_t*)q;
  P.Hq = Hq;
  P.kv_dtype = (int)kv->dtype;
  P.data = (const uint8_t*)kv->data;
  P.rope = (const uint16_t*)kv->rope;
  P.scale = kv->scale;
  P.N = N;
  P.ids = ids;
  P.count = count;
  P.k_cap = k_cap;
  P.window = Wc;
  P.scale_log2 = scale * LOG2E;
  P.out = out;
  P.lse = lse;
  P.part = (float*)ws;
  const int nw = (Hq + 15) / 16;
  dim3 grid((unsigned)(B * P.splits));
  switch (nw) {
    case 1: attn_mfma_kernel<1><<<grid, 64, 0, st>>>(P); break;
    case 2: attn_mfma_kernel<2><<<grid, 128, 0, st>>>(P); break;
    case 3: attn_mfma_kernel<3><<<grid, 192, 0, st>>>(P); break;
    default: attn_mfma_kernel<4><<<grid, 256, 0, st>>>(P); break;
  }
  LIT_CHECK_LAUNCH(who);
  if (P.splits > 1) {
    attn_combine_kernel<<<dim3((unsigned)(B * Hq)), dim3(512), 0, st>>>((const float*)ws, P.splits, Hq, out, lse);
    LIT_CHECK_LAUNCH(who);
  }
  return LIT_OK;
}
