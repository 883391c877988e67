// lsa_gate.hip - a8: the FlashMemory / LSA sigmoid chunk gate.
//
// zhichai.net, "FlashMemory-DeepSeek-V4 深度解读：用预言家替代记忆海绵":
//   section 2.2 - every tau = 64 decode steps a memory indexer looks at the hidden
//   state and scores each compressed chunk with a sigmoid; chunks at or above
//   0.5 are fetched, the native indexer then picks its top-k inside that set;
//   section 3.1 - only the query side (three small projections) is trained, the
//   keys are the frozen compressed index keys;
//   section 4.1 - independent indexers at layers 10, 12 and 20, their kept
//   sets OR-ed;
//   second reply - the gated score sigma(sum_h w_h * ReLU(q_h . k)).
// ai-muninn.com, "FlashMemory can't improve ...", section "Act 2", names the
// projections wq_a, wq_b and weights_proj.
//
// Per layer: u = wq_a h, q = wq_b u, w = w_proj h in fp64 with sequential sums
// (so they are bit-identical to a CPU loop), then z[n] for every chunk. The bulk
// of z runs in fp32 on the VALU; a proven bound on its rounding decides which
// chunks sit close enough to the threshold to need the canonical fp64 value.
#include <algorithm>
#include <math.h>

#include "lit_common.h"

namespace lit {
namespace {

constexpr int MV_ROWS = 256;  // matrix rows per workgroup
constexpr int MV_COLS = 32;   // columns staged per step
constexpr double GATE_SAFETY = 4.0;

// y[b][r] = sum_i M[r][i] * x[b][i] (fp64, i ascending, each product rounded
// before it is added). M is BF16 [R][C]; x is fp32 or fp64 [B][C].
template <typename XT>
__global__ __launch_bounds__(MV_ROWS) void matvec_kernel(const uint16_t* __restrict__ M, const XT* __restrict__ x,
                                                         int R, int C, double* __restrict__ y) {
#pragma clang fp contract(off)
  __shared__ float ms[MV_COLS][MV_ROWS + 1];
  __shared__ double xs[MV_COLS];
  const int b = blockIdx.y, r0 = blockIdx.x * MV_ROWS, tid = threadIdx.x;
  const XT* xb = x + (size_t)b * C;
  double acc = 0.0;
  for (int c0 = 0; c0 < C; c0 += MV_COLS) {
    for (int u = tid; u < MV_COLS * MV_ROWS; u += MV_ROWS) {
      const int rr = u / MV_COLS, cc = u % MV_COLS;
      const int r = r0 + rr, c = c0 + cc;
      ms[cc][rr] = (r < R && c < C) ? bf16_to_f32(M[(size_t)r * C + c]) : 0.f;
    }
    if (tid < MV_COLS) xs[tid] = (c0 + tid < C) ? (double)xb[c0 + tid] : 0.0;
    __syncthreads();
    const int n = min(MV_COLS, C - c0);
    for (int cc = 0; cc < n; cc++) {
      const double p = (double)ms[cc][tid] * xs[cc];
      acc = acc + p;
    }
    __syncthreads();
  }
  if (r0 + tid < R) y[(size_t)b * R + r0 + tid] = acc;
}

// z for every chunk of one layer; keep = z >= thr, OR-ed into gate.
__global__ __launch_bounds__(256) void gate_score_kernel(const double* __restrict__ q64, const double* __restrict__ w64,
                                                         const uint16_t* __restrict__ k, int H, int N, double thr,
                                                         uint8_t* __restrict__ gate, int first) {
#pragma clang fp contract(off)
  __shared__ float q32[64 * LIT_IDX_DIM];
  __shared__ float w32[64];
  __shared__ double qn[64];
  const int b = blockIdx.y, tid = threadIdx.x;
  const double* qb = q64 + (size_t)b * H * LIT_IDX_DIM;
  for (int i = tid; i < H * LIT_IDX_DIM; i += 256) q32[i] = (float)qb[i];
  if (tid < H) {
    w32[tid] = (float)w64[(size_t)b * H + tid];
    double s = 0.0;
    for (int d = 0; d < LIT_IDX_DIM; d++) s += qb[tid * LIT_IDX_DIM + d] * qb[tid * LIT_IDX_DIM + d];
    qn[tid] = fabs(w64[(size_t)b * H + tid]) * sqrt(s);
  }
  __syncthreads();
  const int n = blockIdx.x * 256 + tid;
  if (n >= N) return;
  double Q = 0.0;
  for (int h = 0; h < H; h++) Q += qn[h];
  const uint16_t* kr = k + ((size_t)b * N + n) * LIT_IDX_DIM;
  float kv[LIT_IDX_DIM];
  float kn2 = 0.f;
#pragma unroll
  for (int c = 0; c < LIT_IDX_DIM / 8; c++) {
    const u32x4 v = *(const u32x4*)(kr + 8 * c);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      kv[8 * c + 2 * i] = bf16_lo(v[i]);
      kv[8 * c + 2 * i + 1] = bf16_hi(v[i]);
    }
  }
#pragma unroll
  for (int d = 0; d < LIT_IDX_DIM; d++) kn2 = fmaf(kv[d], kv[d], kn2);
  float z = 0.f;
  for (int h = 0; h < H; h++) {
    float acc = 0.f;
#pragma unroll
    for (int d = 0; d < LIT_IDX_DIM; d++) acc = fmaf(q32[h * LIT_IDX_DIM + d], kv[d], acc);
    z = fmaf(w32[h], fmaxf(acc, 0.f), z);
  }
  // |z - z64| <= (134 + H) u Q |k|, u = 2^-24 (rounding of q and w to fp32,
  // 128 products and sums per head, the head sum), times a safety factor.
  const double delta = GATE_SAFETY * 0x1p-24 * (134.0 + H) * Q * sqrt((double)kn2) * (1.0 + 0x1p-16) + 1e-300;
  bool keep;
  if (fabs((double)z - thr) > delta) {
    keep = (double)z >= thr;
  } else {
    const double* wb = w64 + (size_t)b * H;
    double zz = 0.0;
    for (int h = 0; h < H; h++) {
      double acc = 0.0;
      for (int d = 0; d < LIT_IDX_DIM; d++) {
        const double p = qb[h * LIT_IDX_DIM + d] * (double)kv[d];
        acc = acc + p;
      }
      const double r = acc > 0.0 ? acc : 0.0;
      const double p = wb[h] * r;
      zz = zz + p;
    }
    keep = zz >= thr;
  }
  uint8_t* gp = gate + (size_t)b * N + n;
  *gp = first ? (uint8_t)keep : (uint8_t)(*gp | (uint8_t)keep);
}

__global__ __launch_bounds__(256) void count_kernel(const uint8_t* __restrict__ m, int N, int32_t* __restrict__ out) {
  __shared__ int red[4];
  const int b = blockIdx.x, tid = threadIdx.x;
  int c = 0;
  for (int n = tid; n < N; n += 256) c += m[(size_t)b * N + n] != 0;
  c = wave_sum(c);
  if ((tid & 63) == 0) red[tid >> 6] = c;
  __syncthreads();
  if (tid == 0) out[b] = red[0] + red[1] + red[2] + red[3];
}

}  // namespace
}  // namespace lit

using namespace lit;

extern "C" size_t lit_gate_workspace_bytes(int32_t n_layers, int32_t B, int32_t H, int32_t rank, int32_t N) {
  (void)n_layers;
  (void)N;
  if (B < 1 || H < 1 || rank < 1) return 0;
  return round_up((size_t)B * rank * sizeof(double), 256) +
         round_up((size_t)B * H * LIT_IDX_DIM * sizeof(double), 256) + round_up((size_t)B * H * sizeof(double), 256);
}

extern "C" lit_status lit_lsa_gate(const lit_gate_layer* layers, int32_t n_layers, int32_t B, int32_t N, int32_t H,
                                   int32_t d_model, int32_t rank, double threshold, uint8_t* gate,
                                   int32_t* gate_count, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  const char* who = "lit_lsa_gate";
  if (!layers || !gate || !gate_count) return fail(LIT_ERR_NULL, "%s: layers, gate and gate_count are required", who);
  if (n_layers < 1 || n_layers > 8 || B < 1 || N < 1 || H < 1 || H > 64 || d_model < 1 || rank < 1)
    return fail(LIT_ERR_SHAPE, "%s: n_layers=%d B=%d N=%d H=%d d_model=%d rank=%d", who, n_layers, B, N, H, d_model,
                rank);
  if (!(threshold > 0.0 && threshold < 1.0))
    return fail(LIT_ERR_SHAPE, "%s: threshold=%g outside (0,1)", who, threshold);
  for (int l = 0; l < n_layers; l++) {
    const lit_gate_layer& L = layers[l];
    if (!L.h || !L.wq_a || !L.wq_b || !L.w_proj || !L.k)
      return fail(LIT_ERR_NULL, "%s: layer %d has a NULL array", who, l);
    if (!aligned(L.k, 16)) return fail(LIT_ERR_ALIGN, "%s: layer %d keys must be 16-byte aligned", who, l);
  }
  const size_t need = lit_gate_workspace_bytes(n_layers, B, H, rank, N);
  if (!ws || ws_bytes < need)
    return fail(LIT_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", who, ws_bytes, need);
  if (!aligned(ws, 256)) return fail(LIT_ERR_ALIGN, "%s: workspace must be 256-byte aligned", who);
  // sigmoid(z) >= t  <=>  z >= log(t / (1 - t)), exactly 0 at t = 0.5
  const double thr = threshold == 0.5 ? 0.0 : log(threshold / (1.0 - threshold));
  uint8_t* p = (uint8_t*)ws;
  double* u = (double*)p;
  p += round_up((size_t)B * rank * sizeof(double), 256);
  double* q = (double*)p;
  p += round_up((size_t)B * H * LIT_IDX_DIM * sizeof(double), 256);
  double* w = (double*)p;
  hipStream_t st = (hipStream_t)stream;
  for (int l = 0; l < n_layers; l++) {
    const lit_gate_layer& L = layers[l];
    matvec_kernel<float><<<dim3((unsigned)cdiv(rank, MV_ROWS), (unsigned)B), MV_ROWS, 0, st>>>(
        (const uint16_t*)L.wq_a, L.h, rank, d_model, u);
    LIT_CHECK_LAUNCH(who);
    matvec_kernel<double><<<dim3((unsigned)cdiv(H * LIT_IDX_DIM, MV_ROWS), (unsigned)B), MV_ROWS, 0, st>>>(
        (const uint16_t*)L.wq_b, u, H * LIT_IDX_DIM, rank, q);
    LIT_CHECK_LAUNCH(who);
    matvec_kernel<float><<<dim3((unsigned)cdiv(H, MV_ROWS), (unsigned)B), MV_ROWS, 0, st>>>(
        (const uint16_t*)L.w_proj, L.h, H, d_model, w);
    LIT_CHECK_LAUNCH(who);
    gate_score_kernel<<<dim3((unsigned)cdiv(N, 256), (unsigned)B), 256, 0, st>>>(
        q, w, (const uint16_t*)L.k, H, N, thr, gate, l == 0);
    LIT_CHECK_LAUNCH(who);
  }
  count_kernel<<<dim3((unsigned)B), 256, 0, st>>>(gate, N, gate_count);
  LIT_CHECK_LAUNCH(who);
  return LIT_OK;
}
