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
// of z runs in fp32 on the matrix cores; a proven bound on its rounding decides
// which chunks sit close enough to the threshold to need the canonical fp64 value.
#include <algorithm>
#include <math.h>

#include "lit_common.h"

namespace lit {
namespace {

constexpr int MV_ROWS = 64;  // matrix rows per workgroup: one wave, one row per lane
constexpr int MV_AHEAD = 8;  // 16-byte loads of the row in flight per lane
constexpr int MV_MAX_C = 4096;  // columns the LDS copy of x holds (d_model, rank)
constexpr double GATE_SAFETY = 4.0;

// One matrix-vector product of a batch: y[b][r] = sum_i M[r][i] * x[b][i]
// (fp64, i ascending, each product rounded before it is added). M is BF16
// [R][C] (C a multiple of 8 * MV_AHEAD, at most MV_MAX_C); x is fp32 or fp64 [B][C].
struct MvJob {
  const uint16_t* M;
  const void* x;
  double* y;
  int R, C, x_f64, blocks;
};
constexpr int MV_MAX_JOBS = 16;
struct MvJobs {
  MvJob j[MV_MAX_JOBS];
  int n;
};

// Several independent products in one launch (the gate layers' projections
// that do not depend on each other): the sum of a row is one dependent chain,
// so each launch wants as many rows as it can get. Rows go one per lane, x is
// staged in LDS once per workgroup, and each lane streams its row with 16-byte
// loads, MV_AHEAD of them in flight.
__global__ __launch_bounds__(MV_ROWS) void matvec_kernel(MvJobs J) {
#pragma clang fp contract(off)
  __shared__ double xs[MV_MAX_C];
  int bx = blockIdx.x, ji = 0;
  while (ji < J.n - 1 && bx >= J.j[ji].blocks) {
    bx -= J.j[ji].blocks;
    ji++;
  }
  const uint16_t* M = J.j[ji].M;
  const int R = J.j[ji].R, C = J.j[ji].C;
  const int b = blockIdx.y, tid = threadIdx.x;
  if (J.j[ji].x_f64) {
    const double* xb = (const double*)J.j[ji].x + (size_t)b * C;
    for (int i = tid; i < C; i += MV_ROWS) xs[i] = xb[i];
  } else {
    const float* xb = (const float*)J.j[ji].x + (size_t)b * C;
    for (int i = tid; i < C; i += MV_ROWS) xs[i] = (double)xb[i];
  }
  __syncthreads();
  const int r = bx * MV_ROWS + tid;
  const u32x4* row = (const u32x4*)(M + (size_t)min(r, R - 1) * C);  // lanes past R read row R-1, store nothing
  const int nv = C / 8;  // a multiple of MV_AHEAD
  u32x4 ring[MV_AHEAD];
#pragma unroll
  for (int j = 0; j < MV_AHEAD; j++) ring[j] = row[j];
  double acc = 0.0;
  for (int v0 = 0; v0 < nv; v0 += MV_AHEAD) {
#pragma unroll
    for (int j = 0; j < MV_AHEAD; j++) {
      const int v = v0 + j;
      const u32x4 m8 = ring[j];
      ring[j] = row[min(v + MV_AHEAD, nv - 1)];  // the last block's refills re-read a row piece, unused
      const double* xv = xs + 8 * v;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const double p0 = (double)bf16_lo(m8[i]) * xv[2 * i];
        acc = acc + p0;
        const double p1 = (double)bf16_hi(m8[i]) * xv[2 * i + 1];
        acc = acc + p1;
      }
    }
  }
  if (r < R) J.j[ji].y[(size_t)b * R + r] = acc;
}

// z for every chunk of one layer; keep = z >= thr, OR-ed into gate.
//
// The bulk runs on the fp32 matrix cores (v_mfma_f32_16x16x4_f32: lane l holds
// A[l%16][l/16] and B[l/16][l%16], result register i holds D[4(l/16) + i][l%16]):
// A = 16 heads x 4 dims of q rounded to fp32 (staged in LDS in operand order),
// B = 4 dims x 16 entries of keys (K-step j pairs lane group g with dim 32g + j,
// so each lane holds 32 dims of one entry), D = 16 heads x 16 entries. The
// weighted ReLU sum over the lane's heads and across the four lane groups gives
// every lane of a column the entry's z. A workgroup covers 256 entries (four
// waves of 64, four column groups each).
template <int MT>
__global__ __launch_bounds__(256) void gate_score_kernel(const double* __restrict__ q64, const double* __restrict__ w64,
                                                         const uint16_t* __restrict__ k, int H, int N, double thr,
                                                         uint8_t* __restrict__ gate, int first) {
#pragma clang fp contract(off)
  __shared__ float qlds[MT * 32 * 64];
  __shared__ float wlds[64];
  __shared__ double qn[64];
  __shared__ double Qs;
  const int b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const double* qb = q64 + (size_t)b * H * LIT_IDX_DIM;
  for (int idx = tid; idx < MT * 16 * LIT_IDX_DIM; idx += 256) {
    const int h = idx >> 7, d = idx & 127;
    const float v = h < H ? (float)qb[h * LIT_IDX_DIM + d] : 0.f;
    qlds[((h >> 4) * 32 + (d & 31)) * 64 + (h & 15) + 16 * (d >> 5)] = v;
  }
  if (tid < 64) {
    wlds[tid] = tid < H ? (float)w64[(size_t)b * H + tid] : 0.f;
    double ss = 0.0;
    if (tid < H)
      for (int d = 0; d < LIT_IDX_DIM; d++) ss += qb[tid * LIT_IDX_DIM + d] * qb[tid * LIT_IDX_DIM + d];
    qn[tid] = tid < H ? fabs(w64[(size_t)b * H + tid]) * sqrt(ss) : 0.0;
  }
  __syncthreads();
  if (tid == 0) {
    double Q = 0.0;
    for (int h = 0; h < H; h++) Q += qn[h];
    Qs = Q;
  }
  float wr[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; mt++)
#pragma unroll
    for (int i = 0; i < 4; i++) wr[mt][i] = wlds[16 * mt + 4 * g + i];
  const uint16_t* kb = k + (size_t)b * N * LIT_IDX_DIM;
  const int base = blockIdx.x * 256 + wid * 64;
  float my_z = 0.f, my_n2 = 0.f;
#pragma unroll 1
  for (int G = 0; G < 4; G++) {
    const int e = base + 16 * G + c;
    float kr[32];
#pragma unroll
    for (int v8 = 0; v8 < 4; v8++) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (e < N) v = *(const u32x4*)(kb + (size_t)e * LIT_IDX_DIM + 32 * g + 8 * v8);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        kr[8 * v8 + 2 * i] = bf16_lo(v[i]);
        kr[8 * v8 + 2 * i + 1] = bf16_hi(v[i]);
      }
    }
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int j = 0; j < 32; j++)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(qlds[(mt * 32 + j) * 64 + lane], kr[j], acc[mt], 0, 0, 0);
    float z = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int i = 0; i < 4; i++) z = fmaf(wr[mt][i], fmaxf(acc[mt][i], 0.f), z);
    z += __shfl_xor(z, 16);
    z += __shfl_xor(z, 32);
    float n2 = 0.f;
#pragma unroll
    for (int j = 0; j < 32; j++) n2 = fmaf(kr[j], kr[j], n2);
    n2 += __shfl_xor(n2, 16);
    n2 += __shfl_xor(n2, 32);
    if (G == g) {  // the column group that holds this lane's entry
      my_z = z;
      my_n2 = n2;
    }
  }
  __syncthreads();  // Qs
  const int n = base + lane;
  // |z - z64| <= (134 + H) u Q |k|, u = 2^-24 (rounding of q and w to fp32,
  // 128 products and sums per head, the head sum), times a safety factor that
  // also covers the matrix cores' order of accumulation.
  const double delta = GATE_SAFETY * 0x1p-24 * (134.0 + H) * Qs * sqrt((double)my_n2) * (1.0 + 0x1p-16) + 1e-300;
  const bool live = n < N;
  const bool band = live && !(fabs((double)my_z - thr) > delta);
  bool keep = (double)my_z >= thr;
  // Entries in the band get the canonical fp64 z, one at a time, by the whole
  // wave: lane h sums head h over d ascending (each product rounded before it
  // is added), then the heads' w_h * ReLU terms are added in h order.
  uint64_t todo = __ballot(band);
  const double* wb = w64 + (size_t)b * H;
  while (todo) {
    const int src = __ffsll((unsigned long long)todo) - 1;
    todo &= todo - 1;
    const int e = base + src;
    const uint16_t* kn = kb + (size_t)e * LIT_IDX_DIM;
    double t = 0.0;
    if (lane < H) {
      double acc = 0.0;
      for (int d = 0; d < LIT_IDX_DIM; d++) {
        const double p = qb[lane * LIT_IDX_DIM + d] * (double)bf16_to_f32(kn[d]);
        acc = acc + p;
      }
      const double r = acc > 0.0 ? acc : 0.0;
      t = wb[lane] * r;
    }
    double zz = 0.0;
    for (int h = 0; h < H; h++) {
      const double th = __shfl(t, h);
      zz = zz + th;
    }
    if (lane == src) keep = zz >= thr;
  }
  if (!live) return;
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

// u, q and w of every layer (the stages run across layers at once)
extern "C" size_t lit_gate_workspace_bytes(int32_t n_layers, int32_t B, int32_t H, int32_t rank, int32_t N) {
  (void)N;
  if (n_layers < 1 || B < 1 || H < 1 || rank < 1) return 0;
  return (size_t)n_layers * (round_up((size_t)B * rank * sizeof(double), 256) +
                             round_up((size_t)B * H * LIT_IDX_DIM * sizeof(double), 256) +
                             round_up((size_t)B * H * sizeof(double), 256));
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
  if (d_model % (8 * MV_AHEAD) != 0 || rank % (8 * MV_AHEAD) != 0 || d_model > MV_MAX_C || rank > MV_MAX_C)
    return fail(LIT_ERR_SHAPE, "%s: d_model=%d and rank=%d must be multiples of %d, at most %d", who, d_model, rank,
                8 * MV_AHEAD, MV_MAX_C);
  for (int l = 0; l < n_layers; l++) {
    const lit_gate_layer& L = layers[l];
    if (!L.h || !L.wq_a || !L.wq_b || !L.w_proj || !L.k)
      return fail(LIT_ERR_NULL, "%s: layer %d has a NULL array", who, l);
    if (!aligned(L.k, 16) || !aligned(L.wq_a, 16) || !aligned(L.wq_b, 16) || !aligned(L.w_proj, 16))
      return fail(LIT_ERR_ALIGN, "%s: layer %d keys and projection matrices must be 16-byte aligned", who, l);
  }
  const size_t need = lit_gate_workspace_bytes(n_layers, B, H, rank, N);
  if (!ws || ws_bytes < need)
    return fail(LIT_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", who, ws_bytes, need);
  if (!aligned(ws, 256)) return fail(LIT_ERR_ALIGN, "%s: workspace must be 256-byte aligned", who);
  // sigmoid(z) >= t  <=>  z >= log(t / (1 - t)), exactly 0 at t = 0.5
  const double thr = threshold == 0.5 ? 0.0 : log(threshold / (1.0 - threshold));
  uint8_t* p = (uint8_t*)ws;
  double* u[8];
  double* q[8];
  double* w[8];
  for (int l = 0; l < n_layers; l++) {
    u[l] = (double*)p;
    p += round_up((size_t)B * rank * sizeof(double), 256);
    q[l] = (double*)p;
    p += round_up((size_t)B * H * LIT_IDX_DIM * sizeof(double), 256);
    w[l] = (double*)p;
    p += round_up((size_t)B * H * sizeof(double), 256);
  }
  hipStream_t st = (hipStream_t)stream;
  // stage 1: u = wq_a h and w = w_proj h of every layer; stage 2: q = wq_b u
  MvJobs s1{}, s2{};
  int blocks1 = 0, blocks2 = 0;
  for (int l = 0; l < n_layers; l++) {
    const lit_gate_layer& L = layers[l];
    const int ba = (int)cdiv(rank, MV_ROWS), bw = (int)cdiv(H, MV_ROWS), bq = (int)cdiv(H * LIT_IDX_DIM, MV_ROWS);
    s1.j[s1.n++] = MvJob{(const uint16_t*)L.wq_a, L.h, u[l], rank, d_model, 0, ba};
    s1.j[s1.n++] = MvJob{(const uint16_t*)L.w_proj, L.h, w[l], H, d_model, 0, bw};
    s2.j[s2.n++] = MvJob{(const uint16_t*)L.wq_b, u[l], q[l], H * LIT_IDX_DIM, rank, 1, bq};
    blocks1 += ba + bw;
    blocks2 += bq;
  }
  matvec_kernel<<<dim3((unsigned)blocks1, (unsigned)B), MV_ROWS, 0, st>>>(s1);
  LIT_CHECK_LAUNCH(who);
  matvec_kernel<<<dim3((unsigned)blocks2, (unsigned)B), MV_ROWS, 0, st>>>(s2);
  LIT_CHECK_LAUNCH(who);
  for (int l = 0; l < n_layers; l++) {
    const lit_gate_layer& L = layers[l];
    const dim3 gs((unsigned)cdiv(N, 256), (unsigned)B);
    const uint16_t* kk = (const uint16_t*)L.k;
    switch ((H + 15) / 16) {
      case 1: gate_score_kernel<1><<<gs, 256, 0, st>>>(q[l], w[l], kk, H, N, thr, gate, l == 0); break;
      case 2: gate_score_kernel<2><<<gs, 256, 0, st>>>(q[l], w[l], kk, H, N, thr, gate, l == 0); break;
      case 3: gate_score_kernel<3><<<gs, 256, 0, st>>>(q[l], w[l], kk, H, N, thr, gate, l == 0); break;
      default: gate_score_kernel<4><<<gs, 256, 0, st>>>(q[l], w[l], kk, H, N, thr, gate, l == 0); break;
    }
    LIT_CHECK_LAUNCH(who);
  }
  count_kernel<<<dim3((unsigned)B), 256, 0, st>>>(gate, N, gate_count);
  LIT_CHECK_LAUNCH(who);
  return LIT_OK;
}
