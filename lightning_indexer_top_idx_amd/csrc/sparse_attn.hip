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
// Layout of the work: a workgroup of four waves owns 16 query heads of one
// sequence and a contiguous slice of its row list (ids first, then the window
// rows not already selected; a dense layer's rows are simply its positions).
// Tiles of 64 rows arrive in LDS by direct-to-LDS loads, double-buffered, the
// next tile's loads issued during the current tile's scores; FP8 rows arrive
// raw and are widened to BF16 in place (exactly: an E4M3 value times a power of
// two). Each wave scores 16 rows against the 16 heads (S^T = K Q^T on
// v_mfma_f32_16x16x32_bf16, the queries in registers), the online softmax runs
// in fp32, and O^T += V^T P^T uses the same instruction (A = V^T read from LDS
// with transposed reads, B = P straight from the S^T accumulators). Slices of
// one sequence are merged by a log-sum-exp combine kernel.
#include <algorithm>
#include <math.h>

#include <mutex>

#include "lit_common.h"

// Library-owned scratch of the allocation-free call: the per-slice partial
// results of the split attention. Each GPU the library runs on holds its own
// copy until the process ends. Host code never uses the array's name as an
// address: the device address of each GPU's copy is looked up once per device
// (hipGetSymbolAddress, with that device current) and kept in scratch_dev.
static __device__ __align__(256) uint8_t scratch[LIT_ATTN_SCRATCH_BYTES];

namespace lit {
namespace {

constexpr int PART = 516;        // floats per partial: O[512], m, l, 2 pad
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

struct AttnParams {
  const uint16_t* q;  // [B][Hq][512] bf16
  int Hq;
  int kv_dtype;
  KvArr kd, kr, ks;  // data, rope and scale rows
  int N;
  const int32_t* ids;
  const int32_t* count;
  int k_cap, window;  // window already clamped to N
  float scale_log2;   // scale * log2(e)
  int splits, rows_per_split;
  int B;
  float* out;
  float* lse;
  float* part;  // [B][splits][Hq][PART] when splits > 1
};

__device__ __forceinline__ float e8m0_f32(uint32_t b) {
  if (b == 255u) return __uint_as_float(0x7fc00000u);
  if (b == 0u) return 0x1p-127f;
  return __uint_as_float(b << 23);
}

typedef const __attribute__((address_space(3))) int32_t* lds_ids_t;

struct RowList {
  const int32_t* ids;
  lds_ids_t lids;  // the ids' copy in LDS, or null: read as LDS, not through a generic pointer
  int c, N, Wc, total;
  bool dense;
  // The read behind list position p (any p: the index is clamped into the
  // ids, so the load needs no branch and can be issued ahead of its use).
  __device__ __forceinline__ int fetch(int p) const {
    if (dense || c <= 0) return 0;
    const int j = max(min(p - Wc, c - 1), 0);
    return lids ? lids[j] : ids[j];
  }
  // The row of list position p, given f = fetch(p): positions 0 .. Wc-1 are
  // the window rows N-Wc .. N-1, then the ids follow; an id inside the window
  // (already attended) or outside the rows is skipped.
  __device__ __forceinline__ int resolve(int p, int f) const {
    if (p >= total) return -1;
    if (dense) return p;
    if (p < Wc) return N - Wc + p;
    return (f >= 0 && f < N - Wc) ? f : -1;
  }
  __device__ __forceinline__ int row(int p) const { return resolve(p, fetch(p)); }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Row slices and head groups -> workgroups: the head groups of one slice get
// workgroup ids equal modulo 8, i.e. the same XCD, so its L2 serves the rows
// to all of them.
__device__ __forceinline__ bool decode_unit(int X, int HG, int U, int* u, int* hg) {
  const int per = 8 * HG;
  const int blk = X / per, rem = X % per;
  *hg = rem / 8;
  *u = blk * 8 + rem % 8;
  return *u < U;
}

// Unit u (XCD u % 8) -> sequence and slice. When the batch is a multiple of 8
// every slice of sequence b gets a unit equal to b modulo 8, so its rows, ids
// and the selection that wrote them meet on XCD b % 8; otherwise slices of a
// sequence are consecutive units.
__device__ __forceinline__ void unit_seq(int u, int B, int splits, int* b, int* s) {
  if (B % 8 == 0) {
    const int t = u >> 3;
    *s = t % splits;
    *b = (t / splits) * 8 + (u & 7);
  } else {
    *b = u / splits;
    *s = u % splits;
  }
}

// Log-sum-exp merge of the row slices of one (sequence, head): 128 threads,
// four dims each. When the batch is a multiple of 8 the workgroups of sequence b
// sit on XCD b % 8, where its slices wrote their partials. Up to SM slices are
// merged per pass; every load of a pass (each slice's m, l and four partial
// dims) is requested before any is used.
template <int SM>
__global__ __launch_bounds__(128) void attn_combine_kernel(const float* __restrict__ part, int B, int splits, int Hq,
                                                           const int32_t* __restrict__ count, float* __restrict__ out,
                                                           float* __restrict__ lse) {
  const int x = blockIdx.x, d4 = threadIdx.x;
  int b, h;
  if (B % 8 == 0) {
    b = ((x >> 3) / Hq) * 8 + (x & 7);
    h = (x >> 3) % Hq;
  } else {
    b = x / Hq;
    h = x % Hq;
  }
  const float* base = part + ((size_t)b * splits * Hq + h) * PART;
  const size_t stride = (size_t)Hq * PART;
  float M = -INFINITY, L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < splits; s0 += SM) {
    f32x4 ov[SM];
    float mv[SM], lv[SM];
#pragma unroll
    for (int i = 0; i < SM; i++) {
      const float* ps = base + (size_t)min(s0 + i, splits - 1) * stride;
      ov[i] = *(const f32x4*)(ps + 4 * d4);
      mv[i] = s0 + i < splits ? ps[512] : -INFINITY;
      lv[i] = ps[513];
    }
    float Mp = M;
#pragma unroll
    for (int i = 0; i < SM; i++) Mp = fmaxf(Mp, mv[i]);
    if (Mp == -INFINITY) continue;
    const float r = exp2f(M - Mp);  // earlier passes, rescaled (0 when M was -inf)
    L *= r;
#pragma unroll
    for (int j = 0; j < 4; j++) acc[j] *= r;
#pragma unroll
    for (int i = 0; i < SM; i++) {
      const float wgt = exp2f(mv[i] - Mp);  // empty slices and padding have m = -inf -> 0
      if (wgt > 0.f) {
        L += wgt * lv[i];
#pragma unroll
        for (int j = 0; j < 4; j++) acc[j] += wgt * ov[i][j];
      }
    }
    M = Mp;
  }
  const bool bad = count && count[b] < 0;  // the selection failed: NaN outputs
  const float inv = bad ? __builtin_nanf("") : (L > 0.f ? 1.f / L : 0.f);
  *(f32x4*)(out + ((size_t)b * Hq + h) * LIT_KV_DIM + 4 * d4) = acc * inv;
  if (lse && d4 == 0) lse[(size_t)b * Hq + h] = bad ? __builtin_nanf("") : (L > 0.f ? M * LN2 + logf(L) : -INFINITY);
}

void launch_combine(const float* part, int B, int splits, int Hq, const int32_t* count, float* out, float* lse,
                    hipStream_t st) {
  const dim3 grid((unsigned)(B * Hq)), block(128);
  if (splits <= 2)
    attn_combine_kernel<2><<<grid, block, 0, st>>>(part, B, splits, Hq, count, out, lse);
  else if (splits <= 4)
    attn_combine_kernel<4><<<grid, block, 0, st>>>(part, B, splits, Hq, count, out, lse);
  else if (splits <= 8)
    attn_combine_kernel<8><<<grid, block, 0, st>>>(part, B, splits, Hq, count, out, lse);
  else
    attn_combine_kernel<16><<<grid, block, 0, st>>>(part, B, splits, Hq, count, out, lse);
}

// FP32 rows and queries: one workgroup per (sequence, head), fp32 VALU with an
// online softmax over chunks of 1024 list positions.
__global__ __launch_bounds__(256) void attn_f32_kernel(const float* __restrict__ q, int Hq, KvArr kv,
                                                       int N, const int32_t* __restrict__ ids,
                                                       const int32_t* __restrict__ count, int k_cap, int window,
                                                       float scale, float* __restrict__ out, float* __restrict__ lse) {
  __shared__ float xs[1024];
  __shared__ int rs[1024];
  __shared__ float red[8];
  const int b = blockIdx.x / Hq, h = blockIdx.x % Hq;
  const int tid = threadIdx.x;
  bool bad = false;  // count[b] < 0: the selection failed; the outputs say so with NaN
  RowList RL;
  RL.dense = ids == nullptr;
  RL.N = N;
  RL.lids = nullptr;
  if (RL.dense) {
    RL.ids = nullptr;
    RL.c = 0;
    RL.Wc = 0;
    RL.total = N;
  } else {
    RL.ids = ids + (size_t)b * k_cap;
    const int cap = min(k_cap, N);
    int c = count[b];
    bad = c < 0;
    c = c < 0 ? 0 : (c > cap ? cap : c);
    RL.c = c;
    RL.Wc = window;
    RL.total = c + window;
  }
  const float* qh = q + ((size_t)b * Hq + h) * LIT_KV_DIM;
  const uint8_t* kvb = kv.at(b, 0);
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int c0 = 0; c0 < RL.total; c0 += 1024) {
    const int len = min(1024, RL.total - c0);
    float cmax = -INFINITY;
    for (int p = tid; p < len; p += 256) {
      const int r = RL.row(c0 + p);
      float xv = -INFINITY;
      if (r >= 0) {
        const float* kr = (const float*)(kvb + kv.row * r);
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
      const float* kr = (const float*)(kvb + kv.row * r);
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
  const float inv = bad ? __builtin_nanf("") : (l > 0.f ? 1.f / l : 0.f);
  oh[tid] = o0 * inv;
  oh[tid + 256] = o1 * inv;
  if (lse && tid == 0) lse[(size_t)b * Hq + h] = bad ? __builtin_nanf("") : (l > 0.f ? m + logf(l) : -INFINITY);
}

// ---------------------------------------------------------------- BF16 rows, 16 heads per workgroup

// One workgroup of 4 waves: one sequence, one group of 16 query heads, one
// slice of the row list. The head groups of a slice sit on one XCD (workgroup
// ids equal modulo 8), so its L2 serves the slice's rows to all of them. Tiles
// of 64 rows go straight from global memory into LDS (global_load_lds, 16 bytes
// per lane: one wave instruction moves one 1 KiB row), double-buffered in two
// separate LDS arrays so that reading one buffer never waits for the loads into
// the other. Wave w:
//   scores: tile rows 16w .. +15, S^T = K Q^T on v_mfma_f32_16x16x32_bf16
//           (A = rows from LDS, B = the 16 queries in registers), the 16 K-steps
//           spread over four accumulators so that four MFMA chains are in flight;
//   output: dims 128w .. +127, O^T += V^T P^T on the same instruction, so that
//           a lane's output column is the head whose softmax it keeps; the V^T
//           operand is read transposed by ds_read_b64_tr_b16 (lane (g, s) points
//           at row 8g + s/4 (+4), dims 4(s % 4) .. +3 of the 16-dim block).
// The four waves post their tile maxima to LDS; P is taken against the shared
// running reference and retaken only when a maximum outgrows it by 2^8.
constexpr int MH_THREADS = 256;
constexpr int MH_WAVES = MH_THREADS / 64;
constexpr int MH_TR = 64;                           // rows per tile
constexpr int MH_ROWS_PER_WAVE = MH_TR / MH_WAVES;  // tile rows each wave loads
constexpr int MH_HEADS = 16;                        // query heads per workgroup
constexpr int MH_RS = 520;         // bf16 per LDS row: 1040 B keeps rows 16-byte aligned and spreads banks
constexpr int MH_PS = MH_TR + 8;   // bf16 per LDS row of P (one head)
constexpr int MH_TARGET = 256;     // workgroups aimed at: one per CU
constexpr int MH_ROWS_CAP = 1152;  // rows of a selection slice resolved up front (a multiple of MH_TR)
constexpr int MH_IDS_CACHE = 1024;  // ids copied to LDS up front (k_cap at most this; a multiple of 64)

struct MhTile {
  uint16_t v[MH_TR * MH_RS];
};

typedef short s16x4v __attribute__((ext_vector_type(4)));

// The 16 query rows of head group hg of sequence b into rows 0..15 of a tile
// buffer (heads past Hq repeat the last head: their outputs are never written).
__device__ __forceinline__ void mh_issue_q(const AttnParams& P, int b, int hg, MhTile& T) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < MH_HEADS / MH_WAVES; i++) {
    const int hl = (MH_HEADS / MH_WAVES) * wid + i;
    const int h = min(MH_HEADS * hg + hl, P.Hq - 1);
    const uint16_t* src = P.q + ((size_t)b * P.Hq + h) * LIT_KV_DIM + 8 * lane;
    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)(T.v + hl * MH_RS), 16, 0, 0);
  }
}

__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)
// vmcnt(16): all but the last 16 loads (one tile's rows of this wave) have landed
__device__ __forceinline__ void wait_vm_tile() { __builtin_amdgcn_s_waitcnt(0x4F70); }
static_assert(MH_ROWS_PER_WAVE == 16, "wait_vm_tile counts one load per row");

struct MhState {
  f32x4 o[8];   // O[head c16][dim 128 w + 16 nt + 4g + i]
  float m_run;  // running max of head c16 (log2 domain), the same in every wave
  float l_run;  // this lane's share of head c16's sum (its wave's rows)
};

// The row ids of this wave's share of a tile (wave-uniform), read before any
// of their loads is issued.
__device__ __forceinline__ void mh_row_ids(const int* rws, int (&rid)[MH_ROWS_PER_WAVE]) {
  const int wid = threadIdx.x >> 6;
#pragma unroll
  for (int v = 0; v < MH_ROWS_PER_WAVE / 4; v++) {
    const u32x4 r4 = *(const u32x4*)(rws + MH_ROWS_PER_WAVE * wid + 4 * v);
#pragma unroll
    for (int i = 0; i < 4; i++) rid[4 * v + i] = __builtin_amdgcn_readfirstlane((int)r4[i]);
  }
}

// One tile row (slot i of this wave's share) straight into LDS. A row that is
// not attended (-1) loads row 0 instead: its weight is 0, and a finite value
// keeps 0 * value = 0. BF16 rows: 64 lanes x 16 B, the row as it is. FP8 rows
// arrive raw in the row's slot, widened to BF16 in place before use (see
// mh_widen_fp8): bytes 0..447 the E4M3 dims (lanes 0-27), 448..575 the BF16
// RoPE dims (lanes 28-35), 576..583 the E8M0 scale bytes (a second, 4-byte
// load by lanes 0-1); the other lanes load nothing.
// The row arrays of one sequence (row n of each at its base + its row stride * n).
struct KvSeq {
  const uint8_t* d;
  const uint8_t* r;
  const uint8_t* s;
};

template <bool FP8>
__device__ __forceinline__ void mh_issue_row(const AttnParams& P, const KvSeq& K, int r, int i, MhTile& T) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t n = r >= 0 ? r : 0;
  uint16_t* dst = T.v + (MH_ROWS_PER_WAVE * wid + i) * MH_RS;
  if (!FP8) {
    const uint8_t* src = K.d + P.kd.row * n + 16 * lane;
    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
  } else {
    if (lane < 36) {
      const uint8_t* src = lane < 28 ? K.d + P.kd.row * n + 16 * lane : K.r + P.kr.row * n + 16 * (lane - 28);
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
    }
    if (lane < 2)
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(K.s + P.ks.row * n + 4 * lane),
                                       (__attribute__((address_space(3))) void*)(reinterpret_cast<uint8_t*>(dst) + 576),
                                       4, 0, 0);
  }
}

// A tile of raw FP8 rows widened to the BF16 row layout in place: thread t
// takes row t / 4, quarter t % 4 (112 E4M3 dims and 16 RoPE dims), reads its
// bytes into registers, and after a barrier writes them back as BF16. An
// E4M3 value times its group's power of two is exact in BF16, which the scaled
// conversion instruction produces (the same values the FP8 decode gives).
__device__ __forceinline__ void mh_widen_fp8(MhTile& T) {
  const int tid = threadIdx.x;
  const int r = tid >> 2, qq = tid & 3;
  uint8_t* row = reinterpret_cast<uint8_t*>(T.v + r * MH_RS);
  u32x4 f[7], ro[2];
#pragma unroll
  for (int i = 0; i < 7; i++) f[i] = *(const u32x4*)(row + 112 * qq + 16 * i);
#pragma unroll
  for (int i = 0; i < 2; i++) ro[i] = *(const u32x4*)(row + 448 + 32 * qq + 16 * i);
  const u32x2 sc = *(const u32x2*)(row + 576);
  lds_barrier();
#pragma unroll
  for (int j = 0; j < 14; j++) {
    const int d0 = 112 * qq + 8 * j;  // dims d0 .. d0+7 share one 64-dim scale group
    const int grp = d0 >> 6;
    const float scl = e8m0_f32((sc[grp >> 2] >> (8 * (grp & 3))) & 255u);
    const uint32_t w0 = f[j >> 1][2 * (j & 1)], w1 = f[j >> 1][2 * (j & 1) + 1];
    u32x4 o;
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scl, false));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scl, true));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scl, false));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scl, true));
    *(u32x4*)(row + 2 * d0) = o;
  }
#pragma unroll
  for (int i = 0; i < 2; i++) *(u32x4*)(row + 2 * LIT_KV_FP8_DIMS + 32 * qq + 16 * i) = ro[i];
  lds_barrier();
}

// This wave's share of a whole tile.
template <bool FP8>
__device__ __forceinline__ void mh_issue(const AttnParams& P, const KvSeq& K, const int* rws, MhTile& T) {
  int rid[MH_ROWS_PER_WAVE];
  mh_row_ids(rws, rid);
#pragma unroll
  for (int i = 0; i < MH_ROWS_PER_WAVE; i++) mh_issue_row<FP8>(P, K, rid[i], i, T);
}

// nvalid: rows 0 .. nvalid-1 of the tile are attended, the rest are padding.
// When NT is given, this wave's loads of that next tile (rows nrid) are issued
// one per K-step of the scores, so that their issue overlaps the multiplies.
template <bool FP8>
__device__ __forceinline__ void mh_tile(const AttnParams& P, const MhTile& T, int nvalid, const u32x4 (&qreg)[16],
                                        MhState& S, float (*smax)[16], uint16_t* pbuf, MhTile* NT, const KvSeq& K,
                                        const int (&nrid)[MH_ROWS_PER_WAVE]) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  // S^T: rows 16w + 4g + i, head c16. K-step j accumulates into chain j % 4;
  // the operands of step j + KD are read while step j multiplies (the
  // scheduling barrier keeps the compiler from hoisting every read)
  f32x4 acc[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  const uint16_t* krow = T.v + (16 * wid + c16) * MH_RS + 8 * g;
  constexpr int KD = 4;  // operand reads in flight ahead of the multiply
  static_assert(MH_ROWS_PER_WAVE == 16, "one next-tile row per K-step");
  u32x4 kq[KD];
#pragma unroll
  for (int j = 0; j < KD; j++) kq[j] = *(const u32x4*)(krow + 32 * j);
#pragma unroll
  for (int j = 0; j < 16; j++) {
    const u32x4 ka = kq[j % KD];
    if (j + KD < 16) kq[j % KD] = *(const u32x4*)(krow + 32 * (j + KD));
    if (NT) mh_issue_row<FP8>(P, K, nrid[j], j, *NT);
    acc[j & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka), __builtin_bit_cast(bf16x8, qreg[j]),
                                                         acc[j & 3], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  float xs[4];
  float tmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const bool valid = 16 * wid + 4 * g + i < nvalid;
    const float sv = (acc[0][i] + acc[1][i]) + (acc[2][i] + acc[3][i]);
    xs[i] = valid ? sv * P.scale_log2 : -INFINITY;
    tmax = fmaxf(tmax, xs[i]);
  }
  tmax = max_xor32(max_xor16(tmax));
  if (g == 0) smax[wid][c16] = tmax;
  // P = exp2(x - m) for the tile's rows, rounded to bf16 into pbuf; returns the
  // lane's share of sum P
  auto write_p = [&](float m_use) {
    float psum = 0.f;
    uint32_t hbits[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float pv = exp2f(xs[i] - m_use);
      psum += pv;
      const uint32_t bits = __float_as_uint(pv);
      hbits[i] = (bits + 0x7fffu + ((bits >> 16) & 1u)) >> 16;  // round to nearest even
    }
    u32x2 pk;
    pk[0] = hbits[0] | (hbits[1] << 16);
    pk[1] = hbits[2] | (hbits[3] << 16);
    *(u32x2*)(pbuf + c16 * MH_PS + 16 * wid + 4 * g) = pk;
    return psum;
  };
  auto tile_max = [&]() {
    return fmaxf(S.m_run, fmaxf(fmaxf(smax[0][c16], smax[1][c16]), fmaxf(smax[2][c16], smax[3][c16])));
  };
  // The running max m_run is only a reference point: P is taken against the
  // one every wave already holds, and the four waves' tile maxima (posted to
  // smax) are checked after the barrier that publishes P. Only when some
  // head's maximum passed m_run + 8 (weights above 2^8) is P taken again
  // against the new maximum and the running state rescaled; the first tile
  // (m_run = -inf in every lane) always takes that path.
  float alpha = 1.f;
  if (__any(S.m_run == -INFINITY)) {
    lds_barrier();
    const float m_new = tile_max();
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    alpha = exp2f(S.m_run - m_use);
    S.m_run = m_new;
    S.l_run = S.l_run * alpha + write_p(m_use);
    lds_barrier();
  } else {
    const float psum = write_p(S.m_run);
    lds_barrier();
    const float m_new = tile_max();
    if (__any(m_new > S.m_run + 8.f)) {  // the same verdict in every wave: all read the same smax
      alpha = exp2f(S.m_run - m_new);
      S.m_run = m_new;
      S.l_run = S.l_run * alpha + write_p(m_new);
      lds_barrier();
    } else {
      S.l_run += psum;
    }
  }
  // rescale O (this lane's head) when its reference moved
  if (alpha != 1.0f) {
#pragma unroll
    for (int nt = 0; nt < 8; nt++)
#pragma unroll
      for (int i = 0; i < 4; i++) S.o[nt][i] *= alpha;
  }
  // O += P V over the 64 rows (two K-steps of 32, eight 16-dim blocks each);
  // the V operands of step it + VD are read while step it multiplies
  const uint16_t* vbase = T.v + (8 * g + (c16 >> 2)) * MH_RS + 128 * wid + 4 * (c16 & 3);
  auto vld = [&](int it) {
    const uint16_t* vb = vbase + 32 * (it >> 3) * MH_RS + 16 * (it & 7);
    const s16x4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4v*)vb);
    const s16x4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4v*)(vb + 4 * MH_RS));
    u32x4 bv;
    bv[0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
    bv[1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
    bv[2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
    bv[3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
    return bv;
  };
  bf16x8 pa[2];
#pragma unroll
  for (int kk = 0; kk < 2; kk++) pa[kk] = __builtin_bit_cast(bf16x8, *(const u32x4*)(pbuf + c16 * MH_PS + 32 * kk + 8 * g));
  constexpr int VD = 4;  // transposed reads in flight ahead of the multiply
  u32x4 vq[VD];
#pragma unroll
  for (int it = 0; it < VD; it++) vq[it] = vld(it);
#pragma unroll
  for (int it = 0; it < 16; it++) {
    const u32x4 va = vq[it % VD];
    if (it + VD < 16) vq[it % VD] = vld(it + VD);
    S.o[it & 7] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va), pa[it >> 3], S.o[it & 7], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <bool FP8>
__global__ __launch_bounds__(MH_THREADS, 1) void attn_mh_kernel(AttnParams P) {
  __shared__ MhTile TA, TB;
  __shared__ __align__(16) uint16_t pbuf[MH_HEADS * MH_PS];
  __shared__ __align__(16) int rows_all[MH_ROWS_CAP];  // the slice's rows, or a ring of 4 tiles for long dense slices
  __shared__ float smax[MH_WAVES][16];
  __shared__ float ssum[MH_WAVES][16];
  __shared__ int part[16];
  const int HG = (P.Hq + MH_HEADS - 1) / MH_HEADS;
  int u, hg;
  if (!decode_unit(blockIdx.x, HG, P.B * P.splits, &u, &hg)) return;
  int b, s;
  unit_seq(u, P.B, P.splits, &b, &s);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int Hq = P.Hq;
  KvSeq K;
  K.d = P.kd.at(b, 0);
  K.r = FP8 ? P.kr.at(b, 0) : nullptr;
  K.s = FP8 ? P.ks.at(b, 0) : nullptr;
  // the count as a scalar load (issued first: its wait does not hold the
  // vector loads below)
  const int count_b = P.ids ? *(const __attribute__((address_space(4))) int32_t*)(P.count + b) : 0;
  // the queries travel first, into the second tile buffer, while the row list is built
  mh_issue_q(P, b, hg, TB);
  // The sequence's ids travel with them (all k_cap, so that their copy does not
  // wait for the count), into the same buffer after the 16 query rows; the
  // row list then reads LDS, and the count's load and the ids' copy are one
  // round trip instead of two dependent ones.
  int* ids_l = reinterpret_cast<int*>(TB.v + MH_HEADS * MH_RS);
  const bool ids_cached = P.ids != nullptr && P.k_cap <= MH_IDS_CACHE;
  if (ids_cached) {
    // a fixed count of copies per wave (slots past k_cap repeat the last id and
    // are never read), so that the loads issued after them are counted exactly
    const int32_t* src = P.ids + (size_t)b * P.k_cap;
#pragma unroll
    for (int it = 0; it < MH_IDS_CACHE / (64 * MH_WAVES); it++) {
      const int j0 = 64 * (wid + MH_WAVES * it);
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(src + min(j0 + lane, P.k_cap - 1)),
                                       (__attribute__((address_space(3))) void*)(ids_l + j0), 4, 0, 0);
    }
  }
  // A selection's list holds the window rows first, and slice s takes the
  // list's tiles s, s + splits, ...: when its first tile is window rows (BF16),
  // their rows are known now and their loads go out behind the ids', into
  // registers, so that they land while the ids are read and the row list is
  // built (loads into registers, not LDS: reads of LDS would otherwise wait
  // for them). They are stored to the first tile buffer before the tile loop.
  const bool early = !FP8 && P.ids != nullptr && P.window >= MH_TR * (s + 1);
  u32x4 t0[MH_ROWS_PER_WAVE];
  __builtin_amdgcn_sched_barrier(0);  // the ids' copy is issued before these loads
  if (early) {
#pragma unroll
    for (int i = 0; i < MH_ROWS_PER_WAVE; i++) {
      const int64_t n = P.N - P.window + MH_TR * s + MH_ROWS_PER_WAVE * wid + i;
      t0[i] = *(const u32x4*)(K.d + P.kd.row * n + 16 * lane);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  bool bad = false;  // count[b] < 0: the selection failed; the outputs say so with NaN
  RowList RL;
  RL.dense = P.ids == nullptr;
  RL.N = P.N;
  RL.lids = ids_cached ? (lds_ids_t)ids_l : nullptr;
  if (RL.dense) {
    RL.ids = nullptr;
    RL.c = 0;
    RL.Wc = 0;
    RL.total = P.N;
  } else {
    RL.ids = P.ids + (size_t)b * P.k_cap;
    const int cap = min(P.k_cap, P.N);
    int c = count_b;
    bad = c < 0;
    c = c < 0 ? 0 : (c > cap ? cap : c);
    RL.c = c;
    RL.Wc = P.window;
    RL.total = c + P.window;
  }
  if (ids_cached) {
    // this wave's share of the ids (and queries) has landed; the first tile's
    // loads, issued after them, may still be in flight
    if (early)
      wait_vm_tile();
    else
      wait_vm0();
  }
  lds_barrier();  // ... and every wave's
  // Every row of a selection slice is resolved here (the planner keeps those
  // slices within MH_ROWS_CAP) and compacted, so the attended rows are list
  // positions 0 .. n-1 and the tile loop reads nothing but the tiles. Longer
  // slices are dense: their rows are their positions, computed per tile.
  const bool all_rows = !RL.dense;
  int n;                        // attended rows of the slice
  int p0 = 0, p1 = 0;           // a dense slice's positions
  if (all_rows) {
    // slice-local index i -> list position: tile s + splits * (i / MH_TR)
    const int T = (RL.total + MH_TR - 1) / MH_TR;
    const int ntile = T > s ? (T - s + P.splits - 1) / P.splits : 0;
    const int i0 = early ? MH_TR : 0;  // an early first tile is complete: 64 window rows
    const int nloc = ntile * MH_TR;
    constexpr int PER = (MH_ROWS_CAP + MH_THREADS - 1) / MH_THREADS;
    static_assert(PER == 5, "the LDS reads below are written out for five positions per thread");
    int r[PER], p[PER], f[PER];
#pragma unroll
    for (int k = 0; k < PER; k++) {
      const int i = i0 + tid + MH_THREADS * k;
      p[k] = i < nloc ? MH_TR * (s + P.splits * (i / MH_TR)) + i % MH_TR : RL.total;
    }
    if (RL.lids && RL.c > 0) {
      // the ids from LDS in one asm block that waits for its own reads: the
      // compiler would otherwise make each read wait for every load in flight
      // (it cannot tell this copy, which has landed, from the tile loads)
      uint32_t a[PER];
#pragma unroll
      for (int k = 0; k < PER; k++)
        a[k] = (uint32_t)(uintptr_t)(RL.lids + max(min(p[k] - RL.Wc, RL.c - 1), 0));
      asm volatile(
          "ds_read_b32 %0, %5\n\tds_read_b32 %1, %6\n\tds_read_b32 %2, %7\n\tds_read_b32 %3, %8\n\t"
          "ds_read_b32 %4, %9\n\ts_waitcnt lgkmcnt(0)"
          : "=v"(f[0]), "=v"(f[1]), "=v"(f[2]), "=v"(f[3]), "=v"(f[4])
          : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4])
          : "memory");
    } else {
#pragma unroll
      for (int k = 0; k < PER; k++) f[k] = RL.fetch(p[k]);
      // (their loads waited for here, on this path only: where the two paths
      // meet, f holds nothing in flight)
      __builtin_amdgcn_s_waitcnt(0);
    }
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < PER; k++) {
      r[k] = RL.resolve(p[k], f[k]);
      cnt += r[k] >= 0;
    }
    int pos = block_excl_scan1<MH_WAVES>(cnt, part, &n);
    pos += i0;
#pragma unroll
    for (int k = 0; k < PER; k++)
      if (r[k] >= 0) rows_all[pos++] = r[k];
    n += i0;
    lds_barrier();
    const int upto = (n + MH_TR - 1) / MH_TR * MH_TR;
    for (int i = max(n, i0) + tid; i < upto; i += MH_THREADS) rows_all[i] = -1;
  } else {
    p0 = s * P.rows_per_split;
    p1 = min(RL.total, p0 + P.rows_per_split);
    n = max(p1 - p0, 0);
    for (int i = tid; i < 2 * MH_TR; i += MH_THREADS) {
      const int p = p0 + i;
      rows_all[i] = p < p1 ? p : -1;
    }
  }
  // (one LDS array, so that the compiler can tell its reads from the tile loads in flight)
  auto tile_rows = [&](int tt) -> const int* { return rows_all + MH_TR * (all_rows ? tt : (tt & 3)); };
  // a dense slice's first tile needs no row list: its loads go out now,
  // alongside the queries'
  if (!all_rows) {
    lds_barrier();
    if (0 < n) mh_issue<FP8>(P, K, tile_rows(0), TA);
  }
  // the queries as B operands, from the second tile buffer: K-step j, lane
  // (g, c16) holds dims 32j + 8g .. +7 of head c16 of the group
  if (early)
    wait_vm_tile();
  else
    wait_vm0();
  lds_barrier();
  u32x4 qreg[16];
#pragma unroll
  for (int j = 0; j < 16; j++) qreg[j] = *(const u32x4*)(TB.v + c16 * MH_RS + 32 * j + 8 * g);
  if (early) {
#pragma unroll
    for (int i = 0; i < MH_ROWS_PER_WAVE; i++) *(u32x4*)(TA.v + (MH_ROWS_PER_WAVE * wid + i) * MH_RS + 8 * lane) = t0[i];
  }
  lds_barrier();
  if (all_rows && !early && 0 < n) mh_issue<FP8>(P, K, tile_rows(0), TA);

  MhState S;
#pragma unroll
  for (int nt = 0; nt < 8; nt++) S.o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  S.m_run = -INFINITY;
  S.l_run = 0.f;

  // tile t uses buffer t & 1; the loads of tile t + 1 go into the other
  // buffer (free since the barrier that ended tile t - 1) during tile t's
  // score multiplies, so each tile waits only for its own loads
#pragma unroll 1
  for (int t = 0; MH_TR * t < n; t += 2) {
#pragma unroll
    for (int ab = 0; ab < 2; ab++) {
      const int tt = t + ab;
      const int q0 = MH_TR * tt;
      if (q0 >= n) break;
      wait_vm0();
      if (!all_rows && tid < MH_TR) {
        const int p = p0 + q0 + 2 * MH_TR + tid;
        rows_all[MH_TR * ((tt + 2) & 3) + tid] = p < p1 ? p : -1;
      }
      lds_barrier();
      if (FP8) mh_widen_fp8(ab == 0 ? TA : TB);
      const bool more = q0 + MH_TR < n;
      int nrid[MH_ROWS_PER_WAVE];
      if (more) mh_row_ids(tile_rows(tt + 1), nrid);
      mh_tile<FP8>(P, ab == 0 ? TA : TB, n - q0, qreg, S, smax, pbuf, more ? (ab == 0 ? &TB : &TA) : nullptr, K,
              nrid);
      // no barrier here: the next tile's opening barrier orders this tile's
      // reads of its buffer, pbuf and smax before anything rewrites them
    }
  }

  // l per head: the four waves' rows
  const float lw = sum_xor32(sum_xor16(S.l_run));  // every lane takes part in the lane swaps
  if (g == 0) ssum[wid][c16] = lw;
  lds_barrier();
  const int hh = MH_HEADS * hg + c16;
  const float Ls = (ssum[0][c16] + ssum[1][c16]) + (ssum[2][c16] + ssum[3][c16]);
  if (hh < Hq) {
    if (P.splits == 1) {
      float* oh = P.out + ((size_t)b * Hq + hh) * LIT_KV_DIM + 128 * wid + 4 * g;
      const float inv = bad ? __builtin_nanf("") : (Ls > 0.f ? 1.f / Ls : 0.f);
#pragma unroll
      for (int nt = 0; nt < 8; nt++) *(f32x4*)(oh + 16 * nt) = S.o[nt] * inv;
      if (P.lse && wid == 0 && g == 0)
        P.lse[(size_t)b * Hq + hh] = bad ? __builtin_nanf("") : (Ls > 0.f ? S.m_run * LN2 + logf(Ls) : -INFINITY);
    } else {
      float* ph = P.part + (((size_t)b * P.splits + s) * Hq + hh) * PART;
#pragma unroll
      for (int nt = 0; nt < 8; nt++) *(f32x4*)(ph + 128 * wid + 16 * nt + 4 * g) = S.o[nt];
      if (wid == 0 && g == 0) {
        ph[512] = S.m_run;
        ph[513] = Ls;
      }
    }
  }
}

// Slices of the row list per sequence. Up to one round of workgroups (slices x
// head groups x sequences <= MH_TARGET), and selection slices (sparse) no
// longer than MH_ROWS_CAP rows; within that, the count that minimises the
// measured cost: ~2.1 us per 64-row tile of a slice, plus ~5 us for the
// combine kernel once the rows are split. (A 128-row window is then one slice
// of two tiles rather than two of one tile and a combine.)
void plan_mh(int B, int HG, int rows_max, bool sparse, int* splits, int* rows_per_split) {
  constexpr double TILE_US = 2.1, COMBINE_US = 5.0;
  const int tiles = std::max(1, (rows_max + MH_TR - 1) / MH_TR);
  const int want = std::max(1, (MH_TARGET + B * HG - 1) / (B * HG));
  const int s_min = sparse ? std::max(1, (tiles * MH_TR + MH_ROWS_CAP - 1) / MH_ROWS_CAP) : 1;
  const int s_max = std::max(s_min, std::min(tiles, want));
  int best = s_min;
  double best_us = 1e30;
  for (int s = s_min; s <= s_max; s++) {
    const double us = ((tiles + s - 1) / s) * TILE_US + (s > 1 ? COMBINE_US : 0.0);
    if (us < best_us) {
      best_us = us;
      best = s;
    }
  }
  const int tiles_per = (tiles + best - 1) / best;
  *splits = (tiles + tiles_per - 1) / tiles_per;
  *rows_per_split = tiles_per * MH_TR;
}

}  // namespace
}  // namespace lit

using namespace lit;

extern "C" size_t lit_attn_workspace_bytes(int32_t B, int32_t Hq, int32_t N) {
  if (B < 1 || Hq < 1 || N < 1) return 0;
  // A bound on the slices of any call on these shapes, whatever its k_cap and
  // window: a call plans at most min(k_cap, N) + window <= N + LIT_MAX_WINDOW
  // selected rows or N dense rows, and plan_mh never picks more slices than
  // the larger of the round's share (capped by the tiles) and the slices that
  // the LDS row list forces on the longest selection.
  const int HGm = (Hq + MH_HEADS - 1) / MH_HEADS;
  const int tiles = (N + LIT_MAX_WINDOW + MH_TR - 1) / MH_TR;
  const int want = std::max(1, (MH_TARGET + B * HGm - 1) / (B * HGm));
  const int s_forced = (tiles * MH_TR + MH_ROWS_CAP - 1) / MH_ROWS_CAP;
  const int s = std::max(std::min(tiles, want), s_forced);
  if (s <= 1) return 256;
  return round_up((size_t)B * s * Hq * PART * sizeof(float), 256);
}

namespace lit {
namespace {

lit_status scratch_address(const char* who, void** out);

// The attention call behind both entry points: `ws` is the caller's workspace;
// with from_scratch the library's scratch array takes its place once the
// arguments are validated (a plan larger than the array is refused the same way
// as a short workspace).
lit_status attn_decode(const char* who, bool from_scratch, const void* q, lit_dtype q_dtype, int32_t Hq, const lit_kv* kv, int32_t B,
                       const int32_t* ids, const int32_t* count, int32_t k_cap, int32_t window, float scale,
                       float* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
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
  if (!aligned(q, 16) || !aligned(kv->data, 16) || (kv->rope && !aligned(kv->rope, 16)) || !aligned(out, 16) ||
      (kv->scale && !aligned(kv->scale, 4)))
    return fail(LIT_ERR_ALIGN, "%s: q, kv->data, kv->rope and out must be 16-byte aligned, kv->scale 4-byte", who);
  KvArr kd, kr, ks;
  const lit_status kst = kv_arrays(kv, &kd, &kr, &ks, who);
  if (kst != LIT_OK) return kst;
  hipStream_t st = (hipStream_t)stream;
  if (kv->dtype == LIT_F32) {
    attn_f32_kernel<<<dim3((unsigned)(B * Hq)), dim3(256), 0, st>>>((const float*)q, Hq, kd, N,
                                                                     ids, count, k_cap, Wc, scale, out, lse);
    LIT_CHECK_LAUNCH(who);
    return LIT_OK;
  }
  if (ws && !aligned(ws, 16)) return fail(LIT_ERR_ALIGN, "%s: workspace must be 16-byte aligned", who);
  // a selection holds at most N distinct ids (the kernel clamps count[b] to
  // min(k_cap, N)), so a k_cap beyond N plans no more rows than N does
  const int rows_max = ids ? (std::min(k_cap, N) + Wc) : N;
  AttnParams P;
  const int HGm = (Hq + MH_HEADS - 1) / MH_HEADS;
  plan_mh(B, HGm, rows_max, ids != nullptr, &P.splits, &P.rows_per_split);
  P.B = B;
  if (P.splits > 1) {
    const size_t need = round_up((size_t)B * P.splits * Hq * PART * sizeof(float), 256);
    if (from_scratch) {
      const lit_status sst = scratch_address(who, &ws);
      if (sst != LIT_OK) return sst;
      ws_bytes = (size_t)LIT_ATTN_SCRATCH_BYTES;
    }
    if (!ws || ws_bytes < need)
      return fail(LIT_ERR_WORKSPACE, "%s: %zu bytes of partial results needed, the %s holds %zu", who, need,
                  from_scratch ? "library's scratch array" : "workspace given", ws_bytes);
  }
  P.q = (const uint16_t*)q;
  P.Hq = Hq;
  P.kv_dtype = (int)kv->dtype;
  P.kd = kd;
  P.kr = kr;
  P.ks = ks;
  P.N = N;
  P.ids = ids;
  P.count = count;
  P.k_cap = k_cap;
  P.window = Wc;
  P.scale_log2 = scale * LOG2E;
  P.out = out;
  P.lse = lse;
  P.part = (float*)ws;
  const int U = B * P.splits;
  const dim3 grid((unsigned)(((U + 7) / 8) * 8 * HGm));
  if (kv->dtype == LIT_FP8E4M3_G64_ROPE_BF16)
    attn_mh_kernel<true><<<grid, dim3(MH_THREADS), 0, st>>>(P);
  else
    attn_mh_kernel<false><<<grid, dim3(MH_THREADS), 0, st>>>(P);
  LIT_CHECK_LAUNCH(who);
  if (P.splits > 1) {
    launch_combine((const float*)ws, B, P.splits, Hq, ids ? count : nullptr, out, lse, st);
    LIT_CHECK_LAUNCH(who);
  }
  return LIT_OK;
}

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_dev[MAX_DEVICES];

lit_status scratch_address(const char* who, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(LIT_ERR_LAUNCH, "%s: no current HIP device: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEVICES) return fail(LIT_ERR_LAUNCH, "%s: device %d beyond %d", who, dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(LIT_ERR_LAUNCH, "%s: cannot find the scratch array on device %d: %s", who, dev, hipGetErrorString(e));
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return LIT_OK;
}

}  // namespace
}  // namespace lit

extern "C" lit_status lit_sparse_attn_decode(const void* q, lit_dtype q_dtype, int32_t Hq, const lit_kv* kv, int32_t B,
                                             const int32_t* ids, const int32_t* count, int32_t k_cap, int32_t window,
                                             float scale, float* out, float* lse, void* ws, size_t ws_bytes,
                                             void* stream) {
  clear_error();
  return attn_decode("lit_sparse_attn_decode", false, q, q_dtype, Hq, kv, B, ids, count, k_cap, window, scale, out, lse, ws,
                     ws_bytes, stream);
}

extern "C" lit_status lit_sparse_attn_decode_noalloc(const void* q, lit_dtype q_dtype, int32_t Hq, const lit_kv* kv,
                                                     int32_t B, const int32_t* ids, const int32_t* count,
                                                     int32_t k_cap, int32_t window, float scale, float* out,
                                                     float* lse, void* stream) {
  clear_error();
  return attn_decode("lit_sparse_attn_decode_noalloc", true, q, q_dtype, Hq, kv, B, ids, count, k_cap, window, scale,
                     out, lse, nullptr, 0, stream);
}
