// idx_score.hip - a1: lightning-indexer scores on MFMA (gfx950).
//
// [ARCH] ai-muninn.com, "284B 塞得進 128GB、長 context 還跑得動:DeepSeek-V4-Flash 打的是
// KV cache,不是參數量", section "(B) 只讀你需要的": a light indexer scores every
// compressed entry with its own 128-dim key (index_comp_kv). The score form is the
// "native ReLU-MQA" named with the gated equation of zhichai.net, "FlashMemory-DeepSeek-V4
// 深度解读" (second reply), without the sigmoid:
//     s[n] = sum_h w[h] * max(0, q[h] . k[n])
//
// Shape of the work: per sequence a [H x 128] x [128 x N] product, reduced over h
// with the weights. At 64 heads that is 64 flop per key byte, far below the MFMA
// ridge (~312 flop/B), so the kernel is HBM-bound on the key stream; MFMA keeps
// the arithmetic off the VALU (fp32 VALU alone would be ~3x slower than HBM).
//
// Mapping (v_mfma_f32_16x16x32_bf16, wave64): A = 16 heads x 32 dims of q (staged
// in LDS once per workgroup, already in operand order, and held in registers
// when the workgroup scores one query), B = 32 dims x 16 entries
// of keys loaded straight from HBM into registers (lane l holds entry l%16 and 8
// consecutive dims), C = 16 heads x 16 entries. The dims are assigned to the 128
// K positions so that each lane's four 16-byte key loads cover one contiguous
// 64-byte piece per K-step; A uses the same assignment, so the dot products are
// unchanged. A wave handles 64 entries per step (4 column groups), a workgroup
// handles S chunks of 256 entries; the key-norm side output is one value per
// 256-entry chunk.
#include <math.h>

#include "exact.h"
#include "lit_common.h"

namespace lit {
namespace {

constexpr int CHUNK = LIT_KNORM_CHUNK;  // 256 entries: 4 waves x 64
constexpr int KEY_RING = 3;             // key register buffers per wave (half-steps of 32 entries)
constexpr int KEY_RING_1Q = 2;          // the same for one query per workgroup (its q operands take the registers)
constexpr bool KEY_CONTIG = true;       // whole-line key loads, turned into operands through LDS
static_assert(CHUNK == 256, "kernel tiling assumes 256-entry chunks");

// Per-lane weights of the heads this lane's accumulators hold.
template <int MT>
__device__ __forceinline__ void load_lane_weights(const float* wlds, float (&wr)[MT][4]) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int mt = 0; mt < MT; mt++)
#pragma unroll
    for (int i = 0; i < 4; i++) wr[mt][i] = wlds[16 * mt + 4 * g + i];
}

// max(x, 0) as an integer max on the bits: negative values (and -0) become +0.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Epilogue shared by both dtypes: weighted ReLU over the lane's heads, summed
// across the four 16-lane groups (which hold the other heads of the same
// entry) by lane swaps; every lane of the entry ends with the same sum.
template <int MT>
__device__ __forceinline__ float weighted_relu(const f32x4 (&acc)[MT], const float (&wr)[MT][4]) {
  float p = 0.f;
#pragma unroll
  for (int mt = 0; mt < MT; mt++)
#pragma unroll
    for (int i = 0; i < 4; i++) p = fmaf(wr[mt][i], relu_bits(acc[mt][i]), p);
  return sum_xor32(sum_xor16(p));
}

// Upper bound of a key norm from a computed sum of squares m of 128 values:
// 128 x 2^-126 covers any product lost below the normal range, and the factor
// the fp32 rounding of the sum (<= 128 x 2^-24 relative for sequential adds,
// taken four times over for the matrix cores' accumulation, as for the scores)
// and of the sqrt.
__device__ __forceinline__ float norm_bound(float m) { return sqrtf(m + 0x1p-119f) * (1.0f + 0x1p-14f); }

// The two sums the exact selection scales its rounding bound by, written
// after the key-norm bounds and group maxima: sum_h |w_h| * ||q_h|| and
// sum_h |w_h|, in fp64 (the squares of bf16 or fp32 values are exact there),
// each as the two 32-bit words of a double. One wave reads the per-head terms
// (lanes past the staged heads count 0).
__device__ __forceinline__ void write_q_bounds(const double* qn, const double* wa, int nheads, float* hb) {
  const int lane = threadIdx.x & 63;
  double q = lane < nheads ? qn[lane] : 0.0, a = lane < nheads ? wa[lane] : 0.0;
  q = wave_sum_f64_dpp(q);
  a = wave_sum_f64_dpp(a);
  if (lane == 0) {
    uint32_t* u = reinterpret_cast<uint32_t*>(hb);
    const uint64_t qb = (uint64_t)__double_as_longlong(q), ab = (uint64_t)__double_as_longlong(a);
    u[0] = (uint32_t)qb;
    u[1] = (uint32_t)(qb >> 32);
    u[2] = (uint32_t)ab;
    u[3] = (uint32_t)(ab >> 32);
  }
}

// Loads the keys of 32 entries (2 column groups of 16) as B operands. Entries
// at or past N load row N-1 instead (in bounds; their scores are never stored
// and a real row's norm keeps the chunk bound valid), so no load sits in a
// branch and later half-steps' loads stay in flight during this one's math.
__device__ __forceinline__ void load_keys_half(const uint16_t* kb, int base, int N, int g, int c,
                                               u32x4 (&kr)[2][4]) {
#pragma unroll
  for (int G = 0; G < 2; G++) {
    const int e = min(base + 16 * G + c, N - 1);
#pragma unroll
    for (int j = 0; j < 4; j++)
      kr[G][j] = __builtin_nontemporal_load((const u32x4*)(kb + (size_t)e * LIT_IDX_DIM + 8 * g + 32 * j));
  }
}

// Contiguous form: the 32 rows of a half-step are one 8 KB block; instruction i
// reads its 1 KB (rows 4i .. 4i+3, lane l: row 4i + l/16, dims 8(l%16) .. +7),
// so every request covers whole cache lines. Rows at or past N read row N-1.
__device__ __forceinline__ void load_keys_contig(const uint16_t* kb, int base, int N, int lane, u32x4 (&kr)[8]) {
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int e = min(base + 4 * i + (lane >> 4), N - 1);
    kr[i] = __builtin_nontemporal_load((const u32x4*)(kb + (size_t)e * LIT_IDX_DIM + 8 * (lane & 15)));
  }
}

// Wave-private LDS slab for turning the contiguous block into B operands:
// 32 rows of 16 pieces of 16 bytes plus one pad piece (272-byte rows, so that
// the 16 lanes reading one piece of 16 rows hit distinct banks).
constexpr int KT_LD = 17;
__device__ __forceinline__ void keys_to_operands(u32x4* slab, const u32x4 (&kr)[8], int lane, int g, int c,
                                                 u32x4 (&op)[2][4]) {
#pragma unroll
  for (int i = 0; i < 8; i++) slab[(4 * i + (lane >> 4)) * KT_LD + (lane & 15)] = kr[i];
  // operand (G, j), lane (g, c): row 16G + c, piece g + 4j (dims 8g + 32j .. +7);
  // LDS keeps one wave's accesses in order, so the reads see the writes
#pragma unroll
  for (int G = 0; G < 2; G++)
#pragma unroll
    for (int j = 0; j < 4; j++) op[G][j] = slab[(16 * G + c) * KT_LD + g + 4 * j];
}

// Scores of the lane's entry (lane = 16 g + c holds entry base + lane): the
// allowed mask and the visible length nv applied (entries at or past nv are
// not visible to the query and score -inf), the score stored, and the group
// maximum returned in the group's last lane (c = 15; a running maximum along
// the 16-lane row on DPP shifts; entries at or past N count as -inf).
__device__ __forceinline__ float store_score(float v, int e, int N, int nv, const uint8_t* ab, float* sb) {
  if (e < N) {
    if (e >= nv || (ab && ab[e] == 0)) v = -INFINITY;
    sb[e] = v;
  } else {
    v = -INFINITY;
  }
  constexpr uint32_t NEG_INF = 0xff800000u;
  v = fmaxf(v, __uint_as_float(dpp_u32<0x111>(NEG_INF, __float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<0x112>(NEG_INF, __float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<0x114>(NEG_INF, __float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u32<0x118>(NEG_INF, __float_as_uint(v))));
  return v;
}

// A wave works through its 64 entries of each chunk in two half-steps of 32
// (two column groups); its keys pass through a ring of NB register buffers, so
// NB - 1 half-steps (NB - 1 times 8 KB per wave) are in flight while one is
// multiplied (several queries: three buffers measured fastest, a fourth adds
// registers, not bandwidth). With one query per workgroup its A operands are
// read from LDS once into registers instead of once per half-step, which
// halves the LDS traffic of a half-step; the registers come from the ring,
// which then holds two buffers (one query: 25.8 against 27.1-27.9 us per
// 32 x 16384 launch).
//
// A workgroup scores QW queries of one sequence (a "unit"): every key operand
// it loads is multiplied with each query's heads in turn, so a sequence with
// Q queries (draft tokens, a prefill chunk) streams its keys once per QW
// queries. Row r = b * Q + query of scores and hints belongs to query
// r - b * Q of sequence b; lengths[r] (or N) entries are visible to it.
template <int MT, int S, int NB, bool CONTIG, int QW>
__global__ __launch_bounds__(256, 2) void idx_score_bf16_kernel(const uint16_t* __restrict__ q,
                                                             const float* __restrict__ w,
                                                             const uint16_t* __restrict__ k,
                                                             const uint8_t* __restrict__ allowed,
                                                             const int32_t* __restrict__ lengths, int H, int N,
                                                             int Q, int nqg, int nchunks, float* __restrict__ scores,
                                                             float* __restrict__ hints, int hints_len, int seq_xcd) {
  constexpr int NH = 2 * S;  // half-steps per wave
  static_assert(QW >= 1 && QW <= 4, "one wave writes each query's bound sums");
  __shared__ u32x4 qlds[QW][MT * 4 * 64];
  __shared__ float wlds[QW][64];
  __shared__ float nmax[4][S];
  __shared__ double qterm[QW][2][MT * 16];  // |w_h| ||q_h||, |w_h| (first workgroup of a unit)
  __shared__ u32x4 kslab[CONTIG ? 4 : 1][CONTIG ? 32 * KT_LD : 1];
  // seq_xcd: a 1-D grid in which unit u's workgroups all have ids equal to
  // u modulo 8, i.e. run on XCD u % 8, where the selection of a single-query
  // sequence u (one workgroup, id u) then finds its scores in that XCD's L2
  int u, bx;
  if (seq_xcd) {
    const int nx = (nchunks + S - 1) / S, slot = (int)blockIdx.x >> 3;
    bx = slot % nx;
    u = (slot / nx) * 8 + ((int)blockIdx.x & 7);
  } else {
    u = blockIdx.y;
    bx = blockIdx.x;
  }
  const int b = u / nqg, q0 = (u - b * nqg) * QW;
  const int nq = min(QW, Q - q0);  // queries of this unit (the last unit of a sequence may have fewer)
  const int r0 = b * Q + q0;       // its first row
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const uint16_t* kb = k + (size_t)b * N * LIT_IDX_DIM;
  const int wg_base = bx * (S * CHUNK);
  const bool bounds = hints && bx == 0;
  // half-step h: entries hbase(h) .. +31 of chunk h/2
  auto hbase = [&](int h) { return wg_base + (h >> 1) * CHUNK + wid * 64 + 32 * (h & 1); };
  // the first NB - 1 half-steps' keys are in flight while q is staged
  u32x4 kr[NB][2][4];
  auto load_half = [&](int h, u32x4 (&dst)[2][4]) {
    if (CONTIG)
      load_keys_contig(kb, hbase(h), N, lane, reinterpret_cast<u32x4(&)[8]>(dst));
    else
      load_keys_half(kb, hbase(h), N, g, c, dst);
  };
#pragma unroll
  for (int h = 0; h < NB - 1; h++)
    if (h < NH) load_half(h, kr[h]);

  // Stage q as MFMA A operands: operand (mt, j) lane (hh + 16*gg) holds head
  // 16*mt + hh, dims 8*gg + 32*j .. +7. Queries past nq stage zeros.
  for (int idx = tid; idx < QW * MT * 16 * 16; idx += 256) {
    const int qi = idx / (MT * 256), hd = idx - qi * (MT * 256);
    const int h = hd >> 4, d8 = hd & 15;  // the 16 lanes of a row hold one head
    const bool live = h < H && qi < nq;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (live) v = *(const u32x4*)(q + ((size_t)(r0 + qi) * H + h) * LIT_IDX_DIM + d8 * 8);
    const int mt = h >> 4, hh = h & 15, gg = d8 & 3, j = d8 >> 2;
    qlds[qi][(mt * 4 + j) * 64 + hh + 16 * gg] = v;
    if (bounds) {
      double ss = 0.0;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const double lo = (double)bf16_lo(v[i]), hi = (double)bf16_hi(v[i]);
        ss += lo * lo;
        ss += hi * hi;
      }
      ss += dpp_f64<0x111>(ss);
      ss += dpp_f64<0x112>(ss);
      ss += dpp_f64<0x114>(ss);
      ss += dpp_f64<0x118>(ss);
      if (d8 == 15) {
        const double a = live ? fabs((double)w[(size_t)(r0 + qi) * H + h]) : 0.0;
        qterm[qi][0][h] = a * sqrt(ss);
        qterm[qi][1][h] = a;
      }
    }
  }
  for (int i = tid; i < QW * 64; i += 256) {
    const int qi = i >> 6, h = i & 63;
    wlds[qi][h] = h < H && qi < nq ? w[(size_t)(r0 + qi) * H + h] : 0.f;
  }
  lds_barrier();
  const int hq_off = nchunks + (N + LIT_HINT_GROUP - 1) / LIT_HINT_GROUP;  // the query-side sums in a hints row
  if (bounds && wid < nq)  // one wave per query (QW <= 4)
    write_q_bounds(qterm[wid][0], qterm[wid][1], MT * 16, hints + (size_t)(r0 + wid) * hints_len + hq_off);
  float wr[QW][MT][4];
#pragma unroll
  for (int qi = 0; qi < QW; qi++) load_lane_weights<MT>(wlds[qi], wr[qi]);
  u32x4 qreg[QW == 1 ? MT * 4 : 1];  // one query's A operands, held for the whole launch
  if (QW == 1) {
#pragma unroll
    for (int i = 0; i < MT * 4; i++) qreg[i] = qlds[0][i * 64 + lane];
  }
  int nv[QW];  // entries visible to each query
#pragma unroll
  for (int qi = 0; qi < QW; qi++) nv[qi] = lengths && qi < nq ? lengths[r0 + qi] : N;

  const uint8_t* ab = allowed ? allowed + (size_t)b * N : nullptr;

  float my_score[QW], my_n2 = 0.f;
#pragma unroll
  for (int qi = 0; qi < QW; qi++) my_score[qi] = 0.f;
#pragma unroll
  for (int h = 0; h < NH; h++) {
    if (h + NB - 1 < NH) load_half(h + NB - 1, kr[(h + NB - 1) % NB]);
    // keep the loads ahead of this half-step's math (the scheduler would sink them)
    __builtin_amdgcn_sched_barrier(0);
    u32x4 kt[2][4];
    if (CONTIG) keys_to_operands(kslab[wid], reinterpret_cast<const u32x4(&)[8]>(kr[h % NB]), lane, g, c, kt);
    const u32x4 (&kc)[2][4] = CONTIG ? kt : kr[h % NB];
    f32x4 gram[2];
#pragma unroll
    for (int qi = 0; qi < QW; qi++) {
      f32x4 acc[2][MT];
#pragma unroll
      for (int G = 0; G < 2; G++)
#pragma unroll
        for (int mt = 0; mt < MT; mt++) acc[G][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, QW == 1 ? qreg[mt * 4 + j] : qlds[qi][(mt * 4 + j) * 64 + lane]);
#pragma unroll
          for (int G = 0; G < 2; G++)
            acc[G][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, kc[G][j]),
                                                                 acc[G][mt], 0, 0, 0);
        }
      if (qi == 0) {
        // key norms: the 16 x 16 Gram matrix of each column group on the matrix
        // cores (A = B = the group's key registers). Its largest entry is its
        // largest diagonal entry (Cauchy-Schwarz), the largest squared norm.
#pragma unroll
        for (int G = 0; G < 2; G++) {
          gram[G] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < 4; j++)
            gram[G] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kc[G][j]),
                                                              __builtin_bit_cast(bf16x8, kc[G][j]), gram[G], 0, 0, 0);
        }
      }
#pragma unroll
      for (int G = 0; G < 2; G++) {
        const float p = weighted_relu<MT>(acc[G], wr[qi]);
        if (2 * (h & 1) + G == g) my_score[qi] = p;  // the column group that holds this lane's entry
      }
    }
#pragma unroll
    for (int G = 0; G < 2; G++)
#pragma unroll
      for (int i = 0; i < 4; i++) my_n2 = fmaxf(my_n2, gram[G][i]);
    if (h & 1) {
      // chunk h/2 done: lane = 16*g + c holds entry base + lane
      const int s = h >> 1;
      const int base = wg_base + s * CHUNK + wid * 64;
      const int e = base + lane;
#pragma unroll
      for (int qi = 0; qi < QW; qi++) {
        if (qi < nq) {
          const size_t row = (size_t)(r0 + qi);
          const float gmax = store_score(my_score[qi], e, N, nv[qi], ab, scores + row * N);
          if (hints && c == 15 && base + 16 * g < N) hints[row * hints_len + nchunks + (base + 16 * g) / 16] = gmax;
        }
      }
      const float m = wave_max(my_n2);
      if (lane == 0) nmax[wid][s] = m;
      my_n2 = 0.f;
    }
  }
  __syncthreads();
  if (hints && tid < S * QW) {
    const int s = tid % S, qi = tid / S;
    const int chunk = bx * S + s;
    if (chunk < nchunks && qi < nq) {
      const float m = fmaxf(fmaxf(nmax[0][s], nmax[1][s]), fmaxf(nmax[2][s], nmax[3][s]));
      hints[(size_t)(r0 + qi) * hints_len + chunk] = norm_bound(m);
    }
  }
}

// Many queries per sequence (a prefill chunk): the scores are a [Q*H x 128] x
// [128 x N] product followed by the weighted ReLU over each query's heads, far
// above the matrix cores' ridge, so the work is arranged as a GEMM. Each wave
// keeps two queries' 64 heads as A operands in registers for the whole launch;
// the eight waves of a workgroup (16 queries) share 64-entry key tiles staged
// in LDS, double-buffered, the next tile's loads in flight while the current
// one is multiplied. Per 16-entry column block a wave reads the four K-steps'
// B operands once and issues 2 x 16 MFMAs, so LDS supplies 1 KiB per 8 MFMAs.
// Outputs and hints are those of idx_score_bf16_kernel for the same rows.
constexpr int GM_WAVES = 8;                  // waves per workgroup
constexpr int GM_QPW = 2;                    // queries per wave
constexpr int GM_QPB = GM_WAVES * GM_QPW;    // queries per workgroup
constexpr int GM_ET = 64;                    // entries per key tile
constexpr int GM_KS = LIT_IDX_DIM + 8;       // bf16 per LDS key row (pad spreads banks)
constexpr int GM_TILES_PER_CHUNK = CHUNK / GM_ET;

__global__ __launch_bounds__(GM_WAVES * 64, 1) void idx_score_gemm_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint16_t* __restrict__ k,
    const uint8_t* __restrict__ allowed, const int32_t* __restrict__ lengths, int H, int N, int Q, int tiles_per_wg,
    int nchunks, float* __restrict__ scores, float* __restrict__ hints, int hints_len) {
  constexpr int MT = 4;  // head blocks of 16 (heads past H are zeros)
  __shared__ __align__(16) uint16_t ks[2][GM_ET * GM_KS];
  __shared__ float nmax_s[2][GM_WAVES];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int b = blockIdx.z, qg = blockIdx.y;
  const int ntiles = (N + GM_ET - 1) / GM_ET;
  const int t0 = blockIdx.x * tiles_per_wg, t1 = min(ntiles, t0 + tiles_per_wg);
  const uint16_t* kb = k + (size_t)b * N * LIT_IDX_DIM;
  const uint8_t* ab = allowed ? allowed + (size_t)b * N : nullptr;
  const int hq_off = nchunks + (N + LIT_HINT_GROUP - 1) / LIT_HINT_GROUP;

  // this wave's queries: A operands (qi, mt, j), lane (c + 16 g) = head 16 mt + c, dims 8 g + 32 j .. +7
  int rq[GM_QPW], nv[GM_QPW];
  bool qlive[GM_QPW];
  u32x4 A[GM_QPW][MT][4];
  float wr[GM_QPW][MT][4];
#pragma unroll
  for (int qi = 0; qi < GM_QPW; qi++) {
    const int jq = qg * GM_QPB + wid * GM_QPW + qi;
    qlive[qi] = jq < Q;
    rq[qi] = b * Q + min(jq, Q - 1);
    nv[qi] = lengths && qlive[qi] ? lengths[rq[qi]] : N;
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
      const int h = 16 * mt + c;
#pragma unroll
      for (int j = 0; j < 4; j++)
        A[qi][mt][j] = h < H && qlive[qi] ? *(const u32x4*)(q + ((size_t)rq[qi] * H + h) * LIT_IDX_DIM + 8 * g + 32 * j)
                                          : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int hw = 16 * mt + 4 * g + i;
        wr[qi][mt][i] = hw < H && qlive[qi] ? w[(size_t)rq[qi] * H + hw] : 0.f;
      }
    }
  }
  // the query-side bound sums of each live query (first workgroup along the entries)
  if (hints && blockIdx.x == 0) {
#pragma unroll
    for (int qi = 0; qi < GM_QPW; qi++) {
      double qs = 0.0, as = 0.0;
#pragma unroll
      for (int mt = 0; mt < MT; mt++) {
        double ss = 0.0;
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const double lo = (double)bf16_lo(A[qi][mt][j][i]), hi = (double)bf16_hi(A[qi][mt][j][i]);
            ss += lo * lo;
            ss += hi * hi;
          }
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        const int h = 16 * mt + c;
        const double a = h < H && qlive[qi] ? fabs((double)w[(size_t)rq[qi] * H + h]) : 0.0;
        qs += a * sqrt(ss);
        as += a;
      }
      qs = wave_sum_f64_dpp(g == 0 ? qs : 0.0);
      as = wave_sum_f64_dpp(g == 0 ? as : 0.0);
      if (lane == 0 && qlive[qi]) {
        uint32_t* u = reinterpret_cast<uint32_t*>(hints + (size_t)rq[qi] * hints_len + hq_off);
        const uint64_t qb = (uint64_t)__double_as_longlong(qs), abb = (uint64_t)__double_as_longlong(as);
        u[0] = (uint32_t)qb;
        u[1] = (uint32_t)(qb >> 32);
        u[2] = (uint32_t)abb;
        u[3] = (uint32_t)(abb >> 32);
      }
    }
  }

  // key tile staging: thread tid takes entry tid / 8, dims 16 (tid % 8) .. +15
  const int se = tid >> 3, sp = tid & 7;
  auto load_tile = [&](int t, u32x4 (&r)[2]) {
    const int e = min(t * GM_ET + se, N - 1);  // past N: row N-1 (in bounds; a real row keeps the norm bound valid)
    const u32x4* src = (const u32x4*)(kb + (size_t)e * LIT_IDX_DIM + 16 * sp);
    r[0] = src[0];
    r[1] = src[1];
  };
  // Key-norm bounds: the largest squared norm of a 256-entry chunk, reduced
  // when the chunk's last tile is staged and written (to every row of the
  // workgroup) after the next barrier; two slots, as chunks alternate.
  float cmax = 0.f;
  int pend = -1;  // chunk whose maximum waits in nmax_s[pend & 1] (the same in every thread)
  auto stage_tile = [&](int u, int buf, const u32x4 (&r)[2]) {
    uint16_t* dst = &ks[buf][se * GM_KS + 16 * sp];
    *(u32x4*)dst = r[0];
    *(u32x4*)(dst + 8) = r[1];
    float n2 = 0.f;
#pragma unroll
    for (int h2 = 0; h2 < 2; h2++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const float lo = bf16_lo(r[h2][i]), hi = bf16_hi(r[h2][i]);
        n2 = fmaf(lo, lo, n2);
        n2 = fmaf(hi, hi, n2);
      }
    n2 += __shfl_xor(n2, 1);
    n2 += __shfl_xor(n2, 2);
    n2 += __shfl_xor(n2, 4);
    if (u % GM_TILES_PER_CHUNK == 0) cmax = 0.f;
    cmax = fmaxf(cmax, n2);
    if ((u + 1) % GM_TILES_PER_CHUNK == 0 || u + 1 == ntiles) {
      const float m = wave_max(cmax);
      const int ch = u / GM_TILES_PER_CHUNK;
      if (lane == 0) nmax_s[ch & 1][wid] = m;
      pend = ch;
    }
  };
  auto flush_norm = [&]() {  // after a barrier
    if (pend >= 0) {
      if (hints && tid < GM_QPB && qg * GM_QPB + tid < Q) {
        float m = nmax_s[pend & 1][0];
#pragma unroll
        for (int i = 1; i < GM_WAVES; i++) m = fmaxf(m, nmax_s[pend & 1][i]);
        hints[((size_t)b * Q + qg * GM_QPB + tid) * hints_len + pend] = norm_bound(m);
      }
      pend = -1;
    }
  };
  u32x4 raw[2];
  if (t0 < t1) {
    load_tile(t0, raw);
    stage_tile(t0, 0, raw);
  }
  lds_barrier();
  flush_norm();
#pragma unroll 1
  for (int t = t0; t < t1; t++) {
    const int buf = (t - t0) & 1;
    const bool more = t + 1 < t1;
    if (more) load_tile(t + 1, raw);
    const int tb = t * GM_ET;
    // the B operands of column block cb + 1 are read while block cb multiplies
    u32x4 kB[2][4];
#pragma unroll
    for (int j = 0; j < 4; j++) kB[0][j] = *(const u32x4*)&ks[buf][c * GM_KS + 8 * g + 32 * j];
#pragma unroll
    for (int cb = 0; cb < GM_ET / 16; cb++) {
      if (cb + 1 < GM_ET / 16) {
#pragma unroll
        for (int j = 0; j < 4; j++)
          kB[(cb + 1) & 1][j] = *(const u32x4*)&ks[buf][(16 * (cb + 1) + c) * GM_KS + 8 * g + 32 * j];
      }
      const int e = tb + 16 * cb + c;
      const bool hidden = e >= N || (ab && ab[min(e, N - 1)] == 0);
#pragma unroll
      for (int qi = 0; qi < GM_QPW; qi++) {
        f32x4 acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; mt++) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
          for (int mt = 0; mt < MT; mt++)
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, A[qi][mt][j]),
                                                              __builtin_bit_cast(bf16x8, kB[cb & 1][j]), acc[mt], 0,
                                                              0, 0);
        float v = weighted_relu<MT>(acc, wr[qi]);  // every lane of column c: entry e's score
        if (hidden || e >= nv[qi]) v = -INFINITY;
        if (qlive[qi] && g == 0 && e < N) scores[(size_t)rq[qi] * N + e] = v;
        // the 16-entry group maximum along the row of 16 lanes (lane c = 15 ends with it)
        constexpr uint32_t NEG_INF = 0xff800000u;
        v = fmaxf(v, __uint_as_float(dpp_u32<0x111>(NEG_INF, __float_as_uint(v))));
        v = fmaxf(v, __uint_as_float(dpp_u32<0x112>(NEG_INF, __float_as_uint(v))));
        v = fmaxf(v, __uint_as_float(dpp_u32<0x114>(NEG_INF, __float_as_uint(v))));
        v = fmaxf(v, __uint_as_float(dpp_u32<0x118>(NEG_INF, __float_as_uint(v))));
        if (hints && qlive[qi] && lane == 15 && tb + 16 * cb < N)
          hints[(size_t)rq[qi] * hints_len + nchunks + (tb + 16 * cb) / 16] = v;
      }
    }
    if (more) stage_tile(t + 1, (t + 1 - t0) & 1, raw);
    lds_barrier();
    flush_norm();
  }
}

// FP32 inputs: v_mfma_f32_16x16x4_f32, lane l holds A[l%16][l/16] and
// B[l/16][l%16]; K-step j pairs lane group g with dim 32*g + j. One query (row
// b of scores; its keys are those of sequence b / Q) per workgroup row.
template <int MT>
__global__ __launch_bounds__(256) void idx_score_f32_kernel(const float* __restrict__ q,
                                                            const float* __restrict__ w,
                                                            const float* __restrict__ k,
                                                            const uint8_t* __restrict__ allowed,
                                                            const int32_t* __restrict__ lengths, int H,
                                                            int N, int Q, int nchunks, float* __restrict__ scores,
                                                            float* __restrict__ hints, int hints_len) {
  __shared__ float qlds[MT * 32 * 64];
  __shared__ float wlds[64];
  __shared__ float nmax[4];
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const float* qb = q + (size_t)b * H * LIT_IDX_DIM;
  for (int idx = tid; idx < MT * 16 * LIT_IDX_DIM; idx += 256) {
    const int h = idx >> 7, d = idx & 127;
    const float v = h < H ? qb[h * LIT_IDX_DIM + d] : 0.f;
    const int mt = h >> 4, hh = h & 15, gg = d >> 5, j = d & 31;
    qlds[(mt * 32 + j) * 64 + hh + 16 * gg] = v;
  }
  if (tid < 64) wlds[tid] = tid < H ? w[(size_t)b * H + tid] : 0.f;
  __syncthreads();
  if (hints && blockIdx.x == 0 && wid == 0) {
    // lane h: its head's squared norm from the staged operands (fp64, exact squares)
    __shared__ double qterm[2][64];
    double ss = 0.0;
    if (lane < MT * 16)
      for (int d = 0; d < LIT_IDX_DIM; d++) {
        const double x = (double)qlds[((lane >> 4) * 32 + (d & 31)) * 64 + (lane & 15) + 16 * (d >> 5)];
        ss += x * x;
      }
    const double a = lane < H ? fabs((double)wlds[lane]) : 0.0;
    qterm[0][lane] = a * sqrt(ss);
    qterm[1][lane] = a;
    write_q_bounds(qterm[0], qterm[1], 64, hints + (size_t)b * hints_len + nchunks + (N + LIT_HINT_GROUP - 1) / LIT_HINT_GROUP);
  }
  float wr[MT][4];
  load_lane_weights<MT>(wlds, wr);

  const int bk = b / Q;  // the sequence whose keys this query reads
  const float* kb = k + (size_t)bk * N * LIT_IDX_DIM;
  const uint8_t* ab = allowed ? allowed + (size_t)bk * N : nullptr;
  float* sb = scores + (size_t)b * N;
  const int nv = lengths ? lengths[b] : N;
  const int base = blockIdx.x * CHUNK + wid * 64;
  float my_score = 0.f, my_n2 = 0.f;
#pragma unroll 1
  for (int G = 0; G < 4; G++) {
    const int e = base + 16 * G + c;
    float kr[32];
#pragma unroll
    for (int v4 = 0; v4 < 8; v4++) {
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (e < N) v = *(const f32x4*)(kb + (size_t)e * LIT_IDX_DIM + 32 * g + 4 * v4);
#pragma unroll
      for (int i = 0; i < 4; i++) kr[4 * v4 + i] = v[i];
    }
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
      for (int j = 0; j < 32; j++)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(qlds[(mt * 32 + j) * 64 + lane], kr[j], acc[mt], 0, 0, 0);
    const float p = weighted_relu<MT>(acc, wr);
    float n2 = 0.f;
#pragma unroll
    for (int j = 0; j < 32; j++) n2 = fmaf(kr[j], kr[j], n2);
    n2 += __shfl_xor(n2, 16);
    n2 += __shfl_xor(n2, 32);
    if (G == g) {
      my_score = p;
      my_n2 = n2;
    }
  }
  const int e = base + lane;
  const float gmax = store_score(my_score, e, N, nv, ab, sb);
  if (hints && c == 15 && base + 16 * g < N) hints[(size_t)b * hints_len + nchunks + (base + 16 * g) / 16] = gmax;
  const float m = wave_max(my_n2);
  if (lane == 0) nmax[wid] = m;
  __syncthreads();
  if (hints && tid == 0 && (int)blockIdx.x < nchunks) {
    const float mm = fmaxf(fmaxf(nmax[0], nmax[1]), fmaxf(nmax[2], nmax[3]));
    hints[(size_t)b * hints_len + blockIdx.x] = norm_bound(mm);
  }
}

// Canonical fp64 scores of every entry: one wave per entry (slow; for labels).
__global__ __launch_bounds__(256) void idx_score_exact_kernel(const void* __restrict__ q,
                                                              const float* __restrict__ w,
                                                              const void* __restrict__ k,
                                                              const uint8_t* __restrict__ allowed, int dtype,
                                                              int H, int N, double* __restrict__ out) {
  __shared__ float qT[LIT_IDX_DIM * 64];
  __shared__ float krow[4][LIT_IDX_DIM];
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  for (int idx = tid; idx < LIT_IDX_DIM * 64; idx += 256) {
    const int d = idx >> 6, h = idx & 63;
    float v = 0.f;
    if (h < H) {
      const size_t off = ((size_t)b * H + h) * LIT_IDX_DIM + d;
      v = dtype == LIT_F32 ? ((const float*)q)[off] : bf16_to_f32(((const uint16_t*)q)[off]);
    }
    qT[idx] = v;
  }
  __syncthreads();
  const float w_h = lane < H ? w[(size_t)b * H + lane] : 0.f;
  const int waves = gridDim.x * 4;
  for (int n = blockIdx.x * 4 + wid; n < N; n += waves) {
    const size_t row = ((size_t)b * N + n) * LIT_IDX_DIM;
    for (int d = lane; d < LIT_IDX_DIM; d += 64)
      krow[wid][d] = dtype == LIT_F32 ? ((const float*)k)[row + d] : bf16_to_f32(((const uint16_t*)k)[row + d]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    double s = exact_score_wave(qT, krow[wid], w_h, H);
    if (allowed && allowed[(size_t)b * N + n] == 0) s = -INFINITY;
    if (lane == 0) out[(size_t)b * N + n] = s;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

lit_status check_idx_in(const lit_idx_in* in, int32_t B, int32_t N, const char* who) {
  if (!in) return fail(LIT_ERR_NULL, "%s: inputs struct is NULL", who);
  if (!in->q || !in->w || !in->k) return fail(LIT_ERR_NULL, "%s: q, w and k must be non-NULL", who);
  if (B < 1 || N < 1) return fail(LIT_ERR_SHAPE, "%s: B=%d and N=%d must be >= 1", who, B, N);
  if (in->H < 1 || in->H > LIT_MAX_IDX_HEADS)
    return fail(LIT_ERR_SHAPE, "%s: H=%d outside 1..%d", who, in->H, LIT_MAX_IDX_HEADS);
  if (in->dtype != LIT_F32 && in->dtype != LIT_BF16)
    return fail(LIT_ERR_DTYPE, "%s: index q/k dtype %d unsupported (F32 or BF16)", who, (int)in->dtype);
  if (!aligned(in->q, 16) || !aligned(in->k, 16) || !aligned(in->w, 4))
    return fail(LIT_ERR_ALIGN, "%s: q and k must be 16-byte aligned, w 4-byte aligned", who);
  return LIT_OK;
}

}  // namespace

lit_status check_idx_inputs(const lit_idx_in* in, int32_t B, int32_t N, const char* who) {
  return check_idx_in(in, B, N, who);
}

}  // namespace lit

using namespace lit;

template <int MT, int QW>
static void launch_bf16(int S, dim3 grid, hipStream_t st, const lit_idx_in* in, const uint8_t* allowed,
                        const int32_t* lengths, int N, int Q, int nqg, int nchunks, float* scores, float* hints,
                        int hl) {
  const uint16_t* q = (const uint16_t*)in->q;
  const uint16_t* k = (const uint16_t*)in->k;
  // unit counts that fill the 8 XCDs evenly keep each unit on one XCD
  const int seq_xcd = grid.y % 8 == 0;
  const dim3 g = seq_xcd ? dim3(grid.x * grid.y) : grid;
  constexpr int NB = QW == 1 ? KEY_RING_1Q : KEY_RING;
  if (S == 4)
    idx_score_bf16_kernel<MT, 4, NB, KEY_CONTIG, QW><<<g, 256, 0, st>>>(q, in->w, k, allowed, lengths, in->H, N, Q, nqg, nchunks, scores, hints, hl, seq_xcd);
  else
    idx_score_bf16_kernel<MT, 1, NB, KEY_CONTIG, QW><<<g, 256, 0, st>>>(q, in->w, k, allowed, lengths, in->H, N, Q, nqg, nchunks, scores, hints, hl, seq_xcd);
}

template <int MT>
static void launch_f32(dim3 grid, hipStream_t st, const lit_idx_in* in, const uint8_t* allowed,
                       const int32_t* lengths, int N, int Q, int nchunks, float* scores, float* hints, int hl) {
  idx_score_f32_kernel<MT><<<grid, 256, 0, st>>>((const float*)in->q, in->w, (const float*)in->k, allowed, lengths,
                                                 in->H, N, Q, nchunks, scores, hints, hl);
}

extern "C" int32_t lit_idx_hints_len(int32_t N) {
  if (N < 1) return 0;
  return (int32_t)(cdiv(N, LIT_KNORM_CHUNK) + cdiv(N, LIT_HINT_GROUP) + LIT_HINT_QBOUND);
}

// Q queries per sequence; Q == 1 with lengths == NULL is lit_idx_score.
static lit_status idx_score_rows(const lit_idx_in* in, int32_t Q, const int32_t* lengths, const uint8_t* allowed,
                                 int32_t B, int32_t N, float* scores, float* hints, void* stream, const char* who) {
  const int nchunks = (int)cdiv(N, CHUNK);
  const int hl = lit_idx_hints_len(N);
  const int MT = (in->H + 15) / 16;
  hipStream_t hs = (hipStream_t)stream;
  if (in->dtype == LIT_BF16 && Q >= GM_QPB) {
    // many queries: the GEMM arrangement, 16 queries per workgroup, the entries
    // split into ranges of whole chunks until about two workgroups per CU
    const int qgs = (Q + GM_QPB - 1) / GM_QPB;
    const int64_t rows = (int64_t)B * qgs;
    if (qgs > 65535 || B > 65535) return fail(LIT_ERR_SHAPE, "%s: B=%d, Q=%d too large for the grid", who, B, Q);
    const int splits = (int)std::max<int64_t>(1, std::min<int64_t>(nchunks, (512 + rows - 1) / rows));
    const int chunks_per = (nchunks + splits - 1) / splits;
    const int tiles_per = chunks_per * GM_TILES_PER_CHUNK;
    const int ntiles = (int)cdiv(N, GM_ET);
    dim3 grid((unsigned)cdiv(ntiles, tiles_per), (unsigned)qgs, (unsigned)B);
    idx_score_gemm_kernel<<<grid, GM_WAVES * 64, 0, hs>>>((const uint16_t*)in->q, in->w, (const uint16_t*)in->k, allowed,
                                                          lengths, in->H, N, Q, tiles_per, nchunks, scores, hints, hl);
  } else if (in->dtype == LIT_BF16) {
    // Queries per workgroup: one for single queries; two for a pair of draft
    // tokens; four for many queries, where the key operands are reused the most.
    const int QW = Q == 1 ? 1 : (Q == 2 ? 2 : 4);
    const int nqg = (Q + QW - 1) / QW;
    const int64_t units = (int64_t)B * nqg;
    if (units > 65535 * 8) return fail(LIT_ERR_SHAPE, "%s: B x ceil(Q/%d) = %lld workgroup rows, above 524280", who, QW, (long long)units);
    // More chunks per workgroup when there is plenty of work: amortises the q
    // staging and lets every workgroup keep its next chunk's keys in flight;
    // at most about 512 workgroups (two per CU) keep all of them resident at
    // once (4 x 125,000 entries: one round of 492 workgroups of four chunks
    // measured 26.1 us against 28.2 for two rounds of two chunks).
    const int64_t total = units * nchunks;
    const int S = total >= 2048 || (total >= 1024 && QW == 1) ? 4 : 1;
    dim3 grid((unsigned)cdiv(nchunks, S), (unsigned)units);
    if (grid.y > 65535 && grid.y % 8 != 0)
      return fail(LIT_ERR_SHAPE, "%s: %u workgroup rows (above 65535 they must be a multiple of 8)", who, grid.y);
#define LIT_MT_CASES(QWV)                                                                                   \
  switch (MT) {                                                                                             \
    case 1: launch_bf16<1, QWV>(S, grid, hs, in, allowed, lengths, N, Q, nqg, nchunks, scores, hints, hl); break; \
    case 2: launch_bf16<2, QWV>(S, grid, hs, in, allowed, lengths, N, Q, nqg, nchunks, scores, hints, hl); break; \
    case 3: launch_bf16<3, QWV>(S, grid, hs, in, allowed, lengths, N, Q, nqg, nchunks, scores, hints, hl); break; \
    default: launch_bf16<4, QWV>(S, grid, hs, in, allowed, lengths, N, Q, nqg, nchunks, scores, hints, hl); break; \
  }
    if (QW == 1) {
      LIT_MT_CASES(1)
    } else if (QW == 2) {
      LIT_MT_CASES(2)
    } else {
      LIT_MT_CASES(4)
    }
#undef LIT_MT_CASES
  } else {
    const int64_t rows = (int64_t)B * Q;
    if (rows > 65535) return fail(LIT_ERR_SHAPE, "%s: B x Q = %lld fp32 query rows, above 65535", who, (long long)rows);
    dim3 grid((unsigned)nchunks, (unsigned)rows);
    switch (MT) {
      case 1: launch_f32<1>(grid, hs, in, allowed, lengths, N, Q, nchunks, scores, hints, hl); break;
      case 2: launch_f32<2>(grid, hs, in, allowed, lengths, N, Q, nchunks, scores, hints, hl); break;
      case 3: launch_f32<3>(grid, hs, in, allowed, lengths, N, Q, nchunks, scores, hints, hl); break;
      default: launch_f32<4>(grid, hs, in, allowed, lengths, N, Q, nchunks, scores, hints, hl); break;
    }
  }
  LIT_CHECK_LAUNCH(who);
  return LIT_OK;
}

extern "C" lit_status lit_idx_score(const lit_idx_in* in, const uint8_t* allowed, int32_t B, int32_t N,
                                    float* scores, float* hints, void* stream) {
  clear_error();
  lit_status st = check_idx_in(in, B, N, "lit_idx_score");
  if (st != LIT_OK) return st;
  if (!scores) return fail(LIT_ERR_NULL, "lit_idx_score: scores is NULL");
  if (!aligned(scores, 4) || (hints && !aligned(hints, 4)))
    return fail(LIT_ERR_ALIGN, "lit_idx_score: scores/hints must be 4-byte aligned");
  return idx_score_rows(in, 1, nullptr, allowed, B, N, scores, hints, stream, "lit_idx_score");
}

extern "C" lit_status lit_idx_score_mq(const lit_idx_in* in, int32_t Q, const int32_t* lengths,
                                       const uint8_t* allowed, int32_t B, int32_t N, float* scores, float* hints,
                                       void* stream) {
  clear_error();
  const char* who = "lit_idx_score_mq";
  lit_status st = check_idx_in(in, B, N, who);
  if (st != LIT_OK) return st;
  if (Q < 1 || Q > LIT_MAX_QUERIES) return fail(LIT_ERR_SHAPE, "%s: Q=%d outside 1..%d", who, Q, LIT_MAX_QUERIES);
  if ((int64_t)B * Q * N > ((int64_t)1 << 40)) return fail(LIT_ERR_SHAPE, "%s: B x Q x N above 2^40", who);
  if (!scores) return fail(LIT_ERR_NULL, "%s: scores is NULL", who);
  if (!aligned(scores, 4) || (hints && !aligned(hints, 4)) || (lengths && !aligned(lengths, 4)))
    return fail(LIT_ERR_ALIGN, "%s: scores, hints and lengths must be 4-byte aligned", who);
  return idx_score_rows(in, Q, lengths, allowed, B, N, scores, hints, stream, who);
}

extern "C" lit_status lit_idx_score_exact(const lit_idx_in* in, const uint8_t* allowed, int32_t B, int32_t N,
                                          double* scores64, void* stream) {
  clear_error();
  lit_status st = check_idx_in(in, B, N, "lit_idx_score_exact");
  if (st != LIT_OK) return st;
  if (!scores64) return fail(LIT_ERR_NULL, "lit_idx_score_exact: scores64 is NULL");
  if (!aligned(scores64, 8)) return fail(LIT_ERR_ALIGN, "lit_idx_score_exact: scores64 must be 8-byte aligned");
  const int per_b = (int)std::min<int64_t>(cdiv(N, 4), 1024);
  dim3 grid((unsigned)per_b, (unsigned)B);
  idx_score_exact_kernel<<<grid, 256, 0, (hipStream_t)stream>>>(in->q, in->w, in->k, allowed, (int)in->dtype,
                                                                in->H, N, scores64);
  LIT_CHECK_LAUNCH("lit_idx_score_exact");
  return LIT_OK;
}
