// exact.h - the indexer score evaluated in fp64 in canonical order, by one wave.
//
// Canonical order (the order lit_topk_select's exact mode reproduces): for each
// head h the 128 products q[h][d]*k[d] are added for d = 0..127, starting from
// +0.0; then s = sum over h = 0..H-1 of (w[h] * max(0, acc_h)), each product
// rounded to fp64 before it is added, starting from +0.0. BF16 and FP32 inputs
// make q*k exact in fp64, so fma(q, k, acc) equals acc + q*k there; the outer
// product w*relu(acc) is not exact and must not be fused with the add.
#pragma once

#include "lit_common.h"

namespace lit {

// Sequential fp64 sum over lanes 0..n-1 of `v` (every lane gets the result):
// ((0 + v_0) + v_1) + ... + v_{n-1}.
__device__ __forceinline__ double wave_seq_sum_f64(double v, int n) {
#pragma clang fp contract(off)
  double s = 0.0;
  for (int i = 0; i < n; i++) s = s + __shfl(v, i);
  return s;
}

// One wave scores one entry. Lane h < H owns head h.
//   qT   : LDS, q transposed as float [128][64] (q[h][d] at qT[d*64 + h]).
//   krow : LDS, the entry's key as float [128].
//   w_h  : the lane's head weight (0 for lanes >= H).
__device__ __forceinline__ double exact_score_wave(const float* qT, const float* krow, float w_h, int H) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  double acc = 0.0;
#pragma unroll 8
  for (int d = 0; d < 128; d++) acc = fma((double)qT[d * 64 + lane], (double)krow[d], acc);
  const double r = acc > 0.0 ? acc : 0.0;
  const double p = (double)w_h * r;
  return wave_seq_sum_f64(p, H);
}

}  // namespace lit
