// lit_common.h - shared device helpers and host-side error plumbing of the
// lightning-indexer library (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lit.h"

namespace lit {

// ---------------------------------------------------------------- host side

// Records a printf-style message as the calling thread's last error and
// returns `s` (so validation reads `return fail(LIT_ERR_SHAPE, "...")`).
lit_status fail(lit_status s, const char* fmt, ...);
// Maps the HIP runtime's sticky launch error (if any) to LIT_ERR_LAUNCH.
lit_status launch_status(const char* what);
// Clears the calling thread's last error.
void clear_error();

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Opt a kernel in to more than 64 KiB of dynamic LDS (gfx950 has 160 KiB per CU).
lit_status allow_lds(const void* kernel, size_t bytes, const char* what);

// ---------------------------------------------------------------- device side

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

constexpr int WAVE = 64;

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// Order-preserving 32-bit key of an fp32 score: larger score -> larger key.
// -inf and NaN map to 0, the "never selected" key; every finite score and
// +inf map above 0.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f || u == 0xff800000u) return 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}
// Same for fp64 values.
__device__ __forceinline__ uint64_t score_key64(double d) {
  uint64_t u = (uint64_t)__double_as_longlong(d);
  if (d != d || u == 0xfff0000000000000ull) return 0ull;
  return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}

// Workgroup barrier that orders LDS only: it waits for this wave's LDS
// operations (lgkmcnt) but not for outstanding global loads, so prefetches
// stay in flight across it. (__syncthreads also drains vmcnt.) Use it only
// where no thread reads global memory written by another thread of the block.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Wave-level reductions over all 64 lanes.
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive prefix sum over the whole block in thread order. `tmp` holds at
// least (blockDim/64 + 1) ints of LDS. Returns the thread's exclusive prefix;
// *total receives the block total. Contains two barriers.
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int inc = wave_incl_scan(v);
  if (lane == 63) tmp[wid] = inc;
  lds_barrier();
  if (wid == 0) {
    int t = lane < nw ? tmp[lane] : 0;
    int ti = wave_incl_scan(t);
    if (lane < nw) tmp[lane] = ti - t;
    if (lane == nw - 1) tmp[nw] = ti;
  }
  lds_barrier();
  int r = tmp[wid] + inc - v;
  *total = tmp[nw];
  return r;
}

}  // namespace lit

#define LIT_CHECK_LAUNCH(what)                  \
  do {                                          \
    lit_status st_ = lit::launch_status(what);  \
    if (st_ != LIT_OK) return st_;              \
  } while (0)
