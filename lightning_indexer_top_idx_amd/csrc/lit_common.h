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

// One array of a KV descriptor as the kernels read it: row n of sequence b
// starts seq * b + row * n bytes past base.
struct KvArr {
  const uint8_t* base;
  int64_t seq, row;
  __host__ __device__ const uint8_t* at(int b, int n) const { return base + seq * b + row * (int64_t)n; }
};
// The data, rope and scale arrays of a descriptor with every stride of 0
// replaced by the dense layout's; a negative stride is refused with
// LIT_ERR_SHAPE, one that breaks the arrays' alignment with LIT_ERR_ALIGN.
lit_status kv_arrays(const lit_kv* kv, KvArr* data, KvArr* rope, KvArr* scale, const char* who);

// ---------------------------------------------------------------- device side

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

constexpr int WAVE = 64;

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// Order-preserving 32-bit key of an fp32 score: larger score -> larger key,
// equal scores -> equal keys. -inf and NaN map to 0, the "never selected" key;
// every finite score and +inf map above 0.
__device__ __forceinline__ uint32_t score_key(float f) {
  // -0.0 becomes +0.0 first (the two compare equal); then every bit of a
  // negative value is flipped, only the sign bit of a positive one; keys below
  // that of -FLT_MAX (-inf, negative NaNs) or above that of +inf (positive
  // NaNs) become 0. Branch-free: one add, one compare and one select.
  const uint32_t u = __float_as_uint(f + 0.0f);
  const uint32_t key = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
  return key - 0x00800000u <= 0xff800000u - 0x00800000u ? key : 0u;
}
__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}
// Same for fp64 values.
__device__ __forceinline__ uint64_t score_key64(double d) {
  uint64_t u = (uint64_t)__double_as_longlong(d + 0.0);  // -0.0 -> +0.0
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

// ---- wave primitives on DPP lane moves (VALU only, no LDS round trip).
// GFX9 DPP controls: row_shr:n = 0x110 + n, row_bcast:15 = 0x142 (lane 15 of
// each row into the next row), row_bcast:31 = 0x143 (lane 31 into rows 2, 3).
// A lane whose source lies outside its row, or whose row is masked off,
// receives `old`, the identity of the operation.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROWS, 0xf, false);
}
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ double dpp_f64(double v) {  // identity +0.0
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = dpp_u32<CTRL, ROWS>(0u, (uint32_t)u), hi = dpp_u32<CTRL, ROWS>(0u, (uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Inclusive prefix sum over the 64 lanes (Hillis-Steele inside each row of 16,
// then the row totals carried up by the two broadcasts).
__device__ __forceinline__ int wave_incl_scan_dpp(int v) {
  v += (int)dpp_u32<0x111>(0u, (uint32_t)v);
  v += (int)dpp_u32<0x112>(0u, (uint32_t)v);
  v += (int)dpp_u32<0x114>(0u, (uint32_t)v);
  v += (int)dpp_u32<0x118>(0u, (uint32_t)v);
  v += (int)dpp_u32<0x142, 0xa>(0u, (uint32_t)v);
  v += (int)dpp_u32<0x143, 0xc>(0u, (uint32_t)v);
  return v;
}
// Wave totals (the scan's last lane, read back as a wave-uniform value).
__device__ __forceinline__ int wave_sum_dpp(int v) { return __builtin_amdgcn_readlane(wave_incl_scan_dpp(v), 63); }
__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t v) {  // identity 0
  v = max(v, dpp_u32<0x111>(0u, v));
  v = max(v, dpp_u32<0x112>(0u, v));
  v = max(v, dpp_u32<0x114>(0u, v));
  v = max(v, dpp_u32<0x118>(0u, v));
  v = max(v, dpp_u32<0x142, 0xa>(0u, v));
  v = max(v, dpp_u32<0x143, 0xc>(0u, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_min_dpp(uint32_t v) {  // identity ~0
  v = min(v, dpp_u32<0x111>(~0u, v));
  v = min(v, dpp_u32<0x112>(~0u, v));
  v = min(v, dpp_u32<0x114>(~0u, v));
  v = min(v, dpp_u32<0x118>(~0u, v));
  v = min(v, dpp_u32<0x142, 0xa>(~0u, v));
  v = min(v, dpp_u32<0x143, 0xc>(~0u, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ double wave_sum_f64_dpp(double v) {
  v += dpp_f64<0x111>(v);
  v += dpp_f64<0x112>(v);
  v += dpp_f64<0x114>(v);
  v += dpp_f64<0x118>(v);
  v += dpp_f64<0x142, 0xa>(v);
  v += dpp_f64<0x143, 0xc>(v);
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// Butterfly steps across 16-lane rows with no LDS round trip: gfx950's
// v_permlane16_swap / v_permlane32_swap, given the same value twice, hand every
// lane the pair {v[l], v[l ^ 16]} (resp. l ^ 32); max and sum are symmetric in it.
// Call them with every lane of the wave active (inactive lanes are not read).
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Lane l's value of a double, wave-uniform.
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Inclusive prefix sum inside each row of 16 lanes.
__device__ __forceinline__ int row_incl_scan_dpp(int v) {
  v += (int)dpp_u32<0x111>(0u, (uint32_t)v);
  v += (int)dpp_u32<0x112>(0u, (uint32_t)v);
  v += (int)dpp_u32<0x114>(0u, (uint32_t)v);
  v += (int)dpp_u32<0x118>(0u, (uint32_t)v);
  return v;
}

// Exclusive prefix sum over a block of up to 16 waves in thread order, with
// one barrier: every wave posts its total to part[wid] (part[] is LDS that no
// other scan may reuse before a later barrier); then each wave scans the posted
// totals in one row of lanes and reads off its own offset. *total receives the
// block total.
template <int NW>
__device__ __forceinline__ int block_excl_scan1(int v, int* part, int* total) {
  static_assert(NW >= 1 && NW <= 16, "one row of lanes scans the wave totals");
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int inc = wave_incl_scan_dpp(v);
  if (lane == 63) part[wid] = inc;
  lds_barrier();
  const int ps = row_incl_scan_dpp((lane & 15) < NW ? part[lane & 15] : 0);
  *total = __builtin_amdgcn_readlane(ps, NW - 1);
  const int before = __builtin_amdgcn_readlane(ps, wid > 0 ? wid - 1 : 0);
  return (wid > 0 ? before : 0) + inc - v;
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
