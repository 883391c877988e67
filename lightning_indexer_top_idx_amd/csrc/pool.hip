// pool.hip - the LSA cold-pool fetch: gated entries gathered into a compact pool.
//
// zhichai.net, "FlashMemory-DeepSeek-V4 深度解读：用预言家替代记忆海绵", section 2.2:
// every tau = 64 decode steps the gate predicts which compressed blocks the next
// 64 steps will need; those are moved from a CPU "cold pool" to the GPU, the
// rest stay on the host, and the steps in between attend only inside the moved
// set, so that GPU memory follows the gate rather than the context length.
// The same page's later section notes that the swap engine itself was not
// published; this is one written for MI355X:
//   lit_pool_plan      gate [B][N] -> the compact index map of each sequence:
//                      the gated entries plus the SWA window, ascending and
//                      right-aligned in C slots (so the window stays last)
//   lit_pool_gather    rows of any per-entry array copied through that map,
//                      read straight from pinned host memory (or from device
//                      memory) by the kernel, over the host link
//   lit_pool_remap_ids selected compact ids back to the original entry ids
#include "lit_common.h"

namespace lit {
namespace {

constexpr int PLAN_THREADS = 1024;

// One workgroup per sequence: entry n is kept when gated or in the window; a
// block scan over contiguous per-thread segments gives each kept entry its
// rank, which is its slot after the C - count leading empty slots.
__global__ __launch_bounds__(PLAN_THREADS) void pool_plan_kernel(const uint8_t* __restrict__ gate, int N, int window,
                                                                 int C, int32_t* __restrict__ map,
                                                                 int32_t* __restrict__ count,
                                                                 uint8_t* __restrict__ allowed_c) {
  __shared__ int part[PLAN_THREADS / 64];
  const int b = blockIdx.x, tid = threadIdx.x;
  const uint8_t* g = gate + (size_t)b * N;
  int32_t* mp = map + (size_t)b * C;
  uint8_t* ac = allowed_c ? allowed_c + (size_t)b * C : nullptr;
  const int wlo = N - window;  // window entries: wlo .. N-1
  const int seg = (N + PLAN_THREADS - 1) / PLAN_THREADS;
  const int a = min(N, tid * seg), e = min(N, a + seg);
  int kept = 0;
  for (int n = a; n < e; n++) kept += g[n] != 0 || n >= wlo;
  int total;
  int pos = block_excl_scan1<PLAN_THREADS / 64>(kept, part, &total);
  const bool fits = total <= C;
  const int lead = C - total;  // empty slots before the first kept entry
  if (fits) {
    for (int n = a; n < e; n++) {
      const bool gn = g[n] != 0;
      if (gn || n >= wlo) {
        mp[lead + pos] = n;
        if (ac) ac[lead + pos] = gn ? 1 : 0;
        pos++;
      }
    }
  }
  for (int j = tid; j < (fits ? lead : C); j += PLAN_THREADS) {
    mp[j] = -1;
    if (ac) ac[j] = 0;
  }
  if (tid == 0) count[b] = total;
}

// dst row (b, j) = src row (b, map[b][j]) or zeros for an empty slot. Each
// thread copies pieces (16, 8 or 4 bytes, as the row width allows) in a
// grid-stride loop, UNROLL of them loaded before any is stored: reads over the
// host link take microseconds, so many must be in flight at once.
constexpr int GATHER_UNROLL = 8;

template <typename T>
__global__ __launch_bounds__(256) void pool_gather_kernel(const T* __restrict__ src, int src_rows, int pieces, int C,
                                                          const int32_t* __restrict__ map, size_t total,
                                                          T* __restrict__ dst) {
  const size_t step = (size_t)gridDim.x * blockDim.x;
  for (size_t i0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i0 < total; i0 += step * GATHER_UNROLL) {
    T v[GATHER_UNROLL];
#pragma unroll
    for (int u = 0; u < GATHER_UNROLL; u++) {
      const size_t i = i0 + step * u;
      v[u] = T{};
      if (i < total) {
        const size_t row = i / pieces;  // b * C + j
        const int piece = (int)(i - row * pieces);
        const int b = (int)(row / C);
        const int r = map[row];
        if (r >= 0 && r < src_rows) v[u] = src[((size_t)b * src_rows + r) * pieces + piece];
      }
    }
#pragma unroll
    for (int u = 0; u < GATHER_UNROLL; u++) {
      const size_t i = i0 + step * u;
      if (i < total) dst[i] = v[u];
    }
  }
}

__global__ __launch_bounds__(256) void pool_remap_kernel(const int32_t* __restrict__ ids_c,
                                                         const int32_t* __restrict__ count, int k,
                                                         const int32_t* __restrict__ map, int C,
                                                         int32_t* __restrict__ ids) {
  const int b = blockIdx.y;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= k) return;
  const int c = count[b];
  const int v = ids_c[(size_t)b * k + j];
  ids[(size_t)b * k + j] = j < c && v >= 0 && v < C ? map[(size_t)b * C + v] : -1;
}

}  // namespace
}  // namespace lit

using namespace lit;

extern "C" lit_status lit_pool_plan(const uint8_t* gate, int32_t B, int32_t N, int32_t window, int32_t C,
                                    int32_t* map, int32_t* count, uint8_t* allowed_c, void* stream) {
  clear_error();
  const char* who = "lit_pool_plan";
  if (!gate || !map || !count) return fail(LIT_ERR_NULL, "%s: gate, map and count must be non-NULL", who);
  if (B < 1 || N < 1 || C < 1) return fail(LIT_ERR_SHAPE, "%s: B=%d N=%d C=%d must be >= 1", who, B, N, C);
  if (window < 0 || window > LIT_MAX_WINDOW)
    return fail(LIT_ERR_SHAPE, "%s: window=%d outside 0..%d", who, window, LIT_MAX_WINDOW);
  if (!aligned(map, 4) || !aligned(count, 4)) return fail(LIT_ERR_ALIGN, "%s: map and count must be 4-byte aligned", who);
  pool_plan_kernel<<<dim3((unsigned)B), dim3(PLAN_THREADS), 0, (hipStream_t)stream>>>(gate, N, std::min(window, N), C,
                                                                                      map, count, allowed_c);
  LIT_CHECK_LAUNCH(who);
  return LIT_OK;
}

extern "C" lit_status lit_pool_gather(const void* src, int32_t src_rows, int64_t row_bytes, int32_t B,
                                      const int32_t* map, int32_t C, void* dst, void* stream) {
  clear_error();
  const char* who = "lit_pool_gather";
  if (!src || !map || !dst) return fail(LIT_ERR_NULL, "%s: src, map and dst must be non-NULL", who);
  if (B < 1 || src_rows < 1 || C < 1 || row_bytes < 4 || row_bytes % 4 != 0 || row_bytes > (1 << 20))
    return fail(LIT_ERR_SHAPE, "%s: B=%d src_rows=%d C=%d row_bytes=%lld (a multiple of 4, 4..2^20)", who, B,
                src_rows, C, (long long)row_bytes);
  if (!aligned(src, 4) || !aligned(dst, 4) || !aligned(map, 4))
    return fail(LIT_ERR_ALIGN, "%s: src, dst and map must be 4-byte aligned", who);
  // Host memory is read in place over the host link: it must be page-locked
  // (then the runtime gives its device-side address); pageable memory is refused.
  hipPointerAttribute_t attr;
  const void* dsrc = src;
  if (hipPointerGetAttributes(&attr, src) != hipSuccess || attr.type == hipMemoryTypeUnregistered) {
    (void)hipGetLastError();  // clears the error the query may have left
    return fail(LIT_ERR_MEMORY, "%s: src is host memory that is not page-locked (allocate it pinned)", who);
  }
  if (attr.type == hipMemoryTypeHost) {
    if (!attr.devicePointer) return fail(LIT_ERR_MEMORY, "%s: pinned src has no device-side address", who);
    dsrc = attr.devicePointer;
  }
  // the widest piece that divides the row and both base addresses
  const int piece = row_bytes % 16 == 0 && aligned(dsrc, 16) && aligned(dst, 16) ? 16
                    : row_bytes % 8 == 0 && aligned(dsrc, 8) && aligned(dst, 8) ? 8
                                                                                 : 4;
  const int pieces = (int)(row_bytes / piece);
  const size_t total = (size_t)B * C * pieces;
  const dim3 grid((unsigned)std::min<size_t>((total + 255) / 256, 4096)), block(256);
  hipStream_t st = (hipStream_t)stream;
  if (piece == 16)
    pool_gather_kernel<u32x4><<<grid, block, 0, st>>>((const u32x4*)dsrc, src_rows, pieces, C, map, total, (u32x4*)dst);
  else if (piece == 8)
    pool_gather_kernel<u32x2><<<grid, block, 0, st>>>((const u32x2*)dsrc, src_rows, pieces, C, map, total, (u32x2*)dst);
  else
    pool_gather_kernel<uint32_t><<<grid, block, 0, st>>>((const uint32_t*)dsrc, src_rows, pieces, C, map, total,
                                                         (uint32_t*)dst);
  LIT_CHECK_LAUNCH(who);
  return LIT_OK;
}

extern "C" lit_status lit_pool_remap_ids(const int32_t* ids_c, const int32_t* count, int32_t B, int32_t k,
                                         const int32_t* map, int32_t C, int32_t* ids, void* stream) {
  clear_error();
  const char* who = "lit_pool_remap_ids";
  if (!ids_c || !count || !map || !ids) return fail(LIT_ERR_NULL, "%s: every pointer must be non-NULL", who);
  if (B < 1 || k < 1 || C < 1) return fail(LIT_ERR_SHAPE, "%s: B=%d k=%d C=%d must be >= 1", who, B, k, C);
  if (!aligned(ids_c, 4) || !aligned(count, 4) || !aligned(map, 4) || !aligned(ids, 4))
    return fail(LIT_ERR_ALIGN, "%s: arrays must be 4-byte aligned", who);
  pool_remap_kernel<<<dim3((unsigned)((k + 255) / 256), (unsigned)B), dim3(256), 0, (hipStream_t)stream>>>(
      ids_c, count, k, map, C, ids);
  LIT_CHECK_LAUNCH(who);
  return LIT_OK;
}
