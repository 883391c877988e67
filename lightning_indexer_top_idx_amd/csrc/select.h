// select.h - block-level radix selection used by top-k and the golden top-k.
//
// One workgroup selects, from M keyed items, the r largest keys; among equal
// keys the item that comes first (lower position) wins, which is the pages'
// "lower index wins" order because the callers keep items in index order.
// Keys are order-preserving unsigned integers (larger key = larger value).
#pragma once

#include "lit_common.h"

namespace lit {

// LDS scratch the routines below need (all block-shared).
struct SelectScratch {
  uint32_t hist[256];
  int scan[40];
  int misc[8];
};

// Finds the r-th largest key T (1 <= r <= number of items with a non-zero key)
// by MSB-first radix passes of 8 bits. On return *r_eq holds how many items
// equal to T belong to the top r (the rest of the top r are > T).
// `key(i)` yields item i's key. KeyT is uint32_t or uint64_t. Block-wide call.
template <typename KeyT, typename KeyFn>
__device__ KeyT radix_select(KeyFn key, int M, int r, SelectScratch* sc, int* r_eq) {
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63, wid = tid >> 6;
  KeyT prefix = 0, pmask = 0;
  constexpr int BITS = 8 * sizeof(KeyT);
#pragma unroll 1
  for (int shift = BITS - 8; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += nthr) sc->hist[i] = 0u;
    lds_barrier();
    for (int i = tid; i < M; i += nthr) {
      const KeyT kk = key(i);
      if ((kk & pmask) == prefix) atomicAdd(&sc->hist[(uint32_t)(kk >> shift) & 255u], 1u);
    }
    lds_barrier();
    if (wid == 0) {
      int c[4];
#pragma unroll
      for (int t = 0; t < 4; t++) c[t] = (int)sc->hist[4 * lane + t];
      const int ls = c[0] + c[1] + c[2] + c[3];
      const int incl = wave_incl_scan(ls);
      const int total = __shfl(incl, 63);
      int above = total - incl;  // items in bins above this lane's four
      if (above < r && r <= above + ls) {
        for (int t = 3; t >= 0; t--) {
          if (r <= above + c[t]) {
            sc->misc[0] = 4 * lane + t;
            sc->misc[1] = r - above;
            break;
          }
          above += c[t];
        }
      }
    }
    lds_barrier();
    prefix |= (KeyT)sc->misc[0] << shift;
    pmask |= (KeyT)255 << shift;
    r = sc->misc[1];
    lds_barrier();
  }
  *r_eq = r;
  return prefix;
}

// Marks the r best of M items (keys > T, then the first r_eq items equal to T
// in position order) into sel[0..M). Items are split into one contiguous
// segment per thread so a single block scan orders the ties.
template <typename KeyT, typename KeyFn>
__device__ void mark_top(KeyFn key, int M, KeyT T, int r_eq, uint8_t* sel, SelectScratch* sc) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int seg = (M + nthr - 1) / nthr;
  const int a = min(M, tid * seg), e = min(M, a + seg);
  int ties = 0;
  for (int i = a; i < e; i++) ties += key(i) == T;
  int total;
  int before = block_excl_scan(ties, sc->scan, &total);
  for (int i = a; i < e; i++) {
    const KeyT kk = key(i);
    uint8_t s = 0;
    if (kk > T) {
      s = 1;
    } else if (kk == T) {
      s = before < r_eq;
      before++;
    }
    sel[i] = s;
  }
  lds_barrier();
}

// Writes ids (ascending, tail -1 up to k), count and the optional mask of one
// sequence from per-item selection flags sel[0..N). Block-wide call.
__device__ inline void emit_selection(const uint8_t* sel, int N, int k, int32_t* ids, int32_t* count,
                                      uint8_t* mask, SelectScratch* sc) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int seg = (N + nthr - 1) / nthr;
  const int a = min(N, tid * seg), e = min(N, a + seg);
  int c = 0;
  for (int i = a; i < e; i++) c += sel[i] != 0;
  int total;
  int pos = block_excl_scan(c, sc->scan, &total);
  for (int i = a; i < e; i++) {
    const uint8_t s = sel[i] != 0;
    if (s) ids[pos++] = i;
    if (mask) mask[i] = s;
  }
  for (int j = total + tid; j < k; j += nthr) ids[j] = -1;
  if (tid == 0) *count = total;
}

}  // namespace lit
