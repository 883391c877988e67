// recall.hip - a7: overlap of two selections.
//
// ai-muninn.com, "FlashMemory can't improve DeepSeek-V4-Flash's own lightning indexer",
// sections "Act 1" and "Act 3": a selector is scored by how many of its kept
// chunks another selection (the native top-512, or the dense golden set) also
// keeps. Per sequence: inter = |A and M|, plus |A| and |M|.
#include "lit_common.h"

namespace lit {
namespace {

__global__ __launch_bounds__(256) void recall_kernel(const uint8_t* __restrict__ a, const uint8_t* __restrict__ m,
                                                     int N, int32_t* inter, int32_t* ca, int32_t* cb) {
  __shared__ int red[3][4];
  const int b = blockIdx.x, tid = threadIdx.x;
  const uint8_t* ab = a + (size_t)b * N;
  const uint8_t* mb = m + (size_t)b * N;
  int i_ = 0, x = 0, y = 0;
  for (int n = tid; n < N; n += 256) {
    const bool p = ab[n] != 0, q = mb[n] != 0;
    x += p;
    y += q;
    i_ += p && q;
  }
  i_ = wave_sum(i_);
  x = wave_sum(x);
  y = wave_sum(y);
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = i_;
    red[1][tid >> 6] = x;
    red[2][tid >> 6] = y;
  }
  __syncthreads();
  if (tid == 0) {
    if (inter) inter[b] = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    if (ca) ca[b] = red[1][0] + red[1][1] + red[1][2] + red[1][3];
    if (cb) cb[b] = red[2][0] + red[2][1] + red[2][2] + red[2][3];
  }
}

}  // namespace
}  // namespace lit

using namespace lit;

extern "C" lit_status lit_recall(const uint8_t* a, const uint8_t* m, int32_t B, int32_t N, int32_t* inter,
                                 int32_t* count_a, int32_t* count_b, void* stream) {
  clear_error();
  if (!a || !m) return fail(LIT_ERR_NULL, "lit_recall: both masks must be non-NULL");
  if (B < 1 || N < 1) return fail(LIT_ERR_SHAPE, "lit_recall: B=%d N=%d must be >= 1", B, N);
  if ((inter && !aligned(inter, 4)) || (count_a && !aligned(count_a, 4)) || (count_b && !aligned(count_b, 4)))
    return fail(LIT_ERR_ALIGN, "lit_recall: outputs must be 4-byte aligned");
  recall_kernel<<<dim3((unsigned)B), dim3(256), 0, (hipStream_t)stream>>>(a, m, N, inter, count_a, count_b);
  LIT_CHECK_LAUNCH("lit_recall");
  return LIT_OK;
}
