// capi.hip - library-wide entry points and the host-side error plumbing.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <vector>

#include "lit_common.h"

namespace {
thread_local char g_last_error[512] = "";
}

namespace lit {

lit_status fail(lit_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

void clear_error() { g_last_error[0] = 0; }

lit_status launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(LIT_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return LIT_OK;
}

lit_status allow_lds(const void* kernel, size_t bytes, const char* what) {
  if (bytes <= 65536) return LIT_OK;
  // Once per (kernel, device, size): keeps the attribute call out of captured graphs' hot path.
  struct Entry {
    const void* k;
    int dev;
    size_t bytes;
  };
  static std::mutex mu;
  static std::vector<Entry> done;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(LIT_ERR_LAUNCH, "%s: no current HIP device", what);
  std::lock_guard<std::mutex> lock(mu);
  for (const Entry& e : done)
    if (e.k == kernel && e.dev == dev && e.bytes >= bytes) return LIT_OK;
  hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess)
    return fail(LIT_ERR_LAUNCH, "%s: cannot reserve %zu bytes of LDS: %s", what, bytes, hipGetErrorString(e));
  done.push_back({kernel, dev, bytes});
  return LIT_OK;
}

lit_status kv_arrays(const lit_kv* kv, KvArr* data, KvArr* rope, KvArr* scale, const char* who) {
  const int64_t st[6] = {kv->seq_stride,      kv->row_stride,       kv->rope_seq_stride,
                         kv->rope_row_stride, kv->scale_seq_stride, kv->scale_row_stride};
  for (int i = 0; i < 6; i++)
    if (st[i] < 0) return fail(LIT_ERR_SHAPE, "%s: kv stride %lld is negative", who, (long long)st[i]);
  for (int i = 0; i < 4; i++)
    if (st[i] % 16) return fail(LIT_ERR_ALIGN, "%s: kv data and rope strides must be multiples of 16 bytes", who);
  for (int i = 4; i < 6; i++)
    if (st[i] % 4) return fail(LIT_ERR_ALIGN, "%s: kv scale strides must be multiples of 4 bytes", who);
  const int64_t N = kv->n_rows;
  const int64_t drow = kv->dtype == LIT_F32 ? LIT_KV_DIM * 4
                                            : (kv->dtype == LIT_FP8E4M3_G64_ROPE_BF16 ? LIT_KV_FP8_DIMS : LIT_KV_DIM * 2);
  auto arr = [N](const void* base, int64_t seq, int64_t row, int64_t dense_row) {
    KvArr a;
    a.base = (const uint8_t*)base;
    a.row = row ? row : dense_row;
    a.seq = seq ? seq : N * a.row;
    return a;
  };
  *data = arr(kv->data, st[0], st[1], drow);
  *rope = arr(kv->rope, st[2], st[3], LIT_KV_ROPE_DIMS * 2);
  *scale = arr(kv->scale, st[4], st[5], LIT_KV_SCALE_STRIDE);
  return LIT_OK;
}

}  // namespace lit

extern "C" int lit_abi_version(void) { return LIT_ABI_VERSION; }

extern "C" const char* lit_last_error(void) { return g_last_error; }
