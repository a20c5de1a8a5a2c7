// Helpers shared by the HIP entry points (host side).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "wf_attn.h"
#include "wf_error.h"

namespace wf {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// 16-byte store that streams past the caches (nontemporal): page writes are
// not read back by the launch that writes them, and keeping them out of the
// caches leaves room for the data that is. On a page write stream this raises
// the achieved bandwidth by about a third over plain stores (measured).
__device__ __forceinline__ void store_stream16(uint4* dst, const uint4& v) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u*>(dst));
}

// 16-byte load that streams past the caches (nontemporal): for sources a
// kernel reads exactly once.
__device__ __forceinline__ uint4 load_stream16(const uint4* src) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(src));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Maps a failed HIP call to WF_EHIP with the runtime's text.
inline int32_t hip_fail(hipError_t e, const char* where) {
  return fail(WF_EHIP, "%s: %s (%d)", where, hipGetErrorString(e), int(e));
}

// Launch-error check after a kernel launch on `stream`.
inline int32_t check_launch(const char* where) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, where);
  return WF_OK;
}

// Compute units of the current device (cached per device; 0 if unknown).
inline int device_cu_count() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev] = n;
  }
  return cache[dev];
}

inline bool check_pages_enabled() {
  const char* v = std::getenv("WF_CHECK_PAGES");
  return v && v[0] == '1';
}

// Debug mode (WF_CHECK_PAGES=1): copy `n` device page ids to the host on `stream`
// (synchronising it) and range-check them against [0, num_pages).
inline int32_t check_device_pages(const int32_t* ids, int64_t n, int32_t num_pages,
                                  hipStream_t stream, const char* where) {
  if (n <= 0) return WF_OK;
  std::vector<int32_t> h(static_cast<size_t>(n));
  hipError_t e = hipMemcpyAsync(h.data(), ids, size_t(n) * sizeof(int32_t), hipMemcpyDeviceToHost,
                                stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, where);
  for (int64_t i = 0; i < n; ++i)
    if (h[size_t(i)] < 0 || h[size_t(i)] >= num_pages)
      return fail(WF_EINVAL, "%s: page id %d at index %lld outside [0, %d)", where, h[size_t(i)],
                  static_cast<long long>(i), num_pages);
  return WF_OK;
}

}  // namespace wf
