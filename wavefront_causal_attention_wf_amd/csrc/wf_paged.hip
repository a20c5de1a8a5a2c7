// Paged K/V scatter (wf_store_paged) and its diagnostic inverse (wf_gather_paged).
//
// "Wave Forcing: Towards Speed-of-Light Streaming Video Generation", full text
// §4.2 and Appendix B.3: the store chunk's K/V is written straight into the
// attention pages that later ticks read as history, instead of being assembled
// by the consumer.
//
// Layout: a page is P consecutive tokens of one chunk with all heads, i.e. the
// source rows [p*P, p*P + P) of a [T][H][D] chunk are one contiguous block of
// P*H*D bf16, and so is the destination page. Each page is therefore a plain
// block copy; the kernel is bound by HBM bandwidth. Work is split into 16-byte
// lanes, four independent loads in flight per thread before the stores; the
// page writes are nontemporal (streamed past the caches).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "wf_internal.h"

namespace wf {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;

// One block copies kCopyThreads*kCopyUnroll 16-byte units of one page of K
// (blockIdx.z == 0) or V (blockIdx.z == 1). Units past the chunk's last token
// are written as zero.
__global__ __launch_bounds__(kCopyThreads) void store_paged_kernel(
    const uint4* __restrict__ k_src, const uint4* __restrict__ v_src, uint4* __restrict__ k_pool,
    uint4* __restrict__ v_pool, const int32_t* __restrict__ page_ids, int32_t T, int32_t row16,
    int32_t P) {
  const int32_t p = blockIdx.y;
  const uint4* src = blockIdx.z ? v_src : k_src;
  uint4* pool = blockIdx.z ? v_pool : k_pool;
  const int64_t page16 = int64_t(P) * row16;
  const int64_t tok0 = int64_t(p) * P;
  const int64_t valid16 = (T - tok0 < P ? T - tok0 : P) * int64_t(row16);
  const int64_t pid = page_ids[p];
  const uint4* s = src + tok0 * row16;
  uint4* d = pool + pid * page16;
  const int64_t base = int64_t(blockIdx.x) * (kCopyThreads * kCopyUnroll) + threadIdx.x;
  uint4 val[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = base + u * kCopyThreads;
    val[u] = (i < valid16) ? s[i] : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = base + u * kCopyThreads;
    if (i < page16) store_stream16(d + i, val[u]);
  }
}

// Inverse: page p of chunk c -> rows [p*P, min(T, p*P+P)) of chunk c in dst.
__global__ __launch_bounds__(kCopyThreads) void gather_paged_kernel(
    const uint4* __restrict__ k_pool, const uint4* __restrict__ v_pool,
    const int32_t* __restrict__ page_ids, uint4* __restrict__ k_dst, uint4* __restrict__ v_dst,
    int32_t T, int32_t row16, int32_t P, int32_t ppc) {
  const int32_t c = blockIdx.y / ppc;
  const int32_t p = blockIdx.y - c * ppc;
  const uint4* pool = blockIdx.z ? v_pool : k_pool;
  uint4* dst = blockIdx.z ? v_dst : k_dst;
  const int64_t page16 = int64_t(P) * row16;
  const int64_t tok0 = int64_t(p) * P;
  const int64_t valid16 = (T - tok0 < P ? T - tok0 : P) * int64_t(row16);
  const int64_t pid = page_ids[blockIdx.y];
  const uint4* s = pool + pid * page16;
  uint4* d = dst + (int64_t(c) * T + tok0) * row16;
  const int64_t base = int64_t(blockIdx.x) * (kCopyThreads * kCopyUnroll) + threadIdx.x;
  uint4 val[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = base + u * kCopyThreads;
    if (i < valid16) val[u] = s[i];
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const int64_t i = base + u * kCopyThreads;
    if (i < valid16) store_stream16(d + i, val[u]);
  }
}

int32_t validate_paged(const char* where, const void* a, const void* b, const void* c,
                       const void* d, const int32_t* ids, int32_t T, int32_t H, int32_t D,
                       int32_t num_pages, int32_t P) {
  if (T < 0 || H <= 0 || D <= 0 || num_pages <= 0 || P <= 0)
    return fail(WF_EINVAL, "%s: bad sizes T=%d H=%d D=%d num_pages=%d P=%d", where, T, H, D,
                num_pages, P);
  if ((int64_t(H) * D * 2) % 16 != 0)
    return fail(WF_EINVAL, "%s: H*D*2 = %lld bytes is not a multiple of 16", where,
                static_cast<long long>(int64_t(H) * D * 2));
  if (T == 0) return WF_OK;
  if (!a || !b || !c || !d || !ids) return fail(WF_EINVAL, "%s: NULL pointer", where);
  if (!aligned16(a) || !aligned16(b) || !aligned16(c) || !aligned16(d))
    return fail(WF_EINVAL, "%s: tensors must be 16-byte aligned", where);
  const int64_t ppc = (int64_t(T) + P - 1) / P;
  if (ppc > num_pages)
    return fail(WF_EINVAL, "%s: chunk needs %lld pages, pool has %d", where,
                static_cast<long long>(ppc), num_pages);
  if (ppc > 65535) return fail(WF_EUNSUPPORTED, "%s: more than 65535 pages per chunk", where);
  return WF_OK;
}

}  // namespace
}  // namespace wf

extern "C" wf_status wf_store_paged(const void* k_src, const void* v_src, void* k_pool,
                                    void* v_pool, const int32_t* page_ids, int32_t T, int32_t H,
                                    int32_t D, int32_t num_pages, int32_t P, hipStream_t stream) {
  using namespace wf;
  try {
    int32_t st = validate_paged("wf_store_paged", k_src, v_src, k_pool, v_pool, page_ids, T, H, D,
                                num_pages, P);
    if (st != WF_OK || T == 0) return st;
    const int32_t ppc = int32_t((int64_t(T) + P - 1) / P);
    if (check_pages_enabled()) {
      st = check_device_pages(page_ids, ppc, num_pages, stream, "wf_store_paged");
      if (st != WF_OK) return st;
    }
    const int32_t row16 = int32_t(int64_t(H) * D * 2 / 16);
    const int64_t page16 = int64_t(P) * row16;
    const int64_t per_block = kCopyThreads * kCopyUnroll;
    dim3 grid(unsigned((page16 + per_block - 1) / per_block), unsigned(ppc), 2);
    store_paged_kernel<<<grid, kCopyThreads, 0, stream>>>(
        static_cast<const uint4*>(k_src), static_cast<const uint4*>(v_src),
        static_cast<uint4*>(k_pool), static_cast<uint4*>(v_pool), page_ids, T, row16, P);
    return check_launch("wf_store_paged");
  } catch (...) {
    return fail(WF_EINVAL, "wf_store_paged: internal error");
  }
}

extern "C" wf_status wf_gather_paged(const void* k_pool, const void* v_pool,
                                     const int32_t* page_ids, int32_t n_chunks, void* k_dst,
                                     void* v_dst, int32_t T, int32_t H, int32_t D,
                                     int32_t num_pages, int32_t P, hipStream_t stream) {
  using namespace wf;
  try {
    if (n_chunks < 0) return fail(WF_EINVAL, "wf_gather_paged: n_chunks = %d", n_chunks);
    int32_t st = validate_paged("wf_gather_paged", k_pool, v_pool, k_dst, v_dst, page_ids, T, H,
                                D, num_pages, P);
    if (st != WF_OK || T == 0 || n_chunks == 0) return st;
    const int32_t ppc = int32_t((int64_t(T) + P - 1) / P);
    if (int64_t(n_chunks) * ppc > 65535)
      return fail(WF_EUNSUPPORTED, "wf_gather_paged: more than 65535 pages in one call");
    if (check_pages_enabled()) {
      st = check_device_pages(page_ids, int64_t(n_chunks) * ppc, num_pages, stream,
                              "wf_gather_paged");
      if (st != WF_OK) return st;
    }
    const int32_t row16 = int32_t(int64_t(H) * D * 2 / 16);
    const int64_t page16 = int64_t(P) * row16;
    const int64_t per_block = kCopyThreads * kCopyUnroll;
    dim3 grid(unsigned((page16 + per_block - 1) / per_block), unsigned(n_chunks * ppc), 2);
    gather_paged_kernel<<<grid, kCopyThreads, 0, stream>>>(
        static_cast<const uint4*>(k_pool), static_cast<const uint4*>(v_pool), page_ids,
        static_cast<uint4*>(k_dst), static_cast<uint4*>(v_dst), T, row16, P, ppc);
    return check_launch("wf_gather_paged");
  } catch (...) {
    return fail(WF_EINVAL, "wf_gather_paged: internal error");
  }
}
