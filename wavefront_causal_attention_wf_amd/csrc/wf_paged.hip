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
// block copy; the kernels are bound by HBM bandwidth.
//
// Work split (measured on the 4680-token, 12 x 128 chunk with its sources
// rotated beyond the last-level cache): one flat index space over both tensors'
// units (16 bytes each), K's then V's, each thread taking kCopyUnroll units a
// grid-stride apart, so a block's loads are contiguous while a thread's lie far
// apart. That spreads each wave's requests over the memory channels better than
// giving a block a contiguous range of one page (5.2 -> 5.6 TB/s for the store).
// Sources are read once, so loads and stores are both nontemporal.
//
// The store runs as many blocks as the GPU keeps resident at once (8 of 256
// threads per CU, so every SIMD holds 8 waves) and each thread works through
// batches of up to kCopyUnroll units a grid-stride apart, the next batch's
// loads issued before the current batch's stores. For the 4680-token chunk
// that is one batch of 3-4 units per thread: 10.4 -> 10.1 us against one block
// per 4 units per thread (1776 blocks, 6.9 waves per SIMD). More blocks than
// stay resident measured slower, and so did issuing all of a thread's loads
// before any wait (13 us: in-flight requests spread over distant addresses).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "wf_internal.h"

namespace wf {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;

constexpr int kStoreBlocksPerCu = 8;  // 32 waves per CU: 8 per SIMD at <= 64 VGPRs

// Units [0, 2 * total): K's pages (z = 0), then V's (z = 1); unit e of a
// tensor is unit e % page16 of its page e / page16. Units at or past the
// chunk's last token (valid16) are written as zero. Batch j of a thread holds
// its units first + (j * kCopyUnroll + u) * stride.
struct CopyBatch {
  uint4 val[kCopyUnroll];
  uint64_t dst[kCopyUnroll];  // unit offset in its pool (bit 63: V); ~0: none
};

__device__ __forceinline__ void store_batch_load(CopyBatch& b, uint32_t base, uint32_t stride,
                                                 const uint4* __restrict__ k_src,
                                                 const uint4* __restrict__ v_src,
                                                 const int32_t* __restrict__ page_ids,
                                                 uint32_t valid16, uint32_t page16, uint32_t total) {
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const uint32_t e2 = base + u * stride;
    const bool z = e2 >= total;
    const uint32_t e = z ? e2 - total : e2;
    const bool in = e2 < 2 * total;
    b.val[u] = (in && e < valid16) ? load_stream16((z ? v_src : k_src) + e)
                                   : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t pg = e / page16;
    b.dst[u] = in ? (uint64_t(uint32_t(page_ids[pg])) * page16 + (e - pg * page16)) |
                        (uint64_t(z) << 63)
                  : ~uint64_t(0);
  }
}

__global__ __launch_bounds__(kCopyThreads) __attribute__((amdgpu_waves_per_eu(kStoreBlocksPerCu)))
void store_paged_kernel(const uint4* __restrict__ k_src, const uint4* __restrict__ v_src,
                        uint4* __restrict__ k_pool, uint4* __restrict__ v_pool,
                        const int32_t* __restrict__ page_ids, uint32_t valid16, uint32_t page16,
                        uint32_t total) {
  const uint32_t stride = gridDim.x * kCopyThreads;
  const uint32_t step = kCopyUnroll * stride;
  uint32_t base = blockIdx.x * kCopyThreads + threadIdx.x;
  CopyBatch cur;
  store_batch_load(cur, base, stride, k_src, v_src, page_ids, valid16, page16, total);
  while (true) {
    const bool more = base + step < 2 * total;  // (no wrap: checked on the host)
    CopyBatch nxt;
    if (more)
      store_batch_load(nxt, base + step, stride, k_src, v_src, page_ids, valid16, page16, total);
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      if (cur.dst[u] == ~uint64_t(0)) continue;
      const bool z = cur.dst[u] >> 63;
      store_stream16((z ? v_pool : k_pool) + (cur.dst[u] & ~(uint64_t(1) << 63)), cur.val[u]);
    }
    if (!more) break;
    cur = nxt;
    base += step;
  }
}

// Inverse: unit e of chunk c (tokens [0, T) only) comes from page
// page_ids[c * ppc + e / page16]. Units [0, 2 * n * valid16): K's chunks, then
// V's.
__global__ __launch_bounds__(kCopyThreads) void gather_paged_kernel(
    const uint4* __restrict__ k_pool, const uint4* __restrict__ v_pool,
    const int32_t* __restrict__ page_ids, uint4* __restrict__ k_dst, uint4* __restrict__ v_dst,
    uint32_t valid16, uint32_t page16, uint32_t ppc, uint32_t total) {
  const uint32_t stride = gridDim.x * kCopyThreads;
  const uint32_t first = blockIdx.x * kCopyThreads + threadIdx.x;
  uint4 val[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const uint32_t e2 = first + u * stride;
    if (e2 >= 2 * total) continue;
    const bool z = e2 >= total;
    const uint32_t ec = z ? e2 - total : e2;     // unit within the n chunks
    const uint32_t c = ec / valid16;
    const uint32_t e = ec - c * valid16;
    const uint32_t pg = e / page16;
    const uint64_t src = uint64_t(uint32_t(page_ids[c * ppc + pg])) * page16 + (e - pg * page16);
    val[u] = load_stream16((z ? v_pool : k_pool) + src);
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const uint32_t e2 = first + u * stride;
    if (e2 >= 2 * total) continue;
    const bool z = e2 >= total;
    store_stream16((z ? v_dst : k_dst) + (z ? e2 - total : e2), val[u]);
  }
}

// Blocks for the store's n_units 16-byte units: every resident slot filled (a
// thread may hold fewer than kCopyUnroll units), unless there are fewer units
// than threads.
int64_t copy_blocks(int64_t n_units) {
  const int64_t per_block = kCopyThreads * kCopyUnroll;
  const int cus = device_cu_count();
  const int64_t blocks = (n_units + kCopyThreads - 1) / kCopyThreads;
  return std::min<int64_t>(blocks, cus > 0 ? int64_t(kStoreBlocksPerCu) * cus
                                           : (n_units + per_block - 1) / per_block);
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
    const int64_t row16 = int64_t(H) * D * 2 / 16;
    const int64_t page16 = int64_t(P) * row16;
    const int64_t total = int64_t(ppc) * page16;  // units per tensor (whole pages)
    const int64_t blocks = copy_blocks(2 * total);
    // a thread's last batch start plus one step stays below 2^32
    if (2 * total + 2 * blocks * kCopyThreads * kCopyUnroll >= (int64_t(1) << 32) ||
        int64_t(num_pages) * page16 >= (int64_t(1) << 62))
      return fail(WF_EUNSUPPORTED, "wf_store_paged: chunk of %lld bytes too large",
                  static_cast<long long>(total * 16));
    const dim3 grid(static_cast<unsigned>(blocks));
    store_paged_kernel<<<grid, kCopyThreads, 0, stream>>>(
        static_cast<const uint4*>(k_src), static_cast<const uint4*>(v_src),
        static_cast<uint4*>(k_pool), static_cast<uint4*>(v_pool), page_ids,
        uint32_t(int64_t(T) * row16), uint32_t(page16), uint32_t(total));
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
    if (check_pages_enabled()) {
      st = check_device_pages(page_ids, int64_t(n_chunks) * ppc, num_pages, stream,
                              "wf_gather_paged");
      if (st != WF_OK) return st;
    }
    const int64_t row16 = int64_t(H) * D * 2 / 16;
    const int64_t page16 = int64_t(P) * row16;
    const int64_t valid16 = int64_t(T) * row16;
    const int64_t total = int64_t(n_chunks) * valid16;  // units per tensor
    if (2 * total + int64_t(kCopyThreads) * kCopyUnroll >= (int64_t(1) << 32) ||
        int64_t(num_pages) * page16 >= (int64_t(1) << 62))
      return fail(WF_EUNSUPPORTED, "wf_gather_paged: %lld bytes per tensor too large",
                  static_cast<long long>(total * 16));
    const int64_t per_block = kCopyThreads * kCopyUnroll;
    const dim3 grid(unsigned((2 * total + per_block - 1) / per_block));
    gather_paged_kernel<<<grid, kCopyThreads, 0, stream>>>(
        static_cast<const uint4*>(k_pool), static_cast<const uint4*>(v_pool), page_ids,
        static_cast<uint4*>(k_dst), static_cast<uint4*>(v_dst), uint32_t(valid16),
        uint32_t(page16), uint32_t(ppc), uint32_t(total));
    return check_launch("wf_gather_paged");
  } catch (...) {
    return fail(WF_EINVAL, "wf_gather_paged: internal error");
  }
}
