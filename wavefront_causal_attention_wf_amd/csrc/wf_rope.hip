// wf_rope_store_paged: rotary position embedding of a chunk's keys fused with
// the page write of its K and V.
//
// "Wave Forcing: Towards Speed-of-Light Streaming Video Generation":
//   summary page, Methodology 3, and full text Appendix B.1 — K/V are published
//     after the QKV projection and RoPE, so pages hold rotated keys;
//   full text Appendix B.8, Eq. (13) — the K/V arrays hold the anchor, the
//     bounded history, the live store and the denoising chunks, so every live
//     chunk is written into pages by its producer;
//   full text Appendix B.3 — the anchor keeps its unrotated key and is rotated
//     again when the window shifts (the same call, K only, at the new frames).
//
// Rotation (the pages do not spell it out; the common rotary form, applied per
// axis of the latent grid): token t of a F x R x C grid sits at frame
// frame0 + t / (R*C), row (t / C) % R, column t % C; channel pair (2i, 2i+1) of
// every head turns by coordinate * frequency, the coordinate being the one of
// the axis group the pair belongs to (split[0] frame channels, then split[1]
// row channels, then split[2] column channels), frequency theta^(-2i'/d) with
// i' the pair index inside its group of d channels. fp32 arithmetic, bf16
// result rounded to nearest even.
//
// Layout and cost: one thread owns one 16-byte unit (four channel pairs) of one
// token for four heads, so each angle's sine and cosine serve four heads and
// four 16-byte loads are in flight per thread. A wave covers 4 (D = 128) or 8
// (D = 64) tokens, 256 contiguous bytes per (token, head) row. HBM-bound: reads
// K and V once and writes whole pages (zeros past the chunk's last token), both
// nontemporal.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "wf_internal.h"

namespace wf {
namespace {

constexpr int kRopeThreads = 256;
constexpr int kRopeHeads = 4;  // heads per thread: four 16-byte loads in flight
constexpr int kMaxPairs = 64;  // D <= 128

struct RopeParams {
  const uint4* k_src;
  const uint4* v_src;
  uint4* k_pool;
  uint4* v_pool;
  const int32_t* page_ids;
  int32_t T, H, P;
  int32_t tokens;         // ceil(T / P) * P: every slot of the chunk's pages
  int32_t rows, cols;     // R and C of the latent grid
  int32_t frame0;         // first frame of chunk 0
  int32_t frame_step;     // chunk c starts at frame0 + c * frame_step
  int32_t tblocks;        // token blocks per chunk
  int32_t ppc;            // pages per chunk
  float inv_freq[kMaxPairs];  // per channel pair
  int32_t axis[kMaxPairs];    // 0 frame, 1 row, 2 column
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> two bf16 (nearest even) packed low | high << 16.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const __bf16 a = static_cast<__bf16>(lo);
  const __bf16 b = static_cast<__bf16>(hi);
  return uint32_t(__builtin_bit_cast(uint16_t, a)) | (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

// Rotate the two channel pairs held in one 32-bit word pair-wise: word w holds
// channels (2i, 2i+1) as (low, high).
__device__ __forceinline__ uint32_t rotate_word(uint32_t w, float c, float s) {
  const float x0 = bf16_lo(w), x1 = bf16_hi(w);
  return pack_bf16(x0 * c - x1 * s, x0 * s + x1 * c);
}

// blockIdx.x: chunk c = x / tblocks, token block x % tblocks; blockIdx.z == 0:
// K (rotated), 1: V (copied); blockIdx.y: heads [kRopeHeads * y, kRopeHeads *
// y + kRopeHeads). Tokens [T, ppc*P) of the last page are written as zero.
template <int D>
__global__ __launch_bounds__(kRopeThreads) void rope_store_kernel(const RopeParams p) {
  constexpr int U = D / 8;                 // 16-byte units per (token, head) row
  constexpr int TPB = kRopeThreads / U;    // tokens per block
  const int u = threadIdx.x % U;
  const int chunk = int(blockIdx.x) / p.tblocks;
  const int t = (int(blockIdx.x) - chunk * p.tblocks) * TPB + threadIdx.x / U;
  if (t >= p.tokens) return;  // past the last page
  const int H = p.H;
  const int h0 = blockIdx.y * kRopeHeads;
  const int nh = H - h0 < kRopeHeads ? H - h0 : kRopeHeads;
  const int32_t page = t / p.P;
  const int32_t slot = t - page * p.P;
  const int64_t pid = p.page_ids[int64_t(chunk) * p.ppc + page];
  const bool is_v = blockIdx.z != 0;
  uint4* dst = (is_v ? p.v_pool : p.k_pool) + ((pid * p.P + slot) * H + h0) * U + u;
  uint4 x[kRopeHeads] = {};  // (heads past H stay zero: rotated, never stored)
  if (t >= p.T) {  // tail slot of the last page
#pragma unroll
    for (int i = 0; i < kRopeHeads; ++i)
      if (i < nh) store_stream16(dst + int64_t(i) * U, make_uint4(0u, 0u, 0u, 0u));
    return;
  }
  const uint4* src = (is_v ? p.v_src : p.k_src) + ((int64_t(chunk) * p.T + t) * H + h0) * U + u;
#pragma unroll
  for (int i = 0; i < kRopeHeads; ++i)  // every load in flight before any store
    if (i < nh) x[i] = load_stream16(src + int64_t(i) * U);
  if (!is_v) {
    // the four pairs of this unit: 4u .. 4u+3
    const int rc = p.rows * p.cols;
    const int f = t / rc;
    const int rem = t - f * rc;
    const int row = rem / p.cols;
    const float cf = float(p.frame0 + chunk * p.frame_step + f), cr = float(row),
                cc = float(rem - row * p.cols);
    float cs[4], sn[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int pr = 4 * u + j;
      const int a = p.axis[pr];
      const float ang = (a == 0 ? cf : (a == 1 ? cr : cc)) * p.inv_freq[pr];
      sincosf(ang, &sn[j], &cs[j]);
    }
#pragma unroll
    for (int i = 0; i < kRopeHeads; ++i)
      x[i] = make_uint4(rotate_word(x[i].x, cs[0], sn[0]), rotate_word(x[i].y, cs[1], sn[1]),
                        rotate_word(x[i].z, cs[2], sn[2]), rotate_word(x[i].w, cs[3], sn[3]));
  }
#pragma unroll
  for (int i = 0; i < kRopeHeads; ++i)
    if (i < nh) store_stream16(dst + int64_t(i) * U, x[i]);
}

}  // namespace
}  // namespace wf

namespace wf {
namespace {

int32_t rope_store(const char* where, const void* k_src, const void* v_src, int32_t n_chunks,
                   void* k_pool, void* v_pool, const int32_t* page_ids, int32_t T, int32_t H,
                   int32_t D, int32_t num_pages, int32_t P, const wf_rope_desc* rope,
                   int32_t frame_step, hipStream_t stream) {
  if (!rope) return fail(WF_EINVAL, "%s: NULL rope descriptor", where);
  if (T < 0 || H <= 0 || num_pages <= 0 || P <= 0 || n_chunks < 0)
    return fail(WF_EINVAL, "%s: bad sizes T=%d H=%d num_pages=%d P=%d n_chunks=%d", where, T, H,
                num_pages, P, n_chunks);
  if (D != 64 && D != 128) return fail(WF_EUNSUPPORTED, "%s: D=%d (64 or 128)", where, D);
  if (T == 0 || n_chunks == 0) return WF_OK;
  const int64_t cells = int64_t(rope->grid[0]) * rope->grid[1] * rope->grid[2];
  if (rope->grid[0] <= 0 || rope->grid[1] <= 0 || rope->grid[2] <= 0 || cells != T)
    return fail(WF_EINVAL, "%s: grid %d x %d x %d does not hold T=%d tokens", where,
                rope->grid[0], rope->grid[1], rope->grid[2], T);
  for (int64_t c : {int64_t(0), int64_t(n_chunks) - 1}) {  // first frames are monotone in c
    const int64_t f0 = int64_t(rope->frame0) + c * frame_step;
    if (f0 < 0 || f0 + rope->grid[0] > (int64_t(1) << 24))
      return fail(WF_EINVAL, "%s: chunk %lld starts at frame %lld, outside [0, 2^24 - frames]",
                  where, static_cast<long long>(c), static_cast<long long>(f0));
  }
  for (int a = 0; a < 3; ++a)
    if (rope->split[a] < 0 || rope->split[a] % 2)
      return fail(WF_EINVAL, "%s: split[%d]=%d must be even and >= 0", where, a, rope->split[a]);
  if (int64_t(rope->split[0]) + rope->split[1] + rope->split[2] != D)
    return fail(WF_EINVAL, "%s: split %d+%d+%d != D=%d", where, rope->split[0], rope->split[1],
                rope->split[2], D);
  if (!(rope->theta > 0.0f) || !std::isfinite(rope->theta))
    return fail(WF_EINVAL, "%s: theta must be positive and finite", where);
  if (!k_src || !k_pool || !page_ids) return fail(WF_EINVAL, "%s: NULL pointer", where);
  if ((v_src == nullptr) != (v_pool == nullptr))
    return fail(WF_EINVAL, "%s: v_src and v_pool must both be given or both be NULL", where);
  if (!aligned16(k_src) || !aligned16(k_pool) || (v_src && (!aligned16(v_src) || !aligned16(v_pool))))
    return fail(WF_EINVAL, "%s: tensors must be 16-byte aligned", where);
  const int64_t ppc = (int64_t(T) + P - 1) / P;
  if (ppc > num_pages)
    return fail(WF_EINVAL, "%s: chunk needs %lld pages, pool has %d", where,
                static_cast<long long>(ppc), num_pages);
  if (ppc * P >= (int64_t(1) << 31))
    return fail(WF_EUNSUPPORTED, "%s: ceil(T/P)*P must stay below 2^31", where);
  const int tpb = kRopeThreads / (D / 8);
  const int64_t tblocks = (ppc * P + tpb - 1) / tpb;
  if (int64_t(n_chunks) * tblocks > 0x7fffffff)
    return fail(WF_EUNSUPPORTED, "%s: %d chunks exceed the grid", where, n_chunks);
  if (check_pages_enabled()) {
    int32_t st = check_device_pages(page_ids, int64_t(n_chunks) * ppc, num_pages, stream, where);
    if (st != WF_OK) return st;
  }
  RopeParams p{};
  p.k_src = static_cast<const uint4*>(k_src);
  p.v_src = static_cast<const uint4*>(v_src);
  p.k_pool = static_cast<uint4*>(k_pool);
  p.v_pool = static_cast<uint4*>(v_pool);
  p.page_ids = page_ids;
  p.T = T;
  p.H = H;
  p.P = P;
  p.rows = rope->grid[1];
  p.cols = rope->grid[2];
  p.frame0 = rope->frame0;
  p.frame_step = frame_step;
  p.tblocks = int32_t(tblocks);
  p.ppc = int32_t(ppc);
  p.tokens = int32_t(ppc * P);
  int pr = 0;
  for (int a = 0; a < 3; ++a)
    for (int i = 0; i < rope->split[a] / 2; ++i, ++pr) {
      p.axis[pr] = a;
      p.inv_freq[pr] = float(std::pow(double(rope->theta), -2.0 * i / rope->split[a]));
    }
  dim3 grid(unsigned(int64_t(n_chunks) * tblocks), unsigned((H + kRopeHeads - 1) / kRopeHeads),
            v_src ? 2 : 1);
  if (D == 128) rope_store_kernel<128><<<grid, kRopeThreads, 0, stream>>>(p);
  else rope_store_kernel<64><<<grid, kRopeThreads, 0, stream>>>(p);
  return check_launch(where);
}

}  // namespace
}  // namespace wf

extern "C" wf_status wf_rope_store_paged(const void* k_src, const void* v_src, void* k_pool,
                                         void* v_pool, const int32_t* page_ids, int32_t T,
                                         int32_t H, int32_t D, int32_t num_pages, int32_t P,
                                         const wf_rope_desc* rope, hipStream_t stream) {
  try {
    return wf::rope_store("wf_rope_store_paged", k_src, v_src, 1, k_pool, v_pool, page_ids, T, H,
                          D, num_pages, P, rope, 0, stream);
  } catch (...) {
    return wf::fail(WF_EINVAL, "wf_rope_store_paged: internal error");
  }
}

extern "C" wf_status wf_rope_store_paged_chunks(const void* k_src, const void* v_src,
                                                int32_t n_chunks, void* k_pool, void* v_pool,
                                                const int32_t* page_ids, int32_t T, int32_t H,
                                                int32_t D, int32_t num_pages, int32_t P,
                                                const wf_rope_desc* rope, int32_t frame_step,
                                                hipStream_t stream) {
  try {
    return wf::rope_store("wf_rope_store_paged_chunks", k_src, v_src, n_chunks, k_pool, v_pool,
                          page_ids, T, H, D, num_pages, P, rope, frame_step, stream);
  } catch (...) {
    return wf::fail(WF_EINVAL, "wf_rope_store_paged_chunks: internal error");
  }
}
