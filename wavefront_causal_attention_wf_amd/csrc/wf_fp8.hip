// wf_store_paged_fp8: a producer's write of one chunk into the pages of the
// 8-bit tier — keys as e4m3 codes with one fp32 scale per (64-token tile,
// head), values copied as bf16.
//
// "Wave Forcing: Towards Speed-of-Light Streaming Video Generation", full text
// §4.3 (K/V quantisation shrinks the K/V payload; an 8-bit attention backend
// for local computation), Appendix C.5 Table 8 and C.6 (FP8 K/V): the pages
// name the technique but not the format or the scale granularity. Here: e4m3
// (largest finite value 448), scale = amax / 448 over the tile's keys of one
// head, code = e4m3(x * (448 / amax)) rounded to nearest even, both divisions
// and the product in fp32 (correctly rounded). A tile is 64 consecutive tokens
// of one page (pages hold a multiple of 64 tokens), so the attention kernel's
// 64-key tiles each carry one scale per head.
//
// Layout: K codes [num_pages][P][H][D] bytes, scales [num_pages][P/64][H]
// fp32, V [num_pages][P][H][D] bf16; token t of the chunk goes to slot t % P of
// page page_ids[t / P]. Slots past the chunk's last token hold zero codes (and
// zero V), and a tile with no token of the chunk has scale 0.
//
// With 8-bit values (v_exp set) V is quantised too, per (64-token tile, head)
// with a power-of-two scale 2^e (e the smallest integer with amax <= 448 * 2^e,
// 0 for an all-zero tile; v_exp holds e + 127) and stored the way the
// attention kernel's P.V operand reads it: the V pool is
// [num_pages][P/64][H][D][64] bytes, row d of tile (page, sub-tile, head)
// holding channel d of its 64 tokens in the order of the kernel's score
// registers — byte 32*g + j of a row is token
// 32*(j / 16) + 16*((j / 8) % 2) + 8*g + j % 8 of the tile.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "wf_internal.h"

namespace wf {
namespace {

constexpr int kQThreads = 256;
constexpr int kScaleTile = 64;
constexpr float kE4m3Max = 448.0f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Four bf16 values (two words) times inv -> four e4m3 codes, first value in
// the lowest byte.
__device__ __forceinline__ uint32_t e4m3x4(uint32_t w0, uint32_t w1, float inv) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(w0) * inv, bf16_hi(w0) * inv, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(w1) * inv, bf16_hi(w1) * inv, r, true);
  return uint32_t(r);
}

// Smallest e with amax <= 448 * 2^e (amax > 0 and finite): amax = f * 2^E with
// 0.5 <= f < 1 and 448 = 0.875 * 2^9, so e = E - 9 when f <= 0.875, else E - 8.
__device__ __forceinline__ int pow2_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  uint32_t u = __float_as_uint(amax);
  int E = int(u >> 23) - 126;
  if ((u >> 23) == 0) {  // subnormal m * 2^-149: leading one at bit 31 - clz
    const int shift = __clz(u) - 8;  // moves the leading one to bit 23
    E = -117 - __clz(u);
    u <<= shift;
  }
  return ((u & 0x7fffffu) <= 0x600000u) ? E - 9 : E - 8;  // f <= 0.875 <=> mantissa <= 0.75
}

// Column of token t (0..63) within a transposed 8-bit V row (see above).
__device__ __forceinline__ int v8_column(int t) {
  return 32 * ((t >> 3) & 1) + 16 * ((t >> 5) & 1) + 8 * ((t >> 4) & 1) + (t & 7);
}

// Block (x = 64-token tile in page order, y = head, z = 0): the tile's keys of
// head h -> codes and scale, and (bf16 values) its values of head h copied;
// z = 1 (8-bit values only): its values of head h -> codes in the transposed
// tile and the exponent. One thread owns UPT 16-byte units (8 channels of one
// token), all loaded before any store; bf16 values are copied before the
// block's amax reduction.
template <int D>
__global__ __launch_bounds__(kQThreads) void store_fp8_kernel(
    const uint4* __restrict__ k_src, const uint4* __restrict__ v_src, uint8_t* __restrict__ k_pool,
    float* __restrict__ k_scale, uint4* __restrict__ v_pool, uint8_t* __restrict__ v_exp,
    const int32_t* __restrict__ page_ids, int32_t T, int32_t H, int32_t P) {
  constexpr int UPR = D / 8;                             // 16-byte units per head row
  constexpr int UPT = kScaleTile * UPR / kQThreads;      // units per thread
  static_assert(UPT * kQThreads == kScaleTile * UPR, "tile must split evenly");
  const int tile = blockIdx.x;
  const int h = blockIdx.y;
  const bool v8 = v_exp != nullptr;
  const bool is_v = blockIdx.z != 0;                     // (only with 8-bit values)
  const int spp = P / kScaleTile;
  const int pg = tile / spp;
  const int sub = tile - pg * spp;
  const int64_t pid = page_ids[pg];
  const int tok0 = tile * kScaleTile;

  uint4 x[UPT], vx[UPT];
  int64_t dst_row[UPT];
  float am = 0.f;
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const int e = threadIdx.x + u * kQThreads;
    const int tok = e / UPR;
    const int c = e - tok * UPR;
    const int t = tok0 + tok;
    const int64_t src = (int64_t(t) * H + h) * UPR + c;
    x[u] = t < T ? (is_v ? v_src : k_src)[src] : make_uint4(0u, 0u, 0u, 0u);
    vx[u] = (t < T && !v8) ? v_src[src] : make_uint4(0u, 0u, 0u, 0u);
    dst_row[u] = ((pid * P + sub * kScaleTile + tok) * H + h) * UPR + c;  // in 16-byte units
  }
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const uint32_t w[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) am = fmaxf(am, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
  }
  // bf16 values need no scale: their copy drains while the block reduces
  if (!v8) {
#pragma unroll
    for (int u = 0; u < UPT; ++u) store_stream16(v_pool + dst_row[u], vx[u]);
  }
  // block max: within each wave, then across the four waves
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
  __shared__ float wave_max[kQThreads / 64];
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = am;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kQThreads / 64; ++i) am = fmaxf(am, wave_max[i]);

  if (is_v) {  // 8-bit values: power-of-two scale, transposed tile
    __shared__ __attribute__((aligned(16))) uint8_t tile_t[D * kScaleTile];
    const int e = pow2_exponent(am);
    const float mul = __uint_as_float(uint32_t(127 - e) << 23);  // 2^-e (exact)
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int unit = threadIdx.x + u * kQThreads;
      const int col = v8_column(unit / UPR);
      const int d0 = (unit % UPR) * 8;
      const uint32_t codes[2] = {e4m3x4(x[u].x, x[u].y, mul), e4m3x4(x[u].z, x[u].w, mul)};
#pragma unroll
      for (int i = 0; i < 8; ++i)
        tile_t[(d0 + i) * kScaleTile + col] = uint8_t(codes[i >> 2] >> (8 * (i & 3)));
    }
    __syncthreads();
    const int64_t tile16 = ((pid * spp + sub) * H + h) * int64_t(D * kScaleTile / 16);
    for (int i = threadIdx.x; i < D * kScaleTile / 16; i += kQThreads)
      store_stream16(v_pool + tile16 + i, reinterpret_cast<const uint4*>(tile_t)[i]);
    if (threadIdx.x == 0) v_exp[(pid * spp + sub) * H + h] = uint8_t(e + 127);
    return;
  }
  const float inv = am > 0.f ? kE4m3Max / am : 0.f;
  if (threadIdx.x == 0) k_scale[(pid * spp + sub) * H + h] = am / kE4m3Max;

  typedef unsigned v2u __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const v2u codes = {e4m3x4(x[u].x, x[u].y, inv), e4m3x4(x[u].z, x[u].w, inv)};
    // unit (16 bytes of bf16) -> 8 bytes of codes at half the offset
    __builtin_nontemporal_store(codes, reinterpret_cast<v2u*>(k_pool + dst_row[u] * 8));
  }
}

}  // namespace
}  // namespace wf

extern "C" wf_status wf_store_paged_fp8(const void* k_src, const void* v_src, void* k_pool,
                                        float* k_scale, void* v_pool, uint8_t* v_exp,
                                        const int32_t* page_ids, int32_t T, int32_t H, int32_t D,
                                        int32_t num_pages, int32_t P, hipStream_t stream) {
  using namespace wf;
  try {
    const char* where = "wf_store_paged_fp8";
    if (T < 0 || H <= 0 || num_pages <= 0 || P <= 0)
      return fail(WF_EINVAL, "%s: bad sizes T=%d H=%d num_pages=%d P=%d", where, T, H, num_pages,
                  P);
    if (D != 64 && D != 128)
      return fail(WF_EUNSUPPORTED, "%s: head dim D = %d (supported: 64, 128)", where, D);
    if (P % kScaleTile != 0)
      return fail(WF_EINVAL, "%s: page size P = %d must be a multiple of 64", where, P);
    if (T == 0) return WF_OK;
    if (!k_src || !v_src || !k_pool || !k_scale || !v_pool || !page_ids)
      return fail(WF_EINVAL, "%s: NULL pointer", where);
    if (!aligned16(k_src) || !aligned16(v_src) || !aligned16(k_pool) || !aligned16(v_pool) ||
        (reinterpret_cast<uintptr_t>(k_scale) & 3u))
      return fail(WF_EINVAL, "%s: tensors must be 16-byte aligned (scales 4-byte)", where);
    const int64_t ppc = (int64_t(T) + P - 1) / P;
    if (ppc > num_pages)
      return fail(WF_EINVAL, "%s: chunk needs %lld pages, pool has %d", where,
                  static_cast<long long>(ppc), num_pages);
    if (H > 65535) return fail(WF_EUNSUPPORTED, "%s: H = %d exceeds 65535", where, H);
    if (check_pages_enabled()) {
      const int32_t st = check_device_pages(page_ids, ppc, num_pages, stream, where);
      if (st != WF_OK) return st;
    }
    const dim3 grid(unsigned(ppc * (P / kScaleTile)), unsigned(H), v_exp ? 2 : 1);
    if (D == 128)
      store_fp8_kernel<128><<<grid, kQThreads, 0, stream>>>(
          static_cast<const uint4*>(k_src), static_cast<const uint4*>(v_src),
          static_cast<uint8_t*>(k_pool), k_scale, static_cast<uint4*>(v_pool), v_exp, page_ids, T,
          H, P);
    else
      store_fp8_kernel<64><<<grid, kQThreads, 0, stream>>>(
          static_cast<const uint4*>(k_src), static_cast<const uint4*>(v_src),
          static_cast<uint8_t*>(k_pool), k_scale, static_cast<uint4*>(v_pool), v_exp, page_ids, T,
          H, P);
    return check_launch(where);
  } catch (...) {
    return fail(WF_EINVAL, "wf_store_paged_fp8: internal error");
  }
}
