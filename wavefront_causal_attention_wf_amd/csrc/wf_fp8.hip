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
// and the product in fp32 (correctly rounded); a tile with amax below 2^-100
// is stored as zero (scale 0, zero codes). A tile is 64 consecutive tokens
// of one page (pages hold a multiple of 64 tokens), so the attention kernel's
// 64-key tiles each carry one scale per head.
//
// Layout: K codes [num_pages][P][H][D] bytes, scales [num_pages][P/64][H]
// fp32, V [num_pages][P][H][D] bf16; token t of the chunk goes to slot t % P of
// page page_ids[t / P]. Slots past the chunk's last token hold zero codes (and
// zero V), and a tile with no token of the chunk has scale 0.
//
// With 8-bit values (v_exp set) V is quantised too, per (64-token tile, head)
// with a power-of-two scale 2^e (e the smallest integer >= -127 with
// amax <= 448 * 2^e, 0 for an all-zero tile; v_exp holds e + 127) and stored the way the
// attention kernel's P.V operand reads it: the V pool is
// [num_pages][P/64][H][D][64] bytes, row d of tile (page, sub-tile, head)
// holding channel d of its 64 tokens in the order of the kernel's score
// registers — byte 32*g + j of a row is token
// 32*(j / 16) + 16*((j / 8) % 2) + 8*g + j % 8 of the tile.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "wf_internal.h"

namespace wf {
namespace {

constexpr int kQThreads = 256;
constexpr int kScaleTile = 64;
constexpr float kE4m3Max = 448.0f;
constexpr float kTinyAmax = 0x1p-100f;  // smaller key tiles are stored as zero

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Four bf16 values (two words) times inv -> four e4m3 codes, first value in
// the lowest byte.
__device__ __forceinline__ uint32_t e4m3x4(uint32_t w0, uint32_t w1, float inv) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(w0) * inv, bf16_hi(w0) * inv, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(w1) * inv, bf16_hi(w1) * inv, r, true);
  return uint32_t(r);
}

// Smallest e >= -127 with amax <= 448 * 2^e (amax > 0 and finite): amax =
// f * 2^E with 0.5 <= f < 1 and 448 = 0.875 * 2^9, so e = E - 9 when
// f <= 0.875, else E - 8; -127 is the smallest exponent of the E8M0 scale byte
// (a smaller tile keeps e = -127: its values times 2^127 stay below 448).
__device__ __forceinline__ int pow2_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  uint32_t u = __float_as_uint(amax);
  int E = int(u >> 23) - 126;
  if ((u >> 23) == 0) {  // subnormal m * 2^-149: leading one at bit 31 - clz
    const int shift = __clz(u) - 8;  // moves the leading one to bit 23
    E = -117 - __clz(u);
    u <<= shift;
  }
  const int e = ((u & 0x7fffffu) <= 0x600000u) ? E - 9 : E - 8;  // f <= 0.875 <=> mantissa <= 0.75
  return e < -127 ? -127 : e;
}

// Column of token t (0..63) within a transposed 8-bit V row (see above).
__device__ __forceinline__ int v8_column(int t) {
  return 32 * ((t >> 3) & 1) + 16 * ((t >> 5) & 1) + 8 * ((t >> 4) & 1) + (t & 7);
}

// bf16 values (v_exp NULL): a persistent grid. Each block walks units (chunk,
// tile, head) a grid-stride apart, the next unit's loads in flight while the
// current one is reduced and written; the grid is sized so that every block
// gets the same number of units and a CU at most two blocks (measured on a
// 4-step tick's five live chunks in one launch: 62 -> 68 % of HBM peak
// against one block per unit).
template <int D>
__global__ __launch_bounds__(kQThreads) void store_fp8_stream_kernel(
    const uint4* __restrict__ k_src, const uint4* __restrict__ v_src, uint8_t* __restrict__ k_pool,
    float* __restrict__ k_scale, uint4* __restrict__ v_pool, const int32_t* __restrict__ page_ids,
    int32_t T, int32_t H, int32_t P, int32_t tiles, int32_t ppc, int32_t n_units) {
  constexpr int UPR = D / 8;                             // 16-byte units per head row
  constexpr int UPT = kScaleTile * UPR / kQThreads;      // units per thread
  static_assert(UPT * kQThreads == kScaleTile * UPR, "tile must split evenly");
  const int spp = P / kScaleTile;
  __shared__ float wave_max[2][kQThreads / 64];  // by unit parity: no write waits on a read
  struct Buf { uint4 x[UPT], vx[UPT]; };
  auto load = [&](Buf& b, int unit) __attribute__((always_inline)) {
    const int h = unit % H;
    const int ct = unit / H;
    const int chunk = ct / tiles;
    const int tok0 = (ct - chunk * tiles) * kScaleTile;
    const uint4* ks = k_src + int64_t(chunk) * T * H * UPR;
    const uint4* vs = v_src + int64_t(chunk) * T * H * UPR;
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int e = threadIdx.x + u * kQThreads;
      const int tok = e / UPR;
      const int t = tok0 + tok;
      const int64_t src = (int64_t(t) * H + h) * UPR + (e - tok * UPR);
      b.x[u] = t < T ? load_stream16(ks + src) : make_uint4(0u, 0u, 0u, 0u);
      b.vx[u] = t < T ? load_stream16(vs + src) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto process = [&](const Buf& b, int unit, int par) __attribute__((always_inline)) {
    const int h = unit % H;
    const int ct = unit / H;
    const int chunk = ct / tiles;
    const int tile = ct - chunk * tiles;
    const int pg = tile / spp;
    const int sub = tile - pg * spp;
    const int64_t pid = page_ids[int64_t(chunk) * ppc + pg];
    float am = 0.f;
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const uint32_t w[4] = {b.x[u].x, b.x[u].y, b.x[u].z, b.x[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) am = fmaxf(am, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
    }
    // the value copy drains while the block reduces
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int e = threadIdx.x + u * kQThreads;
      const int tok = e / UPR;
      store_stream16(v_pool + ((pid * P + sub * kScaleTile + tok) * H + h) * UPR + (e - tok * UPR),
                     b.vx[u]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
    if ((threadIdx.x & 63) == 0) wave_max[par][threadIdx.x >> 6] = am;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kQThreads / 64; ++i) am = fmaxf(am, wave_max[par][i]);
    // a tile with amax below kTinyAmax is stored as zero (scale 0, zero codes)
    const bool big = am >= kTinyAmax;
    const float inv = big ? kE4m3Max / am : 0.f;
    if (threadIdx.x == 0) k_scale[(pid * spp + sub) * H + h] = big ? am / kE4m3Max : 0.f;
    typedef unsigned v2u __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int e = threadIdx.x + u * kQThreads;
      const int tok = e / UPR;
      const int64_t row = ((pid * P + sub * kScaleTile + tok) * H + h) * UPR + (e - tok * UPR);
      const v2u codes = {e4m3x4(b.x[u].x, b.x[u].y, inv), e4m3x4(b.x[u].z, b.x[u].w, inv)};
      // unit (16 bytes of bf16) -> 8 bytes of codes at half the offset
      __builtin_nontemporal_store(codes, reinterpret_cast<v2u*>(k_pool + row * 8));
    }
  };
  const int stride = gridDim.x;
  int unit = blockIdx.x;
  if (unit >= n_units) return;  // (the grid never exceeds the units)
  Buf a, b;
  load(a, unit);
  for (;;) {  // two units per pass, so that the buffers keep their names
    const int u1 = unit + stride;
    if (u1 < n_units) load(b, u1);
    process(a, unit, 0);
    if (u1 >= n_units) break;
    const int u2 = u1 + stride;
    if (u2 < n_units) load(a, u2);
    process(b, u1, 1);
    if (u2 >= n_units) break;
    unit = u2;
  }
}

// 8-bit values (v_exp set): block b handles unit b = (chunk, 64-token tile,
// head), head fastest, keys and values both: one reduction pass gives both
// maxima; the key codes and scale go out as in store_fp8_stream_kernel, the
// values as a power-of-two scale and codes written through a transposed LDS
// tile. One thread owns UPT 16-byte units (8 channels of one token) of each
// tensor, all loaded before any store. (One unit per block, keys and values
// together, measured 56.0 -> 41.7 us for a 4-step tick's five live chunks,
// against one block per unit and tensor; a persistent grid with the next
// unit's loads in flight needs twice the registers and was slower.)
template <int D>
__global__ __launch_bounds__(kQThreads) void store_fp8_v8_kernel(
    const uint4* __restrict__ k_src, const uint4* __restrict__ v_src, uint8_t* __restrict__ k_pool,
    float* __restrict__ k_scale, uint4* __restrict__ v_pool, uint8_t* __restrict__ v_exp,
    const int32_t* __restrict__ page_ids, int32_t T, int32_t H, int32_t P, int32_t tiles,
    int32_t ppc) {
  constexpr int UPR = D / 8;                             // 16-byte units per head row
  constexpr int UPT = kScaleTile * UPR / kQThreads;      // units per thread
  static_assert(UPT * kQThreads == kScaleTile * UPR, "tile must split evenly");
  const int spp = P / kScaleTile;
  const int unit = blockIdx.x;
  const int h = unit % H;
  const int ct = unit / H;
  const int chunk = ct / tiles;
  const int tile = ct - chunk * tiles;
  const int pg = tile / spp;
  const int sub = tile - pg * spp;
  const int tok0 = tile * kScaleTile;
  const uint4* ks = k_src + int64_t(chunk) * T * H * UPR;
  const uint4* vs = v_src + int64_t(chunk) * T * H * UPR;
  uint4 x[UPT], vx[UPT];
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const int e = threadIdx.x + u * kQThreads;
    const int tok = e / UPR;
    const int t = tok0 + tok;
    const int64_t src = (int64_t(t) * H + h) * UPR + (e - tok * UPR);
    x[u] = t < T ? load_stream16(ks + src) : make_uint4(0u, 0u, 0u, 0u);
    vx[u] = t < T ? load_stream16(vs + src) : make_uint4(0u, 0u, 0u, 0u);
  }
  const int64_t pid = page_ids[int64_t(chunk) * ppc + pg];
  float am = 0.f, vm = 0.f;
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const uint32_t w[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
    const uint32_t wv[4] = {vx[u].x, vx[u].y, vx[u].z, vx[u].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      am = fmaxf(am, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
      vm = fmaxf(vm, fmaxf(fabsf(bf16_lo(wv[i])), fabsf(bf16_hi(wv[i]))));
    }
  }
  // block maxima: within each wave, then across the four waves
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    am = fmaxf(am, __shfl_xor(am, off));
    vm = fmaxf(vm, __shfl_xor(vm, off));
  }
  __shared__ float wave_max[2][kQThreads / 64];  // [K, V][wave]
  __shared__ __attribute__((aligned(16))) uint8_t tile_t[D * kScaleTile];
  if ((threadIdx.x & 63) == 0) {
    wave_max[0][threadIdx.x >> 6] = am;
    wave_max[1][threadIdx.x >> 6] = vm;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kQThreads / 64; ++i) {
    am = fmaxf(am, wave_max[0][i]);
    vm = fmaxf(vm, wave_max[1][i]);
  }
  // values: power-of-two scale, codes into the transposed tile
  const int ev = pow2_exponent(vm);
  const float mul = __uint_as_float(uint32_t(127 - ev) << 23);  // 2^-e (exact)
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const int e = threadIdx.x + u * kQThreads;
    const int col = v8_column(e / UPR);
    const int d0 = (e % UPR) * 8;
    const uint32_t codes[2] = {e4m3x4(vx[u].x, vx[u].y, mul), e4m3x4(vx[u].z, vx[u].w, mul)};
#pragma unroll
    for (int i = 0; i < 8; ++i)
      tile_t[(d0 + i) * kScaleTile + col] = uint8_t(codes[i >> 2] >> (8 * (i & 3)));
  }
  // keys: a tile with amax below kTinyAmax is stored as zero (scale 0, zero
  // codes): 448 / amax would leave float32's range, or amax / 448 its normal range
  const bool big = am >= kTinyAmax;
  const float inv = big ? kE4m3Max / am : 0.f;
  if (threadIdx.x == 0) {
    k_scale[(pid * spp + sub) * H + h] = big ? am / kE4m3Max : 0.f;
    v_exp[(pid * spp + sub) * H + h] = uint8_t(ev + 127);
  }
  typedef unsigned v2u __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int u = 0; u < UPT; ++u) {
    const int e = threadIdx.x + u * kQThreads;
    const int tok = e / UPR;
    const int64_t row = ((pid * P + sub * kScaleTile + tok) * H + h) * UPR + (e - tok * UPR);
    const v2u codes = {e4m3x4(x[u].x, x[u].y, inv), e4m3x4(x[u].z, x[u].w, inv)};
    // unit (16 bytes of bf16) -> 8 bytes of codes at half the offset
    __builtin_nontemporal_store(codes, reinterpret_cast<v2u*>(k_pool + row * 8));
  }
  __syncthreads();
  const int64_t tile16 = ((pid * spp + sub) * H + h) * int64_t(D * kScaleTile / 16);
#pragma unroll
  for (int i = threadIdx.x; i < D * kScaleTile / 16; i += kQThreads)
    store_stream16(v_pool + tile16 + i, reinterpret_cast<const uint4*>(tile_t)[i]);
}
}  // namespace
}  // namespace wf

namespace wf {
namespace {

int32_t store_fp8(const char* where, const void* k_src, const void* v_src, int32_t n_chunks,
                  void* k_pool, float* k_scale, void* v_pool, uint8_t* v_exp,
                  const int32_t* page_ids, int32_t T, int32_t H, int32_t D, int32_t num_pages,
                  int32_t P, hipStream_t stream) {
  if (T < 0 || H <= 0 || num_pages <= 0 || P <= 0 || n_chunks < 0)
    return fail(WF_EINVAL, "%s: bad sizes T=%d H=%d num_pages=%d P=%d n_chunks=%d", where, T, H,
                num_pages, P, n_chunks);
  if (D != 64 && D != 128)
    return fail(WF_EUNSUPPORTED, "%s: head dim D = %d (supported: 64, 128)", where, D);
  if (P % kScaleTile != 0)
    return fail(WF_EINVAL, "%s: page size P = %d must be a multiple of 64", where, P);
  if (T == 0 || n_chunks == 0) return WF_OK;
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
  const int64_t tiles = ppc * (P / kScaleTile);
  if (int64_t(n_chunks) * tiles > 0x7fffffff)
    return fail(WF_EUNSUPPORTED, "%s: %d chunks of %lld tiles exceed the grid", where, n_chunks,
                static_cast<long long>(tiles));
  if (check_pages_enabled()) {
    const int32_t st = check_device_pages(page_ids, int64_t(n_chunks) * ppc, num_pages, stream, where);
    if (st != WF_OK) return st;
  }
  if (!v_exp) {
    // every block the same number of units, at most two blocks per CU
    const int64_t n_units = int64_t(n_chunks) * tiles * H;
    if (n_units > 0x7fffffff)
      return fail(WF_EUNSUPPORTED, "%s: %lld (tile, head) units exceed 2^31", where,
                  static_cast<long long>(n_units));
    const int64_t slots = 2 * int64_t(std::max(device_cu_count(), 1));
    const int64_t per_block = (n_units + slots - 1) / slots;
    const unsigned blocks = unsigned((n_units + per_block - 1) / per_block);
    if (D == 128)
      store_fp8_stream_kernel<128><<<blocks, kQThreads, 0, stream>>>(
          static_cast<const uint4*>(k_src), static_cast<const uint4*>(v_src),
          static_cast<uint8_t*>(k_pool), k_scale, static_cast<uint4*>(v_pool), page_ids, T, H, P,
          int32_t(tiles), int32_t(ppc), int32_t(n_units));
    else
      store_fp8_stream_kernel<64><<<blocks, kQThreads, 0, stream>>>(
          static_cast<const uint4*>(k_src), static_cast<const uint4*>(v_src),
          static_cast<uint8_t*>(k_pool), k_scale, static_cast<uint4*>(v_pool), page_ids, T, H, P,
          int32_t(tiles), int32_t(ppc), int32_t(n_units));
    return check_launch(where);
  }
  // 8-bit values: one block per (chunk, tile, head)
  const int64_t n_units = int64_t(n_chunks) * tiles * H;
  if (n_units > 0x7fffffff)
    return fail(WF_EUNSUPPORTED, "%s: %lld (tile, head) units exceed 2^31", where,
                static_cast<long long>(n_units));
  if (D == 128)
    store_fp8_v8_kernel<128><<<unsigned(n_units), kQThreads, 0, stream>>>(
        static_cast<const uint4*>(k_src), static_cast<const uint4*>(v_src),
        static_cast<uint8_t*>(k_pool), k_scale, static_cast<uint4*>(v_pool), v_exp, page_ids, T,
        H, P, int32_t(tiles), int32_t(ppc));
  else
    store_fp8_v8_kernel<64><<<unsigned(n_units), kQThreads, 0, stream>>>(
        static_cast<const uint4*>(k_src), static_cast<const uint4*>(v_src),
        static_cast<uint8_t*>(k_pool), k_scale, static_cast<uint4*>(v_pool), v_exp, page_ids, T,
        H, P, int32_t(tiles), int32_t(ppc));
  return check_launch(where);
}

}  // namespace
}  // namespace wf

extern "C" wf_status wf_store_paged_fp8(const void* k_src, const void* v_src, void* k_pool,
                                        float* k_scale, void* v_pool, uint8_t* v_exp,
                                        const int32_t* page_ids, int32_t T, int32_t H, int32_t D,
                                        int32_t num_pages, int32_t P, hipStream_t stream) {
  try {
    return wf::store_fp8("wf_store_paged_fp8", k_src, v_src, 1, k_pool, k_scale, v_pool, v_exp,
                         page_ids, T, H, D, num_pages, P, stream);
  } catch (...) {
    return wf::fail(WF_EINVAL, "wf_store_paged_fp8: internal error");
  }
}

extern "C" wf_status wf_store_paged_fp8_chunks(const void* k_src, const void* v_src,
                                               int32_t n_chunks, void* k_pool, float* k_scale,
                                               void* v_pool, uint8_t* v_exp,
                                               const int32_t* page_ids, int32_t T, int32_t H,
                                               int32_t D, int32_t num_pages, int32_t P,
                                               hipStream_t stream) {
  try {
    return wf::store_fp8("wf_store_paged_fp8_chunks", k_src, v_src, n_chunks, k_pool, k_scale,
                         v_pool, v_exp, page_ids, T, H, D, num_pages, P, stream);
  } catch (...) {
    return wf::fail(WF_EINVAL, "wf_store_paged_fp8_chunks: internal error");
  }
}
