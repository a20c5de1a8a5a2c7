// wf_attn_tick: every query chunk of one wave tick in a single launch.
//
// "Wave Forcing: Towards Speed-of-Light Streaming Video Generation":
//   summary page, Methodology 1 — tick sets F_k, W_k (store = stage S) and the
//     ordered context C_{k,s} = anchor + history + live store + live j >= s;
//   full text Eq. (4) — wave mask M_WF(s, j) = 1[j >= s];
//   full text Eq. (5), Appendix B.3 — context order and store visibility
//     (history + itself);
//   summary page, Methodology 3 — rank s reads N_s = N_prefix + (S - s) N_C
//     keys, so stage 0 is the heaviest.
//
// Design (gfx950, wave64, MFMA):
//  * One workgroup = 8 waves = 256 query rows of one (stage, head); each wave
//    owns 32 query rows (two waves per SIMD, one workgroup per CU). The context
//    of the stage is walked chunk by chunk (history chunks through the page
//    table, live store, live j >= s), each chunk cut into ceil(T/64) tiles of
//    64 keys whose last one is masked past T; noisier chunks j < s are not in
//    the walk at all (block-sparse skip).
//  * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_bf16: the query is the
//    MFMA column, so each lane holds one query row's scores and output and the
//    softmax needs only one cross-lane exchange (lane l <-> l+32) per tile.
//    K rows are fed to the MFMA in a bit-2/bit-3-swapped order so that the score
//    registers already are the P operand of the P.V product (no shuffles).
//  * K and V tiles [64 keys][D] stream from global memory straight into LDS
//    (16-byte direct loads, no register staging) into three buffers: the loads
//    of tile i+2 are issued between the Q.K^T MFMAs of tile i, and a tile ends
//    with one barrier that waits only for tile i+1. With pages of a multiple of
//    64 tokens a tile is one contiguous span of a page or a live chunk: its
//    base is a scalar (the page id comes from a scalar load of the page table)
//    and each lane adds a fixed offset. Rows are XOR-swizzled so that the MFMA
//    operand reads are free of LDS bank conflicts; V^T operands are fetched
//    with the gfx950 transposing LDS read (ds_read_b64_tr_b16), so V needs no
//    transpose on its way in.
//  * Online softmax in the exp2 domain (log2 e folded into the scale), fp32
//    state; the running max is only raised when a tile exceeds it by more than
//    8 (in log2 units), so the O rescale is rare (exact: numerator and
//    denominator share the same reference).
//  * Work order: (stage, head) groups, heaviest stage first, dealt to the 8
//    XCDs so that each XCD streams about the same number of keys and the query
//    tiles of a group share that XCD's L2.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>

#include "wf_internal.h"

namespace wf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int KT = 64;              // keys per tile
#ifndef WF_NWAVES
#define WF_NWAVES 8
#endif
constexpr int NWAVES = WF_NWAVES;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int QROWS = 32 * NWAVES;  // query rows per workgroup
constexpr float kLazyTau = 8.0f;    // raise the running max only beyond this (log2 units)
constexpr int kNumXcd = 8;          // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kXcdTable = 512;      // max (stage, head) groups in the XCD table
// History page table held in LDS (ids of all history pages of one tick).
constexpr int kMaxPageIds = 8192;

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* hist_pages;
  int32_t T, H, P, ppc;
  int32_t tps;            // tiles per chunk, ceil(T / 64)
  int32_t t_last;         // keys in a chunk's last tile, T - 64 * (tps - 1)
  uint32_t p_magic;       // floor(2^32 / P) + 1: t / P == umulhi(t, p_magic) for t*P < 2^32
  float c;                // scale * log2(e)
  int32_t ntq;            // query tiles per chunk
  int32_t items_per_stage;  // H * ntq
  int32_t n_page_ids;     // n_hist * ppc entries of hist_pages
  // XCD-aware order: block b runs on XCD b % 8 (round-robin dispatch); its
  // (b / 8)-th item is query tile (b / 8) % ntq of group xcd_groups[x][(b / 8) / ntq],
  // group = rank * H + head. Blocks past an XCD's list exit at once.
  int32_t use_xcd;
  int32_t xcd_stride;
  int16_t xcd_n[kNumXcd];
  int16_t xcd_groups[kXcdTable];
  // (32-bit entries: the kernel reads them with scalar loads, which are
  // dword-granular; a narrower type would turn them into vector loads)
  int32_t stage_of_rank[WF_MAX_STAGES];  // work order, heaviest stage first
  int32_t nseg[WF_MAX_STAGES];
  // per stage: segment code >= 0 is live slot j, < 0 is history chunk (-code - 1)
  int32_t seg[WF_MAX_STAGES][WF_MAX_SEGMENTS];
};

__device__ __forceinline__ int swap_bits23(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// XOR swizzles (on the 16-byte chunk index) of K and V tile rows, chosen so
// that the MFMA operand reads are free of LDS bank conflicts whether the LDS
// serves 128 or 256 bytes per clock (8 or 16 lanes of a 16-byte read, 16 or 32
// lanes of an 8-byte read, per pass):
//  * K: a read touches rows {0..3, 8..11} (+4, +16, ...) at one logical chunk;
//    any 8 such rows land in distinct chunks mod 8, and for D = 128 rows 0..15
//    in distinct chunks mod 16; for D = 64 (two rows per 256 bytes) the 8 rows
//    of one parity among 0..15 land in distinct chunks.
//  * V (transposed reads): a pass reads 32 contiguous bytes (16 lanes) or 64
//    bytes (32 lanes) from each of 4 consecutive rows; the row swizzle places
//    those pieces in distinct bank ranges.
template <int D>
__device__ __forceinline__ int kswz(int row) {
  if constexpr (D == 128) return (row & 3) | ((row >> 1) & 4) | ((row << 1) & 8);
  return (row & 3) ^ ((row >> 2) & 1) ^ ((row >> 1) & 4);
}
template <int D>
__device__ __forceinline__ int vswz(int row) {
  const int q = row & 3;
  if constexpr (D == 128) return (4 * q) ^ (2 * (q >> 1));
  return 2 * q;
}

__device__ __forceinline__ float xlane32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xlane32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef short i16x4 __attribute__((ext_vector_type(4)));

// LDS destination of a direct tile load, passed through an empty asm so that the
// compiler no longer knows which LDS buffer the load writes. It then inserts no
// waits of its own for these loads before LDS reads (which it would place
// conservatively, draining loads meant to stay in flight); the kernel orders
// them itself with tile_barrier(). Every LDS read is of a buffer whose loads
// have landed and been published by that barrier.
__device__ __forceinline__ lds_void* opaque_lds(const uint16_t* p) {
  uint32_t a = uint32_t(reinterpret_cast<uintptr_t>((const lds_void*)p));
  asm volatile("" : "+s"(a));
  return reinterpret_cast<lds_void*>(uintptr_t(a));
}

typedef const __attribute__((address_space(4))) int32_t* const_i32p;

// Tile loads straight from global memory into LDS (16 bytes per lane).
//
// The stage's key sequence is walked segment by segment (a segment = one chunk
// of T keys: a history chunk through its pages, or a live chunk), each cut into
// tps = ceil(T / 64) tiles of 64 keys; only the last tile of a segment is
// partial (its rows past the chunk re-read the chunk's last key and are masked
// in the softmax). Wave w fills rows [RW*w, RW*w + RW) of the K and V tiles; one
// wave instruction writes 1 KB = RPI whole rows, lane l landing at chunk l % DC
// of row l / DC, so each lane fetches the logical chunk that the row swizzle
// maps to that position.
//
// kFast (page size a multiple of 64, and every live chunk): a tile is 64
// consecutive rows of one page or chunk, so its source is one uniform base
// (scalar registers; the page id comes from a scalar load of the page table)
// plus a fixed per-lane offset, and a tile costs no vector address math.
// Otherwise history tiles resolve each lane's page through the page table in
// LDS. prepare() resolves the next tile and advances the cursor; emit(i) issues
// the two loads of row group i, so the caller can spread them between MFMAs.
// Past the last tile the cursor reads tile 0 again (finite, masked).
template <int D, bool kFast>
struct TileLoader {
  static constexpr int DC = D / 8;        // 16-byte chunks per row
  static constexpr int RPI = 64 / DC;     // rows per wave instruction
  static constexpr int RW = KT / NWAVES;  // tile rows loaded by each wave
  static constexpr int NI = RW / RPI;     // instructions per wave per tensor

  // per lane (bytes): row offset + swizzled column, full and last-tile rows
  uint32_t koff[NI], voff[NI], koff_r[NI], voff_r[NI];
  int32_t row[NI];
  // cursor: next tile to resolve
  int seg, m;
  // resolved tile: uniform bases (+ the per-lane offsets), or for per-lane
  // history tiles the pool bases of head h and each lane's pool row
  const char* kb;
  const char* vb;
  bool ragged;
  bool per_lane;
  uint32_t prow[NI];

  __device__ __forceinline__ void init(const AttnParams& p, int wave, int lane) {
    const uint32_t row_bytes = uint32_t(p.H) * D * 2;
    const int pc = lane % DC;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      row[i] = wave * RW + RPI * i + lane / DC;
      const int rr = row[i] < p.t_last ? row[i] : p.t_last - 1;
      const uint32_t kc = uint32_t(pc ^ kswz<D>(row[i])) * 16;
      const uint32_t vc = uint32_t(pc ^ vswz<D>(row[i])) * 16;
      koff[i] = uint32_t(row[i]) * row_bytes + kc;
      voff[i] = uint32_t(row[i]) * row_bytes + vc;
      koff_r[i] = uint32_t(rr) * row_bytes + kc;
      voff_r[i] = uint32_t(rr) * row_bytes + vc;
    }
    seg = 0;
    m = 0;
  }

  __device__ __forceinline__ void prepare(const AttnParams& p, const int32_t* pages_lds, int s,
                                          int h, int nseg) {
    const int sg = seg < nseg ? seg : 0;
    const int mm = seg < nseg ? m : 0;
    const int code = p.seg[s][sg];
    const int64_t t0 = int64_t(KT) * mm;  // first token of the tile within the chunk
    ragged = mm == p.tps - 1;
    per_lane = false;
    if (code >= 0) {  // live chunk `code` of the tick's q/k/v
      const int64_t e = ((int64_t(code) * p.T + t0) * p.H + h) * D;
      kb = reinterpret_cast<const char*>(p.k + e);
      vb = reinterpret_cast<const char*>(p.v + e);
    } else if constexpr (kFast) {  // history chunk: one page holds the whole tile
      const int c = -code - 1;
      const int pid = ((const_i32p)p.hist_pages)[c * p.ppc + int(t0 / p.P)];
      const int64_t prow = int64_t(pid) * p.P + (t0 % p.P);
      const int64_t e = (prow * p.H + h) * D;
      kb = reinterpret_cast<const char*>(p.k_pool + e);
      vb = reinterpret_cast<const char*>(p.v_pool + e);
    } else {  // history chunk, pages smaller than or not aligned to a tile
      const int c = -code - 1;
      per_lane = true;
      kb = reinterpret_cast<const char*>(p.k_pool + int64_t(h) * D);
      vb = reinterpret_cast<const char*>(p.v_pool + int64_t(h) * D);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int rr = ragged && row[i] >= p.t_last ? p.t_last - 1 : row[i];
        const uint32_t tok = uint32_t(t0) + uint32_t(rr);
        const uint32_t pg = __umulhi(tok, p.p_magic);
        const int32_t pid = pages_lds[c * p.ppc + int(pg)];
        // pool rows fit in 31 bits (checked on the host)
        prow[i] = uint32_t(pid) * uint32_t(p.P) + (tok - pg * uint32_t(p.P));
      }
    }
    if (++m == p.tps) {
      m = 0;
      ++seg;
    }
  }

  __device__ __forceinline__ void emit(int i, const AttnParams& p, uint16_t* kbuf,
                                       uint16_t* vbuf, int wave) const {
    lds_void* kdst = opaque_lds(kbuf + (wave * RW + RPI * i) * D);
    lds_void* vdst = opaque_lds(vbuf + (wave * RW + RPI * i) * D);
    const char* ks;
    const char* vs;
    if (!kFast && per_lane) {
      const uint32_t row_bytes = uint32_t(p.H) * D * 2;
      const uint64_t o = uint64_t(prow[i]) * row_bytes;
      const uint32_t rb = uint32_t(row[i]) * row_bytes;
      ks = kb + o + (koff[i] - rb);
      vs = vb + o + (voff[i] - rb);
    } else {
      ks = kb + (ragged ? koff_r[i] : koff[i]);
      vs = vb + (ragged ? voff_r[i] : voff[i]);
    }
    __builtin_amdgcn_global_load_lds(ks, kdst, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vs, vdst, 16, 0, 0);
  }
};

// End of a tile: this wave's tile loads except the newest N have landed in LDS
// and its LDS reads are done, then all waves meet. (__syncthreads() would also
// wait for the newest loads: its fence drains every outstanding memory op.)
// The asm's memory clobber keeps LDS accesses on their side of the barrier.
template <int N>
__device__ __forceinline__ void tile_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // s_waitcnt: vmcnt(N) (bits 3:0 and 15:14), expcnt(7) (no wait), lgkmcnt(0)
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  asm volatile("s_barrier" ::: "memory");
}

template <int D, bool kFast>
__global__ __attribute__((amdgpu_flat_work_group_size(NTHREADS, NTHREADS),
                          amdgpu_waves_per_eu(2, 2))) void
attn_tick_kernel(const AttnParams p) {
  constexpr int KS = D / 16;  // MFMA k-steps over the head dim
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  using Loader = TileLoader<D, kFast>;
  constexpr int NI = Loader::NI;
  // Three K and three V tile buffers as six distinct LDS objects; the loop is
  // unrolled by three so that every access names its buffer statically. Tile
  // it+2 is loaded while tile it is computed.
  __shared__ __attribute__((aligned(16))) uint16_t k_lds0[KT * D];
  __shared__ __attribute__((aligned(16))) uint16_t k_lds1[KT * D];
  __shared__ __attribute__((aligned(16))) uint16_t k_lds2[KT * D];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds0[KT * D];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds1[KT * D];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds2[KT * D];
  __shared__ int32_t pages_lds[kFast ? 1 : kMaxPageIds];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 31;
  const int g = lane >> 5;

  // ---- work item: heaviest stage first, then head, then query tile --------
  const int b = blockIdx.x;
  int rank, h, qt;
  if (p.use_xcd) {
    const int x = b & (kNumXcd - 1);
    const int k = b / kNumXcd;
    const int gi = k / p.ntq;
    if (gi >= p.xcd_n[x]) return;  // whole block: this XCD's list is shorter
    const int grp = p.xcd_groups[x * p.xcd_stride + gi];
    qt = k - gi * p.ntq;
    rank = grp / p.H;
    h = grp - rank * p.H;
  } else {
    rank = b / p.items_per_stage;
    const int rem = b - rank * p.items_per_stage;
    h = rem / p.ntq;
    qt = rem - h * p.ntq;
  }
  const int s = p.stage_of_rank[rank];
  const int nseg = p.nseg[s];
  const int T = p.T;
  const int ntiles = nseg * p.tps;

  if constexpr (!kFast) {  // page table of the history into LDS
    for (int i = tid; i < p.n_page_ids; i += NTHREADS) pages_lds[i] = p.hist_pages[i];
    __syncthreads();
  }

  const int q0w = qt * QROWS + wave * 32;  // first query row of this wave
  const bool wave_active = q0w < T;
  const int qrow = q0w + r;

  // ---- Q^T operand: lane holds query qrow, head dims 16*ks + 8*g .. +7 -----
  bf16x8 qf[KS];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(p.q + ((int64_t(s) * T + qrow) * p.H + h) * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 u = (qrow < T) ? qp[2 * ks + g] : make_uint4(0u, 0u, 0u, 0u);
      qf[ks] = __builtin_bit_cast(bf16x8, u);
    }
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.f;

  // per-lane LDS read offsets (elements)
  const int krow0 = swap_bits23(r);   // K row feeding MFMA row r of block 0 (+32: block 1)
  const int kx = kswz<D>(krow0);      // same swizzle for row + 32
  const int a16 = lane & 15;          // lane within its 16-lane group (transposed V reads)
  const int vrow = 8 * g + (a16 >> 2);
  const int vx = vswz<D>(vrow);
  const int vcx = 2 * ((lane >> 4) & 1) + ((a16 >> 1) & 1);
  const int vsub = 4 * (a16 & 1);

  Loader ld;
  ld.init(p, wave, lane);
  ld.prepare(p, pages_lds, s, h, nseg);
#pragma unroll
  for (int i = 0; i < NI; ++i) ld.emit(i, p, k_lds0, v_lds0, wave);
  ld.prepare(p, pages_lds, s, h, nseg);
#pragma unroll
  for (int i = 0; i < NI; ++i) ld.emit(i, p, k_lds1, v_lds1, wave);
  ld.prepare(p, pages_lds, s, h, nseg);  // tile 2, issued by the first step
  tile_barrier<2 * NI>();  // tile 0 has landed (tile 1 may still be in flight)

  // keys of the computed tile that are real: 64, the chunk's remainder on a
  // segment's last tile, 0 past the end (the loop runs in groups of three)
  int m_c = 0;
  auto valid_keys = [&](int it) {
    const int v = it >= ntiles ? 0 : (m_c == p.tps - 1 ? p.t_last : KT);
    if (++m_c == p.tps) m_c = 0;
    return v;
  };

  // One tile: compute tile it from (kb, vb); the loads of tile it+2 go to
  // (kn, vn), spread between the S^T MFMAs; tile it+3 is resolved for the next.
  auto step = [&](int it, const uint16_t* kb, const uint16_t* vb, uint16_t* kn, uint16_t* vn) {
    const int valid = valid_keys(it);
    if (!wave_active) {
#pragma unroll
      for (int i = 0; i < NI; ++i) ld.emit(i, p, kn, vn, wave);
      ld.prepare(p, pages_lds, s, h, nseg);
    } else {
      // ---- S^T = K Q^T: two 32-key blocks; K operands two k-steps ahead, one
      // row group of next-tile loads after each k-step (scheduling fences keep
      // the interleave). Each LDS address is one offset added to the buffer:
      // the compiler tags LDS accesses with the buffer they touch only through
      // a short chain of address steps.
      auto kload = [&](int kk, bf16x8* dst) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
          dst[blk] = *reinterpret_cast<const bf16x8*>(
              kb + ((krow0 + 32 * blk) * D + ((2 * kk + g) ^ kx) * 8));
      };
      f32x16 sacc[2] = {f32x16{}, f32x16{}};
      bf16x8 ka[3][2];
      kload(0, ka[0]);
      kload(1, ka[1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
          sacc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk % 3][blk], qf[kk], sacc[blk],
                                                              0, 0, 0);
        if (kk + 2 < KS) kload(kk + 2, ka[(kk + 2) % 3]);
        if (kk < NI) ld.emit(kk, p, kn, vn, wave);
        __builtin_amdgcn_sched_barrier(0);
      }
      ld.prepare(p, pages_lds, s, h, nseg);
      // V^T operand of one 16-key step for all DB blocks: two transposed reads each
      auto vload = [&](int kk, bf16x8* dst) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int e0 = (16 * kk + vrow) * D + ((4 * db + vcx) ^ vx) * 8 + vsub;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(vb + e0));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(vb + (e0 + 4 * D)));
          dst[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      };
      // the first V^T operands load while the softmax runs
      bf16x8 va[2][DB];
      vload(0, va[0]);
      // Register x of block blk holds key 32*blk + 16*(x>>3) + 8*g + (x&7).
      if (valid < KT) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int x = 0; x < 16; ++x) {
            const int key = 32 * blk + 16 * (x >> 3) + 8 * g + (x & 7);
            if (key >= valid) sacc[blk][x] = -INFINITY;
          }
      }
      // ---- online softmax (exp2 domain) ------------------------------------
      float mx = sacc[0][0];
#pragma unroll
      for (int x = 1; x < 16; ++x) mx = fmaxf(mx, sacc[0][x]);
#pragma unroll
      for (int x = 0; x < 16; ++x) mx = fmaxf(mx, sacc[1][x]);
      mx = xlane32_max(mx) * p.c;
      const bool raise = mx > m_run + kLazyTau;
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {
        const float m_new = raise ? mx : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < DB; ++i)
#pragma unroll
          for (int x = 0; x < 16; ++x) oacc[i][x] *= alpha;
      }
      bf16x8 pb[4];
      float lsum = 0.f;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const float e = __builtin_amdgcn_exp2f(fmaf(sacc[blk][x], p.c, -m_run));
          lsum += e;
          pb[2 * blk + (x >> 3)][x & 7] = static_cast<__bf16>(e);
        }
      l_run += lsum;
      // ---- O^T += V^T P^T : four 16-key steps, operands one step ahead ------
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (kk + 1 < 4) vload(kk + 1, va[(kk + 1) & 1]);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kk & 1][db], pb[kk], oacc[db], 0,
                                                             0, 0);
      }
    }

    tile_barrier<2 * NI>();  // tile it+1 has landed; tile it+2 may still be in flight
  };

  // Whole groups of three (a tile past the end is fully masked and adds
  // nothing), so that each step names its buffers statically.
  for (int it = 0; it < ntiles; it += 3) {
    step(it, k_lds0, v_lds0, k_lds2, v_lds2);
    step(it + 1, k_lds1, v_lds1, k_lds0, v_lds0);
    step(it + 2, k_lds2, v_lds2, k_lds1, v_lds1);
  }

  // ---- epilogue: O = O^T / l, bf16 ----------------------------------------
  if (wave_active && qrow < T) {
    const float inv = 1.0f / xlane32_sum(l_run);
    uint16_t* op = p.o + ((int64_t(s) * T + qrow) * p.H + h) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 32 * db + 8 * i + 4 * g;
        bf16x4 v4;
#pragma unroll
        for (int j = 0; j < 4; ++j) v4[j] = static_cast<__bf16>(oacc[db][4 * i + j] * inv);
        *reinterpret_cast<uint2*>(op + d) = __builtin_bit_cast(uint2, v4);
      }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct StagePlan {
  int n_active = 0;
  int order[WF_MAX_STAGES];
  int nseg[WF_MAX_STAGES];
  int8_t seg[WF_MAX_STAGES][WF_MAX_SEGMENTS];
  int64_t keys[WF_MAX_STAGES];
};

// Segments of each active slot's context in the Eq. (5) order.
void plan_stages(const wf_tick_desc& d, StagePlan& pl) {
  std::memset(&pl, 0, sizeof(pl));
  const int S = d.S;
  const uint32_t A = d.active_mask;
  for (int s = 0; s <= S; ++s) {
    if (!((A >> s) & 1u)) continue;
    int n = 0;
    for (int c = d.hist_first[s]; c < d.n_hist; ++c) pl.seg[s][n++] = int8_t(-c - 1);
    if ((A >> S) & 1u) pl.seg[s][n++] = int8_t(S);  // live store (self when s == S)
    for (int j = s; j < S; ++j)
      if ((A >> j) & 1u) pl.seg[s][n++] = int8_t(j);
    pl.nseg[s] = n;
    pl.keys[s] = int64_t(n) * d.T;
    pl.order[pl.n_active++] = s;
  }
  std::stable_sort(pl.order, pl.order + pl.n_active,
                   [&](int a, int b) { return pl.keys[a] > pl.keys[b]; });
}

// XCD-aware work order. The (stage, head) groups, heaviest stage first, are
// dealt to the 8 XCDs by longest-processing-time (each to the least-loaded XCD),
// so every XCD gets about the same number of keys to stream and the query tiles
// of one group run together on one XCD and share its L2. Falls back to the
// plain order when the table does not fit.
void plan_xcd_order(const StagePlan& pl, int H, AttnParams& p, int64_t& blocks) {
  p.use_xcd = 0;
  const int G = pl.n_active * H;
  if (G > kXcdTable) return;
  int16_t lists[kNumXcd][kXcdTable];
  int n[kNumXcd] = {0};
  int64_t load[kNumXcd] = {0};
  for (int rank = 0; rank < pl.n_active; ++rank) {
    const int64_t w = pl.keys[pl.order[rank]];
    for (int h = 0; h < H; ++h) {
      int best = 0;
      for (int x = 1; x < kNumXcd; ++x)
        if (load[x] < load[best]) best = x;
      lists[best][n[best]++] = int16_t(rank * H + h);
      load[best] += w;
    }
  }
  int stride = 0;
  for (int x = 0; x < kNumXcd; ++x) stride = std::max(stride, n[x]);
  if (stride * kNumXcd > kXcdTable) return;
  p.use_xcd = 1;
  p.xcd_stride = stride;
  for (int x = 0; x < kNumXcd; ++x) {
    p.xcd_n[x] = int16_t(n[x]);
    for (int i = 0; i < n[x]; ++i) p.xcd_groups[x * stride + i] = lists[x][i];
  }
  blocks = int64_t(kNumXcd) * stride * p.ntq;
}

// kFast: every tile is one uniform span of a page or live chunk (page size a
// multiple of 64, or no history); otherwise history tiles resolve per lane.
template <int D, bool kFast>
int32_t launch_attn(const AttnParams& p, unsigned blocks, hipStream_t stream) {
  attn_tick_kernel<D, kFast><<<dim3(blocks), NTHREADS, 0, stream>>>(p);
  return WF_OK;
}

int32_t validate_tick(const wf_tick_desc* d) {
  if (!d) return fail(WF_EINVAL, "wf_attn_tick: desc is NULL");
  if (d->S < 0 || d->S > WF_MAX_STAGES - 1)
    return fail(WF_EINVAL, "wf_attn_tick: S = %d outside [0, %d]", d->S, WF_MAX_STAGES - 1);
  const uint32_t all = (2u << d->S) - 1u;
  if (d->active_mask & ~all)
    return fail(WF_EINVAL, "wf_attn_tick: active_mask 0x%x has bits above S = %d",
                d->active_mask, d->S);
  if (d->T < 0 || d->H <= 0)
    return fail(WF_EINVAL, "wf_attn_tick: bad sizes T = %d H = %d", d->T, d->H);
  if (d->D != 64 && d->D != 128)
    return fail(WF_EUNSUPPORTED, "wf_attn_tick: head dim D = %d (supported: 64, 128)", d->D);
  if (!(d->scale > 0.f) || !std::isfinite(d->scale))
    return fail(WF_EINVAL, "wf_attn_tick: scale must be positive and finite");
  if (d->n_hist < 0) return fail(WF_EINVAL, "wf_attn_tick: n_hist = %d", d->n_hist);
  if (d->n_hist + d->S + 1 > WF_MAX_SEGMENTS)
    return fail(WF_EUNSUPPORTED, "wf_attn_tick: n_hist + S + 1 = %d exceeds %d",
                d->n_hist + d->S + 1, WF_MAX_SEGMENTS);
  for (int s = 0; s <= d->S; ++s)
    if (d->hist_first[s] < 0 || d->hist_first[s] > d->n_hist)
      return fail(WF_EINVAL, "wf_attn_tick: hist_first[%d] = %d outside [0, %d]", s,
                  d->hist_first[s], d->n_hist);
  if (d->T == 0 || d->active_mask == 0) return WF_OK;
  if (!d->q || !d->k || !d->v || !d->o)
    return fail(WF_EINVAL, "wf_attn_tick: q, k, v and o must be non-NULL");
  if (!aligned16(d->q) || !aligned16(d->k) || !aligned16(d->v) || !aligned16(d->o))
    return fail(WF_EINVAL, "wf_attn_tick: q, k, v and o must be 16-byte aligned");
  if (int64_t(d->T) > (int64_t(1) << 24))
    return fail(WF_EUNSUPPORTED, "wf_attn_tick: T = %d too large", d->T);
  if (d->n_hist > 0) {
    if (!d->k_pool || !d->v_pool || !d->hist_pages)
      return fail(WF_EINVAL, "wf_attn_tick: n_hist > 0 needs k_pool, v_pool and hist_pages");
    if (!aligned16(d->k_pool) || !aligned16(d->v_pool))
      return fail(WF_EINVAL, "wf_attn_tick: pools must be 16-byte aligned");
    if (d->P <= 0 || d->P % 16 != 0)
      return fail(WF_EINVAL, "wf_attn_tick: page size P = %d must be a positive multiple of 16",
                  d->P);
    if (d->num_pages <= 0) return fail(WF_EINVAL, "wf_attn_tick: num_pages = %d", d->num_pages);
    const int64_t ppc = (int64_t(d->T) + d->P - 1) / d->P;
    if (int64_t(d->n_hist) * ppc > d->num_pages)
      return fail(WF_EINVAL, "wf_attn_tick: n_hist * ceil(T/P) = %lld exceeds num_pages = %d",
                  static_cast<long long>(int64_t(d->n_hist) * ppc), d->num_pages);
    if (int64_t(d->T) * d->P >= (int64_t(1) << 32))
      return fail(WF_EUNSUPPORTED, "wf_attn_tick: T * P too large");
    if (int64_t(d->num_pages) * d->P >= (int64_t(1) << 31))
      return fail(WF_EUNSUPPORTED, "wf_attn_tick: num_pages * P = %lld pool rows exceed 2^31",
                  static_cast<long long>(int64_t(d->num_pages) * d->P));
  }
  return WF_OK;
}

}  // namespace
}  // namespace wf

extern "C" wf_status wf_tick_useful_flops(const wf_tick_desc* desc, double* out) {
  using namespace wf;
  try {
    if (!out) return fail(WF_EINVAL, "wf_tick_useful_flops: out is NULL");
    int32_t st = validate_tick(desc);
    if (st != WF_OK) return st;
    StagePlan pl;
    plan_stages(*desc, pl);
    double pairs = 0;
    for (int i = 0; i < pl.n_active; ++i) pairs += double(desc->T) * double(pl.keys[pl.order[i]]);
    *out = 4.0 * desc->D * desc->H * pairs;
    return WF_OK;
  } catch (...) {
    return fail(WF_EINVAL, "wf_tick_useful_flops: internal error");
  }
}

extern "C" wf_status wf_attn_tick(const wf_tick_desc* desc, hipStream_t stream) {
  using namespace wf;
  try {
    int32_t st = validate_tick(desc);
    if (st != WF_OK) return st;
    const wf_tick_desc& d = *desc;
    if (d.T == 0 || d.active_mask == 0) return WF_OK;
    StagePlan pl;
    plan_stages(d, pl);
    const int32_t ppc = d.n_hist > 0 ? int32_t((int64_t(d.T) + d.P - 1) / d.P) : 0;
    if (d.n_hist > 0 && check_pages_enabled()) {
      st = check_device_pages(d.hist_pages, int64_t(d.n_hist) * ppc, d.num_pages, stream,
                              "wf_attn_tick");
      if (st != WF_OK) return st;
    }
    AttnParams p;
    std::memset(&p, 0, sizeof(p));
    p.q = static_cast<const uint16_t*>(d.q);
    p.k = static_cast<const uint16_t*>(d.k);
    p.v = static_cast<const uint16_t*>(d.v);
    p.o = static_cast<uint16_t*>(d.o);
    p.k_pool = static_cast<const uint16_t*>(d.k_pool);
    p.v_pool = static_cast<const uint16_t*>(d.v_pool);
    p.hist_pages = d.hist_pages;
    p.T = d.T;
    p.H = d.H;
    p.P = d.n_hist > 0 ? d.P : 16;
    p.ppc = ppc;
    p.tps = (d.T + KT - 1) / KT;
    p.t_last = d.T - KT * (p.tps - 1);
    p.p_magic = uint32_t((uint64_t(1) << 32) / uint64_t(p.P) + 1);
    p.c = float(double(d.scale) * 1.4426950408889634);
    p.ntq = (d.T + QROWS - 1) / QROWS;
    p.items_per_stage = d.H * p.ntq;
    p.n_page_ids = d.n_hist * ppc;
    for (int i = 0; i < pl.n_active; ++i) p.stage_of_rank[i] = pl.order[i];
    for (int s = 0; s <= d.S; ++s) {
      p.nseg[s] = pl.nseg[s];
      for (int i = 0; i < pl.nseg[s]; ++i) p.seg[s][i] = pl.seg[s][i];
    }
    int64_t blocks = int64_t(pl.n_active) * p.items_per_stage;
    plan_xcd_order(pl, d.H, p, blocks);
    if (blocks > 0x7fffffff) return fail(WF_EUNSUPPORTED, "wf_attn_tick: grid too large");
    const bool fast = d.n_hist == 0 || d.P % KT == 0;
    if (!fast && p.n_page_ids > kMaxPageIds)  // the per-lane path keeps the table in LDS
      return fail(WF_EUNSUPPORTED, "wf_attn_tick: page table of %d ids exceeds %d (page sizes "
                  "that are a multiple of 64 have no such limit)", p.n_page_ids, kMaxPageIds);
    if (d.D == 128)
      st = fast ? launch_attn<128, true>(p, unsigned(blocks), stream)
                : launch_attn<128, false>(p, unsigned(blocks), stream);
    else
      st = fast ? launch_attn<64, true>(p, unsigned(blocks), stream)
                : launch_attn<64, false>(p, unsigned(blocks), stream);
    if (st != WF_OK) return st;
    return check_launch("wf_attn_tick");
  } catch (...) {
    return fail(WF_EINVAL, "wf_attn_tick: internal error");
  }
}
