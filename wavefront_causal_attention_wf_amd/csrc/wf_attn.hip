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
//  * Ping-pong: the waves of a SIMD run the same sequence one barrier slot
//    apart, one in its MFMA slot (P.V of tile j interleaved with Q.K^T of tile
//    j+1) while the other runs its softmax, so MFMA and VALU work overlap.
//  * K and V tiles [64 keys][D] stream from global memory straight into LDS
//    (16-byte buffer loads into LDS, no register staging) through four
//    buffers; each wave issues its share of a tile two slots before the tile is
//    needed, at the start of its softmax slot, and every slot ends with a
//    barrier that waits only for the loads it must. A tile is one contiguous
//    span of a page or a live chunk (pages of a multiple of 64 tokens): its
//    source is a table entry in LDS plus a fixed per-lane offset. Rows are
//    XOR-swizzled so that the MFMA operand reads are free of LDS bank
//    conflicts; V^T operands are fetched with the gfx950 transposing LDS read
//    (ds_read_b64_tr_b16), so V needs no transpose on its way in.
//  * Online softmax in the exp2 domain (log2 e folded into the scale), fp32
//    state; the running max is only raised when a tile exceeds it by more than
//    8 (in log2 units), so the O rescale is rare (exact: numerator and
//    denominator share the same reference), and the tile's max is only
//    computed when the sum of its exponentials says it might.
//  * Work order: (stage, head) groups, heaviest stage first, dealt to the 8
//    XCDs so that each XCD streams about the same number of keys and the query
//    tiles of a group share that XCD's L2. Optionally the launch also writes
//    the store chunk's pages (leading blocks).
//  * 8-bit tier (full text §4.3: K/V quantisation, an 8-bit attention
//    backend): keys come from e4m3 pages with one fp32 scale per (64-key tile,
//    head), each query row is quantised to e4m3 in the kernel with its own
//    scale, and Q.K^T runs on v_mfma_f32_32x32x64_f8f6f4 (half the MFMA time and
//    half the K bytes in LDS of the bf16 product); the two scales fold into the
//    softmax's per-tile multiplier, and P.V stays bf16.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <vector>

#include "wf_internal.h"

// Workspace of wf_attn_tick_noalloc: one array per GPU in the code object,
// held until the process ends. Host code takes its device address from
// hipGetSymbolAddress (once per device), never from the name.
static __device__ __attribute__((aligned(256))) uint8_t scratch[WF_NOALLOC_SCRATCH_BYTES];

namespace wf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int KT = 64;              // keys per tile
#ifndef WF_NWAVES
#define WF_NWAVES 8
#endif
constexpr int NWAVES = WF_NWAVES;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int QROWS = 32 * NWAVES;  // query rows per workgroup
constexpr float kLazyTau = 8.0f;    // raise the running max only beyond this (log2 units)
constexpr float kLazyBound = 256.0f;  // 2^kLazyTau
constexpr int kNumXcd = 8;          // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kXcdTable = 256;      // max (stage, head) groups in the XCD group table
// Packed work order (below): per XCD at most kPackSegs runs of query tiles and
// kPackItems workgroups, each named by a 4-bit run index.
constexpr int kPackSegs = 16;
constexpr int kPackItems = 192;
constexpr int kPackBins = 40;  // CUs per XCD the packed order can fill
// Run-time pool (see AttnParams): at most kMaxPool items; the workspace holds
// kWsHeader bytes of counters, then one partial softmax state per piece.
constexpr int kMaxPool = 128;
constexpr int kWsHeader = 1024;
static_assert((1 + kMaxPool) * 4 <= kWsHeader, "pool counters exceed the workspace header");
constexpr double kPoolShare = 0.08;  // share of a tick's work the pool takes
constexpr int kMaxHeadParts = 8;     // launches a tick's heads may be split into
constexpr int kMinSplitItems = 4;    // items per CU below which a tick is not split
// A piece's partial state: [QROWS][D] unnormalised output, then the QROWS row
// maxima and the QROWS row sums (fp32).
constexpr int64_t state_bytes(int D) { return int64_t(QROWS) * (D + 2) * 4; }
// History page table held in LDS (ids of all history pages of one tick) when
// pages are not a multiple of 64 tokens; otherwise a table of tile sources.
constexpr int kMaxPageIds = 4096;
constexpr int kMaxTiles = 1536;  // 64-key tiles per (stage, head): 24 KB of sources
// Word 3 of a raw buffer resource on gfx9-family parts (32-bit data format, no
// swizzle, stride 0): plain byte-addressed loads.
constexpr int kBufferFlags = 0x00020000;
// Cache-policy operand of a buffer access with device scope (the SC1 bit): the
// access is coherent across the XCDs' separate L2 caches without writing back
// or invalidating them, as the device-scope atomic loads and stores are.
constexpr int kDeviceScope = 16;

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* hist_pages;
  const int32_t* live_pages;  // NULL: live K/V from k and v
  const int32_t* store_pages; // non-NULL: the launch also writes the store chunk's pages
  int32_t n_store_blocks;     // leading blocks that do that copy (a multiple of 8)
  int32_t store_row16;        // 16-byte units per token row (H * D * 2 / 16)
  int32_t store_slot;         // S
  int32_t n_hist;
  const float* k_scale;   // 8-bit tier: [num_pages][P / 64][H] key tile scales
  const uint8_t* v_exp;   // 8-bit values: [num_pages][P / 64][H] tile exponents + 127
  int32_t spp;            // 64-token scale tiles per page (P / 64)
  int32_t T, H, P, ppc;
  int32_t tps;            // tiles per chunk, ceil(T / 64)
  int32_t t_last;         // keys in a chunk's last tile, T - 64 * (tps - 1)
  uint32_t p_magic;       // floor(2^32 / P) + 1: t / P == umulhi(t, p_magic) for t*P < 2^32
  float c;                // scale * log2(e)
  int32_t ntq;            // query tiles per chunk
  // A tick with too many heads for one packed plan runs as several launches,
  // each over heads [h0, h0 + hp); the plan counts heads of its launch.
  int32_t hp, h0;
  int32_t items_per_stage;  // hp * ntq
  int32_t n_page_ids;     // page ids staged in LDS (non-fast path): history, then live
  // Work order; block b runs on XCD x = b % 8 (round-robin dispatch).
  // use_xcd = 1: block b is that XCD's item k = b / 8, query tile k % ntq of
  // group xcd_groups[x][k / ntq] (group = rank * H + head); blocks past an
  // XCD's list exit at once. use_xcd = 2 (packed, one block per CU): block b
  // runs items pack_bin[x][c] .. pack_bin[x][c + 1] - 1 of XCD x's list, c =
  // b / 8; item i belongs to run r = the 4-bit code i of pack_code[x] and is
  // the run's query tile pack_qt0[x][r] + (number of earlier items of run r in
  // the list); its group is pack_grp[x][r].
  int32_t use_xcd;
  int32_t xcd_stride;
  // Tail items (packed order only). The last query tile of every active slot
  // (rows tail_row0 .. T-1, tail_spr 32-row slices) is not an item of its own:
  // the slices of all slots of a head, laid out slot by slot in rank order, are
  // cut into tail_per_head items of NWAVES slices, one slice per wave. An item
  // walks the context of its first slice's slot with the live chunks in
  // descending order (history, live store, S-1, S-2, ...), so each other
  // slice's slot sees the first nseg[s] chunks of that walk, and its wave stops
  // there. Item k of a packed list names one with group n_active * H + h *
  // tail_per_head + m.
  int32_t tail;           // 0: every query tile is an item of its own
  int32_t tail_row0;
  int32_t tail_spr;
  int32_t tail_per_head;
  int32_t tail_npre;      // leading chunks of every slot's walk: history + live store
  int32_t n_active;       // active slots
  // Run-time pool (packed order with a workspace). pool_items query tiles of
  // the heaviest slot (rank 0), item i being tile pool_qt0 - i / H of head
  // i % H (the last full tiles of each head in turn), are not on any list:
  // each is cut into its pool_nseg chunks of keys, piece k being chunk k %
  // pool_nseg of item k / pool_nseg. A block that has run its
  // list takes pieces from a counter in the workspace until none are left, so
  // CUs that run faster (whole XCDs differ by several per cent) take more. A
  // piece leaves its partial softmax state — the unnormalised O, the running
  // reference m and the row sum l of every row — in the workspace, and the
  // block that completes an item's last piece merges the item's states.
  uint32_t* ws;           // [0]: next piece, [1 + i]: pieces done of item i
  int32_t pool_pieces;
  int32_t pool_nseg;
  int32_t pool_items;
  int32_t pool_qt0;
  int16_t xcd_n[kNumXcd];
  int16_t xcd_groups[kXcdTable];
  int16_t pack_grp[kNumXcd][kPackSegs];
  int16_t pack_qt0[kNumXcd][kPackSegs];
  int16_t pack_bin[kNumXcd][kPackBins + 1];
  uint32_t pack_code[kNumXcd][kPackItems / 8];  // eight 4-bit run indices per word
  // (32-bit entries: the kernel reads them with scalar loads, which are
  // dword-granular; a narrower type would turn them into vector loads)
  int32_t stage_of_rank[WF_MAX_STAGES];  // work order, heaviest stage first
  int32_t nseg[WF_MAX_STAGES];
  // per stage: segment code >= 0 is live slot j, < 0 is history chunk (-code - 1)
  int32_t seg[WF_MAX_STAGES][WF_MAX_SEGMENTS];
};

// passed by value as the kernel argument: keep it within 4 KB
static_assert(sizeof(AttnParams) <= 4096, "kernel argument too large");

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
// 8-bit keys (D = 128: rows of 128 bytes, 8 chunks; two rows per 256 bytes):
// a read touches rows {0..3, 8..11} (+4, ...) at one logical chunk; bits 0, 1
// and 3 of the row (bit 0 mixed with bit 2) pick the chunk, so any such 8 rows
// land in distinct chunks, and rows 0..15 of one parity too.
__device__ __forceinline__ int kswz8(int row) {
  return ((row ^ (row >> 2)) & 1) | (row & 2) | ((row >> 1) & 4);
}
// 8-bit values (transposed tile, rows of 64 bytes = four 16-byte chunks): a
// read touches one chunk of 16 consecutive rows; rows r and r + 4k land in
// distinct chunks when the chunk is XORed with bits 2-3 of the row.
__device__ __forceinline__ int v8swz(int drow) { return (drow >> 2) & 3; }
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

// Loop-invariant scalars of a launch, read from the kernel arguments once and
// kept in scalar registers (readfirstlane makes them values the compiler will
// not re-load from the argument buffer inside the loop: scalar-memory loads
// there would force waits that drain every LDS read in flight).
struct Uniforms {
  const char* k;
  const char* v;
  const char* k_pool;
  const char* v_pool;
  int32_t T, H, P, ppc, tps, t_last;
  uint32_t p_magic, row_bytes, krow_bytes;  // token row bytes of V (and bf16 K), of K
  float c;  // softmax scale * log2(e)
};

__device__ __forceinline__ int32_t uniform_i32(int32_t x) {
  return __builtin_amdgcn_readfirstlane(x);
}
__device__ __forceinline__ const char* uniform_ptr(const void* ptr) {
  const uint64_t x = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(x));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(x >> 32));
  return reinterpret_cast<const char*>((uint64_t(hi) << 32) | lo);
}

template <int D, int KB>
__device__ __forceinline__ Uniforms load_uniforms(const AttnParams& p, int h) {
  Uniforms u;
  u.T = uniform_i32(p.T);
  u.H = uniform_i32(p.H);
  u.P = uniform_i32(p.P);
  u.ppc = uniform_i32(p.ppc);
  u.tps = uniform_i32(p.tps);
  u.t_last = uniform_i32(p.t_last);
  u.p_magic = uint32_t(uniform_i32(int32_t(p.p_magic)));
  u.row_bytes = uint32_t(u.H) * D * 2;
  u.krow_bytes = uint32_t(u.H) * D * KB;
  u.c = __builtin_bit_cast(float, uniform_i32(__builtin_bit_cast(int32_t, p.c)));
  // head h's column block of every tensor
  u.k = uniform_ptr(p.k + int64_t(h) * D);
  u.v = uniform_ptr(p.v + int64_t(h) * D);
  u.k_pool = uniform_ptr(reinterpret_cast<const char*>(p.k_pool) + int64_t(h) * D * KB);
  u.v_pool = uniform_ptr(p.v_pool + int64_t(h) * D);
  return u;
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

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
// (from a table of tile sources built in LDS per workgroup) plus a fixed
// per-lane offset, and a tile costs no vector address math. Otherwise history
// tiles resolve each lane's page through the page table in LDS, and the
// segment's code is read (a scalar load) only when the cursor enters a new
// segment. prepare*() resolves the next tile and advances the cursor; emit(i)
// issues the loads of row group i. Past the last tile the cursor reads tile 0
// again (finite, masked). KB = bytes per key element: 2 (bf16), or 1 (e4m3
// keys of the 8-bit tier, whose rows are half as long, so a wave needs half
// as many K instructions per tile; kFast only). VB = bytes per value
// element: 2, or 1 (8-bit values: a V tile is D rows of 64 token bytes, one
// contiguous 64*D-byte block of its page, which each wave loads 16 rows of
// with one instruction).
template <int D, bool kFast, int KB, int VB = 2>
struct TileLoader {
  static_assert(KB == 2 || kFast, "8-bit keys need whole-tile sources");
  static_assert(VB == 2 || (KB == 1 && D == 128 && NWAVES == 8), "8-bit values: D = 128");
  static constexpr int DC = D / 8;        // 16-byte chunks per V row
  static constexpr int RPI = 64 / DC;     // V rows per wave instruction
  static constexpr int RW = KT / NWAVES;  // tile rows loaded by each wave
  static constexpr int NI = VB == 2 ? RW / RPI : 1;  // V instructions per wave per tile
  static constexpr int DCK = D * KB / 16; // 16-byte chunks per K row
  static constexpr int RPIK = 64 / DCK;   // K rows per wave instruction
  static constexpr int NIK = RW / RPIK;   // K instructions per wave per tile (<= NI)
  static constexpr int LPT = NI + NIK;    // loads per wave per tile

  // per lane (bytes): row offset + swizzled column, full and last-tile rows
  uint32_t koff[NIK], voff[NI], koff_r[NIK], voff_r[NI];
  int32_t row[NI];
  // cursor: next tile to resolve
  int seg, m;
  // the cursor's segment: index, history chunk (-1: live), chunk bases
  int cur_seg;
  int hist_c;
  const char* seg_k;
  const char* seg_v;
  // resolved tile: uniform bases (+ the per-lane offsets), or for per-lane
  // history tiles the pool bases of head h and each lane's pool row
  const char* kb;
  const char* vb;
  bool ragged;
  bool per_lane;
  uint32_t prow[NI];

  __device__ __forceinline__ void init(const Uniforms& u, int wave, int lane) {
    const int pc = lane % DC;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      row[i] = wave * RW + RPI * i + lane / DC;
      const int rr = row[i] < u.t_last ? row[i] : u.t_last - 1;
      const uint32_t vc = uint32_t(pc ^ vswz<D>(row[i])) * 16;
      voff[i] = uint32_t(row[i]) * u.row_bytes + vc;
      voff_r[i] = uint32_t(rr) * u.row_bytes + vc;
      if constexpr (VB == 1) {  // channel row of the transposed tile, its 16-byte chunk
        const int drow = wave * (D / NWAVES) + lane / 4;
        voff[i] = uint32_t(drow * 64 + (((lane & 3) ^ v8swz(drow)) << 4));
        voff_r[i] = voff[i];  // tokens past the chunk are zero codes
      }
    }
    const int pck = lane % DCK;
#pragma unroll
    for (int i = 0; i < NIK; ++i) {
      const int kr = wave * RW + RPIK * i + lane / DCK;
      const int rr = kr < u.t_last ? kr : u.t_last - 1;
      const uint32_t kc = uint32_t(pck ^ (KB == 2 ? kswz<D>(kr) : kswz8(kr))) * 16;
      koff[i] = uint32_t(kr) * u.krow_bytes + kc;
      koff_r[i] = uint32_t(rr) * u.krow_bytes + kc;
    }
    seg = 0;
    m = 0;
    cur_seg = -1;
  }

  // kFast: the sources of tile t are entry t of a table built once per
  // workgroup in LDS: K base (bit 0 = last, partial tile of its chunk) and V
  // base. The entry of the next tile is read one tile ahead, so resolving a
  // tile waits for nothing.
  int next_t;
  uint4 pre;

  __device__ __forceinline__ void start_table(const uint4* tab) {
    next_t = 0;
    pre = tab[0];
  }

  __device__ __forceinline__ void prepare_table(const uint4* tab, int ntiles) {
    const uint64_t kr = (uint64_t(uint32_t(uniform_i32(int32_t(pre.y)))) << 32) |
                        uint32_t(uniform_i32(int32_t(pre.x)));
    const uint64_t vr = (uint64_t(uint32_t(uniform_i32(int32_t(pre.w)))) << 32) |
                        uint32_t(uniform_i32(int32_t(pre.z)));
    ragged = kr & 1;
    kb = reinterpret_cast<const char*>(kr & ~uint64_t(1));
    vb = reinterpret_cast<const char*>(vr);
    per_lane = false;
    ++next_t;
    pre = tab[next_t < ntiles ? next_t : 0];
  }

  __device__ __forceinline__ void prepare(const AttnParams& p, const Uniforms& u,
                                          const int32_t* pages_lds, int s, int nseg) {
    const int sg = seg < nseg ? seg : 0;
    const int mm = seg < nseg ? m : 0;
    if (sg != cur_seg) {  // entering a segment: its code, once
      cur_seg = sg;
      const int code = uniform_i32(p.seg[s][sg]);
      if (code >= 0 && p.live_pages) {  // live chunk `code` through its pages
        hist_c = uniform_i32(p.n_hist) + code;
      } else if (code >= 0) {  // live chunk `code` of the tick's q/k/v
        hist_c = -1;
        const uint64_t e = uint64_t(code) * uint64_t(u.T) * u.row_bytes;
        seg_k = u.k + e;
        seg_v = u.v + e;
      } else {
        hist_c = -code - 1;
      }
    }
    const uint32_t t0 = uint32_t(KT) * uint32_t(mm);  // first token of the tile in the chunk
    ragged = mm == u.tps - 1;
    per_lane = false;
    if (hist_c < 0) {
      kb = seg_k + uint64_t(t0) * u.row_bytes;
      vb = seg_v + uint64_t(t0) * u.row_bytes;
    } else if constexpr (kFast) {  // history chunk: one page holds the whole tile
      const uint32_t pg = t0 / uint32_t(u.P);
      const int pid = uniform_i32(pages_lds[hist_c * u.ppc + int(pg)]);
      const uint64_t prow = uint64_t(uint32_t(pid)) * uint32_t(u.P) + (t0 - pg * uint32_t(u.P));
      kb = u.k_pool + prow * u.row_bytes;
      vb = u.v_pool + prow * u.row_bytes;
    } else {  // history chunk, pages smaller than or not aligned to a tile
      per_lane = true;
      kb = u.k_pool;
      vb = u.v_pool;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int rr = ragged && row[i] >= u.t_last ? u.t_last - 1 : row[i];
        const uint32_t tok = t0 + uint32_t(rr);
        const uint32_t pg = __umulhi(tok, u.p_magic);
        const int32_t pid = pages_lds[hist_c * u.ppc + int(pg)];
        // pool rows fit in 31 bits (checked on the host)
        prow[i] = uint32_t(pid) * uint32_t(u.P) + (tok - pg * uint32_t(u.P));
      }
    }
    if (++m == u.tps) {
      m = 0;
      ++seg;
    }
  }

  __device__ __forceinline__ void emit(int i, const Uniforms& u, uint16_t* kbuf, uint16_t* vbuf,
                                       int wave) const {
    // (K buffer offset in 16-bit elements: rows of D * KB bytes)
    lds_void* kdst = opaque_lds(kbuf + (wave * RW + RPIK * (i < NIK ? i : 0)) * D * KB / 2);
    lds_void* vdst = opaque_lds(vbuf + (VB == 2 ? (wave * RW + RPI * i) * D : wave * (D / NWAVES) * 32));
    if (!kFast && per_lane) {
      const uint64_t o = uint64_t(prow[i]) * u.row_bytes;
      const uint32_t rb = uint32_t(row[i]) * u.row_bytes;
      __builtin_amdgcn_global_load_lds(kb + o + (koff[i] - rb), kdst, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vb + o + (voff[i] - rb), vdst, 16, 0, 0);
    } else {
      // Uniform tile base as a buffer resource, per-lane byte offset: a buffer
      // load into LDS counts only on vmcnt, whereas the compiler treats a
      // global load into LDS as possibly also pending on lgkmcnt, which turns
      // every LDS operand wait while tile loads are in flight into a wait for
      // all of them. (Offsets stay below 64 rows, far inside the record range.)
      const __amdgpu_buffer_rsrc_t kr =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kb), 0, 0x7fffffff, kBufferFlags);
      const __amdgpu_buffer_rsrc_t vr =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vb), 0, 0x7fffffff, kBufferFlags);
      // last tile of a chunk: rows past its end re-read its last row (a mask
      // blend rather than a select, which the compiler would turn into an
      // indexed load of the offset arrays from scratch)
      const uint32_t rmask = 0u - uint32_t(ragged);
      if (i < NIK) {
        const uint32_t ko = koff[i] + ((koff_r[i] - koff[i]) & rmask);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, kdst, 16, int(ko), 0, 0, 0);
      }
      const uint32_t vo = voff[i] + ((voff_r[i] - voff[i]) & rmask);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, vdst, 16, int(vo), 0, 0, 0);
    }
  }
};

// End of a slot: this wave's tile loads except the newest N have landed in
// LDS, then all waves meet. (__syncthreads() would also wait for the newest
// loads: its fence drains every outstanding memory op.) LDS reads are not
// waited for: every operand read of a tile buffer has been consumed by an MFMA
// before the slot ends, and the only other LDS read that may still be in flight
// is of the tile-source table, which is never written after the start. The
// asm's memory clobber keeps LDS accesses on their side of the barrier.
template <int N>
__device__ __forceinline__ void tile_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // s_waitcnt: vmcnt(N) (bits 3:0 and 15:14), expcnt(7) and lgkmcnt(15): no wait
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("s_barrier" ::: "memory");
}

// The store chunk's pages written by the attention launch itself: block i of
// the leading n_store_blocks copies page i (K and V) of live slot S exactly as
// wf_store_paged does (bit copy, zeros past the chunk's last token). Its K/V
// are read by attention from the live buffers, not from these pages, so the
// copy and the attention blocks do not depend on each other.
__device__ __forceinline__ void store_page_block(const AttnParams& p, int S) {
  const int i = blockIdx.x;
  if (i >= p.ppc) return;
  const int64_t row16 = p.store_row16;
  const int64_t page16 = int64_t(p.P) * row16;
  const int64_t tok0 = int64_t(i) * p.P;
  const int64_t valid16 = (p.T - tok0 < p.P ? p.T - tok0 : p.P) * row16;
  const int64_t pid = p.store_pages[i];
  const int64_t src0 = (int64_t(S) * p.T + tok0) * row16;
#pragma unroll
  for (int tensor = 0; tensor < 2; ++tensor) {
    const uint4* src = reinterpret_cast<const uint4*>(tensor ? p.v : p.k) + src0;
    uint4* dst = reinterpret_cast<uint4*>(const_cast<uint16_t*>(tensor ? p.v_pool : p.k_pool)) +
                 pid * page16;
    for (int64_t base = threadIdx.x; base < page16; base += 4 * NTHREADS) {
      uint4 x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t e = base + u * NTHREADS;
        x[u] = e < valid16 ? src[e] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t e = base + u * NTHREADS;
        if (e < page16) store_stream16(dst + e, x[u]);
      }
    }
  }
}

template <int D, bool kFast, bool kF8, bool kV8 = false>
__global__ __attribute__((amdgpu_flat_work_group_size(NTHREADS, NTHREADS),
                          amdgpu_waves_per_eu(2, 2))) void
attn_tick_kernel(const AttnParams p) {
  static_assert(!kF8 || (D == 128 && kFast), "8-bit keys: D = 128, whole-tile sources");
  static_assert(!kV8 || kF8, "8-bit values come with 8-bit keys");
  constexpr int KS = D / 16;  // MFMA k-steps over the head dim
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  constexpr int KB = kF8 ? 1 : 2;  // bytes per key element
  constexpr int VB = kV8 ? 1 : 2;  // bytes per value element
  using Loader = TileLoader<D, kFast, KB, VB>;
  constexpr int NI = Loader::NI;
  constexpr int LPT = Loader::LPT;
  constexpr int KTILE = KT * D * KB / 2;  // one K tile in 16-bit elements
  constexpr int VTILE = KT * D * VB / 2;  // one V tile in 16-bit elements
  // Four K and four V tile buffers (one array each, 256-byte aligned); the loop
  // is unrolled by four so that every access names its buffer statically.
  __shared__ __attribute__((aligned(256))) uint16_t k_tiles[4 * KTILE];
  __shared__ __attribute__((aligned(256))) uint16_t v_tiles[4 * VTILE];
  uint16_t* const k_lds0 = k_tiles;
  uint16_t* const k_lds1 = k_tiles + KTILE;
  uint16_t* const k_lds2 = k_tiles + 2 * KTILE;
  uint16_t* const k_lds3 = k_tiles + 3 * KTILE;
  uint16_t* const v_lds0 = v_tiles;
  uint16_t* const v_lds1 = v_tiles + VTILE;
  uint16_t* const v_lds2 = v_tiles + 2 * VTILE;
  uint16_t* const v_lds3 = v_tiles + 3 * VTILE;
  __shared__ int32_t pages_lds[kFast ? 1 : kMaxPageIds];
  __shared__ uint4 tile_tab[kFast ? kMaxTiles : 1];
  // 8-bit tier: each tile's key scale for this head (0 replaced by 1: an
  // all-zero tile has zero codes, so any finite multiplier gives its scores)
  __shared__ float tile_scale[kF8 ? kMaxTiles : 1];
  // 8-bit values: each tile's value exponent for this head (E8M0: e + 127)
  __shared__ int32_t tile_vexp[kV8 ? kMaxTiles : 1];

  // ---- the store chunk's page copy (leading blocks, optional) --------------
  if (int(blockIdx.x) < p.n_store_blocks) {
    store_page_block(p, p.store_slot);
    return;
  }
  // ---- work items: one per block, or (packed order) a CU's list -----------
  const int b = blockIdx.x - p.n_store_blocks;
  int item = 0, item_end = 1;
  if (p.use_xcd == 2) {
    const int c = b / kNumXcd;
    item = p.pack_bin[b & (kNumXcd - 1)][c];
    item_end = p.pack_bin[b & (kNumXcd - 1)][c + 1];
  }
  // pieces of the run-time pool follow the list (an empty list goes straight to them)
  __shared__ int32_t pool_slot[2];  // [0]: the piece taken; [1]: 1 = this block merges its item
  bool in_pool = item >= item_end;
  if (in_pool && p.pool_pieces == 0) return;
  for (;;) {
    int piece = 0;
    if (in_pool) {
      if (threadIdx.x == 0) pool_slot[0] = int(atomicAdd(p.ws, 1u));
      __syncthreads();
      piece = pool_slot[0];
      if (piece >= p.pool_pieces) break;  // (uniform: every thread read the same value)
    }
    // Thread coordinates, opaque per item so that nothing derived from them
    // (per-lane offsets and bases, a few dozen registers) is hoisted out of
    // the item loop and kept live, or spilled, across it.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 31;
    const int g = lane >> 5;
    int rank = 0, h, qt;
    int tail_m = -1;  // tail item index within its head, or -1
    int seg0 = 0;     // pieces: the chunk of the walk this piece covers
    if (in_pool) {
      const int pi = piece / p.pool_nseg;
      h = pi % p.hp;
      qt = p.pool_qt0 - pi / p.hp;
      seg0 = piece - pi * p.pool_nseg;
    } else if (p.use_xcd == 2) {
      const int x = b & (kNumXcd - 1);
      const int k = item;
      const int run = (p.pack_code[x][k >> 3] >> (4 * (k & 7))) & 15;
      // earlier items of the same run: zero nibbles of (codes XOR run * 0x11111111)
      int before = 0;
      const uint32_t rep8 = uint32_t(run) * 0x11111111u;
      for (int w = 0; w <= (k >> 3); ++w) {
        uint32_t y = p.pack_code[x][w] ^ rep8;
        if (w == (k >> 3)) y |= ~((1u << (4 * (k & 7))) - 1u);  // only items before k
        const uint32_t z = ~(((y & 0x77777777u) + 0x77777777u) | y | 0x77777777u);
        before += __builtin_popcount(z);
      }
      const int grp = p.pack_grp[x][run];
      qt = p.pack_qt0[x][run] + before;
      const int n_groups = p.n_active * p.hp;
      if (grp >= n_groups) {  // a tail item
        h = (grp - n_groups) / p.tail_per_head;
        tail_m = grp - n_groups - h * p.tail_per_head;
      } else {
        rank = grp / p.hp;
        h = grp - rank * p.hp;
      }
    } else if (p.use_xcd) {
      const int x = b & (kNumXcd - 1);
      const int k = b / kNumXcd;
      const int gi = k / p.ntq;
      if (gi >= p.xcd_n[x]) return;  // whole block: this XCD's list is shorter
      const int grp = p.xcd_groups[x * p.xcd_stride + gi];
      qt = k - gi * p.ntq;
      rank = grp / p.hp;
      h = grp - rank * p.hp;
    } else {
      rank = b / p.items_per_stage;
      const int rem = b - rank * p.items_per_stage;
      h = rem / p.ntq;
      qt = rem - h * p.ntq;
    }
    h += p.h0;  // the plan counts this launch's heads
    const int T = p.T;
    // s_blk: the slot whose context the item walks; s: the slot of this wave's
    // query rows (they differ only in tail items); ntiles_w: the tiles of the
    // walk this wave uses (a prefix)
    int s_blk, s, q0w, ntiles_w;
    bool wave_active;
    if (tail_m >= 0) {
      const int g0 = tail_m * NWAVES;
      s_blk = p.stage_of_rank[g0 / p.tail_spr];
      const int gw = g0 + wave;
      const bool has = gw < p.n_active * p.tail_spr;
      const int rank_w = has ? gw / p.tail_spr : 0;
      s = p.stage_of_rank[rank_w];
      q0w = p.tail_row0 + (gw - rank_w * p.tail_spr) * 32;
      wave_active = has && q0w < T;
      ntiles_w = p.nseg[s] * p.tps;
    } else {
      s_blk = s = p.stage_of_rank[rank];
      q0w = qt * QROWS + wave * 32;  // first query row of this wave
      wave_active = q0w < T;
      ntiles_w = p.nseg[s] * p.tps;
    }
    const int nseg = in_pool ? 1 : p.nseg[s_blk];  // chunks of this item's walk
    const int ntiles = nseg * p.tps;
    if (in_pool) ntiles_w = ntiles;

    const Uniforms u = load_uniforms<D, KB>(p, h);
    if constexpr (kFast) {
      // sources of every tile of this (stage, head), one thread per tile
      for (int t = tid; t < ntiles; t += NTHREADS) {
        const int sw = t / u.tps;  // chunk index of the walk
        const int mm = t - sw * u.tps;
        // tail items walk the live chunks in descending order; a piece walks one chunk
        const int sg = (tail_m >= 0 && sw >= p.tail_npre) ? p.tail_npre + nseg - 1 - sw : seg0 + sw;
        const int code = p.seg[s_blk][sg];
        const uint32_t t0 = uint32_t(KT) * uint32_t(mm);
        uint64_t kr, vr;
        if (code >= 0 && !p.live_pages) {  // live chunk `code`, contiguous
          const uint64_t e = (uint64_t(code) * uint32_t(u.T) + t0) * u.row_bytes;
          kr = reinterpret_cast<uint64_t>(u.k + e);
          vr = reinterpret_cast<uint64_t>(u.v + e);
        } else {  // history chunk or paged live chunk: rows t0 % P .. of one page
          const int32_t* ids = code >= 0 ? p.live_pages + code * u.ppc
                                         : p.hist_pages + (-code - 1) * u.ppc;
          const uint32_t pg = t0 / uint32_t(u.P);
          const int pid = ids[int(pg)];
          const uint32_t off = t0 - pg * uint32_t(u.P);
          const uint64_t prow = uint64_t(uint32_t(pid)) * uint32_t(u.P) + off;
          kr = reinterpret_cast<uint64_t>(u.k_pool + prow * u.krow_bytes);
          vr = reinterpret_cast<uint64_t>(u.v_pool + prow * u.row_bytes);
          if constexpr (kV8) {  // the tile's transposed block of D x 64 bytes
            const int64_t vt = (int64_t(pid) * p.spp + int(off / uint32_t(KT))) * u.H + h;
            vr = reinterpret_cast<uint64_t>(reinterpret_cast<const char*>(p.v_pool) + vt * (D * KT));
            tile_vexp[t] = p.v_exp[vt];
          }
          if constexpr (kF8) {
            const float ks =
                p.k_scale[(int64_t(pid) * p.spp + int(off / uint32_t(KT))) * u.H + h];
            tile_scale[t] = ks > 0.f ? ks : 1.f;
          }
        }
        kr |= (mm == u.tps - 1) ? 1u : 0u;  // bases are 16-byte aligned: bit 0 is free
        tile_tab[t] = make_uint4(uint32_t(kr), uint32_t(kr >> 32), uint32_t(vr), uint32_t(vr >> 32));
      }
    } else {  // page ids into LDS: history chunks, then (paged) live slots
      const int nh = p.n_hist * p.ppc;
      for (int i = tid; i < p.n_page_ids; i += NTHREADS)
        pages_lds[i] = i < nh ? p.hist_pages[i] : p.live_pages[i - nh];
    }
    __syncthreads();

    const int qrow = q0w + r;

    // ---- Q^T operand: lane holds query qrow, head dims 16*ks + 8*g .. +7 -----
    // (8-bit tier: head dims 64*dh + 32*g .. +31 of MFMA dh, as e4m3 codes)
    bf16x8 qf[kF8 ? 1 : KS];
    i32x8 qf8[2];
    float cq = u.c;  // multiplier of this lane's raw scores (8-bit: times its query scale)
    if constexpr (kF8) {
      const uint4* qp = reinterpret_cast<const uint4*>(p.q + ((int64_t(s) * T + qrow) * p.H + h) * D);
      uint4 raw[2][4];
      float am = 0.f;
#pragma unroll
      for (int dh = 0; dh < 2; ++dh)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          raw[dh][c] = (qrow < T) ? qp[8 * dh + 4 * g + c] : make_uint4(0u, 0u, 0u, 0u);
          const uint32_t w[4] = {raw[dh][c].x, raw[dh][c].y, raw[dh][c].z, raw[dh][c].w};
#pragma unroll
          for (int i = 0; i < 4; ++i)
            am = fmaxf(am, fmaxf(fabsf(__uint_as_float(w[i] << 16)),
                                 fabsf(__uint_as_float(w[i] & 0xffff0000u))));
        }
      // the row's amax (lanes l and l + 32 hold the two halves of one row), its
      // scale amax / 448 and the codes of q * (448 / amax), as the keys' producer
      // (a row with amax below 2^-100 is stored as zero, as its producer does
      // for key tiles: 448 / amax would leave float32's range)
      am = xlane32_max(am);
      const bool big = am >= 0x1p-100f;
      const float inv = big ? 448.0f / am : 0.f;
      const float qscale = am / 448.0f;
      cq = big ? u.c * qscale : u.c;  // zero row: zero codes, any multiplier
#pragma unroll
      for (int dh = 0; dh < 2; ++dh)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t w[4] = {raw[dh][c].x, raw[dh][c].y, raw[dh][c].z, raw[dh][c].w};
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const uint32_t a = w[2 * half], b = w[2 * half + 1];
            int r4 = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(a << 16) * inv,
                                                     __uint_as_float(a & 0xffff0000u) * inv, 0,
                                                     false);
            r4 = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(b << 16) * inv,
                                                 __uint_as_float(b & 0xffff0000u) * inv, r4, true);
            qf8[dh][2 * c + half] = r4;
          }
        }
    } else {
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
    // The same reads as LDS byte addresses. Rows are 2*D bytes and the swizzles
    // act on the 16-byte chunk index only (address bits 4..7 within a row), so
    // the address of K step kk is this lane's base XOR (kk << 5), and that of V
    // output block db is the base XOR (db << 6); buffer, 32-row block, 16-key
    // step and row half are constant offsets. One base per tensor then serves
    // every operand read (addresses formed from it inside each MFMA slot rather
    // than dozens of precomputed address registers).
    constexpr uint32_t TILE_BYTES = KT * D * 2;      // one V (and bf16 K) tile
    constexpr uint32_t KTILE_BYTES = KT * D * KB;   // one K tile
    // 8-bit keys: rows of D bytes, 16-byte chunk 4*dh + 2*g + piece of MFMA dh
    // (the two pieces of one 32-byte operand), swizzled by kswz8; as for bf16 the
    // address of (dh, piece) is the base XOR ((4*dh + piece) << 4).
    // (byte offsets into the tile arrays; reads are formed from the arrays
    // themselves so that the compiler knows which LDS objects they touch)
    const uint32_t k_lane = kF8 ? uint32_t(krow0 * D + (((2 * g) ^ kswz8(krow0)) << 4))
                                : uint32_t(krow0 * D * 2 + ((g ^ kx) << 4));
    // (8-bit values: row r of the transposed tile, logical chunks 2g, 2g + 1,
    // swizzled with v8swz; the second chunk is the base XOR 16)
    const uint32_t v_lane = kV8 ? uint32_t(r * 64 + (((2 * g) ^ v8swz(r)) << 4))
                                : uint32_t(vrow * D * 2 + ((vcx ^ vx) << 4) + vsub * 2);
    const char* const k_bytes = reinterpret_cast<const char*>(k_tiles);
    const char* const v_bytes = reinterpret_cast<const char*>(v_tiles);

    Loader ld;
    ld.init(u, wave, lane);
    auto resolve = [&]() __attribute__((always_inline)) {
      if constexpr (kFast) ld.prepare_table(tile_tab, ntiles);
      else ld.prepare(p, u, pages_lds, s_blk, nseg);
    };
    if constexpr (kFast) ld.start_table(tile_tab);
    resolve();
#pragma unroll
    for (int i = 0; i < NI; ++i) ld.emit(i, u, k_lds0, v_lds0, wave);
    resolve();
#pragma unroll
    for (int i = 0; i < NI; ++i) ld.emit(i, u, k_lds1, v_lds1, wave);
    resolve();
    const bool grp_a = wave < NWAVES / 2 && !kV8;
    if (!grp_a) {  // B: tile 2 as well (A issues it in its first softmax slot)
#pragma unroll
      for (int i = 0; i < NI; ++i) ld.emit(i, u, k_lds2, v_lds2, wave);
      resolve();
    }
    // tile 0 has landed (A: tile 1 may still be in flight; B: tiles 1 and 2)
    if (grp_a) tile_barrier<LPT>();
    else tile_barrier<2 * LPT>();

    // Keys of tile j that are real: 64, the chunk's remainder on a segment's last
    // tile, 0 past the end (the loop runs in groups of four tiles).
    auto valid_keys = [&](int j) __attribute__((always_inline)) {
      if (j >= ntiles) return 0;
      const int m = j - (j / u.tps) * u.tps;
      return m == u.tps - 1 ? u.t_last : KT;
    };

    f32x16 sacc[2];
    bf16x8 pb[4];
    i32x8 pb8;  // 8-bit values: P of the tile as e4m3 codes (byte j = score register j)
    float ks_next = 1.f;  // 8-bit tier: key scale of the tile whose scores are in sacc

    // 8-bit K operand op = 2*dh + blk of K tile buffer kbuf: rows of 32-key block
    // blk, head dims 64*dh + 32*g .. +31 (two 16-byte reads). The swizzled
    // chunk (dh, piece) sits at the lane base XOR ((4*dh + piece) << 4) plus
    // the buffer's and block's offsets, multiples of 32 that leave the XORed
    // bits alone: kb holds the four XORed bases (formed once per tile) and
    // every read is a base plus an immediate offset.
    struct KBase8 {
      uint32_t b[2][2];  // [dh][piece]
    };
    auto kbase8 = [&](uint32_t kl) __attribute__((always_inline)) {
      return KBase8{{{kl, kl ^ 16u}, {kl ^ 64u, kl ^ 80u}}};
    };
    auto kload8 = [&](const KBase8& kb, int kbuf, int op) __attribute__((always_inline)) {
      const uint32_t c = kbuf * KTILE_BYTES + (op & 1) * (32 * D);
      const i32x4 lo = *reinterpret_cast<const i32x4*>(k_bytes + (kb.b[op >> 1][0] + c));
      const i32x4 hi = *reinterpret_cast<const i32x4*>(k_bytes + (kb.b[op >> 1][1] + c));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    // 8-bit V^T operand of 32-channel block db of V tile buffer vbuf: row
    // 32*db + r of the transposed tile, bytes 32*g .. +31 (two 16-byte reads;
    // vl: this lane's base, vl16 = vl ^ 16 the second chunk's, the offsets
    // again multiples of 32)
    auto vload8 = [&](uint32_t vl, uint32_t vl16, int vbuf, int db) __attribute__((always_inline)) {
      const uint32_t c = vbuf * uint32_t(KT * D * VB) + db * (32 * 64);
      const i32x4 lo = *reinterpret_cast<const i32x4*>(v_bytes + (vl + c));
      const i32x4 hi = *reinterpret_cast<const i32x4*>(v_bytes + (vl16 + c));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    auto mfma8 = [&](const i32x8& a, const i32x8& b, const f32x16& c)
                     __attribute__((always_inline)) {
      // formats 0, 0: both operands e4m3; unit block scales
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
    };

    // S^T = K Q^T for one tile (the first one, before the slot pairs start): two
    // 32-key blocks, K operands two k-steps ahead.
    auto qk = [&](int kbuf) __attribute__((always_inline)) {
      uint32_t kl = k_lane;
      asm volatile("" : "+v"(kl));
      if constexpr (kF8) {
        ks_next = tile_scale[0];
        sacc[0] = f32x16{};
        sacc[1] = f32x16{};
        i32x8 ka[4];
        const KBase8 kb = kbase8(kl);
#pragma unroll
        for (int op = 0; op < 4; ++op) ka[op] = kload8(kb, kbuf, op);
#pragma unroll
        for (int op = 0; op < 4; ++op) sacc[op & 1] = mfma8(ka[op], qf8[op >> 1], sacc[op & 1]);
      } else {
        auto kload = [&](int kk, bf16x8* dst) __attribute__((always_inline)) {
          const uint32_t a = (kl ^ uint32_t(kk << 5)) + kbuf * TILE_BYTES;
#pragma unroll
          for (int blk = 0; blk < 2; ++blk)
            dst[blk] = *reinterpret_cast<const bf16x8*>(k_bytes + (a + blk * (32 * D * 2)));
        };
        sacc[0] = f32x16{};
        sacc[1] = f32x16{};
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
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };

    // Online softmax of the scores of tile j (exp2 domain): P as bf16 into pb.
    // Register x of block blk holds key 32*blk + 16*(x>>3) + 8*g + (x&7).
    // ce: the scores' multiplier (softmax scale * log2 e, times the query and
    // key scales in the 8-bit tier).
    auto softmax = [&](int j, float ce, f32x16* sc) __attribute__((always_inline)) {
      const int valid = valid_keys(j);
      if (valid < KT) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int x = 0; x < 16; ++x) {
            const int key = 32 * blk + 16 * (x >> 3) + 8 * g + (x & 7);
            if (key >= valid) sc[blk][x] = -INFINITY;
          }
      }
      // P = 2^(c s - m_run) (bf16 for the P.V product) and this lane's fp32 sum
      float lsum;
      auto exps = [&]() __attribute__((always_inline)) {
        // -0 + x is x exactly, so the first additions fold away
        float part[4] = {-0.f, -0.f, -0.f, -0.f};
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int x = 0; x < 16; x += 4) {
            float ev[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              ev[i] = __builtin_amdgcn_exp2f(fmaf(sc[blk][x + i], ce, -m_run));
              part[i] += ev[i];
            }
            if constexpr (kV8) {  // e4m3 P (at most 2^kLazyTau, inside the range)
              // (the first conversion's high half, taken from ev[0]'s register
              // rather than a zeroed one, is replaced by the second)
              int w = __builtin_amdgcn_cvt_pk_fp8_f32(ev[0], ev[1], __float_as_int(ev[0]), false);
              pb8[4 * blk + x / 4] = __builtin_amdgcn_cvt_pk_fp8_f32(ev[2], ev[3], w, true);
            } else {
#pragma unroll
              for (int i = 0; i < 4; ++i)
                pb[2 * blk + (x >> 3)][(x & 7) + i] = static_cast<__bf16>(ev[i]);
            }
          }
        lsum = (part[0] + part[1]) + (part[2] + part[3]);
      };
      exps();
      // The running reference is raised only when the tile's max exceeds it by
      // more than kLazyTau (log2 units). No P can then exceed 2^kLazyTau, and as
      // P >= 0 a sum at or below 2^kLazyTau on both lanes of every query rules
      // that out without computing the max (the first tile, against -inf, always
      // takes the check).
      if (__builtin_amdgcn_ballot_w64(!(lsum <= kLazyBound)) != 0) {
        float mx = sc[0][0];
#pragma unroll
        for (int x = 1; x < 16; ++x) mx = fmaxf(mx, sc[0][x]);
#pragma unroll
        for (int x = 0; x < 16; ++x) mx = fmaxf(mx, sc[1][x]);
        mx = xlane32_max(mx) * ce;
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
          exps();
        }
      }
      l_run += lsum;
    };

    // V^T operands of 16-key step kk of V tile buffer vbuf: two transposed LDS
    // reads per 32-row block of O^T (vl: this lane's V base).
    auto vload = [&](uint32_t vl, int vbuf, int kk, bf16x8* dst) __attribute__((always_inline)) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint32_t a = (vl ^ uint32_t(db << 6)) + vbuf * TILE_BYTES + kk * (16 * D * 2);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v_bytes + a));
        const i16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v_bytes + (a + 4 * D * 2)));
        dst[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };

    // V^T operands of the next MFMA slot's first 16-key step, read at the end of
    // the softmax slot before it (that tile landed a slot earlier), so the MFMA
    // slot starts on them while its first K operands are still in flight.
    bf16x8 vpre[DB];
    // G(j): O^T += V^T P^T of tile j and S^T = K Q^T of tile j+1, interleaved
    // MFMA by MFMA so that consecutive MFMAs never share an accumulator (the
    // score blocks recur every fourth MFMA, the output blocks every eighth). Each
    // k-step first issues the operand reads of a later step (K two k-steps
    // ahead, V one 16-key step = two k-steps ahead), then runs its P.V MFMAs,
    // then its Q.K^T MFMAs.
    auto gphase = [&](int vbuf, int kbuf, int jn) __attribute__((always_inline)) {
      // the lane bases, opaque here so that the read addresses are formed from
      // them inside the slot instead of being kept in registers across the loop
      uint32_t kl = k_lane, vl = v_lane;
      asm volatile("" : "+v"(kl), "+v"(vl));
      if constexpr (kF8) {
        // four 16-key P.V steps (four MFMAs each), each followed by one of the
        // four 8-bit Q.K^T MFMAs (blocks alternate, so no two in a row share an
        // accumulator); K operands two steps ahead, V one
        ks_next = tile_scale[jn < ntiles ? jn : 0];
        sacc[0] = f32x16{};
        sacc[1] = f32x16{};
        i32x8 ka[3];
        bf16x8 va[2][DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) va[0][db] = vpre[db];
        const KBase8 kb = kbase8(kl);
        ka[0] = kload8(kb, kbuf, 0);
        ka[1] = kload8(kb, kbuf, 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (t + 2 < 4) ka[(t + 2) % 3] = kload8(kb, kbuf, t + 2);
          if (t + 1 < 4) vload(vl, vbuf, t + 1, va[(t + 1) & 1]);
#pragma unroll
          for (int db = 0; db < DB; ++db)
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[t & 1][db], pb[t], oacc[db], 0, 0,
                                                               0);
          sacc[t & 1] = mfma8(ka[t % 3], qf8[t >> 1], sacc[t & 1]);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        auto kload = [&](int kk, bf16x8* dst) __attribute__((always_inline)) {
          const uint32_t a = (kl ^ uint32_t(kk << 5)) + kbuf * TILE_BYTES;
#pragma unroll
          for (int blk = 0; blk < 2; ++blk)
            dst[blk] = *reinterpret_cast<const bf16x8*>(k_bytes + (a + blk * (32 * D * 2)));
        };
        constexpr int PV_PER_STEP = 4 * DB / KS;  // P.V MFMAs per Q.K^T k-step
        sacc[0] = f32x16{};  // the previous scores were consumed by the last softmax
        sacc[1] = f32x16{};
        bf16x8 ka[3][2];
        bf16x8 va[2][DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) va[0][db] = vpre[db];
        kload(0, ka[0]);
        kload(1, ka[1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < KS; ++t) {
          // P.V MFMAs number PV_PER_STEP*t .. : 16-key step kk, output blocks db
          const int pv0 = PV_PER_STEP * t;
          const int kk = pv0 / DB;
          // operands of later steps go out before this step's MFMAs
          if (t + 2 < KS) kload(t + 2, ka[(t + 2) % 3]);
          if (pv0 % DB == 0 && kk + 1 < 4) vload(vl, vbuf, kk + 1, va[(kk + 1) & 1]);
#pragma unroll
          for (int e = 0; e < PV_PER_STEP; ++e) {
            const int db = (pv0 + e) % DB;
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kk & 1][db], pb[kk], oacc[db], 0, 0,
                                                               0);
          }
#pragma unroll
          for (int blk = 0; blk < 2; ++blk)
            sacc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[t % 3][blk], qf[t], sacc[blk], 0,
                                                                0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };


    // Ping-pong: waves 0..3 (group A) and 4..7 (group B) share the four SIMDs
    // one to one and run the same sequence one slot apart, so that while one
    // wave of a SIMD runs MFMAs (G(j): P.V of tile j, then Q.K^T of tile j+1,
    // interleaved) the other runs the VALU softmax S of its current tile:
    //   slot 0: A: Q.K^T(0)      B: Q.K^T(0) (early; no data dependence)
    //   slot 1: A: S(0)          B:   "
    //   slot 2: A: G(0)          B: S(0)
    //   slot 3: A: S(1)          B: G(0)      ...
    // A block-wide barrier ends every odd slot (A's softmax slots, B's MFMA
    // slots); within the two slots between barriers each SIMD's waves run one
    // softmax and one MFMA phase each, in opposite order, so they still overlap.
    // Tile t lives in buffer t % 4; all its rows must have landed by the barrier
    // that ends slot 2t-1, and it is last read in slot 2t+3. Each wave issues
    // its loads at the start of its softmax slot: A those of tile j+2 in S(j)
    // (slot 2j+1), B those of tile j+3 in S(j) (slot 2j+2); A loads tiles 0-1
    // and B tiles 0-2 up front. A buffer is refilled (slot 2t-3 or 2t-4 for tile
    // t) only after the barrier that ends the last slot reading its previous
    // tile t-4 (slot 2t-5). So at each barrier a wave may leave the loads of its
    // newest tile in flight (LPT) and every older load has landed.
    auto end_qk_slot = [&]() __attribute__((always_inline)) {
      if (!grp_a) tile_barrier<LPT>();
    };
    auto end_s_slot = [&]() __attribute__((always_inline)) {
      if (grp_a) tile_barrier<LPT>();
    };
    // The softmax slot of tile js: this wave's loads of its next tile go out
    // first (into kn, vn), then the softmax, then the first V^T operands of the
    // next MFMA slot (from tile buffer vnext).
    auto s_slot = [&](int js, uint16_t* kn, uint16_t* vn, int vnext) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < NI; ++i) ld.emit(i, u, kn, vn, wave);
      resolve();  // the tile this wave loads next
      __builtin_amdgcn_sched_barrier(0);
      if (wave_active && js < ntiles_w) {
        softmax(js, kF8 ? cq * ks_next : cq, sacc);
        __builtin_amdgcn_sched_barrier(0);
        uint32_t vl = v_lane;
        asm volatile("" : "+v"(vl));
        vload(vl, vnext, 0, vpre);
      }
      __builtin_amdgcn_sched_barrier(0);
      end_s_slot();
    };

    if constexpr (kV8) {
      // 8-bit K/V: the softmax, not the MFMA, bounds this tier, so instead of
      // the ping-pong every wave runs both phases, both waves of a SIMD in step:
      // tile j's iteration issues tile j+3's loads, the 8-bit Q.K^T of tile
      // j+1 (into the other score registers), the softmax of tile j while
      // those MFMAs run, then P.V of tile j; the two waves of a SIMD share its
      // VALU (which issues faster for two waves than for one) and overlap each
      // other's MFMAs. Tile t is in buffer t % 4; the barrier opening iteration
      // j waits for this wave's loads of tile j+1 (those of tile j+2 may still
      // be in flight) and for every wave to have finished iteration j-1, whose
      // reads were the last of buffer (j+3) % 4.
      f32x16 s0[2], s1[2];
      auto step = [&](int j, int kbuf, int vbuf, uint16_t* kn, uint16_t* vn, f32x16* sc,
                      f32x16* sn) __attribute__((always_inline)) {
        tile_barrier<LPT>();
#pragma unroll
        for (int i = 0; i < NI; ++i) ld.emit(i, u, kn, vn, wave);
        resolve();
        __builtin_amdgcn_sched_barrier(0);
        // (a wave of a tail item stops after its own slot's chunks: the tiles
        // past them are loaded for the other waves only)
        if (wave_active && j < ntiles_w) {
          uint32_t kl = k_lane, vl = v_lane;
          asm volatile("" : "+v"(kl), "+v"(vl));
          const int jj = j < ntiles ? j : 0;
          const float ks = tile_scale[jj];
          const int ve = tile_vexp[jj];
          i32x8 ka[4], va[4];
          const KBase8 kb = kbase8(kl);
          const uint32_t vl16 = vl ^ 16u;
#pragma unroll
          for (int op = 0; op < 4; ++op) ka[op] = kload8(kb, kbuf, op);
#pragma unroll
          for (int db = 0; db < DB; ++db) va[db] = vload8(vl, vl16, vbuf, db);
          sn[0] = f32x16{};
          sn[1] = f32x16{};
#pragma unroll
          for (int op = 0; op < 4; ++op) sn[op & 1] = mfma8(ka[op], qf8[op >> 1], sn[op & 1]);
          softmax(j, cq * ks, sc);
#pragma unroll
          for (int db = 0; db < DB; ++db)
            oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va[db], pb8, oacc[db], 0,
                                                                       0, 0, ve, 0, 127);
        }
        __builtin_amdgcn_sched_barrier(0);
      };
      if (wave_active) {  // Q.K^T of tile 0 (tile 0 has landed)
        uint32_t kl = k_lane;
        asm volatile("" : "+v"(kl));
        s0[0] = f32x16{};
        s0[1] = f32x16{};
        const KBase8 kb = kbase8(kl);
#pragma unroll
        for (int op = 0; op < 4; ++op) s0[op & 1] = mfma8(kload8(kb, 0, op), qf8[op >> 1], s0[op & 1]);
      }
      for (int j = 0; j < ntiles; j += 4) {
        step(j, 1, 0, k_lds3, v_lds3, s0, s1);
        step(j + 1, 2, 1, k_lds0, v_lds0, s1, s0);
        step(j + 2, 3, 2, k_lds1, v_lds1, s0, s1);
        step(j + 3, 0, 3, k_lds2, v_lds2, s1, s0);
      }
    } else {
    if (wave_active) qk(0);
    end_qk_slot();  // B (end of slot 1): tile 1 has landed (tile 2 may be in flight)
    // S(0): A loads tile 2, B tile 3; G(0) reads V of tile 0
    s_slot(0, grp_a ? k_lds2 : k_lds3, grp_a ? v_lds2 : v_lds3, 0);

    // G(j) then S(j+1); buffers vbuf, kbuf: V of tile j and K of tile j+1 (tile
    // t is in buffer t % 4); (ka_, va_) / (kb_, vb_): where A's / B's loads of
    // S(j+1) go (A: tile j+3, B: tile j+4).
    // A wave runs P.V of tile j (and Q.K^T of tile j+1, whose scores are used
    // only if j+1 < ntiles_w) for j < ntiles_w, and the softmax of tile j for
    // j < ntiles_w: tiles past its prefix are loaded for the other waves but
    // never enter its arithmetic, and the group of four tiles that overhangs
    // the walk costs no MFMA.
    auto slot_pair = [&](int j, int vbuf, int kbuf, uint16_t* ka_, uint16_t* va_, uint16_t* kb_,
                         uint16_t* vb_) __attribute__((always_inline)) {
      if (wave_active && j < ntiles_w) {
        // the MFMA phase wins issue arbitration over the other wave's softmax
        __builtin_amdgcn_s_setprio(1);
        gphase(vbuf, kbuf, j + 1);
        __builtin_amdgcn_s_setprio(0);
      }
      __builtin_amdgcn_sched_barrier(0);
      end_qk_slot();
      s_slot(j + 1, grp_a ? ka_ : kb_, grp_a ? va_ : vb_, (vbuf + 1) & 3);
    };

    for (int j = 0; j < ntiles; j += 4) {
      slot_pair(j, 0, 1, k_lds3, v_lds3, k_lds0, v_lds0);
      slot_pair(j + 1, 1, 2, k_lds0, v_lds0, k_lds1, v_lds1);
      slot_pair(j + 2, 2, 3, k_lds1, v_lds1, k_lds2, v_lds2);
      slot_pair(j + 3, 3, 0, k_lds2, v_lds2, k_lds3, v_lds3);
    }
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): no tile load outlives the loop

    // ---- epilogue: O = O^T / l, bf16 ----------------------------------------
    // (a piece: its partial state to the workspace, and the merge of its
    // item's states by the block that completes the item)
    uint16_t* const op = p.o + ((int64_t(s) * T + qrow) * p.H + h) * D;
    auto store_row = [&](const float* acc, float inv) __attribute__((always_inline)) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = 32 * db + 8 * i + 4 * g;
          bf16x4 v4;
#pragma unroll
          for (int j = 0; j < 4; ++j) v4[j] = static_cast<__bf16>(acc[16 * db + 4 * i + j] * inv);
          *reinterpret_cast<uint2*>(op + d) = __builtin_bit_cast(uint2, v4);
        }
    };
    if (!in_pool) {
      if (wave_active && qrow < T) {
        float acc[16 * DB];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int x = 0; x < 16; ++x) acc[16 * db + x] = oacc[db][x];
        store_row(acc, 1.0f / xlane32_sum(l_run));
      }
    } else {
      // Piece state, fp32: the unnormalised O as each lane holds it (16-byte
      // unit (wave, db, i, lane), so that every store and load of a wave is
      // 1 KB contiguous; the merging block's lanes hold the same rows and
      // columns), then m [QROWS] and l [QROWS] by row. Pieces of one item run
      // on any XCD, so the states are written and read with device-scope
      // accesses; a fence would write back and invalidate this XCD's whole
      // L2, the other CUs' cached tiles too.
      typedef unsigned v4u __attribute__((ext_vector_type(4)));
      constexpr int kStateBytes = int(state_bytes(D));
      char* const states = reinterpret_cast<char*>(p.ws) + kWsHeader;
      const int pi = piece / p.pool_nseg;
      const int row = wave * 32 + r;  // row of the query tile
      if (wave_active) {
        const float lsum = xlane32_sum(l_run);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            states + int64_t(piece) * kStateBytes, 0, kStateBytes, kBufferFlags);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const v4u val = {__float_as_uint(oacc[db][4 * i]), __float_as_uint(oacc[db][4 * i + 1]),
                             __float_as_uint(oacc[db][4 * i + 2]), __float_as_uint(oacc[db][4 * i + 3])};
            __builtin_amdgcn_raw_buffer_store_b128(val, rs, (((wave * DB + db) * 4 + i) * 64 + lane) * 16,
                                                   0, kDeviceScope);
          }
        if (g == 0) {
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m_run), rs, (QROWS * D + row) * 4, 0,
                                                kDeviceScope);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lsum), rs,
                                                (QROWS * D + QROWS + row) * 4, 0, kDeviceScope);
        }
      }
      // every store of the state has completed (device-visible) before the
      // count that lets another CU read it
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
      __syncthreads();
      if (threadIdx.x == 0)
        pool_slot[1] = atomicAdd(p.ws + 1 + pi, 1u) == uint32_t(p.pool_nseg - 1);
      __syncthreads();
      if (pool_slot[1] && wave_active && qrow < T) {  // every piece of item pi has left its state
        // merge in walk order (the same sums whichever block merges): the
        // states' maxima first, then each state's O and row sum, weighted
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            states + int64_t(pi) * p.pool_nseg * kStateBytes, 0, p.pool_nseg * kStateBytes,
            kBufferFlags);
        const int nk = p.pool_nseg;
        float m_all = -INFINITY;
        for (int k0 = 0; k0 < nk; k0 += 8) {  // eight loads in flight (repeats past the last are harmless)
          float mk[8];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            mk[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                rs, min(k0 + j, nk - 1) * kStateBytes + (QROWS * D + row) * 4, 0, kDeviceScope));
#pragma unroll
          for (int j = 0; j < 8; ++j) m_all = fmaxf(m_all, mk[j]);
        }
        float acc[16 * DB];
#pragma unroll
        for (int x = 0; x < 16 * DB; ++x) acc[x] = 0.f;
        float l_all = 0.f;
        for (int k = 0; k < nk; ++k) {
          const int base = k * kStateBytes;
          v4u o[4 * DB];
#pragma unroll
          for (int x = 0; x < 4 * DB; ++x)
            o[x] = __builtin_amdgcn_raw_buffer_load_b128(rs, base + ((wave * 4 * DB + x) * 64 + lane) * 16,
                                                         0, kDeviceScope);
          const float mk = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
              rs, base + (QROWS * D + row) * 4, 0, kDeviceScope));
          const float lk = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
              rs, base + (QROWS * D + QROWS + row) * 4, 0, kDeviceScope));
          const float w = __builtin_amdgcn_exp2f(mk - m_all);
          l_all += w * lk;
#pragma unroll
          for (int x = 0; x < 4 * DB; ++x)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[4 * x + j] += w * __uint_as_float(o[x][j]);
        }
        store_row(acc, 1.0f / l_all);
      }
    }
    if (!in_pool && ++item < item_end) {
      __syncthreads();  // the next item rewrites the tile-source table and the tile buffers
      continue;
    }
    if (p.pool_pieces == 0) break;
    in_pool = true;
    __syncthreads();
  }
}

// Zeroes the run-time pool's counters ahead of the attention launch (a kernel
// rather than a memset, so that the pair can be captured in a graph).
__global__ void clear_pool_kernel(uint32_t* ws, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) ws[i] = 0u;
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

// Compute units per XCD of the current device (the packing below fills that
// many bins per XCD); 0 if the runtime cannot say.
int cus_per_xcd() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    v = n / kNumXcd;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Packed work order. One workgroup fills a CU, and work items differ in
// length (a stage's keys). Launching one block per item and letting the
// hardware hand them out leaves CUs idle: the dispatcher deals blocks to the
// XCDs strictly in turn, so a CU that frees up waits until the turn reaches
// its XCD (measured: 23 us between a CU's blocks on average), and dealing
// whole groups heaviest first leaves XCDs uneven and CUs idle at the end (7 %
// of the 4-step tick). Here every CU gets one block that runs a list of items
// planned on the host:
//  1. groups, heaviest first, are dealt to the least-loaded XCD, a group being
//     split between XCDs when it would overshoot the even share (so a group's
//     query tiles stay on one or two XCDs and share their L2);
//  2. each XCD's items are packed into C bins, one per CU (longest first into
//     the emptiest bin, then moves and swaps out of the fullest bin while
//     they lower it); a block runs its bin, longest item first.
// An item's length is modelled as its key tiles plus a fixed start-up cost.
// Falls back (returns false) when the tables would not hold the plan.
bool plan_packed_order(const StagePlan& pl, int H, int tps, int C, int pool_max, AttnParams& p,
                       int64_t& blocks) {
  if (C <= 0 || C > kPackBins) return false;
  const int ntq = p.ntq;
  if (ntq > 32767) return false;
  const int G = pl.n_active * H;
  const int n_tail = p.tail ? H * p.tail_per_head : 0;
  if (int64_t(G) + n_tail > 32767) return false;
  constexpr int kStartup = 2;  // start-up cost of a workgroup, in key tiles
  // work groups: (stage, head) groups of ntq query tiles (ntq - 1 with tail
  // items), and the tail items, one each; heaviest first
  struct Group { int grp, n, w; };
  std::vector<Group> groups;
  const int ntq_full = p.tail ? ntq - 1 : ntq;
  for (int g = 0; g < G && ntq_full > 0; ++g)
    groups.push_back(Group{g, ntq_full, int(pl.nseg[pl.order[g / H]]) * tps + kStartup});
  for (int t = 0; t < n_tail; ++t) {
    const int m = t % p.tail_per_head;
    const int s_walk = pl.order[(m * NWAVES) / p.tail_spr];
    groups.push_back(Group{G + t, 1, int(pl.nseg[s_walk]) * tps + kStartup});
  }
  // the run-time pool: full query tiles of the heaviest slot, the last ones of
  // its heads in turn, about kPoolShare of the tick's work
  p.pool_items = p.pool_pieces = p.pool_nseg = 0;
  if (pool_max > 0 && ntq_full > 0 && pl.nseg[pl.order[0]] >= 2) {
    int64_t all = 0;
    for (const Group& gr : groups) all += int64_t(gr.w) * gr.n;
    const int w0 = groups[0].w;  // a query tile of rank 0 (groups 0 .. H-1 are rank 0's)
    int want = int(std::lround(kPoolShare * double(all) / w0));
    want = std::min({want, pool_max, kMaxPool, H * ntq_full});
    for (int i = 0; i < want; ++i) --groups[i % H].n;  // tile ntq_full - 1 - i / H of head i % H
    p.pool_qt0 = ntq_full - 1;
    p.pool_items = want;
    p.pool_nseg = pl.nseg[pl.order[0]];
    p.pool_pieces = want * p.pool_nseg;
  }
  std::stable_sort(groups.begin(), groups.end(), [](const Group& a, const Group& b) { return a.w > b.w; });
  int64_t total = 0;
  for (const Group& gr : groups) total += int64_t(gr.w) * gr.n;
  struct Run { int grp, qt0, n, w; };
  struct Packed {
    int16_t grp[kNumXcd][kPackSegs], qt0[kNumXcd][kPackSegs], bin[kNumXcd][kPackBins + 1];
    uint32_t code[kNumXcd][kPackItems / 8];
    int16_t n[kNumXcd];
  };
  // Deal the groups to XCDs against a per-XCD target, then pack each XCD's
  // items onto its CUs; returns the busiest CU's load, or -1 if the tables do
  // not hold the plan.
  auto plan_with = [&](double target, Packed& out) -> int64_t {
    Run runs[kNumXcd][kPackSegs];
    int nrun[kNumXcd] = {0};
    int64_t load[kNumXcd] = {0};
    for (const Group& gr : groups) {
      const int w = gr.w;
      int rem = gr.n, qt = 0;
      while (rem > 0) {
        int x = 0;
        for (int i = 1; i < kNumXcd; ++i)
          if (load[i] < load[x]) x = i;
        const double room = target - double(load[x]);
        int n = room <= 0 ? rem : std::min(rem, std::max(1, int(std::ceil(room / w))));
        if (nrun[x] == kPackSegs) return -1;
        runs[x][nrun[x]++] = Run{gr.grp, qt, n, w};
        load[x] += int64_t(n) * w;
        rem -= n;
        qt += n;
      }
    }
    for (int x = 0; x < kNumXcd; ++x) {
      int n_items = 0;
      for (int r = 0; r < nrun[x]; ++r) n_items += runs[x][r].n;
      if (n_items > kPackItems) return -1;
    }
    int64_t busiest = 0;
    for (int x = 0; x < kNumXcd; ++x) {
      // items of this XCD: run index and length, longest first (runs already are)
      int item_run[kPackItems], item_w[kPackItems];
      int n = 0;
      for (int r = 0; r < nrun[x]; ++r)
        for (int i = 0; i < runs[x][r].n; ++i) {
          item_run[n] = r;
          item_w[n] = runs[x][r].w;
          ++n;
        }
      // bins: item indices; longest first into the emptiest bin
      std::vector<std::vector<int>> bin(C);
      std::vector<int64_t> bl(C, 0);
      for (int i = 0; i < n; ++i) {
        int b = 0;
        for (int j = 1; j < C; ++j)
          if (bl[j] < bl[b]) b = j;
        bin[b].push_back(i);
        bl[b] += item_w[i];
      }
      // Local search on the fullest bin: among moving one item out of it and
      // exchanging one or two of its items for zero, one or two of another bin's,
      // take the exchange that leaves the pair's larger load smallest, while that
      // is below the fullest load. (Items come in a few lengths — one per stage —
      // so single moves and swaps alone stall well above the mean load.)
      for (int iter = 0; iter < 4096; ++iter) {
        int hi = 0;
        for (int j = 1; j < C; ++j)
          if (bl[j] > bl[hi]) hi = j;
        // best exchange: sets of up to two positions in bin[hi] and in bin[lo]
        int64_t best = bl[hi];
        int b_lo = -1, b_a[2] = {-1, -1}, b_c[2] = {-1, -1};
        const std::vector<int>& H_ = bin[hi];
        const int nh = int(H_.size());
        for (int lo = 0; lo < C; ++lo) {
          if (lo == hi) continue;
          const std::vector<int>& L_ = bin[lo];
          const int nl = int(L_.size());
          // (a0, a1): positions in hi (a1 = -1: one item); (c0, c1): in lo (-1: none)
          for (int a0 = 0; a0 < nh; ++a0)
            for (int a1 = -1; a1 < nh; ++a1) {
              if (a1 >= 0 && a1 <= a0) continue;
              const int wa = item_w[H_[a0]] + (a1 >= 0 ? item_w[H_[a1]] : 0);
              for (int c0 = -1; c0 < nl; ++c0)
                for (int c1 = -1; c1 < nl; ++c1) {
                  if (c0 < 0 && c1 >= 0) continue;
                  if (c1 >= 0 && c1 <= c0) continue;
                  const int wc = (c0 >= 0 ? item_w[L_[c0]] : 0) + (c1 >= 0 ? item_w[L_[c1]] : 0);
                  const int d = wa - wc;
                  if (d <= 0) continue;
                  const int64_t m = std::max(bl[hi] - d, bl[lo] + d);
                  if (m < best) {
                    best = m;
                    b_lo = lo;
                    b_a[0] = a0; b_a[1] = a1; b_c[0] = c0; b_c[1] = c1;
                  }
                }
            }
        }
        if (b_lo < 0) break;
        std::vector<int> out_hi, out_lo;
        std::vector<int> keep_hi, keep_lo;
        for (int i = 0; i < nh; ++i) (i == b_a[0] || i == b_a[1] ? out_hi : keep_hi).push_back(H_[i]);
        for (int i = 0; i < int(bin[b_lo].size()); ++i)
          (i == b_c[0] || i == b_c[1] ? out_lo : keep_lo).push_back(bin[b_lo][i]);
        for (int it : out_lo) keep_hi.push_back(it);
        for (int it : out_hi) keep_lo.push_back(it);
        int64_t l_hi = 0, l_lo = 0;
        for (int it : keep_hi) l_hi += item_w[it];
        for (int it : keep_lo) l_lo += item_w[it];
        bin[hi] = keep_hi;
        bin[b_lo] = keep_lo;
        bl[hi] = l_hi;
        bl[b_lo] = l_lo;
      }
      // the XCD's list: bin by bin, longest first within a bin
      int order[kPackItems];
      int no = 0;
      for (int j = 0; j < C; ++j) {
        std::sort(bin[j].begin(), bin[j].end(), [&](int a, int b) { return item_w[a] > item_w[b]; });
        out.bin[x][j] = int16_t(no);
        for (int it : bin[j]) order[no++] = it;
      }
      out.bin[x][C] = int16_t(no);
      out.n[x] = int16_t(no);
      for (int r = 0; r < kPackSegs; ++r) {
        out.grp[x][r] = int16_t(r < nrun[x] ? runs[x][r].grp : 0);
        out.qt0[x][r] = int16_t(r < nrun[x] ? runs[x][r].qt0 : 0);
      }
      for (int w = 0; w < kPackItems / 8; ++w) out.code[x][w] = 0;
      for (int k = 0; k < no; ++k)
        out.code[x][k >> 3] |= uint32_t(item_run[order[k]]) << (4 * (k & 7));
      for (int j = 0; j < C; ++j) busiest = std::max(busiest, bl[j]);
    }
    return busiest;
  };
  // The dealing overshoots each XCD's target by up to one item, and items
  // come in a few lengths, so an XCD may end up a fraction of an item above
  // what its CUs can share evenly: a few targets are tried and the plan with
  // the least-loaded busiest CU is kept.
  static const double kTargetScale[] = {1.0, 0.999, 0.998, 0.996, 0.994, 0.992, 0.99, 0.985, 0.98};
  Packed best{}, cand{};
  int64_t best_load = -1;
  for (double f : kTargetScale) {
    const int64_t l = plan_with(f * double(total) / kNumXcd, cand);
    if (l >= 0 && (best_load < 0 || l < best_load)) {
      best_load = l;
      best = cand;
    }
  }
  if (best_load < 0) return false;
  std::memcpy(p.pack_grp, best.grp, sizeof(best.grp));
  std::memcpy(p.pack_qt0, best.qt0, sizeof(best.qt0));
  std::memcpy(p.pack_bin, best.bin, sizeof(best.bin));
  std::memcpy(p.pack_code, best.code, sizeof(best.code));
  std::memcpy(p.xcd_n, best.n, sizeof(best.n));
  p.use_xcd = 2;
  blocks = int64_t(kNumXcd) * C;  // one block per CU
  return true;
}

// Tail items (see AttnParams): used when every active slot's last query tile
// holds at most half a workgroup's rows, so that two or more slots share an
// item, and every active slot's context is, as a set, a prefix of the heaviest
// slot's walk (history and live store as listed, then the live chunks in
// descending order) — true unless the slots' history budgets differ. Only the
// bf16 kernel with whole-tile sources runs them.
void plan_tail(const wf_tick_desc& d, const StagePlan& pl, AttnParams& p) {
  p.tail = 0;
  if (pl.n_active < 2) return;
  const int r = d.T - (p.ntq - 1) * QROWS;
  const int spr = (r + 31) / 32;
  if (2 * spr > NWAVES) return;
  const int s0 = pl.order[0];
  const int n0 = pl.nseg[s0];
  int npre = 0;  // history chunks and the live store lead every list
  while (npre < n0 && (pl.seg[s0][npre] < 0 || pl.seg[s0][npre] == d.S)) ++npre;
  int walk[WF_MAX_SEGMENTS];
  for (int i = 0; i < n0; ++i) walk[i] = i < npre ? pl.seg[s0][i] : pl.seg[s0][npre + n0 - 1 - i];
  auto bit = [](int code) { return uint64_t(1) << (code >= 0 ? 32 + code : -code - 1); };
  for (int k = 0; k < pl.n_active; ++k) {
    const int s = pl.order[k];
    if (pl.nseg[s] > n0) return;
    uint64_t want = 0, got = 0;
    for (int i = 0; i < pl.nseg[s]; ++i) {
      want |= bit(walk[i]);
      got |= bit(pl.seg[s][i]);
    }
    if (want != got) return;
    int lead = 0;  // its list must lead with the same history and store entries
    while (lead < pl.nseg[s] && (pl.seg[s][lead] < 0 || pl.seg[s][lead] == d.S)) ++lead;
    if (lead != std::min(npre, int(pl.nseg[s]))) return;
  }
  p.tail = 1;
  p.tail_row0 = (p.ntq - 1) * QROWS;
  p.tail_spr = spr;
  p.tail_per_head = (pl.n_active * spr + NWAVES - 1) / NWAVES;
  p.tail_npre = npre;
}

// The launch's work order: tail items and the packed per-CU lists when they
// fit, else whole (stage, head) groups dealt to XCDs, else the plain order.
// Pool items a workspace of `bytes` holds for this tick (each item takes one
// partial state per chunk of the heaviest slot's walk); 0 where the pool does
// not apply (per-lane page lookups, or no workspace).
int pool_capacity(const wf_tick_desc& d, const StagePlan& pl, int64_t bytes) {
  const bool paged = d.n_hist > 0 || d.live_pages != nullptr || d.store_pages != nullptr;
  const bool fast = !paged || d.P % KT == 0;
  if (!fast || pl.n_active == 0 || bytes <= kWsHeader) return 0;
  const int64_t per_item = pl.nseg[pl.order[0]] * state_bytes(d.D);
  return int(std::min<int64_t>(kMaxPool, (bytes - kWsHeader) / per_item));
}

void plan_launch_uncached(const wf_tick_desc& d, const StagePlan& pl, int C, int pool_max,
                          AttnParams& p, int64_t& blocks) {
  p.n_active = pl.n_active;
  p.pool_items = p.pool_pieces = p.pool_nseg = 0;
  const bool paged = d.n_hist > 0 || d.live_pages != nullptr || d.store_pages != nullptr;
  const bool fast = !paged || d.P % KT == 0;
  if (fast) plan_tail(d, pl, p);
  blocks = int64_t(pl.n_active) * p.items_per_stage;
  // a pool leaves groups with fewer tiles, which can split into more runs
  // than the tables hold: retry with one pool item fewer (the pool takes at
  // most pool_max and at most its share) before giving up packing
  bool packed = plan_packed_order(pl, d.H, p.tps, C, pool_max, p, blocks);
  for (int cap = p.pool_items - 1; !packed && cap >= 0; --cap)
    packed = plan_packed_order(pl, d.H, p.tps, C, cap, p, blocks);
  if (!packed) {
    p.tail = 0;
    p.pool_items = p.pool_pieces = p.pool_nseg = 0;
    blocks = int64_t(pl.n_active) * p.items_per_stage;
    plan_xcd_order(pl, d.H, p, blocks);
  }
}

// The work-order members of AttnParams, copied between a cached plan and a
// launch's parameters.
void copy_plan(const AttnParams& from, AttnParams& to) {
  to.use_xcd = from.use_xcd;
  to.xcd_stride = from.xcd_stride;
  to.tail = from.tail;
  to.tail_row0 = from.tail_row0;
  to.tail_spr = from.tail_spr;
  to.tail_per_head = from.tail_per_head;
  to.tail_npre = from.tail_npre;
  to.n_active = from.n_active;
  to.pool_pieces = from.pool_pieces;
  to.pool_nseg = from.pool_nseg;
  to.pool_items = from.pool_items;
  to.pool_qt0 = from.pool_qt0;
  std::memcpy(to.xcd_n, from.xcd_n, sizeof(to.xcd_n));
  std::memcpy(to.xcd_groups, from.xcd_groups, sizeof(to.xcd_groups));
  std::memcpy(to.pack_grp, from.pack_grp, sizeof(to.pack_grp));
  std::memcpy(to.pack_qt0, from.pack_qt0, sizeof(to.pack_qt0));
  std::memcpy(to.pack_bin, from.pack_bin, sizeof(to.pack_bin));
  std::memcpy(to.pack_code, from.pack_code, sizeof(to.pack_code));
}

// Plans depend only on the tick's shape (slots, mask, sizes, history budgets,
// formats, paging) and the CU count, and a streaming rollout repeats a few
// shapes tick after tick, so the last kPlanCache plans are kept (the packing
// search costs tens of milliseconds of host time).
constexpr int kPlanCache = 16;
struct PlanKey {
  int32_t v[16 + WF_MAX_STAGES];
  bool operator==(const PlanKey& o) const { return std::memcmp(v, o.v, sizeof(v)) == 0; }
};
struct PlanEntry {
  PlanKey key;
  AttnParams plan;
  int64_t blocks;
  uint64_t used;
};

PlanKey plan_key(const wf_tick_desc& d, int C, int pool_max) {
  PlanKey k;
  std::memset(&k, 0, sizeof(k));
  const int32_t head[] = {d.S, int32_t(d.active_mask), d.T, d.H, d.D, d.n_hist, d.P,
                          d.k_format, d.v_format, d.live_pages != nullptr, d.store_pages != nullptr,
                          C, pool_max};
  std::memcpy(k.v, head, sizeof(head));
  for (int s = 0; s <= d.S && s < WF_MAX_STAGES; ++s) k.v[16 + s] = d.hist_first[s];
  return k;
}

void plan_launch(const wf_tick_desc& d, const StagePlan& pl, int C, int pool_max, AttnParams& p,
                 int64_t& blocks) {
  static std::mutex mu;
  static PlanEntry cache[kPlanCache];
  static int n_cached = 0;
  static uint64_t clock = 0;
  const PlanKey key = plan_key(d, C, pool_max);
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < n_cached; ++i)
      if (cache[i].key == key) {
        cache[i].used = ++clock;
        copy_plan(cache[i].plan, p);
        blocks = cache[i].blocks;
        return;
      }
  }
  plan_launch_uncached(d, pl, C, pool_max, p, blocks);
  std::lock_guard<std::mutex> lock(mu);
  int slot = n_cached < kPlanCache ? n_cached++ : 0;
  if (slot == 0 && n_cached == kPlanCache)  // evict the least recently used
    for (int i = 1; i < kPlanCache; ++i)
      if (cache[i].used < cache[slot].used) slot = i;
  cache[slot].key = key;
  copy_plan(p, cache[slot].plan);
  cache[slot].blocks = blocks;
  cache[slot].used = ++clock;
}

// The work order of the launch over heads [h0, h0 + hp) of a descriptor:
// planned as a tick of hp heads (the plan counts the launch's heads), into the
// plan members of p (p.H, the tensors' head count, is not touched).
void plan_part(const wf_tick_desc& d, const StagePlan& pl, int C, int64_t ws_bytes, int h0, int hp,
               AttnParams& p, int64_t& blocks) {
  wf_tick_desc dp = d;
  dp.H = hp;
  p.hp = hp;
  p.h0 = h0;
  p.items_per_stage = hp * p.ntq;
  blocks = 0;
  plan_launch(dp, pl, C, pool_capacity(dp, pl, ws_bytes), p, blocks);
}

// Heads per launch. One launch covers every head unless its plan cannot be
// packed (one block per CU running a list) while a split into n launches of
// ceil(H / n) heads can: more (stage, head) groups than the tables hold would
// otherwise run one block per item, which leaves CUs waiting for the
// dispatcher between blocks and idle at the end. A tick of a few items per CU
// loses little that way and stays one launch. Returns (h0, hp) per launch.
std::vector<std::array<int, 2>> head_parts(const wf_tick_desc& d, const StagePlan& pl, int C,
                                           int64_t ws_bytes, AttnParams& trial) {
  int64_t blocks = 0;
  plan_part(d, pl, C, ws_bytes, 0, d.H, trial, blocks);
  if (trial.use_xcd == 2 || C <= 0 || blocks < int64_t(kMinSplitItems) * kNumXcd * C)
    return {{0, d.H}};
  for (int n = 2; n <= kMaxHeadParts && n <= d.H; ++n) {
    const int hp = (d.H + n - 1) / n;
    const int last = d.H - (n - 1) * hp;
    if (last <= 0) continue;
    plan_part(d, pl, C, ws_bytes, 0, hp, trial, blocks);
    if (trial.use_xcd != 2) continue;
    plan_part(d, pl, C, ws_bytes, 0, last, trial, blocks);
    if (trial.use_xcd != 2) continue;
    std::vector<std::array<int, 2>> parts;
    for (int i = 0; i < n; ++i) parts.push_back({i * hp, i + 1 < n ? hp : last});
    return parts;
  }
  return {{0, d.H}};
}

// Base members of a launch's parameters that the host-only planners need.
void plan_base(const wf_tick_desc& d, AttnParams& p) {
  std::memset(&p, 0, sizeof(p));
  p.T = d.T;
  p.H = d.H;
  p.tps = (d.T + KT - 1) / KT;
  p.ntq = (d.T + QROWS - 1) / QROWS;
}


// kFast: every tile is one uniform span of a page or live chunk (page size a
// multiple of 64, or no history); otherwise history tiles resolve per lane.
template <int D, bool kFast, bool kF8 = false, bool kV8 = false>
int32_t launch_attn(const AttnParams& p, unsigned blocks, hipStream_t stream) {
  attn_tick_kernel<D, kFast, kF8, kV8><<<dim3(blocks), NTHREADS, 0, stream>>>(p);
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
  if (d->k_format != WF_K_BF16 && d->k_format != WF_K_E4M3)
    return fail(WF_EINVAL, "wf_attn_tick: k_format = %d (WF_K_BF16 or WF_K_E4M3)", d->k_format);
  if (d->v_format != WF_V_BF16 && d->v_format != WF_V_E4M3)
    return fail(WF_EINVAL, "wf_attn_tick: v_format = %d (WF_V_BF16 or WF_V_E4M3)", d->v_format);
  if (d->v_format == WF_V_E4M3 && d->k_format != WF_K_E4M3)
    return fail(WF_EINVAL, "wf_attn_tick: 8-bit values need 8-bit keys (k_format = WF_K_E4M3)");
  if (d->k_format == WF_K_E4M3) {
    if (d->D != 128)
      return fail(WF_EUNSUPPORTED, "wf_attn_tick: 8-bit keys need D = 128 (D = %d)", d->D);
    if (d->P <= 0 || d->P % KT != 0)
      return fail(WF_EINVAL, "wf_attn_tick: 8-bit keys need P a multiple of 64 (P = %d)", d->P);
  }
  if (d->T == 0 || d->active_mask == 0) return WF_OK;
  const bool live_paged = d->live_pages != nullptr;
  if (d->k_format == WF_K_E4M3) {
    if (!live_paged)
      return fail(WF_EINVAL, "wf_attn_tick: 8-bit keys are read through pages: set live_pages");
    if (d->store_pages)
      return fail(WF_EINVAL, "wf_attn_tick: store_pages writes bf16 pages: not with 8-bit keys");
    if (!d->k_scale || (reinterpret_cast<uintptr_t>(d->k_scale) & 3u))
      return fail(WF_EINVAL, "wf_attn_tick: 8-bit keys need k_scale (4-byte aligned)");
    if (d->v_format == WF_V_E4M3 && !d->v_exp)
      return fail(WF_EINVAL, "wf_attn_tick: 8-bit values need v_exp");
  }
  if (!d->q || !d->o || (!live_paged && (!d->k || !d->v)))
    return fail(WF_EINVAL, "wf_attn_tick: q, o (and k, v without live_pages) must be non-NULL");
  if (!aligned16(d->q) || !aligned16(d->o) ||
      (!live_paged && (!aligned16(d->k) || !aligned16(d->v))))
    return fail(WF_EINVAL, "wf_attn_tick: q, k, v and o must be 16-byte aligned");
  if (int64_t(d->T) > (int64_t(1) << 24))
    return fail(WF_EUNSUPPORTED, "wf_attn_tick: T = %d too large", d->T);
  const bool store_fused = d->store_pages != nullptr;
  if (store_fused) {
    if (live_paged)
      return fail(WF_EINVAL, "wf_attn_tick: store_pages and live_pages exclude each other");
    if (!((d->active_mask >> d->S) & 1u))
      return fail(WF_EINVAL, "wf_attn_tick: store_pages needs the store slot S active");
  }
  if (d->n_hist > 0 || live_paged || store_fused) {
    if (!d->k_pool || !d->v_pool || (d->n_hist > 0 && !d->hist_pages))
      return fail(WF_EINVAL,
                  "wf_attn_tick: n_hist > 0 or live_pages needs k_pool, v_pool (and hist_pages)");
    if (!aligned16(d->k_pool) || !aligned16(d->v_pool))
      return fail(WF_EINVAL, "wf_attn_tick: pools must be 16-byte aligned");
    if (d->P <= 0 || d->P % 16 != 0)
      return fail(WF_EINVAL, "wf_attn_tick: page size P = %d must be a positive multiple of 16",
                  d->P);
    if (d->num_pages <= 0) return fail(WF_EINVAL, "wf_attn_tick: num_pages = %d", d->num_pages);
    const int64_t ppc = (int64_t(d->T) + d->P - 1) / d->P;
    if (ppc > d->num_pages)
      return fail(WF_EINVAL, "wf_attn_tick: a chunk needs %lld pages, pool has %d",
                  static_cast<long long>(ppc), d->num_pages);
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

// The work items of attention block b (counted after the store blocks), as
// the kernel decodes them from the plan, appended to `rows` as (item index in
// the block, rank, head, first query row, rows): one row per item, or for a
// tail item one per rank among its slices.
void decode_block(const AttnParams& p, int b, std::vector<std::array<int, 5>>& rows) {
  auto tile = [&](int k, int rank, int h, int qt) {
    const int q0 = qt * QROWS;
    rows.push_back({k, rank, h, q0, std::min(QROWS, p.T - q0)});
  };
  if (p.use_xcd == 2) {
    const int x = b & (kNumXcd - 1);
    const int c = b / kNumXcd;
    const int G = p.n_active * p.hp;
    for (int k = p.pack_bin[x][c]; k < p.pack_bin[x][c + 1]; ++k) {
      const int run = (p.pack_code[x][k >> 3] >> (4 * (k & 7))) & 15;
      int before = 0;
      for (int i = 0; i < k; ++i) before += ((p.pack_code[x][i >> 3] >> (4 * (i & 7))) & 15) == run;
      const int grp = p.pack_grp[x][run];
      const int item = k - p.pack_bin[x][c];
      if (grp < G) {
        tile(item, grp / p.hp, grp % p.hp, p.pack_qt0[x][run] + before);
        continue;
      }
      const int h = (grp - G) / p.tail_per_head;
      const int m = (grp - G) % p.tail_per_head;
      for (int w = 0; w < NWAVES; ++w) {  // slices, grouped by rank
        const int gw = m * NWAVES + w;
        if (gw >= p.n_active * p.tail_spr) break;
        const int rank = gw / p.tail_spr;
        const int q0 = p.tail_row0 + (gw - rank * p.tail_spr) * 32;
        if (q0 >= p.T) continue;
        const int n = std::min(32, p.T - q0);
        if (!rows.empty() && rows.back()[0] == item && rows.back()[1] == rank &&
            rows.back()[2] == h && rows.back()[3] + rows.back()[4] == q0)
          rows.back()[4] += n;
        else
          rows.push_back({item, rank, h, q0, n});
      }
    }
  } else if (p.use_xcd) {
    const int x = b & (kNumXcd - 1);
    const int k = b / kNumXcd;
    const int gi = k / p.ntq;
    if (gi >= p.xcd_n[x]) return;
    const int grp = p.xcd_groups[x * p.xcd_stride + gi];
    tile(0, grp / p.hp, grp % p.hp, k - gi * p.ntq);
  } else {
    const int rank = b / p.items_per_stage;
    const int rem = b - rank * p.items_per_stage;
    tile(0, rank, rem / p.ntq, rem % p.ntq);
  }
}

}  // namespace
}  // namespace wf

extern "C" wf_status wf_tick_work_order(const wf_tick_desc* desc, int32_t cus_per_xcd_hint,
                                        int32_t* out, int64_t capacity, int64_t* n_items) {
  using namespace wf;
  try {
    if (!n_items) return fail(WF_EINVAL, "wf_tick_work_order: n_items is NULL");
    int32_t st = validate_tick(desc);
    if (st != WF_OK) return st;
    const wf_tick_desc& d = *desc;
    *n_items = 0;
    if (d.T == 0 || d.active_mask == 0) return WF_OK;
    StagePlan pl;
    plan_stages(d, pl);
    const int C = cus_per_xcd_hint > 0 ? cus_per_xcd_hint : cus_per_xcd();
    const int64_t ws_bytes = d.workspace ? d.workspace_bytes : 0;
    AttnParams p;
    plan_base(d, p);
    AttnParams trial = p;
    const auto parts = head_parts(d, pl, C, ws_bytes, trial);
    // launches in order, their blocks numbered on; then every launch's pool items
    std::vector<int> out_rows, pool_rows;
    int64_t block0 = 0;
    int pool0 = 0;
    for (const auto& part : parts) {
      int64_t blocks = 0;
      plan_part(d, pl, C, ws_bytes, part[0], part[1], p, blocks);
      for (int64_t b = 0; b < blocks; ++b) {
        std::vector<std::array<int, 5>> items;
        decode_block(p, int(b), items);
        for (const auto& it : items)
          out_rows.insert(out_rows.end(), {int(block0 + b), it[0], pl.order[it[1]], part[0] + it[2],
                                           it[3], it[4]});
      }
      for (int i = 0; i < p.pool_items; ++i) {  // run-time pool: block -1
        const int q0 = (p.pool_qt0 - i / part[1]) * QROWS;
        pool_rows.insert(pool_rows.end(), {-1, pool0 + i, pl.order[0], part[0] + i % part[1], q0,
                                           std::min(QROWS, d.T - q0)});
      }
      block0 += blocks;
      pool0 += p.pool_items;
    }
    out_rows.insert(out_rows.end(), pool_rows.begin(), pool_rows.end());
    *n_items = int64_t(out_rows.size() / 6);
    if (!out) return WF_OK;
    if (capacity < int64_t(out_rows.size()))
      return fail(WF_EINVAL, "wf_tick_work_order: capacity %lld < 6 * %lld rows",
                  static_cast<long long>(capacity), static_cast<long long>(out_rows.size() / 6));
    std::copy(out_rows.begin(), out_rows.end(), out);
    return WF_OK;
  } catch (...) {
    return fail(WF_EINVAL, "wf_tick_work_order: internal error");
  }
}

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

namespace wf {
namespace {
// Device address of the allocation-free entry point's workspace on the
// current device, looked up with that device current on its first call there.
void* scratch_address(int32_t& st) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    st = hip_fail(e, "wf_attn_tick_noalloc (hipGetDevice)");
    return nullptr;
  }
  if (dev < 0 || dev >= 64) {
    st = fail(WF_EUNSUPPORTED, "wf_attn_tick_noalloc: device %d beyond 64", dev);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) {
      st = hip_fail(e, "wf_attn_tick_noalloc (hipGetSymbolAddress)");
      return nullptr;
    }
    addr[dev] = ptr;
  }
  st = WF_OK;
  return addr[dev];
}

int32_t attn_tick_impl(const wf_tick_desc* desc, void* ws, int64_t ws_bytes, hipStream_t stream) {
  {
    int32_t st = validate_tick(desc);
    if (st != WF_OK) return st;
    const wf_tick_desc& d = *desc;
    if (d.T == 0 || d.active_mask == 0) return WF_OK;
    StagePlan pl;
    plan_stages(d, pl);
    const bool live_paged = d.live_pages != nullptr;
    const bool store_fused = d.store_pages != nullptr;
    const bool paged = d.n_hist > 0 || live_paged || store_fused;
    const int32_t ppc = paged ? int32_t((int64_t(d.T) + d.P - 1) / d.P) : 0;
    if (d.n_hist > 0 && check_pages_enabled()) {
      st = check_device_pages(d.hist_pages, int64_t(d.n_hist) * ppc, d.num_pages, stream,
                              "wf_attn_tick");
      if (st != WF_OK) return st;
    }
    if (store_fused && check_pages_enabled()) {
      st = check_device_pages(d.store_pages, ppc, d.num_pages, stream,
                              "wf_attn_tick (store_pages)");
      if (st != WF_OK) return st;
    }
    if (live_paged && check_pages_enabled()) {
      for (int j = 0; j <= d.S; ++j) {
        if (!((d.active_mask >> j) & 1u)) continue;
        st = check_device_pages(d.live_pages + int64_t(j) * ppc, ppc, d.num_pages, stream,
                                "wf_attn_tick (live_pages)");
        if (st != WF_OK) return st;
      }
    }
    AttnParams p;
    std::memset(&p, 0, sizeof(p));
    p.q = static_cast<const uint16_t*>(d.q);
    p.k_pool = static_cast<const uint16_t*>(d.k_pool);
    p.v_pool = static_cast<const uint16_t*>(d.v_pool);
    // with paged live slots k and v are never read (kept non-NULL for the
    // head-offset arithmetic)
    p.k = live_paged ? p.k_pool : static_cast<const uint16_t*>(d.k);
    p.v = live_paged ? p.v_pool : static_cast<const uint16_t*>(d.v);
    p.o = static_cast<uint16_t*>(d.o);
    p.hist_pages = d.hist_pages;
    p.live_pages = d.live_pages;
    p.store_pages = d.store_pages;
    p.store_slot = d.S;
    p.store_row16 = int32_t(int64_t(d.H) * d.D * 2 / 16);
    p.n_store_blocks = store_fused ? (ppc + kNumXcd - 1) / kNumXcd * kNumXcd : 0;
    p.n_hist = d.n_hist;
    const bool f8 = d.k_format == WF_K_E4M3;
    p.k_scale = f8 ? d.k_scale : nullptr;
    const bool v8 = f8 && d.v_format == WF_V_E4M3;
    p.v_exp = v8 ? d.v_exp : nullptr;
    p.spp = f8 ? d.P / KT : 0;
    p.T = d.T;
    p.H = d.H;
    p.P = paged ? d.P : 16;
    p.ppc = ppc;
    p.tps = (d.T + KT - 1) / KT;
    p.t_last = d.T - KT * (p.tps - 1);
    p.p_magic = uint32_t((uint64_t(1) << 32) / uint64_t(p.P) + 1);
    p.c = float(double(d.scale) * 1.4426950408889634);
    p.ntq = (d.T + QROWS - 1) / QROWS;
    p.n_page_ids = (d.n_hist + (live_paged ? d.S + 1 : 0)) * ppc;
    for (int i = 0; i < pl.n_active; ++i) p.stage_of_rank[i] = pl.order[i];
    for (int s = 0; s <= d.S; ++s) {
      p.nseg[s] = pl.nseg[s];
      for (int i = 0; i < pl.nseg[s]; ++i) p.seg[s][i] = pl.seg[s][i];
    }
    const bool fast = !paged || d.P % KT == 0;
    if (fast) {  // the kernel keeps a table of tile sources in LDS
      int max_seg = 0;
      for (int i = 0; i < pl.n_active; ++i) max_seg = std::max(max_seg, pl.nseg[pl.order[i]]);
      if (int64_t(max_seg) * p.tps > kMaxTiles)
        return fail(WF_EUNSUPPORTED, "wf_attn_tick: %d chunks of %d tiles exceed %d tiles", max_seg,
                    p.tps, kMaxTiles);
    } else if (p.n_page_ids > kMaxPageIds) {  // the kernel keeps the page table in LDS
      return fail(WF_EUNSUPPORTED, "wf_attn_tick: page table of %d ids exceeds %d", p.n_page_ids,
                  kMaxPageIds);
    }
    const int C = cus_per_xcd();
    const int64_t pool_bytes = ws ? ws_bytes : 0;
    p.ws = static_cast<uint32_t*>(ws);
    const int n_store_blocks = p.n_store_blocks;
    AttnParams trial = p;
    const auto parts = head_parts(d, pl, C, pool_bytes, trial);
    for (size_t i = 0; i < parts.size(); ++i) {  // launches in stream order, one per head range
      int64_t blocks = 0;
      plan_part(d, pl, C, pool_bytes, parts[i][0], parts[i][1], p, blocks);
      p.n_store_blocks = i == 0 ? n_store_blocks : 0;  // the first launch writes the store pages
      if (p.pool_pieces > 0) {  // counters of the run-time pool start at zero
        clear_pool_kernel<<<1, 64, 0, stream>>>(p.ws, 1 + p.pool_items);
        st = check_launch("wf_attn_tick (pool counters)");
        if (st != WF_OK) return st;
      }
      blocks += p.n_store_blocks;  // a multiple of 8: the XCD of every attention block is kept
      if (blocks > 0x7fffffff) return fail(WF_EUNSUPPORTED, "wf_attn_tick: grid too large");
      if (v8)  // (validated: D = 128, P a multiple of 64, so fast)
        st = launch_attn<128, true, true, true>(p, unsigned(blocks), stream);
      else if (f8)
        st = launch_attn<128, true, true>(p, unsigned(blocks), stream);
      else if (d.D == 128)
        st = fast ? launch_attn<128, true>(p, unsigned(blocks), stream)
                  : launch_attn<128, false>(p, unsigned(blocks), stream);
      else
        st = fast ? launch_attn<64, true>(p, unsigned(blocks), stream)
                  : launch_attn<64, false>(p, unsigned(blocks), stream);
      if (st != WF_OK) return st;
      st = check_launch("wf_attn_tick");
      if (st != WF_OK) return st;
    }
    return WF_OK;
  }
}

}  // namespace
}  // namespace wf

extern "C" wf_status wf_attn_tick(const wf_tick_desc* desc, hipStream_t stream) {
  using namespace wf;
  try {
    if (desc && desc->workspace && (reinterpret_cast<uintptr_t>(desc->workspace) & 255u))
      return fail(WF_EINVAL, "wf_attn_tick: workspace must be 256-byte aligned");
    if (desc && desc->workspace_bytes < 0)
      return fail(WF_EINVAL, "wf_attn_tick: workspace_bytes = %lld",
                  static_cast<long long>(desc->workspace_bytes));
    return attn_tick_impl(desc, desc ? desc->workspace : nullptr,
                          desc ? desc->workspace_bytes : 0, stream);
  } catch (...) {
    return fail(WF_EINVAL, "wf_attn_tick: internal error");
  }
}

extern "C" wf_status wf_tick_workspace_bytes(const wf_tick_desc* desc, int64_t* bytes) {
  using namespace wf;
  try {
    if (!bytes) return fail(WF_EINVAL, "wf_tick_workspace_bytes: bytes is NULL");
    int32_t st = validate_tick(desc);
    if (st != WF_OK) return st;
    *bytes = 0;
    if (desc->T == 0 || desc->active_mask == 0) return WF_OK;
    StagePlan pl;
    plan_stages(*desc, pl);
    if (pool_capacity(*desc, pl, int64_t(1) << 60) == 0) return WF_OK;
    // the items the planner gives the pool when space is no limit (the CU
    // count of the current device, else MI355X's 32 per XCD)
    const int C = cus_per_xcd() > 0 ? cus_per_xcd() : 32;
    const int64_t unlimited = int64_t(1) << 60;
    AttnParams p;
    plan_base(*desc, p);
    AttnParams trial = p;
    for (const auto& part : head_parts(*desc, pl, C, unlimited, trial)) {
      int64_t blocks = 0;
      plan_part(*desc, pl, C, unlimited, part[0], part[1], p, blocks);
      if (p.pool_items > 0)
        *bytes = std::max<int64_t>(
            *bytes, kWsHeader + int64_t(p.pool_items) * p.pool_nseg * state_bytes(desc->D));
    }
    return WF_OK;
  } catch (...) {
    return fail(WF_EINVAL, "wf_tick_workspace_bytes: internal error");
  }
}

extern "C" wf_status wf_attn_tick_noalloc(const wf_tick_desc* desc, hipStream_t stream) {
  using namespace wf;
  try {
    if (!desc) return fail(WF_EINVAL, "wf_attn_tick_noalloc: desc is NULL");
    if (desc->workspace)
      return fail(WF_EINVAL, "wf_attn_tick_noalloc: workspace must be NULL (the library's own is used)");
    if (desc->workspace_bytes < 0 || desc->workspace_bytes > WF_NOALLOC_SCRATCH_BYTES)
      return fail(WF_EINVAL, "wf_attn_tick_noalloc: workspace_bytes = %lld outside [0, %lld]",
                  static_cast<long long>(desc->workspace_bytes),
                  static_cast<long long>(WF_NOALLOC_SCRATCH_BYTES));
    void* ws = nullptr;
    if (desc->workspace_bytes > 0) {
      int32_t st = WF_OK;
      ws = scratch_address(st);
      if (!ws) return st;
    }
    return attn_tick_impl(desc, ws, desc->workspace_bytes, stream);
  } catch (...) {
    return fail(WF_EINVAL, "wf_attn_tick_noalloc: internal error");
  }
}
