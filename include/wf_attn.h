/*
 * wf_attn.h — C ABI of libwfattn.so: one wave tick of chunk-wise causal
 * wavefront attention on an AMD Instinct MI355X (gfx950).
 *
 * Citations name pages of "Wave Forcing: Towards Speed-of-Light Streaming Video
 * Generation": [summary] = the structured summary page (picx.dev);
 * [full text] = the full-text page (paperpeel.com).
 *
 * The method ([summary] Methodology 1, [full text] Eq. (4), Eq. (5), Appendix
 * B.3): at tick k the S denoising stages hold chunks Z_k^(0) .. Z_{k-S+1}^(S-1)
 * and the store holds B_{k-S} as stage S. Every chunk's queries attend, in one
 * softmax, to: clean history chunks (anchor first, oldest first), the live store,
 * then the live chunks at stages j >= s (itself first). Chunks at noisier stages
 * j < s are never read. The store's K/V is written straight into history pages
 * and becomes history after the tick ([full text] §4.2, Appendix B.3, Eq. (13)).
 *
 * Conventions shared by every call:
 *  - Tensors are bf16 (bit pattern uint16), C-contiguous, head-interleaved:
 *      live q/k/v/o  [S+1][T][H][D]       chunk slot s = stage s, slot S = store
 *      K pool, V pool [num_pages][P][H][D] one page = P consecutive tokens of one
 *                                          chunk, all heads; page bytes contiguous
 *      page tables    int32, device memory
 *  - The caller owns all device memory and the stream; the library allocates no
 *    device memory and keeps no pointer after a call returns. Device calls are
 *    stream-ordered and asynchronous: a WF_OK return means "validated and
 *    enqueued".
 *  - Every argument is validated on the host before anything is launched. On any
 *    error nothing is launched, no output and no page-table state changes, and
 *    wf_last_error() describes the problem. C++ exceptions never cross the ABI.
 *  - Page ids inside device page tables are trusted for speed; with the
 *    environment variable WF_CHECK_PAGES=1 the library copies them to the host
 *    (synchronising the stream) and range-checks them first.
 */
#ifndef WF_ATTN_H_
#define WF_ATTN_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t wf_status;
#define WF_OK 0
#define WF_EINVAL (-1)       /* bad shape, pointer, alignment, mask or index      */
#define WF_ENOMEM (-2)       /* page pool exhausted                              */
#define WF_EHIP (-3)         /* a HIP runtime call or kernel launch failed        */
#define WF_EUNSUPPORTED (-4) /* valid but outside what the kernels implement      */
#define WF_ESTATE (-5)       /* call out of order (commit without alloc, ...)     */

#define WF_MAX_STAGES 8      /* S + 1 <= 8 chunk slots per tick                   */
#define WF_MAX_SEGMENTS 32   /* history chunks + live chunks one query may see    */

/* Text of the last non-OK status returned on this thread ("" if none). */
const char* wf_last_error(void);

/* ABI version of this header (bumped on any incompatible change). */
int32_t wf_abi_version(void);
#define WF_ABI_VERSION 7

/* ------------------------------------------------------------------------ */
/* Page table: host-only state for one request's attention pages.            */
/* [full text] Appendix B.3 (promotion of the live store page, persistent     */
/* anchor), Appendix B.8 / Eq. (13) (fixed-capacity K/V arrays, bounded       */
/* history). Policy (the pages give none): FIFO free list — allocation pops   */
/* ceil(T/P) ids from the front, an evicted chunk's ids are appended to the   */
/* back in page order. Eviction removes the oldest history chunk, or the      */
/* oldest after the anchor when pin_anchor != 0. One handle must not be used  */
/* from two threads at once.                                                  */
/* ------------------------------------------------------------------------ */
typedef struct wf_page_table wf_page_table;

/* num_pages, page_size (P), chunk_tokens (T), window_chunks (history capacity,
 * >= 2 when pin_anchor) must be positive. initial_free_order: host array of
 * num_pages distinct ids in [0, num_pages), or NULL for 0..num_pages-1.
 * *out receives a new handle (freed with wf_page_table_destroy). */
wf_status wf_page_table_create(int32_t num_pages, int32_t page_size, int32_t chunk_tokens,
                               int32_t window_chunks, int32_t pin_anchor,
                               const int32_t* initial_free_order, wf_page_table** out);
void wf_page_table_destroy(wf_page_table* pt);

/* Pages per chunk, ceil(T/P). */
wf_status wf_page_table_pages_per_chunk(const wf_page_table* pt, int32_t* out);

/* Allocate the pages of the store chunk about to be written (the live store U).
 * out_ids: host int32[capacity], capacity >= pages per chunk. WF_ENOMEM when the
 * free list is short, WF_ESTATE when a live chunk is already allocated. */
wf_status wf_page_table_alloc_chunk(wf_page_table* pt, int32_t* out_ids, int32_t capacity);

/* Promote the live chunk to history; if history then exceeds the window, evict
 * one chunk and return its ids to the free list. evicted_ids (host, may be NULL
 * when capacity is 0) receives the evicted ids, *n_evicted their count (0 or
 * pages per chunk). WF_ESTATE without a live chunk. */
wf_status wf_page_table_commit(wf_page_table* pt, int32_t* evicted_ids, int32_t capacity,
                               int32_t* n_evicted);

/* History page lists, oldest chunk first: out = host int32[n_hist][ppc]
 * (capacity in int32 elements). *n_hist_chunks receives the chunk count. This
 * is the table wf_attn_tick reads once the caller has copied it to the device. */
wf_status wf_page_table_export(const wf_page_table* pt, int32_t* out, int32_t capacity,
                               int32_t* n_hist_chunks);

wf_status wf_page_table_num_free(const wf_page_table* pt, int32_t* out);

/* ------------------------------------------------------------------------ */
/* wf_store_paged — write the store chunk's K and V into its pages.          */
/* [full text] §4.2 and Appendix B.3: K/V goes directly into its final        */
/* attention slots. Token t -> slot t % P of page page_ids[t / P]; slots past */
/* token T-1 in the last page are written as zero. Bit-exact copy.            */
/* k_src, v_src: device bf16 [T][H][D]; k_pool, v_pool: device bf16           */
/* [num_pages][P][H][D]; page_ids: device int32 [ceil(T/P)], each in          */
/* [0, num_pages). All pointers 16-byte aligned; H*D*2 a multiple of 16 bytes. */
/* Errors: WF_EINVAL for bad sizes, NULL or misaligned pointers, ceil(T/P) >   */
/* num_pages; WF_EUNSUPPORTED when K and V together exceed 2^32 16-byte units */
/* (64 GiB); WF_EHIP if the launch fails. T = 0 is a no-op.                  */
/* ------------------------------------------------------------------------ */
wf_status wf_store_paged(const void* k_src, const void* v_src, void* k_pool, void* v_pool,
                         const int32_t* page_ids, int32_t T, int32_t H, int32_t D,
                         int32_t num_pages, int32_t P, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* wf_rope_store_paged — a producer's write of one chunk's K and V into its   */
/* pages, with the rotary position embedding applied to K on the way.        */
/* [summary] Methodology 3 and [full text] Appendix B.1: K/V are published     */
/* after the QKV projection and RoPE; [full text] Appendix B.8, Eq. (13): the  */
/* K/V arrays hold every chunk of the context, live ones included; [full      */
/* text] Appendix B.3: the anchor keeps its unrotated key and is rotated again */
/* when the window shifts (call with v_src = v_pool = NULL and the anchor's   */
/* pages: only K is rewritten).                                               */
/* Rotation (the pages give no formula; the common rotary form per axis of    */
/* the latent grid): token t of a grid[0] x grid[1] x grid[2] (frames x rows x */
/* columns, row-major) chunk has coordinates (frame0 + t/(R*C), (t/C)%R, t%C); */
/* channel pair (2i, 2i+1) of every head turns by coordinate * frequency:     */
/* (x0, x1) -> (x0 cos a - x1 sin a, x0 sin a + x1 cos a). Pairs are grouped   */
/* by axis: the first split[0] channels follow the frame, the next split[1]   */
/* the row, the last split[2] the column; pair i' of a group of d channels has */
/* frequency theta^(-2i'/d). fp32 arithmetic, bf16 result rounded to nearest  */
/* even; V is copied bit for bit.                                             */
/* Placement as wf_store_paged: token t -> slot t % P of page page_ids[t/P],   */
/* slots past token T-1 of the last page written as zero (K, and V if given). */
/* k_src (pre-rotation keys), v_src: device bf16 [T][H][D]; pools: device bf16 */
/* [num_pages][P][H][D]; page_ids: device int32 [ceil(T/P)]. 16-byte aligned. */
/* Errors: WF_EINVAL for NULL pointers (v_src and v_pool must be both NULL or  */
/* both set), grid not positive or not holding T tokens, frame0 < 0 or        */
/* frame0 + grid[0] > 2^24, odd or negative split parts, split sum != D,       */
/* theta not positive and finite, ceil(T/P) > num_pages; WF_EUNSUPPORTED for  */
/* D not 64/128 or ceil(T/P)*P >= 2^31; WF_EHIP if the launch fails. With   */
/* valid sizes and D, T = 0 is a no-op.                                       */
/* ------------------------------------------------------------------------ */
typedef struct wf_rope_desc {
  int32_t grid[3];  /* latent grid of one chunk: frames, rows, columns; product = T */
  int32_t frame0;   /* latent frame index of the chunk's first frame (>= 0)         */
  int32_t split[3]; /* channels per axis (frame, row, column): even, sum = D         */
  float theta;      /* frequency base, e.g. 10000                                   */
} wf_rope_desc;

wf_status wf_rope_store_paged(const void* k_src, const void* v_src, void* k_pool, void* v_pool,
                              const int32_t* page_ids, int32_t T, int32_t H, int32_t D,
                              int32_t num_pages, int32_t P, const wf_rope_desc* rope,
                              hipStream_t stream);

/* wf_rope_store_paged_chunks — n_chunks producer writes in one launch (a tick's
 * live chunks), chunk c exactly as wf_rope_store_paged writes it with its
 * first frame at rope->frame0 + c * frame_step: k_src (and v_src, or both
 * NULL with v_pool) device bf16 [n_chunks][T][H][D], page_ids device int32
 * [n_chunks][ceil(T/P)], the chunks' pages distinct. In the wave, slot j holds
 * video chunk c_store + S - j, so slots 0..S in order have frame_step = -F
 * ([summary] Methodology 1). Errors as wf_rope_store_paged, each chunk's first
 * frame checked; WF_EINVAL for n_chunks < 0; n_chunks = 0 is a no-op. */
wf_status wf_rope_store_paged_chunks(const void* k_src, const void* v_src, int32_t n_chunks,
                                     void* k_pool, void* v_pool, const int32_t* page_ids,
                                     int32_t T, int32_t H, int32_t D, int32_t num_pages,
                                     int32_t P, const wf_rope_desc* rope, int32_t frame_step,
                                     hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* wf_store_paged_fp8 — a producer's write of one chunk into the pages of the */
/* 8-bit tier: K as e4m3 codes with fp32 scales, V copied as bf16.            */
/* [full text] §4.3 (K/V quantisation shrinks K/V payloads; an 8-bit attention */
/* backend for local computation), Appendix C.5 Table 8 and C.6 (FP8 K/V).    */
/* The pages fix neither the format nor the scale granularity; here: e4m3     */
/* (1 sign, 4 exponent bits of bias 7, 3 mantissa bits, largest finite 448),  */
/* one scale per (64-token tile of a page, head): amax = max |k| over the     */
/* tile's tokens of that head, scale = amax / 448, code = e4m3 of the fp32    */
/* product k * (448 / amax) rounded to nearest even (both quotients fp32,    */
/* correctly rounded; an all-zero tile, or one with amax below 2^-100, has    */
/* scale 0 and zero codes). A key stands for decode(code) * scale.           */
/* Token t -> slot t % P of page                                              */
/* page_ids[t / P]; slots past token T-1 hold zero codes and zero V, and a    */
/* tile holding none of the chunk's tokens has scale 0.                       */
/* k_src, v_src: device bf16 [T][H][D]; k_pool: device uint8                  */
/* [num_pages][P][H][D]; k_scale: device fp32 [num_pages][P/64][H]; page_ids: */
/* device int32 [ceil(T/P)].                                                  */
/* v_exp NULL: v_pool is device bf16 [num_pages][P][H][D] and V is copied.    */
/* v_exp set (8-bit values): V is quantised per (64-token tile, head) with a  */
/* power-of-two scale 2^e, e the smallest integer >= -127 with              */
/* amax <= 448 * 2^e (0 for an all-zero tile; -127 is the least exponent     */
/* v_exp holds), code = e4m3 of v * 2^-e (exact product, rounded to           */
/* nearest even); v_exp: device uint8 [num_pages][P/64][H] receives e + 127;  */
/* v_pool: device uint8 [num_pages][P/64][H][D][64] is written in the layout  */
/* the attention's P.V operand reads: row d of tile (page, sub-tile, head)    */
/* holds channel d of the tile's 64 tokens, byte 32*g + j being token         */
/* 32*(j/16) + 16*((j/8)%2) + 8*g + j%8 (g = 0, 1; j = 0..31); tokens past    */
/* the chunk hold zero codes.                                                 */
/* Errors: WF_EINVAL for bad sizes, P not a multiple of 64, NULL pointers,    */
/* tensors not 16-byte aligned (k_scale: 4-byte), ceil(T/P) > num_pages;      */
/* WF_EUNSUPPORTED for D not 64/128 or H > 65535; WF_EHIP if the launch fails. */
/* T = 0 is a no-op.                                                         */
/* ------------------------------------------------------------------------ */
wf_status wf_store_paged_fp8(const void* k_src, const void* v_src, void* k_pool, float* k_scale,
                             void* v_pool, uint8_t* v_exp, const int32_t* page_ids, int32_t T,
                             int32_t H, int32_t D, int32_t num_pages, int32_t P,
                             hipStream_t stream);

/* wf_store_paged_fp8_chunks — n_chunks producer writes in one launch (a tick's
 * live chunks, each into its own pages), each chunk exactly as
 * wf_store_paged_fp8 writes it: k_src, v_src device bf16 [n_chunks][T][H][D],
 * page_ids device int32 [n_chunks][ceil(T/P)]; pools, scales and v_exp as
 * there. The chunks' pages must be distinct. One launch instead of n keeps the
 * memory system busy across the chunks instead of ramping up and down for
 * each. Errors as wf_store_paged_fp8, plus WF_EINVAL for n_chunks < 0;
 * n_chunks = 0 is a no-op. */
wf_status wf_store_paged_fp8_chunks(const void* k_src, const void* v_src, int32_t n_chunks,
                                    void* k_pool, float* k_scale, void* v_pool, uint8_t* v_exp,
                                    const int32_t* page_ids, int32_t T, int32_t H, int32_t D,
                                    int32_t num_pages, int32_t P, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* wf_gather_paged — diagnostic inverse of the store: copy n_chunks chunks    */
/* from pool pages into contiguous k_dst, v_dst bf16 [n_chunks][T][H][D].     */
/* page_ids: device int32 [n_chunks][ceil(T/P)]. Same alignment rules and     */
/* errors (the 2^32-unit limit counts the n_chunks chunks of K and of V).      */
/* ------------------------------------------------------------------------ */
wf_status wf_gather_paged(const void* k_pool, const void* v_pool, const int32_t* page_ids,
                          int32_t n_chunks, void* k_dst, void* v_dst, int32_t T, int32_t H,
                          int32_t D, int32_t num_pages, int32_t P, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* wf_attn_tick — all S+1 query chunks of one tick in a single launch (a     */
/* tick with more (stage, head) groups than one launch's work plan packs runs */
/* as a few launches over head ranges, in stream order on the same stream).   */
/* For each active stage s and head h:                                        */
/*   O_s = softmax(scale * Q_s K_ctx(s)^T) V_ctx(s), where ctx(s) is, in the  */
/*   Eq. (5) order: history chunks c = hist_first[s] .. n_hist-1 (read through */
/*   hist_pages), the live store (slot S) if active, then live chunks         */
/*   j = s .. S-1 that are active. For s = S the live part is the store only.  */
/* Mask [summary] / [full text] Eq. (4): M_WF(s, j) = 1[j >= s]. Chunks with   */
/* j < s are never enumerated (block skip), so their K/V is never read.        */
/* Arithmetic: bf16 MFMA products, fp32 accumulation and softmax state, P     */
/* rounded to bf16 for the P.V product, bf16 output (round to nearest even).  */
/* With live_pages set, every key of the context is read through pages: the  */
/* results equal those of the same tick with the live K/V in k and v.         */
/* 8-bit tier (k_format = WF_K_E4M3): k_pool holds e4m3 codes with scales in  */
/* k_scale, as written by wf_store_paged_fp8; every key is read through pages */
/* (live_pages required). Each query row (one head) is quantised in the       */
/* kernel the same way with its own scale (amax over its D channels), Q.K^T   */
/* runs on the e4m3 MFMA with fp32 accumulation, and the scores are the       */
/* product of the codes' dot product, the query scale and the key tile's      */
/* scale; the softmax and P.V are those of the bf16 tier. Needs D = 128, P a  */
/* multiple of 64, no store_pages; a query row with amax below 2^-100 is     */
/* taken as zero, as key tiles are.                                           */
/* 8-bit values as well (v_format = WF_V_E4M3, with WF_K_E4M3): v_pool holds  */
/* the transposed e4m3 tiles and v_exp their exponents, as written by          */
/* wf_store_paged_fp8 with v_exp; P is rounded to e4m3 (P <= 2^8: the running */
/* reference lies at most 8 below the row max in log2 units, never above it) */
/* and P.V runs on the e4m3 MFMA with the tile's                             */
/* power-of-two scale applied by the MFMA; the softmax's sum uses the          */
/* unrounded P.                                                               */
/* Errors: WF_EINVAL for bad sizes, masks, pointers (NULL or not 16-byte      */
/* aligned; workspace not 256-byte aligned or workspace_bytes < 0), P not a   */
/* positive multiple of 16, n_hist*ceil(T/P) > num_pages;                     */
/* v_format not WF_V_BF16/WF_V_E4M3, WF_V_E4M3 without WF_K_E4M3 or v_exp;  */
/* k_format not WF_K_BF16/WF_K_E4M3, or WF_K_E4M3 without live_pages or      */
/* k_scale, with store_pages, or with P not a multiple of 64;                 */
/* WF_EUNSUPPORTED for D not 64/128 (WF_K_E4M3: not 128), n_hist + S + 1 > 32, */
/* T > 2^24,                                                                  */
/* T*P >= 2^32, num_pages*P >= 2^31, and tables the kernel stages in LDS    */
/* that would not fit: with P a multiple of 64, more than 1536 64-key tiles   */
/* in one slot's context (segments * ceil(T/64)); otherwise more than 4096    */
/* page ids (n_hist*ceil(T/P), plus (S+1)*ceil(T/P) with live_pages);         */
/* WF_EHIP if the launch fails. T = 0 or active_mask = 0 is a no-op.          */
/* ------------------------------------------------------------------------ */
typedef struct wf_tick_desc {
  int32_t S;              /* denoising stages, 0..7; slot S is the store           */
  uint32_t active_mask;   /* bit s set = slot s occupied; bits above S must be 0    */
  int32_t T, H, D;        /* tokens per chunk (>= 0), heads (>= 1), head dim 64|128 */
  float scale;            /* softmax scale (> 0, finite), e.g. 1/sqrt(D)            */
  const void* q;          /* device bf16 [S+1][T][H][D]                             */
  const void* k;          /* device bf16 [S+1][T][H][D] (unused with live_pages)    */
  const void* v;          /* device bf16 [S+1][T][H][D] (unused with live_pages)    */
  void* o;                /* device bf16 [S+1][T][H][D]; rows of inactive slots are */
                          /* left untouched                                          */
  const void* k_pool;     /* device bf16 [num_pages][P][H][D]; needed when n_hist > 0 */
  const void* v_pool;     /* or live_pages is set, ignored otherwise                */
  int32_t num_pages, P;   /* pool size in pages; tokens per page (multiple of 16)   */
  const int32_t* hist_pages; /* device int32 [n_hist][ceil(T/P)], oldest first      */
  int32_t n_hist;         /* clean history chunks, n_hist + S + 1 <= 32            */
  int32_t hist_first[WF_MAX_STAGES]; /* per slot: first visible history chunk,     */
                          /* 0 = all, n_hist = none (per-rank history budgets)      */
  const int32_t* live_pages; /* device int32 [S+1][ceil(T/P)]: the pages holding    */
                          /* each live slot's K/V (fully paged context, [full text] */
                          /* Appendix B.8, Eq. (13); rows of inactive slots are not */
                          /* read), or NULL: live K/V come from k and v, which may  */
                          /* then be NULL when this is set                          */
  const int32_t* store_pages; /* device int32 [ceil(T/P)], or NULL. Set: the same    */
                          /* launch also writes live slot S's K/V into these pages, */
                          /* exactly as wf_store_paged (one launch per tick instead */
                          /* of two). Needs slot S active, the pools, P, num_pages; */
                          /* excludes live_pages                                    */
  int32_t k_format;       /* WF_K_BF16 (0): k_pool bf16; WF_K_E4M3 (1): k_pool uint8 */
                          /* e4m3 codes [num_pages][P][H][D] with k_scale           */
  const float* k_scale;   /* device fp32 [num_pages][P/64][H] with WF_K_E4M3, else  */
                          /* ignored                                                */
  int32_t v_format;       /* WF_V_BF16 (0), or WF_V_E4M3 (1, needs WF_K_E4M3):      */
                          /* v_pool uint8 transposed tiles [num_pages][P/64][H][D]  */
                          /* [64] with v_exp                                        */
  const uint8_t* v_exp;   /* device uint8 [num_pages][P/64][H] with WF_V_E4M3       */
  void* workspace;        /* device scratch (256-byte aligned), or NULL. Set, with   */
                          /* whole-tile sources (any key format), part of the       */
                          /* work (query tiles of the heaviest slot, cut into one  */
                          /* chunk of keys each) is handed out while the launch    */
                          /* runs to whichever CU is free, and the pieces' partial  */
                          /* softmax states are merged there; the results are those */
                          /* of the same arithmetic in another summation order. The */
                          /* library zeroes the counters it uses before each launch; */
                          /* launches sharing a workspace must not overlap.          */
                          /* wf_tick_workspace_bytes gives the size that lets the   */
                          /* pool reach its full share; a smaller one holds fewer   */
                          /* pieces. Not read or written by the caller.             */
  int64_t workspace_bytes; /* bytes at workspace (>= 0)                              */
} wf_tick_desc;

#define WF_K_BF16 0
#define WF_K_E4M3 1
#define WF_V_BF16 0
#define WF_V_E4M3 1

wf_status wf_attn_tick(const wf_tick_desc* desc, hipStream_t stream);

/* Allocation-free variant of wf_attn_tick, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the run-time pool's workspace is an array of
 * WF_NOALLOC_SCRATCH_BYTES in the library's code object, one per GPU, held
 * until the process ends; the call allocates nothing. desc->workspace must be
 * NULL and desc->workspace_bytes (0 .. WF_NOALLOC_SCRATCH_BYTES) is the part of
 * the array the pool may use: the smaller of wf_tick_workspace_bytes and the
 * maximum gives the same launch as wf_attn_tick with a workspace of that size
 * (0: no pool). Beyond the maximum, or with a workspace pointer: WF_EINVAL.
 * Every call on a GPU uses that GPU's one array, which keeps the last call's
 * contents (the counters are cleared at each call): calls that overlap on one
 * GPU (on different streams, or from several host threads) race. Otherwise as
 * wf_attn_tick. */
#define WF_NOALLOC_SCRATCH_BYTES (64ll << 20)
wf_status wf_attn_tick_noalloc(const wf_tick_desc* desc, hipStream_t stream);

/* Workspace size for wf_attn_tick with this descriptor: the bytes that hold the
 * run-time pool's full share (about 8 % of the tick's work, at most 128 query
 * tiles, one partial state of 256 rows x (D + 2) fp32 per chunk of keys, plus
 * 1 KB of counters); 0 when the tick does not use one. Host only; errors as
 * wf_attn_tick's validation, WF_EINVAL for a NULL bytes. */
wf_status wf_tick_workspace_bytes(const wf_tick_desc* desc, int64_t* bytes);

/* Diagnostic, host only: the work order wf_attn_tick would launch for this
 * descriptor. Row i = out[6i .. 6i+5] = (block, item, slot, head, first query
 * row, rows): attention block `block` (counted after the blocks that write the
 * store's pages; it runs on XCD block % 8) computes query rows [first, first +
 * rows) of that slot and head in its item number `item`, items in the order
 * the block runs them; block -1 lists the run-time pool's items (with a
 * workspace), which whichever blocks are free compute chunk by chunk. An ordinary item is one query tile (256 rows) of one
 * slot; a tail item holds the last query tile's rows of several slots of one
 * head, one row per slot. cus_per_xcd: compute units per XCD to plan for
 * (<= 0: the current device's). *n_items receives the row count; out (host
 * int32, capacity elements, may be NULL to query the count) must hold
 * 6 * n_items.
 * The plan ([summary] Methodology 3: stage s reads N_s keys, so work items
 * differ in length): (slot, head) groups, heaviest first, are dealt to the
 * least-loaded XCD (split between two XCDs to even the loads), and each XCD's
 * items are packed onto its CUs, one block per CU running its list, longest
 * first. When every slot's last query tile holds at most 128 rows and the
 * slots' contexts nest (equal history budgets), those tiles of one head are
 * merged into tail items of eight 32-row slices that walk the heaviest such
 * slot's context with the live chunks in descending order, each slice's wave
 * stopping after its own slot's chunks (whole-tile sources only, any key
 * format). Ticks whose plan does not fit the kernel's tables run one item per
 * block instead, whole groups per XCD. Errors as wf_attn_tick's validation;
 * WF_EINVAL for a short out or a NULL n_items. */
wf_status wf_tick_work_order(const wf_tick_desc* desc, int32_t cus_per_xcd, int32_t* out,
                             int64_t capacity, int64_t* n_items);

/* Useful FLOPs of one call with this descriptor: 4*D*H per visible
 * (query, key) pair (Q.K^T plus P.V), exponentials not counted. Host only. */
wf_status wf_tick_useful_flops(const wf_tick_desc* desc, double* out);

#ifdef __cplusplus
}
#endif
#endif /* WF_ATTN_H_ */
