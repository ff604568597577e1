/*
 * lora.h - C ABI of the MI355X multi-LoRA apply library (gfx950, HIP).
 *
 * What the library computes.  For an adapted linear layer, token i with
 * adapter a(i) needs
 *
 *     y_i = x_i W + scale_a * (x_i A_a^T) B_a
 *
 * ("Multi-LoRA Serving - S-LoRA/Punica Batching" study page, section "The
 * kernel trick: gather, do not merge").  The shared base product x W is one
 * dense GEMM for the whole batch and is NOT computed here: the caller puts it
 * in y first.  This library adds the adapter term, gathering each token's own
 * adapter from a device-resident paged store, without merging weights.
 *
 * Layouts (row-major; elements of the pool's dtype unless noted):
 *   x   [n_tokens][ld_x]   input rows (h_in used)
 *   t   [n_tokens][ld_t]   float32 intermediate x A^T (rank columns used)
 *   y   [n_tokens][ld_y]   output rows (h_out used), updated in place
 *   A   [rank][h_in]       one adapter's rank rows, each of length h_in
 *   B   [rank][h_out]      one adapter's rank rows, each of length h_out
 * Rows of x, t and y are indexed by the ORIGINAL token index.
 *
 * Paged store ("Thousands of adapters", slide 8: a page holds H elements, a
 * rank-R adapter takes R pages).  The pool is an array of pages of
 * page_elems elements.  Each rank row of A (B) spans h_in/page_elems
 * (h_out/page_elems) pages, so one (slot, module) entry uses
 * rank * (h_in + h_out) / page_elems pages, allocated at the adapter's own
 * rank (no padding to the maximum rank).  Pages need not be contiguous.
 *
 * Adapter ids: -1 marks a token without an adapter (y untouched).  An id outside
 * [-1, n_slots) is treated as -1 and counted in the segment meta (word
 * LORA_META_N_BAD); lora_segments_check reports it as LORA_ERR_DEVICE_IDS.
 * A slot with no adapter loaded for a module adds nothing.
 *
 * Streams: `stream` is a hipStream_t passed as void* (NULL = null stream).
 * Every compute call is asynchronous on `stream` and returns after enqueueing.
 * Pointers are device pointers unless marked [host].
 *
 * Errors: every call returns a lora_status.  Argument checks run on the host
 * before anything is enqueued; a call that returns an error has enqueued
 * nothing and changed nothing.  No call aborts or throws.
 *
 * Ownership: the pool owns its pages and slot table.  The caller owns x, t,
 * y, ids, the segment buffer and workspaces; the library never frees them.
 */
#ifndef LORA_MI355X_H
#define LORA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LORA_ABI_VERSION 8

typedef int32_t lora_status;
enum {
    LORA_OK = 0,
    LORA_ERR_ARG = -1,         /* null pointer, bad enum, negative size, misaligned pointer */
    LORA_ERR_SHAPE = -2,       /* dims not multiples of page_elems, module shape mismatch   */
    LORA_ERR_RANK = -3,        /* rank < 1 or rank > the pool's max_rank (the rank cap)      */
    LORA_ERR_NO_PAGES = -4,    /* not enough free pages for the adapter                      */
    LORA_ERR_SLOT = -5,        /* slot/module out of range, already loaded, or empty         */
    LORA_ERR_DTYPE = -6,       /* unsupported dtype combination                              */
    LORA_ERR_HIP = -7,         /* a HIP runtime call failed                                  */
    LORA_ERR_DEVICE_IDS = -8,  /* (segments_check) the batch held ids outside [-1, n_slots)  */
    LORA_ERR_WORKSPACE = -9    /* workspace too small                                        */
};

typedef enum { LORA_F32 = 0, LORA_BF16 = 1 } lora_dtype;

/* Largest rank a pool accepts (the load-time rank cap: study page, "Memory:
 * slots, tiers and paging", cap ranks because slots reserve the maximum). */
#define LORA_MAX_RANK 64

/* Returns LORA_ABI_VERSION. */
int32_t lora_abi_version(void);

/* Static text for a status code. */
const char *lora_status_str(lora_status s);

/* ------------------------------------------------------------------------ */
/* Paged adapter store (GPU slots: study page, "Memory: slots, tiers and   */
/* paging"; unified paging: "Thousands of adapters", slide 8)               */
/* ------------------------------------------------------------------------ */
typedef struct lora_pool lora_pool;   /* opaque, library-owned */

typedef struct {
    int64_t n_pages;         /* pages in the pool                 */
    int64_t free_pages;      /* pages not held by any adapter      */
    int32_t loaded_entries;  /* (slot, module) entries loaded      */
    int32_t loaded_slots;    /* slots with at least one entry      */
    int64_t loads;           /* successful lora_pool_load calls    */
    int64_t evicts;          /* successful lora_pool_evict calls   */
} lora_pool_stats_t;

/* Creates a pool on HIP device `device`.
 *   wdtype      element type of pages (LORA_F32 or LORA_BF16); x uses the same type
 *   page_elems  elements per page; a multiple of 64
 *   n_pages     pages to allocate (n_pages * page_elems elements of device memory)
 *   n_slots     adapter slots (ids 0..n_slots-1), 1..8192
 *   n_modules   adapted linear layers per slot, >= 1
 *   h_in,h_out  [host] [n_modules] input/output widths; multiples of page_elems
 *   max_rank    rank cap, 1..LORA_MAX_RANK
 * On success *out holds the pool.  Synchronous.  Errors: ARG, SHAPE, RANK, HIP. */
lora_status lora_pool_create(lora_pool **out, int32_t device, lora_dtype wdtype,
                             int64_t page_elems, int64_t n_pages, int32_t n_slots,
                             int32_t n_modules, const int64_t *h_in, const int64_t *h_out,
                             int32_t max_rank);

/* Frees the pool's device memory after synchronizing its device.  NULL is OK. */
lora_status lora_pool_destroy(lora_pool *p);

/* Copies one adapter into freshly allocated pages and publishes the
 * (slot, module) entry (the hot-swap strategy of the study page, section
 * "Strategies compared": an adapter's weights are copied into a GPU slot;
 * "Thousands of adapters", slide 9: the copy overlaps the GPU's work).  A and
 * B are [rank][h_in] and [rank][h_out] of the pool's dtype, in host or device
 * memory.  The call returns before the upload completes: A and B in host
 * memory are copied into a page-locked staging buffer before it returns (so
 * they may be reused at once); A and B in device memory are read on `stream`
 * in stream order.  Kernels enqueued later on `stream` see the entry.  Up to
 * 4 uploads are in flight per pool; a fifth call waits for the oldest.
 * Errors: ARG (null), SLOT (range / already loaded), RANK, NO_PAGES, HIP. */
lora_status lora_pool_load(lora_pool *p, int32_t slot, int32_t module, int32_t rank,
                           const void *A, const void *B, float scale, void *stream);

/* Unloads every module of `slot`: the slot's entries read as empty for work
 * enqueued on `stream` after this call, and its pages return to the free list.
 * The pages may be reused by the next load; a load on the same stream is
 * ordered after earlier kernels, so reuse is safe in stream order.  Callers
 * that read the pool from other streams order those streams themselves.
 * Errors: ARG, SLOT (range or nothing loaded), HIP. */
lora_status lora_pool_evict(lora_pool *p, int32_t slot, void *stream);

/* [host] out: counters.  Synchronous, no device work. */
lora_status lora_pool_stats(const lora_pool *p, lora_pool_stats_t *out);

/* Debug read-back of one entry into [host] buffers (A: rank*h_in, B:
 * rank*h_out elements of the pool's dtype, either may be NULL) and its
 * [host] page list (up to max_pages ids, either may be NULL).  Synchronizes
 * the device.  Errors: ARG, SLOT (empty), HIP. */
lora_status lora_pool_read(const lora_pool *p, int32_t slot, int32_t module,
                           int32_t *rank, float *scale, void *A, void *B,
                           int32_t *pages, int32_t max_pages);

/* ------------------------------------------------------------------------ */
/* Segments: tokens grouped by adapter                                      */
/* (the Fastino article's kernel sorts a batch by adapter; the study page's */
/* SGMV runs over runs of tokens with one adapter, "The kernel trick")      */
/* ------------------------------------------------------------------------ */
#define LORA_META_WORDS 16
enum {
    LORA_META_N_SEG = 0,        /* distinct adapters in the batch                       */
    LORA_META_N_ACTIVE = 1,     /* tokens with a valid id                               */
    LORA_META_MAX_SEG_LEN = 2,  /* tokens in the longest segment                        */
    LORA_META_N_BAD = 3,        /* ids outside [-1, n_slots)                            */
    LORA_META_N_UNITS_SHORT = 4,/* GEMV work units of segments shorter than LONG_MIN    */
    LORA_META_N_UNITS_ALL = 5,  /* GEMV work units of all segments                      */
    LORA_META_N_TILES = 6,      /* matrix-core tiles of segments of >= LONG_MIN tokens  */
    LORA_META_UNIT_TOKENS = 7,  /* tokens per GEMV unit                                 */
    LORA_META_TILE_TOKENS = 8,  /* tokens per matrix-core tile                          */
    LORA_META_LONG_MIN = 9,     /* segment length from which tiles are used             */
    LORA_META_N_TOKENS = 10,
    LORA_META_N_SLOTS = 11
};

/* Views into one caller-owned device buffer (see lora_segments_bind). */
typedef struct {
    int32_t *perm;       /* [n_tokens] token indices: ascending slot, original order within a slot */
    int32_t *seg_start;  /* [max_segs + 1] offsets into perm; seg_start[n_seg] = n_active          */
    int32_t *seg_slot;   /* [max_segs] slot of each segment, ascending                             */
    int32_t *meta;       /* [LORA_META_WORDS]                                                      */
    int32_t *units;      /* [2 * max_units] GEMV units: (slot + 65536 * tokens + 2^24 * [segment  */
                         /* spans several units], position in perm)                               */
    int32_t *tiles;      /* [2 * max_tiles] matrix-core tiles: (slot + 65536 * tokens, position)    */
    int32_t *work;       /* builder scratch of large batches (n_chunks > 0), else NULL             */
    int32_t n_tokens, n_slots, max_segs, max_units, max_tiles;
    int32_t n_chunks;    /* 0: one-workgroup build; else the large-batch build's token chunks      */
} lora_segments;

/* Bytes of device memory lora_segments_bind needs for a batch. */
size_t lora_segments_bytes(int32_t n_tokens, int32_t n_slots);

/* [host] Lays out the views over `buf` (device, >= lora_segments_bytes bytes,
 * 256-byte aligned).  No device work.  Errors: ARG, WORKSPACE. */
lora_status lora_segments_bind(void *buf, size_t bytes, int32_t n_tokens, int32_t n_slots,
                               lora_segments *out);

/* Builds the segments of the batch `ids` [n_tokens] (int32, device) on the
 * GPU: a stable sort of token indices by slot that drops ids outside
 * [0, n_slots), the segment offsets and slots, and the work lists of the
 * apply kernels.  Built once per batch and reused by every layer and module.
 * One launch; n_tokens == 0 enqueues nothing.  Errors: ARG, HIP. */
lora_status lora_build_segments(const int32_t *ids, const lora_segments *seg, void *stream);

/* Debug: waits for `stream`, copies the meta words to [host] meta_out (may be
 * NULL) and returns LORA_ERR_DEVICE_IDS if the batch held invalid ids. */
lora_status lora_segments_check(const lora_segments *seg, void *stream, int32_t *meta_out);

/* ------------------------------------------------------------------------ */
/* Apply                                                                    */
/* ------------------------------------------------------------------------ */
/* Shared arguments:
 *   module0, n_modules   consecutive modules [module0, module0+n_modules), all
 *                        with the same h_in (and h_out for expand/bgmv)
 *   module_stride_*      element offset between modules' x / t / y; a stride of
 *                        0 for x means the modules share one x (q, k, v)
 *   seg                  segments built for this batch (n_tokens = seg->n_tokens)
 * x and the pool have the same dtype.  y may be LORA_F32 or LORA_BF16; each y
 * element is rounded once, to nearest even, after y0 + term is formed in fp32.
 * Pointers and leading dimensions must keep every row 16-byte aligned. */

/* Workspace bytes that let lora_shrink split its matrix-core contraction over
 * K as far as it ever does (partial tiles of the splits).  Any smaller size,
 * including 0, is accepted and limits the split. */
size_t lora_shrink_workspace_bytes(const lora_pool *p, int32_t n_tokens, int32_t n_modules);

/* Shrink: t[i][j] = sum_k x_i[k] A_a[j][k] for j < rank_a, i with a valid id
 * ("shrink" of the study page's demo: the per-row product with the gathered
 * A).  t rows of tokens without an adapter, and columns past rank_a, are not
 * written.  Segments of >= LONG_MIN tokens run on bf16 matrix cores.
 * ws: optional device workspace (16-byte aligned, no initialization needed)
 * for splitting the matrix-core contraction over K when there are too few
 * tiles to fill the GPU; with ws_bytes == 0 no split is made.  Calls that
 * share a workspace must be ordered on one stream.
 * t must be 16-byte aligned, with ld_t and module_stride_t multiples of 4.
 * On bf16 pools the call is one launch (plus one for the K splits) that
 * runs long segments on matrix-core tiles and short ones on the GEMV path.
 * Errors: ARG, SHAPE (also: a batch whose launch would exceed 2^31 - 1
 * workgroups; nothing is launched), DTYPE, HIP. */
lora_status lora_shrink(const lora_pool *p, int32_t module0, int32_t n_modules,
                        const void *x, int64_t ld_x, int64_t module_stride_x,
                        const lora_segments *seg,
                        float *t, int64_t ld_t, int64_t module_stride_t,
                        void *ws, size_t ws_bytes, void *stream);

/* lora_shrink for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, serving loops that forbid
 * allocation).  Same arguments and result as lora_shrink with a workspace of
 * lora_shrink_workspace_bytes (the same K split, so the same t bit for bit),
 * but the split's partial tiles go to a device array that the library holds,
 * LORA_NOALLOC_SCRATCH_BYTES per GPU, until the process ends.  Nothing is
 * allocated by the call.
 * Every call on one GPU uses that GPU's array: calls that overlap on one GPU
 * (other streams, other host threads) race and must be ordered by the caller.
 * The array keeps the last call's contents; the call reads only what it wrote.
 * Errors: as lora_shrink, and WORKSPACE when that split needs more than
 * LORA_NOALLOC_SCRATCH_BYTES (nothing is launched; lora_shrink with a
 * workspace serves such calls); HIP when the array's address cannot be had. */
#define LORA_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)
lora_status lora_shrink_noalloc(const lora_pool *p, int32_t module0, int32_t n_modules,
                                const void *x, int64_t ld_x, int64_t module_stride_x,
                                const lora_segments *seg,
                                float *t, int64_t ld_t, int64_t module_stride_t, void *stream);

/* Expand: y_i[c] = round(y_i[c] + scale_a * sum_{j<rank_a} t[i][j] B_a[j][c])
 * for tokens with a valid id ("expand" of the study page's demo, fused into
 * the update of y).  Other rows of y are not touched.
 * On bf16 pools the call is one launch that runs long segments on
 * matrix-core tiles and short ones on the GEMV path.
 * Errors: ARG, SHAPE (also: a batch whose launch would exceed 2^31 - 1
 * workgroups; nothing is launched), DTYPE, HIP. */
lora_status lora_expand(const lora_pool *p, int32_t module0, int32_t n_modules,
                        const float *t, int64_t ld_t, int64_t module_stride_t,
                        const lora_segments *seg,
                        void *y, int64_t ld_y, int64_t module_stride_y, lora_dtype ydtype,
                        void *stream);

/* SGMV: lora_shrink then lora_expand on the same t and workspace, with one
 * difference: when the shrink splits its matrix-core contraction over K, the
 * expand adds the splits' partial tiles itself, in split order as
 * lora_shrink's own sum does, and the launch that would sum them is not
 * made: two launches in place of three ("Thousands of adapters", slide 11:
 * one SGMV call for a mixed batch).  y is the same bit for bit as with the
 * two calls.  t is scratch here: rows of tokens in matrix-core tiles are
 * left unwritten when K is split.  Modules share h_in and h_out; argument
 * rules are those of both calls; the workspace must not be in use by another
 * call in flight.  One call per step pays most: where a step's modules need
 * several calls (q, k, v sharing x beside o), lora_shrink per x and one
 * lora_expand over all of them make fewer, larger launches.
 * Errors: ARG, SHAPE, DTYPE, HIP (nothing is launched on an argument error). */
lora_status lora_apply_sgmv(const lora_pool *p, int32_t module0, int32_t n_modules,
                            const void *x, int64_t ld_x, int64_t module_stride_x,
                            const lora_segments *seg,
                            float *t, int64_t ld_t, int64_t module_stride_t,
                            void *y, int64_t ld_y, int64_t module_stride_y, lora_dtype ydtype,
                            void *ws, size_t ws_bytes, void *stream);

/* One x run of lora_apply_sgmv_multi: n_modules consecutive modules whose x
 * is [n_tokens][ld_x] each, module_stride_x elements apart (0: they share it,
 * as q, k, v do). */
typedef struct {
    const void *x;
    int64_t ld_x;
    int64_t module_stride_x;
    int32_t n_modules;
} lora_x_run;

/* lora_apply_sgmv for modules of one shape whose x comes in several runs (a
 * layer's q, k, v sharing x beside o with its own): one shrink launch per run,
 * all with the same K split, their partial tiles in one layout over the
 * call's modules, then one expand launch over every module that adds them.
 * On bf16 pools two runs (q,k,v beside o) share one shrink launch, and each
 * then aims at half the workgroups lora_shrink aims at, so it may split K
 * fewer ways.  runs[0..n_runs) cover module0 .. module0 + n_modules - 1 in
 * order.  Same result as lora_shrink per run then one lora_expand, bit for
 * bit when those calls take the same split (each run takes the smallest
 * split any run chooses; a smaller workspace limits lora_shrink's split, so
 * with unequal splits t's summation order differs).  The workspace is
 * lora_shrink_workspace_bytes(p, n_tokens, n_modules).  Other rules as
 * lora_apply_sgmv.  Errors: ARG (also: runs that do not cover the modules),
 * SHAPE, DTYPE, HIP; nothing is launched on an argument error. */
lora_status lora_apply_sgmv_multi(const lora_pool *p, int32_t module0, int32_t n_modules,
                                  const lora_x_run *runs, int32_t n_runs, const lora_segments *seg,
                                  float *t, int64_t ld_t, int64_t module_stride_t,
                                  void *y, int64_t ld_y, int64_t module_stride_y, lora_dtype ydtype,
                                  void *ws, size_t ws_bytes, void *stream);

/* Fused BGMV for decode (study page, "The kernel trick": a batched gather
 * matrix-vector product in which each decode token may bring its own
 * adapter): shrink and expand in one
 * launch with t kept on chip; tokens that share an adapter share each read
 * of its pages.  Same result as lora_shrink followed by lora_expand.
 * Errors: ARG, SHAPE, DTYPE, HIP. */
lora_status lora_apply_bgmv(const lora_pool *p, int32_t module0, int32_t n_modules,
                            const void *x, int64_t ld_x, int64_t module_stride_x,
                            const lora_segments *seg,
                            void *y, int64_t ld_y, int64_t module_stride_y, lora_dtype ydtype,
                            void *stream);

/* lora_apply_bgmv straight from the batch's adapter ids, for decode batches
 * of at most LORA_IDS_MAX_TOKENS tokens (study page, "The kernel trick": each
 * decode token brings its own adapter index, and the kernel gathers by it).
 * ids: device int32 [n_tokens], the pool slot of each token; -1 (and any id
 * outside [0, n_slots of the pool)) leaves the token's y rows untouched and is
 * not reported (lora_build_segments + lora_segments_check report bad ids).
 * Every workgroup of the launch builds the batch's unit list in its own LDS,
 * with the same lists lora_build_segments writes, so the step needs no segment
 * build launch and no lora_segments buffer.  Same y as lora_build_segments over
 * the pool's slots followed by lora_apply_bgmv, bit for bit.  x, y and their
 * strides as lora_apply_bgmv.  Errors: ARG, SHAPE (also: n_tokens >
 * LORA_IDS_MAX_TOKENS), DTYPE, HIP; nothing is launched on an error. */
#define LORA_IDS_MAX_TOKENS 64
lora_status lora_apply_bgmv_ids(const lora_pool *p, int32_t module0, int32_t n_modules,
                                const void *x, int64_t ld_x, int64_t module_stride_x,
                                const int32_t *ids, int32_t n_tokens,
                                void *y, int64_t ld_y, int64_t module_stride_y, lora_dtype ydtype,
                                void *stream);

/* lora_apply_bgmv for 2..4 modules that share one x (the q, k, v projections
 * of a layer: "Thousands of adapters", slide 5), taken together: one work
 * item per unit stages the unit's x rows once, shrinks the modules' rank rows
 * as one stacked block, then expands each module's y from its own t columns.
 * Same result as lora_apply_bgmv with module_stride_x = 0 (bit for bit when
 * every rank is a multiple of 8, or on exact inputs).  It saves x reads and
 * per-unit setup but makes each work item as long as all its modules
 * together: it pays only when a launch's units fill the GPU many times over;
 * a decode batch of 64 tokens on q, k, v of 4096 x 4096 takes longer than
 * lora_apply_bgmv's one work item per (unit, module).
 * Requires n_modules * max_rank <= LORA_MAX_RANK and the modules' page ids of
 * one adapter, n_modules * max_rank * (h_in + h_out) / page_elems, <= 1024.
 * Errors: ARG, SHAPE (also: the modules do not fit one work item), DTYPE, HIP. */
lora_status lora_apply_bgmv_packed(const lora_pool *p, int32_t module0, int32_t n_modules,
                                   const void *x, int64_t ld_x, const lora_segments *seg,
                                   void *y, int64_t ld_y, int64_t module_stride_y, lora_dtype ydtype,
                                   void *stream);

/* Base product and adapter term in one matrix-core pass, for batches whose
 * tokens come in runs of one adapter, such as prefills (study page, "The
 * kernel trick: gather, do not merge": one shared base matmul plus each
 * token's low-rank update, whose cost is about 2r/d of the base):
 *   y_i[c] = round(sum_k x_i[k] W[k][c] + scale_a * sum_{j<rank_a} t_i[j] B_a[j][c]),
 *   t_i[j] = sum_k x_i[k] A_a[j][k],
 * with a = ids[i]; a token whose id is -1, outside [0, n_slots) or of an
 * empty slot gets x_i W alone.  Unlike the other apply calls, y is written,
 * not added to: the call computes the base product itself.
 *   module: pool module whose adapters apply; h_in, h_out are its widths.
 *   x [n_tokens][ld_x] bf16, 16-byte aligned rows.
 *   w [h_out][ld_w] bf16: W transposed, row c holds the weights of output
 *     column c (the row-major layout of a linear layer's weight), 16-byte
 *     aligned rows.
 *   ids [n_tokens] int32 per-token slot ids, or NULL for x W alone.  Ids are
 *     read in token order; no segment build is needed.
 *   y [n_tokens][ld_y] bf16, 8-byte aligned rows; written for every token.
 * Tiles of 256 tokens x 256 columns run on bf16 MFMA with fp32
 * accumulation; each element of y is rounded once.  The adapter part of a
 * tile costs about 16/256 of its base part per 16 rank rows of each
 * distinct adapter among its 256 tokens, so batches whose tiles mix many
 * adapters (decode) belong on lora_apply_bgmv after a plain GEMM.
 * The pool must be bf16 and h_in / page_elems at most 32.
 * Errors: ARG (null pointer, bad module, n_tokens < 0, a leading dimension
 * below the width, misalignment), DTYPE (pool not bf16), SHAPE, HIP. */
lora_status lora_fused_gemm(const lora_pool *p, int32_t module,
                            const void *x, int64_t ld_x, const void *w, int64_t ld_w,
                            const int32_t *ids, int32_t n_tokens,
                            void *y, int64_t ld_y, void *stream);

/* lora_fused_gemm with an FP8 base (study page, section "Operating it": a
 * quantized base serves under the bf16 adapters; its design scenario takes
 * the base in FP8).  W is given as OCP FP8 E4M3 codes (1 sign, 4 exponent
 * bits with bias 7, 3 mantissa bits; exponent 0 holds the subnormals m * 2^-9;
 * 0x7F and 0xFF are NaN; largest finite 448) with one float32 scale per output
 * column:
 *   y_i[c] = round(w_scale[c] * sum_k x_i[k] E(w8[c][k]) + scale_a * sum_{j<rank_a} t_i[j] B_a[j][c]),
 * E the exact value of a code.  x, ids, the adapters and y are as for
 * lora_fused_gemm (bf16 activations and adapters: W8A16).  Each code is
 * widened to bf16, which holds every E4M3 value exactly, so the matrix-core
 * products are exact; the sum is fp32, then multiplied by the column scale.
 *   w8 [h_out][ld_w] bytes: row c holds the codes of output column c; 16-byte
 *     aligned, ld_w a multiple of 16.
 *   w_scale [h_out] float32, 16-byte aligned.
 * Errors: as lora_fused_gemm. */
lora_status lora_fused_gemm_fp8w(const lora_pool *p, int32_t module,
                                 const void *x, int64_t ld_x, const void *w8, int64_t ld_w,
                                 const float *w_scale, const int32_t *ids, int32_t n_tokens,
                                 void *y, int64_t ld_y, void *stream);

/* ---- Adapter tiers: GPU slots <- host memory <- cold store ----------------
 * Study page "Multi-LoRA Serving", section "Memory: slots, tiers and paging"
 * and its cache simulation: the engine keeps a fixed number of adapters in
 * GPU slots, a larger least-recently-used set in host memory (a swap is then
 * a PCIe copy, not a download), and loads the rest from a cold store.
 * Policy per request for adapter id a (a >= 0; adapter ids are the caller's,
 * slot ids are the pool's):
 *   GPU tier, least recently used order: a hit refreshes a; a miss gives a
 *   the lowest free slot, else the slot of the least recently used adapter,
 *   which leaves the GPU tier;
 *   host tier, consulted only on a GPU miss, same rule: a hit is a host copy
 *   (LORA_TIER_HOST), a miss a cold load (LORA_TIER_COLD).
 * The state is host-side and not thread-safe: one caller at a time. */
typedef struct lora_tiers lora_tiers;   /* opaque, library-owned */
enum { LORA_TIER_GPU = 0, LORA_TIER_HOST = 1, LORA_TIER_COLD = 2 };

/* Cold store callback: writes adapter `adapter`'s rows for `module` into A
 * ([*rank][h_in], room for max_rank rows) and B ([*rank][h_out]) in the
 * pool's dtype, and sets *rank (0 = no adapter for this module) and *scale.
 * Returns 0 on success; anything else fails the acquire with LORA_ERR_ARG. */
typedef int32_t (*lora_fetch_fn)(void *ctx, int32_t adapter, int32_t module, int32_t *rank, float *scale,
                                 void *A, void *B);

/* gpu_slots >= 1 (the pool's n_slots when used with lora_tiers_acquire),
 * host_slots >= 0.  Errors: ARG. */
lora_status lora_tiers_create(lora_tiers **out, int32_t gpu_slots, int32_t host_slots);
/* Frees the tiers and their host buffers.  Waits for nothing: no upload from
 * them may be pending (synchronize the acquire streams first). */
lora_status lora_tiers_destroy(lora_tiers *t);
/* Policy only: n requests in order.  [host] out arrays, each optional:
 * tier[i], slot[i] (GPU slot after the request), evicted[i] (adapter that
 * left the GPU tier, -1 none).  Errors: ARG (negative id). */
lora_status lora_tiers_touch(lora_tiers *t, const int32_t *ids, int32_t n,
                             int32_t *tier, int32_t *slot, int32_t *evicted);
/* [host] counts since creation. */
lora_status lora_tiers_stats(const lora_tiers *t, int64_t *gpu_hits, int64_t *host_hits, int64_t *cold_loads);
/* [host] *slot = GPU slot of adapter id, -1 if not resident. */
lora_status lora_tiers_slot_of(const lora_tiers *t, int32_t id, int32_t *slot);
/* The policy driving a pool for one batch of n requests ([host] ids, [host]
 * slots out, the slot id to give the apply kernels for each request).  For
 * each GPU miss: the displaced adapter is evicted from the slot and the new
 * adapter's A and B rows of every module are uploaded to it on `stream`,
 * asynchronously, straight from page-locked host buffers that the tiers own
 * (allocated on the first acquire: host_slots x all modules at max_rank);
 * a cold load first calls fetch to fill the buffer.  Kernels of the batch go
 * on the same stream after the call.  All modules of a slot change together.
 * Errors: ARG (bad id, no host tier, another pool), SLOT (more distinct
 * adapters in the batch than slots), RANK, NO_PAGES, HIP; after an error the
 * tiers may disagree with the pool: destroy both. */
lora_status lora_tiers_acquire(lora_tiers *t, lora_pool *p, const int32_t *ids, int32_t n,
                               lora_fetch_fn fetch, void *ctx, int32_t *slots, void *stream);
/* Marks the end of the kernels of the batch last acquired: call it after
 * enqueueing them on `stream`.  Prefetches wait for the batch before it. */
lora_status lora_tiers_batch_done(lora_tiers *t, void *stream);
/* Forecast ("Thousands of adapters", slide 9: a forecast from the waiting
 * queue and an asynchronous copy): uploads, on copy_stream, the adapters of
 * [host] ids that are not resident, in order, as long as a slot can be
 * freed without displacing an adapter of the batch in flight (the last
 * acquire).  copy_stream first waits for the kernels of the batch before
 * the one in flight (the second-latest lora_tiers_batch_done).  The next
 * acquire makes its stream wait for these uploads, and finds the adapters
 * resident.  Prefetches are not requests: the hit counters do not change.
 * [host] *issued = adapters uploaded (optional).
 * Errors: as lora_tiers_acquire. */
lora_status lora_tiers_prefetch(lora_tiers *t, lora_pool *p, const int32_t *ids, int32_t n,
                                lora_fetch_fn fetch, void *ctx, void *copy_stream, int32_t *issued);

#ifdef __cplusplus
}
#endif
#endif /* LORA_MI355X_H */
