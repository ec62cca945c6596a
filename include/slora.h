/*
 * slora.h - C ABI of the paged, heterogeneous-batch LoRA delta on MI355X.
 *
 * The operation (S-LoRA pages): with the base forward h = xW, LoRA adds the
 * product of two thin factors, A (d_in x r) and B (r x d_out), and a server of
 * many adapters keeps that delta separate, computing x A B on the fly for each
 * request's own adapter (summary page "S-LoRA: Serving Thousands of
 * Concurrent LoRA Adapters", sections "What this paper explains", "The
 * mechanism" and "How to read the paper" item 2).  Every token t of a batch
 * names an adapter a with rank r_a and scale s_a and receives
 *
 *     y[t, :] += s_a * (x[t, :] A_a) B_a                      (fp32 accumulate)
 *
 * (blog page "Multiplexing Thousands of Fine-Tuned Adapters", section 2
 * pseudocode: the per-token delta times a scaling factor added to the base
 * output).  A_a and B_a live as non-contiguous pages of one pool shared with
 * KV blocks and found through a block table (summary page, "Unified Paging";
 * blog page section 2; catalog page, mechanism paragraph).  A page here is one
 * row: an adapter of rank r holds, per projection, r pages with the rows of
 * A^T (row j is column j of A) and r pages with the rows of B.
 *
 * Conventions shared by every entry point:
 *  - Every call returns an slora_status; no C++ exception crosses the ABI.
 *    On failure nothing changes (all-or-nothing) and slora_last_error()
 *    returns a message for the calling thread.
 *  - Device memory is owned by the caller: pool classes, x, y, the metadata
 *    buffer and the workspace.  The library never frees it and a pool must not
 *    outlive it.  Host arrays are only borrowed for the duration of a call.
 *    Opaque objects belong to the library and are released by *_destroy.
 *  - Streams are hipStream_t values passed as void* (NULL = default stream).
 *    The library uses the device that is current when the pool is created and
 *    makes it current again for its own HIP calls.
 *  - A pool and its segments are not thread-safe; callers serialise.
 *  - Page offsets are 64-bit: page_id * page_bytes may exceed 4 GiB.
 */
#ifndef SLORA_H
#define SLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct slora_pool slora_pool;
typedef struct slora_segments slora_segments;

typedef enum {
  SLORA_OK = 0,
  SLORA_E_INVAL = -1,  /* bad argument (NULL pointer, size, rank, dtype, layout) */
  SLORA_E_NOMEM = -2,  /* not enough free pages, or a host/device buffer too small */
  SLORA_E_EXIST = -3,  /* adapter id already loaded */
  SLORA_E_NOENT = -4,  /* adapter id not loaded */
  SLORA_E_STALE = -5,  /* segments built against an adapter since unloaded/reloaded */
  SLORA_E_HIP = -6     /* a HIP runtime call failed; the message names it */
} slora_status;

typedef enum { SLORA_F32 = 0, SLORA_F16 = 1 } slora_dtype;

/* Pool description.  With n_classes == 1 every page (A^T rows, B rows and KV
 * blocks) holds h_in elements and h_in must equal h_out.  With n_classes == 2,
 * class 0 pages hold h_in elements (A^T rows, KV) and class 1 pages hold h_out
 * elements (B rows, KV).  class_base[c] is caller-owned device memory of
 * n_pages[c] * page_elems * sizeof(dtype) bytes, 16-byte aligned.
 * free_order[c] (host, borrowed) is the order in which the free list hands out
 * pages: a permutation of [0, n_pages[c]); NULL means ascending ids.
 * h_in and h_out must be multiples of 8; max_rank is at most 256. */
typedef struct {
  int32_t dtype;        /* slora_dtype of pages, x and y */
  int32_t h_in;         /* d_in: elements of x rows and of A^T rows */
  int32_t h_out;        /* d_out: elements of y rows and of B rows */
  int32_t n_proj;       /* projections per adapter sharing one token->adapter map (1..8) */
  int32_t max_adapters; /* adapter ids are 0 .. max_adapters-1 */
  int32_t max_rank;     /* largest rank accepted by slora_load_adapter */
  int32_t n_classes;    /* 1 or 2, see above */
  int32_t reserved0;    /* must be 0 */
  int64_t n_pages[2];
  void* class_base[2];
  const int32_t* free_order[2];
} slora_pool_desc;

/* Create a pool over caller-owned page memory: one allocator and block table
 * for adapter factors of every rank and for KV blocks (summary page, "Unified
 * Paging": a unified memory pool manages adapter weights and KV cache
 * together; blog page, section 2: adapter weights sit in non-contiguous
 * memory blocks).  Host-only: no device memory is touched until the first
 * adapter load with data. */
slora_status slora_pool_create(const slora_pool_desc* desc, slora_pool** out);
void slora_pool_destroy(slora_pool* pool);

/* Tuning knobs of the tile builder (applied by later slora_build_segments):
 *  SLORA_TUNE_MFMA_MIN_TOKENS  - fp16 segments with at least this many tokens
 *                                (and rank at most SLORA_MFMA_MAX_RANK, h_in
 *                                a multiple of 64, n_tokens x h_out x 2
 *                                below 4 GiB) use the matrix-core (MFMA)
 *                                tiles; default 64.
 *  SLORA_TUNE_GEMV_EXPAND_ELEMS- target rank x columns of one vector-ALU
 *                                expand tile; 0 (default): chosen from the
 *                                batch (16K to 256K, growing with the
 *                                batch's vector-ALU expand work, counted
 *                                over all projections when the batch has
 *                                matrix-core tiles or tiles too deep for
 *                                one register set).
 *  SLORA_TUNE_MFMA_EXPAND_COLS - columns of one MFMA expand tile, a multiple
 *                                of 128; 0 (default): 512 when every segment
 *                                of the batch takes the MFMA tiles, else 1024.
 *  SLORA_TUNE_MFMA_SHRINK_SPLITS - K splits of each 64-token MFMA shrink
 *                                block, 1..4; 0 (default): enough for about
 *                                512 shrink tiles.
 *  SLORA_TUNE_FUSED            - 1 (default): slora_lora_delta runs both
 *                                stages in one launch, each expand tile
 *                                waiting for its tokens' x A values;
 *                                0: two launches (shrink, then expand).
 *  SLORA_TUNE_XCDS             - n > 1: the shrink tiles of each token block
 *                                go to one of n XCDs (workgroup i runs on
 *                                XCD i mod n); 1 (default): no grouping.
 *  SLORA_TUNE_TILE_ORDER       - 0: tiles of each stage in segment (adapter
 *                                id) order; 1: clustered by rank, highest
 *                                first (summary page, "Heterogeneous batching
 *                                kernels": clustering of ranks); 2 (default):
 *                                the tiles that move the most bytes first.
 *  SLORA_TUNE_FWD_GROUP        - slora_lora_forward's tile order: tiles
 *                                go row block by row block in groups of n
 *                                row blocks, column by column inside a
 *                                group (1: row-block major); 0 (default):
 *                                groups of 8 for the 32- and 64-row tiles
 *                                and the 256-column ones, row-block major
 *                                for 128 x 128.
 *  SLORA_TUNE_FWD_TILE         - slora_lora_forward's tile: 32 (32 x 128
 *                                everywhere), 64 (64 x 128 everywhere),
 *                                128 (128 x 128 everywhere), 256
 *                                (256 x 256 everywhere, when h_out is a
 *                                multiple of 256) or 0 (default): 256 x 256
 *                                for the leading positions that fill whole
 *                                rounds of 256 such tiles and 128 x 256 for
 *                                the rest; 128 x 128 when the batch is too
 *                                small for one round, 64 x 128 when it is too
 *                                small for 256 tiles of 128 x 128 or its LoRA
 *                                steps outnumber a tile's x W steps, 32 x 128
 *                                when it is too small for 256 tiles of
 *                                64 x 128.
 *  SLORA_TUNE_SHRINK_ROWS      - rank rows of one vector-ALU shrink tile, at
 *                                most 16 / (16-byte chunks of an x row per
 *                                thread); 0 (default): that maximum, and 8
 *                                for blocks of one token at four chunks a
 *                                thread (their x needs a quarter of the
 *                                registers).
 *  SLORA_TUNE_FWD_KSPLIT       - slora_lora_forward's 32- and 64-row tiles:
 *                                1 (one group of waves takes every step of
 *                                a tile) or 2 (two groups take alternate
 *                                steps into sums of their own, added before
 *                                the output is rounded); 0 (default): 2.
 *                                The larger tiles always take 1.
 * They change how the work is cut, never what is computed (only, in floating
 * point, the order in which partial sums meet). */
#define SLORA_MFMA_MAX_RANK 64
typedef enum {
  SLORA_TUNE_MFMA_MIN_TOKENS = 0,
  SLORA_TUNE_GEMV_EXPAND_ELEMS = 1,
  SLORA_TUNE_MFMA_EXPAND_COLS = 2,
  SLORA_TUNE_MFMA_SHRINK_SPLITS = 3,
  SLORA_TUNE_FUSED = 4,
  SLORA_TUNE_XCDS = 5,
  SLORA_TUNE_TILE_ORDER = 6,
  SLORA_TUNE_FWD_GROUP = 7,
  SLORA_TUNE_FWD_TILE = 8,
  SLORA_TUNE_SHRINK_ROWS = 9,
  SLORA_TUNE_FWD_KSPLIT = 10
} slora_tune_key;
slora_status slora_pool_set_tuning(slora_pool* pool, int32_t key, int64_t value);

/* Take n pages of class cls from the head of the free list for KV blocks
 * (summary page, walkthrough step 4: KV growth and adapters share one
 * allocator).  Writes the ids to out_ids (host, n entries). */
slora_status slora_alloc_pages(slora_pool* pool, int32_t cls, int64_t n, int32_t* out_ids);
/* Return KV pages to the tail of the free list, in the order given.  Only
 * pages handed out by slora_alloc_pages and not yet freed are accepted. */
slora_status slora_free_pages(slora_pool* pool, int32_t cls, int64_t n, const int32_t* ids);
/* Free pages of class cls, or -1 on a bad argument. */
int64_t slora_free_count(const slora_pool* pool, int32_t cls);

/* Make adapter `id` resident (summary page, "Host-resident adapter store" and
 * walkthrough step 2: adapters live in host memory and are fetched on demand).
 * Takes from the head of the free list, for each projection p in order, rank
 * pages for the A^T rows j = 0..rank-1 and then rank pages for the B rows (B
 * rows come from class 1 when the pool has two classes).  A and B are host
 * arrays of n_proj pointers: A[p] is h_in x rank row-major, B[p] is
 * rank x h_out row-major, both of the pool dtype.  The rows are packed into a
 * pinned staging image and fetched into the pages on `stream` as by
 * slora_load_adapters_async, and the call returns after the fetch has
 * completed, so A and B may be freed at once.  A == NULL and
 * B == NULL together reserve the pages and block-table entry without writing
 * them (the pages keep their previous content).  1 <= rank <= max_rank; scale
 * must be finite. */
slora_status slora_load_adapter(slora_pool* pool, int32_t id, int32_t rank, float scale,
                                const void* const* A, const void* const* B, void* stream);

/* Asynchronous adapter fetch (summary page, "Host-resident adapter store" and
 * walkthrough step 2: the next iteration's adapters are copied into the pool
 * while the current one computes).  An adapter image is the byte layout one load
 * moves to the device: the n_proj x rank A^T rows (h_in elements each,
 * projection-major), then the n_proj x rank B rows (h_out elements), then
 * 2 x n_proj x rank int32 page ids that the load writes; padded to 256 bytes.
 * slora_adapter_image_bytes returns its size for `rank` (0 on a bad pool or
 * rank). */
size_t slora_adapter_image_bytes(const slora_pool* pool, int32_t rank);
/* Fill an image (host, image_bytes >= slora_adapter_image_bytes(rank)) from
 * A and B laid out as for slora_load_adapter: A^T rows are A's columns.  Host
 * only, no device call; done once when an adapter enters the host store, so
 * that a later fetch is one copy. */
slora_status slora_pack_adapter(const slora_pool* pool, int32_t rank, const void* const* A,
                                const void* const* B, void* image, size_t image_bytes);
/* Fetch n adapters at once.  For k = 0..n-1 in order, take pages for adapter
 * ids[k] (rank ranks[k], scale scales[k]) exactly as slora_load_adapter would
 * (same free-list order) and write their ids into images[k]; then queue on
 * `stream` one host-to-device copy per image into dev_stage (image k at the
 * sum of the earlier images' slora_adapter_image_bytes), all copies first so
 * the copy engine runs them back to back, and then one kernel launch per 64
 * adapters that moves every row into its page; return without waiting.  The
 * copies run on a copy engine, not on the compute units, so a delta running
 * meanwhile loses little.  images[k] is an image packed by slora_pack_adapter
 * for ranks[k], in pinned host memory (hipHostMalloc, or a pinned torch
 * tensor); dev_stage is device memory of the pool's device of dev_stage_bytes
 * >= the images' total size.  Every argument is checked first (bad id, rank or
 * scale, an id twice, an unpinned image, a dev_stage too small or not on the
 * device: SLORA_E_INVAL; an id already loaded: SLORA_E_EXIST; too few free
 * pages for the whole batch: SLORA_E_NOMEM) and a failure takes no page.
 * Ownership stays with the caller; neither the images nor dev_stage may be
 * written, reused or freed until `stream` has passed this call.  The adapters
 * count as loaded at once (segments may be built against them), but their
 * pages hold the rows only once `stream` has passed the call: a
 * slora_lora_delta that reads them must be queued after it on the same stream
 * or wait for an event recorded there.  Likewise, unloading an adapter whose
 * pages a queued delta still reads and fetching another into them races unless
 * the fetch's stream waits for the delta.  A failed queue call returns
 * SLORA_E_HIP with every page given back, after waiting on `stream` for the
 * copies and scatters it had already queued (none of them still writes a
 * page it gave back); device faults surface at the caller's
 * synchronisation.  n == 0 does nothing. */
slora_status slora_load_adapters_async(slora_pool* pool, int32_t n, const int32_t* ids,
                                       const int32_t* ranks, const float* scales, void* const* images,
                                       void* dev_stage, size_t dev_stage_bytes, void* stream);
/* Drop adapter `id` from the pool (summary page, walkthrough step 4: unused
 * adapters leave GPU memory).  Its pages go to the tail of the free list in the
 * order they were taken.  Segments built against it become stale. */
slora_status slora_unload_adapter(slora_pool* pool, int32_t id);
/* Page ids of adapter `id`, projection `proj`: rank A^T pages to a_ids and
 * rank B pages to b_ids (host arrays; either may be NULL).  *rank_out
 * (may be NULL) receives the rank. */
slora_status slora_adapter_pages(const slora_pool* pool, int32_t id, int32_t proj,
                                 int32_t* a_ids, int32_t* b_ids, int32_t* rank_out);

/* Group a batch by adapter (host only; summary page, "Heterogeneous batching
 * kernels": a batch mixes requests of different adapters and ranks, and the
 * kernels gather each request's adapter pages; blog page, section 3: each
 * request's hidden state is matched with its adapter's pages through the
 * paging table).  ids[t] (host, n_tokens entries) is
 * token t's adapter; a negative id means "no adapter" and leaves y[t]
 * untouched.  Tokens are stably sorted by adapter id into segments in
 * ascending id order, each with its rank, scale, rank prefix offset and page
 * lists, and the work is cut into tiles for the shrink (x A) and expand
 * (. B, scale, accumulate) kernels.  Every named adapter must be loaded. */
slora_status slora_build_segments(slora_pool* pool, int32_t n_tokens, const int32_t* ids,
                                  slora_segments** out);
void slora_segments_destroy(slora_segments* seg);

typedef struct {
  int32_t n_tokens;       /* batch size given to slora_build_segments */
  int32_t n_routed;       /* tokens with an adapter */
  int32_t n_segments;     /* distinct adapters in the batch */
  int32_t n_proj;
  int64_t sum_rank;       /* sum over segments of rank: page-list length per projection */
  int64_t sum_rank_tokens;/* sum over routed tokens of their adapter's rank */
  int32_t n_shrink_tiles;
  int32_t n_expand_tiles;
  int32_t n_mfma_segments;/* segments routed to the matrix-core (MFMA) tiles */
  int32_t n_combine_tiles;/* tiles summing the K-split partials of MFMA shrink blocks */
  size_t meta_bytes;      /* device metadata size for slora_segments_upload */
  size_t workspace_bytes; /* device workspace size for slora_lora_delta */
} slora_segments_info;

slora_status slora_segments_get_info(const slora_segments* seg, slora_segments_info* info);

/* Host copies of the segment metadata (the sorted batch and the page lists
 * of the block table that the kernels gather from, summary page "Unified
 * Paging"); any pointer may be NULL.  Sizes:
 * perm[n_routed] (batch index of the i-th sorted token), seg_start[S+1],
 * seg_adapter[S], seg_rank[S], seg_scale[S], seg_page_off[S+1] (prefix sum of
 * ranks), a_pages[n_proj*sum_rank] and b_pages[n_proj*sum_rank] (entry
 * p*sum_rank + seg_page_off[s] + j is row j of segment s, projection p). */
slora_status slora_segments_export(const slora_segments* seg, int32_t* perm, int32_t* seg_start,
                                   int32_t* seg_adapter, int32_t* seg_rank, float* seg_scale,
                                   int32_t* seg_page_off, int32_t* a_pages, int32_t* b_pages);

/* Introspection of the work split (host copies): layout[9] receives
 * {n_tiles, stride, tokcap, pagecap, n_shrink_tiles, n_expand_tiles, hdr,
 *  n_combine_tiles, n_splits} and, when records is not NULL and holds at
 * least n_tiles * stride words, the tile records in launch order (every
 * shrink tile, then every combine tile, then every expand tile), stride int32
 * words each.  Record words:
 * 0 kind (bit 0: matrix-core (MFMA) tile, bit 1: expand tile, bit 2: combine
 * tile), 1 token count, 2 segment rank, 3 first rank row (vector-ALU shrink),
 * first k (MFMA shrink) or first column (expand), 4 rows, k extent or columns
 * covered, 5 workspace offset of the first token's v row, 6 scale (float
 * bits), 7 expand thread-map width / K split of an MFMA shrink tile / splits
 * summed by a combine tile, 8 segment index, 9 K splits of an MFMA shrink
 * tile's token block; from word hdr, tokcap batch indices of the tokens, then
 * per projection pagecap page ids (vector-ALU shrink: the A^T pages of the
 * rows covered; MFMA shrink: all rank A^T pages; expand: all rank B pages).
 * MFMA shrink tiles split over K (n_splits > 1) write partial x A to
 * workspace area `split` (each area sum_rank_tokens values); a combine tile
 * sums the areas of its tokens into area 0.
 * For tests and tools; the layout may change. */
slora_status slora_segments_tiles(const slora_segments* seg, int32_t* layout, int32_t* records,
                                  size_t records_words);

/* Introspection of slora_lora_forward's tables (host copies): layout[8]
 * receives {n_rb, n_rb_big, big_rows, small_bm, n_stages, packed,
 * stage_words, n_proj}.  Sorted positions [0, big_rows) form n_rb_big row
 * blocks of 256 and the rest row blocks of small_bm (32, 64 or 128); rb_info
 * (2 x n_rb words) holds per row block its first LoRA stage and stage count;
 * stages (n_proj x n_stages x stage_words words, projection-major) the LoRA
 * stage entries: 32 B page ids, then, when packed, one word per group of 4
 * rows, segment << 9 | (first rank row / 4) << 3 | rows (0: empty group),
 * else the segment, first rank row and rank of the stage's one segment.
 * Either buffer may be NULL.  For tests and tools; the layout may change. */
slora_status slora_segments_forward_tables(const slora_segments* seg, int32_t* layout, int32_t* rb_info,
                                           size_t rb_words, int32_t* stages, size_t stage_words);

/* Copy the tile metadata (the batch's page lists and work split, summary page
 * "Heterogeneous batching kernels") to caller-owned device memory dev_meta (at least
 * meta_bytes, 16-byte aligned) on `stream` and remember that address for
 * later deltas.  The copy is asynchronous; dev_meta must stay untouched while
 * deltas that use it are in flight.  The metadata also holds the area where
 * a fused launch passes x A between its stages (the upload zeroes it on
 * `stream`), so every slora_lora_delta that uses one upload must be
 * ordered on one stream. */
slora_status slora_segments_upload(slora_segments* seg, void* dev_meta, size_t dev_meta_bytes,
                                   void* stream);

/* The hot path (summary page, "How to read the paper" item 2, h = xW + xAB,
 * with the delta xAB kept separate from the base product; blog page, section
 * 2: each token's product with its adapter's A and B, times the adapter's
 * scaling factor, added to the base output; summary page, "Heterogeneous
 * batching kernels": one launch for a batch of many adapters and ranks
 * gathering non-contiguous pages): y[t] += s_a * (x[t] A_a) B_a for every routed token, for
 * projection `proj` (0 <= proj < n_proj).  x is device memory of
 * n_tokens x h_in and y of n_tokens x h_out, both row-major in batch order
 * and of the pool dtype; y is updated in place with one rounding of
 * fp32(y) + s * d per element, where d is accumulated in fp32.  workspace is
 * device memory of at least workspace_bytes (fp32 x A products and their
 * K-split partials), 16-byte
 * aligned.  Launches the shrink and expand kernels on `stream` and returns
 * without waiting; launch errors return SLORA_E_HIP, device faults surface at
 * the caller's next synchronisation.  Requires a prior slora_segments_upload.
 * Returns SLORA_E_STALE if an adapter of the batch was unloaded since the
 * segments were built.  With no routed tokens it launches nothing. */
slora_status slora_lora_delta(slora_pool* pool, const slora_segments* seg, int32_t proj,
                              const void* x, void* y, void* workspace, size_t workspace_bytes,
                              void* stream);

/* slora_lora_delta with timing: the caller's HIP events (hipEvent_t as void*,
 * created with timing enabled; either may be NULL) are recorded by the kernel
 * dispatch itself, start when its first kernel begins and stop when its last
 * kernel ends, so hipEventElapsedTime gives the kernels' own duration without
 * the queue overhead of a separate hipEventRecord.  With no routed tokens
 * nothing is launched and the events are not recorded. */
slora_status slora_lora_delta_timed(slora_pool* pool, const slora_segments* seg, int32_t proj,
                                    const void* x, void* y, void* workspace, size_t workspace_bytes,
                                    void* stream, void* start_event, void* stop_event);

/* Several projections of one batch in one launch (summary page, "Algorithm /
 * figure walkthrough" step 3: each request's adapter is applied to the
 * layer's projections; catalog page, mechanism paragraph: custom kernels
 * batch the LoRA products of many adapters together).  For i = 0 .. n-1,
 * projection projs[i] (distinct, each 0 <= projs[i] < n_proj) reads xs[i] and
 * updates ys[i] exactly as slora_lora_delta(projs[i], xs[i], ys[i]) would, to
 * the bit: several projections may share one x (q, k and v of an attention
 * layer) and each has its own y.  The workspace holds n areas of
 * workspace_bytes (n x slora_segments_info.workspace_bytes in all).  With
 * SLORA_TUNE_FUSED (the default) the n projections run as one kernel launch
 * whose grid holds every projection's tiles, so one launch pays one ramp and
 * one tail instead of n; otherwise the projections run one after another as
 * staged launches.  1 <= n <= 8; errors and ordering as for
 * slora_lora_delta. */
slora_status slora_lora_delta_multi(slora_pool* pool, const slora_segments* seg, int32_t n,
                                    const int32_t* projs, const void* const* xs, void* const* ys,
                                    void* workspace, size_t workspace_bytes, void* stream);
/* slora_lora_delta_multi with dispatch-recorded HIP events, as for
 * slora_lora_delta_timed. */
slora_status slora_lora_delta_multi_timed(slora_pool* pool, const slora_segments* seg, int32_t n,
                                          const int32_t* projs, const void* const* xs, void* const* ys,
                                          void* workspace, size_t workspace_bytes, void* stream,
                                          void* start_event, void* stop_event);

/* Reads (synchronously, on `stream`) whether any fused launch since the last
 * upload gave up waiting for the x A values of its tokens: *flag = 1 if so,
 * which would mean its results are wrong; 0 otherwise.  A wait gives up only
 * after about 2^20 polls, so a healthy GPU never raises it. */
slora_status slora_segments_read_error(const slora_segments* seg, void* stream, int32_t* flag);

/* For tests of the epoch counter: fused launches tag the x A values they
 * exchange with an epoch that counts 1, 2, ... per launch since the upload
 * and, once it reaches 2^31 - 1, clear the exchange pairs on the stream and
 * start again at 1.  Moves the count of fused launches since the upload
 * forward to `launches` (from the current count up to 2^31 - 1; SLORA_E_INVAL
 * otherwise, nothing changed), so that the next launch takes epoch
 * launches + 1, or clears and takes 1.  Only forward: pairs left by earlier
 * launches then carry smaller epochs and can never match a later one. */
slora_status slora_segments_set_launch_count(slora_segments* seg, int64_t launches);

/* The two stages of slora_lora_delta, for callers that schedule or time them
 * apart: slora_lora_shrink writes v = x A (fp32) for every routed token into
 * the workspace; slora_lora_expand then applies y += s v B.  Same arguments,
 * checks and kernels as slora_lora_delta; expand must follow a shrink of the
 * same segments, projection and x on the same stream, with the workspace
 * untouched in between. */
slora_status slora_lora_shrink(slora_pool* pool, const slora_segments* seg, int32_t proj,
                               const void* x, void* workspace, size_t workspace_bytes,
                               void* stream);
slora_status slora_lora_expand(slora_pool* pool, const slora_segments* seg, int32_t proj, void* y,
                               const void* workspace, size_t workspace_bytes, void* stream);

/* The base projection with the delta in the same pass (summary page, "How to
 * read the paper" item 2: h = xW + xAB; blog page, section 2: the batched
 * forward returns the base output plus the adapter output):
 *   y[t, o] = round( sum_k x[t, k] W[k, o] + s_a * sum_j v[t, j] B_a[j, o] ),
 *   v[t, :] = x[t, :] A_a,
 * one fp32 sum per output element and one rounding to fp16; a token with no
 * adapter (negative id) gets y[t] = round(x[t] W).  y is WRITTEN (not
 * accumulated): the delta costs no extra read and write of y.  w is device
 * memory holding the base weight of projection `proj`, h_in x h_out fp16
 * row-major (W[k, o] at w[k * h_out + o]), caller-owned and only read;
 * x (n_tokens x h_in) and y (n_tokens x h_out) are device memory in batch
 * order, as for slora_lora_delta; workspace as for slora_lora_delta.  All
 * four 16-byte aligned.  fp16 pools only, with h_in a multiple of 64 and
 * h_out a multiple of 128 (SLORA_E_INVAL otherwise).  A batch without
 * 256-row tiles packs its LoRA stages with 23-bit segment fields, so it may
 * hold at most 2^23 - 1 segments (SLORA_E_INVAL otherwise).  Launches the
 * shrink kernels (v into the workspace) and then one matrix-core kernel over
 * tiles of 32, 64, 128 or 256 tokens (in segment order) x 128 or 256 columns
 * on `stream` (SLORA_TUNE_FWD_TILE), and returns
 * without waiting; launch errors return SLORA_E_HIP, device faults surface
 * at the caller's next synchronisation.  Requires a prior
 * slora_segments_upload; returns SLORA_E_STALE like slora_lora_delta.  With
 * n_tokens == 0 it launches nothing. */
slora_status slora_lora_forward(slora_pool* pool, const slora_segments* seg, int32_t proj,
                                const void* x, const void* w, void* y, void* workspace,
                                size_t workspace_bytes, void* stream);

/* slora_lora_forward with the caller's HIP events recorded by the dispatches
 * themselves (start when the first kernel begins, stop when the last ends),
 * as for slora_lora_delta_timed. */
slora_status slora_lora_forward_timed(slora_pool* pool, const slora_segments* seg, int32_t proj,
                                      const void* x, const void* w, void* y, void* workspace,
                                      size_t workspace_bytes, void* stream, void* start_event,
                                      void* stop_event);

/* slora_lora_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation, arguments and checks, but the workspace
 * (the fp32 x A products and their K-split partials) is the library's own
 * device array of 8 MiB, one per GPU, held until the process ends.  The call
 * allocates nothing.  A batch whose workspace_bytes exceed 8 MiB is refused
 * with SLORA_E_NOMEM before any device work.  Every call on one GPU shares
 * that GPU's array and leaves its contents behind (each call writes every
 * value it reads before reading it): calls on one GPU that overlap in time
 * (different streams, or different host threads without ordering) race and
 * must be serialised by the caller. */
slora_status slora_lora_forward_noalloc(slora_pool* pool, const slora_segments* seg, int32_t proj,
                                        const void* x, const void* w, void* y, void* stream);

/* Message for the calling thread's last failed call ("" if none). */
const char* slora_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SLORA_H */
