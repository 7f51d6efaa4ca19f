/*
 * ukv.h - unified page-major KV-cache pool on AMD Instinct MI355X (gfx950).
 *
 * One raw uint8 HBM buffer holds every sub-pool's KV cache.  A page of an MHA
 * sub-pool is the envelope [L0_K*ps | L0_V*ps | L1_K*ps | ...]: 2L blocks of
 * ps equally wide rows.  Every (layer, K/V) pair is a dense view
 * (n_rows, head_num, head_dim) whose base is the start of block 2l (K) or
 * 2l+1 (V), so all views share one kernel-facing id space
 *
 *     kernel_id(t) = (t / ps) * (ps * blocks_per_page) + t % ps,
 *
 * with blocks_per_page = 2L for MHA and L for MLA.  On that pool this library
 * runs HIP kernels for id translation, the per-layer K/V scatter-store, the
 * block-table gather, the row and page moves, and, on the read path, the
 * prefix-only page-table build and a decode attention over the views.
 *
 * Source for the method: the report page "PR #34602: feat(unified-memory):
 * dense KV views for uniform-row MHA/SWA models" (sgl-project/sglang), cited
 * below as DKV with its section headings: 执行摘要 (summary), 功能与动机
 * (motivation), 实现拆解 (implementation) steps 1-5, 关键文件 (key files),
 * 关键源码片段 (key excerpts: unified_memory_pool.py, multi_ended_allocator.py,
 * layout/page_major.py), 评论区精华 (review), 风险与影响 (risks).
 *
 * Conventions for every entry point:
 *  - Return UKV_OK (0) or a negative UKV_ERR_* code; on error
 *    ukv_last_error() gives a readable message (thread-local).  Nothing is
 *    launched when a call returns an error.
 *  - Pointers named *_dev are device pointers on the pool's device; the
 *    caller owns them (the library never frees caller memory).
 *  - Data-path calls are asynchronous on `stream` (0 = the null stream),
 *    never allocate and never synchronise.  They only check host-visible
 *    arguments; conditions found on the device (an id off the kernel-facing
 *    id space, a bad block-table entry, ...) skip the affected row and set a
 *    sticky per-pool flag, read with ukv_pool_error_flags().
 *  - The calling thread's current HIP device must be the pool's device.
 */
#ifndef UKV_H
#define UKV_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes --------------------------------------------------------- */
#define UKV_OK 0
#define UKV_ERR_INVALID_ARG -1
#define UKV_ERR_ASYMMETRIC_KV -2   /* MHA spec with head_dim != v_head_dim */
#define UKV_ERR_KERNEL_ID_BOUND -3 /* kernel-facing rows would reach 2^31 */
#define UKV_ERR_OVERFLOW -4        /* byte sizes overflow 64 bits */
#define UKV_ERR_ALIGNMENT -5       /* misaligned anchor or buffer */
#define UKV_ERR_TAIL_PAD -6        /* raw buffer smaller than envelopes + tail pad */
#define UKV_ERR_HIP -7             /* a HIP runtime call failed */
#define UKV_ERR_RACE -8            /* debug validation: ids whose rows would race (nothing launched) */

/* ---- sticky device flags (ukv_pool_error_flags) --------------------------- */
#define UKV_FLAG_SLOT_RANGE 1u /* translate: slot / page past the pool or the v2p table; wrote 0 */
#define UKV_FLAG_BAD_ID 2u     /* store/move: id not a kernel-facing row id; row skipped */
#define UKV_FLAG_BAD_BLOCK 4u  /* gather: block-table entry not a kernel-facing page; row skipped */
#define UKV_FLAG_LAYOUT 8u     /* gather: cu_out / seq_lens / out_rows disagree; row skipped */

/* ---- sub-pool kinds -------------------------------------------------------- */
#define UKV_MHA 0 /* a K row and a V row per token per layer: blocks_per_page = 2L */
#define UKV_MLA 1 /* one latent row per token per layer:   blocks_per_page = L  */

#define UKV_MAX_SUB 8

/*
 * One sub-pool.  Row bytes = head_num * head_dim * elem_bytes.  MLA: the
 * latent row is head_num = 1, head_dim = 576 for the usual 512 + 64 latent;
 * v_head_dim is ignored.  elem_bytes is the stored dtype's itemsize
 * (1, 2, 4 or 8); rows are moved as bytes, never converted.
 */
typedef struct ukv_subpool_spec {
    int32_t kind;
    int32_t layer_num;
    int32_t head_num;
    int32_t head_dim;
    int32_t v_head_dim;
    int32_t elem_bytes;
    int64_t num_pages; /* pages of this sub-pool; page 0 serves as the tombstone sink */
} ukv_subpool_spec;

typedef struct ukv_subpool_plan {
    uint64_t row_bytes;
    int64_t blocks_per_page; /* 2L (MHA) or L (MLA) */
    uint64_t page_bytes;     /* one page envelope = ps * blocks_per_page * row_bytes */
    int64_t n_rows;          /* rows of each dense view = num_pages * blocks_per_page * ps */
    uint64_t anchor_bytes;   /* byte offset of the sub-pool's first page in the raw buffer */
    uint64_t envelope_bytes; /* num_pages * page_bytes */
    uint64_t tail_pad_bytes; /* this spec's view tail pad: one page envelope */
} ukv_subpool_plan;

typedef struct ukv_plan {
    int32_t n_sub;
    int32_t reserved;
    int64_t page_size;
    uint64_t envelope_bytes; /* all sub-pools, back to back in spec order */
    uint64_t tail_pad_bytes; /* max over the specs */
    uint64_t required_bytes; /* envelope_bytes + tail_pad_bytes: the raw buffer size */
    ukv_subpool_plan sub[UKV_MAX_SUB];
} ukv_plan;

/* A dense per-layer view: element (row, h, d) of type elem_bytes sits at byte
 * byte_offset + row * row_bytes + (h * head_dim + d) * elem_bytes of the raw buffer. */
typedef struct ukv_view {
    uint64_t byte_offset;
    int64_t n_rows;
    int32_t head_num;
    int32_t head_dim;
    int32_t elem_bytes;
    int32_t reserved;
    uint64_t row_bytes;
    int64_t stride_elems[3]; /* (head_num * head_dim, head_dim, 1) */
} ukv_view;

typedef struct ukv_pool ukv_pool;

/*
 * Pool plan: spec arithmetic and the start-up gates, pure host code (no
 * device, no allocation).  DKV 实现拆解 step 2 and the unified_memory_pool.py
 * excerpt: blocks_per_page from the spec (MHA 2L, MLA L); the view tail pad
 * derived from the specs as their maximum (MHA: page_size * entry bytes, one
 * page envelope; MLA read the same way); the asymmetric-KV gate (an MHA spec
 * needs head_dim == v_head_dim, MLA is exempt); the kernel-facing row bound
 * num_pages * blocks_per_page * ps < 2^31 (DKV 风险 item 5).  Sub-pools sit
 * back to back in spec order from byte 0.
 *
 * specs: host array of n_specs (1..UKV_MAX_SUB) specs; page_size >= 1.
 * out:   host struct, filled on success.
 * Errors: INVALID_ARG, ASYMMETRIC_KV, KERNEL_ID_BOUND, OVERFLOW, ALIGNMENT
 * (an anchor that is not a multiple of its sub-pool's itemsize).
 */
int ukv_pool_plan(const ukv_subpool_spec *specs, int32_t n_specs, int64_t page_size, ukv_plan *out);

/*
 * Pool over a caller-owned device buffer (DKV unified_memory_pool.py excerpt:
 * one uint8 buffer of total bytes + the derived tail pad).  Plans the specs,
 * then borrows raw_dev: it must be a device allocation on the current
 * device, 16-byte aligned, of at least plan.required_bytes (else
 * UKV_ERR_TAIL_PAD: no caller can under-allocate the pad).  The handle owns
 * two 4-byte device words for the sticky flags (allocated here, freed by
 * ukv_pool_destroy); it never frees raw_dev.  Does not touch the buffer's
 * contents.  *out is set only on success.
 */
int ukv_pool_create(const ukv_subpool_spec *specs, int32_t n_specs, int64_t page_size, void *raw_dev,
                    uint64_t raw_bytes, ukv_pool **out);

/* Frees the handle and its flag words (not the raw buffer).  NULL is a no-op. */
int ukv_pool_destroy(ukv_pool *pool);

/* Copy of the pool's plan. */
int ukv_pool_get_plan(const ukv_pool *pool, ukv_plan *out);

/*
 * Dense view of (sub, layer, kv) (DKV 实现拆解 step 1, layout/page_major.py
 * excerpt build_mha_views): base = anchor + (2*layer + kv) * ps * row_bytes
 * for MHA (kv 0 = K, 1 = V), anchor + layer * ps * row_bytes for MLA (kv
 * must be 0); n_rows rows.  The last view reaches (blocks_per_page-1)*ps
 * rows past the last envelope, into the tail pad.
 */
int ukv_pool_view(const ukv_pool *pool, int32_t sub, int32_t layer, int32_t kv, ukv_view *out);

/* The same view from a plan and its specs, pure host code (no pool, no device). */
int ukv_plan_view(const ukv_plan *plan, const ukv_subpool_spec *specs, int32_t sub, int32_t layer, int32_t kv,
                  ukv_view *out);

/*
 * Token slots -> kernel-facing row ids (DKV 实现拆解 step 3 and the
 * multi_ended_allocator.py excerpt, translate_kv_loc_for_kernel): for each
 * slot t, page = t / ps, offset = t % ps, phys = v2p[page] (identity when
 * v2p_dev is NULL), id = phys * ps * blocks_per_page + offset.
 *   t < 0 (tombstone) -> 0, the page-0 sink; phys < 0 (unmapped) -> 0;
 *   page >= v2p_len, or phys >= num_pages -> 0 and UKV_FLAG_SLOT_RANGE.
 * slots_dev: int64[n]; v2p_dev: int32[v2p_len] or NULL; out_dev: int32[n].
 * out_dev may be slots_dev itself (the pages' out= path aliases its input, so
 * a graph-captured batch can translate into its own slot buffer): the int32
 * ids then fill the buffer's first 4n bytes, translated by one workgroup that
 * reads each chunk of slots before writing its ids (a few microseconds per
 * thousand slots); any other overlap of out_dev with slots_dev or v2p_dev is
 * UKV_ERR_INVALID_ARG.  n in [0, 2^31).  Translate once per batch; every
 * layer reuses the ids.
 */
int ukv_translate_loc_for_kernel(const ukv_pool *pool, int32_t sub, const int64_t *slots_dev, int64_t n,
                                 const int32_t *v2p_dev, int64_t v2p_len, int32_t *out_dev, hipStream_t stream);

/*
 * Page ids -> block-table entries of the dense views (DKV 功能与动机: every
 * layer is read through one contiguous tensor and one shared block table):
 * out = kernel_id(phys * ps) / ps = phys * blocks_per_page, with the same
 * tombstone / unmapped / range rules as ukv_translate_loc_for_kernel.
 * pages_dev, out_dev: int32[n]; either the same buffer (each element is read
 * and then written by one thread) or not overlapping (UKV_ERR_INVALID_ARG).
 * v2p_dev as above.
 */
int ukv_translate_pages_for_kernel(const ukv_pool *pool, int32_t sub, const int32_t *pages_dev, int64_t n,
                                   const int32_t *v2p_dev, int64_t v2p_len, int32_t *out_dev, hipStream_t stream);

/*
 * Token slots -> internal physical slot ids (DKV multi_ended_allocator.py
 * excerpt: compaction and the in-flight write set keep physical ids; only
 * kernels see kernel-facing ids): phys * ps + t % ps with phys = v2p[t / ps]
 * (identity when v2p_dev is NULL).  Tombstones (t < 0) and unmapped pages
 * give -1; a page past the table or the pool gives -1 and raises
 * UKV_FLAG_SLOT_RANGE.  slots_dev int64[n] -> out_dev int32[n], which may be
 * slots_dev itself (as in ukv_translate_loc_for_kernel).
 */
int ukv_translate_loc(const ukv_pool *pool, int32_t sub, const int64_t *slots_dev, int64_t n, const int32_t *v2p_dev,
                      int64_t v2p_len, int32_t *out_dev, hipStream_t stream);

/*
 * Per-layer scatter-store (DKV 关键文件, memory_pool.py: _store_kv_layer is a
 * plain 3-D row assignment): K_view[layer][ids[i]] = k[i] and
 * V_view[layer][ids[i]] = v[i], each a row_bytes byte copy.
 * ids_dev: int32[n] KERNEL-FACING ids (from ukv_translate_loc_for_kernel):
 *   virtual or physical slots here silently hit other layers' rows (the
 *   hazard DKV's review names for an unguarded fused store), so an id that
 *   is not on some page's block-0 rows is skipped and raises UKV_FLAG_BAD_ID.
 * k_dev, v_dev: rows of row_bytes at k_dev + i * src_row_stride_bytes
 *   (src_row_stride_bytes >= row_bytes).  MLA: k_dev is the latent, v_dev
 *   must be NULL.
 * Id 0 is the sink row: tombstoned entries all write it and race.  Each
 * chunk of the copy's vector width comes whole from one of them: the width
 * is the largest of 16, 8, 4, 2 and 1 bytes that divides row_bytes, the K and
 * V views' byte offsets, the pool's, k_dev's and v_dev's addresses and the
 * source strides (16 bytes for 16-byte aligned rows).  Repeated live ids
 * race the same way.
 */
int ukv_store_kv(const ukv_pool *pool, int32_t sub, int32_t layer, const int32_t *ids_dev, int64_t n,
                 const void *k_dev, const void *v_dev, int64_t src_row_stride_bytes, hipStream_t stream);

/*
 * The store on several layers in one launch: layers layer_begin + i*layer_step
 * for i < layer_count (step >= 1, all inside the sub-pool), each exactly as
 * ukv_store_kv, with layer i's K / V source rows at
 * k_dev / v_dev + i * src_layer_stride_bytes + entry * src_row_stride_bytes.
 * The ids are translated once for the batch and serve every layer (DKV
 * 实现拆解 and 关联脉络: the write location is translated once per forward
 * batch, #35245).  layer_count = 0 is a no-op; at most 65535 layers.
 */
int ukv_store_kv_layers(const ukv_pool *pool, int32_t sub, int32_t layer_begin, int32_t layer_count,
                        int32_t layer_step, const int32_t *ids_dev, int64_t n, const void *k_dev, const void *v_dev,
                        int64_t src_row_stride_bytes, int64_t src_layer_stride_bytes, hipStream_t stream);

/*
 * Block-table gather into contiguous ragged K / V (DKV 功能与动机: a backend
 * reads a layer through one contiguous tensor plus one shared block table).
 * Output row o belongs to request r with cu_out[r] <= o < cu_out[r+1] and holds
 * position j = j0 + (o - cu_out[r]), j0 = seq_lens[r] - window when
 * 0 < window < seq_lens[r] (a sliding-window layer keeps its last `window`
 * positions) and 0 otherwise; the source row of position j is
 * block_table[r * bt_stride + j / ps] * ps + j % ps of the dense view.
 * block_table_dev: int32[num_reqs * bt_stride], entries from
 *   ukv_translate_pages_for_kernel (phys * blocks_per_page).  A bad entry
 *   skips the row and raises UKV_FLAG_BAD_BLOCK.
 * seq_lens_dev: int32[num_reqs]; cu_out_dev: int64[num_reqs + 1], non-decreasing,
 *   cu_out[0] = 0, cu_out[num_reqs] = out_rows, cu_out[r+1] - cu_out[r] = kept
 *   positions of r; a mismatch raises UKV_FLAG_LAYOUT and skips the rows concerned.
 * k_out_dev, v_out_dev: out_rows * row_bytes bytes each (MLA: v_out_dev NULL).
 * out_rows in [0, 2^31).  The pool is only read.
 */
int ukv_gather_kv(const ukv_pool *pool, int32_t sub, int32_t layer, const int32_t *block_table_dev,
                  int64_t bt_stride, const int32_t *seq_lens_dev, const int64_t *cu_out_dev, int32_t num_reqs,
                  int32_t window, void *k_out_dev, void *v_out_dev, int64_t out_rows, hipStream_t stream);

/*
 * The gather on several layers in one launch: layers layer_begin + i*layer_step
 * for i < layer_count, each exactly as ukv_gather_kv with one block table,
 * seq_lens, cu_out and window for all of them; layer i's rows go to
 * k_out_dev / v_out_dev + i * out_layer_stride_bytes.  With more than one
 * layer, |out_layer_stride_bytes| must be at least out_rows * row_bytes (the
 * layers' outputs may not overlap), else UKV_ERR_INVALID_ARG.
 */
int ukv_gather_kv_layers(const ukv_pool *pool, int32_t sub, int32_t layer_begin, int32_t layer_count,
                         int32_t layer_step, const int32_t *block_table_dev, int64_t bt_stride,
                         const int32_t *seq_lens_dev, const int64_t *cu_out_dev, int32_t num_reqs, int32_t window,
                         void *k_out_dev, void *v_out_dev, int64_t out_rows, int64_t out_layer_stride_bytes,
                         hipStream_t stream);

/*
 * Row move on every layer in [layer_begin, layer_end), K and V (DKV 关键文件,
 * memory_pool.py: _move_kv_cache_impl is a 3-D row copy):
 * view[l][dst[i]] = view[l][src[i]].  dst_dev, src_dev: int32[n]
 * kernel-facing ids; the src and dst sets must be disjoint and dst ids
 * distinct (otherwise rows race).  A pair with an id off the kernel-facing
 * space is skipped and raises UKV_FLAG_BAD_ID.
 */
int ukv_move_kv(const ukv_pool *pool, int32_t sub, const int32_t *dst_dev, const int32_t *src_dev, int64_t n,
                int32_t layer_begin, int32_t layer_end, hipStream_t stream);

/*
 * Page relocation for compaction (DKV multi_ended_allocator.py excerpt and
 * 关键文件: lazy compaction relocates KV with move_kv_cache, then rewrites
 * the virtual-to-physical table): physical page src_pages[i] is copied to
 * physical page dst_pages[i] on every layer, K and V.  A page's rows on all
 * layers are one contiguous page envelope, so this is a copy of page_bytes
 * per pair; it equals ukv_move_kv on the pages' kernel-facing row ids.
 * dst_pages_dev, src_pages_dev: int32[n] in [0, num_pages) (a pair outside
 * is skipped with UKV_FLAG_BAD_ID); the src and dst sets must be disjoint.
 */
int ukv_move_pages(const ukv_pool *pool, int32_t sub, const int32_t *dst_pages_dev, const int32_t *src_pages_dev,
                   int64_t n, hipStream_t stream);

/*
 * Table rewrite after a relocation: v2p_dev[virt[i]] = phys[i] (-1 unmaps).
 * v2p_dev: the caller's int32[v2p_len] virtual-to-physical table on the
 * device; virt_pages_dev, phys_pages_dev: int32[n], virt distinct.  An entry
 * with virt outside the table or phys outside [-1, num_pages) is skipped
 * with UKV_FLAG_SLOT_RANGE.  The table may not overlap the page lists.
 */
int ukv_remap_pages(const ukv_pool *pool, int32_t sub, int32_t *v2p_dev, int64_t v2p_len,
                    const int32_t *virt_pages_dev, const int32_t *phys_pages_dev, int64_t n, hipStream_t stream);

/*
 * Sliding-window eviction (DKV 功能与动机 and 关联脉络: SWA layers live in a
 * sub-pool of their own, and the tombstone fix clears the full-to-SWA
 * mapping of tokens that left the window).  mapping_dev: the caller's
 * int32[map_len] full virtual page -> SWA physical page table (-1 = not
 * resident), which is also the v2p argument of the translations on the SWA
 * sub-pool, so a write through an evicted page goes to the sink row.  For
 * each request r and page i of its block table (int32[num_reqs * bt_stride],
 * full virtual pages) with (i + 1) * ps <= seq_lens[r] - window:
 * mapping[table[r][i]] = -1.  A page past the mapping raises
 * UKV_FLAG_SLOT_RANGE; negative entries are skipped; window <= 0 is a no-op.
 * Pages must not be shared between requests.  The page size is the pool's.
 */
int ukv_evict_window(const ukv_pool *pool, int32_t *mapping_dev, int64_t map_len, const int32_t *table_dev,
                     int64_t bt_stride, const int32_t *seq_lens_dev, int32_t num_reqs, int32_t window,
                     hipStream_t stream);

/*
 * Kernel-facing page table for the read path, built from the prefix only
 * (DKV 关联脉络: the stacked change #35247 translates, for the attention
 * backends, only the pages that hold a request's prefix).
 * req_pages_dev: int32[num_reqs * bt_stride], row r = request r's allocator
 *   pages in position order (entry i holds positions [i*ps, (i+1)*ps));
 * prefix_lens_dev: int32[num_reqs];
 * out_dev: int32[num_reqs * bt_stride], the same buffer as req_pages_dev or
 *   not overlapping it (nor the lengths or v2p).
 * Entry i of row r is translated exactly when i < ceil(prefix_lens[r] / ps),
 * as ukv_translate_pages_for_kernel (through v2p_dev when not NULL): the
 * result is phys * blocks_per_page, 0 for a negative or unmapped page, and
 * 0 plus UKV_FLAG_SLOT_RANGE past the v2p table or the pool.  Every other
 * entry is written 0 and its input is never read for translation.  A prefix
 * needing more than bt_stride entries raises UKV_FLAG_LAYOUT.
 */
int ukv_build_page_table(const ukv_pool *pool, int32_t sub, const int32_t *req_pages_dev, int64_t bt_stride,
                         const int32_t *prefix_lens_dev, int32_t num_reqs, const int32_t *v2p_dev, int64_t v2p_len,
                         int32_t *out_dev, hipStream_t stream);

/*
 * Decode attention straight from the dense views (DKV 功能与动机: a backend
 * reads each layer through one dense tensor plus one block table shared by
 * all layers).  The pages print no attention kernel; this is the textbook
 * scaled dot-product attention of one query token per request with grouped
 * KV heads.  For request r with len = seq_lens[r] > 0, positions
 * j0 <= j < len (j0 = len - window when 0 < window < len, else 0), query
 * head g reading KV head h = g / G (G = q_heads / head_num):
 *     out[r][g] = sum_j softmax_j(scale * q[r][g] . K_j[h]) * V_j[h],
 * K_j / V_j being row block_table[r][j / ps] * ps + j % ps of the layer's
 * K / V views.
 * Sub-pool: MHA, bf16, head_dim 64, 128 or 256; G in {1, 2, 4, 8}.
 * q_dev: bf16 [num_reqs, q_heads, head_dim], contiguous, 16-byte aligned.
 * block_table_dev: int32[num_reqs * bt_stride] kernel-facing page indices
 *   (ukv_build_page_table / ukv_translate_pages_for_kernel).
 * seq_lens_dev: int32[num_reqs]; max_seq_len: a host bound on them that
 *   sizes the launch.
 * out_dev: fp32 [num_reqs, q_heads, head_dim], 16-byte aligned, overlapping
 *   neither q, the workspace nor the pool.
 * workspace_dev: at least ukv_decode_attention_workspace_bytes(...) bytes,
 *   16-byte aligned, owned by the caller (partial results per chunk of
 *   positions; its contents on entry do not matter).
 * Arithmetic: scores on the matrix cores from bf16 inputs with fp32
 * accumulation, softmax and the weighted sum of V in fp32.
 * Conditions: a request with len <= 0 gives zeros; len > max_seq_len gives
 * zeros and UKV_FLAG_LAYOUT; a position whose table column is past
 * bt_stride, or whose entry is negative, not a multiple of blocks_per_page
 * or past the pool, gives zeros for the whole request and UKV_FLAG_BAD_BLOCK.
 */
int ukv_decode_attention(const ukv_pool *pool, int32_t sub, int32_t layer, const void *q_dev, int32_t q_heads,
                         const int32_t *block_table_dev, int64_t bt_stride, const int32_t *seq_lens_dev,
                         int32_t num_reqs, int32_t max_seq_len, int32_t window, float scale, float *out_dev,
                         void *workspace_dev, uint64_t workspace_bytes, hipStream_t stream);

/*
 * Workspace bytes ukv_decode_attention needs on this sub-pool for these
 * sizes (0 when none, or for a bad pool / sub-pool).  The call splits each
 * request into units of up to 1,024 positions, fewer when the batch is small,
 * so the size depends on num_reqs, max_seq_len and window together.
 */
uint64_t ukv_decode_attention_workspace_bytes(const ukv_pool *pool, int32_t sub, int32_t num_reqs, int32_t q_heads,
                                              int32_t max_seq_len, int32_t window);

/*
 * ukv_decode_attention without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, arithmetic, conditions and results
 * as ukv_decode_attention (the same kernels run); the partial results live in
 * a fixed 64 MiB device array of the library, one per GPU it runs on, held
 * until the process ends.  The call itself allocates nothing: the array's
 * device address is looked up once per device, on the first call there.
 * Errors: as ukv_decode_attention, plus UKV_ERR_INVALID_ARG when
 * ukv_decode_attention_workspace_bytes(...) for these sizes exceeds 64 MiB
 * (256 requests of up to 8,192 positions with 32 query heads of dim 128 need
 * 34 MB), and UKV_ERR_HIP when the address lookup fails.  Every call on one
 * GPU shares that GPU's array: calls that overlap in time on one GPU (other
 * streams, or other threads) race on it and must be ordered by the caller.
 * Nothing in the array needs clearing: each call writes every partial it
 * reads.
 */
int ukv_decode_attention_noalloc(const ukv_pool *pool, int32_t sub, int32_t layer, const void *q_dev, int32_t q_heads,
                                 const int32_t *block_table_dev, int64_t bt_stride, const int32_t *seq_lens_dev,
                                 int32_t num_reqs, int32_t max_seq_len, int32_t window, float scale, float *out_dev,
                                 hipStream_t stream);

/*
 * Decode attention over an MLA sub-pool's dense latent view (DKV 功能与动机:
 * the MLA sub-pool already exposes dense per-layer views, read through one
 * dense tensor plus the shared block table).  The pages print no MLA
 * attention; this is the absorbed form: every query head attends to the one
 * latent row c_j of each position, the scores using the whole row and the
 * values its first v_dim elements.  For request r with len = seq_lens[r] > 0,
 * positions j0 <= j < len (j0 = len - window when 0 < window < len, else 0):
 *     out[r][g] = sum_j softmax_j(scale * q[r][g] . c_j) * c_j[0 : v_dim],
 * c_j being row block_table[r][j / ps] * ps + j % ps of the layer's view.
 * Sub-pool: MLA, bf16, latent width (head_dim) 576; v_dim must be 512;
 * q_heads a positive multiple of 16.
 * q_dev: bf16 [num_reqs, q_heads, 576], contiguous, 16-byte aligned (the
 *   query in the latent space: its non-rotary part already absorbed).
 * block_table_dev, seq_lens_dev, max_seq_len: as ukv_decode_attention.
 * out_dev: fp32 [num_reqs, q_heads, v_dim], 16-byte aligned, overlapping
 *   neither q, the workspace nor the pool.
 * workspace_dev: at least ukv_mla_decode_attention_workspace_bytes(...)
 *   bytes, 16-byte aligned, owned by the caller.
 * Arithmetic: both products on the matrix cores from bf16 inputs with fp32
 * accumulation; each softmax weight enters the value product as two bf16
 * parts (relative error <= 2^-16); softmax and the merge in fp32.
 * Conditions: as ukv_decode_attention (zeros for len <= 0; zeros and
 * UKV_FLAG_LAYOUT past max_seq_len; zeros and UKV_FLAG_BAD_BLOCK for a bad
 * or missing table entry).
 */
int ukv_mla_decode_attention(const ukv_pool *pool, int32_t sub, int32_t layer, const void *q_dev, int32_t q_heads,
                             int32_t v_dim, const int32_t *block_table_dev, int64_t bt_stride,
                             const int32_t *seq_lens_dev, int32_t num_reqs, int32_t max_seq_len, int32_t window,
                             float scale, float *out_dev, void *workspace_dev, uint64_t workspace_bytes,
                             hipStream_t stream);

/*
 * Workspace bytes ukv_mla_decode_attention needs for these sizes (0 when
 * none, or for a bad pool / sub-pool or q_heads not a multiple of 16).
 */
uint64_t ukv_mla_decode_attention_workspace_bytes(const ukv_pool *pool, int32_t sub, int32_t num_reqs,
                                                  int32_t q_heads, int32_t v_dim, int32_t max_seq_len,
                                                  int32_t window);

/*
 * Debug validation (for tests and bring-up; not for the data path).  The
 * pages' fused-store review (DKV 评论区精华, 风险与影响) shows what goes wrong
 * when ids are not what a kernel expects; rows that collide are the quieter
 * failure: two live store entries on one row, or a move whose destinations
 * repeat or meet its sources, race on the device with no error.
 * ukv_check_store_ids: UKV_ERR_RACE when two entries of ids (host array) name
 * the same row, row 0 excepted (the sink row that tombstones share).
 * ukv_check_move_ids: UKV_ERR_RACE when dst (host array) repeats an id or an
 * id of src is also in dst.  Both are host-only (no device), O(n log n), and
 * name the first offending pair in ukv_last_error().
 * ukv_pool_set_debug(pool, 1): from then on ukv_store_kv[_layers],
 * ukv_move_kv and ukv_move_pages first copy their id arrays to the host on
 * their stream (the call then synchronises that stream and allocates host
 * memory) and run these checks; on UKV_ERR_RACE nothing is launched.  0
 * turns it off (the default).
 */
int ukv_check_store_ids(const int32_t *ids, int64_t n);
int ukv_check_move_ids(const int32_t *dst, const int32_t *src, int64_t n);
int ukv_pool_set_debug(ukv_pool *pool, int32_t on);

/*
 * Reads and clears the pool's sticky flags (UKV_FLAG_*): enqueued on
 * `stream` after the work already there, then synchronises that stream.
 */
int ukv_pool_error_flags(ukv_pool *pool, hipStream_t stream, uint32_t *out_and_clear);

/* Message of the calling thread's last failed call ("" if none). */
const char *ukv_last_error(void);

/* Name of a status code, e.g. "UKV_ERR_TAIL_PAD". */
const char *ukv_status_name(int status);

#ifdef __cplusplus
}
#endif

#endif /* UKV_H */
