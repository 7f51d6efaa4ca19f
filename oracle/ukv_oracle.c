/*
 * CPU oracle for the unified page-major KV-cache pool.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the GPU library: it restates, slowly and
 * plainly, what the method computes, in the order the source pages give it.
 *
 * Sources.  "DKV" below is the report page "PR #34602: feat(unified-memory):
 * dense KV views for uniform-row MHA/SWA models" (sgl-project/sglang); its
 * sections are cited by their headings:
 *   DKV/impl-1..3   - 实现拆解 (implementation breakdown), steps 1-3
 *   DKV/pool        - 关键源码片段 (key excerpts): unified_memory_pool.py
 *   DKV/alloc       - 关键源码片段: multi_ended_allocator.py
 *   DKV/views       - 关键源码片段: layout/page_major.py (build_mha_views)
 *   DKV/files       - 关键文件 (key files): memory_pool.py, cache_move.py
 *   DKV/risk        - 风险与影响 (risks), item 5 (the int32 row bound)
 * "CKV" is the report page of vLLM PR #51689 (KV offload canonical layout
 * gate); its test table names an MLA latent head of 576 elements.
 *
 * Readings of points the pages leave open are marked READING.
 * Pins: every function here is checked in tests/test_oracle_pins.py against
 * brute-force enumeration of the envelope, an independent numpy strided 4-D
 * builder, closed forms and derived boundary values.  No function here is
 * "parity unpinned".
 *
 * Integer-only: nothing here converts or rounds a value; rows are moved as
 * bytes with memcpy.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Return codes. */
#define ORC_OK 0
#define ORC_INVALID -1
#define ORC_ASYMMETRIC_KV -2
#define ORC_KERNEL_ID_BOUND -3
#define ORC_OVERFLOW -4
#define ORC_ALIGNMENT -5
#define ORC_TAIL_PAD -6

/* Sticky condition bits reported by the data-path functions. */
#define ORC_F_SLOT_RANGE 1u  /* translate: slot or page past the pool / table */
#define ORC_F_BAD_ID 2u      /* store/move: id is not a kernel-facing row id */
#define ORC_F_BAD_BLOCK 4u   /* gather: block-table entry is not a kernel-facing page */
#define ORC_F_LAYOUT 8u      /* gather: output row not covered by cu_out / seq_lens */

#define ORC_MAX_SUB 8

typedef struct {
    int32_t kind; /* 0 = MHA: a K row and a V row per layer; 1 = MLA: one latent row per layer */
    int32_t layer_num;
    int32_t head_num;
    int32_t head_dim;
    int32_t v_head_dim; /* MHA only */
    int32_t elem_bytes; /* itemsize of the stored dtype */
    int64_t num_pages;
} orc_spec;

typedef struct {
    uint64_t row_bytes;
    uint64_t blocks_per_page;
    uint64_t page_bytes;     /* one page envelope */
    uint64_t n_rows;         /* rows of every dense view = kernel-facing id space */
    uint64_t anchor_bytes;   /* where this sub-pool's first page envelope starts */
    uint64_t envelope_bytes; /* num_pages page envelopes */
    uint64_t tail_pad_bytes; /* this spec's own view tail pad */
} orc_sub_plan;

typedef unsigned __int128 u128;

/*
 * Spec arithmetic and the start-up gates (DKV/impl-2, DKV/pool, DKV/views).
 *
 *  - asymmetric-KV gate: the unified pool is allowed when the model uses MLA
 *    or has no asymmetric KV, i.e. an MHA spec needs head_dim == v_head_dim.
 *  - row bytes = head_num * head_dim * itemsize (DKV/views).
 *  - blocks_per_page: MHA 2 * layer_num, MLA layer_num (DKV/impl-2, DKV/pool).
 *  - page envelope = page_size * blocks * row bytes; view rows
 *    n_rows = num_pages * blocks * page_size (DKV/views).
 *  - MHA view tail pad = page_size * entry_bytes().  READING: entry_bytes()
 *    is never shown; it is the bytes one token takes over all layers' K and
 *    V rows, blocks * row bytes, because the same pages call the required pad
 *    "a whole page envelope" and the builder's error text sizes it as
 *    page_size * blocks * row bytes.
 *  - MLA view tail pad: READING, one MLA page envelope by the same argument
 *    (its last dense view also reaches (blocks-1)*page_size rows past the end).
 *  - pool tail pad = the max over specs (DKV/pool, UnifiedKVPool.__init__);
 *    pool size = the envelopes + that pad.
 *  - READING: sub-pools sit back to back in spec order; the first at byte 0.
 *  - kernel-facing row bound: num_pages * blocks * page_size must be below
 *    2^31 (DKV/impl-2, DKV/risk item 5).
 *  - anchors must be multiples of the itemsize (DKV/views asserts).
 */
int orc_plan(const orc_spec *specs, int n_specs, int64_t page_size,
             orc_sub_plan *subs, uint64_t *pool_tail_pad, uint64_t *required_bytes)
{
    if (specs == NULL || subs == NULL || pool_tail_pad == NULL || required_bytes == NULL)
        return ORC_INVALID;
    if (n_specs < 1 || n_specs > ORC_MAX_SUB || page_size < 1)
        return ORC_INVALID;

    u128 anchor = 0;
    u128 tail = 0;
    for (int i = 0; i < n_specs; i++) {
        const orc_spec *s = &specs[i];
        if (s->kind != 0 && s->kind != 1)
            return ORC_INVALID;
        if (s->layer_num < 1 || s->head_num < 1 || s->head_dim < 1 || s->num_pages < 1)
            return ORC_INVALID;
        if (s->elem_bytes != 1 && s->elem_bytes != 2 && s->elem_bytes != 4 && s->elem_bytes != 8)
            return ORC_INVALID;
        /* unified_memory_supported_for_model: use_mla_backend or not has_asymmetric_kv */
        if (s->kind == 0 && s->head_dim != s->v_head_dim)
            return ORC_ASYMMETRIC_KV;

        u128 row_bytes = (u128)s->head_num * (u128)s->head_dim * (u128)s->elem_bytes;
        u128 blocks = (s->kind == 0) ? 2 * (u128)s->layer_num : (u128)s->layer_num;
        u128 page_bytes = (u128)page_size * blocks * row_bytes;
        u128 n_rows = (u128)s->num_pages * blocks * (u128)page_size;
        u128 entry_bytes = blocks * row_bytes;
        u128 pad = (u128)page_size * entry_bytes;
        u128 env = (u128)s->num_pages * page_bytes;

        if (n_rows >= ((u128)1 << 31))
            return ORC_KERNEL_ID_BOUND;
        if (anchor % (u128)s->elem_bytes != 0)
            return ORC_ALIGNMENT;
        if (anchor + env > (u128)UINT64_MAX || page_bytes > (u128)UINT64_MAX)
            return ORC_OVERFLOW;

        subs[i].row_bytes = (uint64_t)row_bytes;
        subs[i].blocks_per_page = (uint64_t)blocks;
        subs[i].page_bytes = (uint64_t)page_bytes;
        subs[i].n_rows = (uint64_t)n_rows;
        subs[i].anchor_bytes = (uint64_t)anchor;
        subs[i].envelope_bytes = (uint64_t)env;
        subs[i].tail_pad_bytes = (uint64_t)pad;

        anchor += env;
        if (pad > tail)
            tail = pad;
    }
    if (anchor + tail > (u128)UINT64_MAX)
        return ORC_OVERFLOW;
    *pool_tail_pad = (uint64_t)tail;
    *required_bytes = (uint64_t)(anchor + tail);
    return ORC_OK;
}

/*
 * Base byte offset of the dense view of (layer, kv) (DKV/views): layer l's K
 * starts at block 2l and V one block (page_size rows) later; MLA layer l's
 * latent view starts at block l.  kv: 0 = K (or latent), 1 = V.
 */
int orc_view_base(const orc_sub_plan *sp, int kind, int64_t page_size, int layer_num,
                  int layer, int kv, uint64_t *base_bytes)
{
    if (layer < 0 || layer >= layer_num)
        return ORC_INVALID;
    if (kind == 0) {
        if (kv != 0 && kv != 1)
            return ORC_INVALID;
        uint64_t k_base = sp->anchor_bytes + (uint64_t)(2 * layer) * (uint64_t)page_size * sp->row_bytes;
        *base_bytes = kv == 0 ? k_base : k_base + (uint64_t)page_size * sp->row_bytes;
    } else {
        if (kv != 0)
            return ORC_INVALID;
        *base_bytes = sp->anchor_bytes + (uint64_t)layer * (uint64_t)page_size * sp->row_bytes;
    }
    return ORC_OK;
}

/*
 * The view builder's own bounds assert (DKV/views): the last view, block
 * blocks-1, ends at anchor + (blocks-1)*ps*row_bytes + n_rows*row_bytes and
 * must fit in the raw buffer.  Returns ORC_TAIL_PAD when it does not.
 */
int orc_builder_check(const orc_sub_plan *sp, int64_t page_size, uint64_t raw_bytes,
                      uint64_t *last_view_end)
{
    u128 end = (u128)sp->anchor_bytes +
               (u128)(sp->blocks_per_page - 1) * (u128)page_size * (u128)sp->row_bytes +
               (u128)sp->n_rows * (u128)sp->row_bytes;
    *last_view_end = (uint64_t)end;
    return end <= (u128)raw_bytes ? ORC_OK : ORC_TAIL_PAD;
}

/* kernel_id(t) = (t // ps) * (ps * multiplier) + t % ps, for t >= 0 (DKV/impl-1). */
int64_t orc_kernel_id(int64_t t, int64_t page_size, int64_t multiplier)
{
    return (t / page_size) * (page_size * multiplier) + t % page_size;
}

/*
 * translate_kv_loc_for_kernel (DKV/impl-3, DKV/alloc), one slot at a time:
 * split into page and offset, look the page up in the virtual-to-physical
 * table (identity when no table is given), scale by the page stride
 * ps * blocks_per_page, add the offset, clamp negatives to 0.
 *
 * READINGS: a negative slot is a tombstone and goes to 0 (the page-0 sink)
 * before any lookup; an unmapped page (negative table entry) goes to 0; a
 * page past the table or a physical page past the pool goes to 0 and raises
 * ORC_F_SLOT_RANGE.
 */
void orc_translate(const int64_t *slots, int64_t n, int64_t page_size, int64_t blocks_per_page,
                   int64_t num_pages, const int32_t *v2p, int64_t v2p_len, int32_t *out,
                   uint32_t *flags)
{
    for (int64_t i = 0; i < n; i++) {
        int64_t t = slots[i];
        if (t < 0) {
            out[i] = 0;
            continue;
        }
        int64_t page = t / page_size;
        int64_t offset = t % page_size;
        int64_t phys;
        if (v2p != NULL) {
            if (page >= v2p_len) {
                out[i] = 0;
                *flags |= ORC_F_SLOT_RANGE;
                continue;
            }
            phys = v2p[page];
        } else {
            phys = page;
        }
        if (phys < 0) {
            out[i] = 0;
            continue;
        }
        if (phys >= num_pages) {
            out[i] = 0;
            *flags |= ORC_F_SLOT_RANGE;
            continue;
        }
        int64_t id = phys * (page_size * blocks_per_page) + offset;
        out[i] = (int32_t)id;
    }
}

/*
 * Block-table entries for the read path (DKV/motivation: every layer is
 * read through one contiguous tensor and one shared block table).  The
 * dense view's page index of a page is the kernel id of its first slot
 * divided by page_size.  Same tombstone / unmapped / range readings as
 * orc_translate.
 */
void orc_translate_pages(const int32_t *pages, int64_t n, int64_t page_size, int64_t blocks_per_page,
                         int64_t num_pages, const int32_t *v2p, int64_t v2p_len, int32_t *out,
                         uint32_t *flags)
{
    for (int64_t i = 0; i < n; i++) {
        int64_t q = pages[i];
        if (q < 0) {
            out[i] = 0;
            continue;
        }
        int64_t phys;
        if (v2p != NULL) {
            if (q >= v2p_len) {
                out[i] = 0;
                *flags |= ORC_F_SLOT_RANGE;
                continue;
            }
            phys = v2p[q];
        } else {
            phys = q;
        }
        if (phys < 0) {
            out[i] = 0;
            continue;
        }
        if (phys >= num_pages) {
            out[i] = 0;
            *flags |= ORC_F_SLOT_RANGE;
            continue;
        }
        int64_t first_slot_id = orc_kernel_id(phys * page_size, page_size, blocks_per_page);
        out[i] = (int32_t)(first_slot_id / page_size);
    }
}

/* A row id is kernel-facing when it lies on some page's block 0 rows. */
static int is_kernel_facing(int64_t id, int64_t page_size, int64_t blocks_per_page, int64_t num_pages)
{
    if (id < 0)
        return 0;
    int64_t stride = page_size * blocks_per_page;
    return id / stride < num_pages && id % stride < page_size;
}

typedef struct {
    uint8_t *raw;
    uint64_t raw_bytes;
    int32_t kind;
    int32_t layer_num;
    int64_t page_size;
    int64_t num_pages;
    orc_sub_plan sp;
} orc_pool;

/* Byte offset of row `id` of the (layer, kv) dense view inside raw. */
static int64_t row_off(const orc_pool *p, int layer, int kv, int64_t id)
{
    uint64_t base = 0;
    orc_view_base(&p->sp, p->kind, p->page_size, p->layer_num, layer, kv, &base);
    return (int64_t)(base + (uint64_t)id * p->sp.row_bytes);
}

/*
 * Per-layer store (DKV/files: _store_kv_layer is a plain 3-D row
 * assignment): k_view[layer][ids] = k, v_view[layer][ids] = v.  MLA stores
 * the latent row only (v is NULL).  An id off the kernel-facing id space is
 * not written and raises ORC_F_BAD_ID.
 *
 * orc_store_map gives, for entry i, the byte offset its K (and V) row lands
 * at, or -1 when the entry is skipped; orc_store copies the rows there, in
 * entry order, so among repeated ids the last one wins.
 */
void orc_store_map(const orc_pool *p, int layer, const int32_t *ids, int64_t n, int64_t *k_off, int64_t *v_off,
                   uint32_t *flags)
{
    for (int64_t i = 0; i < n; i++) {
        int64_t id = ids[i];
        if (!is_kernel_facing(id, p->page_size, (int64_t)p->sp.blocks_per_page, p->num_pages)) {
            *flags |= ORC_F_BAD_ID;
            k_off[i] = -1;
            if (v_off != NULL)
                v_off[i] = -1;
            continue;
        }
        k_off[i] = row_off(p, layer, 0, id);
        if (v_off != NULL)
            v_off[i] = p->kind == 0 ? row_off(p, layer, 1, id) : -1;
    }
}

void orc_store(const orc_pool *p, int layer, const int32_t *ids, int64_t n, const uint8_t *k, const uint8_t *v,
               int64_t src_row_stride, uint32_t *flags)
{
    int64_t *k_off = (int64_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
    int64_t *v_off = (int64_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
    if (k_off == NULL || v_off == NULL)
        abort();
    orc_store_map(p, layer, ids, n, k_off, v_off, flags);
    for (int64_t i = 0; i < n; i++) {
        if (k_off[i] < 0)
            continue;
        memcpy(p->raw + k_off[i], k + i * src_row_stride, p->sp.row_bytes);
        if (p->kind == 0)
            memcpy(p->raw + v_off[i], v + i * src_row_stride, p->sp.row_bytes);
    }
    free(k_off);
    free(v_off);
}

/*
 * Block-table gather (DKV/motivation: a backend reads each layer through one
 * contiguous tensor plus one shared block table).  The pages print no gather
 * kernel; READING of the operation:
 *   output row o belongs to the request r with cu_out[r] <= o < cu_out[r+1];
 *   it holds position j = j0 + (o - cu_out[r]) of that request, where
 *   j0 = 0, or len - window for a sliding-window layer shorter than len;
 *   the source row of position j is bt[r][j / ps] * ps + j % ps in the dense
 *   view, whose block-table entries are kernel-facing page indices.
 * Rows not covered (or past their request's length) raise ORC_F_LAYOUT,
 * bad block-table entries ORC_F_BAD_BLOCK; such rows are not written.
 *
 * orc_gather_map gives the byte offsets each output row is read from (-1 for
 * a skipped row); orc_gather copies them.
 */
void orc_gather_map(const orc_pool *p, int layer, const int32_t *bt, int64_t bt_stride, const int32_t *seq_lens,
                    const int64_t *cu_out, int32_t num_reqs, int32_t window, int64_t out_rows, int64_t *k_src,
                    int64_t *v_src, uint32_t *flags)
{
    int64_t bpp = (int64_t)p->sp.blocks_per_page;
    if (cu_out[0] != 0 || cu_out[num_reqs] != out_rows)
        *flags |= ORC_F_LAYOUT;
    for (int64_t o = 0; o < out_rows; o++) {
        k_src[o] = -1;
        if (v_src != NULL)
            v_src[o] = -1;
        int32_t r = 0;
        while (r < num_reqs && !(o < cu_out[r + 1]))
            r++;
        if (r == num_reqs || o < cu_out[r]) {
            *flags |= ORC_F_LAYOUT;
            continue;
        }
        int64_t len = seq_lens[r];
        int64_t j0 = (window > 0 && len > window) ? len - window : 0;
        int64_t q = o - cu_out[r];
        if (q >= len - j0) {
            *flags |= ORC_F_LAYOUT;
            continue;
        }
        int64_t j = j0 + q;
        int64_t page_idx = j / p->page_size;
        if (page_idx >= bt_stride) {
            *flags |= ORC_F_BAD_BLOCK;
            continue;
        }
        int64_t kp = bt[(int64_t)r * bt_stride + page_idx];
        if (kp < 0 || kp % bpp != 0 || kp / bpp >= p->num_pages) {
            *flags |= ORC_F_BAD_BLOCK;
            continue;
        }
        int64_t row = kp * p->page_size + j % p->page_size;
        k_src[o] = row_off(p, layer, 0, row);
        if (v_src != NULL && p->kind == 0)
            v_src[o] = row_off(p, layer, 1, row);
    }
}

void orc_gather(const orc_pool *p, int layer, const int32_t *bt, int64_t bt_stride, const int32_t *seq_lens,
                const int64_t *cu_out, int32_t num_reqs, int32_t window, uint8_t *k_out, uint8_t *v_out,
                int64_t out_rows, uint32_t *flags)
{
    int64_t *k_src = (int64_t *)malloc((size_t)(out_rows > 0 ? out_rows : 1) * sizeof(int64_t));
    int64_t *v_src = (int64_t *)malloc((size_t)(out_rows > 0 ? out_rows : 1) * sizeof(int64_t));
    if (k_src == NULL || v_src == NULL)
        abort();
    orc_gather_map(p, layer, bt, bt_stride, seq_lens, cu_out, num_reqs, window, out_rows, k_src, v_src, flags);
    uint64_t rb = p->sp.row_bytes;
    for (int64_t o = 0; o < out_rows; o++) {
        if (k_src[o] < 0)
            continue;
        memcpy(k_out + o * (int64_t)rb, p->raw + k_src[o], rb);
        if (p->kind == 0)
            memcpy(v_out + o * (int64_t)rb, p->raw + v_src[o], rb);
    }
    free(k_src);
    free(v_src);
}

/*
 * move_kv_cache (DKV/files: _move_kv_cache_impl is a 3-D row copy on every
 * layer, K and V): view[l][dst] = view[l][src] for l in [layer_begin,
 * layer_end).  The right-hand side is read whole before any write, as a
 * tensor assignment does.  A pair with either id off the kernel-facing id
 * space is skipped and raises ORC_F_BAD_ID.
 *
 * orc_move_map lists, for every (layer, kv, i) in that order, the byte
 * offsets a row is read from and written to (-1 for a skipped pair).
 */
void orc_move_map(const orc_pool *p, const int32_t *dst, const int32_t *src, int64_t n, int layer_begin,
                  int layer_end, int64_t *dst_off, int64_t *src_off, uint32_t *flags)
{
    int kvs = p->kind == 0 ? 2 : 1;
    int64_t bpp = (int64_t)p->sp.blocks_per_page;
    int64_t at = 0;
    for (int layer = layer_begin; layer < layer_end; layer++) {
        for (int kv = 0; kv < kvs; kv++) {
            for (int64_t i = 0; i < n; i++, at++) {
                if (!is_kernel_facing(src[i], p->page_size, bpp, p->num_pages) ||
                    !is_kernel_facing(dst[i], p->page_size, bpp, p->num_pages)) {
                    *flags |= ORC_F_BAD_ID;
                    dst_off[at] = -1;
                    src_off[at] = -1;
                    continue;
                }
                src_off[at] = row_off(p, layer, kv, src[i]);
                dst_off[at] = row_off(p, layer, kv, dst[i]);
            }
        }
    }
}

int orc_move(const orc_pool *p, const int32_t *dst, const int32_t *src, int64_t n, int layer_begin, int layer_end,
             uint32_t *flags)
{
    int kvs = p->kind == 0 ? 2 : 1;
    int64_t total = n * (int64_t)(layer_end - layer_begin) * kvs;
    uint64_t rb = p->sp.row_bytes;
    if (total < 0)
        total = 0;
    int64_t *dst_off = (int64_t *)malloc((size_t)(total > 0 ? total : 1) * sizeof(int64_t));
    int64_t *src_off = (int64_t *)malloc((size_t)(total > 0 ? total : 1) * sizeof(int64_t));
    uint8_t *snap = (uint8_t *)malloc(total > 0 ? (size_t)total * rb : 1);
    if (dst_off == NULL || src_off == NULL || snap == NULL) {
        free(dst_off);
        free(src_off);
        free(snap);
        return ORC_INVALID;
    }
    orc_move_map(p, dst, src, n, layer_begin, layer_end, dst_off, src_off, flags);
    for (int64_t a = 0; a < total; a++)
        if (src_off[a] >= 0)
            memcpy(snap + a * rb, p->raw + src_off[a], rb);
    for (int64_t a = 0; a < total; a++)
        if (dst_off[a] >= 0)
            memcpy(p->raw + dst_off[a], snap + a * rb, rb);
    free(dst_off);
    free(src_off);
    free(snap);
    return ORC_OK;
}

/* Size of orc_pool, so the Python side can check its struct mirror. */
int orc_sizeof_pool(void) { return (int)sizeof(orc_pool); }
int orc_sizeof_sub_plan(void) { return (int)sizeof(orc_sub_plan); }
int orc_sizeof_spec(void) { return (int)sizeof(orc_spec); }

/*
 * translate_kv_loc (DKV/alloc: the allocator's internal mechanisms, such as
 * compaction and the in-flight write set, keep physical ids; kernel-facing
 * ids are for kernels only).  READING: the internal id of slot t is the
 * physical slot phys * ps + t % ps with phys = v2p[t / ps] (identity
 * without a table); tombstones and unmapped pages stay -1 (internal
 * bookkeeping must still see them), a page past the table or the pool gives
 * -1 and raises ORC_F_SLOT_RANGE.
 */
void orc_translate_loc(const int64_t *slots, int64_t n, int64_t page_size, int64_t num_pages, const int32_t *v2p,
                       int64_t v2p_len, int32_t *out, uint32_t *flags)
{
    for (int64_t i = 0; i < n; i++) {
        int64_t t = slots[i];
        out[i] = -1;
        if (t < 0)
            continue;
        int64_t page = t / page_size;
        int64_t phys = page;
        if (v2p != NULL) {
            if (page >= v2p_len) {
                *flags |= ORC_F_SLOT_RANGE;
                continue;
            }
            phys = v2p[page];
        }
        if (phys < 0)
            continue;
        if (phys >= num_pages) {
            *flags |= ORC_F_SLOT_RANGE;
            continue;
        }
        out[i] = (int32_t)(phys * page_size + t % page_size);
    }
}

/*
 * Page relocation for compaction (DKV 关键文件 and alloc: lazy compaction moves
 * KV through move_kv_cache and rewrites the virtual-to-physical table).
 * READING: moving physical page s to physical page d is the row move of all
 * ps slots of page s to page d on every layer, K and V; here it is stated
 * exactly that way, through orc_move on the pages' kernel-facing row ids.
 * Pages must lie in [0, num_pages) (else ORC_F_BAD_ID, pair skipped).
 */
int orc_move_pages(const orc_pool *p, const int32_t *dst_pages, const int32_t *src_pages, int64_t n, uint32_t *flags)
{
    int64_t ps = p->page_size;
    int64_t bpp = (int64_t)p->sp.blocks_per_page;
    int32_t *d = (int32_t *)malloc((size_t)(n > 0 ? n * ps : 1) * sizeof(int32_t));
    int32_t *s = (int32_t *)malloc((size_t)(n > 0 ? n * ps : 1) * sizeof(int32_t));
    if (d == NULL || s == NULL) {
        free(d);
        free(s);
        return ORC_INVALID;
    }
    int64_t m = 0;
    for (int64_t i = 0; i < n; i++) {
        if (dst_pages[i] < 0 || dst_pages[i] >= p->num_pages || src_pages[i] < 0 || src_pages[i] >= p->num_pages) {
            *flags |= ORC_F_BAD_ID;
            continue;
        }
        for (int64_t o = 0; o < ps; o++) {
            d[m] = (int32_t)orc_kernel_id((int64_t)dst_pages[i] * ps + o, ps, bpp);
            s[m] = (int32_t)orc_kernel_id((int64_t)src_pages[i] * ps + o, ps, bpp);
            m++;
        }
    }
    int rc = orc_move(p, d, s, m, 0, p->layer_num, flags);
    free(d);
    free(s);
    return rc;
}

/*
 * Table rewrite after a relocation: v2p[virt[i]] = phys[i], in entry order.
 * virt past the table or phys outside [-1, num_pages) raise ORC_F_SLOT_RANGE
 * and the entry is skipped (-1 unmaps a virtual page).
 */
void orc_remap_pages(int32_t *v2p, int64_t v2p_len, const int32_t *virt, const int32_t *phys, int64_t n,
                     int64_t num_pages, uint32_t *flags)
{
    for (int64_t i = 0; i < n; i++) {
        if (virt[i] < 0 || virt[i] >= v2p_len || phys[i] < -1 || phys[i] >= num_pages) {
            *flags |= ORC_F_SLOT_RANGE;
            continue;
        }
        v2p[virt[i]] = phys[i];
    }
}

/*
 * Sliding-window eviction (DKV 功能与动机 and 关联脉络: the unified pool holds
 * SWA layers in their own sub-pool; the tombstone fix clears the full-to-SWA
 * mapping of tokens that left the window).  READING: the mapping is per page
 * (full virtual page -> SWA physical page, -1 = not resident); page i of
 * request r (positions [i*ps, (i+1)*ps)) is evicted when it lies wholly
 * before the window, (i+1)*ps <= len - window: mapping[table[r][i]] = -1.
 * A table entry past the mapping raises ORC_F_SLOT_RANGE; negative entries
 * are skipped.  window <= 0 evicts nothing.  Requests do not share pages.
 */
void orc_evict_window(int32_t *mapping, int64_t map_len, const int32_t *table, int64_t bt_stride,
                      const int32_t *seq_lens, int32_t num_reqs, int32_t window, int64_t page_size, uint32_t *flags)
{
    if (window <= 0)
        return;
    for (int32_t r = 0; r < num_reqs; r++) {
        int64_t len = seq_lens[r];
        if (len <= window)
            continue;
        int64_t start = len - window;
        for (int64_t i = 0; i < bt_stride && (i + 1) * page_size <= start; i++) {
            int64_t page = table[(int64_t)r * bt_stride + i];
            if (page < 0)
                continue;
            if (page >= map_len) {
                *flags |= ORC_F_SLOT_RANGE;
                continue;
            }
            mapping[page] = -1;
        }
    }
}

/*
 * Prefix-only page-table build for the read path (DKV 关联脉络: the stacked
 * change #35247 builds the kernel-facing page table of the attention
 * backends by translating the prefix only).  READING: row r of req_pages
 * lists the request's allocator pages in position order; entry i holds
 * positions [i*ps, (i+1)*ps), so it is translated (as orc_translate_pages,
 * through v2p when given) exactly when i < ceil(prefix_len[r] / ps); every
 * other entry is written as page 0 (the sink page) and is never read, so it
 * raises nothing.  A prefix needing more than bt_stride entries raises
 * ORC_F_LAYOUT (the covered entries are still translated); range conditions
 * of translated entries raise ORC_F_SLOT_RANGE as in orc_translate_pages.
 */
void orc_build_page_table(const int32_t *req_pages, int64_t bt_stride, const int32_t *prefix_lens, int32_t num_reqs,
                          int64_t page_size, int64_t blocks_per_page, int64_t num_pages, const int32_t *v2p,
                          int64_t v2p_len, int32_t *out, uint32_t *flags)
{
    for (int32_t r = 0; r < num_reqs; r++) {
        int64_t len = prefix_lens[r] > 0 ? prefix_lens[r] : 0;
        int64_t used = (len + page_size - 1) / page_size;
        if (used > bt_stride)
            *flags |= ORC_F_LAYOUT;
        for (int64_t i = 0; i < bt_stride; i++) {
            int64_t at = (int64_t)r * bt_stride + i;
            if (i < used)
                orc_translate_pages(&req_pages[at], 1, page_size, blocks_per_page, num_pages, v2p, v2p_len, &out[at],
                                    flags);
            else
                out[at] = 0;
        }
    }
}
