// Pool plan: spec arithmetic and start-up gates of the unified page-major
// KV pool.  Pure host code: no device call, no allocation.
//
// Source: report page "PR #34602: feat(unified-memory): dense KV views for
// uniform-row MHA/SWA models" (DKV), 实现拆解 (implementation) steps 1-2, its
// unified_memory_pool.py and layout/page_major.py excerpts, and 风险与影响
// (risks) item 5.  The readings of what those pages leave open (the size of
// entry_bytes(), the MLA tail pad, where sub-pools sit) are stated at each
// step below.
#include "ukv_internal.h"

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

namespace ukv {

namespace {
thread_local char g_last_error[1024] = "";
}

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_last_error[0] = '\0'; }

const char *last_error() { return g_last_error; }

bool ranges_overlap(const void *a, uint64_t na, const void *b, uint64_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na != 0 && nb != 0 && x < y + nb && y < x + na;
}

namespace {

bool mul_u64(uint64_t a, uint64_t b, uint64_t *out) { return !__builtin_mul_overflow(a, b, out); }
bool add_u64(uint64_t a, uint64_t b, uint64_t *out) { return !__builtin_add_overflow(a, b, out); }

bool valid_elem_bytes(int32_t e) { return e == 1 || e == 2 || e == 4 || e == 8; }

}  // namespace

int plan_pool(const ukv_subpool_spec *specs, int32_t n_specs, int64_t page_size, ukv_plan *out) {
    if (specs == nullptr || out == nullptr)
        return fail(UKV_ERR_INVALID_ARG, "ukv_pool_plan: null specs or out");
    if (n_specs < 1 || n_specs > UKV_MAX_SUB)
        return fail(UKV_ERR_INVALID_ARG, "ukv_pool_plan: n_specs=%d outside [1, %d]", n_specs, UKV_MAX_SUB);
    if (page_size < 1)
        return fail(UKV_ERR_INVALID_ARG, "ukv_pool_plan: page_size=%lld < 1", (long long)page_size);

    ukv_plan p;
    std::memset(&p, 0, sizeof(p));
    p.n_sub = n_specs;
    p.page_size = page_size;
    const uint64_t ps = (uint64_t)page_size;
    uint64_t cursor = 0;  // next sub-pool's anchor: sub-pools are laid back to back in spec order
    uint64_t pad_max = 0;

    for (int32_t i = 0; i < n_specs; ++i) {
        const ukv_subpool_spec &s = specs[i];
        if (s.kind != UKV_MHA && s.kind != UKV_MLA)
            return fail(UKV_ERR_INVALID_ARG, "sub-pool %d: kind=%d is neither UKV_MHA nor UKV_MLA", i, s.kind);
        if (s.layer_num < 1 || s.head_num < 1 || s.head_dim < 1 || s.num_pages < 1)
            return fail(UKV_ERR_INVALID_ARG,
                        "sub-pool %d: layer_num=%d head_num=%d head_dim=%d num_pages=%lld must all be >= 1", i,
                        s.layer_num, s.head_num, s.head_dim, (long long)s.num_pages);
        if (!valid_elem_bytes(s.elem_bytes))
            return fail(UKV_ERR_INVALID_ARG, "sub-pool %d: elem_bytes=%d is not 1, 2, 4 or 8", i, s.elem_bytes);
        // Asymmetric-KV gate: the 2L-block row array exists only when K and V
        // rows are equally wide; MLA keeps one latent row and is exempt.
        if (s.kind == UKV_MHA && s.head_dim != s.v_head_dim)
            return fail(UKV_ERR_ASYMMETRIC_KV,
                        "sub-pool %d: asymmetric KV (head_num=%d, head_dim=%d, v_head_num=%d, v_head_dim=%d) cannot "
                        "use the unified pool: its page envelope is 2L equal-width row blocks; use an MLA backend "
                        "or a non-unified KV layout",
                        i, s.head_num, s.head_dim, s.head_num, s.v_head_dim);

        uint64_t row_bytes, blocks, rows_per_page, page_bytes, n_rows, envelope;
        blocks = s.kind == UKV_MHA ? 2ull * (uint64_t)s.layer_num : (uint64_t)s.layer_num;
        if (!mul_u64((uint64_t)s.head_num, (uint64_t)s.head_dim, &row_bytes) ||
            !mul_u64(row_bytes, (uint64_t)s.elem_bytes, &row_bytes) || !mul_u64(blocks, ps, &rows_per_page) ||
            !mul_u64(rows_per_page, row_bytes, &page_bytes))
            return fail(UKV_ERR_OVERFLOW, "sub-pool %d: page envelope size overflows 64 bits", i);
        // Kernel-facing row bound: every dense view has num_pages * blocks * ps
        // rows, indexed through int32 read-index buffers, so it must stay < 2^31.
        if (!mul_u64((uint64_t)s.num_pages, rows_per_page, &n_rows) || n_rows >= (1ull << 31))
            return fail(UKV_ERR_KERNEL_ID_BOUND,
                        "sub-pool %d: kernel-facing rows num_pages(%lld) * blocks_per_page(%llu) * page_size(%lld) "
                        "must be < 2^31",
                        i, (long long)s.num_pages, (unsigned long long)blocks, (long long)page_size);
        if (!mul_u64((uint64_t)s.num_pages, page_bytes, &envelope))
            return fail(UKV_ERR_OVERFLOW, "sub-pool %d: envelope size overflows 64 bits", i);
        if (cursor % (uint64_t)s.elem_bytes != 0)
            return fail(UKV_ERR_ALIGNMENT, "sub-pool %d: anchor %llu is not a multiple of its itemsize %d", i,
                        (unsigned long long)cursor, s.elem_bytes);
        // View tail pad: the last dense view starts (blocks-1)*ps rows into the
        // first page and spans n_rows rows, so it ends (blocks-1)*ps rows past
        // the last envelope.  The pad is one whole page envelope, ps * entry
        // bytes with entry bytes = blocks * row bytes (one token over all of
        // the sub-pool's row blocks); the same rule is applied to MLA.
        const uint64_t pad = page_bytes;

        ukv_subpool_plan &q = p.sub[i];
        q.row_bytes = row_bytes;
        q.blocks_per_page = (int64_t)blocks;
        q.page_bytes = page_bytes;
        q.n_rows = (int64_t)n_rows;
        q.anchor_bytes = cursor;
        q.envelope_bytes = envelope;
        q.tail_pad_bytes = pad;
        if (!add_u64(cursor, envelope, &cursor))
            return fail(UKV_ERR_OVERFLOW, "sub-pool %d: pool size overflows 64 bits", i);
        if (pad > pad_max)
            pad_max = pad;
    }
    p.envelope_bytes = cursor;
    p.tail_pad_bytes = pad_max;  // the max over the specs: no caller can under-allocate it
    if (!add_u64(cursor, pad_max, &p.required_bytes))
        return fail(UKV_ERR_OVERFLOW, "pool size plus tail pad overflows 64 bits");
    *out = p;
    return UKV_OK;
}

int view_of(const ukv_plan &p, const ukv_subpool_spec &s, int32_t sub, int32_t layer, int32_t kv, ukv_view *out) {
    if (layer < 0 || layer >= s.layer_num)
        return fail(UKV_ERR_INVALID_ARG, "view: layer %d outside [0, %d)", layer, s.layer_num);
    const int32_t kvs = s.kind == UKV_MHA ? 2 : 1;
    if (kv < 0 || kv >= kvs)
        return fail(UKV_ERR_INVALID_ARG, "view: kv=%d invalid for this sub-pool (0%s)", kv,
                    kvs == 2 ? " = K, 1 = V" : " = latent");
    const ukv_subpool_plan &q = p.sub[sub];
    // Block of (layer, kv) inside every page: K of layer l is block 2l, V is
    // block 2l+1; an MLA layer's latent is block l.  The view's base folds the
    // block start in, so row k of every view is kernel-facing id k.
    const uint64_t block = s.kind == UKV_MHA ? 2ull * (uint64_t)layer + (uint64_t)kv : (uint64_t)layer;
    ukv_view v;
    std::memset(&v, 0, sizeof(v));
    v.byte_offset = q.anchor_bytes + block * (uint64_t)p.page_size * q.row_bytes;
    v.n_rows = q.n_rows;
    v.head_num = s.head_num;
    v.head_dim = s.head_dim;
    v.elem_bytes = s.elem_bytes;
    v.row_bytes = q.row_bytes;
    v.stride_elems[0] = (int64_t)s.head_num * s.head_dim;
    v.stride_elems[1] = s.head_dim;
    v.stride_elems[2] = 1;
    *out = v;
    return UKV_OK;
}

// Positions of entries sorted by value, ties by position: the first equal
// neighbours are the first repeated value.
static std::vector<int64_t> order_by_value(const int32_t *v, int64_t n) {
    std::vector<int64_t> idx((size_t)n);
    for (int64_t i = 0; i < n; ++i) idx[(size_t)i] = i;
    std::sort(idx.begin(), idx.end(), [v](int64_t a, int64_t b) { return v[a] != v[b] ? v[a] < v[b] : a < b; });
    return idx;
}

int check_store_ids(const int32_t *ids, int64_t n, const char *who) {
    if (n < 0 || (n > 0 && ids == nullptr)) return fail(UKV_ERR_INVALID_ARG, "%s: null ids or n < 0", who);
    const std::vector<int64_t> idx = order_by_value(ids, n);
    for (size_t k = 1; k < idx.size(); ++k) {
        const int32_t id = ids[idx[k]];
        if (id != 0 && id == ids[idx[k - 1]])
            return fail(UKV_ERR_RACE,
                        "%s: ids[%lld] and ids[%lld] are both row %d: their rows would race (only the sink row 0, "
                        "which tombstones share, may repeat)",
                        who, (long long)idx[k - 1], (long long)idx[k], id);
    }
    return UKV_OK;
}

int check_move_ids(const int32_t *dst, const int32_t *src, int64_t n, const char *who) {
    if (n < 0 || (n > 0 && (dst == nullptr || src == nullptr)))
        return fail(UKV_ERR_INVALID_ARG, "%s: null dst / src or n < 0", who);
    const std::vector<int64_t> idx = order_by_value(dst, n);
    for (size_t k = 1; k < idx.size(); ++k)
        if (dst[idx[k]] == dst[idx[k - 1]])
            return fail(UKV_ERR_RACE, "%s: dst[%lld] and dst[%lld] are both %d: their writes would race", who,
                        (long long)idx[k - 1], (long long)idx[k], dst[idx[k]]);
    for (int64_t i = 0; i < n; ++i) {  // a source that is also a destination: read and write race
        const int32_t x = src[i];
        auto it = std::lower_bound(idx.begin(), idx.end(), x, [dst](int64_t a, int32_t val) { return dst[a] < val; });
        if (it != idx.end() && dst[*it] == x)
            return fail(UKV_ERR_RACE, "%s: src[%lld] = %d is also dst[%lld]: the sets must be disjoint", who,
                        (long long)i, x, (long long)*it);
    }
    return UKV_OK;
}

}  // namespace ukv

// Host-only entry points (no device, no HIP call).
extern "C" {

int ukv_pool_plan(const ukv_subpool_spec *specs, int32_t n_specs, int64_t page_size, ukv_plan *out) {
    return ukv::plan_pool(specs, n_specs, page_size, out);
}

int ukv_plan_view(const ukv_plan *plan, const ukv_subpool_spec *specs, int32_t sub, int32_t layer, int32_t kv,
                  ukv_view *out) {
    if (plan == nullptr || specs == nullptr || out == nullptr)
        return ukv::fail(UKV_ERR_INVALID_ARG, "ukv_plan_view: null argument");
    if (sub < 0 || sub >= plan->n_sub || plan->n_sub > UKV_MAX_SUB)
        return ukv::fail(UKV_ERR_INVALID_ARG, "ukv_plan_view: sub-pool %d outside [0, %d)", sub, plan->n_sub);
    return ukv::view_of(*plan, specs[sub], sub, layer, kv, out);
}

int ukv_check_store_ids(const int32_t *ids, int64_t n) { return ukv::check_store_ids(ids, n, "ukv_check_store_ids"); }

int ukv_check_move_ids(const int32_t *dst, const int32_t *src, int64_t n) {
    return ukv::check_move_ids(dst, src, n, "ukv_check_move_ids");
}

const char *ukv_last_error(void) { return ukv::last_error(); }

const char *ukv_status_name(int status) {
    switch (status) {
        case UKV_OK: return "UKV_OK";
        case UKV_ERR_INVALID_ARG: return "UKV_ERR_INVALID_ARG";
        case UKV_ERR_ASYMMETRIC_KV: return "UKV_ERR_ASYMMETRIC_KV";
        case UKV_ERR_KERNEL_ID_BOUND: return "UKV_ERR_KERNEL_ID_BOUND";
        case UKV_ERR_OVERFLOW: return "UKV_ERR_OVERFLOW";
        case UKV_ERR_ALIGNMENT: return "UKV_ERR_ALIGNMENT";
        case UKV_ERR_TAIL_PAD: return "UKV_ERR_TAIL_PAD";
        case UKV_ERR_HIP: return "UKV_ERR_HIP";
        case UKV_ERR_RACE: return "UKV_ERR_RACE";
        default: return "UKV_ERR_UNKNOWN";
    }
}

}  // extern "C"
