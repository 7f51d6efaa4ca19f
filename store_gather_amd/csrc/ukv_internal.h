// Internal declarations shared by the host and kernel translation units of
// libukv (not installed; the public ABI is include/ukv.h).
#pragma once

#include "ukv.h"

#include <cstdint>

struct ukv_pool;

namespace ukv {

// Records a thread-local message for ukv_last_error() and returns `code`.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
const char *last_error();

// Host-side checks shared by the entry points.
int check_pool_call(const ukv_pool *pool, int32_t sub, const char *who);  // pool, sub-pool, current device
int check_launch(const char *who);                                       // hipGetLastError after a launch
bool ranges_overlap(const void *a, uint64_t na, const void *b, uint64_t nb);

int plan_pool(const ukv_subpool_spec *specs, int32_t n_specs, int64_t page_size, ukv_plan *out);
// Race checks of the debug validation (host arrays): UKV_ERR_RACE with the first offending pair.
int check_store_ids(const int32_t *ids, int64_t n, const char *who);
int check_move_ids(const int32_t *dst, const int32_t *src, int64_t n, const char *who);
int view_of(const ukv_plan &p, const ukv_subpool_spec &s, int32_t sub, int32_t layer, int32_t kv, ukv_view *out);

}  // namespace ukv

struct ukv_pool {
    ukv_subpool_spec spec[UKV_MAX_SUB];
    ukv_plan plan;
    uint8_t *raw;        // borrowed device buffer
    uint64_t raw_bytes;
    int device;
    uint32_t *flags_dev;  // [0] sticky flags, [1] read-back slot; owned
    int32_t debug;        // ukv_pool_set_debug: store / move ids checked for races before each launch
};
