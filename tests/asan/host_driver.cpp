// Host-only driver for the sanitizer build of the library's plan, view and race-check
// code (tests/test_debug_validation.py).  Exercises the C entry points the way the host
// ABI tests do, with a seeded fuzz; prints "<n> cases ok" when every call returned a
// defined status.  No device code.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "ukv.h"

static int check_status(int rc) {
    switch (rc) {
        case UKV_OK: case UKV_ERR_INVALID_ARG: case UKV_ERR_ASYMMETRIC_KV: case UKV_ERR_KERNEL_ID_BOUND:
        case UKV_ERR_OVERFLOW: case UKV_ERR_ALIGNMENT: case UKV_ERR_TAIL_PAD: case UKV_ERR_RACE:
            return 0;
        default:
            std::printf("undefined status %d\n", rc);
            return 1;
    }
}

int main() {
    std::mt19937_64 g(12345);
    int bad = 0;
    long cases = 0;
    auto pick = [&](int64_t lo, int64_t hi) { return lo + (int64_t)(g() % (uint64_t)(hi - lo + 1)); };
    // the gates at their boundaries: the 70B shape at 838,860 / 838,861 pages, the 8B shape at 2^21 pages
    const int64_t pages[] = {838860, 838861, (1 << 21) - 1, 1 << 21, 1, 0, -1};
    for (int64_t P : pages) {
        for (int L : {80, 32}) {
            ukv_subpool_spec s = {UKV_MHA, L, 8, 128, 128, 2, P};
            ukv_plan plan;
            bad += check_status(ukv_pool_plan(&s, 1, 16, &plan));
            ++cases;
        }
    }
    for (int it = 0; it < 20000; ++it) {
        const int n = (int)pick(0, UKV_MAX_SUB + 1);
        std::vector<ukv_subpool_spec> specs((size_t)(n > 0 ? n : 1));
        for (int i = 0; i < n; ++i) {
            ukv_subpool_spec &s = specs[(size_t)i];
            s.kind = (int32_t)pick(-1, 2);
            s.layer_num = (int32_t)pick(-1, 130);
            s.head_num = (int32_t)pick(-1, 64);
            s.head_dim = (int32_t)(pick(0, 3) == 0 ? pick(-1, 1 << 20) : pick(1, 576));
            s.v_head_dim = pick(0, 4) == 0 ? (int32_t)pick(1, 576) : s.head_dim;
            s.elem_bytes = (int32_t)pick(0, 9);
            s.num_pages = pick(0, 5) == 0 ? (int64_t)(g() >> pick(1, 40)) : pick(-1, 5000);
        }
        const int64_t ps = pick(0, 5) == 0 ? (int64_t)(g() >> pick(1, 50)) : pick(-1, 128);
        ukv_plan plan;
        const int rc = ukv_pool_plan(n > 0 ? specs.data() : nullptr, n, ps, &plan);
        bad += check_status(rc);
        ++cases;
        if (rc == UKV_OK) {
            for (int sub = -1; sub <= plan.n_sub; ++sub) {
                const int L = sub >= 0 && sub < plan.n_sub ? specs[(size_t)sub].layer_num : 1;
                for (int layer = -1; layer <= L; layer += (L > 8 ? 7 : 1)) {
                    for (int kv = -1; kv <= 2; ++kv) {
                        ukv_view v;
                        bad += check_status(ukv_plan_view(&plan, specs.data(), sub, layer, kv, &v));
                        ++cases;
                    }
                }
            }
        }
        (void)ukv_last_error();
    }
    for (int it = 0; it < 2000; ++it) {
        const int64_t n = pick(0, 300);
        std::vector<int32_t> a((size_t)n), b((size_t)n);
        const int64_t hi = pick(1, 4 * n + 2);
        for (auto &x : a) x = (int32_t)pick(-3, hi);
        for (auto &x : b) x = (int32_t)pick(-3, hi);
        bad += check_status(ukv_check_store_ids(n ? a.data() : nullptr, n));
        bad += check_status(ukv_check_move_ids(n ? a.data() : nullptr, n ? b.data() : nullptr, n));
        cases += 2;
    }
    bad += check_status(ukv_check_store_ids(nullptr, 5)) + check_status(ukv_check_store_ids(nullptr, -1));
    bad += check_status(ukv_pool_plan(nullptr, 1, 16, nullptr));
    for (int s = -9; s <= 1; ++s) (void)ukv_status_name(s);
    if (bad) return 1;
    std::printf("%ld cases ok\n", cases);
    return 0;
}
