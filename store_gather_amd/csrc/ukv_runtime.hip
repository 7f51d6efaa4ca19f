// libukv: the C-ABI entry points and the HIP kernels of the unified
// page-major KV pool for gfx950 (MI355X).
//
// Source for the method: report page "PR #34602: feat(unified-memory): dense
// KV views for uniform-row MHA/SWA models" (DKV), 实现拆解 (implementation)
// steps 1-3, 关键文件 (key files: memory_pool.py, cache_move.py), 功能与动机
// (motivation) and the multi_ended_allocator.py excerpt.  The pages show
// Python/torch code and a retired Triton store kernel; nothing here follows
// either.  Every data-path kernel is a byte copy bounded by HBM bandwidth:
//
//  - rows are moved as 16-byte integer vectors (global_load/store_dwordx4)
//    whenever the row size, the view bases and the caller's pointers allow,
//    so bf16 NaN payloads and denormals pass bit-exact;
//  - store, gather and move work on tiles of rows: lane k of a 64-lane wave
//    resolves row k of the tile (its id, its block-table entry, or its move
//    pair), the row numbers are broadcast with ds_bpermute (__shfl), and the
//    tile's 16-byte chunks are spread over all lanes, loads before stores.
//    Tiles are sized by loads in flight per lane, so 32-byte rows, 1 KiB
//    rows, 1,152-byte MLA latents and 2 KiB rows all keep the memory system
//    equally busy (tile shapes swept on MI355X);
//  - destinations written once (gather outputs, stored and moved pool rows)
//    use the non-temporal store hint;
//  - one launch can cover a strided range of layers (grid y), so one
//    translation of a batch serves every layer;
//  - nothing allocates, nothing synchronises; ids are int32 (the pool plan
//    guarantees every view has fewer than 2^31 rows) and byte addresses are
//    64-bit (base + (uint64) id * row_bytes), since pools reach hundreds of GiB.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <new>
#include <type_traits>
#include <vector>

#include "ukv_internal.h"

// ----------------------------------------------------------------------------
// errors
// ----------------------------------------------------------------------------
namespace ukv {

int check_pool_call(const ukv_pool *pool, int32_t sub, const char *who) {
    if (pool == nullptr) return fail(UKV_ERR_INVALID_ARG, "%s: null pool", who);
    if (sub < 0 || sub >= pool->plan.n_sub)
        return fail(UKV_ERR_INVALID_ARG, "%s: sub-pool %d outside [0, %d)", who, sub, pool->plan.n_sub);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != pool->device)
        return fail(UKV_ERR_INVALID_ARG, "%s: current device %d is not the pool's device %d", who, dev, pool->device);
    return UKV_OK;
}

int check_launch(const char *who) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(UKV_ERR_HIP, "%s: kernel launch failed: %s", who, hipGetErrorString(e));
    return UKV_OK;
}

}  // namespace ukv

using ukv::check_launch;
using ukv::check_pool_call;
using ukv::fail;
using ukv::ranges_overlap;

namespace {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int64_t kMaxGrid = 0x7fffffff;

// The wave's index inside the block, made uniform so that everything derived
// from it is computed in scalar registers.
__device__ __forceinline__ int wave_in_block() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave)); }

// XCD order: workgroups go to the 8 XCDs round-robin in launch order (launch index i
// on XCD i % 8); this gives the workgroups of one XCD consecutive logical blocks, a
// bijection of [0, g).  Only the speed depends on that dispatch order: any other
// still covers every block once.
__device__ __forceinline__ uint32_t xcd_logical_block(uint32_t i, uint32_t g) {
    const uint32_t xcd = i & 7;
    return xcd * (g >> 3) + min(xcd, g & 7) + (i >> 3);
}
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// A kernel-facing row id lies on block 0 of some page: id = page * (ps *
// blocks_per_page) + offset with offset < ps and page < num_pages.  The view
// row count n_rows = num_pages * page_stride is below 2^31.
__device__ __forceinline__ bool kernel_facing(int32_t id, uint32_t n_rows, uint32_t page_stride, uint32_t ps) {
    return id >= 0 && (uint32_t)id < n_rows && ((uint32_t)id % page_stride) < ps;
}

// Integer vectors the rows are moved in.  Clang's ext vectors (not HIP's
// struct vector types), so that the non-temporal builtins accept them.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Store with the non-temporal (streaming) hint when NT: for destinations
// written once and not read again by this kernel (gather outputs, moved
// rows), it keeps them from displacing reusable lines in L2 / MALL.
// Measured on the decode-shape gather: +10% HBM throughput.
template <bool NT, typename V>
__device__ __forceinline__ void put(V *p, V v) {
    if constexpr (NT)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

// ----------------------------------------------------------------------------
// translate (DKV 实现拆解 step 3; multi_ended_allocator.py excerpt)
// ----------------------------------------------------------------------------
struct TranslateArgs {
    const int64_t *slots;  // or int32 page ids (pages mode)
    const int32_t *pages;
    const int32_t *v2p;
    int32_t *out;
    uint32_t *flags;
    int64_t n;
    int64_t v2p_len;
    int64_t ps;
    int64_t page_stride;  // ps * blocks_per_page
    int64_t bpp;
    int64_t num_pages;
    int32_t internal;  // 1: physical slot ids (translate_kv_loc), tombstones stay -1
};

// slot t -> id: tombstone (t < 0) -> 0; page = t / ps, offset = t % ps;
// phys = v2p[page] (identity without a table); unmapped (phys < 0) -> 0;
// past the table or the pool -> 0 plus UKV_FLAG_SLOT_RANGE;
// else phys * ps * blocks_per_page + offset.
__device__ __forceinline__ int32_t translate_one(const TranslateArgs &a, int64_t t, bool &out_of_range) {
    int32_t id = a.internal ? -1 : 0;
    out_of_range = false;
    if (t >= 0) {
        const int64_t page = t / a.ps;
        const int64_t offset = t - page * a.ps;
        int64_t phys = page;
        if (a.v2p != nullptr) {
            if (page >= a.v2p_len) {
                out_of_range = true;
                phys = -1;
            } else {
                phys = a.v2p[page];
            }
        }
        if (phys >= a.num_pages) {
            out_of_range = true;
        } else if (phys >= 0) {
            id = (int32_t)(phys * (a.internal ? a.ps : a.page_stride) + offset);
        }
    }
    return id;
}

__global__ __launch_bounds__(kBlock) void translate_slots_kernel(TranslateArgs a) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= a.n) return;
    bool out_of_range;
    a.out[i] = translate_one(a, a.slots[i], out_of_range);
    if (out_of_range) atomicOr(a.flags, UKV_FLAG_SLOT_RANGE);
}

// The same with the int32 ids written over the int64 slots they come from (the
// pages' out= path, which may alias its input).  Id i occupies bytes [4i, 4i+4),
// inside slot i/2, so one workgroup walks the array in chunks: every thread reads
// its slot, the workgroup waits, then writes.  A chunk's writes land on slots of
// that chunk or earlier ones, all read before its barrier; later chunks' slots
// lie past every byte written so far.
constexpr int kInPlaceBlock = 1024;

__global__ __launch_bounds__(kInPlaceBlock) void translate_inplace_kernel(TranslateArgs a) {
    bool any_out = false;
    for (int64_t c = 0; c < a.n; c += kInPlaceBlock) {
        const int64_t i = c + threadIdx.x;
        bool out_of_range = false;
        int32_t id = 0;
        if (i < a.n) id = translate_one(a, a.slots[i], out_of_range);
        any_out |= out_of_range;
        __syncthreads();
        if (i < a.n) a.out[i] = id;
        __syncthreads();
    }
    if (any_out) atomicOr(a.flags, UKV_FLAG_SLOT_RANGE);
}

// page q -> the dense views' page index of its first slot, phys * blocks_per_page.
__global__ __launch_bounds__(kBlock) void translate_pages_kernel(TranslateArgs a) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= a.n) return;
    const int64_t q = a.pages[i];
    int32_t kp = 0;
    bool out_of_range = false;
    if (q >= 0) {
        int64_t phys = q;
        if (a.v2p != nullptr) {
            if (q >= a.v2p_len) {
                out_of_range = true;
                phys = -1;
            } else {
                phys = a.v2p[q];
            }
        }
        if (phys >= a.num_pages) {
            out_of_range = true;
        } else if (phys >= 0) {
            kp = (int32_t)(phys * a.bpp);
        }
    }
    a.out[i] = kp;
    if (out_of_range) atomicOr(a.flags, UKV_FLAG_SLOT_RANGE);
}

// ----------------------------------------------------------------------------
// store (DKV 关键文件: _store_kv_layer, a plain 3-D row assignment)
// ----------------------------------------------------------------------------
// Store and gather move rows in tiles.  A tile is `tile_rows` rows whose
// 16-byte chunks are spread over the wave: lane k first resolves row k of
// the tile (its id or block-table entry), the row numbers are broadcast with
// ds_bpermute (__shfl), then every lane copies up to TPL chunks of K and V of
// the tile, loads first, then stores (several rounds when the tile holds more
// than 64 * TPL chunks).  The host sizes tiles by loads in flight per lane
// (tiling_for), so every row size keeps about the same bytes in flight per
// wave: e.g. 2 rows of 2 KiB K+V per gather tile, 5 MLA latents of 1,152 B.
constexpr int kTasksPerLane = 4;

struct StoreArgs {
    uint8_t *pool;
    uint64_t base[2];  // byte offsets of the K and V views of the layer
    const int32_t *ids;
    const uint8_t *src[2];
    int64_t src_stride;
    int64_t n;
    uint32_t n_rows;
    uint32_t page_stride;
    uint32_t ps;
    uint32_t row_bytes;
    int32_t vecs;          // row_bytes / sizeof(V)
    int32_t tile_rows;     // rows per tile, <= 64
    int32_t tiles_per_wave;
    uint32_t layers;           // grid y (in the struct's alignment gap: the arguments stay within 128 bytes)
    uint64_t layer_base_step;  // view bytes from one stored layer to the next (grid y)
    int64_t src_layer_stride;  // source bytes from one stored layer to the next
    uint32_t *flags;
};

// K_view[l][ids[i]] = k[l][i], V_view[l][ids[i]] = v[l][i] for the layer of
// grid row blockIdx.y; waves own runs of tiles, kStoreTileWaves to a workgroup:
// eight (512 threads) took the hybrid MHA store of 1 KiB rows (1.05 M rows, 4.3 GB)
// 684-704 us against 704-716 us with four, in five A/B pairs on three boxes.
constexpr int kStoreTileWaves = 8;

template <typename V, int NKV, int TPL = kTasksPerLane, bool NT = false>
__global__ __launch_bounds__(kStoreTileWaves * kWave) void store_kernel(StoreArgs a) {
    const int lane = lane_id();
    const int64_t wave = (int64_t)blockIdx.x * kStoreTileWaves + wave_in_block();
    const int64_t per_wave = (int64_t)a.tile_rows * a.tiles_per_wave;
    const int64_t i_begin = wave * per_wave;
    if (i_begin >= a.n) return;
    const int64_t i_end = i_begin + per_wave < a.n ? i_begin + per_wave : a.n;
    const int tasks = a.tile_rows * a.vecs;
    const uint64_t view0 = (uint64_t)blockIdx.y * a.layer_base_step;
    const int64_t src0 = (int64_t)blockIdx.y * a.src_layer_stride;
    bool bad = false;
    for (int64_t i0 = i_begin; i0 < i_end; i0 += a.tile_rows) {
        // lane k: the destination row of entry i0 + k (-1: skipped)
        int32_t id = -1;
        if (lane < a.tile_rows && i0 + lane < i_end) {
            const int32_t v = a.ids[i0 + lane];
            if (kernel_facing(v, a.n_rows, a.page_stride, a.ps))
                id = v;
            else
                bad = true;
        }
        for (int base = 0; base < tasks; base += kWave * TPL) {
            V buf[NKV][TPL];
            int32_t rows[TPL];
            int32_t ks[TPL];
            int32_t cs[TPL];
#pragma unroll
            for (int j = 0; j < TPL; ++j) {
                const int t = base + lane + j * kWave;
                const int k = t / a.vecs;
                const int c = t - k * a.vecs;
                const int32_t row = __shfl(id, k < kWave ? k : 0);
                rows[j] = (t < tasks) ? row : -1;
                ks[j] = k;
                cs[j] = c;
                // sources are read once: non-temporal loads (+2% on the
                // prefill-shape store, interleaved medians)
                if (rows[j] >= 0) {
#pragma unroll
                    for (int h = 0; h < NKV; ++h)
                        buf[h][j] = __builtin_nontemporal_load(
                            &reinterpret_cast<const V *>(a.src[h] + src0 + (i0 + k) * a.src_stride)[c]);
                }
            }
#pragma unroll
            for (int j = 0; j < TPL; ++j) {
                if (rows[j] >= 0) {
#pragma unroll
                    for (int h = 0; h < NKV; ++h)
                        put<NT>(&reinterpret_cast<V *>(a.pool + a.base[h] + view0 +
                                                       (uint64_t)(uint32_t)rows[j] * a.row_bytes)[cs[j]],
                                buf[h][j]);
                }
            }
            (void)ks;
        }
    }
    if (bad && blockIdx.y == 0) atomicOr(a.flags, UKV_FLAG_BAD_ID);
}

// ----------------------------------------------------------------------------
// gather (DKV 功能与动机: one contiguous tensor + one shared block table)
// ----------------------------------------------------------------------------
struct GatherArgs {
    const uint8_t *pool;
    uint64_t base[2];
    const int32_t *bt;
    int64_t bt_stride;
    const int32_t *seq_lens;
    const int64_t *cu_out;
    uint8_t *out[2];
    int64_t out_rows;
    int32_t num_reqs;
    int32_t window;
    uint32_t ps;
    uint32_t bpp;
    uint32_t num_pages;
    uint32_t row_bytes;
    int32_t vecs;
    int32_t tile_rows;
    int32_t tiles_per_wave;
    uint64_t layer_base_step;  // view bytes from one gathered layer to the next (grid y)
    int64_t out_layer_stride;  // output bytes from one gathered layer to the next
    uint32_t *flags;
};

// Source row of output row o (in request r, found by the caller), or -1 with
// the reason added to `bad`.  Row o of request r holds position
// j = j0 + (o - cu_out[r]) and reads dense row bt[r][j / ps] * ps + j % ps.
__device__ __forceinline__ int32_t gather_source_row(const GatherArgs &a, int64_t o, int32_t r, uint32_t &bad) {
    if (r >= a.num_reqs || o < a.cu_out[r]) {
        bad |= UKV_FLAG_LAYOUT;
        return -1;
    }
    const int64_t len = a.seq_lens[r];
    const int64_t j0 = (a.window > 0 && len > a.window) ? len - a.window : 0;
    const int64_t q = o - a.cu_out[r];
    if (q >= len - j0) {
        bad |= UKV_FLAG_LAYOUT;
        return -1;
    }
    const uint32_t j = (uint32_t)(j0 + q);  // < seq_lens[r] <= INT32_MAX
    const uint32_t page_idx = j / a.ps;
    if ((int64_t)page_idx >= a.bt_stride) {
        bad |= UKV_FLAG_BAD_BLOCK;
        return -1;
    }
    const int32_t kp = a.bt[(int64_t)r * a.bt_stride + page_idx];
    if (kp < 0 || (uint32_t)kp % a.bpp != 0 || (uint32_t)kp / a.bpp >= a.num_pages) {
        bad |= UKV_FLAG_BAD_BLOCK;
        return -1;
    }
    return (int32_t)((uint32_t)kp * a.ps + (j - page_idx * a.ps));  // < n_rows < 2^31
}

// A wave owns a run of output rows.  The request of its first row is found
// by binary search over cu_out (scalar); each tile's lanes advance from there
// to their own row's request.
template <typename V, int NKV, int TPL = kTasksPerLane>
__global__ __launch_bounds__(kBlock) void gather_kernel(GatherArgs a) {
    const int lane = lane_id();
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
        if (a.cu_out[0] != 0 || a.cu_out[a.num_reqs] != a.out_rows) atomicOr(a.flags, UKV_FLAG_LAYOUT);
    }
    const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + wave_in_block();
    const int64_t per_wave = (int64_t)a.tile_rows * a.tiles_per_wave;
    const int64_t o_begin = wave * per_wave;
    const uint64_t view0 = (uint64_t)blockIdx.y * a.layer_base_step;
    uint8_t *const out_l[2] = {a.out[0] + (int64_t)blockIdx.y * a.out_layer_stride,
                               a.out[1] + (int64_t)blockIdx.y * a.out_layer_stride};
    if (o_begin >= a.out_rows) return;
    const int64_t o_end = o_begin + per_wave < a.out_rows ? o_begin + per_wave : a.out_rows;

    // r = number of requests r' >= 1 with cu_out[r'] <= o_begin (upper bound)
    int32_t lo = 0, hi = a.num_reqs;
    while (lo < hi) {
        const int32_t mid = (lo + hi) >> 1;
        if (a.cu_out[mid + 1] <= o_begin)
            lo = mid + 1;
        else
            hi = mid;
    }
    int32_t r = lo;
    uint32_t bad = 0;
    const int tasks = a.tile_rows * a.vecs;
    for (int64_t o0 = o_begin; o0 < o_end; o0 += a.tile_rows) {
        // lane k: the source row of output row o0 + k (-1: skipped)
        int32_t src_row = -1;
        int32_t rk = r;
        const int64_t o = o0 + lane;
        if (lane < a.tile_rows && o < o_end) {
            while (rk < a.num_reqs && a.cu_out[rk + 1] <= o) ++rk;
            src_row = gather_source_row(a, o, rk, bad);
        }
        r = __builtin_amdgcn_readlane(rk, a.tile_rows - 1);  // rows grow with the lane: the tile's last request
        for (int base = 0; base < tasks; base += kWave * TPL) {
            V buf[NKV][TPL];
            int32_t rows[TPL];
            int32_t ks[TPL];
            int32_t cs[TPL];
#pragma unroll
            for (int j = 0; j < TPL; ++j) {
                const int t = base + lane + j * kWave;
                const int k = t / a.vecs;
                const int c = t - k * a.vecs;
                const int32_t row = __shfl(src_row, k < kWave ? k : 0);
                rows[j] = (t < tasks) ? row : -1;
                ks[j] = k;
                cs[j] = c;
                if (rows[j] >= 0) {
#pragma unroll
                    for (int h = 0; h < NKV; ++h)
                        buf[h][j] = reinterpret_cast<const V *>(a.pool + a.base[h] + view0 +
                                                                (uint64_t)(uint32_t)rows[j] * a.row_bytes)[c];
                }
            }
#pragma unroll
            for (int j = 0; j < TPL; ++j) {
                if (rows[j] >= 0) {
#pragma unroll
                    for (int h = 0; h < NKV; ++h)
                        put<true>(&reinterpret_cast<V *>(out_l[h] + (uint64_t)(o0 + ks[j]) * a.row_bytes)[cs[j]],
                                  buf[h][j]);
                }
            }
        }
    }
    if (bad != 0 && blockIdx.y == 0) atomicOr(a.flags, bad);
}

// ----------------------------------------------------------------------------
// move (DKV 关键文件: _move_kv_cache_impl, a 3-D row copy per layer, K and V)
// ----------------------------------------------------------------------------
struct MoveArgs {
    uint8_t *pool;
    uint64_t base0;       // byte offset of view (layer_begin, kv 0)
    uint64_t layer_step;  // bytes between consecutive layers' views
    uint64_t kv_step;     // bytes between a layer's K and V views
    const int32_t *dst;
    const int32_t *src;
    int64_t n;
    int32_t nl;
    uint32_t n_rows;
    uint32_t page_stride;
    uint32_t ps;
    uint32_t row_bytes;
    int32_t vecs;
    int32_t tile_units;  // (pair, layer) units per tile, <= 64
    uint32_t *flags;
};

// Tiles of `tile_units` units u = (pair i, layer l), u = i * nl + l: lane k
// resolves unit u0 + k to its source and destination row offsets (K view;
// V is kv_step further), broadcast as two 32-bit halves with __shfl; then
// every lane copies up to TPL chunks per round, K and V, loads first.
template <typename V, int NKV, int TPL>
__global__ __launch_bounds__(kBlock) void move_kernel(MoveArgs a) {
    const int lane = lane_id();
    const int64_t total = a.n * a.nl;
    const int64_t u0 = ((int64_t)blockIdx.x * kWavesPerBlock + wave_in_block()) * a.tile_units;
    if (u0 >= total) return;
    int64_t s_off = -1, d_off = -1;
    bool bad = false;
    if (lane < a.tile_units && u0 + lane < total) {
        const int64_t u = u0 + lane;
        const int64_t i = u / a.nl;
        const int32_t l = (int32_t)(u - i * a.nl);
        const int32_t d = a.dst[i];
        const int32_t s = a.src[i];
        if (kernel_facing(d, a.n_rows, a.page_stride, a.ps) && kernel_facing(s, a.n_rows, a.page_stride, a.ps)) {
            const uint64_t layer_base = a.base0 + (uint64_t)l * a.layer_step;
            s_off = (int64_t)(layer_base + (uint64_t)(uint32_t)s * a.row_bytes);
            d_off = (int64_t)(layer_base + (uint64_t)(uint32_t)d * a.row_bytes);
        } else {
            bad = (l == 0);  // one report per pair
        }
    }
    const int tasks = a.tile_units * a.vecs;
    for (int base = 0; base < tasks; base += kWave * TPL) {
        V buf[NKV][TPL];
        int64_t dst_off[TPL];
        int32_t cs[TPL];
#pragma unroll
        for (int j = 0; j < TPL; ++j) {
            const int t = base + lane + j * kWave;
            const int k = t / a.vecs;
            const int c = t - k * a.vecs;
            const int kk = k < kWave ? k : 0;
            const uint32_t s_lo = (uint32_t)__shfl((int)(uint32_t)s_off, kk);
            const uint32_t s_hi = (uint32_t)__shfl((int)(uint32_t)(s_off >> 32), kk);
            const uint32_t d_lo = (uint32_t)__shfl((int)(uint32_t)d_off, kk);
            const uint32_t d_hi = (uint32_t)__shfl((int)(uint32_t)(d_off >> 32), kk);
            const int64_t so = (int64_t)(((uint64_t)s_hi << 32) | s_lo);
            const int64_t dof = (int64_t)(((uint64_t)d_hi << 32) | d_lo);
            dst_off[j] = (t < tasks && so >= 0) ? dof : -1;
            cs[j] = c;
            if (dst_off[j] >= 0) {
#pragma unroll
                for (int h = 0; h < NKV; ++h)
                    buf[h][j] = reinterpret_cast<const V *>(a.pool + so + h * a.kv_step)[c];
            }
        }
#pragma unroll
        for (int j = 0; j < TPL; ++j) {
            if (dst_off[j] >= 0) {
#pragma unroll
                for (int h = 0; h < NKV; ++h)
                    put<true>(&reinterpret_cast<V *>(a.pool + dst_off[j] + h * a.kv_step)[cs[j]], buf[h][j]);
            }
        }
    }
    if (bad) atomicOr(a.flags, UKV_FLAG_BAD_ID);
}

// ----------------------------------------------------------------------------
// row-piece kernels: store, gather and move of rows that are whole 1 KiB pieces
// ----------------------------------------------------------------------------
// For rows of 2^k KiB (k >= 0) moved as 16-byte vectors, a wave copies one
// 1 KiB piece of one view's row (gather: two consecutive pieces): one
// non-temporal load and one non-temporal store per lane, so the memory system
// sees short, fully coalesced accesses issued in address order from many
// waves.  Measured on MI355X against the tile kernels above, same pools and
// inputs, bit-identical results (% of 8 TB/s, medians of interleaved runs):
// prefill-shape store of 2 KiB rows, 32 layers in one launch, 71 -> 75%; its
// gather-back 74 -> 80.5%; the 65,536-row move 71 -> 79%; the 70B-shape move
// 75 -> 79%; the 1 KiB-row hybrid gather 73 -> 77%; a decode-size store launch
// (256 rows) 14 -> 7.6 us.  One case goes the other way: the decode gather whose
// requests share pages (most reads hit the Infinity Cache) ran at 81% with the
// tile kernel's 8 KiB per wave and runs at 78% here.  Plain loads instead of
// non-temporal ones lost 4-5 points on the gather-back; 2 and 4 KiB per wave
// (K and V of a piece together, whole rows, pairs of rows) and a wave-wide
// request search instead of the binary search were no faster.  1 KiB rows
// keep the tile store (75 vs 74%).  A piece index w = (row, view, piece) with
// the piece count a power of two splits into shifts.
constexpr int kPieceVecs = kWave;  // 16-byte vectors per piece: 1 KiB

// Waves MI355X-class GPUs hold at once for these kernels: CUs x 32.  The CU count is
// read once per device.
int64_t resident_waves() {
    static int64_t cache[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256 * 32;
    if (cache[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cache[dev] = (int64_t)cus * 32;
    }
    return cache[dev];
}

// Pieces per store wave for a launch of `pieces` 1 KiB pieces: `base` for
// launches of more than eight rounds of resident waves (there one piece per
// wave measured fastest); a small launch gets enough per wave (at most 8) to
// finish in one round, so it pays one chain of load latencies instead of
// several.  Measured on the 32-layer decode store (256 rows x 32 layers, 67 MB,
// four pieces per wave): 13.1-13.6 against 13.6-14.2 us.  Small launches of
// 2 KiB rows now take the row-group store instead (11.7-11.8 us); rows of 4 KiB
// and more keep this.
int pieces_per_wave(int64_t pieces, int base) {
    const int64_t round = resident_waves();
    if (pieces > 8 * round) return base;
    int k = base;
    while (k < 8 && pieces > round * k) k *= 2;
    return k;
}

// Loads per lane of the row-group store (V / 8 for rows of V 16-byte vectors,
// 64 < V < 128, V a multiple of 8), or 0 when the rows are no such shape.
int group_loads(int vec_bytes, uint64_t row_bytes) {
    if (vec_bytes != 16 || row_bytes % 128 != 0 || row_bytes <= 1024 || row_bytes >= 2048) return 0;
    return (int)(row_bytes / 128);
}

// Launch kernel template K<NKV, J> for J = loads per lane (9..16) through f(tag).
template <typename F>
void with_group_loads(int j, F &&f) {
    switch (j) {
        case 16: f(std::integral_constant<int, 16>()); break;
        case 9: f(std::integral_constant<int, 9>()); break;
        case 10: f(std::integral_constant<int, 10>()); break;
        case 11: f(std::integral_constant<int, 11>()); break;
        case 12: f(std::integral_constant<int, 12>()); break;
        case 13: f(std::integral_constant<int, 13>()); break;
        case 14: f(std::integral_constant<int, 14>()); break;
        default: f(std::integral_constant<int, 15>()); break;
    }
}

// log2 of the 1 KiB pieces per row, or -1 when rows are not 2^k whole pieces of
// 16-byte vectors (then the row-group store or the tile kernels run).
int piece_shift(int vec_bytes, uint64_t row_bytes) {
    if (vec_bytes != 16 || row_bytes % 1024 != 0) return -1;
    const uint64_t pcs = row_bytes / 1024;
    int lp = 0;
    while ((1ull << lp) < pcs) ++lp;
    return (1ull << lp) == pcs ? lp : -1;
}

// K_view[l][ids[i]] = k[l][i], V_view[l][ids[i]] = v[l][i]: piece u = (entry, view,
// piece of the row) = u >> (lp + log2 NKV), (u >> lp) & (NKV - 1), u & (2^lp - 1),
// for the layer of logical grid row y.  Wave w copies pieces K*w .. K*w + K-1,
// their loads issued together (K > 1 only for launches small enough to finish in
// one round of resident waves: see pieces_per_wave).
//
// XL (launches of several layers): workgroups go to the 8 XCDs round-robin in
// launch order, and the workgroups of one XCD take consecutive logical blocks, so
// each XCD stores its own run of layers instead of every XCD working on the same
// layer.  Measured on the 32-layer prefill store (32,768 rows x 32 layers, 8.6 GB)
// on six boxes: 1,328-1,406 us (76-81% of 8 TB/s) against 1,404-1,443 us in launch
// order, with a twentieth of the cycles L2's writes waited for DRAM credits (2.8e6
// against 5.75e7 per launch).  The same order made the gathers 5-9% and the row move
// 2% slower, and did not speed up the single-layer prefill store: those keep launch
// order.  The
// kernel recomputes the grid from its arguments, and the layer count sits in the
// argument block's alignment gap: two more argument words, which took the block past
// 128 bytes, made the latency-bound 256-row decode store 2.7-2.8 us against 2.5 us.
template <int NKV, int K, bool XL>
__global__ __launch_bounds__(kBlock) void store_piece_kernel(StoreArgs a, int lp) {
    const int lane = lane_id();
    constexpr int hb = NKV == 2 ? 1 : 0;
    uint32_t x = blockIdx.x, y = blockIdx.y;
    if constexpr (XL) {  // the host's grid: gx = ceil(ceil(pieces / K) / waves per block); gx * layers < 2^32
        const uint32_t gx = (uint32_t)(((((a.n << hb) << lp) + K - 1) / K + kWavesPerBlock - 1) / kWavesPerBlock);
        const uint32_t l = xcd_logical_block(y * gx + x, gx * a.layers);
        y = l / gx;
        x = l - y * gx;
    }
    const int64_t u0 = ((int64_t)x * kWavesPerBlock + wave_in_block()) * K;
    if ((u0 >> (lp + hb)) >= a.n) return;
    const int64_t src0 = (int64_t)y * a.src_layer_stride;
    const uint64_t view0 = (uint64_t)y * a.layer_base_step;
    u32x4 buf[K];
    u32x4 *dst[K];
    bool bad = false;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int64_t u = u0 + k;
        const int64_t i = u >> (lp + hb);
        dst[k] = nullptr;
        if (i >= a.n) continue;
        const int h = (int)((u >> lp) & (NKV - 1));
        const int64_t p = u & ((1ll << lp) - 1);
        const int32_t id = a.ids[i];
        if (!kernel_facing(id, a.n_rows, a.page_stride, a.ps)) {
            bad = true;
            continue;
        }
        const int64_t c = p * kPieceVecs + lane;
        buf[k] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(a.src[h] + src0 + i * a.src_stride) + c);
        dst[k] = reinterpret_cast<u32x4 *>(a.pool + a.base[h] + view0 + (uint64_t)(uint32_t)id * a.row_bytes) + c;
    }
#pragma unroll
    for (int k = 0; k < K; ++k)
        if (dst[k] != nullptr) __builtin_nontemporal_store(buf[k], dst[k]);
    if (bad && lane == 0 && y == 0) atomicOr(a.flags, UKV_FLAG_BAD_ID);
}

// Each wave copies K consecutive pieces u = K*w, ... of the (output row, view,
// piece) sequence (K = 2: a whole 2 KiB row of one view, or, for 1 KiB rows, the
// K and the V row of one output row).  The request of the first
// row is found by binary search over cu_out (scalar); the others advance from it.
template <int NKV, int K>
__global__ __launch_bounds__(kBlock) void gather_piece_kernel(GatherArgs a, int lp) {
    const int lane = lane_id();
    constexpr int hb = NKV == 2 ? 1 : 0;
    const int64_t u0 = ((int64_t)blockIdx.x * kWavesPerBlock + wave_in_block()) * K;
    const int64_t o0 = u0 >> (lp + hb);
    if (o0 >= a.out_rows) return;
    const uint64_t view0 = (uint64_t)blockIdx.y * a.layer_base_step;
    const int64_t out0 = (int64_t)blockIdx.y * a.out_layer_stride;
    int32_t lo = 0, hi = a.num_reqs;  // r = number of requests r' >= 1 with cu_out[r'] <= o0
    while (lo < hi) {
        const int32_t mid = (lo + hi) >> 1;
        if (a.cu_out[mid + 1] <= o0)
            lo = mid + 1;
        else
            hi = mid;
    }
    int32_t r = lo;
    uint32_t bad = 0;
    u32x4 buf[K];
    u32x4 *dst[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int64_t u = u0 + k;
        const int64_t o = u >> (lp + hb);
        dst[k] = nullptr;
        if (o >= a.out_rows) continue;
        while (r < a.num_reqs && a.cu_out[r + 1] <= o) ++r;
        const int32_t row = gather_source_row(a, o, r, bad);
        if (row < 0) continue;
        const int h = (int)((u >> lp) & (NKV - 1));
        const int64_t c = (u & ((1ll << lp) - 1)) * kPieceVecs + lane;
        buf[k] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(a.pool + a.base[h] + view0 + (uint64_t)(uint32_t)row * a.row_bytes) + c);
        dst[k] = reinterpret_cast<u32x4 *>(a.out[h] + out0 + o * (int64_t)a.row_bytes) + c;
    }
#pragma unroll
    for (int k = 0; k < K; ++k)
        if (dst[k] != nullptr) __builtin_nontemporal_store(buf[k], dst[k]);
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0 &&
        (a.cu_out[0] != 0 || a.cu_out[a.num_reqs] != a.out_rows))
        bad |= UKV_FLAG_LAYOUT;  // the launch's one check of the ragged layout as a whole
    if (bad != 0 && lane == 0 && blockIdx.y == 0) atomicOr(a.flags, bad);
}

// Stores of rows of V = 8 J 16-byte vectors with 64 < V < 128 (1,152 to 1,920
// bytes; the MLA latent of 576 bf16 among them), which are no whole number of
// 1 KiB pieces, and small launches of 2 KiB rows (V = 128; each load then stays
// within one row): a wave copies kGroupRows = 8 consecutive entries of one view as J
// loads and J stores per lane, lane l of load j taking vector f = 64 j + l of the
// 8 rows' 8 V vectors (row f / V, vector f % V).  Every load and store moves a
// whole 1 KiB (the sources are contiguous rows); one instruction spans at most
// two rows, whose ids are wave-uniform and come through the scalar cache.
// Measured on the hybrid workload's MLA store (1.05 M latents, 2.43 GB): 376-383
// us (80% of 8 TB/s) in 12 of 14 runs (431 and 475 us in the other two), against
// 427-469 us for the tile kernel in 9 of 12 runs (377-379 us in three).  Groups of
// whole 1 KiB rows ran 45% slower than the tiles, of 2 KiB rows faster on the small
// 32-layer decode store but slower on the single-layer prefill store, so only these
// widths take them.  The compiler waits for every memory operation before each
// store here; a variant with the loads issued unconditionally, one wait for them
// and then the stores back to back ran at 431 us, and a gather built the same
// way stayed behind the tile gather (434-455 against 404-427 us).
constexpr int kGroupRows = 8;

template <int NKV, int J>
__global__ __launch_bounds__(kBlock) void store_group_kernel(StoreArgs a) {
    constexpr int V = 8 * J;
    constexpr int hb = NKV == 2 ? 1 : 0;
    const int lane = lane_id();
    const int64_t w = (int64_t)blockIdx.x * kWavesPerBlock + wave_in_block();
    const int64_t i0 = (w >> hb) * kGroupRows;
    if (i0 >= a.n) return;
    const int h = (int)(w & (NKV - 1));
    int32_t id[kGroupRows];
    bool bad = false;
#pragma unroll
    for (int r = 0; r < kGroupRows; ++r) {
        id[r] = -1;
        if (i0 + r < a.n) {
            const int32_t v = a.ids[i0 + r];
            if (kernel_facing(v, a.n_rows, a.page_stride, a.ps))
                id[r] = v;
            else
                bad = true;
        }
    }
    // the view's pointers by fixed indices, not through a runtime index into the
    // argument array
    const uint8_t *src = (h == 0 ? a.src[0] : a.src[1]) + (int64_t)blockIdx.y * a.src_layer_stride + i0 * a.src_stride;
    uint8_t *dst = a.pool + (h == 0 ? a.base[0] : a.base[1]) + (uint64_t)blockIdx.y * a.layer_base_step;
    u32x4 buf[J];
    u32x4 *to[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int lo = (64 * j) / V;  // the load's first row of the group; its second is lo + 1
        const int f = 64 * j + lane;
        const bool second = f >= (lo + 1) * V;
        const int r = second ? lo + 1 : lo;
        const int c = f - r * V;
        const int32_t row = second ? id[lo + 1 < kGroupRows ? lo + 1 : lo] : id[lo];
        to[j] = nullptr;
        if (row < 0) continue;  // past n, or a bad id
        buf[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src + r * a.src_stride) + c);
        to[j] = reinterpret_cast<u32x4 *>(dst + (uint64_t)(uint32_t)row * a.row_bytes) + c;
    }
#pragma unroll
    for (int j = 0; j < J; ++j)
        if (to[j] != nullptr) __builtin_nontemporal_store(buf[j], to[j]);
    if (bad && lane == 0 && h == 0 && blockIdx.y == 0) atomicOr(a.flags, UKV_FLAG_BAD_ID);
}

// view[l][dst[i]] = view[l][src[i]]: wave w copies piece w & (2^lp - 1) of view
// (w >> lp) & (NKV - 1) of unit u = w >> (lp + log2 NKV) = pair * nl + layer
// (layers of one pair are neighbours: their rows share the pair's two pages).
template <int NKV>
__global__ __launch_bounds__(kBlock) void move_piece_kernel(MoveArgs a, int lp) {
    const int lane = lane_id();
    const int64_t w = (int64_t)blockIdx.x * kWavesPerBlock + wave_in_block();
    constexpr int hb = NKV == 2 ? 1 : 0;
    const int64_t u = w >> (lp + hb);
    if (u >= a.n * a.nl) return;
    const int h = (int)((w >> lp) & (NKV - 1));
    const int64_t p = w & ((1ll << lp) - 1);
    const int64_t i = u / a.nl;
    const int32_t l = (int32_t)(u - i * a.nl);
    const int32_t d = a.dst[i];
    const int32_t s = a.src[i];
    if (!kernel_facing(d, a.n_rows, a.page_stride, a.ps) || !kernel_facing(s, a.n_rows, a.page_stride, a.ps)) {
        if (lane == 0 && l == 0 && h == 0 && p == 0) atomicOr(a.flags, UKV_FLAG_BAD_ID);  // one report per pair
        return;
    }
    const uint64_t view = a.base0 + (uint64_t)l * a.layer_step + (uint64_t)h * a.kv_step;
    const int64_t c = p * kPieceVecs + lane;
    const u32x4 *from = reinterpret_cast<const u32x4 *>(a.pool + view + (uint64_t)(uint32_t)s * a.row_bytes) + c;
    u32x4 *to = reinterpret_cast<u32x4 *>(a.pool + view + (uint64_t)(uint32_t)d * a.row_bytes) + c;
    __builtin_nontemporal_store(__builtin_nontemporal_load(from), to);
}

// ----------------------------------------------------------------------------
// page relocation and table rewrite (compaction: DKV alloc excerpt and 关键文件)
// ----------------------------------------------------------------------------
struct PageMoveArgs {
    uint8_t *pool;
    uint64_t anchor;
    uint64_t page_bytes;
    const int32_t *dst;
    const int32_t *src;
    int64_t n;
    int64_t num_pages;
    int64_t vecs;       // page_bytes / sizeof(V)
    int64_t segs;       // segments per page
    uint32_t *flags;
    uint32_t grid;      // workgroups in the launch (< 2^32), for the XCD order
};

// A page's rows on every layer, K and V, are one contiguous envelope, so a
// page relocation is a straight copy of page_bytes.  One wave per
// (pair, 64 * TPL-chunk segment); the pair index is wave-uniform, so the
// page lookups are scalar loads.  The workgroups of one XCD take consecutive
// blocks (XCD order): each XCD copies its own run of pages.  Measured on the
// compaction of 1,789 pages of 2 MiB (7.5 GB), three A/B pairs in one run:
// 1,152-1,158 us (81% of 8 TB/s) against 1,231-1,234 us (76%) in launch order,
// where the eight XCDs copy the same few pages at once.
template <typename V, int TPL>
__global__ __launch_bounds__(kBlock) void move_pages_kernel(PageMoveArgs a) {
    const int64_t w = (int64_t)xcd_logical_block(blockIdx.x, a.grid) * kWavesPerBlock + wave_in_block();
    const int64_t pair = w / a.segs;
    if (pair >= a.n) return;
    const int64_t seg = w - pair * a.segs;
    const int lane = lane_id();
    const int32_t d = a.dst[pair];
    const int32_t s = a.src[pair];
    if (d < 0 || d >= a.num_pages || s < 0 || s >= a.num_pages) {
        if (lane == 0 && seg == 0) atomicOr(a.flags, UKV_FLAG_BAD_ID);
        return;
    }
    const V *src = reinterpret_cast<const V *>(a.pool + a.anchor + (uint64_t)s * a.page_bytes);
    V *dst = reinterpret_cast<V *>(a.pool + a.anchor + (uint64_t)d * a.page_bytes);
    const int64_t c0 = seg * (int64_t)(kWave * TPL) + lane;
    V buf[TPL];
#pragma unroll
    for (int j = 0; j < TPL; ++j) {
        const int64_t c = c0 + (int64_t)j * kWave;
        if (c < a.vecs) buf[j] = __builtin_nontemporal_load(&src[c]);
    }
#pragma unroll
    for (int j = 0; j < TPL; ++j) {
        const int64_t c = c0 + (int64_t)j * kWave;
        if (c < a.vecs) put<true>(&dst[c], buf[j]);
    }
}

// v2p[virt[i]] = phys[i]; virt past the table or phys outside [-1, num_pages)
// skip the entry and raise UKV_FLAG_SLOT_RANGE.
__global__ __launch_bounds__(kBlock) void remap_pages_kernel(int32_t *v2p, int64_t v2p_len, const int32_t *virt,
                                                            const int32_t *phys, int64_t n, int64_t num_pages,
                                                            uint32_t *flags) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= n) return;
    const int32_t v = virt[i];
    const int32_t p = phys[i];
    if (v < 0 || v >= v2p_len || p < -1 || p >= num_pages) {
        atomicOr(flags, UKV_FLAG_SLOT_RANGE);
        return;
    }
    v2p[v] = p;
}

// Sliding-window eviction: thread per block-table entry (r, i); page i of
// request r is evicted when it lies wholly before the window.
__global__ __launch_bounds__(kBlock) void evict_window_kernel(int32_t *mapping, int64_t map_len, const int32_t *table,
                                                             int64_t bt_stride, const int32_t *seq_lens,
                                                             int32_t num_reqs, int32_t window, int64_t ps,
                                                             uint32_t *flags) {
    const int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (e >= (int64_t)num_reqs * bt_stride) return;
    const int64_t r = e / bt_stride;
    const int64_t i = e - r * bt_stride;
    const int64_t len = seq_lens[r];
    if (len <= window || (i + 1) * ps > len - window) return;
    const int32_t page = table[e];
    if (page < 0) return;
    if (page >= map_len) {
        atomicOr(flags, UKV_FLAG_SLOT_RANGE);
        return;
    }
    mapping[page] = -1;
}

__global__ void flags_fetch_clear_kernel(uint32_t *f) {
    if (threadIdx.x == 0) f[1] = atomicExch(&f[0], 0u);
}

// ----------------------------------------------------------------------------
// host helpers
// ----------------------------------------------------------------------------

// Debug validation: the id arrays of a store (b == nullptr) or a move, copied to
// the host on the call's stream, checked for rows that would race.
int debug_check(const ukv_pool *pool, const int32_t *a_dev, const int32_t *b_dev, int64_t n, hipStream_t stream,
                const char *who) {
    if (!pool->debug || n == 0) return UKV_OK;
    std::vector<int32_t> a((size_t)n), b(b_dev != nullptr ? (size_t)n : 0);
    hipError_t e = hipMemcpyAsync(a.data(), a_dev, (size_t)n * 4, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess && b_dev != nullptr)
        e = hipMemcpyAsync(b.data(), b_dev, (size_t)n * 4, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(UKV_ERR_HIP, "%s: debug validation copy: %s", who, hipGetErrorString(e));
    return b_dev == nullptr ? ukv::check_store_ids(a.data(), n, who) : ukv::check_move_ids(a.data(), b.data(), n, who);
}

// Largest power of two <= 16 dividing every value: the widest integer vector
// every row access of a call can use.
int vec_bytes_for(std::initializer_list<uint64_t> values) {
    uint64_t acc = 16;
    for (uint64_t v : values) {
        while (acc > 1 && (v % acc) != 0) acc >>= 1;
    }
    return (int)acc;
}

template <int NKV, typename F>
int dispatch_vec(int vb, F &&f) {
    switch (vb) {
        case 16: return f((u32x4 *)nullptr);
        case 8: return f((u32x2 *)nullptr);
        case 4: return f((uint32_t *)nullptr);
        case 2: return f((uint16_t *)nullptr);
        default: return f((uint8_t *)nullptr);
    }
}

// Tile shape of a store / gather launch.  One tile per wave; the tile's rows
// are chosen so that each lane has a few 16-byte loads in flight: about 6
// (K and V together) for a gather, about 3 for a store, whose sources are
// plain contiguous rows.  Chunks per lane per round (TPL) is 4, or 8 when a
// tile needs more than 4.  Measured on MI355X against 1-8 rows per tile,
// 1-16 tiles per wave and TPL 2-8, for 2,048-byte (K+V), 1,024-byte (K+V)
// and 1,152-byte (MLA) rows at 32 K to 1.2 M rows per launch: within a few
// percent of the best shape for every one.
struct Tiling {
    int32_t tile_rows;
    int32_t tiles_per_wave;
    int32_t tpl;
    int64_t waves;  // one tile per wave
    int64_t grid;   // workgroups of kWavesPerBlock waves
};

Tiling tiling_for(int32_t vecs, int32_t nkv, int64_t rows, bool gather) {
    Tiling t;
    const int64_t target = gather ? 6 * kWave : 3 * kWave;  // 16-byte loads per wave per round, K and V together
    int64_t tr = gather ? (target + (int64_t)nkv * vecs / 2) / ((int64_t)nkv * vecs)  // rounded
                        : target / ((int64_t)nkv * vecs);                             // rounded down
    t.tile_rows = (int32_t)(tr < 1 ? 1 : (tr > kWave ? kWave : tr));
    t.tpl = gather && (int64_t)t.tile_rows * vecs > 4 * kWave ? 8 : (gather ? 4 : 8);
    t.tiles_per_wave = 1;
    t.waves = (rows + t.tile_rows - 1) / t.tile_rows;
    t.grid = (t.waves + kWavesPerBlock - 1) / kWavesPerBlock;
    return t;
}

}  // namespace

// ----------------------------------------------------------------------------
// C ABI
// ----------------------------------------------------------------------------
extern "C" {

int ukv_pool_create(const ukv_subpool_spec *specs, int32_t n_specs, int64_t page_size, void *raw_dev,
                    uint64_t raw_bytes, ukv_pool **out) {
    if (out == nullptr) return fail(UKV_ERR_INVALID_ARG, "ukv_pool_create: null out");
    ukv_plan plan;
    int rc = ukv::plan_pool(specs, n_specs, page_size, &plan);
    if (rc != UKV_OK) return rc;
    if (raw_dev == nullptr) return fail(UKV_ERR_INVALID_ARG, "ukv_pool_create: null raw buffer");
    if (((uintptr_t)raw_dev & 15u) != 0)
        return fail(UKV_ERR_ALIGNMENT, "ukv_pool_create: raw buffer %p is not 16-byte aligned", raw_dev);
    if (raw_bytes < plan.required_bytes)
        return fail(UKV_ERR_TAIL_PAD,
                    "ukv_pool_create: raw buffer holds %llu bytes but the pool needs %llu: %llu of page envelopes "
                    "plus a %llu-byte view tail pad (one page envelope, the max over the sub-pool specs)",
                    (unsigned long long)raw_bytes, (unsigned long long)plan.required_bytes,
                    (unsigned long long)plan.envelope_bytes, (unsigned long long)plan.tail_pad_bytes);
    hipPointerAttribute_t attr;
    std::memset(&attr, 0, sizeof(attr));
    if (hipPointerGetAttributes(&attr, raw_dev) != hipSuccess || attr.type != hipMemoryTypeDevice) {
        (void)hipGetLastError();
        return fail(UKV_ERR_INVALID_ARG, "ukv_pool_create: raw buffer %p is not device memory", raw_dev);
    }
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != attr.device)
        return fail(UKV_ERR_INVALID_ARG, "ukv_pool_create: buffer lives on device %d, current device is %d",
                    attr.device, dev);
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)raw_dev) == hipSuccess && base != nullptr) {
        if ((uintptr_t)raw_dev + raw_bytes > (uintptr_t)base + size)
            return fail(UKV_ERR_INVALID_ARG,
                        "ukv_pool_create: %llu bytes from %p run past the device allocation (%zu bytes at %p)",
                        (unsigned long long)raw_bytes, raw_dev, size, (void *)base);
    } else {
        (void)hipGetLastError();
    }
    ukv_pool *p = new (std::nothrow) ukv_pool;
    if (p == nullptr) return fail(UKV_ERR_INVALID_ARG, "ukv_pool_create: out of host memory");
    std::memset(p, 0, sizeof(*p));
    std::memcpy(p->spec, specs, sizeof(ukv_subpool_spec) * (size_t)n_specs);
    p->plan = plan;
    p->raw = (uint8_t *)raw_dev;
    p->raw_bytes = raw_bytes;
    p->device = dev;
    hipError_t e = hipMalloc((void **)&p->flags_dev, 2 * sizeof(uint32_t));
    if (e == hipSuccess) e = hipMemset(p->flags_dev, 0, 2 * sizeof(uint32_t));
    if (e != hipSuccess) {
        if (p->flags_dev) (void)hipFree(p->flags_dev);
        delete p;
        return fail(UKV_ERR_HIP, "ukv_pool_create: flag words: %s", hipGetErrorString(e));
    }
    *out = p;
    return UKV_OK;
}

int ukv_pool_destroy(ukv_pool *pool) {
    if (pool == nullptr) return UKV_OK;
    hipError_t e = hipFree(pool->flags_dev);
    delete pool;
    if (e != hipSuccess) return fail(UKV_ERR_HIP, "ukv_pool_destroy: %s", hipGetErrorString(e));
    return UKV_OK;
}

int ukv_pool_get_plan(const ukv_pool *pool, ukv_plan *out) {
    if (pool == nullptr || out == nullptr) return fail(UKV_ERR_INVALID_ARG, "ukv_pool_get_plan: null argument");
    *out = pool->plan;
    return UKV_OK;
}

int ukv_pool_view(const ukv_pool *pool, int32_t sub, int32_t layer, int32_t kv, ukv_view *out) {
    if (pool == nullptr || out == nullptr) return fail(UKV_ERR_INVALID_ARG, "ukv_pool_view: null argument");
    if (sub < 0 || sub >= pool->plan.n_sub)
        return fail(UKV_ERR_INVALID_ARG, "ukv_pool_view: sub-pool %d outside [0, %d)", sub, pool->plan.n_sub);
    return ukv::view_of(pool->plan, pool->spec[sub], sub, layer, kv, out);
}

static int translate_common(const ukv_pool *pool, int32_t sub, const void *in, uint64_t in_elem, int64_t n,
                            const int32_t *v2p, int64_t v2p_len, int32_t *out, hipStream_t stream, bool pages,
                            const char *who, bool internal = false) {
    int rc = check_pool_call(pool, sub, who);
    if (rc != UKV_OK) return rc;
    if (n < 0 || n > kMaxGrid) return fail(UKV_ERR_INVALID_ARG, "%s: n=%lld outside [0, 2^31)", who, (long long)n);
    if (n == 0) return UKV_OK;
    if (in == nullptr || out == nullptr) return fail(UKV_ERR_INVALID_ARG, "%s: null input or output", who);
    if (v2p != nullptr && v2p_len < 0) return fail(UKV_ERR_INVALID_ARG, "%s: v2p_len < 0", who);
    // out may be the input buffer itself (same start): int32 ids over int64 slots take the
    // one-workgroup in-place kernel; any other overlap is refused
    const bool same = (const void *)out == in;
    if (!same && ranges_overlap(in, (uint64_t)n * in_elem, out, (uint64_t)n * sizeof(int32_t)))
        return fail(UKV_ERR_INVALID_ARG, "%s: output overlaps the input without starting where it starts", who);
    if (v2p != nullptr && ranges_overlap(v2p, (uint64_t)v2p_len * 4, out, (uint64_t)n * sizeof(int32_t)))
        return fail(UKV_ERR_INVALID_ARG, "%s: output overlaps the v2p table", who);
    const ukv_subpool_spec &s = pool->spec[sub];
    const ukv_subpool_plan &q = pool->plan.sub[sub];
    TranslateArgs a;
    std::memset(&a, 0, sizeof(a));
    a.slots = (const int64_t *)in;
    a.pages = (const int32_t *)in;
    a.v2p = v2p;
    a.out = out;
    a.flags = pool->flags_dev;
    a.n = n;
    a.v2p_len = v2p == nullptr ? 0 : v2p_len;
    a.ps = pool->plan.page_size;
    a.bpp = q.blocks_per_page;
    a.page_stride = pool->plan.page_size * q.blocks_per_page;
    a.num_pages = s.num_pages;
    a.internal = internal ? 1 : 0;
    const unsigned grid = (unsigned)((n + kBlock - 1) / kBlock);
    if (pages)
        hipLaunchKernelGGL(translate_pages_kernel, dim3(grid), dim3(kBlock), 0, stream, a);
    else if (same)
        hipLaunchKernelGGL(translate_inplace_kernel, dim3(1), dim3(kInPlaceBlock), 0, stream, a);
    else
        hipLaunchKernelGGL(translate_slots_kernel, dim3(grid), dim3(kBlock), 0, stream, a);
    return check_launch(who);
}

int ukv_translate_loc_for_kernel(const ukv_pool *pool, int32_t sub, const int64_t *slots_dev, int64_t n,
                                 const int32_t *v2p_dev, int64_t v2p_len, int32_t *out_dev, hipStream_t stream) {
    return translate_common(pool, sub, slots_dev, sizeof(int64_t), n, v2p_dev, v2p_len, out_dev, stream, false,
                            "ukv_translate_loc_for_kernel");
}

int ukv_translate_loc(const ukv_pool *pool, int32_t sub, const int64_t *slots_dev, int64_t n, const int32_t *v2p_dev,
                      int64_t v2p_len, int32_t *out_dev, hipStream_t stream) {
    return translate_common(pool, sub, slots_dev, sizeof(int64_t), n, v2p_dev, v2p_len, out_dev, stream, false,
                            "ukv_translate_loc", true);
}

int ukv_translate_pages_for_kernel(const ukv_pool *pool, int32_t sub, const int32_t *pages_dev, int64_t n,
                                   const int32_t *v2p_dev, int64_t v2p_len, int32_t *out_dev, hipStream_t stream) {
    return translate_common(pool, sub, pages_dev, sizeof(int32_t), n, v2p_dev, v2p_len, out_dev, stream, true,
                            "ukv_translate_pages_for_kernel");
}

// Checks a layer range [begin, begin + count*step) with step >= 1 against the
// sub-pool and returns the view byte step between consecutive layers in it.
static int check_layer_range(const ukv_pool *pool, int32_t sub, int32_t begin, int32_t count, int32_t step,
                             const char *who, uint64_t *base_step) {
    const ukv_subpool_spec &s = pool->spec[sub];
    if (begin < 0 || count < 0 || step < 1 ||
        (count > 0 && (int64_t)begin + (int64_t)(count - 1) * step >= (int64_t)s.layer_num))
        return fail(UKV_ERR_INVALID_ARG, "%s: layers %d + k*%d for k < %d run outside [0, %d)", who, begin, step, count,
                    s.layer_num);
    if (count > 65535) return fail(UKV_ERR_INVALID_ARG, "%s: more than 65535 layers in one call", who);
    const uint64_t blocks_per_layer = s.kind == UKV_MHA ? 2 : 1;
    *base_step = (uint64_t)step * blocks_per_layer * (uint64_t)pool->plan.page_size * pool->plan.sub[sub].row_bytes;
    return UKV_OK;
}

static uint64_t magnitude(int64_t v) { return v < 0 ? (uint64_t)(-(v + 1)) + 1 : (uint64_t)v; }

int ukv_store_kv_layers(const ukv_pool *pool, int32_t sub, int32_t layer_begin, int32_t layer_count,
                        int32_t layer_step, const int32_t *ids_dev, int64_t n, const void *k_dev, const void *v_dev,
                        int64_t src_row_stride_bytes, int64_t src_layer_stride_bytes, hipStream_t stream) {
    const char *who = "ukv_store_kv";
    int rc = check_pool_call(pool, sub, who);
    if (rc != UKV_OK) return rc;
    const ukv_subpool_spec &s = pool->spec[sub];
    const ukv_subpool_plan &q = pool->plan.sub[sub];
    uint64_t base_step = 0;
    rc = check_layer_range(pool, sub, layer_begin, layer_count, layer_step, who, &base_step);
    if (rc != UKV_OK) return rc;
    if (n < 0 || n > kMaxGrid) return fail(UKV_ERR_INVALID_ARG, "%s: n=%lld outside [0, 2^31)", who, (long long)n);
    const int nkv = s.kind == UKV_MHA ? 2 : 1;
    if (nkv == 1 && v_dev != nullptr) return fail(UKV_ERR_INVALID_ARG, "%s: MLA sub-pool takes no V rows", who);
    if (n == 0 || layer_count == 0) return UKV_OK;
    if (ids_dev == nullptr || k_dev == nullptr || (nkv == 2 && v_dev == nullptr))
        return fail(UKV_ERR_INVALID_ARG, "%s: null ids, K or V", who);
    if (src_row_stride_bytes < (int64_t)q.row_bytes)
        return fail(UKV_ERR_INVALID_ARG, "%s: src_row_stride_bytes=%lld < row bytes %llu", who,
                    (long long)src_row_stride_bytes, (unsigned long long)q.row_bytes);
    rc = debug_check(pool, ids_dev, nullptr, n, stream, who);
    if (rc != UKV_OK) return rc;
    StoreArgs a;
    std::memset(&a, 0, sizeof(a));
    ukv_view vk, vv;
    ukv::view_of(pool->plan, s, sub, layer_begin, 0, &vk);
    vv = vk;
    if (nkv == 2) ukv::view_of(pool->plan, s, sub, layer_begin, 1, &vv);
    a.pool = pool->raw;
    a.base[0] = vk.byte_offset;
    a.base[1] = vv.byte_offset;
    a.ids = ids_dev;
    a.src[0] = (const uint8_t *)k_dev;
    a.src[1] = (const uint8_t *)(nkv == 2 ? v_dev : k_dev);
    a.src_stride = src_row_stride_bytes;
    a.n = n;
    a.n_rows = (uint32_t)q.n_rows;
    a.page_stride = (uint32_t)(pool->plan.page_size * q.blocks_per_page);
    a.ps = (uint32_t)pool->plan.page_size;
    a.row_bytes = (uint32_t)q.row_bytes;
    a.layer_base_step = base_step;
    a.src_layer_stride = layer_count > 1 ? src_layer_stride_bytes : 0;
    a.flags = pool->flags_dev;
    const int vb = vec_bytes_for({q.row_bytes, vk.byte_offset, vv.byte_offset, (uint64_t)(uintptr_t)pool->raw,
                                  (uint64_t)(uintptr_t)k_dev, (uint64_t)(uintptr_t)a.src[1],
                                  (uint64_t)src_row_stride_bytes, magnitude(a.src_layer_stride)});
    a.vecs = (int32_t)(q.row_bytes / (uint64_t)vb);
    const int lp = piece_shift(vb, q.row_bytes);
    // A small launch of 2 KiB rows (one that would give a wave more than one piece)
    // takes the row-group store, 16 loads per lane: the 32-layer decode store (256
    // rows x 32 layers, 67 MB) ran 11.7-11.8 against 13.2-13.5 us on pieces; a large
    // one keeps its pieces (groups made the single-layer prefill store 53-54 against
    // 47.4 us).
    const bool small_2k = lp == 1 && pieces_per_wave(((n * nkv) << lp) * layer_count, 1) > 1;
    if (lp >= 1 && !small_2k) {  // rows of 2 KiB and more: a wave per 1 KiB piece (1 KiB rows measured faster in tiles)
        const int64_t pieces = (n * nkv) << lp;
        const int k = pieces_per_wave(pieces * layer_count, 1);
        const int64_t grid = ((pieces + k - 1) / k + kWavesPerBlock - 1) / kWavesPerBlock;
        if (grid > kMaxGrid) return fail(UKV_ERR_INVALID_ARG, "%s: n too large for one launch", who);
        const dim3 g((unsigned)grid, (unsigned)layer_count), b(kBlock);
        a.layers = (uint32_t)layer_count;
        const bool xl = layer_count > 1 && (uint64_t)grid * (uint64_t)layer_count < (1ull << 32);
        auto go = [&](auto kv, auto kk) {
            constexpr int NKV = decltype(kv)::value, K = decltype(kk)::value;
            if (xl)
                hipLaunchKernelGGL((store_piece_kernel<NKV, K, true>), g, b, 0, stream, a, lp);
            else
                hipLaunchKernelGGL((store_piece_kernel<NKV, K, false>), g, b, 0, stream, a, lp);
        };
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        using I4 = std::integral_constant<int, 4>;
        using I8 = std::integral_constant<int, 8>;
        if (nkv == 2) {
            if (k == 1) go(I2(), I1()); else if (k == 2) go(I2(), I2()); else if (k == 4) go(I2(), I4()); else go(I2(), I8());
        } else {
            if (k == 1) go(I1(), I1()); else if (k == 2) go(I1(), I2()); else if (k == 4) go(I1(), I4()); else go(I1(), I8());
        }
        return check_launch(who);
    }
    if (const int gj = small_2k ? 16 : group_loads(vb, q.row_bytes)) {  // a wave per 8 rows of a view
        const int64_t grid = (((n + kGroupRows - 1) / kGroupRows) * nkv + kWavesPerBlock - 1) / kWavesPerBlock;
        if (grid > kMaxGrid) return fail(UKV_ERR_INVALID_ARG, "%s: n too large for one launch", who);
        const dim3 g((unsigned)grid, (unsigned)layer_count), b(kBlock);
        with_group_loads(gj, [&](auto jt) {
            constexpr int J = decltype(jt)::value;
            if (nkv == 2)
                hipLaunchKernelGGL((store_group_kernel<2, J>), g, b, 0, stream, a);
            else
                hipLaunchKernelGGL((store_group_kernel<1, J>), g, b, 0, stream, a);
        });
        return check_launch(who);
    }
    const Tiling tl = tiling_for(a.vecs, nkv, n, false);
    a.tile_rows = tl.tile_rows;
    a.tiles_per_wave = tl.tiles_per_wave;
    const int64_t grid = (tl.waves + kStoreTileWaves - 1) / kStoreTileWaves;
    if (grid > kMaxGrid) return fail(UKV_ERR_INVALID_ARG, "%s: n too large for one launch", who);
    auto launch = [&](auto *tag) {
        using V = std::remove_pointer_t<decltype(tag)>;
        const dim3 g((unsigned)grid, (unsigned)layer_count), b(kStoreTileWaves * kWave);
        if (nkv == 2 && tl.tpl == 8)
            hipLaunchKernelGGL((store_kernel<V, 2, 8, true>), g, b, 0, stream, a);
        else if (nkv == 2)
            hipLaunchKernelGGL((store_kernel<V, 2, 4, true>), g, b, 0, stream, a);
        else if (tl.tpl == 8)
            hipLaunchKernelGGL((store_kernel<V, 1, 8, true>), g, b, 0, stream, a);
        else
            hipLaunchKernelGGL((store_kernel<V, 1, 4, true>), g, b, 0, stream, a);
        return check_launch(who);
    };
    return dispatch_vec<2>(vb, launch);
}

int ukv_store_kv(const ukv_pool *pool, int32_t sub, int32_t layer, const int32_t *ids_dev, int64_t n,
                 const void *k_dev, const void *v_dev, int64_t src_row_stride_bytes, hipStream_t stream) {
    return ukv_store_kv_layers(pool, sub, layer, 1, 1, ids_dev, n, k_dev, v_dev, src_row_stride_bytes, 0, stream);
}

int ukv_gather_kv_layers(const ukv_pool *pool, int32_t sub, int32_t layer_begin, int32_t layer_count,
                         int32_t layer_step, const int32_t *block_table_dev, int64_t bt_stride,
                         const int32_t *seq_lens_dev, const int64_t *cu_out_dev, int32_t num_reqs, int32_t window,
                         void *k_out_dev, void *v_out_dev, int64_t out_rows, int64_t out_layer_stride_bytes,
                         hipStream_t stream) {
    const char *who = "ukv_gather_kv";
    int rc = check_pool_call(pool, sub, who);
    if (rc != UKV_OK) return rc;
    const ukv_subpool_spec &s = pool->spec[sub];
    const ukv_subpool_plan &q = pool->plan.sub[sub];
    uint64_t base_step = 0;
    rc = check_layer_range(pool, sub, layer_begin, layer_count, layer_step, who, &base_step);
    if (rc != UKV_OK) return rc;
    if (num_reqs < 0 || window < 0 || out_rows < 0 || out_rows > kMaxGrid)
        return fail(UKV_ERR_INVALID_ARG, "%s: num_reqs=%d window=%d out_rows=%lld out of range", who, num_reqs,
                    window, (long long)out_rows);
    const int nkv = s.kind == UKV_MHA ? 2 : 1;
    if (nkv == 1 && v_out_dev != nullptr) return fail(UKV_ERR_INVALID_ARG, "%s: MLA sub-pool has no V output", who);
    if (out_rows == 0 || layer_count == 0) return UKV_OK;
    if (cu_out_dev == nullptr || k_out_dev == nullptr || (nkv == 2 && v_out_dev == nullptr))
        return fail(UKV_ERR_INVALID_ARG, "%s: null cu_out or output", who);
    if (num_reqs > 0 && (block_table_dev == nullptr || seq_lens_dev == nullptr || bt_stride < 1))
        return fail(UKV_ERR_INVALID_ARG, "%s: null block table / seq_lens or bt_stride < 1", who);
    if (layer_count > 1 && magnitude(out_layer_stride_bytes) < (uint64_t)out_rows * q.row_bytes)
        return fail(UKV_ERR_INVALID_ARG, "%s: out_layer_stride_bytes=%lld makes the layers' outputs overlap", who,
                    (long long)out_layer_stride_bytes);
    GatherArgs a;
    std::memset(&a, 0, sizeof(a));
    ukv_view vk, vv;
    ukv::view_of(pool->plan, s, sub, layer_begin, 0, &vk);
    vv = vk;
    if (nkv == 2) ukv::view_of(pool->plan, s, sub, layer_begin, 1, &vv);
    a.pool = pool->raw;
    a.base[0] = vk.byte_offset;
    a.base[1] = vv.byte_offset;
    a.bt = block_table_dev;
    a.bt_stride = bt_stride;
    a.seq_lens = seq_lens_dev;
    a.cu_out = cu_out_dev;
    a.out[0] = (uint8_t *)k_out_dev;
    a.out[1] = (uint8_t *)(nkv == 2 ? v_out_dev : k_out_dev);
    a.out_rows = out_rows;
    a.num_reqs = num_reqs;
    a.window = window;
    a.ps = (uint32_t)pool->plan.page_size;
    a.bpp = (uint32_t)q.blocks_per_page;
    a.num_pages = (uint32_t)s.num_pages;
    a.row_bytes = (uint32_t)q.row_bytes;
    a.layer_base_step = base_step;
    a.out_layer_stride = layer_count > 1 ? out_layer_stride_bytes : 0;
    a.flags = pool->flags_dev;
    const int vb = vec_bytes_for({q.row_bytes, vk.byte_offset, vv.byte_offset, (uint64_t)(uintptr_t)pool->raw,
                                  (uint64_t)(uintptr_t)k_out_dev, (uint64_t)(uintptr_t)a.out[1],
                                  magnitude(a.out_layer_stride)});
    a.vecs = (int32_t)(q.row_bytes / (uint64_t)vb);
    const int lp = piece_shift(vb, q.row_bytes);
    if (lp >= 0) {  // rows of whole 1 KiB pieces: a wave per two pieces
        // (four per wave in a small launch was slower: a window gather of 16,384
        // rows took 17.9 against 15.6 us)
        const int64_t pieces = (out_rows * nkv) << lp;
        const int64_t grid = ((pieces + 1) / 2 + kWavesPerBlock - 1) / kWavesPerBlock;
        if (grid > kMaxGrid) return fail(UKV_ERR_INVALID_ARG, "%s: out_rows too large for one launch", who);
        const dim3 g((unsigned)grid, (unsigned)layer_count), b(kBlock);
        if (nkv == 2)
            hipLaunchKernelGGL((gather_piece_kernel<2, 2>), g, b, 0, stream, a, lp);
        else
            hipLaunchKernelGGL((gather_piece_kernel<1, 2>), g, b, 0, stream, a, lp);
        return check_launch(who);
    }
    const Tiling tl = tiling_for(a.vecs, nkv, out_rows, true);
    a.tile_rows = tl.tile_rows;
    a.tiles_per_wave = tl.tiles_per_wave;
    const int64_t grid = tl.grid;
    if (grid > kMaxGrid) return fail(UKV_ERR_INVALID_ARG, "%s: out_rows too large for one launch", who);
    auto launch = [&](auto *tag) {
        using V = std::remove_pointer_t<decltype(tag)>;
        const dim3 g((unsigned)grid, (unsigned)layer_count), b(kBlock);
        if (nkv == 2 && tl.tpl == 8)
            hipLaunchKernelGGL((gather_kernel<V, 2, 8>), g, b, 0, stream, a);
        else if (nkv == 2)
            hipLaunchKernelGGL((gather_kernel<V, 2, 4>), g, b, 0, stream, a);
        else if (tl.tpl == 8)
            hipLaunchKernelGGL((gather_kernel<V, 1, 8>), g, b, 0, stream, a);
        else
            hipLaunchKernelGGL((gather_kernel<V, 1, 4>), g, b, 0, stream, a);
        return check_launch(who);
    };
    return dispatch_vec<2>(vb, launch);
}

int ukv_gather_kv(const ukv_pool *pool, int32_t sub, int32_t layer, const int32_t *block_table_dev,
                  int64_t bt_stride, const int32_t *seq_lens_dev, const int64_t *cu_out_dev, int32_t num_reqs,
                  int32_t window, void *k_out_dev, void *v_out_dev, int64_t out_rows, hipStream_t stream) {
    return ukv_gather_kv_layers(pool, sub, layer, 1, 1, block_table_dev, bt_stride, seq_lens_dev, cu_out_dev,
                                num_reqs, window, k_out_dev, v_out_dev, out_rows, 0, stream);
}

int ukv_move_kv(const ukv_pool *pool, int32_t sub, const int32_t *dst_dev, const int32_t *src_dev, int64_t n,
                int32_t layer_begin, int32_t layer_end, hipStream_t stream) {
    const char *who = "ukv_move_kv";
    int rc = check_pool_call(pool, sub, who);
    if (rc != UKV_OK) return rc;
    const ukv_subpool_spec &s = pool->spec[sub];
    const ukv_subpool_plan &q = pool->plan.sub[sub];
    if (layer_begin < 0 || layer_begin > layer_end || layer_end > s.layer_num)
        return fail(UKV_ERR_INVALID_ARG, "%s: layer range [%d, %d) outside [0, %d]", who, layer_begin, layer_end,
                    s.layer_num);
    if (n < 0 || n > kMaxGrid) return fail(UKV_ERR_INVALID_ARG, "%s: n=%lld outside [0, 2^31)", who, (long long)n);
    const int32_t nl = layer_end - layer_begin;
    if (n == 0 || nl == 0) return UKV_OK;
    if (dst_dev == nullptr || src_dev == nullptr) return fail(UKV_ERR_INVALID_ARG, "%s: null dst or src", who);
    rc = debug_check(pool, dst_dev, src_dev, n, stream, who);
    if (rc != UKV_OK) return rc;
    const int64_t units = n * (int64_t)nl;
    const int nkv = s.kind == UKV_MHA ? 2 : 1;
    ukv_view v0;
    ukv::view_of(pool->plan, s, sub, layer_begin, 0, &v0);
    MoveArgs a;
    std::memset(&a, 0, sizeof(a));
    a.pool = pool->raw;
    a.base0 = v0.byte_offset;
    a.kv_step = (uint64_t)pool->plan.page_size * q.row_bytes;
    a.layer_step = (uint64_t)nkv * a.kv_step;
    a.dst = dst_dev;
    a.src = src_dev;
    a.n = n;
    a.nl = nl;
    a.n_rows = (uint32_t)q.n_rows;
    a.page_stride = (uint32_t)(pool->plan.page_size * q.blocks_per_page);
    a.ps = (uint32_t)pool->plan.page_size;
    a.row_bytes = (uint32_t)q.row_bytes;
    a.flags = pool->flags_dev;
    const int vb = vec_bytes_for({q.row_bytes, v0.byte_offset, a.kv_step, (uint64_t)(uintptr_t)pool->raw});
    a.vecs = (int32_t)(q.row_bytes / (uint64_t)vb);
    const int lp = piece_shift(vb, q.row_bytes);
    if (lp >= 0) {  // rows of whole 1 KiB pieces: a wave per piece
        const int64_t grid = (((units * nkv) << lp) + kWavesPerBlock - 1) / kWavesPerBlock;
        if (grid > kMaxGrid) return fail(UKV_ERR_INVALID_ARG, "%s: n * layers too large for one launch", who);
        if (nkv == 2)
            hipLaunchKernelGGL(move_piece_kernel<2>, dim3((unsigned)grid), dim3(kBlock), 0, stream, a, lp);
        else
            hipLaunchKernelGGL(move_piece_kernel<1>, dim3((unsigned)grid), dim3(kBlock), 0, stream, a, lp);
        return check_launch(who);
    }
    // units per tile: about 512 chunks of one view per tile, two rounds of 4 per lane
    // (4 rows of 2 KiB; measured on MI355X against 1 and 2 units and 2 or 8 per lane)
    const int64_t tu = (int64_t)2 * kWave * kTasksPerLane / a.vecs;
    a.tile_units = (int32_t)(tu < 1 ? 1 : (tu > kWave ? kWave : tu));
    const int64_t waves = (units + a.tile_units - 1) / a.tile_units;
    const int64_t grid = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
    if (grid > kMaxGrid) return fail(UKV_ERR_INVALID_ARG, "%s: n * layers too large for one launch", who);
    auto launch = [&](auto *tag) {
        using V = std::remove_pointer_t<decltype(tag)>;
        if (nkv == 2)
            hipLaunchKernelGGL((move_kernel<V, 2, kTasksPerLane>), dim3((unsigned)grid), dim3(kBlock), 0, stream, a);
        else
            hipLaunchKernelGGL((move_kernel<V, 1, kTasksPerLane>), dim3((unsigned)grid), dim3(kBlock), 0, stream, a);
        return check_launch(who);
    };
    return dispatch_vec<2>(vb, launch);
}

int ukv_move_pages(const ukv_pool *pool, int32_t sub, const int32_t *dst_pages_dev, const int32_t *src_pages_dev,
                   int64_t n, hipStream_t stream) {
    const char *who = "ukv_move_pages";
    int rc = check_pool_call(pool, sub, who);
    if (rc != UKV_OK) return rc;
    if (n < 0 || n > kMaxGrid) return fail(UKV_ERR_INVALID_ARG, "%s: n=%lld outside [0, 2^31)", who, (long long)n);
    if (n == 0) return UKV_OK;
    if (dst_pages_dev == nullptr || src_pages_dev == nullptr)
        return fail(UKV_ERR_INVALID_ARG, "%s: null dst or src", who);
    rc = debug_check(pool, dst_pages_dev, src_pages_dev, n, stream, who);
    if (rc != UKV_OK) return rc;
    const ukv_subpool_plan &q = pool->plan.sub[sub];
    PageMoveArgs a;
    std::memset(&a, 0, sizeof(a));
    a.pool = pool->raw;
    a.anchor = q.anchor_bytes;
    a.page_bytes = q.page_bytes;
    a.dst = dst_pages_dev;
    a.src = src_pages_dev;
    a.n = n;
    a.num_pages = pool->spec[sub].num_pages;
    a.flags = pool->flags_dev;
    const int vb = vec_bytes_for({q.page_bytes, q.anchor_bytes, (uint64_t)(uintptr_t)pool->raw});
    // one 16-byte chunk per lane (1 KiB per wave of 16-byte vectors): measured on
    // MI355X at 5.9 TB/s for 2 MiB pages, against 5.6 at 2-4 chunks per lane and
    // 4.0 at 8 (8 KiB per wave)
    constexpr int kTpl = 1;
    a.vecs = (int64_t)(q.page_bytes / (uint64_t)vb);
    a.segs = (a.vecs + kWave * kTpl - 1) / (kWave * kTpl);
    const int64_t waves = n * a.segs;
    const int64_t grid = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
    if (grid > kMaxGrid) return fail(UKV_ERR_INVALID_ARG, "%s: n pages too large for one launch", who);
    a.grid = (uint32_t)grid;
    auto launch = [&](auto *tag) {
        using V = std::remove_pointer_t<decltype(tag)>;
        hipLaunchKernelGGL((move_pages_kernel<V, kTpl>), dim3((unsigned)grid), dim3(kBlock), 0, stream, a);
        return check_launch(who);
    };
    return dispatch_vec<1>(vb, launch);
}

int ukv_remap_pages(const ukv_pool *pool, int32_t sub, int32_t *v2p_dev, int64_t v2p_len,
                    const int32_t *virt_pages_dev, const int32_t *phys_pages_dev, int64_t n, hipStream_t stream) {
    const char *who = "ukv_remap_pages";
    int rc = check_pool_call(pool, sub, who);
    if (rc != UKV_OK) return rc;
    if (n < 0 || n > kMaxGrid || v2p_len < 0)
        return fail(UKV_ERR_INVALID_ARG, "%s: n=%lld or v2p_len=%lld out of range", who, (long long)n,
                    (long long)v2p_len);
    if (n == 0) return UKV_OK;
    if (v2p_dev == nullptr || virt_pages_dev == nullptr || phys_pages_dev == nullptr)
        return fail(UKV_ERR_INVALID_ARG, "%s: null table or pages", who);
    if (ranges_overlap(v2p_dev, (uint64_t)v2p_len * 4, virt_pages_dev, (uint64_t)n * 4) ||
        ranges_overlap(v2p_dev, (uint64_t)v2p_len * 4, phys_pages_dev, (uint64_t)n * 4))
        return fail(UKV_ERR_INVALID_ARG, "%s: the table overlaps the page lists", who);
    const unsigned grid = (unsigned)((n + kBlock - 1) / kBlock);
    hipLaunchKernelGGL(remap_pages_kernel, dim3(grid), dim3(kBlock), 0, stream, v2p_dev, v2p_len, virt_pages_dev,
                       phys_pages_dev, n, (int64_t)pool->spec[sub].num_pages, pool->flags_dev);
    return check_launch(who);
}

int ukv_evict_window(const ukv_pool *pool, int32_t *mapping_dev, int64_t map_len, const int32_t *table_dev,
                     int64_t bt_stride, const int32_t *seq_lens_dev, int32_t num_reqs, int32_t window,
                     hipStream_t stream) {
    const char *who = "ukv_evict_window";
    int rc = check_pool_call(pool, 0, who);
    if (rc != UKV_OK) return rc;
    if (num_reqs < 0 || map_len < 0 || bt_stride < 0)
        return fail(UKV_ERR_INVALID_ARG, "%s: negative size", who);
    if (window <= 0 || num_reqs == 0 || bt_stride == 0) return UKV_OK;
    if (mapping_dev == nullptr || table_dev == nullptr || seq_lens_dev == nullptr)
        return fail(UKV_ERR_INVALID_ARG, "%s: null mapping, table or seq_lens", who);
    const int64_t entries = (int64_t)num_reqs * bt_stride;
    if (ranges_overlap(mapping_dev, (uint64_t)map_len * 4, table_dev, (uint64_t)entries * 4))
        return fail(UKV_ERR_INVALID_ARG, "%s: the mapping overlaps the table", who);
    const int64_t grid = (entries + kBlock - 1) / kBlock;
    if (grid > kMaxGrid) return fail(UKV_ERR_INVALID_ARG, "%s: table too large for one launch", who);
    hipLaunchKernelGGL(evict_window_kernel, dim3((unsigned)grid), dim3(kBlock), 0, stream, mapping_dev, map_len,
                       table_dev, bt_stride, seq_lens_dev, num_reqs, window, (int64_t)pool->plan.page_size,
                       pool->flags_dev);
    return check_launch(who);
}

int ukv_pool_set_debug(ukv_pool *pool, int32_t on) {
    if (pool == nullptr) return fail(UKV_ERR_INVALID_ARG, "ukv_pool_set_debug: null pool");
    pool->debug = on != 0;
    return UKV_OK;
}

int ukv_pool_error_flags(ukv_pool *pool, hipStream_t stream, uint32_t *out_and_clear) {
    if (pool == nullptr || out_and_clear == nullptr)
        return fail(UKV_ERR_INVALID_ARG, "ukv_pool_error_flags: null argument");
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != pool->device)
        return fail(UKV_ERR_INVALID_ARG, "ukv_pool_error_flags: current device %d is not the pool's device %d", dev,
                    pool->device);
    hipLaunchKernelGGL(flags_fetch_clear_kernel, dim3(1), dim3(kWave), 0, stream, pool->flags_dev);
    int rc = check_launch("ukv_pool_error_flags");
    if (rc != UKV_OK) return rc;
    uint32_t host = 0;
    hipError_t e = hipMemcpyAsync(&host, pool->flags_dev + 1, sizeof(uint32_t), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(UKV_ERR_HIP, "ukv_pool_error_flags: %s", hipGetErrorString(e));
    *out_and_clear = host;
    return UKV_OK;
}

}  // extern "C"
