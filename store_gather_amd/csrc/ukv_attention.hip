// libukv read path for gfx950 (MI355X): the kernel-facing, prefix-only
// page-table build and a paged decode attention that reads the dense
// per-layer K / V views through that table.
//
// Source: report page "PR #34602: feat(unified-memory): dense KV views for
// uniform-row MHA/SWA models": 功能与动机 (motivation: a backend reads each
// layer through one dense tensor and one block table shared by all layers)
// and 关联脉络 (related work: the stacked change #35247 builds the backends'
// kernel-facing page table by translating the prefix only).  The pages print
// no attention kernel; the attention is the textbook scaled dot-product
// decode attention with grouped KV heads (G query heads per KV head).
//
// Design (decode: one query token per request, G <= 8 query heads per KV
// head, bf16 K / V / Q, fp32 accumulation and output):
//
//  - split-K over positions ("flash decoding"): one 64-lane wave owns
//    (request, KV head, chunk of up to 1,024 positions) and writes an unnormalised
//    partial (running max, row sum, G x D sums) to a workspace; a second,
//    small kernel merges the chunks of each (request, KV head).  Tens of
//    thousands of waves for a decode batch, whatever the length mix.
//  - per tile of 16 positions: S^T = K Q^T on the matrix cores
//    (v_mfma_f32_16x16x32_bf16, D / 32 steps).  K is the A operand straight
//    from HBM: lane l loads 16 bytes of position l % 16, so every load is a
//    plain 16-byte vector load of the dense view.  Q is the B operand, its G
//    heads repeated over the 16 columns, so lane l ends with the scores of
//    positions 4 (l / 16) + i (i < 4) for query head (l % 16) % G.
//  - online softmax in base 2 with a lazy rescale: the running max moves
//    only when a tile's max exceeds it by more than 8 (weights stay <= 2^8,
//    no overflow), so the G x D / 4 accumulators are rescaled a handful of
//    times per chunk instead of every tile.
//  - P V on the vector ALUs in fp32: lane l accumulates position group
//    l / 16 and dims [(l % 16) D / 16, +D / 16) of every query head; V is
//    read as 16-byte loads of D / 16 elements, 4 positions per wave load.
//    (P V reduces over positions, which are strided in the dense view, so
//    the matrix cores would need a transpose through LDS; the vector work is
//    a small share of the HBM time at decode's arithmetic intensity.)
//  - K and V of the next tile are loaded before the current tile is
//    computed; the block-table lookups of a tile are done by its 16
//    position lanes and broadcast with ds_bpermute.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>

#include "ukv_internal.h"

using ukv::check_launch;
using ukv::check_pool_call;
using ukv::fail;
using ukv::ranges_overlap;

namespace {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int64_t kMaxGrid = 0x7fffffff;
constexpr int kTile = 16;        // positions per MFMA tile
constexpr int kMaxChunk = 1024;  // positions per wave (split-K unit), at most
constexpr int kMinChunk = 128;
constexpr int64_t kBusyWaves = 4096;  // about 1.3 x the waves MI355X holds at this kernel's occupancy
constexpr float kRescaleGap = 8.0f;  // log2 headroom before the running max moves

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ----------------------------------------------------------------------------
// prefix-only page-table build (关联脉络: #35247)
// ----------------------------------------------------------------------------
struct TableArgs {
    const int32_t *req_pages;  // [num_reqs, width] allocator pages in position order
    const int32_t *prefix_lens;
    const int32_t *v2p;
    int32_t *out;  // [num_reqs, width] kernel-facing page indices
    uint32_t *flags;
    int64_t width;
    int64_t entries;
    int64_t v2p_len;
    int64_t ps;
    int64_t bpp;
    int64_t num_pages;
};

// Entry i of request r is translated when it holds a prefix position
// (i < ceil(len / ps)), through v2p when given: negative or unmapped -> 0,
// past the table or the pool -> 0 plus UKV_FLAG_SLOT_RANGE, else
// phys * blocks_per_page.  Entries past the prefix are written 0 and never
// read.  A prefix needing more than `width` entries raises UKV_FLAG_LAYOUT.
__global__ __launch_bounds__(kBlock) void build_page_table_kernel(TableArgs a) {
    const int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (e >= a.entries) return;
    const int64_t r = e / a.width;
    const int64_t i = e - r * a.width;
    const int64_t len = a.prefix_lens[r];
    const int64_t used = len > 0 ? (len + a.ps - 1) / a.ps : 0;
    if (i == 0 && used > a.width) atomicOr(a.flags, UKV_FLAG_LAYOUT);
    int32_t kp = 0;
    bool out_of_range = false;
    if (i < used) {
        const int64_t q = a.req_pages[e];
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
            if (phys >= a.num_pages)
                out_of_range = true;
            else if (phys >= 0)
                kp = (int32_t)(phys * a.bpp);
        }
    }
    a.out[e] = kp;
    if (out_of_range) atomicOr(a.flags, UKV_FLAG_SLOT_RANGE);
}

// ----------------------------------------------------------------------------
// decode attention
// ----------------------------------------------------------------------------
struct AttnArgs {
    const uint8_t *pool;
    uint64_t k_base;     // byte offset of the layer's K view (row 0)
    uint64_t v_base;     // byte offset of the layer's V view
    uint32_t row_bytes;  // head_num * head_dim * 2
    uint32_t ps;
    uint32_t bpp;
    uint32_t num_pages;
    const uint16_t *q;  // [num_reqs, head_num * G, D] bf16
    const int32_t *bt;  // [num_reqs, bt_stride] kernel-facing page indices
    int64_t bt_stride;
    const int32_t *seq_lens;
    int32_t num_reqs;
    int32_t heads;  // KV heads
    int32_t window;
    int32_t max_seq_len;
    int32_t max_chunks;
    int32_t chunk;     // positions per split-K unit, a multiple of 16
    float scale_log2;  // softmax scale * log2(e)
    double inv_bpp;    // 1 / blocks_per_page
    float *part_o;     // [num_reqs, max_chunks, heads, G, D]
    float *part_ml;    // [num_reqs, max_chunks, heads, G, 2]: running max (log2 units), row sum; sum < 0 marks a bad chunk
    float *out;        // [num_reqs, heads * G, D] fp32
    uint32_t *flags;
};

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Positions [j0, len) of a request: the last `window` ones for a windowed layer.
__device__ __forceinline__ int32_t first_position(int32_t len, int32_t window) {
    return (window > 0 && len > window) ? len - window : 0;
}

__device__ __forceinline__ u32x4 load16(const uint8_t *p) { return *(const u32x4 *)p; }

// bf16 pair in one 32-bit word -> two floats (exact).
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Lane n of each 16-lane row, broadcast to the whole row (DPP row_newbcast).
template <int N>
__device__ __forceinline__ float row_bcast(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + N, 0xF, 0xF, false));
}

// e is a multiple of bpp: floor(e * (1 / bpp)) in double is off by at most one
// for e < 2^31, fixed by one correction step; no integer division.
__device__ __forceinline__ bool multiple_of(int32_t e, int32_t bpp, double inv_bpp) {
    int32_t q = (int32_t)((double)e * inv_bpp);
    int32_t r = e - q * bpp;
    if (r < 0) r += bpp;
    if (r >= bpp) r -= bpp;
    return r == 0;
}

template <int G>
__device__ __forceinline__ float p_of_head(float p, int g) {
    // p of head g at this lane's position: lane g of the lane's row holds it
    switch (g) {
        case 0: return row_bcast<0>(p);
        case 1: return row_bcast<1>(p);
        case 2: return row_bcast<2>(p);
        case 3: return row_bcast<3>(p);
        case 4: return row_bcast<4>(p);
        case 5: return row_bcast<5>(p);
        case 6: return row_bcast<6>(p);
        default: return row_bcast<7>(p);
    }
}

template <int G, int D>
__global__ __launch_bounds__(kWave) void attn_chunk_kernel(AttnArgs a) {
    static_assert(D % 32 == 0 && D >= 64 && D <= 256, "head_dim");
    static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group");
    constexpr int KS = D / 32;   // MFMA k-steps per tile
    constexpr int DL = D / 16;   // V elements per lane per position
    constexpr int VH = DL < 8 ? 1 : DL / 8;  // 16-byte V loads per lane per position
    const int lane = lane_id();
    const int grp = lane >> 4;   // position group of this lane (0..3)
    const int col = lane & 15;   // MFMA column: position (K operand) and query head (Q operand)

    // one wave per block; chunk-major order: every request's chunk 0 first,
    // so the last waves are the late chunks of the longest requests
    const int64_t wave = blockIdx.x;
    const int64_t per_chunk = (int64_t)a.num_reqs * a.heads;
    const int32_t c = (int32_t)(wave / per_chunk);
    if (c >= a.max_chunks) return;
    const int32_t rem = (int32_t)(wave - (int64_t)c * per_chunk);
    const int32_t r = rem / a.heads;
    const int32_t h = rem - r * a.heads;
    const int32_t len = a.seq_lens[r];
    if (len <= 0 || len > a.max_seq_len) return;
    const int32_t j0 = first_position(len, a.window);
    const int32_t pbeg = j0 + c * a.chunk;
    if (pbeg >= len) return;
    const int32_t pend = min(len, pbeg + a.chunk);
    const int32_t tiles = (pend - pbeg + kTile - 1) / kTile;
    const int64_t unit = ((int64_t)r * a.max_chunks + c) * a.heads + h;

    // Q as the B operand: column col holds query head (col % G) of KV head h;
    // lane group grp holds dims [8 (4 s + grp), +8) at k-step s.
    const int qhead = h * G + (col % G);
    const uint16_t *qrow = a.q + ((int64_t)r * a.heads * G + qhead) * D;
    bf16x8 qb[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) qb[s] = __builtin_bit_cast(bf16x8, *(const u32x4 *)(qrow + 8 * (4 * s + grp)));

    const uint8_t *kview = a.pool + a.k_base + (uint64_t)h * D * 2;
    const uint8_t *vview = a.pool + a.v_base + (uint64_t)h * D * 2 + (uint64_t)col * DL * 2;

    // The lane's K position in tile t is pbeg + 16 t + col; its table column
    // and page offset advance by 16 positions per tile without a division.
    const uint32_t ps = a.ps;
    const uint32_t q16 = (uint32_t)kTile / ps, r16 = (uint32_t)kTile - q16 * ps;
    const int32_t *bt_row = a.bt + (int64_t)r * a.bt_stride;
    const int32_t entry_lim = (int32_t)(a.num_pages * a.bpp);  // num_pages * bpp * ps < 2^31
    struct Pos {
        int32_t j;
        uint32_t col, off;
    };
    auto advance = [&](Pos p) {
        p.j += kTile;
        p.col += q16;
        p.off += r16;
        if (p.off >= ps) {
            p.off -= ps;
            ++p.col;
        }
        return p;
    };
    // table entry of a position (a load), -1 past the table; nothing past the chunk
    auto entry = [&](const Pos &p) -> int32_t {
        return (p.j < pend && (int64_t)p.col < a.bt_stride) ? bt_row[p.col] : -1;
    };
    bool bad = false;
    auto row_of = [&](const Pos &p, int32_t e) -> int32_t {
        if (p.j >= pend) return -1;
        if (e < 0 || e >= entry_lim || !multiple_of(e, (int32_t)a.bpp, a.inv_bpp)) {
            bad = true;
            return -1;
        }
        return e * (int32_t)ps + (int32_t)p.off;  // < n_rows < 2^31
    };
    auto bad_chunk = [&]() {
        atomicOr(a.flags, UKV_FLAG_BAD_BLOCK);
        if (lane < G) a.part_ml[(unit * G + lane) * 2 + 1] = -1.0f;
    };

    u32x4 kreg[KS];
    u32x4 vreg[4][VH] = {};
    uint64_t vlo[4] = {};  // D = 64: 8 bytes per lane
    auto load_tile = [&](int32_t krow) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
            kreg[s] = krow >= 0 ? load16(kview + (uint64_t)(uint32_t)krow * a.row_bytes + 16 * (4 * s + grp))
                                : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int32_t vrow = __shfl(krow, 4 * grp + t);
            const uint8_t *p = vview + (uint64_t)(uint32_t)(vrow < 0 ? 0 : vrow) * a.row_bytes;
            if constexpr (DL >= 8) {
#pragma unroll
                for (int v = 0; v < VH; ++v) vreg[t][v] = vrow >= 0 ? load16(p + 16 * v) : u32x4{0, 0, 0, 0};
            } else {
                vlo[t] = vrow >= 0 ? *(const uint64_t *)p : 0ull;
            }
        }
    };

    float acc[G][DL];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int d = 0; d < DL; ++d) acc[g][d] = 0.0f;
    float m_run = -INFINITY;  // running max of this lane's query head, log2 units
    float l_run = 0.0f;       // row sum over this lane's positions

    // prologue: entries of tiles 0 and 1, loads of tile 0
    Pos p0;
    p0.j = pbeg + col;
    p0.col = (uint32_t)p0.j / ps;
    p0.off = (uint32_t)p0.j - p0.col * ps;
    const int32_t e0 = entry(p0);
    Pos p1 = advance(p0);
    int32_t e1 = entry(p1);
    int32_t krow = row_of(p0, e0);
    if (__any(bad)) return bad_chunk();
    load_tile(krow);
    for (int t = 0; t < tiles; ++t) {
        // scores of this tile
        f32x4 sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kreg[s]), qb[s], sacc, 0, 0, 0);
        u32x4 vcur[4][VH] = {};
        uint64_t vcur_lo[4] = {};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (DL >= 8) {
#pragma unroll
                for (int v = 0; v < VH; ++v) vcur[i][v] = vreg[i][v];
            } else {
                vcur_lo[i] = vlo[i];
            }
        }
        // the next tile's loads and the entries of the one after go out
        // before this tile's arithmetic
        if (t + 1 < tiles) {
            const Pos p2 = advance(p1);
            const int32_t e2 = entry(p2);
            krow = row_of(p1, e1);
            if (__any(bad)) return bad_chunk();
            load_tile(krow);
            p1 = p2;
            e1 = e2;
        }
        const int32_t tile0 = pbeg + t * kTile + 4 * grp;
        float x[4];
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = tile0 + i < pend ? sacc[i] * a.scale_log2 : -INFINITY;
            tmax = fmaxf(tmax, x[i]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const bool need = tmax > m_run + kRescaleGap;
        if (__any(need)) {
            const float alpha = need ? exp2f(m_run - tmax) : 1.0f;
            if (need) m_run = tmax;
            l_run *= alpha;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float ag = p_of_head<G>(alpha, g);
#pragma unroll
                for (int d = 0; d < DL; ++d) acc[g][d] *= ag;
            }
        }
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = exp2f(x[i] - m_run);
            l_run += p[i];
        }
        // P V: position 4 grp + i of the tile, dims [col * DL, +DL) of every head
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float vf[DL];
            if constexpr (DL >= 8) {
#pragma unroll
                for (int v = 0; v < VH; ++v)
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        vf[8 * v + 2 * w] = lo_bf16(vcur[i][v][w]);
                        vf[8 * v + 2 * w + 1] = hi_bf16(vcur[i][v][w]);
                    }
            } else {
#pragma unroll
                for (int w = 0; w < 2; ++w) {
                    const uint32_t word = (uint32_t)(vcur_lo[i] >> (32 * w));
                    vf[2 * w] = lo_bf16(word);
                    vf[2 * w + 1] = hi_bf16(word);
                }
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float pg = p_of_head<G>(p[i], g);
#pragma unroll
                for (int d = 0; d < DL; ++d) acc[g][d] = fmaf(pg, vf[d], acc[g][d]);
            }
        }
    }
    // sum the four position groups
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int d = 0; d < DL; ++d) {
            acc[g][d] += __shfl_xor(acc[g][d], 16);
            acc[g][d] += __shfl_xor(acc[g][d], 32);
        }
    if (lane < 16) {
        float *po = a.part_o + unit * G * D + col * DL;
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int d = 0; d < DL; d += 4)
                *(f32x4 *)(po + g * D + d) = f32x4{acc[g][d], acc[g][d + 1], acc[g][d + 2], acc[g][d + 3]};
    }
    if (lane < G) {
        a.part_ml[(unit * G + lane) * 2] = m_run;
        a.part_ml[(unit * G + lane) * 2 + 1] = l_run;
    }
}

// Merge the units of (request, KV head): out = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c.
// A bad unit, a request past max_seq_len (UKV_FLAG_LAYOUT) or an empty one
// gives zeros.  One wave: lanes take the (unit, head) pairs in parallel for
// the maxima and the denominators, the weights go through LDS, and each lane
// sums G * D / 64 outputs over the units with independent loads.
template <int G, int D>
__global__ __launch_bounds__(kWave) void attn_combine_kernel(AttnArgs a) {
    constexpr int E = G * D / kWave;  // outputs per lane
    constexpr int kPiece = 4096 / G;  // units whose weights fit the LDS array at once
    __shared__ float wsh[kPiece * G];
    const int lane = lane_id();
    const int g_lane = lane % G;  // the head of every (unit, head) pair this lane takes
    const int32_t r = (int32_t)(blockIdx.x / (uint32_t)a.heads);
    const int32_t h = (int32_t)(blockIdx.x - (uint32_t)r * a.heads);
    float *o = a.out + ((int64_t)r * a.heads + h) * G * D;
    const int32_t len = a.seq_lens[r];
    int32_t chunks = 0;
    if (len > a.max_seq_len) {
        if (h == 0 && lane == 0) atomicOr(a.flags, UKV_FLAG_LAYOUT);
    } else if (len > 0) {
        const int32_t n = len - first_position(len, a.window);
        chunks = (n + a.chunk - 1) / a.chunk;
    }
    const int64_t unit0 = (int64_t)r * a.max_chunks * a.heads + h;  // unit c: unit0 + c * heads
    auto ml_of = [&](int c) { return *(const float2 *)(a.part_ml + ((unit0 + (int64_t)c * a.heads) * G + g_lane) * 2); };
    // running max and denominator of head g_lane over this lane's pairs
    float mx = -INFINITY, den = 0.0f;
    bool bad = false;
    for (int idx = lane; idx < chunks * G; idx += kWave) {
        const float2 ml = ml_of(idx / G);
        bad |= ml.y < 0.0f;
        if (ml.x > mx) {
            den = den * exp2f(mx - ml.x) + ml.y;
            mx = ml.x;
        } else {
            den += exp2f(ml.x - mx) * ml.y;
        }
    }
    float mh = mx;
    for (int sh = kWave / 2; sh >= G; sh >>= 1) mh = fmaxf(mh, __shfl_xor(mh, sh));
    den = mx == -INFINITY ? 0.0f : den * exp2f(mx - mh);
    for (int sh = kWave / 2; sh >= G; sh >>= 1) den += __shfl_xor(den, sh);
    const bool any_bad = __any(bad);
    float acc[E];
#pragma unroll
    for (int k = 0; k < E; ++k) acc[k] = 0.0f;
    if (chunks > 0 && !any_bad) {
        for (int c0 = 0; c0 < chunks; c0 += kPiece) {
            const int cn = min(kPiece, chunks - c0);
            for (int idx = lane; idx < cn * G; idx += kWave) wsh[idx] = exp2f(ml_of(c0 + idx / G).x - mh);
            __syncthreads();
#pragma unroll 4
            for (int c = 0; c < cn; ++c) {
                const float *po = a.part_o + (unit0 + (int64_t)(c0 + c) * a.heads) * G * D;
#pragma unroll
                for (int k = 0; k < E; ++k) {
                    const int e = lane + kWave * k;
                    acc[k] = fmaf(wsh[c * G + e / D], po[e], acc[k]);
                }
            }
            __syncthreads();
        }
    }
#pragma unroll
    for (int k = 0; k < E; ++k) {
        const int e = lane + kWave * k;
        const float dg = __shfl(den, e / D);  // lane g holds head g's denominator
        o[e] = (chunks > 0 && !any_bad) ? acc[k] / dg : 0.0f;
    }
}

// Positions per split-K unit: the largest of 1024, 768, 512, 384, 256, 128
// that still gives about kBusyWaves waves for the batch's bound (long units
// amortise each wave's start and its partial result; enough of them keep
// every CU busy).  Measured on the decode-shape batch: 1024 (6.5 TB/s) over
// 512 (6.2 TB/s) in chunk-major order.
int32_t chunk_for(int32_t num_reqs, int32_t heads, int32_t max_seq_len, int32_t window) {
    const int64_t n = (window > 0 && window < max_seq_len) ? window : max_seq_len;
    int32_t chunk = kMaxChunk;
    while (chunk > kMinChunk && (int64_t)num_reqs * heads * ((n + chunk - 1) / chunk) < kBusyWaves)
        chunk = chunk > 512 ? chunk - 256 : chunk - 128;
    return chunk;
}

int64_t max_chunks_for(int32_t max_seq_len, int32_t window, int32_t chunk) {
    const int64_t n = (window > 0 && window < max_seq_len) ? window : max_seq_len;
    return n > 0 ? (n + chunk - 1) / chunk : 0;
}

// ukv_decode_attention_noalloc's partials: a fixed device array, one per GPU the
// library runs on, held until the process ends (64 MiB: the decode batch of 256
// requests of up to 8,192 positions with 32 query heads of 128 needs 34 MB).  In
// host code `scratch` only names the symbol; its device address, looked up once
// per device, is what kernels and copies take.
constexpr uint64_t kNoAllocScratchBytes = 64ull << 20;
__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_lock;
void *g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch`, found with hipGetSymbolAddress on the
// first call on that device (the device is current: check_pool_call checked it).
int device_scratch(void **out, const char *who) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return fail(UKV_ERR_HIP, "%s: current device %d unusable for the fixed scratch", who, dev);
    std::lock_guard<std::mutex> hold(g_scratch_lock);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(UKV_ERR_HIP, "%s: device address of the fixed scratch: %s", who, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return UKV_OK;
}

int decode_attention_with(const ukv_pool *pool, int32_t sub, int32_t layer, const void *q_dev, int32_t q_heads,
                          const int32_t *block_table_dev, int64_t bt_stride, const int32_t *seq_lens_dev,
                          int32_t num_reqs, int32_t max_seq_len, int32_t window, float scale, float *out_dev,
                          void *workspace_dev, uint64_t workspace_bytes, hipStream_t stream, const char *who);

}  // namespace

extern "C" {

int ukv_build_page_table(const ukv_pool *pool, int32_t sub, const int32_t *req_pages_dev, int64_t bt_stride,
                         const int32_t *prefix_lens_dev, int32_t num_reqs, const int32_t *v2p_dev, int64_t v2p_len,
                         int32_t *out_dev, hipStream_t stream) {
    const char *who = "ukv_build_page_table";
    int rc = check_pool_call(pool, sub, who);
    if (rc != UKV_OK) return rc;
    if (num_reqs < 0 || bt_stride < 0) return fail(UKV_ERR_INVALID_ARG, "%s: negative size", who);
    if (v2p_dev != nullptr && v2p_len < 0) return fail(UKV_ERR_INVALID_ARG, "%s: v2p_len < 0", who);
    const int64_t entries = (int64_t)num_reqs * bt_stride;
    if (entries == 0) return UKV_OK;
    if (req_pages_dev == nullptr || prefix_lens_dev == nullptr || out_dev == nullptr)
        return fail(UKV_ERR_INVALID_ARG, "%s: null page lists, lengths or output", who);
    const uint64_t bytes = (uint64_t)entries * sizeof(int32_t);
    if ((const void *)out_dev != (const void *)req_pages_dev && ranges_overlap(out_dev, bytes, req_pages_dev, bytes))
        return fail(UKV_ERR_INVALID_ARG, "%s: output overlaps the page lists (same buffer or disjoint)", who);
    if (ranges_overlap(out_dev, bytes, prefix_lens_dev, (uint64_t)num_reqs * 4) ||
        (v2p_dev != nullptr && ranges_overlap(out_dev, bytes, v2p_dev, (uint64_t)v2p_len * 4)))
        return fail(UKV_ERR_INVALID_ARG, "%s: output overlaps the lengths or the v2p table", who);
    const int64_t grid = (entries + kBlock - 1) / kBlock;
    if (grid > kMaxGrid) return fail(UKV_ERR_INVALID_ARG, "%s: table too large for one launch", who);
    TableArgs a;
    std::memset(&a, 0, sizeof(a));
    a.req_pages = req_pages_dev;
    a.prefix_lens = prefix_lens_dev;
    a.v2p = v2p_dev;
    a.out = out_dev;
    a.flags = pool->flags_dev;
    a.width = bt_stride;
    a.entries = entries;
    a.v2p_len = v2p_dev == nullptr ? 0 : v2p_len;
    a.ps = pool->plan.page_size;
    a.bpp = pool->plan.sub[sub].blocks_per_page;
    a.num_pages = pool->spec[sub].num_pages;
    hipLaunchKernelGGL(build_page_table_kernel, dim3((unsigned)grid), dim3(kBlock), 0, stream, a);
    return check_launch(who);
}

uint64_t ukv_decode_attention_workspace_bytes(const ukv_pool *pool, int32_t sub, int32_t num_reqs, int32_t q_heads,
                                              int32_t max_seq_len, int32_t window) {
    if (pool == nullptr || sub < 0 || sub >= pool->plan.n_sub) return 0;
    const ukv_subpool_spec &s = pool->spec[sub];
    if (num_reqs <= 0 || q_heads <= 0 || max_seq_len <= 0 || s.head_num <= 0) return 0;
    if (window < 0) window = 0;
    const int32_t chunk = chunk_for(num_reqs, s.head_num, max_seq_len, window);
    return (uint64_t)num_reqs * (uint64_t)max_chunks_for(max_seq_len, window, chunk) * (uint64_t)q_heads *
           ((uint64_t)s.head_dim + 2) * sizeof(float);
}

int ukv_decode_attention(const ukv_pool *pool, int32_t sub, int32_t layer, const void *q_dev, int32_t q_heads,
                         const int32_t *block_table_dev, int64_t bt_stride, const int32_t *seq_lens_dev,
                         int32_t num_reqs, int32_t max_seq_len, int32_t window, float scale, float *out_dev,
                         void *workspace_dev, uint64_t workspace_bytes, hipStream_t stream) {
    return decode_attention_with(pool, sub, layer, q_dev, q_heads, block_table_dev, bt_stride, seq_lens_dev, num_reqs,
                                 max_seq_len, window, scale, out_dev, workspace_dev, workspace_bytes, stream,
                                 "ukv_decode_attention");
}

int ukv_decode_attention_noalloc(const ukv_pool *pool, int32_t sub, int32_t layer, const void *q_dev, int32_t q_heads,
                                 const int32_t *block_table_dev, int64_t bt_stride, const int32_t *seq_lens_dev,
                                 int32_t num_reqs, int32_t max_seq_len, int32_t window, float scale, float *out_dev,
                                 hipStream_t stream) {
    const char *who = "ukv_decode_attention_noalloc";
    int rc = check_pool_call(pool, sub, who);
    if (rc != UKV_OK) return rc;
    const uint64_t need = ukv_decode_attention_workspace_bytes(pool, sub, num_reqs, q_heads, max_seq_len, window);
    if (need > kNoAllocScratchBytes)
        return fail(UKV_ERR_INVALID_ARG,
                    "%s: this batch needs %llu bytes of partial results; the fixed scratch holds %llu "
                    "(pass a workspace to ukv_decode_attention instead)",
                    who, (unsigned long long)need, (unsigned long long)kNoAllocScratchBytes);
    void *ws = nullptr;
    if (need > 0) {
        rc = device_scratch(&ws, who);
        if (rc != UKV_OK) return rc;
    }
    return decode_attention_with(pool, sub, layer, q_dev, q_heads, block_table_dev, bt_stride, seq_lens_dev, num_reqs,
                                 max_seq_len, window, scale, out_dev, ws, need > 0 ? kNoAllocScratchBytes : 0, stream,
                                 who);
}

}  // extern "C"

namespace {

int decode_attention_with(const ukv_pool *pool, int32_t sub, int32_t layer, const void *q_dev, int32_t q_heads,
                          const int32_t *block_table_dev, int64_t bt_stride, const int32_t *seq_lens_dev,
                          int32_t num_reqs, int32_t max_seq_len, int32_t window, float scale, float *out_dev,
                          void *workspace_dev, uint64_t workspace_bytes, hipStream_t stream, const char *who) {
    int rc = check_pool_call(pool, sub, who);
    if (rc != UKV_OK) return rc;
    const ukv_subpool_spec &s = pool->spec[sub];
    const ukv_subpool_plan &p = pool->plan.sub[sub];
    if (s.kind != UKV_MHA) return fail(UKV_ERR_INVALID_ARG, "%s: sub-pool %d is not MHA", who, sub);
    if (s.elem_bytes != 2) return fail(UKV_ERR_INVALID_ARG, "%s: K / V must be bf16 (itemsize %d)", who, s.elem_bytes);
    if (layer < 0 || layer >= s.layer_num)
        return fail(UKV_ERR_INVALID_ARG, "%s: layer %d outside [0, %d)", who, layer, s.layer_num);
    const int D = s.head_dim;
    if (D != 64 && D != 128 && D != 256) return fail(UKV_ERR_INVALID_ARG, "%s: head_dim %d not 64, 128 or 256", who, D);
    if (q_heads <= 0 || q_heads % s.head_num != 0)
        return fail(UKV_ERR_INVALID_ARG, "%s: q_heads %d is not a multiple of head_num %d", who, q_heads, s.head_num);
    const int G = q_heads / s.head_num;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(UKV_ERR_INVALID_ARG, "%s: %d query heads per KV head (supported: 1, 2, 4, 8)", who, G);
    if (num_reqs < 0 || window < 0 || max_seq_len < 0 || bt_stride < 0)
        return fail(UKV_ERR_INVALID_ARG, "%s: negative size", who);
    if (!std::isfinite(scale)) return fail(UKV_ERR_INVALID_ARG, "%s: scale is not finite", who);
    if (num_reqs == 0) return UKV_OK;
    if (q_dev == nullptr || seq_lens_dev == nullptr || out_dev == nullptr)
        return fail(UKV_ERR_INVALID_ARG, "%s: null q, seq_lens or output", who);
    if (((uintptr_t)q_dev % 16) != 0 || ((uintptr_t)out_dev % 16) != 0)
        return fail(UKV_ERR_ALIGNMENT, "%s: q and out must be 16-byte aligned", who);
    ukv_view vk, vv;
    ukv::view_of(pool->plan, s, sub, layer, 0, &vk);
    ukv::view_of(pool->plan, s, sub, layer, 1, &vv);
    if (((uintptr_t)pool->raw + vk.byte_offset) % 16 != 0 || ((uintptr_t)pool->raw + vv.byte_offset) % 16 != 0)
        return fail(UKV_ERR_ALIGNMENT, "%s: the layer's views are not 16-byte aligned", who);
    const int32_t chunk = chunk_for(num_reqs, s.head_num, max_seq_len, window);
    const int64_t chunks = max_chunks_for(max_seq_len, window, chunk);
    const uint64_t need = ukv_decode_attention_workspace_bytes(pool, sub, num_reqs, q_heads, max_seq_len, window);
    if (chunks > 0) {
        if (block_table_dev == nullptr || bt_stride < 1)
            return fail(UKV_ERR_INVALID_ARG, "%s: null block table or bt_stride < 1", who);
        if (workspace_dev == nullptr || workspace_bytes < need)
            return fail(UKV_ERR_INVALID_ARG, "%s: workspace of %llu bytes, %llu needed", who,
                        (unsigned long long)workspace_bytes, (unsigned long long)need);
        if (((uintptr_t)workspace_dev % 16) != 0)
            return fail(UKV_ERR_ALIGNMENT, "%s: workspace must be 16-byte aligned", who);
    }
    const uint64_t out_bytes = (uint64_t)num_reqs * q_heads * D * sizeof(float);
    if (ranges_overlap(out_dev, out_bytes, q_dev, (uint64_t)num_reqs * q_heads * D * 2) ||
        ranges_overlap(out_dev, out_bytes, workspace_dev, need) ||
        ranges_overlap(out_dev, out_bytes, pool->raw, pool->raw_bytes))
        return fail(UKV_ERR_INVALID_ARG, "%s: output overlaps q, the workspace or the pool", who);
    const int64_t grid = (int64_t)num_reqs * chunks * s.head_num;  // one wave per block
    if (grid > kMaxGrid || (int64_t)num_reqs * s.head_num > kMaxGrid)
        return fail(UKV_ERR_INVALID_ARG, "%s: batch too large for one launch", who);
    AttnArgs a;
    std::memset(&a, 0, sizeof(a));
    a.pool = pool->raw;
    a.k_base = vk.byte_offset;
    a.v_base = vv.byte_offset;
    a.row_bytes = (uint32_t)p.row_bytes;
    a.ps = (uint32_t)pool->plan.page_size;
    a.bpp = (uint32_t)p.blocks_per_page;
    a.num_pages = (uint32_t)s.num_pages;
    a.q = (const uint16_t *)q_dev;
    a.bt = block_table_dev;
    a.bt_stride = bt_stride;
    a.seq_lens = seq_lens_dev;
    a.num_reqs = num_reqs;
    a.heads = s.head_num;
    a.window = window;
    a.max_seq_len = max_seq_len;
    a.max_chunks = (int32_t)chunks;
    a.chunk = chunk;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);
    a.inv_bpp = 1.0 / (double)p.blocks_per_page;
    float *ws = (float *)workspace_dev;
    a.part_o = ws;
    a.part_ml = ws == nullptr ? nullptr : ws + (uint64_t)num_reqs * chunks * q_heads * D;
    a.out = out_dev;
    a.flags = pool->flags_dev;
    auto launch = [&](auto gtag, auto dtag) {
        constexpr int GG = decltype(gtag)::value;
        constexpr int DD = decltype(dtag)::value;
        if (grid > 0) hipLaunchKernelGGL((attn_chunk_kernel<GG, DD>), dim3((unsigned)grid), dim3(kWave), 0, stream, a);
        hipLaunchKernelGGL((attn_combine_kernel<GG, DD>), dim3((unsigned)(num_reqs * s.head_num)), dim3(kWave), 0,
                           stream, a);
        return check_launch(who);
    };
    auto by_dim = [&](auto gtag) {
        switch (D) {
            case 64: return launch(gtag, std::integral_constant<int, 64>());
            case 128: return launch(gtag, std::integral_constant<int, 128>());
            default: return launch(gtag, std::integral_constant<int, 256>());
        }
    };
    switch (G) {
        case 1: return by_dim(std::integral_constant<int, 1>());
        case 2: return by_dim(std::integral_constant<int, 2>());
        case 4: return by_dim(std::integral_constant<int, 4>());
        default: return by_dim(std::integral_constant<int, 8>());
    }
}

}  // namespace
