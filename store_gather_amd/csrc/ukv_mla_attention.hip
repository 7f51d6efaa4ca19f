// libukv read path for MLA sub-pools on gfx950 (MI355X): paged decode
// attention straight from a layer's dense latent view.
//
// Source: report page "PR #34602: feat(unified-memory): dense KV views for
// uniform-row MHA/SWA models", 功能与动机 (motivation): the MLA sub-pool
// already exposes dense per-layer views, and a backend reads a layer through
// one dense tensor and one block table shared by all layers.  The pages print
// no attention kernel; this is the textbook decode attention of the
// absorbed MLA form: every query head attends to the one latent row per
// position, scores over the whole row (576 wide: the compressed KV part and
// the rotary part), values the row's first 512 elements.
//
// Design (one query token per request, q_heads a multiple of 16, bf16 latent
// rows and queries, fp32 accumulation and output).  At 16 query heads the
// read is ~30 FLOP per byte, beyond what the vector ALUs sustain at HBM
// bandwidth, so both products run on the matrix cores:
//
//  - balanced split-K: the batch's positions, request after request, form
//    one sequence that is cut into equal spans, one per workgroup (1,024
//    over all head groups: four per CU, so every workgroup has the same work
//    and none is left over for a second round).  The cut is by cost: each
//    request costs its positions plus a fixed start-up share (its queries,
//    the restart of the tile stream, its partial), so a span that takes a
//    request boundary takes fewer positions.  A workgroup walks its span
//    request by request and writes an unnormalised partial (max, row sum,
//    16 x 512 sums) for each request it touches to slot (span + request),
//    which is unique; a second kernel merges each request's slots.  Every
//    wave finds its first request by a prefix sum over the costs; the first
//    wave also leaves, per request, where its positions start, for the
//    merge.
//  - the query-head groups of one span sit on one XCD (blocks b with the
//    same b % 8), so the latent rows they share are read once into that
//    XCD's L2.
//  - per 16 positions, S^T = C Q^T on v_mfma_f32_16x16x32_bf16 (18 k-steps
//    over 576): the latent rows are the A operand, the 16 heads' queries the
//    B operand, so lane l ends with the scores of positions 4 (l / 16) + i
//    for head l % 16 -- the weights of those four positions are then already
//    where the P V product wants them, with no exchange between lanes.
//  - the rows are not loaded in that operand layout (16 rows x 64 bytes per
//    load, which holds a plain read of the view to about 65% of HBM
//    bandwidth): each wave loads its half of the rows' first 512 elements two
//    rows per load (whole 128-byte lines), with the streaming hint, and stages
//    them in LDS (row-major); the A operand of the score product comes back
//    from LDS, and the value operand through the gfx950 transposing read
//    ds_read_b64_tr_b16 (four positions of one dim per lane per read).  Only
//    the small rotary chunk is loaded in the operand layout.
//  - each weight p enters the product as two bf16 parts, bf16(p) and
//    bf16(p - bf16(p)), so the weights keep about 16 significant bits
//    (relative error <= 2^-16): one K = 32 product per 16 value dims takes
//    both parts of a lane's four positions, against the four transposed
//    values twice (v_mfma_f32_16x16x32_bf16 again).
//  - base-2 softmax against a fixed reference per segment (the first tile's
//    max score): the sums never need a vector rescale, which keeps the
//    register pressure where the compiler does not spill.  A score that
//    outgrows the reference by more than 2^64 sends the segment through a
//    max-first pass instead (weights then never exceed 1).
//  - two waves per workgroup split each row: wave h loads the chunks of
//    its 256 value dims and 32 of the rotary dims, computes the partial
//    scores over them, and the two add each other's partials through LDS
//    (the same sum, bit for bit, in both), then each multiplies the weights
//    into its own 256 value dims.  Per wave: 16 x 256 fp32 sums, one 9-chunk
//    row buffer and its 9 chunks of the 16 queries (the score product's B
//    operand, loaded once per request), ~226 registers, so two waves per
//    SIMD.  (Queries in LDS cost 9 KB of LDS reads per wave and tile: 229
//    against 217 us per layer on the decode batch.)
//  - once a tile has been staged and its scores taken, the next tile's rows
//    go out into the same registers and stay in flight during the value
//    product; block-table entries are read a tile ahead of their rows.  Every
//    load is issued on every path, so the compiler's count of loads in
//    flight is exact.  (A second row buffer, for two tiles in flight, took
//    the registers the queries now hold, and was no faster.)
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <type_traits>

#include "ukv_internal.h"

using ukv::check_launch;
using ukv::check_pool_call;
using ukv::fail;
using ukv::ranges_overlap;

namespace {

constexpr int kWave = 64;
constexpr int64_t kMaxGrid = 0x7fffffff;
constexpr int kTile = 16;                // positions per tile
constexpr int kHeads = 16;               // query heads per wave (the MFMA width)
constexpr int64_t kTargetGroups = 1024;  // two-wave workgroups: 4 per CU x 256 CUs, one round
constexpr int64_t kMinSpan = 256;        // positions per wave, at least (a partial is 32 KiB)
constexpr int64_t kSegCost = 128;        // a span's cost of starting a request, in positions' worth of time
constexpr int kXcds = 8;                 // workgroups go round-robin over the 8 XCDs
constexpr float kGrowGap = 64.0f;       // log2 headroom of the weights over their reference
constexpr int kLatent = 576;             // supported latent width (elements)
constexpr int kValue = 512;              // supported value width (elements)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct MlaArgs {
    const uint8_t *pool;
    uint64_t base;       // byte offset of the layer's latent view (row 0)
    uint32_t row_bytes;  // latent width * 2
    uint32_t ps;
    uint32_t bpp;
    uint32_t num_pages;
    const uint16_t *q;  // [num_reqs, q_heads, latent] bf16
    const int32_t *bt;  // [num_reqs, bt_stride] kernel-facing page indices
    int64_t bt_stride;
    const int32_t *seq_lens;
    int32_t num_reqs;
    int32_t q_heads;
    int32_t groups;  // q_heads / 16
    int32_t window;
    int32_t max_seq_len;
    int32_t spans;     // waves per head group, a multiple of 8
    float scale_log2;  // softmax scale * log2(e)
    double inv_bpp;
    int64_t *cum;    // [num_reqs + 2]: where each request's positions start in cost units, the total cost, the span
    float *part_o;   // [spans + num_reqs slots, q_heads, value]
    float *part_ml;  // [spans + num_reqs slots, q_heads, 2]: running max (log2 units), row sum; sum < 0: bad
    float *out;      // [num_reqs, q_heads, value]
    uint32_t *flags;
};

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

__device__ __forceinline__ int32_t first_position(int32_t len, int32_t window) {
    return (window > 0 && len > window) ? len - window : 0;
}

// Positions request r attends to: 0 when it is empty or past the caller's bound.
__device__ __forceinline__ int32_t attended(const MlaArgs &a, int32_t len) {
    return (len <= 0 || len > a.max_seq_len) ? 0 : len - first_position(len, a.window);
}

__device__ __forceinline__ int64_t wave_inclusive_scan(int64_t v, int lane) {
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int64_t u = __shfl_up(v, (unsigned)d);
        if (lane >= d) v += u;
    }
    return v;
}

__device__ __forceinline__ u32x4 load16(const uint8_t *p) { return *(const u32x4 *)p; }
// A latent row's bytes: read once per launch, with the streaming hint.
__device__ __forceinline__ u32x4 load16_nt(const uint8_t *p) {
    return __builtin_nontemporal_load((const u32x4 *)p);
}

// e is a multiple of bpp: floor(e / bpp) by a double reciprocal is off by at
// most one for e < 2^31, fixed by one correction step.
__device__ __forceinline__ bool multiple_of(int32_t e, int32_t bpp, double inv_bpp) {
    int32_t q = (int32_t)((double)e * inv_bpp);
    int32_t r = e - q * bpp;
    if (r < 0) r += bpp;
    if (r >= bpp) r -= bpp;
    return r == 0;
}

// Row pitch of the LDS value tile: 512 bf16 plus 32 bytes, so that the
// sixteen rows one transposing read touches spread over the banks.
constexpr int kPitch = kValue * 2 + 32;

// A workgroup of two waves owns (span, head group).  Wave `half` loads the
// row chunks s = 8 half .. 8 half + 7 (its 256 value dims) and s = 16 + half
// (its 32 rotary dims) of every row, computes the partial scores over those
// 288 dims, and the two waves add each other's partials through LDS; both
// then hold the same scores and take the same softmax decisions, and each
// multiplies the weights into its own 256 value dims.  Per wave: 16 x 256
// fp32 sums (64 registers), one 9-chunk row buffer and the queries' 9 chunks
// -- two waves per SIMD.
template <int KS, int NB>
__global__ __launch_bounds__(2 * kWave) __attribute__((amdgpu_waves_per_eu(2, 2))) void mla_attn_span_kernel(MlaArgs a) {
    static_assert(KS * 32 == kLatent && NB * 16 == kValue && KS == NB / 2 + 2, "latent / value width");
    constexpr int KH = KS / 2;      // row chunks per wave: 8 value chunks and 1 rotary chunk
    constexpr int VH = NB / 2;      // 16-dim value blocks per wave
    __shared__ __attribute__((aligned(16))) uint8_t lds[kTile * kPitch];
    __shared__ __attribute__((aligned(16))) f32x4 xch[2][2][kWave];  // partial scores by tile parity and wave
    const int half = (int)(threadIdx.x / kWave);
    const int lane = lane_id();
    const int grp = lane >> 4;
    const int col = lane & 15;
    // the wave's row chunks: j < 8 -> value chunk 8 half + j, j = 8 -> rotary chunk 16 + half
    auto chunk = [&](int j) { return j < KH - 1 ? (KH - 1) * half + j : 2 * (KH - 1) + half; };

    // block b -> (span w, head group hg), with every group of a span on XCD b % 8
    const int32_t b = (int32_t)blockIdx.x;
    const int32_t y = b / kXcds;
    const int32_t hg = y % a.groups;
    const int32_t w = (y / a.groups) * kXcds + (b - y * kXcds);
    const bool writer = w == 0 && hg == 0 && half == 0;

    // The split runs in cost units: a request of n > 0 attended positions costs
    // kSegCost + n (its positions come after the start-up share), so a span
    // that takes a request boundary gets that many fewer positions.  Total
    // cost T (the first wave records, per request, where its positions start
    // in cost units), then the span.
    int64_t carry = 0;
    for (int32_t base = 0; base < a.num_reqs; base += kWave) {
        const int32_t r = base + lane;
        const int64_t n = r < a.num_reqs ? attended(a, a.seq_lens[r]) : 0;
        const int64_t c = n > 0 ? n + kSegCost : 0;
        const int64_t incl = wave_inclusive_scan(c, lane);
        if (writer && r < a.num_reqs) a.cum[r] = carry + incl - c + kSegCost;
        carry += __shfl(incl, kWave - 1);
    }
    const int64_t total = carry;
    int64_t span = (total + a.spans - 1) / a.spans;
    span = span < kMinSpan ? kMinSpan : span;
    if (writer && lane == 0) {
        a.cum[a.num_reqs] = total;
        a.cum[a.num_reqs + 1] = span;
    }
    const int64_t start = (int64_t)w * span;
    if (start >= total) return;  // both waves of the workgroup leave together
    const int64_t end = start + span < total ? start + span : total;
    // the request whose cost interval holds `start`, and its cost base
    int32_t r = -1;
    int64_t rbase = 0;
    carry = 0;
    for (int32_t base = 0; base < a.num_reqs && r < 0; base += kWave) {
        const int32_t rr = base + lane;
        const int64_t n = rr < a.num_reqs ? attended(a, a.seq_lens[rr]) : 0;
        const int64_t c = n > 0 ? n + kSegCost : 0;
        const int64_t incl = wave_inclusive_scan(c, lane);
        const int64_t excl = carry + incl - c;
        const uint64_t hit = __ballot(c > 0 && excl <= start && start < excl + c);
        if (hit != 0) {
            const int l = __ffsll((unsigned long long)hit) - 1;
            r = base + l;
            rbase = __shfl(excl, l);
        }
        carry += __shfl(incl, kWave - 1);
    }

    // the queries are the B operand, in registers: column col is head hg*16 + col,
    // lane group grp holds dims [8 (4 s + grp), +8) at k-step s
    const uint8_t *view = a.pool + a.base;
    const uint32_t ps = a.ps;
    const uint32_t q16 = (uint32_t)kTile / ps, r16 = (uint32_t)kTile - q16 * ps;
    const int32_t entry_lim = (int32_t)(a.num_pages * a.bpp);  // num_pages * bpp * ps < 2^31
    // transposing reads: lane (grp, col) points at position 4 grp + col / 4 of
    // the tile, dims 16 nb + 4 (col % 4) .. +3; it receives dim 16 nb + col of
    // positions 4 grp .. 4 grp + 3 (nb in this wave's blocks)
    const int tr_off = (4 * grp + col / 4) * kPitch + 8 * (col % 4) + 32 * VH * half;

    u32x4 kA[KH];
    int64_t cur = start;
    while (cur < end) {
        r = __builtin_amdgcn_readfirstlane(r);
        const int32_t len = a.seq_lens[r];
        const int32_t n = attended(a, len);
        if (n == 0) {
            ++r;
            continue;
        }
        // this span's positions of request r: cost [cur, end) against the
        // request's positions at [rbase + kSegCost, rbase + kSegCost + n)
        const int64_t p0 = cur - rbase - kSegCost > 0 ? cur - rbase - kSegCost : 0;
        const int64_t p1 = end - rbase - kSegCost < n ? end - rbase - kSegCost : n;
        if (p1 <= p0) {  // only the request's start-up share falls in this span
            cur = rbase + n + kSegCost;
            rbase = cur;
            ++r;
            continue;
        }
        const int64_t seg = p1 - p0;
        const int32_t pbeg = first_position(len, a.window) + (int32_t)p0;
        const int32_t pend = pbeg + (int32_t)seg;
        const int32_t tiles = (pend - pbeg + kTile - 1) / kTile;
        const int64_t slot = (int64_t)w + r;
        u32x4 qreg[KH];  // the score product's B operand: head col's dims of this wave's chunks
        {
            const uint8_t *qg = (const uint8_t *)(a.q + ((int64_t)r * a.q_heads + hg * kHeads + col) * kLatent) + 16 * grp;
#pragma unroll
            for (int j = 0; j < KH; ++j) qreg[j] = load16(qg + 64 * chunk(j));
        }
        f32x4 o[VH];
        float m_run = -INFINITY;  // the weights' reference (log2 units) of head col
        float l_run = 0.0f;       // row sum over this lane's positions
        // the lane's position in tile t is pbeg + 16 t + col; (table column,
        // page offset) advance by 16 positions per tile without a division.
        const int32_t *bt_row = a.bt + (int64_t)r * a.bt_stride;
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
        // table entry of a position, raw: read by every lane (at the row's last
        // column when past it), so that every tile issues the same loads and the
        // compiler's count of loads in flight is exact on every path; row_of
        // makes the range checks, where the value is first used (a check here
        // would wait for this load, the newest, and with it for every row load
        // before it).
        auto entry = [&](const Pos &p) -> int32_t {
            return bt_row[(int64_t)p.col < a.bt_stride ? (int64_t)p.col : a.bt_stride - 1];
        };
        bool bad = false;
        auto row_of = [&](const Pos &p, int32_t e) -> int32_t {
            if (p.j >= pend) return -1;
            if ((int64_t)p.col >= a.bt_stride || e < 0 || e >= entry_lim ||
                !multiple_of(e, (int32_t)a.bpp, a.inv_bpp)) {
                bad = true;
                return -1;
            }
            return e * (int32_t)ps + (int32_t)p.off;  // < n_rows < 2^31
        };
        // The wave's share of a tile's rows, loaded unconditionally (a position
        // past the segment reads row 0; its scores are masked and its values
        // zeroed in LDS).  k[0..7]: its 512-byte value half of all 16 rows, two
        // rows per load (lane l: row of position 2 i + l / 32, 16 bytes at
        // 512 half + 16 (l % 32)), so that each load reads whole 128-byte lines
        // -- reading the rows in the matrix cores' operand layout instead (16
        // rows x 64 bytes per load) holds a plain read of this layer view to
        // about 65% of HBM bandwidth, against 75-79% this way.  The rows of the
        // other positions come from the lanes that computed them.  k[8]: its
        // half of the rotary chunk, in the operand layout (lane (grp, col):
        // position col, 16 bytes at 1024 + 64 half + 16 grp).
        auto row_at = [&](int32_t row, int i) {  // row of position 2 i + lane / 32
            const int32_t ra = __builtin_amdgcn_readlane(row, 2 * i);
            const int32_t rb = __builtin_amdgcn_readlane(row, 2 * i + 1);
            return lane < 32 ? ra : rb;
        };
        auto load_tile = [&](u32x4 (&k)[KH], int32_t row) {
            const int32_t rr = row < 0 ? 0 : row;
            const uint8_t *vp = view + 512 * half + 16 * (lane & 31);
#pragma unroll
            for (int i = 0; i < KH - 1; ++i) k[i] = load16_nt(vp + (uint64_t)(uint32_t)row_at(rr, i) * a.row_bytes);
            k[KH - 1] = load16_nt(view + (uint64_t)(uint32_t)rr * a.row_bytes + 16 * grp + 64 * chunk(KH - 1));
        };
        // the value half into LDS (row-major, this wave's columns only); rows past
        // the segment stage zeros
        auto stage = [&](const u32x4 (&k)[KH], int32_t row, int32_t t) {
            uint8_t *st = lds + (lane >> 5) * kPitch + 512 * half + 16 * (lane & 31);
            if (pbeg + (t + 1) * kTile <= pend) {  // every position of the tile is in the segment (uniform)
#pragma unroll
                for (int i = 0; i < KH - 1; ++i) *(u32x4 *)(st + 2 * i * kPitch) = k[i];
            } else {  // the segment's last tile
#pragma unroll
                for (int i = 0; i < KH - 1; ++i)
                    *(u32x4 *)(st + 2 * i * kPitch) = row_at(row, i) >= 0 ? k[i] : u32x4{0, 0, 0, 0};
            }
        };
        // this wave's partial scores, then the other wave's added (through LDS, by
        // tile parity).  The value chunks' operands come back from the wave's own
        // LDS columns (LDS runs a wave's operations in order, and the compiler
        // may not move the reads above the writes of the same array).
        auto scores = [&](const u32x4 (&k)[KH], int32_t t) {
            const uint8_t *ap = lds + col * kPitch + 512 * half + 16 * grp;
            // three accumulators: chains of three dependent products instead of nine
            f32x4 part[3] = {};
#pragma unroll
            for (int j = 0; j < KH; ++j)
                part[j % 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, j < KH - 1 ? load16(ap + 64 * j) : k[KH - 1]),
                    __builtin_bit_cast(bf16x8, qreg[j]), part[j % 3], 0, 0, 0);
            const f32x4 acc = (part[0] + part[1]) + part[2];
            xch[t & 1][half][lane] = acc;
            __syncthreads();
            const f32x4 other = xch[t & 1][1 - half][lane];
            return half == 0 ? acc + other : other + acc;  // the same sum, bit for bit, in both waves
        };
        // One pass over the segment, one tile at a time: once tile t has been
        // staged and its scores taken, the rows of tile t + 1 go out into the
        // same registers and stay in flight during the value product.  Table
        // entries are read a tile ahead of their rows' loads.  The weights are 2^(x - ref) for a fixed reference ref,
        // so the sums are never rescaled (they stay in the matrix cores'
        // accumulators):
        //   MODE 0: ref = the first tile's max score; returns false (sums
        //           unusable) as soon as a score exceeds ref + kGrowGap;
        //   MODE 1: a given ref, at least every score (nothing to check);
        //   MODE 2: no sums, ref becomes the segment's max score.
        // Both waves see the same scores, so they take every branch together.
        auto pass = [&](auto mode_tag) -> bool {
            constexpr int MODE = decltype(mode_tag)::value;
            // the score exchange restarts at tile 0: the other wave has read the last one
            __syncthreads();
#pragma unroll
            for (int nb = 0; nb < VH; ++nb) o[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            l_run = 0.0f;
            Pos q0 = {pbeg + col, 0u, 0u};
            q0.col = (uint32_t)q0.j / ps;
            q0.off = (uint32_t)q0.j - q0.col * ps;
            const int32_t e0 = entry(q0);
            Pos qa = advance(q0);
            const int32_t row0 = row_of(q0, e0);
            if (__any(bad)) return true;
            load_tile(kA, row0);
            int32_t ea = entry(qa);
            int32_t va = row0;
            // scores of tile t -> weights, row sums and P V; false: the reference was outgrown
            auto tile_math = [&](const f32x4 &sc, int32_t t) -> bool {
                const int32_t p0 = pbeg + t * kTile + 4 * grp;
                float x[4];
                float lmax = -INFINITY;  // over this lane's four positions
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[i] = p0 + i < pend ? sc[i] * a.scale_log2 : -INFINITY;
                    lmax = fmaxf(lmax, x[i]);
                }
                // The lanes of one head (same col) hold the same reference, so a
                // score outgrows it exactly when some lane's own max does: only
                // the first tile needs the tile's max over the four lane groups,
                // and the max-first pass reduces its per-lane maxima once at its end.
                if constexpr (MODE == 2) {
                    m_run = fmaxf(m_run, lmax);
                    return true;
                } else {
                    if constexpr (MODE == 0) {
                        if (t == 0) {
                            float tmax = fmaxf(lmax, __shfl_xor(lmax, 16));
                            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
                            m_run = tmax;
                        }
                        if (__any(lmax > m_run + kGrowGap)) return false;
                    }
                    s16x4 whi, wlo;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float pw = exp2f(x[i] - m_run);
                        l_run += pw;
                        const __bf16 h = (__bf16)pw;
                        const __bf16 lo = (__bf16)(pw - (float)h);
                        whi[i] = __builtin_bit_cast(short, h);
                        wlo[i] = __builtin_bit_cast(short, lo);
                    }
                    // one K = 32 product per block: k = 8 grp + i is position 4 grp + i % 4,
                    // its high part for i < 4 and its low part for i >= 4, so the value
                    // operand is the four transposed values twice.  The wave reads only
                    // the value half it staged itself: LDS runs a wave's operations in
                    // order, and the compiler may not move the reads above the writes of
                    // the same array.
                    const s16x8 w8 = __builtin_shufflevector(whi, wlo, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                    for (int nb = 0; nb < VH; ++nb) {
                        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) s16x4 *)(lds + tr_off + 32 * nb));
                        const s16x8 v8 = __builtin_shufflevector(v, v, 0, 1, 2, 3, 0, 1, 2, 3);
                        o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w8),
                                                                        __builtin_bit_cast(bf16x8, v8), o[nb], 0, 0, 0);
                    }
                    return true;
                }
            };
            // tile t from buffer k (its rows v); then the rows of tile t + 1 from (q, e) into k
            // and the entry of tile t + 2 into e.  Both loads are issued on every path (row 0
            // past the segment's last tile or for a bad entry), the check for a bad entry after
            // them: a path that skipped them would join the others with fewer loads in flight,
            // and the compiler would then wait for every load at each step.  Every mode
            // stages the tile: the scores read it back.
            auto step = [&](u32x4 (&k)[KH], int32_t &v, Pos &q, int32_t &e, int32_t t) -> int {
                stage(k, v, t);
                const f32x4 sc = scores(k, t);
                const int32_t rown = row_of(q, e);
                q = advance(q);
                load_tile(k, rown);
                e = entry(q);
                v = rown;
                if (__any(bad)) return 1;
                return tile_math(sc, t) ? 0 : 2;
            };
            // the loads in flight at the loop's head: [rows t, entry t + 1]
            int st = 0;
            for (int32_t t = 0; t < tiles; ++t) {
                st = step(kA, va, qa, ea, t);
                if (st != 0) break;
            }
            return st != 2;
        };
        if (!pass(std::integral_constant<int, 0>())) {
            // a score outgrew the first tile's by more than 2^kGrowGap: the
            // segment's max first, then the sums against it
            m_run = -INFINITY;
            pass(std::integral_constant<int, 2>());
            m_run = fmaxf(m_run, __shfl_xor(m_run, 16));  // the head's max over the four lane groups
            m_run = fmaxf(m_run, __shfl_xor(m_run, 32));
            if (!__any(bad)) pass(std::integral_constant<int, 1>());
        }
        const bool seg_bad = __any(bad);
        // the partial of (slot, head group): this wave's value half
        const int64_t head0 = slot * a.q_heads + (int64_t)hg * kHeads;
        if (seg_bad) {
            if (half == 0) {
                atomicOr(a.flags, UKV_FLAG_BAD_BLOCK);
                if (lane < kHeads) a.part_ml[(head0 + lane) * 2 + 1] = -1.0f;
            }
        } else {
            l_run += __shfl_xor(l_run, 16);
            l_run += __shfl_xor(l_run, 32);
            // o[nb][i]: head 4 grp + i, dim 256 half + 16 nb + col
            float *po = a.part_o + head0 * kValue + (kValue / 2) * half + col;
#pragma unroll
            for (int nb = 0; nb < VH; ++nb)
#pragma unroll
                for (int i = 0; i < 4; ++i) po[(4 * grp + i) * kValue + 16 * nb] = o[nb][i];
            if (half == 0 && lane < kHeads) {
                a.part_ml[(head0 + lane) * 2] = m_run;
                a.part_ml[(head0 + lane) * 2 + 1] = l_run;
            }
        }
        cur = rbase + n + kSegCost;
        rbase = cur;
        ++r;
    }
}

// Merge the slots of (request, head): out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s
// over the slots w + r of the spans w that hold its positions.  A bad
// slot, a request past max_seq_len (UKV_FLAG_LAYOUT) or an empty one gives
// zeros.  One wave per (request, head); lane l sums dims l + 64 k.
__global__ __launch_bounds__(kWave) void mla_attn_combine_kernel(MlaArgs a) {
    constexpr int E = kValue / kWave;
    const int lane = lane_id();
    const int32_t r = (int32_t)(blockIdx.x / (uint32_t)a.q_heads);
    const int32_t h = (int32_t)(blockIdx.x - (uint32_t)r * a.q_heads);
    float *o = a.out + ((int64_t)r * a.q_heads + h) * kValue;
    const int32_t len = a.seq_lens[r];
    if (len > a.max_seq_len && h == 0 && lane == 0) atomicOr(a.flags, UKV_FLAG_LAYOUT);
    const int32_t n = attended(a, len);
    int64_t w0 = 0, slots = 0;
    if (n > 0) {
        const int64_t c0 = a.cum[r], span = a.cum[a.num_reqs + 1];
        w0 = c0 / span;
        slots = (c0 + n - 1) / span - w0 + 1;
    }
    auto head_of = [&](int64_t k) { return ((w0 + k + r) * a.q_heads + h); };  // slot w0 + k + r, head h
    float mx = -INFINITY, den = 0.0f;
    bool bad = false;
    for (int64_t k = lane; k < slots; k += kWave) {
        const float2 ml = *(const float2 *)(a.part_ml + head_of(k) * 2);
        bad |= ml.y < 0.0f;
        if (ml.x > mx) {
            den = den * exp2f(mx - ml.x) + ml.y;
            mx = ml.x;
        } else {
            den += exp2f(ml.x - mx) * ml.y;
        }
    }
    float mh = mx;
    for (int sh = kWave / 2; sh >= 1; sh >>= 1) mh = fmaxf(mh, __shfl_xor(mh, sh));
    den = mx == -INFINITY ? 0.0f : den * exp2f(mx - mh);
    for (int sh = kWave / 2; sh >= 1; sh >>= 1) den += __shfl_xor(den, sh);
    const bool ok = slots > 0 && !__any(bad);
    float acc[E];
#pragma unroll
    for (int k = 0; k < E; ++k) acc[k] = 0.0f;
    if (ok) {
        for (int64_t k = 0; k < slots; ++k) {
            const int64_t hs = head_of(k);
            const float wgt = exp2f(a.part_ml[hs * 2] - mh);
            const float *po = a.part_o + hs * kValue;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] = fmaf(wgt, po[lane + kWave * e], acc[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) o[lane + kWave * e] = ok ? acc[e] / den : 0.0f;
}

// Waves per head group (a multiple of 8): about one per SIMD over all groups,
// fewer when the batch's bound would give spans under kMinSpan positions.
int64_t mla_spans_for(int32_t num_reqs, int32_t groups, int32_t max_seq_len, int32_t window) {
    const int64_t n = (window > 0 && window < max_seq_len) ? window : max_seq_len;
    const int64_t bound = (int64_t)num_reqs * (n > 0 ? n : 0);
    if (bound <= 0) return 0;
    int64_t w = kTargetGroups / groups;
    const int64_t by_span = (bound + kMinSpan - 1) / kMinSpan;
    w = w < by_span ? w : by_span;
    w = w < 1 ? 1 : w;
    return (w + kXcds - 1) / kXcds * kXcds;
}

uint64_t mla_header_bytes(int32_t num_reqs) { return ((uint64_t)(num_reqs + 2) * 8 + 15) / 16 * 16; }

}  // namespace

extern "C" {

uint64_t ukv_mla_decode_attention_workspace_bytes(const ukv_pool *pool, int32_t sub, int32_t num_reqs,
                                                  int32_t q_heads, int32_t v_dim, int32_t max_seq_len,
                                                  int32_t window) {
    if (pool == nullptr || sub < 0 || sub >= pool->plan.n_sub) return 0;
    if (num_reqs <= 0 || q_heads <= 0 || q_heads % kHeads != 0 || v_dim <= 0 || max_seq_len <= 0) return 0;
    if (window < 0) window = 0;
    const int64_t spans = mla_spans_for(num_reqs, q_heads / kHeads, max_seq_len, window);
    return mla_header_bytes(num_reqs) +
           (uint64_t)(spans + num_reqs) * (uint64_t)q_heads * ((uint64_t)v_dim + 2) * sizeof(float);
}

int ukv_mla_decode_attention(const ukv_pool *pool, int32_t sub, int32_t layer, const void *q_dev, int32_t q_heads,
                             int32_t v_dim, const int32_t *block_table_dev, int64_t bt_stride,
                             const int32_t *seq_lens_dev, int32_t num_reqs, int32_t max_seq_len, int32_t window,
                             float scale, float *out_dev, void *workspace_dev, uint64_t workspace_bytes,
                             hipStream_t stream) {
    const char *who = "ukv_mla_decode_attention";
    int rc = check_pool_call(pool, sub, who);
    if (rc != UKV_OK) return rc;
    const ukv_subpool_spec &s = pool->spec[sub];
    const ukv_subpool_plan &p = pool->plan.sub[sub];
    if (s.kind != UKV_MLA) return fail(UKV_ERR_INVALID_ARG, "%s: sub-pool %d is not MLA", who, sub);
    if (s.elem_bytes != 2) return fail(UKV_ERR_INVALID_ARG, "%s: latent rows must be bf16 (itemsize %d)", who, s.elem_bytes);
    if (layer < 0 || layer >= s.layer_num)
        return fail(UKV_ERR_INVALID_ARG, "%s: layer %d outside [0, %d)", who, layer, s.layer_num);
    if (s.head_dim != kLatent || v_dim != kValue)
        return fail(UKV_ERR_INVALID_ARG, "%s: latent width %d / value width %d (supported: %d / %d)", who, s.head_dim,
                    v_dim, kLatent, kValue);
    if (q_heads <= 0 || q_heads % kHeads != 0)
        return fail(UKV_ERR_INVALID_ARG, "%s: q_heads %d is not a positive multiple of %d", who, q_heads, kHeads);
    if (num_reqs < 0 || window < 0 || max_seq_len < 0 || bt_stride < 0)
        return fail(UKV_ERR_INVALID_ARG, "%s: negative size", who);
    if (!std::isfinite(scale)) return fail(UKV_ERR_INVALID_ARG, "%s: scale is not finite", who);
    if (num_reqs == 0) return UKV_OK;
    if (q_dev == nullptr || seq_lens_dev == nullptr || out_dev == nullptr)
        return fail(UKV_ERR_INVALID_ARG, "%s: null q, seq_lens or output", who);
    if (((uintptr_t)q_dev % 16) != 0 || ((uintptr_t)out_dev % 16) != 0)
        return fail(UKV_ERR_ALIGNMENT, "%s: q and out must be 16-byte aligned", who);
    ukv_view vw;
    ukv::view_of(pool->plan, s, sub, layer, 0, &vw);
    if (((uintptr_t)pool->raw + vw.byte_offset) % 16 != 0)
        return fail(UKV_ERR_ALIGNMENT, "%s: the layer's view is not 16-byte aligned", who);
    const int32_t groups = q_heads / kHeads;
    const int64_t spans = mla_spans_for(num_reqs, groups, max_seq_len, window);
    const uint64_t need =
        ukv_mla_decode_attention_workspace_bytes(pool, sub, num_reqs, q_heads, v_dim, max_seq_len, window);
    if (spans > 0) {
        if (block_table_dev == nullptr || bt_stride < 1)
            return fail(UKV_ERR_INVALID_ARG, "%s: null block table or bt_stride < 1", who);
        if (workspace_dev == nullptr || workspace_bytes < need)
            return fail(UKV_ERR_INVALID_ARG, "%s: workspace of %llu bytes, %llu needed", who,
                        (unsigned long long)workspace_bytes, (unsigned long long)need);
        if (((uintptr_t)workspace_dev % 16) != 0)
            return fail(UKV_ERR_ALIGNMENT, "%s: workspace must be 16-byte aligned", who);
    }
    const uint64_t out_bytes = (uint64_t)num_reqs * q_heads * kValue * sizeof(float);
    if (ranges_overlap(out_dev, out_bytes, q_dev, (uint64_t)num_reqs * q_heads * kLatent * 2) ||
        ranges_overlap(out_dev, out_bytes, workspace_dev, need) ||
        ranges_overlap(out_dev, out_bytes, pool->raw, pool->raw_bytes))
        return fail(UKV_ERR_INVALID_ARG, "%s: output overlaps q, the workspace or the pool", who);
    const int64_t grid = spans * groups;  // two waves per block
    if (grid > kMaxGrid || (int64_t)num_reqs * q_heads > kMaxGrid)
        return fail(UKV_ERR_INVALID_ARG, "%s: batch too large for one launch", who);
    MlaArgs a;
    std::memset(&a, 0, sizeof(a));
    a.pool = pool->raw;
    a.base = vw.byte_offset;
    a.row_bytes = (uint32_t)p.row_bytes;
    a.ps = (uint32_t)pool->plan.page_size;
    a.bpp = (uint32_t)p.blocks_per_page;
    a.num_pages = (uint32_t)s.num_pages;
    a.q = (const uint16_t *)q_dev;
    a.bt = block_table_dev;
    a.bt_stride = bt_stride;
    a.seq_lens = seq_lens_dev;
    a.num_reqs = num_reqs;
    a.q_heads = q_heads;
    a.groups = groups;
    a.window = window;
    a.max_seq_len = max_seq_len;
    a.spans = (int32_t)spans;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);
    a.inv_bpp = 1.0 / (double)p.blocks_per_page;
    if (workspace_dev != nullptr && spans > 0) {
        uint8_t *ws = (uint8_t *)workspace_dev;
        a.cum = (int64_t *)ws;
        a.part_ml = (float *)(ws + mla_header_bytes(num_reqs));
        a.part_o = a.part_ml + (uint64_t)(spans + num_reqs) * q_heads * 2;
    }
    a.out = out_dev;
    a.flags = pool->flags_dev;
    if (grid > 0)
        hipLaunchKernelGGL((mla_attn_span_kernel<kLatent / 32, kValue / 16>), dim3((unsigned)grid), dim3(2 * kWave), 0,
                           stream, a);
    hipLaunchKernelGGL(mla_attn_combine_kernel, dim3((unsigned)(num_reqs * q_heads)), dim3(kWave), 0, stream, a);
    return check_launch(who);
}

}  // extern "C"
