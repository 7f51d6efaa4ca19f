"""Reference decode attention read straight from the dense per-layer views (fp64, CPU).

TEST INFRASTRUCTURE ONLY: like the rest of oracle/, only the tests, the
package smoke check and the benchmark's CPU-baseline leg may import this.

Source: the report page "PR #34602: feat(unified-memory): dense KV views for
uniform-row MHA/SWA models", section 功能与动机 (motivation): once every layer
of the pool is a dense (n_rows, head_num, head_dim) view, an attention
backend reads a layer through that one tensor and one block table shared by
all layers; section 关联脉络 (related work) places the kernel-facing,
prefix-only page-table build (#35247) on that read path.  The pages print
no attention kernel.  READING: the attention is the textbook scaled
dot-product decode attention with grouped KV heads, written out in float64.
For request r with length len (positions j0 <= j < len, j0 = len - window
for a sliding-window layer longer than its window, else 0), query head g
(KV head h = g // G, G = q_heads / head_num):

    s_j = scale * sum_d q[r, g, d] * K_j[h, d]
    p_j = exp(s_j - max_j s_j) / sum_j exp(s_j - max_j s_j)
    out[r, g, d] = sum_j p_j * V_j[h, d]

K_j / V_j are the rows of the layer's K / V views at row
bt[r][j // ps] * ps + j % ps (block-table entries are kernel-facing page
indices, phys * blocks_per_page), decoded from their bf16 bits.

MLA sub-pools (one latent row per token per layer, e.g. 576 wide) have one
dense view per layer and no separate V rows.  READING (the pages print no MLA
attention either): every query head attends to the single latent "head" —
the scores use the whole latent row, K_j = c_j, and the values are its
first v_dim elements, V_j = c_j[:v_dim] (the compressed KV part ahead of the
rotary part, 512 of 576 in the models with 576-wide latents); the query is
given in the latent space (its no-position part already absorbed).  That is
the formula above with one KV head, G = q_heads.

Conditions (the same readings as the block-table gather): a request with
len <= 0 attends to nothing and its output is zero; a request longer than
the caller's bound max_seq_len raises LAYOUT; one whose positions need a
table column past the table width, or a negative / non-kernel-facing /
out-of-pool entry, raises BAD_BLOCK.  Such a request's output is all zeros.

Pinned in tests/test_oracle_pins.py: against torch's scaled_dot_product_attention
in float64 over rows fetched by the independent strided builder, against
the closed forms of uniform keys and of a single position, and on the
error conditions above.
"""
from __future__ import annotations

import math

import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact: every bf16 value is a float32 value)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """One request: q [Hq, D], k [n, Hkv, D], v [n, Hkv, Dv] (float64) -> [Hq, Dv].

    Query head g reads KV head g // (Hq // Hkv).  n == 0 gives zeros.
    """
    hq = q.shape[0]
    n, hkv = k.shape[0], k.shape[1]
    group = hq // hkv
    out = np.zeros((hq, v.shape[2]))
    if n == 0:
        return out
    for g in range(hq):
        h = g // group
        s = scale * (k[:, h, :] @ q[g])
        e = np.exp(s - s.max())
        out[g] = (e / e.sum()) @ v[:, h, :]
    return out


U32 = 2.0 ** -24  # unit roundoff of float32


def gamma(n: int) -> float:
    """n u / (1 - n u): the bound on the relative error of an n-term float32 sum."""
    return n * U32 / (1.0 - n * U32)


def fp32_error_bound(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, sum_terms: int,
                     weight_rel: float = 0.0) -> np.ndarray:
    """Bound on |out_fp32 - out| per query head for an fp32 evaluation of `attend`.

    q [Hq, D], k [n, Hkv, D], v [n, Hkv, Dv] as in `attend`.  An fp32
    evaluation computes each score from exact products (bf16 x bf16 fits in
    float32) with a D-term fp32 sum, so |ds_j| <= scale * gamma(D) *
    sum_d |q_d k_jd| (A); scaling and the exponential add a few units of
    roundoff relative to the argument (4 u (|scale s_j| log2 e + 1)).  Weights
    perturbed by at most delta relative change the weighted mean by at most
    4 delta max|v|, and the numerator / denominator sums of at most
    `sum_terms` terms add 2 gamma(sum_terms) max|v|.  ``weight_rel`` is any
    further relative error of each weight as the evaluation uses it (e.g. a
    weight split into two bf16 parts for a matrix-core product: 2^-16); it
    adds to delta.
    """
    hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    bound = np.zeros(hq)
    if k.shape[0] == 0:
        return bound
    for g in range(hq):
        h = g // group
        a = (np.abs(k[:, h, :]) @ np.abs(q[g])).max()
        s_max = np.abs(scale * (k[:, h, :] @ q[g])).max() * 1.4426950408889634
        delta = scale * gamma(d) * a + 4 * U32 * (s_max + 1.0) + weight_rel
        vmax = np.abs(v[:, h, :]).max()
        bound[g] = 4 * delta * vmax + 2 * gamma(sum_terms) * vmax
    return bound


def chain_terms_any_split(n: int, parts_per_weight: int = 1) -> int:
    """Longest fp32 sum chain any split of n positions can form, from n alone.

    Whatever way an evaluation cuts a request into pieces, one chain sums at
    most ``parts_per_weight * n`` products (the whole request in one piece,
    each weight entering as that many parts), then at most n partial results
    (a piece holds at least one position), plus a few reduction and division
    steps.  The bound of :func:`fp32_error_bound` computed with this many
    terms holds for every split, so it does not depend on how a kernel
    distributes positions.
    """
    return (parts_per_weight + 1) * n + 8


# With every score equal (a zero query), every weight of an evaluation that
# takes exp2(score - reference) is exactly 1; with integer values (|v| <= 8,
# at most 2^21 positions) every float32 partial sum of weights and of
# weighted values is then exact, whatever the split and the merge order, and
# the output is the exact mean S/n up to the final division: one rounding, or
# two for a reciprocal and a product.  This bound allows four.
EXACT_MEAN_REL = 4 * 2.0 ** -24


def exact_mean_tolerance(expected: np.ndarray) -> np.ndarray:
    """Allowed |fp32 output - exact mean| per element for zero-query, integer-valued inputs."""
    return EXACT_MEAN_REL * np.abs(expected)


def decode_attention(pool, sub: int, layer: int, q_bits: np.ndarray, block_table, seq_lens, window: int,
                     scale: float, max_seq_len: int | None = None, read=None, requests=None,
                     bound_terms=None, v_dim: int | None = None, weight_rel: float = 0.0, uniform: bool = False,
                     read_words=None):
    """Decode attention of every request over its positions in the pool's dense views.

    q_bits: [R, Hq, D] bf16 bits (uint16); block_table: [R, width] int32
    kernel-facing page indices; seq_lens: [R].  ``read(offset, nbytes)``
    returns the uint16 words at a byte offset of the pool (default: the
    pool's own buffer), so that an addresses-only pool can be served from
    values generated on demand; ``read_words(indices)`` does the same for an
    array of 2-byte word indices at once.  ``requests`` limits the work to some
    requests (the others stay zero).  An MLA sub-pool needs ``v_dim``, the
    value width taken from the front of each latent row.  Returns (out
    float64 [R, Hq, Dv], set of condition names raised), and with
    ``bound_terms`` also the fp32_error_bound [R, Hq] of every request (0
    where nothing is read; ``weight_rel`` as there).  ``bound_terms`` is the
    longest sum chain: an int for every request, or a function of the
    request's attended position count (e.g. :func:`chain_terms_any_split`).
    ``uniform`` takes the closed form of equal scores (a zero query or a zero
    scale), where softmax weights every position 1/n: the output is the mean
    of the attended value rows, summed in float64 before one division, so
    that for integer values it is the exact mean correctly rounded.
    """
    def read_rows(base, rows, row_bytes):
        """uint16 words of the view rows ``rows`` (row r at byte base + r * row_bytes)."""
        offs = base + rows * row_bytes
        idx = (offs // 2)[:, None] + np.arange(row_bytes // 2)
        if read_words is not None:
            return read_words(idx)
        if read is None:
            return pool.raw[: pool.raw.size // 2 * 2].view(np.uint16)[idx]
        return np.stack([read(int(off), row_bytes) for off in offs])
    spec = pool.specs[sub]
    mla = spec.kind == 1
    if mla:
        assert v_dim is not None and 0 < v_dim <= spec.head_dim, "MLA attention needs 0 < v_dim <= latent width"
        hkv, d, dv = 1, spec.head_dim, v_dim
    else:
        hkv, d, dv = spec.head_num, spec.head_dim, spec.v_head_dim
    ps = pool.page_size
    bpp = pool.plan.subs[sub].blocks_per_page
    bt = np.asarray(block_table, dtype=np.int64)
    width = bt.shape[1] if bt.ndim == 2 else 0
    lens = np.asarray(seq_lens, dtype=np.int64)
    R, hq = q_bits.shape[0], q_bits.shape[1]
    assert hq % hkv == 0
    k_base = pool.view_base(sub, layer, 0)
    v_base = k_base if mla else pool.view_base(sub, layer, 1)  # MLA: values are the latent rows' front
    k_row_bytes = hkv * d * spec.elem_bytes
    v_row_bytes = k_row_bytes if mla else hkv * dv * spec.elem_bytes
    out = np.zeros((R, hq, dv))
    bound = np.zeros((R, hq))
    flags = set()
    for r in (range(R) if requests is None else requests):
        n = int(lens[r])
        if n <= 0:
            continue
        if max_seq_len is not None and n > max_seq_len:
            flags.add("layout")
            continue
        j0 = n - window if (window > 0 and n > window) else 0
        j = np.arange(j0, n, dtype=np.int64)  # attended positions
        col = j // ps
        if (col >= width).any():
            flags.add("bad_block")
            continue
        entry = bt[r, col]
        if ((entry < 0) | (entry % bpp != 0) | (entry // bpp >= spec.num_pages)).any():
            flags.add("bad_block")
            continue
        rows = entry * ps + j % ps
        qf = bf16_bits_to_f64(q_bits[r])
        if uniform:  # the values alone decide the output
            assert scale == 0.0 or not qf.any(), "the uniform closed form needs equal scores"
            v = read_rows(k_base, rows, k_row_bytes)[:, :dv] if mla else read_rows(v_base, rows, v_row_bytes)
            vf = bf16_bits_to_f64(v).reshape(-1, hkv, dv)
            out[r] = vf.sum(axis=0)[np.arange(hq) // (hq // hkv)] / len(rows)
            continue
        k = read_rows(k_base, rows, k_row_bytes)
        v = k[:, :dv] if mla else read_rows(v_base, rows, v_row_bytes)
        kf, vf = bf16_bits_to_f64(k).reshape(-1, hkv, d), bf16_bits_to_f64(v).reshape(-1, hkv, dv)
        out[r] = attend(qf, kf, vf, scale)
        if bound_terms is not None:
            terms = bound_terms(len(rows)) if callable(bound_terms) else bound_terms
            bound[r] = fp32_error_bound(qf, kf, vf, scale, terms, weight_rel)
    if bound_terms is not None:
        return out, frozenset(flags), bound
    return out, frozenset(flags)


# A weight p split into bf16 parts p_hi = bf16(p), p_lo = bf16(p - p_hi) keeps
# p_hi + p_lo within 2^-16 |p| (two 8-bit significands, round to nearest).
BF16_SPLIT_REL = 2.0 ** -16


def default_scale(head_dim: int) -> float:
    """The usual softmax scale, 1 / sqrt(head_dim)."""
    return 1.0 / math.sqrt(head_dim)
