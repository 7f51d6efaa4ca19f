"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module holds none of the method's arithmetic: it never forms a
kernel-facing id, a block count, a view offset or a block-table entry.  It
only draws what a caller of the pool would hold:

* sub-pool shapes (layer count, heads, head dim, itemsize, page count),
* token slots in the allocator's numbering (slot t is offset t % ps of page
  t // ps; -1 is a tombstone),
* per-request physical page lists and lengths,
* row values: bf16 draws from N(0, 1), and a counter-based byte pattern used
  to pre-fill a pool so that every byte that a kernel must not touch is known.

Generators (both published, both re-implemented here from their definitions):

* SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014; output mix as in Vigna's public-domain reference):
  element w of the stream seeded with s is mix(s + (w + 1) * 0x9E3779B97F4A7C15).
* Irwin-Hall (1927): the sum of n independent uniforms; with n = 4 it stands
  in for N(0, 1) where the values must be generated bit-identically on the
  device and on the host (pools of many GiB that attention reads).
* Small integers: the top four bits of a SplitMix64 output, minus 8: values
  whose float32 sums are exact, for checks whose result is known exactly.
* Box-Muller (1958): z0 = sqrt(-2 ln u1) cos(2 pi u2), z1 = sqrt(-2 ln u1) sin(2 pi u2),
  with u1, u2 in (0, 1] from 53-bit SplitMix64 draws; z is rounded to float32
  and then to bfloat16 with round-to-nearest-even on the bit pattern.

Structure (slots, pages, lengths) comes from numpy's PCG64 seeded with
``[seed, sub]`` where sub = 1 slots, 2 pages, 3 tombstones, 4 lengths,
5 values.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
M1 = 0xBF58476D1CE4E5B9
M2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

SUB_SLOTS, SUB_PAGES, SUB_TOMB, SUB_LENS, SUB_VALUES = 1, 2, 3, 4, 5

MHA, MLA = 0, 1


# ----------------------------------------------------------------------------
# SplitMix64 and the pool pre-fill pattern
# ----------------------------------------------------------------------------

def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Elements [start, start+count) of the SplitMix64 stream seeded with ``seed``."""
    w = np.arange(start, start + count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & MASK64) + (w + np.uint64(1)) * np.uint64(GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(M2)
        z = z ^ (z >> np.uint64(31))
    return z


def fill_pattern_host(seed: int, byte_start: int, nbytes: int) -> np.ndarray:
    """Pre-fill bytes [byte_start, byte_start+nbytes) of a pool: 8-byte word w holds element w.

    Both bounds must be multiples of 8.  Little-endian byte order.
    """
    assert byte_start % 8 == 0 and nbytes % 8 == 0
    return splitmix64(seed, byte_start // 8, nbytes // 8).view(np.uint8)


def _i64(c: int) -> int:
    """An unsigned 64-bit constant as the signed int64 with the same bits."""
    return c - (1 << 64) if c >= (1 << 63) else c


def fill_pattern_device(t, seed: int, byte_start: int = 0, chunk_words: int = 1 << 27):
    """Write the pre-fill pattern into a device uint8 tensor ``t`` with torch ops.

    ``t`` holds bytes [byte_start, byte_start + t.numel()).  The same stream as
    :func:`fill_pattern_host`, evaluated in wrapping int64 arithmetic; the
    logical right shift is an arithmetic shift with the sign bits masked off.
    """
    import torch

    assert t.dtype == torch.uint8 and t.is_contiguous()
    assert byte_start % 8 == 0 and t.numel() % 8 == 0
    words = t.view(torch.int64)
    n = words.numel()
    w0 = byte_start // 8
    for a in range(0, n, chunk_words):
        b = min(n, a + chunk_words)
        z = torch.arange(w0 + a + 1, w0 + b + 1, dtype=torch.int64, device=t.device)
        z.mul_(_i64(GAMMA)).add_(_i64(seed & MASK64))
        z ^= (z >> 30) & ((1 << 34) - 1)
        z.mul_(_i64(M1))
        z ^= (z >> 27) & ((1 << 37) - 1)
        z.mul_(_i64(M2))
        z ^= (z >> 31) & ((1 << 33) - 1)
        words[a:b].copy_(z)
        del z


# ----------------------------------------------------------------------------
# bf16 N(0, 1) values
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit pattern, round to nearest even (NaN stays NaN)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    rounded = np.where(nan, (u >> np.uint64(16)) | np.uint64(0x40), rounded)
    return rounded.astype(np.uint16)


def normal_bf16_host(seed: int, count: int, stream: int = SUB_VALUES) -> np.ndarray:
    """``count`` bf16 N(0, 1) draws (as uint16 bit patterns) by Box-Muller over SplitMix64."""
    pairs = (count + 1) // 2
    base_seed = (seed * 0x100000001B3 + stream * GAMMA) & MASK64
    u = splitmix64(base_seed, 0, 2 * pairs)
    u53 = (u >> np.uint64(11)).astype(np.float64)
    uni = (u53 + 1.0) / float(1 << 53)  # (0, 1]
    u1, u2 = uni[0::2], uni[1::2]
    r = np.sqrt(-2.0 * np.log(u1))
    z = np.empty(2 * pairs, dtype=np.float64)
    z[0::2] = r * np.cos(2.0 * np.pi * u2)
    z[1::2] = r * np.sin(2.0 * np.pi * u2)
    return f32_to_bf16_bits(z[:count].astype(np.float32))


def normal_bf16_device(shape, seed: int, device):
    """bf16 N(0, 1) values drawn on the device (torch's Philox generator, seeded)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(*shape, generator=g, dtype=torch.float32, device=device)
    return x.to(torch.bfloat16)


# ----------------------------------------------------------------------------
# Counter-based bf16 values with an approximately N(0, 1) distribution
# ----------------------------------------------------------------------------

# Irwin-Hall sum of four uniform 16-bit integers: mean 4 * 65535 / 2 and
# variance 4 * (65536^2 - 1) / 12; scaled to unit variance.
IH_MEAN = 2 * 65535
IH_SCALE = 1.0 / float(np.sqrt(4.0 * (65536.0 * 65536.0 - 1.0) / 12.0))


def irwin_hall_bf16_host(seed: int, byte_start: int, nbytes: int) -> np.ndarray:
    """bf16 values (as uint16 bit patterns) for bytes [byte_start, byte_start+nbytes) of a buffer.

    The bf16 element at byte 2e is drawn from SplitMix64 element e of the
    stream seeded with ``seed``: the four 16-bit fields of that output are
    summed exactly, centred and scaled in float64 (one rounding), rounded to
    float32 and then to bf16 with round-to-nearest-even on the bits.  The
    result has mean 0, variance 1 and range about +-3.46, and is bit-identical
    to :func:`irwin_hall_bf16_device` (every step is an exact integer step or
    one correctly rounded IEEE operation).
    """
    assert byte_start % 2 == 0 and nbytes % 2 == 0
    z = splitmix64(seed, byte_start // 2, nbytes // 2)
    m = np.uint64(0xFFFF)
    s = ((z & m) + ((z >> np.uint64(16)) & m) + ((z >> np.uint64(32)) & m) + (z >> np.uint64(48))).astype(np.int64)
    x = (s - IH_MEAN).astype(np.float64) * IH_SCALE
    return f32_to_bf16_bits(x.astype(np.float32))


def irwin_hall_fill_device(t, seed: int, byte_start: int = 0, chunk_elems: int = 1 << 27):
    """Write :func:`irwin_hall_bf16_host`'s values for bytes [byte_start, ...) into device uint8 ``t``."""
    import torch

    assert t.dtype == torch.uint8 and t.is_contiguous()
    assert byte_start % 2 == 0 and t.numel() % 2 == 0
    out = t.view(torch.int16)
    n = out.numel()
    e0 = byte_start // 2
    for a in range(0, n, chunk_elems):
        b = min(n, a + chunk_elems)
        z = torch.arange(e0 + a + 1, e0 + b + 1, dtype=torch.int64, device=t.device)
        z.mul_(_i64(GAMMA)).add_(_i64(seed & MASK64))
        z ^= (z >> 30) & ((1 << 34) - 1)
        z.mul_(_i64(M1))
        z ^= (z >> 27) & ((1 << 37) - 1)
        z.mul_(_i64(M2))
        z ^= (z >> 31) & ((1 << 33) - 1)
        s = (z & 0xFFFF) + ((z >> 16) & 0xFFFF) + ((z >> 32) & 0xFFFF) + ((z >> 48) & 0xFFFF)
        del z
        x = (s - IH_MEAN).to(torch.float64).mul_(IH_SCALE).to(torch.float32)
        del s
        u = x.view(torch.int32).to(torch.int64) & 0xFFFFFFFF
        del x
        bits = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        out[a:b].copy_(bits.to(torch.int16))
        del u, bits


# ----------------------------------------------------------------------------
# Small-integer bf16 values
# ----------------------------------------------------------------------------

def small_int_bf16_host(seed: int, byte_start: int, nbytes: int) -> np.ndarray:
    """bf16 bit patterns of integers in [-8, 7] for bytes [byte_start, byte_start+nbytes) of a buffer.

    The element at byte 2e is the top four bits of SplitMix64 element e of the
    stream seeded with ``seed``, minus 8.  Every such integer is exact in bf16,
    and sums of up to 2^21 of them are exact in float32.
    """
    assert byte_start % 2 == 0 and nbytes % 2 == 0
    z = splitmix64(seed, byte_start // 2, nbytes // 2)
    v = (z >> np.uint64(60)).astype(np.int64) - 8
    return (v.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def small_int_bf16_words(seed: int, words: np.ndarray) -> np.ndarray:
    """:func:`small_int_bf16_host`'s values at arbitrary 2-byte word indices (any shape)."""
    w = np.asarray(words, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & MASK64) + (w + np.uint64(1)) * np.uint64(GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(M2)
        z = z ^ (z >> np.uint64(31))
    v = (z >> np.uint64(60)).astype(np.int64) - 8
    return (v.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def small_int_fill_device(t, seed: int, byte_start: int = 0, chunk_elems: int = 1 << 27):
    """Write :func:`small_int_bf16_host`'s values for bytes [byte_start, ...) into device uint8 ``t``."""
    import torch

    assert t.dtype == torch.uint8 and t.is_contiguous()
    assert byte_start % 2 == 0 and t.numel() % 2 == 0
    out = t.view(torch.int16)
    n = out.numel()
    e0 = byte_start // 2
    for a in range(0, n, chunk_elems):
        b = min(n, a + chunk_elems)
        z = torch.arange(e0 + a + 1, e0 + b + 1, dtype=torch.int64, device=t.device)
        z.mul_(_i64(GAMMA)).add_(_i64(seed & MASK64))
        z ^= (z >> 30) & ((1 << 34) - 1)
        z.mul_(_i64(M1))
        z ^= (z >> 27) & ((1 << 37) - 1)
        z.mul_(_i64(M2))
        z ^= (z >> 31) & ((1 << 33) - 1)
        v = ((z >> 60) & 15) - 8
        del z
        bits = (v.to(torch.float32).view(torch.int32) >> 16) & 0xFFFF
        out[a:b].copy_(bits.to(torch.int16))
        del v, bits


# ----------------------------------------------------------------------------
# Shapes of the workloads
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class SubPoolShape:
    kind: int
    layer_num: int
    head_num: int
    head_dim: int
    v_head_dim: int
    elem_bytes: int
    num_pages: int

    @property
    def row_bytes(self) -> int:
        """Bytes of one token's row of one layer (heads x head dim x itemsize)."""
        return self.head_num * self.head_dim * self.elem_bytes


def mha(layer_num, head_num, head_dim, num_pages, elem_bytes=2, v_head_dim=None) -> SubPoolShape:
    return SubPoolShape(MHA, layer_num, head_num, head_dim, head_dim if v_head_dim is None else v_head_dim,
                        elem_bytes, num_pages)


def mla(layer_num, num_pages, latent_dim=576, elem_bytes=2) -> SubPoolShape:
    """MLA latent sub-pool: one latent row of ``latent_dim`` elements per token per layer."""
    return SubPoolShape(MLA, layer_num, 1, latent_dim, 0, elem_bytes, num_pages)


def rng(seed: int, sub: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([seed, sub]))


def live_slots(seed: int, num_pages: int, page_size: int, count: int, first_page: int = 1,
               sub: int = SUB_SLOTS) -> np.ndarray:
    """``count`` distinct token slots on pages [first_page, num_pages) (page 0 is the sink page)."""
    lo = first_page * page_size
    hi = num_pages * page_size
    assert count <= hi - lo
    g = rng(seed, sub)
    if hi - lo <= 4 * count or hi - lo < (1 << 22):
        return (g.permutation(hi - lo)[:count] + lo).astype(np.int64)
    picked = np.unique(g.integers(lo, hi, size=int(count * 1.2) + 16))
    while picked.size < count:
        picked = np.unique(np.concatenate([picked, g.integers(lo, hi, size=count)]))
    return g.permutation(picked)[:count].astype(np.int64)


def page_permutation(seed: int, num_pages: int, sub: int = SUB_PAGES) -> np.ndarray:
    """A seeded permutation of the live pages 1 .. num_pages-1."""
    return (rng(seed, sub).permutation(num_pages - 1) + 1).astype(np.int32)


def slots_of_requests(pages_per_req: Sequence[np.ndarray], lens: Sequence[int], page_size: int) -> np.ndarray:
    """Token slots of each request's positions 0..len-1, concatenated (allocator numbering)."""
    out = []
    for pages, n in zip(pages_per_req, lens):
        j = np.arange(n, dtype=np.int64)
        out.append(np.asarray(pages, dtype=np.int64)[j // page_size] * page_size + j % page_size)
    return np.concatenate(out) if out else np.zeros(0, dtype=np.int64)


def padded_table(pages_per_req: Sequence[np.ndarray], width: Optional[int] = None, pad: int = 0) -> np.ndarray:
    """Per-request page lists as a [num_reqs, width] int32 table (unused entries = ``pad``)."""
    width = max((len(p) for p in pages_per_req), default=0) if width is None else width
    t = np.full((len(pages_per_req), max(width, 1)), pad, dtype=np.int32)
    for r, p in enumerate(pages_per_req):
        t[r, : len(p)] = p
    return t


def out_offsets(lens: Sequence[int], window: int = 0) -> np.ndarray:
    """Ragged output layout: request r's rows start at cu[r]; it keeps its last ``window``
    positions when window > 0, else all of them."""
    lens = np.asarray(lens, dtype=np.int64)
    kept = np.minimum(lens, window) if window > 0 else lens
    return np.concatenate([[0], np.cumsum(kept)]).astype(np.int64)


def compaction_plan(live_pages, num_pages: int):
    """An allocator's compaction choice: live pages above the watermark (the live count,
    counting the sink page 0) move into the free pages below it, lowest first.
    Returns (src_pages, dst_pages) as int32 arrays."""
    live = np.unique(np.asarray(live_pages, dtype=np.int64))
    mark = live.size + 1  # pages [1, mark) can hold every live page
    src = live[live >= mark]
    free_low = np.setdiff1d(np.arange(1, mark), live)
    assert free_low.size >= src.size
    return src.astype(np.int32), free_low[: src.size].astype(np.int32)


# ----------------------------------------------------------------------------
# The five workloads
# ----------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    page_size: int
    shapes: List[SubPoolShape]
    seed: int = 0
    # store: token slots (with -1 tombstones), per sub-pool
    store_slots: Dict[int, np.ndarray] = field(default_factory=dict)
    # gather: per sub-pool, per-request physical page lists and lengths
    req_pages: Dict[int, List[np.ndarray]] = field(default_factory=dict)
    req_lens: Dict[int, np.ndarray] = field(default_factory=dict)
    # per sub-pool list of per-layer windows (0 = full)
    windows: Dict[int, List[int]] = field(default_factory=dict)
    # move: disjoint src / dst slots, per sub-pool
    move_src: Dict[int, np.ndarray] = field(default_factory=dict)
    move_dst: Dict[int, np.ndarray] = field(default_factory=dict)
    notes: str = ""


def tiny_mha(seed: int = 0) -> Workload:
    """Two layers, two heads of dim 8, bf16, page size 4, 16 pages (page 0 = sink page).

    Store 37 entries: 34 distinct live slots on pages 1-15 and 3 tombstones,
    shuffled.  Gather 3 requests of 5, 11 and 21 tokens (2, 3 and 6 pages) whose
    pages are the first 11 entries of a seeded permutation of pages 1-15.  Move 8
    rows to 8 other rows, the two sets disjoint.
    """
    ps, P = 4, 16
    w = Workload("tiny_mha", ps, [mha(2, 2, 8, P)], seed)
    live = live_slots(seed, P, ps, 34)
    slots = np.concatenate([live, np.full(3, -1, dtype=np.int64)])
    w.store_slots[0] = rng(seed, SUB_TOMB).permutation(slots)
    perm = page_permutation(seed, P)
    lens = np.array([5, 11, 21], dtype=np.int32)
    counts = [2, 3, 6]
    starts = np.concatenate([[0], np.cumsum(counts)])
    w.req_pages[0] = [perm[starts[r]: starts[r + 1]] for r in range(3)]
    w.req_lens[0] = lens
    w.windows[0] = [0, 0]
    mv = live_slots(seed, P, ps, 16, sub=SUB_SLOTS + 100)
    w.move_src[0], w.move_dst[0] = mv[:8], mv[8:]
    return w


def decode_8b(num_pages: int = 4096, num_reqs: int = 256, len_lo: int = 1024, len_hi: int = 8192,
              new_tokens: int = 256, layer_num: int = 32, seed: int = 0, share_pages: bool = True) -> Workload:
    """Llama-3-8B-shape decode step: 32 layers, 8 KV heads of dim 128, bf16, page size 16.

    ``num_reqs`` requests with lengths uniform in [len_lo, len_hi].  The pool
    (4,096 pages = 65,536 slots) cannot hold 256 such contexts apart, so each
    request reads its pages cyclically from one seeded permutation of the live
    pages, continuing where the previous request stopped: pages are shared
    between requests (read-only, as prefix sharing would).  The decode store
    writes ``new_tokens`` distinct live slots per layer.

    ``share_pages=False`` keeps the same requests and lengths but sizes the pool
    to hold every context apart (1 + the pages they need, ~74 K pages, ~144 GiB):
    no page is read twice in a layer.
    """
    ps = 16
    g = rng(seed, SUB_LENS)
    lens = g.integers(len_lo, len_hi, endpoint=True, size=num_reqs).astype(np.int32)
    npages = (lens.astype(np.int64) + ps - 1) // ps
    if not share_pages:
        num_pages = int(1 + npages.sum())
    w = Workload("decode_8b", ps, [mha(layer_num, 8, 128, num_pages)], seed)
    perm = page_permutation(seed, num_pages)
    start = np.concatenate([[0], np.cumsum(npages)])
    w.req_pages[0] = [perm[(start[r] + np.arange(npages[r])) % perm.size] for r in range(num_reqs)]
    w.req_lens[0] = lens
    w.windows[0] = [0] * layer_num
    w.store_slots[0] = live_slots(seed, num_pages, ps, new_tokens)
    return w


def dirichlet_lengths(seed: int, total: int, parts: int, alpha: float = 1.0) -> np.ndarray:
    """Split ``total`` tokens into ``parts`` lengths >= 1: a seeded Dirichlet(alpha) share,
    rounded by largest remainder."""
    g = rng(seed, SUB_LENS)
    share = g.dirichlet(np.full(parts, alpha)) * (total - parts)
    base = np.floor(share).astype(np.int64)
    rem = (total - parts) - int(base.sum())
    order = np.argsort(-(share - base), kind="stable")
    base[order[:rem]] += 1
    return (base + 1).astype(np.int32)


def prefill_8b(num_pages: int = 16384, tokens: int = 32768, num_reqs: int = 16, tomb_frac: float = 0.01,
               layer_num: int = 32, move_rows: int = 65536, seed: int = 0) -> Workload:
    """Llama-3-8B-shape prefill/extend: 262,144 slots; 32,768 new tokens over 16 requests.

    Lengths are a seeded Dirichlet(1) split; each request takes ceil(len/16)
    pages in a row from one seeded page permutation and fills them in order,
    so its tokens form runs of whole pages.  1% of the slots are tombstones.
    The same pool also serves a gather of the 16 requests back and a move of
    ``move_rows`` distinct live rows to ``move_rows`` other live rows.
    """
    ps = 16
    w = Workload("prefill_8b", ps, [mha(layer_num, 8, 128, num_pages)], seed)
    lens = dirichlet_lengths(seed, tokens, num_reqs)
    perm = page_permutation(seed, num_pages)
    npages = (lens.astype(np.int64) + ps - 1) // ps
    start = np.concatenate([[0], np.cumsum(npages)])
    assert start[-1] <= perm.size, "pool too small for the requests"
    pages = [perm[start[r]: start[r + 1]] for r in range(num_reqs)]
    slots = slots_of_requests(pages, lens, ps)
    n_tomb = int(round(tomb_frac * slots.size))
    tomb_at = rng(seed, SUB_TOMB).choice(slots.size, size=n_tomb, replace=False)
    store = slots.copy()
    store[tomb_at] = -1
    w.store_slots[0] = store
    w.req_pages[0] = pages
    w.req_lens[0] = lens
    w.windows[0] = [0] * layer_num
    if move_rows:
        s = live_slots(seed, num_pages, ps, 2 * move_rows, sub=SUB_SLOTS + 100)
        w.move_src[0], w.move_dst[0] = s[:move_rows], s[move_rows:]
    return w


def hybrid(num_reqs: int = 128, len_lo: int = 256, len_hi: int = 16384, layer_num: int = 24,
           window: int = 128, seed: int = 0) -> Workload:
    """Hybrid unified pool: an MHA sub-pool (24 layers, 8 KV heads of dim 64, bf16) whose
    layers alternate full / sliding-window 128, beside an MLA sub-pool (24 layers, one
    576-wide latent row per token per layer).  Page size 64.

    Each sub-pool holds every request apart: 1 sink page + sum(ceil(len/64)) pages,
    each sub-pool with its own seeded page permutation.  Every request's whole context
    is stored on every layer of both sub-pools, then gathered back: MHA layer l is
    full when l is even and keeps the last ``window`` positions when l is odd; every
    MLA layer is full.
    """
    ps = 64
    g = rng(seed, SUB_LENS)
    lens = g.integers(len_lo, len_hi, endpoint=True, size=num_reqs).astype(np.int32)
    npages = (lens.astype(np.int64) + ps - 1) // ps
    P = int(1 + npages.sum())
    w = Workload("hybrid", ps, [mha(layer_num, 8, 64, P), mla(layer_num, P)], seed)
    start = np.concatenate([[0], np.cumsum(npages)])
    for sub in (0, 1):
        perm = page_permutation(seed, P, sub=SUB_PAGES + 10 * sub)
        pages = [perm[start[r]: start[r + 1]] for r in range(num_reqs)]
        w.req_pages[sub] = pages
        w.req_lens[sub] = lens
        w.store_slots[sub] = slots_of_requests(pages, lens, ps)
    w.windows[0] = [0 if l % 2 == 0 else window for l in range(layer_num)]
    w.windows[1] = [0] * layer_num
    return w


def swa_decode(num_reqs: int = 128, len_lo: int = 256, len_hi: int = 16384, layer_num: int = 24, window: int = 128,
               seed: int = 0) -> Workload:
    """Hybrid decode step with the sliding-window layers in a sub-pool of their own.

    Sub-pool 0 holds the full-attention layers (even layers of a 24-layer model,
    8 KV heads of dim 64, bf16, page 64), sub-pool 1 the sliding-window ones (odd
    layers, window 128).  ``num_reqs`` requests of U[len_lo, len_hi] tokens get
    one new token each.  Full pages come from a seeded permutation (room for the
    new token included); every full page that overlaps a request's window after
    the new token, and ``stale`` older pages, are mapped to SWA pages from their
    own permutation (``mapping``: full page -> SWA page, -1 = not resident).
    """
    ps = 64
    g = rng(seed, SUB_LENS)
    lens = g.integers(len_lo, len_hi, endpoint=True, size=num_reqs).astype(np.int32)
    new_len = lens.astype(np.int64) + 1
    npages = (new_len + ps - 1) // ps
    P_full = int(1 + npages.sum())
    first = np.maximum(new_len - window, 0) // ps  # first page overlapping the window
    stale = np.minimum(first, 2)  # two pages that left the window still mapped
    n_swa = int((npages - first + stale).sum())
    P_swa = 1 + n_swa
    half = layer_num // 2
    w = Workload("swa_decode", ps, [mha(half, 8, 64, P_full), mha(half, 8, 64, P_swa)], seed)
    perm = page_permutation(seed, P_full)
    start = np.concatenate([[0], np.cumsum(npages)])
    pages = [perm[start[r]: start[r + 1]] for r in range(num_reqs)]
    w.req_pages[0] = pages
    w.req_lens[0] = new_len.astype(np.int32)
    w.windows[0] = [0] * half
    w.windows[1] = [window] * half
    mapping = np.full(P_full, -1, dtype=np.int32)
    swa_perm = page_permutation(seed, P_swa, sub=SUB_PAGES + 10)
    at = 0
    for r in range(num_reqs):
        for i in range(int(first[r] - stale[r]), int(npages[r])):
            mapping[pages[r][i]] = swa_perm[at]
            at += 1
    w.store_slots[0] = np.array([pages[r][lens[r] // ps] * ps + lens[r] % ps for r in range(num_reqs)],
                                dtype=np.int64)
    w.notes = "mapping"
    w.swa_mapping = mapping
    w.window = window
    return w


def move_70b(num_pages: int = 32768, rows: int = 65536, layer_num: int = 80, seed: int = 0) -> Workload:
    """Llama-3-70B-shape pool: 80 layers, 8 KV heads of dim 128, bf16, page size 16;
    32,768 pages (160 GiB of envelopes).  Move ``rows`` live rows to ``rows`` other
    live rows, src and dst disjoint, on every layer."""
    ps = 16
    w = Workload("move_70b", ps, [mha(layer_num, 8, 128, num_pages)], seed)
    s = live_slots(seed, num_pages, ps, 2 * rows)
    w.move_src[0], w.move_dst[0] = s[:rows], s[rows:]
    return w


__all__ = [
    "splitmix64", "fill_pattern_host", "fill_pattern_device", "f32_to_bf16_bits", "normal_bf16_host",
    "normal_bf16_device", "SubPoolShape", "mha", "mla", "rng", "live_slots", "page_permutation",
    "slots_of_requests", "padded_table", "out_offsets", "Workload", "tiny_mha", "decode_8b",
    "dirichlet_lengths", "prefill_8b", "hybrid", "move_70b", "compaction_plan", "swa_decode", "MHA", "MLA",
    "irwin_hall_bf16_host", "irwin_hall_fill_device", "small_int_bf16_host", "small_int_bf16_words", "small_int_fill_device",
]
