"""Pins for the CPU oracle, against facts that do not come from the oracle itself.

Source page: "PR #34602: feat(unified-memory): dense KV views for uniform-row
MHA/SWA models" (sglang report).  What pins what:

* ``walk()`` below enumerates a page envelope in memory order straight from its
  description ``[L0_K*ps | L0_V*ps | L1_K*ps | ...]`` (implementation step 1):
  it never uses a kernel id, a block index or a view offset.  Addressing,
  view bases, translate, the tail pad and the row bound are checked against it
  by brute force on tiny pools.
* ``oracle/strided.py`` (the nested strided reference, the page's own test
  oracle) checks the oracle's store / gather / move byte for byte.
* Gates are checked at boundary values that the walk determines.
"""
import itertools

import numpy as np
import pytest

import oracle
from oracle import MHA, MLA, Spec
from oracle.strided import StridedPool, layer_view_4d
import ukv_workloads as W


def walk(num_pages, layer_num, kind, page_size, row_bytes, anchor=0):
    """Byte address of every (page, layer, kv, offset) row, walking the envelope in order."""
    addr = anchor
    out = {}
    kvs = (0, 1) if kind == MHA else (0,)
    for p in range(num_pages):
        for l in range(layer_num):
            for kv in kvs:
                for o in range(page_size):
                    out[(p, l, kv, o)] = addr
                    addr += row_bytes
    return out, addr


SHAPES = [
    (kind, L, ps, P, H, D, es)
    for kind in (MHA, MLA)
    for L in (1, 2, 3)
    for ps in (1, 2, 4)
    for P in (1, 2, 5)
    for (H, D, es) in ((1, 4, 2), (2, 8, 2), (3, 2, 1))
]


def make_spec(kind, L, P, H, D, es):
    return Spec(kind, L, H, D, D if kind == MHA else 0, es, P)


@pytest.mark.parametrize("kind,L,ps,P,H,D,es", SHAPES)
def test_addressing_matches_envelope_walk(kind, L, ps, P, H, D, es):
    pool = oracle.OraclePool([make_spec(kind, L, P, H, D, es)], ps)
    sp = pool.plan.subs[0]
    rb = H * D * es
    addrs, end = walk(P, L, kind, ps, rb)
    assert sp.row_bytes == rb
    assert sp.envelope_bytes == end
    assert sp.page_bytes == end // P
    for (p, l, kv, o), a in addrs.items():
        base = pool.view_base(0, l, kv)
        kid = oracle.kernel_id(p * ps + o, ps, sp.blocks_per_page)
        assert base + kid * rb == a, (p, l, kv, o)
        assert 0 <= kid < sp.n_rows


@pytest.mark.parametrize("kind,L,ps,P,H,D,es", SHAPES[::5])
def test_spec_offsets_equal_block_origins(kind, L, ps, P, H, D, es):
    pool = oracle.OraclePool([make_spec(kind, L, P, H, D, es)], ps)
    addrs, _ = walk(P, L, kind, ps, H * D * es)
    for l in range(L):
        for kv in ((0, 1) if kind == MHA else (0,)):
            assert pool.view_base(0, l, kv) == addrs[(0, l, kv, 0)]


@pytest.mark.parametrize("L,ps,P", [(1, 1, 1), (2, 4, 3), (3, 2, 5)])
def test_k_and_v_share_an_id_without_aliasing(L, ps, P):
    spec = make_spec(MHA, L, P, 2, 8, 2)
    pool = oracle.OraclePool([spec], ps)
    sp = pool.plan.subs[0]
    rb = sp.row_bytes
    seen = set()
    for t in range(P * ps):
        kid = oracle.kernel_id(t, ps, sp.blocks_per_page)
        for l in range(L):
            k = pool.view_base(0, l, 0) + kid * rb
            v = pool.view_base(0, l, 1) + kid * rb
            assert v - k == ps * rb
            seen.update((k, v))
    # a bijection onto the envelope, one row per rb bytes
    assert sorted(seen) == list(range(0, sp.envelope_bytes, rb))


@pytest.mark.parametrize("kind,L,ps,P", [(MHA, 2, 4, 16), (MHA, 3, 1, 2), (MLA, 3, 4, 5), (MLA, 1, 2, 3)])
def test_tail_pad_covers_view_overrun_and_is_one_envelope(kind, L, ps, P):
    spec = make_spec(kind, L, P, 2, 8, 2)
    pool = oracle.OraclePool([spec], ps)
    sp = pool.plan.subs[0]
    addrs, end = walk(P, L, kind, ps, sp.row_bytes)
    # furthest byte any dense view reaches, from the view bases the walk pinned
    reach = max(pool.view_base(0, l, kv) + sp.n_rows * sp.row_bytes
                for l in range(L) for kv in ((0, 1) if kind == MHA else (0,)))
    assert reach - end <= sp.tail_pad_bytes
    # "a whole page envelope" of pad: the bytes of one page in the walk
    assert sp.tail_pad_bytes == end // P
    assert pool.plan.required_bytes == end + sp.tail_pad_bytes
    # valid kernel ids never reach the pad: the last row the walk knows ends the envelope
    assert max(addrs.values()) + sp.row_bytes == end


def test_builder_check_boundaries_tiny_pool():
    """Two layers, two heads of dim 8, bf16, page size 4, 16 pages."""
    spec = make_spec(MHA, 2, 16, 2, 8, 2)
    pool = oracle.OraclePool([spec], 4)
    sp = pool.plan.subs[0]
    _, end = walk(16, 2, MHA, 4, 32)
    overrun = max(pool.view_base(0, l, kv) + sp.n_rows * 32 for l in range(2) for kv in (0, 1)) - end
    assert overrun == 3 * 4 * 32  # three blocks of four 32-byte rows past the last envelope
    assert pool.builder_check(0, end)[0] == "tail_pad"
    assert pool.builder_check(0, end + overrun - 1)[0] == "tail_pad"
    assert pool.builder_check(0, end + overrun) == ("ok", end + overrun)
    assert pool.plan.required_bytes == end + sp.page_bytes == 8192 + 512


def test_pool_tail_pad_is_max_over_specs_and_subpools_back_to_back():
    a = make_spec(MHA, 2, 3, 2, 8, 2)
    b = make_spec(MLA, 5, 4, 1, 16, 2)
    pool = oracle.OraclePool([a, b], 4)
    sa, sb = pool.plan.subs
    wa, ea = walk(3, 2, MHA, 4, 32)
    wb, eb = walk(4, 5, MLA, 4, 32, anchor=ea)
    assert sb.anchor_bytes == ea
    assert pool.plan.tail_pad_bytes == max(sa.tail_pad_bytes, sb.tail_pad_bytes) == max(ea // 3, (eb - ea) // 4)
    assert pool.plan.required_bytes == eb + pool.plan.tail_pad_bytes
    for (p, l, kv, o), addr in wb.items():
        kid = oracle.kernel_id(p * 4 + o, 4, sb.blocks_per_page)
        assert pool.view_base(1, l, kv) + kid * 32 == addr


def test_multiplier_one_collapse_aliases_k_over_v():
    """With a page multiplier of 1 (the override the pages keep only for tests), a K write
    for a slot on page 1 lands in page 0's V rows: physical ids written into dense rows."""
    ps, L, P = 4, 2, 3
    pool = oracle.OraclePool([make_spec(MHA, L, P, 2, 8, 2)], ps)
    rb = 32
    addrs, _ = walk(P, L, MHA, ps, rb)
    for o in range(ps):
        wrong = pool.view_base(0, 0, 0) + oracle.kernel_id(1 * ps + o, ps, 1) * rb
        assert wrong == addrs[(0, 0, 1, o)]  # page 0, layer 0, V
        assert wrong != addrs[(1, 0, 0, o)]
        right = pool.view_base(0, 0, 0) + oracle.kernel_id(1 * ps + o, ps, 2 * L) * rb
        assert right == addrs[(1, 0, 0, o)]


def test_asymmetric_kv_rejected_mla_exempt():
    assert oracle.plan([Spec(MHA, 2, 8, 192, 128, 2, 4)], 16).code == "asymmetric_kv"
    assert oracle.plan([Spec(MHA, 2, 8, 128, 128, 2, 4)], 16).code == "ok"
    assert oracle.plan([Spec(MLA, 2, 1, 576, 512, 2, 4)], 16).code == "ok"
    # a later asymmetric spec rejects the whole pool
    assert oracle.plan([Spec(MLA, 2, 1, 576, 0, 2, 4), Spec(MHA, 2, 8, 64, 128, 2, 4)], 16).code == "asymmetric_kv"


def _rows_per_page(L, kind, ps):
    addrs, _ = walk(1, L, kind, ps, 1)
    return len(addrs)


@pytest.mark.parametrize("L,ps", [(80, 16), (32, 16), (3, 4)])
def test_int32_row_bound_boundary(L, ps):
    per_page = _rows_per_page(L, MHA, ps)  # rows one page adds to every dense view
    limit = 1 << 31
    p_max = (limit - 1) // per_page  # the largest page count whose rows stay below 2^31
    ok = oracle.plan([Spec(MHA, L, 8, 128, 128, 2, p_max)], ps)
    bad = oracle.plan([Spec(MHA, L, 8, 128, 128, 2, p_max + 1)], ps)
    assert ok.code == "ok" and ok.subs[0].n_rows == p_max * per_page < limit
    assert bad.code == "kernel_id_bound"
    if (L, ps) == (80, 16):
        assert (p_max, p_max * per_page) == (838860, 2147481600)
    if (L, ps) == (32, 16):
        # 2^21 pages give exactly 2^31 rows: rejected, "must be less than 2^31"
        assert oracle.plan([Spec(MHA, L, 8, 128, 128, 2, 1 << 21)], ps).code == "kernel_id_bound"
        assert p_max == (1 << 21) - 1


def test_invalid_and_overflow_specs():
    good = Spec(MHA, 2, 2, 8, 8, 2, 4)
    assert oracle.plan([], 4).code == "invalid_arg"
    assert oracle.plan([good], 0).code == "invalid_arg"
    for bad in (Spec(MHA, 0, 2, 8, 8, 2, 4), Spec(MHA, 2, 0, 8, 8, 2, 4), Spec(MHA, 2, 2, 0, 0, 2, 4),
                Spec(MHA, 2, 2, 8, 8, 3, 4), Spec(MHA, 2, 2, 8, 8, 2, 0), Spec(7, 2, 2, 8, 8, 2, 4)):
        assert oracle.plan([bad], 4).code == "invalid_arg", bad
    assert oracle.plan([good] * 9, 4).code == "invalid_arg"
    huge = Spec(MHA, 1, 1 << 30, 1 << 30, 1 << 30, 8, 1)
    assert oracle.plan([huge], 1).code == "overflow"
    # anchors must be multiples of the itemsize: a 1-byte sub-pool of odd size, then a 2-byte one
    odd = Spec(MLA, 1, 1, 3, 0, 1, 1)
    assert oracle.plan([odd, Spec(MLA, 1, 1, 4, 0, 2, 1)], 1).code == "alignment"


# ---------------------------------------------------------------------------
# translate
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind,L,ps,P", [(MHA, 2, 4, 5), (MHA, 1, 1, 3), (MLA, 3, 2, 4), (MHA, 3, 16, 2)])
def test_translate_brute_force_against_walk(kind, L, ps, P):
    spec = make_spec(kind, L, P, 1, 4, 2)
    pool = oracle.OraclePool([spec], ps)
    rb = pool.plan.subs[0].row_bytes
    addrs, _ = walk(P, L, kind, ps, rb)
    slots = np.arange(P * ps, dtype=np.int64)
    ids, flags = pool.translate(0, slots)
    assert flags == frozenset()
    base = pool.view_base(0, 0, 0)
    for t, kid in zip(slots, ids):
        p, o = divmod(int(t), ps)
        assert base + int(kid) * rb == addrs[(p, 0, 0, o)]


def test_translate_tombstones_unmapped_and_range():
    ps, L, P = 4, 2, 6
    bpp = 2 * L
    pool = oracle.OraclePool([make_spec(MHA, L, P, 2, 8, 2)], ps)
    ids, flags = pool.translate(0, [-1, -5, -4, 0, 3])
    assert ids.tolist() == [0, 0, 0, 0, 3] and flags == frozenset()
    ids, flags = pool.translate(0, [P * ps])
    assert ids.tolist() == [0] and flags == {"slot_range"}
    # with a virtual-to-physical table: page 0 -> 2, page 1 unmapped, page 2 -> 5, page 3 -> 9 (past the pool)
    v2p = np.array([2, -1, 5, 9], dtype=np.int32)
    slots = np.array([1, 5, 10, -1, 14, 17], dtype=np.int64)
    ids, flags = pool.translate(0, slots, v2p)
    exp = [2 * ps * bpp + 1, 0, 5 * ps * bpp + 2, 0, 0, 0]
    assert ids.tolist() == exp
    assert flags == {"slot_range"}
    # ps == 1: phys * blocks_per_page
    pool1 = oracle.OraclePool([make_spec(MHA, L, P, 2, 8, 2)], 1)
    ids, _ = pool1.translate(0, np.arange(P))
    assert ids.tolist() == [p * bpp for p in range(P)]
    # one block per page: the kernel-facing id is the physical slot
    ids = [oracle.kernel_id(t, ps, 1) for t in range(P * ps)]
    assert ids == list(range(P * ps))


def test_translate_pages_matches_first_slot_rows():
    ps, L, P = 4, 3, 7
    pool = oracle.OraclePool([make_spec(MHA, L, P, 2, 8, 2)], ps)
    rb = 32
    addrs, _ = walk(P, L, MHA, ps, rb)
    pages = np.array([0, 3, 6, -1, 2], dtype=np.int32)
    kp, flags = pool.translate_pages(0, pages)
    assert flags == frozenset()
    base = pool.view_base(0, 0, 0)
    for q, e in zip(pages, kp):
        if q < 0:
            assert e == 0
            continue
        for o in range(ps):
            assert base + (int(e) * ps + o) * rb == addrs[(int(q), 0, 0, o)]
    kp, flags = pool.translate_pages(0, np.array([7], dtype=np.int32))
    assert kp.tolist() == [0] and flags == {"slot_range"}
    kp, flags = pool.translate_pages(0, np.array([1, 0, 2], dtype=np.int32), v2p=np.array([4, -3], dtype=np.int32))
    assert kp.tolist() == [0, 4 * 2 * L, 0] and flags == {"slot_range"}


# ---------------------------------------------------------------------------
# store / gather / move against the strided reference
# ---------------------------------------------------------------------------

def _filled_pool(shapes, ps, seed=7):
    specs = [Spec(s.kind, s.layer_num, s.head_num, s.head_dim, s.v_head_dim, s.elem_bytes, s.num_pages) for s in shapes]
    req = oracle.plan(specs, ps).required_bytes
    n = (req + 7) // 8 * 8
    raw = W.fill_pattern_host(seed, 0, n).copy()
    return oracle.OraclePool(specs, ps, raw), raw


def _strided(pool, sub):
    s, sp = pool.specs[sub], pool.plan.subs[sub]
    return StridedPool(pool.raw, sp.anchor_bytes, s.num_pages, s.layer_num, s.kind == MLA, pool.page_size, sp.row_bytes)


def _rows(seed, n, rb):
    return W.normal_bf16_host(seed, n * rb // 2).view(np.uint8).reshape(n, rb)


def test_store_matches_strided_reference_tiny():
    w = W.tiny_mha()
    pool, raw = _filled_pool(w.shapes, w.page_size)
    ref_raw = raw.copy()
    ref = StridedPool(ref_raw, 0, 16, 2, False, 4, 32)
    slots = w.store_slots[0]
    ids, flags = pool.translate(0, slots)
    assert flags == frozenset()
    for layer in range(2):
        k = _rows(10 + layer, slots.size, 32)
        v = _rows(20 + layer, slots.size, 32)
        assert pool.store(0, layer, ids, k, v) == frozenset()
        # reference: live slots at (page, offset); tombstones at the page-0 sink row, in order
        ref.store_slots(layer, slots, k, v)
        for i in np.nonzero(slots < 0)[0]:
            ref.env[0, layer, 0, 0] = k[i]
            ref.env[0, layer, 1, 0] = v[i]
    assert np.array_equal(raw, ref_raw)


def test_store_skips_and_flags_ids_off_the_kernel_space():
    pool, raw = _filled_pool([W.mha(2, 2, 8, 4)], 4)
    before = raw.copy()
    bad = [4, 15, 4 * 16, -2]  # block 1 of page 0, block 3 of page 0, page 4 (past the pool), negative
    for i in bad:
        assert pool.store(0, 0, [i], _rows(1, 1, 32), _rows(2, 1, 32)) == {"bad_id"}
    assert np.array_equal(raw, before)


@pytest.mark.parametrize("window", [0, 3, 8, 100])
def test_gather_matches_strided_reference(window):
    w = W.tiny_mha()
    pool, raw = _filled_pool(w.shapes, w.page_size)
    ref = _strided(pool, 0)
    pages, lens = w.req_pages[0], w.req_lens[0]
    table = W.padded_table(pages)
    bt, flags = pool.translate_pages(0, table)
    assert flags == frozenset()
    cu = W.out_offsets(lens, window)
    for layer in range(2):
        k_out = np.zeros((cu[-1], 32), dtype=np.uint8)
        v_out = np.zeros((cu[-1], 32), dtype=np.uint8)
        assert pool.gather(0, layer, bt, lens, cu, window, k_out, v_out) == frozenset()
        rk, rv = ref.gather_pages(layer, pages, lens, window)
        assert np.array_equal(k_out, rk) and np.array_equal(v_out, rv)


def test_store_then_gather_round_trip_and_mla():
    w = W.hybrid(num_reqs=3, len_lo=5, len_hi=150, layer_num=2, window=7)
    pool, raw = _filled_pool(w.shapes, w.page_size)
    for sub in (0, 1):
        rb = pool.row_bytes(sub)
        slots = w.store_slots[sub]
        ids, _ = pool.translate(sub, slots)
        bt, _ = pool.translate_pages(sub, W.padded_table(w.req_pages[sub]))
        lens = w.req_lens[sub]
        for layer in range(2):
            k = _rows(30 + layer + 10 * sub, slots.size, rb)
            v = _rows(40 + layer, slots.size, rb) if sub == 0 else None
            assert pool.store(sub, layer, ids, k, v) == frozenset()
            win = w.windows[sub][layer]
            cu = W.out_offsets(lens, win)
            ko = np.zeros((cu[-1], rb), dtype=np.uint8)
            vo = np.zeros((cu[-1], rb), dtype=np.uint8) if sub == 0 else None
            assert pool.gather(sub, layer, bt, lens, cu, win, ko, vo) == frozenset()
            # expected: request r keeps its last `win` positions (all when win == 0)
            starts = np.concatenate([[0], np.cumsum(lens)])
            keep = np.concatenate([np.arange(starts[r] + (lens[r] - win if 0 < win < lens[r] else 0), starts[r + 1])
                                   for r in range(len(lens))])
            assert np.array_equal(ko, k[keep])
            if sub == 0:
                assert np.array_equal(vo, v[keep])
    # nothing outside the two sub-pools' envelopes moved: the tail pad is intact
    end = pool.plan.subs[1].anchor_bytes + pool.plan.subs[1].envelope_bytes
    fill = W.fill_pattern_host(7, 0, (pool.plan.required_bytes + 7) // 8 * 8)
    assert np.array_equal(raw[end:], fill[end:])


def test_gather_flags_bad_blocks_and_layout():
    pool, raw = _filled_pool([W.mha(2, 2, 8, 4)], 4)
    lens = np.array([3, 2], dtype=np.int32)
    bt = np.array([[4, 0], [5, 0]], dtype=np.int32)  # 5 is not a multiple of the 4 blocks per page
    cu = W.out_offsets(lens)
    ko = np.zeros((5, 32), np.uint8)
    vo = np.zeros((5, 32), np.uint8)
    assert pool.gather(0, 0, bt, lens, cu, 0, ko, vo) == {"bad_block"}
    assert not ko[3:].any()
    cu_bad = np.array([0, 2, 5], dtype=np.int64)  # request 0 gets 2 rows for 3 positions, request 1 gets 3 for 2
    assert "layout" in pool.gather(0, 0, np.array([[4, 0], [8, 0]], np.int32), lens, cu_bad, 0, ko, vo)
    ko2 = np.zeros((6, 32), np.uint8)
    assert pool.gather(0, 0, np.array([[4, 0], [8, 0]], np.int32), lens, cu, 0, ko2, ko2.copy()) == {"layout"}


def test_move_matches_strided_reference_and_is_reversible():
    w = W.tiny_mha()
    pool, raw = _filled_pool(w.shapes, w.page_size)
    orig = raw.copy()
    ref_raw = raw.copy()
    ref = StridedPool(ref_raw, 0, 16, 2, False, 4, 32)
    src_ids, _ = pool.translate(0, w.move_src[0])
    dst_ids, _ = pool.translate(0, w.move_dst[0])
    assert pool.move(0, dst_ids, src_ids, 0, 2) == frozenset()
    for layer in range(2):
        for kv in (0, 1):
            snap = [ref.row(layer, kv, *divmod(int(s), 4)).copy() for s in w.move_src[0]]
            for d, row in zip(w.move_dst[0], snap):
                ref.env[divmod(int(d), 4)[0], layer, kv, divmod(int(d), 4)[1]] = row
    assert np.array_equal(raw, ref_raw)
    # moving the original dst contents back needs them saved: a move is a gather(src) then a store(dst)
    pool2, raw2 = _filled_pool(w.shapes, w.page_size)
    for layer in range(2):
        rows_k = np.stack([orig[pool.view_base(0, layer, 0) + int(i) * 32:][:32] for i in src_ids])
        rows_v = np.stack([orig[pool.view_base(0, layer, 1) + int(i) * 32:][:32] for i in src_ids])
        pool2.store(0, layer, dst_ids, rows_k, rows_v)
    assert np.array_equal(raw2, raw)
    # src and dst swapped twice restores the pool
    pool3, raw3 = _filled_pool(w.shapes, w.page_size)
    both_a = np.concatenate([src_ids, dst_ids])
    both_b = np.concatenate([dst_ids, src_ids])
    pool3.move(0, both_b, both_a, 0, 2)
    assert not np.array_equal(raw3, orig)
    pool3.move(0, both_b, both_a, 0, 2)
    assert np.array_equal(raw3, orig)


def test_move_partial_layer_range_and_bad_ids():
    w = W.tiny_mha()
    pool, raw = _filled_pool(w.shapes, w.page_size)
    orig = raw.copy()
    src_ids, _ = pool.translate(0, w.move_src[0])
    dst_ids, _ = pool.translate(0, w.move_dst[0])
    pool.move(0, dst_ids, src_ids, 1, 2)
    for kv in (0, 1):
        b0 = pool.view_base(0, 0, kv)
        for i in dst_ids:
            assert np.array_equal(raw[b0 + int(i) * 32:][:32], orig[b0 + int(i) * 32:][:32])  # layer 0 untouched
    raw[:] = orig
    assert pool.move(0, np.array([5], np.int32), src_ids[:1], 0, 2) == {"bad_id"}
    assert np.array_equal(raw, orig)


def test_layer_view_4d_agrees_with_dense_rows():
    """The old 4-D per-layer view (page, offset, head, dim) and the dense 3-D view read the same words."""
    spec = make_spec(MHA, 3, 4, 2, 8, 2)
    pool, raw = _filled_pool([W.mha(3, 2, 8, 4)], 2)
    for l, kv in itertools.product(range(3), (0, 1)):
        v4 = layer_view_4d(raw, 0, 4, 3, 2, 2, 2, 8, 2, l, kv)
        base = pool.view_base(0, l, kv)
        for p, o in itertools.product(range(4), range(2)):
            kid = oracle.kernel_id(p * 2 + o, 2, 6)
            dense = raw[base + kid * 32: base + kid * 32 + 32].view(np.uint16).reshape(2, 8)
            assert np.array_equal(v4[p, o], dense)


def test_address_maps_match_strided_reference_and_need_no_buffer():
    """The store / gather / move address maps (used for pool-sized checks) give the
    strided reference's row addresses, and an addresses-only pool gives the same."""
    w = W.hybrid(num_reqs=4, len_lo=3, len_hi=200, layer_num=3, window=5)
    pool, raw = _filled_pool(w.shapes, w.page_size)
    bare = oracle.OraclePool(pool.specs, w.page_size, addresses_only=True)
    for sub in (0, 1):
        ref = _strided(pool, sub)
        kvs = (0, 1) if sub == 0 else (0,)
        slots = w.store_slots[sub]
        ids, _ = pool.translate(sub, slots)
        for layer in range(3):
            maps = pool.store_map(sub, layer, ids)
            assert all(np.array_equal(a, b) for a, b in zip(maps[:2], bare.store_map(sub, layer, ids)[:2]) if a is not None)
            for kv in kvs:
                exp = [ref.row_address(layer, kv, *divmod(int(t), w.page_size)) for t in slots]
                assert maps[kv].tolist() == exp
            lens = w.req_lens[sub]
            bt, _ = pool.translate_pages(sub, W.padded_table(w.req_pages[sub]))
            win = w.windows[sub][layer]
            cu = W.out_offsets(lens, win)
            gm = pool.gather_map(sub, layer, bt, lens, cu, win, int(cu[-1]))
            assert gm[2] == frozenset()
            exp_k = []
            for pages, n in zip(w.req_pages[sub], lens):
                j0 = n - win if 0 < win < n else 0
                exp_k += [ref.row_address(layer, 0, int(pages[j // w.page_size]), j % w.page_size) for j in range(j0, n)]
            assert gm[0].tolist() == exp_k
            assert np.array_equal(gm[0], bare.gather_map(sub, layer, bt, lens, cu, win, int(cu[-1]))[0])
        mv = W.live_slots(3, w.shapes[sub].num_pages, w.page_size, 10, sub=31)
        src, _ = pool.translate(sub, mv[:5])
        dst, _ = pool.translate(sub, mv[5:])
        d_off, s_off, fl = pool.move_map(sub, dst, src, 1, 3)
        assert fl == frozenset()
        at = 0
        for layer in (1, 2):
            for kv in kvs:
                for i in range(5):
                    assert s_off[at] == ref.row_address(layer, kv, *divmod(int(mv[i]), w.page_size))
                    assert d_off[at] == ref.row_address(layer, kv, *divmod(int(mv[5 + i]), w.page_size))
                    at += 1
        assert at == d_off.size


# ---------------------------------------------------------------------------
# virtual-to-physical indirection and compaction
# ---------------------------------------------------------------------------

def test_translate_loc_is_the_physical_slot_behind_every_kernel_id():
    ps, L, P = 4, 3, 9
    pool = oracle.OraclePool([make_spec(MHA, L, P, 2, 8, 2)], ps)
    bpp = 2 * L
    v2p = np.array([5, -1, 2, 8, 0, 11], dtype=np.int32)  # 11 is past the pool
    slots = np.arange(-2, 6 * ps + 3, dtype=np.int64)
    internal, f_int = pool.translate_loc(0, slots, v2p)
    kernel, f_ker = pool.translate(0, slots, v2p)
    assert f_int == f_ker == {"slot_range"}
    for t, i, k in zip(slots, internal, kernel):
        if i >= 0:
            assert oracle.kernel_id(int(i), ps, bpp) == k
        else:
            assert k == 0  # tombstone, unmapped or out of range: the kernel id is the sink
    assert internal[slots == -1][0] == -1
    ident, _ = pool.translate_loc(0, np.arange(P * ps))
    assert ident.tolist() == list(range(P * ps))


def test_page_move_copies_whole_envelopes():
    """A page's rows on every layer, K and V, are one contiguous envelope (the walk):
    moving page s to d copies exactly those bytes and nothing else."""
    shapes = [W.mha(3, 2, 8, 7), W.mla(2, 5, latent_dim=16)]
    pool, raw = _filled_pool(shapes, 4)
    orig = raw.copy()
    for sub in (0, 1):
        sp = pool.plan.subs[sub]
        assert pool.move_pages(sub, [1, 6 if sub == 0 else 4], [3, 2]) == frozenset()
        for d, s in ((1, 3), (6 if sub == 0 else 4, 2)):
            a_d = sp.anchor_bytes + d * sp.page_bytes
            a_s = sp.anchor_bytes + s * sp.page_bytes
            assert np.array_equal(raw[a_d:a_d + sp.page_bytes], orig[a_s:a_s + sp.page_bytes])
            orig[a_d:a_d + sp.page_bytes] = orig[a_s:a_s + sp.page_bytes]
    assert np.array_equal(raw, orig)
    assert pool.move_pages(0, [7], [1]) == {"bad_id"}
    assert np.array_equal(raw, orig)


def test_compaction_preserves_what_requests_read():
    """Relocate the pages above a watermark into free pages below it, rewrite the table:
    every request gathers the same rows through the new table as through the old."""
    w = W.prefill_8b(num_pages=40, tokens=300, num_reqs=3, move_rows=0, layer_num=2)
    pool, raw = _filled_pool(w.shapes, w.page_size)
    P = w.shapes[0].num_pages
    pages = w.req_pages[0]
    lens = w.req_lens[0]
    used = np.unique(np.concatenate(pages))
    # virtual page v of the batch = its index in `used`; the table maps it to its physical page
    v2p = used.astype(np.int32).copy()
    vpages = [np.searchsorted(used, p).astype(np.int32) for p in pages]
    table = W.padded_table(vpages)
    cu = W.out_offsets(lens)

    def read_all():
        bt, _ = pool.translate_pages(0, table, v2p)
        out = []
        for layer in range(2):
            ko = np.zeros((int(cu[-1]), pool.row_bytes(0)), np.uint8)
            vo = np.zeros_like(ko)
            assert pool.gather(0, layer, bt, lens, cu, 0, ko, vo) == frozenset()
            out += [ko, vo]
        return out

    before = read_all()
    plan = W.compaction_plan(used, P)
    assert len(plan[0]) > 0
    assert pool.move_pages(0, plan[1], plan[0]) == frozenset()
    virt = np.searchsorted(used, plan[0]).astype(np.int32)
    assert pool.remap_pages(0, v2p, virt, plan[1]) == frozenset()
    assert v2p.max() < len(used) + 1  # every live page now sits below the watermark
    after = read_all()
    assert all(np.array_equal(a, b) for a, b in zip(before, after))


def test_window_eviction_brute_force_and_window_reads_unchanged():
    w = W.swa_decode(num_reqs=5, len_lo=20, len_hi=700, layer_num=4, window=70)
    ps = w.page_size
    mapping = w.swa_mapping.copy()
    pool, raw = _filled_pool(w.shapes, ps)
    table = W.padded_table(w.req_pages[0], pad=-1)
    lens = w.req_lens[0]
    win = w.window
    bt_before, _ = pool.translate_pages(1, W.padded_table(w.req_pages[0]), mapping)
    cu = W.out_offsets(lens, win)
    rb = pool.row_bytes(1)

    def read(bt):
        ko = np.zeros((int(cu[-1]), rb), np.uint8)
        vo = np.zeros_like(ko)
        assert pool.gather(1, 1, bt, lens, cu, win, ko, vo) == frozenset()
        return ko, vo

    before = read(bt_before)
    exp = mapping.copy()
    for r, pages in enumerate(w.req_pages[0]):
        for i, page in enumerate(pages):
            positions = range(i * ps, (i + 1) * ps)
            if all(p < lens[r] - win for p in positions):
                exp[page] = -1
    assert (exp != mapping).sum() > 0
    assert pool.evict_window(mapping, table, lens, win) == frozenset()
    assert np.array_equal(mapping, exp)
    after = read(pool.translate_pages(1, W.padded_table(w.req_pages[0]), mapping)[0])
    assert np.array_equal(before[0], after[0]) and np.array_equal(before[1], after[1])
    # a slot on an evicted page now translates to the sink
    evicted = np.nonzero((exp == -1) & (w.swa_mapping >= 0))[0]
    ids, _ = pool.translate(1, [int(evicted[0]) * ps + 3], mapping)
    assert ids.tolist() == [0]
    assert pool.evict_window(mapping, np.array([[len(mapping)]], np.int32), np.array([1000], np.int32), 10) == {"slot_range"}


# ---------------------------------------------------------------------------
# read path: prefix-only page table and decode attention over the dense views
# ---------------------------------------------------------------------------

from oracle import attention as A  # noqa: E402


def _gauss_pool(shapes, ps, seed=11):
    """A pool whose every byte pair is a finite bf16 value (attention reads whole rows)."""
    specs = [Spec(s.kind, s.layer_num, s.head_num, s.head_dim, s.v_head_dim, s.elem_bytes, s.num_pages) for s in shapes]
    req = oracle.plan(specs, ps).required_bytes
    raw = W.irwin_hall_bf16_host(seed, 0, (req + 7) // 8 * 8).view(np.uint8).copy()
    return oracle.OraclePool(specs, ps, raw), raw


def _requests(seed, P, ps, lens):
    """Per-request physical page lists drawn from pages 1..P-1, pages not shared."""
    perm = W.page_permutation(seed, P)
    perm = perm[perm != 0]
    out, at = [], 0
    for n in lens:
        k = (int(n) + ps - 1) // ps
        out.append(perm[at: at + k])
        at += k
    assert at <= perm.size
    return out


def _sdpa_reference(ref, layer, pages, lens, window, q_bits, hkv, d, scale):
    """torch's scaled_dot_product_attention in float64, rows fetched by the strided builder."""
    import torch

    out = np.zeros((len(lens), q_bits.shape[1], d))
    group = q_bits.shape[1] // hkv
    for r, (pg, n) in enumerate(zip(pages, lens)):
        if n <= 0:
            continue
        k, v = ref.gather_pages(layer, [pg], [n], window)
        kt = torch.from_numpy(A.bf16_bits_to_f64(k.view(np.uint16)).reshape(-1, hkv, d)).transpose(0, 1)
        vt = torch.from_numpy(A.bf16_bits_to_f64(v.view(np.uint16)).reshape(-1, hkv, d)).transpose(0, 1)
        kt = kt.repeat_interleave(group, dim=0).unsqueeze(0)  # [1, Hq, n, d]: q head g reads KV head g // G
        vt = vt.repeat_interleave(group, dim=0).unsqueeze(0)
        q = torch.from_numpy(A.bf16_bits_to_f64(q_bits[r])).unsqueeze(0).unsqueeze(2)  # [1, Hq, 1, d]
        o = torch.nn.functional.scaled_dot_product_attention(q, kt.contiguous(), vt.contiguous(), scale=scale)
        out[r] = o[0, :, 0, :].numpy()
    return out


@pytest.mark.parametrize("hkv,group,d,window", [(2, 2, 16, 0), (2, 2, 16, 6), (1, 4, 8, 0), (3, 1, 8, 9)])
def test_decode_attention_matches_torch_sdpa(hkv, group, d, window):
    ps, P, L = 4, 24, 2
    lens = np.array([1, 5, 13, 4, 22, 0], dtype=np.int32)
    pool, raw = _gauss_pool([W.mha(L, hkv, d, P)], ps)
    pages = _requests(3, P, ps, lens)
    bt, flags = pool.translate_pages(0, W.padded_table(pages))
    assert flags == frozenset()
    q = W.irwin_hall_bf16_host(5, 0, 2 * lens.size * hkv * group * d).reshape(lens.size, hkv * group, d)
    scale = A.default_scale(d)
    ref = _strided(pool, 0)
    for layer in range(L):
        out, fl = A.decode_attention(pool, 0, layer, q, bt, lens, window, scale)
        assert fl == frozenset()
        exp = _sdpa_reference(ref, layer, pages, lens, window, q, hkv, d, scale)
        assert np.abs(out - exp).max() < 1e-12
        assert not np.allclose(out[1:5], 0)


def test_decode_attention_closed_forms():
    ps, P, hkv, group, d = 4, 12, 2, 2, 8
    lens = np.array([7, 1], dtype=np.int32)
    pool, raw = _gauss_pool([W.mha(1, hkv, d, P)], ps)
    ref = _strided(pool, 0)
    pages = _requests(8, P, ps, lens)
    bt, _ = pool.translate_pages(0, W.padded_table(pages))
    q = W.irwin_hall_bf16_host(9, 0, 2 * 2 * hkv * group * d).reshape(2, hkv * group, d)
    # request 0: every K row the same -> uniform weights -> the mean of its V rows
    k0 = ref.row(0, 0, int(pages[0][0]), 0).copy()
    for j in range(7):
        ref.env[int(pages[0][j // ps]), 0, 0, j % ps] = k0
    out, fl = A.decode_attention(pool, 0, 0, q, bt, lens, 0, 0.3)
    assert fl == frozenset()
    _, v = ref.gather_pages(0, [pages[0]], [7], 0)
    vmean = A.bf16_bits_to_f64(v.view(np.uint16)).reshape(7, hkv, d).mean(axis=0)
    for g in range(hkv * group):
        assert np.allclose(out[0, g], vmean[g // group], rtol=0, atol=1e-14)
    # request 1: a single position -> exactly its V row, whatever q and the scale
    _, v1 = ref.gather_pages(0, [pages[1]], [1], 0)
    v1 = A.bf16_bits_to_f64(v1.view(np.uint16)).reshape(hkv, d)
    for g in range(hkv * group):
        assert np.array_equal(out[1, g], v1[g // group])
    # scale 0 -> uniform weights for any keys
    out0, _ = A.decode_attention(pool, 0, 0, q, bt, lens, 3, 0.0)
    _, v3 = ref.gather_pages(0, [pages[0]], [7], 3)
    v3 = A.bf16_bits_to_f64(v3.view(np.uint16)).reshape(3, hkv, d).mean(axis=0)
    assert np.allclose(out0[0, 1], v3[0], rtol=0, atol=1e-14)


def test_decode_attention_conditions_zero_the_request():
    ps, P, hkv, d = 4, 12, 2, 8
    lens = np.array([6, 6, 6, 0, 9], dtype=np.int32)
    pool, raw = _gauss_pool([W.mha(1, hkv, d, P)], ps)
    pages = _requests(4, P, ps, lens)
    bt, _ = pool.translate_pages(0, W.padded_table(pages))
    q = W.irwin_hall_bf16_host(2, 0, 2 * lens.size * hkv * d).reshape(lens.size, hkv, d)
    good, fl = A.decode_attention(pool, 0, 0, q, bt, lens, 0, 0.5)
    assert fl == frozenset() and np.allclose(good[3], 0) and not np.allclose(good[0], 0)
    bpp = pool.plan.subs[0].blocks_per_page
    for bad in (-1, 1, P * bpp, bt[1, 0] + 1):
        b = bt.copy()
        b[1, 1] = bad
        out, fl = A.decode_attention(pool, 0, 0, q, b, lens, 0, 0.5)
        assert fl == {"bad_block"}
        assert np.allclose(out[1], 0) and np.array_equal(np.delete(out, 1, 0), np.delete(good, 1, 0))
    # a bad entry outside the window is never read
    b = bt.copy()
    b[4, 0] = -1
    out, fl = A.decode_attention(pool, 0, 0, q, b, lens, 4, 0.5)
    assert fl == frozenset()
    # a table too narrow for the length, and a length past the caller's bound
    out, fl = A.decode_attention(pool, 0, 0, q, bt[:, :2], lens, 0, 0.5)
    assert fl == {"bad_block"} and np.allclose(out[4], 0) and np.array_equal(out[:4], good[:4])
    out, fl = A.decode_attention(pool, 0, 0, q, bt, lens, 0, 0.5, max_seq_len=8)
    assert fl == {"layout"} and np.allclose(out[4], 0) and np.array_equal(out[:4], good[:4])


def test_build_page_table_is_prefix_only():
    ps, P = 4, 16
    pool, raw = _filled_pool([W.mha(2, 2, 8, P)], ps)
    lens = np.array([5, 1, 12, 0], dtype=np.int32)
    pages = _requests(6, P, ps, lens)
    width = 5
    req = np.full((lens.size, width), 10 ** 6, dtype=np.int32)  # entries past the prefix hold garbage
    for r, pg in enumerate(pages):
        req[r, :pg.size] = pg
    out, fl = pool.build_page_table(0, req, lens)
    assert fl == frozenset()
    full, _ = pool.translate_pages(0, W.padded_table(pages))
    for r, pg in enumerate(pages):
        assert np.array_equal(out[r, :pg.size], full[r, :pg.size])
        assert (out[r, pg.size:] == 0).all()
    # the built table reads back, through the block-table gather, what the strided builder holds
    ref = _strided(pool, 0)
    cu = W.out_offsets(lens, 0)
    ko = np.zeros((int(cu[-1]), 32), np.uint8)
    vo = np.zeros_like(ko)
    assert pool.gather(0, 1, out, lens, cu, 0, ko, vo) == frozenset()
    rk, rv = ref.gather_pages(1, pages, lens, 0)
    assert np.array_equal(ko, rk) and np.array_equal(vo, rv)
    # through a virtual-to-physical table: entry i is the kernel-facing index of v2p[page]
    v2p = W.page_permutation(12, P).astype(np.int32)
    out2, fl = pool.build_page_table(0, req, lens, v2p)
    assert fl == frozenset()
    bpp = pool.plan.subs[0].blocks_per_page
    for r, pg in enumerate(pages):
        walk_rows, _ = walk(P, 2, MHA, ps, 32)
        for i, page in enumerate(pg):
            phys = int(v2p[page])
            assert pool.view_base(0, 0, 0) + out2[r, i] * ps * 32 == walk_rows[(phys, 0, 0, 0)]
            assert out2[r, i] % bpp == 0
    # a prefix wider than the table, and an out-of-range page inside the prefix
    _, fl = pool.build_page_table(0, req[:, :2], lens)
    assert fl == {"layout"}
    bad = req.copy()
    bad[2, 1] = P
    out3, fl = pool.build_page_table(0, bad, lens)
    assert fl == {"slot_range"} and out3[2, 1] == 0


@pytest.mark.parametrize("n,hkv,group,d", [(1, 1, 1, 64), (37, 2, 4, 128), (700, 1, 8, 128), (2500, 2, 2, 64)])
def test_fp32_error_bound_covers_a_float32_evaluation(n, hkv, group, d):
    """The derived tolerance is not tighter than the arithmetic: a plain float32
    evaluation of the same attention stays inside it (sums of up to n terms)."""
    g = np.random.default_rng(n + d)
    bits = lambda m: W.irwin_hall_bf16_host(int(g.integers(1 << 30)), 0, 2 * m)
    q = A.bf16_bits_to_f64(bits(hkv * group * d)).reshape(hkv * group, d)
    k = A.bf16_bits_to_f64(bits(n * hkv * d)).reshape(n, hkv, d)
    v = A.bf16_bits_to_f64(bits(n * hkv * d)).reshape(n, hkv, d)
    scale = A.default_scale(d)
    exact = A.attend(q, k, v, scale)
    bound = A.fp32_error_bound(q, k, v, scale, n + 2)
    out32 = np.zeros_like(exact)
    for gh in range(hkv * group):
        h = gh // group
        s = (k[:, h, :].astype(np.float32) @ q[gh].astype(np.float32)) * np.float32(scale)
        e = np.exp(s - s.max())
        out32[gh] = (e @ v[:, h, :].astype(np.float32)) / e.sum(dtype=np.float32)
    err = np.abs(out32 - exact).max(axis=1)
    assert (err <= bound).all(), (err, bound)
    assert (bound < 5e-3).all()


# ---------------------------------------------------------------------------
# decode attention over an MLA sub-pool's latent view
# ---------------------------------------------------------------------------

def _sdpa_reference_mla(ref, layer, pages, lens, window, q_bits, lat, v_dim, scale):
    """torch's SDPA in float64: one latent 'head' for every query head, values its front."""
    import torch

    hq = q_bits.shape[1]
    out = np.zeros((len(lens), hq, v_dim))
    for r, (pg, n) in enumerate(zip(pages, lens)):
        if n <= 0:
            continue
        c, none = ref.gather_pages(layer, [pg], [n], window)
        assert none is None
        c = torch.from_numpy(A.bf16_bits_to_f64(c.view(np.uint16)).reshape(-1, lat))
        k = c.unsqueeze(0).expand(hq, -1, -1).unsqueeze(0).contiguous()  # [1, Hq, n, lat]
        v = c[:, :v_dim].unsqueeze(0).expand(hq, -1, -1).unsqueeze(0).contiguous()
        q = torch.from_numpy(A.bf16_bits_to_f64(q_bits[r])).unsqueeze(0).unsqueeze(2)  # [1, Hq, 1, lat]
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)
        out[r] = o[0, :, 0, :].numpy()
    return out


@pytest.mark.parametrize("lat,v_dim,hq,window", [(24, 16, 4, 0), (24, 16, 4, 5), (576, 512, 16, 0), (40, 40, 2, 7)])
def test_mla_decode_attention_matches_torch_sdpa(lat, v_dim, hq, window):
    ps, P, L = 4, 20, 3
    lens = np.array([1, 6, 15, 0, 19], dtype=np.int32)
    pool, raw = _gauss_pool([W.mla(L, P, latent_dim=lat)], ps)
    pages = _requests(21, P, ps, lens)
    bt, flags = pool.translate_pages(0, W.padded_table(pages))
    assert flags == frozenset()
    q = W.irwin_hall_bf16_host(23, 0, 2 * lens.size * hq * lat).reshape(lens.size, hq, lat)
    scale = A.default_scale(lat)
    ref = _strided(pool, 0)
    for layer in (0, L - 1):
        out, fl = A.decode_attention(pool, 0, layer, q, bt, lens, window, scale, v_dim=v_dim)
        assert fl == frozenset() and out.shape == (lens.size, hq, v_dim)
        exp = _sdpa_reference_mla(ref, layer, pages, lens, window, q, lat, v_dim, scale)
        assert np.abs(out - exp).max() < 1e-12
        assert not np.allclose(out[1], 0) and np.allclose(out[3], 0)


def test_mla_decode_attention_closed_forms_and_conditions():
    ps, P, lat, v_dim, hq = 4, 12, 24, 16, 4
    lens = np.array([7, 1, 9], dtype=np.int32)
    pool, raw = _gauss_pool([W.mla(2, P, latent_dim=lat)], ps)
    ref = _strided(pool, 0)
    pages = _requests(5, P, ps, lens)
    bt, _ = pool.translate_pages(0, W.padded_table(pages))
    q = W.irwin_hall_bf16_host(6, 0, 2 * lens.size * hq * lat).reshape(lens.size, hq, lat)
    # request 0: latent rows that differ only in their value front, and a query that is
    # zero there: every score is the same, so the weights are uniform and the output is
    # the mean of the value fronts (the scores read the part past the values too)
    k0 = ref.row(1, 0, int(pages[0][0]), 0).copy()
    for j in range(7):
        row = ref.env[int(pages[0][j // ps]), 1, 0, j % ps]
        row[2 * v_dim:] = k0[2 * v_dim:]
    q0 = q.copy()
    q0[0, :, :v_dim] = 0
    out, fl = A.decode_attention(pool, 0, 1, q0, bt, lens, 0, 0.7, v_dim=v_dim)
    assert fl == frozenset()
    c, _ = ref.gather_pages(1, [pages[0]], [7], 0)
    cmean = A.bf16_bits_to_f64(c.view(np.uint16)).reshape(7, lat)[:, :v_dim].mean(axis=0)
    for g in range(hq):
        assert np.allclose(out[0, g], cmean, rtol=0, atol=1e-14)
    assert not np.allclose(out[2], cmean)  # other requests keep their own weights
    # a single position: exactly its value front, whatever q and the scale
    out, _ = A.decode_attention(pool, 0, 1, q, bt, lens, 0, 3.0, v_dim=v_dim)
    c1, _ = ref.gather_pages(1, [pages[1]], [1], 0)
    c1 = A.bf16_bits_to_f64(c1.view(np.uint16)).reshape(lat)[:v_dim]
    for g in range(hq):
        assert np.array_equal(out[1, g], c1)
    # scale 0 over a window: the mean of the window's value fronts
    out0, _ = A.decode_attention(pool, 0, 0, q, bt, lens, 3, 0.0, v_dim=v_dim)
    c3, _ = ref.gather_pages(0, [pages[2]], [9], 3)
    c3 = A.bf16_bits_to_f64(c3.view(np.uint16)).reshape(3, lat)[:, :v_dim].mean(axis=0)
    assert np.allclose(out0[2, 2], c3, rtol=0, atol=1e-14)
    # the same conditions as the MHA read: bad entries, narrow tables, lengths past the bound
    good, _ = A.decode_attention(pool, 0, 0, q, bt, lens, 0, 0.5, v_dim=v_dim)
    b = bt.copy()
    b[2, 1] = bt[2, 1] + 1  # not a multiple of blocks_per_page
    out, fl = A.decode_attention(pool, 0, 0, q, b, lens, 0, 0.5, v_dim=v_dim)
    assert fl == {"bad_block"} and np.allclose(out[2], 0) and np.array_equal(out[:2], good[:2])
    out, fl = A.decode_attention(pool, 0, 0, q, bt, lens, 0, 0.5, max_seq_len=8, v_dim=v_dim)
    assert fl == {"layout"} and np.allclose(out[2], 0) and np.array_equal(out[:2], good[:2])
    with pytest.raises(AssertionError):
        A.decode_attention(pool, 0, 0, q, bt, lens, 0, 0.5)  # an MLA read needs its value width


@pytest.mark.parametrize("n,hq,sparse", [(1, 16, False), (45, 16, False), (900, 32, False), (3000, 16, False),
                                         (45, 16, True), (3000, 16, True)])
def test_split_weight_bound_covers_a_matrix_core_style_evaluation(n, hq, sparse):
    """An fp32 evaluation that splits each weight into bf16 high and low parts
    (scores from exact bf16 products, fp32 sums) stays inside the bound with
    weight_rel = 2^-16 and the chain length any split of n positions can form
    (from n alone), on 576-wide latents with 512-wide values.  With a
    query that is zero but for a few dims (some in the value part, some past
    it) the score term of the bound all but vanishes, and the bound is tight
    enough to reject the same evaluation with the low parts dropped (on
    short requests: over thousands of positions the sums' own term leads)."""
    g = np.random.default_rng(n + hq + 7 * sparse)
    bits = lambda m: W.irwin_hall_bf16_host(int(g.integers(1 << 30)), 0, 2 * m)
    lat, v_dim = 576, 512
    q = A.bf16_bits_to_f64(bits(hq * lat)).reshape(hq, lat)
    if sparse:
        keep = np.zeros(lat, bool)
        keep[[3, 200, 511, 512, 575]] = True
        q[:, ~keep] = 0.0
    c = A.bf16_bits_to_f64(bits(n * lat)).reshape(n, 1, lat)
    scale = A.default_scale(192)
    exact = A.attend(q, c, c[:, :, :v_dim], scale)
    bound = A.fp32_error_bound(q, c, c[:, :, :v_dim], scale, A.chain_terms_any_split(n, 2), A.BF16_SPLIT_REL)
    import torch

    def bf16(x):
        return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float32).numpy()

    out = np.zeros_like(exact)
    hi_only = np.zeros_like(exact)
    for h in range(hq):
        s = (c[:, 0, :].astype(np.float32) @ q[h].astype(np.float32)) * np.float32(scale)
        p = np.exp2((s - s.max()) * np.float32(1.4426950408889634)).astype(np.float32)
        hi = bf16(p)
        lo = bf16(p - hi)
        num = hi @ c[:, 0, :v_dim].astype(np.float32) + lo @ c[:, 0, :v_dim].astype(np.float32)
        out[h] = num / p.sum(dtype=np.float32)
        hi_only[h] = (hi @ c[:, 0, :v_dim].astype(np.float32)) / p.sum(dtype=np.float32)
        assert (np.abs(hi + lo - p) <= A.BF16_SPLIT_REL * p).all()
    err = np.abs(out - exact).max(axis=1)
    assert (err <= bound).all(), (err, bound)
    assert (bound < (6e-3 if sparse else 0.05)).all()
    if sparse and n <= 100:  # a dropped low part (bf16 weights) is caught on short requests, where
        # the sums' term 2 gamma(n) max|v| stays small
        assert (np.abs(hi_only - exact).max(axis=1) > bound).any()


def _int_pool(shapes, ps, seed=13):
    """A pool whose every byte pair is a small integer in bf16 (exact float32 sums)."""
    specs = [Spec(s.kind, s.layer_num, s.head_num, s.head_dim, s.v_head_dim, s.elem_bytes, s.num_pages) for s in shapes]
    req = oracle.plan(specs, ps).required_bytes
    raw = W.small_int_bf16_host(seed, 0, (req + 7) // 8 * 8).view(np.uint8).copy()
    return oracle.OraclePool(specs, ps, raw)


def _float32_pieces(vals, cuts, reciprocal):
    """A float32 evaluation of the mean of ``vals`` [n, dv] with every weight 1: the
    positions cut into pieces at ``cuts``, each piece summed on its own, the pieces'
    sums merged, then one division (or a reciprocal and a product)."""
    edges = np.concatenate([[0], np.sort(cuts), [vals.shape[0]]]).astype(np.int64)
    num = np.zeros(vals.shape[1], np.float32)
    den = np.float32(0)
    for a, b in zip(edges[:-1], edges[1:]):
        num = num + vals[a:b].astype(np.float32).sum(axis=0, dtype=np.float32)
        den = den + np.float32(b - a)
    if reciprocal:
        return (num * (np.float32(1) / den)).astype(np.float64)
    return (num / den).astype(np.float64)


@pytest.mark.parametrize("mla", [True, False])
def test_exact_mean_tolerance_rejects_dropped_or_doubled_positions(mla):
    """With a zero query every weight is 1, and with small-integer values every float32
    partial sum is exact, so a split evaluation returns the mean up to its final
    division.  The tolerance the GPU tests use for that case accepts a float32
    evaluation cut into arbitrary pieces (both division forms), and rejects the mean
    taken with one 16-position tile dropped, one 256-position span dropped, one
    256-position span counted twice, or one position dropped, on a 60,000-position MLA
    request (576-wide latents, 512-wide values, 16 query heads) and an 8,192-position
    MHA request (8 KV heads x 128, 4 query heads per KV head)."""
    if mla:
        n, ps, hq = 60000, 64, 16
        shape = W.mla(1, (n + ps - 1) // ps + 3)
    else:
        n, ps, hq = 8192, 16, 32
        shape = W.mha(1, 8, 128, n // ps + 3)
    pool = _int_pool([shape], ps)
    pages = _requests(6, shape.num_pages, ps, [n])
    bt, fl = pool.translate_pages(0, W.padded_table(pages))
    assert fl == frozenset()
    lat = shape.head_dim if mla else 128
    q = np.zeros((1, hq, lat), np.uint16)
    kw = {"v_dim": 512} if mla else {}
    exp, fl = A.decode_attention(pool, 0, 0, q, bt, [n], 0, 1.0, uniform=True, **kw)
    assert fl == frozenset()
    # the closed form agrees with the softmax formula on the same rows
    ref, _ = A.decode_attention(pool, 0, 0, q, bt, [n], 0, 1.0, **kw)
    assert np.abs(ref - exp).max() < 1e-9
    tol = A.exact_mean_tolerance(exp[0])
    # the attended value rows, fetched by the independent strided builder
    if mla:
        c, _ = _strided(pool, 0).gather_pages(0, [pages[0]], [n], 0)
        vals = A.bf16_bits_to_f64(c.view(np.uint16)).reshape(n, lat)[:, :512]
        heads = [vals] * hq
    else:
        _, v = _strided(pool, 0).gather_pages(0, [pages[0]], [n], 0)
        v = A.bf16_bits_to_f64(v.view(np.uint16)).reshape(n, 8, 128)
        heads = [v[:, g // 4] for g in range(hq)]
    assert all(float(np.abs(h).max()) <= 8 for h in heads)
    g = np.random.default_rng(n)
    for recip in (False, True):
        cuts = g.choice(np.arange(1, n), size=37, replace=False)
        got = np.stack([_float32_pieces(h, cuts, recip) for h in heads])
        assert (np.abs(got - exp[0]) <= tol).all()
    mutants = {
        "tile dropped": np.delete(np.arange(n), np.arange(4096, 4112)),
        "span dropped": np.delete(np.arange(n), np.arange(n // 2, n // 2 + 256)),
        "span doubled": np.concatenate([np.arange(n), np.arange(1024, 1280)]),
        "position dropped": np.arange(1, n),
    }
    for what, keep in mutants.items():
        bad = np.stack([h[keep].sum(axis=0) / keep.size for h in heads])
        assert (np.abs(bad - exp[0]) > tol).any(), what
        # the fp32 bound derived from the length alone cannot see a dropped tile this long
        # (why the tests add the exact case)
    bound = A.fp32_error_bound(np.zeros((hq, lat)), np.zeros((n, 1, lat)), heads[0][:, None, :], 1.0,
                               A.chain_terms_any_split(n, 2 if mla else 1))
    assert (bound > 1e-3).all()
