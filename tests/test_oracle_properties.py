"""Randomised pins for the CPU oracle (hypothesis, seeded and bounded).

Source page: "PR #34602: feat(unified-memory): dense KV views for uniform-row
MHA/SWA models" (sglang report).  Every expectation here comes from outside
the oracle's arithmetic:

* the page envelope walked in memory order, ``[L0_K*ps | L0_V*ps | ...]``
  (implementation step 1), for where a (page, layer, kv, offset) row lives;
* round trips: rows stored at a request's slots come back from a gather
  through its block table; a move leaves every byte but its destinations
  alone;
* plan sums: sub-pools sit back to back, and one tail pad follows the last.

The shapes go beyond the fixed lists of test_oracle_pins.py: page sizes that
are not powers of two, 4-byte elements, up to three sub-pools.
"""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from oracle import MHA, MLA, Spec
import ukv_workloads as W

SETTINGS = settings(max_examples=40, deadline=None, derandomize=True, database=None,
                    suppress_health_check=[HealthCheck.too_slow])


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


@st.composite
def specs(draw):
    kind = draw(st.sampled_from([MHA, MLA]))
    L = draw(st.integers(1, 4))
    H = 1 if kind == MLA else draw(st.integers(1, 3))
    D = draw(st.sampled_from([2, 4, 6, 8]))
    es = draw(st.sampled_from([1, 2, 4]))
    P = draw(st.integers(1, 6))
    return Spec(kind, L, H, D, D if kind == MHA else 0, es, P)


def row_bytes_of(spec):
    return spec.head_num * spec.head_dim * spec.elem_bytes


def filled(spec_list, ps, seed=3):
    req = oracle.plan(spec_list, ps).required_bytes
    raw = W.fill_pattern_host(seed, 0, (req + 7) // 8 * 8).copy()
    return oracle.OraclePool(spec_list, ps, raw), raw


@SETTINGS
@given(st.lists(specs(), min_size=1, max_size=3), st.integers(1, 9))
def test_plan_places_subpools_back_to_back_with_one_tail_pad(spec_list, ps):
    """Anchors follow each other in spec order, each envelope is num_pages page envelopes
    of the walk's length, and the pool ends one largest page envelope after the last."""
    p = oracle.plan(spec_list, ps)
    if p.code != "ok":  # only the alignment gate can refuse these small shapes
        assert p.code == "alignment"
        return
    anchor = 0
    envelopes = []
    for spec, sp in zip(spec_list, p.subs):
        _, end = walk(spec.num_pages, spec.layer_num, spec.kind, ps, row_bytes_of(spec), anchor)
        assert sp.anchor_bytes == anchor and sp.envelope_bytes == end - anchor
        envelopes.append((end - anchor) // spec.num_pages)
        anchor = end
    assert p.required_bytes == anchor + max(envelopes)


@SETTINGS
@given(specs(), st.integers(1, 9))
def test_every_kernel_id_lands_where_the_walk_puts_its_row(spec, ps):
    """view_base(layer, kv) + id * row_bytes, for the id translate gives slot p*ps + o,
    is the walk's address of row (p, layer, kv, o), for every row of the pool."""
    pool, _ = filled([spec], ps)
    if pool.plan.code != "ok":
        return
    rb = row_bytes_of(spec)
    addrs, _ = walk(spec.num_pages, spec.layer_num, spec.kind, ps, rb)
    slots = np.arange(spec.num_pages * ps, dtype=np.int64)
    ids, flags = pool.translate(0, slots)
    assert flags == frozenset()
    kvs = (0, 1) if spec.kind == MHA else (0,)
    for layer in range(spec.layer_num):
        for kv in kvs:
            base = pool.view_base(0, layer, kv)
            got = base + ids.astype(np.int64) * rb
            exp = [addrs[(int(t) // ps, layer, kv, int(t) % ps)] for t in slots]
            assert got.tolist() == exp


@SETTINGS
@given(specs(), st.integers(1, 6), st.data())
def test_translate_through_a_random_page_table(spec, ps, data):
    """Through a virtual-to-physical table with unmapped (-1) and out-of-pool entries:
    a mapped slot reaches the walk's row of its physical page; a tombstone, an unmapped
    page or a page past the table or the pool gives the sink row 0, and only the last
    two raise the range flag."""
    pool, _ = filled([spec], ps)
    if pool.plan.code != "ok":
        return
    P = spec.num_pages
    rb = row_bytes_of(spec)
    addrs, _ = walk(P, spec.layer_num, spec.kind, ps, rb)
    nv = data.draw(st.integers(2, 8))
    v2p = np.array(data.draw(st.lists(st.integers(-1, P + 2), min_size=nv, max_size=nv)), dtype=np.int32)
    # at least one unmapped and one mapped page, each with a slot on it
    u, m = data.draw(st.lists(st.integers(0, nv - 1), min_size=2, max_size=2, unique=True))
    v2p[u], v2p[m] = -1, data.draw(st.integers(0, P - 1))
    slots = data.draw(st.lists(st.integers(-3, (nv + 1) * ps), min_size=1, max_size=40))
    slots += [u * ps + data.draw(st.integers(0, ps - 1)), m * ps + data.draw(st.integers(0, ps - 1))]
    slots = np.array(data.draw(st.permutations(slots)), dtype=np.int64)
    ids, flags = pool.translate(0, slots, v2p)
    base = pool.view_base(0, 0, 0)
    out_of_range = False
    for t, kid in zip(slots.tolist(), ids.tolist()):
        page, off = divmod(t, ps) if t >= 0 else (None, None)
        if t < 0:
            assert kid == 0
        elif page >= nv or v2p[page] >= P:
            assert kid == 0
            out_of_range = True
        elif v2p[page] < 0:
            assert kid == 0
        else:
            assert base + kid * rb == addrs[(int(v2p[page]), 0, 0, off)]
    assert flags == (frozenset({"slot_range"}) if out_of_range else frozenset())
    # tombstones and unmapped pages alone raise nothing
    inside = [t for t in slots.tolist() if t < 0 or (t // ps < nv and v2p[t // ps] < P)]
    if inside:
        assert pool.translate(0, np.array(inside, dtype=np.int64), v2p)[1] == frozenset()


@SETTINGS
@given(specs(), st.integers(1, 5), st.data())
def test_rows_stored_at_a_requests_slots_come_back_from_its_gather(spec, ps, data):
    """Requests own disjoint random pages; every position's row is stored at its slot's
    kernel id, then gathered (all positions, or the last `window`) through the requests'
    block table: the rows come back in request order, and the gather flags nothing."""
    pool, raw = filled([spec], ps)
    if pool.plan.code != "ok":
        return
    P = spec.num_pages
    rb = row_bytes_of(spec)
    perm = np.array(data.draw(st.permutations(range(P))), dtype=np.int32)
    nreq = data.draw(st.integers(1, min(3, P)))
    cuts = sorted(data.draw(st.lists(st.integers(1, P - 1), min_size=nreq - 1, max_size=nreq - 1, unique=True))) \
        if nreq > 1 else []
    pages = np.split(perm, cuts)
    lens = np.array([data.draw(st.integers(1, len(pg) * ps)) for pg in pages], dtype=np.int32)
    window = data.draw(st.sampled_from([0, 1, 3, 100]))
    layer = data.draw(st.integers(0, spec.layer_num - 1))
    slots = np.concatenate([pg[np.arange(n) // ps].astype(np.int64) * ps + np.arange(n) % ps
                            for pg, n in zip(pages, lens)])
    g = np.random.default_rng(int(slots.sum()) + 7)
    k = g.integers(0, 256, (slots.size, rb), dtype=np.uint8)
    v = g.integers(0, 256, (slots.size, rb), dtype=np.uint8) if spec.kind == MHA else None
    ids, flags = pool.translate(0, slots)
    assert flags == frozenset()
    assert pool.store(0, layer, ids, k, v) == frozenset()
    bt, flags = pool.translate_pages(0, W.padded_table(pages))
    assert flags == frozenset()
    cu = W.out_offsets(lens, window)
    ko = np.zeros((int(cu[-1]), rb), np.uint8)
    vo = np.zeros_like(ko) if v is not None else None
    assert pool.gather(0, layer, bt, lens, cu, window, ko, vo) == frozenset()
    starts = np.concatenate([[0], np.cumsum(lens)])
    keep = np.concatenate([np.arange(starts[r] + (lens[r] - window if 0 < window < lens[r] else 0), starts[r + 1])
                           for r in range(len(lens))])
    assert np.array_equal(ko, k[keep])
    if v is not None:
        assert np.array_equal(vo, v[keep])


@SETTINGS
@given(specs(), st.integers(1, 5), st.data())
def test_move_changes_only_its_destination_rows(spec, ps, data):
    """A move over a layer range copies each source row onto its destination on those
    layers (K and V), read at the walk's addresses before and after; every other byte of
    the buffer, the tail pad included, is unchanged."""
    pool, raw = filled([spec], ps)
    if pool.plan.code != "ok":
        return
    P = spec.num_pages
    rb = row_bytes_of(spec)
    addrs, _ = walk(P, spec.layer_num, spec.kind, ps, rb)
    nslots = P * ps
    n = data.draw(st.integers(1, max(1, nslots // 2)))
    chosen = data.draw(st.permutations(range(nslots)))[: 2 * n]
    if len(chosen) < 2:
        return
    n = len(chosen) // 2
    src = np.array(chosen[:n], dtype=np.int64)
    dst = np.array(chosen[n:2 * n], dtype=np.int64)
    l0 = data.draw(st.integers(0, spec.layer_num - 1))
    l1 = data.draw(st.integers(l0 + 1, spec.layer_num))
    before = raw.copy()
    sid, _ = pool.translate(0, src)
    did, _ = pool.translate(0, dst)
    assert pool.move(0, did, sid, l0, l1) == frozenset()
    expect = before.copy()
    kvs = (0, 1) if spec.kind == MHA else (0,)
    for layer in range(l0, l1):
        for kv in kvs:
            for s, d in zip(src.tolist(), dst.tolist()):
                a_s = addrs[(s // ps, layer, kv, s % ps)]
                a_d = addrs[(d // ps, layer, kv, d % ps)]
                expect[a_d:a_d + rb] = before[a_s:a_s + rb]
    assert np.array_equal(raw, expect)
