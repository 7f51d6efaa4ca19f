"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

The oracle cannot hold a 32-160 GiB envelope on the host, so it answers with
addresses: for every row a store / gather / move touches, the byte offsets it
reads and writes (oracle/ukv_oracle.c *_map, an addresses-only pool).  On the
device the test then checks
  * every written row against its source (a torch index of the input, never
    of the HIP path's output),
  * every gathered row against the envelope row at the oracle's address,
  * every byte nothing may write against the pre-fill pattern, regenerated
    from its definition (SplitMix64 over 8-byte words) chunk by chunk,
  * the sink rows with the tombstone rule (each chunk of the store's vector
    width, 16 bytes here, whole from one of the tombstoned entries of that call).
Every output row of every layer is compared; nothing is sampled.
"""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import oracle
import store_gather_amd as U
import ukv_workloads as W
from parity_util import (assert_bytes_are_pattern, assert_rows_subset, copy_unit, equal_rows_chunked, log,
                         offsets_to_rows, ospecs, pattern_mismatch_rows, round8, rows_view)

pytestmark = pytest.mark.gpu
SEED = 21


@pytest.fixture(autouse=True)
def _name(request):
    log(f"\n[gpu-full] {request.node.name}")
    torch.cuda.synchronize()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _make(w):
    plan = U.ukv_pool_plan(w.shapes, w.page_size)
    n = round8(int(plan.required_bytes))
    pool = U.allocate_pool(w.shapes, w.page_size, extra_bytes=n - int(plan.required_bytes))
    W.fill_pattern_device(pool.raw, SEED)
    orc = oracle.OraclePool(ospecs(w.shapes), w.page_size, addresses_only=True)
    torch.cuda.synchronize()
    log(f"  pool {n / 2**30:.2f} GiB filled")
    return pool, orc


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _translate(pool, orc, sub, slots):
    ids = U.ukv_translate_loc_for_kernel(pool, sub, _dev(slots))
    exp, ef = orc.translate(sub, slots)
    assert np.array_equal(ids.cpu().numpy(), exp) and ef == frozenset()
    return ids, exp


def _block_table(pool, orc, sub, pages):
    table = W.padded_table(pages)
    bt = U.ukv_translate_pages_for_kernel(pool, sub, _dev(table))
    exp, ef = orc.translate_pages(sub, table)
    assert np.array_equal(bt.cpu().numpy(), exp) and ef == frozenset()
    return bt, exp


def _sub_geom(pool, sub):
    q = pool.plan.sub[sub]
    return int(q.anchor_bytes), int(q.envelope_bytes), int(q.row_bytes)


def _store_layers(pool, orc, sub, ids_d, ids, slots, masks, value_seed):
    """Store every layer; check written rows against the sources and the sink rows
    against the tombstone rule; mark written rows in masks[sub]."""
    anchor, env, rb = _sub_geom(pool, sub)
    rows = rows_view(pool.raw, anchor, env, rb)
    shape = pool.specs[sub]
    nkv = 2 if shape.kind == W.MHA else 1
    live = torch.from_numpy(np.nonzero(slots >= 0)[0]).cuda()
    tomb = torch.from_numpy(np.nonzero(slots < 0)[0]).cuda()
    n = ids.size
    for layer in range(shape.layer_num):
        src = [W.normal_bf16_device((n, rb // 2), value_seed + 2 * layer + h, "cuda").view(torch.uint8)
               for h in range(nkv)]
        U.ukv_store_kv(pool, sub, layer, ids_d, src[0], src[1] if nkv == 2 else None)
        maps = orc.store_map(sub, layer, ids)
        assert maps[2] == frozenset()
        for h in range(nkv):
            r = torch.from_numpy(offsets_to_rows(maps[h], anchor, rb)).cuda()
            masks[sub][r] = True
            assert equal_rows_chunked(rows, r[live], src[h], live), f"layer {layer} kv {h}: stored rows"
            if tomb.numel():
                # each chunk of the store's vector width whole from one tombstoned row
                unit = copy_unit(rb, *[orc.view_base(sub, layer, x) for x in range(nkv)],
                                 *[t.data_ptr() for t in src])
                sink = rows[int(r[tomb[0]])].view(-1, unit)
                cand = src[h].index_select(0, tomb).view(tomb.numel(), -1, unit)
                ok = (cand == sink.unsqueeze(0)).all(dim=2).any(dim=0)
                assert bool(ok.all()), f"layer {layer} kv {h}: sink row ({unit}-byte chunks)"
    torch.cuda.synchronize()


def _check_untouched(pool, masks):
    for sub in range(len(pool.specs)):
        anchor, env, rb = _sub_geom(pool, sub)
        changed = pattern_mismatch_rows(pool.raw, SEED, anchor, env, rb)
        assert_rows_subset(changed, masks[sub], f"sub-pool {sub}")
    end = int(pool.plan.envelope_bytes)
    assert_bytes_are_pattern(pool.raw, SEED, end, pool.raw.numel())  # the tail pad


def _gather_layers(pool, orc, sub, bt_d, bt, lens, windows, layers):
    anchor, env, rb = _sub_geom(pool, sub)
    rows = rows_view(pool.raw, anchor, env, rb)
    nkv = 2 if pool.specs[sub].kind == W.MHA else 1
    lens = np.asarray(lens, dtype=np.int32)
    lens_d = _dev(lens)
    for layer in layers:
        win = windows[layer]
        cu = W.out_offsets(lens, win)
        n_out = int(cu[-1])
        outs = [torch.empty((n_out, rb), dtype=torch.uint8, device="cuda") for _ in range(nkv)]
        U.ukv_gather_kv(pool, sub, layer, bt_d, lens_d, _dev(cu), win, outs[0], outs[1] if nkv == 2 else None)
        maps = orc.gather_map(sub, layer, bt, lens, cu, win, n_out)
        assert maps[2] == frozenset()
        for h in range(nkv):
            r = torch.from_numpy(offsets_to_rows(maps[h], anchor, rb)).cuda()
            assert equal_rows_chunked(rows, r, outs[h], None), f"layer {layer} kv {h}: gathered rows"
        del outs


def _masks(pool):
    out = []
    for sub in range(len(pool.specs)):
        _, env, rb = _sub_geom(pool, sub)
        out.append(torch.zeros(env // rb, dtype=torch.bool, device="cuda"))
    return out


def test_full_decode_8b_store_and_gather_all_layers():
    """Llama-3-8B-shape pool (8 GiB), 256 new rows per layer, 256 requests gathered in full, 32 layers."""
    w = W.decode_8b()
    pool, orc = _make(w)
    slots = w.store_slots[0]
    ids_d, ids = _translate(pool, orc, 0, slots)
    masks = _masks(pool)
    _store_layers(pool, orc, 0, ids_d, ids, slots, masks, 500)
    log("  stores checked")
    _check_untouched(pool, masks)
    log("  untouched bytes checked")
    bt_d, bt = _block_table(pool, orc, 0, w.req_pages[0])
    _gather_layers(pool, orc, 0, bt_d, bt, w.req_lens[0], w.windows[0], range(32))
    log("  gathers checked (32 layers x 1,179,779 rows)")
    assert U.ukv_pool_error_flags(pool) == frozenset()


def test_full_prefill_8b_store_gather_move():
    """32 GiB pool; 32,768 tokens (1% tombstones) stored on 32 layers, gathered back,
    then 65,536 rows moved to disjoint rows on every layer."""
    w = W.prefill_8b()
    pool, orc = _make(w)
    slots = w.store_slots[0]
    ids_d, ids = _translate(pool, orc, 0, slots)
    masks = _masks(pool)
    _store_layers(pool, orc, 0, ids_d, ids, slots, masks, 900)
    log("  stores checked")
    _check_untouched(pool, masks)
    log("  untouched bytes checked")
    bt_d, bt = _block_table(pool, orc, 0, w.req_pages[0])
    _gather_layers(pool, orc, 0, bt_d, bt, w.req_lens[0], w.windows[0], range(32))
    log("  gathers checked")
    src_d, src = _translate(pool, orc, 0, w.move_src[0])
    dst_d, dst = _translate(pool, orc, 0, w.move_dst[0])
    before = pool.raw.clone()
    U.ukv_move_kv(pool, 0, dst_d, src_d)
    d_off, s_off, fl = orc.move_map(0, dst, src, 0, 32)
    assert fl == frozenset()
    anchor, env, rb = _sub_geom(pool, 0)
    d_rows = torch.from_numpy(offsets_to_rows(d_off, anchor, rb)).cuda()
    s_rows = torch.from_numpy(offsets_to_rows(s_off, anchor, rb)).cuda()
    rows_after = rows_view(pool.raw, anchor, env, rb)
    rows_before = rows_view(before, anchor, env, rb)
    assert equal_rows_chunked(rows_after, d_rows, rows_before, s_rows), "moved rows"
    allowed = torch.zeros(env // rb, dtype=torch.bool, device="cuda")
    allowed[d_rows] = True
    for c0 in range(0, env // rb, 1 << 19):
        c1 = min(env // rb, c0 + (1 << 19))
        changed = (rows_after[c0:c1] != rows_before[c0:c1]).any(dim=1).nonzero().flatten() + c0
        assert_rows_subset(changed, allowed, "move")
    assert torch.equal(pool.raw[anchor + env:], before[anchor + env:])
    del before
    log("  move checked")
    assert U.ukv_pool_error_flags(pool) == frozenset()


def test_full_hybrid_mha_swa_and_mla():
    """MHA (24 layers, 8x64, page 64, odd layers window 128) and MLA (24 layers, 576 latent)
    sub-pools holding 128 requests of 256..16384 tokens; every token stored on every layer of
    both sub-pools, every layer gathered back."""
    w = W.hybrid()
    pool, orc = _make(w)
    masks = _masks(pool)
    for sub in (0, 1):
        slots = w.store_slots[sub]
        ids_d, ids = _translate(pool, orc, sub, slots)
        _store_layers(pool, orc, sub, ids_d, ids, slots, masks, 1300 + 100 * sub)
        log(f"  sub-pool {sub} stores checked")
    _check_untouched(pool, masks)
    log("  untouched bytes checked")
    for sub in (0, 1):
        bt_d, bt = _block_table(pool, orc, sub, w.req_pages[sub])
        _gather_layers(pool, orc, sub, bt_d, bt, w.req_lens[sub], w.windows[sub], range(24))
        log(f"  sub-pool {sub} gathers checked")
    assert U.ukv_pool_error_flags(pool) == frozenset()


def test_full_move_70b():
    """Llama-3-70B-shape pool, 32,768 pages (160 GiB): 65,536 rows moved to 65,536 disjoint rows
    on all 80 layers, K and V, in one launch."""
    w = W.move_70b()
    pool, orc = _make(w)
    src_d, src = _translate(pool, orc, 0, w.move_src[0])
    dst_d, dst = _translate(pool, orc, 0, w.move_dst[0])
    U.ukv_move_kv(pool, 0, dst_d, src_d)
    d_off, s_off, fl = orc.move_map(0, dst, src, 0, 80)
    assert fl == frozenset()
    anchor, env, rb = _sub_geom(pool, 0)
    rows = rows_view(pool.raw, anchor, env, rb)
    d_rows = torch.from_numpy(offsets_to_rows(d_off, anchor, rb)).cuda()
    s_rows = torch.from_numpy(offsets_to_rows(s_off, anchor, rb)).cuda()
    # sources are disjoint from destinations, so they still hold their pre-fill bytes
    assert equal_rows_chunked(rows, d_rows, rows, s_rows), "moved rows"
    allowed = torch.zeros(env // rb, dtype=torch.bool, device="cuda")
    allowed[d_rows] = True
    changed = pattern_mismatch_rows(pool.raw, SEED, anchor, env, rb)
    assert changed.numel() == d_rows.numel()
    assert_rows_subset(changed, allowed, "move")
    assert_bytes_are_pattern(pool.raw, SEED, anchor + env, pool.raw.numel())
    assert U.ukv_pool_error_flags(pool) == frozenset()
    log("  move checked (10,485,760 rows)")


def test_full_bound_rejected_without_allocation():
    """The 70B-shape spec whose kernel-facing rows would reach 2^31 is rejected by the host
    plan; no device memory is touched (allocation stays where it was)."""
    before = torch.cuda.memory_allocated()
    assert U.plan_status([W.mha(80, 8, 128, 838861)], 16) == "UKV_ERR_KERNEL_ID_BOUND"
    assert U.plan_status([W.mha(80, 8, 128, 838860)], 16) == "UKV_OK"
    assert torch.cuda.memory_allocated() == before


def test_full_compaction_prefill_8b():
    """32 GiB pool; the 16 requests' pages (scattered over 16,383) are relocated below the
    watermark (whole page envelopes, all 32 layers, K and V) and the table rewritten; every
    gathered row is the same before and after, and only destination pages change."""
    w = W.prefill_8b(move_rows=0)
    pool, orc = _make(w)
    P, ps = w.shapes[0].num_pages, w.page_size
    used = np.unique(np.concatenate(w.req_pages[0]))
    v2p = used.astype(np.int32).copy()
    vpages = [np.searchsorted(used, p).astype(np.int32) for p in w.req_pages[0]]
    lens = w.req_lens[0]
    v2p_d = _dev(v2p)
    table = W.padded_table(vpages)
    cu = W.out_offsets(lens)
    rows = int(cu[-1])
    anchor, env, rb = _sub_geom(pool, 0)

    def read():
        bt = U.ukv_translate_pages_for_kernel(pool, 0, _dev(table), v2p=v2p_d)
        ko = torch.empty((32, rows, rb), dtype=torch.uint8, device="cuda")
        vo = torch.empty_like(ko)
        U.ukv_gather_kv_layers(pool, 0, 0, 32, bt, _dev(lens), _dev(cu), 0, ko, vo)
        return ko, vo

    before = read()
    src, dst = W.compaction_plan(used, P)
    log(f"  relocating {src.size} pages ({src.size * pool.plan.sub[0].page_bytes / 1e9:.2f} GB)")
    snap = pool.raw.clone()
    U.ukv_move_pages(pool, 0, _dev(dst), _dev(src))
    U.ukv_remap_pages(pool, 0, v2p_d, _dev(np.searchsorted(used, src).astype(np.int32)), _dev(dst))
    after = read()
    assert torch.equal(before[0], after[0]) and torch.equal(before[1], after[1])
    pb = int(pool.plan.sub[0].page_bytes)
    pages_now = pool.raw[anchor: anchor + env].view(P, pb)
    pages_then = snap[anchor: anchor + env].view(P, pb)
    d_t, s_t = _dev(dst.astype(np.int64)), _dev(src.astype(np.int64))
    assert torch.equal(pages_now.index_select(0, d_t), pages_then.index_select(0, s_t))
    changed = (pages_now != pages_then).any(dim=1).nonzero().flatten()
    allowed = torch.zeros(P, dtype=torch.bool, device="cuda")
    allowed[d_t] = True
    assert_rows_subset(changed, allowed, "page move")
    v2p_exp = v2p.copy()
    orc.remap_pages(0, v2p_exp, np.searchsorted(used, src).astype(np.int32), dst)
    assert np.array_equal(v2p_d.cpu().numpy(), v2p_exp)
    assert U.ukv_pool_error_flags(pool) == frozenset()
    del snap


def _top_pages(ps):
    """The largest page count the host plan admits for one layer of one 8-element bf16 head
    (16-byte rows) at page size ps: kernel-facing rows then reach just below 2^31."""
    lo, hi = 1, 1 << 28
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if U.plan_status([W.mha(1, 1, 8, mid)], ps) == "UKV_OK":
            lo = mid
        else:
            hi = mid - 1
    return lo


def test_full_top_of_the_kernel_id_space():
    """16-byte rows (one layer, one head of 8 bf16), page size 16, the largest page count the
    2^31 row bound admits (32 GiB, 2^31 rows): the last two pages, page 1 and a middle one
    stored (K and V, one tombstone; the last V row is the envelope's last row; page 0 is the
    sink and holds no live slot), gathered back in full and windowed through a table that
    lists the last page first, then rows of the top and middle pages moved to page 2 and to
    one near the top.  Every touched row against the oracle's addresses, every other byte
    against the pre-fill."""
    ps = 16
    P = _top_pages(ps)
    assert U.plan_status([W.mha(1, 1, 8, P + 1)], ps) == "UKV_ERR_KERNEL_ID_BOUND"
    assert oracle.plan(ospecs([W.mha(1, 1, 8, P)]), ps).code == "ok"
    assert oracle.plan(ospecs([W.mha(1, 1, 8, P + 1)]), ps).code != "ok"
    w = SimpleNamespace(shapes=[W.mha(1, 1, 8, P)], page_size=ps)
    pool, orc = _make(w)
    anchor, env, rb = _sub_geom(pool, 0)
    assert rb == 16 and env // rb > (1 << 31) - 64
    top, mid = P - 1, P // 2
    pages = [top, top - 1, 1, mid]
    slots = np.concatenate([np.arange(p * ps, (p + 1) * ps) for p in pages]).astype(np.int64)
    slots[5] = -1  # a tombstone
    ids_d, ids = _translate(pool, orc, 0, slots)
    assert int(ids.max()) == top * 2 * ps + ps - 1
    masks = _masks(pool)
    _store_layers(pool, orc, 0, ids_d, ids, slots, masks, 1700)
    assert bool(masks[0][env // rb - 1])  # the envelope's last row was written
    log("  stores checked")
    req_pages = [np.array([top, top - 1], np.int32), np.array([mid, 1], np.int32)]
    lens = [2 * ps, ps + 4]
    bt_d, bt = _block_table(pool, orc, 0, req_pages)
    _gather_layers(pool, orc, 0, bt_d, bt, lens, [0], [0])
    _gather_layers(pool, orc, 0, bt_d, bt, lens, [5], [0])
    log("  gathers checked")
    src = np.concatenate([np.arange(top * ps, (top + 1) * ps), np.arange(mid * ps, (mid + 1) * ps)]).astype(np.int64)
    dst = np.concatenate([np.arange(2 * ps, 3 * ps), np.arange((top - 2) * ps, (top - 1) * ps)]).astype(np.int64)
    src_d, s_ids = _translate(pool, orc, 0, src)
    dst_d, d_ids = _translate(pool, orc, 0, dst)
    U.ukv_move_kv(pool, 0, dst_d, src_d)
    d_off, s_off, fl = orc.move_map(0, d_ids, s_ids, 0, 1)
    assert fl == frozenset()
    rows = rows_view(pool.raw, anchor, env, rb)
    d_rows = torch.from_numpy(offsets_to_rows(d_off, anchor, rb)).cuda()
    s_rows = torch.from_numpy(offsets_to_rows(s_off, anchor, rb)).cuda()
    # sources and destinations are disjoint, so the sources still hold what was stored
    assert equal_rows_chunked(rows, d_rows, rows, s_rows), "moved rows"
    masks[0][d_rows] = True
    _check_untouched(pool, masks)
    log("  move and untouched bytes checked")
    assert U.ukv_pool_error_flags(pool) == frozenset()
