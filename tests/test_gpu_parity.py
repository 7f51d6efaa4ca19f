"""GPU parity: the HIP path (through the C-ABI) against the CPU oracle.

Integer / byte work, so the bar is bit-exact on every byte of the pool and of
every output, with one documented exception: the sink row (id 0 of each view)
that tombstoned store entries all write, where each chunk of the store's vector
width (16 bytes for aligned rows) must come whole from one of those entries'
source rows.  Sizes here span several waves and blocks
with ragged tails; the workload-sized cases are in test_gpu_full.py.
"""
import numpy as np
import pytest
import torch

import oracle
import store_gather_amd as U
import ukv_workloads as W
from parity_util import Pair, bf16_rows, log, rows_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _name(request):
    log(f"\n[gpu] {request.node.name}")
    torch.cuda.synchronize()
    yield
    torch.cuda.synchronize()


def test_device_fill_matches_host_fill():
    t = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    W.fill_pattern_device(t, 11, byte_start=4096, chunk_words=3000)
    assert np.array_equal(t.cpu().numpy(), W.fill_pattern_host(11, 4096, 1 << 20))


# ---------------------------------------------------------------------------
# translate
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape,ps", [(W.mha(2, 2, 8, 16), 4), (W.mha(32, 8, 128, 300), 16), (W.mla(24, 77), 64),
                                      (W.mha(3, 1, 8, 9), 1)])
def test_translate_parity(shape, ps):
    pair = Pair([shape], ps)
    P = shape.num_pages
    g = np.random.default_rng(5)
    n = 3000
    slots = g.integers(-3, P * ps + 40, size=n).astype(np.int64)
    slots[:5] = [-1, 0, P * ps - 1, P * ps, (1 << 40)]
    ids = U.ukv_translate_loc_for_kernel(pair.gpu, 0, to_dev(slots))
    exp, ef = pair.orc.translate(0, slots)
    assert np.array_equal(ids.cpu().numpy(), exp)
    assert U.ukv_pool_error_flags(pair.gpu) == ef == {"slot_range"}
    # virtual-to-physical table with unmapped entries and entries past the pool
    v2p = g.integers(-2, P + 3, size=P + 5).astype(np.int32)
    slots = g.integers(-2, (P + 7) * ps, size=n).astype(np.int64)
    ids = U.ukv_translate_loc_for_kernel(pair.gpu, 0, to_dev(slots), v2p=to_dev(v2p))
    exp, ef = pair.orc.translate(0, slots, v2p)
    assert np.array_equal(ids.cpu().numpy(), exp)
    assert U.ukv_pool_error_flags(pair.gpu) == ef
    # all in range: no flag
    live = W.live_slots(1, P, ps, min(500, (P - 1) * ps))
    ids = U.ukv_translate_loc_for_kernel(pair.gpu, 0, to_dev(live))
    exp, ef = pair.orc.translate(0, live)
    assert np.array_equal(ids.cpu().numpy(), exp) and ef == frozenset()
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()


def test_translate_pages_parity_and_in_place():
    pair = Pair([W.mha(4, 2, 8, 50)], 8)
    g = np.random.default_rng(9)
    pages = g.integers(-2, 60, size=(37, 11)).astype(np.int32)
    kp = U.ukv_translate_pages_for_kernel(pair.gpu, 0, to_dev(pages))
    exp, ef = pair.orc.translate_pages(0, pages)
    assert np.array_equal(kp.cpu().numpy(), exp)
    assert U.ukv_pool_error_flags(pair.gpu) == ef == {"slot_range"}
    # in place (same buffer) is allowed for pages
    d = to_dev(np.clip(pages, -1, 49))
    U.ukv_translate_pages_for_kernel(pair.gpu, 0, d, out=d)
    exp, ef = pair.orc.translate_pages(0, np.clip(pages, -1, 49))
    assert np.array_equal(d.cpu().numpy(), exp) and ef == frozenset()
    v2p = g.integers(-1, 50, size=40).astype(np.int32)
    kp = U.ukv_translate_pages_for_kernel(pair.gpu, 0, to_dev(pages), v2p=to_dev(v2p))
    exp, ef = pair.orc.translate_pages(0, pages, v2p)
    assert np.array_equal(kp.cpu().numpy(), exp)
    assert U.ukv_pool_error_flags(pair.gpu) == ef


@pytest.mark.parametrize("n", [1, 2, 1023, 1024, 1025, 5000, 70001])
def test_translate_in_place_over_its_slots(n):
    """The int32 ids written over the int64 slots they come from (out = the slots' own
    buffer): bit-exact against the oracle for the kernel-facing and the internal ids, with
    and without a v2p table, across the one-workgroup kernel's chunk boundaries, with
    tombstones, unmapped pages and out-of-range slots (flagged)."""
    P, ps = 300, 16
    pair = Pair([W.mha(3, 2, 8, P)], ps)
    g = np.random.default_rng(n)
    slots = g.integers(-3, P * ps + 40, size=n).astype(np.int64)
    v2p = g.permutation(P + 20).astype(np.int32)[:P + 5]
    v2p[g.choice(P + 5, 30, replace=False)] = -1
    v2p[v2p >= P + 3] = P + 1  # some mapped past the pool
    for table in (None, v2p):
        for internal in (False, True):
            buf = to_dev(slots)
            out = buf.view(torch.int32)[:n]
            fn = U.ukv_translate_loc if internal else U.ukv_translate_loc_for_kernel
            fn(pair.gpu, 0, buf, v2p=None if table is None else to_dev(table), out=out)
            ofn = pair.orc.translate_loc if internal else pair.orc.translate
            exp, ef = ofn(0, slots, table)
            assert np.array_equal(out.cpu().numpy(), exp), (internal, table is None)
            assert U.ukv_pool_error_flags(pair.gpu) == ef


def test_translate_rejects_other_overlaps():
    pair = Pair([W.mha(2, 2, 8, 16)], 4)
    buf = torch.zeros(64, dtype=torch.int64, device="cuda")
    for out in (buf.view(torch.int32)[1:65], buf.view(torch.int32)[64:128]):
        with pytest.raises(U.UkvError) as e:
            U.ukv_translate_loc_for_kernel(pair.gpu, 0, buf, out=out)
        assert e.value.status == "UKV_ERR_INVALID_ARG"
    table = torch.zeros(80, dtype=torch.int32, device="cuda")
    with pytest.raises(U.UkvError, match="v2p"):
        U.ukv_translate_loc_for_kernel(pair.gpu, 0, buf, v2p=table, out=table[8:72])
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()


# ---------------------------------------------------------------------------
# the tiny pool: store, gather, move
# ---------------------------------------------------------------------------

def test_tiny_store_gather_move():
    w = W.tiny_mha(seed=0)
    pair = Pair(w.shapes, w.page_size)
    rb = pair.rb(0)
    slots = w.store_slots[0]
    ids_d = U.ukv_translate_loc_for_kernel(pair.gpu, 0, to_dev(slots))
    ids, ef = pair.orc.translate(0, slots)
    assert np.array_equal(ids_d.cpu().numpy(), ids) and ef == frozenset()
    for layer in range(2):
        k = bf16_rows(100 + layer, slots.size, rb)
        v = bf16_rows(200 + layer, slots.size, rb)
        U.ukv_store_kv(pair.gpu, 0, layer, ids_d, rows_dev(k), rows_dev(v))
        assert pair.orc.store(0, layer, ids, k, v) == frozenset()
        pair.record_store(0, layer, ids, k, v)
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()
    pair.assert_pools_equal()

    pages, lens = w.req_pages[0], w.req_lens[0]
    table = W.padded_table(pages)
    bt_d = U.ukv_translate_pages_for_kernel(pair.gpu, 0, to_dev(table))
    bt, _ = pair.orc.translate_pages(0, table)
    assert np.array_equal(bt_d.cpu().numpy(), bt)
    for window in (0, 3, 8):
        cu = W.out_offsets(lens, window)
        for layer in range(2):
            ko = torch.zeros((int(cu[-1]), rb), dtype=torch.uint8, device="cuda")
            vo = torch.zeros_like(ko)
            U.ukv_gather_kv(pair.gpu, 0, layer, bt_d, to_dev(lens), to_dev(cu), window, ko, vo)
            eko = np.zeros((int(cu[-1]), rb), np.uint8)
            evo = np.zeros_like(eko)
            assert pair.orc.gather(0, layer, bt, lens, cu, window, eko, evo) == frozenset()
            assert np.array_equal(ko.cpu().numpy(), eko) and np.array_equal(vo.cpu().numpy(), evo)
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()

    src, _ = pair.orc.translate(0, w.move_src[0])
    dst, _ = pair.orc.translate(0, w.move_dst[0])
    U.ukv_move_kv(pair.gpu, 0, to_dev(dst), to_dev(src))
    assert pair.orc.move(0, dst, src, 0, 2) == frozenset()
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()
    pair.assert_pools_equal()


# ---------------------------------------------------------------------------
# scaled-down workloads: the real row shapes, fewer pages and requests
# ---------------------------------------------------------------------------

def _store_all_layers(pair, sub, slots, seed, layers=None):
    rb = pair.rb(sub)
    ids_d = U.ukv_translate_loc_for_kernel(pair.gpu, sub, to_dev(slots))
    ids, ef = pair.orc.translate(sub, slots)
    assert np.array_equal(ids_d.cpu().numpy(), ids) and ef == frozenset()
    for layer in (range(pair.shapes[sub].layer_num) if layers is None else layers):
        k = bf16_rows(seed + 2 * layer, slots.size, rb)
        v = bf16_rows(seed + 2 * layer + 1, slots.size, rb) if pair.kvs(sub) == 2 else None
        U.ukv_store_kv(pair.gpu, sub, layer, ids_d, rows_dev(k), None if v is None else rows_dev(v))
        assert pair.orc.store(sub, layer, ids, k, v) == frozenset()
        pair.record_store(sub, layer, ids, k, v)
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()


def _gather_all_layers(pair, sub, pages, lens, windows, layers=None):
    rb = pair.rb(sub)
    table = W.padded_table(pages)
    bt_d = U.ukv_translate_pages_for_kernel(pair.gpu, sub, to_dev(table))
    bt, _ = pair.orc.translate_pages(sub, table)
    lens = np.asarray(lens, dtype=np.int32)
    lens_d = to_dev(lens)
    for layer in (range(pair.shapes[sub].layer_num) if layers is None else layers):
        win = windows[layer]
        cu = W.out_offsets(lens, win)
        ko = torch.empty((int(cu[-1]), rb), dtype=torch.uint8, device="cuda")
        vo = torch.empty_like(ko) if pair.kvs(sub) == 2 else None
        U.ukv_gather_kv(pair.gpu, sub, layer, bt_d, lens_d, to_dev(cu), win, ko, vo)
        eko = np.zeros((int(cu[-1]), rb), np.uint8)
        evo = np.zeros_like(eko) if vo is not None else None
        assert pair.orc.gather(sub, layer, bt, lens, cu, win, eko, evo) == frozenset()
        assert np.array_equal(ko.cpu().numpy(), eko), f"layer {layer} K"
        if vo is not None:
            assert np.array_equal(vo.cpu().numpy(), evo), f"layer {layer} V"
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()


def test_scaled_decode_8b():
    w = W.decode_8b(num_pages=64, num_reqs=7, len_lo=50, len_hi=700, new_tokens=37)
    pair = Pair(w.shapes, w.page_size)
    _store_all_layers(pair, 0, w.store_slots[0], 1000)
    pair.assert_pools_equal()
    _gather_all_layers(pair, 0, w.req_pages[0], w.req_lens[0], w.windows[0])


def test_scaled_prefill_8b_with_tombstones_and_move():
    w = W.prefill_8b(num_pages=96, tokens=900, num_reqs=5, move_rows=150)
    assert (w.store_slots[0] < 0).sum() == 9
    pair = Pair(w.shapes, w.page_size)
    _store_all_layers(pair, 0, w.store_slots[0], 2000)
    pair.assert_pools_equal()
    _gather_all_layers(pair, 0, w.req_pages[0], w.req_lens[0], w.windows[0], layers=[0, 13, 31])
    src, _ = pair.orc.translate(0, w.move_src[0])
    dst, _ = pair.orc.translate(0, w.move_dst[0])
    U.ukv_move_kv(pair.gpu, 0, to_dev(dst), to_dev(src))
    pair.orc.move(0, dst, src, 0, 32)
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()
    pair.assert_pools_equal()


def test_scaled_hybrid_mha_swa_and_mla():
    w = W.hybrid(num_reqs=6, len_lo=20, len_hi=700, layer_num=24, window=128)
    pair = Pair(w.shapes, w.page_size)
    for sub in (0, 1):
        _store_all_layers(pair, sub, w.store_slots[sub], 3000 + 100 * sub)
    pair.assert_pools_equal()
    for sub in (0, 1):
        _gather_all_layers(pair, sub, w.req_pages[sub], w.req_lens[sub], w.windows[sub])
    # move within the MLA sub-pool, a partial layer range
    mv = W.live_slots(4, w.shapes[1].num_pages, 64, 60, sub=77)
    src, _ = pair.orc.translate(1, mv[:30])
    dst, _ = pair.orc.translate(1, mv[30:])
    U.ukv_move_kv(pair.gpu, 1, to_dev(dst), to_dev(src), 5, 19)
    pair.orc.move(1, dst, src, 5, 19)
    pair.assert_pools_equal()


def test_scaled_move_70b():
    w = W.move_70b(num_pages=40, rows=200)
    pair = Pair(w.shapes, w.page_size)
    src, _ = pair.orc.translate(0, w.move_src[0])
    dst, _ = pair.orc.translate(0, w.move_dst[0])
    U.ukv_move_kv(pair.gpu, 0, to_dev(dst), to_dev(src))
    pair.orc.move(0, dst, src, 0, 80)
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()
    pair.assert_pools_equal()


# ---------------------------------------------------------------------------
# row widths that need narrower vectors, strided / misaligned sources
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape,ps", [
    (W.mha(3, 1, 3, 11), 3),                  # 6-byte rows: 2-byte vectors
    (W.mha(2, 1, 7, 9, elem_bytes=1), 4),     # 7-byte rows: bytes
    (W.mha(2, 2, 2, 9), 5),                   # 8-byte rows
    (W.mla(3, 13, latent_dim=20), 2),         # 40-byte rows: 8-byte vectors
    (W.mha(2, 4, 96, 10, elem_bytes=4), 4),   # 1536-byte rows, fp32 itemsize
])
def test_odd_row_sizes(shape, ps):
    pair = Pair([shape], ps)
    P = shape.num_pages
    slots = W.live_slots(3, P, ps, min(40, (P - 1) * ps))
    _store_all_layers(pair, 0, slots, 4000)
    pair.assert_pools_equal()
    g = np.random.default_rng(1)
    lens = np.array([1, ps, 2 * ps + 1, 0, 3 * ps - 1], dtype=np.int32)
    pages = [g.integers(1, P, size=max(1, -(-int(n) // ps))).astype(np.int32) for n in lens]
    _gather_all_layers(pair, 0, pages, lens, [0, 2, 0][: shape.layer_num])
    mv = W.live_slots(8, P, ps, 20, sub=9)
    src, _ = pair.orc.translate(0, mv[:10])
    dst, _ = pair.orc.translate(0, mv[10:])
    U.ukv_move_kv(pair.gpu, 0, to_dev(dst), to_dev(src))
    pair.orc.move(0, dst, src, 0, shape.layer_num)
    pair.assert_pools_equal()


@pytest.mark.parametrize("shape,ps", [
    (W.mla(3, 24, latent_dim=512), 8),        # 1 KiB latents: one-view pieces, one per row
    (W.mla(2, 24, latent_dim=1024), 4),       # 2 KiB latents: one-view pieces, two per row
    (W.mha(2, 8, 256, 24), 4),                # 4 KiB rows: four pieces per row and view
    (W.mha(3, 4, 128, 24), 16),               # 1 KiB rows: gather pieces K and V of one row, tiled store
])
def test_row_piece_shapes(shape, ps):
    """The row-piece kernels on the row shapes the workloads do not cover: latents of
    whole KiB (one view), 4 KiB rows, 1 KiB MHA rows; stores, gathers (full and
    windowed, ragged) and a move, against the oracle byte for byte."""
    pair = Pair([shape], ps)
    P = shape.num_pages
    slots = W.live_slots(5, P, ps, min(70, (P - 1) * ps))
    _store_all_layers(pair, 0, slots, 4500)
    pair.assert_pools_equal()
    g = np.random.default_rng(2)
    lens = np.array([1, ps, 2 * ps + 1, 0, 5 * ps - 1, 3], dtype=np.int32)
    pages = [g.integers(1, P, size=max(1, -(-int(n) // ps))).astype(np.int32) for n in lens]
    _gather_all_layers(pair, 0, pages, lens, [0, ps + 1, 0][: shape.layer_num])
    mv = W.live_slots(9, P, ps, 24, sub=9)
    src, _ = pair.orc.translate(0, mv[:12])
    dst, _ = pair.orc.translate(0, mv[12:])
    U.ukv_move_kv(pair.gpu, 0, to_dev(dst), to_dev(src), 0, shape.layer_num)
    pair.orc.move(0, dst, src, 0, shape.layer_num)
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()
    pair.assert_pools_equal()


@pytest.mark.parametrize("shape,n", [
    (W.mla(4, 40, latent_dim=576), 203),      # 1,152-byte latents: 9 loads per lane, one view
    (W.mla(3, 40, latent_dim=640), 64),       # 1,280 bytes: 10 loads
    (W.mha(3, 9, 64, 40), 77),                # 1,152-byte MHA rows: K and V groups
    (W.mha(2, 12, 64, 40), 8),                # 1,536 bytes: 12 loads, one whole group
    (W.mha(2, 15, 64, 40), 131),              # 1,920 bytes: 15 loads
])
def test_store_group_shapes(shape, n):
    """The row-group store (rows of 1,152 to 1,920 bytes, eight entries of one view per
    wave) on ragged entry counts, with tombstones and a bad id among the entries, one
    layer at a time and fused over the layers: byte for byte against the oracle, flags
    too."""
    ps = 16
    pair = Pair([shape], ps)
    rb = pair.rb(0)
    assert 1024 < rb < 2048 and rb % 128 == 0
    L = shape.layer_num
    nkv = pair.kvs(0)
    slots = W.live_slots(n + 3, shape.num_pages, ps, n).copy()
    slots[::11] = -1  # tombstones
    ids, _ = pair.orc.translate(0, slots)
    ids = ids.copy()
    ids[min(6, n - 1)] = ps + 1  # on page 0's second block: skipped and flagged
    for layer in range(L):  # one layer per launch
        k = bf16_rows(8100 + layer, n, rb)
        v = bf16_rows(8200 + layer, n, rb) if nkv == 2 else None
        U.ukv_store_kv(pair.gpu, 0, layer, to_dev(ids), rows_dev(k), None if v is None else rows_dev(v))
        assert pair.orc.store(0, layer, ids, k, v) == {"bad_id"}
        pair.record_store(0, layer, ids, k, v)
    assert U.ukv_pool_error_flags(pair.gpu) == {"bad_id"}
    pair.assert_pools_equal()
    k = bf16_rows(8300, L * n, rb)  # all layers in one launch, new values
    v = bf16_rows(8400, L * n, rb) if nkv == 2 else None
    U.ukv_store_kv_layers(pair.gpu, 0, 0, L, to_dev(ids), rows_dev(k).view(L, n, -1),
                          None if v is None else rows_dev(v).view(L, n, -1))
    for layer in range(L):
        kl = k[layer * n:(layer + 1) * n]
        vl = None if v is None else v[layer * n:(layer + 1) * n]
        assert pair.orc.store(0, layer, ids, kl, vl) == {"bad_id"}
        pair.record_store(0, layer, ids, kl, vl)
    assert U.ukv_pool_error_flags(pair.gpu) == {"bad_id"}
    pair.assert_pools_equal()


# (entries, layers) -> pieces per wave on 256 CUs: 1 (small), 2, 4, 8 (a ragged last wave
# in each layer), 1 (more than eight rounds of resident waves); multi-layer launches take
# the XCD order, (101, 3) and (7, 5) with a grid that is no multiple of the 8 XCDs
@pytest.mark.parametrize("n,layers", [(256, 1), (101, 32), (256, 32), (401, 32), (1500, 32), (40, 32), (101, 3),
                                      (7, 5)])
def test_store_pieces_per_wave(n, layers):
    """Fused stores whose size gives each wave 1, 2, 4 or 8 pieces (a small launch is
    packed into one round of resident waves), with tombstones and a bad id among the
    entries: byte for byte against the oracle, flags too."""
    P, ps = 160, 16
    shape = W.mha(32, 8, 128, P)
    pair = Pair([shape], ps)
    rb = pair.rb(0)
    slots = W.live_slots(n, P, ps, n).copy()
    slots[::37] = -1  # tombstones
    ids, _ = pair.orc.translate(0, slots)
    ids = ids.copy()
    ids[5] = 2 * ps + 3  # on page 0's third block, not its first: skipped and flagged
    k = bf16_rows(6000 + n, layers * n, rb)
    v = bf16_rows(7000 + n, layers * n, rb)
    U.ukv_store_kv_layers(pair.gpu, 0, 32 - layers, layers, to_dev(ids), rows_dev(k).view(layers, n, -1),
                          rows_dev(v).view(layers, n, -1))
    flags = set()
    for i in range(layers):
        l = 32 - layers + i
        flags |= pair.orc.store(0, l, ids, k[i * n:(i + 1) * n], v[i * n:(i + 1) * n])
        pair.record_store(0, l, ids, k[i * n:(i + 1) * n], v[i * n:(i + 1) * n])
    assert U.ukv_pool_error_flags(pair.gpu) == flags == {"bad_id"}
    pair.assert_pools_equal()


def test_strided_and_misaligned_sources():
    pair = Pair([W.mha(4, 2, 64, 20)], 8)
    rb = pair.rb(0)
    slots = W.live_slots(2, 20, 8, 50)
    ids_d = U.ukv_translate_loc_for_kernel(pair.gpu, 0, to_dev(slots))
    ids, _ = pair.orc.translate(0, slots)
    # K and V as halves of one fused [n, 2, rb] tensor: row stride 2 * rb
    kv = bf16_rows(50, 2 * slots.size, rb).reshape(slots.size, 2, rb)
    fused = to_dev(kv)
    U.ukv_store_kv(pair.gpu, 0, 1, ids_d, fused[:, 0], fused[:, 1])
    pair.orc.store(0, 1, ids, kv[:, 0], kv[:, 1])
    # sources that start 2 bytes past a 16-byte boundary: narrower vectors
    big = torch.zeros(slots.size * rb + 2, dtype=torch.uint8, device="cuda")
    k = bf16_rows(60, slots.size, rb)
    big[2:].copy_(torch.from_numpy(k.reshape(-1)).cuda())
    kmis = big[2:].view(slots.size, rb)
    assert kmis.data_ptr() % 16 == 2
    U.ukv_store_kv(pair.gpu, 0, 2, ids_d, kmis, kmis)
    pair.orc.store(0, 2, ids, k, k)
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()
    pair.assert_pools_equal()


# ---------------------------------------------------------------------------
# device-side conditions: flags raised, rows skipped, exactly as the oracle
# ---------------------------------------------------------------------------

def test_bad_ids_and_tables_are_flagged_and_skipped():
    pair = Pair([W.mha(2, 2, 8, 6)], 4)
    rb = pair.rb(0)
    # block 1 of page 0, offset 5 >= ps on page 5, block 3 of page 0, negative, past the pool, huge; then a valid id
    ids = np.array([4, 5 * 16 + 5, 15, -7, 6 * 16, 1 << 30, 16 + 2], dtype=np.int32)
    k = bf16_rows(1, ids.size, rb)
    v = bf16_rows(2, ids.size, rb)
    U.ukv_store_kv(pair.gpu, 0, 1, to_dev(ids), rows_dev(k), rows_dev(v))
    assert pair.orc.store(0, 1, ids, k, v) == {"bad_id"}
    assert U.ukv_pool_error_flags(pair.gpu) == {"bad_id"}
    pair.assert_pools_equal()
    # move with one bad pair among good ones
    dst = np.array([16 + 1, 37, 2 * 16 + 3], dtype=np.int32)  # 37 is block 0, offset 5 >= ps
    src = np.array([3 * 16, 4 * 16 + 2, 5 * 16], dtype=np.int32)
    U.ukv_move_kv(pair.gpu, 0, to_dev(dst), to_dev(src))
    assert pair.orc.move(0, dst, src, 0, 2) == {"bad_id"}
    assert U.ukv_pool_error_flags(pair.gpu) == {"bad_id"}
    pair.assert_pools_equal()
    # gather: a block entry that is not a multiple of blocks_per_page, one past the pool,
    # a table too narrow for the length, and an inconsistent cu_out
    lens = np.array([5, 3, 9, 2], dtype=np.int32)
    bt = np.array([[4, 9], [6, 0], [8, 12], [24, 0]], dtype=np.int32)
    for cu in (W.out_offsets(lens), np.array([0, 5, 7, 16, 19], dtype=np.int64)):
        rows = int(cu[-1])
        ko = torch.zeros((rows, rb), dtype=torch.uint8, device="cuda")
        vo = torch.zeros_like(ko)
        U.ukv_gather_kv(pair.gpu, 0, 0, to_dev(bt), to_dev(lens), to_dev(cu), 0, ko, vo)
        eko = np.zeros((rows, rb), np.uint8)
        evo = np.zeros_like(eko)
        ef = pair.orc.gather(0, 0, bt, lens, cu, 0, eko, evo)
        assert U.ukv_pool_error_flags(pair.gpu) == ef and "bad_block" in ef
        assert np.array_equal(ko.cpu().numpy(), eko) and np.array_equal(vo.cpu().numpy(), evo)
    # out_rows larger than cu_out[-1]
    cu = W.out_offsets(lens)
    ko = torch.zeros((int(cu[-1]) + 3, rb), dtype=torch.uint8, device="cuda")
    vo = torch.zeros_like(ko)
    okbt = np.array([[4, 8, 0], [12, 0, 0], [16, 20, 4], [4, 0, 0]], dtype=np.int32)
    U.ukv_gather_kv(pair.gpu, 0, 1, to_dev(okbt), to_dev(lens), to_dev(cu), 0, ko, vo)
    eko = np.zeros(ko.shape, np.uint8)
    evo = np.zeros_like(eko)
    ef = pair.orc.gather(0, 1, okbt, lens, cu, 0, eko, evo)
    assert ef == {"layout"} and U.ukv_pool_error_flags(pair.gpu) == ef
    assert np.array_equal(ko.cpu().numpy(), eko) and np.array_equal(vo.cpu().numpy(), evo)


def test_empty_and_degenerate_calls():
    pair = Pair([W.mha(2, 2, 8, 6), W.mla(2, 5, latent_dim=8)], 4)
    e64 = torch.empty(0, dtype=torch.int64, device="cuda")
    e32 = torch.empty(0, dtype=torch.int32, device="cuda")
    assert U.ukv_translate_loc_for_kernel(pair.gpu, 0, e64).numel() == 0
    U.ukv_store_kv(pair.gpu, 0, 0, e32, torch.empty((0, 32), dtype=torch.uint8, device="cuda"),
                   torch.empty((0, 32), dtype=torch.uint8, device="cuda"))
    U.ukv_move_kv(pair.gpu, 0, e32, e32)
    ids = to_dev(np.array([17], dtype=np.int32))
    U.ukv_move_kv(pair.gpu, 0, ids, ids, 1, 1)  # empty layer range
    # a zero-length request between two others, and an all-tombstone store
    lens = np.array([3, 0, 2], dtype=np.int32)
    bt = np.array([[4], [0], [8]], dtype=np.int32)
    cu = W.out_offsets(lens)
    ko = torch.zeros((5, 32), dtype=torch.uint8, device="cuda")
    vo = torch.zeros_like(ko)
    U.ukv_gather_kv(pair.gpu, 0, 1, to_dev(bt), to_dev(lens), to_dev(cu), 0, ko, vo)
    eko = np.zeros((5, 32), np.uint8)
    evo = np.zeros_like(eko)
    assert pair.orc.gather(0, 1, bt, lens, cu, 0, eko, evo) == frozenset()
    assert np.array_equal(ko.cpu().numpy(), eko) and np.array_equal(vo.cpu().numpy(), evo)
    tomb = np.full(5, -1, dtype=np.int64)
    ids_d = U.ukv_translate_loc_for_kernel(pair.gpu, 1, to_dev(tomb))
    ids, _ = pair.orc.translate(1, tomb)
    k = bf16_rows(9, 5, 16)
    U.ukv_store_kv(pair.gpu, 1, 1, ids_d, rows_dev(k))
    pair.orc.store(1, 1, ids, k, None)
    pair.record_store(1, 1, ids, k, None)
    # no requests, no rows
    U.ukv_gather_kv(pair.gpu, 1, 0, to_dev(np.zeros((0, 1), np.int32)), e32, to_dev(np.zeros(1, np.int64)), 0,
                    torch.empty((0, 16), dtype=torch.uint8, device="cuda"))
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()
    pair.assert_pools_equal()


def test_host_argument_errors():
    pair = Pair([W.mha(2, 2, 8, 6), W.mla(2, 5, latent_dim=8)], 4)
    ids = to_dev(np.array([16], dtype=np.int32))
    rows = torch.zeros((1, 32), dtype=torch.uint8, device="cuda")
    for call in (
        lambda: U.ukv_store_kv(pair.gpu, 0, 2, ids, rows, rows),           # layer out of range
        lambda: U.ukv_store_kv(pair.gpu, 1, 0, ids, rows[:, :16], rows[:, :16]),  # MLA takes no V
        lambda: U.ukv_move_kv(pair.gpu, 0, ids, ids, 1, 3),                # layer range
    ):
        with pytest.raises(U.UkvError) as e:
            call()
        assert e.value.status == "UKV_ERR_INVALID_ARG"
    with pytest.raises(U.UkvError) as e:
        U.ukv_move_kv(pair.gpu, 2, ids, ids, 0, 1)  # no such sub-pool
    assert e.value.status == "UKV_ERR_INVALID_ARG"
    with pytest.raises(ValueError):
        U.ukv_store_kv(pair.gpu, 0, 0, ids.cpu(), rows, rows)  # host tensor never reaches the library
    # a raw buffer one byte short of the tail pad
    plan = U.ukv_pool_plan([W.mha(2, 2, 8, 16)], 4)
    short = torch.empty(int(plan.required_bytes) - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(U.UkvError) as e:
        U.ukv_pool_create([W.mha(2, 2, 8, 16)], 4, short)
    assert e.value.status == "UKV_ERR_TAIL_PAD"
    # host memory is refused before any launch
    import ctypes
    host = np.zeros(int(plan.required_bytes), dtype=np.uint8)
    h = ctypes.c_void_p()
    rc = U.lib().ukv_pool_create(U._specs_array([W.mha(2, 2, 8, 16)]), 1, 4, host.ctypes.data, host.size,
                                 ctypes.byref(h))
    assert rc == -1 and "not device memory" in U.ukv_last_error()


# ---------------------------------------------------------------------------
# several layers per launch (one translation serves every layer)
# ---------------------------------------------------------------------------

def test_fused_layer_store_and_gather():
    w = W.decode_8b(num_pages=48, num_reqs=5, len_lo=30, len_hi=400, new_tokens=61)
    pair = Pair(w.shapes, w.page_size)
    rb = pair.rb(0)
    slots = w.store_slots[0]
    ids_d = U.ukv_translate_loc_for_kernel(pair.gpu, 0, to_dev(slots))
    ids, _ = pair.orc.translate(0, slots)
    layers = list(range(3, 30, 2))  # 14 layers, step 2
    k = bf16_rows(70, len(layers) * slots.size, rb).reshape(len(layers), slots.size, rb)
    v = bf16_rows(71, len(layers) * slots.size, rb).reshape(len(layers), slots.size, rb)
    U.ukv_store_kv_layers(pair.gpu, 0, 3, len(layers), ids_d, to_dev(k), to_dev(v), layer_step=2)
    for i, layer in enumerate(layers):
        pair.orc.store(0, layer, ids, k[i], v[i])
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()
    pair.assert_pools_equal()
    table = W.padded_table(w.req_pages[0])
    bt_d = U.ukv_translate_pages_for_kernel(pair.gpu, 0, to_dev(table))
    bt, _ = pair.orc.translate_pages(0, table)
    lens = w.req_lens[0]
    for window, begin, count, step in ((0, 0, 32, 1), (100, 1, 11, 3)):
        cu = W.out_offsets(lens, window)
        rows = int(cu[-1])
        ko = torch.zeros((count, rows, rb), dtype=torch.uint8, device="cuda")
        vo = torch.zeros_like(ko)
        U.ukv_gather_kv_layers(pair.gpu, 0, begin, count, bt_d, to_dev(lens), to_dev(cu), window, ko, vo,
                               layer_step=step)
        kh, vh = ko.cpu().numpy(), vo.cpu().numpy()
        for i in range(count):
            eko = np.zeros((rows, rb), np.uint8)
            evo = np.zeros_like(eko)
            pair.orc.gather(0, begin + i * step, bt, lens, cu, window, eko, evo)
            assert np.array_equal(kh[i], eko) and np.array_equal(vh[i], evo), (window, i)
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()


def test_fused_layers_mla_and_argument_errors():
    w = W.hybrid(num_reqs=4, len_lo=10, len_hi=300, layer_num=24, window=128)
    pair = Pair(w.shapes, w.page_size)
    rb = pair.rb(1)
    slots = w.store_slots[1]
    ids_d = U.ukv_translate_loc_for_kernel(pair.gpu, 1, to_dev(slots))
    ids, _ = pair.orc.translate(1, slots)
    lat = bf16_rows(80, 24 * slots.size, rb).reshape(24, slots.size, rb)
    U.ukv_store_kv_layers(pair.gpu, 1, 0, 24, ids_d, to_dev(lat))
    for layer in range(24):
        pair.orc.store(1, layer, ids, lat[layer], None)
    pair.assert_pools_equal()
    lens = w.req_lens[1]
    table = W.padded_table(w.req_pages[1])
    bt_d = U.ukv_translate_pages_for_kernel(pair.gpu, 1, to_dev(table))
    bt, _ = pair.orc.translate_pages(1, table)
    cu = W.out_offsets(lens)
    rows = int(cu[-1])
    ko = torch.zeros((6, rows, rb), dtype=torch.uint8, device="cuda")
    U.ukv_gather_kv_layers(pair.gpu, 1, 2, 6, bt_d, to_dev(lens), to_dev(cu), 0, ko, layer_step=4)
    kh = ko.cpu().numpy()
    for i in range(6):
        eko = np.zeros((rows, rb), np.uint8)
        pair.orc.gather(1, 2 + 4 * i, bt, lens, cu, 0, eko, None)
        assert np.array_equal(kh[i], eko)
    # a layer range past the sub-pool, and overlapping per-layer outputs, are refused
    with pytest.raises(U.UkvError) as e:
        U.ukv_gather_kv_layers(pair.gpu, 1, 2, 6, bt_d, to_dev(lens), to_dev(cu), 0, ko, layer_step=5)
    assert e.value.status == "UKV_ERR_INVALID_ARG"
    rc = U.lib().ukv_gather_kv_layers(pair.gpu.handle, 1, 0, 2, 1, bt_d.data_ptr(), bt_d.stride(0),
                                      to_dev(lens).data_ptr(), to_dev(cu).data_ptr(), len(lens), 0, ko.data_ptr(),
                                      None, rows, rb * rows - 1, None)
    assert rc == -1 and "overlap" in U.ukv_last_error()
    with pytest.raises(U.UkvError):
        U.ukv_store_kv_layers(pair.gpu, 1, 20, 5, ids_d, to_dev(lat[:5]))
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()


# ---------------------------------------------------------------------------
# virtual-to-physical indirection and compaction
# ---------------------------------------------------------------------------

def test_translate_loc_parity():
    pair = Pair([W.mha(4, 2, 8, 30)], 8)
    g = np.random.default_rng(12)
    slots = g.integers(-3, 40 * 8, size=2000).astype(np.int64)
    v2p = g.integers(-2, 33, size=37).astype(np.int32)
    for table in (None, v2p):
        got = U.ukv_translate_loc(pair.gpu, 0, to_dev(slots), v2p=None if table is None else to_dev(table))
        exp, ef = pair.orc.translate_loc(0, slots, table)
        assert np.array_equal(got.cpu().numpy(), exp)
        assert U.ukv_pool_error_flags(pair.gpu) == ef


def test_move_pages_and_remap_parity():
    pair = Pair([W.mha(3, 2, 16, 12), W.mla(5, 9, latent_dim=24)], 4)
    for sub, (dst, src) in ((0, ([1, 2, 11], [7, 4, 5])), (1, ([3, 8], [1, 6]))):
        U.ukv_move_pages(pair.gpu, sub, to_dev(np.array(dst, np.int32)), to_dev(np.array(src, np.int32)))
        assert pair.orc.move_pages(sub, dst, src) == frozenset()
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()
    pair.assert_pools_equal()
    U.ukv_move_pages(pair.gpu, 0, to_dev(np.array([12, 3], np.int32)), to_dev(np.array([2, 3], np.int32)))
    assert pair.orc.move_pages(0, [12, 3], [2, 3]) == {"bad_id"}
    assert U.ukv_pool_error_flags(pair.gpu) == {"bad_id"}
    pair.assert_pools_equal()
    v2p = np.arange(20, dtype=np.int32)
    vd = to_dev(v2p)
    virt = np.array([3, 19, 25, 0, 7], np.int32)
    phys = np.array([11, -1, 2, 12, -2], np.int32)
    U.ukv_remap_pages(pair.gpu, 0, vd, to_dev(virt), to_dev(phys))
    assert pair.orc.remap_pages(0, v2p, virt, phys) == {"slot_range"}
    assert U.ukv_pool_error_flags(pair.gpu) == {"slot_range"}
    assert np.array_equal(vd.cpu().numpy(), v2p)


@pytest.mark.parametrize("n", [37, 101])
def test_move_pages_ragged_xcd_grid(n):
    """Page relocations whose launch grid is no multiple of the 8 XCDs (1 KiB pages: one
    wave per page, ceil(n / 4) = 10 and 26 workgroups), so both terms of the XCD order
    run: byte for byte against the oracle."""
    pair = Pair([W.mha(2, 2, 16, 256)], 4)
    assert pair.rb(0) * 4 * 4 == 1024  # page bytes: ps x 2L blocks x row bytes
    g = np.random.default_rng(n)
    perm = g.permutation(256).astype(np.int32)
    dst, src = perm[:n], perm[n:2 * n]
    U.ukv_move_pages(pair.gpu, 0, to_dev(dst), to_dev(src))
    assert pair.orc.move_pages(0, dst, src) == frozenset()
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()
    pair.assert_pools_equal()


def test_compaction_end_to_end():
    """Requests written through a virtual-to-physical table; the pages above the watermark are
    relocated below it and the table rewritten; every request reads the same K/V after."""
    w = W.prefill_8b(num_pages=160, tokens=1500, num_reqs=6, move_rows=0, layer_num=6)
    pair = Pair(w.shapes, w.page_size)
    P, ps, rb = w.shapes[0].num_pages, w.page_size, pair.rb(0)
    used = np.unique(np.concatenate(w.req_pages[0]))
    v2p = used.astype(np.int32).copy()
    vpages = [np.searchsorted(used, p).astype(np.int32) for p in w.req_pages[0]]
    lens = w.req_lens[0]
    vslots = W.slots_of_requests(vpages, lens, ps)
    v2p_d = to_dev(v2p)
    ids_d = U.ukv_translate_loc_for_kernel(pair.gpu, 0, to_dev(vslots), v2p=v2p_d)
    ids, _ = pair.orc.translate(0, vslots, v2p)
    assert np.array_equal(ids_d.cpu().numpy(), ids)
    internal = U.ukv_translate_loc(pair.gpu, 0, to_dev(vslots), v2p=v2p_d)
    assert np.array_equal(internal.cpu().numpy(), W.slots_of_requests(w.req_pages[0], lens, ps))
    for layer in range(6):
        k = bf16_rows(300 + layer, vslots.size, rb)
        v = bf16_rows(400 + layer, vslots.size, rb)
        U.ukv_store_kv(pair.gpu, 0, layer, ids_d, rows_dev(k), rows_dev(v))
        pair.orc.store(0, layer, ids, k, v)
    table = W.padded_table(vpages)
    cu = W.out_offsets(lens)

    def read(vt):
        bt = U.ukv_translate_pages_for_kernel(pair.gpu, 0, to_dev(table), v2p=vt)
        ko = torch.empty((6, int(cu[-1]), rb), dtype=torch.uint8, device="cuda")
        vo = torch.empty_like(ko)
        U.ukv_gather_kv_layers(pair.gpu, 0, 0, 6, bt, to_dev(lens), to_dev(cu), 0, ko, vo)
        return ko.cpu().numpy(), vo.cpu().numpy()

    before = read(v2p_d)
    src, dst = W.compaction_plan(used, P)
    assert src.size > 10
    U.ukv_move_pages(pair.gpu, 0, to_dev(dst), to_dev(src))
    U.ukv_remap_pages(pair.gpu, 0, v2p_d, to_dev(np.searchsorted(used, src).astype(np.int32)), to_dev(dst))
    pair.orc.move_pages(0, dst, src)
    pair.orc.remap_pages(0, v2p, np.searchsorted(used, src).astype(np.int32), dst)
    assert np.array_equal(v2p_d.cpu().numpy(), v2p) and v2p.max() <= used.size
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()
    pair.assert_pools_equal()
    after = read(v2p_d)
    assert np.array_equal(before[0], after[0]) and np.array_equal(before[1], after[1])


# ---------------------------------------------------------------------------
# sliding-window layers in a sub-pool of their own
# ---------------------------------------------------------------------------

def test_swa_subpool_store_gather_and_eviction():
    w = W.swa_decode(num_reqs=7, len_lo=40, len_hi=900, layer_num=6, window=100)
    pair = Pair(w.shapes, w.page_size)
    ps = w.page_size
    mapping = w.swa_mapping.copy()
    map_d = to_dev(mapping)
    slots = w.store_slots[0]
    lens = w.req_lens[0]
    # the new token of every request: full layers directly, window layers through the mapping
    for sub, v2p in ((0, None), (1, mapping)):
        ids_d = U.ukv_translate_loc_for_kernel(pair.gpu, sub, to_dev(slots), v2p=None if v2p is None else map_d)
        ids, _ = pair.orc.translate(sub, slots, v2p)
        assert np.array_equal(ids_d.cpu().numpy(), ids)
        rb = pair.rb(sub)
        for layer in range(3):
            k = bf16_rows(500 + 10 * sub + layer, slots.size, rb)
            v = bf16_rows(600 + 10 * sub + layer, slots.size, rb)
            U.ukv_store_kv(pair.gpu, sub, layer, ids_d, rows_dev(k), rows_dev(v))
            pair.orc.store(sub, layer, ids, k, v)
            pair.record_store(sub, layer, ids, k, v)
    pair.assert_pools_equal()
    table = W.padded_table(w.req_pages[0])
    for sub, win in ((0, 0), (1, w.window)):
        bt_d = U.ukv_translate_pages_for_kernel(pair.gpu, sub, to_dev(table), v2p=None if sub == 0 else map_d)
        bt, _ = pair.orc.translate_pages(sub, table, None if sub == 0 else mapping)
        assert np.array_equal(bt_d.cpu().numpy(), bt)
        cu = W.out_offsets(lens, win)
        rb = pair.rb(sub)
        ko = torch.empty((3, int(cu[-1]), rb), dtype=torch.uint8, device="cuda")
        vo = torch.empty_like(ko)
        U.ukv_gather_kv_layers(pair.gpu, sub, 0, 3, bt_d, to_dev(lens), to_dev(cu), win, ko, vo)
        for layer in range(3):
            eko = np.zeros((int(cu[-1]), rb), np.uint8)
            evo = np.zeros_like(eko)
            assert pair.orc.gather(sub, layer, bt, lens, cu, win, eko, evo) == frozenset()
            assert np.array_equal(ko[layer].cpu().numpy(), eko) and np.array_equal(vo[layer].cpu().numpy(), evo)
    # eviction clears exactly the oracle's entries; window reads are unchanged
    padded = W.padded_table(w.req_pages[0], pad=-1)
    U.ukv_evict_window(pair.gpu, map_d, to_dev(padded), to_dev(lens), w.window)
    assert pair.orc.evict_window(mapping, padded, lens, w.window) == frozenset()
    assert np.array_equal(map_d.cpu().numpy(), mapping)
    assert (mapping != w.swa_mapping).sum() > 0
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()


def test_debug_validation_refuses_racing_ids_before_launch():
    """With the pool's debug validation on, stores and moves whose ids would race are
    refused (UKV_ERR_RACE) before anything is launched, so the pool keeps every byte;
    ids that do not race (tombstones sharing the sink row included) run exactly as
    without it.  Only the non-racing calls reach the device."""
    w = W.tiny_mha(seed=0)
    pair = Pair(w.shapes, w.page_size)
    rb = pair.rb(0)
    U.ukv_pool_set_debug(pair.gpu, True)
    slots = w.store_slots[0]  # 34 live slots and 3 tombstones
    ids_d = U.ukv_translate_loc_for_kernel(pair.gpu, 0, to_dev(slots))
    ids, _ = pair.orc.translate(0, slots)
    k = bf16_rows(300, slots.size, rb)
    v = bf16_rows(301, slots.size, rb)
    U.ukv_store_kv(pair.gpu, 0, 1, ids_d, rows_dev(k), rows_dev(v))
    assert pair.orc.store(0, 1, ids, k, v) == frozenset()
    pair.record_store(0, 1, ids, k, v)
    pair.assert_pools_equal()
    before = pair.gpu.raw.clone()
    live = np.nonzero(ids != 0)[0]
    dup = ids.copy()
    dup[live[5]] = dup[live[20]]
    with pytest.raises(U.UkvError, match="UKV_ERR_RACE.*would race"):
        U.ukv_store_kv(pair.gpu, 0, 0, to_dev(dup), rows_dev(k), rows_dev(v))
    with pytest.raises(U.UkvError, match="UKV_ERR_RACE"):
        U.ukv_store_kv_layers(pair.gpu, 0, 0, 2, to_dev(dup), rows_dev(np.concatenate([k, k])).view(2, slots.size, -1),
                              rows_dev(np.concatenate([v, v])).view(2, slots.size, -1))
    src, _ = pair.orc.translate(0, w.move_src[0])
    dst, _ = pair.orc.translate(0, w.move_dst[0])
    overlap = dst.copy()
    overlap[3] = src[6]
    with pytest.raises(U.UkvError, match="UKV_ERR_RACE.*disjoint"):
        U.ukv_move_kv(pair.gpu, 0, to_dev(overlap), to_dev(src))
    with pytest.raises(U.UkvError, match="UKV_ERR_RACE"):
        U.ukv_move_pages(pair.gpu, 0, to_dev(np.array([3, 4, 3], np.int32)), to_dev(np.array([7, 8, 9], np.int32)))
    torch.cuda.synchronize()
    assert torch.equal(pair.gpu.raw, before), "a refused call wrote to the pool"
    U.ukv_move_kv(pair.gpu, 0, to_dev(dst), to_dev(src))  # disjoint: runs
    assert pair.orc.move(0, dst, src, 0, 2) == frozenset()
    U.ukv_pool_set_debug(pair.gpu, False)
    U.ukv_move_kv(pair.gpu, 0, to_dev(src), to_dev(dst))  # off again: no host copy, same result as the oracle
    assert pair.orc.move(0, src, dst, 0, 2) == frozenset()
    assert U.ukv_pool_error_flags(pair.gpu) == frozenset()
    pair.assert_pools_equal()
