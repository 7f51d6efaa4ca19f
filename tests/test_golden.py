"""The oracle and the library's host plan against pool geometry worked by hand
from the pages' closed forms (tests/golden/geometry.txt, which cites its
passages: the envelope and kernel_id of the dense-KV-views page's
implementation step 1, the spec-derived tail pad, blocks per page and row
bound of step 2, and the row count of its risk item 5)."""
import os
from collections import defaultdict

import pytest

import oracle
import store_gather_amd as U
import ukv_workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "geometry.txt")


def _records():
    recs = defaultdict(list)
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].split()
            if line:
                recs[line[0]].append(line[1:])
    return recs


REC = _records()


def _pools():
    """pool name -> (page size, [(kind, L, H, D, P, expected sub-plan fields)])"""
    subs = defaultdict(list)
    for name, kind, L, H, D, ps, P, *rest in REC["sub"]:
        subs[name].append((kind, int(L), int(H), int(D), int(ps), int(P), [int(x) for x in rest]))
    return subs


POOLS = _pools()


def _specs(name):
    rows = POOLS[name]
    o, lib = [], []
    for kind, L, H, D, ps, P, _ in rows:
        if kind == "mha":
            o.append(oracle.Spec(oracle.MHA, L, H, D, D, 2, P))
            lib.append(W.mha(L, H, D, P))
        else:
            o.append(oracle.Spec(oracle.MLA, L, H, D, 0, 2, P))
            lib.append(W.mla(L, P))
    return o, lib, rows[0][4]


def test_golden_file_is_complete():
    assert len(REC["sub"]) == 7 and len(REC["pool"]) == 7
    assert len(REC["kid"]) >= 10 and len(REC["addr"]) >= 6


@pytest.mark.parametrize("name", sorted(POOLS))
def test_sub_pool_geometry(name):
    ospecs, lspecs, ps = _specs(name)
    o = oracle.plan(ospecs, ps)
    lp = U.ukv_pool_plan(lspecs, ps)
    pool = oracle.OraclePool(ospecs, ps, addresses_only=True)
    for sub, (kind, L, H, D, _, P, exp) in enumerate(POOLS[name]):
        rb, bpp, page_bytes, n_rows, anchor, envelope, overrun = exp
        for got in (o.subs[sub], lp.sub[sub]):
            assert (got.row_bytes, got.blocks_per_page, got.page_bytes, got.n_rows, got.anchor_bytes,
                    got.envelope_bytes) == (rb, bpp, page_bytes, n_rows, anchor, envelope)
        last_kv = 1 if kind == "mha" else 0
        end = pool.view_base(sub, L - 1, last_kv) + n_rows * rb
        assert end - (anchor + envelope) == overrun
        v = U.ukv_plan_view(lp, lspecs, sub, L - 1, last_kv)
        assert v.byte_offset + n_rows * rb - (anchor + envelope) == overrun


@pytest.mark.parametrize("rec", REC["pool"], ids=[r[0] for r in REC["pool"]])
def test_pool_tail_pad_required_and_status(rec):
    name, ps, tail, required, status = rec
    if name in POOLS:
        ospecs, lspecs, _ = _specs(name)
    else:  # the rejected 70B shape: one page past the largest accepted count
        assert name == "bound_reject_70b"
        ospecs = [oracle.Spec(oracle.MHA, 80, 8, 128, 128, 2, 838861)]
        lspecs = [W.mha(80, 8, 128, 838861)]
    o = oracle.plan(ospecs, int(ps))
    assert o.code == status
    if status != "ok":
        assert U.plan_status(lspecs, int(ps)) == "UKV_ERR_KERNEL_ID_BOUND"
        return
    lp = U.ukv_pool_plan(lspecs, int(ps))
    assert (o.tail_pad_bytes, o.required_bytes) == (int(tail), int(required))
    assert (lp.tail_pad_bytes, lp.required_bytes) == (int(tail), int(required))


@pytest.mark.parametrize("rec", REC["kid"], ids=[f"{r[0]}-{r[2]}" for r in REC["kid"]])
def test_worked_kernel_ids(rec):
    name, sub, t, kid = rec[0], int(rec[1]), int(rec[2]), int(rec[3])
    ospecs, _, ps = _specs(name)
    pool = oracle.OraclePool(ospecs, ps, addresses_only=True)
    ids, flags = pool.translate(sub, [t])
    assert int(ids[0]) == kid and not flags
    if t >= 0:
        assert oracle.kernel_id(t, ps, pool.plan.subs[sub].blocks_per_page) == kid


@pytest.mark.parametrize("rec", REC["addr"], ids=[f"{r[0]}-{r[2]}-{r[3]}-{r[4]}" for r in REC["addr"]])
def test_worked_row_addresses(rec):
    name, sub, t, layer, kv, addr = rec[0], *map(int, rec[1:])
    ospecs, lspecs, ps = _specs(name)
    pool = oracle.OraclePool(ospecs, ps, addresses_only=True)
    rb = pool.plan.subs[sub].row_bytes
    kid = int(pool.translate(sub, [t])[0][0])
    assert pool.view_base(sub, layer, kv) + kid * rb == addr
    lp = U.ukv_pool_plan(lspecs, ps)
    assert U.ukv_plan_view(lp, lspecs, sub, layer, kv).byte_offset + kid * rb == addr
