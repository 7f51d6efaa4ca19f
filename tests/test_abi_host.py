"""Host-side checks of the C-ABI library (no GPU): it loads, exports every
symbol include/ukv.h declares, and its pure-host plan and view arithmetic
agrees with the oracle, rejections included."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import store_gather_amd as U
import ukv_workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

ORACLE_TO_STATUS = {
    "ok": "UKV_OK",
    "invalid_arg": "UKV_ERR_INVALID_ARG",
    "asymmetric_kv": "UKV_ERR_ASYMMETRIC_KV",
    "kernel_id_bound": "UKV_ERR_KERNEL_ID_BOUND",
    "overflow": "UKV_ERR_OVERFLOW",
    "alignment": "UKV_ERR_ALIGNMENT",
    "tail_pad": "UKV_ERR_TAIL_PAD",
}


def header_functions():
    text = open(os.path.join(ROOT, "include", "ukv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ukv_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = header_functions()
    assert len(names) >= 14
    lib = ctypes.CDLL(U.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(U.EXPORTS)


def test_status_names_match_header():
    text = open(os.path.join(ROOT, "include", "ukv.h")).read()
    for name, val in re.findall(r"#define (UKV_(?:OK|ERR_[A-Z_]+))\s+(-?\d+)", text):
        assert U.STATUS[int(val)] == name
        assert U.lib().ukv_status_name(int(val)).decode() == name
    for name, val in re.findall(r"#define UKV_FLAG_([A-Z_]+)\s+(\d+)u", text):
        assert U.FLAGS[int(val)] == name.lower()


def _ospec(s):
    return oracle.Spec(s.kind, s.layer_num, s.head_num, s.head_dim, s.v_head_dim, s.elem_bytes, s.num_pages)


def _compare(specs, ps):
    o = oracle.plan([_ospec(s) for s in specs], ps)
    status = U.plan_status(specs, ps)
    assert status == ORACLE_TO_STATUS[o.code], (specs, ps, status, o.code)
    if o.code != "ok":
        return None
    p = U.ukv_pool_plan(specs, ps)
    assert p.n_sub == len(specs) and p.page_size == ps
    assert p.required_bytes == o.required_bytes
    assert p.tail_pad_bytes == o.tail_pad_bytes
    for i, (a, b) in enumerate(zip(p.sub, o.subs)):
        assert (a.row_bytes, a.blocks_per_page, a.page_bytes, a.n_rows, a.anchor_bytes, a.envelope_bytes,
                a.tail_pad_bytes) == (b.row_bytes, b.blocks_per_page, b.page_bytes, b.n_rows, b.anchor_bytes,
                                      b.envelope_bytes, b.tail_pad_bytes), i
    return p


WORKLOAD_SHAPES = [
    ("tiny", [W.mha(2, 2, 8, 16)], 4),
    ("decode_8b", [W.mha(32, 8, 128, 4096)], 16),
    ("prefill_8b", [W.mha(32, 8, 128, 16384)], 16),
    ("hybrid", [W.mha(24, 8, 64, 16538), W.mla(24, 16538)], 64),
    ("move_70b", [W.mha(80, 8, 128, 32768)], 16),
    ("bound_ok_70b", [W.mha(80, 8, 128, 838860)], 16),
    ("bound_reject_70b", [W.mha(80, 8, 128, 838861)], 16),
    ("bound_reject_8b", [W.mha(32, 8, 128, 1 << 21)], 16),
    ("asym", [W.mha(2, 8, 192, 4, v_head_dim=128)], 16),
    ("mla_only", [W.mla(61, 100)], 64),
    ("fp8_rows", [W.mha(3, 1, 7, 5, elem_bytes=1), W.mha(2, 2, 4, 3, elem_bytes=2)], 3),
]


@pytest.mark.parametrize("name,specs,ps", WORKLOAD_SHAPES, ids=[w[0] for w in WORKLOAD_SHAPES])
def test_plan_matches_oracle_on_workload_shapes(name, specs, ps):
    _compare(specs, ps)


def test_plan_matches_oracle_fuzz():
    g = np.random.default_rng(123)
    for _ in range(2000):
        n = int(g.integers(1, 4))
        specs = []
        for _ in range(n):
            kind = int(g.integers(0, 2))
            hd = int(g.integers(1, 300))
            specs.append(W.SubPoolShape(kind, int(g.integers(0, 100)), int(g.integers(0, 20)), hd,
                                        hd if g.random() < 0.9 else int(g.integers(1, 300)),
                                        int(g.choice([1, 2, 3, 4, 8])), int(g.integers(0, 1 << int(g.integers(1, 24))))))
        _compare(specs, int(g.integers(0, 130)))


def test_views_match_oracle():
    for specs, ps in (([W.mha(2, 2, 8, 16)], 4), ([W.mha(24, 8, 64, 50), W.mla(24, 50)], 64),
                      ([W.mha(3, 1, 7, 5, elem_bytes=1), W.mha(2, 2, 4, 3)], 3)):
        p = U.ukv_pool_plan(specs, ps)
        o = oracle.OraclePool([_ospec(s) for s in specs], ps, raw=np.zeros(oracle.plan([_ospec(s) for s in specs], ps).required_bytes, np.uint8))
        for sub, s in enumerate(specs):
            for layer in range(s.layer_num):
                for kv in range(2 if s.kind == W.MHA else 1):
                    v = U.ukv_plan_view(p, specs, sub, layer, kv)
                    assert v.byte_offset == o.view_base(sub, layer, kv)
                    assert v.n_rows == p.sub[sub].n_rows
                    assert (v.head_num, v.head_dim, v.elem_bytes) == (s.head_num, s.head_dim, s.elem_bytes)
                    assert list(v.stride_elems) == [s.head_num * s.head_dim, s.head_dim, 1]
            with pytest.raises(U.UkvError):
                U.ukv_plan_view(p, specs, sub, s.layer_num, 0)
            with pytest.raises(U.UkvError):
                U.ukv_plan_view(p, specs, sub, 0, 2 if s.kind == W.MHA else 1)


def test_rejection_messages_are_readable():
    with pytest.raises(U.UkvError) as e:
        U.ukv_pool_plan([W.mha(2, 8, 192, 4, v_head_dim=128)], 16)
    msg = str(e.value)
    assert e.value.status == "UKV_ERR_ASYMMETRIC_KV"
    assert all(x in msg for x in ("head_num=8", "head_dim=192", "v_head_dim=128"))
    with pytest.raises(U.UkvError) as e:
        U.ukv_pool_plan([W.mha(80, 8, 128, 838861)], 16)
    assert e.value.status == "UKV_ERR_KERNEL_ID_BOUND" and "2^31" in str(e.value)


def test_bound_check_needs_no_allocation():
    """The 70B-shape bound check runs on the host only: a pool that would need
    4 PiB plans to a rejection without touching any device."""
    assert U.plan_status([W.mha(80, 8, 128, 838861)], 16) == "UKV_ERR_KERNEL_ID_BOUND"
    p = U.ukv_pool_plan([W.mha(80, 8, 128, 838860)], 16)
    assert p.sub[0].n_rows == 2147481600 and p.required_bytes == (838860 + 1) * 5 * 1024 * 1024


def test_create_rejects_without_device_work():
    """Argument errors are reported before any device call."""
    specs = U._specs_array([W.mha(2, 2, 8, 16)])
    h = ctypes.c_void_p()
    assert U.lib().ukv_pool_create(specs, 1, 4, None, 1 << 20, ctypes.byref(h)) == -1
    assert U.lib().ukv_pool_create(specs, 1, 4, ctypes.c_void_p(0x1008), 1 << 20, ctypes.byref(h)) == -5
    assert U.lib().ukv_pool_create(specs, 1, 4, ctypes.c_void_p(0x1000), 8192, ctypes.byref(h)) == -6
    assert "8704" in U.ukv_last_error()
    assert h.value is None
    assert U.lib().ukv_store_kv(None, 0, 0, None, 0, None, None, 0, None) == -1
    assert U.lib().ukv_pool_destroy(None) == 0
