"""CPU oracle for the unified page-major KV-cache pool.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the GPU library (``store_gather_amd``) and imports nothing from it.

Two independent statements of the layout live here:

* ``ukv_oracle.c`` (loaded through ctypes): byte-level envelope arithmetic,
  kernel-facing ids and the store / gather / move row copies, written from the
  report page "PR #34602: feat(unified-memory): dense KV views for uniform-row
  MHA/SWA models" (implementation steps 1-3 and its excerpts of
  unified_memory_pool.py, multi_ended_allocator.py and layout/page_major.py);
* ``strided.py``: the envelope as a nested numpy strided array
  ``(page, layer, kv, offset, row byte)``, the independent 4-D reference
  builder the same page's test file uses as its oracle.

Every function is pinned by ``tests/test_oracle_pins.py``; none is "parity
unpinned".
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

MHA = 0
MLA = 1
MAX_SUB = 8

CODE_NAMES = {
    0: "ok",
    -1: "invalid_arg",
    -2: "asymmetric_kv",
    -3: "kernel_id_bound",
    -4: "overflow",
    -5: "alignment",
    -6: "tail_pad",
}
FLAG_NAMES = {1: "slot_range", 2: "bad_id", 4: "bad_block", 8: "layout"}


def flag_names(bits: int) -> frozenset:
    return frozenset(name for bit, name in FLAG_NAMES.items() if bits & bit)


class _Spec(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("layer_num", ctypes.c_int32),
        ("head_num", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("v_head_dim", ctypes.c_int32),
        ("elem_bytes", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
    ]


class _SubPlan(ctypes.Structure):
    _fields_ = [
        ("row_bytes", ctypes.c_uint64),
        ("blocks_per_page", ctypes.c_uint64),
        ("page_bytes", ctypes.c_uint64),
        ("n_rows", ctypes.c_uint64),
        ("anchor_bytes", ctypes.c_uint64),
        ("envelope_bytes", ctypes.c_uint64),
        ("tail_pad_bytes", ctypes.c_uint64),
    ]


class _Pool(ctypes.Structure):
    _fields_ = [
        ("raw", ctypes.c_void_p),
        ("raw_bytes", ctypes.c_uint64),
        ("kind", ctypes.c_int32),
        ("layer_num", ctypes.c_int32),
        ("page_size", ctypes.c_int64),
        ("num_pages", ctypes.c_int64),
        ("sp", _SubPlan),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load liboracle.so, building it with gcc when it is not there yet."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build

            _build.build()
        L = ctypes.CDLL(_LIB_PATH)
        vp, i64, i32, u64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint64
        L.orc_plan.argtypes = [ctypes.POINTER(_Spec), ctypes.c_int, i64, ctypes.POINTER(_SubPlan), ctypes.POINTER(u64), ctypes.POINTER(u64)]
        L.orc_plan.restype = ctypes.c_int
        L.orc_view_base.argtypes = [ctypes.POINTER(_SubPlan), ctypes.c_int, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(u64)]
        L.orc_view_base.restype = ctypes.c_int
        L.orc_builder_check.argtypes = [ctypes.POINTER(_SubPlan), i64, u64, ctypes.POINTER(u64)]
        L.orc_builder_check.restype = ctypes.c_int
        L.orc_kernel_id.argtypes = [i64, i64, i64]
        L.orc_kernel_id.restype = i64
        L.orc_translate.argtypes = [vp, i64, i64, i64, i64, vp, i64, vp, ctypes.POINTER(ctypes.c_uint32)]
        L.orc_translate.restype = None
        L.orc_translate_pages.argtypes = [vp, i64, i64, i64, i64, vp, i64, vp, ctypes.POINTER(ctypes.c_uint32)]
        L.orc_translate_pages.restype = None
        L.orc_store.argtypes = [ctypes.POINTER(_Pool), ctypes.c_int, vp, i64, vp, vp, i64, ctypes.POINTER(ctypes.c_uint32)]
        L.orc_store.restype = None
        L.orc_gather.argtypes = [ctypes.POINTER(_Pool), ctypes.c_int, vp, i64, vp, vp, i32, i32, vp, vp, i64, ctypes.POINTER(ctypes.c_uint32)]
        L.orc_gather.restype = None
        L.orc_move.argtypes = [ctypes.POINTER(_Pool), vp, vp, i64, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_uint32)]
        L.orc_move.restype = ctypes.c_int
        L.orc_store_map.argtypes = [ctypes.POINTER(_Pool), ctypes.c_int, vp, i64, vp, vp, ctypes.POINTER(ctypes.c_uint32)]
        L.orc_store_map.restype = None
        L.orc_gather_map.argtypes = [ctypes.POINTER(_Pool), ctypes.c_int, vp, i64, vp, vp, i32, i32, i64, vp, vp,
                                     ctypes.POINTER(ctypes.c_uint32)]
        L.orc_gather_map.restype = None
        L.orc_move_map.argtypes = [ctypes.POINTER(_Pool), vp, vp, i64, ctypes.c_int, ctypes.c_int, vp, vp,
                                   ctypes.POINTER(ctypes.c_uint32)]
        L.orc_move_map.restype = None
        L.orc_translate_loc.argtypes = [vp, i64, i64, i64, vp, i64, vp, ctypes.POINTER(ctypes.c_uint32)]
        L.orc_translate_loc.restype = None
        L.orc_move_pages.argtypes = [ctypes.POINTER(_Pool), vp, vp, i64, ctypes.POINTER(ctypes.c_uint32)]
        L.orc_move_pages.restype = ctypes.c_int
        L.orc_remap_pages.argtypes = [vp, i64, vp, vp, i64, i64, ctypes.POINTER(ctypes.c_uint32)]
        L.orc_remap_pages.restype = None
        L.orc_evict_window.argtypes = [vp, i64, vp, i64, vp, i32, i32, i64, ctypes.POINTER(ctypes.c_uint32)]
        L.orc_evict_window.restype = None
        L.orc_build_page_table.argtypes = [vp, i64, vp, i32, i64, i64, i64, vp, i64, vp, ctypes.POINTER(ctypes.c_uint32)]
        L.orc_build_page_table.restype = None
        for fn in ("orc_sizeof_pool", "orc_sizeof_sub_plan", "orc_sizeof_spec"):
            getattr(L, fn).restype = ctypes.c_int
        assert L.orc_sizeof_pool() == ctypes.sizeof(_Pool)
        assert L.orc_sizeof_sub_plan() == ctypes.sizeof(_SubPlan)
        assert L.orc_sizeof_spec() == ctypes.sizeof(_Spec)
        _lib = L
    return _lib


@dataclass(frozen=True)
class Spec:
    """One sub-pool: MHA (K and V rows per layer) or MLA (one latent row per layer)."""

    kind: int
    layer_num: int
    head_num: int
    head_dim: int
    v_head_dim: int
    elem_bytes: int
    num_pages: int


@dataclass(frozen=True)
class SubPlan:
    row_bytes: int
    blocks_per_page: int
    page_bytes: int
    n_rows: int
    anchor_bytes: int
    envelope_bytes: int
    tail_pad_bytes: int


@dataclass(frozen=True)
class Plan:
    code: str
    subs: Tuple[SubPlan, ...] = ()
    tail_pad_bytes: int = 0
    required_bytes: int = 0


def plan(specs: Sequence[Spec], page_size: int) -> Plan:
    n = len(specs)
    arr = (_Spec * max(n, 1))()
    for i, s in enumerate(specs):
        arr[i] = _Spec(s.kind, s.layer_num, s.head_num, s.head_dim, s.v_head_dim, s.elem_bytes, s.num_pages)
    subs = (_SubPlan * MAX_SUB)()
    tail = ctypes.c_uint64(0)
    req = ctypes.c_uint64(0)
    rc = lib().orc_plan(arr, n, page_size, subs, ctypes.byref(tail), ctypes.byref(req))
    if rc != 0:
        return Plan(CODE_NAMES[rc])
    out = tuple(
        SubPlan(s.row_bytes, s.blocks_per_page, s.page_bytes, s.n_rows, s.anchor_bytes, s.envelope_bytes, s.tail_pad_bytes)
        for s in list(subs)[:n]
    )
    return Plan("ok", out, tail.value, req.value)


def kernel_id(t: int, page_size: int, multiplier: int) -> int:
    """kernel_id(t) = (t // ps) * (ps * multiplier) + t % ps, for t >= 0."""
    return int(lib().orc_kernel_id(t, page_size, multiplier))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def translate(slots, page_size, blocks_per_page, num_pages, v2p=None):
    """Token slots (int64) -> kernel-facing ids (int32), plus raised flag names."""
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    out = np.empty(slots.shape, dtype=np.int32)
    flags = ctypes.c_uint32(0)
    v = None if v2p is None else np.ascontiguousarray(v2p, dtype=np.int32)
    lib().orc_translate(_ptr(slots), slots.size, page_size, blocks_per_page, num_pages, _ptr(v),
                        0 if v is None else v.size, _ptr(out), ctypes.byref(flags))
    return out, flag_names(flags.value)


def translate_pages(pages, page_size, blocks_per_page, num_pages, v2p=None):
    """Page ids (int32) -> kernel-facing page indices of the dense views (int32), plus flags."""
    pages = np.ascontiguousarray(pages, dtype=np.int32)
    out = np.empty(pages.shape, dtype=np.int32)
    flags = ctypes.c_uint32(0)
    v = None if v2p is None else np.ascontiguousarray(v2p, dtype=np.int32)
    lib().orc_translate_pages(_ptr(pages), pages.size, page_size, blocks_per_page, num_pages, _ptr(v),
                              0 if v is None else v.size, _ptr(out), ctypes.byref(flags))
    return out, flag_names(flags.value)


class OraclePool:
    """A pool over a host uint8 buffer (the raw envelope + tail pad).

    ``raw`` may be ``None`` together with ``addresses_only=True``: the pool then
    only answers the *_map queries (byte offsets), which never touch the buffer,
    so pools of any size can be described without host memory."""

    def __init__(self, specs: Sequence[Spec], page_size: int, raw: Optional[np.ndarray] = None,
                 addresses_only: bool = False):
        self.specs = tuple(specs)
        self.page_size = page_size
        self.plan = plan(self.specs, page_size)
        if self.plan.code != "ok":
            raise ValueError(f"oracle plan rejected: {self.plan.code}")
        self.addresses_only = addresses_only
        if addresses_only:
            raw = None
        else:
            if raw is None:
                raw = np.zeros(self.plan.required_bytes, dtype=np.uint8)
            assert raw.dtype == np.uint8 and raw.ndim == 1 and raw.flags.c_contiguous
            assert raw.size >= self.plan.required_bytes
        self.raw = raw

    def _pool(self, sub: int) -> _Pool:
        s, sp = self.specs[sub], self.plan.subs[sub]
        # addresses-only pools: a null base, so row pointers are plain byte offsets
        base = 0 if self.raw is None else self.raw.ctypes.data
        size = self.plan.required_bytes if self.raw is None else self.raw.size
        return _Pool(base, size, s.kind, s.layer_num, self.page_size, s.num_pages,
                     _SubPlan(sp.row_bytes, sp.blocks_per_page, sp.page_bytes, sp.n_rows, sp.anchor_bytes,
                              sp.envelope_bytes, sp.tail_pad_bytes))

    def view_base(self, sub: int, layer: int, kv: int) -> int:
        s = self.specs[sub]
        sp = self._pool(sub).sp
        out = ctypes.c_uint64(0)
        rc = lib().orc_view_base(ctypes.byref(sp), s.kind, self.page_size, s.layer_num, layer, kv, ctypes.byref(out))
        if rc != 0:
            raise ValueError("bad (layer, kv)")
        return out.value

    def builder_check(self, sub: int, raw_bytes: int) -> Tuple[str, int]:
        sp = self._pool(sub).sp
        end = ctypes.c_uint64(0)
        rc = lib().orc_builder_check(ctypes.byref(sp), self.page_size, raw_bytes, ctypes.byref(end))
        return CODE_NAMES[rc], end.value

    def row_bytes(self, sub: int) -> int:
        return self.plan.subs[sub].row_bytes

    def translate(self, sub: int, slots, v2p=None):
        s, sp = self.specs[sub], self.plan.subs[sub]
        return translate(slots, self.page_size, sp.blocks_per_page, s.num_pages, v2p)

    def translate_pages(self, sub: int, pages, v2p=None):
        s, sp = self.specs[sub], self.plan.subs[sub]
        return translate_pages(pages, self.page_size, sp.blocks_per_page, s.num_pages, v2p)

    def translate_loc(self, sub: int, slots, v2p=None):
        """Token slots -> internal physical slot ids (int32; -1 for tombstones / unmapped)."""
        slots = np.ascontiguousarray(slots, dtype=np.int64)
        out = np.empty(slots.shape, dtype=np.int32)
        flags = ctypes.c_uint32(0)
        v = None if v2p is None else np.ascontiguousarray(v2p, dtype=np.int32)
        lib().orc_translate_loc(_ptr(slots), slots.size, self.page_size, self.specs[sub].num_pages, _ptr(v),
                                0 if v is None else v.size, _ptr(out), ctypes.byref(flags))
        return out, flag_names(flags.value)

    def move_pages(self, sub: int, dst_pages, src_pages):
        dst = np.ascontiguousarray(dst_pages, dtype=np.int32)
        src = np.ascontiguousarray(src_pages, dtype=np.int32)
        flags = ctypes.c_uint32(0)
        pool = self._pool(sub)
        rc = lib().orc_move_pages(ctypes.byref(pool), _ptr(dst), _ptr(src), dst.size, ctypes.byref(flags))
        if rc != 0:
            raise MemoryError("oracle page move")
        return flag_names(flags.value)

    def remap_pages(self, sub: int, v2p: np.ndarray, virt, phys):
        """In place on the int32 table ``v2p``."""
        assert v2p.dtype == np.int32 and v2p.flags.c_contiguous
        virt = np.ascontiguousarray(virt, dtype=np.int32)
        phys = np.ascontiguousarray(phys, dtype=np.int32)
        flags = ctypes.c_uint32(0)
        lib().orc_remap_pages(_ptr(v2p), v2p.size, _ptr(virt), _ptr(phys), virt.size, self.specs[sub].num_pages,
                              ctypes.byref(flags))
        return flag_names(flags.value)

    def build_page_table(self, sub: int, req_pages, prefix_lens, v2p=None):
        """Prefix-only kernel-facing page table [num_reqs, width] (int32), plus flags."""
        t = np.ascontiguousarray(req_pages, dtype=np.int32)
        lens = np.ascontiguousarray(prefix_lens, dtype=np.int32)
        out = np.empty(t.shape, dtype=np.int32)
        flags = ctypes.c_uint32(0)
        v = None if v2p is None else np.ascontiguousarray(v2p, dtype=np.int32)
        sp = self.plan.subs[sub]
        lib().orc_build_page_table(_ptr(t), t.shape[1], _ptr(lens), lens.size, self.page_size, sp.blocks_per_page,
                                   self.specs[sub].num_pages, _ptr(v), 0 if v is None else v.size, _ptr(out),
                                   ctypes.byref(flags))
        return out, flag_names(flags.value)

    def evict_window(self, mapping: np.ndarray, table, seq_lens, window: int):
        """In place on the int32 full-to-SWA page mapping."""
        assert mapping.dtype == np.int32 and mapping.flags.c_contiguous
        bt = np.ascontiguousarray(table, dtype=np.int32)
        if bt.ndim == 1:
            bt = bt.reshape(len(seq_lens), -1)
        lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        flags = ctypes.c_uint32(0)
        lib().orc_evict_window(_ptr(mapping), mapping.size, _ptr(bt), bt.shape[1], _ptr(lens), lens.size, window,
                               self.page_size, ctypes.byref(flags))
        return flag_names(flags.value)

    def store(self, sub: int, layer: int, ids, k: np.ndarray, v: Optional[np.ndarray]):
        """k, v: uint8 arrays of shape [n, row_bytes] (MLA: v is None)."""
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        rb = self.row_bytes(sub)
        k = np.ascontiguousarray(k, dtype=np.uint8).reshape(ids.size, rb)
        if v is not None:
            v = np.ascontiguousarray(v, dtype=np.uint8).reshape(ids.size, rb)
        flags = ctypes.c_uint32(0)
        pool = self._pool(sub)
        lib().orc_store(ctypes.byref(pool), layer, _ptr(ids), ids.size, _ptr(k), _ptr(v), rb, ctypes.byref(flags))
        return flag_names(flags.value)

    def gather(self, sub: int, layer: int, block_table: np.ndarray, seq_lens, cu_out, window: int,
               k_out: np.ndarray, v_out: Optional[np.ndarray]):
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        if bt.ndim == 1:
            bt = bt.reshape(len(seq_lens), -1)
        lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        cu = np.ascontiguousarray(cu_out, dtype=np.int64)
        assert k_out.dtype == np.uint8 and k_out.flags.c_contiguous
        out_rows = k_out.size // self.row_bytes(sub)
        flags = ctypes.c_uint32(0)
        pool = self._pool(sub)
        lib().orc_gather(ctypes.byref(pool), layer, _ptr(bt), bt.shape[1], _ptr(lens), _ptr(cu), lens.size,
                         window, _ptr(k_out), _ptr(v_out), out_rows, ctypes.byref(flags))
        return flag_names(flags.value)

    # -- address maps: byte offsets into raw, -1 for a skipped row --------------
    def store_map(self, sub: int, layer: int, ids):
        """(K offsets, V offsets or None, flags) of each store entry."""
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        k_off = np.empty(ids.size, np.int64)
        v_off = np.empty(ids.size, np.int64) if self.specs[sub].kind == MHA else None
        flags = ctypes.c_uint32(0)
        pool = self._pool(sub)
        lib().orc_store_map(ctypes.byref(pool), layer, _ptr(ids), ids.size, _ptr(k_off), _ptr(v_off),
                            ctypes.byref(flags))
        return k_off, v_off, flag_names(flags.value)

    def gather_map(self, sub: int, layer: int, block_table, seq_lens, cu_out, window: int, out_rows: int):
        """(K source offsets, V source offsets or None, flags) of every output row."""
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        if bt.ndim == 1:
            bt = bt.reshape(len(seq_lens), -1)
        lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        cu = np.ascontiguousarray(cu_out, dtype=np.int64)
        k_src = np.empty(out_rows, np.int64)
        v_src = np.empty(out_rows, np.int64) if self.specs[sub].kind == MHA else None
        flags = ctypes.c_uint32(0)
        pool = self._pool(sub)
        lib().orc_gather_map(ctypes.byref(pool), layer, _ptr(bt), bt.shape[1], _ptr(lens), _ptr(cu), lens.size,
                             window, out_rows, _ptr(k_src), _ptr(v_src), ctypes.byref(flags))
        return k_src, v_src, flag_names(flags.value)

    def move_map(self, sub: int, dst, src, layer_begin: int, layer_end: int):
        """(dst offsets, src offsets, flags) for every (layer, kv, pair), in that order."""
        dst = np.ascontiguousarray(dst, dtype=np.int32)
        src = np.ascontiguousarray(src, dtype=np.int32)
        kvs = 2 if self.specs[sub].kind == MHA else 1
        total = dst.size * (layer_end - layer_begin) * kvs
        d_off = np.empty(total, np.int64)
        s_off = np.empty(total, np.int64)
        flags = ctypes.c_uint32(0)
        pool = self._pool(sub)
        lib().orc_move_map(ctypes.byref(pool), _ptr(dst), _ptr(src), dst.size, layer_begin, layer_end, _ptr(d_off),
                           _ptr(s_off), ctypes.byref(flags))
        return d_off, s_off, flag_names(flags.value)

    def move(self, sub: int, dst, src, layer_begin: int, layer_end: int):
        dst = np.ascontiguousarray(dst, dtype=np.int32)
        src = np.ascontiguousarray(src, dtype=np.int32)
        assert dst.size == src.size
        flags = ctypes.c_uint32(0)
        pool = self._pool(sub)
        rc = lib().orc_move(ctypes.byref(pool), _ptr(dst), _ptr(src), dst.size, layer_begin, layer_end,
                            ctypes.byref(flags))
        if rc != 0:
            raise MemoryError("oracle move snapshot")
        return flag_names(flags.value)


__all__ = [
    "MHA", "MLA", "Spec", "SubPlan", "Plan", "plan", "kernel_id", "translate", "translate_pages",
    "OraclePool", "flag_names", "CODE_NAMES", "FLAG_NAMES",
]
