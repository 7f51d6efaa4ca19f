"""Python binding of libukv (include/ukv.h): argument marshalling only.

Every step of the path (translate, store, gather, move) runs in the HIP
kernels of libukv.so; this module checks tensors, passes their device
pointers and the current torch stream, and turns status codes into
exceptions.  torch supplies device memory and streams.  There is no
fallback: importing this package without a built libukv.so raises.

The method is the unified page-major KV pool of the report page "PR #34602:
feat(unified-memory): dense KV views for uniform-row MHA/SWA models"; the
entry points mirror the C names.
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, Optional, Sequence

import torch  # loads the HIP runtime libukv shares with torch (same soname)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libukv.so")

UKV_MHA = 0
UKV_MLA = 1
UKV_MAX_SUB = 8

STATUS = {
    0: "UKV_OK",
    -1: "UKV_ERR_INVALID_ARG",
    -2: "UKV_ERR_ASYMMETRIC_KV",
    -3: "UKV_ERR_KERNEL_ID_BOUND",
    -4: "UKV_ERR_OVERFLOW",
    -5: "UKV_ERR_ALIGNMENT",
    -6: "UKV_ERR_TAIL_PAD",
    -7: "UKV_ERR_HIP",
    -8: "UKV_ERR_RACE",
}
FLAGS = {1: "slot_range", 2: "bad_id", 4: "bad_block", 8: "layout"}

EXPORTS = (
    "ukv_pool_plan", "ukv_pool_create", "ukv_pool_destroy", "ukv_pool_get_plan", "ukv_pool_view", "ukv_plan_view",
    "ukv_translate_loc_for_kernel", "ukv_translate_pages_for_kernel", "ukv_store_kv", "ukv_store_kv_layers",
    "ukv_gather_kv", "ukv_gather_kv_layers", "ukv_move_kv", "ukv_pool_error_flags", "ukv_last_error",
    "ukv_status_name", "ukv_translate_loc", "ukv_move_pages", "ukv_remap_pages", "ukv_evict_window",
    "ukv_build_page_table", "ukv_decode_attention", "ukv_decode_attention_workspace_bytes",
    "ukv_mla_decode_attention", "ukv_mla_decode_attention_workspace_bytes", "ukv_decode_attention_noalloc",
    "ukv_check_store_ids", "ukv_check_move_ids", "ukv_pool_set_debug",
)


class UkvError(RuntimeError):
    def __init__(self, code: int, message: str):
        self.code = code
        self.status = STATUS.get(code, f"UKV_ERR_{code}")
        super().__init__(f"{self.status}: {message}")


class SubpoolSpec(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32), ("layer_num", ctypes.c_int32), ("head_num", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("v_head_dim", ctypes.c_int32), ("elem_bytes", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
    ]


class SubpoolPlan(ctypes.Structure):
    _fields_ = [
        ("row_bytes", ctypes.c_uint64), ("blocks_per_page", ctypes.c_int64), ("page_bytes", ctypes.c_uint64),
        ("n_rows", ctypes.c_int64), ("anchor_bytes", ctypes.c_uint64), ("envelope_bytes", ctypes.c_uint64),
        ("tail_pad_bytes", ctypes.c_uint64),
    ]


class Plan(ctypes.Structure):
    _fields_ = [
        ("n_sub", ctypes.c_int32), ("reserved", ctypes.c_int32), ("page_size", ctypes.c_int64),
        ("envelope_bytes", ctypes.c_uint64), ("tail_pad_bytes", ctypes.c_uint64),
        ("required_bytes", ctypes.c_uint64), ("sub", SubpoolPlan * UKV_MAX_SUB),
    ]


class View(ctypes.Structure):
    _fields_ = [
        ("byte_offset", ctypes.c_uint64), ("n_rows", ctypes.c_int64), ("head_num", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("elem_bytes", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("row_bytes", ctypes.c_uint64), ("stride_elems", ctypes.c_int64 * 3),
    ]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libukv.so is not built ({LIB_PATH}); run `python store_gather_amd/build.py` "
            "(there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
    P = ctypes.POINTER
    sigs = {
        "ukv_pool_plan": [P(SubpoolSpec), i32, i64, P(Plan)],
        "ukv_pool_create": [P(SubpoolSpec), i32, i64, vp, u64, P(vp)],
        "ukv_pool_destroy": [vp],
        "ukv_pool_get_plan": [vp, P(Plan)],
        "ukv_pool_view": [vp, i32, i32, i32, P(View)],
        "ukv_plan_view": [P(Plan), P(SubpoolSpec), i32, i32, i32, P(View)],
        "ukv_translate_loc_for_kernel": [vp, i32, vp, i64, vp, i64, vp, vp],
        "ukv_translate_pages_for_kernel": [vp, i32, vp, i64, vp, i64, vp, vp],
        "ukv_store_kv": [vp, i32, i32, vp, i64, vp, vp, i64, vp],
        "ukv_store_kv_layers": [vp, i32, i32, i32, i32, vp, i64, vp, vp, i64, i64, vp],
        "ukv_gather_kv": [vp, i32, i32, vp, i64, vp, vp, i32, i32, vp, vp, i64, vp],
        "ukv_gather_kv_layers": [vp, i32, i32, i32, i32, vp, i64, vp, vp, i32, i32, vp, vp, i64, i64, vp],
        "ukv_move_kv": [vp, i32, vp, vp, i64, i32, i32, vp],
        "ukv_pool_error_flags": [vp, vp, P(ctypes.c_uint32)],
        "ukv_translate_loc": [vp, i32, vp, i64, vp, i64, vp, vp],
        "ukv_move_pages": [vp, i32, vp, vp, i64, vp],
        "ukv_remap_pages": [vp, i32, vp, i64, vp, vp, i64, vp],
        "ukv_evict_window": [vp, vp, i64, vp, i64, vp, i32, i32, vp],
        "ukv_build_page_table": [vp, i32, vp, i64, vp, i32, vp, i64, vp, vp],
        "ukv_decode_attention": [vp, i32, i32, vp, i32, vp, i64, vp, i32, i32, i32, ctypes.c_float, vp, vp, u64, vp],
        "ukv_decode_attention_noalloc": [vp, i32, i32, vp, i32, vp, i64, vp, i32, i32, i32, ctypes.c_float, vp, vp],
        "ukv_check_store_ids": [vp, i64],
        "ukv_check_move_ids": [vp, vp, i64],
        "ukv_pool_set_debug": [vp, i32],
        "ukv_mla_decode_attention": [vp, i32, i32, vp, i32, i32, vp, i64, vp, i32, i32, i32, ctypes.c_float, vp, vp,
                                     u64, vp],
    }
    for name, args in sigs.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.ukv_decode_attention_workspace_bytes.argtypes = [vp, i32, i32, i32, i32, i32]
    L.ukv_decode_attention_workspace_bytes.restype = u64
    L.ukv_mla_decode_attention_workspace_bytes.argtypes = [vp, i32, i32, i32, i32, i32, i32]
    L.ukv_mla_decode_attention_workspace_bytes.restype = u64
    L.ukv_last_error.argtypes = []
    L.ukv_last_error.restype = ctypes.c_char_p
    L.ukv_status_name.argtypes = [ctypes.c_int]
    L.ukv_status_name.restype = ctypes.c_char_p
    return L


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def ukv_last_error() -> str:
    return _lib.ukv_last_error().decode()


def _check(rc: int) -> None:
    if rc != 0:
        raise UkvError(rc, ukv_last_error())


def _specs_array(specs: Sequence) -> "ctypes.Array":
    arr = (SubpoolSpec * max(1, len(specs)))()
    for i, s in enumerate(specs):
        arr[i] = SubpoolSpec(int(s.kind), int(s.layer_num), int(s.head_num), int(s.head_dim), int(s.v_head_dim),
                             int(s.elem_bytes), int(s.num_pages))
    return arr


def ukv_check_store_ids(ids) -> None:
    """Host-side race check of a store's kernel-facing ids (numpy int32): raises
    UkvError(UKV_ERR_RACE) when two entries other than the sink row 0 name one row."""
    import numpy as np

    a = np.ascontiguousarray(ids, dtype=np.int32)
    _check(_lib.ukv_check_store_ids(a.ctypes.data if a.size else None, a.size))


def ukv_check_move_ids(dst, src) -> None:
    """Host-side race check of a move's ids: dst distinct, src and dst disjoint."""
    import numpy as np

    d = np.ascontiguousarray(dst, dtype=np.int32)
    s_ = np.ascontiguousarray(src, dtype=np.int32)
    if d.size != s_.size:
        raise ValueError("dst and src differ in length")
    _check(_lib.ukv_check_move_ids(d.ctypes.data if d.size else None, s_.ctypes.data if s_.size else None, d.size))


def ukv_pool_plan(specs: Sequence, page_size: int) -> Plan:
    """Spec arithmetic and the start-up gates; raises UkvError on a rejection."""
    out = Plan()
    _check(_lib.ukv_pool_plan(_specs_array(specs), len(specs), int(page_size), ctypes.byref(out)))
    return out


def plan_status(specs: Sequence, page_size: int) -> str:
    """Status name of ukv_pool_plan for these specs ("UKV_OK" when accepted)."""
    out = Plan()
    return STATUS[_lib.ukv_pool_plan(_specs_array(specs), len(specs), int(page_size), ctypes.byref(out))]


def _stream_handle(stream: Optional[torch.cuda.Stream]) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev_ptr(t: Optional[torch.Tensor], name: str, device: torch.device, dtype=None) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a tensor on {device}, got {t.device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


class Pool:
    """A pool handle over a device uint8 buffer; keeps the buffer alive."""

    def __init__(self, handle: int, raw: torch.Tensor, specs: Sequence, page_size: int):
        self.handle = ctypes.c_void_p(handle)
        self.raw = raw
        self.specs = tuple(specs)
        self.page_size = int(page_size)
        self.plan = Plan()
        _check(_lib.ukv_pool_get_plan(self.handle, ctypes.byref(self.plan)))
        self.device = raw.device

    def row_bytes(self, sub: int) -> int:
        return int(self.plan.sub[sub].row_bytes)

    def close(self) -> None:
        if self.handle is not None and self.handle.value:
            _check(_lib.ukv_pool_destroy(self.handle))
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def ukv_pool_create(specs: Sequence, page_size: int, raw: torch.Tensor) -> Pool:
    """Pool over the caller's device buffer ``raw`` (uint8, contiguous)."""
    if raw.dtype != torch.uint8 or not raw.is_contiguous() or not raw.is_cuda:
        raise ValueError("raw must be a contiguous uint8 CUDA tensor")
    h = ctypes.c_void_p()
    with torch.cuda.device(raw.device):
        _check(_lib.ukv_pool_create(_specs_array(specs), len(specs), int(page_size), raw.data_ptr(), raw.numel(),
                                    ctypes.byref(h)))
    return Pool(h.value, raw, specs, page_size)


def allocate_pool(specs: Sequence, page_size: int, device="cuda", extra_bytes: int = 0) -> Pool:
    """Allocate exactly the planned bytes (envelopes + tail pad) with torch and create the pool."""
    plan = ukv_pool_plan(specs, page_size)
    raw = torch.empty(int(plan.required_bytes) + extra_bytes, dtype=torch.uint8, device=device)
    return ukv_pool_create(specs, page_size, raw)


def ukv_pool_destroy(pool: Pool) -> None:
    pool.close()


def ukv_pool_view(pool: Pool, sub: int, layer: int, kv: int) -> View:
    out = View()
    _check(_lib.ukv_pool_view(pool.handle, sub, layer, kv, ctypes.byref(out)))
    return out


def ukv_plan_view(plan: Plan, specs: Sequence, sub: int, layer: int, kv: int) -> View:
    """View of (sub, layer, kv) computed from a plan alone (host only)."""
    out = View()
    _check(_lib.ukv_plan_view(ctypes.byref(plan), _specs_array(specs), sub, layer, kv, ctypes.byref(out)))
    return out


def dense_view(pool: Pool, sub: int, layer: int, kv: int, dtype: torch.dtype) -> torch.Tensor:
    """The (n_rows, head_num, head_dim) tensor view of (sub, layer, kv) over the raw buffer."""
    v = ukv_pool_view(pool, sub, layer, kv)
    item = torch.empty((), dtype=dtype).element_size()
    assert item == v.elem_bytes and v.byte_offset % item == 0
    return torch.as_strided(pool.raw.view(dtype), (v.n_rows, v.head_num, v.head_dim),
                            tuple(v.stride_elems), v.byte_offset // item)


def ukv_translate_loc_for_kernel(pool: Pool, sub: int, slots: torch.Tensor, v2p: Optional[torch.Tensor] = None,
                                 out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """int64 token slots -> int32 kernel-facing ids (launched on the current stream)."""
    d = pool.device
    _dev_ptr(slots, "slots", d, torch.int64)
    if not slots.is_contiguous():
        raise ValueError("slots must be contiguous")
    if out is None:
        out = torch.empty(slots.shape, dtype=torch.int32, device=d)
    _dev_ptr(out, "out", d, torch.int32)
    if out.numel() != slots.numel() or not out.is_contiguous():
        raise ValueError("out must be a contiguous int32 tensor of slots' size")
    vp = _dev_ptr(v2p, "v2p", d, torch.int32)
    _check(_lib.ukv_translate_loc_for_kernel(pool.handle, sub, slots.data_ptr(), slots.numel(), vp,
                                             0 if v2p is None else v2p.numel(), out.data_ptr(),
                                             _stream_handle(stream)))
    return out


def ukv_translate_pages_for_kernel(pool: Pool, sub: int, pages: torch.Tensor, v2p: Optional[torch.Tensor] = None,
                                   out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """int32 page ids -> int32 block-table entries of the dense views."""
    d = pool.device
    _dev_ptr(pages, "pages", d, torch.int32)
    if not pages.is_contiguous():
        raise ValueError("pages must be contiguous")
    if out is None:
        out = torch.empty(pages.shape, dtype=torch.int32, device=d)
    _dev_ptr(out, "out", d, torch.int32)
    if out.numel() != pages.numel() or not out.is_contiguous():
        raise ValueError("out must be a contiguous int32 tensor of pages' size")
    vp = _dev_ptr(v2p, "v2p", d, torch.int32)
    _check(_lib.ukv_translate_pages_for_kernel(pool.handle, sub, pages.data_ptr(), pages.numel(), vp,
                                               0 if v2p is None else v2p.numel(), out.data_ptr(),
                                               _stream_handle(stream)))
    return out


def _rows_arg(t: Optional[torch.Tensor], name: str, n: int, row_bytes: int, d) -> tuple:
    """(pointer, row stride in bytes) of an [n, ...] tensor whose rows are contiguous."""
    if t is None:
        return None, 0
    _dev_ptr(t, name, d)
    if t.shape[0] != n:
        raise ValueError(f"{name} has {t.shape[0]} rows, expected {n}")
    row = t[0] if n > 0 else t
    if n > 0 and (not row.is_contiguous() or row.numel() * t.element_size() != row_bytes):
        raise ValueError(f"each row of {name} must be {row_bytes} contiguous bytes")
    return t.data_ptr(), t.stride(0) * t.element_size()


def ukv_store_kv(pool: Pool, sub: int, layer: int, ids: torch.Tensor, k: torch.Tensor,
                 v: Optional[torch.Tensor] = None, stream=None) -> None:
    """K_view[layer][ids] = k and V_view[layer][ids] = v (MLA: k is the latent, v None)."""
    d = pool.device
    _dev_ptr(ids, "ids", d, torch.int32)
    if not ids.is_contiguous():
        raise ValueError("ids must be contiguous")
    n = ids.numel()
    rb = pool.row_bytes(sub)
    kp, ks = _rows_arg(k, "k", n, rb, d)
    vpt, vs = _rows_arg(v, "v", n, rb, d)
    if v is not None and vs != ks:
        raise ValueError("k and v must share one row stride")
    _check(_lib.ukv_store_kv(pool.handle, sub, layer, ids.data_ptr(), n, kp, vpt, ks if n else rb,
                             _stream_handle(stream)))


def ukv_store_kv_layers(pool: Pool, sub: int, layer_begin: int, layer_count: int, ids: torch.Tensor,
                        k: torch.Tensor, v: Optional[torch.Tensor] = None, layer_step: int = 1, stream=None) -> None:
    """Store on layers layer_begin + i*layer_step (i < layer_count) in one launch; k / v are
    [layer_count, n, ...] with each layer's rows contiguous (MLA: v None)."""
    d = pool.device
    _dev_ptr(ids, "ids", d, torch.int32)
    if not ids.is_contiguous():
        raise ValueError("ids must be contiguous")
    n = ids.numel()
    rb = pool.row_bytes(sub)
    for name, t in (("k", k), ("v", v)):
        if t is not None and (t.dim() < 2 or t.shape[0] != layer_count):
            raise ValueError(f"{name} must be [layer_count, n, ...]")
    if layer_count == 0 or n == 0:
        return
    _, ks = _rows_arg(k[0], "k", n, rb, d)
    vs = _rows_arg(v[0], "v", n, rb, d)[1] if v is not None else ks
    if vs != ks:
        raise ValueError("k and v must share one row stride")
    kl = k.stride(0) * k.element_size()
    if v is not None and v.stride(0) * v.element_size() != kl:
        raise ValueError("k and v must share one layer stride")
    _check(_lib.ukv_store_kv_layers(pool.handle, sub, layer_begin, layer_count, layer_step, ids.data_ptr(), n,
                                    k.data_ptr(), None if v is None else v.data_ptr(), ks, kl,
                                    _stream_handle(stream)))


def ukv_gather_kv(pool: Pool, sub: int, layer: int, block_table: torch.Tensor, seq_lens: torch.Tensor,
                  cu_out: torch.Tensor, window: int, k_out: torch.Tensor, v_out: Optional[torch.Tensor] = None,
                  stream=None) -> None:
    """Gather each request's rows (all, or its last ``window``) into contiguous k_out / v_out."""
    d = pool.device
    _dev_ptr(block_table, "block_table", d, torch.int32)
    _dev_ptr(seq_lens, "seq_lens", d, torch.int32)
    _dev_ptr(cu_out, "cu_out", d, torch.int64)
    if block_table.dim() != 2 or (block_table.numel() > 0 and block_table.stride(1) != 1):
        raise ValueError("block_table must be [num_reqs, width] with unit inner stride")
    num_reqs = seq_lens.numel()
    if block_table.shape[0] != num_reqs or cu_out.numel() != num_reqs + 1:
        raise ValueError("block_table rows / cu_out size do not match seq_lens")
    if not (seq_lens.is_contiguous() and cu_out.is_contiguous()):
        raise ValueError("seq_lens and cu_out must be contiguous")
    rb = pool.row_bytes(sub)
    for name, t in (("k_out", k_out), ("v_out", v_out)):
        if t is not None:
            _dev_ptr(t, name, d)
            if not t.is_contiguous() or (t.numel() * t.element_size()) % rb != 0:
                raise ValueError(f"{name} must be contiguous whole rows of {rb} bytes")
    out_rows = k_out.numel() * k_out.element_size() // rb
    if v_out is not None and v_out.numel() * v_out.element_size() // rb != out_rows:
        raise ValueError("k_out and v_out differ in rows")
    _check(_lib.ukv_gather_kv(pool.handle, sub, layer, block_table.data_ptr(),
                              block_table.stride(0) if block_table.numel() else 0, seq_lens.data_ptr(),
                              cu_out.data_ptr(),
                              num_reqs, int(window), k_out.data_ptr(),
                              None if v_out is None else v_out.data_ptr(), out_rows, _stream_handle(stream)))


def ukv_gather_kv_layers(pool: Pool, sub: int, layer_begin: int, layer_count: int, block_table: torch.Tensor,
                         seq_lens: torch.Tensor, cu_out: torch.Tensor, window: int, k_out: torch.Tensor,
                         v_out: Optional[torch.Tensor] = None, layer_step: int = 1, stream=None) -> None:
    """Gather layers layer_begin + i*layer_step (i < layer_count) in one launch into
    k_out / v_out of shape [layer_count, out_rows, ...]."""
    d = pool.device
    _dev_ptr(block_table, "block_table", d, torch.int32)
    _dev_ptr(seq_lens, "seq_lens", d, torch.int32)
    _dev_ptr(cu_out, "cu_out", d, torch.int64)
    if block_table.dim() != 2 or (block_table.numel() > 0 and block_table.stride(1) != 1):
        raise ValueError("block_table must be [num_reqs, width] with unit inner stride")
    num_reqs = seq_lens.numel()
    if block_table.shape[0] != num_reqs or cu_out.numel() != num_reqs + 1:
        raise ValueError("block_table rows / cu_out size do not match seq_lens")
    rb = pool.row_bytes(sub)
    for name, t in (("k_out", k_out), ("v_out", v_out)):
        if t is not None:
            _dev_ptr(t, name, d)
            if not t.is_contiguous() or t.dim() < 2 or t.shape[0] != layer_count:
                raise ValueError(f"{name} must be a contiguous [layer_count, out_rows, ...] tensor")
            if (t[0].numel() * t.element_size()) % rb != 0:
                raise ValueError(f"{name} rows must be whole rows of {rb} bytes")
    out_rows = k_out[0].numel() * k_out.element_size() // rb if layer_count else 0
    if v_out is not None and v_out.shape != k_out.shape:
        raise ValueError("k_out and v_out differ in shape")
    _check(_lib.ukv_gather_kv_layers(pool.handle, sub, layer_begin, layer_count, layer_step, block_table.data_ptr(),
                                     block_table.stride(0) if block_table.numel() else 0, seq_lens.data_ptr(),
                                     cu_out.data_ptr(), num_reqs, int(window), k_out.data_ptr(),
                                     None if v_out is None else v_out.data_ptr(), out_rows,
                                     k_out.stride(0) * k_out.element_size(), _stream_handle(stream)))


def ukv_move_kv(pool: Pool, sub: int, dst: torch.Tensor, src: torch.Tensor, layer_begin: int = 0,
                layer_end: Optional[int] = None, stream=None) -> None:
    """view[l][dst] = view[l][src] for every layer in [layer_begin, layer_end), K and V."""
    d = pool.device
    _dev_ptr(dst, "dst", d, torch.int32)
    _dev_ptr(src, "src", d, torch.int32)
    if dst.numel() != src.numel() or not (dst.is_contiguous() and src.is_contiguous()):
        raise ValueError("dst and src must be contiguous and of one size")
    if layer_end is None:
        layer_end = pool.specs[sub].layer_num
    _check(_lib.ukv_move_kv(pool.handle, sub, dst.data_ptr(), src.data_ptr(), dst.numel(), int(layer_begin),
                            int(layer_end), _stream_handle(stream)))


def ukv_translate_loc(pool: Pool, sub: int, slots: torch.Tensor, v2p: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """int64 token slots -> int32 internal physical slot ids (-1: tombstone / unmapped)."""
    d = pool.device
    _dev_ptr(slots, "slots", d, torch.int64)
    if not slots.is_contiguous():
        raise ValueError("slots must be contiguous")
    if out is None:
        out = torch.empty(slots.shape, dtype=torch.int32, device=d)
    _dev_ptr(out, "out", d, torch.int32)
    if out.numel() != slots.numel() or not out.is_contiguous():
        raise ValueError("out must be a contiguous int32 tensor of slots' size")
    vp = _dev_ptr(v2p, "v2p", d, torch.int32)
    _check(_lib.ukv_translate_loc(pool.handle, sub, slots.data_ptr(), slots.numel(), vp,
                                  0 if v2p is None else v2p.numel(), out.data_ptr(), _stream_handle(stream)))
    return out


def ukv_move_pages(pool: Pool, sub: int, dst_pages: torch.Tensor, src_pages: torch.Tensor, stream=None) -> None:
    """Relocate whole physical pages (every layer, K and V): page src[i] -> page dst[i]."""
    d = pool.device
    _dev_ptr(dst_pages, "dst_pages", d, torch.int32)
    _dev_ptr(src_pages, "src_pages", d, torch.int32)
    if dst_pages.numel() != src_pages.numel() or not (dst_pages.is_contiguous() and src_pages.is_contiguous()):
        raise ValueError("dst_pages and src_pages must be contiguous and of one size")
    _check(_lib.ukv_move_pages(pool.handle, sub, dst_pages.data_ptr(), src_pages.data_ptr(), dst_pages.numel(),
                               _stream_handle(stream)))


def ukv_remap_pages(pool: Pool, sub: int, v2p: torch.Tensor, virt_pages: torch.Tensor, phys_pages: torch.Tensor,
                    stream=None) -> None:
    """v2p[virt[i]] = phys[i] on the device (in place)."""
    d = pool.device
    for name, t in (("v2p", v2p), ("virt_pages", virt_pages), ("phys_pages", phys_pages)):
        _dev_ptr(t, name, d, torch.int32)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if virt_pages.numel() != phys_pages.numel():
        raise ValueError("virt_pages and phys_pages differ in size")
    _check(_lib.ukv_remap_pages(pool.handle, sub, v2p.data_ptr(), v2p.numel(), virt_pages.data_ptr(),
                                phys_pages.data_ptr(), virt_pages.numel(), _stream_handle(stream)))


def ukv_evict_window(pool: Pool, mapping: torch.Tensor, table: torch.Tensor, seq_lens: torch.Tensor, window: int,
                     stream=None) -> None:
    """Clear the full-to-SWA page mapping of pages wholly before each request's window (in place)."""
    d = pool.device
    _dev_ptr(mapping, "mapping", d, torch.int32)
    _dev_ptr(table, "table", d, torch.int32)
    _dev_ptr(seq_lens, "seq_lens", d, torch.int32)
    if table.dim() != 2 or not table.is_contiguous() or table.shape[0] != seq_lens.numel():
        raise ValueError("table must be a contiguous [num_reqs, width] tensor")
    if not (mapping.is_contiguous() and seq_lens.is_contiguous()):
        raise ValueError("mapping and seq_lens must be contiguous")
    _check(_lib.ukv_evict_window(pool.handle, mapping.data_ptr(), mapping.numel(), table.data_ptr(), table.shape[1],
                                 seq_lens.data_ptr(), seq_lens.numel(), int(window), _stream_handle(stream)))


def ukv_build_page_table(pool: Pool, sub: int, req_pages: torch.Tensor, prefix_lens: torch.Tensor,
                         out: Optional[torch.Tensor] = None, v2p: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    """Kernel-facing page table [num_reqs, width] translated from the prefix pages only
    (``out`` may be ``req_pages`` itself; a new tensor when None)."""
    d = pool.device
    _dev_ptr(req_pages, "req_pages", d, torch.int32)
    _dev_ptr(prefix_lens, "prefix_lens", d, torch.int32)
    _dev_ptr(v2p, "v2p", d, torch.int32)
    if req_pages.dim() != 2 or not req_pages.is_contiguous() or req_pages.shape[0] != prefix_lens.numel():
        raise ValueError("req_pages must be a contiguous [num_reqs, width] tensor")
    if not prefix_lens.is_contiguous() or (v2p is not None and not v2p.is_contiguous()):
        raise ValueError("prefix_lens and v2p must be contiguous")
    if out is None:
        out = torch.empty_like(req_pages)
    _dev_ptr(out, "out", d, torch.int32)
    if out.shape != req_pages.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped like req_pages")
    _check(_lib.ukv_build_page_table(pool.handle, sub, req_pages.data_ptr(), req_pages.shape[1],
                                     prefix_lens.data_ptr(), prefix_lens.numel(),
                                     None if v2p is None else v2p.data_ptr(), 0 if v2p is None else v2p.numel(),
                                     out.data_ptr(), _stream_handle(stream)))
    return out


def ukv_decode_attention_workspace_bytes(pool: Pool, sub: int, num_reqs: int, q_heads: int, max_seq_len: int,
                                         window: int = 0) -> int:
    return int(_lib.ukv_decode_attention_workspace_bytes(pool.handle, sub, num_reqs, q_heads, max_seq_len, window))


def ukv_decode_attention(pool: Pool, sub: int, layer: int, q: torch.Tensor, block_table: torch.Tensor,
                         seq_lens: torch.Tensor, max_seq_len: int, window: int, scale: float,
                         out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    """Decode attention of q [num_reqs, q_heads, head_dim] (bf16) over each request's
    positions in the layer's dense K / V views; returns fp32 [num_reqs, q_heads, head_dim].
    ``workspace`` (uint8, at least ukv_decode_attention_workspace_bytes) is allocated when None."""
    d = pool.device
    _dev_ptr(q, "q", d, torch.bfloat16)
    _dev_ptr(block_table, "block_table", d, torch.int32)
    _dev_ptr(seq_lens, "seq_lens", d, torch.int32)
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [num_reqs, q_heads, head_dim] tensor")
    num_reqs, q_heads, head_dim = q.shape
    if seq_lens.numel() != num_reqs or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be contiguous with one length per request")
    if block_table.dim() != 2 or block_table.shape[0] != num_reqs or (
            block_table.numel() > 0 and block_table.stride(1) != 1):
        raise ValueError("block_table must be [num_reqs, width] with unit inner stride")
    if out is None:
        out = torch.empty((num_reqs, q_heads, head_dim), dtype=torch.float32, device=d)
    _dev_ptr(out, "out", d, torch.float32)
    if tuple(out.shape) != (num_reqs, q_heads, head_dim) or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 tensor shaped like q")
    need = ukv_decode_attention_workspace_bytes(pool, sub, num_reqs, q_heads, max_seq_len, window)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=d)
    _dev_ptr(workspace, "workspace", d)
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    _check(_lib.ukv_decode_attention(pool.handle, sub, layer, q.data_ptr(), q_heads, block_table.data_ptr(),
                                     block_table.stride(0) if block_table.numel() else 0, seq_lens.data_ptr(),
                                     num_reqs, int(max_seq_len), int(window), float(scale), out.data_ptr(),
                                     workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                     _stream_handle(stream)))
    return out


def ukv_pool_set_debug(pool: "Pool", on: bool) -> None:
    """Debug validation on the pool's stores and moves (host copies of their ids, checked
    for races before each launch; the calls then synchronise their stream)."""
    _check(_lib.ukv_pool_set_debug(pool.handle, 1 if on else 0))


def ukv_decode_attention_noalloc(pool: Pool, sub: int, layer: int, q: torch.Tensor, block_table: torch.Tensor,
                                 seq_lens: torch.Tensor, max_seq_len: int, window: int, scale: float,
                                 out: torch.Tensor, stream=None) -> torch.Tensor:
    """ukv_decode_attention with the partial results in the library's fixed device array
    (nothing allocated: the caller passes the output too)."""
    d = pool.device
    _dev_ptr(q, "q", d, torch.bfloat16)
    _dev_ptr(block_table, "block_table", d, torch.int32)
    _dev_ptr(seq_lens, "seq_lens", d, torch.int32)
    _dev_ptr(out, "out", d, torch.float32)
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [num_reqs, q_heads, head_dim] tensor")
    num_reqs, q_heads, head_dim = q.shape
    if seq_lens.numel() != num_reqs or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be contiguous with one length per request")
    if block_table.dim() != 2 or block_table.shape[0] != num_reqs or (
            block_table.numel() > 0 and block_table.stride(1) != 1):
        raise ValueError("block_table must be [num_reqs, width] with unit inner stride")
    if tuple(out.shape) != (num_reqs, q_heads, head_dim) or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 tensor shaped like q")
    _check(_lib.ukv_decode_attention_noalloc(pool.handle, sub, layer, q.data_ptr(), q_heads, block_table.data_ptr(),
                                             block_table.stride(0) if block_table.numel() else 0,
                                             seq_lens.data_ptr(), num_reqs, int(max_seq_len), int(window),
                                             float(scale), out.data_ptr(), _stream_handle(stream)))
    return out


def ukv_mla_decode_attention_workspace_bytes(pool: Pool, sub: int, num_reqs: int, q_heads: int, v_dim: int,
                                             max_seq_len: int, window: int = 0) -> int:
    return int(_lib.ukv_mla_decode_attention_workspace_bytes(pool.handle, sub, num_reqs, q_heads, v_dim, max_seq_len,
                                                             window))


def ukv_mla_decode_attention(pool: Pool, sub: int, layer: int, q: torch.Tensor, block_table: torch.Tensor,
                             seq_lens: torch.Tensor, max_seq_len: int, window: int, scale: float, v_dim: int = 512,
                             out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                             stream=None) -> torch.Tensor:
    """Decode attention of q [num_reqs, q_heads, latent] (bf16) over each request's latent rows
    in the layer's dense MLA view; returns fp32 [num_reqs, q_heads, v_dim].  ``workspace``
    (uint8, at least ukv_mla_decode_attention_workspace_bytes) is allocated when None."""
    d = pool.device
    _dev_ptr(q, "q", d, torch.bfloat16)
    _dev_ptr(block_table, "block_table", d, torch.int32)
    _dev_ptr(seq_lens, "seq_lens", d, torch.int32)
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [num_reqs, q_heads, latent] tensor")
    num_reqs, q_heads, _ = q.shape
    if seq_lens.numel() != num_reqs or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be contiguous with one length per request")
    if block_table.dim() != 2 or block_table.shape[0] != num_reqs or (
            block_table.numel() > 0 and block_table.stride(1) != 1):
        raise ValueError("block_table must be [num_reqs, width] with unit inner stride")
    if out is None:
        out = torch.empty((num_reqs, q_heads, v_dim), dtype=torch.float32, device=d)
    _dev_ptr(out, "out", d, torch.float32)
    if tuple(out.shape) != (num_reqs, q_heads, v_dim) or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 [num_reqs, q_heads, v_dim] tensor")
    need = ukv_mla_decode_attention_workspace_bytes(pool, sub, num_reqs, q_heads, v_dim, max_seq_len, window)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=d)
    _dev_ptr(workspace, "workspace", d)
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    _check(_lib.ukv_mla_decode_attention(pool.handle, sub, layer, q.data_ptr(), q_heads, v_dim,
                                         block_table.data_ptr(), block_table.stride(0) if block_table.numel() else 0,
                                         seq_lens.data_ptr(), num_reqs, int(max_seq_len), int(window), float(scale),
                                         out.data_ptr(), workspace.data_ptr(),
                                         workspace.numel() * workspace.element_size(), _stream_handle(stream)))
    return out


def ukv_pool_error_flags(pool: Pool, stream=None) -> frozenset:
    """Read and clear the pool's sticky flags (synchronises the stream)."""
    out = ctypes.c_uint32(0)
    _check(_lib.ukv_pool_error_flags(pool.handle, _stream_handle(stream), ctypes.byref(out)))
    return frozenset(name for bit, name in FLAGS.items() if out.value & bit)


__all__ = [
    "UKV_MHA", "UKV_MLA", "UkvError", "SubpoolSpec", "Plan", "View", "Pool", "lib", "ukv_pool_plan",
    "plan_status", "ukv_pool_create", "allocate_pool", "ukv_pool_destroy", "ukv_pool_view", "ukv_plan_view", "dense_view",
    "ukv_translate_loc_for_kernel", "ukv_translate_pages_for_kernel", "ukv_store_kv", "ukv_store_kv_layers",
    "ukv_gather_kv", "ukv_gather_kv_layers", "ukv_move_kv", "ukv_pool_error_flags", "ukv_last_error", "EXPORTS",
    "STATUS", "FLAGS", "ukv_translate_loc", "ukv_move_pages", "ukv_remap_pages", "ukv_evict_window",
    "ukv_build_page_table", "ukv_decode_attention", "ukv_decode_attention_workspace_bytes",
    "ukv_mla_decode_attention", "ukv_mla_decode_attention_workspace_bytes",
]
