"""Helpers for the GPU parity tests: a GPU pool and an oracle pool over
identical pre-filled bytes, and the byte comparison with the sink-row rule."""
from __future__ import annotations

import sys
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

import oracle
import store_gather_amd as U
import ukv_workloads as W

SEED = 7


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def ospecs(shapes) -> List[oracle.Spec]:
    return [oracle.Spec(s.kind, s.layer_num, s.head_num, s.head_dim, s.v_head_dim, s.elem_bytes, s.num_pages)
            for s in shapes]


def round8(n: int) -> int:
    return (n + 7) // 8 * 8


class Pair:
    """A GPU pool and the oracle pool, both pre-filled with the SplitMix64 byte pattern."""

    def __init__(self, shapes: Sequence[W.SubPoolShape], page_size: int, seed: int = SEED, device="cuda"):
        self.shapes = list(shapes)
        self.ps = page_size
        plan = U.ukv_pool_plan(self.shapes, page_size)
        n = round8(int(plan.required_bytes))
        self.gpu = U.allocate_pool(self.shapes, page_size, device=device, extra_bytes=n - int(plan.required_bytes))
        W.fill_pattern_device(self.gpu.raw, seed)
        self.orc = oracle.OraclePool(ospecs(self.shapes), page_size, W.fill_pattern_host(seed, 0, n).copy())
        # tombstoned source rows per (sub, layer): candidates for the sink rows
        self.sink: Dict[tuple, List[np.ndarray]] = {}

    def rb(self, sub: int) -> int:
        return self.gpu.row_bytes(sub)

    def kvs(self, sub: int) -> int:
        return 2 if self.shapes[sub].kind == W.MHA else 1

    def record_store(self, sub: int, layer: int, ids: np.ndarray, k: np.ndarray, v: Optional[np.ndarray],
                     unit: Optional[int] = None) -> None:
        """Remember the rows a store sends to the sink row (id 0) of each view, and the unit
        each of them writes whole: the store's vector width, by the rule include/ukv.h states
        for ukv_store_kv.  The default takes 16-byte aligned sources with rows back to back
        (what rows_dev gives); a test with other sources passes the width its call gets."""
        at = np.nonzero(np.asarray(ids) == 0)[0]
        rb = self.rb(sub)
        bases = [self.orc.view_base(sub, layer, kv) for kv in range(self.kvs(sub))]
        if unit is None:
            unit = copy_unit(rb, *bases)
        for kv, rows in enumerate((k, v)[: self.kvs(sub)]):
            key = (sub, layer, kv)
            if at.size:
                self.sink[key] = (unit, [rows[i] for i in at])

    def assert_pools_equal(self) -> None:
        got = self.gpu.raw.cpu().numpy()
        assert_bytes_equal_with_sinks(got, self.orc, self.sink)


def copy_unit(*values: int) -> int:
    """The largest of 16, 8, 4, 2, 1 bytes dividing every value: the vector width a store
    copies in for these row bytes, view offsets, addresses and strides."""
    u = 16
    for v in values:
        while u > 1 and int(v) % u:
            u //= 2
    return u


def assert_bytes_equal_with_sinks(got: np.ndarray, orc: oracle.OraclePool, sink: Dict[tuple, tuple]):
    """Every byte equal to the oracle's, except on the sink rows of `sink` ((sub, layer, kv) ->
    (unit, tombstoned source rows)): racing stores leave each `unit`-byte chunk of a sink row
    whole from one of its tombstoned rows (the one rule the library promises there)."""
    exp = orc.raw
    assert got.shape == exp.shape
    diff = got != exp
    if not diff.any():
        return
    for (sub, layer, kv), (unit, cands) in sink.items():
        rb = orc.row_bytes(sub)
        assert rb % unit == 0
        off = orc.view_base(sub, layer, kv)  # row 0 of the view: the sink row
        seg = got[off: off + rb].reshape(-1, unit)
        c = np.stack([np.asarray(x, dtype=np.uint8).reshape(-1, unit) for x in cands])
        ok = (c == seg[None]).all(axis=2).any(axis=0)
        assert ok.all(), (f"sink row of {(sub, layer, kv)}: {unit}-byte chunks {np.nonzero(~ok)[0][:8]} "
                          "whole from no tombstoned row")
        diff[off: off + rb] = False
    bad = np.nonzero(diff)[0]
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]} (of {got.size})"


def to_dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def bf16_rows(seed: int, n: int, row_bytes: int) -> np.ndarray:
    """n rows of bf16 N(0,1) draws as uint8 [n, row_bytes]."""
    vals = W.normal_bf16_host(seed, (n * row_bytes + 1) // 2)
    return vals.view(np.uint8)[: n * row_bytes].reshape(n, row_bytes)


def rows_dev(rows: np.ndarray) -> torch.Tensor:
    return to_dev(rows)  # uint8 [n, row_bytes] on the device


def gather_inputs(pair: Pair, sub: int, pages_per_req, lens, window: int):
    """Block table (physical pages, padded), lens, cu_out for one gather."""
    table = W.padded_table(pages_per_req)
    cu = W.out_offsets(lens, window)
    return table, np.asarray(lens, dtype=np.int32), cu


# ---------------------------------------------------------------------------
# pool-sized checks on the device (oracle addresses, regenerated pre-fill)
# ---------------------------------------------------------------------------

def rows_view(raw: torch.Tensor, anchor: int, envelope: int, rb: int) -> torch.Tensor:
    """A sub-pool's envelope as [rows, row_bytes] (rows counted from its anchor)."""
    return raw[anchor: anchor + envelope].view(-1, rb)


def offsets_to_rows(off: np.ndarray, anchor: int, rb: int) -> np.ndarray:
    off = np.asarray(off, dtype=np.int64)
    assert (off >= anchor).all() and ((off - anchor) % rb == 0).all()
    return (off - anchor) // rb


def pattern_mismatch_rows(raw: torch.Tensor, seed: int, anchor: int, envelope: int, rb: int,
                          chunk_bytes: int = 1 << 30) -> torch.Tensor:
    """Rows of [anchor, anchor + envelope) whose bytes differ from the pre-fill pattern."""
    rows_per_chunk = max(1, chunk_bytes // rb)
    nrows = envelope // rb
    out = []
    scratch = torch.empty(rows_per_chunk * rb, dtype=torch.uint8, device=raw.device)
    for r0 in range(0, nrows, rows_per_chunk):
        n = min(rows_per_chunk, nrows - r0)
        b0 = anchor + r0 * rb
        exp = scratch[: n * rb]
        fill_at(exp, seed, b0)
        diff = (raw[b0: b0 + n * rb].view(n, rb) != exp.view(n, rb)).any(dim=1)
        out.append(diff.nonzero().flatten() + r0)
    return torch.cat(out) if out else torch.empty(0, dtype=torch.int64, device=raw.device)


def fill_at(t: torch.Tensor, seed: int, byte_start: int) -> None:
    """The pre-fill pattern for bytes [byte_start, byte_start + t.numel()) of a pool,
    for any byte alignment (the generator works on 8-byte words)."""
    lo = byte_start - byte_start % 8
    hi = byte_start + t.numel()
    hi8 = (hi + 7) // 8 * 8
    if lo == byte_start and hi8 == hi:
        W.fill_pattern_device(t, seed, byte_start=lo)
        return
    tmp = torch.empty(hi8 - lo, dtype=torch.uint8, device=t.device)
    W.fill_pattern_device(tmp, seed, byte_start=lo)
    t.copy_(tmp[byte_start - lo: byte_start - lo + t.numel()])


def assert_bytes_are_pattern(raw: torch.Tensor, seed: int, start: int, end: int) -> None:
    if end <= start:
        return
    exp = torch.empty(end - start, dtype=torch.uint8, device=raw.device)
    fill_at(exp, seed, start)
    assert torch.equal(raw[start:end], exp), f"bytes [{start}, {end}) changed"


def assert_rows_subset(changed: torch.Tensor, allowed_mask: torch.Tensor, what: str) -> None:
    """Every changed row is one the operation was meant to write."""
    if changed.numel() == 0:
        return
    bad = changed[~allowed_mask[changed]]
    assert bad.numel() == 0, f"{what}: {bad.numel()} rows changed that no operation writes, e.g. {bad[:8].tolist()}"


def equal_rows_chunked(a: torch.Tensor, a_idx: torch.Tensor, b: torch.Tensor, b_idx, chunk: int = 1 << 20) -> bool:
    """a[a_idx] == b[b_idx] row for row (b_idx None: b itself), in chunks."""
    for c0 in range(0, a_idx.numel(), chunk):
        x = a.index_select(0, a_idx[c0: c0 + chunk])
        y = b[c0: c0 + chunk] if b_idx is None else b.index_select(0, b_idx[c0: c0 + chunk])
        if not torch.equal(x, y):
            return False
    return True
