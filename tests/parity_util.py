"""Helpers for the GPU parity tests: a GPU pool and an oracle pool over
identical pre-filled bytes, and the byte comparison with the sink-row rule."""
from __future__ import annotations

import math
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

    def record_store(self, sub: int, layer: int, ids: np.ndarray, k: np.ndarray, v: Optional[np.ndarray]) -> None:
        """Remember the rows a store sends to the sink row (id 0) of each view."""
        at = np.nonzero(np.asarray(ids) == 0)[0]
        for kv, rows in enumerate((k, v)[: self.kvs(sub)]):
            key = (sub, layer, kv)
            if at.size:
                self.sink[key] = [rows[i] for i in at]

    def assert_pools_equal(self) -> None:
        got = self.gpu.raw.cpu().numpy()
        assert_bytes_equal_with_sinks(got, self.orc, self.sink)


def assert_bytes_equal_with_sinks(got: np.ndarray, orc: oracle.OraclePool, sink: Dict[tuple, List[np.ndarray]]):
    exp = orc.raw
    assert got.shape == exp.shape
    diff = got != exp
    if not diff.any():
        return
    for (sub, layer, kv), cands in sink.items():
        rb = orc.row_bytes(sub)
        off = orc.view_base(sub, layer, kv)  # row 0 of the view: the sink row
        g = math.gcd(rb, 4)
        dt = {1: np.uint8, 2: np.uint16, 4: np.uint32}[g]
        seg = got[off: off + rb].view(dt)
        c = np.stack([np.asarray(x, dtype=np.uint8).view(dt) for x in cands])
        ok = (c == seg[None, :]).any(axis=0)
        assert ok.all(), f"sink row of {(sub, layer, kv)}: word {np.nonzero(~ok)[0][:8]} from no tombstoned row"
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
