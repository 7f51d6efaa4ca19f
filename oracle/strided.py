"""Independent strided reference builder for the page envelope (numpy).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The report page "PR #34602: feat(unified-memory): dense KV views for
uniform-row MHA/SWA models" describes each page of an MHA sub-pool as the
envelope ``[L0_K*ps | L0_V*ps | L1_K*ps | ...]`` (implementation step 1), and
its test file checks the dense views byte for byte against an independent
strided reference builder (key files: test_unified_mha_views.py; review:
test_addressing_matches_strided_reference).  This module is that reference:
it never forms a kernel-facing id.  It addresses a token by (page, offset)
through a nested strided array

    MHA: (page, layer, kv, offset, byte)   MLA: (page, layer, offset, byte)

built only from the envelope's description (pages back to back, inside a
page the layers in order, inside a layer K then V, each ps rows of
row_bytes), and from the anchor and page count of the sub-pool.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def envelope_array(raw: np.ndarray, anchor: int, num_pages: int, layer_num: int, kv_per_layer: int,
                   page_size: int, row_bytes: int) -> np.ndarray:
    """The sub-pool's envelope as a nested view of ``raw`` (no copy)."""
    shape = (num_pages, layer_num, kv_per_layer, page_size, row_bytes)
    strides = (
        layer_num * kv_per_layer * page_size * row_bytes,  # next page envelope
        kv_per_layer * page_size * row_bytes,  # next layer inside the page
        page_size * row_bytes,  # K -> V inside the layer
        row_bytes,  # next token offset inside the block
        1,
    )
    end = anchor + num_pages * strides[0]
    assert end <= raw.size, "envelope runs past the raw buffer"
    return np.ndarray(shape=shape, dtype=np.uint8, buffer=raw, offset=anchor, strides=strides)


def layer_view_4d(raw: np.ndarray, anchor: int, num_pages: int, layer_num: int, kv_per_layer: int,
                  page_size: int, head_num: int, head_dim: int, elem_bytes: int, layer: int, kv: int) -> np.ndarray:
    """The old strided per-layer view (page, offset, head, dim) in raw element words."""
    dt = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[elem_bytes]
    row_bytes = head_num * head_dim * elem_bytes
    env = envelope_array(raw, anchor, num_pages, layer_num, kv_per_layer, page_size, row_bytes)
    blk = env[:, layer, kv]  # (page, offset, byte)
    return np.ndarray(
        shape=(num_pages, page_size, head_num, head_dim),
        dtype=dt,
        buffer=raw,
        offset=blk.__array_interface__["data"][0] - raw.__array_interface__["data"][0],
        strides=(blk.strides[0], blk.strides[1], head_dim * elem_bytes, elem_bytes),
    )


class StridedPool:
    """Reference ops addressed by (page, offset) only; ``slots`` are token slots."""

    def __init__(self, raw: np.ndarray, anchor: int, num_pages: int, layer_num: int, mla: bool,
                 page_size: int, row_bytes: int):
        self.raw = raw
        self.kv_per_layer = 1 if mla else 2
        self.page_size = page_size
        self.row_bytes = row_bytes
        self.num_pages = num_pages
        self.env = envelope_array(raw, anchor, num_pages, layer_num, self.kv_per_layer, page_size, row_bytes)

    def row(self, layer: int, kv: int, page: int, offset: int) -> np.ndarray:
        return self.env[page, layer, kv, offset]

    def row_address(self, layer: int, kv: int, page: int, offset: int) -> int:
        """Byte offset of a row inside raw."""
        return self.row(layer, kv, page, offset).__array_interface__["data"][0] - self.raw.__array_interface__["data"][0]

    def store_slots(self, layer: int, slots, k: np.ndarray, v: Optional[np.ndarray]):
        """Write token rows at their (page, offset); negative slots are skipped."""
        for i, t in enumerate(np.asarray(slots, dtype=np.int64)):
            if t < 0:
                continue
            p, o = divmod(int(t), self.page_size)
            self.env[p, layer, 0, o] = k[i]
            if v is not None:
                self.env[p, layer, 1, o] = v[i]

    def gather_pages(self, layer: int, pages_per_req, seq_lens, window: int):
        """Concatenate each request's positions, read through its physical page list."""
        ks, vs = [], []
        for pages, n in zip(pages_per_req, seq_lens):
            j0 = n - window if (window > 0 and n > window) else 0
            for j in range(j0, n):
                p = int(pages[j // self.page_size])
                o = j % self.page_size
                ks.append(self.env[p, layer, 0, o].copy())
                if self.kv_per_layer == 2:
                    vs.append(self.env[p, layer, 1, o].copy())
        k = np.array(ks, dtype=np.uint8).reshape(-1, self.row_bytes)
        v = np.array(vs, dtype=np.uint8).reshape(-1, self.row_bytes) if vs else None
        return k, v
