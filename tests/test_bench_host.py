"""Host-side checks of bench.py (no GPU): every workload's step script builds,
its byte and row accounting matches the per-unit figures the step is made of,
the multi-GPU request is refused, the CPU-oracle baseline leg runs, and the
counter figure is taken from a profile summary only when its kernel source
hash matches."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import ukv_workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("name", bench.WORKLOADS)
def test_every_workload_script_builds(name):
    s = bench.build_script(name, W, reduced=True)
    assert s.ops and all(op.nbytes > 0 for op in s.ops if not op.kind.startswith("translate"))
    assert any(s.roofline(op) for op in s.ops), "the roofline kernel must run in the step"
    kinds = {op.kind for op in s.ops}
    for op in s.ops:
        assert bench.op_rows(op, s) >= 0
    assert kinds <= {"translate", "translate_pages", "translate_loc", "store", "gather", "move", "store_layers",
                      "gather_layers", "move_pages", "remap_pages", "evict", "build_table", "attention",
                      "mla_attention"}


def test_decode_8b_step_bytes_by_hand():
    """The default workload's step: 256 slots and the block table translated once, then per layer a store of
    256 rows (4 rows of 2 KiB each and a 4-byte id) and a gather of every request (4 rows of 2 KiB per output
    row, 4 bytes per block-table page read, 12 bytes per request)."""
    s = bench.build_script("decode_8b", W)
    w = W.decode_8b()
    lens = w.req_lens[0].astype(np.int64)
    pages = sum(len(p) for p in w.req_pages[0])
    rows = int(lens.sum())
    store = 256 * (4 * 2048 + 4)
    gather = rows * 4 * 2048 + pages * 4 + 256 * 12 + 8
    table = W.padded_table(w.req_pages[0]).size * 8
    assert sum(op.nbytes for op in s.ops) == 256 * 12 + table + 32 * (store + gather)
    assert sum(bench.op_rows(op, s) for op in s.ops if not op.kind.startswith("translate")) == 32 * (256 + rows)


def test_fused_workloads_keep_the_step_bytes():
    for base in ("decode_8b", "prefill_8b", "swa_decode"):
        a = bench.build_script(base, W, reduced=True)
        b = bench.build_script(base + "_fused", W, reduced=True)
        assert sum(op.nbytes for op in a.ops) == sum(op.nbytes for op in b.ops)
        assert len(b.ops) < len(a.ops)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_cpu_baseline_runs_the_oracle():
    cpu = bench.cpu_baseline("tiny", W, budget_s=0.5)
    assert cpu["kind"] == "oracle" and cpu["cores"] == 1 and cpu["unit"] == "GB/s" and cpu["value"] > 0
    assert "tiny" in cpu["sample"]


def test_traffic_only_from_a_summary_of_the_same_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    assert bench.traffic_from_profile("decode_8b", "gather") is None
    good = bench.kernel_source_hash("gather")
    f = tmp_path / "gather_decode_8b_counters.txt"
    f.write_text(f"hbm_bytes_per_launch: 12345\nkernel_source_sha256_16: {good}\n")
    assert bench.traffic_from_profile("decode_8b", "gather") == 12345
    f.write_text("hbm_bytes_per_launch: 12345\nkernel_source_sha256_16: 0000000000000000\n")
    assert bench.traffic_from_profile("decode_8b", "gather") is None
    # each kernel family hashes its own source file
    assert bench.kernel_source_hash("mla_attn_span") != bench.kernel_source_hash("attn_chunk") != good
