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
    """The oracle timed on every allowed core (its row copies split into disjoint slices) and on
    one thread; the core count and the CPU model are recorded."""
    cpu = bench.cpu_baseline("tiny", W, budget_s=0.5)
    assert cpu["kind"] == "oracle" and cpu["unit"] == "GB/s" and cpu["value"] > 0
    assert cpu["cores"] == bench.host_threads() and cpu["cpu_model"] and "tiny" in cpu["sample"]
    if cpu["cores"] > 1:
        assert cpu["single_thread"]["value"] > 0 and "1 thread" in cpu["single_thread"]["sample"]
    one = bench.cpu_baseline("tiny", W, budget_s=0.5, threads=1)
    assert one["cores"] == 1 and "single_thread" not in one


def test_threaded_oracle_leg_gives_the_same_bytes():
    """The row copies split over threads leave the host pool and outputs as one thread does."""
    import oracle

    s = bench.build_script("tiny", W)
    specs = [oracle.Spec(x.kind, x.layer_num, x.head_num, x.head_dim, x.v_head_dim, x.elem_bytes, x.num_pages)
             for x in s.shapes]
    req = oracle.plan(specs, s.page_size).required_bytes
    results = []
    for threads in (1, 3):
        pool = oracle.OraclePool(specs, s.page_size, W.fill_pattern_host(5, 0, (req + 7) // 8 * 8).copy())
        bufs = {k: np.arange(rows * rb, dtype=np.uint64).astype(np.uint8).reshape(rows, rb)
                for k, (rows, rb) in s.buffers.items()}
        live = dict(s.arrays)
        live["slots0"] = live["slots0"][live["slots0"] >= 0]  # tombstones race on the sink row
        bench._oracle_step(s, pool, live, bufs, threads, 60.0)
        results.append((pool.raw.copy(), {k: v.copy() for k, v in bufs.items()}))
    assert np.array_equal(results[0][0], results[1][0])
    for k in results[0][1]:
        assert np.array_equal(results[0][1][k], results[1][1][k])


def test_traffic_only_from_a_summary_of_the_same_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    assert bench.traffic_from_profile("decode_8b", "gather") is None
    good = bench.kernel_source_hash("gather")
    f = tmp_path / "gather_decode_8b_counters.txt"
    f.write_text(f"beyond_l2_bytes_per_launch: 12345\nkernel_source_sha256_16: {good}\n")
    assert bench.traffic_from_profile("decode_8b", "gather") == 12345
    f.write_text("beyond_l2_bytes_per_launch: 12345\nkernel_source_sha256_16: 0000000000000000\n")
    assert bench.traffic_from_profile("decode_8b", "gather") is None
    # each kernel family hashes its own source file
    assert bench.kernel_source_hash("mla_attn_span") != bench.kernel_source_hash("attn_chunk") != good


FIXTURE = os.path.join(ROOT, "tests", "fixtures", "rocprof_tiny")


def test_rocprof_summary_from_fixture_csvs(tmp_path):
    """The summariser on hand-made rocprofv3 CSV files (tests/fixtures/rocprof_tiny): the
    calibration copy reads 524,288 KiB of FETCH_SIZE and 1,048,576 KiB of WRITE_SIZE for the
    1 GiB it moves each way (scales 2 and 1); the two gather dispatches read 1 and 3 KiB of
    FETCH_SIZE and 2 KiB of WRITE_SIZE each, so bytes beyond L2 per roofline launch =
    (2 x 2 + 2 x 1) KiB = 6,144 B, against the 4,096 algorithmic bytes of the trace log's
    bench line; their trace durations (1,000 and 3,000 ns) average 2.0 us.  bench.py then
    publishes 6,144 as roofline.traffic, because the summary carries the current source hash."""
    paths = bench.rocprof_summary(FIXTURE, "tiny", out_dir=str(tmp_path))
    assert [os.path.basename(p) for p in paths] == ["gather_tiny_kernel_trace.txt", "gather_tiny_counters.txt"]
    trace = open(paths[0]).read()
    counters = open(paths[1]).read()
    assert "average 2.0 us" in trace and "2 of 2 gather dispatches" in trace
    assert "store_kernel" in trace and "fillBufferAligned" not in trace
    assert "scale 2.0000" in counters and "scale 1.0000" in counters
    assert "beyond_l2_bytes_per_launch: 6144" in counters
    assert "traffic / algorithmic: 1.5000" in counters
    assert f"kernel_source_sha256_16: {bench.kernel_source_hash('gather')}" in counters
    assert "rocprofv3 --pmc FETCH_SIZE" in counters and "--rocprof-summary" in counters
    # the stall run: means over the two gather dispatches only (the store's rows are ignored)
    for line in ("TCC_EA0_RDREQ_sum: 20", "TCC_EA0_WRREQ_sum: 30", "TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum: 2",
                 "TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum: 100"):
        assert "  " + line + "\n" in counters, line
    assert "rocprofv3 --pmc TCC_EA0_RDREQ_sum" in counters
    assert bench.traffic_from_profile("tiny", "gather", profile_dir=str(tmp_path)) == 6144


def test_rocprof_summary_command_line(tmp_path):
    """`bench.py --rocprof-summary DIR --workload W` writes the summaries without a GPU."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--rocprof-summary", FIXTURE, "--workload",
                        "tiny", "--profile-dir", str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "\n".join(str(tmp_path / f) for f in ("gather_tiny_kernel_trace.txt",
                                                                     "gather_tiny_counters.txt"))
