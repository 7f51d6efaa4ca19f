"""Throughput of the unified page-major KV pool's hot path on one MI355X.

A step is one pass of the whole path over one batch of a workload: translate
the batch's token slots and its block table once, then, layer by layer, the
stores and gathers, then the move where the workload has one.  Every launch
goes through the C ABI (libukv.so) on torch's current stream.

Default workload (decode_8b, the configuration the metric is quoted on):
Llama-3-8B-shape pool, 32 layers x 8 KV heads x head dim 128, bf16, page
size 16, 4,096 pages = 65,536 slots (8 GiB of envelopes); 256 requests with
lengths uniform in [1024, 8192]; per layer store 256 new rows and gather every
request in full.  `--workload` selects the others (prefill_8b, hybrid,
move_70b, tiny); each prints its own JSON line.

Output: one JSON line per workload.  `value` is algorithmic GB/s (bytes the
method must read and write, 1e9 B/s) over the whole step with inputs resident
in HBM.  `roofline` reports the dominant kernel per launch, from HIP events
recorded around each of its launches inside the timed region, on the stream
the kernels run on.  `ops` gives every launch kind's time per launch, from
all its launches in step order run back to back (outside the timed region).
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
`tokens_per_s` counts token rows (one token's K and V, or its MLA latent, in
one layer) stored, gathered, moved or attended over the step time; each `ops`
entry gives its own rows per launch and rate.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
import time
from dataclasses import dataclass, field
from typing import Callable, Dict, List

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0  # MI355X HBM3E, 8 TB/s
METRIC = "KV store/gather/move HBM GB/s and % of peak, Llama-3-8B-shape pool"
KERNEL_SRC = os.path.join(ROOT, "store_gather_amd", "csrc", "ukv_runtime.hip")
ATTN_SRC = os.path.join(ROOT, "store_gather_amd", "csrc", "ukv_attention.hip")
MLA_ATTN_SRC = os.path.join(ROOT, "store_gather_amd", "csrc", "ukv_mla_attention.hip")
PROFILE_DIR = os.path.join(ROOT, "profiles")
WORKLOADS = ("decode_8b", "prefill_8b", "hybrid", "move_70b", "tiny", "decode_8b_fused", "prefill_8b_fused",
             "compact_8b", "swa_decode", "swa_decode_fused", "decode_attn_8b", "decode_attn_mla", "decode_8b_noreuse")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def num(x, nd):
    """Rounded float, or None for a figure that was not measured."""
    return None if x is None or x != x else round(float(x), nd)


def kernel_source_hash(kernel: str = "") -> str:
    """First 16 hex digits of the SHA-256 of the source file that holds `kernel`."""
    src = MLA_ATTN_SRC if kernel.startswith("mla_attn") else ATTN_SRC if kernel.startswith("attn") else KERNEL_SRC
    with open(src, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile(workload: str, kernel: str, profile_dir: str = None):
    """Bytes beyond L2 per launch of the roofline kernel (FETCH_SIZE + WRITE_SIZE, each
    scaled by a plain copy's reading) from the committed counter summary, or None when
    there is none or it was taken on a different kernel source."""
    path = os.path.join(profile_dir or PROFILE_DIR, f"{kernel}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"beyond_l2_bytes_per_launch:\s*([0-9]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash(kernel):
        return None
    return int(m_bytes.group(1))


# ----------------------------------------------------------------------------
# rocprofv3 harness: kernel-trace and counter runs -> the summaries under profiles/
# ----------------------------------------------------------------------------

# The library's kernels, as they appear in rocprofv3's kernel names.
LIB_KERNELS = ("store_kernel", "store_piece_kernel", "store_group_kernel", "gather_kernel", "gather_piece_kernel", "move_kernel",
               "move_piece_kernel", "translate_slots_kernel", "translate_pages_kernel", "move_pages_kernel",
               "remap_pages_kernel", "evict_window_kernel", "build_page_table_kernel", "attn_chunk_kernel",
               "attn_combine_kernel", "mla_attn_span_kernel", "mla_attn_combine_kernel", "flags_fetch_clear_kernel",
               "validate_mark_kernel", "validate_check_kernel", "translate_inplace_kernel")


# The attention entry points: one call is the split kernel, then the kernel that merges its
# partials; bench.py's HIP events bracket the call, so its roofline time holds both.
ROOFLINE_MERGE_KERNEL = {"attn_chunk": "attn_combine_kernel", "mla_attn_span": "mla_attn_combine_kernel"}


STALL_COUNTERS = ("TCC_EA0_RDREQ_sum", "TCC_EA0_WRREQ_sum", "TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum",
                  "TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum")


def profile_commands(workload: str, out: str = "$OUT") -> Dict[str, str]:
    """The four profiler runs one summary needs (run from /tmp with TMPDIR=/tmp; $R is the
    repository root, $OUT a directory for rocprofv3's CSV files): a kernel trace, then one
    counter per run (FETCH_SIZE, WRITE_SIZE), each beside a plain 1 GiB copy that
    calibrates the counter, then L2's requests to memory and the cycles they waited for
    DRAM credits (four L2 counters, one run)."""
    bench = f"python3 $R/bench.py --workload {workload} --no-cpu-baseline --no-bar"
    return {
        "trace": f"rocprofv3 --kernel-trace --stats --output-format csv -d {out}/trace -o run -- {bench} "
                 f"--steps 5 --warmup 2 > {out}/trace.log",
        "fetch": f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {out}/fetch -o run -- {bench} "
                 f"--steps 1 --warmup 1 --copy-calibration",
        "write": f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {out}/write -o run -- {bench} "
                 f"--steps 1 --warmup 1 --copy-calibration",
        "stalls": f"rocprofv3 --pmc {' '.join(STALL_COUNTERS)} --output-format csv -d {out}/stalls -o run -- {bench} "
                  f"--steps 1 --warmup 1",
    }


def _is_lib_kernel(name: str) -> bool:
    return any(re.search(r"(^|::|\s)" + k + r"\b", name) for k in LIB_KERNELS)


def _matches(name: str, kernel: str) -> bool:
    """Kernel names of one launch kind: `kernel` is the short name (store, gather, move,
    move_pages, attn_chunk, mla_attn_span); the row-piece, row-group and tile kernels all
    count."""
    return re.search(r"(^|::|\s)" + kernel + r"(_piece|_group)?_kernel\b", name) is not None


def _grid(row: dict, keys) -> int:
    g = 1
    for k in keys:
        g *= int(row[k])
    return g


def rocprof_summary(directory: str, workload: str, out_dir: str = PROFILE_DIR) -> List[str]:
    """Write the kernel-trace and counter summaries of one workload from the
    rocprofv3 runs of :func:`profile_commands` kept under ``directory`` (the stall run is
    optional: without it the counters summary ends after the bytes beyond L2).

    Kernel trace: the stats rows of this library's kernels, and the roofline kind's
    average duration (only its largest-grid dispatches where the workload's script
    says that one kernel also serves a smaller launch kind) beside bench.py's
    HIP-event figure from the same run.  Counters: FETCH_SIZE and WRITE_SIZE per
    dispatch (KiB) are scaled by what they read for the plain 1 GiB device copy
    (__amd_rocclr_copyBuffer, 1,048,576 KiB each way) and summed: bytes moved beyond
    L2 per dispatch (L2 misses, which MALL hits still count), against the algorithmic
    bytes per launch.  Each summary records the SHA-256 (16 hex digits) of the kernel
    source it was taken on; bench.py publishes the counter figure only while it
    matches."""
    import ukv_workloads as W

    script = build_script(workload, W)
    kernel = script.roofline_kernel
    src = MLA_ATTN_SRC if kernel.startswith("mla_attn") else ATTN_SRC if kernel.startswith("attn") else KERNEL_SRC
    h = kernel_source_hash(kernel)
    cmds = profile_commands(workload)

    def rows(path):
        with open(path, newline="") as f:
            return list(csv.DictReader(f))

    bench_line = None
    log_path = os.path.join(directory, "trace.log")
    if os.path.exists(log_path):
        for line in open(log_path):
            if line.startswith("{"):
                bench_line = json.loads(line)
    stats = rows(os.path.join(directory, "trace", "run_kernel_stats.csv"))
    def is_roof(name):
        return _matches(name, kernel) and (not script.roofline_nkv or
                                           re.search(r"<[^,]*, %d[,>]" % script.roofline_nkv, name) is not None)

    trace = [r for r in rows(os.path.join(directory, "trace", "run_kernel_trace.csv")) if is_roof(r["Kernel_Name"])]
    if not trace:
        raise ValueError(f"no {kernel} kernel dispatches in the trace")
    gk = ("Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z")
    gmax = max(_grid(r, gk) for r in trace)
    sel = [r for r in trace if _grid(r, gk) == gmax] if script.roofline_largest_grid else trace
    durs = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in sel]
    roof_avg = sum(durs) / len(durs)
    lines = [f"# Kernel trace: {workload} workload ({kernel} kernels are the roofline kind)", "",
             "Command (from /tmp with TMPDIR=/tmp; R = repository root, OUT = a scratch directory):",
             "  " + cmds["trace"], "",
             f"Summarised by: python3 bench.py --rocprof-summary $OUT --workload {workload}",
             f"kernel source: {os.path.relpath(src, ROOT)}, kernel_source_sha256_16: {h}",
             "Rows of rocprofv3's run_kernel_stats.csv for this library's kernels (durations in ns):", "",
             '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"']
    for r in stats:
        if _is_lib_kernel(r["Name"]):
            lines.append(",".join(f'"{r[k]}"' if k == "Name" else r[k] for k in
                                  ("Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs",
                                   "StdDev")))
    lines += ["", f"Roofline dispatches: {len(sel)} of {len(trace)} {kernel} dispatches"
              + (f" (the largest grid, {gmax} work-items; the smaller ones are another launch kind)"
                 if script.roofline_largest_grid else "") + f", average {roof_avg / 1e3:.1f} us"]
    merge = ROOFLINE_MERGE_KERNEL.get(kernel)
    if merge:  # the attention entry points launch the split kernel, then a merge kernel
        md = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
              for r in rows(os.path.join(directory, "trace", "run_kernel_trace.csv"))
              if re.search(r"(^|::|\s)" + merge + r"\b", r["Kernel_Name"])]
        if md:
            m_avg = sum(md) / len(md)
            lines.append(f"Each call also launches its merge kernel ({merge}): average {m_avg / 1e3:.1f} us; "
                         f"both kernels {(roof_avg + m_avg) / 1e3:.1f} us per call, the interval bench.py's events bracket")
    if bench_line:
        rl = bench_line["roofline"]
        lines += [f"Same run, bench.py's HIP events around every roofline launch: {rl['ms_per_launch'] * 1e3:.1f} us "
                  f"per launch; roofline achieved {rl['achieved']} GB/s ({rl['frac']})",
                  f"bench value {bench_line['value']} GB/s for the whole step ({bench_line['pct_of_peak']}% of 8 TB/s)"]
    trace_path = os.path.join(out_dir, f"{kernel}_{workload}_kernel_trace.txt")
    with open(trace_path, "w") as f:
        f.write("\n".join(lines) + "\n")

    def counters(name, run=None):
        out, grids = {}, {}
        for r in rows(os.path.join(directory, run or name.split("_")[0].lower(), "run_counter_collection.csv")):
            if r["Counter_Name"] == name:
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
                grids.setdefault(r["Kernel_Name"], []).append(int(r["Grid_Size"]))
        if script.roofline_largest_grid:  # the largest grid over all the roofline kind's kernels
            g = max(max(v) for k, v in grids.items() if is_roof(k))
            for k in list(out):
                if is_roof(k):
                    out[k] = [v for v, gg in zip(out[k], grids[k]) if gg == g]
                    if not out[k]:
                        del out[k]
        return out

    fetch, write = counters("FETCH_SIZE"), counters("WRITE_SIZE")
    copies = [k for k in fetch if "copyBuffer" in k]
    if not copies or not any("copyBuffer" in k for k in write):
        raise ValueError("no calibration copy (__amd_rocclr_copyBuffer) in the counter runs")
    kib = float(1 << 20)  # the copy reads and writes 1 GiB
    f_scale = kib / max(fetch[copies[0]])
    w_scale = kib / max(next(v for k, v in write.items() if "copyBuffer" in k))
    lines = [f"# Bytes beyond L2 per dispatch, {workload} workload ({kernel} kernels are the roofline kind)", "",
             "Commands (from /tmp with TMPDIR=/tmp; R = repository root, OUT = a scratch directory), one counter "
             "per run:", "  " + cmds["fetch"], "  " + cmds["write"], "",
             f"Summarised by: python3 bench.py --rocprof-summary $OUT --workload {workload}", "",
             "FETCH_SIZE and WRITE_SIZE count traffic between L2 and the memory fabric (L2 misses and write-backs),",
             "so MALL (Infinity Cache) hits count as well: these are bytes beyond L2, an upper bound on DRAM bytes.",
             "Calibration: --copy-calibration runs a plain 1 GiB device copy (torch copy_, dispatched as",
             "__amd_rocclr_copyBuffer); its counters per dispatch against the 1,048,576 KiB it reads and writes:",
             f"  FETCH_SIZE {max(fetch[copies[0]]):.3f} KiB -> scale {f_scale:.4f}",
             f"  WRITE_SIZE {kib / w_scale:.3f} KiB -> scale {w_scale:.4f}", "",
             "Per kernel: mean counters per dispatch, and (FETCH x scale + WRITE x scale) x 1024 bytes:"]
    roof = []  # (dispatches, bytes per dispatch) of the roofline kind's kernels
    for k in sorted(fetch):
        if not _is_lib_kernel(k):
            continue
        fm = sum(fetch[k]) / len(fetch[k])
        wv = write.get(k, [0.0])
        wm = sum(wv) / len(wv)
        b = int(round((fm * f_scale + wm * w_scale) * 1024))
        lines.append(f"  {k}: {len(fetch[k])} dispatches, FETCH_SIZE {fm:.3f} KiB, WRITE_SIZE {wm:.3f} KiB -> {b} B")
        if is_roof(k):
            roof.append((len(fetch[k]), b))
    n_roof = sum(n for n, _ in roof)
    roof_bytes = int(round(sum(n * b for n, b in roof) / n_roof)) if n_roof else None
    alg = bench_line["roofline"]["algorithmic_bytes_per_launch"] if bench_line else None
    lines += ["", f"roofline kind: the {kernel} dispatches" + (", largest grid only" if script.roofline_largest_grid
                                                                else ""),
              f"beyond_l2_bytes_per_launch: {roof_bytes}",
              f"algorithmic_bytes_per_launch: {alg}",
              f"traffic / algorithmic: {roof_bytes / alg:.4f}" if (roof_bytes and alg) else "traffic / algorithmic: n/a"]
    if os.path.exists(os.path.join(directory, "stalls", "run_counter_collection.csv")):
        # L2's requests to memory and the cycles they waited because the memory side had
        # no credits left, summed over the L2 channels, per roofline dispatch
        st = {c: counters(c, "stalls") for c in STALL_COUNTERS}
        per = {}
        for c, by_kernel in st.items():
            vals = [v for k, vs in by_kernel.items() if is_roof(k) for v in vs]
            per[c] = sum(vals) / len(vals) if vals else None
        lines += ["", "DRAM credit stalls (one more run):", "  " + cmds["stalls"],
                  "Per roofline dispatch, summed over the L2 channels: requests from L2 to memory, and the",
                  "cycles they waited because the memory side had no credits (room) left for them:"]
        for c in STALL_COUNTERS:
            lines.append(f"  {c}: {per[c]:.4g}" if per[c] is not None else f"  {c}: n/a")
    lines.append(f"kernel_source_sha256_16: {h}")
    counters_path = os.path.join(out_dir, f"{kernel}_{workload}_counters.txt")
    with open(counters_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return [trace_path, counters_path]


# ----------------------------------------------------------------------------
# A workload's step as a script of operations, run on the GPU (libukv) or the CPU oracle
# ----------------------------------------------------------------------------

@dataclass
class Op:
    kind: str  # translate | translate_pages | store | gather | move
    sub: int
    label: str
    args: dict
    nbytes: int = 0  # algorithmic bytes (reads + writes the method must do)


@dataclass
class Script:
    name: str
    description: str
    shapes: list
    page_size: int
    arrays: Dict[str, np.ndarray]  # host inputs: slots, tables, lens, cu_out
    buffers: Dict[str, tuple]  # name -> (rows, row_bytes): store sources and gather outputs
    ops: List[Op]
    roofline: Callable[[Op], bool]
    roofline_kernel: str
    counts: dict = field(default_factory=dict)
    dtype: str = "u8"  # what the path computes in: bytes moved as integers
    roofline_largest_grid: bool = False  # the roofline kernel also serves a smaller launch kind
    roofline_nkv: int = 0  # when set: only the kernels instantiated for this many views (2 = K and V)


def op_rows(op: Op, s: "Script") -> int:
    """Token rows one launch moves or reads: one token's K and V (MHA) or latent (MLA) in one
    layer is one row.  Translations count the slots they translate; table work counts none."""
    a = op.args
    if op.kind in ("translate", "translate_loc"):
        return int(s.arrays[a["inp"]].size)
    if op.kind == "store":
        return int(a["n"])
    if op.kind == "store_layers":
        return int(a["n"]) * int(a["count"])
    if op.kind == "gather":
        return int(a["rows"])
    if op.kind == "gather_layers":
        return int(a["rows"]) * int(a["count"])
    if op.kind == "move":
        return int(s.arrays[f"msrc{op.sub}"].size) * (int(a["l1"]) - int(a["l0"]))
    if op.kind == "move_pages":
        return int(s.arrays[f"psrc{op.sub}"].size) * s.page_size * s.shapes[op.sub].layer_num
    if op.kind in ("attention", "mla_attention"):
        return int(s.arrays[f"lens{op.sub}"].astype(np.int64).sum())
    return 0


def _pages_read(pages_per_req, lens, window, ps):
    n = 0
    for pages, ln in zip(pages_per_req, lens):
        ln = int(ln)
        j0 = ln - window if 0 < window < ln else 0
        if ln > j0:
            n += (ln - 1) // ps - j0 // ps + 1
    return n


DESCRIPTIONS = {
    "decode_8b": "decode_8b: Llama-3-8B-shape pool (32 layers, 8 KV heads x 128, bf16, page 16, 4096 pages = 65,536 "
                 "slots, 8 GiB); 256 requests, lengths U[1024, 8192], pages shared cyclically from one seeded "
                 "permutation; per step: translate 256 slots and the block table once, then per layer store 256 new "
                 "K/V rows and gather every request in full",
    "decode_8b_noreuse": "decode_8b_noreuse: the decode_8b batch (256 requests, lengths U[1024, 8192], same seeds) on "
                         "a pool sized to hold every context apart (73,857 pages of 2 MiB, 144 GiB): no page is read "
                         "twice in a layer, so the gathers' bytes cannot come from the Infinity Cache; per step: "
                         "translate once, then per layer store 256 new K/V rows and gather every request in full",
    "prefill_8b": "prefill_8b: Llama-3-8B-shape pool (16,384 pages = 262,144 slots, 32 GiB); 32,768 new tokens over "
                  "16 requests (Dirichlet split, runs of whole pages, 1% tombstones); per step: translate, then per "
                  "layer store all 32,768 tokens and gather the 16 requests back, then move 65,536 rows to disjoint "
                  "rows on all 32 layers",
    "hybrid": "hybrid: MHA sub-pool (24 layers, 8 KV heads x 64, bf16, page 64, odd layers sliding-window 128) and "
              "MLA sub-pool (24 layers, 576-wide latent) holding 128 requests of U[256, 16384] tokens apart (16,538 "
              "pages each, ~76 GiB); per step: translate both, then per layer store every token in both sub-pools "
              "and gather every request (MHA full or its last 128, MLA full); one set of source rows serves every "
              "layer",
    "move_70b": "move_70b: Llama-3-70B-shape pool (80 layers, 8 KV heads x 128, bf16, page 16, 32,768 pages, "
                "160 GiB); per step: translate 131,072 slots, move 65,536 rows to 65,536 disjoint rows on all 80 "
                "layers, K and V, in one launch",
    "tiny": "tiny: 2 layers, 2 KV heads x 8, bf16, page 4, 16 pages; store 37 entries (3 tombstones), gather 3 "
            "requests of 5/11/21 tokens, move 8 rows",
    "decode_8b_fused": "decode_8b_fused: the decode_8b batch with the 256 new rows of all 32 layers stored in one "
                       "launch (ukv_store_kv_layers), then the per-layer gathers",
    "prefill_8b_fused": "prefill_8b_fused: the prefill_8b batch with all 32 layers stored in one launch and gathered "
                        "back in one launch (ukv_store_kv_layers / ukv_gather_kv_layers), then the move",
    "swa_decode_fused": "swa_decode_fused: the swa_decode batch with each sub-pool's 12 layers stored in one launch "
                        "and gathered in one launch (the full layers in full, the window layers their last 128 "
                        "positions; ukv_store_kv_layers / ukv_gather_kv_layers), then the eviction",
    "swa_decode": "swa_decode: a 24-layer hybrid model (8 KV heads x 64, bf16, page 64) whose 12 full-attention "
                  "layers use a full sub-pool (16,540 pages) and whose 12 sliding-window-128 layers use their own "
                  "sub-pool (638 pages) reached through a full-to-SWA page mapping; 128 requests of U[256, 16384] "
                  "tokens get one new token each; per step: translate (the window layers through the mapping), "
                  "per layer store the new rows and gather every request (full, or its last 128 positions), then "
                  "evict the pages that left the window",
    "decode_attn_8b": "decode_attn_8b: the decode_8b batch on the read path: a Llama-3-8B-shape pool (32 layers, "
                      "8 KV heads x 128, bf16, page 16, 4,096 pages, 8 GiB) of Irwin-Hall bf16 values, 256 requests "
                      "of U[1024, 8192] positions with 32 query heads each (GQA 4); per step: translate the 256 new "
                      "slots and build the prefix-only page table once, then per layer store the 256 new K/V rows "
                      "and run decode attention over every request straight from the dense views (fp32 output)",
    "decode_attn_mla": "decode_attn_mla: the read path on the hybrid workload's MLA sub-pool (24 layers, one "
                       "576-wide bf16 latent row per token, page 64, 16,538 pages, ~28 GiB) of Irwin-Hall bf16 "
                       "values; 128 requests of U[256, 16384] positions, 16 query heads each (a 128-head MLA model's "
                       "share of one GPU at 8-way tensor parallelism); per step: translate the 128 new slots and "
                       "build the prefix-only page table once, then per layer store the 128 new latent rows and run "
                       "decode attention over every request straight from the dense latent view (scores over the "
                       "whole row, values its first 512 elements, fp32 output)",
    "compact_8b": "compact_8b: the prefill_8b pool (16,384 pages of 2 MiB) with its 16 requests addressed through a "
                  "virtual-to-physical table; per step: internal ids of the batch (translate_loc), relocation of every "
                  "live page above the watermark into the free pages below it (whole page envelopes, all 32 layers, "
                  "K and V), the table rewrite, and the block table through the new table",
}


def build_script(name: str, W, reduced: bool = False) -> Script:
    """The step of workload `name`.  `reduced` shrinks the pools (same row and page geometry,
    envelopes of at most ~8 GiB) for the CPU-oracle sample."""
    if name == "compact_8b":
        return compaction_script(W, reduced)
    if name == "swa_decode":
        return swa_script(W, reduced)
    if name == "decode_attn_8b":
        return attention_script(W, reduced)
    if name == "decode_attn_mla":
        return attention_mla_script(W, reduced)
    if name.endswith("_fused"):
        return fuse_layers(build_script(name[: -len("_fused")], W, reduced), name,
                           gathers=name.startswith(("prefill", "swa")))
    if name == "decode_8b":
        w = W.decode_8b()
    elif name == "decode_8b_noreuse":
        w = W.decode_8b(num_reqs=12, share_pages=False) if reduced else W.decode_8b(share_pages=False)
    elif name == "prefill_8b":
        w = W.prefill_8b(num_pages=4096, move_rows=16384) if reduced else W.prefill_8b()
    elif name == "hybrid":
        w = W.hybrid(num_reqs=12) if reduced else W.hybrid()
    elif name == "move_70b":
        w = W.move_70b(num_pages=1600, rows=8192) if reduced else W.move_70b()
    elif name == "tiny":
        w = W.tiny_mha()
    else:
        raise ValueError(name)

    ps = w.page_size
    arrays: Dict[str, np.ndarray] = {}
    buffers: Dict[str, tuple] = {}
    ops: List[Op] = []
    nsub = len(w.shapes)
    rb = [s.row_bytes for s in w.shapes]
    nkv = [2 if s.kind == W.MHA else 1 for s in w.shapes]
    kind_name = ["mha" if k == 2 else "mla" for k in nkv]

    # translation, once per batch
    for sub in range(nsub):
        if sub in w.store_slots:
            arrays[f"slots{sub}"] = w.store_slots[sub].astype(np.int64)
            n = arrays[f"slots{sub}"].size
            ops.append(Op("translate", sub, f"translate sub{sub}", {"inp": f"slots{sub}", "out": f"ids{sub}"}, n * 12))
        if sub in w.req_pages:
            arrays[f"table{sub}"] = W.padded_table(w.req_pages[sub])
            arrays[f"lens{sub}"] = w.req_lens[sub].astype(np.int32)
            t = arrays[f"table{sub}"]
            ops.append(Op("translate_pages", sub, f"translate_pages sub{sub}", {"inp": f"table{sub}", "out": f"bt{sub}"},
                          t.size * 8))
        if sub in w.move_src:
            arrays[f"msrc{sub}"] = w.move_src[sub].astype(np.int64)
            arrays[f"mdst{sub}"] = w.move_dst[sub].astype(np.int64)
            m = arrays[f"msrc{sub}"].size
            ops.append(Op("translate", sub, f"translate move src sub{sub}", {"inp": f"msrc{sub}", "out": f"msrcid{sub}"},
                          m * 12))
            ops.append(Op("translate", sub, f"translate move dst sub{sub}", {"inp": f"mdst{sub}", "out": f"mdstid{sub}"},
                          m * 12))

    # sources and outputs
    per_layer_sources = name in ("decode_8b", "decode_8b_noreuse", "prefill_8b", "tiny")
    for sub in range(nsub):
        if sub in w.store_slots:
            n = arrays[f"slots{sub}"].size
            L = w.shapes[sub].layer_num if per_layer_sources else 1
            for h in range(nkv[sub]):
                buffers[f"src{sub}_{h}"] = (L * n, rb[sub])
        if sub in w.req_pages:
            wins = sorted(set(w.windows[sub]))
            for win in wins:
                arrays[f"cu{sub}_{win}"] = W.out_offsets(arrays[f"lens{sub}"], win)
            rows = max(int(arrays[f"cu{sub}_{win}"][-1]) for win in wins)
            for h in range(nkv[sub]):
                buffers[f"out{sub}_{h}"] = (rows, rb[sub])

    # per layer: stores, then gathers
    layer_num = max(s.layer_num for s in w.shapes)
    for layer in range(layer_num):
        for sub in range(nsub):
            if layer >= w.shapes[sub].layer_num or sub not in w.store_slots:
                continue
            n = arrays[f"slots{sub}"].size
            row0 = layer * n if per_layer_sources else 0
            ops.append(Op("store", sub, f"store {kind_name[sub]} sub{sub}",
                          {"layer": layer, "ids": f"ids{sub}", "row0": row0, "n": n},
                          n * (2 * nkv[sub] * rb[sub] + 4)))
        for sub in range(nsub):
            if layer >= w.shapes[sub].layer_num or sub not in w.req_pages:
                continue
            win = w.windows[sub][layer]
            cu = arrays[f"cu{sub}_{win}"]
            rows = int(cu[-1])
            R = arrays[f"lens{sub}"].size
            pr = _pages_read(w.req_pages[sub], arrays[f"lens{sub}"], win, ps)
            ops.append(Op("gather", sub, f"gather {kind_name[sub]}{' swa' if win else ''} sub{sub}",
                          {"layer": layer, "window": win, "cu": f"cu{sub}_{win}", "rows": rows},
                          rows * 2 * nkv[sub] * rb[sub] + pr * 4 + R * 12 + 8))
    # the move, over every layer in one launch
    for sub in range(nsub):
        if sub in w.move_src:
            m = arrays[f"msrc{sub}"].size
            L = w.shapes[sub].layer_num
            ops.append(Op("move", sub, f"move sub{sub}", {"l0": 0, "l1": L}, m * L * 2 * nkv[sub] * rb[sub] + m * 8))

    roof = {
        "decode_8b": (lambda op: op.kind == "gather", "gather"),
        "decode_8b_noreuse": (lambda op: op.kind == "gather", "gather"),
        "prefill_8b": (lambda op: op.kind == "move", "move"),
        "hybrid": (lambda op: op.label.startswith("store mha"), "store"),
        "move_70b": (lambda op: op.kind == "move", "move"),
        "tiny": (lambda op: op.kind == "gather", "gather"),
    }[name]
    counts = {"layers": layer_num}
    for sub in range(nsub):
        if sub in w.store_slots:
            counts[f"stored_rows_per_layer_sub{sub}"] = int(arrays[f"slots{sub}"].size)
        if sub in w.req_lens:
            counts[f"requests_sub{sub}"] = int(arrays[f"lens{sub}"].size)
            counts[f"gathered_rows_per_full_layer_sub{sub}"] = int(arrays[f"lens{sub}"].astype(np.int64).sum())
        if sub in w.move_src:
            counts[f"moved_rows_sub{sub}"] = int(arrays[f"msrc{sub}"].size)
    return Script(name, DESCRIPTIONS[name], list(w.shapes), ps, arrays, buffers, ops, roof[0], roof[1], counts,
                  roofline_nkv=2 if name == "hybrid" else 0)


def compaction_script(W, reduced: bool) -> Script:
    w = W.prefill_8b(num_pages=4096, move_rows=0) if reduced else W.prefill_8b(move_rows=0)
    ps = w.page_size
    shape = w.shapes[0]
    P = shape.num_pages
    used = np.unique(np.concatenate(w.req_pages[0]))
    vpages = [np.searchsorted(used, p).astype(np.int32) for p in w.req_pages[0]]
    src, dst = W.compaction_plan(used, P)
    arrays = {
        "vslots0": W.slots_of_requests(vpages, w.req_lens[0], ps).astype(np.int64),
        "v2p0": used.astype(np.int32),
        "psrc0": src,
        "pdst0": dst,
        "pvirt0": np.searchsorted(used, src).astype(np.int32),
        "table0": W.padded_table(vpages),
    }
    page_bytes = ps * 2 * shape.layer_num * shape.row_bytes
    n, m, t = arrays["vslots0"].size, src.size, arrays["table0"].size
    ops = [
        Op("translate_loc", 0, "translate_loc sub0", {"inp": "vslots0", "out": "int0", "v2p": "v2p0"}, n * 16),
        Op("move_pages", 0, "move_pages sub0", {}, m * 2 * page_bytes + m * 8),
        Op("remap_pages", 0, "remap_pages sub0", {}, m * 12),
        Op("translate_pages", 0, "translate_pages sub0", {"inp": "table0", "out": "bt0", "v2p": "v2p0"}, t * 12),
    ]
    counts = {"layers": shape.layer_num, "relocated_pages": int(m), "live_pages": int(used.size),
              "page_bytes": int(page_bytes)}
    return Script("compact_8b", DESCRIPTIONS["compact_8b"], list(w.shapes), ps, arrays, {}, ops,
                  lambda op: op.kind == "move_pages", "move_pages", counts)


def swa_script(W, reduced: bool) -> Script:
    w = W.swa_decode(num_reqs=24 if reduced else 128)
    ps = w.page_size
    full, swa = w.shapes
    lens = w.req_lens[0]
    table = W.padded_table(w.req_pages[0])
    arrays = {"slots0": w.store_slots[0], "slots1": w.store_slots[0].copy(), "map1": w.swa_mapping.copy(),
              "table0": table, "table1": table.copy(), "ptable": W.padded_table(w.req_pages[0], pad=-1),
              "lens0": lens, "lens1": lens, "cu0_0": W.out_offsets(lens), "cu1_win": W.out_offsets(lens, w.window)}
    n, R, rb = lens.size, lens.size, full.row_bytes
    ops = [Op("translate", 0, "translate sub0", {"inp": "slots0", "out": "ids0"}, n * 12),
           Op("translate", 1, "translate swa sub1", {"inp": "slots1", "out": "ids1", "v2p": "map1"}, n * 16),
           Op("translate_pages", 0, "translate_pages sub0", {"inp": "table0", "out": "bt0"}, table.size * 8),
           Op("translate_pages", 1, "translate_pages swa sub1", {"inp": "table1", "out": "bt1", "v2p": "map1"},
              table.size * 12)]
    rows_full = int(arrays["cu0_0"][-1])
    rows_win = int(arrays["cu1_win"][-1])
    pr_full = _pages_read(w.req_pages[0], lens, 0, ps)
    pr_win = _pages_read(w.req_pages[0], lens, w.window, ps)
    for layer in range(full.layer_num):
        for sub in (0, 1):
            ops.append(Op("store", sub, f"store {'swa ' if sub else ''}sub{sub}",
                          {"layer": layer, "ids": f"ids{sub}", "row0": layer * n, "n": n}, n * (4 * rb + 4)))
        ops.append(Op("gather", 0, "gather sub0", {"layer": layer, "window": 0, "cu": "cu0_0", "rows": rows_full},
                      rows_full * 4 * rb + pr_full * 4 + R * 12 + 8))
        ops.append(Op("gather", 1, "gather swa sub1",
                      {"layer": layer, "window": w.window, "cu": "cu1_win", "rows": rows_win},
                      rows_win * 4 * rb + pr_win * 4 + R * 12 + 8))
    ops.append(Op("evict", 1, "evict_window sub1", {"window": w.window}, table.size * 4 + n * 4))
    buffers = {"src0_0": (full.layer_num * n, rb), "src0_1": (full.layer_num * n, rb),
               "src1_0": (swa.layer_num * n, rb), "src1_1": (swa.layer_num * n, rb),
               "out0_0": (rows_full, rb), "out0_1": (rows_full, rb), "out1_0": (rows_win, rb), "out1_1": (rows_win, rb)}
    counts = {"layers": 2 * full.layer_num, "requests": int(n), "gathered_rows_full_layer": rows_full,
              "gathered_rows_window_layer": rows_win, "full_pages": int(full.num_pages),
              "swa_pages": int(swa.num_pages)}
    return Script("swa_decode", DESCRIPTIONS["swa_decode"], list(w.shapes), ps, arrays, buffers, ops,
                  lambda op: op.kind == "gather" and op.sub == 0, "gather", counts, roofline_largest_grid=True)


ATTN_Q_HEADS = 32  # Llama-3-8B: 32 query heads on 8 KV heads
ATTN_SCALE = 128 ** -0.5


def attention_script(W, reduced: bool) -> Script:
    """The decode step of the read path: page table, then per layer store + decode attention."""
    w = W.decode_8b(num_pages=1024, num_reqs=16) if reduced else W.decode_8b()
    ps = w.page_size
    shape = w.shapes[0]
    lens = w.req_lens[0].astype(np.int32)
    R, d, hq = lens.size, shape.head_dim, ATTN_Q_HEADS
    rb = shape.row_bytes
    slots = w.store_slots[0].astype(np.int64)
    n = slots.size
    req = W.padded_table(w.req_pages[0])
    arrays = {"slots0": slots, "req0": req, "lens0": lens,
              "q0": W.irwin_hall_bf16_host(41, 0, 2 * R * hq * d).view(np.int16).reshape(R, hq, d)}
    pages_read = _pages_read(w.req_pages[0], lens, 0, ps)
    attn_bytes = int(lens.astype(np.int64).sum()) * 2 * rb + R * hq * d * (2 + 4) + pages_read * 4 + R * 4
    ops = [Op("translate", 0, "translate sub0", {"inp": "slots0", "out": "ids0"}, n * 12),
           Op("build_table", 0, "build_page_table sub0", {"inp": "req0", "out": "bt0"}, req.size * 8 + R * 4)]
    for layer in range(shape.layer_num):
        ops.append(Op("store", 0, "store mha sub0", {"layer": layer, "ids": "ids0", "row0": layer * n, "n": n},
                      n * (4 * rb + 4)))
        ops.append(Op("attention", 0, "attention sub0", {"layer": layer, "max_len": int(lens.max())}, attn_bytes))
    buffers = {"src0_0": (shape.layer_num * n, rb), "src0_1": (shape.layer_num * n, rb)}
    counts = {"layers": shape.layer_num, "requests": int(R), "q_heads": hq,
              "attended_positions_per_layer": int(lens.astype(np.int64).sum()),
              "attention_flops_per_layer": int(4 * lens.astype(np.int64).sum() * hq * d)}
    return Script("decode_attn_8b", DESCRIPTIONS["decode_attn_8b"], list(w.shapes), ps, arrays, buffers, ops,
                  lambda op: op.kind == "attention", "attn_chunk", counts, dtype="bf16")


ATTN_MLA_Q_HEADS = 16  # a 128-head MLA model at 8-way tensor parallelism
ATTN_MLA_SCALE = 192 ** -0.5  # 1 / sqrt(query-key head dim of the unabsorbed form: 128 + 64)
MLA_V_DIM = 512  # value width: the latent's compressed part ahead of its 64 rotary elements


def attention_mla_script(W, reduced: bool) -> Script:
    """The MLA read path's decode step: page table, then per layer store + MLA decode attention."""
    w = W.hybrid(num_reqs=12) if reduced else W.hybrid()
    ps = w.page_size
    shape = w.shapes[1]
    lens = w.req_lens[1].astype(np.int32)
    pages = w.req_pages[1]
    R, hq, lat = lens.size, ATTN_MLA_Q_HEADS, shape.head_dim
    rb = shape.row_bytes
    # the token decoded now sits at each request's last position
    slots = W.slots_of_requests(pages, lens, ps).astype(np.int64)[np.cumsum(lens.astype(np.int64)) - 1]
    req = W.padded_table(pages)
    arrays = {"slots0": slots, "req0": req, "lens0": lens,
              "q0": W.irwin_hall_bf16_host(43, 0, 2 * R * hq * lat).view(np.int16).reshape(R, hq, lat)}
    pages_read = _pages_read(pages, lens, 0, ps)
    attn_bytes = (int(lens.astype(np.int64).sum()) * rb + R * hq * (lat * 2 + MLA_V_DIM * 4) + pages_read * 4
                  + R * 4)
    ops = [Op("translate", 0, "translate sub0", {"inp": "slots0", "out": "ids0"}, R * 12),
           Op("build_table", 0, "build_page_table sub0", {"inp": "req0", "out": "bt0"}, req.size * 8 + R * 4)]
    for layer in range(shape.layer_num):
        ops.append(Op("store", 0, "store mla sub0", {"layer": layer, "ids": "ids0", "row0": layer * R, "n": R},
                      R * (2 * rb + 4)))
        ops.append(Op("mla_attention", 0, "mla_attention sub0", {"layer": layer, "max_len": int(lens.max())},
                      attn_bytes))
    buffers = {"src0_0": (shape.layer_num * R, rb)}
    pos = int(lens.astype(np.int64).sum())
    counts = {"layers": shape.layer_num, "requests": int(R), "q_heads": hq, "latent": lat, "v_dim": MLA_V_DIM,
              "attended_positions_per_layer": pos,
              "attention_flops_per_layer": int(2 * pos * hq * (lat + MLA_V_DIM))}
    return Script("decode_attn_mla", DESCRIPTIONS["decode_attn_mla"], [shape], ps, arrays, buffers, ops,
                  lambda op: op.kind == "mla_attention", "mla_attn_span", counts, dtype="bf16")


def fuse_layers(s: Script, name: str, gathers: bool) -> Script:
    """The same step with each sub-pool's per-layer stores (and, if asked, its per-layer
    gathers, when they share one window) replaced by one launch over all layers."""
    ops: List[Op] = []
    for op in s.ops:
        if op.kind == "store":
            prev = next((o for o in ops if o.kind == "store_layers" and o.sub == op.sub), None)
            if prev is None:
                ops.append(Op("store_layers", op.sub, op.label.replace("store", "store_layers"),
                              {"layer": op.args["layer"], "count": 1, "ids": op.args["ids"], "n": op.args["n"]},
                              op.nbytes))
            else:
                prev.args["count"] += 1
                prev.nbytes += op.nbytes
        elif op.kind == "gather" and gathers:
            prev = next((o for o in ops if o.kind == "gather_layers" and o.sub == op.sub), None)
            if prev is None:
                ops.append(Op("gather_layers", op.sub, op.label.replace("gather", "gather_layers"),
                              dict(op.args, count=1), op.nbytes))
            else:
                assert prev.args["window"] == op.args["window"]
                prev.args["count"] += 1
                prev.nbytes += op.nbytes
        else:
            ops.append(op)
    buffers = dict(s.buffers)
    if gathers:
        for k, (rows, rb) in s.buffers.items():
            if k.startswith("out"):
                count = next(o.args["count"] for o in ops if o.kind == "gather_layers" and f"out{o.sub}_" in k)
                buffers[k] = (rows * count, rb)
    totals: Dict[str, int] = {}
    for op in ops:
        totals[op.label] = totals.get(op.label, 0) + op.nbytes
    top = max(totals, key=totals.get)  # the roofline: the launch kind (label) that moves the most bytes
    kind = next(op.kind for op in ops if op.label == top)
    return Script(name, DESCRIPTIONS[name], s.shapes, s.page_size, s.arrays, buffers, ops,
                  lambda op: op.label == top, kind.split("_")[0], dict(s.counts),
                  roofline_largest_grid=s.roofline_largest_grid, roofline_nkv=s.roofline_nkv)


class GpuRunner:
    """Runs a script through libukv on the current device and stream."""

    def __init__(self, script: Script, torch, U, W, device, fill: bool = True):
        self.s = script
        self.U = U
        plan = U.ukv_pool_plan(script.shapes, script.page_size)
        n = (int(plan.required_bytes) + 7) // 8 * 8
        self.pool = U.allocate_pool(script.shapes, script.page_size, device=device,
                                    extra_bytes=n - int(plan.required_bytes))
        attn = any(op.kind in ("attention", "mla_attention") for op in script.ops)
        if fill and attn:
            W.irwin_hall_fill_device(self.pool.raw, 1)  # attention reads whole rows: finite bf16 values
        elif fill:
            W.fill_pattern_device(self.pool.raw, 1)
        self.t = {k: torch.from_numpy(np.ascontiguousarray(v)).to(device) for k, v in script.arrays.items()}
        if attn:
            q = self.t["q0"].view(torch.bfloat16)
            self.t["q0"] = q
            mx = max(op.args["max_len"] for op in script.ops if op.kind in ("attention", "mla_attention"))
            if any(op.kind == "mla_attention" for op in script.ops):
                self.t["attn_out"] = torch.empty((q.shape[0], q.shape[1], MLA_V_DIM), dtype=torch.float32,
                                                 device=device)
                need = U.ukv_mla_decode_attention_workspace_bytes(self.pool, 0, q.shape[0], q.shape[1], MLA_V_DIM,
                                                                  mx, 0)
            else:
                self.t["attn_out"] = torch.empty(q.shape, dtype=torch.float32, device=device)
                need = U.ukv_decode_attention_workspace_bytes(self.pool, 0, q.shape[0], q.shape[1], mx, 0)
            self.t["attn_ws"] = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
        for op in script.ops:  # int32 outputs of the translations, shaped like their inputs
            if "out" in op.args and op.args["out"] not in self.t:
                self.t[op.args["out"]] = torch.empty(script.arrays[op.args["inp"]].shape, dtype=torch.int32,
                                                     device=device)
        for i, (k, (rows, rb)) in enumerate(script.buffers.items()):
            if k.startswith("src"):
                self.t[k] = W.normal_bf16_device((rows, rb // 2), 100 + i, device).view(torch.uint8)
            else:
                self.t[k] = torch.empty((rows, rb), dtype=torch.uint8, device=device)
        torch.cuda.synchronize()
        self.required = int(plan.required_bytes)

    def launch(self, op: Op) -> None:
        U, t, a, sub = self.U, self.t, op.args, op.sub
        nkv = 2 if self.s.shapes[sub].kind == 0 else 1
        if op.kind == "translate":
            U.ukv_translate_loc_for_kernel(self.pool, sub, t[a["inp"]], out=t[a["out"]],
                                           v2p=t[a["v2p"]] if "v2p" in a else None)
        elif op.kind == "evict":
            U.ukv_evict_window(self.pool, t[f"map{sub}"], t["ptable"], t["lens0"], a["window"])
        elif op.kind == "translate_pages":
            U.ukv_translate_pages_for_kernel(self.pool, sub, t[a["inp"]], out=t[a["out"]],
                                             v2p=t[a["v2p"]] if "v2p" in a else None)
        elif op.kind == "translate_loc":
            U.ukv_translate_loc(self.pool, sub, t[a["inp"]], v2p=t[a["v2p"]], out=t[a["out"]])
        elif op.kind == "build_table":
            U.ukv_build_page_table(self.pool, sub, t[a["inp"]], t[f"lens{sub}"], out=t[a["out"]])
        elif op.kind == "attention":
            U.ukv_decode_attention(self.pool, sub, a["layer"], t["q0"], t[f"bt{sub}"], t[f"lens{sub}"], a["max_len"],
                                   0, ATTN_SCALE, out=t["attn_out"], workspace=t["attn_ws"])
        elif op.kind == "mla_attention":
            U.ukv_mla_decode_attention(self.pool, sub, a["layer"], t["q0"], t[f"bt{sub}"], t[f"lens{sub}"],
                                       a["max_len"], 0, ATTN_MLA_SCALE, v_dim=MLA_V_DIM, out=t["attn_out"],
                                       workspace=t["attn_ws"])
        elif op.kind == "move_pages":
            U.ukv_move_pages(self.pool, sub, t[f"pdst{sub}"], t[f"psrc{sub}"])
        elif op.kind == "remap_pages":
            U.ukv_remap_pages(self.pool, sub, t[f"v2p{sub}"], t[f"pvirt{sub}"], t[f"pdst{sub}"])
        elif op.kind == "store":
            r0, n = a["row0"], a["n"]
            k = t[f"src{sub}_0"][r0: r0 + n]
            v = t[f"src{sub}_1"][r0: r0 + n] if nkv == 2 else None
            U.ukv_store_kv(self.pool, sub, a["layer"], t[a["ids"]], k, v)
        elif op.kind == "gather":
            rows = a["rows"]
            ko = t[f"out{sub}_0"][:rows]
            vo = t[f"out{sub}_1"][:rows] if nkv == 2 else None
            U.ukv_gather_kv(self.pool, sub, a["layer"], t[f"bt{sub}"], t[f"lens{sub}"], t[a["cu"]], a["window"], ko, vo)
        elif op.kind == "move":
            U.ukv_move_kv(self.pool, sub, t[f"mdstid{sub}"], t[f"msrcid{sub}"], a["l0"], a["l1"])
        elif op.kind == "store_layers":
            n, c, l0 = a["n"], a["count"], a["layer"]
            k = t[f"src{sub}_0"][l0 * n: (l0 + c) * n].view(c, n, -1)
            v = t[f"src{sub}_1"][l0 * n: (l0 + c) * n].view(c, n, -1) if nkv == 2 else None
            U.ukv_store_kv_layers(self.pool, sub, l0, c, t[a["ids"]], k, v)
        elif op.kind == "gather_layers":
            rows, c = a["rows"], a["count"]
            ko = t[f"out{sub}_0"][: c * rows].view(c, rows, -1)
            vo = t[f"out{sub}_1"][: c * rows].view(c, rows, -1) if nkv == 2 else None
            U.ukv_gather_kv_layers(self.pool, sub, a["layer"], c, t[f"bt{sub}"], t[f"lens{sub}"], t[a["cu"]],
                                   a["window"], ko, vo)
        else:
            raise ValueError(op.kind)


def host_threads() -> int:
    """Threads for the CPU baseline: the cores this process may run on (sched_getaffinity),
    capped by OMP_NUM_THREADS where the environment sets it (a GPU machine's CPU share)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or 'unknown'."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _slices(n: int, parts: int):
    """[a, b) bounds of ``parts`` nearly equal slices of range(n) (empty ones dropped)."""
    edges = np.linspace(0, n, parts + 1).astype(np.int64)
    return [(int(a), int(b)) for a, b in zip(edges[:-1], edges[1:]) if b > a]


def _oracle_step(s: "Script", pool, h: dict, bufs: dict, threads: int, budget_s: float):
    """The step's operations in order on the CPU oracle until ``budget_s`` is spent: store,
    gather and move (the row copies) each split into ``threads`` disjoint slices run by as
    many threads at once (the oracle's C calls release the GIL; its code is unchanged), the
    rest on one thread.  Returns (bytes done, seconds, operations done)."""
    import oracle  # noqa: F401  (the pool's methods load it)
    from concurrent.futures import ThreadPoolExecutor

    ex = ThreadPoolExecutor(max_workers=threads) if threads > 1 else None

    def run(fns):
        if ex is None:
            for f in fns:
                f()
        else:
            for f in [ex.submit(f) for f in fns]:
                f.result()

    def store(sub, layer, ids, k, v):
        run([lambda a=a, b=b: pool.store(sub, layer, ids[a:b], k[a:b], None if v is None else v[a:b])
             for a, b in _slices(ids.size, threads)])

    def gather(sub, layer, bt, lens, cu, window, ko, vo):
        fns = []
        for a, b in _slices(lens.size, threads):
            c0, c1 = int(cu[a]), int(cu[b])
            fns.append(lambda a=a, b=b, c0=c0, c1=c1: pool.gather(
                sub, layer, bt[a:b], lens[a:b], cu[a:b + 1] - c0, window, ko[c0:c1], None if vo is None else vo[c0:c1]))
        run(fns)

    def move(sub, dst, src, l0, l1):
        run([lambda a=a, b=b: pool.move(sub, dst[a:b], src[a:b], l0, l1) for a, b in _slices(dst.size, threads)])

    done_bytes = done_ops = 0
    t0 = time.perf_counter()
    for op in s.ops:
        a, sub = op.args, op.sub
        nkv = 2 if s.shapes[sub].kind == 0 else 1
        if op.kind == "translate":
            h[a["out"]], _ = pool.translate(sub, h[a["inp"]], h[a["v2p"]] if "v2p" in a else None)
        elif op.kind == "evict":
            h[f"map{sub}"] = h[f"map{sub}"].copy()
            pool.evict_window(h[f"map{sub}"], h["ptable"], h["lens0"], a["window"])
        elif op.kind == "translate_pages":
            h[a["out"]], _ = pool.translate_pages(sub, h[a["inp"]], h[a["v2p"]] if "v2p" in a else None)
        elif op.kind == "translate_loc":
            h[a["out"]], _ = pool.translate_loc(sub, h[a["inp"]], h[a["v2p"]])
        elif op.kind == "build_table":
            h[a["out"]], _ = pool.build_page_table(sub, h[a["inp"]], h[f"lens{sub}"])
        elif op.kind in ("attention", "mla_attention"):
            from threadpoolctl import threadpool_limits

            from oracle import attention as oracle_attention
            mla = op.kind == "mla_attention"
            with threadpool_limits(limits=threads):  # numpy's BLAS on the same threads
                oracle_attention.decode_attention(pool, sub, a["layer"], h["q0"].view(np.uint16), h[f"bt{sub}"],
                                                  h[f"lens{sub}"], 0, ATTN_MLA_SCALE if mla else ATTN_SCALE,
                                                  a["max_len"], v_dim=MLA_V_DIM if mla else None)
        elif op.kind == "move_pages":
            pool.move_pages(sub, h[f"pdst{sub}"], h[f"psrc{sub}"])
        elif op.kind == "remap_pages":
            h[f"v2p{sub}"] = h[f"v2p{sub}"].copy()
            pool.remap_pages(sub, h[f"v2p{sub}"], h[f"pvirt{sub}"], h[f"pdst{sub}"])
        elif op.kind in ("store", "store_layers"):
            n = a["n"]
            for i in range(a.get("count", 1)):
                r0 = a["row0"] if op.kind == "store" else (a["layer"] + i) * n
                store(sub, a["layer"] + i, h[a["ids"]], bufs[f"src{sub}_0"][r0: r0 + n],
                      bufs[f"src{sub}_1"][r0: r0 + n] if nkv == 2 else None)
        elif op.kind in ("gather", "gather_layers"):
            rows = a["rows"]
            for i in range(a.get("count", 1)):
                ko = bufs[f"out{sub}_0"][i * rows:(i + 1) * rows]
                vo = bufs[f"out{sub}_1"][i * rows:(i + 1) * rows] if nkv == 2 else None
                gather(sub, a["layer"] + i, h[f"bt{sub}"], h[f"lens{sub}"], h[a["cu"]], a["window"], ko, vo)
        elif op.kind == "move":
            move(sub, h[f"mdstid{sub}"], h[f"msrcid{sub}"], a["l0"], a["l1"])
        done_bytes += op.nbytes
        done_ops += 1
        if time.perf_counter() - t0 > budget_s and not op.kind.startswith("translate"):
            break
    dt = time.perf_counter() - t0
    if ex is not None:
        ex.shutdown()
    return done_bytes, dt, done_ops


def cpu_baseline(name: str, W, budget_s: float = 10.0, threads: int = None) -> dict:
    """The CPU oracle, as written, on a bounded sample of the same workload: the step's
    operations in order until the time budget is spent, on a host envelope of the same
    row and page geometry (at most ~8 GiB), once with one thread per core the process may
    use (the row copies split into disjoint slices) and once single-threaded."""
    import oracle

    threads = host_threads() if threads is None else threads
    s = build_script(name, W, reduced=True)
    specs = [oracle.Spec(x.kind, x.layer_num, x.head_num, x.head_dim, x.v_head_dim, x.elem_bytes, x.num_pages)
             for x in s.shapes]
    req = oracle.plan(specs, s.page_size).required_bytes
    # pages touched up front; 0x3F3F is the finite bf16 value 0.746 for the attention reads
    attn = name in ("decode_attn_8b", "decode_attn_mla")
    pool = oracle.OraclePool(specs, s.page_size, np.full(req, 0x3F if attn else 0x5A, dtype=np.uint8))
    bufs = {k: np.full((rows, rb), 7, dtype=np.uint8) for k, (rows, rb) in s.buffers.items()}
    legs = {}
    for t in ((threads, 1) if threads > 1 else (1,)):
        legs[t] = _oracle_step(s, pool, dict(s.arrays), bufs, t, budget_s)
    envelope = sum(p.envelope_bytes for p in pool.plan.subs)
    shrunk = " (same row and page geometry, fewer pages)" if name.split("_fused")[0] in (
        "prefill_8b", "hybrid", "move_70b", "compact_8b", "swa_decode", "decode_8b_noreuse") else ""
    if name == "decode_attn_8b":
        shrunk = " (16 of the 256 requests on 1,024 pages of the same geometry; fp64 numpy attention over rows the " \
                 "C oracle addresses)"
    if name == "decode_attn_mla":
        shrunk = " (12 of the 128 requests, their pool sized to fit, same latent geometry; fp64 numpy attention " \
                 "over rows the C oracle addresses)"

    def describe(t):
        b, dt, n = legs[t]
        return (f"the first {n} of {len(s.ops)} operations of one step ({b / 1e9:.2f} GB) in {dt:.1f} s on "
                f"{t} thread{'s' if t > 1 else ''}")

    b, dt, _ = legs[threads]
    out = {
        "value": round(b / dt / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{name}: {describe(threads)}, host envelope {envelope / 2**30:.2f} GiB{shrunk}; row copies split "
                  f"into disjoint slices, one per thread",
        "cpu_model": cpu_model(),
        "cores_allowed": len(os.sched_getaffinity(0)),
    }
    if threads > 1:
        b1, dt1, _ = legs[1]
        out["single_thread"] = {"value": round(b1 / dt1 / 1e9, 3), "unit": "GB/s", "sample": describe(1)}
    return out


# The launches the 70% bar is judged on (row copies on the Llama-3-8B-shape pools) and the
# controls reported beside them: (key, workload, op kind, what one launch does).
BAR = (
    ("store", "prefill_8b_fused", "store_layers",
     "prefill_8b: 32,768 new tokens stored on all 32 layers in one launch (8.59 GB)"),
    ("gather_back", "prefill_8b_fused", "gather_layers",
     "prefill_8b: the 16 requests gathered back from all 32 layers in one launch (8.59 GB)"),
    ("move", "prefill_8b_fused", "move",
     "prefill_8b: 65,536 rows moved to disjoint rows on all 32 layers, K and V, in one launch (17.18 GB)"),
    ("move_70b", "move_70b", "move",
     "move_70b: 65,536 rows moved on all 80 layers of the 160 GiB Llama-3-70B-shape pool (42.95 GB)"),
    ("decode_gather_no_reuse", "decode_8b_noreuse", "gather",
     "decode_8b_noreuse: one layer's gather of the decode batch with every request on pages of its own, "
     "so no page is read twice (control for the Infinity Cache; 9.67 GB per launch)"),
)


def _launch_times(g, torch, ops, launches: int):
    """Per-launch milliseconds of ``ops`` run in order, cycled to at least ``launches``
    launches, each between two HIP events on the current stream, right after an untimed
    warm pass of the same launches (_warm_pass)."""
    seq = (ops * (-(-launches // len(ops))))[:max(launches, len(ops))]
    for op in seq[:2]:
        g.launch(op)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in seq]
    warm = _warm_pass(seq)
    torch.cuda.synchronize()
    # a spin kernel holds the GPU while the host queues the warm and the timed launches
    torch.cuda._sleep(int(spin_cycles_per_ms(torch) * (2.0 + 0.1 * (len(warm) + 2 * len(seq)))))
    for op in warm:
        g.launch(op)
    for op, (e0, e1) in zip(seq, evs):
        e0.record()
        g.launch(op)
        e1.record()
    torch.cuda.synchronize()
    return seq, [e0.elapsed_time(e1) for e0, e1 in evs]


def run_bar(torch, U, W, device, launches: int = 12) -> dict:
    """The bar's launches, each on its own pool (inputs resident in HBM, pools not
    pre-filled: a copy does not depend on the bytes it moves), plus the plain device copy
    of 4 GiB as the platform's achievable ceiling."""
    out: Dict[str, dict] = {}
    groups: Dict[str, list] = {}
    for key, wl, kind, what in BAR:
        groups.setdefault(wl, []).append((key, kind, what))
    for wl, items in groups.items():
        script = build_script(wl, W)
        t0 = time.time()
        g = GpuRunner(script, torch, U, W, device, fill=False)
        for op in script.ops:
            if op.kind.startswith("translate"):
                g.launch(op)
        log(f"[bench] bar {wl}: setup {time.time() - t0:.1f}s, pool {g.required / 2**30:.2f} GiB")
        for key, kind, what in items:
            ops = [op for op in script.ops if op.kind == kind]
            seq, ms = _launch_times(g, torch, ops, launches)
            nbytes = float(np.mean([op.nbytes for op in seq]))
            mean, med, mn = float(np.mean(ms)), float(np.median(ms)), float(np.min(ms))
            out[key] = {"what": what, "launches": len(ms), "bytes_per_launch": int(nbytes),
                        "ms_mean": num(mean, 5), "ms_median": num(med, 5), "ms_min": num(mn, 5),
                        "GBps": num(nbytes / mean / 1e6, 1), "frac": num(nbytes / mean / 1e6 / PEAK_GBPS, 4),
                        "frac_of_median": num(nbytes / med / 1e6 / PEAK_GBPS, 4)}
        flags = U.ukv_pool_error_flags(g.pool)
        assert flags == frozenset(), f"device flags raised: {flags}"
        del g
        torch.cuda.empty_cache()
    n = 4 << 30
    src = torch.empty(n, dtype=torch.uint8, device=device)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record()
        dst.copy_(src)
        e1.record()
    torch.cuda.synchronize()
    mean = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    del src, dst
    torch.cuda.empty_cache()
    return {
        "note": "per-launch HIP events on the launch's stream; GB/s and frac from the mean, frac_of_median from the "
                "median; algorithmic bytes (reads + writes the method must do)",
        "target_frac": 0.70,
        "peak_GBps": PEAK_GBPS,
        "ops": out,
        "copy_ceiling": {"what": "plain 4 GiB device-to-device copy (torch copy_)", "bytes_per_launch": 2 * n,
                         "ms_mean": num(mean, 5), "GBps": num(2 * n / mean / 1e6, 1),
                         "frac": num(2 * n / mean / 1e6 / PEAK_GBPS, 4)},
    }


_SPIN = {}


WARM_MS = 15.0  # GPU time the untimed warm pass runs for, at least (see _warm_pass)


def _warm_pass(seq) -> list:
    """The untimed launches queued just ahead of a timed pass: ``seq`` repeated until it
    moves about WARM_MS of work at 6.5 TB/s (1 to 100 times).  Started from an idle GPU, a
    sequence of bandwidth-bound launches slows down for its first ~10 ms and then recovers
    (the swa_decode full-layer gather, back to back: 725, 735, 752, 810, 846, 838, 827,
    811, 803, 779, 761, 750 us per launch; the same launches after such a pass: 698-712
    us), which looks like the GPU's power management reacting to the load; without the
    pass, short sequences measured that transient, not the kernels."""
    total = sum(op.nbytes for op in seq)
    reps = int(min(100, max(1, -(-WARM_MS * 6.5e9 // max(total, 1)))))
    return list(seq) * reps


def spin_cycles_per_ms(torch) -> float:
    """Cycles of torch's spin kernel (torch.cuda._sleep) per millisecond on this GPU, measured once."""
    if "c" not in _SPIN:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        torch.cuda.synchronize()
        e0.record()
        torch.cuda._sleep(10_000_000)
        e1.record()
        torch.cuda.synchronize()
        _SPIN["c"] = 10_000_000 / max(e0.elapsed_time(e1), 1e-3)
    return _SPIN["c"]


def run_workload(name, args, torch, U, W, device) -> dict:
    script = build_script(name, W)
    t0 = time.time()
    g = GpuRunner(script, torch, U, W, device)
    log(f"[bench] {name}: setup {time.time() - t0:.1f}s, pool {g.required / 2**30:.2f} GiB, "
        f"{len(script.ops)} launches per step")
    if args.copy_calibration:
        src = torch.full((1 << 30,), 7, dtype=torch.uint8, device=device)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        for op in script.ops:
            g.launch(op)
    torch.cuda.synchronize()
    flags = U.ukv_pool_error_flags(g.pool)
    assert flags == frozenset(), f"device flags raised: {flags}"

    mk = lambda: torch.cuda.Event(enable_timing=True)
    use_ev = args.launch_events == "roofline"
    timed = [(op, mk(), mk()) for _ in range(args.steps) for op in script.ops if use_ev and script.roofline(op)]
    it = iter(timed)
    start, end = mk(), mk()
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        for op in script.ops:
            if use_ev and script.roofline(op):
                _, e0, e1 = next(it)
                e0.record()
                g.launch(op)
                e1.record()
            else:
                g.launch(op)
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    flags = U.ukv_pool_error_flags(g.pool)
    assert flags == frozenset(), f"device flags raised: {flags}"

    step_bytes = sum(op.nbytes for op in script.ops)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    step_rows = sum(op_rows(op, script) for op in script.ops if not op.kind.startswith("translate"))
    roof_ms = roof_bytes = achieved = roof_med = roof_min = None
    if timed:
        roof_times = [e0.elapsed_time(e1) for _, e0, e1 in timed]
        roof_ms = float(np.mean(roof_times))
        roof_med, roof_min = float(np.median(roof_times)), float(np.min(roof_times))
        roof_bytes = float(np.mean([op.nbytes for op, _, _ in timed]))
        achieved = roof_bytes / (roof_ms * 1e-3) / 1e9

    # per-kind launch times, outside the timed region: all launches of a kind in step order
    # (distinct layers, so no launch re-reads what the previous one left in cache), back to
    # back between two events; a kind with a single launch per step is run three times
    agg: Dict[str, dict] = {}
    kinds: Dict[str, List[Op]] = {}
    for op in script.ops:
        kinds.setdefault(op.label.split(" sub")[0], []).append(op)
    spin = spin_cycles_per_ms(torch)
    for key, group in kinds.items():
        seq = group if len(group) > 1 else group * 3
        for op in seq[:2]:
            g.launch(op)
        e0, e1 = mk(), mk()
        torch.cuda.synchronize()
        # a spin kernel holds the GPU while the host queues the warm pass and the
        # timed sequence, so the events bracket back-to-back kernels, not the host's
        # launch rate (short kernels finish faster than Python issues them)
        warm = _warm_pass(seq)
        torch.cuda._sleep(int(spin * (2.0 + 0.1 * (len(warm) + len(seq)))))
        for op in warm:
            g.launch(op)
        e0.record()
        for op in seq:
            g.launch(op)
        e1.record()
        torch.cuda.synchronize()
        agg[key] = {"launches": len(group), "ms": e0.elapsed_time(e1) / len(seq),
                    "bytes": sum(op.nbytes for op in seq) / len(seq)}
    ops_out = {}
    for k, d in agg.items():
        gbps = d["bytes"] / (d["ms"] * 1e-3) / 1e9
        rows = sum(op_rows(op, script) for op in kinds[k]) / len(kinds[k])
        ops_out[k] = {"launches_per_step": d["launches"], "ms_per_launch": num(d["ms"], 5),
                      "bytes_per_launch": int(d["bytes"]), "GBps": num(gbps, 1),
                      "pct_of_peak": num(100 * gbps / PEAK_GBPS, 2), "rows_per_launch": int(rows),
                      "Mrows_per_s": num(rows / (d["ms"] * 1e-3) / 1e6, 2)}
    flags = U.ukv_pool_error_flags(g.pool)
    assert flags == frozenset(), f"device flags raised: {flags}"
    del g
    torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] {name}: timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(name, W)

    return {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": script.dtype,
        "data": "synthetic",
        "config": dict({"workload": script.description, "kv_dtype": "bf16", "parallelism": "single GPU",
                        "step_bytes": step_bytes, "token_rows_per_step": step_rows,
                        "launches_per_step": len(script.ops)}, **script.counts),
        "pct_of_peak": round(100.0 * value / PEAK_GBPS, 2),
        "tokens_per_s": round(step_rows / (ms_step * 1e-3), 1),
        "roofline": {
            "bound": "hbm",
            "kernel": f"{script.roofline_kernel}_kernel",
            "achieved": num(achieved, 1),
            "peak": PEAK_GBPS,
            "unit": "GB/s",
            "frac": num(achieved / PEAK_GBPS if achieved else None, 4),
            "traffic": traffic_from_profile(name, script.roofline_kernel),
            "algorithmic_bytes_per_launch": int(roof_bytes) if roof_bytes else None,
            "ms_per_launch": num(roof_ms, 5),
            "ms_per_launch_median": num(roof_med, 5),
            "ms_per_launch_min": num(roof_min, 5),
        },
        "ops": ops_out,
        "cpu_baseline": cpu,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decode_8b", help=f"one of {WORKLOADS}, a comma list, or 'all'")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--launch-events", choices=("roofline", "none"), default="roofline",
                    help="HIP events recorded inside the timed region around every launch of the roofline "
                         "kernel (default), or none")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (3 times), the reference kernel for scaling "
                         "hardware byte counters")
    ap.add_argument("--no-bar", action="store_true",
                    help="skip the bar's launches (prefill_8b store / gather-back / move, the 70B-shape move, the "
                         "no-reuse decode gather, the plain-copy ceiling) that the first line carries")
    ap.add_argument("--rocprof-summary", metavar="DIR",
                    help="no GPU work: write the kernel-trace and counter summaries of --workload under profiles/ "
                         "from the rocprofv3 runs kept in DIR (see profile_commands)")
    ap.add_argument("--profile-dir", default=PROFILE_DIR, help="where --rocprof-summary writes (default profiles/)")
    args = ap.parse_args()
    if args.rocprof_summary:
        for path in rocprof_summary(args.rocprof_summary, args.workload, out_dir=args.profile_dir):
            print(path)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path has no cross-GPU exchange (each GPU holds its own pool); "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    names = WORKLOADS if args.workload == "all" else tuple(args.workload.split(","))
    for n in names:
        if n not in WORKLOADS:
            ap.error(f"unknown workload {n}")

    import torch

    import store_gather_amd as U
    import ukv_workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    for i, n in enumerate(names):
        line = run_workload(n, args, torch, U, W, device)
        if i == 0 and not args.no_bar:
            log("[bench] the bar's launches")
            line["bar"] = run_bar(torch, U, W, device)
        print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
