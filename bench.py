"""Throughput of the unified page-major KV pool's hot path on one MI355X.

A step is one pass of the whole path over one batch: translate the batch's
token slots once, translate its block table once, then for every layer
store the batch's new K/V rows and gather every request's K/V through the
block table (plus, for the workloads that have one, the move).

Default workload (decode_8b): Llama-3-8B-shape pool, 32 layers x 8 KV heads
x head dim 128, bf16, page size 16, 4,096 pages = 65,536 slots (8 GiB of
envelopes); 256 requests with lengths uniform in [1024, 8192]; per layer
store 256 new rows and gather every request in full.

Prints one JSON line.  `value` is algorithmic GB/s (bytes the method must
read and write, 1e9 B/s) over the whole step with inputs resident in HBM;
`roofline` reports the dominant kernel (the gather) per launch, timed with
HIP events around each launch on the stream it runs on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0  # MI355X HBM3E, 8 TB/s
KERNEL_SRC = os.path.join(ROOT, "store_gather_amd", "csrc", "ukv_runtime.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gather_decode_8b_counters.txt")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def num(x, nd):
    """Rounded float, or None for a figure that was not measured."""
    return None if x != x else round(x, nd)


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile():
    """HBM bytes per gather launch from the committed counter summary, or None when
    the summary is missing or was taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return int(m_bytes.group(1))


# ----------------------------------------------------------------------------
# the decode_8b workload on the GPU
# ----------------------------------------------------------------------------

class DecodeStep:
    def __init__(self, torch, U, W, device, seed=0):
        self.torch = torch
        self.U = U
        w = W.decode_8b(seed=seed)
        self.w = w
        shape = w.shapes[0]
        self.L = shape.layer_num
        self.ps = w.page_size
        plan = U.ukv_pool_plan(w.shapes, self.ps)
        n = (int(plan.required_bytes) + 7) // 8 * 8
        t0 = time.time()
        self.pool = U.allocate_pool(w.shapes, self.ps, device=device, extra_bytes=n - int(plan.required_bytes))
        W.fill_pattern_device(self.pool.raw, 1)
        self.rb = self.pool.row_bytes(0)
        slots = w.store_slots[0]
        self.n_new = slots.size
        self.slots = torch.from_numpy(slots).to(device)
        table = W.padded_table(w.req_pages[0])
        self.table = torch.from_numpy(table).to(device)
        self.lens_np = w.req_lens[0].astype(np.int32)
        self.lens = torch.from_numpy(self.lens_np).to(device)
        cu = W.out_offsets(self.lens_np)
        self.cu = torch.from_numpy(cu).to(device)
        self.out_rows = int(cu[-1])
        self.pages_read = int(sum(len(p) for p in w.req_pages[0]))
        H, D = shape.head_num, shape.head_dim
        # new K / V rows of every layer: bf16 N(0,1), drawn on the device
        self.k_new = W.normal_bf16_device((self.L, self.n_new, H, D), seed + 101, device)
        self.v_new = W.normal_bf16_device((self.L, self.n_new, H, D), seed + 202, device)
        self.k_out = torch.empty((self.out_rows, H, D), dtype=torch.bfloat16, device=device)
        self.v_out = torch.empty_like(self.k_out)
        self.ids = torch.empty(self.n_new, dtype=torch.int32, device=device)
        self.bt = torch.empty_like(self.table)
        torch.cuda.synchronize()
        log(f"[bench] decode_8b setup {time.time() - t0:.1f}s: pool {plan.required_bytes / 2**30:.2f} GiB, "
            f"{len(self.lens_np)} requests, {self.out_rows} gathered rows per layer, {self.n_new} new rows")

    # algorithmic bytes (reads + writes the method must do)
    def bytes_translate(self):
        return self.n_new * (8 + 4) + self.table.numel() * (4 + 4)

    def bytes_store_launch(self):
        return self.n_new * (4 * self.rb + 4)

    def bytes_gather_launch(self):
        R = len(self.lens_np)
        return self.out_rows * 4 * self.rb + self.pages_read * 4 + R * 4 + (R + 1) * 8

    def bytes_step(self):
        return self.bytes_translate() + self.L * (self.bytes_store_launch() + self.bytes_gather_launch())

    def run(self, timers=None):
        """One step; ``timers`` (optional) is an iterator of (store, gather) event pairs,
        recorded around every launch on the stream the kernels run on."""
        U = self.U
        U.ukv_translate_loc_for_kernel(self.pool, 0, self.slots, out=self.ids)
        U.ukv_translate_pages_for_kernel(self.pool, 0, self.table, out=self.bt)
        for l in range(self.L):
            ev = next(timers) if timers is not None else None
            if ev and ev[0]:
                ev[0][0].record()
            U.ukv_store_kv(self.pool, 0, l, self.ids, self.k_new[l], self.v_new[l])
            if ev and ev[0]:
                ev[0][1].record()
            if ev and ev[1]:
                ev[1][0].record()
            U.ukv_gather_kv(self.pool, 0, l, self.bt, self.lens, self.cu, 0, self.k_out, self.v_out)
            if ev and ev[1]:
                ev[1][1].record()


def cpu_baseline(W, budget_s=12.0, seed=0):
    """The CPU oracle, as written, on a bounded sample of the same workload: translate
    the batch and the block table, then store + gather layer by layer until the
    time budget is spent.  Same pool geometry (8 GiB host envelope)."""
    import oracle

    w = W.decode_8b(seed=seed)
    shape = w.shapes[0]
    ps = w.page_size
    spec = oracle.Spec(shape.kind, shape.layer_num, shape.head_num, shape.head_dim, shape.v_head_dim,
                       shape.elem_bytes, shape.num_pages)
    req = oracle.plan([spec], ps).required_bytes
    raw = np.full(req, 0x5A, dtype=np.uint8)  # touched, so the timing sees no first-touch faults
    pool = oracle.OraclePool([spec], ps, raw)
    rb = pool.row_bytes(0)
    slots = w.store_slots[0]
    table = W.padded_table(w.req_pages[0])
    lens = w.req_lens[0]
    cu = W.out_offsets(lens)
    rows = int(cu[-1])
    k_out = np.full((rows, rb), 1, np.uint8)
    v_out = np.full((rows, rb), 2, np.uint8)
    k_new = np.full((slots.size, rb), 3, np.uint8)
    v_new = np.full((slots.size, rb), 4, np.uint8)
    pages_read = int(sum(len(p) for p in w.req_pages[0]))
    t0 = time.perf_counter()
    ids, _ = pool.translate(0, slots)
    bt, _ = pool.translate_pages(0, table)
    nbytes = slots.size * 12 + table.size * 8
    layers = 0
    while layers < shape.layer_num:
        pool.store(0, layers, ids, k_new, v_new)
        pool.gather(0, layers, bt, lens, cu, 0, k_out, v_out)
        nbytes += slots.size * (4 * rb + 4) + rows * 4 * rb + pages_read * 4 + len(lens) * 12 + 8
        layers += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {
        "value": round(nbytes / dt / 1e9, 3),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"decode_8b: translate + {layers} of {shape.layer_num} layers of (store 256 rows + gather "
                  f"{rows} rows) on an 8 GiB host envelope, single-threaded C oracle, {dt:.1f} s",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--launch-events", choices=("gather", "all", "none"), default="gather",
                    help="HIP events recorded around launches inside the timed region: around every "
                         "gather (default), around gathers and stores, or none")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (3 times), the reference kernel for "
                         "scaling hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path has no cross-GPU exchange (each GPU holds its own pool); "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import store_gather_amd as U
    import ukv_workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    step = DecodeStep(torch, U, W, device)
    if args.copy_calibration:
        src = torch.full((1 << 30,), 7, dtype=torch.uint8, device=device)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    flags = U.ukv_pool_error_flags(step.pool)
    assert flags == frozenset(), f"device flags raised: {flags}"

    n_ev = args.steps * step.L
    mk = lambda: torch.cuda.Event(enable_timing=True)
    ev_store = [(mk(), mk()) if args.launch_events == "all" else None for _ in range(n_ev)]
    ev_gather = [(mk(), mk()) if args.launch_events != "none" else None for _ in range(n_ev)]
    start, end = mk(), mk()
    torch.cuda.synchronize()
    start.record()
    timers = iter(list(zip(ev_store, ev_gather)))
    for _ in range(args.steps):
        step.run(timers)
    end.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps
    g_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev_gather])) if ev_gather[0] else float("nan")
    s_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev_store])) if ev_store[0] else float("nan")
    flags = U.ukv_pool_error_flags(step.pool)
    assert flags == frozenset(), f"device flags raised: {flags}"

    value = step.bytes_step() / (ms_step * 1e-3) / 1e9
    g_gbps = step.bytes_gather_launch() / (g_ms * 1e-3) / 1e9
    s_gbps = step.bytes_store_launch() / (s_ms * 1e-3) / 1e9
    traffic = traffic_from_profile()

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(W)

    out = {
        "metric": "KV store/gather/move HBM GB/s and % of peak, Llama-3-8B-shape pool",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {
            "workload": "decode_8b: Llama-3-8B-shape pool (32 layers, 8 KV heads x 128, bf16, page 16, "
                        "4096 pages = 65,536 slots, 8 GiB); 256 requests, lengths U[1024, 8192], pages shared "
                        "cyclically from one seeded permutation; per step: translate 256 slots and the block "
                        "table once, then per layer store 256 new K/V rows and gather every request in full",
            "kv_dtype": "bf16",
            "global_batch": len(step.lens_np),
            "gathered_rows_per_layer": step.out_rows,
            "new_rows_per_layer": step.n_new,
            "layers": step.L,
            "parallelism": "single GPU",
        },
        "pct_of_peak": round(100.0 * value / PEAK_GBPS, 2),
        "tokens_per_s": {
            "gathered": round(step.out_rows * step.L / (ms_step * 1e-3), 1),
            "stored": round(step.n_new * step.L / (ms_step * 1e-3), 1),
        },
        "per_launch": {
            "gather_ms": num(g_ms, 4), "gather_GBps": num(g_gbps, 1),
            "store_ms": num(s_ms, 5), "store_GBps": num(s_gbps, 1),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "gather_kernel",
            "achieved": num(g_gbps, 1),
            "peak": PEAK_GBPS,
            "unit": "GB/s",
            "frac": num(g_gbps / PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": step.bytes_gather_launch(),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
