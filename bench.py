#!/usr/bin/env python3
"""Benchmark of the quantized-embedding hot path on one MI355X.

Headline (the step that is timed for `value`): the fused dequantize +
weighted-sum pooled lookup (qemb_bag_forward) of the multi-hot workload --
64 tables x 1M rows, d=128, rows range-quantized to INT4 with fp16 scale and
bias, batch 16384 per table, bag lengths U{1..64}, Zipf(1.05) ids, U(0,1)
per-id weights -- reported as pooled lookups/s, with the kernel's achieved
algorithmic HBM bandwidth against the 8 TB/s peak.  Four pre-generated index
batches rotate across steps.  The table is generated on the GPU and packed by
the library's own quantizer before timing starts; inputs are resident in HBM.

Beside it, in the same run: the INT8 table, a uniform-id control (no Zipf
reuse), the same lookups over k-means codebook rows, the dot interaction
of the pooled output with a dense vector per sample, the quantizer workload
(5e7 x 64 rows: range, greedy and codebook quantize, dequantize, normalized
l2), and the CPU oracle timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F32_PEAK_TFLOPS = 157.3   # MI355X dense fp32 matrix
# fp32 VALU issue peak in lane-instructions/s: 256 CUs x 128 lanes x 2.4 GHz
# (the published 157.3 TFLOP/s fp32 vector peak counts an FMA as 2 flops;
# the counters show more than one wave64 VALU instruction per CU per cycle,
# so the 128 lanes per CU per clock are two wave64 instructions)
VALU_PEAK_LANE_INSTS = 256 * 128 * 2.4e9
HEADLINE_KERNEL = "bag_seg_kernel<4, int, true, 24, 1>"
COUNTERS = os.path.join(ROOT, "profiles", "bag_seg_int4_multihot_counters.md")
QUANT_COUNTERS = os.path.join(ROOT, "profiles", "quantizer_workload_counters.md")


def log(msg: str) -> None:
    print("[bench] " + msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batches", type=int, default=4, help="index batches rotated across steps")
    ap.add_argument("--no-extras", action="store_true", help="headline only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--codebook-only", action="store_true",
                    help="only the codebook-row lookup of the multi-hot workload (for profiling)")
    ap.add_argument("--compress-only", action="store_true",
                    help="error-bounded compression of the pooled output only")
    ap.add_argument("--interaction-only", action="store_true",
                    help="only one INT4 lookup and the dot interaction on its output (for profiling)")
    ap.add_argument("--gather-floor", action="store_true",
                    help="only the INT4 lookup and the gather floor of its memory traffic")
    ap.add_argument("--quantizer-only", action="store_true",
                    help="only the quantizer workload (for profiling)")
    ap.add_argument("--uniform-ids", action="store_true",
                    help="only the INT4 lookup with ids uniform over each table (the no-reuse "
                         "control, for profiling)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    return ap.parse_args()


def algorithmic_bag_bytes(nnz: int, n_bags: int, dim: int, bits: int, idx_bytes: int,
                          weighted: bool) -> int:
    """Bytes one lookup call must move at minimum: the unpadded packed row
    (codes + fp16 scale + fp16 bias) and the id (+ weight) per lookup, the CSR
    offsets, and the fp32 output."""
    row = (dim * bits + 7) // 8 + 4
    per = row + idx_bytes + (4 if weighted else 0)
    return nnz * per + (n_bags + 1) * idx_bytes + n_bags * dim * 4


def algorithmic_codebook_bytes(nnz: int, n_bags: int, dim: int, idx_bytes: int,
                               weighted: bool) -> int:
    """The same minimum for codebook rows: 16 fp32 levels (64 bytes) and the
    unpadded 4-bit codes per lookup."""
    per = 64 + (dim + 1) // 2 + idx_bytes + (4 if weighted else 0)
    return nnz * per + (n_bags + 1) * idx_bytes + n_bags * dim * 4


def counter_record(path):
    """The json block of a committed counter summary, or None when the
    summary is missing or was taken on a different kernel source."""
    try:
        text = open(path).read()
    except OSError:
        return None
    start = text.find("```json")
    if start < 0:
        return None
    end = text.find("```", start + 7)
    rec = json.loads(text[start + 7:end])
    from int4_row_wise_amd import build as qbuild
    src = qbuild.source_sha256()
    if rec.get("source_sha256") != src or qbuild.built_source_sha256() != src:
        return None
    return rec


def measured_traffic():
    """HBM bytes per launch of the headline kernel from the committed counter
    summary (FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by what the
    counter reads for a plain device copy of known size), or None."""
    rec = counter_record(COUNTERS)
    if rec is None:
        return None
    return 1024.0 * (rec["fetch_kib_per_dispatch"] * rec["fetch_scale"] +
                     rec["write_kib_per_dispatch"] * rec["write_scale"])


class Timer:
    """HIP events on torch's current stream (the stream the library launches on)."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def __enter__(self):
        self.s = self.torch.cuda.Event(enable_timing=True)
        self.e = self.torch.cuda.Event(enable_timing=True)
        self.s.record()
        return self

    def __exit__(self, *a):
        self.e.record()
        self.pairs.append((self.s, self.e))

    def ms(self):
        self.torch.cuda.synchronize()
        return [s.elapsed_time(e) for s, e in self.pairs]


def build_table(q, synth, torch, w, bits_list, dev):
    """Generate each fp32 table on the GPU and pack it with the library's
    range quantizer; returns {bits: packed [total_rows, S]}."""
    out = {}
    for bits in bits_list:
        out[bits] = torch.empty((w.total_rows, q.row_stride(w.dim, bits)), dtype=torch.uint8,
                                device=dev)
    r0 = 0
    for t in range(w.n_tables):
        n = w.rows[t]
        x = synth.table_values_torch(w, t, 0, n, dev)
        for bits in bits_list:
            q.quantize_rowwise(x, bits, q.RANGE, out=out[bits][r0:r0 + n])
        del x
        r0 += n
    torch.cuda.synchronize()
    return out


def to_dev(torch, a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def bench_bags(q, torch, packed, toff, batches, w, bits, steps, warmup, out):
    """Time `steps` lookups rotating over the batches; returns per-launch ms
    (HIP events around each launch) and the wall time of the timed region.
    bits None: codebook rows."""
    def call(k):
        b = batches[k % len(batches)]
        if bits is None:
            q.bag_forward_codebook(packed, toff, w.batch, w.dim, b["idx"], b["offs"], b["w"], out=out)
        else:
            q.bag_forward(packed, toff, w.batch, w.dim, bits, b["idx"], b["offs"], b["w"], out=out)

    for k in range(warmup):
        call(k)
    torch.cuda.synchronize()
    tm = Timer(torch)
    t0 = time.perf_counter()
    for k in range(steps):
        with tm:
            call(k)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return tm.ms(), wall


def cpu_baseline(oracle, synth, torch, w, bits, batch0, dev, budget_s=15.0):
    """The oracle (plain C, OpenMP over bags) on the first tables of the
    workload: every bag of those tables, over the oracle's own packing of
    the same generated values.  Returns lookups/s over the sample."""
    n_tab = 8
    xs = [synth.table_values_torch(w, t, 0, w.rows[t], dev).cpu().numpy() for t in range(n_tab)]
    x = np.concatenate(xs)
    del xs
    packed = oracle.quantize_rowwise(x, bits, oracle.RANGE)
    del x
    B = w.batch
    offs = batch0["offs_np"][: n_tab * B + 1]
    nnz = int(offs[-1])
    idx = batch0["idx_np"][:nnz]
    wts = batch0["w_np"][:nnz]
    toff = np.array([0] + list(np.cumsum(w.rows[:n_tab])), dtype=np.int64)
    reps, t_total = 0, 0.0
    while t_total < budget_s and reps < 1000:
        t0 = time.perf_counter()
        oracle.bag_forward(packed, toff, B, w.dim, bits, idx, offs, wts)
        t_total += time.perf_counter() - t0
        reps += 1
    threads = oracle.num_threads()
    # one thread, one table (a shorter sample)
    offs1 = offs[: B + 1]
    n1 = int(offs1[-1])
    oracle.set_threads(1)
    try:
        t0 = time.perf_counter()
        oracle.bag_forward(packed, toff, B, w.dim, bits, idx[:n1], offs1, wts[:n1])
        t1 = time.perf_counter() - t0
    finally:
        oracle.set_threads(threads)
    return {
        "value": nnz * reps / t_total, "unit": "lookups/s", "cores": threads,
        "kind": "oracle",
        "sample": "tables 0-%d of %d (all %d bags each, %d lookups), %d repetitions, oracle-packed "
                  "INT4 rows of the same generated values" % (n_tab - 1, w.n_tables, B, nnz, reps),
        "seconds": round(t_total, 2),
        "one_thread_lookups_per_s": n1 / t1,
        "affinity_cores": len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model(),
    }


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def launch_stats(ms):
    a = np.asarray(ms, dtype=np.float64)
    return {"mean_ms": float(a.mean()), "median_ms": float(np.median(a)), "min_ms": float(a.min()),
            "p90_ms": float(np.percentile(a, 90)), "launches": int(a.size)}


def device_copy_gbps(torch, dev, nbytes=1 << 30, reps=10):
    """Achievable bandwidth of a plain device-to-device copy on this GPU
    (read + write bytes per second), for context next to the rooflines."""
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    a.fill_(1)
    b.copy_(a)
    torch.cuda.synchronize()
    tm = Timer(torch)
    for _ in range(reps):
        with tm:
            b.copy_(a)
    ms = float(np.median(tm.ms()))
    del a, b
    return 2 * nbytes / (ms * 1e-3) / 1e9


def stream_ceiling(torch, dev, nbytes=2 << 30, reps=10):
    """HBM rates of the plainest access patterns on this GPU (libqemb_floor.so:
    16-byte non-temporal loads and stores, u words per lane and round, a
    grid-stride loop): read only, write only, and a copy (read + write
    bytes), GB/s of the median launch over `nbytes` per array, the best of a
    few launch shapes (workgroups, u)."""
    import ctypes
    from int4_row_wise_amd import build as qbuild
    lib = ctypes.CDLL(qbuild.FLOOR_LIB)
    p, i32 = ctypes.c_void_p, ctypes.c_int32
    lib.qemb_floor_stream.argtypes = [p, p, ctypes.c_int64, i32, i32, i32, p, p]
    lib.qemb_floor_stream.restype = ctypes.c_int
    a = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    b = torch.empty(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    n = nbytes // 16
    res = {"bytes_per_array": nbytes}
    for mode, name, moved in ((0, "read", nbytes), (1, "write", nbytes), (2, "copy", 2 * nbytes)):
        best = (0.0, None)
        for grid, u in ((1024, 2), (4096, 4), (8192, 8), (16384, 4)):
            def call():
                rc = lib.qemb_floor_stream(a.data_ptr(), b.data_ptr(), n, mode, grid, u, sink.data_ptr(), st)
                assert rc == 0, rc
            call()
            torch.cuda.synchronize()
            tm = Timer(torch)
            for _ in range(reps):
                with tm:
                    call()
            rate = moved / (float(np.median(tm.ms())) * 1e-3) / 1e9
            best = max(best, (rate, "%d workgroups, %d words per lane" % (grid, u)), key=lambda x: x[0])
        res[name + "_GBps"], res[name + "_shape"] = best
    del a, b
    return res


def bench_cold(q, torch, packed, toff, batch, w, bits, out, dev, reps=5):
    """Lookups with L2 and the MALL flushed first: each launch follows a
    write of a 1 GiB scratch buffer (not timed)."""
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    ms = []
    for _ in range(reps):
        scratch.fill_(reps)
        torch.cuda.synchronize()
        tm = Timer(torch)
        with tm:
            q.bag_forward(packed, toff, w.batch, w.dim, bits, batch["idx"], batch["offs"], batch["w"],
                          out=out)
        ms.extend(tm.ms())
    del scratch
    return ms


def quantizer_extras(q, synth, torch, dev, oracle=None, reps=3):
    """The quantizer workload: one 5e7 x 64 table (99% N(0,0.02) / 1%
    Laplace(0,0.2)), range and greedy INT4 quantization (200 bins, 100
    steps), full-table dequantize, normalized l2 of both encodings; with
    `oracle`, the oracle's rows/s for the same operations on a row prefix."""
    w = synth.workload(5)
    rows, dim = w.rows[0], w.dim
    x = synth.table_values_torch(w, 0, 0, rows, dev)
    S = q.row_stride(dim, 4)
    packed = torch.empty((rows, S), dtype=torch.uint8, device=dev)
    y = torch.empty((rows, dim), dtype=torch.float32, device=dev)
    res = {"workload": w.name, "rows": rows, "dim": dim}
    in_b, out_b = rows * dim * 4, rows * ((dim * 4 + 7) // 8 + 4)

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        tm = Timer(torch)
        for _ in range(n):
            with tm:
                fn()
        return float(np.mean(tm.ms()))

    ms = timed(lambda: q.quantize_rowwise(x, 4, q.RANGE, out=packed), reps)
    res["range_quantize"] = {"ms": ms, "rows_per_s": rows / ms * 1e3,
                             "GBps": (in_b + out_b) / ms / 1e6,
                             "hbm_frac": (in_b + out_b) / ms / 1e6 / HBM_PEAK_GBS}
    res["range_l2"] = q.l2_error(x, packed, 4)
    ms = timed(lambda: q.dequantize(packed, dim, 4, out=y), reps)
    res["dequantize"] = {"ms": ms, "rows_per_s": rows / ms * 1e3, "GBps": (in_b + out_b) / ms / 1e6,
                         "hbm_frac": (in_b + out_b) / ms / 1e6 / HBM_PEAK_GBS}
    ms = timed(lambda: q.quantize_rowwise(x, 4, q.GREEDY, w.n_bins, w.n_steps, out=packed), 1)
    res["greedy_quantize"] = {"ms": ms, "rows_per_s": rows / ms * 1e3,
                              "windows_per_row": 2 * w.n_steps + 1}
    # VALU issue rate: the kernel's wave64 VALU instructions per launch as
    # counted by SQ_INSTS_VALU on this source (committed summary), over this
    # run's launch time, against 128 lanes per CU per clock
    rec = counter_record(QUANT_COUNTERS)
    if rec is not None and rec["rows"] == rows and rec["dim"] == dim and \
            rec["windows_per_row"] == 2 * w.n_steps + 1:
        lane_insts = rec["valu_insts_per_dispatch"] * 64
        cycles = rec["grbm_gui_active_per_dispatch"] / rec["xcds"]
        res["greedy_quantize"].update({
            "bound": "alu", "valu_lane_insts_per_launch": lane_insts,
            "lane_insts_per_element_window": lane_insts / (rows * dim * (2 * w.n_steps + 1)),
            "valu_lane_insts_per_s": lane_insts / ms * 1e3,
            "valu_frac": lane_insts / ms * 1e3 / VALU_PEAK_LANE_INSTS,
            "valu_peak_lane_insts_per_s": VALU_PEAK_LANE_INSTS,
            "counted_insts_per_cu_cycle": rec["valu_insts_per_dispatch"] / (256 * cycles),
            "counted_clock_ghz": cycles / (rec["traced_avg_us"] * 1e-6) / 1e9})
    res["greedy_l2"] = q.l2_error(x, packed, 4)
    del packed
    cb = torch.empty((rows, q.codebook_row_stride(dim)), dtype=torch.uint8, device=dev)
    ms = timed(lambda: q.quantize_codebook(x, q.CODEBOOK_ITERS, out=cb), 1)
    res["codebook_quantize"] = {"ms": ms, "rows_per_s": rows / ms * 1e3, "n_iter": q.CODEBOOK_ITERS,
                                "bytes_per_row": cb.shape[1]}
    res["codebook_l2"] = q.l2_error_codebook(x, cb)
    # the baselines the greedy search is compared with, same packed format
    pk = torch.empty((rows, S), dtype=torch.uint8, device=dev)
    for name, method, param in (("symmetric", q.SYMMETRIC, 0.0), ("percentile_0.99", q.PERCENTILE, 0.99),
                                ("aciq", q.ACIQ, 0.0)):
        ms = timed(lambda: q.quantize_baseline(x, 4, method, param, out=pk), 1)
        res["baseline_" + name] = {"ms": ms, "rows_per_s": rows / ms * 1e3,
                                   "GBps": (in_b + out_b) / ms / 1e6,
                                   "hbm_frac": (in_b + out_b) / ms / 1e6 / HBM_PEAK_GBS,
                                   "l2": q.l2_error(x, pk, 4)}
    del pk
    # 2-bit rows (range), the narrowest width of the comparison
    pk2 = torch.empty((rows, q.row_stride(dim, 2)), dtype=torch.uint8, device=dev)
    out2_b = rows * ((dim * 2 + 7) // 8 + 4)
    ms = timed(lambda: q.quantize_rowwise(x, 2, q.RANGE, out=pk2), reps)
    res["int2_range_quantize"] = {"ms": ms, "rows_per_s": rows / ms * 1e3,
                                  "GBps": (in_b + out2_b) / ms / 1e6,
                                  "hbm_frac": (in_b + out2_b) / ms / 1e6 / HBM_PEAK_GBS,
                                  "l2": q.l2_error(x, pk2, 2)}
    del pk2
    res["l2_mean_row_by_method"] = {
        k: res[k]["mean_row"] for k in ("codebook_l2", "greedy_l2", "range_l2")} | {
        "baseline_" + n + "_l2": res["baseline_" + n]["l2"]["mean_row"]
        for n in ("symmetric", "percentile_0.99", "aciq")} | {
        "int2_range_l2": res["int2_range_quantize"]["l2"]["mean_row"]}
    cb_out = rows * cb.shape[1]
    ms = timed(lambda: q.dequantize_codebook(cb, dim, out=y), reps)
    res["codebook_dequantize"] = {"ms": ms, "rows_per_s": rows / ms * 1e3,
                                  "GBps": (in_b + cb_out) / ms / 1e6,
                                  "hbm_frac": (in_b + cb_out) / ms / 1e6 / HBM_PEAK_GBS}
    if oracle is not None:
        x_np = x[: 1 << 20].cpu().numpy()
        rr = oracle_quantizer_rates(oracle, x_np, 4, oracle.RANGE, w.n_bins, w.n_steps, 1 << 20, 1 << 16)
        rg = oracle_quantizer_rates(oracle, x_np, 4, oracle.GREEDY, w.n_bins, w.n_steps, 1 << 16, 1 << 12)
        res["cpu_oracle"] = {
            "kind": "oracle", "cores": rr["quantize"]["cores"],
            "range_rows_per_s": rr["quantize"]["per_s"],
            "range_rows_per_s_one_thread": rr["quantize"]["one_thread_per_s"],
            "greedy_rows_per_s": rg["quantize"]["per_s"],
            "greedy_rows_per_s_one_thread": rg["quantize"]["one_thread_per_s"],
            "dequantize_rows_per_s": rr["dequantize"]["per_s"],
            "dequantize_rows_per_s_one_thread": rr["dequantize"]["one_thread_per_s"],
            "sample": "first 2^20 rows (range, dequantize; one thread 2^16) and 2^16 rows (greedy; "
                      "one thread 2^12) of the table"}
    del x, y, cb
    torch.cuda.empty_cache()
    return res


def codebook_extras(q, synth, torch, w, toff, batches, out, dev, n_bags, steps=20, warmup=3):
    """The multi-hot workload over codebook rows (16 fp32 levels per row from
    k-means, 4-bit codes): the tables quantized by the library's codebook
    quantizer, then the same rotating batches through the codebook lookup."""
    S = q.codebook_row_stride(w.dim)
    cb = torch.empty((w.total_rows, S), dtype=torch.uint8, device=dev)
    tm = Timer(torch)
    r0 = 0
    for t in range(w.n_tables):
        n = w.rows[t]
        x = synth.table_values_torch(w, t, 0, n, dev)
        with tm:
            q.quantize_codebook(x, q.CODEBOOK_ITERS, out=cb[r0:r0 + n])
        del x
        r0 += n
    qms = float(np.sum(tm.ms()))
    ms, _ = bench_bags(q, torch, cb, toff, batches, w, None, steps, warmup, out)
    nnz = [batches[k % len(batches)]["nnz"] for k in range(steps)]
    byt = [algorithmic_codebook_bytes(n, n_bags, w.dim, 4, True) for n in nnz]
    gbps = float(np.mean(byt)) / (np.mean(ms) * 1e-3) / 1e9
    del cb
    torch.cuda.empty_cache()
    return {"quantize_ms_all_tables": qms, "quantize_rows_per_s": w.total_rows / qms * 1e3,
            "n_iter": q.CODEBOOK_ITERS, "row_bytes": S,
            "lookups_per_s": float(np.mean(nnz)) / (np.mean(ms) * 1e-3),
            "avg_launch_ms": float(np.mean(ms)), "launch_ms": launch_stats(ms),
            "GBps": gbps, "hbm_frac": gbps / HBM_PEAK_GBS}


def interaction_extras(q, torch, pooled, w, dev, steps=20, warmup=3):
    """The dot interaction on the lookup's pooled output of the multi-hot
    workload (B=16384 samples, T=64 tables, d=128) with a N(0,1) dense
    vector per sample: the dense vector, then the dots of every pair of
    distinct rows of [dense; pooled]."""
    B, T, dim = pooled.shape
    gen = torch.Generator(device=dev)
    gen.manual_seed(4)
    dense = torch.randn((B, dim), generator=gen, device=dev, dtype=torch.float32)
    W = q.interaction_width(T, dim)
    res_out = torch.empty((B, W), dtype=torch.float32, device=dev)
    for _ in range(warmup):
        q.dot_interaction(dense, pooled, out=res_out)
    torch.cuda.synchronize()
    tm = Timer(torch)
    for _ in range(steps):
        with tm:
            q.dot_interaction(dense, pooled, out=res_out)
    ms = float(np.mean(tm.ms()))
    # bytes: every input row read once, the output row written once
    byt = B * (4 * dim * (T + 1) + 4 * W)
    # matrix-core flops issued: 16x16 tiles on or below the diagonal of the
    # pooled Gram matrix, 2*16*16*16 flops per 16 columns
    nbp = (T + 15) // 16
    kc = (dim + 15) // 16
    mfma_flops = B * (nbp * (nbp + 1) // 2) * kc * 2 * 16 * 16 * 16
    useful = B * 2 * dim * T * (T + 1) // 2
    return {"samples": B, "tables": T, "dim": dim, "out_width": W, "avg_launch_ms": ms,
            "samples_per_s": B / (ms * 1e-3), "GBps": byt / (ms * 1e-3) / 1e9,
            "hbm_frac": byt / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "mfma_TFLOPs": mfma_flops / (ms * 1e-3) / 1e12,
            "mfma_frac": mfma_flops / (ms * 1e-3) / 1e12 / MFMA_F32_PEAK_TFLOPS,
            "useful_TFLOPs": useful / (ms * 1e-3) / 1e12, "bytes_per_launch": byt}


def compress_extras(q, torch, pooled, dev, steps=20, warmup=3):
    """Error-bounded compression of the lookup's pooled output (the payload a
    table-sharded model sends in its all-to-all) and its inverse.  The pages
    give no bound; each table's bound is 1 % of the standard deviation of its
    pooled values.  Algorithmic bytes: compression reads every vector once and
    writes the records and offsets; decompression reads the records and
    offsets and writes every vector."""
    B, T, dim = pooled.shape
    n = B * T
    eb = (0.01 * pooled.std(dim=(0, 2))).float().contiguous()
    buf = torch.empty(q.compress_bound(n, dim), dtype=torch.uint8, device=dev)
    offs = torch.empty(n + 1, dtype=torch.int64, device=dev)
    ws = torch.empty(max(q.compress_workspace_bytes(n), 16), dtype=torch.uint8, device=dev)
    y = torch.empty((n, dim), dtype=torch.float32, device=dev)
    for _ in range(warmup):
        q.compress_pooled(pooled, eb, out=buf, offs=offs, workspace=ws)
        q.decompress_pooled(buf, offs, dim, eb, y=y)
    torch.cuda.synchronize()
    total = int(offs[-1].item())
    tc, td = Timer(torch), Timer(torch)
    for _ in range(steps):
        with tc:
            q.compress_pooled(pooled, eb, out=buf, offs=offs, workspace=ws)
    for _ in range(steps):
        with td:
            q.decompress_pooled(buf, offs, dim, eb, y=y, in_bytes=total)
    msc, msd = float(np.mean(tc.ms())), float(np.mean(td.ms()))
    err = float((y.view(B, T, dim) - pooled).abs().div(eb.view(1, T, 1)).max().item())
    raw = n * dim * 4
    bc = raw + total + 8 * (n + 1)
    bd = total + 8 * (n + 1) + raw
    return {"vectors": n, "dim": dim, "tables": T, "bound": "1 % of each table's std",
            "compressed_bytes": total, "ratio": raw / total, "max_err_over_bound": err,
            "compress_ms": msc, "compress_GBps": bc / (msc * 1e-3) / 1e9,
            "compress_hbm_frac": bc / (msc * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "decompress_ms": msd, "decompress_GBps": bd / (msd * 1e-3) / 1e9,
            "decompress_hbm_frac": bd / (msd * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "compress_bytes_per_call": bc, "decompress_bytes_per_call": bd}


def oracle_rate(oracle, fn, n_all: int, n_one: int, budget_s: float = 4.0):
    """Units/s of the oracle running fn(n) over the first n units: all of the
    oracle's threads on n_all units (repeated within budget_s), and one
    thread on n_one units."""
    threads = oracle.num_threads()
    reps, t_all = 0, 0.0
    while reps == 0 or (t_all < budget_s and reps < 20):
        t0 = time.perf_counter()
        fn(n_all)
        t_all += time.perf_counter() - t0
        reps += 1
    oracle.set_threads(1)
    try:
        t0 = time.perf_counter()
        fn(n_one)
        t_one = time.perf_counter() - t0
    finally:
        oracle.set_threads(threads)
    return {"per_s": n_all * reps / t_all, "cores": threads, "sample": n_all, "reps": reps,
            "one_thread_per_s": n_one / t_one, "one_thread_sample": n_one}


def oracle_quantizer_rates(oracle, x_np, bits, mode, n_bins, n_steps, n_all, n_one):
    """Oracle rows/s for quantize (mode) and dequantize over a row prefix."""
    def quant(n):
        oracle.quantize_rowwise(x_np[:n], bits, mode, n_bins, n_steps)
    packed = oracle.quantize_rowwise(x_np[:max(n_all, n_one)], bits, mode, n_bins, n_steps)
    dim = x_np.shape[1]

    def deq(n):
        oracle.dequantize(packed[:n], dim, bits)
    return {"quantize": oracle_rate(oracle, quant, n_all, n_one),
            "dequantize": oracle_rate(oracle, deq, min(n_all * 4, packed.shape[0]), n_one)}


def gather_floor(q, torch, packed, w, batches, out, dev, runs=(16, 32), steps=20, warmup=3):
    """The memory traffic of the INT4 lookup with none of its arithmetic
    (libqemb_floor.so: every id and weight read once, contiguously; every row
    read as the lookup reads it, 8 lanes x 12 bytes; the output's bytes
    written), over the same table and rotating batches: a floor for any
    kernel that reads rows this way.  `runs`: batches of 64 ids per wave."""
    import ctypes
    from int4_row_wise_amd import build as qbuild
    lib = ctypes.CDLL(qbuild.FLOOR_LIB)
    p, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.qemb_floor_gather.argtypes = [p, i64, p, p, p, p, i64, p, p, i32, p, i64, i64, p, p]
    lib.qemb_floor_gather.restype = ctypes.c_int
    T, B = w.n_tables, w.batch
    toff = to_dev(torch, np.array([0] + list(np.cumsum(w.rows)), dtype=np.int64), dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    out_bytes = out.numel() * 4
    res = {}
    for run in runs:
        plans = []
        for b in batches:
            id_start = b["offs_np"][::B].astype(np.int64)  # table t's ids start at offsets[t * B]
            waves = -(-(id_start[1:] - id_start[:-1]) // (64 * run))
            wave_start = np.concatenate([[0], np.cumsum(waves)]).astype(np.int64)
            n_waves = int(wave_start[-1])
            store = -(-out_bytes // (n_waves * run) // 512) * 512  # output bytes per batch of 64 ids
            plans.append((to_dev(torch, id_start, dev), to_dev(torch, np.repeat(np.arange(T, dtype=np.int32), waves), dev),
                          to_dev(torch, wave_start, dev), n_waves, b, store * run))
        st = torch.cuda.current_stream().cuda_stream

        def call(k):
            ids_start, wave_table, wave_start, n_waves, b, opw = plans[k % len(plans)]
            rc = lib.qemb_floor_gather(packed.data_ptr(), packed.shape[1], toff.data_ptr(), ids_start.data_ptr(),
                                       wave_table.data_ptr(), wave_start.data_ptr(), n_waves, b["idx"].data_ptr(),
                                       b["w"].data_ptr(), run, out.data_ptr(), out_bytes, opw, sink.data_ptr(), st)
            assert rc == 0, rc
        for k in range(warmup):
            call(k)
        torch.cuda.synchronize()
        tm = Timer(torch)
        for k in range(steps):
            with tm:
                call(k)
        ms = tm.ms()
        nnz = float(np.mean([batches[k % len(batches)]["nnz"] for k in range(steps)]))
        byt = algorithmic_bag_bytes(int(nnz), T * B, w.dim, 4, 4, True)
        res["run_%d_bags_per_wave_eq_%d" % (run, run * 2)] = {
            "avg_launch_ms": float(np.mean(ms)), "median_ms": float(np.median(ms)),
            "GBps": byt / (np.mean(ms) * 1e-3) / 1e9, "hbm_frac": byt / (np.mean(ms) * 1e-3) / 1e9 / HBM_PEAK_GBS}
    return res


def ctr_extras(q, synth, torch, oracle, dev, wid, steps=50, warmup=5, with_oracle=True):
    """A one-hot workload end to end: every table drawn on the GPU and
    quantized by the library (timed per chunk of at most 2^24 rows; HIP
    events), then the one-hot pooled lookup of one batch (timed per launch),
    and the oracle on the same operations: quantize of a row prefix of the
    largest table, the lookup of the whole batch over oracle-packed copies
    of the rows it references."""
    w = synth.workload(wid)
    bits = 4
    mode = q.GREEDY if w.clip == "greedy" else q.RANGE
    S = q.row_stride(w.dim, bits)
    C = (w.dim * bits + 7) // 8
    packed = torch.empty((w.total_rows, S), dtype=torch.uint8, device=dev)
    tm = Timer(torch)
    r0 = 0
    for t in range(w.n_tables):
        n = w.rows[t]
        for c0 in range(0, n, 1 << 24):
            m = min(1 << 24, n - c0)
            x = synth.table_values_torch(w, t, c0, m, dev)
            if mode == q.GREEDY:
                fn = lambda: q.quantize_rowwise(x, bits, mode, w.n_bins, w.n_steps, out=packed[r0 + c0:r0 + c0 + m])
            else:
                fn = lambda: q.quantize_rowwise(x, bits, mode, out=packed[r0 + c0:r0 + c0 + m])
            with tm:
                fn()
            del x
        r0 += n
    qms = float(np.sum(tm.ms()))
    qbytes = w.total_rows * (w.dim * 4 + C + 4)
    res = {"workload": w.name, "rows": w.total_rows, "tables": w.n_tables, "dim": w.dim,
           "quantize": {"clip": w.clip, "ms_all_tables": qms, "rows_per_s": w.total_rows / qms * 1e3,
                        "GBps": qbytes / qms / 1e6, "hbm_frac": qbytes / qms / 1e6 / HBM_PEAK_GBS}}
    bt = synth.batch(w, batch_seed=0, index_dtype=np.int32)
    toff = to_dev(torch, bt.table_offsets, dev)
    idx, offs = to_dev(torch, bt.indices, dev), to_dev(torch, bt.offsets, dev)
    out = torch.empty((bt.B, bt.T, w.dim), dtype=torch.float32, device=dev)
    for _ in range(warmup):
        q.bag_forward(packed, toff, bt.B, w.dim, bits, idx, offs, out=out)
    torch.cuda.synchronize()
    tl = Timer(torch)
    for _ in range(steps):
        with tl:
            q.bag_forward(packed, toff, bt.B, w.dim, bits, idx, offs, out=out)
    ms = tl.ms()
    n_bags = bt.T * bt.B
    lb = algorithmic_bag_bytes(bt.nnz, n_bags, w.dim, bits, 4, False)
    res["lookup"] = {"batch": bt.B, "lookups": bt.nnz, "launch_ms": launch_stats(ms),
                     "lookups_per_s": bt.nnz / (np.mean(ms) * 1e-3),
                     "GBps": lb / (np.mean(ms) * 1e-3) / 1e9,
                     "hbm_frac": lb / (np.mean(ms) * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "bytes_per_launch": lb}
    del packed
    torch.cuda.empty_cache()
    if not with_oracle:
        return res
    omode = oracle.GREEDY if w.clip == "greedy" else oracle.RANGE
    big = int(np.argmax(w.rows))
    n_pre = min(w.rows[big], 1 << 20 if omode == oracle.RANGE else 1 << 16)
    x_np = synth.table_values_torch(w, big, 0, n_pre, dev).cpu().numpy()
    rates = oracle_quantizer_rates(oracle, x_np, bits, omode, w.n_bins, w.n_steps, n_pre,
                                   max(1, n_pre // 16))
    # the lookup: oracle-packed copies of the referenced rows, ids remapped
    idx64 = bt.indices.astype(np.int64)
    mini, sub = [], np.empty_like(idx64)
    base = 0
    for t in range(bt.T):
        sl = slice(bt.offsets[t * bt.B], bt.offsets[(t + 1) * bt.B])
        u, inv = np.unique(idx64[sl], return_inverse=True)
        xr = torch.empty((u.size, w.dim), dtype=torch.float32)
        for c in np.unique(u // synth.CHUNK_ROWS):
            sel = np.nonzero(u // synth.CHUNK_ROWS == c)[0]
            r0c = int(c) * synth.CHUNK_ROWS
            blk = synth.table_values_torch(w, t, r0c, min(synth.CHUNK_ROWS, w.rows[t] - r0c), dev)
            xr[torch.from_numpy(sel)] = blk[torch.from_numpy(u[sel] - r0c).to(dev)].cpu()
            del blk
        mini.append(oracle.quantize_rowwise(xr.numpy(), bits, omode, w.n_bins, w.n_steps))
        sub[sl] = inv + base
        base += u.size
    mp = np.concatenate(mini)
    mtoff = np.array([0, mp.shape[0]], np.int64)
    n_bag = bt.T * bt.B

    def look(nb):
        oracle.bag_forward(mp, mtoff, nb, w.dim, bits, sub[:bt.offsets[nb]], bt.offsets[:nb + 1])
    lr = oracle_rate(oracle, look, n_bag, max(1, n_bag // 16))
    res["cpu_oracle"] = {
        "kind": "oracle", "cores": rates["quantize"]["cores"],
        "quantize_rows_per_s": rates["quantize"]["per_s"],
        "quantize_rows_per_s_one_thread": rates["quantize"]["one_thread_per_s"],
        "quantize_sample": "first %d rows of table %d (one thread: first %d)" % (
            n_pre, big, rates["quantize"]["one_thread_sample"]),
        "dequantize_rows_per_s": rates["dequantize"]["per_s"],
        "dequantize_rows_per_s_one_thread": rates["dequantize"]["one_thread_per_s"],
        "lookups_per_s": lr["per_s"] * (bt.nnz / n_bag),
        "lookups_per_s_one_thread": lr["one_thread_per_s"] * (bt.nnz / n_bag),
        "lookup_sample": "the whole batch (%d bags) over oracle-packed copies of its rows" % n_bag}
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    if args.calibrate_copy:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty(n, dtype=torch.uint8, device="cuda")
        a.fill_(1)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 5}))
        return

    import int4_row_wise_amd as q
    from int4_row_wise_amd import build as qbuild
    from int4_row_wise_amd import synth
    qbuild.ensure_built()
    q.load_library()  # raises unless the library was built from the current kernel sources
    dev = torch.device("cuda:0")
    if args.quantizer_only:
        print(json.dumps({"quantizer": quantizer_extras(q, synth, torch, dev)}), flush=True)
        return
    w = synth.workload(4)
    if args.uniform_ids:
        import dataclasses
        w = dataclasses.replace(w, alpha=None)
    bits_list = (4,) if (args.no_extras or args.interaction_only or args.compress_only or
                         args.gather_floor or args.uniform_ids) else (4, 8)

    # the index batches (seconds of host work) come first and the tables
    # (GPU work) right before the timed lookups: a GPU left idle for seconds
    # before the warm-up starts the lookup in a power-management transient
    # (launches 4-40 after an idle period run up to 35 % slower than the
    # steady state while the board's power limit pulls the clock back)
    t0 = time.time()
    batches = []
    for k in range(args.batches):
        b = synth.batch(w, batch_seed=k, index_dtype=np.int32)
        batches.append({"idx": to_dev(torch, b.indices, dev), "offs": to_dev(torch, b.offsets, dev),
                        "w": to_dev(torch, b.weights, dev), "nnz": b.nnz,
                        "idx_np": b.indices, "offs_np": b.offsets, "w_np": b.weights})
    log("%d index batches generated in %.1fs (nnz %s)" % (
        len(batches), time.time() - t0, [b["nnz"] for b in batches]))
    t0 = time.time()
    packed = {} if args.codebook_only else build_table(q, synth, torch, w, bits_list, dev)
    log("tables generated and packed in %.1fs" % (time.time() - t0))
    toff = to_dev(torch, np.array([0] + list(np.cumsum(w.rows)), dtype=np.int64), dev)
    n_bags = w.n_tables * w.batch
    out = torch.empty((w.batch, w.n_tables, w.dim), dtype=torch.float32, device=dev)
    if args.interaction_only or args.compress_only:
        b0 = batches[0]
        q.bag_forward(packed[4], toff, w.batch, w.dim, 4, b0["idx"], b0["offs"], b0["w"], out=out)
        if args.compress_only:
            res = compress_extras(q, torch, out, dev, args.steps, args.warmup)
            print(json.dumps({"compress": res, "workload": w.name}), flush=True)
        else:
            res = interaction_extras(q, torch, out, w, dev, args.steps, args.warmup)
            print(json.dumps({"interaction": res, "workload": w.name}), flush=True)
        return
    if args.codebook_only:
        del packed
        res = codebook_extras(q, synth, torch, w, toff, batches, out, dev, n_bags, args.steps,
                              args.warmup)
        print(json.dumps({"codebook": res, "workload": w.name}), flush=True)
        return

    if args.uniform_ids:
        ms, _ = bench_bags(q, torch, packed[4], toff, batches, w, 4, args.steps, args.warmup, out)
        bu = algorithmic_bag_bytes(batches[0]["nnz"], n_bags, w.dim, 4, 4, True)
        print(json.dumps({"uniform_ids_lookup": {
            "avg_launch_ms": float(np.mean(ms)), "lookups": batches[0]["nnz"],
            "GBps": bu / (np.mean(ms) * 1e-3) / 1e9,
            "hbm_frac": bu / (np.mean(ms) * 1e-3) / 1e9 / HBM_PEAK_GBS}, "workload": w.name + ", uniform ids"}),
              flush=True)
        return
    if args.gather_floor:
        ms, _ = bench_bags(q, torch, packed[4], toff, batches, w, 4, args.steps, args.warmup, out)
        floor = gather_floor(q, torch, packed[4], w, batches, out, dev, steps=args.steps)
        print(json.dumps({"lookup_avg_launch_ms": float(np.mean(ms)), "gather_floor": floor,
                          "workload": w.name}), flush=True)
        return
    ms, wall = bench_bags(q, torch, packed[4], toff, batches, w, 4, args.steps, args.warmup, out)
    nnz_timed = sum(batches[k % len(batches)]["nnz"] for k in range(args.steps))
    bytes_timed = sum(algorithmic_bag_bytes(batches[k % len(batches)]["nnz"], n_bags, w.dim, 4, 4,
                                            True) for k in range(args.steps))
    avg_ms = float(np.mean(ms))
    achieved = bytes_timed / args.steps / (avg_ms * 1e-3) / 1e9
    log("INT4 bag forward: %.3f ms/launch (median %.3f), %.0f GB/s algorithmic" % (
        avg_ms, float(np.median(ms)), achieved))
    stats = launch_stats(ms)

    result = {
        "metric": "pooled lookups/sec and achieved HBM GB/s (% of roofline), INT4 bag fwd",
        "value": nnz_timed / wall,
        "unit": "lookups/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "storage": "int4 codes + fp16 scale/bias per row",
        "data": "synthetic (seeded generators; no dataset)",
        "config": {
            "workload": w.name,
            "tables": w.n_tables, "rows_per_table": w.rows[0], "dim": w.dim, "bits": 4,
            "batch": w.batch, "bag_length": "U{1..64}", "ids": "Zipf(1.05), int32",
            "weights": "U(0,1) fp32", "index_batches": len(batches),
            "mean_nnz": float(np.mean([b["nnz"] for b in batches])),
        },
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(),
            "traffic_unit": "bytes per launch (HBM, from FETCH_SIZE/WRITE_SIZE)",
            "kernel": HEADLINE_KERNEL,
            "bytes_per_launch": bytes_timed / args.steps,
            "avg_launch_ms": avg_ms,
        },
        "launch_ms": stats,
    }

    if not args.no_extras:
        ms8, wall8 = bench_bags(q, torch, packed[8], toff, batches, w, 8, max(10, args.steps // 2),
                                3, out)
        b8 = algorithmic_bag_bytes(batches[0]["nnz"], n_bags, w.dim, 8, 4, True)
        result["int8"] = {"lookups_per_s": batches[0]["nnz"] / (np.mean(ms8) * 1e-3),
                          "avg_launch_ms": float(np.mean(ms8)),
                          "GBps": b8 / (np.mean(ms8) * 1e-3) / 1e9,
                          "hbm_frac": b8 / (np.mean(ms8) * 1e-3) / 1e9 / HBM_PEAK_GBS}
        # uniform-id control: same shapes, ids uniform over each table
        import dataclasses
        wu = dataclasses.replace(w, alpha=None)
        bu = synth.batch(wu, batch_seed=0, index_dtype=np.int32)
        ub = [{"idx": to_dev(torch, bu.indices, dev), "offs": to_dev(torch, bu.offsets, dev),
               "w": to_dev(torch, bu.weights, dev), "nnz": bu.nnz}]
        msu, _ = bench_bags(q, torch, packed[4], toff, ub, w, 4, 10, 3, out)
        bb = algorithmic_bag_bytes(bu.nnz, n_bags, w.dim, 4, 4, True)
        result["uniform_ids_control"] = {
            "lookups_per_s": bu.nnz / (np.mean(msu) * 1e-3), "avg_launch_ms": float(np.mean(msu)),
            "GBps": bb / (np.mean(msu) * 1e-3) / 1e9,
            "hbm_frac": bb / (np.mean(msu) * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del ub
        b0 = algorithmic_bag_bytes(batches[0]["nnz"], n_bags, w.dim, 4, 4, True)
        msc = bench_cold(q, torch, packed[4], toff, batches[0], w, 4, out, dev)
        result["cold_cache"] = {
            "note": "each launch after writing a 1 GiB scratch buffer (L2 and MALL flushed)",
            "launch_ms": launch_stats(msc), "GBps": b0 / (np.median(msc) * 1e-3) / 1e9,
            "hbm_frac": b0 / (np.median(msc) * 1e-3) / 1e9 / HBM_PEAK_GBS}
        result["stream_ceiling"] = stream_ceiling(torch, dev)
        result["interaction"] = interaction_extras(q, torch, out, w, dev)
        result["compress"] = compress_extras(q, torch, out, dev)
        # (after the consumers of the pooled output: the floor overwrites it)
        result["gather_floor"] = gather_floor(q, torch, packed[4], w, batches, out, dev)
        # 2-bit rows of the same tables (range), same batches
        p2 = build_table(q, synth, torch, w, (2,), dev)[2]
        ms2, _ = bench_bags(q, torch, p2, toff, batches, w, 2, 10, 3, out)
        b2 = algorithmic_bag_bytes(batches[0]["nnz"], n_bags, w.dim, 2, 4, True)
        result["int2"] = {"lookups_per_s": batches[0]["nnz"] / (np.mean(ms2) * 1e-3),
                          "avg_launch_ms": float(np.mean(ms2)),
                          "GBps": b2 / (np.mean(ms2) * 1e-3) / 1e9,
                          "hbm_frac": b2 / (np.mean(ms2) * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del p2
        result["device_copy_GBps"] = device_copy_gbps(torch, dev)
        del packed[8]
        torch.cuda.empty_cache()
        result["codebook"] = codebook_extras(q, synth, torch, w, toff, batches, out, dev, n_bags)
        t0 = time.time()
        oracle_mod = None
        if not args.no_cpu_baseline:
            import oracle as oracle_mod
        result["quantizer"] = quantizer_extras(q, synth, torch, dev, oracle_mod)
        log("quantizer workload done in %.1fs" % (time.time() - t0))
        for wid, key in ((1, "tiny"), (2, "ctr_one_hot"), (3, "large_ctr_one_hot")):
            t0 = time.time()
            result[key] = ctr_extras(q, synth, torch, oracle_mod, dev, wid,
                                     with_oracle=oracle_mod is not None)
            log("%s workload done in %.1fs" % (key, time.time() - t0))

    if not args.no_cpu_baseline:
        import oracle
        t0 = time.time()
        result["cpu_baseline"] = cpu_baseline(oracle, synth, torch, w, 4, batches[0], dev)
        log("cpu baseline done in %.1fs" % (time.time() - t0))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
