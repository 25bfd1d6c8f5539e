"""Benchmark of one step of the paged-attention hot path on one MI355X.

A step is the whole hot path over one batch: prepare_inputs_and_plan (the
flat-batch indices, the slot mapping and the attention work list, in one
launch) -> kv_cache_write (this step's K/V rows into the block pool) -> the
attention run (main kernel, and the split-KV reduce when a context is
partitioned).  Plan then run is the same work as one paged_attention_varlen
call.  Inputs are resident in HBM before timing; outputs, workspace and index
buffers are preallocated, so a step allocates nothing.

Default workload: the mixed chunked-prefill step ("Building the Batch", "Why
flatten": one 5,000-token prompt chunk with 3,000 tokens already computed,
next to 200 single-token decodes with contexts uniform in [1024, 8192]; 32 q
/ 8 kv heads, head_dim 128, bf16, 16-token blocks placed at random), the
largest of the five configurations.  ``--workload`` selects another.

Timing protocol: every timed iteration starts after a 512 MiB write that
flushes L2 and the MALL, and is bracketed by HIP events on the stream the
library launches on; medians, p10 and p90 are reported, and the GPU clocks are
sampled while the loops run.  The roofline is that of the attention run
(max(t_bytes, t_flops) / t), for the whole batch and for its decode rows and
prompt rows alone over the same pools.

Prints one JSON line: tokens/s of the whole step, the roofline figures, and
the fp64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attn tokens/s; decode HBM GB/s % peak; prefill MFMA TFLOP/s % peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
FP8_SCALES = (0.0125, 0.0125)    # k_scale, v_scale of --kv-dtype fp8 (N(0,1) history / scale)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", type=int, default=4, choices=[1, 2, 3, 4, 5])
    p.add_argument("--rows", default="all", choices=["all", "decode", "prefill"],
                   help="time the whole batch, or only its single-token/short (decode) "
                        "or prompt-chunk (prefill) requests over the same pools")
    p.add_argument("--split-tokens", type=int, default=0,
                   help="context partition size of decode items (0 = library default)")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="approximate budget of the CPU oracle baseline (all threads)")
    p.add_argument("--cpu-single-seconds", type=float, default=5.0,
                   help="approximate budget of the single-thread CPU oracle baseline")
    p.add_argument("--kv-dtype", default="bf16", choices=["bf16", "fp8"],
                   help="cache element type: bf16, or FP8 E4M3 codes with per-pool scales "
                        "(the same history quantised; q and out stay bf16)")
    p.add_argument("--graph", action="store_true",
                   help="also capture the step in a HIP graph and time K replays (reported "
                        "beside the eager figures)")
    p.add_argument("--op", default="step", choices=["step", "input_ids", "copy_blocks",
                                                     "zero_blocks"],
                   help="step: the hot path above.  input_ids: prepare_inputs + "
                        "prepare_input_ids of the workload's step.  copy_blocks / "
                        "zero_blocks: --blocks block copies (fresh destinations) or clears "
                        "in both pools of the workload's cache geometry")
    p.add_argument("--blocks", type=int, default=8192,
                   help="blocks per copy_blocks / zero_blocks launch")
    p.add_argument("--clock-runs", type=int, default=300,
                   help="attention runs queued back to back while the GPU clocks are read "
                        "(0: no clock reading)")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="instead of the step, time a plain device-to-device copy of this many "
                        "MiB (the known-size kernel that HBM byte counters are scaled by)")
    return p.parse_args()


def copy_probe(mib, launches=10):
    """Device-to-device copy of a known size: reads and writes ``mib`` MiB per launch."""
    import torch
    dev = torch.device("cuda:0")
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(launches):
        dst.copy_(src)
    ev[1].record()
    torch.cuda.synchronize(dev)
    ms = ev[0].elapsed_time(ev[1]) / launches
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": launches + 1,
                      "ms_per_copy": round(ms, 4), "copy_gbs": round(2 * n / ms / 1e6, 1)}),
          flush=True)


def algorithmic_work(wl):
    """Bytes and flops the attention call must move / compute (one layer)."""
    nst = wl.num_scheduled_tokens.astype(np.int64)
    seq = nst + wl.num_computed_tokens.astype(np.int64)
    e = 2 if str(wl.dtype).endswith("bfloat16") else 4
    e_kv = 1 if wl.kv_scales is not None else e  # FP8 pools: one byte per element
    Hq, Hkv, d, bs = wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size
    kv_token_bytes = 2 * Hkv * d * e_kv
    # unique context tokens: blocks shared by several requests are read once
    shared = 0
    if wl.notes.get("shared_blocks"):
        blocks_logical = int(((seq + bs - 1) // bs).sum())
        blocks_unique = len(np.unique(wl.block_table[wl.block_table >= 0]))
        shared = (blocks_logical - blocks_unique) * bs
    unique_ctx = int(seq.sum()) - shared
    T = int(nst.sum())
    q_o_bytes = 2 * T * Hq * d * e
    table_bytes = int(((seq + bs - 1) // bs).sum()) * 4 + (2 * wl.num_reqs + 1) * 4
    # visible (query, key) pairs: row t of a request sees seq - q_len + t + 1 keys
    pairs_dec = pairs_pre = 0
    for n, L in zip(nst, seq):
        vis = int(n * (L - n) + n * (n + 1) // 2)
        if n * (Hq // Hkv) <= 16:
            pairs_dec += vis
        else:
            pairs_pre += vis
    flops_per_pair = 4 * d * Hq
    return {
        "context_tokens": int(seq.sum()),
        "kv_token_bytes": kv_token_bytes,
        "bytes_logical": int(seq.sum()) * kv_token_bytes + q_o_bytes + table_bytes,
        "bytes_unique": unique_ctx * kv_token_bytes + q_o_bytes + table_bytes,
        "flops_decode": pairs_dec * flops_per_pair,
        "flops_prefill": pairs_pre * flops_per_pair,
        "write_bytes": 2 * T * Hkv * d * (e + e_kv),
    }


_CSRC = os.path.join(ROOT, "paged_kv_cache_prepare_amd", "csrc")
TRAFFIC = (os.path.join(ROOT, "profiles", "attention_hbm_traffic.txt"),
           [os.path.join(_CSRC, f) for f in ("attention.hip", "pkv_internal.h")])
BLOCK_OPS_TRAFFIC = (os.path.join(ROOT, "profiles", "block_ops_hbm_traffic.txt"),
                     [os.path.join(_CSRC, "block_ops.hip")])


def source_hash(sources):
    h = hashlib.sha256()
    for f in sources:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(key, which=TRAFFIC):
    """HBM bytes per launch from the rocprofv3 FETCH_SIZE / WRITE_SIZE figures
    in profiles/, or None when there are none for this workload or the kernel
    source has changed since they were taken."""
    path, sources = which
    try:
        with open(path) as fh:
            kv = dict(line.split("=", 1) for line in (l.strip() for l in fh)
                      if line and not line.startswith("#") and "=" in line)
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("source_sha256") != source_hash(sources) or key not in kv:
        return None
    return int(kv[key])


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, budget_s, single_s):
    """The fp64 oracle, as it is, timed on host cores on a bounded sample of
    the same step, phase by phase.

    prepare and the KV write run on the whole batch; attention runs on an
    evenly strided sample of rows (prompt-chunk and decode rows in the batch's
    proportions), sized by a short calibration run to take about
    ``budget_s`` with every OpenMP thread, then a smaller sample on one
    thread for about ``single_s``.  Rate = sampled rows / (attention time of
    the sample + prepare and write time scaled to the sample's share of the
    rows)."""
    import oracle
    T = wl.num_tokens
    kc, vc = wl.key_cache.cpu(), wl.value_cache.cpu()
    key, val, q = wl.key.cpu(), wl.value.cpu(), wl.q.cpu()
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    prep = oracle.prepare(wl.num_scheduled_tokens, wl.num_computed_tokens, wl.block_table,
                          wl.block_size, wl.num_blocks)
    t_prep = time.perf_counter() - t0
    t0 = time.perf_counter()
    if wl.kv_scales is None:
        oracle.kv_write(key, val, kc, vc, prep["slot_mapping"], wl.block_size)
    else:
        oracle.kv_write_fp8(key, val, kc, vc, prep["slot_mapping"], wl.block_size, *wl.kv_scales)
    t_write = time.perf_counter() - t0

    def attn(rows, nthreads):
        t1 = time.perf_counter()
        oracle.attention(q, kc, vc, prep["query_start_loc"], prep["seq_lens"], wl.block_table,
                         wl.block_size, wl.scale, rows=rows, kv_scales=wl.kv_scales,
                         num_threads=nthreads)
        return time.perf_counter() - t1

    def sample(budget, nthreads):
        n = min(T, max(2, 2 * nthreads))
        rows = np.unique(np.linspace(0, T - 1, n).astype(np.int32))
        dt = attn(rows, nthreads)
        while len(rows) < T and dt < budget / 3:
            n = min(T, max(len(rows) + 1, int(len(rows) * min(16.0, 0.8 * budget /
                                                              max(dt, 1e-3)))))
            rows = np.unique(np.linspace(0, T - 1, n).astype(np.int32))
            dt = attn(rows, nthreads)
        reps = 1
        if len(rows) == T:  # the whole batch is cheap: repeat it for a stable time
            while dt < budget / 3 and reps < 1000:
                dt += attn(rows, nthreads)
                reps += 1
        n = len(rows)
        total = dt + (t_prep + t_write) * reps * n / T
        what = (f"all {T} rows, {reps} times" if reps > 1 else f"{n} evenly strided rows of {T}")
        return reps * n / total, dt, what

    rate, dt, what = sample(budget_s, threads)
    rate1, dt1, what1 = sample(single_s, 1)
    return {"value": round(rate, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"fp64 oracle; prepare ({t_prep:.3f} s) and kv_write ({t_write:.3f} s) "
                      f"on all {T} rows, prorated; attention on {what} ({dt:.2f} s)",
            "phases_s": {"prepare": round(t_prep, 4), "kv_write": round(t_write, 4),
                         "attention_sample": round(dt, 3)},
            "single_thread": {"value": round(rate1, 2), "unit": "tokens/s", "cores": 1,
                              "sample": f"attention on {what1} ({dt1:.2f} s), prepare and "
                                        f"kv_write prorated"}}


class ClockReader:
    """SCLK / MCLK of the GPU (amdsmi's clock query; sysfs pp_dpm_* as a
    fallback).  ``under_load`` samples them while a long queue of the
    benchmark's own kernels runs.  Never fails the benchmark: where neither
    source is readable it reports that."""

    def __init__(self):
        self.source = None
        try:
            self._read = self._init_reader()
        except Exception:
            self._read = None

    def _init_reader(self):
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            h = handles[0]
            try:
                import torch
                bus = getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None)
                for cand in handles:
                    bdf = amdsmi.amdsmi_get_gpu_device_bdf(cand)
                    if bus is not None and int(bdf.split(":")[1], 16) == int(bus):
                        h = cand
            except Exception:
                pass

            def valid(x):
                return isinstance(x, (int, float)) and 0 < x < 0xFFFF

            def from_metrics():
                # per-XCC current gfx clocks where the metrics table has them
                mt = amdsmi.amdsmi_get_gpu_metrics_info(h)
                g = mt.get("current_gfxclks")
                if isinstance(g, (list, tuple)):
                    g = [x for x in g if valid(x)]
                    g = float(np.median(g)) if g else None
                else:
                    g = None
                if g is None:
                    for key in ("current_gfxclk", "average_gfxclk_frequency"):
                        if valid(mt.get(key)):
                            g = float(mt[key])
                            break
                m = next((float(mt[k]) for k in ("current_uclk", "average_uclk_frequency")
                          if valid(mt.get(k))), None)
                if g is None or m is None:
                    raise ValueError("no clock in the metrics table")
                return g, m

            def from_clock_info():
                g = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)["clk"]
                m = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.MEM)["clk"]
                return float(g), float(m)
            try:
                from_metrics()
                self.source = ("amdsmi_get_gpu_metrics_info (median of the per-XCC current "
                               "gfx clocks; current uclk)")
                return from_metrics
            except Exception:
                from_clock_info()
                self.source = "amdsmi_get_clock_info (GFX, MEM)"
                return from_clock_info
        except Exception:
            pass
        import glob
        for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
            sc, mc = os.path.join(dev, "pp_dpm_sclk"), os.path.join(dev, "pp_dpm_mclk")

            def cur(path):
                with open(path) as fh:
                    for line in fh:
                        if "*" in line:
                            return float(line.split(":")[1].strip().rstrip("*").strip()
                                         .lower().replace("mhz", ""))
                raise ValueError(path)
            try:
                def read(sc=sc, mc=mc):
                    return cur(sc), cur(mc)
                read()
                self.source = f"{sc} and pp_dpm_mclk"
                return read
            except Exception:
                continue
        return None

    def under_load(self, enqueue, done, period_s=0.01):
        """Call ``enqueue`` (which queues GPU work without waiting), then read
        the clocks every ``period_s`` until ``done()`` is true."""
        if self._read is None:
            enqueue()
            return {"source": None, "note": "no clock source readable"}
        sclk, mclk = [], []
        enqueue()
        t_end = time.perf_counter() + 30.0
        while not done() and time.perf_counter() < t_end:
            try:
                g, m = self._read()
                sclk.append(g)
                mclk.append(m)
            except Exception:
                pass
            time.sleep(period_s)
        if not sclk:
            return {"source": self.source, "note": "no readings while the kernels ran"}
        return {"source": self.source, "samples": len(sclk),
                "sclk_mhz": {"median": float(np.median(sclk)), "min": float(np.min(sclk)),
                             "max": float(np.max(sclk))},
                "mclk_mhz": {"median": float(np.median(mclk)), "min": float(np.min(mclk)),
                             "max": float(np.max(mclk))}}


class Calib:
    """The benchmark's measurement kernels (libpkv_calib.so, include/pkv_calib.h):
    the shader clock seen by a spinning wave, and a plain read kernel over a
    list of K/V runs.  Neither is part of the measured path."""

    def __init__(self):
        import ctypes
        from paged_kv_cache_prepare_amd import _build
        if not os.path.exists(_build.CALIB_LIB_PATH):
            raise RuntimeError(f"{_build.CALIB_LIB_PATH} is not built: run __graft_entry__.build()")
        self.lib = ctypes.CDLL(_build.CALIB_LIB_PATH)
        P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        self.lib.pkv_calib_clock.argtypes = [P, i64, P]
        self.lib.pkv_calib_read_runs.argtypes = [P, P, i64, i32, P, P]

    def clock(self, ms, stream):
        """Enqueue a wave that spins for ``ms`` on ``stream``; returns a
        function giving the shader clock in MHz once the stream is done."""
        import torch
        with torch.cuda.stream(stream):  # allocated for this stream; the kernel writes both words
            out = torch.empty(2, dtype=torch.int64, device=stream.device)
        ticks = int(min(max(ms, 0.01), 9000.0) * 1e5)
        rc = self.lib.pkv_calib_clock(out.data_ptr(), ticks, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"pkv_calib_clock: {rc}")
        return lambda: 100.0 * float(out[0]) / float(out[1])

    def read_runs(self, addrs, wave_begin, run_kib, sink, stream):
        rc = self.lib.pkv_calib_read_runs(addrs.data_ptr(), wave_begin.data_ptr(),
                                          wave_begin.numel() - 1, run_kib, sink.data_ptr(),
                                          stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"pkv_calib_read_runs: {rc}")


def decode_run_stream(wl, b):
    """The K/V runs the decode items of ``wl``'s work list read, per wave, in
    the order the kernels issue them: item by item as the plan lists them,
    the item's four waves splitting its partition's 32-token steps, each
    step's two K runs then its two V runs.  Returns (run addresses, wave
    offsets, run KiB) as CPU int64 arrays, or None without decode items."""
    import torch
    ws = b["ws"].cpu()
    head = ws[:256].view(torch.int32).numpy()
    n = int(head[0])
    items = ws[256:256 + 16 * n].view(torch.int32).numpy().reshape(n, 4)
    items = items[items[:, 3] >= 1]
    if len(items) == 0:
        return None
    seq = b["prep"]["seq_lens"].cpu().numpy().astype(np.int64)
    run = 16 * wl.head_dim * wl.key_cache.element_size()
    stride = wl.num_kv_heads * run
    kbase, vbase = wl.key_cache.data_ptr(), wl.value_cache.data_ptr()
    addrs, begin = [], [0]
    for r, h, k, ns in items.tolist():
        nblk = -(-int(seq[r]) // 16)
        steps_all = -(-nblk // 2)
        per_split = -(-steps_all // ns)
        sp_b = k * per_split
        sp_e = min(steps_all, sp_b + per_split)
        per_wave = -(-max(0, sp_e - sp_b) // 4)
        row = wl.block_table[r].astype(np.int64)
        for w in range(4):
            s = np.arange(sp_b + w * per_wave, min(sp_e, sp_b + (w + 1) * per_wave))
            j = np.stack([2 * s, 2 * s + 1], 1)
            ok = j < nblk
            off = row[np.minimum(j, nblk - 1)] * stride + h * run
            a = np.concatenate([kbase + off, vbase + off], 1)       # K0 K1 V0 V1 per step
            a = a[np.concatenate([ok, ok], 1)]
            addrs.append(a)
            begin.append(begin[-1] + len(a))
    return (np.concatenate(addrs).astype(np.int64), np.asarray(begin, np.int64), run // 1024)


def read_ceiling(calib, wl, b, kernel_ms, unique_bytes, flush, steps, stream):
    """Time a plain read kernel over the decode run stream of ``wl`` (each
    iteration after the cache flush, HIP events) and compare."""
    import torch
    st = decode_run_stream(wl, b)
    if st is None:
        return None
    addrs, begin, kib = st
    dev = wl.q.device
    a_d = torch.from_numpy(addrs).to(dev)
    b_d = torch.from_numpy(begin).to(dev)
    sink = torch.empty(64 * (len(begin) - 1), dtype=torch.int32, device=dev)
    for _ in range(2):
        flush()
        calib.read_runs(a_d, b_d, kib, sink, stream)
    ts = []
    for _ in range(steps):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        calib.read_runs(a_d, b_d, kib, sink, stream)
        e1.record(stream)
        torch.cuda.synchronize(dev)
        ts.append(e0.elapsed_time(e1))
    ms = pct(ts)
    t = ms["median"] / 1e3
    logical = int(len(addrs)) * kib * 1024
    return {"reader_ms": ms, "runs": int(len(addrs)), "logical_bytes": logical,
            "reader_logical_gbs": round(logical / t / 1e9, 1),
            "reader_frac_of_peak": round(unique_bytes / t / 1e9 / HBM_PEAK_GBS, 4),
            "kernel_over_reader_time": round(kernel_ms / ms["median"], 4),
            "note": "a plain read kernel (no arithmetic, the same non-temporal loads, 32 KiB in "
                    "flight per wave) over exactly the K/V runs the decode items read, in the "
                    "work list's order; reader_frac_of_peak is the roofline fraction that "
                    "reader attains on the same algorithmic bytes"}


def pct(xs):
    xs = np.asarray(xs, np.float64)
    return {"median": round(float(np.median(xs)), 4), "p10": round(float(np.percentile(xs, 10)), 4),
            "p90": round(float(np.percentile(xs, 90)), 4), "mean": round(float(xs.mean()), 4),
            "n": int(xs.size)}


def _timed_launches(fn, steps, warmup):
    """Average ms per call of ``fn`` over ``steps`` calls, from HIP events on
    torch's current stream (the stream the library launches on), after
    ``warmup`` untimed calls; plus the host-clock ms per call of the same loop."""
    import torch
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    for _ in range(warmup):
        fn()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    ev[0].record(stream)
    for _ in range(steps):
        fn()
    ev[1].record(stream)
    torch.cuda.synchronize(dev)
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return ev[0].elapsed_time(ev[1]) / steps, wall


def bench_op(args):
    """One JSON line for a batch-side operation (--op), HBM roofline and the
    oracle timed beside it."""
    import torch
    import oracle
    import paged_kv_cache_prepare_amd as pkv
    from paged_kv_cache_prepare_amd import workloads

    dev = torch.device("cuda:0")
    st = workloads.config_structure(args.workload)
    nst, nct = st["num_scheduled_tokens"], st["num_computed_tokens"]
    Hkv, d, bs = st["num_kv_heads"], st["head_dim"], workloads.BLOCK_SIZE
    rng = np.random.default_rng(2000 + args.workload)
    line = {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "data": "synthetic (seeded)"}
    if args.op == "input_ids":
        R, T = len(nst), int(nst.sum())
        seq = (nst + nct).astype(np.int64)
        width = int(seq.max())
        # requests given more than one token this step are prompt chunks that
        # do not finish the prompt: their sampled token is discarded
        total = (seq + (nst > 1)).astype(np.int32)
        table = rng.integers(0, 152064, (R, width)).astype(np.int32)
        g = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in
             dict(nst=nst, nct=nct, total=total, table=table,
                  bt=np.zeros((R, 1), np.int32)).items()}
        i32 = dict(dtype=torch.int32, device=dev)
        prep = {"req_indices": torch.empty(T, **i32), "positions": torch.empty(T, **i32),
                "slot_mapping": torch.empty(T, dtype=torch.int64, device=dev),
                "query_start_loc": torch.empty(R + 1, **i32), "seq_lens": torch.empty(R, **i32),
                "logits_indices": torch.empty(R, **i32)}
        ids = {"input_ids": torch.empty(T, **i32),
               "discard_request_mask": torch.empty(R, dtype=torch.uint8, device=dev)}

        def fn():
            pkv.prepare_inputs(g["nst"], g["nct"], g["bt"], num_tokens=T, block_size=1 << 30,
                               num_blocks=1, out=prep)
            pkv.prepare_input_ids(g["table"], prep["req_indices"], prep["positions"],
                                  prep["seq_lens"], g["total"], out=ids)

        ms, wall = _timed_launches(fn, args.steps, args.warmup)
        # prepare: nst, nct, table column read, 3 per-row + 3 per-request outputs;
        # ids: req_indices, positions, token id read + write; seq_lens, total, mask
        nbytes = R * 8 + T * 4 + T * 16 + R * 12 + T * 16 + R * 9
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0) or reps == 0:
            ref = oracle.prepare(nst, nct, np.zeros((R, 1), np.int32), 1 << 30, 1)
            oracle.input_ids(table, ref["req_indices"], ref["positions"], ref["seq_lens"], total)
            reps += 1
        cpu_s = (time.perf_counter() - t0) / reps
        gbs = nbytes / (ms / 1e3) / 1e9
        line.update({
            "metric": "input prep tokens/s (prepare_inputs + prepare_input_ids)",
            "value": round(T / (ms / 1e3), 1), "unit": "tokens/s", "ms_per_step": round(ms, 4),
            "dtype": "int32",
            "config": {"workload": workloads.CONFIG_NAMES[args.workload], "op": args.op,
                       "num_reqs": R, "num_tokens": T, "row_width": width},
            "host_ms_per_step": round(wall, 4),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 6), "traffic": None,
                         "kernel": "prepare_kernel + input_ids_kernel (launch-latency bound)",
                         "algorithmic_bytes": nbytes, "avg_ms": round(ms, 4)},
            "cpu_baseline": {"value": round(T / cpu_s, 1), "unit": "tokens/s", "cores": 1,
                             "kind": "oracle",
                             "sample": f"oracle prepare + input_ids on the whole step, "
                                       f"{reps} times"}})
        print(json.dumps(line), flush=True)
        return

    # copy_blocks / zero_blocks on the workload's pool geometry
    fp8 = args.kv_dtype == "fp8"
    e = 1 if fp8 else (4 if st["dtype"] == torch.float32 else 2)
    block_bytes = Hkv * bs * d * e
    need = int(((nst.astype(np.int64) + nct + bs - 1) // bs).sum())
    nb = max(int(math.ceil(1.25 * need)), 2 * args.blocks)
    n = args.blocks
    gen = torch.Generator(device=dev).manual_seed(2000 + args.workload)
    pools = [torch.randint(0, 256, (nb, block_bytes), generator=gen, dtype=torch.uint8,
                           device=dev) for _ in range(2)]
    perm = rng.permutation(nb)
    if args.op == "copy_blocks":
        items = np.stack([rng.choice(perm[n:], n), perm[:n]], 1).astype(np.int32)
        moved = 2 * 2 * n * block_bytes                 # both pools, read + write
    else:
        items = perm[:n].astype(np.int32)
        moved = 2 * n * block_bytes                     # both pools, write
    dev_items = torch.from_numpy(np.ascontiguousarray(items)).to(dev)
    op = getattr(pkv, args.op)
    ms, wall = _timed_launches(lambda: op(pools[0], pools[1], dev_items), args.steps,
                               args.warmup)
    gbs = moved / (ms / 1e3) / 1e9
    # oracle on host pools: a bounded sample of the same list in a compact pool
    m = min(n, 1024)
    hk = np.zeros((2 * m, block_bytes), np.uint8)
    hv = np.zeros((2 * m, block_bytes), np.uint8)
    h_items = (np.stack([np.arange(m, 2 * m), np.arange(m)], 1) if args.op == "copy_blocks"
               else np.arange(m)).astype(np.int32)
    ofn = oracle.copy_blocks if args.op == "copy_blocks" else oracle.zero_blocks
    t0 = time.perf_counter()
    reps = 0
    while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0) or reps == 0:
        ofn(hk, hv, h_items)
        reps += 1
    cpu_s = (time.perf_counter() - t0) / reps
    line.update({
        "metric": f"{args.op} HBM GB/s", "value": round(gbs, 1), "unit": "GB/s",
        "ms_per_step": round(ms, 4), "dtype": "u8",
        "config": {"workload": f"{n} blocks of {block_bytes} B per pool, pools of "
                               f"{workloads.CONFIG_NAMES[args.workload]}"
                               + (" with an FP8 cache" if fp8 else ""),
                   "op": args.op, "blocks": n, "block_bytes": block_bytes,
                   "num_blocks": nb},
        "host_ms_per_step": round(wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(f"{args.op}_w{args.workload}_n{n}"
                                                 + ("_fp8" if fp8 else ""), BLOCK_OPS_TRAFFIC),
                     "kernel": f"{args.op}_kernel, HIP events", "algorithmic_bytes": moved,
                     "avg_ms": round(ms, 4)},
        "cpu_baseline": {"value": round((moved * m / n) / cpu_s / 1e9, 2), "unit": "GB/s",
                         "cores": 1, "kind": "oracle",
                         "sample": f"oracle {args.op} of {m} blocks in a {2 * m}-block host "
                                   f"pool pair, {reps} times"}})
    print(json.dumps(line), flush=True)


def step_buffers(wl, split_tokens):
    """Device inputs and preallocated outputs / workspace of one step of ``wl``."""
    import torch
    import paged_kv_cache_prepare_amd as pkv
    dev = wl.q.device
    T, R = wl.num_tokens, wl.num_reqs
    i32 = dict(dtype=torch.int32, device=dev)
    b = {"nst": torch.from_numpy(wl.num_scheduled_tokens).to(dev),
         "nct": torch.from_numpy(wl.num_computed_tokens).to(dev),
         "bt": torch.from_numpy(wl.block_table).to(dev),
         "prep": {"req_indices": torch.empty(T, **i32), "positions": torch.empty(T, **i32),
                  "slot_mapping": torch.empty(T, dtype=torch.int64, device=dev),
                  "query_start_loc": torch.empty(R + 1, **i32),
                  "seq_lens": torch.empty(R, **i32), "logits_indices": torch.empty(R, **i32)},
         "out": torch.empty_like(wl.q), "ks": None, "vs": None}
    if wl.kv_scales is not None:
        b["ks"] = torch.tensor([wl.kv_scales[0]], dtype=torch.float32, device=dev)
        b["vs"] = torch.tensor([wl.kv_scales[1]], dtype=torch.float32, device=dev)
    need = pkv.attention_workspace_bytes(R, T, wl.num_q_heads, wl.num_kv_heads, wl.head_dim,
                                         wl.max_query_len, wl.max_seq_len, split_tokens, wl.dtype)
    b["ws"] = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    return b


def make_phases(wl, b, split_tokens):
    """The step's calls: prepare_inputs_and_plan (index tensors and the
    attention work list), kv_cache_write, and the attention run (main +
    reduce) over that list.  Plan followed by run is the same work as one
    paged_attention_varlen call."""
    import paged_kv_cache_prepare_amd as pkv
    prep = b["prep"]
    kc, vc = wl.key_cache, wl.value_cache

    def prepare_plan():
        pkv.prepare_inputs_and_plan(b["nst"], b["nct"], b["bt"], num_tokens=wl.num_tokens,
                                    block_size=wl.block_size, num_blocks=wl.num_blocks,
                                    num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
                                    head_dim=wl.head_dim, max_query_len=wl.max_query_len,
                                    max_seq_len=wl.max_seq_len, dtype=wl.dtype,
                                    split_tokens=split_tokens, workspace=b["ws"], out=prep)

    def write():
        if b["ks"] is None:
            pkv.kv_cache_write(wl.key, wl.value, kc, vc, prep["slot_mapping"],
                               block_size=wl.block_size)
        else:
            pkv.kv_cache_write_fp8(wl.key, wl.value, kc, vc, prep["slot_mapping"], b["ks"],
                                   b["vs"], block_size=wl.block_size)

    def run():
        pkv.paged_attention(wl.q, kc, vc, prep["query_start_loc"], prep["seq_lens"], b["bt"],
                            max_query_len=wl.max_query_len, max_seq_len=wl.max_seq_len,
                            scale=wl.scale, out=b["out"], split_tokens=split_tokens,
                            workspace=b["ws"], k_scale=b["ks"], v_scale=b["vs"], planned=True)

    return prepare_plan, write, run


def roofline_of(work, t_ms):
    """Fraction of the roofline for the attention work ``work`` done in
    ``t_ms``: the bound is max(t_bytes, t_flops) with t_bytes = unique
    algorithmic bytes / HBM peak and t_flops = visible-pair flops / bf16 MFMA
    peak; achieved is reported in the unit of the larger one."""
    t = t_ms / 1e3
    flops = work["flops_decode"] + work["flops_prefill"]
    t_bytes = work["bytes_unique"] / (HBM_PEAK_GBS * 1e9)
    t_flops = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    if t_flops > t_bytes:
        ach = flops / t / 1e12
        r = {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
             "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        ach = work["bytes_unique"] / t / 1e9
        r = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(ach / HBM_PEAK_GBS, 4)}
    r.update({"algorithmic_bytes": work["bytes_unique"], "algorithmic_flops": flops,
              "avg_ms": round(t_ms, 4), "hbm_gbs": round(work["bytes_unique"] / t / 1e9, 1),
              "tflops": round(flops / t / 1e12, 2),
              "t_bytes_ms": round(t_bytes * 1e3, 4), "t_flops_ms": round(t_flops * 1e3, 4)})
    return r


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path: the hot path is measured on one GPU's share at its real shape.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib)
        return
    if args.op != "step":
        bench_op(args)
        return
    import torch
    from paged_kv_cache_prepare_amd import workloads

    dev = torch.device("cuda:0")
    full = workloads.config(args.workload, device=dev)
    if args.kv_dtype == "fp8":
        if full.dtype != torch.bfloat16:
            print("an FP8 cache needs bf16 queries (workloads 2-5)", file=sys.stderr)
            sys.exit(2)
        full = workloads.to_fp8(full, *FP8_SCALES)
    group = full.num_q_heads // full.num_kv_heads
    short = full.num_scheduled_tokens * group <= 16
    subs = {"decode": np.nonzero(short)[0], "prefill": np.nonzero(~short)[0]}
    wl = full
    if args.rows != "all":
        if len(subs[args.rows]) == 0:
            print(f"workload {args.workload} has no {args.rows} rows", file=sys.stderr)
            sys.exit(2)
        wl = workloads.select(full, subs[args.rows])
    work = algorithmic_work(wl)
    T = wl.num_tokens
    stream = torch.cuda.current_stream(dev)
    # the cache flush: a 512 MiB write (twice the 256 MB MALL) before every timed
    # iteration, outside the event brackets, so no timed call finds the pools
    # in L2 or the MALL from the previous iteration
    scratch = torch.empty((512 << 20) // 4, dtype=torch.float32, device=dev)

    def flush():
        scratch.fill_(1.0)

    b = step_buffers(wl, args.split_tokens)
    prepare_plan, write, run = make_phases(wl, b, args.split_tokens)

    def step():
        prepare_plan()
        write()
        run()

    def events(n):
        return [torch.cuda.Event(enable_timing=True) for _ in range(n)]

    for _ in range(args.warmup):
        flush()
        step()
    clock_reader = ClockReader()
    try:
        calib = Calib()
    except Exception as exc:  # measurement extras only: the bench line stands without them
        print(f"calibration kernels unavailable: {exc}", file=sys.stderr)
        calib = None
    # timed region: K steps, each after a flush, each bracketed by events
    ev = [events(2) for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for k in range(args.steps):
        flush()
        ev[k][0].record(stream)
        step()
        ev[k][1].record(stream)
    torch.cuda.synchronize(dev)
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    step_ms = [e[0].elapsed_time(e[1]) for e in ev]
    # phase pass, same protocol: events between the calls
    ph = [events(4) for _ in range(args.steps)]
    for k in range(args.steps):
        flush()
        ph[k][0].record(stream)
        prepare_plan()
        ph[k][1].record(stream)
        write()
        ph[k][2].record(stream)
        run()
        ph[k][3].record(stream)
    torch.cuda.synchronize(dev)
    phase_ms = {name: [e[i].elapsed_time(e[i + 1]) for e in ph]
                for i, name in enumerate(("prepare_and_plan", "kv_write", "run"))}
    # the decode rows and the prompt rows alone over the same pools: the
    # per-path fractions (same protocol, attention run only)
    sub_lines = {}
    if args.rows == "all":
        for name, reqs in subs.items():
            if len(reqs) == 0 or len(reqs) == wl.num_reqs:
                continue
            sw = workloads.select(full, reqs)
            sb = step_buffers(sw, args.split_tokens)
            s_prep_plan, _, s_run = make_phases(sw, sb, args.split_tokens)
            s_prep_plan()
            for _ in range(max(2, args.warmup // 2)):
                flush()
                s_run()
            sev = [events(2) for _ in range(args.steps)]
            for k in range(args.steps):
                flush()
                sev[k][0].record(stream)
                s_run()
                sev[k][1].record(stream)
            torch.cuda.synchronize(dev)
            ms = pct([e[0].elapsed_time(e[1]) for e in sev])
            sr = roofline_of(algorithmic_work(sw), ms["median"])
            sr["traffic"] = measured_traffic(f"w{args.workload}_{name}_split{args.split_tokens}"
                                             + ("_fp8" if args.kv_dtype == "fp8" else ""))
            sub_lines[name] = {"rows": sw.num_tokens, "requests": sw.num_reqs,
                               "run_ms": ms, **sr}
            if name == "decode" and calib is not None:
                sub_lines[name]["read_ceiling"] = read_ceiling(
                    calib, sw, sb, ms["median"], algorithmic_work(sw)["bytes_unique"], flush,
                    args.steps, stream)
            del sb
    run_ceiling = None
    if calib is not None and len(subs["prefill"]) == 0 and args.rows != "prefill":
        run_ceiling = read_ceiling(calib, wl, b, pct(phase_ms["run"])["median"],
                                   work["bytes_unique"], flush, args.steps, stream)

    # clocks while the attention run executes: --clock-runs runs queued back
    # to back (no flush).  The shader clock comes from a wave that spins on a
    # second stream from the end of the second run for 80 % of the expected
    # rest; the memory clock from amdsmi, read until the last run ends.
    done_ev = torch.cuda.Event()
    start_ev = torch.cuda.Event()
    side = torch.cuda.Stream(dev)
    wave_clock = {}

    def enqueue():
        for i in range(args.clock_runs):
            run()
            if i == 1:
                start_ev.record(stream)
        done_ev.record(stream)
        if calib is not None and args.clock_runs > 2:
            side.wait_event(start_ev)
            spin = 0.8 * pct(phase_ms["run"])["median"] * (args.clock_runs - 2)
            wave_clock["under_load"] = calib.clock(spin, side)

    if args.clock_runs > 0:
        amd = clock_reader.under_load(enqueue, done_ev.query)
        torch.cuda.synchronize(dev)
        clocks = {"sclk_mhz": None, "mclk_mhz": None}
        if "under_load" in wave_clock:
            clocks["sclk_mhz"] = round(wave_clock["under_load"](), 1)
            idle = calib.clock(20.0, side)
            torch.cuda.synchronize(dev)
            clocks["sclk_idle_mhz"] = round(idle(), 1)
            clocks["sclk_source"] = ("one wave spinning on a second stream beside the runs: "
                                     "s_memtime ticks over s_memrealtime (100 MHz) ticks; "
                                     "sclk_idle_mhz is the same wave alone")
        if isinstance(amd.get("mclk_mhz"), dict):
            clocks["mclk_mhz"] = amd["mclk_mhz"]["median"]
            clocks["mclk_source"] = f"{amd['source']}, {amd['samples']} samples"
        clocks["note"] = (f"{args.clock_runs} attention runs of the workload back to back")
    else:
        clocks = {"note": "not read (--clock-runs 0)"}
    torch.cuda.synchronize(dev)

    graph_ms = None
    if args.graph:
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize(dev)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        gms = []
        for k in range(args.warmup + args.steps):
            flush()
            e0, e1 = events(2)
            e0.record(stream)
            graph.replay()
            e1.record(stream)
            torch.cuda.synchronize(dev)
            if k >= args.warmup:
                gms.append(e0.elapsed_time(e1))
        graph_ms = pct(gms)

    st = pct(step_ms)
    run_ms = pct(phase_ms["run"])
    roof = roofline_of(work, run_ms["median"])
    key = f"w{args.workload}_{args.rows}_split{args.split_tokens}"
    roof["traffic"] = measured_traffic(key + ("_fp8" if args.kv_dtype == "fp8" else ""))
    roof["kernel"] = ("attn_main_kernel + attn_reduce_kernel (pkv_paged_attention_run over "
                      "the step's plan), HIP events, median of the timed iterations, each after "
                      "a 512 MiB cache flush")
    roof["rule"] = "frac = max(t_bytes, t_flops) / t"
    if sub_lines:
        roof["sub_batches"] = sub_lines
    if run_ceiling is not None:
        roof["read_ceiling"] = run_ceiling

    cpu = cpu_baseline(wl, args.cpu_seconds, args.cpu_single_seconds)
    line = {
        "metric": METRIC,
        "value": round(T / (st["median"] / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": st["median"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16" if wl.dtype == torch.bfloat16 else "f32") +
                 ("+fp8kv" if args.kv_dtype == "fp8" else ""),
        "data": "synthetic (seeded N(0,1) K/V/Q, random block placement)",
        "config": {"workload": workloads.CONFIG_NAMES[args.workload], "num_reqs": wl.num_reqs,
                   "num_tokens": T, "context_tokens": work["context_tokens"],
                   "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads,
                   "head_dim": wl.head_dim, "block_size": wl.block_size, "seed": wl.seed,
                   "split_tokens": args.split_tokens, "rows": args.rows,
                   "kv_dtype": args.kv_dtype},
        "timing": {"protocol": "each of the K timed steps runs after a 512 MiB write (L2 and "
                               "MALL flush) and is bracketed by HIP events on the library's "
                               "stream; value = num_tokens / median step time",
                   "step_ms": st, "wall_ms_per_iteration_with_flush": round(wall_ms, 4)},
        "phases_ms": {name: pct(v) for name, v in phase_ms.items()},
        "context_tokens_per_s": round(work["context_tokens"] / (st["median"] / 1e3), 1),
        "roofline": roof,
        "clocks": clocks,
        "cpu_baseline": cpu,
    }
    if graph_ms is not None:
        line["graph"] = {"step_ms": graph_ms,
                         "note": "HIP-graph replays of the step, same flush protocol"}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
