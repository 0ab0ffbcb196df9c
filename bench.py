#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X: µs/step and achieved KV-read GB/s.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--workload c2] [--mode fused|two]

A step is one full decode call over one batch of synthetic input (map + merge,
or the single fused kernel; with append or cascade workloads those parts
too). Inputs are resident in HBM before timing starts. To keep the 256 MB
last-level cache (MALL) from serving repeated reads, steps rotate through
enough copies of the KV cache to cover >= 1 GiB; the single-copy ("warm")
figure is reported separately. The K timed steps are captured as one HIP graph
and replayed between two events (the median of three replays) (how a serving loop launches decode
steps: a graph launch costs ~5 µs once, its kernels then dispatch back to back);
the same K steps launched eagerly are timed too (`eager_us_per_step`, the median
of three regions), and
`--launch eager` makes those the headline.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_TFLOPS = 2500.0  # dense bf16 / fp16 matrix peak
METRIC = "decode attention µs/step + achieved KV-read GB/s (% of 8 TB/s HBM peak)"
WORKLOAD_TEXT = {
    "c1": "unpaged MHA decode: B=1, Hq=Hkv=32, D=128, 4096 contiguous fp16 tokens, 16 splits",
    "c2": "long-context GQA decode: B=1, Hq=32, Hkv=8, D=128, 131072 contiguous bf16 tokens",
    "c3": "paged batched decode: B=32, Hq=32, Hkv=8, D=128, page 16, lengths U[512,8192], bf16",
    "c4": "decode with KV append + NeoX rotary: B=4, Hq=32, Hkv=8, D=128, max_seqlen 2048, fp16",
    "c5": "cascade: 64 requests, Hq=32, Hkv=8, D=128, shared 16384-token prefix + U[256,2048] suffix, "
          "page 64, bf16",
    "c2f8": "long-context GQA decode: B=1, Hq=32, Hkv=8, D=128, 131072 contiguous float8 e4m3fn tokens, "
            "per-(request, KV head) descales, bf16 queries",
    "c3f8": "paged batched decode: B=32, Hq=32, Hkv=8, D=128, page 16, lengths U[512,8192], float8 e4m3fn "
            "KV with per-(request, KV head) descales, bf16 queries",
    "c2g8": "long-context GQA decode with eight query heads per KV head: B=1, Hq=64, Hkv=8, D=128, "
            "131072 contiguous bf16 tokens",
    "c1f8": "unpaged MHA decode: B=1, Hq=Hkv=32, D=128, 4096 contiguous float8 e4m3fn tokens, "
            "per-(request, KV head) descales, bf16 queries, 16 splits",
    "c2g2f8": "long-context GQA decode with two query heads per KV head: B=1, Hq=16, Hkv=8, D=128, "
              "131072 contiguous float8 e4m3fn tokens, per-(request, KV head) descales, bf16 queries",
    "c5f8": "cascade: 64 requests, Hq=32, Hkv=8, D=128, shared 16384-token prefix + U[256,2048] suffix, "
            "page 64, float8 e4m3fn pool with per-(request, KV head) descales, bf16 queries",
}
# every library source: a change to any of them (kernels, launch code, planner) marks stored counters stale
KERNEL_SOURCES = sorted(f for f in os.listdir(os.path.join(ROOT, "decode_attention_fdec_amd", "csrc"))
                        if f.endswith((".hip", ".h", ".cpp")))


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "decode_attention_fdec_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Runner:
    """Device copies of one workload plus a step function (rotates KV copies)."""

    def __init__(self, F, case, mode: str, splits: int, min_footprint: int, dev):
        import torch

        self.F, self.case, self.mode = F, case, mode
        self.dev = dev
        self.q = case.q.to(dev)
        self.lens = case.seq_lens.to(dev)
        self.table = None if case.page_table is None else case.page_table.to(dev)
        # float8 caches: per (request, KV head) descales
        self.kd = None if case.k_descale is None else case.k_descale.to(dev)
        self.vd = None if case.v_descale is None else case.v_descale.to(dev)
        kv_footprint = 2 * case.k.numel() * case.k.element_size()
        self.copies = max(1, min(64, math.ceil(min_footprint / kv_footprint)))
        self.k = [case.k.to(dev) for _ in range(self.copies)]
        self.v = [case.v.to(dev) for _ in range(self.copies)]
        self.append = None
        if case.k_new is not None:
            self.k_new, self.v_new = case.k_new.to(dev), case.v_new.to(dev)
            self.cos = None if case.rope_cos is None else case.rope_cos.to(dev)
            self.sin = None if case.rope_sin is None else case.rope_sin.to(dev)
            self.append = F.make_append(self.k_new, self.v_new, self.cos, self.sin, case.rotary_dim)
        B, Hq, D = case.q.shape
        self.cascade = case.prefix_pages is not None
        if self.cascade:
            self.prefix_pages = case.prefix_pages.to(dev)
            sp, ss = F.cascade_plan(B, Hq, case.Hkv, case.prefix_len, case.capacity, case.page_size,
                                    kv_dtype=case.dtype)
            self.S = (sp, ss)
            self.out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
            self.lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
            self.ws = F.Workspace(F.cascade_workspace_size(B, Hq, case.Hkv, D, sp, ss), dev)
            self.i = 0
            return
        if mode == "bal":
            # balanced split: `splits` is the block count per group of KV heads (0 = default)
            self.S = max(0, splits)
            self.out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
            self.lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
            self.ws = F.Workspace(F.balanced_workspace_size(B, Hq, case.Hkv, D, self.S), dev)
            self.i = 0
            return
        if splits <= 0:
            splits = case.num_splits
        if splits <= 0:
            lens_host = (case.seq_lens + (1 if case.k_new is not None else 0)).tolist()
            splits = F.plan(B, Hq, case.Hkv, lens_host, case.capacity, case.page_size, kv_dtype=case.dtype)
        self.S = splits
        self.i = 0
        if mode.startswith("multi"):
            # q_len query tokens per request (speculative decode), the case's cache
            import synth

            self.q_len = int(mode[len("multi"):])
            self.q = synth.multi_query(300 + self.q_len, case, self.q_len).to(dev)
            self.out = torch.empty(B, self.q_len, Hq, D, dtype=torch.float32, device=dev)
            self.lse = torch.empty(B, Hq, self.q_len, dtype=torch.float32, device=dev)
            self.ws = F.Workspace(F.workspace_size(B * self.q_len, Hq, case.Hkv, D, splits), dev)
            return
        self.out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
        self.lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
        self.ws = F.Workspace(F.workspace_size(B, Hq, case.Hkv, D, splits), dev)

    def step(self, copy: int | None = None) -> None:
        c = self.i % self.copies if copy is None else copy
        self.i += 1
        if self.cascade:
            self.F.cascade_decode(self.q, self.k[c], self.v[c], self.table, self.prefix_pages,
                                  self.case.prefix_len, self.lens, self.S[0], self.S[1], out=self.out,
                                  lse=self.lse, workspace=self.ws, k_descale=self.kd, v_descale=self.vd)
            return
        if self.mode.startswith("multi"):
            self.F.decode_multi(self.q, self.k[c], self.v[c], self.lens, page_table=self.table, num_splits=self.S,
                                out=self.out, lse=self.lse, workspace=self.ws, k_descale=self.kd, v_descale=self.vd)
            return
        if self.mode == "bal":
            self.F.decode_balanced(self.q, self.k[c], self.v[c], self.lens, page_table=self.table,
                                   num_blocks=self.S, out=self.out, lse=self.lse, workspace=self.ws,
                                   k_descale=self.kd, v_descale=self.vd)
            return
        self.F.decode(self.q, self.k[c], self.v[c], self.lens, page_table=self.table, num_splits=self.S,
                      append=self.append, fused=(self.mode == "fused"), out=self.out, lse=self.lse,
                      workspace=self.ws, k_descale=self.kd, v_descale=self.vd)


def time_region(runner: Runner, steps: int, warmup: int, copy=None):
    """Whole-region time of `steps` back-to-back steps (events on the launch stream)."""
    import torch

    for _ in range(warmup):
        runner.step(copy)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        runner.step(copy)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps  # ms


def time_region_graph(runner: Runner, steps: int, warmup: int):
    """Whole-region time of `steps` steps captured as one HIP graph (on a side stream)
    and replayed between events on the launch stream: one untimed replay, then the
    median of three timed ones.
    The steps rotate KV copies as eager steps do, so the graph holds `steps`
    distinct steps."""
    import torch

    for _ in range(warmup):
        runner.step()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for _ in range(steps):
                runner.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / steps)
    return sorted(times)[1]  # ms, the median of three replays


def time_per_launch(runner: Runner, steps: int, copy=None):
    """Per-step durations from an event pair around each step (launch-gap free)."""
    import torch

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        runner.step(copy)
        b.record()
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in ev)  # ms


CASCADE_SINGLE = "cascade prefix + suffix (single kernel)"


def stage_labels(runner: Runner, nkernels: int = 0):
    """The kernels one step launches, in order (a cascade step launches two when
    its prefix and suffix blocks share one grid, three otherwise)."""
    if runner.cascade:
        if nkernels == 2:
            return [CASCADE_SINGLE, "cascade merge"]
        return ["cascade prefix (matrix cores)", "suffix map (balanced split)", "cascade merge"]
    if runner.mode == "bal":
        return ["map (balanced split)", "segment merge"]
    if runner.mode == "fused":
        return ["map + merge (single kernel)"]
    return ["map", "merge"]


def time_stages(F, runner: Runner, steps: int) -> dict:
    """Mean duration (us) of each kernel of a step, from the library's stage-timing
    events (fdec_trace_start / fdec_trace_stop) on the launch stream, over `steps`
    back-to-back steps."""
    import torch

    for _ in range(3):
        runner.step()
    torch.cuda.synchronize()
    F.trace_start(8 * steps + 8)
    for _ in range(steps):
        runner.step()
    ms, kinds = F.trace_stop()
    by = {}
    for m, k in zip(ms, kinds):
        if k >= 1:
            by.setdefault(k, []).append(m * 1e3)
    labels = stage_labels(runner, len(by))
    return {(labels[k - 1] if k - 1 < len(labels) else f"kernel {k}"): round(sum(v) / len(v), 2)
            for k, v in sorted(by.items())}


def roofline_entry(case, stages: dict, runner: Runner) -> dict:
    """HBM roofline of the step's dominant kernel(s): algorithmic bytes / mean duration."""
    out = {}
    if runner.cascade and CASCADE_SINGLE in stages:
        # prefix and suffix blocks in one kernel: its bytes are every attended K/V
        # byte (the prefix once), its flops the prefix's; floor = max of the two
        nb = case.kv_bytes()
        t = stages[CASCADE_SINGLE]
        flops = 4.0 * case.D * case.B * case.Hq * case.prefix_len
        floor = max(nb / HBM_PEAK_GBS / 1e3, flops / MFMA_BF16_TFLOPS / 1e6)
        out["prefix_suffix"] = {"bound": "hbm", "achieved": round(nb / (t * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                                "unit": "GB/s", "frac": round(nb / (t * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                "kernel": CASCADE_SINGLE, "avg_launch_us": t, "algorithmic_bytes_per_launch": nb,
                                "prefix_tflops": round(flops / (t * 1e-6) / 1e12, 1), "floor_us": round(floor, 2),
                                "frac_of_floor": round(floor / t, 4)}
        return out
    if runner.cascade:
        pre = case.prefix_len * case.Hkv * 2 * case.D * case.k.element_size()
        suf = case.kv_bytes() - pre
        t_pre = stages["cascade prefix (matrix cores)"]
        t_suf = stages["suffix map (balanced split)"]
        rows = case.B * case.Hq
        flops = 4.0 * case.D * rows * case.prefix_len
        out["prefix"] = {"bound": "hbm", "achieved": round(pre / (t_pre * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(pre / (t_pre * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                         "avg_launch_us": t_pre, "algorithmic_bytes_per_launch": pre,
                         "tflops": round(flops / (t_pre * 1e-6) / 1e12, 1), "mfma_peak_tflops": MFMA_BF16_TFLOPS,
                         "floor_us": round(max(pre / HBM_PEAK_GBS / 1e3, flops / MFMA_BF16_TFLOPS / 1e6), 2),
                         "frac_of_floor": round(max(pre / HBM_PEAK_GBS / 1e3, flops / MFMA_BF16_TFLOPS / 1e6) / t_pre,
                                                4)}
        out["suffix"] = {"bound": "hbm", "achieved": round(suf / (t_suf * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(suf / (t_suf * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                         "avg_launch_us": t_suf, "algorithmic_bytes_per_launch": suf}
        return out
    label = next(iter(stages))
    t = stages[label]
    nb = case.kv_bytes()
    return {"bound": "hbm", "achieved": round(nb / (t * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(nb / (t * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "kernel": label, "avg_launch_us": t,
            "algorithmic_bytes_per_launch": nb}


CALIB_BYTES = 256 << 20


def summarize_pmc(fetch_csv: str, write_csv: str) -> dict:
    """HBM traffic of the step's dominant kernel (the map kernel, or the
    single-launch cascade kernel) from rocprofv3 counter csv files.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what the same
    counter reads for the calibration probes: a plain read (FETCH) and a plain
    copy (WRITE) of CALIB_BYTES each.
    """
    import csv

    def per_kernel(path, counter):
        out = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                out.setdefault(r["Kernel_Name"], []).append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
        return out

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")

    def pick(d, key):  # median over the dispatches of the kernel
        vals = [v for k, vs in d.items() if key in k for _, v in vs]
        return sorted(vals)[len(vals) // 2] if vals else None

    def last(d, key):  # the calibration probes are the last read / copy dispatches of the run
        vals = [dv for k, vs in d.items() if key in k for dv in vs]
        return max(vals)[1] if vals else None

    fetch_scale = CALIB_BYTES / 1024.0 / last(f, "read_kernel")
    write_scale = CALIB_BYTES / 1024.0 / last(w, "copy_kernel")
    dom = "map_kernel" if any("map_kernel" in k for k in f) else "cascade_fused_kernel"
    fk, wk = pick(f, dom), pick(w, dom)
    kernels = {}  # every library kernel of the run: median scaled bytes per dispatch
    for name in sorted(set(f) | set(w)):
        short = re.sub(r"\(.*", "", name).replace("void ", "").strip()
        if not short.startswith("fdec::"):
            continue
        fr, wr = pick(f, name), pick(w, name)
        kernels[short] = {"read_bytes": None if fr is None else int(round(fr * fetch_scale * 1024)),
                          "write_bytes": None if wr is None else int(round(wr * write_scale * 1024))}
    res = {"fetch_kib": fk, "write_kib": wk, "fetch_scale": round(fetch_scale, 4),
           "write_scale": round(write_scale, 4), "kernels": kernels, "kernel_hash": kernel_hash()}
    if fk is not None and wk is not None:
        res.update({"traffic_bytes": int(round((fk * fetch_scale + wk * write_scale) * 1024)),
                    "read_bytes": int(round(fk * fetch_scale * 1024)),
                    "write_bytes": int(round(wk * write_scale * 1024))})
    return res


def probe_ceiling(F, nbytes: int, dev, reps: int = 20) -> dict:
    """What the memory system delivers at this footprint: the median rate of
    fdec_probe_read (best-effort streaming read, non-temporal 16-byte loads) and
    of fdec_probe_stream (the map kernels' LDS-DMA load path, static slices) over
    nbytes, rotating three buffers so the last-level cache cannot serve repeats."""
    import torch

    n = max(64 << 20, (nbytes + (256 << 10) - 1) // (256 << 10) * (256 << 10))
    bufs = [torch.ones(n, dtype=torch.uint8, device=dev) for _ in range(3)]
    sink = torch.zeros(F.PROBE_BLOCKS + 1, dtype=torch.int32, device=dev)
    out = {}
    for key, fn in (("probe_read_GBps", lambda b: F.probe_read(b, sink)),
                    ("probe_lds_dma_GBps", lambda b: F.probe_stream(b, F.PROBE_STATIC, 1, sink))):
        for i in range(3):
            fn(bufs[i])
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(ev):
            a.record()
            fn(bufs[i % 3])
            b.record()
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) for a, b in ev)
        out[key] = round(n / (t[len(t) // 2] * 1e-3) / 1e9, 1)
    out["probe_bytes"] = n
    del bufs
    return out


SQ_COUNTERS = ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_INSTS_LDS", "SQ_LDS_IDX_ACTIVE",
               "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE"]


def summarize_counters(paths, cu_count: int = 256, xcc_count: int = 8) -> dict:
    """Per-kernel medians (over dispatches) of rocprofv3 --pmc csv files, with the
    derived figures rocprofv3 defines for them. The csv holds each counter summed
    over the GPU's dies; GRBM_GUI_ACTIVE (cycles the GPU is busy) is counted once
    per die, and rocprofv3's formulas take one die's value (its max), here the
    sum over xcc_count dies divided by that count:
      occupancy_pct  = 400 * SQ_WAVE_CYCLES / busy / CUs / 32
                       (resident waves as % of 32 per CU; SQ_WAVE_CYCLES is in quad-cycles),
      waves_per_cu   = 4 * SQ_WAVE_CYCLES / busy / CUs,
      lds_bank_conflicts_per_access = SQ_LDS_BANK_CONFLICT / (SQ_LDS_IDX_ACTIVE - SQ_LDS_BANK_CONFLICT)
                       (stall cycles per cycle of useful indexed LDS work),
      lds_bank_conflict_pct_of_time = 100 * SQ_LDS_BANK_CONFLICT / busy / CUs."""
    import csv

    per = {}  # kernel -> counter -> dispatch -> value (summed over dimensions)
    for path in paths:
        for r in csv.DictReader(open(path)):
            k = re.sub(r"\(.*", "", r["Kernel_Name"]).replace("void ", "").strip()
            c = r["Counter_Name"]
            d = per.setdefault(k, {}).setdefault(c, {})
            d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    out = {}
    for k, cs in per.items():
        med = {c: sorted(v.values())[len(v) // 2] for c, v in cs.items()}
        med["dispatches"] = max(len(v) for v in cs.values())
        g = med.get("GRBM_GUI_ACTIVE")
        g = g / xcc_count if g else g
        if g:
            med["busy_cycles_per_die"] = round(g)
        if g and "SQ_WAVE_CYCLES" in med:
            med["occupancy_pct"] = round(400.0 * med["SQ_WAVE_CYCLES"] / g / cu_count / 32, 2)
            med["waves_per_cu"] = round(4.0 * med["SQ_WAVE_CYCLES"] / g / cu_count, 3)
        if "SQ_LDS_BANK_CONFLICT" in med and "SQ_LDS_IDX_ACTIVE" in med:
            act = med["SQ_LDS_IDX_ACTIVE"] - med["SQ_LDS_BANK_CONFLICT"]
            med["lds_bank_conflicts_per_access"] = round(med["SQ_LDS_BANK_CONFLICT"] / act, 5) if act > 0 else None
            if g:
                med["lds_bank_conflict_pct_of_time"] = round(100.0 * med["SQ_LDS_BANK_CONFLICT"] / g / cu_count, 4)
        out[k] = med
    return out


def pct(xs, p):
    return xs[min(len(xs) - 1, int(round(p / 100.0 * (len(xs) - 1))))]


def map_kernel_name(case) -> str:
    """The map kernel fdec_decode_partials runs for a case (default kernel paths)."""
    G = case.q.shape[1] // case.Hkv
    if case.D == 128 and G in (4, 8) and os.environ.get("FDEC_MAP_PATH") != "vector":
        return "map_kernel_mfma_g4 (matrix cores)" if G == 4 else "map_kernel_mfma_g8 (matrix cores)"
    return "map_kernel (vector)"


def load_traffic(workload: str):
    """HBM traffic per launch from committed rocprofv3 counter summaries, if current."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_hash") != kernel_hash():
        return None  # the kernel changed since the counters were taken
    return t.get("traffic_bytes")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(case, budget_s: float):
    """The fp64 oracle on the same workload, timed on this host's cores: whole
    passes over the workload with every host thread (OpenMP over (request, query
    head)) and with one thread, median of 3 timed runs each. A run repeats passes
    until it has taken budget_s / 6 seconds (at least one pass)."""
    import oracle

    oracle.build(force=False)
    kv = oracle.KV(case.k, case.v, oracle.dtype_code(case.k), case.Hq, case.B, case.page_size, case.page_table,
                   case.prefix_pages, case.prefix_len, case.k_descale, case.v_descale)
    q = oracle.to_f64(case.q, oracle.dtype_code(case.q))
    scale = 1.0 / math.sqrt(case.D)

    def rate(threads):
        runs = []
        for _ in range(3):
            reps, t0 = 0, oracle.now()
            while True:
                oracle.decode(kv, q, case.seq_lens, scale, threads)
                reps += 1
                if oracle.now() - t0 >= budget_s / 6 or reps >= 1000:
                    break
            runs.append(case.kv_bytes() * reps / (oracle.now() - t0) / 1e9)
        return sorted(runs)[1], [round(r, 4) for r in runs]

    threads = oracle.max_threads()
    all_rate, all_runs = rate(threads)
    one_rate, one_runs = rate(1)
    return {"value": round(all_rate, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"whole passes of the fp64 oracle over the full workload ({case.name}, "
                      f"{case.kv_bytes()} KV bytes per pass), median of 3 runs of >= {budget_s / 6:.1f} s with "
                      f"{threads} OpenMP threads; rate = KV bytes per pass x passes / time",
            "runs_GBps": all_runs, "single_thread_GBps": round(one_rate, 4), "single_thread_runs_GBps": one_runs,
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


def measure_workload(F, name: str, mode: str, splits: int, steps: int, warmup: int, dev, launch: str = "graph"):
    import synth

    t0 = time.time()
    case = synth.workload(name)
    runner = Runner(F, case, mode, splits, 1 << 30, dev)
    log(f"[bench] {name}: inputs ready in {time.time() - t0:.1f}s, copies={runner.copies}, S={runner.S}")
    eager = sorted([time_region(runner, steps, warmup)] + [time_region(runner, steps, 0) for _ in range(2)])[1]
    ms, how = eager, "eager"
    if launch == "graph":
        try:
            ms, how = time_region_graph(runner, steps, 2), "hip_graph"
        except Exception as e:  # keep the eager figure if this runtime cannot capture
            how = f"eager (graph capture failed: {type(e).__name__})"
    per = time_per_launch(runner, steps)
    warm = time_region(runner, steps, 2, copy=0)
    stages = time_stages(F, runner, steps)
    nbytes = case.kv_bytes()
    res = {"us_per_step": round(ms * 1e3, 2), "kv_bytes": nbytes, "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
           "pct_of_peak": round(100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
           "step_us_p10_p50_p90": [round(pct(per, p) * 1e3, 2) for p in (10, 50, 90)],
           "launch": how, "eager_us_per_step": round(eager * 1e3, 2),
           "warm_us_per_step": round(warm * 1e3, 2), "num_splits": runner.S, "mode": mode,
           "kv_copies_rotated": runner.copies, "kernel_us": stages,
           "roofline": roofline_entry(case, stages, runner)}
    rl = res["roofline"] if not runner.cascade else res["roofline"].get("prefix_suffix", res["roofline"].get("suffix"))
    rl["traffic"] = load_traffic(name)  # HBM bytes of the map kernel from the stored counters, if current
    log(f"[bench] {name}: {res['us_per_step']} us/step, {res['GBps']} GB/s ({res['pct_of_peak']}% of peak)")
    return case, runner, res, per


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c2",
                    choices=["c1", "c2", "c3", "c4", "c5", "c2f8", "c3f8", "c2g8", "c1f8", "c2g2f8", "c5f8"])
    ap.add_argument("--mode", default="two", choices=["fused", "two", "bal"])
    ap.add_argument("--launch", default="graph", choices=["graph", "eager"],
                    help="time the K steps as one captured HIP graph replay (default) or as eager launches")
    ap.add_argument("--splits", type=int, default=0, help="0 = the planner's choice")
    ap.add_argument("--also", default="c1,c3,c4,c5,c2f8,c3f8,c2q2,c2q4,c2f8q4,c2g8,c1f8,c2g2f8,c5f8",
                    help="other workloads timed for context ('' = none)")
    ap.add_argument("--cpu-seconds", type=float, default=24.0, help="CPU oracle timing budget (all runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the streaming-read probes (profiler runs)")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run a plain read and a plain copy of 256 MiB (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarize rocprofv3 FETCH_SIZE / WRITE_SIZE csv files and exit")
    ap.add_argument("--summarize-counters", nargs="+", metavar="CSV",
                    help="per-kernel medians of rocprofv3 --pmc csv files (occupancy, LDS bank conflicts) and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        print(json.dumps(summarize_counters(args.summarize_counters), indent=1))
        return 0
    if args.summarize_pmc:
        print(json.dumps(summarize_pmc(*args.summarize_pmc), indent=1))
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the decode path runs on one GPU and has no multi-GPU mode", file=sys.stderr)
        return 2

    import torch

    import decode_attention_fdec_amd as F

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    F.load_library()
    dev = torch.device("cuda:0")

    case, runner, res, per = measure_workload(F, args.workload, args.mode, args.splits, args.steps,
                                              args.warmup, dev, args.launch)
    # the dominant kernel: the split-KV map kernel of the step (the suffix map of a
    # cascade), timed with the library's stage-timing events on its stream
    rl = res["roofline"] if not runner.cascade else res["roofline"].get("prefix_suffix", res["roofline"].get("suffix"))
    achieved = rl["achieved"]
    roofline = dict(rl)
    kname = ("cascade_fused_kernel (prefix and suffix blocks)" if rl.get("kernel") == CASCADE_SINGLE
             else map_kernel_name(case) + f" ({rl.get('kernel', 'suffix map')} stage of the timed step)")
    roofline.update({"traffic": load_traffic(args.workload), "kernel": kname, "kernel_hash": kernel_hash()})

    # attainable streaming read at the map kernel's footprint (the probes)
    import torch as _t

    if not args.no_probe:
        res.update(probe_ceiling(F, case.kv_bytes(), dev))
    if args.calibrate:
        src = _t.empty(CALIB_BYTES, dtype=_t.uint8, device=dev)
        dst = _t.empty(CALIB_BYTES, dtype=_t.uint8, device=dev)
        F.probe_read(src)
        F.probe_copy(dst, src)
        _t.cuda.synchronize()
        del src, dst
    if "probe_read_GBps" in res:
        res["pct_of_probe"] = round(100 * res["GBps"] / res["probe_read_GBps"], 1)
        roofline["kernel_pct_of_probe"] = round(100 * achieved / res["probe_read_GBps"], 1)
    del runner

    # the paged batch of mixed lengths runs on the balanced split (equal work per
    # block whatever the length mix); its uniform-split time is kept beside it
    others = {}
    runs = []
    for name in [x for x in args.also.split(",") if x and x != args.workload]:
        if name == "c3":
            runs += [("c3", "c3", "bal"), ("c3_uniform_splits", "c3", args.mode)]
        elif name == "c3f8":
            runs.append((name, name, "bal"))
        elif re.fullmatch(r"c\d+\w*?q\d+", name):  # e.g. c2q4 / c2f8q4: c2 / c2f8 with 4 query tokens
            base, q = name.rsplit("q", 1)
            runs.append((name, base, f"multi{q}"))
        else:
            runs.append((name, name, args.mode))
    for key, name, mode in runs:
        try:
            _, r2, res2, _ = measure_workload(F, name, mode, 0, args.steps, args.warmup, dev, args.launch)
            others[key] = res2
            del r2
        except F.FdecError as e:  # a workload whose path is not built yet
            others[key] = {"error": str(e)}
            log(f"[bench] {key}: {e}")
        _t.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle ...")
        cpu = cpu_baseline(case, args.cpu_seconds)
        log(f"[bench] oracle: {cpu['value']} GB/s on {cpu['cores']} threads")

    line = {
        "metric": METRIC,
        "value": res["GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["us_per_step"] / 1e3, 5),
        "us_per_step": res["us_per_step"],
        "pct_of_peak": res["pct_of_peak"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",  # arithmetic type: fp32 math on fp16/bf16 KV (kv_dtype in config)
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.workload],
                   "kv_dtype": {_t.bfloat16: "bf16", _t.float16: "fp16"}.get(case.dtype, "fp8_e4m3fn"), **res},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "other_workloads": others,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
