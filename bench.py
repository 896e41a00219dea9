#!/usr/bin/env python3
"""Benchmark of one verify step (split kernel + combine kernel) on one MI355X.

Default workload: batch 1, live length 261,888 + 256 = 262,144 tokens with the
q = 8 verify rows at the end, 16 query heads / 2 KV heads, head_dim 256,
E4M3 K/V with per-head scales and 1% outlier tokens, page size 64 (the
256K-context q8 case the metric is quoted on). Inputs are synthetic, seeded and
resident in HBM before the timed region starts.

Timing follows the pages' protocol of graph-replayed operator timing ("[Bugfix]
Use FP32 state and E4M3 defaults for DFlash2", Test Plan and Results: 20
warmups, then timed replays): the step (split and combine) is captured once
as a HIP graph; after a 0.3 s pre-warm and W untimed warmup rounds, K timed
rounds follow. Before every timed run an untimed read of a clean 1 GiB
buffer evicts the 256 MB Infinity Cache and the L2s, so the KV bytes come
from HBM. The scrub only reads: a scrub that writes leaves dirty lines whose
write-back then competes with the timed kernel's reads. Each replay is
bracketed by HIP events on the stream the graph is launched on. `value`,
`ms_per_step` and `kv_pct_of_peak_hbm` are those replays. Each round also
times the same step launched eagerly (the two kernels back to back, events
around the step) and an eager step with an event between the kernels for
the per-kernel figures (the split kernel's mean launch time is the
roofline's denominator); the three alternate in mirrored order round by
round, as the pages alternate their variants in ABBA blocks, so that all
three see the same clocks.

Prints one JSON line. `value` is the achieved KV read rate: live K+V bytes of
the step divided by the mean step time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verify-step us + achieved KV HBM GB/s (% peak), q8 E4M3 at 256K ctx"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, AMD published
PEAK_FP16_MFMA_TFLOPS = 2500.0  # MI355X dense FP16 matrix peak, AMD published
KERNEL_SRC = os.path.join(ROOT, "paged_fp8_split_amd", "csrc", "pfs_kernels.hip")


def note(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    """sha256[:16] of the kernel source with comments and blank lines removed,
    so that profiles stay valid across comment-only edits."""
    import re

    with open(KERNEL_SRC) as f:
        text = f.read()
    lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
    code = "\n".join(ln for ln in lines if ln.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def traffic_from_profiles(cfg: int):
    """HBM bytes per split-kernel launch measured with rocprofv3 PMC counters
    (profiles/traffic_split_config<cfg>.json), if those counters were taken on
    the current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"traffic_split_config{cfg}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    return t.get("bytes_per_launch")


def sq_counters_from_profiles(cfg: int):
    """Split-kernel SQ counter figures (profiles/sq_split_config<cfg>.json:
    MFMA busy fraction per SIMD and the like), if those counters were taken on
    the current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"sq_split_config{cfg}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    return t.get("derived")


def split_mfma_flops(w) -> int:
    """Dense matrix work of the split kernel: S = Q K^T and O = P V over every
    live key, 2 flops per multiply-add, for the G x q rows of each KV head."""
    import numpy as np

    L = np.clip(w.live_len.astype(np.int64), 0, w.capacity)
    rows = w.q * w.group
    return int(L.sum()) * w.num_kv_heads * rows * w.head_dim * 2 * 2


def split_algorithmic_bytes(w, plan) -> int:
    """Bytes the split kernel must move: live K+V, Q, the block-table entries of
    the live pages, and the FP32 partials (max, sum, D accumulators per row) of
    every split that holds live tokens."""
    import numpy as np

    L = np.clip(w.live_len.astype(np.int64), 0, w.capacity)
    kv = int(L.sum()) * w.num_kv_heads * w.head_dim * 2
    qb = w.batch * w.q * w.num_q_heads * w.head_dim * 2
    bt = int((-(-L // w.page_size)).sum()) * 4
    rows = w.q * w.group
    splits = int((-(-L // plan.tokens_per_split)).sum())
    ws = splits * w.num_kv_heads * rows * (w.head_dim + 2) * 4
    return kv + qb + bt + ws


def step_algorithmic_bytes(w, plan) -> int:
    """Bytes one verify step must move: the split kernel's (live K+V, Q,
    block-table entries, FP32 partials written), the combine's read of those
    partials, and the FP16 output."""
    import numpy as np

    L = np.clip(w.live_len.astype(np.int64), 0, w.capacity)
    rows = w.q * w.group
    splits = int((-(-L // plan.tokens_per_split)).sum())
    ws = splits * w.num_kv_heads * rows * (w.head_dim + 2) * 4
    out = w.batch * w.q * w.num_q_heads * w.head_dim * 2
    return split_algorithmic_bytes(w, plan) + ws + out


def mfma_report(w, split_ms: float, cfg) -> dict:
    """Matrix-core use of the split kernel: the dense FP16 work over the mean
    launch time against the FP16 MFMA peak, and the MFMA-busy fraction that
    the SQ counters measured on this kernel source for the default mode of
    workload cfg (None if they are stale, or for cfg None)."""
    flops = split_mfma_flops(w)
    tf = flops / (split_ms * 1e-3) / 1e12
    sq = (sq_counters_from_profiles(cfg) if cfg is not None else None) or {}
    return {
        "kernel": "pfs_split_kernel",
        "flop_per_launch": flops,
        "achieved": round(tf, 2),
        "peak": PEAK_FP16_MFMA_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(tf / PEAK_FP16_MFMA_TFLOPS, 4),
        "busy_frac_counters": sq.get("mfma_busy_frac"),
        "valu_busy_frac_counters": sq.get("valu_busy_frac"),
        "counters_source": (f"rocprofv3 --pmc SQ counters of this kernel source, read from "
                            f"profiles/sq_split_config{cfg}.json (not measured in this run)") if sq else None,
    }


def codec_timing(w, t, dev, evict, reps: int = 20) -> dict:
    """The two codec kernels on the same workload, HIP events on the current
    stream: the draft-token quantize-on-write (q rows x KV heads, launch
    bound) and the scaled paged E4M3 -> FP16 bridge over every live token of
    the K pool (cache scrubbed before each launch). Runs last: the append
    writes the draft slots of the pools."""
    import numpy as np
    import torch

    import paged_fp8_split_amd as pfs

    rng = np.random.default_rng(12)
    shape = (w.batch, w.q, w.num_kv_heads, w.head_dim)
    kn = torch.from_numpy(rng.normal(0, 1, shape).astype(np.float16)).to(dev)
    vn = torch.from_numpy(rng.normal(0, 1, shape).astype(np.float16)).to(dev)
    out = torch.empty((w.batch, w.capacity, w.num_kv_heads, w.head_dim), dtype=torch.float16, device=dev)

    def timed(fn, scrub):
        ms = []
        for k in range(reps + 3):
            if scrub:
                evict()
            T = timer()
            e0, e1 = T.event(), T.event()
            stream = torch.cuda.current_stream()
            T.record(e0, stream)
            fn()
            T.record(e1, stream)
            torch.cuda.synchronize()
            if k >= 3:
                ms.append(T.elapsed_ms(e0, e1))
            T.destroy([e0, e1])
        return float(np.median(ms)) * 1e3

    # the append is a few microseconds of GPU work: time a graph of `chain`
    # back-to-back appends (idempotent) so that neither the binding's host
    # overhead nor the graph launch is inside the per-append figure
    append = lambda: pfs.kv_append(kn, vn, t["k_scale"], t["v_scale"], t["block_table"], t["live_len"],
                                   t["k_pool"], t["v_pool"])
    append()
    torch.cuda.synchronize()
    chain = 50
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(chain):
            append()
    torch.cuda.synchronize()
    app_us = timed(graph.replay, False) / chain
    br_us = timed(lambda: pfs.dequant_paged(t["k_pool"], t["block_table"], t["live_len"], scale=t["k_scale"],
                                            out=out), True)
    live = int(np.clip(w.live_len.astype(np.int64), 0, w.capacity).sum())
    br_bytes = live * w.num_kv_heads * w.head_dim * 3 + (w.batch * w.capacity - live) * w.num_kv_heads * w.head_dim * 2
    app_bytes = int(np.prod(shape)) * (2 * 2 + 2)
    return {
        "kv_append_us": round(app_us, 2),  # per append in a graph of back-to-back appends
        "kv_append_bytes": app_bytes,
        "bridge_scaled_us": round(br_us, 2),
        "bridge_bytes": br_bytes,
        "bridge_GBps": round(br_bytes / (br_us * 1e-6) / 1e9, 1),
        "bridge_frac_of_peak": round(br_bytes / (br_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
    }


class HipTimer:
    """Timing events recorded on a HIP stream through the HIP runtime that
    torch itself loaded, created with hipEventDisableSystemFence: recording
    such an event skips the system-scope cache write-back and invalidate that
    a default event performs (HIP's documentation offers the flag for timing
    events for exactly that reason). A default event between two kernels
    leaves the GPU idle for about 5.5 us on this stack (rocprofv3 kernel
    trace: scrub end -> split start is 0 without an event, 5.5 us with one),
    which would be counted inside the timed step."""

    FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        import ctypes

        import torch

        torch.cuda.init()
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64.so" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime (libamdhip64.so) is not loaded")
        self.hip = ctypes.CDLL(path)
        self.c = ctypes
        for fn, args in (("hipEventCreateWithFlags", [ctypes.c_void_p, ctypes.c_uint]),
                         ("hipEventRecord", [ctypes.c_void_p, ctypes.c_void_p]),
                         ("hipEventSynchronize", [ctypes.c_void_p]),
                         ("hipEventElapsedTime", [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
                         ("hipEventDestroy", [ctypes.c_void_p])):
            getattr(self.hip, fn).argtypes = args
            getattr(self.hip, fn).restype = ctypes.c_int

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed: hipError {rc}")

    def event(self):
        ev = self.c.c_void_p()
        self._ok(self.hip.hipEventCreateWithFlags(self.c.byref(ev), self.FLAGS), "hipEventCreateWithFlags")
        return ev

    def record(self, ev, stream):
        self._ok(self.hip.hipEventRecord(ev, self.c.c_void_p(stream.cuda_stream)), "hipEventRecord")

    def elapsed_ms(self, a, b) -> float:
        self._ok(self.hip.hipEventSynchronize(b), "hipEventSynchronize")
        ms = self.c.c_float()
        self._ok(self.hip.hipEventElapsedTime(self.c.byref(ms), a, b), "hipEventElapsedTime")
        return float(ms.value)

    def destroy(self, evs):
        for ev in evs:
            self.hip.hipEventDestroy(ev)


_TIMER = None


def timer() -> HipTimer:
    global _TIMER
    if _TIMER is None:
        _TIMER = HipTimer()
    return _TIMER


def time_steps(split, combine, evict, stream, steps: int, warmup: int, mid_event: bool):
    """Warm up, then time `steps` scrubbed split + combine steps with HIP
    events (HipTimer) on `stream`. With `mid_event` an event between the two
    kernels also splits each step into its kernels (the step itself is timed
    without it). Returns (split_ms, combine_ms, step_ms, wall_s); the first
    two are None without `mid_event`."""
    import numpy as np
    import torch

    for _ in range(warmup):
        evict()
        split()
        combine()
    torch.cuda.synchronize()
    note("warmup done; timing")
    T = timer()
    evs = [[T.event() for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    for k in range(steps):
        evict()
        T.record(evs[k][0], stream)
        split()
        if mid_event:
            T.record(evs[k][1], stream)
        combine()
        T.record(evs[k][2], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    step_ms = np.array([T.elapsed_ms(e[0], e[2]) for e in evs])
    split_ms = np.array([T.elapsed_ms(e[0], e[1]) for e in evs]) if mid_event else None
    comb_ms = np.array([T.elapsed_ms(e[1], e[2]) for e in evs]) if mid_event else None
    T.destroy([x for e in evs for x in e])
    return split_ms, comb_ms, step_ms, wall


def time_interleaved(graph, split, combine, evict, stream, steps: int, warmup: int, prewarm_s: float = 0.3):
    """The step three ways, interleaved so that each sees the same GPU state
    (clock ramp, temperature): as one replay of `graph`, eagerly (split and
    combine back to back), and eagerly with an event between the kernels
    (per-kernel times). Each timed run follows an untimed scrub and has HIP
    events (HipTimer) on `stream` around it; a round runs the three in one
    order and the next round in the reverse order (A B C, C B A, ...). Before
    the `warmup` untimed rounds, steps run for `prewarm_s` seconds so that the
    clocks have ramped up. Returns (graph_ms, eager_ms, split_ms, combine_ms,
    wall_s) with one entry per timed round."""
    import numpy as np
    import torch

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < prewarm_s:
        evict()
        graph.replay()
        evict()
        split()
        combine()
        torch.cuda.synchronize()
    for _ in range(warmup):
        evict()
        graph.replay()
        evict()
        split()
        combine()
    torch.cuda.synchronize()
    note("warmup done; timing")
    T = timer()
    evs = {"g": [[T.event(), T.event()] for _ in range(steps)],
           "e": [[T.event(), T.event()] for _ in range(steps)],
           "m": [[T.event(), T.event(), T.event()] for _ in range(steps)]}

    def run_graph(ev):
        T.record(ev[0], stream)
        graph.replay()
        T.record(ev[1], stream)

    def run_eager(ev):
        T.record(ev[0], stream)
        split()
        combine()
        T.record(ev[1], stream)

    def run_mid(ev):
        T.record(ev[0], stream)
        split()
        T.record(ev[1], stream)
        combine()
        T.record(ev[2], stream)

    order = [("g", run_graph), ("e", run_eager), ("m", run_mid)]
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    for k in range(steps):
        for key, fn in (order if k % 2 == 0 else order[::-1]):
            evict()
            fn(evs[key][k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    graph_ms = np.array([T.elapsed_ms(a, b) for a, b in evs["g"]])
    eager_ms = np.array([T.elapsed_ms(a, b) for a, b in evs["e"]])
    split_ms = np.array([T.elapsed_ms(e[0], e[1]) for e in evs["m"]])
    comb_ms = np.array([T.elapsed_ms(e[1], e[2]) for e in evs["m"]])
    T.destroy([x for v in evs.values() for e in v for x in e])
    return graph_ms, eager_ms, split_ms, comb_ms, wall


def variant(cfg: int, dev, evict, steps: int, warmup: int, kv_format: str = "e4m3",
            pv_mode: str = "high_residual", w=None) -> dict:
    """The workload in another mode of the path (E5M2 bytes, or the opt-in
    single FP16 probability operand): step and split-kernel times, measured
    eagerly like the main line's per-kernel pass."""
    import torch

    import paged_fp8_split_amd as pfs
    from paged_fp8_split_amd import _lib
    from paged_fp8_split_amd import workloads as W

    if w is None:
        note(f"generating the {kv_format} workload")
        w = W.config(cfg, kv_format=kv_format)
    t = W.device_tensors(w, dev)
    plan = pfs.make_plan(batch=w.batch, q=w.q, num_q_heads=w.num_q_heads, head_map=t["head_map"], k_pool=t["k_pool"],
                         max_pages_per_row=w.max_pages_per_row, sm_scale=t["sm_scale"], kv_format=kv_format,
                         pv_mode=pv_mode)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty_like(t["q"])
    stream = torch.cuda.current_stream(dev)
    split = lambda: _lib.verify_split(plan, t["q"], t["k_pool"], t["v_pool"], t["k_scale"], t["block_table"],
                                      t["live_len"], ws, stream)
    combine = lambda: _lib.verify_combine(plan, t["v_scale"], t["live_len"], out, ws, stream)
    _, _, step_ms, _ = time_steps(split, combine, evict, stream, steps, warmup, mid_event=False)
    split_ms, comb_ms, _, _ = time_steps(split, combine, evict, stream, steps, 0, mid_event=True)
    sb = split_algorithmic_bytes(w, plan)
    ach = sb / (float(split_ms.mean()) * 1e-3) / 1e9
    res = {
        "workload": w.name + ("-e5m2" if kv_format == "e5m2" else "") + ("-pv-fp16" if pv_mode == "fp16" else ""),
        "us_per_step": round(float(step_ms.mean()) * 1e3, 2),
        "kv_GBps": round(w.kv_bytes() / (float(step_ms.mean()) * 1e-3) / 1e9, 2),
        "split_mean_launch_us": round(float(split_ms.mean()) * 1e3, 2),
        "split_achieved_GBps": round(ach, 2),
        "split_frac": round(ach / PEAK_HBM_GBS, 4),
        "mfma": mfma_report(w, float(split_ms.mean()), None),
        "combine_us": round(float(comb_ms.mean()) * 1e3, 2),
    }
    del t, ws, out
    torch.cuda.empty_cache()
    return res


def ceiling(args, dev) -> dict:
    """Read-bandwidth probes (libpfs_probe.so) on the timed workload's pools:
    the live K and V bytes of the step, read in the split kernel's units
    (one 512-thread workgroup per (split, KV head), pages resolved through
    the block table) with no arithmetic, once with register loads and once
    straight into LDS through the split kernel's pipeline of stages; then the
    same number of bytes read from one flat buffer; the split kernel alone
    for comparison. Each launch after the read-only scrub, HIP events
    (HipTimer) around it; bytes = the live K and V bytes. Then the combine
    against a flat read of the same partial bytes, each straight after a
    split (its floor for one burst of reads of that size)."""
    import ctypes

    import numpy as np
    import torch

    import paged_fp8_split_amd as pfs
    from paged_fp8_split_amd import _lib
    from paged_fp8_split_amd import workloads as W

    lib = ctypes.CDLL(os.path.join(ROOT, "paged_fp8_split_amd", "libpfs_probe.so"))
    lib.pfs_probe_paged.restype = ctypes.c_int32
    lib.pfs_probe_paged.argtypes = [ctypes.c_int32] + [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 3 + \
        [ctypes.c_int32] * 6 + [ctypes.c_void_p] * 2
    lib.pfs_probe_flat.restype = ctypes.c_int32
    lib.pfs_probe_flat.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    w = W.config(args.config, q=args.q)
    if w.batch != 1:
        raise SystemExit("--ceiling probes one request (configs 1, 2 and 3)")
    t = W.device_tensors(w, dev)
    plan = pfs.make_plan(batch=1, q=w.q, num_q_heads=w.num_q_heads, head_map=t["head_map"], k_pool=t["k_pool"],
                         max_pages_per_row=w.max_pages_per_row, sm_scale=t["sm_scale"])
    L = int(w.live_len[0])
    kv = w.kv_bytes()
    grid = plan.num_splits * w.num_kv_heads
    sink = torch.empty(grid * 512, dtype=torch.int32, device=dev)
    flat = torch.ones(kv // 4, dtype=torch.int32, device=dev)
    scrub = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    scrub_sink = torch.empty((), dtype=torch.float32, device=dev)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    T = timer()

    def paged(mode):
        rc = lib.pfs_probe_paged(mode, t["k_pool"].data_ptr(), t["v_pool"].data_ptr(), t["block_table"].data_ptr(),
                                 w.page_stride, w.token_stride, w.head_stride, w.page_size, w.head_dim,
                                 w.num_kv_heads, plan.tokens_per_split, plan.num_splits, L, sink.data_ptr(), sp)
        assert rc == 0, rc

    def flat_read():
        assert lib.pfs_probe_flat(flat.data_ptr(), kv, grid, sink.data_ptr(), sp) == 0

    def split():
        _lib.verify_split(plan, t["q"], t["k_pool"], t["v_pool"], t["k_scale"], t["block_table"], t["live_len"], ws,
                          stream)

    cases = {"paged_register_loads": lambda: paged(0), "paged_direct_to_lds": lambda: paged(1),
             "flat_register_loads": flat_read, "split_kernel": split}
    times = {k: [] for k in cases}
    for fn in cases.values():  # warm up every path
        for _ in range(3):
            fn()
    torch.cuda.synchronize()
    for r in range(args.steps):  # interleaved, every launch after a scrub
        for name, fn in cases.items():
            torch.sum(scrub, 0, out=scrub_sink)
            e0, e1 = T.event(), T.event()
            T.record(e0, stream)
            fn()
            T.record(e1, stream)
            times[name].append(T.elapsed_ms(e0, e1))
            T.destroy([e0, e1])
    note(f"ceiling: {args.steps} interleaved rounds")
    res = {"workload": w.name, "kv_bytes": kv, "workgroups": grid, "tokens_per_split": plan.tokens_per_split}
    for name, ms in times.items():
        ms = np.array(ms)
        res[name] = {"us_mean": round(float(ms.mean()) * 1e3, 2), "us_p10": round(float(np.percentile(ms, 10)) * 1e3, 2),
                     "kv_TBps": round(kv / (float(ms.mean()) * 1e-3) / 1e12, 3),
                     "frac_of_8TBps": round(kv / (float(ms.mean()) * 1e-3) / 1e12 / 8.0, 4)}

    # the combine's floor: the workspace's partial bytes read flat (register
    # loads, 512 workgroups) straight after a split, as the combine reads them,
    # against the combine itself; each after an untimed scrub and split
    out = torch.empty_like(t["q"])
    part_bytes = (plan.workspace_bytes // 16) * 16
    part_grid = 512
    psink = torch.empty(part_grid * 512, dtype=torch.int32, device=dev)

    def combine():
        _lib.verify_combine(plan, t["v_scale"], t["live_len"], out, ws, stream)

    def partials_read():
        assert lib.pfs_probe_flat(ws.data_ptr(), part_bytes, part_grid, psink.data_ptr(), sp) == 0

    ccases = {"combine": combine, "partials_flat_read": partials_read}
    ctimes = {k: [] for k in ccases}
    for r in range(args.steps):
        for name, fn in ccases.items():
            torch.sum(scrub, 0, out=scrub_sink)
            split()
            e0, e1 = T.event(), T.event()
            T.record(e0, stream)
            fn()
            T.record(e1, stream)
            ctimes[name].append(T.elapsed_ms(e0, e1))
            T.destroy([e0, e1])
    res["combine_floor"] = {"partial_bytes": part_bytes, "flat_read_workgroups": part_grid}
    for name, ms in ctimes.items():
        ms = np.array(ms)
        res["combine_floor"][name] = {"us_mean": round(float(ms.mean()) * 1e3, 2),
                                      "us_p10": round(float(np.percentile(ms, 10)) * 1e3, 2),
                                      "TBps": round(part_bytes / (float(ms.mean()) * 1e-3) / 1e12, 3)}
    return res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_baseline(w, cfg_of_w: int, seconds: float, single_thread_configs=(1, 3)):
    """The FP64 oracle, as it stands, on the host cores: whole verify steps of
    the same workload with one OpenMP thread per core this process may run on,
    repeated until `seconds` have elapsed (at least one step); then one
    single-thread step of each named workload in `single_thread_configs`.
    Returns (report, oracle result of the timed workload)."""
    import oracle
    from paged_fp8_split_amd import workloads as W

    threads = len(os.sched_getaffinity(0))
    units = w.batch * w.num_q_heads * w.q
    t0 = time.perf_counter()
    reps = 0
    while True:
        ref = oracle.verify(w, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        note(f"cpu oracle step {reps}: {el:.1f} s elapsed")
        if el >= seconds:
            break
    per_step = el / reps
    single = {}
    for cfg in single_thread_configs:
        wc = w if cfg == cfg_of_w else W.config(cfg)
        t1 = time.perf_counter()
        oracle.verify(wc, threads=1)
        dt = time.perf_counter() - t1
        note(f"cpu oracle, one thread, {wc.name}: {dt:.2f} s")
        single[wc.name] = round(dt, 4)
    rep = {
        "value": round(w.kv_bytes() / per_step / 1e9, 4),
        "unit": "GB/s",
        "cores": int(min(threads, units)),
        "kind": "oracle",
        "sample": f"{reps} whole verify step(s) of the timed workload ({w.name}), FP64, "
                  f"{per_step:.2f} s per step",
        "seconds_per_step": round(per_step, 4),
        "threads": threads,
        "cpu_model": cpu_model(),
        "single_thread_seconds_per_step": single,
    }
    return rep, ref


def parity_report(y16, r) -> dict:
    """The timed output against the oracle: relative L2, max abs per band of
    |r|, and the pages' count of FP16 outputs that differ from the oracle
    result rounded to FP16 ("[Kernel][SM70] Add opt-in E4M3 grouped attention
    with FP32 partials", test plan and results)."""
    import numpy as np

    y = y16.astype(np.float64)
    err = np.abs(y - r)
    ar = np.abs(r)
    bands = {}
    for lo, hi in ((0.0, 8.0), (8.0, 16.0), (16.0, float("inf"))):
        m = (ar >= lo) & (ar < hi)
        bands[f"[{lo:g},{hi:g})"] = round(float(err[m].max()), 6) if m.any() else None
    return {
        "rel_l2": float(np.linalg.norm(err) / np.linalg.norm(r)),
        "max_abs_by_band": bands,
        "fp16_disagreements": int((y16.view(np.uint16) != r.astype(np.float16).view(np.uint16)).sum()),
        "elements": int(r.size),
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3, help="named workload (default 3: 256K context, q8)")
    ap.add_argument("--tokens-per-split", type=int, default=0)
    ap.add_argument("--q", type=int, default=None,
                    help="draft rows per request (the 8 x 64K batch also runs at q = 1 and q = 16)")
    ap.add_argument("--pv-mode", default="high_residual", choices=["high_residual", "fp16"],
                    help="probability operands of the timed line (default high_residual)")
    ap.add_argument("--kv-format", default="e4m3", choices=["e4m3", "e5m2"], help="KV byte format of the timed line")
    ap.add_argument("--no-scrub", action="store_true", help="do not evict the Infinity Cache between steps")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the residual-probability and E5M2 variants of the workload")
    ap.add_argument("--ceiling", action="store_true",
                    help="only run the read-bandwidth probes (libpfs_probe.so) on the workload's pools and exit")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run device-to-device copies of MIB MiB (to scale HBM byte counters) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} (WORLD_SIZE {world}) is not supported: "
              "bench.py measures the single-GPU verify step only (no collectives, no sharding).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 3}), flush=True)
        return 0

    import paged_fp8_split_amd as pfs
    from paged_fp8_split_amd import _lib
    from paged_fp8_split_amd import workloads as W

    dev = torch.device("cuda:0")
    if args.ceiling:
        print(json.dumps({"ceiling": ceiling(args, dev)}), flush=True)
        return 0
    note(f"generating workload config {args.config}")
    w = W.config(args.config, q=args.q, kv_format=args.kv_format)
    t = W.device_tensors(w, dev)
    plan = pfs.make_plan(batch=w.batch, q=w.q, num_q_heads=w.num_q_heads, head_map=t["head_map"], k_pool=t["k_pool"],
                         max_pages_per_row=w.max_pages_per_row, sm_scale=t["sm_scale"],
                         tokens_per_split=args.tokens_per_split, kv_format=args.kv_format, pv_mode=args.pv_mode)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty_like(t["q"])
    scrub = None if args.no_scrub else torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB, read only
    scrub_sink = torch.empty((), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def evict():
        if scrub is not None:
            torch.sum(scrub, 0, out=scrub_sink)
    stream = torch.cuda.current_stream(dev)

    def split():
        _lib.verify_split(plan, t["q"], t["k_pool"], t["v_pool"], t["k_scale"], t["block_table"], t["live_len"], ws,
                          stream)

    def combine():
        _lib.verify_combine(plan, t["v_scale"], t["live_len"], out, ws, stream)

    note(f"plan: {plan.num_splits} splits x {plan.tokens_per_split} tokens, workspace {plan.workspace_bytes} B, "
         f"{plan.num_cus} CUs")
    # the headline: the step captured once as a HIP graph, replayed after
    # each scrub, HIP events (hipEventDisableSystemFence) around each replay
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _lib.verify(plan, t["q"], t["k_pool"], t["v_pool"], t["k_scale"], t["v_scale"], t["block_table"],
                    t["live_len"], out, ws)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    y = out.cpu().numpy()
    out_sha = hashlib.sha256(y.tobytes()).hexdigest()
    split()
    combine()
    eager_same = hashlib.sha256(out.cpu().numpy().tobytes()).hexdigest() == out_sha
    note("graph captured; timing replays, eager steps and per-kernel steps, interleaved")
    # graph replays (the headline), the same step launched eagerly, and an
    # eager pass with an event between the kernels (the split kernel's launch
    # time is the roofline's denominator), interleaved round by round
    graph_step_ms, step_ms, split_ms, comb_ms, wall = time_interleaved(g, split, combine, evict, stream,
                                                                        args.steps, args.warmup)

    # the graph replayed back to back without scrubs (cache-warm: context only)
    T = timer()
    ga, gb = T.event(), T.event()
    reps = 50
    T.record(ga, stream)
    for _ in range(reps):
        g.replay()
    T.record(gb, stream)
    torch.cuda.synchronize()
    graph_warm_ms = T.elapsed_ms(ga, gb) / reps
    T.destroy([ga, gb])
    # context: the same scrubbed replays timed with torch's default events,
    # whose system-scope fence idles the GPU before the step starts
    dflt = []
    for _ in range(10):
        evict()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        dflt.append(e0.elapsed_time(e1))

    kv = w.kv_bytes()
    mean_ms = float(graph_step_ms.mean())
    eager_ms = float(step_ms.mean())
    value = kv / (mean_ms * 1e-3) / 1e9
    split_bytes = split_algorithmic_bytes(w, plan)
    step_bytes = step_algorithmic_bytes(w, plan)
    split_mean_ms = float(split_ms.mean())
    achieved = split_bytes / (split_mean_ms * 1e-3) / 1e9
    default_line = args.pv_mode == "high_residual" and args.kv_format == "e4m3" and args.tokens_per_split == 0
    traffic = traffic_from_profiles(args.config) if default_line else None
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mean_ms, 5),
        "us_per_step": round(mean_ms * 1e3, 2),
        "us_per_step_p10_p50_p90": [round(float(np.percentile(graph_step_ms, p)) * 1e3, 2) for p in (10, 50, 90)],
        "kv_pct_of_peak_hbm": round(100.0 * value / PEAK_HBM_GBS, 2),
        # every byte the step must move (the split kernel's, plus the combine's
        # read of the partials and its FP16 output) over the same replay time
        "step_algorithmic_bytes": step_bytes,
        "step_algorithmic_GBps": round(step_bytes / (mean_ms * 1e-3) / 1e9, 2),
        "timing": "HIP-graph replay of split + combine, HIP events (hipEventDisableSystemFence) around each replay on "
                  "its stream (the graph launch inside the interval), Infinity Cache scrubbed before each replay; "
                  "replays interleaved round by round (A B C, C B A) with the eager step and the per-kernel pass "
                  "after a 0.3 s pre-warm",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "precision": f"{args.kv_format.upper()} KV bytes; FP16 MFMA operands (probabilities as "
                     + ("FP16 high + FP16 residual" if args.pv_mode == "high_residual" else "one FP16 operand")
                     + "); FP32 accumulation and split partials; FP16 output",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "batch": w.batch,
            "context": int(w.live_len.max()),
            "q": w.q,
            "num_q_heads": w.num_q_heads,
            "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim,
            "page_size": w.page_size,
            "partition_tokens": 64,
            "tokens_per_split": plan.tokens_per_split,
            "num_splits": plan.num_splits,
            "num_cus": plan.num_cus,
            "pv_mode": args.pv_mode,
            "kv_format": args.kv_format,
            "kv_bytes": kv,
            "infinity_cache_scrub": scrub is not None,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "pfs_split_kernel",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "traffic_source": ("rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE of this kernel source, read from "
                               f"profiles/traffic_split_config{args.config}.json (not measured in this run)")
            if traffic is not None else None,
            "algorithmic_bytes_per_launch": split_bytes,
            "mean_launch_us": round(split_mean_ms * 1e3, 2),
        },
        "mfma": mfma_report(w, split_mean_ms, args.config if default_line else None),
        "us_per_step_eager": round(eager_ms * 1e3, 2),
        "kv_pct_of_peak_hbm_eager": round(100.0 * kv / (eager_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
        "eager_output_matches_graph": bool(eager_same),
        "combine_us": round(float(comb_ms.mean()) * 1e3, 2),
        "graph_replay_cache_warm_us": round(graph_warm_ms * 1e3, 2),
        "us_per_step_graph_default_events": round(float(np.mean(dflt)) * 1e3, 2),
        "timed_loop_wall_s": round(wall, 4),
        "output_sha256": out_sha,
        "kernel_source_sha": kernel_source_sha(),
    }
    note("timing the codec kernels")
    res["codec"] = codec_timing(w, t, dev, evict)
    if not args.no_variants:
        vs, vw = max(args.steps // 2, 10), max(args.warmup // 2, 3)
        res["variants"] = {
            "pv_fp16": variant(args.config, dev, evict, vs, vw, pv_mode="fp16", w=w),
            "e5m2": variant(args.config, dev, evict, vs, vw, kv_format="e5m2"),
        }
    if not args.no_cpu_baseline:
        note("timing the CPU oracle")
        res["cpu_baseline"], ref = cpu_baseline(w, args.config, args.cpu_seconds)
        res["parity_vs_oracle"] = parity_report(y, ref)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
