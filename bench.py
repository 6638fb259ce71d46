#!/usr/bin/env python3
"""Benchmark of batch-invariant split-KV decode attention on one MI355X.

Workload: absorbed-MLA decode, B=64 rows, 128 query heads over one shared
576-wide latent KV (512 + 64 rope), value width 512, scale 1/sqrt(192),
bf16 values N(0, 0.5^2), KV lengths lognormal (median 4096, sigma 1) clipped
to [64, 32768], 64-token pages with a seeded permuted block table.  Inputs
are synthetic and resident in HBM before timing starts.

One step = the whole hot path: host re-planning of the per-row splits, the
split list's hand-over (by value in the kernel arguments for this batch),
the split kernel and the fixed-order combine.  Untimed steps first run for
`--settle-ms` of wall time while the shader clock settles (reported as
`clock_settle`, apart from `warmup`); then the timed region is exactly
`--steps` steps after `--warmup` untimed ones, bracketed by device
synchronisation, with nothing else recorded on the stream (per-step timing
events would add their own gaps to the step).  The split kernel's
duration for the roofline comes from a second pass of `--steps` steps right
after it, in which the library launches the split kernel through
hipExtLaunchKernel with a start and a stop HIP event, so the events carry the
kernel's own start and end on its stream.  Prints one JSON line: the metric,
the roofline of the split kernel (against the 8 TB/s published peak and the
read peak the streaming-read probe measures), the CPU oracle baseline and
the parity of the timed configuration against the oracle on the rows the
baseline computed.
"""

import argparse
import ctypes
import gc
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X published HBM3E bandwidth
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "mla_split_b64_hbm_traffic.txt")
# The B=64 split kernel: mla_h128.hip with the tile loop gen_mla_h128.py writes.
SPLIT_KERNEL_SRC = [os.path.join(ROOT, "invariant_split_kv_amd", "csrc", f)
                    for f in ("mla_h128.hip", "gen_mla_h128.py")]
SPLIT_KERNEL_NAME = "mla_h128_kernel"


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in SPLIT_KERNEL_SRC:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per split-kernel launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    try:
        fields = dict(l.split(":", 1) for l in open(TRAFFIC_SUMMARY) if ":" in l and not l.startswith("#"))
    except OSError:
        return None
    fields = {k.strip(): v.strip() for k, v in fields.items()}
    if fields.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return int(fields["hbm_bytes_per_launch"])


def copy_calibration():
    """A plain device copy of 1 GiB, three times (reference for the byte counters)."""
    import torch
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": 1 << 30, "copies": 3}), flush=True)
METRIC = "decode-attn KV GB/s + % HBM roofline (MLA B=64); row batch-invariance pass rate"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles through the HIP runtime already loaded by torch."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        assert self.rt.hipEventCreate(ctypes.byref(ev)) == 0
        return ev.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.rt.hipEventSynchronize(b) == 0
        assert self.rt.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, ev):
        self.rt.hipEventDestroy(ev)


def clock_settle(dc, torch, lens_host, settle_ms):
    """Untimed steps until `settle_ms` of wall time has passed (checked every
    ten steps, after a device synchronisation): the shader clock of a cold
    part takes some tens of milliseconds of this load to reach its steady
    level.  Reported as its own field, apart from `warmup`."""
    stream = torch.cuda.current_stream()
    steps = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < settle_ms:
        for _ in range(10):
            dc.plan.update(lens_host)
            dc.run(stream)
        steps += 10
        torch.cuda.synchronize()
    return {"steps": steps, "ms": round((time.perf_counter() - t0) * 1e3, 1)}


def hbm_read_peak(isk, torch, nbytes=2 << 30, launches=10):
    """Achievable HBM read rate: isk_hbm_read_probe over a 2 GiB buffer (8x
    the 256 MB last-level cache), best of four grid sizes, each timed over
    `launches` launches after two untimed ones."""
    stream = torch.cuda.current_stream()
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(3)
    sink = torch.empty(16384, dtype=torch.int32, device="cuda")
    by_blocks = {}
    for blocks in (1024, 2048, 4096, 8192):
        for _ in range(2):
            isk.hbm_read_probe(buf, nbytes, sink, blocks, stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(launches):
            isk.hbm_read_probe(buf, nbytes, sink, blocks, stream)
        b.record(stream)
        torch.cuda.synchronize()
        by_blocks[blocks] = round(nbytes * launches / (a.elapsed_time(b) * 1e-3) / 1e9, 1)
    del buf, sink
    torch.cuda.empty_cache()
    best = max(by_blocks, key=by_blocks.get)
    return {"gbs": by_blocks[best], "bytes": nbytes, "blocks": best, "gbs_by_blocks": by_blocks,
            "frac_of_published_peak": round(by_blocks[best] / HBM_PEAK_GBS, 4)}


def timed_steps(dc, isk, torch, evs, steps, warmup, lens_host, instrument):
    """Warm up, then time exactly `steps` steps.  With `instrument`, the
    library's timing hook stamps HIP events with every split kernel's start and
    end and records one after every combine; their per-step durations are
    returned too (None otherwise)."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        dc.plan.update(lens_host)
        dc.run(stream)
    torch.cuda.synchronize()
    marks = [(evs.create(), evs.create(), evs.create()) for _ in range(steps)] if instrument else None
    # Python's cyclic collector paused over the timed loop: a full collection
    # of this process's objects takes tens of milliseconds of host time,
    # which would show up as idle GPU time inside the region.
    gc.collect()
    gc.disable()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(steps):
        if instrument:
            isk.plan_set_timing_events(dc.plan.handle, *marks[i])
        dc.plan.update(lens_host)
        dc.run(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gc.enable()
    total_ms = t_start.elapsed_time(t_end)
    if not instrument:
        return total_ms, wall, None, None
    isk.plan_set_timing_events(dc.plan.handle, None, None, None)
    split = [evs.elapsed_ms(a, b) for a, b, _ in marks]
    comb = [evs.elapsed_ms(b, c) for _, b, c in marks]
    for m in marks:
        for e in m:
            evs.destroy(e)
    return total_ms, wall, split, comb


def interleaved_ms(torch, calls_by_name, rounds=10, calls=10, warm=20):
    """Median milliseconds per call of each named step under the same clock
    state: after `warm` untimed calls of each, `rounds` rounds in which every
    step is timed over `calls` calls in turn (the order reversed on every
    other round, so that a drifting clock favours neither)."""
    stream = torch.cuda.current_stream()
    names = list(calls_by_name)
    for n in names:
        for _ in range(warm):
            calls_by_name[n]()
    per = {n: [] for n in names}
    for r in range(rounds):
        for n in (names if r % 2 == 0 else names[::-1]):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(calls):
                calls_by_name[n]()
            b.record(stream)
            torch.cuda.synchronize()
            per[n].append(a.elapsed_time(b) / calls)
    import numpy as np
    return {n: float(np.median(v)) for n, v in per.items()}


# Length-band split tables (isk_plan_create_banded) for two regimes.  Both
# keep a row's splits a function of its own length; they differ in which
# batches they favour.  Latency: rows up to 16384 tokens get 512-token splits
# (a lone row spreads over more compute units).  Throughput: rows above 32768
# tokens get at most 24 splits (fewer partials for very long rows).
BANDS_LATENCY = [(16384, 512), (1 << 30, 1536)]
BANDS_THROUGHPUT = [(32768, 1536), (1 << 30, 1536, 24)]


def per_row_vs_balanced_sizes(isk, synth, torch, np, sizes=(1, 2, 8, 32, 128), calls=50):
    """Per-row over balanced call time on the invariance-stress batches (probe
    row of 16384 tokens among batchmates of 1..131072 tokens, composition 0),
    one batch per size, with the per-row plan under the two band tables too.
    The four plans of a batch are timed interleaved (interleaved_ms), so they
    see the same clock state.  Values are drawn on the GPU (N(0, 0.5^2),
    bf16); only the timing is used."""
    res = {}
    stream = torch.cuda.current_stream()
    batches = [(str(B), synth.config5_composition(B, 0)[0]) for B in sizes]
    # Two lognormal batches (median 4096, sigma 1, at most 32768 tokens) on
    # either side of the B=64 headline batch.
    batches += [(f"lognormal_{B}", synth.config3_mla_lens(100, B)) for B in (16, 128)]
    for key, lens in batches:
        lens = np.asarray(lens, dtype=np.int32)
        B = len(lens)
        paging = synth.make_paging(lens, 64, np.random.default_rng([B, 77]))
        g = torch.Generator(device="cuda").manual_seed(B)
        pool = (torch.randn((paging.num_pages, 64, synth.MLA_DQK), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
        q = (torch.randn((B, 128, synth.MLA_DQK), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
        bt = torch.from_numpy(paging.block_table).cuda()
        lens_d = torch.from_numpy(lens).cuda()
        out = torch.empty((B, 128, synth.MLA_DV), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, 128), dtype=torch.float32, device="cuda")
        plans, steps = [], {}
        for name, mode, bands in (("per_row", isk.SPLIT_PER_ROW, None),
                                  ("bands_latency", isk.SPLIT_PER_ROW, BANDS_LATENCY),
                                  ("bands_throughput", isk.SPLIT_PER_ROW, BANDS_THROUGHPUT),
                                  ("balanced", isk.SPLIT_BATCH_BALANCED, None)):
            desc = isk.IskDesc(isk.KIND_MLA, 128, 1, synth.MLA_DQK, synth.MLA_DV, 64, paging.num_pages,
                               paging.max_pages_per_row, 0, mode, 0, isk.OUT_BF16, 0, 1.0 / math.sqrt(192.0))
            plan = isk.Plan(desc, lens, bands=bands)
            ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device="cuda")
            plans.append((plan, ws))
            steps[name] = (lambda plan=plan, ws=ws: isk.attn_decode(plan.handle, q, pool, bt, lens_d, None, None,
                                                                    out, lse, ws, ws.numel(), stream))
        ms = interleaved_ms(torch, steps, rounds=6, calls=max(1, calls // 6))
        for plan, _ in plans:
            plan.close()
        res[key] = {"kv_tokens": int(lens.sum()), "per_row_ms": round(ms["per_row"], 5),
                       "balanced_ms": round(ms["balanced"], 5),
                       "per_row_over_balanced": round(ms["per_row"] / ms["balanced"], 4),
                       "bands_latency_ms": round(ms["bands_latency"], 5),
                       "bands_throughput_ms": round(ms["bands_throughput"], 5)}
        del pool, q
        torch.cuda.empty_cache()
    return res


class CacheFlush:
    """Evicts the inputs from L2 and the 256 MB Infinity Cache by reading a
    1 GiB buffer (written once, read once here so that no dirty line of it
    is left).  A read leaves the caches full of clean lines; a write fill
    (`dirty=True`) leaves up to 256 MB of dirty lines that the next kernel's
    reads must first write back to HBM, which charges that kernel for the
    flush's own traffic."""

    def __init__(self, torch):
        self.torch = torch
        self.buf = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
        self.buf.sum(dtype=torch.int64)
        torch.cuda.synchronize()

    def __call__(self, dirty=False):
        if dirty:
            self.buf.fill_(1)
        else:
            self.buf.sum(dtype=self.torch.int64)


def cold_steps(dc, torch, n, dirty=False):
    """Per-call time with L2 and the 256 MB Infinity Cache flushed first (a
    1 GiB read; `dirty`: a 1 GiB write fill, see CacheFlush)."""
    flush = CacheFlush(torch)
    times = []
    stream = torch.cuda.current_stream()
    for _ in range(n):
        flush(dirty)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dc.run(stream)
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    del flush
    return times


def gather_rows(case, np):
    """Pool rows a sparse case attends, row by row in top-k slot order."""
    out = []
    for b, r in enumerate(case.rows):
        n = min(max(int(r.topk_len), 0), len(r.topk_idx))
        pos = np.asarray(r.topk_idx[:n])
        pos = pos[(pos >= 0) & (pos < int(case.lens[b]))]
        out.append(case.paging.token_slots(b, pos))
    return np.concatenate(out).astype(np.int32)


def gather_ceiling(isk, torch, np, dc, rows, launches=20):
    """isk_hbm_gather_probe over the rows a sparse batch gathers from its
    pool (the same bytes as its split kernels' tile loads, in the same 1 KiB
    pieces): warm (best of four grid sizes, `launches` launches) and cold
    (1 GiB read flush before each launch, median of 15) rates."""
    stream = torch.cuda.current_stream()
    rows_d = torch.from_numpy(rows).cuda()
    row_bytes = 2 * 576
    src_bytes = dc.pool.numel() * dc.pool.element_size()
    sink = torch.empty(16384, dtype=torch.int32, device="cuda")
    nbytes = len(rows) * row_bytes
    probe = lambda blocks: isk.hbm_gather_probe(dc.pool, src_bytes, rows_d, len(rows), row_bytes, sink, blocks,
                                                stream)
    warm = {}
    for blocks in (512, 1024, 2048, 4096):
        for _ in range(2):
            probe(blocks)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(launches):
            probe(blocks)
        b.record(stream)
        torch.cuda.synchronize()
        warm[blocks] = a.elapsed_time(b) / launches
    best = min(warm, key=warm.get)
    flush = CacheFlush(torch)
    cold = []
    for _ in range(15):
        flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        probe(best)
        b.record(stream)
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    del flush, rows_d, sink
    cold_ms = float(np.median(cold))
    return {"bytes": nbytes, "blocks": best, "warm_ms": round(warm[best], 5),
            "warm_gbs": round(nbytes / (warm[best] * 1e-3) / 1e9, 1), "cold_ms": round(cold_ms, 5),
            "cold_gbs": round(nbytes / (cold_ms * 1e-3) / 1e9, 1)}


def sparse_extras(isk, synth, torch, np, DeviceCase, kv_bytes, calls=100):
    """The config-4 sparse batch (B=64, 2048 top-k positions per row) and the
    same batch with an extra KV source (512 more positions per row from a
    second cache): warm and cold (1 GiB read flush first) call times and gathered
    KV GB/s.  The gathered bytes (151 MB, 189 MB with the extra set) fit in
    the 256 MB Infinity Cache, so the cold figure is the HBM one."""
    res = {}
    stream = torch.cuda.current_stream()
    for name, make in (("sparse_b64_k2048", synth.config4_sparse),
                       ("sparse_extra_b64_k2048_x512", synth.config4_sparse_extra)):
        case = make()
        dc = DeviceCase(case)
        kvb = kv_bytes(case)
        for _ in range(20):
            dc.run(stream)
        gc.collect()
        gc.disable()   # no cyclic collection inside the timed calls
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(calls):
            dc.run(stream)
        b.record(stream)
        torch.cuda.synchronize()
        gc.enable()
        warm = a.elapsed_time(b) / calls
        cold = float(np.median(cold_steps(dc, torch, 30)))
        info = dc.plan.info()
        res[name] = {"gathered_tokens": kvb // (synth.MLA_DQK * 2), "splits": info["num_segments"],
                     "split_kernel": info["split_kernel"],
                     "warm_ms_per_call": round(warm, 5), "warm_kv_gbs": round(kvb / (warm * 1e-3) / 1e9, 2),
                     "cold_ms_per_call": round(cold, 5), "cold_kv_gbs": round(kvb / (cold * 1e-3) / 1e9, 2)}
        if getattr(case, "extra", None) is None:
            res[name]["cold_dirty_flush_ms_per_call"] = round(float(np.median(cold_steps(dc, torch, 15, dirty=True))), 5)
            g = gather_ceiling(isk, torch, np, dc, gather_rows(case, np))
            g["cold_call_over_gather"] = round(cold / g["cold_ms"], 3)
            res[name]["gather_probe"] = g
        dc.close()
        del dc
        torch.cuda.empty_cache()
    return res


def gqa_extras(isk, synth, torch, np, DeviceCase, kv_bytes, calls=50):
    """The dense GQA Llama-8B-shaped batch (B=32, Hq=32, Hkv=8, D=128, lens
    uniform in [128, 8192], 16-token pages): warm and cold call times, KV
    GB/s and the split kernel's share of the 8 TB/s peak (kernel-bound
    events)."""
    stream = torch.cuda.current_stream()
    case = synth.config2_gqa()
    dc = DeviceCase(case)
    kvb = kv_bytes(case)
    for _ in range(20):
        dc.run(stream)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(calls):
        dc.run(stream)
    b.record(stream)
    torch.cuda.synchronize()
    warm = a.elapsed_time(b) / calls
    cold = float(np.median(cold_steps(dc, torch, 20)))
    evs = HipEvents()
    marks = [(evs.create(), evs.create()) for _ in range(calls)]
    for m in marks:
        isk.plan_set_timing_events(dc.plan.handle, m[0], m[1], None)
        dc.run(stream)
    torch.cuda.synchronize()
    isk.plan_set_timing_events(dc.plan.handle, None, None, None)
    split = float(np.mean([evs.elapsed_ms(x, y) for x, y in marks]))
    for x, y in marks:
        evs.destroy(x)
        evs.destroy(y)
    info = dc.plan.info()
    dc.close()
    q_bytes = case.batch * case.hq * case.d * 2
    return {"kv_bytes": kvb, "splits": info["num_segments"], "warm_ms_per_call": round(warm, 5),
            "warm_kv_gbs": round(kvb / (warm * 1e-3) / 1e9, 2), "cold_ms_per_call": round(cold, 5),
            "cold_kv_gbs": round(kvb / (cold * 1e-3) / 1e9, 2), "split_kernel_ms": round(split, 5),
            "split_kernel_frac_of_hbm_peak": round((kvb + q_bytes) / (split * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def rmsnorm_extras(isk, torch, calls=200):
    """Batch-invariant RMSNorm (one workgroup per row) at hidden size 7168:
    a decode batch of 64 rows and a large batch of 16384 rows; bytes moved
    are x read + y written (+ w once), against the 8 TB/s peak."""
    res = {}
    stream = torch.cuda.current_stream()
    dim = 7168
    g = torch.Generator(device="cuda").manual_seed(5)
    w = (1.0 + 0.1 * torch.randn(dim, generator=g, device="cuda")).to(torch.bfloat16)
    for rows in (64, 16384):
        x = torch.randn((rows, dim), generator=g, device="cuda").to(torch.bfloat16)
        y = torch.empty_like(x)
        for _ in range(20):
            isk.rmsnorm(x, w, y, rows, dim, 1e-6, stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(calls):
            isk.rmsnorm(x, w, y, rows, dim, 1e-6, stream)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / calls
        nbytes = 2 * rows * dim * 2 + dim * 2
        res[f"rows{rows}_dim{dim}"] = {"us_per_call": round(ms * 1e3, 2), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                                       "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del x, y
    return res


def linear_extras(isk, torch, calls=50):
    """Batch-invariant linear layer at n = k = 7168 (weights 103 MB, bf16):
    decode-sized rows (1, 8: one 16-row tile, bound by the weight read; 32:
    one 32-row tile, bound by the activation reads from L2), 256 rows (128 x
    64 LDS-staged tiles, one round on the CUs) and 4096 rows (256 x 128
    LDS-staged tiles, bound by the matrix cores' issue)."""
    res = {}
    stream = torch.cuda.current_stream()
    n = k = 7168
    g = torch.Generator(device="cuda").manual_seed(7)
    w = (0.02 * torch.randn((n, k), generator=g, device="cuda")).to(torch.bfloat16)
    for m in (1, 8, 32, 256, 4096):
        x = torch.randn((m, k), generator=g, device="cuda").to(torch.bfloat16)
        y = torch.empty((m, n), dtype=torch.float32, device="cuda")
        for _ in range(5):
            isk.linear_bf16(x, w, y, m, n, k, stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(calls):
            isk.linear_bf16(x, w, y, m, n, k, stream)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / calls
        nbytes = n * k * 2 + m * k * 2 + m * n * 4
        flops = 2.0 * m * n * k
        res[f"m{m}"] = {"us_per_call": round(ms * 1e3, 2), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                        "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
                        "frac_of_bf16_mfma_peak": round(flops / (ms * 1e-3) / 2.5e15, 4)}
        del x, y
    return res


def invariance_pass_rate(case, out_bits, lse_bits, mode, synth, DeviceCase, rows):
    """Rows re-run alone in a freshly permuted page pool with a fresh plan:
    bit equality of out (bf16) and lse (fp32) with the batched run."""
    ok = 0
    for b in rows:
        one = synth.mla_case([case.lens[b]], case.hq, case.scale, 64, structure_seed=5000 + int(b), seeds=[0])
        one.rows = [case.rows[b]]
        d1 = DeviceCase(one, split_mode=mode)
        d1.run()
        _, _, sb, sl = d1.result()
        d1.close()
        ok += int(sb[0].tobytes() == out_bits[b].tobytes() and sl[0].tobytes() == lse_bits[b].tobytes())
    return ok


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(case, seconds, gpu_out=None, gpu_lse=None):
    """The fp64 oracle on the host cores over a bounded sample of rows: most
    of `seconds` with the BLAS pool as configured, a quarter more with one
    thread.  With the GPU's output of the batch, the sampled rows also give
    the parity statistics of the timed configuration against the oracle."""
    import numpy as np
    import oracle
    from workloads import synth
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threadpool_limits = None
        threads = os.cpu_count() or 1
    q = synth.bf16_value(case.q_bits())
    lat = [synth.bf16_value(r.latent) for r in case.rows]
    refs = {}

    def run(budget, keep):
        done_tokens, rows, passes = 0, 0, 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget:   # whole passes over the batch, row by row
            for b in range(case.batch):
                ro, rl = oracle.mla_decode(q[b:b + 1], [lat[b]], case.scale)
                if keep and b not in refs:
                    refs[b] = (ro[0], rl[0])
                done_tokens += int(case.lens[b])
                rows += 1
                if time.perf_counter() - t0 >= budget:
                    break
            passes += 1
        return done_tokens, rows, passes, time.perf_counter() - t0

    tokens, rows, passes, dt = run(seconds, True)
    gbs = tokens * synth.MLA_DQK * 2 / dt / 1e9
    res = {"value": round(gbs, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{rows} rows ({tokens} KV tokens; {passes} pass(es) over the 64-row batch) of the "
                     f"same workload, fp64 numpy oracle, {dt:.1f} s wall",
           "nproc": os.cpu_count(), "cpu_model": cpu_model()}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1, user_api="blas"):
            t1, r1, _, d1 = run(seconds / 4, False)
        res["single_thread"] = {"value": round(t1 * synth.MLA_DQK * 2 / d1 / 1e9, 4), "unit": "GB/s",
                                "sample": f"{r1} rows ({t1} KV tokens), {d1:.1f} s wall, 1 BLAS thread"}
    if gpu_out is not None and refs:
        def ordered(bits):   # bf16 bit patterns -> integers in value order
            bits = bits.astype(np.int32)
            return np.where(bits & 0x8000, -(bits & 0x7fff), bits & 0x7fff)

        def to_bf16_bits(x):   # float64 -> bf16 bits, round to nearest even (via fp32)
            u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
            u = (u + 0x7fff + ((u >> 16) & 1)) >> 16
            return u.astype(np.int32) & 0xffff

        errs, over, lerr, n = [], [], [], 0
        hist = np.zeros(4, np.int64)   # ulp distance 0, 1, 2, > 2
        for b, (ro, rl) in refs.items():
            e = np.abs(gpu_out[b] - ro)
            ax = np.maximum(np.abs(ro), 2.0 ** -126)
            bar = np.maximum(2e-3, 2.0 ** (np.floor(np.log2(ax)) - 7))
            errs.append(e.max())
            over.append((e / bar).max())
            d = np.abs(ordered(to_bf16_bits(gpu_out[b])) - ordered(to_bf16_bits(ro)))
            hist += np.bincount(np.minimum(d, 3).ravel(), minlength=4)[:4]
            lerr.append(np.max(np.abs(np.where(np.isneginf(rl), 0, gpu_lse[b] - rl))))
            n += e.size
        res["parity"] = {"rows": len(refs), "elements": int(n), "max_abs": float(max(errs)),
                         "max_err_over_bar": round(float(max(over)), 4), "lse_max_abs": float(max(lerr)),
                         "bf16_ulp_distance_to_rounded_oracle": {"0": int(hist[0]), "1": int(hist[1]), "2": int(hist[2]),
                                                                 ">2": int(hist[3])},
                         "bar": "|gpu - oracle| <= max(2e-3, 1 bf16 ulp of the oracle value); lse 1e-3"}
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    # The shader clock of a cold part takes some tens of milliseconds of this
    # load to settle; that phase runs before the warm-up and is reported as
    # its own field (clock_settle), never counted in warmup.
    ap.add_argument("--settle-ms", type=float, default=60.0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the timed region (for profiler runs); no balanced/cold/invariance/CPU legs")
    ap.add_argument("--mode", choices=["per_row", "balanced"], default="per_row",
                    help="split rule of the timed region (the headline line uses per_row)")
    ap.add_argument("--only", choices=["linear", "rmsnorm", "gqa", "sparse"], default=None,
                    help="run one side measurement alone and print its JSON (for profiler runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy three times (byte-counter calibration run)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import invariant_split_kv_amd as isk
    from workloads import synth
    from workloads.device import DeviceCase, io_bytes, kv_bytes

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.only is not None:
        legs = {"linear": lambda: linear_extras(isk, torch), "rmsnorm": lambda: rmsnorm_extras(isk, torch),
                "gqa": lambda: gqa_extras(isk, synth, torch, np, DeviceCase, kv_bytes),
                "sparse": lambda: sparse_extras(isk, synth, torch, np, DeviceCase, kv_bytes)}
        log(f"side measurement {args.only} only")
        print(json.dumps({args.only: legs[args.only]()}), flush=True)
        return
    mode = isk.SPLIT_PER_ROW if args.mode == "per_row" else isk.SPLIT_BATCH_BALANCED

    log("generating the B=64 MLA batch")
    case = synth.config3_mla()
    lens_host = np.asarray(case.lens, dtype=np.int32)
    dc = DeviceCase(case, split_mode=mode)
    info = dc.plan.info()
    kvb = kv_bytes(case)
    iob = io_bytes(case)
    q_bytes = case.batch * case.hq * synth.MLA_DQK * 2
    evs = HipEvents()

    log(f"clock settle: {args.settle_ms:.0f} ms of untimed steps")
    settle = clock_settle(dc, torch, lens_host, args.settle_ms)
    log(f"timing {args.steps} steps after {args.warmup} warm-up steps (mode {args.mode})")
    total_ms, wall, _, _ = timed_steps(dc, isk, torch, evs, args.steps, args.warmup, lens_host, False)
    log(f"kernel durations: {args.steps} more steps with kernel-bound HIP events")
    inst_ms, _, split, comb = timed_steps(dc, isk, torch, evs, args.steps, 0, lens_host, True)
    ms_step = total_ms / args.steps
    # Host cost of re-planning the batch (part of every step above).
    plan_us = []
    for _ in range(200):
        t0 = time.perf_counter()
        dc.plan.update(lens_host)
        plan_us.append((time.perf_counter() - t0) * 1e6)
    split_ms = float(np.mean(split))
    comb_ms = float(np.mean(comb))
    gbs = kvb / (ms_step * 1e-3) / 1e9
    achieved = (kvb + q_bytes) / (split_ms * 1e-3) / 1e9

    res = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; no dataset)",
        "config": {
            "workload": "absorbed MLA decode B=64, Hq=128, latent 576 (512+64), Dv=512, scale 1/sqrt(192), "
                        "lens lognormal(median 4096, sigma 1) clipped [64,32768], 64-token pages, permuted table",
            "batch": case.batch, "kv_tokens": int(lens_host.sum()), "split_mode": args.mode,
            "split_tokens": info["split_tokens"], "splits": info["num_segments"],
            "partials": info["num_partials"], "workgroups": info["num_groups"],
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "kernel": SPLIT_KERNEL_NAME,
            "algorithmic_bytes_per_launch": kvb + q_bytes,
            "avg_launch_ms": round(split_ms, 5),
        },
        "kv_bytes_per_step": kvb,
        "pct_hbm_roofline": round(100.0 * (kvb + iob) / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(case.batch / (ms_step * 1e-3), 1),
        "kv_tokens_per_s": round(float(lens_host.sum()) / (ms_step * 1e-3), 1),
        "combine_ms": round(comb_ms, 5),
        "host_plan_us": round(float(np.median(plan_us)), 1),
        "mfma_tflops_split": round(float(lens_host.sum()) * case.hq * (576 + 512) * 2 / (split_ms * 1e-3) / 1e12, 1),
        "wall_s_timed_region": round(wall, 4),
        "clock_settle": settle,
        "ms_per_step_with_kernel_events": round(inst_ms / args.steps, 5),
        "numerics_id": isk.numerics_id(),
    }

    if not args.no_extras:
        log("HBM read peak: streaming-read probe over 2 GiB")
        peak = hbm_read_peak(isk, torch)
        res["hbm_read_probe"] = peak
        res["roofline"]["measured_read_peak_gbs"] = peak["gbs"]
        res["roofline"]["frac_of_measured_read_peak"] = round(achieved / peak["gbs"], 4)
        res["pct_measured_read_peak"] = round(100.0 * (kvb + iob) / (ms_step * 1e-3) / 1e9 / peak["gbs"], 2)
        torch.cuda.synchronize()
        gpu_out, gpu_lse, bits, lbits = dc.result()
        log("invariance: every row re-run alone vs batched")
        ok = invariance_pass_rate(case, bits, lbits, mode, synth, DeviceCase, range(case.batch))
        res["invariance"] = {"pass": ok, "total": case.batch, "rate": round(ok / case.batch, 4),
                             "check": "out bf16 bits + lse fp32 bits, solo (fresh pages, fresh plan) vs batched"}
        log("cold-cache calls (1 GiB read flush before each; then a 1 GiB write fill before each)")
        cold = cold_steps(dc, torch, 50)
        res["cold_ms_per_call"] = round(float(np.median(cold)), 5)
        res["cold_kv_gbs"] = round(kvb / (np.median(cold) * 1e-3) / 1e9, 2)
        cold_dirty = cold_steps(dc, torch, 30, dirty=True)
        res["cold_dirty_flush_ms_per_call"] = round(float(np.median(cold_dirty)), 5)
        if mode == isk.SPLIT_PER_ROW:
            log("batch-balanced comparison mode on the same batch, interleaved with per-row steps")
            dcb = DeviceCase(case, split_mode=isk.SPLIT_BATCH_BALANCED, pool=dc.pool)
            stream = torch.cuda.current_stream()

            def step_of(d):
                def step():
                    d.plan.update(lens_host)
                    d.run(stream)
                return step

            il = interleaved_ms(torch, {"per_row": step_of(dc), "balanced": step_of(dcb)}, rounds=10, calls=20)
            _, _, sb, _ = timed_steps(dcb, isk, torch, evs, args.steps, 0, lens_host, True)
            _, _, bb, bl = dcb.result()
            okb = invariance_pass_rate(case, bb, bl, isk.SPLIT_BATCH_BALANCED, synth, DeviceCase,
                                       range(0, case.batch, 4))
            res["balanced"] = {"per_row_ms_per_step": round(il["per_row"], 5),
                               "balanced_ms_per_step": round(il["balanced"], 5),
                               "per_row_over_balanced": round(il["per_row"] / il["balanced"], 4),
                               "timing": "interleaved: 10 rounds of 20 steps of each, order alternating",
                               "balanced_split_ms": round(float(np.mean(sb)), 5),
                               "invariance_pass": okb, "invariance_total": len(range(0, case.batch, 4))}
            dcb.close()
            log("per-row (plain and two band tables) vs balanced: stress batches B=1..128, lognormal B=16, 128")
            res["per_row_over_balanced_by_batch"] = per_row_vs_balanced_sizes(isk, synth, torch, np)
        log("dense GQA (Llama-8B-shaped batch)")
        res["gqa"] = gqa_extras(isk, synth, torch, np, DeviceCase, kv_bytes)
        log("batch-invariant linear layer")
        res["linear"] = linear_extras(isk, torch)
        log("batch-invariant RMSNorm")
        res["rmsnorm"] = rmsnorm_extras(isk, torch)
        log("sparse decode (config-4 batch) with and without an extra KV source")
        res["sparse"] = sparse_extras(isk, synth, torch, np, DeviceCase, kv_bytes)
        if not args.no_cpu_baseline:
            log(f"CPU baseline: fp64 oracle for ~{args.cpu_seconds:.0f} s")
            res["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds, gpu_out, gpu_lse)
            if "parity" in res["cpu_baseline"]:
                res["parity"] = res["cpu_baseline"].pop("parity")
    dc.close()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
