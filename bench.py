#!/usr/bin/env python3
"""Benchmark: one packed continuous-batching tick of paged attention on one MI355X.

A step is one whole tick of the hot path over one batch of synthetic input, one
pa_tick_forward call: slot mapping -> RoPE on the new Q/K + K/V page write ->
paged attention (decode rows with split-KV and its merge, prefill chunks on
MFMA). --separate enqueues the same step as the three separate calls.

Default workload: the Qwen3-4B-shaped packed mixed tick (48 decode rows with
contexts U[256, 4096] plus prefill chunks of 512/512/1024 tokens after 0-3
cached 256-token pages; 32 query / 8 KV heads, head_dim 128, bf16, seed 1004).
Inputs sit in HBM before timing starts; three copies of every buffer are
rotated between steps so no step finds the previous step's pages in the
256 MB Infinity Cache ("cold"); the same steps on one copy are reported as
"warm".

Prints ONE JSON line. `value` = tick tokens per second. `roofline` refers to
the dominant kernel of the step (the fused decode + prefill kernel), timed per
launch with HIP events the library records on its launch stream: its HBM
fraction counts the decode rows' algorithmic bytes (unique physical pages) over
the kernel's median duration; the prefill chunks' work is flops, scored on
their own leg. `legs` times, attention only, the same tick's decode rows alone
(HBM) and prefill chunks alone (MFMA), and the Qwen3-4B decode tick and the
prefix-shared long-context tick whole (their decode kernel's HBM fraction on
unique pages, logical bytes beside it). `practical_peak` is a plain read-only
stream over 2 GiB on the same GPU. `cpu_baseline` = the CPU oracle (RoPE +
write + float64 attention) on the same tick.
"""

import argparse
import json
import math
import os
import re
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged-attn KV read GB/s (% HBM peak) + packed-tick attn tokens/s, Qwen3-4B"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure
MFMA_BF16_FLOP_PER_CLK_CU = 4096  # 4 SIMDs x 1024 dense bf16 flops per clock (gfx950)
WORKLOADS = {"cfg2": 2, "cfg3": 3, "cfg4": 4, "cfg5": 5}
ROTATE = 3
ATTN_NAMES = ("tick_attention", "decode_attention", "prefill_attention_mfma")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------- accounting
def decode_work(t):
    """Algorithmic bytes of the tick's decode rows (query length 1).

    Per row with n keys: its K and V rows (n*Hkv*D*e each), its query and
    output rows (Hq*D*e each) and 4 bytes per page-table entry used. `unique`
    counts each physical page's rows once however many sequences read it
    (pages shared by a prefix are read by every sharer, but a kernel that
    streams them from HBM once per tick needs them once); `logical` sums every
    row's own K/V bytes.
    """
    e = 2 if t.dtype == "bf16" else 4
    row_bytes = t.Hkv * t.D * e
    rows_of_page = {}
    logical_kv = 0
    other = 0
    n_rows = 0
    for s in range(t.S):
        n, L = int(t.seq_lens[s]), int(t.query_lens[s])
        if L != 1:
            continue
        n_rows += 1
        logical_kv += 2 * n * row_bytes
        pages = math.ceil(n / t.P)
        other += 2 * t.Hq * t.D * e + 4 * pages
        for j in range(pages):
            pg = int(t.block_tables[s, j])
            rows_of_page[pg] = max(rows_of_page.get(pg, 0), min(t.P, n - j * t.P))
    unique_kv = 2 * row_bytes * sum(rows_of_page.values())
    return {"rows": n_rows, "unique_kv_bytes": unique_kv, "logical_kv_bytes": logical_kv,
            "bytes": unique_kv + other, "logical_bytes": logical_kv + other}


def prefill_work(t):
    """Flops of the tick's prefill chunks: 4*D*Hq per unmasked (row, key) pair,
    pairs = L*P0 + L(L+1)/2 for a chunk of L rows after P0 cached keys."""
    flops = 0
    for s in range(t.S):
        n, L = int(t.seq_lens[s]), int(t.query_lens[s])
        if L > 1:
            p0 = n - L
            flops += 4 * t.D * t.Hq * (L * p0 + L * (L + 1) // 2)
    return flops


def prep_bytes(t):
    """Algorithmic bytes of the launch before the attention (slot mapping, RoPE,
    page write). Every token reads its k and v rows, its position, cos/sin row
    and page-table entry, and writes its slot and its K and V rows into the
    pools. A bf16 tick leaves q and k as they are and stages each decode row's
    rotated query in `out` (read q row, write out row); the prefill rows'
    queries are rotated by the attention kernel where it reads them. A float32
    tick reads and writes q and k back in place."""
    e = 2 if t.dtype == "bf16" else 4
    kv = 2 * t.Hkv * t.D * e
    per_token = kv + 4 + 4 * t.D + 4 + 4 + kv
    if t.dtype == "bf16":
        qrow = t.Hq * t.D * e
        dec = int((t.query_lens == 1).sum())
        return t.T * per_token + dec * 2 * qrow
    return t.T * (per_token + (2 * t.Hq + t.Hkv) * t.D * e)  # q read and written, k written


def stats(v):
    a = np.asarray(v, dtype=np.float64)
    return {"median_ms": round(float(np.median(a)), 5), "min_ms": round(float(a.min()), 5),
            "p90_ms": round(float(np.percentile(a, 90)), 5), "mean_ms": round(float(a.mean()), 5),
            "launches": int(a.size)}


def kernel_stats(recs):
    per = {}
    for name, ms in recs:
        per.setdefault(name, []).append(ms)
    return {n: stats(v) for n, v in per.items()}


# --------------------------------------------------------------- the machine
def rocminfo_peaks():
    """CU count and peak engine clock of the gfx950 agent from rocminfo, and
    the bf16 dense MFMA peak they give (CUs x clock x 4096 flops/clock)."""
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except Exception as e:  # noqa: BLE001 - reported, not fatal
        return {"error": f"rocminfo: {e}"}
    for agent in out.split("Agent ")[1:]:
        if "gfx950" not in agent:
            continue
        cu = re.search(r"Compute Unit:\s+(\d+)", agent)
        mhz = re.search(r"Max Clock Freq\. \(MHz\):\s+(\d+)", agent)
        if cu and mhz:
            cus, clk = int(cu.group(1)), int(mhz.group(1))
            return {"compute_units": cus, "max_clock_mhz": clk,
                    "mfma_bf16_dense_tflops": round(cus * clk * 1e6 * MFMA_BF16_FLOP_PER_CLK_CU
                                                    / 1e12, 1)}
    return {"error": "no gfx950 agent in rocminfo"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def practical_peak(pa, torch, dev, steps):
    """A plain read-only stream over 2 GiB (16-byte loads, the whole GPU):
    median bandwidth over `steps` launches."""
    buf = torch.ones(2 << 30, dtype=torch.uint8, device=dev)
    sink = None
    for _ in range(3):
        sink = pa.pa_probe_stream_read(buf, sink)
    torch.cuda.synchronize()
    pa.pa_profile_start(steps + 4)
    for _ in range(steps):
        pa.pa_probe_stream_read(buf, sink)
    recs = pa.pa_profile_stop()
    pa.pa_profile_reset()
    ms = float(np.median([m for _, m in recs]))
    del buf, sink
    return {"read_only_gbps": round((2 << 30) / (ms / 1e3) / 1e9, 1),
            "bytes": 2 << 30, "median_ms": round(ms, 5), "kernel": "stream_read"}


# ------------------------------------------------------------------ the tick
class DeviceTick:
    """`copies` copies of a tick's buffers in HBM, and one step of it."""

    def __init__(self, t, torch, pa, dev, copies, kv_split, separate=False):
        self.t, self.torch, self.pa = t, torch, pa
        self.kv_split, self.separate = kv_split, separate

        def st(a):
            if t.dtype == "f32":
                return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(
                torch.bfloat16)

        def i32(a):
            return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)

        self.copies = []
        for _ in range(copies):
            self.copies.append({
                "q": st(t.q), "k": st(t.k), "v": st(t.v), "kp": st(t.k_pool),
                "vp": st(t.v_pool), "bt": i32(t.block_tables), "sl": i32(t.seq_lens),
                "qsl": i32(t.qsl), "pos": i32(t.positions),
                "slots": torch.empty(t.T, dtype=torch.int32, device=dev),
                "out": torch.empty((t.T, t.Hq, t.D), dtype=torch.bfloat16 if t.dtype == "bf16"
                                   else torch.float32, device=dev),
            })
        self.table = pa.pa_rope_cos_sin_table(t.max_pos, t.D, t.theta, device=dev)
        self.dt = pa.PA_BF16 if t.dtype == "bf16" else pa.PA_F32
        ws = pa.pa_paged_attention_workspace_size(t.S, t.T, t.Hq, t.D, t.max_query_len,
                                                  t.max_seq_len, t.P, kv_split, self.dt)
        self.ws = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream()

    def step(self, i):
        t, pa, c = self.t, self.pa, self.copies[i % len(self.copies)]
        if not self.separate:
            pa.pa_tick_forward(c["q"], c["k"], c["v"], c["pos"], c["bt"], c["sl"], c["qsl"],
                               self.table, c["kp"], c["vp"], t.max_query_len, t.max_seq_len,
                               scale=t.scale, kv_split_tokens=self.kv_split, out=c["out"],
                               slot_mapping=c["slots"], workspace=self.ws, stream=self.stream)
            return
        pa.pa_compute_slot_mapping(c["bt"], c["qsl"], c["pos"], t.P, t.num_pages, out=c["slots"],
                                   stream=self.stream)
        pa.pa_rope_and_cache_write(c["q"], c["k"], c["v"], c["pos"], c["slots"], self.table,
                                   c["kp"], c["vp"], stream=self.stream)
        pa.pa_paged_attention_varlen(c["q"], c["kp"], c["vp"], c["bt"], c["sl"], c["qsl"],
                                     t.max_query_len, t.max_seq_len, scale=t.scale,
                                     kv_split_tokens=self.kv_split, out=c["out"],
                                     workspace=self.ws, stream=self.stream)

    def sub(self, mask):
        """Attention-only steps over the sequences in `mask` (rows, tables and
        lengths selected; the pools of each copy shared)."""
        t, torch, pa = self.t, self.torch, self.pa
        seqs = np.nonzero(mask)[0]
        rows = np.concatenate([np.arange(t.qsl[s], t.qsl[s + 1]) for s in seqs]).astype(np.int64)
        ql = t.query_lens[seqs].astype(np.int64)
        qsl = np.zeros(len(seqs) + 1, np.int32)
        qsl[1:] = np.cumsum(ql)
        dev = self.copies[0]["q"].device
        ridx = torch.from_numpy(rows).to(dev)
        sidx = torch.from_numpy(seqs.astype(np.int64)).to(dev)
        subs = []
        for c in self.copies:
            q = c["q"].index_select(0, ridx).contiguous()
            subs.append({"q": q, "out": torch.empty_like(q),
                         "bt": c["bt"].index_select(0, sidx).contiguous(),
                         "sl": c["sl"].index_select(0, sidx).contiguous(),
                         "qsl": torch.from_numpy(qsl).to(dev)})
        S, T = int(len(seqs)), int(qsl[-1])
        mql, msl = int(ql.max()), int(t.seq_lens[seqs].max())
        ws = torch.empty(max(pa.pa_paged_attention_workspace_size(
            S, T, t.Hq, t.D, mql, msl, t.P, self.kv_split, self.dt), 1), dtype=torch.uint8,
            device=dev)

        def sub_step(i):
            c, u = self.copies[i % len(self.copies)], subs[i % len(subs)]
            pa.pa_paged_attention_varlen(u["q"], c["kp"], c["vp"], u["bt"], u["sl"], u["qsl"],
                                         mql, msl, scale=t.scale, kv_split_tokens=self.kv_split,
                                         out=u["out"], workspace=ws, stream=self.stream)
        return sub_step


def prewarm(torch, step, ms):
    """Untimed steps for about `ms` ms of wall time, before the warm-up steps:
    a GPU that has been idle raises its clocks over its first milliseconds of
    work, and a serving loop runs ticks back to back at the clocks this
    reaches. Returns the number of steps run."""
    n, t0 = 0, time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            step(n)
            n += 1
        torch.cuda.synchronize()
    return n


PREWARM_MS = 0.0  # --prewarm-ms, for every timed pass


def timed(torch, step, steps, warmup, stream, wall=None, prewarm_ms=None):
    """Pre-warm (PREWARM_MS unless given), warm-up, then `steps` steps between
    two events (synchronised on both sides): ms per step. `wall`, a list,
    receives the host seconds of the timed region."""
    prewarm(torch, step, PREWARM_MS if prewarm_ms is None else prewarm_ms)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    if wall is not None:
        wall.append(time.perf_counter() - w0)
    return ev0.elapsed_time(ev1) / steps


def profiled(pa, torch, step, steps):
    """The same steps again with the library's per-launch events."""
    torch.cuda.synchronize()
    pa.pa_profile_start(16 * steps + 16)
    for i in range(steps):
        step(i)
    recs = pa.pa_profile_stop()
    pa.pa_profile_reset()
    return kernel_stats(recs)


def hbm_entry(kernel, ks, nbytes, extra=None):
    ms = ks[kernel]["median_ms"]
    gbps = nbytes / (ms / 1e3) / 1e9
    e = {"kernel": kernel, "bound": "hbm", "bytes_per_launch": int(nbytes),
         "achieved_gbps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4), **ks[kernel]}
    if extra:
        e.update(extra)
    return e


def dominant(ks):
    return max((n for n in ks if n in ATTN_NAMES), key=lambda n: ks[n]["median_ms"], default=None)


def decode_config_leg(cfg, pa, torch, W, dev, steps, warmup, kv_split):
    """A whole decode tick of workload `cfg` (pa_tick_forward), and its decode
    kernel against the HBM roofline on unique and logical bytes."""
    t = W.make_config(cfg, poison=False)
    dt_ = DeviceTick(t, torch, pa, dev, ROTATE, kv_split)
    ms = timed(torch, dt_.step, steps, warmup, dt_.stream)
    ks = profiled(pa, torch, dt_.step, steps)
    work = decode_work(t)
    k = dominant(ks)
    kms = ks[k]["median_ms"]
    leg = hbm_entry(k, ks, work["bytes"], {
        "workload": t.name, "ms_per_step": round(ms, 5),
        "tick_tokens_per_s": round(t.T / (ms / 1e3), 1),
        "unique_kv_bytes": work["unique_kv_bytes"], "logical_kv_bytes": work["logical_kv_bytes"],
        "logical_gbps": round(work["logical_bytes"] / (kms / 1e3) / 1e9, 1),
        "all_kernels": ks})
    del dt_
    torch.cuda.empty_cache()
    return leg


def cpu_baseline(t, reps):
    """The oracle as it stands, on the same tick, timed on the host."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    table = oracle.rope_table(t.max_pos, t.D, t.theta) if t.theta is not None else None
    times = []
    # at least `reps` runs, and more (up to 30) until about 10 s of CPU work
    while len(times) < reps or (sum(times) < 10.0 and len(times) < 30):
        t0 = time.perf_counter()
        oracle.run_tick(t.dtype, t.q, t.k, t.v, t.positions, t.block_tables, t.qsl, t.seq_lens,
                        t.k_pool, t.v_pool, table, t.scale)
        times.append(time.perf_counter() - t0)
    med = float(np.median(times))
    return {"value": t.T / med, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"the full tick ({t.T} query rows, {t.S} sequences), {len(times)} runs, median "
                      f"{med:.2f} s per tick; numpy float32 RoPE + float64 attention",
            "seconds_per_tick": med, "host_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": cpu_model()}


# The sources of the kernels a tick runs (and their launch set-up): a counter
# summary taken on other sources no longer describes these kernels.
TICK_SOURCES = ("pa_api.hip", "pa_decode.hip", "pa_decode_mfma.h", "pa_device.h", "pa_internal.h",
                "pa_plan.h", "pa_plan.hip", "pa_prefill_mfma.h", "pa_rope_cache.hip", "pa_tick.hip")


def kernel_sources_digest():
    """sha256 over the sources of the tick's kernels (TICK_SOURCES in csrc/, and
    include/pa.h)."""
    import hashlib
    h = hashlib.sha256()
    files = [os.path.join(ROOT, "paged_kv_cache_page_amd", "csrc", f) for f in TICK_SOURCES]
    files.append(os.path.join(ROOT, "include", "pa.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def committed_record(path, tag):
    """The `<tag>: {...}` JSON record of a committed counter summary under
    profiles/, or None when there is none or the tick's kernel sources changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", path)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            if line.startswith(tag + ":"):
                rec = json.loads(line.split(":", 1)[1])
                return rec if rec.get("sources_sha256") == kernel_sources_digest() else None
    return None


def committed_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` (profiles/<kernel>_<workload>_traffic.md)."""
    rec = committed_record(f"{kernel}_{workload}_traffic.md", "traffic-json")
    return rec.get("bytes_per_launch") if rec else None


# ------------------------------------------------------------- other benches
def bench_sample(steps, warmup, with_cpu):
    """pa_sample_tokens over one logits row per sequence of the packed mixed tick
    (51 rows) at Qwen3's vocabulary (151936), float32 logits N(0, 4^2), with the
    request defaults temperature 0.2 and top-p 0.95 (top-k off), a fresh uniform
    per row. Algorithmic bytes per launch: each logit read once plus the
    settings and the tokens. Prints one JSON line."""
    import torch
    import paged_kv_cache_page_amd as pa
    R, V = 51, 151936
    rng = np.random.default_rng(5)
    logits_h = (rng.standard_normal((R, V)) * 4).astype(np.float32)
    dev = "cuda:0"
    logits = torch.from_numpy(logits_h).to(dev)
    T = torch.full((R,), 0.2, dtype=torch.float32, device=dev)
    k = torch.zeros(R, dtype=torch.int32, device=dev)
    p = torch.full((R,), 0.95, dtype=torch.float32, device=dev)
    u = torch.from_numpy(rng.random(R, dtype=np.float32)).to(dev)
    out = torch.empty(R, dtype=torch.int32, device=dev)
    prewarm(torch, lambda i: pa.pa_sample_tokens(logits, T, k, p, u, out=out), PREWARM_MS)
    for _ in range(warmup):
        pa.pa_sample_tokens(logits, T, k, p, u, out=out)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(steps):
        pa.pa_sample_tokens(logits, T, k, p, u, out=out)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    nbytes = R * V * 4 + R * 5 * 4
    rec = {"metric": "sampled rows/s", "value": round(R / (ms * 1e-3), 1), "unit": "rows/s",
           "ms_per_launch": round(ms, 5), "steps": steps, "warmup": warmup,
           "config": {"workload": "sampling, 51 rows x 151936 vocab, float32 logits, "
                                  "temperature 0.2, top-p 0.95", "rows": R, "vocab": V},
           "roofline": {"bound": "hbm", "kernel": "sample_screen_kernel + sample_draw_kernel",
                        "achieved": round(nbytes / (ms * 1e-3) / 1e9, 1), "peak": 8000.0,
                        "unit": "GB/s", "frac": round(nbytes / (ms * 1e-3) / 8e12, 4),
                        "bytes_per_launch": nbytes, "traffic": None}}
    if with_cpu:
        from oracle import sampling as osm
        n = 8
        t0 = time.perf_counter()
        osm.sample_rows(logits_h[:n], np.full(n, 0.2, np.float32), np.zeros(n, np.int32),
                        np.full(n, 0.95, np.float32), u[:n].cpu().numpy())
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": round(n / dt, 2), "unit": "rows/s", "cores": 1,
                               "kind": "oracle", "sample": f"{n} of the rows"}
    got = out.cpu().numpy()
    rec["tokens_in_range"] = bool(((got >= 0) & (got < V)).all())
    print(json.dumps(rec))


def bench_block_manager(steps):
    """Host block manager over a synthetic continuous-batching trace at the Qwen
    serving shape: 256-token pages, a 4096-page pool, 64 requests live, prompts
    that share one of four 2048-token prefixes plus U[64, 1024] own tokens,
    U[64, 512] new tokens each. One tick = admit as many waiting requests as fit
    (restoring cached prefixes), record one prefill (the uncached prompt) or one
    decode token per live request, finish the requests that are done (publishing
    their prompt blocks). Prints one JSON line: ticks/s and manager calls/s."""
    import paged_kv_cache_page_amd as pa
    P, N, LIVE = 256, 4096, 64
    rng = np.random.default_rng(0)
    prefixes = [rng.integers(0, 150000, 2048).astype(np.int32) for _ in range(4)]
    bm = pa.BlockManager(N, P)
    live, next_id, calls = {}, 0, 0

    def tick():
        nonlocal next_id, calls
        while len(live) < LIVE:
            prompt = np.concatenate([prefixes[next_id % 4],
                                     rng.integers(0, 150000, int(rng.integers(64, 1025)))
                                     .astype(np.int32)])
            new = int(rng.integers(64, 513))
            calls += 1
            try:
                cached = bm.admit(next_id, prompt, new)
            except pa.PaError:
                calls += 1
                bm.evict(16)
                break
            live[next_id] = [len(prompt) - cached, new]
            next_id += 1
        for req in list(live):
            rest = live[req]
            calls += 1
            if rest[0]:
                bm.append(req, rest[0])
                rest[0] = 0
            else:
                bm.append(req, 1)
                rest[1] -= 1
                if rest[1] == 0:
                    calls += 1
                    bm.finish(req)
                    del live[req]

    for _ in range(20):
        tick()
    calls = 0
    t0 = time.perf_counter()
    for _ in range(steps):
        tick()
    dt = time.perf_counter() - t0
    free, reserved, cached = bm.stats()
    print(json.dumps({"metric": "block_manager_ticks_per_s", "value": round(steps / dt, 1),
                      "unit": "ticks/s", "calls_per_s": round(calls / dt, 1),
                      "us_per_call": round(dt / calls * 1e6, 3), "steps": steps,
                      "config": {"workload": "host block manager, 64 live requests, P=256, "
                                             "4096 pages, 4 shared 2048-token prefixes",
                                 "free": free, "reserved": reserved, "cached_blocks": cached},
                      "note": "includes the ctypes binding's per-call cost"}))


# ---------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--prewarm-ms", type=float, default=300.0,
                    help="untimed steps run for this many ms before the warm-up steps, so that "
                         "the timed steps see the clocks of a GPU in steady use (0 = none)")
    ap.add_argument("--workload", default="cfg4", choices=sorted(WORKLOADS))
    ap.add_argument("--kv-split", type=int, default=0)
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-legs", action="store_true",
                    help="time the step only (no decode/prefill legs, no other workloads)")
    ap.add_argument("--only", choices=["step", "decode-rows", "prefill-chunks"], default=None,
                    help="run just this part of the default workload (for profiler runs): the "
                         "whole step, or its decode rows or prefill chunks alone")
    ap.add_argument("--separate", action="store_true",
                    help="enqueue the step as three calls (slot mapping, RoPE + write, attention) "
                         "instead of pa_tick_forward")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (reference for HBM traffic counters)")
    ap.add_argument("--block-manager", action="store_true",
                    help="only time the host block manager over a synthetic serving trace "
                         "(no GPU)")
    ap.add_argument("--sample", action="store_true",
                    help="only time pa_sample_tokens over one tick's logits rows")
    args = ap.parse_args()
    global PREWARM_MS
    PREWARM_MS = args.prewarm_ms
    if args.sample:
        bench_sample(args.steps, args.warmup, not args.no_cpu)
        return
    if args.block_manager:
        bench_block_manager(args.steps)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_page_amd as pa
    from paged_kv_cache_page_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        # a plain copy of known size: the traffic counters' reading for it gives the
        # scale factor from counter units to bytes
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "reads": n, "writes": n}))
        return
    pa.lib()
    dev = "cuda:0"
    cfg = WORKLOADS[args.workload]
    log("generating", W.CONFIG_NAMES[cfg])
    t = W.make_config(cfg, poison=False)
    tick = DeviceTick(t, torch, pa, dev, ROTATE, args.kv_split, args.separate)

    if args.only in ("decode-rows", "prefill-chunks"):
        mask = t.query_lens == 1 if args.only == "decode-rows" else t.query_lens > 1
        sub = tick.sub(mask)
        ms = timed(torch, sub, args.steps, args.warmup, tick.stream)
        print(json.dumps({"only": args.only, "workload": t.name, "ms_per_call": round(ms, 5),
                          "steps": args.steps}), flush=True)
        return

    log("warmup", args.warmup, "+ timed", args.steps, "steps (cold: 3 rotated copies)")
    prewarm_steps = prewarm(torch, tick.step, args.prewarm_ms)
    walls = []
    ms_per_step = timed(torch, tick.step, args.steps, args.warmup, tick.stream, walls,
                        prewarm_ms=0.0)
    wall = walls[0]
    if args.only == "step":
        print(json.dumps({"only": "step", "workload": t.name, "ms_per_step": round(ms_per_step, 5),
                          "steps": args.steps}), flush=True)
        return
    log("per-kernel timing pass")
    kernels = profiled(pa, torch, tick.step, args.steps)
    log("warm pass (one copy)")
    warm_ms = timed(torch, lambda i: tick.step(0), args.steps, args.warmup, tick.stream)

    dec = decode_work(t)
    flops = prefill_work(t)
    tokens_per_s = t.T / (ms_per_step / 1e3)
    dom = dominant(kernels)
    roof = None
    if dom is not None:
        dms = kernels[dom]["median_ms"]
        if dec["rows"]:
            gbps = dec["bytes"] / (dms / 1e3) / 1e9
            roof = {"bound": "hbm", "kernel": dom, "achieved": round(gbps, 1),
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                    "bytes_per_launch": dec["bytes"], "duration_ms": dms,
                    "note": "decode rows' algorithmic bytes (unique pages) over the fused "
                            "kernel's median duration; its prefill flops are scored on the "
                            "prefill leg"}
            if flops:
                t_hbm = dec["bytes"] / (HBM_PEAK_GBPS * 1e9)
                t_mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
                roof["flops_per_launch"] = flops
                # the kernel's floor if its HBM stream and its MFMA work never
                # overlapped (sum) or overlapped perfectly (max), over its duration
                roof["sum_bound_frac"] = round((t_hbm + t_mfma) / (dms / 1e3), 4)
                roof["max_bound_frac"] = round(max(t_hbm, t_mfma) / (dms / 1e3), 4)
        else:
            tf = flops / (dms / 1e3) / 1e12
            roof = {"bound": "mfma", "kernel": dom, "achieved": round(tf, 1),
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "flops_per_launch": flops,
                    "duration_ms": dms}
        roof["traffic"] = committed_traffic(dom, t.name)
    attn_ms = sum(v["median_ms"] for n, v in kernels.items() if n not in
                  ("slot_mapping", "rope_cache_write"))
    extra = {"attention_only_tokens_per_s": round(t.T / (attn_ms / 1e3), 1) if attn_ms else None,
             "warm_ms_per_step": round(warm_ms, 5),
             "warm_tokens_per_s": round(t.T / (warm_ms / 1e3), 1),
             "prep_bytes_per_step": prep_bytes(t)}

    legs = {}
    if not args.no_legs:
        ql = t.query_lens
        for leg, mask in (("decode_rows_only", ql == 1), ("prefill_chunks_only", ql > 1)):
            if not mask.any() or mask.all():
                continue
            log("leg", leg)
            sub = tick.sub(mask)
            timed(torch, sub, args.steps, args.warmup, tick.stream)
            ks = profiled(pa, torch, sub, args.steps)
            k = dominant(ks)
            if leg == "decode_rows_only":
                legs[leg] = hbm_entry(k, ks, dec["bytes"], {
                    "all_kernels": ks,
                    "traffic": committed_traffic("decode_attention", t.name + "-decode-rows")})
            else:
                tf = flops / (ks[k]["median_ms"] / 1e3) / 1e12
                legs[leg] = {"kernel": k, "bound": "mfma", "flops_per_launch": flops,
                             "achieved_tflops": round(tf, 1),
                             "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), **ks[k],
                             "all_kernels": ks,
                             # MFMA busy cycles / (active cycles x SIMDs) and the bf16 MFMA
                             # flops the counters saw, from the committed summary
                             "counters": committed_record(
                                 f"prefill_chunks_{t.name}_mfma-counters.md", "counters-json")}
        if cfg == 4:
            for name, c in (("cfg3_decode", 3), ("cfg5_decode", 5)):
                log("leg", name)
                legs[name] = decode_config_leg(c, pa, torch, W, dev, args.steps, args.warmup,
                                               args.kv_split)
        if legs:
            extra["legs"] = legs
        log("practical peak (read-only stream)")
        extra["practical_peak"] = practical_peak(pa, torch, dev, max(10, args.steps // 2))
        pp = extra["practical_peak"]["read_only_gbps"]
        for v in list(legs.values()) + ([roof] if roof and roof["bound"] == "hbm" else []):
            g = v.get("achieved_gbps", v.get("achieved")) if v else None
            if g and v.get("bound") == "hbm":
                v["frac_of_practical_peak"] = round(g / pp, 4)
    extra["peaks"] = {"hbm_gbps": HBM_PEAK_GBPS, "mfma_bf16_tflops": MFMA_BF16_PEAK_TFLOPS,
                      "source": "MI355X vendor figures", "rocminfo": rocminfo_peaks()}

    cpu = None
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(t, args.cpu_reps)

    line = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "prewarm": {"ms": args.prewarm_ms, "steps": prewarm_steps,
                    "note": "untimed steps before the warm-up steps (of this pass and of every "
                            "other timed pass), so that the timed steps run at the clocks of a "
                            "GPU in steady use"},
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": t.dtype,
        "data": "synthetic",
        "config": {"workload": t.name, "seqs": t.S, "query_tokens": t.T,
                   "decode_rows": int((t.query_lens == 1).sum()),
                   "chunks": [int(x) for x in t.query_lens[t.query_lens > 1]],
                   "heads_q_kv": [t.Hq, t.Hkv], "head_dim": t.D, "page_size": t.P,
                   "pool_pages": t.num_pages, "seed": t.seed, "parallelism": "none (1 GPU)",
                   "entry": "three calls" if args.separate else "pa_tick_forward"},
        "roofline": roof, "cpu_baseline": cpu, "kernels": kernels,
        "kernel_sources_sha256": kernel_sources_digest(),
        "wall_s_timed_region": round(wall, 4), **extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
