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
256 MB Infinity Cache.

Prints ONE JSON line. `value` = tick tokens per second. `roofline` refers to
the dominant kernel (for a mixed tick the fused decode + prefill kernel, an HBM
stream), timed per launch with HIP events the library records on its launch
stream; `legs` times the same tick's decode rows alone and prefill chunks alone
(attention only). `cpu_baseline` = the CPU oracle (RoPE + write + float64
attention) on the same tick.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged-attn KV read GB/s (% HBM peak) + packed-tick attn tokens/s, Qwen3-4B"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure
WORKLOADS = {"cfg2": 2, "cfg3": 3, "cfg4": 4, "cfg5": 5}
ROTATE = 3


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def algorithmic_work(t):
    """Bytes / flops the method itself must move / compute (no re-reads, no scratch).

    Decode row of a sequence with n keys: K and V rows n*Hkv*D*e each, the
    query and output rows Hq*D*e each, and 4 bytes per page-table entry used.
    Prefill chunk of L rows after P0 cached keys: 4*D*Hq*pairs flops over the
    unmasked (row, key) pairs, pairs = L*P0 + L(L+1)/2; its bytes are the K and
    V rows of its n = P0 + L keys read once per KV head, its query and output
    rows, and its page-table entries.
    """
    e = 2 if t.dtype == "bf16" else 4
    dec_bytes = 0
    dec_kv = 0
    flops = 0
    pf_bytes = 0
    for s in range(t.S):
        n, L = int(t.seq_lens[s]), int(t.query_lens[s])
        if L == 1:
            kv = 2 * n * t.Hkv * t.D * e
            dec_kv += kv
            dec_bytes += kv + 2 * t.Hq * t.D * e + 4 * math.ceil(n / t.P)
        elif L > 1:
            p0 = n - L
            pairs = L * p0 + L * (L + 1) // 2
            flops += 4 * t.D * t.Hq * pairs
            pf_bytes += 2 * n * t.Hkv * t.D * e + 2 * L * t.Hq * t.D * e + 4 * math.ceil(n / t.P)
    T = t.T
    k1_bytes = T * ((t.Hq + 2 * t.Hkv) * t.D * e + 8 + t.D * 4) + T * (t.Hq + 3 * t.Hkv) * t.D * e
    return {"decode_bytes": dec_bytes, "decode_kv_bytes": dec_kv, "prefill_flops": flops,
            "prefill_bytes": pf_bytes, "k1_bytes": k1_bytes}


def cpu_baseline(t, reps):
    """The oracle as it stands, on the same tick, timed on the host."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
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
            "seconds_per_tick": med,
            "host_cpus": len(os.sched_getaffinity(0))}


def sub_tick(t, c, mask, dev):
    """Device tensors of the tick restricted to the sequences in `mask` (rows,
    page tables and lengths selected; the pools are shared)."""
    import torch
    seqs = np.nonzero(mask)[0]
    rows = np.concatenate([np.arange(t.qsl[s], t.qsl[s + 1]) for s in seqs]).astype(np.int64)
    ql = t.query_lens[seqs].astype(np.int64)
    qsl = np.zeros(len(seqs) + 1, np.int32)
    qsl[1:] = np.cumsum(ql)
    ridx = torch.from_numpy(rows).to(dev)
    sidx = torch.from_numpy(seqs.astype(np.int64)).to(dev)
    q = c["q"].index_select(0, ridx).contiguous()
    return {"q": q, "out": torch.empty_like(q),
            "bt": c["bt"].index_select(0, sidx).contiguous(),
            "sl": c["sl"].index_select(0, sidx).contiguous(),
            "qsl": torch.from_numpy(qsl).to(dev), "S": int(len(seqs)), "T": int(qsl[-1]),
            "mql": int(ql.max()), "msl": int(t.seq_lens[seqs].max())}


def kernel_sources_digest():
    """sha256 over the library's kernel sources (csrc/*.hip, csrc/*.h, include/pa.h)."""
    import glob
    import hashlib
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "paged_kv_cache_page_amd", "csrc", "*.hip")) +
                   glob.glob(os.path.join(ROOT, "paged_kv_cache_page_amd", "csrc", "*.h")) +
                   [os.path.join(ROOT, "include", "pa.h")])
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def committed_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (profiles/<kernel>_<workload>_traffic.md, a line `traffic-json: {...}`),
    or None when there is none or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            if line.startswith("traffic-json:"):
                rec = json.loads(line.split(":", 1)[1])
                if rec.get("sources_sha256") != kernel_sources_digest():
                    return None
                return rec.get("bytes_per_launch")
    return None


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="cfg4", choices=sorted(WORKLOADS))
    ap.add_argument("--kv-split", type=int, default=0)
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true")
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

    def dev_st(a):
        if t.dtype == W.F32:
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    def dev_i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)

    copies = []
    for r in range(ROTATE):
        copies.append({
            "q": dev_st(t.q), "k": dev_st(t.k), "v": dev_st(t.v),
            "kp": dev_st(t.k_pool), "vp": dev_st(t.v_pool),
            "bt": dev_i32(t.block_tables), "sl": dev_i32(t.seq_lens), "qsl": dev_i32(t.qsl),
            "pos": dev_i32(t.positions), "slots": torch.empty(t.T, dtype=torch.int32, device=dev),
            "out": torch.empty((t.T, t.Hq, t.D), dtype=torch.bfloat16 if t.dtype == W.BF16
                               else torch.float32, device=dev),
        })
    table = pa.pa_rope_cos_sin_table(t.max_pos, t.D, t.theta, device=dev)
    dt = pa.PA_BF16 if t.dtype == W.BF16 else pa.PA_F32
    ws_bytes = pa.pa_paged_attention_workspace_size(t.S, t.T, t.Hq, t.D, t.max_query_len,
                                                    t.max_seq_len, t.P, args.kv_split, dt)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        c = copies[i % ROTATE]
        if not args.separate:
            pa.pa_tick_forward(c["q"], c["k"], c["v"], c["pos"], c["bt"], c["sl"], c["qsl"], table,
                               c["kp"], c["vp"], t.max_query_len, t.max_seq_len, scale=t.scale,
                               kv_split_tokens=args.kv_split, out=c["out"],
                               slot_mapping=c["slots"], workspace=ws, stream=stream)
            return
        pa.pa_compute_slot_mapping(c["bt"], c["qsl"], c["pos"], t.P, t.num_pages, out=c["slots"],
                                   stream=stream)
        pa.pa_rope_and_cache_write(c["q"], c["k"], c["v"], c["pos"], c["slots"], table, c["kp"],
                                   c["vp"], stream=stream)
        pa.pa_paged_attention_varlen(c["q"], c["kp"], c["vp"], c["bt"], c["sl"], c["qsl"],
                                     t.max_query_len, t.max_seq_len, scale=t.scale,
                                     kv_split_tokens=args.kv_split, out=c["out"], workspace=ws,
                                     stream=stream)

    log("warmup", args.warmup)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    log("timed", args.steps, "steps")
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps

    # second pass with per-kernel events (recorded by the library on its stream)
    log("per-kernel timing pass")
    pa.pa_profile_start(16 * args.steps + 16)
    for i in range(args.steps):
        step(i)
    recs = pa.pa_profile_stop()
    pa.pa_profile_reset()
    per = {}
    for name, ms in recs:
        per.setdefault(name, []).append(ms)
    kernels = {n: {"avg_ms": float(np.mean(v)), "launches": len(v)} for n, v in per.items()}

    work = algorithmic_work(t)
    tokens_per_s = t.T / (ms_per_step / 1e3)
    attn_names = ("tick_attention", "decode_attention", "prefill_attention_mfma")
    dominant = max((n for n in kernels if n in attn_names), key=lambda n: kernels[n]["avg_ms"],
                   default=None)
    roof = None
    extra = {}
    if dominant is not None:
        dms = kernels[dominant]["avg_ms"]
        if dominant == "prefill_attention_mfma":
            tf = work["prefill_flops"] / (dms / 1e3) / 1e12
            roof = {"bound": "mfma", "kernel": dominant, "achieved": round(tf, 1),
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                    "flops_per_launch": work["prefill_flops"]}
        else:
            # decode rows (and, in the fused tick, the prefill chunks' K/V, Q
            # and output) are one HBM stream; the chunks' flops would take
            # prefill_flops / MFMA peak, far below bytes / HBM peak here
            nbytes = work["decode_bytes"] + (work["prefill_bytes"] if dominant == "tick_attention"
                                             else 0)
            gbps = nbytes / (dms / 1e3) / 1e9
            roof = {"bound": "hbm", "kernel": dominant, "achieved": round(gbps, 1),
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                    "bytes_per_launch": nbytes}
            if dominant == "tick_attention" and work["prefill_flops"]:
                t_roof = max(nbytes / (HBM_PEAK_GBPS * 1e9),
                             work["prefill_flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12))
                roof["flops_per_launch"] = work["prefill_flops"]
                roof["time_bound_frac"] = round(t_roof / (dms / 1e3), 4)
        roof["traffic"] = committed_traffic(dominant, t.name)
    attn_ms = sum(v["avg_ms"] for n, v in kernels.items() if n not in
                  ("slot_mapping", "rope_cache_write"))
    extra["attention_only_tokens_per_s"] = round(t.T / (attn_ms / 1e3), 1) if attn_ms else None

    # the same tick's decode rows alone and prefill chunks alone, attention only
    # (their K/V are in the pools since the steps above)
    legs = {}
    ql = t.query_lens
    for leg, mask in (("decode_rows_only", ql == 1), ("prefill_chunks_only", ql > 1)):
        if not mask.any() or mask.all():
            continue
        subs = [sub_tick(t, c, mask, dev) for c in copies]
        sw = torch.empty(max(pa.pa_paged_attention_workspace_size(
            subs[0]["S"], subs[0]["T"], t.Hq, t.D, subs[0]["mql"], subs[0]["msl"], t.P,
            args.kv_split, dt), 1), dtype=torch.uint8, device=dev)

        def sub_step(i, subs=subs, sw=sw):
            c, u = copies[i % ROTATE], subs[i % ROTATE]
            pa.pa_paged_attention_varlen(u["q"], c["kp"], c["vp"], u["bt"], u["sl"], u["qsl"],
                                         u["mql"], u["msl"], scale=t.scale,
                                         kv_split_tokens=args.kv_split, out=u["out"],
                                         workspace=sw, stream=stream)

        for i in range(args.warmup):
            sub_step(i)
        torch.cuda.synchronize()
        pa.pa_profile_start(16 * args.steps + 16)
        for i in range(args.steps):
            sub_step(i)
        rec = pa.pa_profile_stop()
        pa.pa_profile_reset()
        ks = {}
        for name, ms in rec:
            ks.setdefault(name, []).append(ms)
        ks = {n: float(np.mean(v)) for n, v in ks.items()}
        main_k = max((n for n in ks if n in attn_names), key=lambda n: ks[n])
        entry = {"kernel": main_k, "avg_ms": round(ks[main_k], 5),
                 "all_kernels_ms": {n: round(v, 5) for n, v in ks.items()}}
        if leg == "decode_rows_only":
            gbps = work["decode_bytes"] / (ks[main_k] / 1e3) / 1e9
            entry.update({"bound": "hbm", "bytes_per_launch": work["decode_bytes"],
                          "achieved_gbps": round(gbps, 1),
                          "frac": round(gbps / HBM_PEAK_GBPS, 4),
                          "kv_read_gbps": round(work["decode_kv_bytes"] / (ks[main_k] / 1e3) / 1e9,
                                                1)})
        else:
            tf = work["prefill_flops"] / (ks[main_k] / 1e3) / 1e12
            entry.update({"bound": "mfma", "flops_per_launch": work["prefill_flops"],
                          "achieved_tflops": round(tf, 1),
                          "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)})
        legs[leg] = entry
    if legs:
        extra["legs"] = legs

    cpu = None
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(t, args.cpu_reps)

    line = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
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
