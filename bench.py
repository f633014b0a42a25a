#!/usr/bin/env python3
"""Decode-step benchmark of the quantized-KV hot path on one MI355X.

Workload (default): batch 1, 24 query heads, 4 KV heads, head_dim 256, an int8
cache with per-row absmax scales holding 65,536 tokens, one query token.  One
step = quantize-on-append of the new token's K/V row + split-KV decode +
fixed-order combine, i.e. the whole hot path, issued as kvq_append_decode_attend
(the append runs inside the split kernel) unless --separate-append is given.
Steps rotate over 16 layer caches (16 x 130 MiB) so the 256 MB Infinity Cache
cannot serve the KV bytes.  Inputs are seeded synthetic tensors already resident
in HBM when the timed region starts.

Timing: half a second of step replays settles the clocks whatever --warmup is,
then --warmup untimed steps, then 5 back-to-back windows of exactly --steps
steps (one HIP-graph replay each, step i on layer i % 16), each between two HIP
events on its stream; ms_per_step is the median window.  The split kernel alone
is timed the same way over 64 replays of a graph of 16 split launches per
window.

Prints ONE JSON line.  `value` is the effective KV-read bandwidth of the whole
step: algorithmic bytes (K and V codes plus per-row scales of every cached
token) / wall time per step.  `roofline` rates the dominant kernel (the split
decode) by its own duration, measured with HIP events on its stream.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode µs/step + KV-read HBM GB/s, Hq24/Hkv4/D256 int8 at 64K ctx"
PEAK_HBM_GBPS = 8000.0
PEAK_F16_FLOPS = 2.5e15  # MI355X dense fp16 / bf16 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "split_decode_int8_64k_traffic.json")
KERNEL_SOURCES = ["quantized_kv_cache_02_amd/csrc/kvq_split.hip",
                  "quantized_kv_cache_02_amd/csrc/kvq_device.h",
                  "quantized_kv_cache_02_amd/csrc/kvq_params.h",
                  "quantized_kv_cache_02_amd/csrc/kvq_quant.h",
                  "quantized_kv_cache_02_amd/csrc/kvq_sched.h"]


def _code_only(text: str) -> str:
    """The source without its comments and blank space, so that a comment edit
    does not invalidate a counter summary taken on the same code."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_digest() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(bytes_per_launch_alg: float):
    """HBM bytes per split-kernel launch from the committed rocprofv3 counter
    summary, or None when it is missing, was taken on other kernel sources or
    on another workload (other algorithmic bytes)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_digest") != kernel_digest():
        return None
    if t.get("algorithmic_bytes_per_launch") != int(bytes_per_launch_alg):
        return None
    return t.get("hbm_bytes_per_launch")


def algorithmic_bytes(w) -> int:
    """K and V codes plus per-row scales of every cached token the step's queries
    can see (all of them, or those inside a sliding window).  An unquantized
    bf16 cache reads 2 D bytes per row and no scale."""
    row = w.D // 2 if w.dtype == 2 else 2 * w.D if w.dtype == 4 else w.D
    # per-row scales, K side and V side (v_mode 0: the same mode as K)
    per_row_scale = 4 * (w.mode == 1) + 4 * ((w.v_mode or w.mode) == 1)
    tokens = 0
    for L in w.lens:
        L = int(L)
        lo = max(0, L - w.Tq - w.window + 1) if w.window > 0 else 0
        tokens += L - lo
    return int(tokens * w.Hkv * (2 * row + per_row_scale))


def build_layers(kvq, torch, w, layers: int, dev):
    """`layers` caches of the workload, each quantized by kvq_append from the same
    rows, and the step's new rows (the last Tq of each sequence), [B, Tq, Hkv, D]."""
    k = w.k.to(dev)
    v = w.v.to(dev)
    table = None if w.block_table is None else torch.from_numpy(w.block_table).to(dev)
    caches = []
    for _ in range(layers):
        c = kvq.KVCache(w.dtype, w.mode, w.Hkv, w.D, w.block_size, w.num_blocks, w.k_static,
                        w.v_static, device=dev, v_scale_mode=w.v_mode)
        if table is None:
            kvq.append(c, k, v, torch.zeros(w.B, dtype=torch.int32, device=dev))
        else:
            for b in range(w.B):
                L = int(w.lens[b])
                if L > 0:
                    kvq.append(c, k[b:b + 1, :L].contiguous(), v[b:b + 1, :L].contiguous(),
                               torch.zeros(1, dtype=torch.int32, device=dev), table[b:b + 1].contiguous())
        caches.append(c)
    kn = torch.zeros(w.B, w.Tq, w.Hkv, w.D, dtype=torch.bfloat16, device=dev)
    vn = torch.zeros_like(kn)
    for b in range(w.B):
        L = int(w.lens[b])
        for j in range(w.Tq):
            p = L - w.Tq + j
            if p >= 0:
                kn[b, j] = k[b, p]
                vn[b, j] = v[b, p]
    torch.cuda.synchronize()
    return caches, table, kn, vn


SETTLE_S = 0.5   # step-graph replays before any timing, whatever --warmup is (--settle-s)
WINDOWS = 5      # timed windows; the median is reported
SPLIT_REPLAYS = 64  # replays of the 16-launch split-only graph per window


def _median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def time_workload(kvq, torch, w, layers: int, steps: int, warmup: int, dev, fused: bool = True,
                  settle_s: float = SETTLE_S, split_replays: int = SPLIT_REPLAYS):
    """Time decode steps of workload `w` rotated over `layers` caches.

    Clocks are settled first by SETTLE_S seconds of replays of a graph of one
    step per layer.  Then `warmup` untimed steps and WINDOWS timed windows of
    exactly `steps` steps each (a graph of `steps` steps, step i on layer
    i % layers), issued back to back after a synchronize and timed with HIP
    events on their stream; the median window gives ms per step.  The split
    kernel alone is timed the same way over SPLIT_REPLAYS replays of a graph of
    one split launch per layer per window."""
    caches, table, kn, vn = build_layers(kvq, torch, w, layers, dev)
    q = w.q.to(dev)
    lens = torch.from_numpy(w.lens).to(dev)
    pos = (lens - w.Tq).clamp(min=0).contiguous()
    sink = None if w.sink is None else torch.from_numpy(w.sink).to(dev)
    B, Tq, Hq, D = q.shape
    msl = max(int(w.lens.max()), 1)
    ws = torch.empty(kvq.workspace_bytes(caches[0], B, Hq, Tq, msl), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    S = kvq.num_splits(caches[0], B, Hq, Tq, msl)

    options = w.softcap > 0 or w.window > 0

    def step(c, s):
        if options:
            kvq.attend_ex(c, q, lens, msl, w.sm_scale, block_table=table, head_sink=sink,
                          k_new=kn if fused else None, v_new=vn if fused else None,
                          softcap=w.softcap, window=w.window, out=out, workspace=ws, stream=s)
        elif fused:
            kvq.append_decode_attend(c, kn, vn, q, lens, msl, w.sm_scale, block_table=table,
                                     head_sink=sink, out=out, workspace=ws, stream=s)
        else:
            kvq.append(c, kn, vn, pos, block_table=table, stream=s)
            kvq.split_decode(c, q, lens, msl, w.sm_scale, ws, block_table=table, stream=s)
            kvq.combine(c, B, Hq, Tq, lens, msl, ws, out, head_sink=sink, stream=s)

    def split_only(c, s):
        if options:  # the options entry point has no split-only form: time the step
            step(c, s)
        else:
            kvq.split_decode(c, q, lens, msl, w.sm_scale, ws, block_table=table, stream=s)

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graphs = {}
    with torch.cuda.stream(stream):
        for c in caches:  # warm the kernels once outside capture
            step(c, stream)
        plans = (("layers", step, layers), ("window", step, steps), ("split", split_only, layers))
        for name, fn, n in plans:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(n):
                    fn(caches[i % layers], stream)
            graphs[name] = g
    torch.cuda.synchronize()

    def windows(graph, reps: int):
        """WINDOWS back-to-back windows of `reps` replays, each between two events."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(WINDOWS + 1)]
        torch.cuda.synchronize()
        ev[0].record(stream)
        for k in range(WINDOWS):
            for _ in range(reps):
                graph.replay()
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        return [ev[k].elapsed_time(ev[k + 1]) for k in range(WINDOWS)]

    with torch.cuda.stream(stream):
        t_settle = time.perf_counter()
        n_settle = 0
        while time.perf_counter() - t_settle < settle_s:
            for _ in range(8):
                graphs["layers"].replay()
            n_settle += 8 * layers
            torch.cuda.synchronize()
        wsteps = 0
        while wsteps < warmup:
            graphs["layers"].replay()
            wsteps += layers
        t0 = time.perf_counter()
        step_windows = windows(graphs["window"], 1)
        wall_s = time.perf_counter() - t0
        step_ms = _median(step_windows) / steps
        split_windows = windows(graphs["split"], split_replays)
        split_ms = _median(split_windows) / (split_replays * layers)
    del graphs, caches
    return dict(workload=w.name, steps=steps, warmup=wsteps, settle_steps=n_settle, step_ms=step_ms,
                split_ms=split_ms, wall_s=wall_s, bytes=algorithmic_bytes(w), splits=S,
                step_window_ms=[round(x / steps, 6) for x in step_windows],
                split_window_ms=[round(x / (split_replays * layers), 6) for x in split_windows])


STREAM_GRIDS = (256, 512, 1024, 2048)


def time_stream_floor(kvq, torch, nbytes: int, layers: int, dev, reps: int = 8):
    from quantized_kv_cache_02_amd import probe as kprobe

    """The HBM floor for reading `nbytes` once: kvq_stream_read (the decode's
    non-temporal 16-byte loads, nothing else) over `layers` rotated buffers of
    that size, back to back on one stream, timed with HIP events on it; the
    fastest of a few workgroup counts."""
    nbytes = nbytes // 16 * 16
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device=dev) for _ in range(layers)]
    sink = torch.empty(max(STREAM_GRIDS) * 4096, dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    best = None
    with torch.cuda.stream(stream):
        for wg in STREAM_GRIDS:
            for b in bufs:
                kprobe.stream_read(b, wg, sink, stream=stream)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                for b in bufs:
                    kprobe.stream_read(b, wg, sink, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (reps * layers)
            if best is None or us < best[0]:
                best = (us, wg)
    del bufs, sink
    torch.cuda.empty_cache()
    return best


def time_config(kvq, torch, ki, dtype: str, ctx: int, layers: int, steps: int, warmup: int, dev,
                fused: bool = True, **kw):
    w = ki.make_workload(3, ctx=ctx, dtype=dtype)
    r = time_workload(kvq, torch, w, layers, steps, warmup, dev, fused, **kw)
    r.update(ctx=ctx, dtype=dtype, workload=w)
    return r


def time_sdpa_bf16(torch, ctx: int, layers: int, iters: int, dev, expanded: bool):
    """torch's bf16 scaled_dot_product_attention on the same decode geometry
    (B1, 24 query heads over 4 KV heads, D 256, one query token) over `layers`
    rotated unquantized caches: the comparison the kernel page draws its
    crossover against.  expanded: K/V already repeated to the 24 query heads
    (6x the bytes, torch's fused backends); else enable_gqa on the 4 KV heads.
    Returns ms per call (eager launches, HIP events)."""
    import torch.nn.functional as F

    g = torch.Generator(device="cpu").manual_seed(900 + ctx % 997)
    hk = 24 if expanded else 4
    q = torch.randn(1, 24, 1, 256, generator=g).to(torch.bfloat16).to(dev)
    ks = [torch.randn(1, hk, ctx, 256, generator=g).to(torch.bfloat16).to(dev) for _ in range(layers)]
    vs = [torch.randn(1, hk, ctx, 256, generator=g).to(torch.bfloat16).to(dev) for _ in range(layers)]
    for i in range(layers):
        F.scaled_dot_product_attention(q, ks[i], vs[i], enable_gqa=not expanded)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for it in range(iters):
        F.scaled_dot_product_attention(q, ks[it % layers], vs[it % layers], enable_gqa=not expanded)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    del ks, vs
    torch.cuda.empty_cache()
    return ms


def prefill_flops(w) -> int:
    """MFMA work of one chunked-prefill attention: 2 D multiply-adds for Q.K^T and
    2 D for P.V per (query row, visible key)."""
    pairs = 0
    for L in w.lens:
        L = int(L)
        for j in range(w.Tq):
            p = L - w.Tq + j
            lo = max(0, p - w.window + 1) if w.window > 0 else 0
            pairs += max(0, p + 1 - lo)
    return 4 * w.D * w.Hq * pairs


def time_prefill(kvq, torch, ki, dtype: str, past: int, chunk: int, layers: int, reps: int, dev):
    """Chunked prefill of `chunk` tokens after `past` cached ones (workload-3
    geometry), over `layers` rotated caches: kvq_prefill_attend (append + tiled
    attention) as HIP-graph replays, and the attention kernel alone (the chunk
    already in the cache)."""
    w = ki.make_workload(3, ctx=past + chunk, dtype=dtype)
    w.Tq = chunk
    w.q = ki.randn_bf16((1, chunk, w.Hq, w.D), 777)
    caches, table, _, _ = build_layers(kvq, torch, w, layers, dev)
    k = w.k.to(dev)
    v = w.v.to(dev)
    kn = k[:, past:past + chunk].contiguous()
    vn = v[:, past:past + chunk].contiguous()
    q = w.q.to(dev)
    lens = torch.from_numpy(w.lens).to(dev)
    msl = past + chunk
    out = torch.empty_like(q)
    # the context-split workspace of kvq_prefill_attend_ws (0 bytes: unsplit)
    need = kvq.prefill_workspace_bytes(caches[0], 1, w.Hq, chunk, msl)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    res = {}
    with torch.cuda.stream(stream):
        for name, fused in (("step", True), ("attend", False)):
            def run(c):
                kvq.prefill_attend(c, q, lens, msl, w.sm_scale, k_new=kn if fused else None,
                                   v_new=vn if fused else None, out=out, workspace=ws, stream=stream)
            for c in caches:
                run(c)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for c in caches:
                    run(c)
            g.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            res[name] = e0.elapsed_time(e1) / (reps * layers)
            del g
    del caches
    torch.cuda.empty_cache()
    fl = prefill_flops(w)
    return dict(dtype=dtype, past=past, chunk=chunk, workspace_bytes=need,
                step_ms=res["step"], attend_ms=res["attend"],
                flops=fl, attend_TFLOPs=fl / (res["attend"] * 1e-3) / 1e12,
                step_TFLOPs=fl / (res["step"] * 1e-3) / 1e12)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(ki, w, seconds: float, seconds_1t: float):
    """The oracle as it stands on the same workload: one step = dequantize the
    layer cache to fp32, then fp64 attention.  Whole steps until `seconds` of
    wall time have passed (at least one) on the OpenMP threads the process has,
    then on one thread for `seconds_1t`.  Returns both as (steps, s/step) with
    the thread count."""
    import oracle

    oracle.build(force=False)
    ocache = oracle.build_cache(w)
    qb = ki.bf16_bits(w.q)

    def run(budget):
        n = 0
        t0 = time.perf_counter()
        while True:
            K, V = ocache.dequantize(w.lens)
            oracle.attend(qb, K, V, w.lens, w.sm_scale, None, w.Hkv)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget or el / n * (n + 1) > 2.5 * budget:
                return n, el / n

    threads = oracle.num_threads()
    n, sec = run(seconds)
    oracle.set_num_threads(1)
    n1, sec1 = run(seconds_1t)
    oracle.set_num_threads(threads)
    return n, sec, threads, n1, sec1


# Wide query-row sets (G query heads x Tq draft tokens per KV head, more than
# 16 rows per 16-row block budget): dtype, K scale mode, D, B, Hkv, G, Tq,
# context per sequence, paged.
WIDE_ROW_SHAPES = [
    ("int8", "per-row", 256, 1, 4, 4, 8, 65536, False),
    ("int8", "per-row", 256, 1, 4, 6, 8, 65536, False),
    ("int8", "per-row", 256, 1, 4, 8, 8, 65536, False),
    ("int8", "per-row", 128, 4, 8, 8, 8, 16384, True),
    ("int4", "per-row", 128, 4, 8, 6, 8, 16384, True),
    ("fp8", "per-tensor", 256, 2, 4, 6, 4, 32768, True),
    ("fp8", "per-tensor", 256, 2, 4, 8, 8, 32768, True),
]


def time_wide_rows(kvq, torch, ki, args, dev, fused):
    """Split-kernel and step times of the wide row sets above and of workload 5."""
    dts = {"int8": ki.INT8, "int4": ki.INT4, "fp8": ki.FP8}
    mds = {"per-row": ki.PER_ROW, "per-tensor": ki.PER_TENSOR}
    with open(args.wide_rows, "w") as f:
        shapes = [("workload5", None)] + [(sh, None) for sh in WIDE_ROW_SHAPES]
        for sh, _ in shapes:
            if sh == "workload5":
                w = ki.make_workload(5)
                desc = "workload 5: paged int4 per-channel, B4 Hq24 Hkv4 D256, 32,768 + 8 tokens"
            else:
                dt, md, D, B, Hkv, G, Tq, ctx, paged = sh
                w = ki.random_workload(4400 + D + G * Tq, B=B, Hkv=Hkv, G=G, D=D, Tq=Tq, lens=[ctx] * B,
                                       dtype=dts[dt], mode=mds[md], block_size=16 if paged else None)
                desc = (f"{dt} {md}, B{B} Hq{G * Hkv} Hkv{Hkv} D{D}, {ctx} tokens, Tq {Tq} "
                        f"({G * Tq} rows per KV head){', paged' if paged else ''}")
            s = time_workload(kvq, torch, w, 4, max(64, args.steps // 4), args.warmup, dev, fused)
            s["what"] = desc
            s["rows_per_kv_head"] = (w.Hq // w.Hkv) * w.Tq
            s["split_GBps"] = s["bytes"] / (s["split_ms"] * 1e-3) / 1e9
            f.write(json.dumps(s) + "\n")
            f.flush()
            print(f"[wide] {desc}: split {s['split_ms'] * 1e3:.2f} us, step {s['step_ms'] * 1e3:.2f} us",
                  file=sys.stderr, flush=True)
            del w
            torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=640)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--ctx", type=int, default=65536)
    ap.add_argument("--dtype", default="int8", choices=["int8", "int4", "bf16"])
    ap.add_argument("--layers", type=int, default=16)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall seconds of oracle steps on all OpenMP threads")
    ap.add_argument("--cpu-seconds-1t", type=float, default=6.0,
                    help="wall seconds of oracle steps on one thread")
    ap.add_argument("--separate-append", action="store_true",
                    help="run the step as three launches (kvq_append, split, combine) instead of "
                         "kvq_append_decode_attend (append fused into the split kernel, then combine)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream-floor", action="store_true",
                    help="skip the streaming-read floor (e.g. under a profiler)")
    ap.add_argument("--settle-s", type=float, default=SETTLE_S,
                    help="seconds of step replays that settle the clocks before timing (0 under a "
                         "profiler, which serializes every launch)")
    ap.add_argument("--split-replays", type=int, default=SPLIT_REPLAYS,
                    help="replays of the split-only graph per timed window")
    ap.add_argument("--sweep", default="", help="also time the context sweep for int8 and int4 "
                                                "and write the lines to this JSON-lines file")
    ap.add_argument("--workload", type=int, default=3, choices=[2, 3, 4, 5],
                    help="time another of the seeded workloads instead (2, 4, 5: their own "
                         "shapes; the JSON line then reports that workload)")
    ap.add_argument("--crossover", default="",
                    help="time the int8 step against the same step over an unquantized bf16 "
                         "cache (this library's kernel) and torch bf16 SDPA, over the context "
                         "sweep, and write JSON lines to this file")
    ap.add_argument("--prefill-cases", default="",
                    help="with --prefill: comma-separated dtype:past:chunk cases "
                         "(default: int8/int4/fp8/bf16 x 0+2048, 16384+2048, 32768+1024, 4096+512)")
    ap.add_argument("--prefill", default="",
                    help="time chunked prefill (workload-3 geometry, int8 / int4 / bf16 "
                         "caches, several past lengths and chunk sizes) and write JSON lines to this "
                         "file")
    ap.add_argument("--wide-rows", default="",
                    help="time the split kernel on wide query-row sets (17-64 rows per KV head: "
                         "speculative drafts over grouped heads, several dtypes and head dims) and "
                         "write JSON lines to this file")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB, 20 times "
                         "(reference dispatch for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode path is not run across GPUs, and the "
              "figure is that GPU's throughput. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import kvq_inputs as ki
    import quantized_kv_cache_02_amd as kvq

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    kvq.lib()

    if args.crossover:
        with open(args.crossover, "w") as f:
            for ctx in ki.SWEEP_CTX:
                layers = args.layers if ctx <= 65536 else 8
                sd = time_sdpa_bf16(torch, ctx, layers, 8 * layers, dev, expanded=False)
                sde = time_sdpa_bf16(torch, ctx, max(2, layers // 4) if ctx > 65536 else layers,
                                     8 * layers, dev, expanded=True)
                r = time_config(kvq, torch, ki, "int8", ctx, layers, max(64, args.steps // 4),
                                args.warmup, dev, True)
                r.pop("workload")
                rb = time_config(kvq, torch, ki, "bf16", ctx, layers, max(64, args.steps // 4),
                                 args.warmup, dev, True)
                rb.pop("workload")
                line = {"ctx": ctx, "sdpa_bf16_gqa_us": round(sd * 1e3, 2),
                        "sdpa_bf16_expanded_us": round(sde * 1e3, 2),
                        "bf16_step_us": round(rb["step_ms"] * 1e3, 2),
                        "bf16_split_us": round(rb["split_ms"] * 1e3, 2),
                        "int8_step_us": round(r["step_ms"] * 1e3, 2),
                        "int8_split_us": round(r["split_ms"] * 1e3, 2),
                        "bf16_bytes": rb["bytes"], "int8_bytes": r["bytes"]}
                f.write(json.dumps(line) + "\n")
                f.flush()
                print(f"[crossover] {line}", file=sys.stderr, flush=True)
        return

    if args.prefill:
        cases = [(dt, past, chunk) for dt in ("int8", "int4", "fp8", "bf16")
                 for past, chunk in ((0, 2048), (16384, 2048), (32768, 1024), (4096, 512))]
        if args.prefill_cases:
            cases = []
            for item in args.prefill_cases.split(","):
                dt, past, chunk = item.split(":")
                cases.append((dt, int(past), int(chunk)))
        with open(args.prefill, "w") as f:
            for dt, past, chunk in cases:
                r = time_prefill(kvq, torch, ki, dt, past, chunk, 4, 8, dev)
                r["attend_frac_of_fp16_peak"] = r["attend_TFLOPs"] * 1e12 / PEAK_F16_FLOPS
                f.write(json.dumps(r) + "\n")
                f.flush()
                print(f"[prefill] {dt} past={past} chunk={chunk} step {r['step_ms']:.3f} ms "
                      f"attend {r['attend_ms']:.3f} ms {r['attend_TFLOPs']:.0f} TFLOP/s",
                      file=sys.stderr, flush=True)
        return

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(20):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "dispatches": 20}))
        return

    fused = not args.separate_append
    if args.wide_rows:
        time_wide_rows(kvq, torch, ki, args, dev, fused)
        return
    if args.workload != 3:
        w = ki.make_workload(args.workload)
        r = time_workload(kvq, torch, w, args.layers, args.steps, args.warmup, dev, fused,
                          settle_s=args.settle_s, split_replays=args.split_replays)
        r.pop("workload")
        print(json.dumps({"workload": w.name, "us_per_step": round(r["step_ms"] * 1e3, 2),
                          "split_kernel_us": round(r["split_ms"] * 1e3, 2),
                          "split_GBps": round(r["bytes"] / (r["split_ms"] * 1e-3) / 1e9, 1),
                          "algorithmic_bytes_per_step": r["bytes"], "splits": r["splits"]}),
              flush=True)
        return
    r = time_config(kvq, torch, ki, args.dtype, args.ctx, args.layers, args.steps, args.warmup, dev,
                    fused, settle_s=args.settle_s, split_replays=args.split_replays)
    w = r.pop("workload")
    achieved = r["bytes"] / (r["split_ms"] * 1e-3) / 1e9
    value = r["bytes"] / (r["step_ms"] * 1e-3) / 1e9
    traffic = measured_traffic(r["bytes"])
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": r["steps"],
        "warmup": r["warmup"],
        "ms_per_step": round(r["step_ms"], 5),
        "us_per_step": round(r["step_ms"] * 1e3, 2),
        "split_kernel_us": round(r["split_ms"] * 1e3, 2),
        "timing": {
            "settle_steps": r["settle_steps"],
            "windows": WINDOWS,
            "step_us_per_window": [round(x * 1e3, 2) for x in r["step_window_ms"]],
            "split_replays_per_window": args.split_replays * args.layers,
            "split_us_per_window": [round(x * 1e3, 2) for x in r["split_window_ms"]],
            "how": "median of the windows; each window a HIP-graph replay timed with HIP events on "
                   "its stream, after settle_steps steps of clock settling and the warmup steps",
        },
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16 MFMA, f32 accumulate" if args.dtype == "bf16"
                  else "i8 MFMA (Q.K, i32 accumulate) + f16 MFMA (P.V, f32 accumulate)"),
        "data": "synthetic",
        "config": {
            "workload": f"decode B1 Hq24 Hkv4 D256, "
                        f"{'unquantized bf16' if args.dtype == 'bf16' else args.dtype + ' per-row absmax'} "
                        f"cache, {args.ctx}-token context, 1 query token, {args.layers} layer caches "
                        f"rotated",
            "step": ("kvq_append_decode_attend (append fused into the split kernel) + combine"
                     if fused else "kvq_append + split decode + combine"),
            "cache_dtype": args.dtype,
            "context": args.ctx,
            "splits": r["splits"],
            "algorithmic_bytes_per_step": r["bytes"],
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
        },
    }
    fl_us, fl_wg = (None, None) if args.no_stream_floor else time_stream_floor(kvq, torch, r["bytes"],
                                                                                 args.layers, dev)
    if fl_us is not None:
        line["stream_floor"] = {
            "us": round(fl_us, 2),
            "GB/s": round(r["bytes"] / (fl_us * 1e-6) / 1e9, 1),
            "frac_of_peak": round(r["bytes"] / (fl_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
            "workgroups": fl_wg,
            "split_kernel_over_floor": round(r["split_ms"] * 1e3 / fl_us, 3),
            "what": "kvq_stream_read of the same bytes: the decode's loads and nothing else",
        }
    if not args.no_cpu_baseline:
        n, sec, threads, n1, sec1 = cpu_baseline(ki, w, args.cpu_seconds, args.cpu_seconds_1t)
        line["cpu_baseline"] = {
            "value": round(r["bytes"] / sec / 1e9, 4),
            "unit": "GB/s",
            "cores": threads,
            "kind": "oracle",
            "sample": f"{n} oracle steps (dequantize the {args.ctx}-token layer cache to fp32, "
                      f"then fp64 attention) on the same workload, {sec * 1e3:.0f} ms/step on "
                      f"{threads} OpenMP threads; {n1} steps on 1 thread, {sec1 * 1e3:.0f} ms/step",
            "cpu_model": cpu_model(),
            "value_1_thread": round(r["bytes"] / sec1 / 1e9, 4),
            "ms_per_step": round(sec * 1e3, 1),
            "ms_per_step_1_thread": round(sec1 * 1e3, 1),
        }
    print(json.dumps(line), flush=True)

    if args.sweep:
        with open(args.sweep, "w") as f:
            for dt in ("int8", "int4"):
                for ctx in ki.SWEEP_CTX:
                    layers = args.layers if ctx <= 65536 else 8
                    s = time_config(kvq, torch, ki, dt, ctx, layers, max(64, args.steps // 4),
                                    args.warmup, dev, fused)
                    s.pop("workload")
                    s["step_GBps"] = s["bytes"] / (s["step_ms"] * 1e-3) / 1e9
                    s["split_GBps"] = s["bytes"] / (s["split_ms"] * 1e-3) / 1e9
                    s["split_frac_of_peak"] = s["split_GBps"] / PEAK_HBM_GBPS
                    fl_us, fl_wg = time_stream_floor(kvq, torch, s["bytes"], layers, dev)
                    s["stream_floor_us"] = fl_us
                    s["stream_floor_workgroups"] = fl_wg
                    f.write(json.dumps(s) + "\n")
                    f.flush()
                    print(f"[sweep] {dt} ctx={ctx} step {s['step_ms'] * 1e3:.2f} us "
                          f"split {s['split_ms'] * 1e3:.2f} us {s['split_GBps']:.0f} GB/s",
                          file=sys.stderr, flush=True)
                    torch.cuda.empty_cache()
            extra = [ki.make_workload(cfg) for cfg in (2, 4, 5)]
            for win, cap in ((4096, 0.0), (0, 30.0)):
                w = ki.make_workload(3, ctx=65536, dtype="int8")
                w.window, w.softcap = win, cap
                w.name = f"{w.name}-window{win}-softcap{int(cap)}"
                extra.append(w)
            for w in extra:
                cfg = w.cfg
                s = time_workload(kvq, torch, w, args.layers, max(64, args.steps // 4), args.warmup,
                                  dev, fused)
                s["cfg"] = cfg
                s["window"], s["softcap"] = w.window, w.softcap
                s["step_GBps"] = s["bytes"] / (s["step_ms"] * 1e-3) / 1e9
                s["split_GBps"] = s["bytes"] / (s["split_ms"] * 1e-3) / 1e9
                s["split_frac_of_peak"] = s["split_GBps"] / PEAK_HBM_GBPS
                fl_us, fl_wg = time_stream_floor(kvq, torch, s["bytes"], args.layers, dev)
                s["stream_floor_us"] = fl_us
                s["stream_floor_workgroups"] = fl_wg
                f.write(json.dumps(s) + "\n")
                f.flush()
                print(f"[sweep] cfg{cfg} {w.name} step {s['step_ms'] * 1e3:.2f} us "
                      f"split {s['split_ms'] * 1e3:.2f} us {s['split_GBps']:.0f} GB/s",
                      file=sys.stderr, flush=True)
                torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
