"""Benchmark of the MI355X canvas-denoise step (one GPU).

A "step" is one pass of the whole hot path over one 256-token canvas: canvas attention
over the prefix KV cache, the fused logits/entropy/argmax sampler head over the
262144-token vocabulary, entropy-bounded acceptance, renoise, self-conditioning and the
stop test; whenever a canvas reaches its stop or its 48-step cap the commit of its K/V
and the next canvas's initialization fall inside the timed region too.

Workload (default "gemma_head"): V=262144, d=2048, C=256, 16 query / 8 KV heads of
128, FFW 1024, prefix 8192 tokens, N=48, synthetic seeded weights and driver hidden
states (dg_inputs), all resident in HBM before timing starts. Every canvas attends over
the same 8192-token prefix: after each commit the cache length is set back to it, so the
commit's rows are rewritten by the next canvas's commit.

Protocol: one whole warm-up canvas is run and discarded first (the clock ramps during
the first tens of launches of a process), then --warmup untimed steps, then exactly
--steps timed steps (value = steps/s). Canvas tokens/s comes from whole canvases timed
from initialization to commit: the median of --canvases of them.

Prints one JSON line: denoise steps/s (value), canvas tokens/s (also with each canvas
run by the library's own loop, dg_run_canvas), the roofline of the dominant pair of
calls (the sampler head dg_logits_entropy and self-conditioning dg_selfcond_accept,
which together are most of the step; both timed live with HIP events inside real
steps), the same protocol at the tiny and small workloads, and the CPU oracle's rate on
a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "denoise steps/s & canvas tokens/s (256-canvas, 262K vocab); % MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=240)
    ap.add_argument("--warmup", type=int, default=48)
    ap.add_argument("--config", default="gemma_head")
    ap.add_argument("--roofline-reps", type=int, default=20)
    ap.add_argument("--cpu-steps", type=int, default=6, help="oracle steps timed for cpu_baseline (about 10 s)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-batched", action="store_true", help="skip the batched-canvas lines")
    ap.add_argument("--no-moe", action="store_true", help="skip the canvas MoE FFN line")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured HBM and MFMA ceilings")
    ap.add_argument("--no-long-prefix", action="store_true",
                    help="skip the isolated attention call over a 262144-token prefix")
    ap.add_argument("--no-chain", action="store_true",
                    help="skip the 8-canvas block-AR chain with commits")
    ap.add_argument("--no-small", action="store_true",
                    help="skip the protocol lines of the small and tiny workloads")
    ap.add_argument("--no-cache-probe", action="store_true",
                    help="skip the sampler head over a cache-resident slice of E")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the eager-vs-graph lines of fixed-step canvases")
    ap.add_argument("--canvases", type=int, default=7,
                    help="whole canvases timed for canvas tokens/s (median), after one warm-up canvas")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 1 GiB device copy (for HBM counter calibration)")
    return ap.parse_args()


# kernel sources of the pair, the shared header (workspace layout, split counts) and the
# acceptance routines that run beside the self-conditioning reduce
PAIR_SOURCES = ("k_logits.hip", "k_selfcond.hip", "k_gemm.hip", "dg_common.h", "dg_sampler_dev.h")


def pair_traffic_from_profiles():
    """HBM bytes per step of the dominant pair (both calls' kernels), from the committed
    counter summary, if it was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "sampler_pair_gemma_head_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        parts = line.split()
        if len(parts) == 2 and not line.startswith("#"):
            vals[parts[0]] = parts[1]
    h = hashlib.sha256()
    for f in PAIR_SOURCES:
        h.update(open(os.path.join(ROOT, "block_ar_canvas_amd", "csrc", f), "rb").read())
    if vals.get("sources_sha256_16") != h.hexdigest()[:16] or "hbm_bytes_per_step" not in vals:
        return None
    return float(vals["hbm_bytes_per_step"])


def pair_sources_sha():
    h = hashlib.sha256()
    for f in PAIR_SOURCES:
        h.update(open(os.path.join(ROOT, "block_ar_canvas_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def run_protocol(loop, hidden_of, canvases: int, P0: int):
    """One discarded warm-up canvas, then `canvases` whole canvases timed one by one from
    initialization to commit (each over the same P0-token prefix). Returns the per-canvas
    seconds and step counts."""
    import torch

    secs, steps = [], []
    for c in range(canvases + 1):
        loop.P = P0
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        n = loop.run_canvas(c, hidden_of(c))
        torch.cuda.synchronize()
        if c > 0:
            secs.append(time.perf_counter() - t0)
            steps.append(n)
    loop.P = P0
    return secs, steps


def protocol_summary(secs, steps, C):
    i = int(np.argsort(secs)[len(secs) // 2])
    return {"canvases": len(secs), "warmup_canvases": 1,
            "median_ms_per_canvas": round(1e3 * secs[i], 3), "steps_per_canvas": steps[i],
            "steps_per_s": round(steps[i] / secs[i], 2),
            "canvas_tokens_per_s": round(C / secs[i], 1),
            "ms_per_canvas": [round(1e3 * x, 3) for x in secs]}


def graph_canvas_rate(ctx, loop, hidden, reps):
    """Whole canvases enqueued with no host wait (init, every step, commit; no adaptive
    stop), first eagerly and then captured once in a HIP graph and replayed: steps/s of
    each. Against the protocol's canvases (which poll the stop flag between steps) this
    separates what the host's launches cost from what the kernels cost."""
    import torch

    P0 = loop.P
    old = ctx.stream
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    ctx.set_stream(s)
    try:
        with torch.cuda.stream(s):
            loop.enqueue_canvas_fixed(1, hidden)            # warm-up
            loop.P = P0
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(s):
            for _ in range(reps):
                loop.enqueue_canvas_fixed(1, hidden)
                loop.P = P0
        torch.cuda.synchronize()
        eager = time.perf_counter() - t0
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            loop.enqueue_canvas_fixed(1, hidden)
        loop.P = P0
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        graph = time.perf_counter() - t0
        del g
    finally:
        torch.cuda.synchronize()
        ctx.set_stream(old)
    n = reps * loop.N
    return {"canvases": reps, "eager_fixed_steps_per_s": round(n / eager, 2),
            "graph_steps_per_s": round(n / graph, 2),
            "graph_canvas_tokens_per_s": round(reps * loop.dims.C / graph, 1)}


def native_protocol(ctx, cfg, Wd, Kd, Vtd, hidden_of, canvases):
    """The protocol with each canvas run by dg_run_canvas (the loop sequenced inside the
    library: one host call per canvas instead of one per kernel call): one discarded
    warm-up canvas, then `canvases` whole canvases from the same prefix, as in
    run_protocol."""
    import torch

    import block_ar_canvas_amd as dg

    dev = Kd.device
    ws = torch.empty(dg.workspace_bytes(cfg, Kd.shape[1]), dtype=torch.uint8, device=dev)
    lws = torch.empty(dg.loop_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    x0 = torch.empty(cfg.C, dtype=torch.int32, device=dev)
    secs, steps = [], []
    for c in range(canvases + 1):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        n, _ = ctx.run_canvas(cfg, Wd, Kd, Vtd, cfg.P0, hidden_of(c), ws, lws, x0, N=cfg.N,
                              seed=cfg.seed, canvas=c)
        torch.cuda.synchronize()
        if c > 0:
            secs.append(time.perf_counter() - t0)
            steps.append(n)
    ctx.sync()
    return protocol_summary(secs, steps, cfg.C)


def small_workload(ctx, name, canvases):
    """The protocol at a smaller workload (tiny or small): steps/s and canvas tokens/s."""
    import torch

    import dg_inputs as di
    from block_ar_canvas_amd.loop import CanvasLoop
    cfg = di.config(name)
    dev = torch.device("cuda:0")
    W = di.weights(cfg)
    Kp, Vp = di.prefix_kv(cfg, cfg.P0 + cfg.C)
    Wd = {k: _bf(v, dev) for k, v in W.items()}
    Kd = _bf(Kp, dev)
    Vtd = _bf(np.ascontiguousarray(Vp.transpose(0, 2, 1)), dev)
    Hd = [_bf(di.hidden_all(cfg, W["E"], c), dev) for c in range(2)]
    loop = CanvasLoop(ctx, cfg, Wd, Kd, Vtd, cfg.P0, N=cfg.N, seed=cfg.seed)
    secs, steps = run_protocol(loop, lambda c: (lambda k: Hd[c % 2][k]), canvases, cfg.P0)
    ctx.sync()
    out = protocol_summary(secs, steps, cfg.C)
    out["fixed_step_canvases"] = graph_canvas_rate(ctx, loop, lambda k: Hd[0][k], 100 if cfg.V < 4096 else 20)
    out["native_loop"] = native_protocol(ctx, cfg, Wd, Kd, Vtd, lambda c: (lambda k: Hd[c % 2][k]), canvases)
    out["workload"] = (f"{cfg.name}: V={cfg.V} d={cfg.d} C={cfg.C} Hq={cfg.Hq} Hkv={cfg.Hkv} "
                       f"hd={cfg.hd} F={cfg.F} prefix={cfg.P0} N={cfg.N}")
    return out


_T0 = time.time()


def note(what: str):
    """One progress line on stderr as a section of the run finishes (stdout carries only
    the result line)."""
    print(f"bench.py: {what} ({time.time() - _T0:.1f} s)", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); the path has "
              "no multi-GPU sharding, so N > 1 is not supported", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_ar_canvas_amd as dg
    import dg_inputs as di
    from block_ar_canvas_amd.loop import CanvasLoop

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    cfg = di.config(args.config)
    Pcap = -(-(cfg.P0 + cfg.C) // 8) * 8
    n_hidden = 4                                      # driver states cycle over 4 canvases

    t_gen = time.time()
    W = di.weights(cfg)
    Kp, Vp = di.prefix_kv(cfg, Pcap)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    Wd = {k: bf(v) for k, v in W.items()}
    Kd = bf(Kp)
    Vtd = bf(np.ascontiguousarray(Vp.transpose(0, 2, 1)))
    del Vp
    Hd = [bf(di.hidden_all(cfg, W["E"], c)) for c in range(n_hidden)]
    torch.cuda.synchronize()
    t_gen = time.time() - t_gen
    note("inputs on the device")

    ctx = dg.Context(0)
    loop = CanvasLoop(ctx, cfg, Wd, Kd, Vtd, cfg.P0, N=cfg.N, seed=cfg.seed)

    # the protocol's warm-up canvas, discarded
    loop.run_canvas(0, lambda k: Hd[0][k])
    loop.P = cfg.P0
    torch.cuda.synchronize()

    # Drive the block-AR loop step by step so that exactly `steps` steps are timed.
    state = {"canvas": 0, "k": 0, "done": True, "commits": 0}

    def one_step():
        s = state
        if s["done"]:
            s["canvas"] += 1
            s["k"] = 0
            s["done"] = False
            loop.init_canvas(s["canvas"])
            loop.step(0, Hd[s["canvas"] % n_hidden][0])
            return
        k = s["k"]
        if k + 1 < cfg.N:
            loop.step(k + 1, Hd[s["canvas"] % n_hidden][k + 1])
        flag = loop.wait_flag(k)
        if flag != dg.STOP_GO:
            loop.commit(loop.argmax[k & 1])
            loop.P = cfg.P0                            # every canvas over the same prefix
            s["commits"] += 1
            s["done"] = True
            return
        s["k"] = k + 1

    # Each call of one_step enqueues one denoise step (or, at a canvas end, the commit
    # whose step was the speculative one); count enqueued denoise steps.
    def run(n):
        steps = 0
        while steps < n:
            one_step()
            if not state["done"]:
                steps += 1
        return steps

    run(args.warmup)
    torch.cuda.synchronize()
    note("warm-up canvas and steps")
    c0 = state["commits"]
    t0 = time.perf_counter()
    run(args.steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    commits = state["commits"] - c0
    sec = t1 - t0
    steps_per_s = args.steps / sec
    ctx.sync()
    note(f"{args.steps} timed steps")

    # Roofline of the dominant pair: the sampler head (dg_logits_entropy: logits tile
    # kernel and row finalize) and self-conditioning (dg_selfcond_accept: p0 E split
    # kernel, reduce with the acceptance/renoise/stop workgroups beside it, the two FFW
    # GEMMs), timed live with HIP events on the library's stream
    # around each call inside real denoise steps (the same loop, continued for
    # max(reps, 48) steps after the timed region, so the event packets do not touch the
    # headline step time).
    loop.logits_events, loop.selfcond_events = [], []
    run(max(args.roofline_reps, 48))
    torch.cuda.synchronize()
    evl, loop.logits_events = loop.logits_events, None
    evs, loop.selfcond_events = loop.selfcond_events, None
    logits_ms = sum(a.elapsed_time(b) for a, b in evl) / len(evl)
    selfcond_ms = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
    pair_ms = logits_ms + selfcond_ms
    # algorithmic bytes: E read by each call, H, the FFW weights and the outputs
    # (entropy, argmax, z); the bf16 probabilities passed between the calls are a design
    # choice and are not counted, nor are the acceptance's few KiB
    e_bytes = cfg.V * cfg.d * 2
    ffw_bytes = 2 * cfg.F * cfg.d * 2
    alg_bytes = 2 * e_bytes + cfg.C * cfg.d * 2 + ffw_bytes + cfg.C * 8 + cfg.C * cfg.d * 2
    alg_flops = 2 * (2.0 * cfg.C * cfg.V * cfg.d) + 2 * (2.0 * cfg.C * cfg.d * cfg.F)
    achieved = alg_bytes / (pair_ms * 1e-3) / 1e9
    traffic = pair_traffic_from_profiles()

    # the protocol: whole canvases, init to commit
    secs, csteps = run_protocol(loop, lambda c: (lambda k: Hd[c % n_hidden][k]), args.canvases, cfg.P0)
    ctx.sync()
    proto = protocol_summary(secs, csteps, cfg.C)
    note("whole-canvas protocol")
    if not args.no_graph:
        proto["fixed_step_canvases"] = graph_canvas_rate(ctx, loop, lambda k: Hd[0][k], 5)
        note("fixed-step and graph canvases")
    proto["native_loop"] = native_protocol(ctx, cfg, Wd, Kd, Vtd, lambda c: (lambda k: Hd[c % n_hidden][k]),
                                           args.canvases)
    note("whole-canvas protocol in the library's loop")

    if args.calibrate_copy:
        src_t = torch.empty(1 << 29, dtype=torch.int16, device=dev)
        dst_t = torch.empty_like(src_t)
        dst_t.copy_(src_t)
        torch.cuda.synchronize()

    result = {
        "metric": METRIC,
        "value": round(steps_per_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_canvases": 1,
        "ms_per_step": round(1e3 * sec / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: V={cfg.V} d={cfg.d} C={cfg.C} Hq={cfg.Hq} Hkv={cfg.Hkv} "
                               f"hd={cfg.hd} F={cfg.F} prefix={cfg.P0} N={cfg.N}",
                   "canvas": cfg.C, "vocab": cfg.V, "prefix_tokens": cfg.P0, "max_steps": cfg.N,
                   "parallelism": "single-gpu"},
        "canvas_tokens_per_s": proto["canvas_tokens_per_s"],
        "canvas_protocol": proto,
        "canvas_tokens_per_s_at_12_steps": round(steps_per_s * cfg.C / 12, 1),
        "commits_timed": commits,
        "roofline": {"kernel": "dg_logits_entropy + dg_selfcond_accept (logits_tile_kernel, row_finalize_kernel, "
                               "selfcond_split_kernel, selfcond_reduce_kernel with the acceptance workgroups, "
                               "2 FFW gemm_kernel)",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "alg_bytes_per_step": alg_bytes,
                     "alg_flop_per_step": alg_flops,
                     "ms_per_step": round(pair_ms, 4), "launches_timed": len(evl),
                     "logits_ms_per_call": round(logits_ms, 4),
                     "selfcond_ms_per_call": round(selfcond_ms, 4),
                     "mfma_frac": round(alg_flops / (pair_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                     "logits_mfma_frac": round(2.0 * cfg.C * cfg.V * cfg.d / (logits_ms * 1e-3) / 1e12
                                               / BF16_PEAK_TFLOPS, 4)},
        "input_gen_s": round(t_gen, 1),
    }

    if not args.no_cache_probe and cfg.V >= 65536:
        cr = cache_resident_logits(ctx, cfg, Wd, args.roofline_reps)
        # the in-step call: 1024 tiles over 256 CUs, four tiles per CU
        cr["in_step_us_per_tile_per_cu"] = round(1e3 * logits_ms / (cfg.V / 256 / 256), 2)
        result["cache_resident_logits"] = cr
        note("cache-resident sampler head")
    if not args.no_long_prefix:
        result["long_prefix_attention"] = long_prefix_attention(ctx, cfg, Wd, Hd[0], args.roofline_reps)
        note("long-prefix attention")
    del Kd, Vtd, loop
    if not args.no_batched:
        result["batched"] = [batched_canvases(ctx, cfg, Wd, Hd, B) for B in (2, 4)]
        result["confidence_rule"] = variant_canvas(ctx, cfg, Wd, Hd, rule="confidence")
        result["sampled_tokens"] = variant_canvas(ctx, cfg, Wd, Hd, draw="sample")
        note("batched canvases and the acceptance variants")
    del Hd
    if not args.no_small:
        result["small"] = small_workload(ctx, "small", args.canvases)
        note("small workload")
        result["tiny"] = small_workload(ctx, "tiny", args.canvases)
        note("tiny workload")
    if not args.no_chain:
        result["chain8"] = chain(ctx)
        result["chain8_prefill"] = chain(ctx, commit="prefill", rope_base=10000.0)
        note("chains of 8 canvases")
    if not args.no_moe:
        result["moe_ffn"] = moe_ffn(ctx, cfg, args.roofline_reps)
        note("MoE FFN")
    if not args.no_peaks:
        pk = measured_peaks(ctx)
        note("measured ceilings")
        result["measured_peaks"] = pk
        rf = result["roofline"]
        rf["frac_of_measured"] = round(rf["achieved"] / pk["hbm_read_GBs"], 4)
        rf["mfma_frac_of_measured"] = round(rf["mfma_frac"] * BF16_PEAK_TFLOPS / pk["mfma_bf16_TFLOPs"], 4)
        if "long_prefix_attention" in result:
            lp = result["long_prefix_attention"]
            lp["hbm_frac_of_measured"] = round(lp["achieved_GBs"] / pk["hbm_read_GBs"], 4)
            lp["mfma_frac_of_measured"] = round(lp["attention_tflops"] / pk["mfma_bf16_TFLOPs"], 4)
        if "moe_ffn" in result:
            mo = result["moe_ffn"]
            mo["hbm_frac_of_measured"] = round(mo["achieved_GBs"] / pk["hbm_read_GBs"], 4)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, W, Kp, args.cpu_steps)
        note("CPU oracle baseline")
    print(json.dumps(result))


def measured_peaks(ctx):
    """What this GPU reaches in practice: a streaming read of a 4 GiB buffer (16 times the
    256 MB last-level cache, so it measures HBM) and back-to-back bf16 MFMAs with register
    operands. Both through the library (dg_peak_stream_read, dg_peak_mfma_bf16), timed
    with HIP events on the library's stream; best of several launches."""
    import torch

    import block_ar_canvas_amd as dg
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.empty(dg.PEAK_STREAM_BLOCKS, dtype=torch.int32, device=dev)
    fsink = torch.empty(dg.PEAK_MFMA_BLOCKS * 4, dtype=torch.float32, device=dev)

    def best_ms(fn, n):
        fn()
        best = float("inf")
        for _ in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            best = min(best, e0.elapsed_time(e1))
        return best

    ms_r = best_ms(lambda: ctx.peak_stream_read(buf, sink), 5)
    flop = [0]

    def mf():
        flop[0] = ctx.peak_mfma(4096, fsink)
    ms_m = best_ms(mf, 5)
    ctx.sync()
    del buf
    return {"hbm_read_GBs": round(nbytes / (ms_r * 1e-3) / 1e9, 1),
            "hbm_read_frac_of_published": round(nbytes / (ms_r * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_bf16_TFLOPs": round(flop[0] / (ms_m * 1e-3) / 1e12, 1),
            "mfma_frac_of_published": round(flop[0] / (ms_m * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "read_bytes": nbytes, "mfma_flop": flop[0]}


def _bf(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


def cache_resident_logits(ctx, cfg, Wd, reps):
    """dg_logits_entropy over the first 32768 rows of E (128 MiB, held by the 256 MB
    memory-side cache across back-to-back calls) for one 256-column canvas: 128 vocabulary
    tiles, each the same work as one tile of the full-vocabulary call (1024 tiles, four
    rounds of 256). If the full call were waiting on HBM, a tile would take longer there
    than here; the per-tile times are reported side by side with the in-step call."""
    import torch

    import block_ar_canvas_amd as dg
    dev = torch.device("cuda:0")
    Vs = 32768
    dims = dg.Dims(Vs, cfg.d, cfg.C, cfg.Hq, cfg.Hkv, cfg.hd, cfg.F)
    E = Wd["E"][:Vs]
    H = torch.randn(cfg.C, cfg.d, device=dev).to(torch.bfloat16)
    ws = torch.empty(dg.workspace_bytes(dims, 0), dtype=torch.uint8, device=dev)
    ent = torch.empty(cfg.C, dtype=torch.float32, device=dev)
    am = torch.empty(cfg.C, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(10):
        ctx.logits_entropy(dims, H, E, 0.4, ws, ent, am)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = max(reps, 20)
    e0.record(stream)
    for _ in range(n):
        ctx.logits_entropy(dims, H, E, 0.4, ws, ent, am)
    e1.record(stream)
    e1.synchronize()
    ctx.sync()
    ms = e0.elapsed_time(e1) / n
    return {"vocab_rows": Vs, "e_bytes": Vs * cfg.d * 2, "tiles": Vs // 256, "ms_per_call": round(ms, 4),
            "us_per_tile_per_cu": round(1e3 * ms, 2)}


def long_prefix_attention(ctx, cfg, Wd, H, reps):
    """One dg_canvas_attn call over a 262144-token prefix (the long-prefix workload's
    cache, seed 3, with the sampler-head workload's weights), timed with HIP events.
    The rates are per whole call (embedding gather, Q/K/V projection, split attention,
    merge and Wo), so they understate the attention kernel itself."""
    import torch
    import dg_inputs as di

    lp = di.config("long_prefix")
    dev = torch.device("cuda:0")
    P = lp.P0
    Pcap = -(-(P + cfg.C) // 8) * 8
    Kp, Vp = di.prefix_kv(lp, Pcap)
    Kd = _bf(Kp, dev)
    del Kp
    Vtd = _bf(np.ascontiguousarray(Vp.transpose(0, 2, 1)), dev)
    del Vp
    ws = torch.empty(__import__("block_ar_canvas_amd").workspace_bytes(cfg, Pcap), dtype=torch.uint8,
                     device=dev)
    tok = torch.from_numpy(di.targets(lp, 0)).to(dev)
    z = H[cfg.N - 1]
    A = torch.empty(cfg.C, cfg.d, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # ten untimed calls first: the first calls after a pause run at a boost clock that the
    # part does not hold, so a short timed window would overstate the steady rate
    reps = max(reps, 10)
    for _ in range(10):
        ctx.canvas_attn(cfg, tok, z, Wd["E"], Wd["Wq"], Wd["Wk"], Wd["Wv"], Wd["Wo"], Kd, Vtd, P, ws, A)
    e0.record(stream)
    for _ in range(reps):
        ctx.canvas_attn(cfg, tok, z, Wd["E"], Wd["Wq"], Wd["Wk"], Wd["Wv"], Wd["Wo"], Kd, Vtd, P, ws, A)
    e1.record(stream)
    e1.synchronize()
    ctx.sync()
    ms = e0.elapsed_time(e1) / reps
    keys = P + cfg.C
    kv_bytes = 2 * cfg.Hkv * keys * cfg.hd * 2
    flops = 4.0 * cfg.Hq * cfg.C * keys * cfg.hd
    gbs = kv_bytes / (ms * 1e-3) / 1e9
    tfs = flops / (ms * 1e-3) / 1e12
    return {"prefix_tokens": P, "ms_per_call": round(ms, 4), "kv_bytes": kv_bytes,
            "achieved_GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "attention_tflops": round(tfs, 1), "mfma_frac": round(tfs / BF16_PEAK_TFLOPS, 4)}


def batched_canvases(ctx, cfg, Wd, Hd, B):
    """B canvases in lockstep, one per request, each request with its own prefix of
    cfg.P0 tokens (seeded per request): one warm-up batch, then one timed batch from
    init to the last commit. The logits kernel runs on B*C columns here; its in-step time
    (HIP events around each dg_logits_entropy) gives the MFMA fraction at that width."""
    import torch

    import dg_inputs as di
    from block_ar_canvas_amd.loop import BatchLoop
    dev = Hd[0].device
    Pcap = -(-(cfg.P0 + 2 * cfg.C) // 8) * 8
    caches = []
    for r in range(B):
        Kp, Vp = di.prefix_kv(cfg, Pcap, request=r)
        caches.append((_bf(Kp, dev), _bf(np.ascontiguousarray(Vp.transpose(0, 2, 1)), dev), cfg.P0))
        del Kp, Vp
    loop = BatchLoop(ctx, cfg, Wd, caches, N=cfg.N, seed=cfg.seed)
    stream = torch.cuda.current_stream()

    def hidden_of(j):
        hs = [torch.cat([Hd[(j * B + i) % len(Hd)][k] for i in range(B)], dim=0) for k in range(cfg.N)]
        return lambda k: hs[k]

    loop.run_batch(0, hidden_of(0))
    h1 = hidden_of(1)
    torch.cuda.synchronize()
    loop.logits_events = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    steps = loop.run_batch(1, h1)
    e1.record(stream)
    e1.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3
    evs = loop.logits_events
    logits_ms = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
    flops = 2.0 * B * cfg.C * cfg.V * cfg.d
    return {"B": B, "canvas_tokens_per_s": round(B * cfg.C / sec, 1),
            "batched_steps_per_s": round(max(steps) / sec, 2),
            "ms_per_batched_step": round(1e3 * sec / max(steps), 4),
            "logits_ms_per_launch": round(logits_ms, 4),
            "logits_mfma_frac": round(flops / (logits_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "prefix_tokens_per_request": cfg.P0}


def variant_canvas(ctx, cfg, Wd, Hd, rule="entropy", draw="argmax"):
    """The step loop with another acceptance rule (confidence-ranked) or sampled tokens
    instead of the argmax: one warm-up canvas, then one timed canvas (init to commit) at
    the same workload."""
    import torch

    import dg_inputs as di
    from block_ar_canvas_amd.loop import CanvasLoop
    dev = Hd[0].device
    Pcap = -(-(cfg.P0 + 2 * cfg.C) // 8) * 8
    Kp, Vp = di.prefix_kv(cfg, Pcap)
    loop = CanvasLoop(ctx, cfg, Wd, _bf(Kp, dev), _bf(np.ascontiguousarray(Vp.transpose(0, 2, 1)), dev),
                      cfg.P0, N=cfg.N, seed=cfg.seed, rule=rule, draw=draw)
    del Kp, Vp
    loop.run_canvas(0, lambda k: Hd[0][k])
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    steps = loop.run_canvas(1, lambda k: Hd[1 % len(Hd)][k])
    e1.record(stream)
    e1.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3
    return {"rule": rule, "draw": draw, "steps": steps, "ms_per_step": round(1e3 * sec / steps, 4),
            "canvas_tokens_per_s": round(cfg.C / sec, 1)}


def moe_ffn(ctx, cfg, reps):
    """The canvas MoE FFN on one canvas at the workload's width: 128 experts, 8 routed per
    token plus a shared expert, expert width 512, shared width 1024 (stand-in sizes). The
    canvas rows share part of their direction, so the random router sends the canvas to
    about 84 distinct experts, as the pages report for real text. Reports the call time
    and the weight bytes it streams (router, the experts used, the shared expert) as
    achieved GB/s."""
    import torch

    import block_ar_canvas_amd as dg
    import dg_inputs as di
    C, d, E, K, Fe, Fs = cfg.C, cfg.d, 128, 8, 512, 1024
    dev = torch.device("cuda:0")
    inp = di.moe_inputs(C, d, E, K, Fe, Fs, seed=61, share=di.MOE_CANVAS_SHARE)
    dv = {k: _bf(v, dev) for k, v in inp.items()}
    del inp
    md = dg.MoeDims(d, E, K, Fe, Fs)
    ws = torch.empty(dg.moe_workspace_bytes(md, C), dtype=torch.uint8, device=dev)
    Y = torch.empty(C, d, dtype=torch.bfloat16, device=dev)
    nact = torch.zeros(1, dtype=torch.int32, device=dev)
    args = (md, dv["X"], dv["Wr"], dv["W1"], dv["W2"], dv["W1s"], dv["W2s"], ws, Y, nact)
    for _ in range(5):
        ctx.moe_ffn(*args)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = max(reps, 10)
    e0.record(stream)
    for _ in range(n):
        ctx.moe_ffn(*args)
    e1.record(stream)
    e1.synchronize()
    ms = e0.elapsed_time(e1) / n
    na = int(nact.item())
    wbytes = 2 * (E * d + na * 2 * Fe * d + 2 * Fs * d)
    return {"workload": f"canvas MoE FFN: C={C} d={d} experts={E} top-{K} Fe={Fe} shared Fs={Fs}, "
                        f"canvas rows sharing {di.MOE_CANVAS_SHARE:.2f} of their variance",
            "ms_per_call": round(ms, 4), "experts_used": na,
            "weight_bytes": wbytes, "achieved_GBs": round(wbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(wbytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4)}


def chain(ctx, commit="projection", rope_base=0.0):
    """The 8-canvas block-AR chain (chain8 workload: prefix 32768, seed 4): every canvas
    runs its step loop to the stop test or the 48-step cap and commits its K/V before
    the next canvas starts. Returns canvas tokens/s including commits. commit="prefill"
    (with rope_base) commits by the causal re-encode, with rotary positions throughout,
    and also reports the prefill call's own time."""
    import torch
    import dg_inputs as di
    from block_ar_canvas_amd.loop import CanvasLoop

    cc = di.config("chain8")
    dev = torch.device("cuda:0")
    W = di.weights(cc)
    Wd = {k: _bf(v, dev) for k, v in W.items()}
    Kp, Vp = di.prefix_kv(cc)
    Kd = _bf(Kp, dev)
    Vtd = _bf(np.ascontiguousarray(Vp.transpose(0, 2, 1)), dev)
    del Kp, Vp
    Hd = [_bf(di.hidden_all(cc, W["E"], c), dev) for c in range(cc.n_canvas)]
    del W
    loop = CanvasLoop(ctx, cc, Wd, Kd, Vtd, cc.P0, N=cc.N, seed=cc.seed, commit=commit,
                      rope_base=rope_base)
    # warm-up: one canvas on a copy of the cache start, then reset the length
    loop.run_canvas(0, lambda k: Hd[0][k])
    loop.P = cc.P0
    torch.cuda.synchronize()
    steps = 0
    t0 = time.perf_counter()
    for c in range(cc.n_canvas):
        steps += loop.run_canvas(c, lambda k, c=c: Hd[c][k])
    torch.cuda.synchronize()
    sec = time.perf_counter() - t0
    ctx.sync()
    assert loop.P == cc.P0 + cc.n_canvas * cc.C
    out = {"workload": f"chain8: {cc.n_canvas} canvases of {cc.C} from prefix {cc.P0}, V={cc.V} d={cc.d}",
           "commit": commit, "rope_base": rope_base,
           "canvas_tokens_per_s": round(cc.n_canvas * cc.C / sec, 1),
           "steps": steps, "steps_per_s": round(steps / sec, 2), "seconds": round(sec, 4)}
    if commit == "prefill":
        # the commit call alone, at the chain's final length (reset after each call)
        P_end = loop.P - cc.C
        x0 = torch.zeros(cc.C, dtype=torch.int32, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        stream = torch.cuda.current_stream()
        for _ in range(3):
            loop.P = P_end
            loop.commit(x0)
        e0.record(stream)
        for _ in range(10):
            loop.P = P_end
            loop.commit(x0)
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1) / 10
        out["prefill_ms_per_call"] = round(ms, 4)
        # algorithmic work of one prefill call: the cache rows it reads, its weights, the
        # gathered embedding rows and its outputs; causal attention over P_end + i + 1 keys
        # for block row i, plus the QKV and Wo products
        qkv = (cc.Hq + 2 * cc.Hkv) * cc.hd
        pbytes = (2 * cc.Hkv * P_end * cc.hd * 2 + (qkv * cc.d + cc.d * cc.Hq * cc.hd) * 2
                  + cc.C * cc.d * 2 + 2 * cc.Hkv * cc.C * cc.hd * 2 + cc.C * cc.d * 2)
        pflops = (4.0 * cc.Hq * cc.hd * (cc.C * P_end + cc.C * (cc.C + 1) / 2)
                  + 2.0 * cc.C * cc.d * qkv + 2.0 * cc.C * cc.Hq * cc.hd * cc.d)
        out["prefill_keys"] = P_end + cc.C
        out["prefill_GBs"] = round(pbytes / (ms * 1e-3) / 1e9, 1)
        out["prefill_hbm_frac"] = round(pbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        out["prefill_tflops"] = round(pflops / (ms * 1e-3) / 1e12, 1)
        out["prefill_mfma_frac"] = round(pflops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
        out["prefill_prefix_tokens"] = P_end
    ctx.set_rope(0.0)
    return out


def cpu_info():
    """CPU model, BLAS library and its thread count on this host."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas, threads = "unknown", os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            blas = f"{info[0].get('internal_api')} {info[0].get('version')} ({info[0].get('threading_layer')})"
            threads = max(i.get("num_threads", 1) for i in info)
    except Exception:
        pass
    return model, blas, int(threads), len(os.sched_getaffinity(0))


def oracle_steps(cfg, W, Kp, Vp, k0, n_steps):
    """n full oracle denoise steps of one canvas from step k0 (attention, sampler head,
    acceptance, renoise, self-conditioning, stop test). Returns seconds."""
    import oracle as O
    import dg_inputs as di

    tgt = di.targets(cfg, 0)
    tok = np.random.default_rng(0).integers(0, cfg.V, cfg.C).astype(np.int32)
    z = np.zeros((cfg.C, cfg.d), np.uint16)
    H = [di.hidden(cfg, W["E"], 0, k0 + i, tgt) for i in range(n_steps)]
    prev = None
    t0 = time.perf_counter()
    for i in range(n_steps):
        k = k0 + i
        tau = O.temperature(k, cfg.N)
        O.canvas_attn(tok, z, W["E"], W["Wq"], W["Wk"], W["Wv"], W["Wo"], Kp, Vp, cfg.P0,
                      cfg.Hq, cfg.Hkv, cfg.hd)
        ent, am, p, _ = O.logits_entropy(H[i], W["E"], tau)
        acc, _ = O.entropy_accept(ent[None], 0.1)
        tok = O.renoise(am[None], acc, cfg.seed, 0, k, cfg.V)[0]
        z, _ = O.selfcond(p, W["E"], W["W1"], W["W2"])
        O.stop_test(ent, am, prev, 0.005, k, cfg.N)
        prev = am
    return time.perf_counter() - t0


def cpu_baseline(cfg, W, Kp, n_steps):
    """The CPU oracle, as it stands, on bounded samples: n full steps of the workload's
    canvas with every BLAS thread; two steps of the small workload with every thread and
    one step with one thread; a whole tiny-workload canvas; and canvas attention over the
    262144-token prefix for one KV head (scaled to all heads)."""
    import dg_inputs as di

    model, blas, threads, affinity = cpu_info()
    Kp_o = Kp[:, :cfg.P0 + cfg.C].copy()
    _, Vp_o = di.prefix_kv(cfg, cfg.P0 + cfg.C)
    sec = oracle_steps(cfg, W, Kp_o, Vp_o, cfg.N // 2, n_steps)
    del Kp_o, Vp_o
    sm = di.config("small")
    Ws = di.weights(sm)
    Ks, Vs = di.prefix_kv(sm, sm.P0 + sm.C)
    oracle_steps(sm, Ws, Ks, Vs, sm.N // 2, 1)                  # first-touch warm-up
    sec_small = oracle_steps(sm, Ws, Ks, Vs, sm.N // 2, 2) / 2
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            sec_small_1 = oracle_steps(sm, Ws, Ks, Vs, sm.N // 2, 1)
    except Exception:
        sec_small_1 = None
    del Ws, Ks, Vs
    ty = di.config("tiny")
    Wt = di.weights(ty)
    Kt, Vt = di.prefix_kv(ty, ty.P0 + ty.C)
    sec_tiny = oracle_steps(ty, Wt, Kt, Vt, 0, ty.N) / ty.N
    sec_lp_head = long_prefix_attention_oracle_head(cfg, W)
    return {"value": round(n_steps / sec, 5), "unit": "steps/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n_steps} full denoise step(s) of {cfg.name} (k={cfg.N // 2}..), numpy float64, "
                      f"{sec:.1f} s",
            "cpu_model": model, "blas": blas, "blas_threads": threads, "affinity_cpus": affinity,
            "small_s_per_step": round(sec_small, 4),
            "small_s_per_step_1_thread": None if sec_small_1 is None else round(sec_small_1, 4),
            "small_sample": "small workload (V 32768, d 1024, prefix 2048): 2 steps with every "
                            "BLAS thread, 1 step with one thread",
            "tiny_s_per_step": round(sec_tiny, 5),
            "long_prefix_attention_s_per_call": round(sec_lp_head * cfg.Hkv, 2),
            "long_prefix_attention_sample": f"canvas attention over the 262144-token prefix for one of "
                                            f"{cfg.Hkv} KV heads (its {cfg.Hq // cfg.Hkv} query heads, "
                                            f"{sec_lp_head:.1f} s), times {cfg.Hkv}"}


def long_prefix_attention_oracle_head(cfg, W):
    """Seconds the oracle takes for canvas attention over the long-prefix cache restricted
    to KV head 0 and its query heads (the embedding gather, their Q/K/V projections,
    attention over prefix + canvas, and their share of Wo), on the long-prefix workload's
    keys and values for that head."""
    import oracle as O
    import dg_inputs as di

    lp = di.config("long_prefix")
    G, hd = cfg.Hq // cfg.Hkv, cfg.hd
    Kp = di.gaussian_bf16(lp.seed, di.TAG_KP, (1, lp.P0, hd), 1.0)   # = KV head 0 of the cache
    Vp = di.gaussian_bf16(lp.seed, di.TAG_VP, (1, lp.P0, hd), 1.0)
    tok = di.targets(lp, 0)
    Wq, Wk, Wv = W["Wq"][:G * hd], W["Wk"][:hd], W["Wv"][:hd]
    Wo = np.ascontiguousarray(W["Wo"][:, :G * hd])
    t0 = time.perf_counter()
    O.canvas_attn(tok, None, W["E"], Wq, Wk, Wv, Wo, Kp, Vp, lp.P0, G, 1, hd)
    return time.perf_counter() - t0


if __name__ == "__main__":
    main()
