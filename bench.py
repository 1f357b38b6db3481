#!/usr/bin/env python3
"""Benchmark of streaming block-causal chunk attention on one MI355X.

A step is one chunk of a stream in steady state (full window, eviction every
chunk): for each denoising step, append the current block's K/V (fused RoPE +
append kernel) and attend its queries over [sinks, window blocks, current]
(bf16 MFMA attention kernel); then evict the oldest window block and commit the
current one (index remaps).  The headline workload is the largest config, the
720p refiner-style stream (10800 query tokens against 43200 keys, 24 heads,
relative-time RoPE, one step per chunk); the 540p dense stream (6120 against
30600, 4 steps per chunk) is timed after it and reported under `also`.  Other
workloads: TwinCache, block-sparse (tile mask + sparse kernel), variable-length
blocks, frame-aligned editing, fp8.  Inputs are seeded synthetic N(0,1)*0.5
bf16 tensors of the workload's shapes, resident in HBM before timing.

Prints ONE JSON line.  `value` = attention TFLOP per chunk / wall time per
chunk (everything in the step counted in the time).  `roofline` is the
attention kernel alone (HIP events on the launch stream), against the dense
MFMA peak of its arithmetic type (bf16, or fp8 for the fp8 workload), and
against the rate the library's matrix-core probe measures on this device.
`latency_flatness` is the least-squares slope of per-chunk latency over a
further run of chunks.  `cpu_baseline` times the fp64 oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # 256 CU x 2.4 GHz x 4096 flop/clk (dense)
PEAK_FP8_TFLOPS = 5033.2      # 256 CU x 2.4 GHz x 8192 flop/clk (dense)
PEAK_HBM_GBPS = 8000.0

WORKLOADS = {"c2": 2, "c3": 3, "c4": 4, "c5": 5, "c6": 6, "c7": 7, "c8": 8}


def attn_flops(B, H, d, n_keys):
    return 4.0 * B * n_keys * d * H


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("attend.hip", "device_common.h"):
        with open(os.path.join(ROOT, "streaming_block_causal_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload):
    """HBM bytes per attention launch from committed rocprofv3 counter runs, if still current."""
    path = os.path.join(ROOT, "profiles", f"attend_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, sample_heads):
    """Time the fp64 oracle on `sample_heads` heads (all rows) of one steady-state call."""
    from threadpoolctl import threadpool_info

    import oracle.stream as ostream
    n = w.n_sink + w.n_window + 1
    st = ostream.Stream(w)
    q, slots = st.slot_inputs(n, 1)               # warm the input cache (draws are not the oracle)
    t0 = time.perf_counter()
    st.call(n, 1, heads=list(range(sample_heads)))
    dt = time.perf_counter() - t0
    # keys each query sees: every history and current key, plus one source frame when editing
    keys = sum(k.shape[0] for role, _, k, _ in slots if role != "source")
    keys += w.lat_h * w.lat_w if slots[-1][0] == "source" else 0
    flops = attn_flops(q.shape[0], sample_heads, w.head_dim, keys)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
    call_s = dt * w.n_heads / sample_heads          # the whole call (heads are independent)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "nproc": os.cpu_count(),
            "sample": f"one steady-state call (chunk {n}, step 1), {sample_heads} of {w.n_heads} heads, "
                      f"all {q.shape[0]} queries x {keys} keys, fp64 numpy; {dt:.1f} s",
            "seconds": dt, "call_seconds": call_s, "chunk_seconds": call_s * w.n_steps,
            "latent_frames_per_s": w.frames / (call_s * w.n_steps)}


def measured_peak(stream, iters=65536):
    """Sustained matrix-core rate of this device (bf16 and fp8 MFMA chains with register operands,
    the library's probe), best of three launches timed with events on `stream`."""
    import torch

    from streaming_block_causal_amd import native
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(8 * cus, dtype=torch.float32, device="cuda")
    out = {}
    for name, dt in (("bf16", native.SW_BF16), ("fp8", native.SW_FP8)):
        best = None
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            flops = native.sw_probe_mfma(stream.cuda_stream, dt, iters, sink.data_ptr(), sink.numel())
            e1.record(stream)
            e1.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        out[name] = {"tflops": flops / (best * 1e-3) / 1e12, "ms": best,
                     "datasheet_tflops": PEAK_FP8_TFLOPS if name == "fp8" else PEAK_BF16_TFLOPS}
    return out


def run(args, key, stream, flat_chunks, graph, cpu_heads, probe):
    """Time one workload's chunk step on `stream`; returns its JSON record."""
    import torch

    import synth
    from streaming_block_causal_amd.cache import Cache, CacheConfig

    dev = "cuda"
    w = synth.WORKLOADS[WORKLOADS[key]]
    cfg = CacheConfig(n_heads=w.n_heads, head_dim=w.head_dim, frames_per_block=w.frames, lat_h=w.lat_h,
                      lat_w=w.lat_w, n_sink=w.n_sink, n_window=w.n_window, twin=w.twin,
                      sparse=w.sparse_keep is not None, dtype="fp8" if w.attn_fp8 else w.dtype,
                      rope_theta=w.rope_theta,
                      policy=w.policy, editing=w.editing)
    cache = Cache(cfg, device=dev, stream=stream)
    B, H, d, T = w.block_tokens, w.n_heads, w.head_dim, w.n_steps
    shape = (B, H, d)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)

    # per-block lengths: a frame pattern, or an editing stream's reference block
    varlen = w.frame_pattern is not None or w.editing
    hw = w.lat_h * w.lat_w
    frame_counts = sorted({synth.frames_of(w, b) for b in range(64)})

    def draw(frames):
        return (torch.randn((frames * hw, H, d), generator=gen, device=dev, dtype=torch.float32)
                * w.scale).to(torch.bfloat16)

    # two input sets per block length (alternating chunks), resident in HBM before timing
    if args.fused_qkv:
        # packed [B][3][H][d] projection outputs; q/k/v below are views of them (the plain path is
        # unchanged) and the epilogue writes the normalised q into its own buffer
        def packed(f):
            return (torch.randn((f * hw, 3, H, d), generator=gen, device=dev, dtype=torch.float32)
                    * w.scale).to(torch.bfloat16)
        qkv_sets = {f: [[packed(f) for _ in range(T)] for _ in range(2)] for f in frame_counts}
        sets = {f: [[(x[:, 0], x[:, 1], x[:, 2]) for x in qkv_sets[f][i]] for i in range(2)] for f in frame_counts}
        gq = torch.rand(d, generator=gen, device=dev) + 0.5
        gk = torch.rand(d, generator=gen, device=dev) + 0.5
        qn = {f: torch.empty((f * hw, H, d), dtype=torch.bfloat16, device=dev) for f in frame_counts}
    else:
        sets = {f: [[(draw(f), draw(f), draw(f)) for _ in range(T)] for _ in range(2)] for f in frame_counts}
    noisy = {f: [(draw(f), draw(f)) for _ in range(2)] for f in frame_counts}
    source = {f: [(draw(f), draw(f)) for _ in range(2)] for f in frame_counts} if w.editing else None
    outs = {f: torch.empty((f * hw, H, d), dtype=torch.bfloat16, device=dev) for f in frame_counts}
    nt = -(-B // 128)

    def frames_of(b):
        return synth.frames_of(w, b)

    def append_current(k, v, b):
        cache.append("current", k, v, b, n_frames=frames_of(b) if varlen else None)

    n_slots_full = w.n_sink + w.n_window + 1
    state = {"block": 0, "window": 0, "sinks": 0}
    history = []            # frames of the committed blocks the cache holds, logical order

    host_us = {"evict": [], "promote": []}   # host time of the index-remap calls (no device work)

    def commit():
        b = state["block"]
        if state["sinks"] >= w.n_sink and w.n_window > 0 and state["window"] == w.n_window:
            t0 = time.perf_counter()
            cache.evict()
            host_us["evict"].append((time.perf_counter() - t0) * 1e6)
            state["window"] -= 1
            history.pop(state["sinks"])
        t0 = time.perf_counter()
        cache.append("clean", None, None, b)
        host_us["promote"].append((time.perf_counter() - t0) * 1e6)
        if state["sinks"] < w.n_sink:
            state["sinks"] += 1
            history.append(frames_of(b))
        elif w.n_window > 0:
            state["window"] += 1
            history.append(frames_of(b))
        if w.twin:
            kn, vn = noisy[frames_of(b)][b % 2]
            cache.append("noisy", kn, vn, b, n_frames=frames_of(b) if varlen else None)
        state["block"] += 1

    ev = {"attn": [], "append": [], "mask": [], "source": []}
    last_mask = {}

    flops_timed = {"sum": 0.0, "frames": 0}

    def chunk(record):
        b = state["block"]
        fb = frames_of(b)
        out = outs[fb]
        if record:
            # keys per query: history + current block, plus its own source frame when editing
            keys = (sum(history) + fb) * hw + (hw if w.editing else 0)
            flops_timed["sum"] += T * attn_flops(fb * hw, H, d, keys)
            flops_timed["frames"] += fb
        for s in range(T):
            q, k, v = sets[fb][b % 2][s]
            if record:
                e0, e1, es, em, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(5))
                e0.record(stream)
            if args.fused_qkv:
                q = cache.append_qkv(qkv_sets[fb][b % 2][s], gq, gk, 1e-6, b, q_out=qn[fb],
                                     n_frames=fb)
            else:
                append_current(k, v, b)
            if record:
                e1.record(stream)
            if w.editing and s == 0:   # the chunk's source frames, staged once for all its steps
                ks, vs = source[fb][b % 2]
                cache.append("source", ks, vs, b, n_frames=fb)
                if record:
                    ev["source"].append((e1, es))
            if record:
                es.record(stream)
            step = "final" if s == T - 1 else "intermediate"
            if w.sparse_keep is not None:
                idx, k_row = cache.build_tile_mask(q, w.sparse_keep, out=mask_buf["idx"], k_cap=mask_buf["k"],
                                                   step=step)
                last_mask["idx"] = idx
                if record:
                    em.record(stream)
                cache.attend(q, step, tile_idx=idx, k_row=k_row, out=out)
            else:
                if record:
                    em.record(stream)
                cache.attend(q, step, out=out)
            if record:
                e2.record(stream)
                ev["append"].append((e0, e1))
                ev["mask"].append((es, em))
                ev["attn"].append((em, e2))
        commit()

    # fill the cache to steady state (appends and commits only, so every attention launch
    # below -- and in a profiler trace of this script -- has the full key set), then warm up
    while state["block"] < n_slots_full - 1:
        fb0 = frames_of(state["block"])
        q, k, v = sets[fb0][state["block"] % 2][T - 1]
        if args.fused_qkv:
            cache.append_qkv(qkv_sets[fb0][state["block"] % 2][T - 1], gq, gk, 1e-6, state["block"],
                             q_out=qn[fb0], n_frames=fb0)
        else:
            append_current(k, v, state["block"])
        commit()
    mask_buf = {}
    if w.sparse_keep is not None:   # steady-state budget; the buffer is reused (no allocation per call)
        mask_buf["k"] = cache.mask_budget(w.sparse_keep)
        mask_buf["idx"] = torch.empty((H, nt, mask_buf["k"]), dtype=torch.int32, device=dev)
    for _ in range(args.warmup):
        chunk(False)
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for _ in range(args.steps):
        chunk(True)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    if w.sparse_keep is not None:   # the last timed mask (later phases reuse the buffer)
        last_mask["idx"] = mask_buf["idx"].clone()

    # host cost of the cache bookkeeping: evict and promote (index remaps, zero bytes moved) over
    # the warm-up and timed chunks, and a relocation-policy call
    def med(x):
        x = sorted(x)
        return x[len(x) // 2] if x else None
    t0 = time.perf_counter()
    for _ in range(100):
        cache.relocate(w.policy)
    cache_host = {"evict_median": med(host_us["evict"]), "promote_median": med(host_us["promote"]),
                  "relocate_mean": (time.perf_counter() - t0) * 1e4, "calls": len(host_us["evict"]),
                  "bytes_moved": 0}

    flat = None
    if flat_chunks > 0:
        # per-chunk latency over a long steady stream: least-squares slope vs chunk index
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(flat_chunks + 1)]
        marks[0].record(stream)
        for i in range(flat_chunks):
            chunk(False)
            marks[i + 1].record(stream)
        torch.cuda.synchronize()
        lat = [marks[i].elapsed_time(marks[i + 1]) for i in range(flat_chunks)]
        n = len(lat)
        xm, ym = (n - 1) / 2.0, sum(lat) / n
        slope = sum((i - xm) * (y - ym) for i, y in enumerate(lat)) / max(sum((i - xm) ** 2 for i in range(n)), 1e-30)
        flat = {"chunks": n, "first_block": state["block"] - n, "mean_ms": ym,
                "slope_pct_of_mean_per_100_chunks": 100.0 * slope * 100.0 / ym}

    graph_rec = None
    if graph:
        if w.frame_pattern is not None:
            graph_rec = {"skipped": "block lengths follow a pattern: the ring layout does not repeat"}
        else:
            # one recorded chunk per ring phase (the recording only runs host bookkeeping), then
            # replays in turn: the chunk's appends, masks and attention calls of all its steps
            period = cache.ring_period()
            graphs = []
            for _ in range(period):
                cache.graph_begin()
                chunk(False)
                graphs.append(cache.graph_end())
            n_rep = max(args.steps, period)
            for i in range(period):                      # warm-up replays
                graphs[i].launch()
            torch.cuda.synchronize()
            g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            g0.record(stream)
            for i in range(n_rep):
                graphs[i % period].launch()
            g1.record(stream)
            torch.cuda.synchronize()
            ms_graph = g0.elapsed_time(g1) / n_rep
            graph_rec = {"chunks": n_rep, "ring_period": period, "ms_per_step": ms_graph,
                         "eager_ms_per_step": dt / args.steps * 1e3}
            for g in graphs:
                g.close()

    attn_ms = [a.elapsed_time(b) for a, b in ev["attn"]]
    mask_ms = [a.elapsed_time(b) for a, b in ev["mask"]]
    app_ms = [a.elapsed_time(b) for a, b in ev["append"]]
    keys = n_slots_full * B
    if varlen:
        flops_call = flops_timed["sum"] / (T * args.steps)   # mean over the timed calls
    elif w.sparse_keep is None:
        flops_call = attn_flops(B, H, d, keys)
    else:
        # exact kept-tile work of the last mask: sum of valid_q * valid_k over kept tile pairs
        idx = last_mask["idx"].long()
        valid = torch.clamp(B - 128 * torch.arange(nt, device=dev), max=128).double()
        vk = valid[idx % nt]                                   # [H, nt, k_row]
        flops_call = float(4.0 * d * (vk.sum(dim=2) * valid[None, :]).sum().item())
    flops_chunk = flops_timed["sum"] / args.steps if varlen else flops_call * T
    ms_chunk = dt / args.steps * 1e3
    avg_attn = sum(attn_ms) / len(attn_ms)
    avg_mask = sum(mask_ms) / len(mask_ms)
    srt = sorted(attn_ms)
    p50, p95 = srt[len(srt) // 2], srt[min(len(srt) - 1, int(0.95 * len(srt)))]
    achieved = flops_call / (avg_attn * 1e-3) / 1e12
    # plain: read raw K, V + write K, V^T; fused epilogue: read q, k, v + write q, K, V^T (bf16)
    append_bytes = (6 if args.fused_qkv else 4) * B * H * d * 2
    avg_app = sum(app_ms) / len(app_ms)
    peak = PEAK_FP8_TFLOPS if w.attn_fp8 else PEAK_BF16_TFLOPS   # the contraction's own dtype
    res = {
        "metric": "chunk-attention TFLOP/s + latent frames/s (sink+window KV), % of MFMA peak",
        "value": flops_chunk / (ms_chunk * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_chunk,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if w.attn_fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "block_tokens": B, "keys": keys, "heads": H, "head_dim": d,
                   "n_sink": w.n_sink, "n_window": w.n_window, "steps_per_chunk": T,
                   "latent_grid": [w.frames, w.lat_h, w.lat_w],
                   "frame_pattern": list(w.frame_pattern) if w.frame_pattern else None,
                   "editing": {"ref_frames": w.ref_frames, "source_frames": "same instant"} if w.editing else None,
                   "qkv_epilogue": "fused RMSNorm + RoPE + append" if args.fused_qkv else None,
                   "parallelism": "single GPU"},
        "latent_frames_per_s": (flops_timed["frames"] / args.steps if varlen else w.frames) / (ms_chunk * 1e-3),
        "frac_of_bf16_peak_step": flops_chunk / (ms_chunk * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "attention_ms_per_call": avg_attn,
        "attention_ms_p50_p95": [p50, p95],
        "append_ms_per_call": avg_app,
        "append_gbps": append_bytes / (avg_app * 1e-3) / 1e9,
        "latency_flatness": flat,
        "cache_host_us": cache_host,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": load_traffic(key),
                     "kernel": ("attend_fp8_kernel<4>" if w.attn_fp8 else
                                "attend_bf16_kernel<true, 4, false>" if w.sparse_keep else
                                "attend_bf16_kernel<false, 8, true>" if w.editing else "attend_bf16_kernel<false, 8, false>"),
                     "flops_per_launch": flops_call},
    }
    if w.sparse_keep is not None:
        # the mask reads Q once (plus the small pooled-key tables); the sparse attention's
        # compulsory bytes are Q, O and the kept K/V tiles of every query tile
        q_bytes = B * H * d * 2
        idx = last_mask["idx"].long()
        valid = torch.clamp(B - 128 * torch.arange(nt, device=dev), max=128).double()
        kv_bytes = float((valid[idx % nt]).sum().item()) * d * 2 * 2
        res["mask_ms_per_call"] = avg_mask
        res["mask_gbps"] = q_bytes / (avg_mask * 1e-3) / 1e9
        res["attention_ms_per_call_incl_mask"] = avg_attn + avg_mask
        res["sparse_attention_hbm"] = {"bytes": 2 * q_bytes + kv_bytes,
                                       "gbps": (2 * q_bytes + kv_bytes) / (avg_attn * 1e-3) / 1e9,
                                       "frac": (2 * q_bytes + kv_bytes) / (avg_attn * 1e-3) / 1e9 / PEAK_HBM_GBPS}
    if graph_rec is not None:
        if "ms_per_step" in graph_rec:
            graph_rec["value"] = flops_chunk / (graph_rec["ms_per_step"] * 1e-3) / 1e12
        res["graph_replay"] = graph_rec
    if w.editing:
        src_ms = [a.elapsed_time(b) for a, b in ev["source"]]
        res["source_append_ms_per_chunk"] = sum(src_ms) / len(src_ms)
    if probe is not None:
        mp = probe["fp8" if w.attn_fp8 else "bf16"]["tflops"]
        res["roofline"]["measured_peak"] = mp
        res["roofline"]["frac_of_measured_peak"] = achieved / mp
    if cpu_heads < 0:   # about 2.3 TFLOP of oracle work (one whole 540p call)
        cpu_heads = max(1, min(w.n_heads, round(w.n_heads * 2.301e12 / flops_call)))
    if cpu_heads > 0:
        res["cpu_baseline"] = cpu_baseline(w, min(cpu_heads, w.n_heads))
    else:
        res["cpu_baseline"] = None
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed chunks")
    ap.add_argument("--warmup", type=int, default=3, help="untimed chunks")
    ap.add_argument("--workload", default="c4", choices=sorted(WORKLOADS),
                    help="the headline workload (default: the 720p refiner stream, the largest config)")
    ap.add_argument("--also", default=None,
                    help="comma-separated workloads timed after the headline and reported under "
                         "'also' in the same line (default: c2 when the headline is c4; 'none' = skip)")
    ap.add_argument("--cpu-heads", type=int, default=-1,
                    help="heads in the oracle sample (-1 = as many as make about 2.3 TFLOP, i.e. one "
                         "whole 540p call or 10 heads of a 720p call, about 15 s on 16 host threads; "
                         "0 = skip)")
    ap.add_argument("--flat-chunks", type=int, default=200, metavar="N",
                    help="after the timed steps, time N more chunks one by one and report the latency "
                         "slope (headline workload only; 0 = skip)")
    ap.add_argument("--no-probe", action="store_true",
                    help="skip the matrix-core rate probe (measured peak)")
    ap.add_argument("--fused-qkv", action="store_true",
                    help="stage each step from a packed QKV projection output through the fused "
                         "RMSNorm + RoPE + append epilogue (the attention then reads the normalised q)")
    ap.add_argument("--graph", action="store_true",
                    help="after the eager timing, record one chunk graph per ring phase and time their replays")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run device-to-device copies of MIB MiB (scales PMC byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the chunk attention path is single-GPU (its heads are "
              "independent and would shard across GPUs without any exchange).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 3}), flush=True)
        return

    import synth

    torch.cuda.init()
    # a side stream (the NULL stream cannot be recorded into a graph); torch's own work follows it
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    probe = None if args.no_probe else measured_peak(stream)
    res = run(args, args.workload, stream, args.flat_chunks, args.graph, args.cpu_heads, probe)
    also = args.also if args.also is not None else ("c2" if args.workload == "c4" else "none")
    if also != "none":
        res["also"] = {}
        for key in also.split(","):
            r = run(args, key, stream, 0, False, args.cpu_heads, probe)
            res["also"][r["config"]["workload"]] = {
                k: r[k] for k in ("value", "unit", "ms_per_step", "latent_frames_per_s", "attention_ms_per_call",
                                  "attention_ms_p50_p95", "append_ms_per_call", "append_gbps", "dtype")}
            res["also"][r["config"]["workload"]]["roofline"] = r["roofline"]
            res["also"][r["config"]["workload"]]["cpu_baseline"] = r["cpu_baseline"]
    if probe is not None:
        res["measured_peak"] = probe
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
