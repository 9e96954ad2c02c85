#!/usr/bin/env python3
"""Benchmark of the latent-cache chunk-attention hot path on one MI355X.

One step = one chunk-layer at the Wan2.1-1.3B shape (batch 1, 30x52 latent grid,
3-frame query chunk = 4680 tokens, 21-frame window = 32760 keys, 12 heads,
d_c = 192, d_rope = 32, bf16 storage, fp32 accumulation):
  vmla_cache_append     down-projection + 3D-RoPE + ring write of the chunk
  vmla_query_prologue   absorbed, pre-scaled queries
  vmla_latent_attention scores vs the latent window, online softmax, P.c, W_V_up
All inputs are seeded synthetic tensors already resident in HBM when the timed
region starts. Prints one JSON line on stdout.

`--config 3` and `--config 4` time the batch-8 (30 layers, one buffer set per
layer) and batch-16 single-frame workloads instead; their buffers rotate so the
append and the query prologue read HBM, not the 256 MB Infinity Cache, and
their bulk inputs are device-generated N(0,1) tensors (values do not change the
work).

`--long-horizon` (config 2 only) keeps one sink frame plus a 6-frame window
with k_R rotated at read time; `--layer` runs the whole attention layer instead
of the attention core: the d_q = 768 query latent, the latent attention, and
the output mixer W_O with B_h folded in (out [B, N_q, d_model]).

`--chunk-causal` times the whole-clip form instead: the 21 latent frames of a
Wan-1.3B clip (32,760 tokens) appended, every token a query, 3-frame chunks
under the chunk-causal block mask (with `--explicit`: through explicit per-head
K/V of the whole clip).

`--config 5` times the minute-scale rollout at B=8 (80 chunks x 4 denoising steps
x 30 layers over a 21-frame ring) as one step-layer per distinct window length,
weighted by how often the rollout runs it.

The default run also times the append at the batch-8 shape on cold buffers
(`append_cold`, the HBM-graded figure) and reports the attention kernel's
algorithmic GB/s next to its TFLOP/s.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--config 2|3|4|5]
                       [--long-horizon] [--layer] [--explicit] [--d-c 64|128|192] [--chunk-causal]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "latent-cache MLA chunk attention TFLOP/s + ms/chunk-layer (Wan-1.3B shape)"
PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def work(w, layer=False, explicit=False):
    """Algorithmic flops and bytes of one step (absorbed method, bf16 storage).
    ``layer``: the whole layer instead, with the d_q query latent (x W_DQ, then
    the folded [A_h | W_UQ^rope[h]]) and B_h folded into the output mixer."""
    H, Nq, Nk, D = w.n_heads, w.n_q * w.batch, w.n_k, w.d_model
    B = w.batch
    per_qkh = 2 * (w.d_c + w.d_rope) + 2 * w.d_c                # 832
    core = per_qkh * w.n_q * Nk * H * B
    prologue = Nq * (2 * D * H * w.d_head + H * 2 * w.d_nope * w.d_c)
    epilogue = Nq * H * 2 * w.d_c * w.d_v
    append = Nq * 2 * D * w.cache_row
    row = 2 * w.cache_row
    bytes_append = Nq * D * 2 + D * w.cache_row * 2 + Nq * row
    bytes_prologue = Nq * D * 2 + D * H * w.d_head * 2 + H * w.d_c * w.d_nope * 2 + Nq * H * row
    bytes_attn = Nq * H * row + B * Nk * row + H * w.d_c * w.d_v * 2 + Nq * H * w.d_v * 2
    if layer:
        prologue = Nq * (2 * D * w.d_q + 2 * w.d_q * H * w.cache_row)
        epilogue = Nq * 2 * H * w.d_c * D                            # [O_lat / l] x W_VO
    if explicit:
        # queries x W_Q; per-head K/V rebuilt from every valid slot; 2 (128 + 128)
        # flops per (query, key, head)
        prologue = Nq * 2 * D * H * w.d_head + B * Nk * 2 * w.d_c * H * (w.d_nope + w.d_v)
        core = 2 * (w.d_head + w.d_v) * w.n_q * Nk * H * B
        epilogue = 0
    return dict(core=core, prologue=prologue, epilogue=epilogue, append=append,
                attn_kernel=core + epilogue, step=core + prologue + epilogue + append,
                bytes_append=bytes_append, bytes_prologue=bytes_prologue, bytes_attn=bytes_attn)


def clip_work(w, n_frames, window, explicit=False, rows=None):
    """Algorithmic flops of the whole-clip chunk-causal form: every token of
    frames 0 .. n_frames - 1 is a query; chunk c (w.chunk_frames frames) sees
    the frames [max(0, e - window), e), e its end. ``rows``: restrict the
    query-side work to these chunk indices (the append stays whole)."""
    T, H, D, B = w.tokens_per_frame, w.n_heads, w.d_model, w.batch
    C = w.chunk_frames
    n_chunks = -(-n_frames // C)
    per_pair = 2 * (w.d_head + w.d_v) if explicit else 2 * (w.d_c + w.d_rope) + 2 * w.d_c
    core = nq = 0
    for c in range(n_chunks) if rows is None else rows:
        e = min((c + 1) * C, n_frames)
        q = (e - c * C) * T
        core += per_pair * q * (e - max(0, e - window)) * T * H * B
        nq += q * B
    if explicit:
        prologue = nq * 2 * D * H * w.d_head + B * n_frames * T * 2 * w.d_c * H * (w.d_nope + w.d_v)
        epilogue = 0
    else:
        prologue = nq * (2 * D * H * w.d_head + H * 2 * w.d_nope * w.d_c)
        epilogue = nq * H * 2 * w.d_c * w.d_v
    append = B * n_frames * T * 2 * D * w.cache_row
    bytes_append = B * n_frames * T * (D * 2 + 2 * w.cache_row) + D * w.cache_row * 2
    return dict(core=core, prologue=prologue, epilogue=epilogue, append=append,
                attn_kernel=core + epilogue, step=core + prologue + epilogue + append,
                bytes_append=bytes_append)


def measured_mfma_peak():
    """Sustained dense bf16 MFMA rate of this GPU in TFLOP/s: the best of six
    launches of the register-only matrix-core probe (libvmla_probe.so), timed
    with HIP events on the current stream. The measured second reference line
    of the roofline, next to the published peak."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "latent_kv_attention_cache_amd", "libvmla_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m latent_kv_attention_cache_amd.build`")
    lib = ctypes.CDLL(path)
    lib.vmla_probe_sink_floats.restype = ctypes.c_int64
    lib.vmla_probe_mfma_flops.argtypes = [ctypes.c_int32]
    lib.vmla_probe_mfma_flops.restype = ctypes.c_double
    lib.vmla_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    lib.vmla_probe_mfma_bf16.restype = ctypes.c_int32
    sink = torch.empty(lib.vmla_probe_sink_floats(), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    iters = 20000                              # ~4-5 ms per launch
    best = 0.0
    for _ in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        st = lib.vmla_probe_mfma_bf16(ctypes.c_void_p(sink.data_ptr()), iters,
                                      ctypes.c_void_p(stream.cuda_stream))
        e1.record(stream)
        torch.cuda.synchronize()
        if st != 0:
            raise RuntimeError(f"peak probe launch failed ({st})")
        best = max(best, lib.vmla_probe_mfma_flops(iters) / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return best


def measured_hbm_read():
    """Sustained HBM read bandwidth of this GPU in GB/s: the best of five
    launches of the stream probe (libvmla_probe.so) over a 2 GiB buffer, far
    larger than the 256 MB Infinity Cache."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "latent_kv_attention_cache_amd", "libvmla_probe.so"))
    lib.vmla_probe_read_sink_words.restype = ctypes.c_int64
    lib.vmla_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.vmla_probe_hbm_read.restype = ctypes.c_int32
    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(lib.vmla_probe_read_sink_words(), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    best = 0.0
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        st = lib.vmla_probe_hbm_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                     ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
        e1.record(stream)
        torch.cuda.synchronize()
        if st != 0:
            raise RuntimeError(f"HBM probe launch failed ({st})")
        best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf, sink
    return best


def cpu_baseline(w, wts, x_host, step_flops, mix=None):
    """Time the CPU fp64 oracle on the whole step: every query token of the
    chunk, all heads, the full key window (its explicit per-head K/V build
    included). About 10-30 s on a 16-core host."""
    import numpy as np
    import oracle.vmla_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    if mix is not None:
        orc.chunk_layer_reference(w, wts, mix, x_host, np.arange(w.n_q))
    else:
        ref = orc.chunk_attention_reindexed_reference if w.rope_at_read else orc.chunk_attention_reference
        ref(w, wts, x_host, np.arange(w.n_q))
    full_s = time.perf_counter() - t0
    log(f"[cpu_baseline] oracle on the full step: {full_s:.2f} s")
    return {
        "value": step_flops / full_s / 1e12, "unit": "TFLOP/s", "cores": int(threads),
        "kind": "oracle", "ms_per_step": full_s * 1e3,
        "sample": (f"the whole step: numpy fp64 oracle (explicit per-head K/V) on all {w.n_q} "
                   f"query tokens and {w.n_heads} heads over the full {w.n_k}-key window, its "
                   f"cache build included; {full_s:.1f} s wall on the host, rated with the "
                   f"step's algorithmic flops"),
    }


def _threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        return len(os.sched_getaffinity(0))


def cpu_baseline_sampled(w, rows=512):
    """The oracle on a bounded sample of a batch-B step: one batch element of
    one layer (seeded host inputs), its cache window built, then ``rows`` of
    the chunk's query rows over the full window. Rows are independent, so the
    step time is extrapolated linearly: B x (window build + N_q / rows x the
    rows' time); the rate is the sample's own algorithmic flops over its time."""
    import numpy as np
    import oracle.vmla_oracle as orc
    from workloads import weights, x_frame
    wts = weights(w)
    xs = {t: x_frame(w, t) for t in range(w.t_first + w.chunk_frames - min(w.window_frames, w.t_first + w.chunk_frames),
                                           w.t_first + w.chunk_frames)}
    idx = np.linspace(0, w.n_q - 1, rows).astype(np.int64)
    t0 = time.perf_counter()
    orc.chunk_attention_reference(w, wts, lambda t: xs[t], idx[:1])
    t_build = time.perf_counter() - t0
    t0 = time.perf_counter()
    orc.chunk_attention_reference(w, wts, lambda t: xs[t], idx)
    t_all = time.perf_counter() - t0
    t_rows = max(t_all - t_build, 1e-9)
    per_q = 2 * (w.d_c + w.d_rope) * w.n_k * w.n_heads + 2 * w.n_heads * w.d_c * w.d_v + \
        2 * w.d_model * w.n_heads * w.d_head + w.n_heads * 2 * w.d_nope * w.d_c
    step_s = w.batch * (t_build + t_rows * w.n_q / rows)
    log(f"[cpu_baseline] oracle sample: window build {t_build:.2f} s, {rows} rows {t_rows:.2f} s; "
        f"extrapolated step {step_s:.1f} s")
    return {
        "value": rows * per_q / t_all / 1e12, "unit": "TFLOP/s", "cores": int(_threads()),
        "kind": "oracle", "ms_per_step": step_s * 1e3, "extrapolated": True,
        "sample": (f"one batch element of one layer: numpy fp64 oracle (explicit per-head K/V) "
                   f"building its {w.n_k}-key window ({t_build:.1f} s), then {rows} of the "
                   f"chunk's {w.n_q} query rows over it ({t_rows:.1f} s); rate = the sample's "
                   f"algorithmic flops / its time; ms_per_step extrapolated linearly to "
                   f"{w.batch} elements x {w.n_q} rows"),
    }


def _noise_sets(w, dims, n_sets, dev, seed, layer=False):
    """Device-noise buffer sets (x, weights, cache) for the batched workloads:
    values do not change the work, and one set per layer keeps the append and
    the prologue reading HBM rather than the Infinity Cache."""
    import torch
    import latent_kv_attention_cache_amd as vm
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    shapes = {"w_q": (w.d_model, w.n_heads * w.d_head), "w_down": (w.d_model, w.d_c),
              "w_kr": (w.d_model, w.d_rope), "w_k_up": (w.n_heads, w.d_c, w.d_nope),
              "w_v_up": (w.n_heads, w.d_c, w.d_v)}
    if layer:
        shapes.update({"w_dq": (w.d_model, w.d_q), "w_uq": (w.d_q, w.n_heads * w.d_head),
                       "w_o": (w.n_heads * w.d_v, w.d_model)})
    sets = []
    for _ in range(n_sets):
        dw = {k: (torch.randn(shp, generator=g, device=dev) * shp[-2] ** -0.5).to(torch.bfloat16)
              for k, shp in shapes.items()}
        cache = vm.LatentCache.empty(w.batch, w.window_frames, w.grid_h, w.grid_w, device=dev, dims=dims)
        cache.data.normal_(generator=g)
        x = torch.randn((w.batch, w.n_q, w.d_model), generator=g, device=dev).to(torch.bfloat16)
        sets.append((x, dw, cache))
    return sets


def append_cold(dev, reps=60):
    """The append at the batch-8 chunk shape (8 x 4680 tokens, 132.5 MB of
    algorithmic traffic) on 30 rotating buffer sets (7 GB, far beyond the 256 MB
    Infinity Cache), timed with one pair of HIP events on the launch stream
    around 60 back-to-back launches (each on the next buffer set): the
    HBM-graded append figure, the average launch duration."""
    import torch
    import latent_kv_attention_cache_amd as vm
    from workloads import config
    w = config(3)
    dims = vm.default_dims()
    sets = _noise_sets(w, dims, w.n_layers, dev, seed=33)
    stream = torch.cuda.current_stream()
    for i in range(10):
        x, dw, cache = sets[i % len(sets)]
        vm.vmla_cache_append(cache, x, dw["w_down"], dw["w_kr"], w.t_first, w.chunk_frames, dims=dims)
    # one event pair over the back-to-back launches: the average launch
    # duration, with no event packets between the kernels
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        x, dw, cache = sets[i % len(sets)]
        vm.vmla_cache_append(cache, x, dw["w_down"], dw["w_kr"], w.t_first, w.chunk_frames, dims=dims)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    nbytes = work(w)["bytes_append"]
    del sets
    torch.cuda.empty_cache()
    gbs = nbytes / (us * 1e-6) / 1e9
    log(f"[bench] cold append (B=8, 4680 tokens, 30 buffer sets): {us:.1f} us = {gbs:.0f} GB/s")
    return {"workload": "append at the batch-8 chunk shape: 8 x 4680 tokens, 30 rotating buffer sets "
                        "(7 GB, cold: not served by the Infinity Cache)",
            "bound": "hbm", "us": round(us, 2), "bytes_per_launch": nbytes, "achieved": round(gbs, 1),
            "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps first; the shader clock needs tens of ms of load to settle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--config", type=int, default=2, choices=(2, 3, 4, 5),
                    help="2: Wan-1.3B chunk-layer at B=1 (the reported workload); 3: B=8, 30 "
                         "layers; 4: B=16, one-frame chunk; 5: the minute-scale rollout at B=8 "
                         "(80 chunks x 4 steps x 30 layers, as a weighted sum over its window lengths)")
    ap.add_argument("--long-horizon", action="store_true",
                    help="with --config 2: the long-rollout cache instead of the 21-frame window -- "
                         "one sink frame plus a 6-frame window, k_R cached before RoPE and "
                         "rotated in the active context, chunk at t = 18..20 after evictions")
    ap.add_argument("--layer", action="store_true",
                    help="the whole attention layer: d_q = 768 query latent, latent attention, "
                         "B_h folded into the W_O output mixer (out [B, N_q, d_model])")
    ap.add_argument("--explicit", action="store_true",
                    help="the explicit-reconstruction route instead of the latent form: per-head "
                         "K/V rebuilt from the cache each step, then 128-dim attention")
    ap.add_argument("--d-c", type=int, default=192, choices=(64, 128, 192, 256, 512),
                    help="content-latent width of the cache (the latent-budget sweep); the "
                         "--layer and --explicit routes run at 192 only")
    ap.add_argument("--split", type=int, default=32, choices=(16, 32, 64, 96), metavar="D_ROPE",
                    help="NoPE/RoPE split of the 128-wide head: positional width 16, 32 (the "
                         "default 96/32), 64 or 96, at d_c = 192")
    ap.add_argument("--chunk-causal", action="store_true",
                    help="the whole-clip form: 21 latent frames, every token a query, 3-frame "
                         "chunks under the chunk-causal block mask")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run a plain device-to-device copy of MIB MiB, whose counter "
                         "readings calibrate FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the chunk-attention hot path runs on a single "
              "MI355X; run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import latent_kv_attention_cache_amd as vm
    from workloads import config, mixer_weights, weights, x_frame

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    vm.load_library()
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: {nbytes} bytes read and {nbytes} bytes written")
        del src, dst
    if args.config == 5:
        if args.chunk_causal or args.long_horizon or args.layer or args.explicit or args.d_c != 192 \
                or args.split != 32:
            print("--config 5 runs the attention core at the default widths", file=sys.stderr)
            sys.exit(2)
        return rollout_bench(args, dev)
    if args.chunk_causal:
        if args.config != 2 or args.long_horizon or args.layer or args.d_c != 192 or args.split != 32:
            print("--chunk-causal runs the Wan-1.3B clip at B=1 (config 2 shapes), with or without "
                  "--explicit", file=sys.stderr)
            sys.exit(2)
        return clip_bench(args, dev)
    w = config(args.config)
    if args.long_horizon:
        if args.config != 2:
            print("--long-horizon applies to --config 2", file=sys.stderr)
            sys.exit(2)
        w = w.with_(window_frames=6, sink_frames=1, rope_at_read=True,
                    name=w.name + ", sink 1 + window 6, read-time RoPE")
    if args.d_c != 192:
        if args.layer or args.explicit:
            print("--d-c applies to the attention core (not --layer / --explicit)", file=sys.stderr)
            sys.exit(2)
        w = w.with_(d_c=args.d_c, name=w.name + f", d_c = {args.d_c}")
    if args.split != 32:
        if args.layer or args.long_horizon or args.d_c != 192:
            print("--split runs the attention core or --explicit at d_c = 192 with k_R rotated at "
                  "append", file=sys.stderr)
            sys.exit(2)
        from workloads import split_variant
        w = split_variant(w, args.split).with_(
            name=w.name + f", NoPE/RoPE split {128 - args.split}/{args.split}")
    log(f"[bench] workload: {w.name}")
    dims = vm.default_dims(d_c=w.d_c, d_nope=w.d_nope, d_rope=w.d_rope, rope_pairs=w.rope_pairs,
                           rope_axis_dims=w.rope_axis_dims)
    xs = None
    if args.config == 2:
        # seeded host inputs, the same as the parity tests use
        wts = weights(w)
        xs = {t: x_frame(w, t) for t in w.prior_frames + w.chunk_frame_ids}
        dw = {k: torch.from_numpy(v).to(dev).to(torch.bfloat16) for k, v in wts.items()}
        mix = mixer_weights(w) if args.layer else None
        if args.layer:
            dw.update({k: torch.from_numpy(v).to(dev).to(torch.bfloat16) for k, v in mix.items()})

        def xdev(frames):
            return torch.from_numpy(np.concatenate([xs[t] for t in frames]))[None].to(dev).to(torch.bfloat16)

        cache = vm.LatentCache.empty(w.batch, w.window_frames, w.grid_h, w.grid_w, device=dev,
                                     dims=dims, sink_frames=w.sink_frames, rope_at_read=w.rope_at_read)
        prior = w.prior_frames
        i = 0
        while i < len(prior):       # contiguous runs of earlier frames
            j = i
            while j + 1 < len(prior) and prior[j + 1] == prior[j] + 1:
                j += 1
            vm.vmla_cache_append(cache, xdev(prior[i:j + 1]), dw["w_down"], dw["w_kr"], prior[i],
                                 j + 1 - i, dims=dims)
            i = j + 1
        sets = [(xdev(list(w.chunk_frame_ids)).contiguous(), dw, cache)]
    else:
        # one buffer set per layer (config 3) or eight rotating sets (config 4)
        n_sets = w.n_layers if w.n_layers > 1 else 8
        sets = _noise_sets(w, dims, n_sets, dev, seed=w.cfg_id, layer=args.layer)
        log(f"[bench] {n_sets} buffer sets of "
            f"{(sets[0][0].numel() + sets[0][2].data.numel()) * 2 / 1e6:.0f} MB")
    n_valid = w.n_valid_frames
    if args.explicit:
        if args.layer or args.long_horizon:
            print("--explicit runs the attention core with k_R rotated at append", file=sys.stderr)
            sys.exit(2)
        for _, dw, _ in sets:
            dw["w_kv"] = vm.vmla_pack_kv_weights(dw["w_k_up"], dw["w_v_up"], dims=dims)
    if args.layer:
        # the one-time weight folds of the layer (not part of a step)
        for _, dw, _ in sets:
            dw["w_qa"] = vm.vmla_fold_query_weights(dw["w_uq"], dw["w_k_up"], w.d_q, dims=dims)
            dw["w_vo"] = vm.vmla_fold_output_weights(dw["w_v_up"], dw["w_o"], dims=dims)
        ws = torch.empty(vm.vmla_layer_workspace_bytes(w.batch, w.n_q, w.d_q, dims), dtype=torch.uint8,
                         device=dev)
        out = torch.empty((w.batch, w.n_q, w.d_model), dtype=torch.bfloat16, device=dev)
    elif args.explicit:
        ws = torch.empty(vm.vmla_explicit_workspace_bytes(w.batch, w.n_q, w.n_k, dims),
                         dtype=torch.uint8, device=dev)
        out = torch.empty((w.batch, w.n_q, w.n_heads, w.d_v), dtype=torch.bfloat16, device=dev)
    else:
        ws = torch.empty(vm.vmla_attention_workspace_bytes(w.batch, w.n_q, dims), dtype=torch.uint8,
                         device=dev)
        out = torch.empty((w.batch, w.n_q, w.n_heads, w.d_v), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def step(ev=None, i=0):
        x, dw, cache = sets[i % len(sets)]
        if ev is not None:
            ev[0].record(stream)
        vm.vmla_cache_append(cache, x, dw["w_down"], dw["w_kr"], w.t_first, w.chunk_frames, dims=dims)
        if ev is not None:
            ev[1].record(stream)
        if args.layer:
            vm.vmla_layer_query_prologue(cache, x, dw["w_dq"], dw["w_qa"], w.t_first, w.chunk_frames,
                                         n_valid, ws, dims=dims)
        elif args.explicit:
            pass                      # the explicit call below builds its own queries
        else:
            vm.vmla_query_prologue(cache, x, dw["w_q"], dw["w_k_up"], w.t_first, w.chunk_frames,
                                   n_valid, ws, dims=dims)
        if ev is not None:
            ev[2].record(stream)
        if args.layer:
            vm.vmla_layer_attention(cache, w.d_q, dw["w_vo"], w.t_first, w.chunk_frames, n_valid, out,
                                    ws, dims=dims)
        elif args.explicit:
            vm.vmla_chunk_attention_explicit(cache, x, dw["w_q"], dw["w_kv"], w.t_first, w.chunk_frames,
                                             n_valid, out, ws, dims=dims)
        else:
            vm.vmla_latent_attention(cache, dw["w_v_up"], w.t_first, w.chunk_frames, n_valid, out, ws,
                                     dims=dims)
        if ev is not None:
            ev[3].record(stream)

    for i in range(args.warmup):
        step(i=i)
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i], i=i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    k_ms = {"append": 0.0, "query_prologue": 0.0, "latent_attn": 0.0}
    for ev in events:
        k_ms["append"] += ev[0].elapsed_time(ev[1])
        k_ms["query_prologue"] += ev[1].elapsed_time(ev[2])
        k_ms["latent_attn"] += ev[2].elapsed_time(ev[3])
    k_ms = {k: v / args.steps for k, v in k_ms.items()}
    assert torch.isfinite(out.float()).all().item(), "non-finite output"

    wk = work(w, layer=args.layer, explicit=args.explicit)
    tflops = wk["step"] / (ms_step * 1e-3) / 1e12
    attn_tflops = wk["attn_kernel"] / (k_ms["latent_attn"] * 1e-3) / 1e12
    append_gbs = wk["bytes_append"] / (k_ms["append"] * 1e-3) / 1e9
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "latent_attn_config2_traffic.json")
    if (args.config == 2 and not (args.long_horizon or args.layer or args.explicit)
            and args.d_c == 192 and args.split == 32 and os.path.exists(tfile)):
        with open(tfile) as f:
            tr = json.load(f)
        if tr.get("kernel_source_sha") == _kernel_sha():
            traffic = tr.get("bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": {2: "Wan-1.3B-shaped chunk-layer: B=1, 30x52 grid, 3-frame query chunk over "
                            "a 21-frame latent window",
                         3: "Wan-1.3B-shaped chunk-layer at B=8, 30 layers with their own weights, "
                            "inputs and caches, one layer per step",
                         4: "single-frame chunk at B=16: 1560 query tokens per element over a "
                            "21-frame latent window"}[args.config],
            "batch": w.batch, "n_q": w.n_q, "n_k": w.n_k, "n_heads": w.n_heads, "d_model": w.d_model,
            "d_c": w.d_c, "d_rope": w.d_rope, "d_nope": w.d_nope, "d_v": w.d_v,
            "flops_per_step": wk["step"],
        },
        "kernels_ms": {k: round(v, 4) for k, v in k_ms.items()},
        "roofline": {
            "bound": "mfma",
            "kernel": "latent_attn",
            "achieved": round(attn_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "flops_per_launch": wk["attn_kernel"],
            # algorithmic bytes (Qhat, the window's cache rows, W_V_up, out) per
            # launch over its time, next to the 8 TB/s of HBM
            "bytes_per_launch": wk["bytes_attn"],
            "gbs": round(wk["bytes_attn"] / (k_ms["latent_attn"] * 1e-3) / 1e9, 1),
            "gbs_frac_of_hbm": round(wk["bytes_attn"] / (k_ms["latent_attn"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        },
        "append_roofline": {
            "bound": "hbm", "achieved": round(append_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(append_gbs / PEAK_HBM_GBS, 4), "bytes_per_launch": wk["bytes_append"],
        },
    }
    log(f"[bench] ms/step {ms_step:.4f}  kernels {k_ms}  attention {attn_tflops:.1f} TFLOP/s")
    _add_measured_peak(result["roofline"], result["append_roofline"])
    if args.config == 2 and not (args.long_horizon or args.layer or args.explicit) and args.d_c == 192 \
            and args.split == 32:
        # the HBM-graded append figure: the batch-8 shape on cold buffers, timed
        # while the GPU is still under load and before the CPU baseline occupies
        # the host
        ac = append_cold(dev)
        ac["measured_peak"] = result["append_roofline"]["measured_peak"]
        ac["frac_of_measured_peak"] = round(ac["achieved"] / ac["measured_peak"], 4)
        result["append_cold"] = ac
    if not args.no_cpu_baseline and args.config == 2:
        xh = lambda t: xs[t]  # noqa: E731
        result["cpu_baseline"] = cpu_baseline(w, wts, xh, wk["step"], mix)
    elif not args.no_cpu_baseline and args.config in (3, 4) and not (args.layer or args.explicit) \
            and args.d_c == 192 and args.split == 32:
        result["cpu_baseline"] = cpu_baseline_sampled(w)
    if args.long_horizon:
        result["config"]["workload"] = ("Wan-1.3B-shaped chunk-layer, long rollout: B=1, 30x52 "
                                        "grid, 3-frame query chunk at t=18..20 over one sink frame "
                                        "plus a 6-frame window, RoPE applied at read time")
    if args.d_c != 192:
        result["config"]["workload"] += f"; content latent d_c = {args.d_c} (latent-budget sweep)"
    if args.split != 32:
        result["config"]["workload"] += (f"; NoPE/RoPE split {128 - args.split}/{args.split}, "
                                         f"rope pairs {tuple(w.rope_pairs)}")
    if args.explicit:
        result["config"]["workload"] += ("; explicit route: per-head K/V rebuilt from the latent "
                                         "cache each step (201 MB at B=1), then 128-dim attention")
        result["kernels_ms"] = {"append": round(k_ms["append"], 4),
                                "explicit_route": round(k_ms["latent_attn"], 4)}
        result["roofline"]["kernel"] = "explicit route (query GEMM + K/V rebuild GEMM + attention)"
        result["roofline"]["flops_per_launch"] = wk["prologue"] + wk["core"]
        et = (wk["prologue"] + wk["core"]) / (k_ms["latent_attn"] * 1e-3) / 1e12
        result["roofline"]["achieved"] = round(et, 2)
        result["roofline"]["frac"] = round(et / PEAK_BF16_TFLOPS, 4)
        result["roofline"]["frac_of_measured_peak"] = round(et / result["roofline"]["measured_peak"], 4)
        result["absorbed_flops_per_step"] = work(w)["step"]
    if args.layer:
        result["config"]["workload"] += ("; whole attention layer: d_q=768 query latent, latent "
                                         "attention, B_h folded into the W_O output mixer")
        result["config"]["d_q"] = w.d_q
        result["kernels_ms"]["layer_attention"] = result["kernels_ms"].pop("latent_attn")
        result["roofline"]["kernel"] = "latent_attn (folded epilogue) + output-mixer GEMM"
        result["config"]["sink_frames"] = w.sink_frames
        result["config"]["window_frames"] = w.window_frames
    print(json.dumps(result), flush=True)


def rollout_bench(args, dev):
    """The minute-scale rollout (B=8): 240 latent frames in 80 chunks of 3, each
    chunk re-appended and attended at each of 4 denoising steps in each of 30
    layers, over a 21-frame ring (t continues to 239). A step-layer's work
    depends only on its window length, min(3k + 3, 21) frames for chunk k, so
    one step-layer (append + query prologue + attention) is timed at each
    distinct length on 30 rotating layer buffer sets, and the rollout total is
    the sum over the 80 chunks x 4 steps x 30 layers of the matching times."""
    import torch

    import latent_kv_attention_cache_amd as vm
    from workloads import config

    w5 = config(5)
    dims = vm.default_dims()
    log(f"[bench] workload: {w5.name}")
    per_chunk = w5.n_steps * w5.n_layers
    nf_of = [min(w5.chunk_frames * (k + 1), w5.window_frames) for k in range(w5.n_chunks)]
    distinct = sorted(set(nf_of))
    sets = _noise_sets(w5.with_(t_first=18), dims, w5.n_layers, dev, seed=5)
    ws = torch.empty(vm.vmla_attention_workspace_bytes(w5.batch, w5.n_q, dims), dtype=torch.uint8, device=dev)
    out = torch.empty((w5.batch, w5.n_q, w5.n_heads, w5.d_v), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    rows, tot_s, tot_fl, attn_s, attn_fl, app_s = [], 0.0, 0, 0.0, 0, 0.0
    for nf in distinct:
        # the last chunk with this window length: t_first = 3k, the ring wrapped for nf = 21
        k = max(i for i, v in enumerate(nf_of) if v == nf)
        w = w5.with_(t_first=w5.chunk_frames * k)
        n_valid = w.n_valid_frames
        assert n_valid == nf

        def step(i, ev=None):
            x, dw, cache = sets[i % len(sets)]
            if ev is not None:
                ev[0].record(stream)
            vm.vmla_cache_append(cache, x, dw["w_down"], dw["w_kr"], w.t_first, w.chunk_frames, dims=dims)
            if ev is not None:
                ev[1].record(stream)
            vm.vmla_query_prologue(cache, x, dw["w_q"], dw["w_k_up"], w.t_first, w.chunk_frames, n_valid, ws,
                                   dims=dims)
            if ev is not None:
                ev[2].record(stream)
            vm.vmla_latent_attention(cache, dw["w_v_up"], w.t_first, w.chunk_frames, n_valid, out, ws,
                                     dims=dims)
            if ev is not None:
                ev[3].record(stream)

        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i, evs[i])
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        km = [sum(e[j].elapsed_time(e[j + 1]) for e in evs) / args.steps for j in range(3)]
        wk = work(w)
        n = nf_of.count(nf) * per_chunk
        tot_s += n * ms * 1e-3
        tot_fl += n * wk["step"]
        attn_s += n * km[2] * 1e-3
        attn_fl += n * wk["attn_kernel"]
        app_s += n * km[0] * 1e-3
        rows.append({"window_frames": nf, "n_k": w.n_k, "chunks": nf_of.count(nf), "step_layers": n,
                     "ms_per_step_layer": round(ms, 4), "append_us": round(km[0] * 1e3, 2),
                     "query_prologue_us": round(km[1] * 1e3, 2), "latent_attn_ms": round(km[2], 4),
                     "latent_attn_tflops": round(wk["attn_kernel"] / (km[2] * 1e-3) / 1e12, 1)})
        log(f"[bench] window {nf} frames: {ms:.3f} ms per step-layer, attention {km[2]:.3f} ms "
            f"({rows[-1]['latent_attn_tflops']} TFLOP/s) x {n} step-layers")
    assert torch.isfinite(out.float()).all().item(), "non-finite output"
    n_total = w5.n_chunks * per_chunk
    achieved = attn_fl / attn_s / 1e12
    result = {
        "metric": METRIC, "value": round(tot_fl / tot_s / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(tot_s * 1e3 / n_total, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": ("minute-scale streaming rollout at B=8: 240 latent frames of 30x52 in 80 "
                                "3-frame chunks, each appended and attended at 4 denoising steps in 30 "
                                "layers over a 21-frame ring; one step-layer timed per window length, "
                                "the total weighted by the rollout's counts"),
                   "batch": w5.batch, "n_q": w5.n_q, "n_chunks": w5.n_chunks, "n_steps": w5.n_steps,
                   "n_layers": w5.n_layers, "window_frames": w5.window_frames, "d_c": w5.d_c,
                   "d_rope": w5.d_rope, "step_layers": n_total, "flops_total": tot_fl},
        "rollout": {"total_s": round(tot_s, 3), "attention_s": round(attn_s, 3), "append_s": round(app_s, 4),
                    "by_window": rows},
        "roofline": {"bound": "mfma", "kernel": "latent_attn (flop-weighted over the rollout)",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "flops_per_launch": None},
    }
    log(f"[bench] rollout: {tot_s:.2f} s in all ({attn_s:.2f} s of attention at {achieved:.1f} TFLOP/s)")
    _add_measured_peak(result["roofline"])
    print(json.dumps(result), flush=True)


def clip_bench(args, dev):
    """The whole-clip chunk-causal form: append all frames, query prologue over
    the clip, chunk-causal attention (or the explicit route). One step = one
    forward of the clip through the attention of one layer."""
    import numpy as np
    import torch

    import latent_kv_attention_cache_amd as vm
    from workloads import config, weights, x_frame

    F, W = 21, 21
    w = config(2).with_(window_frames=F, chunk_frames=3, t_first=0,
                        name="Wan-1.3B clip, B=1, 21 frames of 30x52, 3-frame chunks, chunk-causal mask")
    log(f"[bench] workload: {w.name}")
    dims = vm.default_dims()
    wts = weights(w)
    xs = {t: x_frame(w, t) for t in range(F)}
    dw = {k: torch.from_numpy(v).to(dev).to(torch.bfloat16) for k, v in wts.items()}
    x = torch.from_numpy(np.concatenate([xs[t] for t in range(F)]))[None].to(dev).to(torch.bfloat16)
    cache = vm.LatentCache.empty(1, F, w.grid_h, w.grid_w, device=dev, dims=dims)
    n_q = F * w.tokens_per_frame
    out = torch.empty((1, n_q, w.n_heads, w.d_v), dtype=torch.bfloat16, device=dev)
    if args.explicit:
        dw["w_kv"] = vm.vmla_pack_kv_weights(dw["w_k_up"], dw["w_v_up"], dims=dims)
        ws = torch.empty(vm.vmla_explicit_workspace_bytes(1, n_q, n_q, dims), dtype=torch.uint8,
                         device=dev)
    else:
        ws = torch.empty(vm.vmla_attention_workspace_bytes(1, n_q, dims), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        vm.vmla_cache_append(cache, x, dw["w_down"], dw["w_kr"], 0, F, dims=dims)
        if ev is not None:
            ev[1].record(stream)
        if not args.explicit:
            vm.vmla_query_prologue(cache, x, dw["w_q"], dw["w_k_up"], 0, F, F, ws, dims=dims)
        if ev is not None:
            ev[2].record(stream)
        if args.explicit:
            vm.vmla_chunk_causal_attention_explicit(cache, x, dw["w_q"], dw["w_kv"], F, w.chunk_frames,
                                                    W, out, ws, dims=dims)
        else:
            vm.vmla_chunk_causal_latent_attention(cache, dw["w_v_up"], F, w.chunk_frames, W, out, ws,
                                                  dims=dims)
        if ev is not None:
            ev[3].record(stream)

    steps, warmup = max(1, args.steps // 5), max(1, args.warmup // 5)   # a clip is ~5 chunk steps
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    k_ms = [sum(ev[j].elapsed_time(ev[j + 1]) for ev in events) / steps for j in range(3)]
    assert torch.isfinite(out.float()).all().item(), "non-finite output"

    wk = clip_work(w, F, W, explicit=args.explicit)
    tflops = wk["step"] / (ms_step * 1e-3) / 1e12
    if args.explicit:
        kflops, kname = wk["prologue"] + wk["core"], "explicit route (query GEMM + K/V rebuild + attention)"
        kms = {"append": k_ms[0], "explicit_route": k_ms[2]}
    else:
        kflops, kname = wk["attn_kernel"], "latent_attn (chunk-causal instance)"
        kms = {"append": k_ms[0], "query_prologue": k_ms[1], "latent_attn": k_ms[2]}
    ach = kflops / (k_ms[2] * 1e-3) / 1e12
    append_gbs = wk["bytes_append"] / (k_ms[0] * 1e-3) / 1e9
    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {
            "workload": ("Wan-1.3B clip through one attention layer: B=1, 21 latent frames of "
                         "30x52 tokens, every token a query, 3-frame chunks under the chunk-causal "
                         "block mask (window = the clip)"
                         + ("; explicit route: per-head K/V of the whole clip rebuilt, then "
                            "128-dim attention" if args.explicit else "")),
            "batch": 1, "n_q": n_q, "n_k": n_q, "n_frames": F, "chunk_frames": w.chunk_frames,
            "mask_window_frames": W, "n_heads": w.n_heads, "d_model": w.d_model, "d_c": w.d_c,
            "d_rope": w.d_rope, "d_nope": w.d_nope, "d_v": w.d_v, "flops_per_step": wk["step"],
        },
        "kernels_ms": {k: round(v, 4) for k, v in kms.items()},
        "roofline": {"bound": "mfma", "kernel": kname, "achieved": round(ach, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "flops_per_launch": kflops},
        "append_roofline": {"bound": "hbm", "achieved": round(append_gbs, 1), "peak": PEAK_HBM_GBS,
                            "unit": "GB/s", "frac": round(append_gbs / PEAK_HBM_GBS, 4),
                            "bytes_per_launch": wk["bytes_append"]},
    }
    if args.explicit:
        result["absorbed_flops_per_step"] = clip_work(w, F, W)["step"]
    log(f"[bench] ms/step {ms_step:.4f}  kernels {kms}  {kname} {ach:.1f} TFLOP/s")
    _add_measured_peak(result["roofline"], result["append_roofline"])
    if not args.no_cpu_baseline:
        # bounded sample: the oracle on the last chunk's 4680 queries (each sees
        # the whole clip), with the whole clip's cache build
        import oracle.vmla_oracle as orc
        n_chunks = -(-F // w.chunk_frames)
        c = n_chunks - 1
        T = w.tokens_per_frame
        rows = np.arange(c * w.chunk_frames * T, F * T)
        t0 = time.perf_counter()
        orc.clip_chunk_causal_reference(w, wts, lambda t: xs[t], F, W, rows)
        sec = time.perf_counter() - t0
        fl = clip_work(w, F, W, rows=[c])["step"]
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:  # pragma: no cover
            threads = len(os.sched_getaffinity(0))
        log(f"[cpu_baseline] oracle on the last chunk: {sec:.2f} s")
        result["cpu_baseline"] = {
            "value": fl / sec / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"the last chunk's {len(rows)} queries (each attends to all {F * T} keys of "
                       f"the clip) through the numpy fp64 oracle, the whole clip's cache build "
                       f"included; {sec:.1f} s wall on the host, rated with that sample's "
                       f"algorithmic flops"),
        }
    print(json.dumps(result), flush=True)


def _add_measured_peak(roof, append_roof=None):
    peak = measured_mfma_peak()
    log(f"[bench] measured MFMA peak {peak:.1f} TFLOP/s")
    roof["measured_peak"] = round(peak, 1)
    roof["frac_of_measured_peak"] = round(roof["achieved"] / peak, 4)
    if append_roof is not None:
        bw = measured_hbm_read()
        log(f"[bench] measured HBM read {bw:.1f} GB/s")
        append_roof["measured_peak"] = round(bw, 1)
        append_roof["frac_of_measured_peak"] = round(append_roof["achieved"] / bw, 4)


def _kernel_sha():
    import hashlib
    h = hashlib.sha256()
    for f in ("latent_attn.hip", "device_common.h", "kernels.h"):
        with open(os.path.join(ROOT, "latent_kv_attention_cache_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
