"""Batched-decode benchmark on one MI355X.

Workload: one Llama-3-8B-shaped attention layer decoding a batch of 32
sequences: H_q=32, H_kv=8, d_h=128, bf16 cache with max_len 4096, per-row
committed lengths drawn uniformly from {1024..4095} (seed 0), T=1.

One step = the whole hot path for one token of every row: truncate the cache
back to its drawn lengths (host bookkeeping), append the step's k/v (append
kernel), attend (split-K decode kernel + combine kernel). Inputs are resident
in HBM before timing starts. Steps rotate over --instances independent caches
(default 4, 2.1 GB of K/V in all) so the 256 MB Infinity Cache cannot hold the
working set between steps.

Prints one JSON line. `value` is the step's algorithmic HBM traffic (K and V of
every visible position, q, the float32 output, and the append's read+write)
divided by the step time. The roofline object times the decode attention
(partial + combine kernels) alone with HIP events on the stream it runs on.

Besides the headline line it reports, under "extra", the chunked-prefill
workload (B=4, 32 chunks of T=512 up to 16384 keys, bf16, MFMA path: TFLOP/s and
% of the bf16 matrix peak) and the long-context decode workload (B=8, H_q=64,
H_kv=8, 32768 cached keys: GB/s for T=1 and T=4 attention calls), and the
tiny decoder (48-token prompt, 160 greedy steps, attention through the C ABI):
wall time of the cached and the uncached generation and their work counters;
the rotary append and query rotation; and latent-cache appends.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]
    python bench.py --pmc-workload c3_attend|c3_step|c5_t1|c5_t4   # for rocprofv3 --pmc
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-attn HBM GB/s (% peak) + tokens/s, GQA 32q/8kv d128 ctx4k B=32"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak, published
PMC_COPY_BYTES = 256 << 20     # calibration copy size for the traffic counters
B, HQ, HKV, D, MAX_LEN = 32, 32, 8, 128, 4096
WORKLOAD = ("batched decode, one Llama-3-8B-shaped layer: B=32, H_q=32, H_kv=8, d_h=128, "
            "bf16 cache max_len 4096, lengths U{1024..4095} seed 0, T=1")


PMC_WORKLOADS_ARG = ("c3_attend", "c3_step", "c5_t1", "c5_t4")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--instances", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU time budget of the oracle sample")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the prefill, long-context and tiny-decoder figures")
    ap.add_argument("--pmc-workload", choices=PMC_WORKLOADS_ARG, default=None,
                    help="run one counter workload (calibration copy, then 40 calls) and exit")
    ap.add_argument("--pmc-prefill", action="store_true",
                    help="run the chunked-prefill workload once (32 chunks) for counter passes and exit")
    return ap.parse_args()


def lengths_seed0() -> np.ndarray:
    from kv_cached_gqa_amd.workloads import batched_lengths
    return batched_lengths(np.random.default_rng(0), B, 1024, MAX_LEN - 1)


def step_bytes(lengths) -> tuple[int, int]:
    from kv_cached_gqa_amd import work
    att = work.attend_bytes(lengths, 1, HQ, HKV, D, "bf16", "bf16")
    app = work.append_bytes(B, HKV, 1, D, "bf16", "bf16")
    return att, app


def make_caches(n_instances, lengths):
    import torch
    from kv_cached_gqa_amd.kvc import KVCache

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    caches = []
    for c in range(n_instances):
        gen.manual_seed(1000 + c)
        cache = KVCache(1, HKV, D, MAX_LEN, batch=B, n_q_heads=HQ, dtype="bf16", device=dev)
        k = torch.randn((B, HKV, MAX_LEN - 1, D), generator=gen, device=dev, dtype=torch.bfloat16)
        v = torch.randn((B, HKV, MAX_LEN - 1, D), generator=gen, device=dev, dtype=torch.bfloat16)
        cache.append(0, k, v)
        del k, v
        cache.truncate(lengths)
        caches.append(cache)
    return caches, gen, dev


def gpu_bench(args, lengths):
    import torch

    caches, gen, dev = make_caches(args.instances, lengths)
    n_in = 8
    gen.manual_seed(7)
    qs = [torch.randn((B, HQ, 1, D), generator=gen, device=dev, dtype=torch.bfloat16) for _ in range(n_in)]
    ks = [torch.randn((B, HKV, 1, D), generator=gen, device=dev, dtype=torch.bfloat16) for _ in range(n_in)]
    vs = [torch.randn((B, HKV, 1, D), generator=gen, device=dev, dtype=torch.bfloat16) for _ in range(n_in)]
    outs = [torch.empty((B, HQ, 1, D), device=dev, dtype=torch.float32) for _ in range(args.instances)]
    torch.cuda.synchronize()

    def step(i):
        # one decode step: roll back to the drawn lengths, append the new token's
        # keys and values, attend (one call: the fused append and attention)
        c = i % args.instances
        cache = caches[c]
        cache.truncate(lengths)
        cache.append_attend(0, ks[i % n_in], vs[i % n_in], qs[i % n_in], out=outs[c])

    def step_two_calls(i):
        c = i % args.instances
        cache = caches[c]
        cache.truncate(lengths)
        cache.append(0, ks[i % n_in], vs[i % n_in])
        cache.attend(0, qs[i % n_in], out=outs[c])

    stream = torch.cuda.current_stream()
    warm_up(step_two_calls, args.warmup)
    ms_step_two = block_times(lambda i: step_two_calls(args.warmup + i), max(50, args.steps), stream)["median"]
    warm_up(step, args.warmup)
    t_wall = time.perf_counter()
    ms_step = event_time(lambda i: step(args.warmup + i), args.steps, stream)     # the timed region: K steps
    wall = time.perf_counter() - t_wall
    blocks = block_times(lambda i: step(args.warmup + args.steps + i), max(50, args.steps), stream)

    # decode attention alone, events on the same stream
    for c in caches:
        c.truncate(lengths)
        c.append(0, ks[0], vs[0])
    warm_up(lambda i: caches[i % args.instances].attend(0, qs[i % n_in], out=outs[i % args.instances]), 0)
    at = block_times(lambda i: caches[i % args.instances].attend(0, qs[i % n_in], out=outs[i % args.instances]),
                     max(50, args.steps), stream)
    for c in caches:
        c.close()
    return ms_step, blocks, at["median"] * 1e3, wall, ms_step_two


# Warm-up by wall time as well as by count: the GPU clocks ramp up from idle
# over the first milliseconds of work.
WARMUP_S = 0.3
# Steps are timed in back-to-back blocks bracketed by two events: an event
# recorded after every step costs ~2.5 us of GPU time per step (measured on the
# batched-decode step: 67.5 us bracketed, 70.2 us with an event per step).
BLOCKS = 5


def warm_up(fn, n, seconds=WARMUP_S):
    """n calls, then more until `seconds` of wall time have passed (the GPU
    clocks ramp up from idle over the first few milliseconds of work, so a
    count alone does not bring them to a steady state), then synchronise."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while i < n or time.perf_counter() - t0 < seconds:
        fn(i)
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def block_times(fn, reps, stream, blocks=BLOCKS) -> dict:
    """`blocks` blocks of `reps` back-to-back calls, each block bracketed by
    two events and synchronised: ms per call of each block, their median,
    minimum and maximum."""
    per = sorted(event_time(lambda i, b=b: fn(b * reps + i), reps, stream) for b in range(blocks))
    return {"median": per[len(per) // 2], "min": per[0], "max": per[-1], "blocks": blocks, "reps": reps}


def pmc_workload(lengths, which: str):
    """What the traffic counters are collected on: a calibration copy of known
    size (PMC_COPY_BYTES read and written), then 40 calls of one workload:
    c3_attend, attention calls of the batched-decode workload over 4 cache
    instances; c3_step, its whole step (truncate, kvc_append_attend); c5_t1 /
    c5_t4, attention calls of the long-context workload at T=1 / T=4."""
    import torch
    src = torch.ones(PMC_COPY_BYTES // 4, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst
    if which.startswith("c3"):
        caches, gen, dev = make_caches(4, lengths)
        kv = torch.randn((B, HKV, 1, D), generator=gen, device=dev, dtype=torch.bfloat16)
        q = torch.randn((B, HQ, 1, D), generator=gen, device=dev, dtype=torch.bfloat16)
        out = torch.empty((B, HQ, 1, D), device=dev, dtype=torch.float32)
        if which == "c3_attend":
            for c in caches:
                c.append(0, kv, kv)
            for i in range(40):
                caches[i % 4].attend(0, q, out=out)
        else:
            for i in range(40):
                caches[i % 4].truncate(lengths)
                caches[i % 4].append_attend(0, kv, kv, q, out=out)
    else:
        t = 1 if which == "c5_t1" else 4
        cache, q, out = long_ctx_cache(t)
        for _ in range(40):
            cache.attend(0, q, out=out)
    torch.cuda.synchronize()


def event_time(fn, reps, stream):
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def call_time_us(fn, reps, stream) -> float:
    """Median over `reps` calls of fn's time on the GPU, each call bracketed by
    its own events and synchronised (the launch latency included), for calls
    too small to time back to back: a queued loop of them is bound by the
    host and its timing depends on what the process ran before."""
    import torch
    times = []
    for i in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    times.sort()
    return times[len(times) // 2]


def new_cache(n_kv_heads, d_head, max_len, batch, n_q_heads, dev, block=None):
    """A bf16 cache of one layer, contiguous or paged (blocks of `block`)."""
    from kv_cached_gqa_amd.kvc import KVCache, PagedKVCache
    if block is None:
        return KVCache(1, n_kv_heads, d_head, max_len, batch=batch, n_q_heads=n_q_heads, dtype="bf16", device=dev)
    return PagedKVCache(1, n_kv_heads, d_head, max_len, batch=batch, n_q_heads=n_q_heads, dtype="bf16", device=dev,
                        block_size=block)


def prefill_bench(block=None, runs=3, precision="rounded"):
    """Chunked prefill: B=4, H_q=32, H_kv=8, d_h=128, bf16, 32 chunks of T=512
    appended and attended in turn (queries at s = 0, 512, ..., 15872); on a
    paged cache with blocks of `block` positions when given; `precision` is the
    cache's prefill precision (kvc_set_prefill_precision)."""
    import torch
    from kv_cached_gqa_amd import work
    b, hq, hkv, d, t, nch = 4, 32, 8, 128, 512, 32
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    cache = new_cache(hkv, d, t * nch, b, hq, dev, block)
    cache.set_prefill_precision(precision)
    ks = [torch.randn((b, hkv, t, d), generator=gen, device=dev, dtype=torch.bfloat16) for _ in range(4)]
    vs = [torch.randn((b, hkv, t, d), generator=gen, device=dev, dtype=torch.bfloat16) for _ in range(4)]
    qs = [torch.randn((b, hq, t, d), generator=gen, device=dev, dtype=torch.bfloat16) for _ in range(4)]
    out = torch.empty((b, hq, t, d), device=dev, dtype=torch.float32)

    def run(_):
        cache.truncate(0)
        for c in range(nch):
            cache.append(0, ks[c % 4], vs[c % 4])
            cache.attend(0, qs[c % 4], out=out)
    run(0)
    torch.cuda.synchronize()
    ms = event_time(run, runs, torch.cuda.current_stream()) if runs > 1 else float("nan")
    flops = sum(work.attend_flops([c * t] * b, t, hq, d) for c in range(nch))
    tf = flops / (ms * 1e-3) / 1e12
    cache.close()
    return {"workload": "chunked prefill: B=4, H_q=32, H_kv=8, d_h=128, bf16, 32 chunks of T=512 (append + attend "
                        "each), keys up to 16384",
            "ms_per_run": round(ms, 4), "tflops": round(tf, 1), "pct_peak_bf16_mfma": round(100 * tf / PEAK_BF16_TFLOPS, 2),
            "flops_per_run": flops}


def tiny_decoder_bench():
    """The random-weight decoder of "kv-cache-decoding" (vocab 96, width 128,
    4 heads, 4 layers; 48-token prompt, 160 greedy steps) on the GPU, attention
    through the C ABI with an fp32 cache: wall time of the cached and of the
    uncached generation (one warm-up run of each first) and their work
    counters."""
    import torch
    from kv_cached_gqa_amd.decoder import GpuDecoder, greedy_cached, greedy_uncached
    from kv_cached_gqa_amd.workloads import DecoderShape, decoder_params, decoder_prompt
    shape = DecoderShape()
    model = GpuDecoder(decoder_params(0, shape), shape)
    prompt, n_new = decoder_prompt(1, 48, shape), 160
    res = {"workload": "random-weight decoder: vocab 96, width 128, 4 heads, 4 layers, fp32 cache; "
                       "48-token prompt, 160 greedy steps"}
    for name, run in (("cached", lambda: greedy_cached(model, prompt, n_new)),
                      ("uncached", lambda: greedy_uncached(model, prompt, n_new))):
        out = run()
        if name == "cached":
            out[2].close()
        torch.cuda.synchronize()
        model.scores_computed = model.positions_processed = 0
        t0 = time.perf_counter()
        out = run()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        if name == "cached":
            out[2].close()
        res[name] = {"ms": round(dt * 1e3, 2), "tokens_per_s": round(n_new / dt, 1),
                     "attention_scores": model.scores_computed, "positions": model.positions_processed,
                     "ids": out[0]}
    res["same_ids"] = res["cached"].pop("ids") == res["uncached"].pop("ids")
    res["speedup"] = round(res["uncached"]["ms"] / res["cached"]["ms"], 2)
    model.close()
    return res


def rope_bench():
    """The batched-decode step's append (B=32, H_kv=8, d_h=128, bf16, T=1, rows
    at 2000 positions) with the keys rotated (kvc_append_rope) against the
    plain append, and the rotation of the step's queries (kvc_rope_q, H_q=32):
    microseconds per call (median of 50 synchronised calls, launch included)."""
    import torch
    from kv_cached_gqa_amd.kvc import KVCache
    b, hq, hkv, d = 32, 32, 8, 128
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(17)
    cache = KVCache(1, hkv, d, 2048, batch=b, n_q_heads=hq, dtype="bf16", device=dev)
    k = torch.randn((b, hkv, 2000, d), generator=gen, device=dev, dtype=torch.bfloat16)
    cache.append(0, k, k)
    del k
    kv = torch.randn((b, hkv, 1, d), generator=gen, device=dev, dtype=torch.bfloat16)
    q = torch.randn((b, hq, 1, d), generator=gen, device=dev, dtype=torch.bfloat16)
    st = torch.cuda.current_stream()
    res = {"workload": "append of one decode step, B=32, H_kv=8, d_h=128, bf16, positions 2000"}

    def step(rope):
        cache.append(0, kv, kv, rope_base=500000.0 if rope else None)
        cache.truncate(2000)

    for name, fn in (("append_us", lambda i: step(False)), ("append_rope_us", lambda i: step(True)),
                     ("rope_q_us", lambda i: cache.rope_q(0, q, 500000.0))):
        if name == "rope_q_us":
            cache.append(0, kv, kv)              # the chunk the queries belong to
        for i in range(10):
            fn(i)
        res[name] = round(call_time_us(fn, 50, st), 2)
    cache.close()
    return res


def latent_bench():
    """Latent-cache appends (B=32, r=512, d_R=64, bf16): one decode step (T=1)
    and one prefill chunk (T=512), microseconds per call (median of 50
    synchronised calls, launch included)."""
    import torch
    from kv_cached_gqa_amd.kvc import LatentCache
    b, r, dr = 32, 512, 64
    dev = torch.device("cuda:0")
    lc = LatentCache(1, r, dr, 1024, batch=b, dtype="bf16", device=dev)
    st = torch.cuda.current_stream()
    res = {"workload": "latent cache append, B=32, r=512, d_R=64, bf16"}
    for t in (1, 512):
        c = torch.randn((b, t, r), device=dev, dtype=torch.bfloat16)
        kr = torch.randn((b, t, dr), device=dev, dtype=torch.bfloat16)

        def step(i):
            lc.append(0, c, kr)
            lc.truncate(0)

        for i in range(10):
            step(i)
        us = call_time_us(step, 50, st)
        moved = 2 * b * t * (r + dr) * 2           # read + write, bf16 in and out
        res[f"T{t}"] = {"us": round(us, 2), "gbs": round(moved / (us * 1e-6) / 1e9, 1)}
    lc.close()
    return res


def paged_bench(lengths, us_contiguous: float):
    """The batched-decode workload on paged caches (blocks of 128 and 256
    positions): each cache grows one block per row per append, so a row's
    blocks are interleaved with every other row's in the pool, as decode
    growth leaves them; then the rows are cut to the drawn lengths, which
    gives the blocks past each length back. One attention call (T=1) per
    repetition over 4 rotating instances, HIP events on the stream; the held
    pool bytes against the contiguous cache's 2 B H_kv max_len d_h itemsize."""
    import torch
    from kv_cached_gqa_amd.kvc import PagedKVCache
    from kv_cached_gqa_amd import work
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(17)
    att = work.attend_bytes(lengths, 1, HQ, HKV, D, "bf16", "bf16")
    contiguous_bytes = 2 * B * HKV * MAX_LEN * D * 2
    res = {"workload": WORKLOAD + ", paged", "contiguous_us_per_attend": round(us_contiguous, 2)}
    st = torch.cuda.current_stream()
    for bs in (128, 256):
        caches = []
        for c in range(4):
            pc = PagedKVCache(1, HKV, D, MAX_LEN, batch=B, n_q_heads=HQ, dtype="bf16", device=dev, block_size=bs)
            chunk = torch.randn((B, HKV, bs, D), generator=gen, device=dev, dtype=torch.bfloat16)
            while int(pc.seq_len()[0]) < MAX_LEN - 1:
                t = min(bs, MAX_LEN - 1 - int(pc.seq_len()[0]))
                part = chunk if t == bs else chunk[:, :, :t].contiguous()
                pc.append(0, part, part)
            del chunk, part
            pc.truncate(lengths)
            kv = torch.randn((B, HKV, 1, D), generator=gen, device=dev, dtype=torch.bfloat16)
            pc.append(0, kv, kv)
            caches.append(pc)
        q = torch.randn((B, HQ, 1, D), generator=gen, device=dev, dtype=torch.bfloat16)
        out = torch.empty((B, HQ, 1, D), device=dev, dtype=torch.float32)
        for i in range(8):
            caches[i % 4].attend(0, q, out=out)
        ms = event_time(lambda i: caches[i % 4].attend(0, q, out=out), 200, st)
        used, _ = caches[0].blocks()
        held = 2 * used * HKV * bs * D * 2
        gbs = att / (ms * 1e-3) / 1e9
        res[f"block{bs}"] = {"us_per_attend": round(ms * 1e3, 2), "gbs": round(gbs, 1),
                             "pct_peak_hbm": round(100 * gbs / PEAK_HBM_GBS, 2),
                             "vs_contiguous": round(us_contiguous / (ms * 1e3), 3),
                             "held_bytes": held, "held_vs_contiguous": round(held / contiguous_bytes, 3)}
        for pc in caches:
            pc.close()
        torch.cuda.synchronize()
    # the matrix-core paths on paged storage: long-context decode (8 and 32
    # query rows per KV head) and chunked prefill, blocks of 128
    res["long_context_decode_block128"] = long_ctx_bench(128)
    pf = prefill_bench(128)
    res["chunked_prefill_block128"] = {k: pf[k] for k in ("ms_per_run", "tflops", "pct_peak_bf16_mfma")}
    return res


def small_configs_bench():
    """The latency-bound configs, decode tokens/s: the tiny GQA cache (L=4,
    B=1, H_q=4, H_kv=2, d_h=32, fp32; a 16-token prefill, then 112 decode
    steps) and the SmolLM2-shaped cache (L=30, B=1, H_q=9, H_kv=3, d_h=64,
    fp16; a 512-token prefill, then 256 decode steps), inputs from their call
    scripts moved to the device first. A decode step is every layer's
    kvc_append_attend; the steps run once untimed, the cache is cut back to
    the prefill, and the second run is timed with HIP events."""
    import torch
    from kv_cached_gqa_amd.kvc import KVCache, torch_dtype
    from kv_cached_gqa_amd import workloads as W
    dev = torch.device("cuda:0")
    res = {}
    for name, (shape, calls) in (("tiny_gqa_fp32", W.script_tiny_gqa()),
                                 ("smollm2_135m_fp16", W.script_smollm2(rollback=0))):
        tdt = torch_dtype(shape.dtype)
        to = lambda x: torch.from_numpy(x).to(dev, tdt)  # noqa: E731
        prefill, decode = [], []
        for c in calls:
            if c.op == "pass":
                (prefill if c.tag == "prefill" else decode).append((c.layer, to(c.k), to(c.v), to(c.q)))
        cache = KVCache(shape.n_layers, shape.n_kv_heads, shape.d_head, shape.max_len, batch=shape.batch,
                        n_q_heads=shape.n_q_heads, dtype=shape.dtype, device=dev)
        out = torch.empty_like(decode[0][3], dtype=torch.float32)
        for layer, k, v, q in prefill:
            cache.append_attend(layer, k, v, q)
        p0 = int(cache.seq_len()[0])
        n_steps = len(decode) // shape.n_layers

        def run(_):
            for layer, k, v, q in decode:
                cache.append_attend(layer, k, v, q, out=out)
        run(0)
        cache.truncate(p0)
        torch.cuda.synchronize()
        ms = event_time(run, 1, torch.cuda.current_stream())
        res[name] = {"layers": shape.n_layers, "decode_steps": n_steps, "ms": round(ms, 3),
                     "tokens_per_s": round(n_steps * shape.batch / (ms * 1e-3), 1),
                     "us_per_layer_call": round(ms * 1e3 / len(decode), 2)}
        cache.close()
    return res


def long_ctx_cache(t, block=None, seed=13):
    """The long-context workload (B=8, H_q=64, H_kv=8, d_h=128, bf16, 32768
    cached keys) with a chunk of t positions appended: (cache, q, out)."""
    import torch
    b, hq, hkv, d, s0, ml = 8, 64, 8, 128, 32768, 32776
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    cache = new_cache(hkv, d, ml, b, hq, dev, block)
    for _ in range(4):
        k = torch.randn((b, hkv, s0 // 4, d), generator=gen, device=dev, dtype=torch.bfloat16)
        cache.append(0, k, k)
        del k
    kv = torch.randn((b, hkv, t, d), generator=gen, device=dev, dtype=torch.bfloat16)
    cache.append(0, kv, kv)
    q = torch.randn((b, hq, t, d), generator=gen, device=dev, dtype=torch.bfloat16)
    out = torch.empty((b, hq, t, d), device=dev, dtype=torch.float32)
    return cache, q, out


def long_ctx_bench(block=None):
    """Long-context decode: B=8, H_q=64, H_kv=8, d_h=128, bf16, 32768 cached keys;
    attention calls with T=1 and T=4 (a draft block) after one append, each
    timed over 20 back-to-back calls after a warm-up; on a paged cache with
    blocks of `block` positions when given."""
    import torch
    from kv_cached_gqa_amd import work
    b, hq, hkv, d, s0 = 8, 64, 8, 128, 32768
    res = {"workload": "long-context decode: B=8, H_q=64, H_kv=8, d_h=128, bf16, 32768 cached keys"}
    for t in (1, 4):
        cache, q, out = long_ctx_cache(t, block)
        warm_up(lambda i: cache.attend(0, q, out=out), 3)
        ms = block_times(lambda i: cache.attend(0, q, out=out), 20, torch.cuda.current_stream())["median"]
        byt = work.attend_bytes([s0] * b, t, hq, hkv, d, "bf16", "bf16")
        res[f"T{t}"] = {"us_per_attend": round(ms * 1e3, 2), "gbs": round(byt / (ms * 1e-3) / 1e9, 1),
                        "pct_peak_hbm": round(100 * byt / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)}
        cache.close()
    return res


def cpu_baseline(lengths, seconds: float, threads=1) -> dict:
    """The oracle, as it stands, on the same workload: whole steps (truncate,
    append, attend of all 32 rows) until `seconds` of CPU time are spent, with
    BLAS limited to `threads` threads (None: all cores). The preload is not
    timed."""
    from threadpoolctl import threadpool_limits
    from oracle import OracleCache
    from kv_cached_gqa_amd.workloads import draw_kv, draw_qkv, SHAPES

    shape = SHAPES["llama3_8b_layer_decode_bf16"]
    oc = OracleCache(1, B, HQ, HKV, D, MAX_LEN, "bf16")
    rng = np.random.default_rng(0)
    rng.integers(1024, MAX_LEN, size=B)          # the lengths draw (already known)
    k, v = draw_kv(rng, shape, MAX_LEN - 1)
    oc.append(0, k, v)
    del k, v
    oc.truncate(lengths)
    inputs = [draw_qkv(rng, shape, 1) for _ in range(4)]
    att, app = step_bytes(lengths)
    steps = 0
    with threadpool_limits(limits=threads):
        t0 = time.perf_counter()
        while True:
            q, k, v = inputs[steps % len(inputs)]
            oc.truncate(lengths)
            oc.append(0, k, v)
            oc.attend(0, q)
            steps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    t_step = el / steps
    cores = 1 if threads == 1 else (os.cpu_count() or 1)
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round((att + app) / t_step / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "host": {"cpu_model": model, "logical_cpus": os.cpu_count()},
            "sample": f"{steps} whole decode steps of the same workload (all 32 rows), float64 NumPy, "
                      f"{cores} BLAS thread(s), {el:.1f} s",
            "tokens_per_s": round(B / t_step, 2), "s_per_step": round(t_step, 4)}


def oracle_config_timings(budget_s: float = 8.0) -> dict:
    """The oracle, as it stands, on the other configurations' call scripts,
    all BLAS threads, each bounded to about `budget_s` seconds of timed calls
    (the set-up and input draws are not timed): seconds, calls timed, tokens/s
    (query positions per second) or TFLOP/s, and effective GB/s (the same
    algorithmic bytes the GPU figures use, divided by the oracle's time)."""
    from threadpoolctl import threadpool_info
    from oracle import OracleCache
    from kv_cached_gqa_amd import work
    from kv_cached_gqa_amd import workloads as W
    threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)

    def timed_script(shape, calls, timed_tag, stop_after=None):
        orc = OracleCache(shape.n_layers, shape.batch, shape.n_q_heads, shape.n_kv_heads, shape.d_head,
                          shape.max_len, shape.dtype)
        el, n_calls, queries, byt, flops = 0.0, 0, 0, 0, 0
        for call in calls:
            timed = call.op != "truncate" and timed_tag(call)
            t0 = time.perf_counter()
            if call.op in ("append", "pass"):
                orc.append(call.layer, call.k, call.v)
            if call.op == "pass":
                orc.attend(call.layer, call.q)
            if call.op == "truncate":
                orc.truncate(call.n)
            dt = time.perf_counter() - t0
            if timed and call.op == "pass":
                el += dt
                n_calls += 1
                offs = orc.seq_len(call.layer) - call.T
                if call.layer == shape.n_layers - 1:
                    queries += shape.batch * call.T
                byt += (work.attend_bytes(offs, call.T, shape.n_q_heads, shape.n_kv_heads, shape.d_head,
                                          shape.dtype, "fp32")
                        + work.append_bytes(shape.batch, shape.n_kv_heads, call.T, shape.d_head, "fp32", shape.dtype))
                flops += work.attend_flops(offs, call.T, shape.n_q_heads, shape.d_head)
                if el >= budget_s or (stop_after is not None and n_calls >= stop_after):
                    break
        return {"seconds": round(el, 3), "calls_timed": n_calls, "tokens_per_s": round(queries / el, 2),
                "gbs": round(byt / el / 1e9, 3), "tflops": round(flops / el / 1e12, 4)}

    res = {"cores": threads, "kind": "oracle",
           "method": "float64 NumPy oracle on the configuration's own call script; timed: the pass "
                     "calls named in each entry (append + attend), until the budget"}
    shape, calls = W.script_tiny_gqa()
    r = timed_script(shape, calls, lambda c: c.tag != "prefill")
    res["tiny_gqa_fp32"] = {"sample": f"decode passes (T=1, 4 layers) of the 112-step script: {r['calls_timed']} calls",
                            **r}
    shape, calls = W.script_smollm2(rollback=0)
    r = timed_script(shape, calls, lambda c: c.tag != "prefill")
    res["smollm2_135m_fp16"] = {"sample": f"decode passes (T=1, 30 layers, after the 512-token prefill): "
                                          f"{r['calls_timed']} calls", **r}
    shape, calls = W.script_chunked_prefill()
    r = timed_script(shape, calls, lambda c: True)
    res["chunked_prefill_bf16"] = {"sample": f"the first {r['calls_timed']} chunks of T=512 (keys up to "
                                             f"{512 * r['calls_timed']}), all rows", **r}
    shape, calls = W.script_long_ctx_spec(n_cycles=1)
    r = timed_script(shape, calls, lambda c: c.op == "pass")
    res["long_ctx_spec_bf16"] = {"sample": f"one speculative cycle after the 32768-key preload: "
                                           f"{r['calls_timed']} passes (a T=4 draft, then T=1 steps), all rows",
                                 **r}
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the path shards by (row, KV head) with no exchange, so no multi-GPU figure is produced.",
              file=sys.stderr)
        sys.exit(2)
    lengths = lengths_seed0()
    if args.pmc_workload:
        pmc_workload(lengths, args.pmc_workload)
        return
    if args.pmc_prefill:
        prefill_bench(runs=1)
        return
    att, app = step_bytes(lengths)
    ms_step, blocks, us_attend, wall, ms_step_two = gpu_bench(args, lengths)
    from kv_cached_gqa_amd.measure import stored_traffic
    traffic = stored_traffic()
    gbs = (att + app) / (ms_step * 1e-3) / 1e9
    att_gbs = att / (us_attend * 1e-6) / 1e9
    rec = {
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
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "batch": B, "n_q_heads": HQ, "n_kv_heads": HKV, "d_head": D,
                   "max_len": MAX_LEN, "T": 1, "cache_instances": args.instances,
                   "mean_context": float(np.mean(lengths) + 1)},
        "tokens_per_s": round(B / (ms_step * 1e-3), 1),
        "step": "truncate to the drawn lengths, then kvc_append_attend (append and attention in one call)",
        "timing": {"ms_per_step": f"{args.steps} back-to-back steps between two events, after {args.warmup} "
                                  f"warm-up steps and at least {WARMUP_S:.1f} s of warm-up",
                   "blocks_median_ms": round(blocks["median"], 5), "blocks_min_ms": round(blocks["min"], 5),
                   "blocks_max_ms": round(blocks["max"], 5),
                   "blocks": f"{blocks['blocks']} further blocks of {blocks['reps']} steps, each between two events"},
        "ms_per_step_append_then_attend": round(ms_step_two, 5),
        "pct_peak_hbm": round(100 * gbs / PEAK_HBM_GBS, 2),
        "bytes_per_step": att + app,
        "roofline": {"bound": "hbm", "kernel": "decode attention: decode_mfma + decode_combine",
                     "achieved": round(att_gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(att_gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": att, "launch_us": round(us_attend, 3)},
    }
    if not args.no_extra:
        pf_split = prefill_bench(precision="split")
        rec["extra"] = {"chunked_prefill": prefill_bench(),
                        "chunked_prefill_split_p": {"precision": "P as a hi + lo pair (kvc_set_prefill_precision)",
                                                    **{k: pf_split[k] for k in ("ms_per_run", "tflops",
                                                                                "pct_peak_bf16_mfma")}},
                        "long_context_decode": long_ctx_bench(),
                        "tiny_decoder": tiny_decoder_bench(), "rope": rope_bench(),
                        "latent_cache": latent_bench(), "paged_decode": paged_bench(lengths, us_attend),
                        "small_configs": small_configs_bench()}
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(lengths, args.cpu_seconds)
        rec["cpu_baseline"]["all_cores"] = cpu_baseline(lengths, args.cpu_seconds / 2, threads=None)
        rec["cpu_baseline"]["other_configs"] = oracle_config_timings()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
