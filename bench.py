#!/usr/bin/env python3
"""Throughput of the MI355X decoder block on its synthetic workloads.

Default (N=1): the 70B-shaped GQA block (dim 8192, 64 query / 8 kv heads, ffn
28672), causal prefill of 4 x 1024 tokens in bf16 -- the largest single-block
workload -- reported as prefill TFLOP/s with the roofline of its dominant
kernel; its decode counterpart (64 sequences against 4096-token caches) as
tokens/s with its HBM roofline; and, as extra keys, the 7B-shaped prefill
(1 x 2048), the 13B-shaped decode (16 x 4096), the tiny fp32 block, and the
40-layer 4-bit 13B stack (512-token prompt pass, greedy, sampled and no-cache
steps).  Beside them: the matrix-core and copy rates measured on this part, and
the CPU oracle timed on this host on bounded samples of every workload.  Prints
ONE JSON line on stdout.

A step is one llama_block_prefill (or llama_block_decode) call over the whole
batch, inputs resident in HBM.  Phase times come from HIP events recorded by
the library on the stream it launches on (llama_block_profile_*).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decoder-block prefill TFLOP/s + decode tokens/s; % MFMA / HBM roofline"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PREFILL_PHASES = ["rms_x", "qkv_gemm_rope_append", "attention_prefill", "wo_gemm_residual_h_stats",
                  "w13_gemm_swiglu", "w2_gemm_residual"]
DECODE_PHASES = ["qkv_gemv_and_x_stats", "qkv_finish_rope_append", "attention_decode", "wo_gemv",
                 "wo_residual_h_stats", "w13_gemv_swiglu", "w2_gemv", "w2_residual"]

HEADLINE = "gqa70b_block_prefill_b4_l1024"
DECODE = "gqa70b_block_decode_b64_kv4096"
EXTRA_PREFILL = "llama7b_block_prefill_b1_l2048"
EXTRA_DECODE = "llama13b_block_decode_b16_kv4096"
TINY = "tiny_f32_d256_prefill32_decode8"
STACK = "q4_llama13b_stack40_prompt512_greedy128"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _setup(wl, max_seq, n_layers, inp=None):
    import torch
    import workloads as W
    import decoder_block_rmsnorm_amd as L
    from tests import gpu_util as G
    t0 = time.time()
    if inp is None:
        inp = W.draw_block_workload(wl)
        log(f"[bench] {wl.name}: inputs drawn in {time.time() - t0:.1f}s")
    s = wl.shape
    blk, wd = G.make_block(s, inp["weights"], max_seq)
    del wd
    cache = L.KVCache(n_layers, wl.batch, max_seq, s.n_kv_heads, s.head_dim, dtype=G.act_code(s.dtype))
    torch.cuda.synchronize()
    return inp, blk, cache


def _traffic_bytes(kernel):
    t = recorded_traffic(kernel)
    return None if t is None else t["bytes"]


def _phase_table(names, ph_ms, ncalls, extra=None):
    out = {}
    for i, (name, ms) in enumerate(zip(names, ph_ms)):
        out[name] = {"avg_us": round(ms / max(ncalls, 1) * 1e3, 2)}
        if extra:
            out[name].update(extra(i, ms / max(ncalls, 1)))
    return out


def bench_prefill(wl, steps, warmup, inp=None):
    """Prefill: the timed region is `steps` back-to-back calls bracketed by two
    events; the dominant kernel (the w1/w3 GEMM) is timed inside it by events
    attached to its own launches.  The per-phase breakdown comes from a separate
    untimed pass with an event at every phase boundary."""
    import torch
    import workloads as W
    from tests import gpu_util as G
    s, B, Lq = wl.shape, wl.batch, wl.seq_len
    # one cache layer per call so that every call starts from an empty cache
    inp, blk, cache = _setup(wl, Lq, warmup + 2 * steps, inp)
    sc = G.scratch(blk, B * Lq, B, Lq)
    x = G.tdev(inp["x"].reshape(B * Lq, s.dim), s.dtype)
    y = torch.empty_like(x)
    layer = 0
    for _ in range(warmup):
        blk.prefill(cache, layer, x, y, B, Lq, sc)
        layer += 1
    flops = W.prefill_flops(s, B, Lq)
    lin = W.linear_flops(s, B * Lq)
    attn_flops = flops - sum(lin.values())
    ph_flops = [0.0, lin["qkv"], attn_flops, lin["wo"], lin["w13"], lin["w2"]]
    assert len(ph_flops) == len(PREFILL_PHASES)
    # breakdown pass
    torch.cuda.synchronize()
    blk.profile_start(steps)
    for _ in range(steps):
        blk.prefill(cache, layer, x, y, B, Lq, sc)
        layer += 1
    ph_ms, ncalls = blk.profile_read()

    def tf(i, avg_ms):
        return {"tflops": round(ph_flops[i] / (avg_ms * 1e-3) / 1e12, 1) if ph_flops[i] and avg_ms > 0 else None}
    phases = _phase_table(PREFILL_PHASES, ph_ms, ncalls, tf)
    # timed region
    dom = PREFILL_PHASES.index("w13_gemm_swiglu")
    blk.profile_start(steps, phases=[dom])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        blk.prefill(cache, layer, x, y, B, Lq, sc)
        layer += 1
    e1.record()
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    dom_ms, dcalls = blk.profile_read()
    avg_dom = dom_ms[dom] / dcalls * 1e-3
    achieved = ph_flops[dom] / avg_dom / 1e12
    ms = total_ms / steps
    return {
        "workload": wl.name, "batch": B, "seq_len": Lq, "ms_per_step": round(ms, 4),
        "tflops": round(flops / (ms * 1e-3) / 1e12, 2), "tokens_per_s": round(B * Lq / (ms * 1e-3), 1),
        "frac_of_peak_block": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "flops_per_step": flops, "phases": phases,
        "roofline": {"kernel": "k_gemm_mfma (w1/w3 + SwiGLU epilogue)", "bound": "mfma",
                     "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": _traffic_bytes(f"prefill_w13:{wl.name}"),
                     "flops_per_launch": ph_flops[dom], "avg_launch_us": round(avg_dom * 1e6, 2)},
    }


def bench_decode(wl, steps, warmup, inp=None):
    """Decode: every step reads 512 MB first (more than the 256 MB last-level
    cache, and a read leaves no dirty lines) so no weight or cache byte is served
    from it.  Step time = (time of `steps` x [flush, decode] - time of `steps` x
    [flush]) / steps, each loop bracketed by two events; the attention kernels
    are timed inside the first loop by events attached to their launches."""
    import torch
    import workloads as W
    from tests import gpu_util as G
    s, B, S0 = wl.shape, wl.batch, wl.cache_len
    max_seq = S0 + warmup + 2 * steps + 1
    inp, blk, cache = _setup(wl, max_seq, 1, inp)
    for b in range(B):
        cache.write(0, b, 0, G.tdev(inp["k_cache"][b], s.dtype), G.tdev(inp["v_cache"][b], s.dtype))
    cache.set_lens(0, [S0] * B)
    sc = G.scratch(blk, B, B, max_seq)
    x = G.tdev(inp["x"].reshape(B, s.dim), s.dtype)
    y = torch.empty_like(x)
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    for _ in range(warmup):
        flush.sum()
        blk.decode(cache, 0, x, y, B, sc)
    torch.cuda.synchronize()
    # breakdown pass (events at every phase boundary)
    blk.profile_start(steps)
    for _ in range(steps):
        flush.sum()
        blk.decode(cache, 0, x, y, B, sc)
    ph_ms, ncalls = blk.profile_read()
    lens0 = S0 + warmup + steps
    att = DECODE_PHASES.index("attention_decode")
    blk.profile_start(steps, phases=[att])
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(steps):
        flush.sum()
        blk.decode(cache, 0, x, y, B, sc)
    ev[1].record()
    for _ in range(steps):
        flush.sum()
    ev[2].record()
    torch.cuda.synchronize()
    t_loop, t_flush = ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2])
    att_ms, acalls = blk.profile_read()
    ms = (t_loop - t_flush) / steps
    byts = [W.decode_bytes(s, B, lens0 + i) for i in range(steps)]
    tot_bytes = sum(b["total"] for b in byts) / steps
    kv_bytes = sum(b["kv_read"] + b["kv_write"] for b in byts) / steps
    attn_us = att_ms[att] / acalls * 1e3
    lb = {0: s.dim * (s.n_heads + 2 * s.n_kv_heads) * s.head_dim, 3: s.n_heads * s.head_dim * s.dim,
          5: 2 * s.dim * s.ffn_dim, 6: s.ffn_dim * s.dim}
    esz = 2 if s.dtype == "bf16" else 4

    def gbs(i, avg_ms):
        if i in lb:
            return {"gbs": round(lb[i] * esz / (avg_ms * 1e-3) / 1e9, 1)}
        if i == att:
            return {"gbs": round(kv_bytes / (avg_ms * 1e-3) / 1e9, 1)}
        return {}
    phases = _phase_table(DECODE_PHASES, ph_ms, ncalls, gbs)
    achieved = kv_bytes / (attn_us * 1e-6) / 1e9
    return {
        "workload": wl.name, "batch": B, "cache_len": S0, "us_per_step": round(ms * 1e3, 2),
        "tokens_per_s": round(B / (ms * 1e-3), 1), "bytes_per_step": tot_bytes,
        "hbm_frac_step": round(tot_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "phases_sum_us": round(sum(ph_ms) / ncalls * 1e3, 2), "phases": phases,
        "roofline": {"kernel": "k_attn_decode_bf16 + k_attn_merge", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": _traffic_bytes(f"decode_attention:{wl.name}"), "bytes_per_launch": kv_bytes,
                     "avg_launch_us": round(attn_us, 2)},
    }


def bench_tiny(wl, reps):
    """The tiny fp32 block: a 32-token prefill, then 8 decode steps (latency
    bound: reported in microseconds per call, best of `reps`)."""
    import torch
    import workloads as W
    from tests import gpu_util as G
    s, P, n = wl.shape, wl.seq_len, wl.decode_steps
    inp = W.draw_block_workload(wl)
    blk, wd = G.make_block(s, inp["weights"], P + n)
    x = G.tdev(inp["x"][0], s.dtype)
    y = torch.empty_like(x)
    sc = G.scratch(blk, P, 1, P + n)
    best_p, best_d = float("inf"), float("inf")
    for _ in range(reps):
        cache = G.make_cache(s, 1, 1, P + n)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        torch.cuda.synchronize()
        ev[0].record()
        blk.prefill(cache, 0, x[:P], y[:P], 1, P, sc)
        ev[1].record()
        for t in range(n):
            blk.decode(cache, 0, x[P + t:P + t + 1], y[P + t:P + t + 1], 1, sc)
        ev[2].record()
        torch.cuda.synchronize()
        best_p = min(best_p, ev[0].elapsed_time(ev[1]) * 1e3)
        best_d = min(best_d, ev[1].elapsed_time(ev[2]) * 1e3 / n)
    return {"workload": wl.name, "prefill_us": round(best_p, 1), "decode_us_per_step": round(best_d, 1),
            "flops_prefill": W.prefill_flops(s, 1, P)}


def bench_stack(wl, reps):
    """The 40-layer 4-bit stack: embedding, blocks, final norm, output head and
    greedy argmax, each call on one stream with its decode step replayed from a
    HIP graph.  Prompt pass = a call with one greedy step; decode step time =
    (call with n steps - call with 1 step) / (n - 1), which leaves the prompt
    pass and the graph capture out.  Best of `reps` calls each."""
    import numpy as np
    import torch
    import workloads as W
    import decoder_block_rmsnorm_amd as L
    from tests import gpu_util as G
    s, P, n = wl.shape, wl.seq_len, wl.decode_steps
    max_seq = P + n
    t0 = time.time()
    blocks, keep = [], []
    for item in W.draw_stack(wl, W.Rng(wl.seed)):
        if item[0] == "ids":
            ids = item[1]
        elif item[0] == "layer":
            blk, wd = G.make_block(s, item[2], max_seq)
            blocks.append(blk)
            del wd
        else:
            head = item[1]
    emb, fn, out = G.tdev(head["embedding"], "bf16"), G.tdev(head["norm"], "bf16"), G.q4_dev(head["output"])
    stack = L.Stack(blocks, emb, wl.vocab, fn, out)
    log(f"[bench] {wl.name}: stack built in {time.time() - t0:.1f}s")
    sc = torch.empty(stack.scratch_bytes(P, max_seq), dtype=torch.uint8, device="cuda")
    prompt = torch.from_numpy(ids.reshape(-1).astype(np.int32)).cuda()
    out_ids = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
    logits = torch.zeros((n + 1, wl.vocab), dtype=torch.float32, device="cuda")
    st = torch.cuda.Stream()

    def run(steps):
        cache = G.make_cache(s, wl.n_layers, 1, max_seq)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(st):
            e0.record(st)
            stack.generate(cache, prompt, steps, out_ids, logits, sc, use_graph=True, stream=st)
            e1.record(st)
        torch.cuda.synchronize()
        del cache
        return e0.elapsed_time(e1)
    run(1)
    t1 = min(run(1) for _ in range(reps))
    tn = min(run(n) for _ in range(reps))
    step_ms = (tn - t1) / (n - 1)
    prompt_ms = t1 - step_ms
    # the same loop with a sampled next id (temperature 0.8, nucleus 0.9, seeded
    # draws) in place of the argmax
    u = torch.from_numpy(W.Rng(wl.seed + 1).g.random(n + 1).astype(np.float32)).cuda()
    stack.set_sampling(0.8, 0.9, u)
    run(1)
    s1 = min(run(1) for _ in range(reps))
    sn = min(run(n) for _ in range(reps))
    sampled_step_ms = (sn - s1) / (n - 1)
    stack.set_sampling(0.0, 1.0, None)
    # the loop without the cache's reuse (every id re-runs the prompt pass over
    # the sequence so far): nr ids, timed once
    nr = 16
    sc_r = torch.empty(stack.scratch_bytes(P + nr, max_seq), dtype=torch.uint8, device="cuda")
    cache = G.make_cache(s, wl.n_layers, 1, max_seq)
    torch.cuda.synchronize()
    t0r = time.perf_counter()
    stack.generate_recompute(cache, prompt, nr, out_ids, None, sc_r, stream=st)
    torch.cuda.synchronize()
    recompute_ms = (time.perf_counter() - t0r) * 1e3 / (nr + 1)
    del cache, sc_r
    # bytes of one step at the mean cache length: every weight and cached K/V
    # byte once, plus the output head (4-bit) and the logits
    mean_cached = P + n / 2
    layer = W.decode_bytes(s, 1, int(mean_cached))["total"]
    head_bytes = wl.vocab * s.dim * (0.5 + 2 * 2 / s.group_size) + wl.vocab * 4
    step_bytes = wl.n_layers * layer + head_bytes
    flops = wl.n_layers * W.prefill_flops(s, 1, P) + 2.0 * wl.vocab * s.dim   # head: last token only
    return {"workload": wl.name, "prompt_tokens": P, "prompt_ms": round(prompt_ms, 3),
            "prompt_tflops": round(flops / (prompt_ms * 1e-3) / 1e12, 1),
            "prompt_frac_of_peak": round(flops / (prompt_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "decode_steps": n, "decode_us_per_step": round(step_ms * 1e3, 1),
            "decode_tokens_per_s": round(1.0 / (step_ms * 1e-3), 1), "bytes_per_step": step_bytes,
            "sampled_decode_us_per_step": round(sampled_step_ms * 1e3, 1),
            "recompute_ms_per_id": round(recompute_ms, 3), "recompute_ids": nr + 1,
            "hbm_frac_step": round(step_bytes / (step_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def measured_peaks():
    """What this part sustains: a register-only loop of bf16 MFMAs (2 and 1
    wavefronts per SIMD on every CU) and a 1 GiB device-to-device copy."""
    import torch
    import decoder_block_rmsnorm_amd as L
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = {"spec_bf16_tflops": PEAK_BF16_TFLOPS, "spec_hbm_gbs": PEAK_HBM_GBS, "compute_units": cus}
    for waves, key in ((2, "mfma_bf16_loop_tflops_2waves_per_simd"), (1, "mfma_bf16_loop_tflops_1wave_per_simd")):
        blocks = cus * waves
        sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
        iters = 20000
        L.llama_probe_mfma_bf16(blocks, 100, sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        L.llama_probe_mfma_bf16(blocks, iters, sink)
        e1.record()
        torch.cuda.synchronize()
        flop = blocks * 4 * iters * 8 * 32768.0
        out[key] = round(flop / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = float("inf")
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    out["copy_gbs"] = round(2 * n / (best * 1e-3) / 1e9, 1)     # read + write
    del src, dst
    return out


# ------------------------------------------------------------------ CPU oracle
def _blas_info():
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return i.get("num_threads", 1), f"{i.get('internal_api', '?')} {i.get('version', '')}".strip()
    except Exception:  # pragma: no cover
        pass
    return len(os.sched_getaffinity(0)), "unknown"


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_prefill(wl, inp, min_seconds):
    """The oracle's causal prefill of the workload's whole batch, repeated until
    at least `min_seconds` have passed (at least once)."""
    import workloads as W
    from oracle import ref
    reps, t0 = 0, time.perf_counter()
    while True:
        ref.block_forward(inp["x"], inp["weights"], wl.shape)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    fl = W.prefill_flops(wl.shape, wl.batch, wl.seq_len) * reps
    return {"value": round(fl / dt / 1e12, 5), "unit": "TFLOP/s",
            "tokens_per_s": round(reps * wl.batch * wl.seq_len / dt, 2),
            "sample": f"{reps} x the causal prefill of the whole batch ({wl.batch} x {wl.seq_len} tokens) of "
                      f"{wl.name}, float64 numpy, {dt:.1f} s; {fl / 1e12:.3f} TFLOP counted"}


def cpu_decode(wl, inp):
    """One decode step of the whole batch through the oracle."""
    from oracle import ref
    x = inp["x"][:, :1]
    t0 = time.perf_counter()
    ref.block_forward(x, inp["weights"], wl.shape, list(inp["k_cache"]), list(inp["v_cache"]))
    dt = time.perf_counter() - t0
    return {"value": round(wl.batch / dt, 3), "unit": "tokens/s", "us_per_step": round(dt * 1e6, 1),
            "sample": f"one decode step of all {wl.batch} sequences against {wl.cache_len} cached positions "
                      f"of {wl.name}, float64 numpy, {dt:.1f} s"}


def cpu_tiny(wl):
    import numpy as np
    import workloads as W
    from oracle import ref
    inp = W.draw_block_workload(wl)
    s, P, n = wl.shape, wl.seq_len, wl.decode_steps
    t0 = time.perf_counter()
    r = ref.block_forward(inp["x"][:, :P], inp["weights"], s)
    kc, vc = r["k_new"], r["v_new"]
    for t in range(n):
        r = ref.block_forward(inp["x"][:, P + t:P + t + 1], inp["weights"], s, kc, vc)
        kc = [np.concatenate([kc[0], r["k_new"][0]])]
        vc = [np.concatenate([vc[0], r["v_new"][0]])]
    dt = time.perf_counter() - t0
    return {"value": round(dt * 1e6, 1), "unit": "us (prefill 32 + 8 decode steps)",
            "sample": f"the whole {wl.name} workload, float64 numpy"}


def cpu_stack(wl, n_layers=2, steps=4):
    """The 4-bit stack on a bounded sample: the 512-token prompt pass and `steps`
    single-token steps through the first `n_layers` of the 40 layers (their
    weights dequantized once to float64 and kept for the steps), per-layer times
    scaled to the 40 layers, plus the output head's share."""
    import numpy as np
    import workloads as W
    from oracle import ref
    s, P = wl.shape, wl.seq_len
    gen = W.draw_stack(wl, W.Rng(wl.seed))
    ids = next(gen)[1]
    layers = [next(gen)[2] for _ in range(n_layers)]
    t0 = time.perf_counter()
    dense = [{k: (v if k.endswith("norm") else ref.weight_matrix(v)) for k, v in w.items()} for w in layers]
    t_deq = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    x = rng.standard_normal((1, P, s.dim))
    t0 = time.perf_counter()
    kc, vc = [], []
    for w in dense:
        r = ref.block_forward(x, w, s)
        kc.append(r["k_new"][0])
        vc.append(r["v_new"][0])
        x = ref.stack_arrays(r, "y")
    t_prompt = time.perf_counter() - t0
    xt = rng.standard_normal((1, 1, s.dim))
    t0 = time.perf_counter()
    for _ in range(steps):
        for i, w in enumerate(dense):
            r = ref.block_forward(xt, w, s, [kc[i]], [vc[i]])
            kc[i] = np.concatenate([kc[i], r["k_new"][0]])
            vc[i] = np.concatenate([vc[i], r["v_new"][0]])
    t_step = (time.perf_counter() - t0) / steps
    scale = wl.n_layers / n_layers
    prompt_s = (t_prompt + t_deq) * scale
    return {"value": round(P / prompt_s, 2), "unit": "tokens/s (prompt pass)",
            "decode_us_per_step": round(t_step * scale * 1e6, 1),
            "sample": f"the {P}-token prompt pass and {steps} decode steps through {n_layers} of the "
                      f"{wl.n_layers} layers of {wl.name} (weights dequantized to float64 once, "
                      f"{t_deq:.1f} s, and kept for the steps), times scaled by {scale:g}; float64 numpy"}


def _source_sha(path):
    import hashlib
    with open(os.path.join(ROOT, path), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def recorded_traffic(kernel):
    """HBM bytes per launch of `kernel` from the counter summary committed in
    profiles/hbm_traffic.md (FETCH_SIZE + WRITE_SIZE, each scaled by the copy
    calibration), or None when none is recorded or the kernel's source file
    has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if not line.startswith("traffic:"):
            continue
        kv = dict(t.split("=", 1) for t in line.split()[1:])
        if kv.get("kernel") != kernel:
            continue
        if _source_sha(kv["source"]) != kv["sha256"]:
            return None
        return {"bytes": int(kv["bytes_per_launch"]), "fetch_bytes": int(kv["fetch_bytes"]),
                "write_bytes": int(kv["write_bytes"]), "source": kv["source"]}
    return None


def copy_probe(mb, reps):
    """A plain device copy of `mb` MiB, `reps` times: the known-size kernel that
    calibrates the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    src = torch.ones(mb << 18, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": mb << 20, "reps": reps}), flush=True)


def blas_probe(workload, steps, warmup):
    """The workload's W1/W3 product through torch.matmul (hipBLASLt), timed with
    events: the vendor library's rate on the same shape, for the profiles that
    set it beside the block's own GEMM (same bf16 operands, fp32 accumulation;
    hipBLASLt writes the whole product, the block's GEMM only g)."""
    import torch
    import workloads as W
    wl = W.get(workload)
    M, K, N = wl.batch * wl.seq_len, wl.shape.dim, 2 * wl.shape.ffn_dim
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn(M, K, device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn(N, K, device="cuda", dtype=torch.bfloat16, generator=g) * 0.02
    for _ in range(warmup):
        c = torch.matmul(a, b.t())
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        c = torch.matmul(a, b.t())
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / max(steps, 1)
    del c
    print(json.dumps({"blas_probe": f"torch.matmul {M}x{K} . ({N}x{K})^T bf16", "workload": wl.name,
                      "ms": round(ms, 4), "tflops": round(2.0 * M * K * N / (ms * 1e-3) / 1e12, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE, help="the headline prefill workload")
    ap.add_argument("--decode-workload", default=DECODE,
                    help="decode workload reported beside the prefill line ('' to skip)")
    ap.add_argument("--extras", default="all", choices=["all", "none"],
                    help="also run the 7B prefill, 13B decode, tiny fp32 and 4-bit stack workloads")
    ap.add_argument("--kv-heads", type=int, default=0,
                    help="run the decode workload with this many kv heads (1 = multi-query attention)")
    ap.add_argument("--window", type=int, default=0,
                    help="run the decode workload with sliding-window attention of this many positions")
    ap.add_argument("--stack-workload", default=STACK,
                    help="the 4-bit stack workload of the extras ('' to skip)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum seconds of oracle time on the headline workload (0: no CPU baselines)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration) and exit")
    ap.add_argument("--blas-probe", action="store_true",
                    help="only time the headline workload's W1/W3 product through torch.matmul and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (no collectives, no sharded "
              "weights); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import dataclasses
    import torch
    import workloads as W
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_probe:
        return copy_probe(args.copy_probe, max(args.steps, 1))
    if args.blas_probe:
        return blas_probe(args.workload, args.steps, args.warmup)
    cpu = args.cpu_seconds > 0
    cpu_rows = {}
    wl = W.get(args.workload)
    if wl.mode != "prefill":
        raise SystemExit("--workload must be a prefill workload; decode workloads go to --decode-workload")
    log(f"[bench] prefill {wl.name}: warmup {args.warmup}, steps {args.steps}")
    inp = W.draw_block_workload(wl)
    pre = bench_prefill(wl, args.steps, args.warmup, inp)
    log(f"[bench] prefill {pre['ms_per_step']:.3f} ms/step, {pre['tflops']:.1f} TFLOP/s")
    torch.cuda.empty_cache()
    if cpu:
        log(f"[bench] cpu oracle, {wl.name}, at least {args.cpu_seconds} s")
        cpu_rows[wl.name] = cpu_prefill(wl, inp, args.cpu_seconds)
    del inp
    out = {
        "metric": METRIC, "value": pre["tflops"], "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": pre["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs, N(0,0.02) weights, 1+U(-0.1,0.1) norm weights)",
        "config": {"workload": wl.name, "batch": wl.batch, "seq_len": wl.seq_len, "dim": wl.shape.dim,
                   "n_heads": wl.shape.n_heads, "n_kv_heads": wl.shape.n_kv_heads, "ffn_dim": wl.shape.ffn_dim,
                   "tokens_per_s": pre["tokens_per_s"], "frac_of_peak_block": pre["frac_of_peak_block"]},
        "roofline": pre["roofline"],
        "prefill_phases": pre["phases"],
    }
    if args.decode_workload:
        dw = W.get(args.decode_workload)
        if args.kv_heads > 0:
            dw = dataclasses.replace(dw, name=f"{dw.name}_kvheads{args.kv_heads}",
                                     shape=dataclasses.replace(dw.shape, n_kv_heads=args.kv_heads))
        if args.window > 0:
            dw = dataclasses.replace(dw, name=f"{dw.name}_window{args.window}",
                                     shape=dataclasses.replace(dw.shape, window=args.window))
        log(f"[bench] decode {dw.name}")
        dinp = W.draw_block_workload(dw)
        out["decode"] = bench_decode(dw, args.steps, args.warmup, dinp)
        log(f"[bench] decode {out['decode']['us_per_step']} us/step, {out['decode']['tokens_per_s']} tok/s")
        torch.cuda.empty_cache()
        if cpu:
            log(f"[bench] cpu oracle, {dw.name}")
            cpu_rows[dw.name] = cpu_decode(dw, dinp)
        del dinp
    if args.extras == "all":
        extra = {}
        ew = W.get(EXTRA_PREFILL)
        log(f"[bench] prefill {ew.name}")
        einp = W.draw_block_workload(ew)
        r = bench_prefill(ew, args.steps, args.warmup, einp)
        log(f"[bench] prefill {r['ms_per_step']:.3f} ms/step, {r['tflops']:.1f} TFLOP/s")
        extra[ew.name] = r
        torch.cuda.empty_cache()
        if cpu:
            cpu_rows[ew.name] = cpu_prefill(ew, einp, 0.0)
        del einp
        dw = W.get(EXTRA_DECODE)
        log(f"[bench] decode {dw.name}")
        dinp = W.draw_block_workload(dw)
        r = bench_decode(dw, args.steps, args.warmup, dinp)
        log(f"[bench] decode {r['us_per_step']} us/step, {r['tokens_per_s']} tok/s")
        extra[dw.name] = r
        torch.cuda.empty_cache()
        if cpu:
            cpu_rows[dw.name] = cpu_decode(dw, dinp)
        del dinp
        tw = W.get(TINY)
        extra[tw.name] = bench_tiny(tw, 5)
        if cpu:
            cpu_rows[tw.name] = cpu_tiny(tw)
        out["extra"] = extra
        if args.stack_workload:
            sw = W.get(args.stack_workload)
            torch.cuda.empty_cache()
            log(f"[bench] stack {sw.name}")
            out["stack"] = bench_stack(sw, 2)
            log(f"[bench] stack decode {out['stack']['decode_us_per_step']} us/step")
            torch.cuda.empty_cache()
            if cpu:
                log(f"[bench] cpu oracle, {sw.name} (sample)")
                cpu_rows[sw.name] = cpu_stack(sw)
    torch.cuda.empty_cache()
    out["measured_peaks"] = measured_peaks()
    if cpu:
        threads, blas = _blas_info()
        head = cpu_rows[wl.name]
        out["cpu_baseline"] = {"value": head["value"], "unit": head["unit"], "cores": threads, "kind": "oracle",
                               "sample": head["sample"], "cpu": _cpu_model(), "blas": blas,
                               "workloads": {k: v for k, v in cpu_rows.items() if k != wl.name}}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
