#!/usr/bin/env python3
"""Benchmark of the MTLA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline workload (the JSON line's ``value``): speech-translation-shaped
decoding, batch 50 (10 sentences x beam 5), 512 tokens, H=8, d_h=64, d_c=256,
d_R=32, s=2, bf16 storage.  One step is the whole 512-token decode of the
batch: for every token, mtla_decode_step (gate + temporal merge of the token,
query absorption, latent attention over ceil(t/s) slots, up-projection).
The 512 launches of a step are captured once in a HIP graph and replayed;
inputs are resident in HBM before the timed region.

The other workloads are reported in ``components``: the s=4 decode loop
(2048 tokens), the summarisation-shaped prefill (B=16, N=4096, s=3), the same
prefill's second half as one chunked call after the first half
(mtla_prefill_at), the LLM-scale step (B=64, cache of 32,768 tokens, one
append + decode), a beam-search reorder of that LLM-scale decode state
(mtla_reorder_state), the whole layer from h (input projections + RoPE,
the core, output projection) for the s=2 decode loop and the prefill, and
the training backward of the summarisation prefill (mtla_prefill_backward).

``roofline`` describes the dominant kernel of the headline step: the fused
decode-step kernel, the step's only kernel, so its average launch duration is
the timed graph replay (HIP events) divided by the 512 launches.  ``cpu_baseline`` is the fp64 oracle (test
infrastructure, single-threaded) timed on this host over the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

METRIC = "MTLA decode tokens/s + HBM GB/s (s=2,4); stride-masked prefill TFLOP/s"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--no-components", action="store_true", help="headline workload only")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only", default=None,
                   help="run one workload and print its record (st_decode_s2, st_decode_s4, prefill, "
                        "prefill_chunk, llm_decode, reorder, layer_decode, layer_prefill, backward, copy: "
                        "the counter-calibration copy kernel)")
    return p.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

def to_dev(x, dtype, torch):
    return torch.from_numpy(x).to("cuda").to(dtype)


def timed_graph(g, reps, torch):
    """Average ms of `reps` replays of graph g, HIP events on torch's stream."""
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / reps


def capture(fn, torch):
    fn()  # eager run first: loads code objects, checks arguments
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def slot_reads(n_tokens, s):
    """sum_{t=1..N} ceil(t/s): slot rows one sequence's decode loop reads."""
    return sum(-(-t // s) for t in range(1, n_tokens + 1))


# ---------------------------------------------------------------------------
# decode loop (headline and the s=4 component)
# ---------------------------------------------------------------------------

class DecodeLoop:
    def __init__(self, w, m, torch, workloads):
        import numpy as np
        self.w, self.m, self.torch = w, m, torch
        B, N, H = w.batch, w.n_tokens, w.heads
        self.dims = m.make_dims(B, H, w.d_h, w.d_c, w.d_r, w.s, -(-N // w.s), "bf16")
        d = self.dims
        lat = workloads.batch_latents(w)                       # c [B, N, d_c], k_r [B, N, d_r]
        qry = workloads.batch_queries(w)                       # q_c [B, N, H, d_h], q_r
        wts = workloads.weights(w)
        bf = torch.bfloat16
        # per-step slices must be contiguous: stage token-major copies
        self.c = to_dev(np.ascontiguousarray(lat["c"].transpose(1, 0, 2)), bf, torch)
        self.k_r = to_dev(np.ascontiguousarray(lat["k_r"].transpose(1, 0, 2)), bf, torch)
        self.q_c = to_dev(np.ascontiguousarray(qry["q_c"].transpose(1, 0, 2, 3)), bf, torch)
        self.q_r = to_dev(np.ascontiguousarray(qry["q_r"].transpose(1, 0, 2, 3)), bf, torch)
        self.w_hyp = to_dev(wts["w_hyp"], torch.float32, torch)
        self.w_uk = to_dev(wts["w_uk"], bf, torch)
        self.w_uv = to_dev(wts["w_uv"], bf, torch)
        self.pos = (torch.arange(1, N + 1, dtype=torch.int32, device="cuda")[:, None]
                    .expand(N, B).contiguous())
        self.pe = torch.empty(N, w.d_c, dtype=torch.float32, device="cuda")
        m.mtla_sinusoidal_pe(self.pe)
        self.cache = torch.zeros(B, d.max_slots, d.width, dtype=bf, device="cuda")
        self.open_acc = torch.zeros(B, 2, d.width, dtype=torch.float32, device="cuda")
        self.ws = torch.zeros(m.mtla_decode_workspace_bytes(d), dtype=torch.uint8, device="cuda")
        self.out = torch.empty(N, B, H, w.d_h, dtype=bf, device="cuda")
        self.host_inputs = (lat, qry, wts)

    def step(self):
        m, d = self.m, self.dims
        for t in range(self.w.n_tokens):
            m.mtla_decode_step(d, self.pos[t], self.c[t], self.k_r[t], self.w_hyp, self.pe,
                               self.q_c[t], self.q_r[t], self.w_uk, self.w_uv, self.cache,
                               self.open_acc, self.out[t], self.ws)


def step_bytes(w, t):
    """Algorithmic HBM bytes of one decode-step launch at token t (bf16
    storage): slot rows read, W_UK and W_UV, and the per-token terms (token
    latent and rope key, queries, outputs, the written slot row, the fp32
    open-slot state read and written, the pe row and W_hyp)."""
    e, B, H = 2, w.batch, w.heads
    n = -(-t // w.s)
    cache = B * n * w.width * e
    weights = 2 * H * w.d_h * w.d_c * e + w.d_c * 4
    token = B * (w.width * e + H * (w.d_h + w.d_r) * e + H * w.d_h * e + w.width * e
                 + 2 * w.width * 4 + w.d_c * 4)
    return cache, weights, token


def run_decode_loop(w, steps, warmup, m, torch, workloads):
    log(f"{w.name}: staging inputs")
    t0 = time.time()
    dl = DecodeLoop(w, m, torch, workloads)
    splits, fused = m.mtla_decode_plan(dl.dims)
    log(f"{w.name}: staged in {time.time() - t0:.1f}s; plan splits={splits} fused={fused}; "
        f"capturing {w.n_tokens} steps")
    g = capture(dl.step, torch)
    for _ in range(warmup):
        g.replay()
    ms = timed_graph(g, steps, torch)
    tokens = w.batch * w.n_tokens
    per_t = [step_bytes(w, t) for t in range(1, w.n_tokens + 1)]
    cache_b = sum(p[0] for p in per_t)
    all_b = sum(sum(p) for p in per_t)
    rec = {"workload": w.name, "ms_per_step": ms, "tokens_per_step": tokens,
           "tokens_per_s": tokens / (ms * 1e-3), "us_per_token": ms * 1e3 / w.n_tokens,
           "plan": {"splits": splits, "fused": fused},
           "step_GBps": all_b / (ms * 1e-3) / 1e9,
           "cache_GBps": cache_b / (ms * 1e-3) / 1e9}
    if fused:
        per_launch = all_b / w.n_tokens
        us = ms * 1e3 / w.n_tokens
        rec["dominant_kernel"] = {
            "name": "decode_step_wave_kernel" if w.d_c == 256 else "decode_step_kernel",
            "launches_per_step": w.n_tokens, "avg_launch_us": us,
            "algorithmic_bytes_per_launch": per_launch, "GBps": per_launch / (us * 1e-6) / 1e9}
    return rec, dl


# ---------------------------------------------------------------------------
# prefill component
# ---------------------------------------------------------------------------

def attended_pairs(N, s):
    """A(N, s) = sum_{i<=N} ceil(i/s): keys attended, per (sequence, head)."""
    q, r = divmod(N, s)
    return s * q * (q + 1) // 2 + r * (q + 1)


def run_prefill(w, steps, warmup, m, torch, workloads):
    log(f"{w.name}: staging inputs")
    B, N, H = w.batch, w.n_tokens, w.heads
    d = m.make_dims(B, H, w.d_h, w.d_c, w.d_r, w.s, -(-N // w.s), "bf16")
    lat, qry, wts = workloads.batch_latents(w), workloads.batch_queries(w), workloads.weights(w)
    bf = torch.bfloat16
    c, k_r = to_dev(lat["c"], bf, torch), to_dev(lat["k_r"], bf, torch)
    q_c, q_r = to_dev(qry["q_c"], bf, torch), to_dev(qry["q_r"], bf, torch)
    w_hyp = to_dev(wts["w_hyp"], torch.float32, torch)
    w_uk, w_uv = to_dev(wts["w_uk"], bf, torch), to_dev(wts["w_uv"], bf, torch)
    pe = torch.empty(N, w.d_c, dtype=torch.float32, device="cuda")
    m.mtla_sinusoidal_pe(pe)
    cache = torch.zeros(B, d.max_slots, d.width, dtype=bf, device="cuda")
    open_acc = torch.zeros(B, 2, d.width, dtype=torch.float32, device="cuda")
    out = torch.empty(B, N, H, w.d_h, dtype=bf, device="cuda")
    ws = torch.empty(m.mtla_prefill_workspace_bytes(d, N), dtype=torch.uint8, device="cuda")

    def fn():
        m.mtla_prefill(d, q_c, q_r, c, k_r, w_hyp, pe, w_uk, w_uv, cache, open_acc, out, ws)
    g = capture(fn, torch)
    for _ in range(warmup):
        g.replay()
    ms = timed_graph(g, steps, torch)
    A = attended_pairs(N, w.s)
    f_attn = 2.0 * B * H * A * (2 * w.d_h + w.d_r)
    f_up = 4.0 * B * N * w.d_c * H * w.d_h
    return {"workload": w.name, "ms_per_call": ms, "attended_pairs_per_bh": A,
            "attn_gflop": f_attn / 1e9, "kv_gemm_gflop": f_up / 1e9,
            "tflops_end_to_end": (f_attn + f_up) / (ms * 1e-3) / 1e12,
            "attn_tflops_over_end_to_end_time": f_attn / (ms * 1e-3) / 1e12}, (out, q_c, q_r, lat, qry, wts)


def run_backward(w, steps, warmup, m, torch, workloads):
    """Training backward of the summarisation prefill (B=16, N=4096, s=3):
    one mtla_prefill_backward call (forward recomputation included) from the
    same inputs as the prefill and a seeded upstream gradient."""
    log(f"{w.name} backward: staging inputs")
    B, N, H = w.batch, w.n_tokens, w.heads
    d = m.make_dims(B, H, w.d_h, w.d_c, w.d_r, w.s, -(-N // w.s), "bf16")
    lat, qry, wts = workloads.batch_latents(w), workloads.batch_queries(w), workloads.weights(w)
    bf, f32 = torch.bfloat16, torch.float32
    c, k_r = to_dev(lat["c"], bf, torch), to_dev(lat["k_r"], bf, torch)
    q_c, q_r = to_dev(qry["q_c"], bf, torch), to_dev(qry["q_r"], bf, torch)
    w_hyp = to_dev(wts["w_hyp"], f32, torch)
    w_uk, w_uv = to_dev(wts["w_uk"], bf, torch), to_dev(wts["w_uv"], bf, torch)
    d_o = to_dev(workloads.batch_grad_out(w), bf, torch)
    pe = torch.empty(N, w.d_c, dtype=f32, device="cuda")
    m.mtla_sinusoidal_pe(pe)
    g_qc, g_qr = torch.empty_like(q_c), torch.empty_like(q_r)
    g_c, g_kr = torch.empty_like(c), torch.empty_like(k_r)
    g_wh = torch.empty(w.d_c, dtype=f32, device="cuda")
    g_uk = torch.empty(H, w.d_h, w.d_c, dtype=f32, device="cuda")
    g_uv = torch.empty_like(g_uk)
    ws = torch.empty(m.mtla_prefill_backward_workspace_bytes(d, N), dtype=torch.uint8, device="cuda")

    def fn():
        m.mtla_prefill_backward(d, q_c, q_r, c, k_r, w_hyp, pe, w_uk, w_uv, d_o, g_qc, g_qr, g_c, g_kr, g_wh,
                                g_uk, g_uv, ws)
    g = capture(fn, torch)
    for _ in range(warmup):
        g.replay()
    ms = timed_graph(g, steps, torch)
    A = attended_pairs(N, w.s)
    QW = w.d_h + w.d_r
    # per attended pair and head: the score recomputation, dP = dO V^T, dV,
    # dK and dQ products; plus the K/V recomputation, dP^c and dW products
    f_attn = 2.0 * B * H * A * (3 * QW + 2 * w.d_h)
    f_gemm = 3 * 4.0 * B * N * w.d_c * H * w.d_h
    return {"workload": w.name + "_backward", "ms_per_call": ms, "attn_gflop": f_attn / 1e9,
            "gemm_gflop": f_gemm / 1e9, "tflops_end_to_end": (f_attn + f_gemm) / (ms * 1e-3) / 1e12}


def run_prefill_chunk(w, steps, warmup, m, torch, workloads):
    """Chunked prefill of the summarisation shape: the first t0 tokens by
    mtla_prefill (untimed), then tokens t0+1..N by one mtla_prefill_at call
    (timed, replayed from a graph).  t0 ends a block, so every replay reads the
    same cache rows and no open-slot state."""
    B, N, H, s = w.batch, w.n_tokens, w.heads, w.s
    t0 = (N // 2) // s * s
    n2 = N - t0
    log(f"{w.name} chunked: staging inputs (t0={t0}, chunk={n2})")
    d = m.make_dims(B, H, w.d_h, w.d_c, w.d_r, s, -(-N // s), "bf16")
    lat, qry, wts = workloads.batch_latents(w), workloads.batch_queries(w), workloads.weights(w)
    bf = torch.bfloat16
    c, k_r = to_dev(lat["c"], bf, torch), to_dev(lat["k_r"], bf, torch)
    q_c, q_r = to_dev(qry["q_c"], bf, torch), to_dev(qry["q_r"], bf, torch)
    w_hyp = to_dev(wts["w_hyp"], torch.float32, torch)
    w_uk, w_uv = to_dev(wts["w_uk"], bf, torch), to_dev(wts["w_uv"], bf, torch)
    pe = torch.empty(N, w.d_c, dtype=torch.float32, device="cuda")
    m.mtla_sinusoidal_pe(pe)
    cache = torch.zeros(B, d.max_slots, d.width, dtype=bf, device="cuda")
    open_acc = torch.zeros(B, 2, d.width, dtype=torch.float32, device="cuda")
    out1 = torch.empty(B, t0, H, w.d_h, dtype=bf, device="cuda")
    out2 = torch.empty(B, n2, H, w.d_h, dtype=bf, device="cuda")
    ws1 = torch.empty(m.mtla_prefill_workspace_bytes(d, t0), dtype=torch.uint8, device="cuda")
    m.mtla_prefill(d, q_c[:, :t0].contiguous(), q_r[:, :t0].contiguous(), c[:, :t0].contiguous(),
                   k_r[:, :t0].contiguous(), w_hyp, pe, w_uk, w_uv, cache, open_acc, out1, ws1)
    del ws1
    ws = torch.empty(m.mtla_prefill_at_workspace_bytes(d, t0, n2), dtype=torch.uint8, device="cuda")
    args2 = [x[:, t0:].contiguous() for x in (q_c, q_r, c, k_r)]

    def fn():
        m.mtla_prefill_at(d, t0, *args2, w_hyp, pe, w_uk, w_uv, cache, open_acc, out2, ws)
    g = capture(fn, torch)
    for _ in range(warmup):
        g.replay()
    ms = timed_graph(g, steps, torch)
    A = attended_pairs(N, s) - attended_pairs(t0, s)
    f_attn = 2.0 * B * H * A * (2 * w.d_h + w.d_r)
    f_up = 4.0 * B * (n2 + d.max_slots) * w.d_c * H * w.d_h
    return {"workload": w.name + "_chunk2", "t0": t0, "tokens": n2, "ms_per_call": ms,
            "attended_pairs_per_bh": A, "attn_gflop": f_attn / 1e9, "kv_gemm_gflop": f_up / 1e9,
            "tflops_end_to_end": (f_attn + f_up) / (ms * 1e-3) / 1e12,
            "attn_tflops_over_end_to_end_time": f_attn / (ms * 1e-3) / 1e12}


def run_layer_decode(w, steps, warmup, m, torch, workloads):
    """The whole layer from h at the speech-translation decode shape: for every
    token, mtla_layer_decode_step (input projections + RoPE, the fused core
    step, output projection), 512 steps per replay.  Weights and h are the
    seeded layer parameters at d_model = 512."""
    B, N = w.batch, w.n_tokens
    d = m.make_dims(B, w.heads, w.d_h, w.d_c, w.d_r, w.s, -(-N // w.s), "bf16")
    p = workloads.layer_params(w)
    bf = torch.bfloat16
    dev = {k: to_dev(v, torch.float32 if k == "w_hyp" else bf, torch) for k, v in p.items()}
    h_t = dev["h"].transpose(0, 1).contiguous()          # token-major: [N, B, d_model]
    pe = torch.empty(N, w.d_c, dtype=torch.float32, device="cuda")
    m.mtla_sinusoidal_pe(pe)
    cache = torch.zeros(B, d.max_slots, d.width, dtype=bf, device="cuda")
    open_acc = torch.zeros(B, 2, d.width, dtype=torch.float32, device="cuda")
    ws = torch.empty(m.mtla_layer_decode_workspace_bytes(d, w.d_model), dtype=torch.uint8, device="cuda")
    y = torch.empty(N, B, w.d_model, dtype=bf, device="cuda")
    pos = (torch.arange(1, N + 1, dtype=torch.int32, device="cuda")[:, None].expand(N, B).contiguous())

    def fn():
        for t in range(N):
            m.mtla_layer_decode_step(d, pos[t], h_t[t], dev["w_dkv"], dev["w_q"], dev["w_r"], dev["w_o"],
                                     dev["w_hyp"], pe, dev["w_uk"], dev["w_uv"], cache, open_acc, y[t], ws)
    g = capture(fn, torch)
    for _ in range(warmup):
        g.replay()
    ms = timed_graph(g, steps, torch)
    return {"workload": "layer_" + w.name, "d_model": w.d_model, "ms_per_step": ms,
            "tokens_per_s": B * N / (ms * 1e-3), "us_per_token_step": ms * 1e3 / N}


def run_layer_prefill(w, steps, warmup, m, torch, workloads):
    """The whole layer from h over the summarisation prefill (B=16, N=4096,
    d_model=512): input projections, mtla_prefill, output projection."""
    B, N = w.batch, w.n_tokens
    d = m.make_dims(B, w.heads, w.d_h, w.d_c, w.d_r, w.s, -(-N // w.s), "bf16")
    p = workloads.layer_params(w)
    bf = torch.bfloat16
    dev = {k: to_dev(v, torch.float32 if k == "w_hyp" else bf, torch) for k, v in p.items()}
    pe = torch.empty(N, w.d_c, dtype=torch.float32, device="cuda")
    m.mtla_sinusoidal_pe(pe)
    cache = torch.zeros(B, d.max_slots, d.width, dtype=bf, device="cuda")
    open_acc = torch.zeros(B, 2, d.width, dtype=torch.float32, device="cuda")
    ws = torch.empty(m.mtla_layer_prefill_workspace_bytes(d, w.d_model, 0, N), dtype=torch.uint8, device="cuda")
    y = torch.empty(B, N, w.d_model, dtype=bf, device="cuda")

    def fn():
        m.mtla_layer_prefill(d, 0, dev["h"], dev["w_dkv"], dev["w_q"], dev["w_r"], dev["w_o"], dev["w_hyp"], pe,
                             dev["w_uk"], dev["w_uv"], cache, open_acc, y, ws)
    g = capture(fn, torch)
    for _ in range(warmup):
        g.replay()
    ms = timed_graph(g, steps, torch)
    Nq = w.heads * (w.d_h + w.d_r)
    f_proj = 2.0 * B * N * w.d_model * (w.d_c + Nq + w.d_r + w.heads * w.d_h)
    A = attended_pairs(N, w.s)
    f_attn = 2.0 * B * w.heads * A * (2 * w.d_h + w.d_r)
    f_up = 4.0 * B * N * w.d_c * w.heads * w.d_h
    return {"workload": "layer_" + w.name, "d_model": w.d_model, "ms_per_call": ms,
            "gflop": (f_proj + f_attn + f_up) / 1e9,
            "tflops_end_to_end": (f_proj + f_attn + f_up) / (ms * 1e-3) / 1e12}


def run_reorder(w, steps, warmup, m, torch):
    """Beam-search reorder of a full decode state at the LLM shape: every
    sequence holds N+1 tokens (16,385 slots); each destination takes a random
    parent.  Pure data movement: the slot rows are read once and written once
    (cache contents are random, their values do not matter to a copy)."""
    B, N, H = w.batch, w.n_tokens, w.heads
    T = N + 1
    d = m.make_dims(B, H, w.d_h, w.d_c, w.d_r, w.s, -(-T // w.s), "bf16")
    gen = torch.Generator(device="cuda").manual_seed(5)
    cache_in = torch.randn(B, d.max_slots, d.width, device="cuda", generator=gen).to(torch.bfloat16)
    cache_out = torch.empty_like(cache_in)
    open_in = torch.randn(B, 2, d.width, device="cuda", generator=gen)
    open_out = torch.empty_like(open_in)
    pos = torch.full((B,), T, dtype=torch.int32, device="cuda")
    pos_out = torch.empty_like(pos)
    src = torch.randint(0, B, (B,), dtype=torch.int32, device="cuda", generator=gen)

    def fn():
        m.mtla_reorder_state(d, src, pos, cache_in, open_in, cache_out, open_out, pos_out)
    g = capture(fn, torch)
    for _ in range(warmup):
        g.replay()
    ms = timed_graph(g, steps, torch)
    moved = 2 * B * (-(-T // w.s)) * d.width * 2 + 2 * B * 2 * d.width * 4
    return {"workload": "beam_reorder_" + w.name, "ms_per_call": ms, "bytes_moved": moved,
            "GBps": moved / (ms * 1e-3) / 1e9, "frac_hbm": moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


# ---------------------------------------------------------------------------
# LLM-scale long-context step
# ---------------------------------------------------------------------------

def run_llm_decode(w, steps, warmup, m, torch, workloads):
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    B, N, H = w.batch, w.n_tokens, w.heads
    T = N + 1  # cache of N tokens, then the appended token N+1
    d = m.make_dims(B, H, w.d_h, w.d_c, w.d_r, w.s, -(-T // w.s), "bf16")
    bf = torch.bfloat16
    log(f"{w.name}: generating {B} x {T} latents")
    t0 = time.time()
    cache = torch.zeros(B, d.max_slots, d.width, dtype=bf, device="cuda")
    open_acc = torch.zeros(B, 2, d.width, dtype=torch.float32, device="cuda")
    pe = torch.empty(T, w.d_c, dtype=torch.float32, device="cuda")
    m.mtla_sinusoidal_pe(pe)
    wts = workloads.weights(w)
    w_hyp = to_dev(wts["w_hyp"], torch.float32, torch)
    w_uk, w_uv = to_dev(wts["w_uk"], bf, torch), to_dev(wts["w_uv"], bf, torch)
    c_dev = torch.empty(B, T, w.d_c, dtype=bf, device="cuda")
    kr_dev = torch.empty(B, T, w.d_r, dtype=bf, device="cuda")

    def gen(b):
        lat = workloads.latents(w, b, T)
        return b, lat["c"], lat["k_r"]
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        for b, cc, kk in ex.map(gen, range(B)):
            c_dev[b].copy_(torch.from_numpy(cc))
            kr_dev[b].copy_(torch.from_numpy(kk))
    qry = workloads.batch_queries(w, 1)
    q_c = to_dev(qry["q_c"][:, 0].copy(), bf, torch)
    q_r = to_dev(qry["q_r"][:, 0].copy(), bf, torch)
    log(f"{w.name}: inputs in {time.time() - t0:.1f}s; building the cache")
    one = torch.ones(B, dtype=torch.int32, device="cuda")
    m.mtla_merge_append(d, one, c_dev[:, :N].contiguous(), kr_dev[:, :N].contiguous(), w_hyp, pe,
                        cache, open_acc)
    pos = torch.full((B,), T, dtype=torch.int32, device="cuda")
    c_t, kr_t = c_dev[:, N].contiguous(), kr_dev[:, N].contiguous()
    out = torch.empty(B, H, w.d_h, dtype=bf, device="cuda")
    ws = torch.zeros(m.mtla_decode_workspace_bytes(d), dtype=torch.uint8, device="cuda")

    def step():
        m.mtla_decode_step(d, pos, c_t, kr_t, w_hyp, pe, q_c, q_r, w_uk, w_uv, cache, open_acc,
                           out, ws)
    g = capture(step, torch)
    reps = max(steps, 20)
    for _ in range(max(warmup, 5)):
        g.replay()
    ms = timed_graph(g, reps, torch)
    # latent attention alone
    q_lat = torch.empty(B, H, d.width, dtype=torch.float32, device="cuda")
    m.mtla_absorb_query(d, q_c, q_r, w_uk, q_lat)
    o_lat = torch.empty(B, H, d.d_c, dtype=torch.float32, device="cuda")
    aws = m.decode_attention_workspace(d)
    ga = capture(lambda: m.mtla_decode_attention(d, pos, q_lat, cache, o_lat, aws), torch)
    for _ in range(5):
        ga.replay()
    ams = timed_graph(ga, reps, torch)
    n_slots = -(-T // w.s)
    cache_bytes = B * n_slots * d.width * 2
    weight_bytes = 2 * H * w.d_h * w.d_c * 2
    flops = 2.0 * B * H * n_slots * (2 * w.d_c + w.d_r) + 4.0 * B * H * w.d_h * w.d_c
    splits, fused = m.mtla_decode_plan(d)
    rec = {"workload": w.name, "ms_per_step": ms, "tokens_per_s": B / (ms * 1e-3),
           "plan": {"splits": splits, "fused": fused},
           "slots_per_seq": n_slots, "step_GBps": (cache_bytes + weight_bytes) / (ms * 1e-3) / 1e9,
           "step_frac_hbm": (cache_bytes + weight_bytes) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "step_tflops": flops / (ms * 1e-3) / 1e12,
           "attention": {"kernels": ("decode_stream_kernel" if (w.d_c, w.d_r) == (512, 64) else "decode_mfma_kernel")
                                        + (" + split_merge_kernel" if splits > 1 else ""),
                         "avg_call_us": ams * 1e3,
                                "algorithmic_bytes_per_launch": cache_bytes,
                                "GBps": cache_bytes / (ams * 1e-3) / 1e9,
                                "frac_hbm": cache_bytes / (ams * 1e-3) / 1e9 / HBM_PEAK_GBS}}
    return rec, (out, cache)


# ---------------------------------------------------------------------------
# copy kernel of known size: calibrates the HBM byte counters
# ---------------------------------------------------------------------------

def run_copy(steps, warmup, torch):
    """A plain elementwise copy (torch.neg) of 1 GiB of bf16: its FETCH_SIZE and
    WRITE_SIZE counters are divided into the known byte count to give the
    factor applied to the same counters of the MTLA kernels."""
    n = 1 << 29
    x = torch.randn(n, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    y = torch.empty_like(x)
    for _ in range(max(warmup, 1)):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        torch.neg(x, out=y)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = x.numel() * x.element_size()
    return {"workload": "copy_bf16_1GiB", "kernel": "torch.neg", "bytes_read": nbytes,
            "bytes_written": nbytes, "ms_per_call": ms, "GBps": 2 * nbytes / (ms * 1e-3) / 1e9}


# ---------------------------------------------------------------------------
# CPU baseline (the fp64 oracle) and parity of the headline run
# ---------------------------------------------------------------------------

def cpu_baseline_and_parity(w, dl, torch):
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    lat, qry, wts = dl.host_inputs
    out = dl.out.float().cpu().numpy().transpose(1, 0, 2, 3)   # [B, N, H, d_h]
    seqs = list(range(w.batch))
    errs = []
    passes = 0
    with threadpool_limits(1):
        t0 = time.time()
        # whole passes over the workload until at least 10 s of CPU work
        while passes == 0 or time.time() - t0 < 10.0:
            for b in seqs:
                ref = oracle.incremental(lat["c"][b], lat["k_r"][b], qry["q_c"][b], qry["q_r"][b],
                                         wts["w_hyp"], wts["w_uk"], wts["w_uv"], w.s, w.softmax_scale)
                if passes == 0:
                    errs.append(oracle.max_rel_err(out[b], ref))
            passes += 1
        dt = time.time() - t0
    tokens = passes * len(seqs) * w.n_tokens
    return ({"value": tokens / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
             "sample": f"{passes} pass(es) over the whole workload ({len(seqs)} sequences x {w.n_tokens} "
                       f"tokens), fp64 NumPy, one thread, {dt:.1f} s"},
            float(max(errs)))


# ---------------------------------------------------------------------------
# measured HBM traffic of the headline kernel (rocprofv3 counter passes)
# ---------------------------------------------------------------------------

def measured_traffic(kernel):
    """Bytes per launch of `kernel` from profiles/traffic.json (two rocprofv3
    --pmc passes, FETCH_SIZE and WRITE_SIZE, scaled by the factors a plain copy
    of known size gives).  None when there is no record for this kernel or when
    its sources have changed since the counters were taken."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None, "no counter record"
    if rec.get("kernel") != kernel:
        return None, "no counter record for this kernel"
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(root, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec["sources_sha256"]:
        return None, "kernel sources changed since the counters were taken"
    return rec["bytes_per_launch"], rec["profile"]


# ---------------------------------------------------------------------------

def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the MTLA path here is "
              "single-GPU and no multi-GPU figure is produced.", file=sys.stderr)
        return 2
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import torch
    import workloads
    import temporally_compressed_latent_amd as m
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1

    W = workloads.WORKLOADS
    if args.only:
        fn = {"st_decode_s2": lambda: run_decode_loop(W[1], args.steps, args.warmup, m, torch, workloads)[0],
              "st_decode_s4": lambda: run_decode_loop(W[2], args.steps, args.warmup, m, torch, workloads)[0],
              "prefill": lambda: run_prefill(W[3], args.steps, args.warmup, m, torch, workloads)[0],
              "prefill_chunk": lambda: run_prefill_chunk(W[3], args.steps, args.warmup, m, torch, workloads),
              "reorder": lambda: run_reorder(W[4], args.steps, args.warmup, m, torch),
              "layer_decode": lambda: run_layer_decode(W[1], args.steps, args.warmup, m, torch, workloads),
              "backward": lambda: run_backward(W[3], args.steps, args.warmup, m, torch, workloads),
              "layer_prefill": lambda: run_layer_prefill(W[3], args.steps, args.warmup, m, torch, workloads),
              "llm_decode": lambda: run_llm_decode(W[4], args.steps, args.warmup, m, torch, workloads)[0],
              "copy": lambda: run_copy(args.steps, args.warmup, torch)}
        print(json.dumps(fn[args.only]()), flush=True)
        return 0

    w = W[1]
    head, dl = run_decode_loop(w, args.steps, args.warmup, m, torch, workloads)
    log("headline:", json.dumps(head))
    comps = {}
    if not args.no_components:
        comps["st_decode_b50_n2048_s4"] = run_decode_loop(W[2], args.steps, args.warmup, m, torch, workloads)[0]
        log("s4:", json.dumps(comps["st_decode_b50_n2048_s4"]))
        torch.cuda.empty_cache()
        comps["sum_prefill_b16_n4096_s3"] = run_prefill(W[3], args.steps, args.warmup, m, torch, workloads)[0]
        log("prefill:", json.dumps(comps["sum_prefill_b16_n4096_s3"]))
        torch.cuda.empty_cache()
        comps["sum_prefill_b16_n4096_s3_chunk2"] = run_prefill_chunk(W[3], args.steps, args.warmup, m, torch,
                                                                     workloads)
        log("prefill chunk:", json.dumps(comps["sum_prefill_b16_n4096_s3_chunk2"]))
        torch.cuda.empty_cache()
        comps["layer_st_decode_b50_n512_s2"] = run_layer_decode(W[1], args.steps, args.warmup, m, torch, workloads)
        log("layer decode:", json.dumps(comps["layer_st_decode_b50_n512_s2"]))
        comps["layer_sum_prefill_b16_n4096_s3"] = run_layer_prefill(W[3], args.steps, args.warmup, m, torch,
                                                                    workloads)
        log("layer prefill:", json.dumps(comps["layer_sum_prefill_b16_n4096_s3"]))
        torch.cuda.empty_cache()
        comps["sum_prefill_b16_n4096_s3_backward"] = run_backward(W[3], args.steps, args.warmup, m, torch, workloads)
        log("backward:", json.dumps(comps["sum_prefill_b16_n4096_s3_backward"]))
        torch.cuda.empty_cache()
        comps["llm_decode_b64_n32768_s2"] = run_llm_decode(W[4], args.steps, args.warmup, m, torch, workloads)[0]
        log("llm:", json.dumps(comps["llm_decode_b64_n32768_s2"]))
        torch.cuda.empty_cache()
        comps["beam_reorder_llm_decode_b64_n32768_s2"] = run_reorder(W[4], args.steps, args.warmup, m, torch)
        log("reorder:", json.dumps(comps["beam_reorder_llm_decode_b64_n32768_s2"]))
    cpu, err = (None, None)
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        cpu, err = cpu_baseline_and_parity(w, dl, torch)

    k = head["dominant_kernel"]
    achieved = k["GBps"]
    traffic, traffic_src = measured_traffic(k["name"])
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded Gaussian latents, rope keys, queries and fan-in-scaled weights",
        "config": {"workload": w.name, "batch": w.batch, "tokens": w.n_tokens, "heads": w.heads,
                   "d_h": w.d_h, "d_c": w.d_c, "d_r": w.d_r, "s": w.s,
                   "tokens_per_step": head["tokens_per_step"], "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": k["name"], "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "traffic_unit": "bytes per launch",
                     "traffic_source": traffic_src, "avg_launch_us": k["avg_launch_us"],
                     "algorithmic_bytes_per_launch": k["algorithmic_bytes_per_launch"]},
        "plan": head["plan"],
        "cpu_baseline": cpu,
        "max_rel_err": err,
        "step_GBps": head["step_GBps"],
        "us_per_token": head["us_per_token"],
        "components": comps,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
