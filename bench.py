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
the timed graph replay (HIP events on the stream the kernels run on) divided
by the 512 launches.  Its algorithmic bytes are the slot rows read plus W_UK
and W_UV (summed over the 512 launches, divided by 512); the per-token terms
(the token's latent and rope key, queries, outputs, the written slot row, the
fp32 open-slot state, the pe row and W_hyp) are reported beside them, not in
them.  ``measured_peaks`` are this GPU's achievable rates from the library's
own measurement kernels (a streaming read of 4 GiB, MFMA chains on registers,
the library's MFMA GEMM on a large product, an empty kernel as a graph node),
taken in the same run; each roofline fraction is given against the published
peak and against the measured one.

``cpu_baseline`` is the fp64 oracle (test infrastructure) timed on this host
with its BLAS on every core the process may use, over a bounded sample of each
workload (stated in ``sample``, scaled to the whole workload where it is a
subset); the host's CPU model and NumPy's BLAS are recorded with it.  It is a
reported baseline, not a target.
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
                        "prefill_chunk, llm_decode, reorder, layer_decode, layer_prefill, layer_fp32, backward; "
                        "measurement kernels: copy (the counter-calibration copy), hbm_read, mfma_peak, "
                        "gemm_peak, launch_floor, tile_stream, load_pattern)")
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
        # W_UV also in the fused step's tile order, packed once (the weights
        # are resident inputs; the step reads them as whole lines)
        self.w_uv_tiles = torch.empty(m.mtla_w_uv_tiles_bytes(d) // 2, dtype=bf, device="cuda")
        m.mtla_pack_w_uv_tiles(d, self.w_uv, self.w_uv_tiles)
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
            m.mtla_decode_step_tiles(d, self.pos[t], self.c[t], self.k_r[t], self.w_hyp, self.pe,
                                     self.q_c[t], self.q_r[t], self.w_uk, self.w_uv, self.w_uv_tiles,
                                     self.cache, self.open_acc, self.out[t], self.ws)


def step_bytes(w, t):
    """Bytes of one decode-step launch at token t (bf16 storage), as
    (slot rows read, W_UK and W_UV, per-token terms).  The first two are the
    algorithmic bytes of the roofline; the per-token terms (token latent and
    rope key, queries, outputs, the written slot row, the fp32 open-slot state
    read and written, the pe row, W_hyp) are counted apart."""
    e, B, H = 2, w.batch, w.heads
    n = -(-t // w.s)
    cache = B * n * w.width * e
    weights = 2 * H * w.d_h * w.d_c * e
    token = (B * (w.width * e + H * (w.d_h + w.d_r) * e + H * w.d_h * e + w.width * e
                  + 2 * w.width * 4 + w.d_c * 4) + w.d_c * 4)
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
    weight_b = sum(p[1] for p in per_t)
    token_b = sum(p[2] for p in per_t)
    alg_b = cache_b + weight_b            # slot rows + W_UK and W_UV (the roofline's bytes)
    rec = {"workload": w.name, "ms_per_step": ms, "tokens_per_step": tokens,
           "tokens_per_s": tokens / (ms * 1e-3), "us_per_token": ms * 1e3 / w.n_tokens,
           "plan": {"splits": splits, "fused": fused},
           "entry_point": "mtla_decode_step_tiles (W_UV packed once by mtla_pack_w_uv_tiles before the loop)",
           "step_GBps": alg_b / (ms * 1e-3) / 1e9,
           "cache_GBps": cache_b / (ms * 1e-3) / 1e9,
           "bytes_per_step": {"cache": cache_b, "w_uk_w_uv": weight_b, "per_token_terms": token_b}}
    if fused:
        us = ms * 1e3 / w.n_tokens
        rec["dominant_kernel"] = {
            "name": "decode_step_wave_kernel" if w.d_c == 256 else "decode_step_kernel",
            "launches_per_step": w.n_tokens, "avg_launch_us": us,
            "algorithmic_bytes_per_launch": alg_b / w.n_tokens,
            "per_token_bytes_per_launch": token_b / w.n_tokens,
            "GBps": alg_b / w.n_tokens / (us * 1e-6) / 1e9}
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
    # the three stages mtla_prefill runs, each replayed alone from its own
    # graph (HIP events on the stream they run on): the attention kernel's own
    # time is the roofline's
    P = torch.empty(B, N, d.width, dtype=bf, device="cuda")
    kc = torch.empty(B, H, m.prefill_slot_keys(d, N), w.d_h, dtype=torch.float16, device="cuda")
    v = torch.empty_like(kc)
    out2 = torch.empty_like(out)
    stages = {"partials": lambda: m.mtla_prefill_partials(d, c, k_r, w_hyp, pe, cache, open_acc, P),
              "keys": lambda: m.mtla_prefill_keys(d, P, w_uk, w_uv, kc, v),
              "attention": lambda: m.mtla_prefill_attention(d, q_c, q_r, P, w_uk, w_uv, kc, v, out2)}
    stage_ms = {}
    for name, fn_s in stages.items():
        gs = capture(fn_s, torch)
        for _ in range(warmup):
            gs.replay()
        stage_ms[name] = timed_graph(gs, steps, torch)
    t_attn = stage_ms["attention"]
    rec = {"workload": w.name, "ms_per_call": ms, "attended_pairs_per_bh": A,
           "attn_gflop": f_attn / 1e9, "kv_gemm_gflop": f_up / 1e9,
           "tflops_end_to_end": (f_attn + f_up) / (ms * 1e-3) / 1e12,
           "attn_tflops_over_end_to_end_time": f_attn / (ms * 1e-3) / 1e12,
           "stages_ms": stage_ms,
           "roofline": {"bound": "mfma", "kernel": "prefill_attn_kernel",
                        "achieved": (f_attn + f_up) / (t_attn * 1e-3) / 1e12,
                        "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": (f_attn + f_up) / (t_attn * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                        "avg_launch_us": t_attn * 1e3, "algorithmic_flops_per_launch": f_attn + f_up,
                        "algorithmic_flops": "2 x attended pairs x heads x (2 d_h + d_r), explicit per-head form, "
                                             "plus each query's own K^C and V (4 x tokens x d_c x heads x d_h), "
                                             "formed in the kernel",
                        "operands": "fp16 scores and values, bf16 diagonal up-projection"}}
    del P, kc, v, out2
    return rec, (out, q_c, q_r, lat, qry, wts)


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
    # K^C and V of the new tokens (each query's own key) and of the completed
    # slots they attend, recomputed from the latent cache
    f_up = 4.0 * B * (n2 + m.prefill_slot_keys(d, n2, t0)) * w.d_c * H * w.d_h
    return {"workload": w.name + "_chunk2", "t0": t0, "tokens": n2, "ms_per_call": ms,
            "attended_pairs_per_bh": A, "attn_gflop": f_attn / 1e9, "kv_gemm_gflop": f_up / 1e9,
            "tflops_end_to_end": (f_attn + f_up) / (ms * 1e-3) / 1e12,
            "attn_tflops_over_end_to_end_time": f_attn / (ms * 1e-3) / 1e12}


def run_layer_decode(w, steps, warmup, m, torch, workloads):
    """The whole layer from h at the speech-translation decode shape: for every
    token, mtla_layer_decode_step_tiles (input projections + RoPE, the fused
    core step, output projection; W_UV packed into tile order once), 512
    steps per replay.  Weights and h are the seeded layer parameters at
    d_model = 512."""
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
    w_uv_tiles = torch.empty(m.mtla_w_uv_tiles_bytes(d) // 2, dtype=bf, device="cuda")
    m.mtla_pack_w_uv_tiles(d, dev["w_uv"], w_uv_tiles)

    def fn():
        for t in range(N):
            m.mtla_layer_decode_step_tiles(d, pos[t], h_t[t], dev["w_dkv"], dev["w_q"], dev["w_r"], dev["w_o"],
                                           dev["w_hyp"], pe, dev["w_uk"], dev["w_uv"], w_uv_tiles, cache,
                                           open_acc, y[t], ws)
    g = capture(fn, torch)
    for _ in range(warmup):
        g.replay()
    ms = timed_graph(g, steps, torch)
    return {"workload": "layer_" + w.name, "d_model": w.d_model, "ms_per_step": ms,
            "tokens_per_s": B * N / (ms * 1e-3), "us_per_token_step": ms * 1e3 / N,
            "entry_point": "mtla_layer_decode_step_tiles (W_UV packed once)"}


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
# this GPU's achievable rates, from the library's measurement kernels
# ---------------------------------------------------------------------------

def timed_calls(fn, reps, torch):
    """Average ms of `reps` eager calls of fn, HIP events on torch's stream
    (the stream the library's kernels are launched on)."""
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def run_step_timeline(w, m, torch, workloads):
    """Phases of the fused decode step over the whole loop, from the step's
    timeline instance (the real-time counter, 100 MHz, read in each
    workgroup): medians over launches and workgroups, in microseconds, by
    quarter of the loop (the cache grows from 1 to ceil(N/s) slots)."""
    import numpy as np
    dl = DecodeLoop(w, m, torch, workloads)
    d, N = dl.dims, w.n_tokens
    # room for the most workgroups a launch can have (one head per group);
    # rows of workgroups that did not run stay zero
    tl = torch.zeros(N, 8 * w.heads * (-(-w.batch // 8)) * 16, dtype=torch.int64, device="cuda")

    def loop():
        for t in range(N):
            m.mtla_calib_step_timeline(d, dl.pos[t], dl.c[t], dl.k_r[t], dl.w_hyp, dl.pe, dl.q_c[t], dl.q_r[t],
                                       dl.w_uk, dl.w_uv, dl.w_uv_tiles, dl.cache, dl.open_acc, dl.out[t],
                                       dl.ws, tl[t])
    g_tl = capture(loop, torch)
    g_plain = capture(dl.step, torch)
    g_tl.replay()
    ms_tl = timed_graph(g_tl, 3, torch)
    ms_plain = timed_graph(g_plain, 3, torch)
    x = tl.cpu().numpy().astype(np.int64).reshape(N, -1, 16)
    live = x[:, :, 0] != 0
    us = 1e-2  # one tick of the 100 MHz counter
    start = np.where(live, x[:, :, 0], np.iinfo(np.int64).max).min(axis=1)
    end = np.where(live, x[:, :, 13], 0).max(axis=1)
    att_end = x[:, :, 4:12].max(axis=2)
    ph = {"dispatch_to_entry": x[:, :, 0] - start[:, None],
          "position": x[:, :, 1] - x[:, :, 0],
          "w_uk_query_absorb": x[:, :, 2] - x[:, :, 1],
          "gate_merge_q_tilde": x[:, :, 3] - x[:, :, 2],
          "attention_slowest_wave": att_end - x[:, :, 3],
          "combine": x[:, :, 12] - att_end,
          "up_projection": x[:, :, 13] - x[:, :, 12],
          "workgroup_total": x[:, :, 13] - x[:, :, 0]}
    quarters = {}
    for qi in range(4):
        sl = slice(qi * N // 4, (qi + 1) * N // 4)
        rec = {k: float(np.median(v[sl][live[sl]]) * us) for k, v in ph.items()}
        rec["launch_span"] = float(np.median((end - start)[sl]) * us)
        nxt = (start[1:] - end[:-1])[sl.start:min(sl.stop, N - 1)]
        rec["gap_to_next_launch"] = float(np.median(nxt) * us)
        quarters[f"tokens_{sl.start + 1}_{sl.stop}"] = rec
    return {"workload": w.name, "kernel": "decode_step_wave_kernel (timeline instance)",
            "workgroups_per_launch": int(live[0].sum()), "ms_per_loop_timeline": ms_tl,
            "ms_per_loop_plain": ms_plain, "phases_us_median": quarters}


def run_launch_floor(steps, warmup, m, torch, n=512):
    """A graph of n empty kernels: the per-launch floor of any one-kernel step
    replayed the way the decode loops are."""
    g = capture(lambda: [m.mtla_calib_empty() for _ in range(n)], torch)
    for _ in range(max(warmup, 1)):
        g.replay()
    ms = timed_graph(g, max(steps, 5), torch)
    return {"kernel": "calib_empty_kernel", "launches_per_graph": n, "us_per_launch": ms * 1e3 / n}


def run_hbm_read(steps, warmup, m, torch, gib=4):
    """Streaming read of a 4 GiB buffer (16x the last-level cache) at several
    grid sizes; the best is the achievable read bandwidth."""
    nbytes = gib << 30
    x = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sweep = {}
    for wg in (256, 512, 1024, 2048, 4096, 8192):
        sink = torch.empty(wg * 4, dtype=torch.int32, device="cuda")
        for _ in range(max(warmup, 1)):
            m.mtla_calib_stream_read(x, wg, sink)
        ms = timed_calls(lambda: m.mtla_calib_stream_read(x, wg, sink), max(steps, 5), torch)
        sweep[wg] = nbytes / (ms * 1e-3) / 1e9
    best = max(sweep, key=sweep.get)
    del x
    return {"kernel": "calib_read_kernel", "bytes": nbytes, "GBps": sweep[best], "workgroups": best,
            "sweep_GBps": {str(k): v for k, v in sweep.items()}, "frac_of_published": sweep[best] / HBM_PEAK_GBS}


def run_tile_stream(steps, warmup, m, torch):
    """The long-cache decode attention's load schedule with no arithmetic
    (mtla_calib_tile_stream) over a cache of the LLM-scale shape (64 x 16,385
    rows of 1,152 B), 4 splits: the ceiling of that access pattern, with and
    without the non-temporal hint, contiguous and interleaved split ranges."""
    seqs, n, splits = 64, 16385, 4
    rows = torch.full((seqs, n, 1152), 0x11, dtype=torch.uint8, device="cuda")
    sink = torch.empty(seqs * splits * 8, dtype=torch.int32, device="cuda")
    nbytes = rows.numel()
    rec = {"kernel": "calib_tile_stream_kernel", "bytes": nbytes, "splits": splits, "GBps": {}}
    for il in (False, True):
        for nt in (False, True):
            for _ in range(max(warmup, 1)):
                m.mtla_calib_tile_stream(rows, splits, il, nt, sink)
            ms = timed_calls(lambda: m.mtla_calib_tile_stream(rows, splits, il, nt, sink), max(steps, 5), torch)
            key = ("interleaved" if il else "contiguous") + ("_nt" if nt else "")
            rec["GBps"][key] = nbytes / (ms * 1e-3) / 1e9
            rec.setdefault("us", {})[key] = ms * 1e3
    del rows
    return rec


def run_load_pattern(steps, warmup, m, torch):
    """A compute unit's issue cost of one 16-byte-per-lane load instruction
    from L2-resident data (mtla_calib_load_pattern, one workgroup of 8 waves
    x 32 loads per compute unit): a contiguous kilobyte per instruction
    against 16 rows x 64 bytes (the MFMA operand layout of row-major rows,
    the decode step's former cache-row and present W_UV loads)."""
    wg = 256
    buf = torch.ones(1 << 20, dtype=torch.int32, device="cuda")  # 4 MiB: stays in L2
    cyc = torch.zeros(wg + 64, dtype=torch.int32, device="cuda")
    rec = {"kernel": "calib_load_pattern_kernel", "workgroups": wg, "loads_per_wave": 32, "waves": 8}
    for name, pat in (("contiguous_1KB", 0), ("16_rows_x_64B", 1)):
        meds = []
        for _ in range(max(steps, 5) + max(warmup, 1)):
            m.mtla_calib_load_pattern(pat, wg, buf, cyc)
            torch.cuda.synchronize()
            meds.append(float(cyc[:wg].float().median()))
        med = sorted(meds[max(warmup, 1):])[len(meds[max(warmup, 1):]) // 2]
        rec[name] = {"cycles_per_workgroup": med, "cycles_per_load_instruction": med / (8 * 32),
                     "bytes_per_cycle": 8 * 32 * 1024 / med}
    return rec


def run_mfma_peak(steps, warmup, m, torch):
    """MFMA chains on registers (32x32x16, fp32 accumulation), bf16 and fp16
    operands, 2 and 4 waves per SIMD; the best is the matrix cores' rate."""
    rec = {"kernel": "calib_mfma_kernel"}
    for name, f16 in (("bf16", False), ("f16", True)):
        best = 0.0
        for wg in (512, 1024):
            out = torch.empty(wg * 256, dtype=torch.float32, device="cuda")
            iters = 4096
            flops = m.mtla_calib_mfma(f16, wg, iters, out)
            for _ in range(max(warmup, 1)):
                m.mtla_calib_mfma(f16, wg, iters, out)
            ms = timed_calls(lambda: m.mtla_calib_mfma(f16, wg, iters, out), max(steps, 5), torch)
            best = max(best, flops / (ms * 1e-3) / 1e12)
        rec[name + "_TFLOPs"] = best
        rec[name + "_frac_of_published"] = best / BF16_PEAK_TFLOPS
    return rec


def run_gemm_peak(steps, warmup, m, torch):
    """The library's own bf16 MFMA GEMM (the layer GEMM, through
    mtla_output_project) on a large product: y[16384, 8192] = o W_O^T with
    K = 8192."""
    R, dm, H, d_h = 16384, 8192, 64, 128
    d = m.make_dims(1, H, d_h, 256, 32, 2, 1, "bf16")
    gen = torch.Generator(device="cuda").manual_seed(3)
    o = (torch.randn(R, H, d_h, device="cuda", generator=gen) * 0.1).to(torch.bfloat16)
    w_o = (torch.randn(dm, H * d_h, device="cuda", generator=gen) * 0.01).to(torch.bfloat16)
    y = torch.empty(R, dm, dtype=torch.bfloat16, device="cuda")
    for _ in range(max(warmup, 1)):
        m.mtla_output_project(d, o, w_o, y)
    ms = timed_calls(lambda: m.mtla_output_project(d, o, w_o, y), max(steps, 5), torch)
    flops = 2.0 * R * dm * H * d_h
    del o, w_o, y
    return {"kernel": "layer_gemm_mfma_kernel", "shape": [R, dm, H * d_h], "ms_per_call": ms,
            "TFLOPs": flops / (ms * 1e-3) / 1e12, "frac_of_published": flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}


def run_gemm_vs_blas(steps, warmup, m, torch):
    """The library's layer GEMM as a plain product (mtla_output_project,
    y = o W^T) beside torch.mm on the ROCm BLAS, on the two projection shapes
    of the summarisation layer prefill (16 x 4096 tokens, K = H d_h = 512):
    N = 1056 (the input projection's width, c + q^C + q^R + k^R) and N = 512
    (the output projection's).  A comparison point only: the layer's own
    input projection also applies RoPE and scatters in its epilogue."""
    R, H, d_h = 65536, 8, 64
    d = m.make_dims(1, H, d_h, 256, 32, 2, 1, "bf16")
    gen = torch.Generator(device="cuda").manual_seed(5)
    out = []
    for N in (1056, 512):
        o = (torch.randn(R, H, d_h, device="cuda", generator=gen) * 0.1).to(torch.bfloat16)
        w = (torch.randn(N, H * d_h, device="cuda", generator=gen) * 0.05).to(torch.bfloat16)
        y = torch.empty(R, N, dtype=torch.bfloat16, device="cuda")
        yb = torch.empty(R, N, dtype=torch.bfloat16, device="cuda")
        a2, wt = o.view(R, H * d_h), w.t()
        for _ in range(max(warmup, 1)):
            m.mtla_output_project(d, o, w, y)
            torch.mm(a2, wt, out=yb)
        ms_own = timed_calls(lambda: m.mtla_output_project(d, o, w, y), max(steps, 5), torch)
        ms_blas = timed_calls(lambda: torch.mm(a2, wt, out=yb), max(steps, 5), torch)
        flops = 2.0 * R * N * H * d_h
        out.append({"shape": [R, N, H * d_h], "own_ms": ms_own, "blas_ms": ms_blas,
                    "own_TFLOPs": flops / (ms_own * 1e-3) / 1e12, "blas_TFLOPs": flops / (ms_blas * 1e-3) / 1e12,
                    "max_abs_diff": float((y.float() - yb.float()).abs().max())})
        del o, w, y, yb, a2, wt
    return {"kernel": "layer_gemm_mfma_kernel vs torch.mm", "products": out}


# ---------------------------------------------------------------------------
# the single fp32 layer (prefill of 64 tokens, 64-step decode), timed
# ---------------------------------------------------------------------------

def run_layer_fp32(w, steps, warmup, m, torch, workloads):
    """The fp32 single-layer workload from h: one mtla_layer_prefill over its
    64 tokens, and the 64-step mtla_layer_decode_step loop from an empty
    cache (the two schedules of the same layer); each replayed from a graph.
    Outputs are kept for parity against the oracle's layer."""
    B, N = w.batch, w.n_tokens
    d = m.make_dims(B, w.heads, w.d_h, w.d_c, w.d_r, w.s, -(-N // w.s), "fp32")
    p = workloads.layer_params(w)
    f32 = torch.float32
    dev = {k: to_dev(v, f32, torch) for k, v in p.items()}
    pe = torch.empty(N, w.d_c, dtype=f32, device="cuda")
    m.mtla_sinusoidal_pe(pe)
    cache = torch.zeros(B, d.max_slots, d.width, dtype=f32, device="cuda")
    open_acc = torch.zeros(B, 2, d.width, dtype=f32, device="cuda")
    y_pre = torch.empty(B, N, w.d_model, dtype=f32, device="cuda")
    y_dec = torch.empty(N, B, w.d_model, dtype=f32, device="cuda")
    wsp = torch.empty(m.mtla_layer_prefill_workspace_bytes(d, w.d_model, 0, N), dtype=torch.uint8, device="cuda")
    wsd = torch.empty(m.mtla_layer_decode_workspace_bytes(d, w.d_model), dtype=torch.uint8, device="cuda")
    h_t = dev["h"].transpose(0, 1).contiguous()
    pos = torch.arange(1, N + 1, dtype=torch.int32, device="cuda")[:, None].expand(N, B).contiguous()

    def prefill():
        m.mtla_layer_prefill(d, 0, dev["h"], dev["w_dkv"], dev["w_q"], dev["w_r"], dev["w_o"], dev["w_hyp"], pe,
                             dev["w_uk"], dev["w_uv"], cache, open_acc, y_pre, wsp)

    def decode():
        for t in range(N):
            m.mtla_layer_decode_step(d, pos[t], h_t[t], dev["w_dkv"], dev["w_q"], dev["w_r"], dev["w_o"],
                                     dev["w_hyp"], pe, dev["w_uk"], dev["w_uv"], cache, open_acc, y_dec[t], wsd)
    gp, gd = capture(prefill, torch), capture(decode, torch)
    for _ in range(warmup):
        gp.replay()
        gd.replay()
    ms_p = timed_graph(gp, steps, torch)
    ms_d = timed_graph(gd, steps, torch)
    rec = {"workload": w.name, "prefill_ms": ms_p, "decode_loop_ms": ms_d,
           "prefill_tokens_per_s": B * N / (ms_p * 1e-3), "decode_tokens_per_s": B * N / (ms_d * 1e-3),
           "us_per_decode_step": ms_d * 1e3 / N}
    return rec, (p, y_pre.cpu().numpy(), y_dec.transpose(0, 1).cpu().numpy())


# ---------------------------------------------------------------------------
# CPU baselines (the fp64 oracle, timed on this host) and parity
# ---------------------------------------------------------------------------

def host_env():
    """The host the oracle runs on: usable cores, CPU model, NumPy's BLAS."""
    import numpy as np
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg.get("Build Dependencies", {}).get("blas", {})
        blas = f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:  # noqa: BLE001 - informational only
        pass
    return {"cores": cores, "cpu_model": model, "numpy": np.__version__, "blas": blas}


def _oracle_threads():
    from threadpoolctl import threadpool_limits
    return threadpool_limits(len(os.sched_getaffinity(0)))


def cpu_decode_loop(w, dl, min_s, torch):
    """The oracle's token-by-token loop over whole sequences of a decode-loop
    workload, until at least min_s seconds; also the parity of those
    sequences' GPU outputs: each step's [b, H, d_h] over the sequences done."""
    import numpy as np
    import oracle
    lat, qry, wts = dl.host_inputs
    out = dl.out.float().cpu().numpy().transpose(1, 0, 2, 3)   # [B, N, H, d_h]
    refs = []
    with _oracle_threads():
        t0 = time.time()
        while len(refs) < w.batch and (not refs or time.time() - t0 < min_s):
            b = len(refs)
            refs.append(oracle.incremental(lat["c"][b], lat["k_r"][b], qry["q_c"][b], qry["q_r"][b],
                                           wts["w_hyp"], wts["w_uk"], wts["w_uv"], w.s, w.softmax_scale))
        dt = time.time() - t0
    n = len(refs)
    want = np.stack(refs)
    got = out[:n]
    step_err = max(oracle.max_rel_err(got[:, t], want[:, t]) for t in range(w.n_tokens))
    tokens = n * w.n_tokens
    env = host_env()
    return ({"value": tokens / dt, "unit": "tokens/s", "cores": env["cores"], "kind": "oracle",
             "sample": f"sequences 0..{n - 1} of {w.batch}, all {w.n_tokens} tokens each (fp64 NumPy "
                       f"incremental loop, {dt:.1f} s); tokens/s needs no scaling", **env},
            float(step_err), n)


def cpu_prefill(w, inputs):
    """The oracle's dense masked N x N pass (every head) on sequence 0, scaled
    to the batch: attended-pair TFLOP/s of the whole prefill."""
    import oracle
    lat, qry, wts = inputs
    N = w.n_tokens
    with _oracle_threads():
        t0 = time.time()
        oracle.parallel(lat["c"][0], lat["k_r"][0], qry["q_c"][0], qry["q_r"][0], wts["w_hyp"], wts["w_uk"],
                        wts["w_uv"], w.s, w.softmax_scale)
        dt = time.time() - t0
    A = attended_pairs(N, w.s)
    f_attn = 2.0 * w.batch * w.heads * A * (2 * w.d_h + w.d_r)
    env = host_env()
    return {"value": f_attn / (dt * w.batch) / 1e12, "unit": "TFLOP/s (attended pairs)", "cores": env["cores"],
            "kind": "oracle", "sample": f"sequence 0 of {w.batch} (dense masked {N}x{N} pass, {w.heads} heads, "
                                        f"fp64 NumPy, {dt:.1f} s), scaled x{w.batch}",
            "seconds_scaled": dt * w.batch, **env}


def cpu_llm_step(w, workloads):
    """The oracle's merge of a 32,768-token history and one decode step over
    16,385 slots, for 4 of the 64 sequences, scaled x16."""
    import numpy as np
    import oracle
    seqs = (0, 21, 42, 63)
    T = w.n_tokens + 1
    wts = workloads.weights(w)
    qry = workloads.batch_queries(w, 1, seqs=seqs)
    lats = [workloads.latents(w, b, T) for b in seqs]
    with _oracle_threads():
        t0 = time.time()
        for k, lat in enumerate(lats):
            c = lat["c"].astype("float64")
            pe = oracle.sinusoidal_pe(T, w.d_c)
            g = oracle.gate(c, pe, wts["w_hyp"])
            x = np.concatenate([c, lat["k_r"]], axis=1)
            slots = oracle.merge_incremental(x, g, w.s)
            oracle.decode_absorbed(qry["q_c"][k, 0], qry["q_r"][k, 0], slots, wts["w_uk"], wts["w_uv"], w.d_c,
                                   w.softmax_scale)
        dt = time.time() - t0
    scale = w.batch / len(seqs)
    env = host_env()
    return {"value": w.batch / (dt * scale), "unit": "tokens/s", "cores": env["cores"], "kind": "oracle",
            "sample": f"sequences {list(seqs)} of {w.batch}: merge of {w.n_tokens} cached tokens plus the appended "
                      f"one and one decode step over {-(-T // w.s)} slots (fp64 NumPy, {dt:.1f} s), scaled "
                      f"x{scale:g}", **env}


def cpu_layer_fp32(w, gpu_out):
    """The oracle's full fp32 layer (both schedules) for the single-layer
    workload, and the parity of the GPU's outputs against it."""
    import oracle
    p, y_pre, y_dec = gpu_out
    with _oracle_threads():
        t0 = time.time()
        inc = oracle.layer(p["h"][0], p, w.heads, w.d_h, w.d_r, w.s, w.softmax_scale, "incremental")
        par = oracle.layer(p["h"][0], p, w.heads, w.d_h, w.d_r, w.s, w.softmax_scale, "parallel")
        dt = time.time() - t0
    env = host_env()
    err_pre = max(oracle.max_rel_err(y_pre[:, t], par[None, t]) for t in range(w.n_tokens))
    err_dec = max(oracle.max_rel_err(y_dec[:, t], inc[None, t]) for t in range(w.n_tokens))
    return ({"value": 2 * w.n_tokens / dt, "unit": "tokens/s", "cores": env["cores"], "kind": "oracle",
             "sample": f"the whole workload: the layer's {w.n_tokens}-token parallel pass and its incremental loop "
                       f"(fp64 NumPy, {dt:.2f} s)", **env},
            {"prefill": float(err_pre), "decode_loop": float(err_dec)})


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
    K, Wu = args.steps, args.warmup
    if args.only:
        fn = {"st_decode_s2": lambda: run_decode_loop(W[1], K, Wu, m, torch, workloads)[0],
              "st_decode_s4": lambda: run_decode_loop(W[2], K, Wu, m, torch, workloads)[0],
              "prefill": lambda: run_prefill(W[3], K, Wu, m, torch, workloads)[0],
              "prefill_chunk": lambda: run_prefill_chunk(W[3], K, Wu, m, torch, workloads),
              "reorder": lambda: run_reorder(W[4], K, Wu, m, torch),
              "layer_decode": lambda: run_layer_decode(W[1], K, Wu, m, torch, workloads),
              "backward": lambda: run_backward(W[3], K, Wu, m, torch, workloads),
              "layer_prefill": lambda: run_layer_prefill(W[3], K, Wu, m, torch, workloads),
              "layer_fp32": lambda: run_layer_fp32(W[0], K, Wu, m, torch, workloads)[0],
              "llm_decode": lambda: run_llm_decode(W[4], K, Wu, m, torch, workloads)[0],
              "copy": lambda: run_copy(K, Wu, torch),
              "hbm_read": lambda: run_hbm_read(K, Wu, m, torch),
              "tile_stream": lambda: run_tile_stream(K, Wu, m, torch),
              "mfma_peak": lambda: run_mfma_peak(K, Wu, m, torch),
              "gemm_peak": lambda: run_gemm_peak(K, Wu, m, torch),
              "gemm_vs_blas": lambda: run_gemm_vs_blas(K, Wu, m, torch),
              "launch_floor": lambda: run_launch_floor(K, Wu, m, torch),
              "load_pattern": lambda: run_load_pattern(K, Wu, m, torch),
              "step_timeline": lambda: run_step_timeline(W[1], m, torch, workloads)}
        print(json.dumps(fn[args.only]()), flush=True)
        return 0

    w = W[1]
    head, dl = run_decode_loop(w, K, Wu, m, torch, workloads)
    log("headline:", json.dumps(head))
    head_out = dl.out.float().cpu()
    dl_inputs = dl.host_inputs
    del dl
    floor = run_launch_floor(K, Wu, m, torch)
    log("launch floor:", json.dumps(floor))
    peaks = {"hbm_read": run_hbm_read(K, Wu, m, torch), "mfma": run_mfma_peak(K, Wu, m, torch),
             "gemm": run_gemm_peak(K, Wu, m, torch), "launch_floor_us": floor["us_per_launch"],
             "decode_tile_stream": run_tile_stream(K, Wu, m, torch),
             "load_pattern": run_load_pattern(K, Wu, m, torch)}
    log("measured peaks:", json.dumps(peaks))
    torch.cuda.empty_cache()
    comps, cpu_jobs = {}, []
    if not args.no_components:
        rec, dl4 = run_decode_loop(W[2], K, Wu, m, torch, workloads)
        rec["launch_floor_us"] = floor["us_per_launch"]
        comps["st_decode_b50_n2048_s4"] = rec
        s4_out, s4_inputs = dl4.out.float().cpu(), dl4.host_inputs
        del dl4
        log("s4:", json.dumps(rec))
        torch.cuda.empty_cache()
        rec, pre = run_prefill(W[3], K, Wu, m, torch, workloads)
        f16_peak = peaks["mfma"]["f16_TFLOPs"]
        rec["roofline"]["measured_peak"] = f16_peak
        rec["roofline"]["frac_of_measured"] = rec["roofline"]["achieved"] / f16_peak
        comps["sum_prefill_b16_n4096_s3"] = rec
        pre_inputs = pre[3:]
        del pre
        log("prefill:", json.dumps(rec))
        torch.cuda.empty_cache()
        comps["sum_prefill_b16_n4096_s3_chunk2"] = run_prefill_chunk(W[3], K, Wu, m, torch, workloads)
        log("prefill chunk:", json.dumps(comps["sum_prefill_b16_n4096_s3_chunk2"]))
        torch.cuda.empty_cache()
        comps["layer_st_decode_b50_n512_s2"] = run_layer_decode(W[1], K, Wu, m, torch, workloads)
        log("layer decode:", json.dumps(comps["layer_st_decode_b50_n512_s2"]))
        comps["layer_sum_prefill_b16_n4096_s3"] = run_layer_prefill(W[3], K, Wu, m, torch, workloads)
        log("layer prefill:", json.dumps(comps["layer_sum_prefill_b16_n4096_s3"]))
        rec, l0_out = run_layer_fp32(W[0], K, Wu, m, torch, workloads)
        comps["layer_fp32_b1_n64_s2"] = rec
        log("fp32 layer:", json.dumps(rec))
        torch.cuda.empty_cache()
        comps["sum_prefill_b16_n4096_s3_backward"] = run_backward(W[3], K, Wu, m, torch, workloads)
        log("backward:", json.dumps(comps["sum_prefill_b16_n4096_s3_backward"]))
        torch.cuda.empty_cache()
        comps["llm_decode_b64_n32768_s2"] = run_llm_decode(W[4], K, Wu, m, torch, workloads)[0]
        att = comps["llm_decode_b64_n32768_s2"]["attention"]
        ceil = peaks["decode_tile_stream"]["GBps"]["interleaved_nt"]
        att["load_schedule_ceiling_GBps"] = ceil
        att["frac_of_load_schedule_ceiling"] = att["GBps"] / ceil
        log("llm:", json.dumps(comps["llm_decode_b64_n32768_s2"]))
        torch.cuda.empty_cache()
        comps["beam_reorder_llm_decode_b64_n32768_s2"] = run_reorder(W[4], K, Wu, m, torch)
        log("reorder:", json.dumps(comps["beam_reorder_llm_decode_b64_n32768_s2"]))

    class _Held:  # host copies of a decode loop's outputs [N, B, H, d_h] and inputs
        def __init__(self, out, inputs):
            self.out = out
            self.host_inputs = inputs
    cpu, err = None, None
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        cpu, err, nseq = cpu_decode_loop(w, _Held(head_out, dl_inputs), 10.0, torch)
        if not args.no_components:
            c4, e4, _ = cpu_decode_loop(W[2], _Held(s4_out, s4_inputs), 5.0, torch)
            comps["st_decode_b50_n2048_s4"]["cpu_baseline"] = c4
            comps["st_decode_b50_n2048_s4"]["max_rel_err"] = e4
            comps["sum_prefill_b16_n4096_s3"]["cpu_baseline"] = cpu_prefill(W[3], pre_inputs)
            comps["llm_decode_b64_n32768_s2"]["cpu_baseline"] = cpu_llm_step(W[4], workloads)
            c0, e0 = cpu_layer_fp32(W[0], l0_out)
            comps["layer_fp32_b1_n64_s2"]["cpu_baseline"] = c0
            comps["layer_fp32_b1_n64_s2"]["max_rel_err"] = e0

    k = head["dominant_kernel"]
    achieved = k["GBps"]
    traffic, traffic_src = measured_traffic(k["name"])
    hbm_meas = peaks["hbm_read"]["GBps"]
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
                     "algorithmic_bytes_per_launch": k["algorithmic_bytes_per_launch"],
                     "algorithmic_bytes": "slot rows read + W_UK + W_UV (per-token terms apart)",
                     "per_token_bytes_per_launch": k["per_token_bytes_per_launch"],
                     "measured_peak": hbm_meas, "frac_of_measured": achieved / hbm_meas,
                     "launch_floor_us": floor["us_per_launch"]},
        "plan": head["plan"],
        "cpu_baseline": cpu,
        "max_rel_err": err,
        "max_rel_err_note": ("worst over the steps of each step's [b, H, d_h] output, over the sequences "
                             "the oracle ran" if err is not None else None),
        "step_GBps": head["step_GBps"],
        "us_per_token": head["us_per_token"],
        "bytes_per_step": head["bytes_per_step"],
        "measured_peaks": peaks,
        "components": comps,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
