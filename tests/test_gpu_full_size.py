"""GPU: parity at the benchmark's full sizes, in the launch configuration
bench.py times, on outputs the oracle can compute one by one:

  * the speech-translation decode loops (B=50, 512 steps at s=2 and 2048
    steps at s=4): every step of every sequence against the oracle's
    token-by-token loop, each step's [B, H, d_h] output on its own;
  * the summarisation prefill (B=16, N=4096, s=3): sampled queries of four
    sequences against the oracle's one-query form of the parallel pass (each
    query position on its own), and their completed slots against the
    oracle's partial merges;
  * the LLM-scale step (B=64, a 32,768-token cache plus one appended token,
    s=2): the step's output and the appended slot of eight sequences against
    the oracle's merge and absorbed decode over all 16,385 slots.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import temporally_compressed_latent_amd as m
import workloads
from tests import oracle_ref
from tests.gpu_util import DEV, host, tdev, tol

pytestmark = pytest.mark.gpu


def _decode_loop_full_size(wid):
    """Every step of every sequence of a decode-loop workload, run by
    mtla_decode_step as the benchmark runs it, against the oracle's
    token-by-token loop: each step's [B, H, d_h] output on its own."""
    w = workloads.WORKLOADS[wid]
    B, N, H = w.batch, w.n_tokens, w.heads
    d = m.make_dims(B, H, w.d_h, w.d_c, w.d_r, w.s, -(-N // w.s), "bf16")
    lat, qry, wts = workloads.batch_latents(w), workloads.batch_queries(w), workloads.weights(w)
    bf = torch.bfloat16
    dev = {"c": tdev(lat["c"], bf), "k_r": tdev(lat["k_r"], bf), "q_c": tdev(qry["q_c"], bf),
           "q_r": tdev(qry["q_r"], bf), "w_hyp": tdev(wts["w_hyp"], torch.float32),
           "w_uk": tdev(wts["w_uk"], bf), "w_uv": tdev(wts["w_uv"], bf)}
    pe = torch.empty(N, w.d_c, dtype=torch.float32, device=DEV)
    m.mtla_sinusoidal_pe(pe)
    cache = torch.zeros(B, d.max_slots, d.width, dtype=bf, device=DEV)
    open_acc = torch.zeros(B, 2, d.width, dtype=torch.float32, device=DEV)
    ws = torch.zeros(m.mtla_decode_workspace_bytes(d), dtype=torch.uint8, device=DEV)
    assert m.mtla_decode_plan(d) == (1, True)  # the fused step the benchmark times
    print(f"full-size decode loop {w.name}: {N} steps at B={B}", flush=True)
    outs = torch.empty(B, N, H, w.d_h, dtype=bf, device=DEV)
    for t in range(1, N + 1):
        pos = torch.full((B,), t, dtype=torch.int32, device=DEV)
        o = torch.empty(B, H, w.d_h, dtype=bf, device=DEV)
        m.mtla_decode_step(d, pos, dev["c"][:, t - 1].contiguous(), dev["k_r"][:, t - 1].contiguous(),
                           dev["w_hyp"], pe, dev["q_c"][:, t - 1].contiguous(), dev["q_r"][:, t - 1].contiguous(),
                           dev["w_uk"], dev["w_uv"], cache, open_acc, o, ws)
        outs[:, t - 1] = o
    got, got_cache = host(outs), host(cache)
    inp = {"c": lat["c"], "k_r": lat["k_r"], "q_c": qry["q_c"], "q_r": qry["q_r"], "w_hyp": wts["w_hyp"],
           "w_uk": wts["w_uk"], "w_uv": wts["w_uv"]}
    print(f"full-size decode loop {w.name}: oracle for all {B} sequences", flush=True)
    want, slots = oracle_ref.loop_outputs(inp, B, N, w.s, d.softmax_scale)
    e = oracle_ref.step_errors(got, want)
    # reported beside the bar: the worst single sequence's step (its own
    # [H, d_h] normalised by its own largest output)
    per_seq = max(oracle.max_rel_err(got[b, t], want[b, t]) for b in range(B) for t in range(N))
    print(f"per-step max rel err: worst {e.max():.3e} at step {int(e.argmax()) + 1}, median {np.median(e):.3e}; "
          f"worst single sequence-step {per_seq:.3e}", flush=True)
    assert e.max() <= tol("bf16"), (int(e.argmax()) + 1, e.max())
    for b in range(B):
        assert oracle.max_rel_err(got_cache[b, :slots[b].shape[0]], slots[b]) <= tol("bf16"), b


def test_decode_loop_full_size():
    w = workloads.WORKLOADS[1]
    assert (w.batch, w.n_tokens, w.s) == (50, 512, 2)
    _decode_loop_full_size(1)


def test_decode_loop_s4_full_size():
    w = workloads.WORKLOADS[2]
    assert (w.batch, w.n_tokens, w.s) == (50, 2048, 4)
    _decode_loop_full_size(2)


def test_prefill_full_size_sampled():
    w = workloads.WORKLOADS[3]
    assert (w.batch, w.n_tokens, w.s) == (16, 4096, 3)
    B, N, H, s = w.batch, w.n_tokens, w.heads, w.s
    d = m.make_dims(B, H, w.d_h, w.d_c, w.d_r, s, -(-N // s), "bf16")
    lat, qry, wts = workloads.batch_latents(w), workloads.batch_queries(w), workloads.weights(w)
    bf = torch.bfloat16
    pe = torch.empty(N, w.d_c, dtype=torch.float32, device=DEV)
    m.mtla_sinusoidal_pe(pe)
    cache = torch.zeros(B, d.max_slots, d.width, dtype=bf, device=DEV)
    open_acc = torch.zeros(B, 2, d.width, dtype=torch.float32, device=DEV)
    out = torch.empty(B, N, H, w.d_h, dtype=bf, device=DEV)
    ws = torch.empty(m.mtla_prefill_workspace_bytes(d, N), dtype=torch.uint8, device=DEV)
    print("full-size prefill: B=16, N=4096", flush=True)
    m.mtla_prefill(d, tdev(qry["q_c"], bf), tdev(qry["q_r"], bf), tdev(lat["c"], bf), tdev(lat["k_r"], bf),
                   tdev(wts["w_hyp"], torch.float32), pe, tdev(wts["w_uk"], bf), tdev(wts["w_uv"], bf),
                   cache, open_acc, out, ws)
    got, got_cache = host(out), host(cache)
    pe_h = oracle.sinusoidal_pe(N, w.d_c)
    rng = np.random.default_rng(3)
    queries = sorted(set([1, 2, 3, 4, 5, 6, 127, 128, 129, 1000, 2047, 2048, 2049, 3000, N - 1, N]
                         + rng.integers(1, N + 1, size=24).tolist()))
    seqs = (0, 5, 10, B - 1)
    wants = []
    for b in seqs:
        print(f"full-size prefill: oracle for sequence {b}, {len(queries)} queries", flush=True)
        gate = oracle.gate(lat["c"][b], pe_h, wts["w_hyp"])
        x = np.concatenate([lat["c"][b], lat["k_r"][b]], axis=1).astype(np.float64)
        P = oracle.partial_merges(x, gate, s)
        wants.append(np.stack([oracle.prefill_query(P, i, qry["q_c"][b, i - 1], qry["q_r"][b, i - 1],
                                                    wts["w_uk"], wts["w_uv"], s, w.d_c, d.softmax_scale)
                               for i in queries]))
        # completed slots are the partial merges at the blocks' last tokens
        nfull = N // s
        assert oracle.max_rel_err(got_cache[b, :nfull], P[s - 1:nfull * s:s]) <= tol("bf16"), b
    # each sampled query position's [4, H, d_h] on its own
    rows = got[list(seqs)][:, [i - 1 for i in queries]]
    e = oracle_ref.assert_steps(rows, np.stack(wants), tol("bf16"))
    print(f"per-query max rel err: worst {e.max():.3e}", flush=True)


def test_llm_step_full_size_sampled():
    w = workloads.WORKLOADS[4]
    assert (w.batch, w.n_tokens, w.s) == (64, 32768, 2)
    B, N, H, s = w.batch, w.n_tokens, w.heads, w.s
    T = N + 1
    d = m.make_dims(B, H, w.d_h, w.d_c, w.d_r, s, -(-T // s), "bf16")
    bf = torch.bfloat16
    wts = workloads.weights(w)
    pe = torch.empty(T, w.d_c, dtype=torch.float32, device=DEV)
    m.mtla_sinusoidal_pe(pe)
    cache = torch.zeros(B, d.max_slots, d.width, dtype=bf, device=DEV)
    open_acc = torch.zeros(B, 2, d.width, dtype=torch.float32, device=DEV)
    c_dev = torch.empty(B, T, w.d_c, dtype=bf, device=DEV)
    kr_dev = torch.empty(B, T, w.d_r, dtype=bf, device=DEV)
    print("full-size LLM step: generating 64 x 32,769 latents", flush=True)

    def gen(b):
        lat = workloads.latents(w, b, T)
        return b, lat["c"], lat["k_r"]
    with ThreadPoolExecutor(16) as ex:
        for b, cc, kk in ex.map(gen, range(B)):
            c_dev[b].copy_(torch.from_numpy(cc))
            kr_dev[b].copy_(torch.from_numpy(kk))
    qry = workloads.batch_queries(w, 1)
    w_hyp = tdev(wts["w_hyp"], torch.float32)
    w_uk, w_uv = tdev(wts["w_uk"], bf), tdev(wts["w_uv"], bf)
    m.mtla_merge_append(d, torch.ones(B, dtype=torch.int32, device=DEV), c_dev[:, :N].contiguous(),
                        kr_dev[:, :N].contiguous(), w_hyp, pe, cache, open_acc)
    out = torch.empty(B, H, w.d_h, dtype=bf, device=DEV)
    ws = torch.zeros(m.mtla_decode_workspace_bytes(d), dtype=torch.uint8, device=DEV)
    print(f"full-size LLM step: plan {m.mtla_decode_plan(d)}", flush=True)
    m.mtla_decode_step(d, torch.full((B,), T, dtype=torch.int32, device=DEV), c_dev[:, N].contiguous(),
                       kr_dev[:, N].contiguous(), w_hyp, pe, tdev(qry["q_c"][:, 0].copy(), bf),
                       tdev(qry["q_r"][:, 0].copy(), bf), w_uk, w_uv, cache, open_acc, out, ws)
    got = host(out)
    for b in (0, 9, 18, 27, 37, 46, 55, B - 1):
        print(f"full-size LLM step: oracle for sequence {b}", flush=True)
        lat = workloads.latents(w, b, T)
        slots, _ = oracle_ref.merged_cache(lat["c"], lat["k_r"], wts["w_hyp"], s)
        want = oracle.decode_absorbed(qry["q_c"][b, 0], qry["q_r"][b, 0], slots, wts["w_uk"], wts["w_uv"], w.d_c,
                                      d.softmax_scale)
        err = oracle.max_rel_err(got[b], want)
        print(f"max rel err {err:.2e}", flush=True)
        assert err <= tol("bf16"), (b, err)
        # the appended token opened slot 16,385; it and the last completed
        # slot follow the oracle's merge
        row = host(cache[b, T // s - 1:T // s + 1])
        assert oracle.max_rel_err(row, slots[T // s - 1:T // s + 1]) <= tol("bf16"), b
