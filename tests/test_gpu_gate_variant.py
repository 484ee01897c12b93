"""GPU: the per-position gate (MTLA_FLAG_GATE_PER_POSITION: W_hyp with s
rows, token t takes row (t-1) mod s) through every entry point that gates a
token -- merge/append (token by token and chunked from mid-block), the decode
step (fused and staged shapes), prefill and its continuation, the layer
prefill, and the training backward -- against the oracle's per-position
gate."""
import numpy as np
import pytest
import torch

import oracle
import temporally_compressed_latent_amd as m
import workloads
from tests import oracle_ref
from tests.gpu_util import DEV, Case, bits, host, make_case, tol

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("d_c,s", [(64, 3), (256, 2), (256, 4), (512, 3)])
def test_merge_per_position(dtype, d_c, s):
    """Tokens 1..k one at a time, then the rest in one chunk that starts
    inside a block: cache, open-slot state and gates against the oracle.
    d_c 256 and 512 take the merge's lane-parallel gate path, 64 the
    generic one."""
    B, N, d_r = 3, 29, 16
    print(f"merge per-position d_c={d_c} s={s} {dtype}", flush=True)
    inp = workloads.boundary_case(40 + s, B, N, 2, 8, d_c, d_r, dtype, gate_rows=s)
    dims = m.make_dims(B, 2, 8, d_c, d_r, s, -(-N // s) + 2, dtype, gate_per_position=True)
    g = Case(dims, inp, N + 4)
    k = s + 1  # the chunk starts at token k + 1, inside the second block when s > 1
    gates = torch.empty(B, N, dtype=torch.float32, device=DEV)
    for t in range(1, k + 1):
        gout = torch.empty(B, 1, dtype=torch.float32, device=DEV)
        g.append(torch.full((B,), t, dtype=torch.int32, device=DEV), t - 1, t, gate_out=gout)
        gates[:, t - 1] = gout[:, 0]
    gout = torch.empty(B, N - k, dtype=torch.float32, device=DEV)
    g.append(torch.full((B,), k + 1, dtype=torch.int32, device=DEV), k, N, gate_out=gout)
    gates[:, k:] = gout
    cache = host(g.cache)
    for b in range(B):
        want, w = oracle_ref.merged_cache(inp["c"][b], inp["k_r"][b], inp["w_hyp"], s)
        n = want.shape[0]
        assert oracle.max_rel_err(cache[b, :n], want) <= tol(dtype), b
        assert np.max(np.abs(host(gates)[b] - w)) <= 2e-6, b
        assert oracle.max_rel_err(host(g.open_state(N))[b], want[n - 1]) <= 1e-5, b


@pytest.mark.parametrize("shape,dtype,s,B,N", [
    ("st", "bf16", 2, 3, 70),    # the fused decode step (its merge picks the row by place)
    ("st", "bf16", 3, 2, 50),
    ("st", "fp32", 2, 2, 40),    # staged: merge, absorb, attention, up-projection
    ("odd", "fp32", 3, 2, 30),
])
def test_decode_step_per_position(shape, dtype, s, B, N):
    print(f"decode step per-position {shape} {dtype} s={s} B={B} N={N}", flush=True)
    inp, g = make_case(shape, 7, B, N, s, dtype, gate_per_position=True)
    out = host(g.step_loop(N))
    want, caches = oracle_ref.loop_outputs(inp, B, N, s, g.d.softmax_scale)
    oracle_ref.assert_steps(out, want, tol(dtype))
    for b, cache in enumerate(caches):
        assert oracle.max_rel_err(host(g.cache)[b, :cache.shape[0]], cache) <= tol(dtype), b


def test_decode_step_per_position_equal_rows_is_one_row_gate():
    """With every W_hyp row equal the per-position fused step gives the
    one-row fused step's outputs, cache and open-slot state bit for bit (the
    gate arithmetic is the same; only the row's address differs)."""
    inp, g1 = make_case("st", 8, 2, 21, 3, "bf16")
    inp2 = dict(inp)
    inp2["w_hyp"] = np.tile(inp["w_hyp"], (3, 1))
    dims = m.make_dims(2, 8, 64, 256, 32, 3, g1.d.max_slots, "bf16", gate_per_position=True)
    g2 = Case(dims, inp2, 25)
    x1, x2 = g1.step_loop(21), g2.step_loop(21)
    assert torch.equal(bits(x1), bits(x2))
    assert torch.equal(bits(g1.cache), bits(g2.cache))
    assert torch.equal(g1.open_acc, g2.open_acc)


@pytest.mark.parametrize("shape,dtype,s,B,N,t0", [
    ("st", "bf16", 3, 2, 200, 0),   # MFMA prefill
    ("st", "bf16", 3, 2, 160, 71),  # continuation from inside a block
    ("st", "fp32", 2, 2, 90, 0),
    ("odd", "fp32", 4, 2, 41, 13),
])
def test_prefill_per_position(shape, dtype, s, B, N, t0):
    print(f"prefill per-position {shape} {dtype} s={s} N={N} t0={t0}", flush=True)
    inp, g = make_case(shape, 9, B, N, s, dtype, gate_per_position=True)
    if t0:
        g.prefill(t0)
        out = host(g.prefill_at(t0, N - t0))
    else:
        out = host(g.prefill(N))
    want = np.stack([oracle_ref.parallel(inp, b, N, s, g.d.softmax_scale)[0] for b in range(B)])
    oracle_ref.assert_steps(out, want[:, t0:], tol(dtype))


def _gpu_backward_pp(inp, s, dtype):
    B, N, d_c = inp["c"].shape
    H, d_h = inp["q_c"].shape[2], inp["q_c"].shape[3]
    d_r = inp["k_r"].shape[2]
    d = m.make_dims(B, H, d_h, d_c, d_r, s, max(1, -(-N // s)), dtype, gate_per_position=True)
    st = d.torch_dtype
    dev = {k: torch.from_numpy(np.ascontiguousarray(inp[k], np.float32)).to(DEV).to(
        torch.float32 if k == "w_hyp" else st) for k in ("c", "k_r", "q_c", "q_r", "w_hyp", "w_uk", "w_uv", "d_o")}
    pe = torch.empty(N, d_c, dtype=torch.float32, device=DEV)
    m.mtla_sinusoidal_pe(pe)
    out = {"dc": torch.empty(B, N, d_c, dtype=st, device=DEV), "dk_r": torch.empty(B, N, d_r, dtype=st, device=DEV),
           "dq_c": torch.empty(B, N, H, d_h, dtype=st, device=DEV),
           "dq_r": torch.empty(B, N, H, d_r, dtype=st, device=DEV),
           "dw_hyp": torch.full((s, d_c), float("nan"), dtype=torch.float32, device=DEV),
           "dw_uk": torch.empty(H, d_h, d_c, dtype=torch.float32, device=DEV),
           "dw_uv": torch.empty(H, d_h, d_c, dtype=torch.float32, device=DEV)}
    ws = torch.empty(m.mtla_prefill_backward_workspace_bytes(d, N), dtype=torch.uint8, device=DEV)
    m.mtla_prefill_backward(d, dev["q_c"], dev["q_r"], dev["c"], dev["k_r"], dev["w_hyp"], pe, dev["w_uk"],
                            dev["w_uv"], dev["d_o"], out["dq_c"], out["dq_r"], out["dc"], out["dk_r"],
                            out["dw_hyp"], out["dw_uk"], out["dw_uv"], ws)
    torch.cuda.synchronize()
    return d, {k: host(v) for k, v in out.items()}


@pytest.mark.parametrize("seed,B,N,s,H,d_h,d_c,d_r,dtype", [
    (21, 2, 37, 3, 2, 16, 32, 8, "fp32"),
    (22, 2, 200, 3, 8, 64, 256, 32, "bf16"),   # the MFMA backward
    (23, 1, 45, 4, 2, 8, 64, 8, "fp32"),
])
def test_backward_per_position(seed, B, N, s, H, d_h, d_c, d_r, dtype):
    print(f"backward per-position seed={seed} N={N} s={s} {dtype}", flush=True)
    inp = workloads.boundary_case(seed, B, N, H, d_h, d_c, d_r, dtype, gate_rows=s)
    inp["d_o"] = workloads.quantize(np.random.default_rng(seed + 7).standard_normal((B, N, H, d_h)).astype(np.float32),
                                    dtype)
    d, got = _gpu_backward_pp(inp, s, dtype)
    per = [oracle.parallel_backward(inp["c"][b], inp["k_r"][b], inp["q_c"][b], inp["q_r"][b], inp["w_hyp"],
                                    inp["w_uk"], inp["w_uv"], s, d.softmax_scale, inp["d_o"][b]) for b in range(B)]
    for k in ("dc", "dk_r", "dq_c", "dq_r"):
        err = oracle.max_rel_err(got[k], np.stack([r[k] for r in per]))
        assert err <= tol(dtype), (k, err)
    for k in ("dw_hyp", "dw_uk", "dw_uv"):
        want = sum(r[k] for r in per)
        assert got[k].shape == want.shape, k
        err = oracle.max_rel_err(got[k], want)
        assert err <= tol(dtype), (k, err)
