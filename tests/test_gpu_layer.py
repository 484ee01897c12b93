"""GPU: the decoder layer around the core (mtla_project_inputs,
mtla_output_project, mtla_layer_prefill, mtla_layer_decode_step) against the
oracle's full layer (projections, RoPE, merge, attention, output projection)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import temporally_compressed_latent_amd as m
from tests import oracle_ref
from tests.gpu_util import DEV, host, tdev, tol

pytestmark = pytest.mark.gpu


def _setup(wid, gate_per_position=False, **kw):
    w = workloads.small(wid, **kw)
    p = workloads.layer_params(w)
    if gate_per_position:
        p["w_hyp"] = workloads.gate_rows_weights(w)
    d = m.make_dims(w.batch, w.heads, w.d_h, w.d_c, w.d_r, w.s, -(-w.n_tokens // w.s) + 1, w.dtype,
                    gate_per_position=gate_per_position)
    st = d.torch_dtype
    dev = {k: tdev(v, torch.float32 if k == "w_hyp" else st) for k, v in p.items()}
    pe = torch.empty(w.n_tokens + 2, w.d_c, dtype=torch.float32, device=DEV)
    m.mtla_sinusoidal_pe(pe)
    cache = torch.zeros(w.batch, d.max_slots, d.width, dtype=st, device=DEV)
    open_acc = torch.zeros(w.batch, 2, d.width, dtype=torch.float32, device=DEV)
    return w, p, d, dev, pe, cache, open_acc


def _oracle_layer(w, p, b, schedule, n=None):
    n = w.n_tokens if n is None else n
    return oracle.layer(p["h"][b, :n], p, w.heads, w.d_h, w.d_r, w.s, w.softmax_scale, schedule)


# (workload, overrides): the fp32 single-layer case as it stands, and the
# speech-translation shape (bf16, d_model 512) at a test-sized batch and length
LAYER_CASES = [(0, {}), (1, dict(batch=2, n_tokens=100)), (1, dict(batch=2, n_tokens=70, s=3)),
               # d_model 200: the GEMMs' K is not a multiple of their 64-wide K step
               (1, dict(batch=2, n_tokens=67, d_model=200))]


@pytest.mark.parametrize("wid,kw", LAYER_CASES)
def test_project_inputs_matches_oracle(wid, kw):
    w, p, d, dev, *_ = _setup(wid, **kw)
    B, T, H = w.batch, w.n_tokens, w.heads
    st = d.torch_dtype
    pos0_h = np.array([1 + 5 * b for b in range(B)], dtype=np.int32)    # sequences start at different tokens
    c = torch.empty(B, T, w.d_c, dtype=st, device=DEV)
    k_r = torch.empty(B, T, w.d_r, dtype=st, device=DEV)
    q_c = torch.empty(B, T, H, w.d_h, dtype=st, device=DEV)
    q_r = torch.empty(B, T, H, w.d_r, dtype=st, device=DEV)
    m.mtla_project_inputs(d, torch.from_numpy(pos0_h).to(DEV), dev["h"], dev["w_dkv"], dev["w_q"], dev["w_r"],
                          c, k_r, q_c, q_r)
    for b in range(B):
        lead = int(pos0_h[b]) - 1          # rows before the first token: RoPE position pos0 - 1 + t
        hf = np.zeros((lead + T, w.d_model))
        hf[lead:] = p["h"][b]
        want = oracle.project(hf, p, H, w.d_h, w.d_r)
        for got, ref in zip((c, k_r, q_c, q_r), want):
            assert oracle.max_rel_err(host(got)[b], ref[lead:]) <= tol(w.dtype), b


# one token per sequence (a decode step's projection) at batch sizes on both
# sides of the few-row GEMM's limits (16, 32, 48, 64 rows), at positions up to
# 2^15 so that the RoPE angle's range reduction is exercised
@pytest.mark.parametrize("wid,B", [(1, 1), (1, 17), (1, 50), (1, 64), (1, 65), (0, 50)])
def test_project_one_token_large_positions(wid, B):
    w, p, d, dev, *_ = _setup(wid, batch=B)
    H = w.heads
    st = d.torch_dtype
    g = np.random.default_rng(11 + B)
    pos0_h = g.integers(1, 1 << 15, size=B).astype(np.int32)
    pos0_h[0] = (1 << 15) - 1
    h1 = dev["h"][:, :1].contiguous()
    c = torch.empty(B, 1, w.d_c, dtype=st, device=DEV)
    k_r = torch.empty(B, 1, w.d_r, dtype=st, device=DEV)
    q_c = torch.empty(B, 1, H, w.d_h, dtype=st, device=DEV)
    q_r = torch.empty(B, 1, H, w.d_r, dtype=st, device=DEV)
    m.mtla_project_inputs(d, torch.from_numpy(pos0_h).to(DEV), h1, dev["w_dkv"], dev["w_q"], dev["w_r"],
                          c, k_r, q_c, q_r)
    for b in range(B):
        # projection of the one row (RoPE at position 0 is the identity), then
        # RoPE at the token's position pos0 - 1
        c0, kr0, qc0, qr0 = oracle.project(p["h"][b, :1], p, H, w.d_h, w.d_r)
        pos = int(pos0_h[b]) - 1
        want = (c0, oracle.rope(kr0, pos), qc0, oracle.rope(qr0, pos))
        for got, ref in zip((c, k_r, q_c, q_r), want):
            assert oracle.max_rel_err(host(got)[b], ref) <= tol(w.dtype), (b, pos)


@pytest.mark.parametrize("R", [37, 600])
@pytest.mark.parametrize("wid,kw", LAYER_CASES)
def test_output_project_matches_oracle(wid, kw, R):
    # 37 rows: the few-row kernel, three 16-row blocks, the last one ragged;
    # 600 rows: the tiled kernel, three 256-row tiles, the last one ragged
    w, p, d, dev, *_ = _setup(wid, **kw)
    H = w.heads
    g = np.random.default_rng(3)
    o = workloads.quantize(g.standard_normal((R, H, w.d_h)).astype(np.float32), w.dtype)
    y = torch.empty(R, w.d_model, dtype=d.torch_dtype, device=DEV)
    m.mtla_output_project(d, tdev(o, d.torch_dtype), dev["w_o"], y)
    want = o.reshape(R, -1).astype(np.float64) @ p["w_o"].astype(np.float64).T    # the layer's last step
    assert oracle.max_rel_err(host(y), want) <= tol(w.dtype)


@pytest.mark.parametrize("wid,kw", LAYER_CASES)
def test_layer_prefill_matches_oracle(wid, kw):
    w, p, d, dev, pe, cache, open_acc = _setup(wid, **kw)
    B, N = w.batch, w.n_tokens
    y = torch.empty(B, N, w.d_model, dtype=d.torch_dtype, device=DEV)
    ws = torch.empty(m.mtla_layer_prefill_workspace_bytes(d, w.d_model, 0, N), dtype=torch.uint8, device=DEV)
    m.mtla_layer_prefill(d, 0, dev["h"], dev["w_dkv"], dev["w_q"], dev["w_r"], dev["w_o"], dev["w_hyp"], pe,
                         dev["w_uk"], dev["w_uv"], cache, open_acc, y, ws)
    want = np.stack([_oracle_layer(w, p, b, "parallel") for b in range(B)])
    oracle_ref.assert_steps(host(y), want, tol(w.dtype))


@pytest.mark.parametrize("wid,kw", LAYER_CASES)
def test_layer_decode_loop_matches_oracle(wid, kw):
    w, p, d, dev, pe, cache, open_acc = _setup(wid, **kw)
    B, N = w.batch, w.n_tokens
    ws = torch.empty(m.mtla_layer_decode_workspace_bytes(d, w.d_model), dtype=torch.uint8, device=DEV)
    ys = []
    for t in range(1, N + 1):
        pos = torch.full((B,), t, dtype=torch.int32, device=DEV)
        y = torch.empty(B, w.d_model, dtype=d.torch_dtype, device=DEV)
        m.mtla_layer_decode_step(d, pos, dev["h"][:, t - 1].contiguous(), dev["w_dkv"], dev["w_q"], dev["w_r"],
                                 dev["w_o"], dev["w_hyp"], pe, dev["w_uk"], dev["w_uv"], cache, open_acc, y, ws)
        ys.append(host(y))
    got = np.stack(ys, axis=1)
    want = np.stack([_oracle_layer(w, p, b, "incremental") for b in range(B)])
    oracle_ref.assert_steps(got, want, tol(w.dtype))


@pytest.mark.parametrize("gate_per_position", [False, True])
def test_layer_prefill_in_chunks_then_decode(gate_per_position):
    """Layer prefill of tokens 1..40, then 41..70 as a chunk, then two decode
    steps: every output follows the oracle's layer over tokens 1..72; also
    with one W_hyp row per place in the block."""
    w, p, d, dev, pe, cache, open_acc = _setup(1, gate_per_position, batch=2, n_tokens=72, s=3)
    B, dm = w.batch, w.d_model
    outs = []
    for t0, n in ((0, 40), (40, 30)):
        y = torch.empty(B, n, dm, dtype=d.torch_dtype, device=DEV)
        ws = torch.empty(m.mtla_layer_prefill_workspace_bytes(d, dm, t0, n), dtype=torch.uint8, device=DEV)
        m.mtla_layer_prefill(d, t0, dev["h"][:, t0:t0 + n].contiguous(), dev["w_dkv"], dev["w_q"], dev["w_r"],
                             dev["w_o"], dev["w_hyp"], pe, dev["w_uk"], dev["w_uv"], cache, open_acc, y, ws)
        outs.append(host(y))
    ws = torch.empty(m.mtla_layer_decode_workspace_bytes(d, dm), dtype=torch.uint8, device=DEV)
    for t in (71, 72):
        y = torch.empty(B, dm, dtype=d.torch_dtype, device=DEV)
        m.mtla_layer_decode_step(d, torch.full((B,), t, dtype=torch.int32, device=DEV),
                                 dev["h"][:, t - 1].contiguous(), dev["w_dkv"], dev["w_q"], dev["w_r"], dev["w_o"],
                                 dev["w_hyp"], pe, dev["w_uk"], dev["w_uv"], cache, open_acc, y, ws)
        outs.append(host(y)[:, None])
    got = np.concatenate(outs, axis=1)
    want = np.stack([_oracle_layer(w, p, b, "incremental") for b in range(B)])
    oracle_ref.assert_steps(got, want, tol(w.dtype))


def test_layer_decode_step_tiles_equals_layer_decode_step():
    """mtla_layer_decode_step_tiles (W_UV packed into tile order) gives the
    bits of mtla_layer_decode_step over a decode loop: outputs, cache rows and
    open-slot state."""
    runs = []
    for tiles in (False, True):
        w, p, d, dev, pe, cache, open_acc = _setup(1, batch=3, n_tokens=60)
        B, dm = w.batch, w.d_model
        ws = torch.empty(m.mtla_layer_decode_workspace_bytes(d, dm), dtype=torch.uint8, device=DEV)
        packed = torch.empty(m.mtla_w_uv_tiles_bytes(d) // 2, dtype=d.torch_dtype, device=DEV)
        m.mtla_pack_w_uv_tiles(d, dev["w_uv"], packed)
        ys = []
        for t in range(1, w.n_tokens + 1):
            pos = torch.full((B,), t, dtype=torch.int32, device=DEV)
            y = torch.empty(B, dm, dtype=d.torch_dtype, device=DEV)
            args = (d, pos, dev["h"][:, t - 1].contiguous(), dev["w_dkv"], dev["w_q"], dev["w_r"], dev["w_o"],
                    dev["w_hyp"], pe, dev["w_uk"], dev["w_uv"])
            if tiles:
                m.mtla_layer_decode_step_tiles(*args, packed, cache, open_acc, y, ws)
            else:
                m.mtla_layer_decode_step(*args, cache, open_acc, y, ws)
            ys.append(y.view(torch.int16).clone())
        runs.append((torch.stack(ys), cache.view(torch.int16).clone(), open_acc.clone()))
    for a, b in zip(*runs):
        assert torch.equal(a, b)


def test_output_project_unaligned_output():
    """An output array that is 4-byte but not 16-byte aligned: the tiled
    GEMM stores column pairs instead of 16-byte chunks, with the same values."""
    w, p, d, dev, *_ = _setup(1, batch=2, n_tokens=40)
    H, R = w.heads, 600
    g = np.random.default_rng(5)
    o = workloads.quantize(g.standard_normal((R, H, w.d_h)).astype(np.float32), w.dtype)
    ot = tdev(o, d.torch_dtype)
    y_al = torch.empty(R, w.d_model, dtype=d.torch_dtype, device=DEV)
    base = torch.empty(R * w.d_model + 8, dtype=d.torch_dtype, device=DEV)
    y_un = base[2:2 + R * w.d_model].view(R, w.d_model)            # 4 bytes past a 16-byte boundary
    assert y_un.data_ptr() % 16 == 4
    m.mtla_output_project(d, ot, dev["w_o"], y_al)
    m.mtla_output_project(d, ot, dev["w_o"], y_un)
    assert torch.equal(y_al.view(torch.int16), y_un.view(torch.int16))
    want = o.reshape(R, -1).astype(np.float64) @ p["w_o"].astype(np.float64).T
    assert oracle.max_rel_err(host(y_un), want) <= tol(w.dtype)
