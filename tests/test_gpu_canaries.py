"""GPU: canary guard bands.  Every workspace and output of the entry points
that use one sits between two 64 KiB bands of 0xA5 bytes, and is passed with
exactly its required size; after the call, both bands must be intact: no
kernel writes outside the ranges the header states.  Covers the one-kernel
and multi-kernel decode paths, prefill and its continuation, the training
backward and the layer entry points."""
import math

import numpy as np
import pytest
import torch

import temporally_compressed_latent_amd as m
import workloads
from tests.gpu_util import DEV, make_case, tdev

pytestmark = pytest.mark.gpu

G = 1 << 16
CANARY = 0xA5


class Guarded:
    """A device buffer of `nbytes` (a view typed as `dtype` with `shape`)
    between two guard bands."""

    def __init__(self, nbytes, dtype=torch.uint8, shape=None):
        self.n = int(nbytes)
        self.buf = torch.full((G + self.n + G,), CANARY, dtype=torch.uint8, device=DEV)
        inner = self.buf[G:G + self.n]
        self.t = inner if dtype == torch.uint8 else inner.view(dtype)
        if shape is not None:
            self.t = self.t.view(shape)

    def intact(self):
        torch.cuda.synchronize()
        return bool((self.buf[:G] == CANARY).all()) and bool((self.buf[G + self.n:] == CANARY).all())


def guarded_like(shape, dtype):
    return Guarded(math.prod(shape) * torch.tensor([], dtype=dtype).element_size(), dtype, shape)


@pytest.mark.parametrize("shape,B,N,s,max_slots", [("st", 3, 130, 2, None),       # one kernel
                                                   ("llm", 4, 1301, 2, 700),     # multi-split pipeline
                                                   ("st", 5, 900, 4, 800)])
def test_decode_and_step_workspaces(shape, B, N, s, max_slots):
    inp, g = make_case(shape, 21, B, N, s, "bf16", max_slots=max_slots)
    d = g.d
    g.append(torch.ones(B, dtype=torch.int32, device=DEV), 0, N - 1)
    pos = torch.full((B,), N, dtype=torch.int32, device=DEV)
    ws = Guarded(m.mtla_decode_workspace_bytes(d))
    out = guarded_like((B, d.heads, d.d_h), torch.bfloat16)
    m.mtla_decode_step(d, pos, g.c[:, N - 1].contiguous(), g.k_r[:, N - 1].contiguous(), g.w_hyp, g.pe,
                       g.q_c[:, N - 1].contiguous(), g.q_r[:, N - 1].contiguous(), g.w_uk, g.w_uv, g.cache,
                       g.open_acc, out.t, ws.t)
    assert ws.intact() and out.intact()
    ws2 = Guarded(m.mtla_decode_workspace_bytes(d))
    out2 = guarded_like((B, d.heads, d.d_h), torch.bfloat16)
    m.mtla_decode(d, pos, g.q_c[:, N - 1].contiguous(), g.q_r[:, N - 1].contiguous(), g.w_uk, g.w_uv, g.cache,
                  out2.t, ws2.t)
    assert ws2.intact() and out2.intact()
    assert torch.isfinite(out.t.float()).all() and torch.isfinite(out2.t.float()).all()


@pytest.mark.parametrize("t0,N", [(0, 300), (100, 200)])
def test_prefill_workspaces(t0, N):
    B, s = 2, 3
    inp, g = make_case("st", 22, B, t0 + N, s, "bf16")
    d = g.d
    if t0:
        g.prefill(t0)
    ws = Guarded(m.mtla_prefill_at_workspace_bytes(d, t0, N))
    out = guarded_like((B, N, d.heads, d.d_h), torch.bfloat16)
    sl = slice(t0, t0 + N)
    m.mtla_prefill_at(d, t0, g.q_c[:, sl].contiguous(), g.q_r[:, sl].contiguous(), g.c[:, sl].contiguous(),
                      g.k_r[:, sl].contiguous(), g.w_hyp, g.pe, g.w_uk, g.w_uv, g.cache, g.open_acc, out.t, ws.t)
    assert ws.intact() and out.intact()
    assert torch.isfinite(out.t.float()).all()


def test_backward_workspace_and_gradients():
    B, N, s = 2, 200, 3
    inp, g = make_case("st", 23, B, N, s, "bf16")
    d = g.d
    rng = np.random.default_rng(5)
    d_o = tdev(workloads.quantize(rng.standard_normal((B, N, d.heads, d.d_h)).astype(np.float32), "bf16"),
               torch.bfloat16)
    ws = Guarded(m.mtla_prefill_backward_workspace_bytes(d, N))
    grads = [guarded_like(t.shape, t.dtype) for t in (g.q_c, g.q_r, g.c, g.k_r)]
    gw = [guarded_like((d.d_c,), torch.float32), guarded_like(tuple(g.w_uk.shape), torch.float32),
          guarded_like(tuple(g.w_uv.shape), torch.float32)]
    m.mtla_prefill_backward(d, g.q_c, g.q_r, g.c, g.k_r, g.w_hyp, g.pe, g.w_uk, g.w_uv, d_o,
                            *[x.t for x in grads], *[x.t for x in gw], ws.t)
    assert ws.intact()
    for x in grads + gw:
        assert x.intact()
        assert torch.isfinite(x.t.float()).all()


def test_layer_workspaces():
    w = workloads.small(1, batch=2, n_tokens=64)
    p = workloads.layer_params(w)
    d = m.make_dims(w.batch, w.heads, w.d_h, w.d_c, w.d_r, w.s, -(-w.n_tokens // w.s) + 1, "bf16")
    dev = {k: tdev(v, torch.float32 if k == "w_hyp" else torch.bfloat16) for k, v in p.items()}
    pe = torch.empty(w.n_tokens + 2, w.d_c, dtype=torch.float32, device=DEV)
    m.mtla_sinusoidal_pe(pe)
    cache = torch.zeros(w.batch, d.max_slots, d.width, dtype=torch.bfloat16, device=DEV)
    open_acc = torch.zeros(w.batch, 2, d.width, dtype=torch.float32, device=DEV)
    n = w.n_tokens - 1
    ws = Guarded(m.mtla_layer_prefill_workspace_bytes(d, w.d_model, 0, n))
    y = guarded_like((w.batch, n, w.d_model), torch.bfloat16)
    m.mtla_layer_prefill(d, 0, dev["h"][:, :n].contiguous(), dev["w_dkv"], dev["w_q"], dev["w_r"], dev["w_o"],
                         dev["w_hyp"], pe, dev["w_uk"], dev["w_uv"], cache, open_acc, y.t, ws.t)
    assert ws.intact() and y.intact()
    ws2 = Guarded(m.mtla_layer_decode_workspace_bytes(d, w.d_model))
    y2 = guarded_like((w.batch, w.d_model), torch.bfloat16)
    m.mtla_layer_decode_step(d, torch.full((w.batch,), w.n_tokens, dtype=torch.int32, device=DEV),
                             dev["h"][:, n].contiguous(), dev["w_dkv"], dev["w_q"], dev["w_r"], dev["w_o"],
                             dev["w_hyp"], pe, dev["w_uk"], dev["w_uv"], cache, open_acc, y2.t, ws2.t)
    assert ws2.intact() and y2.intact()
