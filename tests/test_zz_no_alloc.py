"""The allocation-free decode step (mtla_decode_step_noalloc) against
mtla_decode_step with a caller workspace.  Both run the same kernels, so the
outputs, slot caches and open-slot states must be the same bits; the outputs
also follow the oracle.  Two calls in a row share the one static scratch, the
second on a smaller input.  The size limit is checked on the CPU."""
import ctypes

import pytest
import torch

import oracle
import temporally_compressed_latent_amd as m
from tests import oracle_ref
from tests.gpu_util import DEV, bits, host, make_case


def _states(shape, seed, B, N, s, max_slots):
    """Two identical device states holding tokens 1..N-1 of each sequence."""
    inp, a = make_case(shape, seed, B, N, s, "bf16", max_slots=max_slots)
    _, b = make_case(shape, seed, B, N, s, "bf16", max_slots=max_slots)
    ones = torch.ones(B, dtype=torch.int32, device=DEV)
    a.append(ones, 0, N - 1)
    b.append(ones, 0, N - 1)
    return inp, a, b


def _step(g, N, noalloc):
    d = g.d
    pos = torch.full((d.batch,), N, dtype=torch.int32, device=DEV)
    out = torch.empty(d.batch, d.heads, d.d_h, dtype=g.st, device=DEV)
    args = (d, pos, g.c[:, N - 1].contiguous(), g.k_r[:, N - 1].contiguous(), g.w_hyp, g.pe,
            g.q_c[:, N - 1].contiguous(), g.q_r[:, N - 1].contiguous(), g.w_uk, g.w_uv, g.cache, g.open_acc, out)
    if noalloc:
        m.mtla_decode_step_noalloc(*args)
    else:
        m.mtla_decode_step(*args, g.ws_dec)
    return out


# (shape, seed, B, N, s, max_slots): the LLM-scale row (576 wide) with four
# and then two slot splits, so the call runs the multi-kernel path whose
# kernels keep queries, split partials and latent outputs in the scratch; the
# second call is smaller than the first
CALLS = [("llm", 21, 8, 3001, 2, 1600), ("llm", 22, 3, 1301, 2, 700)]


@pytest.mark.gpu
def test_noalloc_step_equals_workspace_step():
    for shape, seed, B, N, s, ms in CALLS:
        print(f"noalloc step: {shape} B={B} N={N} s={s} max_slots={ms}", flush=True)
        inp, a, b = _states(shape, seed, B, N, s, ms)
        splits, fused = m.mtla_decode_plan(a.d)
        assert splits > 1 and not fused
        x = _step(a, N, noalloc=True)
        y = _step(b, N, noalloc=False)
        torch.cuda.synchronize()
        assert torch.equal(bits(x), bits(y))
        assert torch.equal(bits(a.cache), bits(b.cache))
        assert torch.equal(a.open_acc, b.open_acc)
        got = host(x)
        for bb in sorted({0, B - 1}):
            slots, _ = oracle_ref.merged_cache(inp["c"][bb, :N], inp["k_r"][bb, :N], inp["w_hyp"], s)
            want = oracle.decode_absorbed(inp["q_c"][bb, N - 1], inp["q_r"][bb, N - 1], slots, inp["w_uk"],
                                          inp["w_uv"], a.d.d_c, a.d.softmax_scale)
            assert oracle.max_rel_err(got[bb], want) <= 1e-2, bb


def test_noalloc_rejects_dims_past_the_scratch():
    """Dims whose workspace exceeds the static scratch fail with
    MTLA_ERR_WORKSPACE before anything touches a GPU (the pointers here are
    never dereferenced)."""
    d = m.make_dims(512, 32, 128, 512, 64, 2, 16385)
    assert m.mtla_decode_workspace_bytes(d) > (32 << 20)
    fake = 0x10000
    st = m.lib().mtla_decode_step_noalloc(ctypes.byref(d), fake, fake, fake, fake, fake, 8, fake, fake, fake,
                                          fake, fake, fake, fake, None)
    assert st == m.MTLA_ERR_WORKSPACE
    assert "static scratch" in m.last_error()
