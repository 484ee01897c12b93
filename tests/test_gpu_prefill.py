"""GPU: stride-masked parallel prefill (mtla_prefill) against the oracle's
dense masked pass, and against the device's own token-by-token decode; chunked
prefill (mtla_prefill_at) against the oracle's incremental loop."""
import numpy as np
import pytest
import torch

import oracle
from tests import oracle_ref
from tests.gpu_util import DEV, bits, host, make_case, tol

pytestmark = pytest.mark.gpu

CASES = [
    # shape, dtype, portable, s, B, N
    ("st", "bf16", False, 3, 2, 300),
    ("st", "bf16", False, 1, 1, 200),
    ("st", "bf16", False, 2, 2, 129),
    ("st", "bf16", False, 7, 2, 5),     # s > N: every query sees only its own partial
    ("st", "bf16", False, 3, 3, 1),
    ("llm", "bf16", False, 2, 1, 160),
    ("st", "bf16", True, 3, 2, 100),
    ("st", "fp32", False, 4, 1, 64),
    ("odd", "fp32", False, 2, 2, 37),
    ("odd", "bf16", False, 3, 2, 29),
]


@pytest.mark.parametrize("shape,dtype,portable,s,B,N", CASES)
def test_prefill_matches_oracle(shape, dtype, portable, s, B, N):
    inp, g = make_case(shape, 7, B, N, s, dtype, portable)
    out = host(g.prefill(N))
    cache, acc = host(g.cache), host(g.open_state(N))
    ref = [oracle_ref.parallel(inp, b, N, s, g.d.softmax_scale) for b in range(B)]
    # each query position's [B, H, d_h] on its own (what a decode call at
    # that position returns)
    oracle_ref.assert_steps(out, np.stack([r[0] for r in ref]), tol(dtype))
    for b, (_, P) in enumerate(ref):
        n = oracle.num_slots(N, s)
        slot_rows = [min(s * k, N) - 1 for k in range(1, n + 1)]   # P at each block end
        assert oracle.max_rel_err(cache[b, :n], P[slot_rows]) <= tol(dtype)
        assert oracle.max_rel_err(acc[b], P[N - 1]) <= 1e-5


@pytest.mark.parametrize("shape,s,N,portable", [("st", 3, 200, False), ("llm", 2, 96, False),
                                                ("st", 2, 64, True)])
def test_prefill_equals_device_decode_loop(shape, s, N, portable):
    """The parallel pass and token-by-token decoding agree on the device: the
    same cache bits, the same open-slot state, outputs within tolerance."""
    inp, a = make_case(shape, 8, 2, N, s, "bf16", portable)
    _, b_ = make_case(shape, 8, 2, N, s, "bf16", portable)
    pre = host(a.prefill(N))
    loop = host(b_.decode_loop(N))
    assert torch.equal(bits(a.cache), bits(b_.cache))
    assert torch.equal(a.open_state(N), b_.open_state(N))
    oracle_ref.assert_steps(pre, loop, 1e-2)


@pytest.mark.parametrize("s,N1", [(3, 101), (2, 64), (4, 1)])
def test_prefill_then_decode_continues(s, N1):
    """Prefill N1 tokens (ending inside a block), then keep decoding: the
    outputs follow the oracle's incremental loop."""
    B, N = 2, 160
    inp, g = make_case("st", 9, B, N, s, "bf16")
    g.prefill(N1)
    cont = host(g.decode_loop(N, start=N1))
    want, _ = oracle_ref.loop_outputs(inp, B, N, s, g.d.softmax_scale)
    oracle_ref.assert_steps(cont, want[:, N1:], 1e-2)


@pytest.mark.parametrize("portable", [False, True])
def test_prefill_ignores_cache_rows_past_the_end(portable):
    B, N, s = 2, 150, 3
    inp, a = make_case("st", 10, B, N, s, "bf16", portable, max_slots=90)
    clean = a.prefill(N).clone()
    a.cache[:, oracle.num_slots(N, s):] = float("nan")
    again = a.prefill(N)
    assert torch.isfinite(again.float()).all()
    assert torch.equal(bits(clean), bits(again))


def test_prefill_bit_reproducible():
    B, N, s = 2, 513, 3
    inp, a = make_case("st", 11, B, N, s, "bf16")
    x = a.prefill(N).clone()
    y = a.prefill(N).clone()
    assert torch.equal(bits(x), bits(y))


AT_CASES = [
    # shape, dtype, portable, s, B, t0, N
    ("st", "bf16", False, 3, 2, 100, 200),   # t0 inside a block (100 = 3*33 + 1)
    ("st", "bf16", False, 2, 2, 128, 129),   # t0 at a block boundary
    ("st", "bf16", False, 4, 1, 63, 1),      # one new token, block still open
    ("st", "bf16", False, 3, 1, 2, 300),     # short prefix, long chunk
    ("st", "bf16", True, 3, 2, 50, 60),
    ("st", "fp32", False, 3, 1, 40, 50),
    ("llm", "bf16", False, 2, 1, 70, 90),
    ("odd", "bf16", False, 3, 2, 17, 20),
]


@pytest.mark.parametrize("shape,dtype,portable,s,B,t0,N", AT_CASES)
def test_prefill_at_matches_oracle(shape, dtype, portable, s, B, t0, N):
    """Prefill t0 tokens, then tokens t0+1 .. t0+N in one mtla_prefill_at
    call: outputs, slot rows and the open-slot state follow the oracle's
    token-by-token loop over all t0+N tokens."""
    T = t0 + N
    inp, g = make_case(shape, 12, B, T, s, dtype, portable)
    g.prefill(t0)
    out = host(g.prefill_at(t0, N))
    cache, acc = host(g.cache), host(g.open_state(T))
    n = oracle.num_slots(T, s)
    want, caches = oracle_ref.loop_outputs(inp, B, T, s, g.d.softmax_scale)
    oracle_ref.assert_steps(out, want[:, t0:], tol(dtype))
    for b, slots in enumerate(caches):
        assert oracle.max_rel_err(cache[b, :n], slots) <= tol(dtype), b
        assert oracle.max_rel_err(acc[b], slots[n - 1].astype(np.float64)) <= tol(dtype), b


@pytest.mark.parametrize("shape,s,cuts,portable", [("st", 3, (0, 97, 230, 301), False),
                                                   ("st", 2, (0, 64, 65, 200), False),
                                                   ("llm", 2, (0, 33, 96), False),
                                                   ("st", 3, (0, 40, 101), True)])
def test_prefill_in_chunks_equals_one_pass(shape, s, cuts, portable):
    """Chunked prefill and one pass over the same tokens: the same cache bits
    and open-slot state (the merge continues the open block from its fp32
    state), outputs within tolerance."""
    T = cuts[-1]
    inp, a = make_case(shape, 13, 2, T, s, "bf16", portable)
    _, b_ = make_case(shape, 13, 2, T, s, "bf16", portable)
    one = host(a.prefill(T))
    parts = [host(b_.prefill_at(lo, hi - lo)) for lo, hi in zip(cuts[:-1], cuts[1:])]
    assert torch.equal(bits(a.cache), bits(b_.cache))
    assert torch.equal(a.open_state(T), b_.open_state(T))
    oracle_ref.assert_steps(np.concatenate(parts, axis=1), one, 1e-2)


def test_prefill_at_then_decode_continues():
    """Chunked prefill, then token-by-token decoding: the outputs follow the
    oracle's incremental loop."""
    B, s, T = 2, 3, 180
    inp, g = make_case("st", 14, B, T, s, "bf16")
    g.prefill(50)
    g.prefill_at(50, 71)
    cont = host(g.decode_loop(T, start=121))
    want, _ = oracle_ref.loop_outputs(inp, B, T, s, g.d.softmax_scale)
    oracle_ref.assert_steps(cont, want[:, 121:], 1e-2)


@pytest.mark.parametrize("shape,s,B,N", [("st", 3, 2, 300), ("llm", 2, 1, 160), ("st", 1, 3, 97),
                                         ("st", 8, 2, 8)])   # no completed slot is attended: no slot keys
def test_staged_prefill_equals_one_call(shape, s, B, N):
    """mtla_prefill_partials -> mtla_prefill_keys -> mtla_prefill_attention
    gives the bits of one mtla_prefill call (outputs, slot cache, open-slot
    state): the same kernels on the same data."""
    import temporally_compressed_latent_amd as m
    inp, a = make_case(shape, 16, B, N, s, "bf16")
    _, b_ = make_case(shape, 16, B, N, s, "bf16")
    one = a.prefill(N)
    d = b_.d
    P = torch.empty(B, N, d.width, dtype=torch.bfloat16, device=DEV)
    S = m.prefill_slot_keys(d, N)
    assert S == (N - 1) // s
    kc = torch.empty(B, d.heads, S, d.d_h, dtype=torch.float16, device=DEV)
    v = torch.empty_like(kc)
    out = torch.empty_like(one)
    m.mtla_prefill_partials(d, b_.c[:, :N].contiguous(), b_.k_r[:, :N].contiguous(), b_.w_hyp, b_.pe, b_.cache,
                            b_.open_acc, P)
    m.mtla_prefill_keys(d, P, b_.w_uk, b_.w_uv, kc, v)
    m.mtla_prefill_attention(d, b_.q_c[:, :N].contiguous(), b_.q_r[:, :N].contiguous(), P, b_.w_uk, b_.w_uv,
                             kc, v, out)
    assert torch.equal(bits(out), bits(one))
    assert torch.equal(bits(a.cache), bits(b_.cache))
    assert torch.equal(a.open_state(N), b_.open_state(N))
    # the staged keys are K^C = W_UK P^c_{s b} and V = W_UV P^c_{s b} of the
    # completed slots b = 1 .. (N-1)//s (partial-merge rows s*b - 1, 0-based),
    # which are also the cache's slot rows
    if S == 0:
        return
    rows = torch.arange(S, device=DEV) * s + (s - 1)
    Pc = P.float()[:, rows, :d.d_c]
    assert torch.equal(bits(P[:, rows]), bits(b_.cache[:, :S]))
    for name, w, got in (("K", b_.w_uk, kc), ("V", b_.w_uv, v)):
        want = torch.einsum("hek,bnk->bhne", w.float(), Pc)
        assert (got.float() - want).abs().max().item() <= 2e-3 * want.abs().max().item(), name
