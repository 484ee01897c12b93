"""GPU: absorbed-form decode (mtla_merge_append + mtla_decode, token by
token) against the fp64 oracle's incremental loop."""
import numpy as np
import pytest
import torch

import oracle
from tests import oracle_ref
from tests.gpu_util import DEV, bits, host, make_case, tol

pytestmark = pytest.mark.gpu

LOOP_CASES = [
    # shape, dtype, portable, s, B, N
    ("st", "bf16", False, 2, 2, 150),
    ("st", "bf16", False, 4, 2, 131),
    ("st", "bf16", True, 3, 2, 100),
    ("st", "fp32", False, 2, 2, 90),
    ("llm", "bf16", False, 2, 2, 90),
    ("mid", "bf16", False, 3, 2, 70),
    ("odd", "fp32", False, 3, 3, 40),
    ("odd", "bf16", False, 1, 2, 33),
]


@pytest.mark.parametrize("shape,dtype,portable,s,B,N", LOOP_CASES)
def test_decode_loop_matches_oracle(shape, dtype, portable, s, B, N):
    inp, g = make_case(shape, 1, B, N, s, dtype, portable)
    out = host(g.decode_loop(N))
    want, caches = oracle_ref.loop_outputs(inp, B, N, s, g.d.softmax_scale)
    oracle_ref.assert_steps(out, want, tol(dtype))
    for b, cache in enumerate(caches):
        assert oracle.max_rel_err(host(g.cache)[b, :cache.shape[0]], cache) <= tol(dtype)


@pytest.mark.parametrize("shape,B,N,s", [("st", 40, 3001, 2), ("llm", 64, 1100, 2), ("st", 9, 2048, 4)])
def test_decode_long_cache_many_splits(shape, B, N, s):
    """Cache built by one chunked append, then one decode step; splits hold
    several 64-slot tiles and a ragged last tile."""
    inp, g = make_case(shape, 2, B, N, s, "bf16", max_slots=-(-N // s) + 64, q_rows=1)
    g.append(torch.ones(B, dtype=torch.int32, device=DEV), 0, N)
    out = host(g.decode(torch.full((B,), N, dtype=torch.int32, device=DEV), 0))
    for b in sorted({0, B // 2, B - 1}):
        cache, _ = oracle_ref.merged_cache(inp["c"][b], inp["k_r"][b], inp["w_hyp"], s)
        want = oracle.decode_absorbed(inp["q_c"][b, 0], inp["q_r"][b, 0], cache,
                                      inp["w_uk"], inp["w_uv"], g.d.d_c, g.d.softmax_scale)
        assert oracle.max_rel_err(out[b], want) <= 1e-2, b


@pytest.mark.parametrize("portable", [False, True])
def test_decode_zero_query_is_uniform_mean(portable):
    """q = 0: every slot gets the same weight, so o_h = W_UV[h] mean_j S^c_j,
    computed here from the device's own cache rows."""
    B, N, s = 3, 77, 2
    inp, g = make_case("st", 3, B, N, s, "bf16", portable, q_zero=True)
    g.append(torch.ones(B, dtype=torch.int32, device=DEV), 0, N)
    out = host(g.decode(torch.full((B,), N, dtype=torch.int32, device=DEV), N - 1))
    cache = host(g.cache)
    n = oracle.num_slots(N, s)
    mean = cache[:, :n, :g.d.d_c].mean(axis=1)                       # [B, d_c]
    want = np.einsum("hek,bk->bhe", inp["w_uv"].astype(np.float64), mean)
    assert oracle.max_rel_err(out, want) <= 2 ** -7


@pytest.mark.parametrize("shape,portable", [("st", False), ("llm", False), ("st", True)])
def test_decode_ignores_rows_past_the_open_slot(shape, portable):
    """NaN in every cache row beyond ceil(t/s) must not reach the output."""
    B, N, s = 2, 130, 2
    inp, g = make_case(shape, 4, B, N, s, "bf16", portable, max_slots=200)
    g.append(torch.ones(B, dtype=torch.int32, device=DEV), 0, N)
    pos = torch.full((B,), N, dtype=torch.int32, device=DEV)
    clean = g.decode(pos, N - 1).clone()
    g.cache[:, oracle.num_slots(N, s):] = float("nan")
    poisoned = g.decode(pos, N - 1)
    assert torch.isfinite(poisoned.float()).all()
    assert torch.equal(bits(clean), bits(poisoned))


@pytest.mark.parametrize("shape", ["st", "llm"])
def test_decode_bit_reproducible(shape):
    B, N, s = 4, 700, 2
    inp, g = make_case(shape, 5, B, N, s, "bf16")
    g.append(torch.ones(B, dtype=torch.int32, device=DEV), 0, N)
    pos = torch.full((B,), N, dtype=torch.int32, device=DEV)
    a = g.decode(pos, N - 1).clone()
    b = g.decode(pos, N - 1).clone()
    assert torch.equal(bits(a), bits(b))


@pytest.mark.parametrize("portable", [False, True])
def test_decode_ragged_and_invalid_positions(portable):
    """Each sequence decodes at its own position; an invalid position gives NaN
    for that sequence only."""
    B, N, s = 5, 64, 2
    inp, g = make_case("st", 6, B, N, s, "bf16", portable)
    g.append(torch.ones(B, dtype=torch.int32, device=DEV), 0, N)
    positions = [1, 5, 64, 0, 10_000]
    out = host(g.decode(torch.tensor(positions, dtype=torch.int32, device=DEV), N - 1))
    for b, p in enumerate(positions):
        if not (1 <= p <= N):
            assert np.isnan(out[b]).all(), b
            continue
        cache, _ = oracle_ref.merged_cache(inp["c"][b], inp["k_r"][b], inp["w_hyp"], s)
        want = oracle.decode_absorbed(inp["q_c"][b, N - 1], inp["q_r"][b, N - 1],
                                      cache[: oracle.slot_of(p, s)], inp["w_uk"], inp["w_uv"],
                                      g.d.d_c, g.d.softmax_scale)
        assert oracle.max_rel_err(out[b], want) <= 1e-2, b


@pytest.mark.parametrize("shape,portable,B,N", [("st", False, 3, 900), ("llm", False, 4, 2500),
                                                ("st", True, 2, 900), ("st", False, 80, 3000)])
def test_staged_decode_equals_fused_call(shape, portable, B, N):
    """absorb -> decode_attention -> up_project gives the bits of mtla_decode
    whenever mtla_decode runs the same staged kernels (several splits, or the
    portable path), and agrees within tolerance with the single-kernel step."""
    import temporally_compressed_latent_amd as m
    s = 2
    inp, g = make_case(shape, 12, B, N, s, "bf16", portable, q_rows=1)
    g.append(torch.ones(B, dtype=torch.int32, device=DEV), 0, N)
    pos = torch.full((B,), N, dtype=torch.int32, device=DEV)
    fused = g.decode(pos, 0).clone()
    d = g.d
    q_lat = torch.empty(B, d.heads, d.width, dtype=torch.float32, device=DEV)
    o_lat = torch.empty(B, d.heads, d.d_c, dtype=torch.float32, device=DEV)
    out = torch.empty_like(fused)
    ws = m.decode_attention_workspace(d)
    splits, one_kernel = m.mtla_decode_plan(d)
    for _ in range(3):
        m.mtla_absorb_query(d, g.q_c[:, 0].contiguous(), g.q_r[:, 0].contiguous(), g.w_uk, q_lat)
        m.mtla_decode_attention(d, pos, q_lat, g.cache, o_lat, ws)
        m.mtla_up_project(d, o_lat, g.w_uv, out)
        if one_kernel:
            assert oracle.max_rel_err(host(out), host(fused)) <= 1e-2
        else:
            assert torch.equal(bits(out), bits(fused))


def test_positions_need_only_element_alignment():
    """pos / pos0 may start at any 4-byte boundary (rows of a [T, B] array)."""
    B, N, s = 3, 20, 2
    inp, g = make_case("st", 13, B, N, s, "bf16")
    _, ref = make_case("st", 13, B, N, s, "bf16")
    table = torch.arange(0, N + 1, dtype=torch.int32, device=DEV)[:, None].expand(N + 1, B).contiguous()
    assert table[1].data_ptr() % 16 != 0
    for t in range(1, N + 1):
        g.append(table[t], t - 1, t)
        ref.append(torch.full((B,), t, dtype=torch.int32, device=DEV), t - 1, t)
    a = g.decode(table[N], N - 1)
    b = ref.decode(torch.full((B,), N, dtype=torch.int32, device=DEV), N - 1)
    assert torch.equal(bits(a), bits(b))


@pytest.mark.parametrize("shape,portable,s,B,N,max_slots", [
    ("st", False, 2, 4, 130, None),       # fused single-kernel step
    ("mid", False, 3, 3, 100, None),      # fused, 20 heads in groups of 2
    ("st", False, 4, 2, 90, 700),         # several splits: merge kernel + staged decode
    ("st", True, 2, 2, 60, None),         # portable kernels
])
def test_decode_step_equals_merge_then_decode(shape, portable, s, B, N, max_slots):
    """mtla_decode_step gives the bits of mtla_merge_append + mtla_decode, and
    both follow the oracle's incremental loop."""
    inp, a = make_case(shape, 14, B, N, s, "bf16", portable, max_slots=max_slots)
    _, b_ = make_case(shape, 14, B, N, s, "bf16", portable, max_slots=max_slots)
    x = a.step_loop(N)
    y = b_.decode_loop(N)
    assert torch.equal(bits(x), bits(y))
    assert torch.equal(bits(a.cache), bits(b_.cache))
    assert torch.equal(a.open_acc, b_.open_acc)
    want, _ = oracle_ref.loop_outputs(inp, B, N, s, a.d.softmax_scale)
    oracle_ref.assert_steps(host(x), want, 1e-2)


@pytest.mark.parametrize("groups", [4, 8])
def test_decode_step_head_groups(groups):
    """The fused step with the heads of a sequence split over 4 or 8
    workgroups: outputs follow the oracle, and the merged cache and open-slot
    state are the same bits whatever the split (the merge arithmetic does not
    depend on it)."""
    B, N, s = 5, 70, 3
    outs, caches, states = [], [], []
    for g_ in (groups, 8 if groups == 4 else 4):
        inp, g = make_case("st", 16, B, N, s, "bf16")
        g.d.step_groups = g_
        outs.append(host(g.step_loop(N)))
        caches.append(bits(g.cache))
        states.append(g.open_acc.clone())
    assert torch.equal(caches[0], caches[1])
    assert torch.equal(states[0], states[1])
    want, _ = oracle_ref.loop_outputs(inp, B, N, s, g.d.softmax_scale)
    for out in outs:
        oracle_ref.assert_steps(out, want, 1e-2)


def test_decode_step_invalid_positions():
    """A position the cache cannot hold gives NaN and leaves that sequence's
    cache untouched; the other sequences are unaffected."""
    import temporally_compressed_latent_amd as m
    B, N, s = 3, 16, 2
    inp, g = make_case("st", 15, B, N, s, "bf16")
    before = g.cache.clone()
    pos = torch.tensor([1, 0, 10_000], dtype=torch.int32, device=DEV)
    o = torch.empty(B, g.d.heads, g.d.d_h, dtype=torch.bfloat16, device=DEV)
    m.mtla_decode_step(g.d, pos, g.c[:, 0].contiguous(), g.k_r[:, 0].contiguous(), g.w_hyp, g.pe,
                       g.q_c[:, 0].contiguous(), g.q_r[:, 0].contiguous(), g.w_uk, g.w_uv, g.cache,
                       g.open_acc, o, g.ws_dec)
    out = host(o)
    assert np.isfinite(out[0]).all()
    assert np.isnan(out[1]).all() and np.isnan(out[2]).all()
    assert torch.equal(g.cache[1:], before[1:])


@pytest.mark.parametrize("shape,s,B,N", [("st", 2, 4, 130), ("mid", 3, 3, 100), ("d40", 2, 5, 70)])
def test_decode_step_tiles_equals_decode_step(shape, s, B, N):
    """mtla_pack_w_uv_tiles writes W_UV in the documented tile order (checked
    against a host gather, rows past d_h zero), and mtla_decode_step_tiles
    gives the bits of mtla_decode_step: outputs, cache rows, open-slot state."""
    import numpy as np
    import temporally_compressed_latent_amd as m
    _, a = make_case(shape, 21, B, N, s, "bf16")
    _, b_ = make_case(shape, 21, B, N, s, "bf16")
    d = b_.d
    tiles = torch.full((m.mtla_w_uv_tiles_bytes(d) // 2,), 7.0, dtype=torch.bfloat16, device=DEV)
    m.mtla_pack_w_uv_tiles(d, b_.w_uv, tiles)
    H, d_h, d_c = d.heads, d.d_h, d.d_c
    nt = -(-d_h // 16)
    w = np.zeros((H, nt * 16, d_c), dtype=np.int16)
    w[:, :d_h] = b_.w_uv.view(torch.int16).cpu().numpy()
    want = w.reshape(H, nt, 16, d_c // 32, 4, 8).transpose(0, 1, 3, 4, 2, 5).reshape(-1)
    assert np.array_equal(tiles.view(torch.int16).cpu().numpy(), want)
    x = a.step_loop(N)
    y = b_.step_loop(N, w_uv_tiles=tiles)
    assert torch.equal(bits(x), bits(y))
    assert torch.equal(bits(a.cache), bits(b_.cache))
    assert torch.equal(a.open_acc, b_.open_acc)
