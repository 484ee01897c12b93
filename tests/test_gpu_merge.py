"""GPU: gate + temporal merge (mtla_merge_append) against the oracle, with
bit-exact checks of slot indexing, block resets and chunked appends."""
import numpy as np
import pytest
import torch

import oracle
import temporally_compressed_latent_amd as m
import workloads
from tests import oracle_ref
from tests.gpu_util import DEV, Case, host, tol

pytestmark = pytest.mark.gpu


def _case(seed, B, N, d_c, d_r, s, dtype, **kw):
    inp = workloads.boundary_case(seed, B, N, 2, 8, d_c, d_r, dtype, **kw)
    dims = m.make_dims(B, 2, 8, d_c, d_r, s, -(-N // s) + 3, dtype)
    return inp, Case(dims, inp, N + 8)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("s", [1, 2, 3, 4])
def test_merge_matches_oracle(dtype, s):
    B, N, d_c, d_r = 3, 37, 64, 16
    inp, g = _case(s, B, N, d_c, d_r, s, dtype)
    gates = torch.empty(B, N, dtype=torch.float32, device=DEV)
    for t in range(1, N + 1):
        pos = torch.full((B,), t, dtype=torch.int32, device=DEV)
        gout = torch.empty(B, 1, dtype=torch.float32, device=DEV)
        g.append(pos, t - 1, t, gate_out=gout)
        gates[:, t - 1] = gout[:, 0]
    cache = host(g.cache)
    for b in range(B):
        want, w = oracle_ref.merged_cache(inp["c"][b], inp["k_r"][b], inp["w_hyp"], s)
        n = want.shape[0]
        assert oracle.max_rel_err(cache[b, :n], want) <= tol(dtype)
        assert np.max(np.abs(host(gates)[b] - w)) <= 2e-6
        # fp32 open-slot state holds the unrounded value of the last slot
        assert oracle.max_rel_err(host(g.open_state(N))[b], want[n - 1]) <= 1e-5
        assert np.all(cache[b, n:] == 0)  # rows past the last slot untouched


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_slot_index_sentinel_bit_exact(dtype):
    """Appending token t changes cache row ceil(t/s)-1 and no other row."""
    B, N, s = 2, 23, 3
    inp, g = _case(11, B, N, 32, 8, s, dtype)
    g.cache.fill_(-12345.0)
    prev = g.cache.clone()
    for t in range(1, N + 1):
        g.append(torch.full((B,), t, dtype=torch.int32, device=DEV), t - 1, t)
        changed = (g.cache != prev).any(dim=2).any(dim=0).nonzero().flatten().tolist()
        assert changed == [oracle.slot_of(t, s) - 1], (t, changed)
        prev = g.cache.clone()


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("s", [1, 2, 3, 5])
def test_half_gate_closed_form_bit_exact(dtype, s):
    """W_hyp = 0 makes every gate exactly 1/2; with small-integer latents the
    merged slot is exactly half the block sum in fp32 and in bf16."""
    B, N, d_c, d_r = 2, 17, 32, 8
    rng = np.random.default_rng(s)
    inp = workloads.boundary_case(s, B, N, 2, 8, d_c, d_r, dtype, w_hyp_zero=True)
    inp["c"] = rng.integers(-8, 9, size=(B, N, d_c)).astype(np.float32)
    inp["k_r"] = rng.integers(-8, 9, size=(B, N, d_r)).astype(np.float32)
    dims = m.make_dims(B, 2, 8, d_c, d_r, s, -(-N // s), dtype)
    g = Case(dims, inp, N)
    g.append(torch.ones(B, dtype=torch.int32, device=DEV), 0, N)
    x = np.concatenate([inp["c"], inp["k_r"]], axis=2).astype(np.float64)
    cache = host(g.cache)
    for blk in range(-(-N // s)):
        want = 0.5 * x[:, blk * s: min(N, blk * s + s)].sum(axis=1)
        assert np.array_equal(cache[:, blk], want), blk


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("s", [2, 3])
def test_chunked_append_equals_tokenwise_bit_exact(dtype, s):
    """Appending in chunks (continuing open slots, several workgroups per
    sequence, the open-slot tail pass) gives the same bits as one token at a
    time."""
    B, N, d_c, d_r = 2, 900, 64, 16
    inp, a = _case(21, B, N, d_c, d_r, s, dtype)
    _, b_ = _case(21, B, N, d_c, d_r, s, dtype)
    for t in range(1, N + 1):
        a.append(torch.full((B,), t, dtype=torch.int32, device=DEV), t - 1, t)
    t = 1
    for size in (5, 1, 2, 300, 7, 584, 1):
        b_.append(torch.full((B,), t, dtype=torch.int32, device=DEV), t - 1, t - 1 + size)
        t += size
    assert t == N + 1
    assert torch.equal(a.cache.view(torch.int16 if dtype == "bf16" else torch.int32),
                       b_.cache.view(torch.int16 if dtype == "bf16" else torch.int32))
    assert torch.equal(a.open_state(N), b_.open_state(N))


def test_ragged_positions_and_invalid_sequences():
    """One call with each sequence at its own position; a sequence whose
    position is out of range (t < 1, or beyond the cache / pe table) is left
    untouched."""
    B, N, s, d_c, d_r, T = 5, 40, 2, 32, 8, 6
    inp, g = _case(31, B, N, d_c, d_r, s, "fp32")
    starts = [1, 2, 7, 0, 10_000]
    valid = [1 <= p < 100 for p in starts]
    # earlier tokens of the valid sequences, one at a time (position 0 = skip)
    for t in range(1, max(p for p, v in zip(starts, valid) if v)):
        pos = [t if (v and t < p) else 0 for p, v in zip(starts, valid)]
        g.append(torch.tensor(pos, dtype=torch.int32, device=DEV), t - 1, t)
    before = g.cache.clone()
    rows = [slice(p - 1, p - 1 + T) if v else slice(0, T) for p, v in zip(starts, valid)]
    c = torch.stack([g.c[b, r] for b, r in enumerate(rows)]).contiguous()
    k = torch.stack([g.k_r[b, r] for b, r in enumerate(rows)]).contiguous()
    m.mtla_merge_append(g.d, torch.tensor(starts, dtype=torch.int32, device=DEV), c, k,
                        g.w_hyp, g.pe, g.cache, g.open_acc)
    cache = host(g.cache)
    for b, (p, v) in enumerate(zip(starts, valid)):
        if not v:
            assert torch.equal(g.cache[b], before[b]), b
            continue
        n = p + T - 1
        want, _ = oracle_ref.merged_cache(inp["c"][b, :n], inp["k_r"][b, :n], inp["w_hyp"], s)
        assert oracle.max_rel_err(cache[b, :want.shape[0]], want) <= 1e-5, b


@pytest.mark.parametrize("T", [2, 4])
def test_many_sequences_even_append_across_a_block_boundary(T):
    """B = 1100 puts all blocks of a short append in one workgroup per
    sequence.  An append of an even number of tokens that continues an open
    block reads the open-slot state from the same parity half it writes:
    token 1 first, then tokens 2..T+1 in one call (token 2 closes slot 1,
    token 3 opens slot 2).  The slots and the new open-slot state follow the
    oracle's merge for every sequence."""
    B, s, d_c, d_r = 1100, 2, 64, 16
    N = T + 1
    inp, g = _case(41, B, N, d_c, d_r, s, "fp32")
    g.append(torch.ones(B, dtype=torch.int32, device=DEV), 0, 1)
    g.append(torch.full((B,), 2, dtype=torch.int32, device=DEV), 1, N)
    cache, state = host(g.cache), host(g.open_state(N))
    for b in range(B):
        want, _ = oracle_ref.merged_cache(inp["c"][b], inp["k_r"][b], inp["w_hyp"], s)
        n = want.shape[0]
        assert oracle.max_rel_err(cache[b, :n], want) <= 1e-5, b
        assert oracle.max_rel_err(state[b], want[n - 1]) <= 1e-5, b
