"""Pins of the fp64 oracle against what the MTLA pages and the mathematics fix.

Each ``pin_*`` function takes the oracle module ``o`` and raises
AssertionError when the oracle disagrees with the pinned fact.  They are run
against the real oracle (tests/test_oracle_pins.py) and against deliberately
broken copies of it (tests/test_oracle_mutations.py), which shows that a
plausible mistake anywhere in the oracle fails at least one pin.

None of these checks re-types an oracle formula: each compares the oracle with
an independent construction (enumeration, closed form, library routine, page
value, or a second schedule of the same computation).
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_values.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _rand_case(seed, N, s, H, d_h, d_c, d_r, w_scale=None):
    g = np.random.default_rng(seed)
    c = g.standard_normal((N, d_c))
    k_r = g.standard_normal((N, d_r))
    q_c = g.standard_normal((N, H, d_h))
    q_r = g.standard_normal((N, H, d_r))
    ws = 1.0 / math.sqrt(d_c) if w_scale is None else w_scale
    w_hyp = g.standard_normal(d_c) * ws
    w_uk = g.standard_normal((H, d_h, d_c)) * ws
    w_uv = g.standard_normal((H, d_h, d_c)) * ws
    return c, k_r, q_c, q_r, w_hyp, w_uk, w_uv


# ---------------------------------------------------------------------------
# Integer structure
# ---------------------------------------------------------------------------

def pin_slot_index(o):
    """Slot of each token by enumerating blocks of s tokens (no division)."""
    for s in range(1, 9):
        tokens_to_slot = []
        for b in range(1, 40):
            tokens_to_slot += [b] * s
        for t in range(1, len(tokens_to_slot) + 1):
            assert o.slot_of(t, s) == tokens_to_slot[t - 1], (t, s)


def pin_block_starts(o):
    """Tokens that open a slot are 1, s+1, 2s+1, ... (a range, not a modulus)."""
    for s in range(1, 9):
        starts = set(range(1, 200, s))
        for t in range(1, 200):
            assert o.opens_slot(t, s) == (t in starts), (t, s)


def pin_slot_count(o):
    """ceil(N/s) slots = number of distinct slots the tokens 1..N occupy."""
    for s in range(1, 9):
        for N in range(0, 60):
            distinct = len({o.slot_of(t, s) for t in range(1, N + 1)})
            assert o.num_slots(N, s) == distinct, (N, s)


def pin_mask_special_cases(o):
    """s=1: the ordinary causal mask (np.tril).  s>=N: only the diagonal."""
    for N in range(1, 24):
        assert np.array_equal(o.stride_mask(N, 1), np.tril(np.ones((N, N), dtype=bool)))
        for s in (N, N + 1, N + 5):
            assert np.array_equal(o.stride_mask(N, s), np.eye(N, dtype=bool))


def pin_mask_structure(o):
    """Causal, diagonal always visible, and query i sees ceil(i/s) keys."""
    for s in range(1, 7):
        N = 5 * s + 3
        M = o.stride_mask(N, s)
        assert not np.triu(M, 1).any()
        assert M.diagonal().all()
        for i in range(1, N + 1):
            # its own partial slot plus the completed slots before it
            assert M[i - 1].sum() == len(range(1, i + 1, s)), (i, s)


def pin_mask_matches_incremental_cache(o):
    """The partial merges the mask exposes to query i are exactly the slots the
    incremental decoder holds after token i (the pages' consistency claim at
    the level of the attended rows)."""
    g = np.random.default_rng(7)
    for s in range(1, 6):
        N = 4 * s + 3
        x = g.standard_normal((N, 5))
        w = g.uniform(0.1, 0.9, N)
        P = o.partial_merges(x, w, s)
        M = o.stride_mask(N, s)
        for i in range(1, N + 1):
            cache = o.merge_incremental(x[:i], w[:i], s)
            seen = P[M[i - 1]]
            assert seen.shape == cache.shape, (i, s)
            np.testing.assert_allclose(seen, cache, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# Page values
# ---------------------------------------------------------------------------

def pin_cache_ratio(o):
    g = golden()
    d = g["cache_ratio_default_s2"]["dims"]
    for N in (8, 64, 4096):
        r = o.cache_ratio_vs_mqa(N, d["s"], d["d_h"], d["d_c"], d["d_r"])
        assert r == Fraction(g["cache_ratio_default_s2"]["value"]), r
    f = g["cache_ratio_formula"]
    for d_h in (16, 64, 128):
        for s in range(1, 7):
            N = 12 * s
            r = o.cache_ratio_vs_mqa(N, s, d_h, 4 * d_h, d_h // 2)
            assert r == Fraction(f["numerator"], f["denominator_per_s"] * s), (d_h, s, r)
    # s does not divide N: the stored slot count rounds up, so the ratio is larger
    assert o.cache_ratio_vs_mqa(4096, 3, 64, 256, 32) > Fraction(9, 12)


def pin_row_bytes(o):
    g = golden()
    e = g["latent_row_bytes_bf16"]
    row = o.cache_row_bytes(e["d_c"], e["d_r"], e["bytes_per_element"])
    assert row == e["value"]
    assert row * g["latent_bytes_78_layers"]["layers"] == g["latent_bytes_78_layers"]["value"]
    assert row * 78 * g["latent_bytes_1M_positions"]["positions"] == g["latent_bytes_1M_positions"]["value"]


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------

def pin_gate_zero_weights(o):
    """W_hyp = 0: every gate is sigmoid(0) = 1/2 exactly, whatever c and pe are."""
    g = np.random.default_rng(3)
    c = g.standard_normal((9, 16))
    pe = o.sinusoidal_pe(9, 16)
    w = o.gate(c, pe, np.zeros(16))
    assert np.all(w == 0.5)
    # a positive logit gives a gate above 1/2, a negative one below
    wp = o.gate(np.ones((1, 16)) - pe[:1], pe[:1], np.ones(16))
    assert wp[0] > 0.5 and abs(wp[0] - 1.0 / (1.0 + math.exp(-16.0))) < 1e-15


def pin_gate_per_position(o):
    """One W_hyp row per place in the block: with c + pe a basis vector e_k,
    token t's logit is entry k of row (t - 1) mod s, written out here; rows
    that are all equal give the one-row gate exactly; a continuation starting
    at token t_first keeps its tokens' places."""
    s, d_c, N = 3, 4, 8
    w_hyp = np.arange(s * d_c, dtype=float).reshape(s, d_c) / 7.0 - 0.6
    pe = o.sinusoidal_pe(N, d_c)
    ks = [1, 3, 0, 2, 2, 1, 0, 3]
    c = np.stack([np.eye(d_c)[k] for k in ks]) - pe
    want = np.array([1.0 / (1.0 + math.exp(-w_hyp[(t - 1) % s, ks[t - 1]])) for t in range(1, N + 1)])
    got = o.gate(c, pe, w_hyp)
    assert np.max(np.abs(got - want)) <= 1e-15, (got, want)
    # a continuation from token 5 gives the same gates to tokens 5..8
    assert np.max(np.abs(o.gate(c[4:], pe[4:], w_hyp, t_first=5) - want[4:])) <= 1e-15
    # equal rows: the one-row gate, and the same forward passes
    g = np.random.default_rng(17)
    row = g.standard_normal(d_c)
    c2 = g.standard_normal((N, d_c))
    assert np.array_equal(o.gate(c2, pe, np.tile(row, (s, 1))), o.gate(c2, pe, row))
    args = list(_rand_case(18, 7, s, 2, 3, d_c, 2))
    scale = 0.45
    one = o.parallel(*args, s, scale)
    args[4] = np.tile(args[4], (s, 1))
    assert np.array_equal(o.parallel(*args, s, scale), one)
    assert o.max_rel_err(o.incremental(*args, s, scale), one) <= 1e-12


def pin_merge_half_sum(o):
    """With w = 1/2 the slot is half the block sum; integers keep it exact."""
    g = np.random.default_rng(5)
    for s in range(1, 6):
        N = 3 * s + 2
        x = g.integers(-8, 9, size=(N, 4)).astype(float)
        cache = o.merge_incremental(x, np.full(N, 0.5), s)
        for b in range(cache.shape[0]):
            blk = x[b * s: min(N, (b + 1) * s)]
            assert np.array_equal(cache[b], 0.5 * blk.sum(axis=0)), (s, b)


def pin_block_start_overwrites(o):
    """A token that opens a block writes a new slot: whatever the slot row held
    before (a reused cache) does not leak into the merged value."""
    g = np.random.default_rng(6)
    for s in range(1, 5):
        N = 4 * s + 1
        x = g.standard_normal((N, 3))
        w = g.uniform(0.1, 0.9, N)
        fresh = o.merge_incremental(x, w, s)
        stale = g.standard_normal(fresh.shape) * 100.0
        reused = o.merge_incremental(x, w, s, cache=stale)
        np.testing.assert_allclose(reused, fresh, rtol=0, atol=1e-12)
        # continuing from a block start on a cache with garbage beyond it
        t0 = s + 1
        head = o.merge_incremental(x[: t0 - 1], w[: t0 - 1], s)
        junk = np.vstack([head, g.standard_normal((fresh.shape[0] - head.shape[0], 3))])
        cont = o.merge_incremental(x[t0 - 1:], w[t0 - 1:], s, cache=junk, t0=t0)
        np.testing.assert_allclose(cont, fresh, rtol=0, atol=1e-12)


def pin_uniform_attention_keyset(o):
    """q = 0, W_hyp = 0, basis-vector latents, W_UV = I: output i is
    1/(2 |K(i)|) on tokens 1..i and 0 after, with |K(i)| = 1 + floor((i-1)/s).

    Each token k <= i lies in exactly one attended key (a completed block, or
    the own partial block), so the uniform mean puts equal mass on all of them.
    """
    for s in range(1, 5):
        N = 3 * s + 2
        d = N
        c = np.eye(N)
        k_r = np.zeros((N, 2))
        q_c = np.zeros((N, 1, d))
        q_r = np.zeros((N, 1, 2))
        eye = np.eye(d)[None]
        for sched in (o.incremental, o.parallel):
            out = sched(c, k_r, q_c, q_r, np.zeros(d), eye, eye, s, 0.5, pe=np.zeros((N, d)))
            for i in range(1, N + 1):
                nk = 1 + (i - 1) // s
                want = np.where(np.arange(1, d + 1) <= i, 1.0 / (2 * nk), 0.0)
                np.testing.assert_allclose(out[i - 1, 0], want, rtol=0, atol=1e-14,
                                           err_msg=f"{sched.__name__} s={s} i={i}")


# ---------------------------------------------------------------------------
# Identities and library reductions
# ---------------------------------------------------------------------------

def pin_absorption(o):
    """Absorbed decode (W_UK into the query, W_UV after the sum) equals the
    explicit per-head key/value form."""
    g = np.random.default_rng(11)
    for (H, d_h, d_c, d_r, n) in ((2, 4, 12, 2, 5), (3, 8, 6, 4, 9), (1, 5, 5, 0, 3)):
        S = g.standard_normal((n, d_c + d_r))
        q_c = g.standard_normal((H, d_h))
        q_r = g.standard_normal((H, d_r))
        w_uk = g.standard_normal((H, d_h, d_c))
        w_uv = g.standard_normal((H, d_h, d_c))
        a = o.decode_absorbed(q_c, q_r, S, w_uk, w_uv, d_c, 0.3)
        e = o.decode_explicit(q_c, q_r, S, w_uk, w_uv, d_c, 0.3)
        np.testing.assert_allclose(a, e, rtol=1e-12, atol=1e-12)


def pin_decode_single_slot(o):
    """One slot: softmax of a single score is 1, so o_h = W_UV[h] c_1 exactly."""
    g = np.random.default_rng(12)
    S = g.standard_normal((1, 10))
    w_uv = g.standard_normal((2, 3, 8))
    out = o.decode_absorbed(g.standard_normal((2, 3)), g.standard_normal((2, 2)), S,
                            g.standard_normal((2, 3, 8)), w_uv, 8, 0.7)
    np.testing.assert_allclose(out, np.einsum("hek,k->he", w_uv, S[0, :8]), rtol=1e-13)


def pin_s1_equals_causal_sdpa(o):
    """s = 1 and W_hyp = 0 (w = 1/2) reduce MTLA to causal attention with keys
    [W_UK c_j / 2 ; k^R_j / 2] and values W_UV c_j / 2.  Compared with torch's
    scaled_dot_product_attention in fp64 on the CPU (an independent routine)."""
    import torch
    H, d_h, d_c, d_r, N = 2, 6, 10, 4, 11
    c, k_r, q_c, q_r, _, w_uk, w_uv = _rand_case(21, N, 1, H, d_h, d_c, d_r)
    scale = 1.0 / math.sqrt(d_h + d_r)
    outs = [sched(c, k_r, q_c, q_r, np.zeros(d_c), w_uk, w_uv, 1, scale, pe=np.zeros((N, d_c)))
            for sched in (o.parallel, o.incremental)]
    tq = torch.tensor(np.concatenate([q_c, q_r], axis=2)).permute(1, 0, 2)         # H N d
    K = np.stack([0.5 * c @ w_uk[h].T for h in range(H)])                         # H N d_h
    V = np.stack([0.5 * c @ w_uv[h].T for h in range(H)])
    Kr = np.broadcast_to(0.5 * k_r, (H, N, d_r))
    tk = torch.tensor(np.concatenate([K, Kr], axis=2))
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, torch.tensor(V), is_causal=True, scale=scale).permute(1, 0, 2).numpy()
    for out in outs:
        np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)


def pin_parallel_equals_incremental(o, cases=None):
    """The stride-masked parallel pass equals token-by-token decoding (the pages'
    central claim), in fp64, for the given (seed, N, s, H, d_h, d_c, d_r)."""
    cases = cases or [(1, 13, 2, 2, 4, 8, 2), (2, 17, 3, 1, 3, 5, 4), (3, 9, 4, 2, 2, 6, 2),
                      (4, 10, 1, 1, 4, 4, 2), (5, 7, 9, 2, 3, 7, 2)]
    for (seed, N, s, H, d_h, d_c, d_r) in cases:
        c, k_r, q_c, q_r, w_hyp, w_uk, w_uv = _rand_case(seed, N, s, H, d_h, d_c, d_r)
        scale = 1.0 / math.sqrt(d_h + d_r)
        inc = o.incremental(c, k_r, q_c, q_r, w_hyp, w_uk, w_uv, s, scale)
        par = o.parallel(c, k_r, q_c, q_r, w_hyp, w_uk, w_uv, s, scale)
        assert o.max_rel_err(par, inc) <= 1e-12, (seed, N, s, o.max_rel_err(par, inc))


def pin_prefill_query_rows(o):
    """prefill_query(i) reproduces row i of the dense parallel pass."""
    N, s, H, d_h, d_c, d_r = 11, 3, 2, 4, 6, 2
    c, k_r, q_c, q_r, w_hyp, w_uk, w_uv = _rand_case(31, N, s, H, d_h, d_c, d_r)
    scale = 0.4
    par, P = o.parallel(c, k_r, q_c, q_r, w_hyp, w_uk, w_uv, s, scale, return_partials=True)
    for i in range(1, N + 1):
        row = o.prefill_query(P, i, q_c[i - 1], q_r[i - 1], w_uk, w_uv, s, d_c, scale)
        np.testing.assert_allclose(row, par[i - 1], rtol=1e-12, atol=1e-13)


def pin_rope(o):
    """RoPE: identity at position 0, norm preserving, and scores depend only on
    the relative position (q rotated at p, k at p') ."""
    g = np.random.default_rng(41)
    q, k = g.standard_normal(8), g.standard_normal(8)
    np.testing.assert_allclose(o.rope(q, 0), q, rtol=0, atol=0)
    for p in (1, 7, 300):
        assert abs(np.linalg.norm(o.rope(q, p)) - np.linalg.norm(q)) < 1e-12
    a = o.rope(q, 10) @ o.rope(k, 4)
    b = o.rope(q, 106) @ o.rope(k, 100)
    assert abs(a - b) < 1e-12
    # the pair (2k, 2k+1) rotates as a complex multiplication by e^{i*angle}
    z = complex(q[0], q[1]) * np.exp(1j * 5.0)
    r = o.rope(q, 5)
    assert abs(r[0] - z.real) < 1e-12 and abs(r[1] - z.imag) < 1e-12


def pin_pe(o):
    """pe: position 0 is (sin 0, cos 0) = (0, 1) per pair; pairs lie on the unit
    circle; the first pair advances by one radian per position."""
    pe = o.sinusoidal_pe(50, 12)
    np.testing.assert_array_equal(pe[0], np.tile([0.0, 1.0], 6))
    np.testing.assert_allclose(pe[:, 0::2] ** 2 + pe[:, 1::2] ** 2, 1.0, rtol=1e-14)
    ang = np.arctan2(pe[:, 0], pe[:, 1])
    np.testing.assert_allclose(np.unwrap(ang), np.arange(50.0), atol=1e-12)


def _pairs_as_complex(v):
    """Interleaved real pairs (2k, 2k+1) of the last axis as complex numbers."""
    v = np.asarray(v, dtype=float)
    return v[..., 0::2] + 1j * v[..., 1::2]


def pin_project_worked_example(o):
    """Basis-vector inputs make every projection a known combination of weight
    columns.  Token t (1-based) carries h_t = e_0 + t e_1, so before any
    rotation its projections are W[:, 0] + t W[:, 1] of each weight matrix.
    Then, read off the matrices here (not through a matrix product):
      * c_t is that combination of W_DKV's columns;
      * head h's content query is the combination of W_Q's rows
        h(d_h+d_r) .. h(d_h+d_r)+d_h-1, and its raw rope query of the next
        d_r rows;
      * the rope parts of token t are the raw values with each pair
        (2k, 2k+1), taken as one complex number, multiplied by
        exp(i (t-1) theta_k), theta_k = 10000^(-2k/d_r): the first token is
        not turned at all;
      * hence q^R_t . k^R_u = Re sum_k zq_k conj(zk_k) exp(i (t-u) theta_k)
        depends on the positions only through t - u.
    """
    N, dm, H, d_h, d_r, d_c = 6, 3, 2, 3, 4, 5
    g = np.random.default_rng(71)
    p = {"w_dkv": g.standard_normal((d_c, dm)), "w_q": g.standard_normal((H * (d_h + d_r), dm)),
         "w_r": g.standard_normal((d_r, dm))}
    h = np.zeros((N, dm))
    h[:, 0] = 1.0
    h[:, 1] = np.arange(1, N + 1)
    c, k_r, q_c, q_r = o.project(h, p, H, d_h, d_r)
    assert c.shape == (N, d_c) and k_r.shape == (N, d_r)
    assert q_c.shape == (N, H, d_h) and q_r.shape == (N, H, d_r)
    theta = np.array([10000.0 ** (-2.0 * k / d_r) for k in range(d_r // 2)])
    for t in range(1, N + 1):
        col = lambda w: np.asarray(w)[:, 0] + t * np.asarray(w)[:, 1]
        np.testing.assert_allclose(c[t - 1], col(p["w_dkv"]), rtol=0, atol=1e-12)
        turn = np.exp(1j * (t - 1) * theta)
        zk = _pairs_as_complex(col(p["w_r"])) * turn
        np.testing.assert_allclose(_pairs_as_complex(k_r[t - 1]), zk, rtol=0, atol=1e-12)
        wq = col(p["w_q"])
        for hh in range(H):
            base = hh * (d_h + d_r)
            np.testing.assert_allclose(q_c[t - 1, hh], wq[base:base + d_h], rtol=0, atol=1e-12)
            zq = _pairs_as_complex(wq[base + d_h:base + d_h + d_r]) * turn
            np.testing.assert_allclose(_pairs_as_complex(q_r[t - 1, hh]), zq, rtol=0, atol=1e-12)
    # relative-position property of the rotated dot products
    raw_k = lambda u: _pairs_as_complex(p["w_r"][:, 0] + u * p["w_r"][:, 1])
    for t in range(1, N + 1):
        for u in range(1, N + 1):
            for hh in range(H):
                base = hh * (d_h + d_r) + d_h
                zq = _pairs_as_complex(p["w_q"][base:base + d_r, 0] + t * p["w_q"][base:base + d_r, 1])
                want = np.real(np.sum(zq * np.conj(raw_k(u)) * np.exp(1j * (t - u) * theta)))
                assert abs(float(q_r[t - 1, hh] @ k_r[u - 1]) - want) < 1e-11, (t, u, hh)


def pin_layer_worked_example(o):
    """A layer whose output is known in closed form.  W_Q = 0 and W_R = 0 make
    every score zero (uniform attention over the key set); W_hyp = 0 makes
    every gate 1/2; h_t = e_t and W_DKV = I make c_t = e_t; W_UV[h] = b_h I.
    Each token k <= i lies in exactly one key that query i attends (a
    completed block, or its own partial block), so o_{i,h} is b_h / (2|K(i)|)
    on tokens 1..i and 0 after, with |K(i)| = 1 + floor((i-1)/s).  With
    W_O = [a_1 I, ..., a_H I] (heads side by side in order),
    y_i = (sum_h a_h b_h) / (2|K(i)|) on tokens 1..i.  Also: with the head
    blocks of W_O swapped the sum pairs a_h with b_{H-1-h}, which differs."""
    N, H, s = 7, 2, 3
    d = N
    a, b = (1.0, 3.0), (2.0, 5.0)
    for sched in ("incremental", "parallel"):
        p = {"w_dkv": np.eye(d), "w_q": np.zeros((H * (d + 2), d)), "w_r": np.zeros((2, d)),
             "w_hyp": np.zeros(d), "w_uk": np.stack([np.eye(d)] * H),
             "w_uv": np.stack([b[hh] * np.eye(d) for hh in range(H)]),
             "w_o": np.concatenate([a[hh] * np.eye(d) for hh in range(H)], axis=1)}
        y = o.layer(np.eye(N), p, H, d, 2, s, 0.7, sched)
        assert y.shape == (N, d), y.shape
        for i in range(1, N + 1):
            nk = 1 + (i - 1) // s
            want = np.where(np.arange(1, d + 1) <= i, (a[0] * b[0] + a[1] * b[1]) / (2 * nk), 0.0)
            np.testing.assert_allclose(y[i - 1], want, rtol=0, atol=1e-13, err_msg=f"{sched} i={i}")


def pin_max_rel_err(o):
    """The parity measure ||y - y_ref||_inf / ||y_ref||_inf on hand-computed
    cases: zero for equal tensors; the single worst element decides (not a
    mean); the denominator is the largest |y_ref| (a negative one included),
    never |y| and never the element's own size; any shape."""
    assert o.max_rel_err([1.0, -2.0, 4.0], [1.0, -2.0, 4.0]) == 0.0
    assert o.max_rel_err([1.0, -2.5, 4.0], [1.0, -2.0, 4.0]) == 0.125       # 0.5 / 4
    assert o.max_rel_err([0.0, -2.0, 3.0], [1.0, -2.0, 4.0]) == 0.25        # 1 / 4
    assert o.max_rel_err([2.0, 0.0], [1.0, 0.0]) == 1.0                     # 1 / 1
    assert o.max_rel_err([1.0, 0.0], [2.0, 0.0]) == 0.5                     # 1 / 2
    assert o.max_rel_err([-8.0, 2.0], [-8.0, 1.0]) == 0.125                 # 1 / |-8|
    # an element far smaller than the largest: measured against the largest
    assert abs(o.max_rel_err([2e-6, 10.0], [1e-6, 10.0]) - 1e-7) < 1e-20
    y_ref = np.ones((4, 5, 3))
    y = y_ref.copy()
    y[2, 3, 1] = 0.97
    y[0, 0, 0] = 1.01
    assert abs(o.max_rel_err(y, y_ref) - 0.03) < 1e-15
    assert abs(o.max_rel_err(-5.0 * y, -5.0 * y_ref) - 0.03) < 1e-15


def pin_layer_schedules(o):
    """The full layer gives the same y with either attention schedule, and its
    output projection is linear in the attention output."""
    g = np.random.default_rng(51)
    N, dm, H, d_h, d_c, d_r, s = 7, 12, 2, 4, 8, 2, 2
    p = {"w_dkv": g.standard_normal((d_c, dm)) / math.sqrt(dm),
         "w_q": g.standard_normal((H * (d_h + d_r), dm)) / math.sqrt(dm),
         "w_r": g.standard_normal((d_r, dm)) / math.sqrt(dm),
         "w_o": g.standard_normal((dm, H * d_h)) / math.sqrt(H * d_h),
         "w_hyp": g.standard_normal(d_c) / math.sqrt(d_c),
         "w_uk": g.standard_normal((H, d_h, d_c)) / math.sqrt(d_c),
         "w_uv": g.standard_normal((H, d_h, d_c)) / math.sqrt(d_c)}
    h = g.standard_normal((N, dm))
    y1 = o.layer(h, p, H, d_h, d_r, s, 0.4, "incremental")
    y2 = o.layer(h, p, H, d_h, d_r, s, 0.4, "parallel")
    assert o.max_rel_err(y1, y2) < 1e-12
    p0 = dict(p, w_o=np.zeros_like(p["w_o"]))
    assert np.all(o.layer(h, p0, H, d_h, d_r, s, 0.4) == 0)


def pin_beam_reorder_follows_history(o):
    """A reordered hypothesis carries its parent's state: its slots are the
    merge of the parent's token history (built here from that history, not
    by gathering), the unused rows stay zero, and appending a new token to
    the reordered state equals merging parent history + token from scratch."""
    g = np.random.default_rng(21)
    for s in (1, 2, 3, 5):
        B, W = 6, 4
        lens = g.integers(1, 4 * s + 3, size=B)
        S = o.num_slots(int(lens.max()) + 1, s)
        hist = [g.standard_normal((int(n), W)) for n in lens]
        gates = [g.uniform(0.1, 0.9, int(n)) for n in lens]
        cache = np.zeros((B, S, W))
        open_state = np.zeros((B, W))
        for b in range(B):
            m = o.merge_incremental(hist[b], gates[b], s)
            cache[b, :m.shape[0]] = m
            open_state[b] = m[-1]
        src = g.integers(0, B, size=B)
        src[0] = src[1]                          # a parent kept twice
        out, open_out, pos_out = o.reorder_state(cache, open_state, lens, src, s)
        for b in range(B):
            a = int(src[b])
            want = o.merge_incremental(hist[a], gates[a], s)
            n = want.shape[0]
            np.testing.assert_allclose(out[b, :n], want, rtol=0, atol=1e-12)
            assert not out[b, n:].any()
            assert pos_out[b] == lens[a]
            np.testing.assert_allclose(open_out[b], want[-1], rtol=0, atol=1e-12)
            x_new, w_new = g.standard_normal(W), 0.6
            grown = np.zeros((o.num_slots(int(lens[a]) + 1, s), W))
            grown[:n] = out[b, :n]
            o.append_token(grown, x_new, w_new, int(lens[a]) + 1, s)
            ref = o.merge_incremental(np.vstack([hist[a], x_new]), np.append(gates[a], w_new), s)
            np.testing.assert_allclose(grown, ref, rtol=0, atol=1e-12)


def pin_backward_finite_differences(o):
    """The training backward equals central differences of the forward:
    every element of every gradient of L = sum(d_o * parallel(...)) against
    (L(x + e) - L(x - e)) / 2e, at N a multiple of s, N not a multiple, s = 1
    (the causal mask) and s >= N (the diagonal alone)."""
    H, d_h, d_c, d_r, scale, eps = 2, 3, 4, 2, 0.4, 1e-6
    names = ("dc", "dk_r", "dq_c", "dq_r", "dw_hyp", "dw_uk", "dw_uv")
    # (the last case takes one W_hyp row per place in the block)
    for seed, N, s, per_pos in ((61, 7, 3, False), (62, 6, 2, False), (63, 5, 1, False), (64, 4, 5, False),
                                (65, 7, 3, True)):
        args = list(_rand_case(seed, N, s, H, d_h, d_c, d_r, w_scale=0.5))
        g = np.random.default_rng(seed + 100)
        if per_pos:
            args[4] = g.standard_normal((s, d_c)) * 0.5
        d_o = g.standard_normal((N, H, d_h))
        pe = g.standard_normal((N, d_c))
        grads = o.parallel_backward(*args, s, scale, d_o, pe=pe)

        def loss(a):
            return float(np.sum(d_o * o.parallel(*a, s, scale, pe=pe)))

        for i, name in enumerate(names):
            fd = np.zeros_like(args[i])
            for idx in np.ndindex(args[i].shape):
                a = [x.copy() for x in args]
                a[i][idx] += eps
                lp = loss(a)
                a[i][idx] -= 2 * eps
                fd[idx] = (lp - loss(a)) / (2 * eps)
            got = np.asarray(grads[name])
            assert got.shape == fd.shape, (name, got.shape)
            assert np.max(np.abs(got - fd)) <= 1e-6 * max(1.0, np.max(np.abs(fd))), (seed, name)


ALL_PINS = [
    pin_slot_index, pin_block_starts, pin_slot_count, pin_mask_special_cases,
    pin_mask_structure, pin_mask_matches_incremental_cache, pin_cache_ratio,
    pin_row_bytes, pin_gate_zero_weights, pin_gate_per_position, pin_merge_half_sum,
    pin_block_start_overwrites,
    pin_uniform_attention_keyset, pin_absorption, pin_decode_single_slot,
    pin_s1_equals_causal_sdpa, pin_parallel_equals_incremental,
    pin_prefill_query_rows, pin_rope, pin_pe, pin_project_worked_example,
    pin_layer_worked_example, pin_max_rel_err, pin_layer_schedules,
    pin_beam_reorder_follows_history, pin_backward_finite_differences,
]
