"""CPU: plant plausible mistakes in the oracle and show the pins catch each one.

Every mutation replaces one oracle function with a subtly wrong variant (an
off-by-one key set, a missing block reset, a dropped rope term, a transposed
operand, a wrong scale, ...).  The pin suite must fail for every mutation; if a
mutation survived, the pins would not be strong enough to trust the oracle.
"""
import numpy as np
import pytest

import oracle
from oracle import mtla as O
from tests import oracle_pins as pins


def _visible_keys_block_starts(i, s):
    # completed slots read at the first token of each block instead of the last
    return [s * (b - 1) + 1 for b in range(1, O.slot_of(i, s))] + [i]


def _visible_keys_off_by_one(i, s):
    return [s * b for b in range(1, O.slot_of(i, s) - 1)] + [i]


def _visible_keys_no_diag(i, s):
    ks = [s * b for b in range(1, O.slot_of(i, s))]
    return ks if ks else [i]


def _opens_slot_wrong(t, s):
    return t % s == 0


def _slot_of_floor(t, s):
    return t // s + 1


def _partial_merges_no_reset(x, w, s):
    x = np.asarray(x, dtype=float)
    return np.cumsum(w[:, None] * x, axis=0)


def _append_token_always_add(cache, x_t, w_t, t, s):
    b = O.slot_of(t, s)
    cache[b - 1] = cache[b - 1] + w_t * np.asarray(x_t, dtype=float)


def _decode_absorbed_no_rope(q_c, q_r, slots, w_uk, w_uv, d_c, scale):
    return _ORIG["decode_absorbed"](q_c, np.zeros_like(np.asarray(q_r, dtype=float)), slots, w_uk, w_uv, d_c, scale)


def _decode_absorbed_uv_from_uk(q_c, q_r, slots, w_uk, w_uv, d_c, scale):
    return _ORIG["decode_absorbed"](q_c, q_r, slots, w_uk, w_uk, d_c, scale)


def _decode_absorbed_scale_sq(q_c, q_r, slots, w_uk, w_uv, d_c, scale):
    return _ORIG["decode_absorbed"](q_c, q_r, slots, w_uk, w_uv, d_c, scale * scale)


def _gate_product(c, pe, w_hyp, t_first=1):
    return O.sigmoid((np.asarray(c) * np.asarray(pe)) @ np.asarray(w_hyp))


def _gate_no_pe(c, pe, w_hyp, t_first=1):
    return O.sigmoid(np.asarray(c, dtype=float) @ np.asarray(w_hyp, dtype=float))


def _gate_rows_place_off_by_one(w_hyp, T, t_first=1):
    # token t takes row t mod s instead of its place (t - 1) mod s
    wh = np.asarray(w_hyp, dtype=float)
    if wh.ndim == 1:
        return np.broadcast_to(wh, (T, wh.shape[0]))
    return wh[(t_first + np.arange(T)) % wh.shape[0]]


def _gate_rows_ignore_start(w_hyp, T, t_first=1):
    # a continuation restarts the places at its first token
    return _ORIG["gate_rows"](w_hyp, T, 1)


def _softmax_no_max(z):
    e = np.exp(np.asarray(z, dtype=float))
    return e / e.sum(axis=-1, keepdims=True) * 0.999


def _rope_sign(x, p):
    return _ORIG["rope"](x, -p) if p else np.asarray(x, dtype=float) * 1.0


def _pe_swapped(n, d):
    pe = _ORIG["sinusoidal_pe"](n, d)
    return pe[:, ::-1].copy()


def _cache_elements_floor(n, s, d_c, d_r):
    from fractions import Fraction
    return Fraction((n // s) * (d_c + d_r), n)


def _row_bytes_no_rope(d_c, d_r, e):
    return d_c * e


def _reorder_own_length(cache, open_state, pos, src, s):
    # copies as many slots as the destination held before, not its parent
    out, op, po = _ORIG["reorder_state"](cache, open_state, pos, np.arange(len(src)), s)
    for b in range(len(src)):
        a = int(src[b])
        n = O.num_slots(int(pos[b]), s) if pos[b] > 0 else 0
        out[b] = 0
        out[b, :n] = cache[a, :n]
        op[b] = open_state[a]
        po[b] = pos[a]
    return out, op, po


def _reorder_scatter(cache, open_state, pos, src, s):
    # treats src as destinations (scatter) instead of parents (gather)
    out = np.zeros_like(cache)
    op = np.empty_like(open_state)
    po = np.empty(len(src), dtype=np.int64)
    for a in range(len(src)):
        b = int(src[a])
        n = O.num_slots(int(pos[a]), s)
        out[b, :n] = cache[a, :n]
        op[b] = open_state[a]
        po[b] = pos[a]
    return out, op, po


def _merges_backward_prefix(dP, s):
    # sums the block's tokens up to k (the forward's own direction) instead of from k on
    dP = np.asarray(dP, dtype=float)
    G = np.zeros_like(dP)
    for k in range(1, dP.shape[0] + 1):
        for j in range(s * ((k - 1) // s) + 1, k + 1):
            G[k - 1] += dP[j - 1]
    return G


def _merges_backward_no_reset(dP, s):
    # suffix sum over the whole sequence, ignoring block ends
    return np.cumsum(np.asarray(dP, dtype=float)[::-1], axis=0)[::-1]


def _softmax_backward_no_rowsum(a, da):
    return np.asarray(a, dtype=float) * np.asarray(da, dtype=float)


def _gate_backward_no_pe(c, pe, w_hyp, w, dw, t_first=1):
    return _ORIG["gate_backward"](c, np.zeros_like(np.asarray(pe, dtype=float)), w_hyp, w, dw, t_first)


def _gate_backward_no_sigmoid_slope(c, pe, w_hyp, w, dw, t_first=1):
    # takes dw as du (drops the sigmoid's derivative w (1 - w))
    du = np.asarray(dw, dtype=float)
    w_hyp = np.asarray(w_hyp, dtype=float)
    return du[:, None] * w_hyp[None, :], (np.asarray(c) + np.asarray(pe)).T @ du


def _gate_backward_rows_summed(c, pe, w_hyp, w, dw, t_first=1):
    # per-position W_hyp: every row receives the gradient of all the tokens
    dc, dwh = _ORIG["gate_backward"](c, pe, w_hyp, w, dw, t_first)
    if np.asarray(w_hyp).ndim == 2:
        dwh = np.tile(dwh.sum(axis=0), (dwh.shape[0], 1))
    return dc, dwh


def _project_parts(h, p, heads, d_h, d_r):
    h = np.asarray(h, dtype=float)
    N = h.shape[0]
    c = h @ np.asarray(p["w_dkv"], dtype=float).T
    q = (h @ np.asarray(p["w_q"], dtype=float).T).reshape(N, heads, d_h + d_r)
    k = h @ np.asarray(p["w_r"], dtype=float).T
    return N, c, q, k


def _project_k_unrotated(h, p, heads, d_h, d_r):
    # the shared rope key is cached without its rotation
    N, c, q, k = _project_parts(h, p, heads, d_h, d_r)
    q_r = np.stack([O.rope(q[t, :, d_h:], t) for t in range(N)])
    return c, k, q[:, :, :d_h], q_r


def _project_rope_one_off(h, p, heads, d_h, d_r):
    # both rope parts turned at position t instead of t - 1
    N, c, q, k = _project_parts(h, p, heads, d_h, d_r)
    q_r = np.stack([O.rope(q[t, :, d_h:], t + 1) for t in range(N)])
    k_r = np.stack([O.rope(k[t], t + 1) for t in range(N)])
    return c, k_r, q[:, :, :d_h], q_r


def _project_split_swapped(h, p, heads, d_h, d_r):
    # per head the rope query is taken from the first d_r rows, the content from the rest
    N, c, q, k = _project_parts(h, p, heads, d_h, d_r)
    q_r = np.stack([O.rope(q[t, :, :d_r], t) for t in range(N)])
    k_r = np.stack([O.rope(k[t], t) for t in range(N)])
    return c, k_r, q[:, :, d_r:], q_r


def _layer_heads_reversed(h, p, heads, d_h, d_r, s, scale, schedule="incremental"):
    # heads concatenated last first before the output projection
    c, k_r, q_c, q_r = O.project(h, p, heads, d_h, d_r)
    fn = O.incremental if schedule == "incremental" else O.parallel
    o = fn(c, k_r, q_c, q_r, p["w_hyp"], p["w_uk"], p["w_uv"], s, scale)
    return o[:, ::-1].reshape(o.shape[0], -1) @ np.asarray(p["w_o"], dtype=float).T


def _layer_heads_interleaved(h, p, heads, d_h, d_r, s, scale, schedule="incremental"):
    # the concatenation runs over heads fastest instead of over each head's d_h
    c, k_r, q_c, q_r = O.project(h, p, heads, d_h, d_r)
    fn = O.incremental if schedule == "incremental" else O.parallel
    o = fn(c, k_r, q_c, q_r, p["w_hyp"], p["w_uk"], p["w_uv"], s, scale)
    return o.transpose(0, 2, 1).reshape(o.shape[0], -1) @ np.asarray(p["w_o"], dtype=float).T


def _max_rel_err_zero(y, y_ref):
    return 0.0


def _max_rel_err_by_result(y, y_ref):
    y, y_ref = np.asarray(y, dtype=float), np.asarray(y_ref, dtype=float)
    return float(np.max(np.abs(y - y_ref)) / np.max(np.abs(y)))


def _max_rel_err_mean(y, y_ref):
    y, y_ref = np.asarray(y, dtype=float), np.asarray(y_ref, dtype=float)
    return float(np.mean(np.abs(y - y_ref)) / np.max(np.abs(y_ref)))


def _max_rel_err_elementwise(y, y_ref):
    y, y_ref = np.asarray(y, dtype=float), np.asarray(y_ref, dtype=float)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.abs(y - y_ref) / np.abs(y_ref)
    return float(np.nanmax(np.where(np.isfinite(r), r, 0.0)))


def _max_rel_err_signed_den(y, y_ref):
    y, y_ref = np.asarray(y, dtype=float), np.asarray(y_ref, dtype=float)
    return float(np.max(np.abs(y - y_ref)) / np.max(y_ref))


_ORIG = {name: getattr(O, name) for name in
         ("decode_absorbed", "rope", "sinusoidal_pe", "reorder_state", "gate_backward", "gate_rows")}

MUTATIONS = {
    "visible_keys": [_visible_keys_block_starts, _visible_keys_off_by_one, _visible_keys_no_diag],
    "opens_slot": [_opens_slot_wrong],
    "slot_of": [_slot_of_floor],
    "partial_merges": [_partial_merges_no_reset],
    "append_token": [_append_token_always_add],
    "decode_absorbed": [_decode_absorbed_no_rope, _decode_absorbed_uv_from_uk, _decode_absorbed_scale_sq],
    "gate": [_gate_product, _gate_no_pe],
    "gate_rows": [_gate_rows_place_off_by_one, _gate_rows_ignore_start],
    "softmax": [_softmax_no_max],
    "rope": [_rope_sign],
    "sinusoidal_pe": [_pe_swapped],
    "cache_elements_per_token": [_cache_elements_floor],
    "cache_row_bytes": [_row_bytes_no_rope],
    "reorder_state": [_reorder_own_length, _reorder_scatter],
    "partial_merges_backward": [_merges_backward_prefix, _merges_backward_no_reset],
    "softmax_backward": [_softmax_backward_no_rowsum],
    "gate_backward": [_gate_backward_no_pe, _gate_backward_no_sigmoid_slope, _gate_backward_rows_summed],
    "project": [_project_k_unrotated, _project_rope_one_off, _project_split_swapped],
    "layer": [_layer_heads_reversed, _layer_heads_interleaved],
    "max_rel_err": [_max_rel_err_zero, _max_rel_err_by_result, _max_rel_err_mean,
                    _max_rel_err_elementwise, _max_rel_err_signed_den],
}

CASES = [(name, fn) for name, fns in MUTATIONS.items() for fn in fns]


def _pins_fail(o):
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError, IndexError) as e:  # a pin caught it
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name,fn", CASES, ids=[f"{n}:{f.__name__}" for n, f in CASES])
def test_mutation_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(O, name, fn)
    failed = _pins_fail(O)
    assert failed, f"mutation {fn.__name__} of {name} survived every pin"
