"""Batched calls into the fp64 oracle for the GPU parity tests."""
import numpy as np

import oracle


def incremental(inp: dict, b: int, n: int, s: int, scale: float, q_rows=None):
    c, k_r = inp["c"][b, :n], inp["k_r"][b, :n]
    q_c, q_r = inp["q_c"][b, :n], inp["q_r"][b, :n]
    return oracle.incremental(c, k_r, q_c, q_r, inp["w_hyp"], inp["w_uk"], inp["w_uv"], s, scale,
                              pe=oracle.sinusoidal_pe(n, c.shape[1]), return_cache=True)


def parallel(inp: dict, b: int, n: int, s: int, scale: float):
    c, k_r = inp["c"][b, :n], inp["k_r"][b, :n]
    return oracle.parallel(c, k_r, inp["q_c"][b, :n], inp["q_r"][b, :n], inp["w_hyp"], inp["w_uk"],
                           inp["w_uv"], s, scale, pe=oracle.sinusoidal_pe(n, c.shape[1]),
                           return_partials=True)


def merged_cache(c, k_r, w_hyp, s: int, t0: int = 1, cache=None):
    """Slot cache after appending tokens t0.. (rows of c, k_r) to ``cache``."""
    n = t0 + c.shape[0] - 1
    pe = oracle.sinusoidal_pe(n, c.shape[1])[t0 - 1:]
    w = oracle.gate(c, pe, w_hyp, t_first=t0)
    x = np.concatenate([np.asarray(c, np.float64), np.asarray(k_r, np.float64)], axis=1)
    return oracle.merge_incremental(x, w, s, cache=cache, t0=t0), w


def step_errors(got, want) -> np.ndarray:
    """Parity of every call of a token-by-token loop: got and want hold the
    outputs with the sequence on axis 0 and the step on axis 1; each step's
    [B, ...] tensor is one call's output, measured on its own by
    oracle.max_rel_err.  Returns the error of every step."""
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, (got.shape, want.shape)
    return np.array([oracle.max_rel_err(got[:, t], want[:, t]) for t in range(got.shape[1])])


def assert_steps(got, want, bound: float, what: str = "") -> np.ndarray:
    """step_errors, every step within `bound`; reports the worst step."""
    e = step_errors(got, want)
    worst = int(np.argmax(e)) if e.size else 0
    if e.size:
        assert e[worst] <= bound, f"{what} step {worst + 1}: max relative error {e[worst]:.3e} > {bound}"
    return e


def loop_outputs(inp: dict, B: int, n: int, s: int, scale: float):
    """The oracle's token-by-token outputs [B, n, H, d_h] and final slot
    caches of the first B sequences of a boundary case."""
    outs, caches = [], []
    for b in range(B):
        o, cache = incremental(inp, b, n, s, scale)
        outs.append(o)
        caches.append(cache)
    return np.stack(outs), caches
