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
