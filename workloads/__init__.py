"""Seeded synthetic inputs for the MTLA hot path.

This module is shared by the oracle tests, the GPU parity tests and the
benchmark.  It only draws random numbers, rounds them to the storage dtype and
describes tensor shapes; it holds none of the method's arithmetic (no gate, no
merge, no mask, no attention).

Every tensor is drawn from its own stream,
``SeedSequence([ROOT_SEED, workload_id, tensor_id, b])``, so that any single
sequence ``b`` of a batch can be regenerated on its own (the oracle re-derives a
few sequences of a large workload without holding the whole batch).

Distributions.  The small full-layer workload draws ``h ~ N(0, 1)`` and every
weight ``~ N(0, 1/fan_in)``.  The other workloads enter at the kernel boundary:
the latents ``c_t``, the already-rotated rope keys ``k^R_t`` and the queries are
i.i.d. ``N(0, 1)`` (the statistics a fan-in-scaled projection of ``N(0, 1)``
activations has), and ``W_hyp``, ``W_UK``, ``W_UV`` are ``N(0, 1/d_c)``.
bf16 tensors are rounded to nearest-even from the fp32 draw; both the GPU path
and the oracle consume exactly those rounded values.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import numpy as np

ROOT_SEED = 20250513

# Stream identifiers, one per tensor role.
T_H, T_WDKV, T_WHYP, T_WUK, T_WUV, T_WQ, T_WR, T_WO = 0, 1, 2, 3, 4, 5, 6, 7
T_C, T_KR, T_QC, T_QR = 10, 11, 12, 13
T_DO = 14
T_WHYP_ROWS = 15


@dataclass(frozen=True)
class Workload:
    """Shapes of one synthetic MTLA workload.

    ``mode`` is ``"layer"`` (full layer from ``h``), ``"decode_loop"`` (N
    incremental steps from an empty cache), ``"prefill"`` (one parallel pass
    over N tokens) or ``"long_decode"`` (cache built from N tokens, then one
    appended token and one decode step).
    """
    wid: int
    name: str
    mode: str
    batch: int
    n_tokens: int
    d_model: int
    heads: int
    d_h: int
    d_c: int
    d_r: int
    s: int
    dtype: str  # "fp32" or "bf16" storage

    @property
    def width(self) -> int:
        return self.d_c + self.d_r

    @property
    def softmax_scale(self) -> float:
        return float(1.0 / np.sqrt(self.d_h + self.d_r))

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads: a tiny full-layer case, two speech-translation-shaped
# decode loops (s=2, s=4), a summarisation-shaped prefill and an LLM-scale
# long-context decode step.
WORKLOADS = [
    Workload(0, "layer_fp32_b1_n64_s2", "layer", 1, 64, 256, 4, 64, 256, 32, 2, "fp32"),
    Workload(1, "st_decode_b50_n512_s2", "decode_loop", 50, 512, 512, 8, 64, 256, 32, 2, "bf16"),
    Workload(2, "st_decode_b50_n2048_s4", "decode_loop", 50, 2048, 512, 8, 64, 256, 32, 4, "bf16"),
    Workload(3, "sum_prefill_b16_n4096_s3", "prefill", 16, 4096, 512, 8, 64, 256, 32, 3, "bf16"),
    Workload(4, "llm_decode_b64_n32768_s2", "long_decode", 64, 32768, 4096, 32, 128, 512, 64, 2, "bf16"),
]


def workload(i: int) -> Workload:
    return WORKLOADS[i]


# ----------------------------------------------------------------------------
# bf16 round-to-nearest-even on the host (storage quantisation of inputs).
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    # finite values: u + 0x7fff + lsb stays below 2^32 (largest is 0xff7fffff)
    r = u + np.uint32(0x7FFF)
    r += (u >> np.uint32(16)) & np.uint32(1)
    r >>= np.uint32(16)
    out = r.astype(np.uint16)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round an fp32 array to the storage dtype and return it as fp32 values."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "fp32":
        return x
    if dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(x))
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# Streams
# ----------------------------------------------------------------------------

def rng(wid: int, tensor_id: int, b: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([ROOT_SEED, wid, tensor_id, b])))


def normal(wid: int, tensor_id: int, shape, std: float = 1.0, b: int = 0) -> np.ndarray:
    """fp32 draw of N(0, std^2) from the (wid, tensor_id, b) stream."""
    g = rng(wid, tensor_id, b)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


# ----------------------------------------------------------------------------
# Boundary tensors (what the C-ABI consumes), per workload
# ----------------------------------------------------------------------------

def weights(w: Workload) -> dict:
    """W_hyp [d_c], W_UK [H, d_h, d_c], W_UV [H, d_h, d_c], rounded to storage.

    W_hyp is kept in fp32 (the gate weights are an fp32 operand of the kernel).
    """
    std = 1.0 / np.sqrt(w.d_c)
    return {
        "w_hyp": normal(w.wid, T_WHYP, (w.d_c,), std),
        "w_uk": quantize(normal(w.wid, T_WUK, (w.heads, w.d_h, w.d_c), std), w.dtype),
        "w_uv": quantize(normal(w.wid, T_WUV, (w.heads, w.d_h, w.d_c), std), w.dtype),
    }


def latents(w: Workload, b: int, n_tokens: Optional[int] = None) -> dict:
    """Per-token latents c [T, d_c] and rotated rope keys k_r [T, d_r] of sequence b."""
    T = w.n_tokens if n_tokens is None else n_tokens
    return {
        "c": quantize(normal(w.wid, T_C, (T, w.d_c), b=b), w.dtype),
        "k_r": quantize(normal(w.wid, T_KR, (T, w.d_r), b=b), w.dtype),
    }


def queries(w: Workload, b: int, n_tokens: Optional[int] = None) -> dict:
    """Per-token queries q_c [T, H, d_h] and rotated q_r [T, H, d_r] of sequence b."""
    T = w.n_tokens if n_tokens is None else n_tokens
    return {
        "q_c": quantize(normal(w.wid, T_QC, (T, w.heads, w.d_h), b=b), w.dtype),
        "q_r": quantize(normal(w.wid, T_QR, (T, w.heads, w.d_r), b=b), w.dtype),
    }


def gate_rows_weights(w: Workload) -> np.ndarray:
    """W_hyp with one row per place in the block, [s, d_c] fp32 (the
    per-position gate variant), from a stream of its own."""
    return normal(w.wid, T_WHYP_ROWS, (w.s, w.d_c), 1.0 / np.sqrt(w.d_c))


def batch_latents(w: Workload, n_tokens: Optional[int] = None, seqs=None) -> dict:
    seqs = range(w.batch) if seqs is None else seqs
    parts = [latents(w, b, n_tokens) for b in seqs]
    return {k: np.stack([p[k] for p in parts]) for k in ("c", "k_r")}


def batch_queries(w: Workload, n_tokens: Optional[int] = None, seqs=None) -> dict:
    seqs = range(w.batch) if seqs is None else seqs
    parts = [queries(w, b, n_tokens) for b in seqs]
    return {k: np.stack([p[k] for p in parts]) for k in ("q_c", "q_r")}


def batch_grad_out(w: Workload, seqs=None) -> np.ndarray:
    """Upstream gradient dL/do [B, N, H, d_h] for the training backward: N(0, 1)."""
    seqs = range(w.batch) if seqs is None else seqs
    return np.stack([quantize(normal(w.wid, T_DO, (w.n_tokens, w.heads, w.d_h), b=b), w.dtype) for b in seqs])


def layer_params(w: Workload) -> dict:
    """Full-layer inputs: h [B, N, d_model] and every projection, N(0, 1/fan_in)."""
    dm, H = w.d_model, w.heads
    f = lambda tid, shape, fan: quantize(normal(w.wid, tid, shape, 1.0 / np.sqrt(fan)), w.dtype)
    return {
        "h": np.stack([quantize(normal(w.wid, T_H, (w.n_tokens, dm), b=b), w.dtype) for b in range(w.batch)]),
        "w_dkv": f(T_WDKV, (w.d_c, dm), dm),
        "w_q": f(T_WQ, (H * (w.d_h + w.d_r), dm), dm),
        "w_r": f(T_WR, (w.d_r, dm), dm),
        "w_o": f(T_WO, (dm, H * w.d_h), H * w.d_h),
        **weights(w),
    }


def small(wid: int = 0, **kw) -> Workload:
    """A workload with shapes overridden (for tests at oracle-friendly sizes)."""
    return WORKLOADS[wid].with_(**kw)


def boundary_case(seed: int, B: int, N: int, H: int, d_h: int, d_c: int, d_r: int,
                  dtype: str, w_hyp_zero: bool = False, q_zero: bool = False,
                  q_rows: Optional[int] = None, gate_rows: int = 0) -> dict:
    """Seeded Gaussian kernel-boundary inputs of arbitrary shape (test cases).

    Same distributions as the named workloads; ``w_hyp_zero`` and ``q_zero``
    give the closed-form special cases (every gate 1/2; uniform attention).
    ``q_rows`` limits the queries to that many token rows (default: N).
    ``gate_rows`` > 0 draws W_hyp with that many rows (one per place in the
    block), after every other tensor, so the others are the same draws.
    """
    Q = N if q_rows is None else q_rows
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([ROOT_SEED, 1000 + seed])))
    f = lambda *shape: g.standard_normal(shape, dtype=np.float32)
    std = np.float32(1.0 / np.sqrt(d_c))
    case = {
        "c": quantize(f(B, N, d_c), dtype),
        "k_r": quantize(f(B, N, d_r), dtype),
        "q_c": quantize(f(B, Q, H, d_h), dtype),
        "q_r": quantize(f(B, Q, H, d_r), dtype),
        "w_hyp": f(d_c) * std,
        "w_uk": quantize(f(H, d_h, d_c) * std, dtype),
        "w_uv": quantize(f(H, d_h, d_c) * std, dtype),
    }
    if gate_rows > 0:
        case["w_hyp"] = f(gate_rows, d_c) * std
    if w_hyp_zero:
        case["w_hyp"] = np.zeros(d_c, np.float32)
    if q_zero:
        case["q_c"] = np.zeros_like(case["q_c"])
        case["q_r"] = np.zeros_like(case["q_r"])
    return case
