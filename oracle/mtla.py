"""fp64 CPU oracle for the Multi-head Temporal Latent Attention (MTLA) hot path.

TEST INFRASTRUCTURE.  This module states, as plainly as possible, what the
hot path computes, so that the HIP kernels can be checked against it.  Only
the tests, the smoke check and the benchmark's CPU-baseline leg may import it;
the product path never does.  It shares no code with the HIP library.

Sources (web pages on MTLA; cited by page title and section):
  [MTLA-wiki]  "Multi-head Temporal Latent Attention" (wiki summary of the
               NeurIPS 2025 paper): TL;DR, Key claims, Method.  It cites the
               paper's Sec. 4, Sec. 4.1 Eq. 13, Sec. 4.2 Fig. 2(c), Sec. 4.3
               Eq. 17 and Sec. 6.1.
  [MLA-expl]   "Multi-Head Latent Attention and Sparse Indexers": "Latent
               attention changes the representation" (absorption algebra) and
               "Work the bytes with units and scope" (row bytes).
  [MTLA-repo]  The MTLA repository summary page, "Highlighted Details"
               (evaluation with Fairseq-style parallel beam search).

Indexing.  Tokens and slots are 1-based in the formulas (t, i, j in 1..N;
slot b in 1..ceil(N/s)), as the pages write ceil(t/s).  Arrays are 0-based;
token t lives at array row t-1 and slot b at row b-1.

Readings where the pages are silent or garbled (each is listed, with its
reason, in the design notes):
  * gate input is c_t + pe_t (Key claims: "latent input plus positional
    embedding"; the Method paragraph says "multiplied");
  * one scalar gate per token, w_t = sigmoid(W_hyp . (c_t + pe_t)), no bias;
    the s gates of a block form the merge weights W in R^s, and the same w_t
    scales both c_t and k^R_t.  A variant takes W_hyp in R^{s x d_c}, the
    linear layer's s outputs, of which token t uses output (t - 1) mod s;
  * the first token of a block overwrites its slot, later tokens add to it;
  * sinusoidal pe and RoPE use interleaved (even, odd) pairs, base 10000,
    position t-1; RoPE is applied before merging;
  * softmax scale 1/sqrt(d_h + d_R);
  * no biases, no query compression, no latent normalisation.

Training backward.  ``parallel_backward`` takes reverse mode through the
steps of ``parallel`` (gate, partial merges, explicit keys/values, masked
softmax attention); its pin is central differences of ``parallel`` itself.

Parity status of the conventions (gate input, pe and RoPE formulas, scale):
"parity unpinned" against the pages, which print no worked example.  Every
structural part (slot index, mask, merge, absorption, attention) is pinned by
the CPU tests listed in tests/test_oracle_pins.py.
"""
from __future__ import annotations

from fractions import Fraction
from typing import Dict, List, Optional

import numpy as np

F = np.float64


# ---------------------------------------------------------------------------
# Integer structure: slots, block starts, the stride-aware mask
# ---------------------------------------------------------------------------

def slot_of(t: int, s: int) -> int:
    """Cache slot (1-based) that token t (1-based) is merged into: ceil(t/s).

    [MTLA-wiki] Method (1): every s adjacent latents merge into one slot; only
    every s-th step opens a new slot, the others update the open slot in place.
    """
    if t < 1 or s < 1:
        raise ValueError("t and s are 1-based and positive")
    return -(-t // s)


def opens_slot(t: int, s: int) -> bool:
    """True when token t is the first token of its block, i.e. (t-1) mod s == 0."""
    return (t - 1) % s == 0


def num_slots(n: int, s: int) -> int:
    """Slots a cache holds after n tokens: ceil(n/s)."""
    return -(-n // s) if n > 0 else 0


def visible_keys(i: int, s: int) -> List[int]:
    """Token positions j (1-based) whose cumulative partial merge query i sees.

    [MTLA-wiki] Key claims / Method (2), paper Sec. 4.2 Fig. 2(c): during
    incremental decoding, query i attends the completed slots 1..ceil(i/s)-1
    and its own, partially filled slot ceil(i/s).  With original-length
    cumulative partial merges P_j (Sec. 4.3), the completed slot b is the value
    P_{s*b} and the own partial slot is P_i.  Hence the key set is
    {s*b : b < ceil(i/s)} together with {i}.
    """
    own = slot_of(i, s)
    return [s * b for b in range(1, own)] + [i]


def stride_mask(n: int, s: int) -> np.ndarray:
    """Boolean [n, n] mask, M[i-1, j-1] = True iff query i may attend key j.

    Built from visible_keys, one query at a time (the definition, no algebra).
    """
    m = np.zeros((n, n), dtype=bool)
    for i in range(1, n + 1):
        for j in visible_keys(i, s):
            m[i - 1, j - 1] = True
    return m


def completed_slots(i: int, s: int) -> int:
    """Number of completed slots query i sees: ceil(i/s) - 1 = floor((i-1)/s)."""
    return slot_of(i, s) - 1


def cache_elements_per_token(n: int, s: int, d_c: int, d_r: int) -> Fraction:
    """Stored cache elements per processed token, per layer: ceil(n/s)(d_c+d_r)/n."""
    return Fraction(num_slots(n, s) * (d_c + d_r), n)


def cache_ratio_vs_mqa(n: int, s: int, d_h: int, d_c: int, d_r: int) -> Fraction:
    """Cache size relative to MQA (one K and one V head of width d_h per token).

    [MTLA-wiki] Key claims, paper Sec. 4.3: with d_c = 4 d_h and d_R = d_h/2 the
    average is 9/(4s) elements per token per layer, "close to MQA's 1".
    """
    return cache_elements_per_token(n, s, d_c, d_r) / (2 * d_h)


def cache_row_bytes(d_c: int, d_r: int, bytes_per_element: int) -> int:
    """Bytes of one stored latent row: (latent + rotary) x element size.

    [MLA-expl] "Work the bytes with units and scope".
    """
    return (d_c + d_r) * bytes_per_element


# ---------------------------------------------------------------------------
# Positional embedding, RoPE, gate
# ---------------------------------------------------------------------------

def sinusoidal_pe(n_rows: int, d: int) -> np.ndarray:
    """pe[p, 2k] = sin(p * 10000^(-2k/d)), pe[p, 2k+1] = cos(same); p = t-1.

    [MTLA-wiki] Key claims, paper Sec. 4.1: the hyper-network sees the latent
    plus a positional embedding.  The formula is the sinusoidal reading.
    """
    p = np.arange(n_rows, dtype=F)[:, None]
    e = np.arange(d)[None, :]
    k = (e // 2).astype(F)                      # pair index of element e
    ang = p * 10000.0 ** (-2.0 * k / d)
    return np.where(e % 2 == 0, np.sin(ang), np.cos(ang))


def rope(x: np.ndarray, p: int) -> np.ndarray:
    """Rotate interleaved pairs (2k, 2k+1) of the last axis by p * 10000^(-2k/d).

    [MTLA-wiki] Method (3): decoupled RoPE keys, as in MLA.
    """
    x = np.asarray(x, dtype=F)
    d = x.shape[-1]
    out = np.empty_like(x)
    for k in range(d // 2):
        ang = p * 10000.0 ** (-2.0 * k / d)
        c, s_ = np.cos(ang), np.sin(ang)
        a, b = x[..., 2 * k], x[..., 2 * k + 1]
        out[..., 2 * k] = a * c - b * s_
        out[..., 2 * k + 1] = a * s_ + b * c
    return out


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def gate_rows(w_hyp: np.ndarray, T: int, t_first: int = 1) -> np.ndarray:
    """The W_hyp row each of T consecutive tokens t_first.. takes: [T, d_c].

    w_hyp [d_c] is one weight vector for every token.  w_hyp [s, d_c] is the
    per-position variant: the hyper-network's linear layer has s outputs (the
    merge weights W_t in R^s of [MTLA-wiki] Method (1)), and token t takes
    output (t - 1) mod s, its own place in its block.
    """
    wh = np.asarray(w_hyp, dtype=F)
    if wh.ndim == 1:
        return np.broadcast_to(wh, (T, wh.shape[0]))
    return wh[(t_first - 1 + np.arange(T)) % wh.shape[0]]


def gate(c: np.ndarray, pe: np.ndarray, w_hyp: np.ndarray, t_first: int = 1) -> np.ndarray:
    """w_t = sigmoid(W_hyp . (c_t + pe_t)) for every token row.

    [MTLA-wiki] Key claims, paper Sec. 4.1 Eq. 13.  c: [T, d_c] for tokens
    t_first .. t_first + T - 1; pe: [T, d_c] rows for the same positions;
    w_hyp: [d_c], or [s, d_c] per position in the block (see gate_rows).
    Returns [T].
    """
    c = np.asarray(c, dtype=F)
    x = c + np.asarray(pe, dtype=F)
    return sigmoid(np.sum(x * gate_rows(w_hyp, c.shape[0], t_first), axis=1))


# ---------------------------------------------------------------------------
# Merge: incremental (slot by slot) and parallel (cumulative partial merges)
# ---------------------------------------------------------------------------

def append_token(cache: np.ndarray, x_t: np.ndarray, w_t: float, t: int, s: int) -> None:
    """Merge token t into ``cache`` in place (rows are slots, 0-based).

    [MTLA-wiki] Method (1): the first token of a block writes a new slot; the
    following tokens of the block update that slot in place.
    """
    b = slot_of(t, s)
    if opens_slot(t, s):
        cache[b - 1] = w_t * np.asarray(x_t, dtype=F)
    else:
        cache[b - 1] = cache[b - 1] + w_t * np.asarray(x_t, dtype=F)


def merge_incremental(x: np.ndarray, w: np.ndarray, s: int,
                      cache: Optional[np.ndarray] = None, t0: int = 1) -> np.ndarray:
    """Append tokens t0 .. t0+T-1 into a slot cache, one token at a time.

    x: [T, W] rows x_t = [c_t; k^R_t]; w: [T] gates.  ``cache`` holds the
    slots written so far.  Returns a new cache of ceil((t0+T-1)/s) rows.
    """
    x = np.asarray(x, dtype=F)
    T, W = x.shape
    out = np.zeros((num_slots(t0 + T - 1, s), W), dtype=F)
    if cache is not None:
        out[: cache.shape[0]] = cache
    for k in range(T):
        append_token(out, x[k], w[k], t0 + k, s)
    return out


def partial_merges(x: np.ndarray, w: np.ndarray, s: int) -> np.ndarray:
    """P_j = sum_{k = s*floor((j-1)/s)+1}^{j} w_k x_k for j = 1..N (original length).

    [MTLA-wiki] Key claims, paper Sec. 4.3 Eq. 17: training uses the
    length-N sequence of cumulative in-block merges.  Written as the sum.
    """
    x = np.asarray(x, dtype=F)
    N = x.shape[0]
    P = np.zeros_like(x)
    for j in range(1, N + 1):
        start = s * ((j - 1) // s) + 1
        acc = np.zeros(x.shape[1], dtype=F)
        for k in range(start, j + 1):
            acc = acc + w[k - 1] * x[k - 1]
        P[j - 1] = acc
    return P


# ---------------------------------------------------------------------------
# Beam reorder: the decode state follows the surviving hypotheses
# ---------------------------------------------------------------------------

def reorder_state(cache: np.ndarray, open_state: np.ndarray, pos: np.ndarray, src: np.ndarray,
                  s: int):
    """Beam-search reorder of the per-sequence decode state.

    [MTLA-repo] "Highlighted Details": the models are evaluated with
    Fairseq-style parallel beam search, where after each step every kept
    hypothesis b continues hypothesis src[b] (a parent may be kept several
    times, or dropped).  The state a hypothesis carries is its slot cache
    (slots 1..ceil(pos/s)), its open-slot fp32 value and its token count, so
    the reorder is a gather:

        cache'[b, :ceil(pos[src[b]]/s)] = cache[src[b], :ceil(pos[src[b]]/s)]
        open'[b] = open[src[b]],   pos'[b] = pos[src[b]].

    cache: [B, S, W]; open_state: [B, ...]; pos, src: [B] ints.  Rows of
    cache' past the copied slots are zero (they are never read).
    """
    cache = np.asarray(cache)
    B = cache.shape[0]
    out = np.zeros_like(cache)
    open_out = np.empty_like(np.asarray(open_state))
    pos_out = np.empty(B, dtype=np.int64)
    for b in range(B):
        a = int(src[b])
        n = num_slots(int(pos[a]), s) if pos[a] > 0 else 0
        out[b, :n] = cache[a, :n]
        open_out[b] = open_state[a]
        pos_out[b] = pos[a]
    return out, open_out, pos_out


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def softmax(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=F)
    m = np.max(z, axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def decode_absorbed(q_c, q_r, slots, w_uk, w_uv, d_c: int, scale: float) -> np.ndarray:
    """One decode step in the absorbed form, over the given slot rows.

    [MTLA-wiki] Method: W_UK folds into the query and W_UV is applied after
    the weighted latent sum, so per-step k, v are never rebuilt.
    [MLA-expl] "Latent attention changes the representation":
    q^T (U_K c) = (U_K^T q)^T c and sum_j a_j U_V c_j = U_V sum_j a_j c_j.
    q_c [H, d_h], q_r [H, d_r], slots [n, d_c+d_r], w_uk/w_uv [H, d_h, d_c].
    Returns o [H, d_h].
    """
    q_c, q_r, S = (np.asarray(a, dtype=F) for a in (q_c, q_r, slots))
    Sc, Sr = S[:, :d_c], S[:, d_c:]
    H = q_c.shape[0]
    out = np.zeros((H, w_uv.shape[1]), dtype=F)
    for h in range(H):
        q_t = np.asarray(w_uk[h], dtype=F).T @ q_c[h]          # d_c
        z = scale * (Sc @ q_t + Sr @ q_r[h])                    # n
        a = softmax(z)
        out[h] = np.asarray(w_uv[h], dtype=F) @ (a @ Sc)        # d_h
    return out


def decode_explicit(q_c, q_r, slots, w_uk, w_uv, d_c: int, scale: float) -> np.ndarray:
    """The same step with per-head keys and values rebuilt from the slots.

    k_j = W_UK[h] c_j, v_j = W_UV[h] c_j; score q^C.k_j + q^R.c^R_j.  Used to
    pin the absorption identity.
    """
    q_c, q_r, S = (np.asarray(a, dtype=F) for a in (q_c, q_r, slots))
    Sc, Sr = S[:, :d_c], S[:, d_c:]
    H = q_c.shape[0]
    out = np.zeros((H, w_uv.shape[1]), dtype=F)
    for h in range(H):
        K = Sc @ np.asarray(w_uk[h], dtype=F).T                 # n x d_h
        V = Sc @ np.asarray(w_uv[h], dtype=F).T                 # n x d_h
        a = softmax(scale * (K @ q_c[h] + Sr @ q_r[h]))
        out[h] = a @ V
    return out


def incremental(c, k_r, q_c, q_r, w_hyp, w_uk, w_uv, s: int, scale: float,
                pe: Optional[np.ndarray] = None, return_cache: bool = False):
    """Token-by-token decoding of one sequence, t = 1..N.

    At step t: gate w_t, merge x_t into slot ceil(t/s), then decode with the
    query of token t over slots 1..ceil(t/s) ([MTLA-wiki] Method (1); Key
    claims on the O(N/s) per-token cost).  c [N, d_c], k_r [N, d_r], q_c [N,
    H, d_h], q_r [N, H, d_r].  Returns o [N, H, d_h] (and the final cache).
    """
    c, k_r = np.asarray(c, dtype=F), np.asarray(k_r, dtype=F)
    N, d_c = c.shape
    if pe is None:
        pe = sinusoidal_pe(N, d_c)
    w = gate(c, pe[:N], w_hyp)
    x = np.concatenate([c, k_r], axis=1)
    cache = np.zeros((num_slots(N, s), x.shape[1]), dtype=F)
    outs = []
    for t in range(1, N + 1):
        append_token(cache, x[t - 1], w[t - 1], t, s)
        outs.append(decode_absorbed(q_c[t - 1], q_r[t - 1], cache[: slot_of(t, s)],
                                    w_uk, w_uv, d_c, scale))
    o = np.stack(outs)
    return (o, cache) if return_cache else o


def parallel(c, k_r, q_c, q_r, w_hyp, w_uk, w_uv, s: int, scale: float,
             pe: Optional[np.ndarray] = None, return_partials: bool = False):
    """Parallel (training / prefill) pass under the stride-aware mask.

    [MTLA-wiki] Key claims, Sec. 4.2-4.3: full-length cumulative partial
    merges P_j, explicit per-head keys K^C_j = W_UK[h] P^c_j and values
    V_j = W_UV[h] P^c_j, rope keys P^R_j, and a dense N x N masked softmax.
    Returns o [N, H, d_h] (and P).
    """
    c, k_r = np.asarray(c, dtype=F), np.asarray(k_r, dtype=F)
    q_c, q_r = np.asarray(q_c, dtype=F), np.asarray(q_r, dtype=F)
    N, d_c = c.shape
    if pe is None:
        pe = sinusoidal_pe(N, d_c)
    w = gate(c, pe[:N], w_hyp)
    x = np.concatenate([c, k_r], axis=1)
    P = partial_merges(x, w, s)
    Pc, Pr = P[:, :d_c], P[:, d_c:]
    M = stride_mask(N, s)
    H = q_c.shape[1]
    o = np.zeros((N, H, w_uv.shape[1]), dtype=F)
    for h in range(H):
        K = Pc @ np.asarray(w_uk[h], dtype=F).T                  # N x d_h
        V = Pc @ np.asarray(w_uv[h], dtype=F).T
        z = scale * (q_c[:, h] @ K.T + q_r[:, h] @ Pr.T)         # N x N
        z = np.where(M, z, -np.inf)
        o[:, h] = softmax(z) @ V
    return (o, P) if return_partials else o


# ---------------------------------------------------------------------------
# Training backward of the parallel pass (reverse mode through its steps)
# ---------------------------------------------------------------------------

def softmax_backward(a: np.ndarray, da: np.ndarray) -> np.ndarray:
    """dz for a = softmax(z) along the last axis: a * (da - sum(a * da)).

    Masked entries have a = 0, so their dz is 0.
    """
    a, da = np.asarray(a, dtype=F), np.asarray(da, dtype=F)
    return a * (da - np.sum(a * da, axis=-1, keepdims=True))


def partial_merges_backward(dP: np.ndarray, s: int) -> np.ndarray:
    """Adjoint of ``partial_merges`` in the weighted rows y_k = w_k x_k.

    Token k enters every partial merge P_j of its own block with j >= k (the
    sum that defines P_j starts at the block's first token), so its gradient
    is the sum of dP_j over j = k .. last token of the block (or N).  Written
    as that sum.
    """
    dP = np.asarray(dP, dtype=F)
    N = dP.shape[0]
    G = np.zeros_like(dP)
    for k in range(1, N + 1):
        end = min(s * slot_of(k, s), N)
        for j in range(k, end + 1):
            G[k - 1] = G[k - 1] + dP[j - 1]
    return G


def gate_backward(c, pe, w_hyp, w, dw, t_first: int = 1):
    """Through w_k = sigmoid(u_k), u_k = W_hyp . (c_k + pe_k): returns the
    gate's share of dc ([N, d_c]) and dW_hyp (shaped like w_hyp) given dw
    ([N]).  With one W_hyp row per position in the block, row r collects the
    tokens that take it."""
    c, pe, w_hyp = (np.asarray(a, dtype=F) for a in (c, pe, w_hyp))
    du = np.asarray(dw, dtype=F) * w * (1.0 - w)
    rows = gate_rows(w_hyp, c.shape[0], t_first)
    if w_hyp.ndim == 1:
        return du[:, None] * rows, (c + pe).T @ du
    s = w_hyp.shape[0]
    which = (t_first - 1 + np.arange(c.shape[0])) % s
    dwh = np.zeros_like(w_hyp)
    for r in range(s):
        sel = which == r
        dwh[r] = (c[sel] + pe[sel]).T @ du[sel]
    return du[:, None] * rows, dwh


def parallel_backward(c, k_r, q_c, q_r, w_hyp, w_uk, w_uv, s: int, scale: float,
                      d_o, pe: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Gradients of L = sum(d_o * parallel(...)) for one sequence.

    The training use of the stride-aware mask ([MTLA-wiki] Key claims, paper
    Sec. 4.2-4.3).  Reverse mode through the steps of ``parallel``, last step
    first: the masked softmax attention per head (scores from explicit keys
    K^C_j = W_UK[h] P^c_j and rope keys P^R_j, values W_UV[h] P^c_j), the
    explicit key/value up-projection, the cumulative in-block partial merges,
    and the gate.  d_o [N, H, d_h].  Returns dc, dk_r, dq_c, dq_r, dw_hyp,
    dw_uk, dw_uv, shaped like the inputs.
    """
    c, k_r = np.asarray(c, dtype=F), np.asarray(k_r, dtype=F)
    q_c, q_r = np.asarray(q_c, dtype=F), np.asarray(q_r, dtype=F)
    w_uk, w_uv, d_o = (np.asarray(a, dtype=F) for a in (w_uk, w_uv, d_o))
    N, d_c = c.shape
    H = q_c.shape[1]
    if pe is None:
        pe = sinusoidal_pe(N, d_c)
    pe = np.asarray(pe, dtype=F)[:N]
    # forward, kept for the backward
    w = gate(c, pe, w_hyp)
    x = np.concatenate([c, k_r], axis=1)
    P = partial_merges(x, w, s)
    Pc, Pr = P[:, :d_c], P[:, d_c:]
    M = stride_mask(N, s)
    dPc = np.zeros_like(Pc)
    dPr = np.zeros_like(Pr)
    dq_c = np.zeros_like(q_c)
    dq_r = np.zeros_like(q_r)
    dw_uk = np.zeros_like(w_uk)
    dw_uv = np.zeros_like(w_uv)
    for h in range(H):
        K = Pc @ w_uk[h].T
        V = Pc @ w_uv[h].T
        z = np.where(M, scale * (q_c[:, h] @ K.T + q_r[:, h] @ Pr.T), -np.inf)
        A = softmax(z)
        # o_h = A V
        dA = d_o[:, h] @ V.T
        dV = A.T @ d_o[:, h]
        dz = scale * softmax_backward(A, dA)
        # z = scale (q^C K^T + q^R P^R^T)
        dq_c[:, h] = dz @ K
        dq_r[:, h] = dz @ Pr
        dK = dz.T @ q_c[:, h]
        dPr += dz.T @ q_r[:, h]
        # K = P^c W_UK[h]^T, V = P^c W_UV[h]^T
        dPc += dK @ w_uk[h] + dV @ w_uv[h]
        dw_uk[h] = dK.T @ Pc
        dw_uv[h] = dV.T @ Pc
    # P_j = sum over the block's tokens k <= j of w_k x_k
    G = partial_merges_backward(np.concatenate([dPc, dPr], axis=1), s)
    dx = w[:, None] * G
    dw = np.sum(G * x, axis=1)
    dc_gate, dw_hyp = gate_backward(c, pe, w_hyp, w, dw)
    return {"dc": dx[:, :d_c] + dc_gate, "dk_r": dx[:, d_c:], "dq_c": dq_c, "dq_r": dq_r,
            "dw_hyp": dw_hyp, "dw_uk": dw_uk, "dw_uv": dw_uv}


def prefill_query(P: np.ndarray, i: int, q_c_i, q_r_i, w_uk, w_uv, s: int,
                  d_c: int, scale: float) -> np.ndarray:
    """Output of one query i (1-based) of the parallel pass, from its key set.

    Same definition as ``parallel`` restricted to row i: keys are the partial
    merges at visible_keys(i, s).  Lets large workloads be checked on samples.
    """
    keys = [j - 1 for j in visible_keys(i, s)]
    Pk = np.asarray(P, dtype=F)[keys]
    return decode_explicit(q_c_i, q_r_i, Pk, w_uk, w_uv, d_c, scale)


# ---------------------------------------------------------------------------
# Full layer (projections, RoPE, MTLA attention, output projection)
# ---------------------------------------------------------------------------

def project(h, p: Dict[str, np.ndarray], heads: int, d_h: int, d_r: int):
    """c_t = W_DKV h_t; q_t = W_Q h_t split per head into (q^C, q^R); k^R_t = W_R h_t.

    RoPE at position t-1 is applied to q^R and k^R ([MTLA-wiki] Method).
    h [N, d_model].  Returns c [N,d_c], k_r [N,d_r], q_c [N,H,d_h], q_r [N,H,d_r].
    """
    h = np.asarray(h, dtype=F)
    N = h.shape[0]
    c = h @ np.asarray(p["w_dkv"], dtype=F).T
    q = (h @ np.asarray(p["w_q"], dtype=F).T).reshape(N, heads, d_h + d_r)
    k_r = h @ np.asarray(p["w_r"], dtype=F).T
    q_c = q[:, :, :d_h]
    q_r = np.stack([rope(q[t, :, d_h:], t) for t in range(N)])
    k_r = np.stack([rope(k_r[t], t) for t in range(N)])
    return c, k_r, q_c, q_r


def layer(h, p: Dict[str, np.ndarray], heads: int, d_h: int, d_r: int, s: int,
          scale: float, schedule: str = "incremental"):
    """y_t = W_O [o_{t,1}; ...; o_{t,H}] for one sequence h [N, d_model]."""
    c, k_r, q_c, q_r = project(h, p, heads, d_h, d_r)
    fn = incremental if schedule == "incremental" else parallel
    o = fn(c, k_r, q_c, q_r, p["w_hyp"], p["w_uk"], p["w_uv"], s, scale)
    N = o.shape[0]
    return o.reshape(N, -1) @ np.asarray(p["w_o"], dtype=F).T


# ---------------------------------------------------------------------------
# Error measure used for parity
# ---------------------------------------------------------------------------

def max_rel_err(y, y_ref) -> float:
    """||y - y_ref||_inf / ||y_ref||_inf over a whole output tensor."""
    y = np.asarray(y, dtype=F)
    y_ref = np.asarray(y_ref, dtype=F)
    den = np.max(np.abs(y_ref))
    num = np.max(np.abs(y - y_ref))
    return float(num / den) if den > 0 else float(num)
