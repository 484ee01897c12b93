"""GPU: the training backward of the parallel pass (mtla_prefill_backward)
against the oracle's reverse mode (oracle.parallel_backward), every gradient,
the weight gradients summed over the batch."""
import numpy as np
import pytest
import torch

import oracle
import workloads
import temporally_compressed_latent_amd as m
from tests.gpu_util import DEV, host, tdev, tol

pytestmark = pytest.mark.gpu

NAMES = ("dc", "dk_r", "dq_c", "dq_r", "dw_hyp", "dw_uk", "dw_uv")


def _inputs(seed, B, N, H, d_h, d_c, d_r, dtype):
    inp = workloads.boundary_case(seed, B, N, H, d_h, d_c, d_r, dtype)
    g = np.random.default_rng(seed + 7)
    inp["d_o"] = workloads.quantize(g.standard_normal((B, N, H, d_h)).astype(np.float32), dtype)
    return inp


def _gpu_backward(inp, s, dtype, reps=1, portable=False):
    B, N, d_c = inp["c"].shape
    H, d_h = inp["q_c"].shape[2], inp["q_c"].shape[3]
    d_r = inp["k_r"].shape[2]
    d = m.make_dims(B, H, d_h, d_c, d_r, s, max(1, -(-N // s)), dtype)
    if portable:
        d.flags = m.MTLA_FLAG_PORTABLE
    st = d.torch_dtype
    dev = {k: tdev(inp[k], torch.float32 if k == "w_hyp" else st)
           for k in ("c", "k_r", "q_c", "q_r", "w_hyp", "w_uk", "w_uv", "d_o")}
    pe = torch.empty(max(N, 1), d_c, dtype=torch.float32, device=DEV)
    m.mtla_sinusoidal_pe(pe)
    out = {"dc": torch.empty(B, N, d_c, dtype=st, device=DEV),
           "dk_r": torch.empty(B, N, d_r, dtype=st, device=DEV),
           "dq_c": torch.empty(B, N, H, d_h, dtype=st, device=DEV),
           "dq_r": torch.empty(B, N, H, d_r, dtype=st, device=DEV),
           "dw_hyp": torch.full((d_c,), float("nan"), dtype=torch.float32, device=DEV),
           "dw_uk": torch.full((H, d_h, d_c), float("nan"), dtype=torch.float32, device=DEV),
           "dw_uv": torch.full((H, d_h, d_c), float("nan"), dtype=torch.float32, device=DEV)}
    ws = torch.empty(max(16, m.mtla_prefill_backward_workspace_bytes(d, N)), dtype=torch.uint8, device=DEV)
    runs = []
    for _ in range(reps):
        m.mtla_prefill_backward(d, dev["q_c"], dev["q_r"], dev["c"], dev["k_r"], dev["w_hyp"], pe, dev["w_uk"],
                                dev["w_uv"], dev["d_o"], out["dq_c"], out["dq_r"], out["dc"], out["dk_r"],
                                out["dw_hyp"], out["dw_uk"], out["dw_uv"], ws)
        torch.cuda.synchronize()
        runs.append({k: host(v) for k, v in out.items()})
    return d, runs


def _oracle_backward(inp, s, scale):
    B = inp["c"].shape[0]
    per = [oracle.parallel_backward(inp["c"][b], inp["k_r"][b], inp["q_c"][b], inp["q_r"][b], inp["w_hyp"],
                                    inp["w_uk"], inp["w_uv"], s, scale, inp["d_o"][b]) for b in range(B)]
    want = {k: np.stack([r[k] for r in per]) for k in ("dc", "dk_r", "dq_c", "dq_r")}
    for k in ("dw_hyp", "dw_uk", "dw_uv"):
        want[k] = sum(r[k] for r in per)
    return want


# (seed, B, N, s, H, d_h, d_c, d_r, dtype, portable): several 64-row tiles
# with a ragged tail, s = 1 (the causal mask), s >= N (the diagonal alone), N
# a multiple of s, no rope part; in bf16 the summarisation head shape (the
# MFMA path: several 128-query and 128-slot tiles, B*H a multiple of 8 or
# not, no completed slot at all) and the same shape through the portable
# kernels
CASES = [
    (1, 2, 37, 3, 2, 16, 32, 8, "fp32", False),
    (2, 1, 130, 2, 4, 8, 16, 8, "fp32", False),
    (3, 2, 20, 1, 2, 8, 16, 8, "fp32", False),
    (4, 1, 5, 8, 2, 8, 16, 8, "fp32", False),
    (5, 2, 33, 4, 2, 12, 24, 0, "fp32", False),
    (6, 2, 200, 3, 8, 64, 256, 32, "bf16", False),
    (7, 1, 131, 2, 8, 64, 256, 32, "bf16", False),
    (10, 1, 1000, 3, 8, 64, 256, 32, "bf16", False),
    (11, 3, 300, 2, 2, 64, 256, 32, "bf16", False),
    (12, 1, 7, 9, 8, 64, 256, 32, "bf16", False),
    (13, 2, 257, 1, 8, 64, 256, 32, "bf16", False),
    (14, 2, 200, 3, 8, 64, 256, 32, "bf16", True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}_n{c[2]}_s{c[3]}_{c[8]}{'_portable' if c[9] else ''}"
                                             for c in CASES])
def test_backward_matches_oracle(case):
    seed, B, N, s, H, d_h, d_c, d_r, dtype, portable = case
    print(f"backward case seed={seed} B={B} N={N} s={s} H={H} d_h={d_h} d_c={d_c} d_r={d_r} {dtype} "
          f"portable={portable}", flush=True)
    inp = _inputs(seed, B, N, H, d_h, d_c, d_r, dtype)
    d, (got,) = _gpu_backward(inp, s, dtype, portable=portable)
    want = _oracle_backward(inp, s, d.softmax_scale)
    errs = {}
    for k in NAMES:
        if want[k].size == 0:
            continue
        errs[k] = oracle.max_rel_err(got[k], want[k])
    print("max rel err", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k, err in errs.items():
        assert err <= tol(dtype), (k, err)


def test_backward_is_deterministic():
    inp = _inputs(8, 2, 150, 8, 64, 256, 32, "bf16")
    _, (a, b) = _gpu_backward(inp, 3, "bf16", reps=2)
    for k in NAMES:
        assert np.array_equal(a[k], b[k]), k


def test_backward_empty_sequence_zeroes_weight_gradients():
    inp = _inputs(9, 2, 0, 2, 8, 16, 8, "fp32")
    _, (got,) = _gpu_backward(inp, 2, "fp32")
    for k in ("dw_hyp", "dw_uk", "dw_uv"):
        assert not np.any(got[k]), k


def _workload_inputs(w, seqs=None):
    lat, qry = workloads.batch_latents(w, seqs=seqs), workloads.batch_queries(w, seqs=seqs)
    wts = workloads.weights(w)
    return {"c": lat["c"], "k_r": lat["k_r"], "q_c": qry["q_c"], "q_r": qry["q_r"], "w_hyp": wts["w_hyp"],
            "w_uk": wts["w_uk"], "w_uv": wts["w_uv"], "d_o": workloads.batch_grad_out(w, seqs=seqs)}


def test_backward_full_size_sampled():
    """The summarisation shape (B=16, N=4096, s=3) in the launch configuration
    the benchmark times: sequences 0 and 15 against the oracle's full-length
    backward.  The weight gradients, summed over the batch, are checked on a
    batch of those two sequences at full length."""
    w = workloads.WORKLOADS[3]
    assert (w.batch, w.n_tokens, w.s) == (16, 4096, 3)
    print("full-size backward: GPU at B=16", flush=True)
    d, (got,) = _gpu_backward(_workload_inputs(w), w.s, w.dtype)
    sub = _workload_inputs(w, seqs=[0, 15])
    print("full-size backward: oracle for sequences 0 and 15", flush=True)
    want = _oracle_backward(sub, w.s, d.softmax_scale)
    for k in ("dc", "dk_r", "dq_c", "dq_r"):
        err = oracle.max_rel_err(got[k][[0, 15]], want[k])
        print(k, f"{err:.2e}", flush=True)
        assert err <= tol(w.dtype), (k, err)
    _, (got2,) = _gpu_backward(sub, w.s, w.dtype)
    for k in ("dw_hyp", "dw_uk", "dw_uv"):
        err = oracle.max_rel_err(got2[k], want[k])
        print(k, f"{err:.2e}", flush=True)
        assert err <= tol(w.dtype), (k, err)
