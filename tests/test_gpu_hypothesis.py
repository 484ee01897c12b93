"""GPU: parity over hypothesis-drawn tiny shapes.  Each example draws a layer
shape (the workloads' two, a 20-head one and an odd one only the portable
kernels take), a storage dtype, s, B and N, runs the parallel prefill and the
token-by-token decode loop on the device, and checks both against the
oracle's incremental loop, each step's [B, H, d_h] on its own.  The examples
are derandomized: every run draws the same ones."""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings, strategies as st

from tests import oracle_ref
from tests.gpu_util import host, make_case, tol

pytestmark = pytest.mark.gpu


@settings(max_examples=24, deadline=None, derandomize=True, suppress_health_check=list(HealthCheck))
@given(shape=st.sampled_from(["st", "llm", "mid", "odd"]), dtype=st.sampled_from(["bf16", "fp32"]),
       s=st.integers(1, 6), B=st.integers(1, 3), N=st.integers(1, 40), portable=st.booleans(),
       seed=st.integers(0, 1000))
def test_prefill_and_decode_loop_drawn_shapes(shape, dtype, s, B, N, portable, seed):
    print(f"drawn case: {shape} {dtype} s={s} B={B} N={N} portable={portable} seed={seed}", flush=True)
    inp, a = make_case(shape, seed, B, N, s, dtype, portable)
    _, b = make_case(shape, seed, B, N, s, dtype, portable)
    pre = host(a.prefill(N))
    loop = host(b.decode_loop(N))
    want, _ = oracle_ref.loop_outputs(inp, B, N, s, a.d.softmax_scale)
    oracle_ref.assert_steps(pre, want, tol(dtype), "prefill")
    oracle_ref.assert_steps(loop, want, tol(dtype), "decode loop")
