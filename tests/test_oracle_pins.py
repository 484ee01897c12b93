"""CPU: the fp64 oracle against what the pages and the mathematics fix."""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.mtla)


@settings(max_examples=40, deadline=None)
@given(N=st.integers(1, 24), s=st.integers(1, 6), H=st.integers(1, 2),
       d_h=st.integers(1, 5), d_c=st.integers(1, 7), d_r=st.sampled_from([0, 2, 4]),
       seed=st.integers(0, 10_000))
def test_parallel_equals_incremental_hypothesis(N, s, H, d_h, d_c, d_r, seed):
    pins.pin_parallel_equals_incremental(oracle.mtla, [(seed, N, s, H, d_h, d_c, d_r)])


@settings(max_examples=30, deadline=None)
@given(N=st.integers(1, 40), s=st.integers(1, 9))
def test_mask_row_is_completed_slots_plus_diagonal(N, s):
    M = oracle.stride_mask(N, s)
    for i in range(1, N + 1):
        cols = set(np.nonzero(M[i - 1])[0] + 1)
        completed = {j for j in range(1, i) if j % s == 0}
        assert cols == completed | {i}
        assert len(completed) == oracle.completed_slots(i, s)
