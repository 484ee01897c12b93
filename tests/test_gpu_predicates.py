"""GPU: integer predicates (stride mask, slot limits) bit-exact against the
oracle, and the positional-embedding table."""
import numpy as np
import pytest
import torch

import oracle
import temporally_compressed_latent_amd as m

pytestmark = pytest.mark.gpu

CASES = [(n, s) for n in (1, 2, 3, 7, 16, 33, 64, 100, 257) for s in range(1, 9)] + \
        [(512, 2), (2048, 4), (4096, 3), (300, 300), (5, 9)]


@pytest.mark.parametrize("n,s", CASES)
def test_stride_mask_bit_exact(n, s):
    mask = torch.full((n, n), 7, dtype=torch.uint8, device="cuda")
    m.mtla_debug_stride_mask(n, s, mask)
    got = mask.cpu().numpy()
    want = oracle.stride_mask(n, s).astype(np.uint8)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("n,s", CASES)
def test_slot_limits_bit_exact(n, s):
    hi = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    m.mtla_debug_slot_limits(n, s, hi)
    want = np.array([oracle.completed_slots(i, s) for i in range(1, n + 1)], dtype=np.int32)
    assert np.array_equal(hi.cpu().numpy(), want)


@pytest.mark.parametrize("rows,d", [(1, 2), (64, 256), (4097, 256), (32769, 512), (10, 7)])
def test_sinusoidal_pe(rows, d):
    pe = torch.empty(rows, d, dtype=torch.float32, device="cuda")
    m.mtla_sinusoidal_pe(pe)
    got = pe.cpu().numpy().astype(np.float64)
    want = oracle.sinusoidal_pe(rows, d)
    # the table is the fp64 value rounded to fp32: within one fp32 ulp of |x| <= 1
    assert np.max(np.abs(got - want)) <= 2.0 ** -24 * 1.01
