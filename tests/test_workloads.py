"""CPU: the seeded input generators (shared by oracle tests, GPU tests and
the benchmark) are deterministic, per-sequence, and round like the device."""
import numpy as np
import torch

import workloads


def test_bf16_rounding_matches_torch_rne():
    g = np.random.default_rng(0)
    x = np.concatenate([
        g.standard_normal(100_000).astype(np.float32) * 10,
        # exact ties between two bf16 values, both parities
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, -3.3895314e38], np.float32),
    ])
    mine = workloads.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    assert workloads.f32_to_bf16_bits(np.array([np.nan], np.float32))[0] == 0x7FC0


def test_streams_are_per_sequence_and_reproducible():
    w = workloads.workload(1)
    a = workloads.latents(w, 3, 16)["c"]
    b = workloads.batch_latents(w, 16, seqs=[2, 3])["c"][1]
    assert np.array_equal(a, b)
    assert not np.array_equal(a, workloads.latents(w, 4, 16)["c"])
    assert np.array_equal(a, workloads.quantize(a, "bf16"))   # already bf16-representable


def test_workload_shapes():
    w = workloads.workload(4)
    assert (w.batch, w.n_tokens, w.heads, w.d_h, w.d_c, w.d_r, w.s) == (64, 32768, 32, 128, 512, 64, 2)
    assert w.width * 2 == 1152
    assert workloads.workload(3).s == 3 and workloads.workload(2).n_tokens == 2048
