"""GPU: beam-search reorder of the decode state (mtla_reorder_state) against
the oracle's gather, bit for bit, and decoding that continues after it against
the oracle's loop over each hypothesis' mixed history."""
import numpy as np
import pytest
import torch

import oracle
from tests import oracle_ref
from tests.gpu_util import DEV, bits, host, make_case
import temporally_compressed_latent_amd as m

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,s,shape", [("bf16", 2, "st"), ("bf16", 3, "llm"), ("fp32", 4, "st"),
                                           ("bf16", 1, "odd"), ("fp32", 3, "odd")])
def test_reorder_matches_oracle_bit_exact(dtype, s, shape):
    from tests.gpu_util import SHAPES
    H, d_h, d_c, d_r = SHAPES[shape]
    B, S = 7, 40
    W = d_c + d_r
    d = m.make_dims(B, H, d_h, d_c, d_r, s, S, dtype)
    g = np.random.default_rng(31)
    st = d.torch_dtype
    cache_in = torch.randn(B, S, W, device=DEV).to(st)
    open_in = torch.randn(B, 2, W, device=DEV)
    pos_h = np.array([0, 1, s * S, 5, s * 7 + 1, 13, s * S - 1], dtype=np.int32)
    src_h = np.array([3, 3, 6, 0, 2, -1, 1], dtype=np.int32)   # a repeated parent, one invalid
    pos, src = torch.from_numpy(pos_h).to(DEV), torch.from_numpy(src_h).to(DEV)
    sentinel = torch.full((B, S, W), 7.0, device=DEV).to(st)
    cache_out, open_out = sentinel.clone(), torch.full((B, 2, W), -3.0, device=DEV)
    pos_out = torch.full((B,), -9, dtype=torch.int32, device=DEV)
    m.mtla_reorder_state(d, src, pos, cache_in, open_in, cache_out, open_out, pos_out)
    torch.cuda.synchronize()
    raw_in, raw_out = bits(cache_in).cpu().numpy(), bits(cache_out).cpu().numpy()
    raw_sent = bits(sentinel).cpu().numpy()
    valid = src_h >= 0
    want, want_open, want_pos = oracle.reorder_state(raw_in, host(open_in), pos_h,
                                                     np.where(valid, src_h, 0), s)
    for b in range(B):
        if not valid[b]:
            assert np.array_equal(raw_out[b], raw_sent[b])
            assert (host(open_out)[b] == -3.0).all() and int(pos_out[b]) == -9
            continue
        p = pos_h[src_h[b]]
        n = oracle.num_slots(int(p), s) if p > 0 else 0
        assert np.array_equal(raw_out[b, :n], want[b, :n]), b
        assert np.array_equal(raw_out[b, n:], raw_sent[b, n:]), b      # rows past the slots untouched
        assert np.array_equal(host(open_out)[b], want_open[b]), b
        assert int(pos_out[b]) == want_pos[b]


def test_decode_continues_after_reorder():
    """Decode T1 tokens, reorder beam-style, decode T1+1..T2: hypothesis b then
    holds tokens 1..T1 of its parent and its own tokens after, and the outputs
    follow the oracle's loop over that mixed history."""
    B, s, T1, T2 = 5, 2, 37, 60
    inp, g = make_case("st", 15, B, T2, s, "bf16")
    g.decode_loop(T1)
    src_h = np.array([2, 2, 0, 4, 1], dtype=np.int32)
    src = torch.from_numpy(src_h).to(DEV)
    pos = torch.full((B,), T1, dtype=torch.int32, device=DEV)
    cache2, open2 = torch.empty_like(g.cache), torch.empty_like(g.open_acc)
    m.mtla_reorder_state(g.d, src, pos, g.cache, g.open_acc, cache2, open2)
    g.cache.copy_(cache2)
    g.open_acc.copy_(open2)
    out = host(g.decode_loop(T2, start=T1))
    mixed = {k: np.array(v, copy=True) for k, v in inp.items()}
    for key in ("c", "k_r", "q_c", "q_r"):
        for b in range(B):
            mixed[key][b, :T1] = inp[key][src_h[b], :T1]
    want, _ = oracle_ref.loop_outputs(mixed, B, T2, s, g.d.softmax_scale)
    oracle_ref.assert_steps(out, want[:, T1:], 1e-2)
