"""GPU: the measurement hooks run through the C ABI.  The stream read folds
what it reads into its sink (all-ones words fold to zero); the tile stream
writes its sink only on a pattern no input here holds, so its sink stays
untouched."""
import pytest
import torch

import temporally_compressed_latent_amd as m
from tests.gpu_util import DEV

pytestmark = pytest.mark.gpu


def test_stream_read_and_tile_stream_sinks():
    x = torch.ones(1 << 20, dtype=torch.int32, device=DEV)
    sink = torch.full((64 * 4,), -7, dtype=torch.int32, device=DEV)
    m.mtla_calib_stream_read(x, 64, sink)
    rows = torch.full((3, 200, 1152), 0x11, dtype=torch.uint8, device=DEV)  # ragged last tile
    sink2 = torch.full((3 * 4 * 8,), -7, dtype=torch.int32, device=DEV)
    for il in (False, True):
        for nt in (False, True):
            m.mtla_calib_tile_stream(rows, 4, il, nt, sink2)
    torch.cuda.synchronize()
    assert torch.all(sink == 0) and torch.all(sink2 == -7)


def test_mfma_chains_flop_count():
    out = torch.empty(8 * 256, dtype=torch.float32, device=DEV)
    flops = m.mtla_calib_mfma(False, 8, 16, out)
    torch.cuda.synchronize()
    assert flops == 4 * 8 * 4 * 16 * 2 * 32 * 32 * 16
    assert torch.isfinite(out).all()


def test_load_pattern_cycles():
    """Both load patterns run and report a positive cycle count per
    workgroup; the guard words past the counts stay untouched."""
    buf = torch.ones(1 << 16, dtype=torch.int32, device=DEV)  # 256 KiB
    for pat in (0, 1):
        cyc = torch.full((16 + 64,), -7, dtype=torch.int32, device=DEV)
        m.mtla_calib_load_pattern(pat, 16, buf, cyc)
        torch.cuda.synchronize()
        assert torch.all(cyc[:16] > 0) and torch.all(cyc[16:] == -7)


def test_step_timeline_same_bits_and_ordered_readings():
    """The fused step's timeline instance computes what mtla_decode_step_tiles
    computes (same bits in every step's output and in the final cache and
    open-slot state), and each workgroup's readings follow its phase chain
    (within a few ticks of the 100 MHz counter: waves sample it
    independently).  Shapes it does not cover are refused."""
    g = torch.Generator().manual_seed(11)
    B, H, d_h, d_c, d_r, s, N = 11, 8, 64, 256, 32, 2, 40
    d = m.make_dims(B, H, d_h, d_c, d_r, s, -(-N // s), "bf16")
    bf = torch.bfloat16

    def rnd(*shape, scale=1.0, dtype=bf):
        return (torch.randn(*shape, generator=g) * scale).to(dtype).to(DEV)
    c, k_r = rnd(N, B, d_c), rnd(N, B, d_r)
    q_c, q_r = rnd(N, B, H, d_h), rnd(N, B, H, d_r)
    w_hyp = rnd(d_c, scale=d_c ** -0.5, dtype=torch.float32)
    w_uk, w_uv = rnd(H, d_h, d_c, scale=d_h ** -0.5), rnd(H, d_h, d_c, scale=d_c ** -0.5)
    pe = torch.empty(N, d_c, dtype=torch.float32, device=DEV)
    m.mtla_sinusoidal_pe(pe)
    tiles = torch.empty(m.mtla_w_uv_tiles_bytes(d) // 2, dtype=bf, device=DEV)
    m.mtla_pack_w_uv_tiles(d, w_uv, tiles)
    pos = torch.arange(1, N + 1, dtype=torch.int32, device=DEV)[:, None].expand(N, B).contiguous()
    ws = torch.zeros(m.mtla_decode_workspace_bytes(d), dtype=torch.uint8, device=DEV)
    state = [(torch.zeros(B, d.max_slots, d.width, dtype=bf, device=DEV),
              torch.zeros(B, 2, d.width, dtype=torch.float32, device=DEV)) for _ in range(2)]
    out = [torch.empty(N, B, H, d_h, dtype=bf, device=DEV) for _ in range(2)]
    tl = torch.zeros(N, 8 * H * 2 * 16, dtype=torch.int64, device=DEV)
    for t in range(N):
        m.mtla_decode_step_tiles(d, pos[t], c[t], k_r[t], w_hyp, pe, q_c[t], q_r[t], w_uk, w_uv, tiles,
                                 state[0][0], state[0][1], out[0][t], ws)
        m.mtla_calib_step_timeline(d, pos[t], c[t], k_r[t], w_hyp, pe, q_c[t], q_r[t], w_uk, w_uv, tiles,
                                   state[1][0], state[1][1], out[1][t], ws, tl[t])
    torch.cuda.synchronize()
    assert torch.equal(out[0].view(torch.int16), out[1].view(torch.int16))
    assert torch.equal(state[0][0].view(torch.int16), state[1][0].view(torch.int16))
    assert torch.equal(state[0][1], state[1][1])
    x = tl.cpu().reshape(N, -1, 16)
    live = x[:, :, 0] != 0
    assert all(int(live[t].sum()) in (4 * B, 8 * B) for t in range(N))
    r = x[live]
    slack = 5
    assert torch.all(r[:, 1] >= r[:, 0] - slack) and torch.all(r[:, 2] >= r[:, 1] - slack)
    assert torch.all(r[:, 3] >= r[:, 2] - slack)
    assert torch.all(r[:, 4:12] >= r[:, 2:3] - slack)
    assert torch.all(r[:, 12] >= r[:, 4:12].max(dim=1).values - slack)
    assert torch.all(r[:, 13] >= r[:, 12] - slack)
    assert torch.all(r[:, 14:] == 0)
    # not the one-kernel 256-wide step: refused by the library before any launch
    B2, d_h2, d_c2, d_r2 = 4, 128, 512, 64
    d2 = m.make_dims(B2, H, d_h2, d_c2, d_r2, 2, 8, "bf16")
    z = lambda *shape, dtype=bf: torch.zeros(*shape, dtype=dtype, device=DEV)
    with pytest.raises(Exception, match="timeline covers"):
        m.mtla_calib_step_timeline(d2, pos[0, :B2].contiguous(), z(B2, d_c2), z(B2, d_r2),
                                   z(d_c2, dtype=torch.float32), z(8, d_c2, dtype=torch.float32),
                                   z(B2, H, d_h2), z(B2, H, d_r2), z(H, d_h2, d_c2), z(H, d_h2, d_c2),
                                   z(m.mtla_w_uv_tiles_bytes(d2) // 2), z(B2, 8, d_c2 + d_r2),
                                   z(B2, 2, d_c2 + d_r2, dtype=torch.float32), z(B2, H, d_h2),
                                   z(m.mtla_decode_workspace_bytes(d2), dtype=torch.uint8), tl[0])
