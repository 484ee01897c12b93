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
