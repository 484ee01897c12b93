"""Helpers for GPU parity tests: move seeded inputs to the device and drive
the C-ABI entry points (through the ctypes binding) the way a caller would."""
from __future__ import annotations

import numpy as np
import torch

import temporally_compressed_latent_amd as m

DEV = torch.device("cuda")


def tdev(x: np.ndarray, dtype) -> torch.Tensor:
    """Host fp32 (already storage-representable) -> device tensor of `dtype`."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV).to(dtype)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def tol(dtype: str) -> float:
    """Max relative error bound (||y - y_ref||_inf / ||y_ref||_inf)."""
    return 1e-4 if dtype == "fp32" else 1e-2


class Case:
    """Device-side state for one (dims, inputs) case."""

    def __init__(self, dims: m.MtlaDims, inp: dict, pe_rows: int):
        self.d = dims
        st = dims.torch_dtype
        self.st = st
        B, W = dims.batch, dims.width
        self.c = tdev(inp["c"], st)                     # [B, N, d_c]
        self.k_r = tdev(inp["k_r"], st)                 # [B, N, d_r]
        self.q_c = tdev(inp["q_c"], st)                 # [B, N, H, d_h]
        self.q_r = tdev(inp["q_r"], st)                 # [B, N, H, d_r]
        self.w_hyp = tdev(inp["w_hyp"], torch.float32)
        self.w_uk = tdev(inp["w_uk"], st)
        self.w_uv = tdev(inp["w_uv"], st)
        self.pe = torch.empty(pe_rows, dims.d_c, dtype=torch.float32, device=DEV)
        m.mtla_sinusoidal_pe(self.pe)
        self.cache = torch.zeros(B, dims.max_slots, W, dtype=st, device=DEV)
        # open-slot state: the fp32 value after token t is kept at [b, t % 2]
        self.open_acc = torch.zeros(B, 2, W, dtype=torch.float32, device=DEV)
        self.ws_dec = torch.empty(m.mtla_decode_workspace_bytes(dims), dtype=torch.uint8, device=DEV)

    def open_state(self, t: int) -> torch.Tensor:
        """fp32 state of the open slot after token t, [B, W]."""
        return self.open_acc[:, t % 2]

    def append(self, pos0: torch.Tensor, t_lo: int, t_hi: int, gate_out=None):
        """merge_append tokens t_lo..t_hi-1 (array rows) at device positions pos0."""
        m.mtla_merge_append(self.d, pos0, self.c[:, t_lo:t_hi].contiguous(),
                            self.k_r[:, t_lo:t_hi].contiguous(), self.w_hyp, self.pe,
                            self.cache, self.open_acc, gate_out=gate_out)

    def decode(self, pos: torch.Tensor, t_row: int, out=None) -> torch.Tensor:
        d = self.d
        if out is None:
            out = torch.empty(d.batch, d.heads, d.d_h, dtype=self.st, device=DEV)
        m.mtla_decode(d, pos, self.q_c[:, t_row].contiguous(), self.q_r[:, t_row].contiguous(),
                      self.w_uk, self.w_uv, self.cache, out, self.ws_dec)
        return out

    def decode_loop(self, n_steps: int, start: int = 0) -> torch.Tensor:
        """Token-by-token: for t = start+1..n_steps, merge token t then decode it."""
        d = self.d
        outs = torch.empty(d.batch, n_steps - start, d.heads, d.d_h, dtype=self.st, device=DEV)
        for t in range(start + 1, n_steps + 1):
            pos = torch.full((d.batch,), t, dtype=torch.int32, device=DEV)
            self.append(pos, t - 1, t)
            outs[:, t - 1 - start] = self.decode(pos, t - 1)
        return outs

    def step_loop(self, n_steps: int, start: int = 0, w_uv_tiles=None) -> torch.Tensor:
        """Token-by-token with mtla_decode_step (merge + decode in one call);
        with w_uv_tiles, mtla_decode_step_tiles."""
        d = self.d
        outs = torch.empty(d.batch, n_steps - start, d.heads, d.d_h, dtype=self.st, device=DEV)
        for t in range(start + 1, n_steps + 1):
            pos = torch.full((d.batch,), t, dtype=torch.int32, device=DEV)
            o = torch.empty(d.batch, d.heads, d.d_h, dtype=self.st, device=DEV)
            args = (d, pos, self.c[:, t - 1].contiguous(), self.k_r[:, t - 1].contiguous(), self.w_hyp, self.pe,
                    self.q_c[:, t - 1].contiguous(), self.q_r[:, t - 1].contiguous(), self.w_uk, self.w_uv)
            if w_uv_tiles is None:
                m.mtla_decode_step(*args, self.cache, self.open_acc, o, self.ws_dec)
            else:
                m.mtla_decode_step_tiles(*args, w_uv_tiles, self.cache, self.open_acc, o, self.ws_dec)
            outs[:, t - 1 - start] = o
        return outs

    def prefill(self, n: int) -> torch.Tensor:
        d = self.d
        out = torch.empty(d.batch, n, d.heads, d.d_h, dtype=self.st, device=DEV)
        ws = torch.empty(m.mtla_prefill_workspace_bytes(d, n), dtype=torch.uint8, device=DEV)
        m.mtla_prefill(d, self.q_c[:, :n].contiguous(), self.q_r[:, :n].contiguous(),
                       self.c[:, :n].contiguous(), self.k_r[:, :n].contiguous(), self.w_hyp,
                       self.pe, self.w_uk, self.w_uv, self.cache, self.open_acc, out, ws)
        return out


    def prefill_at(self, t0: int, n: int) -> torch.Tensor:
        """mtla_prefill_at of tokens t0+1 .. t0+n (array rows t0 .. t0+n-1)."""
        d = self.d
        out = torch.empty(d.batch, n, d.heads, d.d_h, dtype=self.st, device=DEV)
        ws = torch.empty(m.mtla_prefill_at_workspace_bytes(d, t0, n), dtype=torch.uint8, device=DEV)
        sl = slice(t0, t0 + n)
        m.mtla_prefill_at(d, t0, self.q_c[:, sl].contiguous(), self.q_r[:, sl].contiguous(),
                          self.c[:, sl].contiguous(), self.k_r[:, sl].contiguous(), self.w_hyp,
                          self.pe, self.w_uk, self.w_uv, self.cache, self.open_acc, out, ws)
        return out


# (H, d_h, d_c, d_r): the two layer shapes of the workloads, a padded-head
# shape for the 32-row MFMA instance, and an odd shape only the portable
# kernels take.
SHAPES = {
    "st": (8, 64, 256, 32),
    "llm": (32, 128, 512, 64),
    "mid": (20, 32, 256, 32),
    "odd": (3, 16, 48, 8),
    "d40": (4, 40, 256, 32),
}


def make_case(shape: str, seed: int, B: int, N: int, s: int, dtype: str, portable: bool = False,
              max_slots=None, gate_per_position: bool = False, **kw):
    import workloads
    H, d_h, d_c, d_r = SHAPES[shape]
    inp = workloads.boundary_case(seed, B, N, H, d_h, d_c, d_r, dtype,
                                  gate_rows=s if gate_per_position else 0, **kw)
    ms = max_slots or (-(-N // s) + 2)
    dims = m.make_dims(B, H, d_h, d_c, d_r, s, ms, dtype, portable=portable,
                       gate_per_position=gate_per_position)
    return inp, Case(dims, inp, N + 4)


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
