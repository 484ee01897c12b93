"""ctypes binding of libmtla.so: argument marshalling only.

Every function here has the name of the C entry point it calls and does no
arithmetic of the method: it checks that the torch tensors it is given match
the shapes, dtypes and devices the C ABI expects (the C library cannot see
tensor sizes), then passes raw device pointers and the current HIP stream.

If the library is missing this module raises at import time: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
import re
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MTLA_LIB", os.path.join(_PKG, "libmtla.so"))
HEADER = os.path.join(os.path.dirname(_PKG), "include", "mtla.h")

MTLA_OK = 0
MTLA_ERR_INVALID_ARG = -1
MTLA_ERR_UNSUPPORTED = -2
MTLA_ERR_WORKSPACE = -3
MTLA_ERR_HIP = -4
MTLA_FP32 = 0
MTLA_BF16 = 1
MTLA_FLAG_PORTABLE = 1
MTLA_FLAG_GATE_PER_POSITION = 2


class MtlaDims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("d_h", ctypes.c_int32),
        ("d_c", ctypes.c_int32),
        ("d_r", ctypes.c_int32),
        ("stride_s", ctypes.c_int32),
        ("max_slots", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("flags", ctypes.c_int32),
        ("decode_splits", ctypes.c_int32),
        ("step_groups", ctypes.c_int32),
    ]

    @property
    def width(self) -> int:
        return self.d_c + self.d_r

    @property
    def gate_shape(self) -> tuple:
        """Shape of W_hyp (and of its gradient): [d_c], or [s, d_c] per position."""
        if self.flags & MTLA_FLAG_GATE_PER_POSITION:
            return (self.stride_s, self.d_c)
        return (self.d_c,)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == MTLA_FP32 else torch.bfloat16

    def copy(self, **kw) -> "MtlaDims":
        d = MtlaDims()
        for name, _ in self._fields_:
            setattr(d, name, kw.get(name, getattr(self, name)))
        return d


class MtlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python temporally_compressed_latent_amd/build.py` "
            "(the MTLA path has no CPU fallback)")
    return ctypes.CDLL(LIB_PATH)


_lib = _load()

_P = ctypes.c_void_p
_I = ctypes.c_int32
_SZ = ctypes.c_size_t
_D = ctypes.POINTER(MtlaDims)

_SIGS = {
    "mtla_version": (_I, []),
    "mtla_status_string": (ctypes.c_char_p, [_I]),
    "mtla_last_error": (ctypes.c_char_p, []),
    "mtla_sinusoidal_pe": (_I, [_I, _I, _P, _P]),
    "mtla_merge_append": (_I, [_D, _P, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P]),
    "mtla_decode_workspace_bytes": (_I, [_D, ctypes.POINTER(_SZ)]),
    "mtla_decode": (_I, [_D, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "mtla_decode_plan": (_I, [_D, ctypes.POINTER(_I), ctypes.POINTER(_I)]),
    "mtla_decode_step": (_I, [_D, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "mtla_decode_step_noalloc": (_I, [_D, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P]),
    "mtla_w_uv_tiles_bytes": (_I, [_D, ctypes.POINTER(_SZ)]),
    "mtla_pack_w_uv_tiles": (_I, [_D, _P, _P, _P]),
    "mtla_decode_step_tiles": (_I, [_D, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "mtla_prefill_partials": (_I, [_D, _I, _P, _P, _P, _P, _I, _P, _P, _P, _P]),
    "mtla_prefill_keys": (_I, [_D, _I, _P, _P, _P, _P, _P, _P]),
    "mtla_prefill_attention": (_I, [_D, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "mtla_calib_stream_read": (_I, [_P, _SZ, _I, _P, _P]),
    "mtla_calib_mfma": (_I, [_I, _I, _I, _P, ctypes.POINTER(ctypes.c_double), _P]),
    "mtla_calib_empty": (_I, [_P]),
    "mtla_calib_load_pattern": (_I, [_I, _I, _P, _SZ, _P, _P]),
    "mtla_calib_tile_stream": (_I, [_P, _I, _I, _I, _I, _P, _P]),
    "mtla_calib_step_timeline": (_I, [_D, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ,
                                      _P, _SZ, _P]),
    "mtla_absorb_query": (_I, [_D, _I, _P, _P, _P, _P, _P]),
    "mtla_decode_attention_workspace_bytes": (_I, [_D, ctypes.POINTER(_SZ)]),
    "mtla_decode_attention": (_I, [_D, _P, _P, _P, _P, _P, _SZ, _P]),
    "mtla_up_project": (_I, [_D, _I, _P, _P, _P, _P]),
    "mtla_prefill_workspace_bytes": (_I, [_D, _I, ctypes.POINTER(_SZ)]),
    "mtla_prefill": (_I, [_D, _I, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "mtla_prefill_at_workspace_bytes": (_I, [_D, _I, _I, ctypes.POINTER(_SZ)]),
    "mtla_reorder_state": (_I, [_D, _P, _P, _P, _P, _P, _P, _P, _P]),
    "mtla_project_inputs": (_I, [_D, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "mtla_output_project": (_I, [_D, _I, _I, _P, _P, _P, _P]),
    "mtla_layer_decode_workspace_bytes": (_I, [_D, _I, ctypes.POINTER(_SZ)]),
    "mtla_layer_decode_step": (_I, [_D, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _SZ,
                                    _P]),
    "mtla_layer_decode_step_tiles": (_I, [_D, _I] + [_P] * 8 + [_I] + [_P] * 7 + [_SZ, _P]),
    "mtla_layer_prefill_workspace_bytes": (_I, [_D, _I, _I, _I, ctypes.POINTER(_SZ)]),
    "mtla_layer_prefill": (_I, [_D, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _SZ,
                                _P]),
    "mtla_prefill_at": (_I, [_D, _I, _I, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "mtla_prefill_backward_workspace_bytes": (_I, [_D, _I, ctypes.POINTER(_SZ)]),
    "mtla_prefill_backward": (_I, [_D, _I, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                   _P, _SZ, _P]),
    "mtla_debug_stride_mask": (_I, [_I, _I, _P, _P]),
    "mtla_debug_slot_limits": (_I, [_I, _I, _P, _P]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def lib() -> ctypes.CDLL:
    return _lib


def header_symbols() -> list:
    """Entry points declared in include/mtla.h."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(mtla_[a-z_]+)\s*\(", text)))


def status_string(status: int) -> str:
    return _lib.mtla_status_string(status).decode()


def last_error() -> str:
    return _lib.mtla_last_error().decode()


def _check(status: int) -> None:
    if status != MTLA_OK:
        raise MtlaError(status, last_error())


def mtla_version() -> int:
    return _lib.mtla_version()


def make_dims(batch: int, heads: int, d_h: int, d_c: int, d_r: int, s: int, max_slots: int,
              dtype="bf16", softmax_scale: Optional[float] = None, portable: bool = False,
              gate_per_position: bool = False, decode_splits: int = 0, step_groups: int = 0) -> MtlaDims:
    d = MtlaDims()
    d.batch, d.heads, d.d_h, d.d_c, d.d_r = batch, heads, d_h, d_c, d_r
    d.stride_s, d.max_slots = s, max_slots
    d.dtype = {"fp32": MTLA_FP32, "bf16": MTLA_BF16, torch.float32: MTLA_FP32,
               torch.bfloat16: MTLA_BF16}[dtype]
    d.softmax_scale = 1.0 / math.sqrt(d_h + d_r) if softmax_scale is None else softmax_scale
    d.flags = (MTLA_FLAG_PORTABLE if portable else 0) | (MTLA_FLAG_GATE_PER_POSITION if gate_per_position else 0)
    d.decode_splits, d.step_groups = decode_splits, step_groups
    return d


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _tensor(name: str, t, shape, dtype, optional: bool = False) -> Optional[int]:
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr() if t.numel() else None


def _ws(name: str, t, need: int) -> tuple:
    if t is None:
        return None, 0
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    return t.data_ptr(), t.numel() * t.element_size()


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def mtla_sinusoidal_pe(pe: torch.Tensor, stream=None) -> None:
    rows, d = pe.shape
    p = _tensor("pe", pe, (rows, d), torch.float32)
    _check(_lib.mtla_sinusoidal_pe(rows, d, p, _stream(stream)))


def mtla_merge_append(dims: MtlaDims, pos0, c, k_r, w_hyp, pe, cache, open_acc,
                      gate_out=None, stream=None) -> None:
    B, W, T = dims.batch, dims.width, int(c.shape[1]) if c.dim() == 3 else -1
    st = dims.torch_dtype
    args = (
        _tensor("pos0", pos0, (B,), torch.int32),
        _tensor("c", c, (B, T, dims.d_c), st),
        _tensor("k_r", k_r, (B, T, dims.d_r), st, optional=dims.d_r == 0),
        _tensor("w_hyp", w_hyp, dims.gate_shape, torch.float32),
        _tensor("pe", pe, (pe.shape[0], dims.d_c), torch.float32),
        _tensor("cache", cache, (B, dims.max_slots, W), st),
        _tensor("open_acc", open_acc, (B, 2, W), torch.float32),
        _tensor("gate_out", gate_out, (B, T), torch.float32, optional=True),
    )
    _check(_lib.mtla_merge_append(ctypes.byref(dims), args[0], T, args[1], args[2], args[3],
                                  args[4], int(pe.shape[0]), args[5], args[6], args[7],
                                  _stream(stream)))


def mtla_decode_workspace_bytes(dims: MtlaDims) -> int:
    n = _SZ(0)
    _check(_lib.mtla_decode_workspace_bytes(ctypes.byref(dims), ctypes.byref(n)))
    return n.value


def mtla_decode(dims: MtlaDims, pos, q_c, q_r, w_uk, w_uv, cache, out, workspace,
                stream=None) -> None:
    B, H, st = dims.batch, dims.heads, dims.torch_dtype
    ws, ws_bytes = _ws("workspace", workspace, 0)
    _check(_lib.mtla_decode(
        ctypes.byref(dims),
        _tensor("pos", pos, (B,), torch.int32),
        _tensor("q_c", q_c, (B, H, dims.d_h), st),
        _tensor("q_r", q_r, (B, H, dims.d_r), st, optional=dims.d_r == 0),
        _tensor("w_uk", w_uk, (H, dims.d_h, dims.d_c), st),
        _tensor("w_uv", w_uv, (H, dims.d_h, dims.d_c), st),
        _tensor("cache", cache, (B, dims.max_slots, dims.width), st),
        _tensor("out", out, (B, H, dims.d_h), st),
        ws, ws_bytes, _stream(stream)))


def mtla_decode_plan(dims: MtlaDims) -> tuple:
    """(splits, fused) of the decode path these dims take."""
    sp, fu = _I(0), _I(0)
    _check(_lib.mtla_decode_plan(ctypes.byref(dims), ctypes.byref(sp), ctypes.byref(fu)))
    return sp.value, bool(fu.value)


def mtla_decode_step(dims: MtlaDims, pos, c, k_r, w_hyp, pe, q_c, q_r, w_uk, w_uv, cache, open_acc,
                     out, workspace, stream=None) -> None:
    B, H, st = dims.batch, dims.heads, dims.torch_dtype
    ws, ws_bytes = _ws("workspace", workspace, 0)
    _check(_lib.mtla_decode_step(
        ctypes.byref(dims),
        _tensor("pos", pos, (B,), torch.int32),
        _tensor("c", c, (B, dims.d_c), st),
        _tensor("k_r", k_r, (B, dims.d_r), st, optional=dims.d_r == 0),
        _tensor("w_hyp", w_hyp, dims.gate_shape, torch.float32),
        _tensor("pe", pe, (pe.shape[0], dims.d_c), torch.float32), int(pe.shape[0]),
        _tensor("q_c", q_c, (B, H, dims.d_h), st),
        _tensor("q_r", q_r, (B, H, dims.d_r), st, optional=dims.d_r == 0),
        _tensor("w_uk", w_uk, (H, dims.d_h, dims.d_c), st),
        _tensor("w_uv", w_uv, (H, dims.d_h, dims.d_c), st),
        _tensor("cache", cache, (B, dims.max_slots, dims.width), st),
        _tensor("open_acc", open_acc, (B, 2, dims.width), torch.float32),
        _tensor("out", out, (B, H, dims.d_h), st),
        ws, ws_bytes, _stream(stream)))


def mtla_w_uv_tiles_bytes(dims: MtlaDims) -> int:
    n = _SZ(0)
    _check(_lib.mtla_w_uv_tiles_bytes(ctypes.byref(dims), ctypes.byref(n)))
    return n.value


def mtla_pack_w_uv_tiles(dims: MtlaDims, w_uv, w_uv_tiles, stream=None) -> None:
    """W_UV [H, d_h, d_c] into the fused decode step's tile order (a flat
    bf16 tensor of mtla_w_uv_tiles_bytes(dims) / 2 elements)."""
    n = mtla_w_uv_tiles_bytes(dims) // 2
    _check(_lib.mtla_pack_w_uv_tiles(
        ctypes.byref(dims),
        _tensor("w_uv", w_uv, (dims.heads, dims.d_h, dims.d_c), dims.torch_dtype),
        _tensor("w_uv_tiles", w_uv_tiles, (n,), dims.torch_dtype), _stream(stream)))


def mtla_decode_step_tiles(dims: MtlaDims, pos, c, k_r, w_hyp, pe, q_c, q_r, w_uk, w_uv, w_uv_tiles, cache,
                           open_acc, out, workspace, stream=None) -> None:
    B, H, st = dims.batch, dims.heads, dims.torch_dtype
    ws, ws_bytes = _ws("workspace", workspace, 0)
    n = mtla_w_uv_tiles_bytes(dims) // 2
    _check(_lib.mtla_decode_step_tiles(
        ctypes.byref(dims),
        _tensor("pos", pos, (B,), torch.int32),
        _tensor("c", c, (B, dims.d_c), st),
        _tensor("k_r", k_r, (B, dims.d_r), st, optional=dims.d_r == 0),
        _tensor("w_hyp", w_hyp, dims.gate_shape, torch.float32),
        _tensor("pe", pe, (pe.shape[0], dims.d_c), torch.float32), int(pe.shape[0]),
        _tensor("q_c", q_c, (B, H, dims.d_h), st),
        _tensor("q_r", q_r, (B, H, dims.d_r), st, optional=dims.d_r == 0),
        _tensor("w_uk", w_uk, (H, dims.d_h, dims.d_c), st),
        _tensor("w_uv", w_uv, (H, dims.d_h, dims.d_c), st),
        _tensor("w_uv_tiles", w_uv_tiles, (n,), st),
        _tensor("cache", cache, (B, dims.max_slots, dims.width), st),
        _tensor("open_acc", open_acc, (B, 2, dims.width), torch.float32),
        _tensor("out", out, (B, H, dims.d_h), st),
        ws, ws_bytes, _stream(stream)))


def mtla_calib_step_timeline(dims: MtlaDims, pos, c, k_r, w_hyp, pe, q_c, q_r, w_uk, w_uv, w_uv_tiles, cache,
                             open_acc, out, workspace, timeline, stream=None) -> None:
    """mtla_decode_step_tiles through the fused step's timeline instance;
    timeline: int64 device tensor of 16 readings per workgroup."""
    B, H, st = dims.batch, dims.heads, dims.torch_dtype
    ws, ws_bytes = _ws("workspace", workspace, 0)
    n = mtla_w_uv_tiles_bytes(dims) // 2
    if timeline.dtype != torch.int64 or timeline.device.type != "cuda" or not timeline.is_contiguous():
        raise ValueError("timeline must be a contiguous int64 device tensor")
    _check(_lib.mtla_calib_step_timeline(
        ctypes.byref(dims),
        _tensor("pos", pos, (B,), torch.int32),
        _tensor("c", c, (B, dims.d_c), st),
        _tensor("k_r", k_r, (B, dims.d_r), st, optional=dims.d_r == 0),
        _tensor("w_hyp", w_hyp, dims.gate_shape, torch.float32),
        _tensor("pe", pe, (pe.shape[0], dims.d_c), torch.float32), int(pe.shape[0]),
        _tensor("q_c", q_c, (B, H, dims.d_h), st),
        _tensor("q_r", q_r, (B, H, dims.d_r), st, optional=dims.d_r == 0),
        _tensor("w_uk", w_uk, (H, dims.d_h, dims.d_c), st),
        _tensor("w_uv", w_uv, (H, dims.d_h, dims.d_c), st),
        _tensor("w_uv_tiles", w_uv_tiles, (n,), st),
        _tensor("cache", cache, (B, dims.max_slots, dims.width), st),
        _tensor("open_acc", open_acc, (B, 2, dims.width), torch.float32),
        _tensor("out", out, (B, H, dims.d_h), st),
        ws, ws_bytes, timeline.data_ptr(), timeline.numel(), _stream(stream)))


def mtla_decode_step_noalloc(dims: MtlaDims, pos, c, k_r, w_hyp, pe, q_c, q_r, w_uk, w_uv, cache, open_acc,
                             out, stream=None) -> None:
    """mtla_decode_step with the library's static scratch as its workspace."""
    B, H, st = dims.batch, dims.heads, dims.torch_dtype
    _check(_lib.mtla_decode_step_noalloc(
        ctypes.byref(dims),
        _tensor("pos", pos, (B,), torch.int32),
        _tensor("c", c, (B, dims.d_c), st),
        _tensor("k_r", k_r, (B, dims.d_r), st, optional=dims.d_r == 0),
        _tensor("w_hyp", w_hyp, dims.gate_shape, torch.float32),
        _tensor("pe", pe, (pe.shape[0], dims.d_c), torch.float32), int(pe.shape[0]),
        _tensor("q_c", q_c, (B, H, dims.d_h), st),
        _tensor("q_r", q_r, (B, H, dims.d_r), st, optional=dims.d_r == 0),
        _tensor("w_uk", w_uk, (H, dims.d_h, dims.d_c), st),
        _tensor("w_uv", w_uv, (H, dims.d_h, dims.d_c), st),
        _tensor("cache", cache, (B, dims.max_slots, dims.width), st),
        _tensor("open_acc", open_acc, (B, 2, dims.width), torch.float32),
        _tensor("out", out, (B, H, dims.d_h), st),
        _stream(stream)))


def mtla_prefill_partials(dims: MtlaDims, c, k_r, w_hyp, pe, cache, open_acc, partials, stream=None) -> None:
    """Staged prefill, stage 1: partial merges P [B, N, W] (and the cache/open slot)."""
    B, st = dims.batch, dims.torch_dtype
    N = int(c.shape[1])
    _check(_lib.mtla_prefill_partials(
        ctypes.byref(dims), N,
        _tensor("c", c, (B, N, dims.d_c), st),
        _tensor("k_r", k_r, (B, N, dims.d_r), st, optional=dims.d_r == 0),
        _tensor("w_hyp", w_hyp, dims.gate_shape, torch.float32),
        _tensor("pe", pe, (pe.shape[0], dims.d_c), torch.float32), int(pe.shape[0]),
        _tensor("cache", cache, (B, dims.max_slots, dims.width), st),
        _tensor("open_acc", open_acc, (B, 2, dims.width), torch.float32),
        _tensor("partials", partials, (B, N, dims.width), st),
        _stream(stream)))


def prefill_slot_keys(dims: MtlaDims, n_tokens: int, t0: int = 0) -> int:
    """Completed slots the queries t0+1..t0+n_tokens attend: floor((t0+n_tokens-1)/s)."""
    return (t0 + n_tokens - 1) // dims.stride_s if n_tokens > 0 else 0


def mtla_prefill_keys(dims: MtlaDims, partials, w_uk, w_uv, k_c, v, stream=None) -> None:
    """Staged prefill, stage 2: K^C and V [B, H, n_keys, d_h] fp16 of the
    completed slots the queries attend (n_keys = prefill_slot_keys)."""
    B, H, st = dims.batch, dims.heads, dims.torch_dtype
    N = int(partials.shape[1])
    S = prefill_slot_keys(dims, N)
    _check(_lib.mtla_prefill_keys(
        ctypes.byref(dims), N,
        _tensor("partials", partials, (B, N, dims.width), st),
        _tensor("w_uk", w_uk, (H, dims.d_h, dims.d_c), st),
        _tensor("w_uv", w_uv, (H, dims.d_h, dims.d_c), st),
        _tensor("k_c", k_c, (B, H, S, dims.d_h), torch.float16, optional=S == 0),
        _tensor("v", v, (B, H, S, dims.d_h), torch.float16, optional=S == 0),
        _stream(stream)))


def mtla_prefill_attention(dims: MtlaDims, q_c, q_r, partials, w_uk, w_uv, k_c, v, out, stream=None) -> None:
    """Staged prefill, stage 3: the stride-masked attention over the staged
    slot keys; each query's own key is formed from partials and the weights."""
    B, H, st = dims.batch, dims.heads, dims.torch_dtype
    N = int(q_c.shape[1])
    S = prefill_slot_keys(dims, N)
    _check(_lib.mtla_prefill_attention(
        ctypes.byref(dims), N,
        _tensor("q_c", q_c, (B, N, H, dims.d_h), st),
        _tensor("q_r", q_r, (B, N, H, dims.d_r), st, optional=dims.d_r == 0),
        _tensor("partials", partials, (B, N, dims.width), st),
        _tensor("w_uk", w_uk, (H, dims.d_h, dims.d_c), st),
        _tensor("w_uv", w_uv, (H, dims.d_h, dims.d_c), st),
        _tensor("k_c", k_c, (B, H, S, dims.d_h), torch.float16, optional=S == 0),
        _tensor("v", v, (B, H, S, dims.d_h), torch.float16, optional=S == 0),
        _tensor("out", out, (B, N, H, dims.d_h), st),
        _stream(stream)))


def mtla_calib_stream_read(src, workgroups: int, sink, stream=None) -> None:
    """Measurement hook: stream-read every byte of `src` (a device tensor)."""
    nbytes = src.numel() * src.element_size()
    if sink.numel() < workgroups * 4 or sink.dtype != torch.int32:
        raise ValueError("sink must be int32 with at least workgroups * 4 elements")
    _check(_lib.mtla_calib_stream_read(src.data_ptr(), nbytes, workgroups, sink.data_ptr(), _stream(stream)))


def mtla_calib_mfma(f16: bool, workgroups: int, iters: int, out, stream=None) -> float:
    """Measurement hook: MFMA chains on registers; returns the flops performed."""
    if out.numel() < workgroups * 256 or out.dtype != torch.float32:
        raise ValueError("out must be float32 with at least workgroups * 256 elements")
    flops = ctypes.c_double(0.0)
    _check(_lib.mtla_calib_mfma(int(f16), workgroups, iters, out.data_ptr(), ctypes.byref(flops), _stream(stream)))
    return flops.value


def mtla_calib_empty(stream=None) -> None:
    """Measurement hook: one kernel that does nothing."""
    _check(_lib.mtla_calib_empty(_stream(stream)))


def mtla_calib_load_pattern(pattern: int, workgroups: int, buf, cycles, stream=None) -> None:
    """Per-workgroup cycles of 8 waves x 32 load instructions (pattern 0:
    contiguous kilobytes, 1: 16 rows x 64 bytes) from L2-resident data."""
    nbytes = buf.numel() * buf.element_size()
    if cycles.dtype != torch.int32 or cycles.numel() < workgroups + 64:
        raise ValueError("cycles: int32 tensor of at least workgroups + 64 elements")
    _check(_lib.mtla_calib_load_pattern(pattern, workgroups, buf.data_ptr(), nbytes, cycles.data_ptr(),
                                        _stream(stream)))


def mtla_calib_tile_stream(rows, splits: int, interleave: bool, nt: bool, sink, stream=None) -> None:
    """Measurement hook: the long-cache decode attention's load schedule over
    `rows` ([seqs, rows_per_seq, 1152] uint8 on the device), no arithmetic."""
    if rows.dim() != 3 or rows.shape[2] != 1152 or rows.dtype != torch.uint8 or not rows.is_contiguous():
        raise ValueError("rows must be a contiguous uint8 tensor [seqs, rows_per_seq, 1152]")
    seqs, n = int(rows.shape[0]), int(rows.shape[1])
    if sink.numel() < seqs * splits * 8 or sink.dtype != torch.int32:
        raise ValueError("sink must be int32 with at least seqs * splits * 8 elements")
    flags = (1 if interleave else 0) | (2 if nt else 0)
    _check(_lib.mtla_calib_tile_stream(rows.data_ptr(), seqs, n, splits, flags, sink.data_ptr(), _stream(stream)))


def mtla_absorb_query(dims: MtlaDims, q_c, q_r, w_uk, q_lat, stream=None) -> None:
    R, H, st = int(q_c.shape[0]), dims.heads, dims.torch_dtype
    _check(_lib.mtla_absorb_query(
        ctypes.byref(dims), R,
        _tensor("q_c", q_c, (R, H, dims.d_h), st),
        _tensor("q_r", q_r, (R, H, dims.d_r), st, optional=dims.d_r == 0),
        _tensor("w_uk", w_uk, (H, dims.d_h, dims.d_c), st),
        _tensor("q_lat", q_lat, (R, H, dims.width), torch.float32), _stream(stream)))


def mtla_decode_attention_workspace_bytes(dims: MtlaDims) -> int:
    n = _SZ(0)
    _check(_lib.mtla_decode_attention_workspace_bytes(ctypes.byref(dims), ctypes.byref(n)))
    return n.value


def mtla_decode_attention(dims: MtlaDims, pos, q_lat, cache, o_lat, workspace, stream=None) -> None:
    B, H = dims.batch, dims.heads
    ws, ws_bytes = _ws("workspace", workspace, 0)
    _check(_lib.mtla_decode_attention(
        ctypes.byref(dims),
        _tensor("pos", pos, (B,), torch.int32),
        _tensor("q_lat", q_lat, (B, H, dims.width), torch.float32),
        _tensor("cache", cache, (B, dims.max_slots, dims.width), dims.torch_dtype),
        _tensor("o_lat", o_lat, (B, H, dims.d_c), torch.float32),
        ws, ws_bytes, _stream(stream)))


def mtla_up_project(dims: MtlaDims, o_lat, w_uv, out, stream=None) -> None:
    R, H, st = int(o_lat.shape[0]), dims.heads, dims.torch_dtype
    _check(_lib.mtla_up_project(
        ctypes.byref(dims), R,
        _tensor("o_lat", o_lat, (R, H, dims.d_c), torch.float32),
        _tensor("w_uv", w_uv, (H, dims.d_h, dims.d_c), st),
        _tensor("out", out, (R, H, dims.d_h), st), _stream(stream)))


def decode_attention_workspace(dims: MtlaDims) -> torch.Tensor:
    """A workspace of the size mtla_decode_attention needs."""
    return torch.empty(mtla_decode_attention_workspace_bytes(dims), dtype=torch.uint8, device="cuda")


def mtla_prefill_workspace_bytes(dims: MtlaDims, n_tokens: int) -> int:
    n = _SZ(0)
    _check(_lib.mtla_prefill_workspace_bytes(ctypes.byref(dims), n_tokens, ctypes.byref(n)))
    return n.value


def mtla_prefill(dims: MtlaDims, q_c, q_r, c, k_r, w_hyp, pe, w_uk, w_uv, cache, open_acc,
                 out, workspace, stream=None) -> None:
    B, H, st = dims.batch, dims.heads, dims.torch_dtype
    N = int(c.shape[1]) if c.dim() == 3 else -1
    ws, ws_bytes = _ws("workspace", workspace, 0)
    _check(_lib.mtla_prefill(
        ctypes.byref(dims), N,
        _tensor("q_c", q_c, (B, N, H, dims.d_h), st),
        _tensor("q_r", q_r, (B, N, H, dims.d_r), st, optional=dims.d_r == 0),
        _tensor("c", c, (B, N, dims.d_c), st),
        _tensor("k_r", k_r, (B, N, dims.d_r), st, optional=dims.d_r == 0),
        _tensor("w_hyp", w_hyp, dims.gate_shape, torch.float32),
        _tensor("pe", pe, (pe.shape[0], dims.d_c), torch.float32), int(pe.shape[0]),
        _tensor("w_uk", w_uk, (H, dims.d_h, dims.d_c), st),
        _tensor("w_uv", w_uv, (H, dims.d_h, dims.d_c), st),
        _tensor("cache", cache, (B, dims.max_slots, dims.width), st),
        _tensor("open_acc", open_acc, (B, 2, dims.width), torch.float32),
        _tensor("out", out, (B, N, H, dims.d_h), st),
        ws, ws_bytes, _stream(stream)))


def mtla_prefill_backward_workspace_bytes(dims: MtlaDims, n_tokens: int) -> int:
    n = _SZ(0)
    _check(_lib.mtla_prefill_backward_workspace_bytes(ctypes.byref(dims), n_tokens, ctypes.byref(n)))
    return n.value


def mtla_prefill_backward(dims: MtlaDims, q_c, q_r, c, k_r, w_hyp, pe, w_uk, w_uv, grad_out,
                          grad_q_c, grad_q_r, grad_c, grad_k_r, grad_w_hyp, grad_w_uk, grad_w_uv,
                          workspace, stream=None) -> None:
    B, H, st = dims.batch, dims.heads, dims.torch_dtype
    N = int(c.shape[1]) if c.dim() == 3 else -1
    ws, ws_bytes = _ws("workspace", workspace, 0)
    nr = dims.d_r == 0
    _check(_lib.mtla_prefill_backward(
        ctypes.byref(dims), N,
        _tensor("q_c", q_c, (B, N, H, dims.d_h), st),
        _tensor("q_r", q_r, (B, N, H, dims.d_r), st, optional=nr),
        _tensor("c", c, (B, N, dims.d_c), st),
        _tensor("k_r", k_r, (B, N, dims.d_r), st, optional=nr),
        _tensor("w_hyp", w_hyp, dims.gate_shape, torch.float32),
        _tensor("pe", pe, (pe.shape[0], dims.d_c), torch.float32), int(pe.shape[0]),
        _tensor("w_uk", w_uk, (H, dims.d_h, dims.d_c), st),
        _tensor("w_uv", w_uv, (H, dims.d_h, dims.d_c), st),
        _tensor("grad_out", grad_out, (B, N, H, dims.d_h), st),
        _tensor("grad_q_c", grad_q_c, (B, N, H, dims.d_h), st),
        _tensor("grad_q_r", grad_q_r, (B, N, H, dims.d_r), st, optional=nr),
        _tensor("grad_c", grad_c, (B, N, dims.d_c), st),
        _tensor("grad_k_r", grad_k_r, (B, N, dims.d_r), st, optional=nr),
        _tensor("grad_w_hyp", grad_w_hyp, dims.gate_shape, torch.float32),
        _tensor("grad_w_uk", grad_w_uk, (H, dims.d_h, dims.d_c), torch.float32),
        _tensor("grad_w_uv", grad_w_uv, (H, dims.d_h, dims.d_c), torch.float32),
        ws, ws_bytes, _stream(stream)))


def mtla_prefill_at_workspace_bytes(dims: MtlaDims, t0: int, n_tokens: int) -> int:
    n = _SZ(0)
    _check(_lib.mtla_prefill_at_workspace_bytes(ctypes.byref(dims), t0, n_tokens, ctypes.byref(n)))
    return n.value


def mtla_prefill_at(dims: MtlaDims, t0: int, q_c, q_r, c, k_r, w_hyp, pe, w_uk, w_uv, cache,
                    open_acc, out, workspace, stream=None) -> None:
    B, H, st = dims.batch, dims.heads, dims.torch_dtype
    N = int(c.shape[1]) if c.dim() == 3 else -1
    ws, ws_bytes = _ws("workspace", workspace, 0)
    _check(_lib.mtla_prefill_at(
        ctypes.byref(dims), int(t0), N,
        _tensor("q_c", q_c, (B, N, H, dims.d_h), st),
        _tensor("q_r", q_r, (B, N, H, dims.d_r), st, optional=dims.d_r == 0),
        _tensor("c", c, (B, N, dims.d_c), st),
        _tensor("k_r", k_r, (B, N, dims.d_r), st, optional=dims.d_r == 0),
        _tensor("w_hyp", w_hyp, dims.gate_shape, torch.float32),
        _tensor("pe", pe, (pe.shape[0], dims.d_c), torch.float32), int(pe.shape[0]),
        _tensor("w_uk", w_uk, (H, dims.d_h, dims.d_c), st),
        _tensor("w_uv", w_uv, (H, dims.d_h, dims.d_c), st),
        _tensor("cache", cache, (B, dims.max_slots, dims.width), st),
        _tensor("open_acc", open_acc, (B, 2, dims.width), torch.float32),
        _tensor("out", out, (B, N, H, dims.d_h), st),
        ws, ws_bytes, _stream(stream)))


def mtla_reorder_state(dims: MtlaDims, src, pos, cache_in, open_in, cache_out, open_out,
                       pos_out=None, stream=None) -> None:
    B, st = dims.batch, dims.torch_dtype
    _check(_lib.mtla_reorder_state(
        ctypes.byref(dims),
        _tensor("src", src, (B,), torch.int32),
        _tensor("pos", pos, (B,), torch.int32),
        _tensor("cache_in", cache_in, (B, dims.max_slots, dims.width), st),
        _tensor("open_in", open_in, (B, 2, dims.width), torch.float32),
        _tensor("cache_out", cache_out, (B, dims.max_slots, dims.width), st),
        _tensor("open_out", open_out, (B, 2, dims.width), torch.float32),
        _tensor("pos_out", pos_out, (B,), torch.int32, optional=True),
        _stream(stream)))


def _layer_weights(dims: MtlaDims, d_model: int, w_dkv, w_q, w_r, w_o):
    H, st = dims.heads, dims.torch_dtype
    return (_tensor("w_dkv", w_dkv, (dims.d_c, d_model), st),
            _tensor("w_q", w_q, (H * (dims.d_h + dims.d_r), d_model), st),
            _tensor("w_r", w_r, (dims.d_r, d_model), st, optional=dims.d_r == 0),
            _tensor("w_o", w_o, (d_model, H * dims.d_h), st))


def mtla_project_inputs(dims: MtlaDims, pos0, h, w_dkv, w_q, w_r, c, k_r, q_c, q_r, stream=None) -> None:
    B, H, st = dims.batch, dims.heads, dims.torch_dtype
    T, dm = (int(h.shape[1]), int(h.shape[2])) if h.dim() == 3 else (-1, -1)
    _check(_lib.mtla_project_inputs(
        ctypes.byref(dims), dm, T,
        _tensor("pos0", pos0, (B,), torch.int32),
        _tensor("h", h, (B, T, dm), st),
        _tensor("w_dkv", w_dkv, (dims.d_c, dm), st),
        _tensor("w_q", w_q, (H * (dims.d_h + dims.d_r), dm), st),
        _tensor("w_r", w_r, (dims.d_r, dm), st, optional=dims.d_r == 0),
        _tensor("c", c, (B, T, dims.d_c), st),
        _tensor("k_r", k_r, (B, T, dims.d_r), st, optional=dims.d_r == 0),
        _tensor("q_c", q_c, (B, T, H, dims.d_h), st),
        _tensor("q_r", q_r, (B, T, H, dims.d_r), st, optional=dims.d_r == 0),
        _stream(stream)))


def mtla_output_project(dims: MtlaDims, o, w_o, y, stream=None) -> None:
    H, st = dims.heads, dims.torch_dtype
    R, dm = int(o.shape[0]), int(y.shape[-1])
    _check(_lib.mtla_output_project(
        ctypes.byref(dims), dm, R,
        _tensor("o", o, (R, H, dims.d_h), st),
        _tensor("w_o", w_o, (dm, H * dims.d_h), st),
        _tensor("y", y, (R, dm), st),
        _stream(stream)))


def mtla_layer_decode_workspace_bytes(dims: MtlaDims, d_model: int) -> int:
    n = _SZ(0)
    _check(_lib.mtla_layer_decode_workspace_bytes(ctypes.byref(dims), d_model, ctypes.byref(n)))
    return n.value


def mtla_layer_decode_step(dims: MtlaDims, pos, h, w_dkv, w_q, w_r, w_o, w_hyp, pe, w_uk, w_uv, cache,
                           open_acc, y, workspace, stream=None) -> None:
    B, H, st = dims.batch, dims.heads, dims.torch_dtype
    dm = int(h.shape[-1])
    ws, ws_bytes = _ws("workspace", workspace, 0)
    wd, wq, wr, wo = _layer_weights(dims, dm, w_dkv, w_q, w_r, w_o)
    _check(_lib.mtla_layer_decode_step(
        ctypes.byref(dims), dm,
        _tensor("pos", pos, (B,), torch.int32),
        _tensor("h", h, (B, dm), st), wd, wq, wr, wo,
        _tensor("w_hyp", w_hyp, dims.gate_shape, torch.float32),
        _tensor("pe", pe, (pe.shape[0], dims.d_c), torch.float32), int(pe.shape[0]),
        _tensor("w_uk", w_uk, (H, dims.d_h, dims.d_c), st),
        _tensor("w_uv", w_uv, (H, dims.d_h, dims.d_c), st),
        _tensor("cache", cache, (B, dims.max_slots, dims.width), st),
        _tensor("open_acc", open_acc, (B, 2, dims.width), torch.float32),
        _tensor("y", y, (B, dm), st),
        ws, ws_bytes, _stream(stream)))


def mtla_layer_decode_step_tiles(dims: MtlaDims, pos, h, w_dkv, w_q, w_r, w_o, w_hyp, pe, w_uk, w_uv, w_uv_tiles,
                                 cache, open_acc, y, workspace, stream=None) -> None:
    B, H, st = dims.batch, dims.heads, dims.torch_dtype
    dm = int(h.shape[-1])
    ws, ws_bytes = _ws("workspace", workspace, 0)
    wd, wq, wr, wo = _layer_weights(dims, dm, w_dkv, w_q, w_r, w_o)
    n = mtla_w_uv_tiles_bytes(dims) // 2
    _check(_lib.mtla_layer_decode_step_tiles(
        ctypes.byref(dims), dm,
        _tensor("pos", pos, (B,), torch.int32),
        _tensor("h", h, (B, dm), st), wd, wq, wr, wo,
        _tensor("w_hyp", w_hyp, dims.gate_shape, torch.float32),
        _tensor("pe", pe, (pe.shape[0], dims.d_c), torch.float32), int(pe.shape[0]),
        _tensor("w_uk", w_uk, (H, dims.d_h, dims.d_c), st),
        _tensor("w_uv", w_uv, (H, dims.d_h, dims.d_c), st),
        _tensor("w_uv_tiles", w_uv_tiles, (n,), st),
        _tensor("cache", cache, (B, dims.max_slots, dims.width), st),
        _tensor("open_acc", open_acc, (B, 2, dims.width), torch.float32),
        _tensor("y", y, (B, dm), st),
        ws, ws_bytes, _stream(stream)))


def mtla_layer_prefill_workspace_bytes(dims: MtlaDims, d_model: int, t0: int, n_tokens: int) -> int:
    n = _SZ(0)
    _check(_lib.mtla_layer_prefill_workspace_bytes(ctypes.byref(dims), d_model, t0, n_tokens, ctypes.byref(n)))
    return n.value


def mtla_layer_prefill(dims: MtlaDims, t0: int, h, w_dkv, w_q, w_r, w_o, w_hyp, pe, w_uk, w_uv, cache,
                       open_acc, y, workspace, stream=None) -> None:
    B, H, st = dims.batch, dims.heads, dims.torch_dtype
    N, dm = (int(h.shape[1]), int(h.shape[2])) if h.dim() == 3 else (-1, -1)
    ws, ws_bytes = _ws("workspace", workspace, 0)
    wd, wq, wr, wo = _layer_weights(dims, dm, w_dkv, w_q, w_r, w_o)
    _check(_lib.mtla_layer_prefill(
        ctypes.byref(dims), dm, int(t0), N,
        _tensor("h", h, (B, N, dm), st), wd, wq, wr, wo,
        _tensor("w_hyp", w_hyp, dims.gate_shape, torch.float32),
        _tensor("pe", pe, (pe.shape[0], dims.d_c), torch.float32), int(pe.shape[0]),
        _tensor("w_uk", w_uk, (H, dims.d_h, dims.d_c), st),
        _tensor("w_uv", w_uv, (H, dims.d_h, dims.d_c), st),
        _tensor("cache", cache, (B, dims.max_slots, dims.width), st),
        _tensor("open_acc", open_acc, (B, 2, dims.width), torch.float32),
        _tensor("y", y, (B, N, dm), st),
        ws, ws_bytes, _stream(stream)))


def mtla_debug_stride_mask(n: int, s: int, mask, stream=None) -> None:
    _check(_lib.mtla_debug_stride_mask(n, s, _tensor("mask", mask, (n, n), torch.uint8),
                                       _stream(stream)))


def mtla_debug_slot_limits(n: int, s: int, hi, stream=None) -> None:
    _check(_lib.mtla_debug_slot_limits(n, s, _tensor("hi", hi, (n,), torch.int32),
                                       _stream(stream)))
