"""CPU: the C-ABI library loads, exports every declared entry point, and
rejects bad arguments before touching the GPU (no kernel is launched here)."""
import ctypes
import re
import subprocess

import pytest

from tests.libmtla import ensure_built

ensure_built()
import temporally_compressed_latent_amd as m  # noqa: E402
from temporally_compressed_latent_amd import _lib  # noqa: E402

FAKE = 0x10000          # 16-byte aligned, never dereferenced (checks fail first)
MISALIGNED = 0x10001


def dims(**kw):
    d = m.make_dims(4, 8, 64, 256, 32, 2, 128)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_exports_every_header_symbol():
    syms = m.header_symbols()
    assert len(syms) == 42
    for s in syms:
        assert hasattr(m.lib(), s), s
    out = subprocess.run(["nm", "-D", "--defined-only", m.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\b(mtla_[a-z_]+)\b", out))
    assert exported == set(syms)


def test_status_strings_and_version():
    assert m.mtla_version() == 10100
    for code, name in [(0, "MTLA_OK"), (-1, "MTLA_ERR_INVALID_ARG"), (-2, "MTLA_ERR_UNSUPPORTED"),
                       (-3, "MTLA_ERR_WORKSPACE"), (-4, "MTLA_ERR_HIP"), (7, "MTLA_UNKNOWN_STATUS")]:
        assert m.status_string(code) == name


def test_workspace_sizes_are_host_only():
    d = dims()
    wd = m.mtla_decode_workspace_bytes(d)
    wp = m.mtla_prefill_workspace_bytes(d, 512)
    assert wd > 0 and wp > 0 and wd % 256 == 0 and wp % 256 == 0
    # more slots -> more split partials; more tokens -> more prefill scratch
    assert m.mtla_decode_workspace_bytes(dims(max_slots=4096)) >= wd
    assert m.mtla_prefill_workspace_bytes(d, 1024) > wp


BAD_DIMS = [
    (dict(batch=-1), m.MTLA_ERR_INVALID_ARG),
    (dict(heads=0), m.MTLA_ERR_INVALID_ARG),
    (dict(d_h=0), m.MTLA_ERR_INVALID_ARG),
    (dict(d_c=0), m.MTLA_ERR_INVALID_ARG),
    (dict(d_r=-2), m.MTLA_ERR_INVALID_ARG),
    (dict(stride_s=0), m.MTLA_ERR_INVALID_ARG),
    (dict(max_slots=0), m.MTLA_ERR_INVALID_ARG),
    (dict(dtype=7), m.MTLA_ERR_INVALID_ARG),
    (dict(softmax_scale=0.0), m.MTLA_ERR_INVALID_ARG),
    (dict(softmax_scale=float("nan")), m.MTLA_ERR_INVALID_ARG),
    (dict(flags=8), m.MTLA_ERR_INVALID_ARG),
    (dict(stride_s=257), m.MTLA_ERR_UNSUPPORTED),
    (dict(d_c=1000, d_r=64), m.MTLA_ERR_UNSUPPORTED),
    (dict(d_h=512), m.MTLA_ERR_UNSUPPORTED),
    (dict(d_c=252), m.MTLA_ERR_UNSUPPORTED),
    (dict(d_r=30), m.MTLA_ERR_UNSUPPORTED),
    (dict(decode_splits=-1), m.MTLA_ERR_INVALID_ARG),
    (dict(decode_splits=65), m.MTLA_ERR_INVALID_ARG),
    (dict(step_groups=-1), m.MTLA_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("kw,status", BAD_DIMS, ids=[str(k) for k, _ in BAD_DIMS])
def test_bad_dims_rejected_everywhere(kw, status):
    L = m.lib()
    d = dims(**kw)
    n = ctypes.c_size_t(0)
    assert L.mtla_decode_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == status
    assert L.mtla_prefill_workspace_bytes(ctypes.byref(d), 16, ctypes.byref(n)) == status
    assert L.mtla_merge_append(ctypes.byref(d), FAKE, 1, FAKE, FAKE, FAKE, FAKE, 8, FAKE, FAKE, None, None) == status
    assert L.mtla_decode(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == status
    assert L.mtla_prefill(ctypes.byref(d), 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, FAKE, FAKE, FAKE, FAKE,
                          FAKE, FAKE, 1 << 30, None) == status
    assert m.last_error() != ""


def test_staged_decode_checks():
    L, d = m.lib(), dims()
    need = m.mtla_decode_attention_workspace_bytes(d)
    assert need > 0
    assert L.mtla_absorb_query(ctypes.byref(d), -1, FAKE, FAKE, FAKE, FAKE, None) == m.MTLA_ERR_INVALID_ARG
    assert L.mtla_absorb_query(ctypes.byref(d), 4, FAKE, FAKE, FAKE, None, None) == m.MTLA_ERR_INVALID_ARG
    assert L.mtla_absorb_query(ctypes.byref(d), 0, None, None, None, None, None) == m.MTLA_OK
    assert L.mtla_up_project(ctypes.byref(d), 4, MISALIGNED, FAKE, FAKE, None) == m.MTLA_ERR_INVALID_ARG
    assert L.mtla_up_project(ctypes.byref(d), 0, None, None, None, None) == m.MTLA_OK
    call = lambda **k: L.mtla_decode_attention(
        ctypes.byref(d), k.get("pos", FAKE), k.get("q", FAKE), k.get("cache", FAKE), k.get("o", FAKE),
        k.get("ws", FAKE), k.get("n", need), None)
    for name in ("pos", "q", "cache", "o"):
        assert call(**{name: None}) == m.MTLA_ERR_INVALID_ARG, name
    assert call(ws=None) == m.MTLA_ERR_WORKSPACE
    assert call(n=need - 1) == m.MTLA_ERR_WORKSPACE


def test_decode_plan():
    # short cache with the workload shapes: one split, fused step kernel
    assert m.mtla_decode_plan(m.make_dims(50, 8, 64, 256, 32, 2, 256)) == (1, True)
    assert m.mtla_decode_plan(m.make_dims(50, 8, 64, 256, 32, 4, 512)) == (1, True)
    # long cache: several splits (one workgroup per compute unit), staged kernels
    sp, fused = m.mtla_decode_plan(m.make_dims(64, 32, 128, 512, 64, 2, 16385))
    assert sp == 4 and not fused
    # fp32 storage and the portable flag never take the MFMA kernels
    assert not m.mtla_decode_plan(m.make_dims(1, 4, 64, 256, 32, 2, 32, "fp32"))[1]
    assert not m.mtla_decode_plan(m.make_dims(2, 8, 64, 256, 32, 2, 32, portable=True))[1]


def test_null_dims():
    L = m.lib()
    assert L.mtla_decode(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None) == m.MTLA_ERR_INVALID_ARG
    assert "dims" in m.last_error()


def test_merge_argument_checks():
    L, d = m.lib(), dims()
    call = lambda **k: L.mtla_merge_append(
        ctypes.byref(d), k.get("pos0", FAKE), k.get("T", 4), k.get("c", FAKE), k.get("k_r", FAKE),
        k.get("w", FAKE), k.get("pe", FAKE), k.get("pe_rows", 64), k.get("cache", FAKE),
        k.get("acc", FAKE), k.get("gate", None), None)
    assert call(T=-1) == m.MTLA_ERR_INVALID_ARG
    assert call(pe_rows=0) == m.MTLA_ERR_INVALID_ARG
    assert call(T=65, pe_rows=64) == m.MTLA_ERR_INVALID_ARG          # more tokens than pe rows
    assert call(T=257, pe_rows=1000) == m.MTLA_ERR_INVALID_ARG       # beyond s * max_slots
    c_names = {"pos0": "pos0", "c": "c", "k_r": "k_r", "w": "w_hyp", "pe": "pe", "cache": "cache",
               "acc": "open_acc"}
    for name, c_name in c_names.items():
        assert call(**{name: None}) == m.MTLA_ERR_INVALID_ARG, name
        assert m.last_error().startswith(c_name + " "), (name, m.last_error())
        assert call(**{name: MISALIGNED}) == m.MTLA_ERR_INVALID_ARG, name
    assert call(gate=MISALIGNED) == m.MTLA_ERR_INVALID_ARG
    # empty work is a no-op, even with null pointers
    assert call(T=0, c=None, cache=None) == m.MTLA_OK
    d0 = dims(batch=0)
    assert L.mtla_merge_append(ctypes.byref(d0), None, 4, None, None, None, None, 8, None, None, None, None) == m.MTLA_OK


def test_decode_argument_checks():
    L, d = m.lib(), dims()
    need = m.mtla_decode_workspace_bytes(d)
    call = lambda **k: L.mtla_decode(
        ctypes.byref(d), k.get("pos", FAKE), k.get("q", FAKE), k.get("qr", FAKE), k.get("uk", FAKE),
        k.get("uv", FAKE), k.get("cache", FAKE), k.get("out", FAKE), k.get("ws", FAKE),
        k.get("n", need), None)
    for name in ("pos", "q", "qr", "uk", "uv", "cache", "out"):
        assert call(**{name: None}) == m.MTLA_ERR_INVALID_ARG, name
        assert call(**{name: MISALIGNED}) == m.MTLA_ERR_INVALID_ARG, name
    assert call(ws=None) == m.MTLA_ERR_WORKSPACE
    assert call(n=need - 1) == m.MTLA_ERR_WORKSPACE
    assert call(ws=MISALIGNED) == m.MTLA_ERR_INVALID_ARG
    d0 = dims(batch=0)
    assert L.mtla_decode(ctypes.byref(d0), None, None, None, None, None, None, None, None, 0, None) == m.MTLA_OK


def test_prefill_argument_checks():
    L, d = m.lib(), dims()
    need = m.mtla_prefill_workspace_bytes(d, 32)
    call = lambda **k: L.mtla_prefill(
        ctypes.byref(d), k.get("N", 32), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, k.get("pe_rows", 64),
        FAKE, FAKE, k.get("cache", FAKE), FAKE, FAKE, k.get("ws", FAKE), k.get("n", need), None)
    assert call(N=-1) == m.MTLA_ERR_INVALID_ARG
    assert call(N=65, pe_rows=64) == m.MTLA_ERR_INVALID_ARG
    assert call(N=300, pe_rows=400) == m.MTLA_ERR_INVALID_ARG        # 300 > s * max_slots = 256
    assert call(cache=None) == m.MTLA_ERR_INVALID_ARG
    assert call(ws=None) == m.MTLA_ERR_WORKSPACE
    assert call(n=need - 16) == m.MTLA_ERR_WORKSPACE
    assert call(N=0, cache=None, ws=None) == m.MTLA_OK


def test_prefill_at_argument_checks():
    L, d = m.lib(), dims()
    need = m.mtla_prefill_at_workspace_bytes(d, 40, 32)
    # continuing after cached tokens: the fast path also holds K^C and V of every slot
    assert need > m.mtla_prefill_workspace_bytes(d, 32)
    assert m.mtla_prefill_at_workspace_bytes(d, 0, 32) == m.mtla_prefill_workspace_bytes(d, 32)
    call = lambda **k: L.mtla_prefill_at(
        ctypes.byref(d), k.get("t0", 40), k.get("N", 32), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
        k.get("pe_rows", 128), FAKE, FAKE, k.get("cache", FAKE), FAKE, FAKE, k.get("ws", FAKE),
        k.get("n", need), None)
    assert call(t0=-1) == m.MTLA_ERR_INVALID_ARG
    assert call(N=-1) == m.MTLA_ERR_INVALID_ARG
    assert call(t0=100, pe_rows=128) == m.MTLA_ERR_INVALID_ARG        # t0 + N = 132 > pe_rows
    assert call(t0=240, pe_rows=400) == m.MTLA_ERR_INVALID_ARG        # 272 > s * max_slots = 256
    assert call(cache=None) == m.MTLA_ERR_INVALID_ARG
    assert call(ws=None) == m.MTLA_ERR_WORKSPACE
    assert call(n=need - 16) == m.MTLA_ERR_WORKSPACE
    assert call(N=0, cache=None, ws=None) == m.MTLA_OK
    n = ctypes.c_size_t(0)
    assert L.mtla_prefill_at_workspace_bytes(ctypes.byref(d), -1, 4, ctypes.byref(n)) == m.MTLA_ERR_INVALID_ARG


def test_reorder_argument_checks():
    L, d = m.lib(), dims()
    A = FAKE
    B_ = FAKE + 4096
    call = lambda **k: L.mtla_reorder_state(
        ctypes.byref(d), k.get("src", A), k.get("pos", A), k.get("ci", A), k.get("oi", A),
        k.get("co", B_), k.get("oo", B_), k.get("po", None), None)
    assert call(src=None) == m.MTLA_ERR_INVALID_ARG
    assert call(pos=None) == m.MTLA_ERR_INVALID_ARG
    assert call(ci=None) == m.MTLA_ERR_INVALID_ARG
    assert call(co=A) == m.MTLA_ERR_INVALID_ARG          # in place
    assert call(oo=A) == m.MTLA_ERR_INVALID_ARG          # in place
    assert call(po=A) == m.MTLA_ERR_INVALID_ARG          # pos_out aliases pos
    assert call(co=MISALIGNED) == m.MTLA_ERR_INVALID_ARG
    d0 = dims(batch=0)
    assert L.mtla_reorder_state(ctypes.byref(d0), None, None, None, None, None, None, None, None) == m.MTLA_OK


def test_layer_argument_checks():
    L, d = m.lib(), dims()
    n = ctypes.c_size_t(0)
    assert L.mtla_layer_decode_workspace_bytes(ctypes.byref(d), 512, ctypes.byref(n)) == m.MTLA_OK
    dec = n.value
    assert dec >= m.mtla_decode_workspace_bytes(d)
    assert L.mtla_layer_decode_workspace_bytes(ctypes.byref(d), 500, ctypes.byref(n)) == m.MTLA_ERR_UNSUPPORTED
    assert L.mtla_layer_prefill_workspace_bytes(ctypes.byref(d), 512, 0, 32, ctypes.byref(n)) == m.MTLA_OK
    assert n.value > m.mtla_prefill_workspace_bytes(d, 32)
    assert L.mtla_layer_prefill_workspace_bytes(ctypes.byref(d), 512, -1, 32, ctypes.byref(n)) == \
        m.MTLA_ERR_INVALID_ARG
    proj = lambda **k: L.mtla_project_inputs(
        ctypes.byref(k.get("d", d)), k.get("dm", 512), k.get("T", 4), k.get("pos0", FAKE), k.get("h", FAKE),
        FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert proj(dm=0) == m.MTLA_ERR_UNSUPPORTED
    assert proj(dm=12) == m.MTLA_ERR_UNSUPPORTED
    assert proj(d=dims(d_h=63)) == m.MTLA_ERR_UNSUPPORTED              # odd d_h: rope pairs
    assert proj(T=-1) == m.MTLA_ERR_INVALID_ARG
    assert proj(pos0=None) == m.MTLA_ERR_INVALID_ARG
    assert proj(h=MISALIGNED) == m.MTLA_ERR_INVALID_ARG
    assert proj(T=0, pos0=None, h=None) == m.MTLA_OK
    outp = lambda **k: L.mtla_output_project(ctypes.byref(d), k.get("dm", 512), k.get("R", 4),
                                             k.get("o", FAKE), k.get("w", FAKE), k.get("y", FAKE), None)
    assert outp(R=-1) == m.MTLA_ERR_INVALID_ARG
    assert outp(o=None) == m.MTLA_ERR_INVALID_ARG
    assert outp(R=0, o=None) == m.MTLA_OK
    step = lambda **k: L.mtla_layer_decode_step(
        ctypes.byref(d), 512, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, k.get("pe_rows", 64), FAKE, FAKE,
        k.get("cache", FAKE), FAKE, FAKE, k.get("ws", FAKE), k.get("n", dec), None)
    assert step(pe_rows=0) == m.MTLA_ERR_INVALID_ARG
    assert step(cache=None) == m.MTLA_ERR_INVALID_ARG                  # the core's check, before any launch
    assert step(ws=None) == m.MTLA_ERR_WORKSPACE
    assert step(n=dec - 16) == m.MTLA_ERR_WORKSPACE
    assert L.mtla_layer_prefill_workspace_bytes(ctypes.byref(d), 512, 40, 32, ctypes.byref(n)) == m.MTLA_OK
    pre_n = n.value
    pre = lambda **k: L.mtla_layer_prefill(
        ctypes.byref(d), 512, k.get("t0", 40), k.get("N", 32), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
        k.get("pe_rows", 128), FAKE, FAKE, k.get("cache", FAKE), FAKE, FAKE, k.get("ws", FAKE),
        k.get("n", pre_n), None)
    assert pre(t0=240, pe_rows=400) == m.MTLA_ERR_INVALID_ARG          # beyond s * max_slots
    assert pre(t0=100) == m.MTLA_ERR_INVALID_ARG                       # t0 + N > pe_rows
    assert pre(cache=None) == m.MTLA_ERR_INVALID_ARG
    assert pre(n=pre_n - 16) == m.MTLA_ERR_WORKSPACE
    assert pre(N=0, cache=None, ws=None) == m.MTLA_OK


def test_debug_hook_checks():
    L = m.lib()
    assert L.mtla_debug_stride_mask(0, 2, FAKE, None) == m.MTLA_ERR_INVALID_ARG
    assert L.mtla_debug_stride_mask(4, 0, FAKE, None) == m.MTLA_ERR_INVALID_ARG
    assert L.mtla_debug_stride_mask(4, 2, None, None) == m.MTLA_ERR_INVALID_ARG
    assert L.mtla_debug_slot_limits(4, 2, None, None) == m.MTLA_ERR_INVALID_ARG
    assert L.mtla_sinusoidal_pe(0, 4, FAKE, None) == m.MTLA_ERR_INVALID_ARG
    assert L.mtla_sinusoidal_pe(4, 4, MISALIGNED, None) == m.MTLA_ERR_INVALID_ARG


def test_binding_rejects_wrong_tensors_before_the_library():
    import torch
    d = dims()
    with pytest.raises((ValueError, TypeError)):
        m.mtla_merge_append(d, torch.zeros(4, dtype=torch.int32), torch.zeros(4, 1, 256),
                            torch.zeros(4, 1, 32), torch.zeros(256), torch.zeros(8, 256),
                            torch.zeros(4, 128, 288), torch.zeros(4, 288), stream=0)


def test_backward_argument_checks():
    L, d = m.lib(), dims()
    n = ctypes.c_size_t(0)
    assert L.mtla_prefill_backward_workspace_bytes(ctypes.byref(d), 32, ctypes.byref(n)) == m.MTLA_OK
    need = n.value
    assert need > 0
    assert L.mtla_prefill_backward_workspace_bytes(ctypes.byref(d), -1, ctypes.byref(n)) == m.MTLA_ERR_INVALID_ARG
    assert L.mtla_prefill_backward_workspace_bytes(ctypes.byref(d), 32, None) == m.MTLA_ERR_INVALID_ARG
    assert L.mtla_prefill_backward_workspace_bytes(ctypes.byref(dims(heads=3, d_h=6)), 32, ctypes.byref(n)) == \
        m.MTLA_ERR_UNSUPPORTED                                            # heads * d_h not a multiple of 4
    bwd = lambda **k: L.mtla_prefill_backward(
        ctypes.byref(k.get("d", d)), k.get("N", 32), k.get("q_c", FAKE), FAKE, FAKE, FAKE, k.get("w_hyp", FAKE),
        FAKE, k.get("pe_rows", 64), FAKE, FAKE, k.get("g_out", FAKE), FAKE, FAKE, k.get("g_c", FAKE), FAKE,
        k.get("g_wh", FAKE), FAKE, FAKE, k.get("ws", FAKE), k.get("n", need), None)
    assert bwd(N=-1) == m.MTLA_ERR_INVALID_ARG
    assert bwd(pe_rows=16) == m.MTLA_ERR_INVALID_ARG                     # pe shorter than the sequence
    assert bwd(w_hyp=None) == m.MTLA_ERR_INVALID_ARG
    assert bwd(g_wh=MISALIGNED) == m.MTLA_ERR_INVALID_ARG
    assert bwd(q_c=None) == m.MTLA_ERR_INVALID_ARG
    assert bwd(g_out=None) == m.MTLA_ERR_INVALID_ARG
    assert bwd(g_c=None) == m.MTLA_ERR_INVALID_ARG
    assert bwd(ws=None) == m.MTLA_ERR_WORKSPACE
    assert bwd(ws=MISALIGNED) == m.MTLA_ERR_INVALID_ARG
    assert bwd(n=need - 16) == m.MTLA_ERR_WORKSPACE


def test_per_position_gate_flag():
    """MTLA_FLAG_GATE_PER_POSITION is a known flag (other unknown bits still
    fail); the backward workspace grows by the extra dW_hyp rows; the binding
    asks for W_hyp of shape [s, d_c] under it and [d_c] without."""
    L = m.lib()
    n1, n2 = ctypes.c_size_t(0), ctypes.c_size_t(0)
    plain = dims()
    pp = dims(flags=m.MTLA_FLAG_GATE_PER_POSITION)
    assert L.mtla_decode_workspace_bytes(ctypes.byref(pp), ctypes.byref(n1)) == m.MTLA_OK
    assert L.mtla_decode_workspace_bytes(ctypes.byref(dims(flags=m.MTLA_FLAG_GATE_PER_POSITION | 4)),
                                         ctypes.byref(n1)) == m.MTLA_ERR_INVALID_ARG
    assert L.mtla_prefill_backward_workspace_bytes(ctypes.byref(plain), 64, ctypes.byref(n1)) == m.MTLA_OK
    assert L.mtla_prefill_backward_workspace_bytes(ctypes.byref(pp), 64, ctypes.byref(n2)) == m.MTLA_OK
    assert n2.value >= n1.value
    assert plain.gate_shape == (plain.d_c,)
    assert pp.gate_shape == (pp.stride_s, pp.d_c)
    mk = m.make_dims(2, 8, 64, 256, 32, 3, 10, "bf16", gate_per_position=True)
    assert mk.flags == m.MTLA_FLAG_GATE_PER_POSITION and mk.gate_shape == (3, 256)


def test_decode_splits_field_sets_the_plan():
    """The launch choice is a field of the dims (0 = the library's choice),
    with no environment override: the plan and the workspace follow it."""
    base = dims(batch=4, max_slots=4096)
    assert m.mtla_decode_plan(base)[0] == 8          # min(ceil(256 / 4), ceil(4096 / 512))
    for k in (1, 3, 8):
        assert m.mtla_decode_plan(dims(batch=4, max_slots=4096, decode_splits=k)) == (k, k == 1)   # one split: the one-kernel step
    assert m.mtla_decode_plan(dims(batch=4, max_slots=4096, decode_splits=64))[0] == 8   # clamped
    assert (m.mtla_decode_workspace_bytes(dims(batch=4, max_slots=4096, decode_splits=2))
            < m.mtla_decode_workspace_bytes(dims(batch=4, max_slots=4096, decode_splits=8)))


def test_no_environment_reads_in_the_library():
    """No getenv on the product path: every launch choice is an argument."""
    import glob
    import os
    for path in glob.glob(os.path.join(os.path.dirname(m.LIB_PATH), "csrc", "*")):
        with open(path) as f:
            assert "getenv" not in f.read(), path


def test_staged_prefill_needs_the_mfma_path():
    """The staged prefill exposes the MFMA path's fp16 keys: fp32 storage or a
    shape without that path is MTLA_ERR_UNSUPPORTED, checked on the host."""
    L = m.lib()
    for d in (dims(dtype=m.MTLA_FP32), dims(d_h=48)):
        assert L.mtla_prefill_keys(ctypes.byref(d), 16, FAKE, FAKE, FAKE, FAKE, FAKE, None) == m.MTLA_ERR_UNSUPPORTED
        assert L.mtla_prefill_attention(ctypes.byref(d), 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                        None) == \
            m.MTLA_ERR_UNSUPPORTED
    assert L.mtla_prefill_partials(ctypes.byref(dims()), 16, FAKE, FAKE, FAKE, FAKE, 8, FAKE, FAKE, FAKE, None) == \
        m.MTLA_ERR_INVALID_ARG          # pe_rows < n_tokens


def test_measurement_hook_checks():
    """The measurement hooks reject bad arguments before any launch."""
    L = m.lib()
    bad = m.MTLA_ERR_INVALID_ARG
    assert L.mtla_calib_stream_read(None, 1024, 4, FAKE, None) == bad
    assert L.mtla_calib_stream_read(FAKE, 1000, 4, FAKE, None) == bad      # not a multiple of 16
    assert L.mtla_calib_stream_read(FAKE, 1024, 0, FAKE, None) == bad
    assert L.mtla_calib_mfma(0, 0, 16, FAKE, None, None) == bad
    assert L.mtla_calib_mfma(0, 4, 0, FAKE, None, None) == bad
    assert L.mtla_calib_tile_stream(None, 4, 64, 4, 0, FAKE, None) == bad
    assert L.mtla_calib_tile_stream(MISALIGNED, 4, 64, 4, 0, FAKE, None) == bad
    assert L.mtla_calib_tile_stream(FAKE, 0, 64, 4, 0, FAKE, None) == bad
    assert L.mtla_calib_tile_stream(FAKE, 4, 0, 4, 0, FAKE, None) == bad
    assert L.mtla_calib_tile_stream(FAKE, 4, (2**31) // 1152 + 1, 4, 0, FAKE, None) == bad
    assert L.mtla_calib_load_pattern(2, 4, FAKE, 1 << 20, FAKE, None) == bad     # no such pattern
    assert L.mtla_calib_load_pattern(0, 0, FAKE, 1 << 20, FAKE, None) == bad
    assert L.mtla_calib_load_pattern(0, 4, None, 1 << 20, FAKE, None) == bad
    assert L.mtla_calib_load_pattern(1, 4, FAKE, 65536, FAKE, None) == bad        # under 128 KiB
    assert L.mtla_calib_load_pattern(1, 4, FAKE, 1 << 20, MISALIGNED, None) == bad
    assert L.mtla_calib_tile_stream(FAKE, 4, 64, 65, 0, FAKE, None) == bad
    assert L.mtla_calib_tile_stream(FAKE, 4, 64, 4, 4, FAKE, None) == bad
    assert L.mtla_calib_tile_stream(FAKE, 4, 64, 4, 3, None, None) == bad


def test_w_uv_tiles_argument_checks():
    """The tile-order W_UV entry points: size, bf16 only, pointers checked
    before any launch; the tiled decode step checks its tiles and then
    everything mtla_decode_step checks."""
    L, d = m.lib(), dims()
    assert m.mtla_w_uv_tiles_bytes(d) == 8 * 4 * 16 * 256 * 2               # H=8, d_h=64: 4 tiles of 16 rows
    assert m.mtla_w_uv_tiles_bytes(dims(d_h=40)) == 8 * 3 * 16 * 256 * 2    # rows padded to 48
    d32 = m.make_dims(4, 8, 64, 256, 32, 2, 128, "fp32")
    n = ctypes.c_size_t(0)
    assert L.mtla_w_uv_tiles_bytes(ctypes.byref(d32), ctypes.byref(n)) == m.MTLA_ERR_UNSUPPORTED
    assert L.mtla_w_uv_tiles_bytes(ctypes.byref(d), None) == m.MTLA_ERR_INVALID_ARG
    assert L.mtla_pack_w_uv_tiles(ctypes.byref(d), None, FAKE, None) == m.MTLA_ERR_INVALID_ARG
    assert L.mtla_pack_w_uv_tiles(ctypes.byref(d), FAKE, MISALIGNED, None) == m.MTLA_ERR_INVALID_ARG
    assert L.mtla_pack_w_uv_tiles(ctypes.byref(d32), FAKE, FAKE, None) == m.MTLA_ERR_UNSUPPORTED
    need = m.mtla_decode_workspace_bytes(d)
    call = lambda dd=d, **k: L.mtla_decode_step_tiles(
        ctypes.byref(dd), FAKE, FAKE, FAKE, FAKE, FAKE, k.get("pe_rows", 64), FAKE, FAKE, FAKE, FAKE,
        k.get("tiles", FAKE), FAKE, FAKE, FAKE, k.get("ws", FAKE), need, None)
    assert call(tiles=None) == m.MTLA_ERR_INVALID_ARG and "w_uv_tiles" in m.last_error()
    assert call(tiles=MISALIGNED) == m.MTLA_ERR_INVALID_ARG
    assert call(dd=d32) == m.MTLA_ERR_UNSUPPORTED
    assert call(pe_rows=0) == m.MTLA_ERR_INVALID_ARG
    assert call(ws=None) == m.MTLA_ERR_WORKSPACE


def test_layer_decode_tiles_argument_checks():
    L, d = m.lib(), dims()
    call = lambda dd=d, **k: L.mtla_layer_decode_step_tiles(
        ctypes.byref(dd), 512, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 64, FAKE, FAKE,
        k.get("tiles", FAKE), FAKE, FAKE, FAKE, k.get("ws", FAKE), 1 << 30, None)
    assert call(tiles=None) == m.MTLA_ERR_INVALID_ARG and "w_uv_tiles" in m.last_error()
    assert call(tiles=MISALIGNED) == m.MTLA_ERR_INVALID_ARG
    assert call(dd=m.make_dims(4, 8, 64, 256, 32, 2, 128, "fp32")) == m.MTLA_ERR_UNSUPPORTED
    assert call(ws=None) == m.MTLA_ERR_WORKSPACE
