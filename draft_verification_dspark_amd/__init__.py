"""Python binding of the gfx950 verify/schedule library (``libdspark.so``).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/dspark.h``.  PyTorch provides
device memory and the current stream.  There is no fallback: if the library
has not been built (``python -m draft_verification_dspark_amd.build`` or
``__graft_entry__.build()``), loading raises.

Names follow the C ABI: ``dspark_schedule``, ``dspark_schedule_load_aware``,
``dspark_verify``, ``dspark_verify_greedy``, ``dspark_schedule_verify`` (each
with a ``*_phase`` twin that enqueues the streaming pass or the rest on its
own), ``dspark_calibrate``, ``dspark_calib_observe``,
``dspark_calib_state_bytes``, ``dspark_markov_draft``,
``dspark_workspace_bytes``, ``dspark_status_string``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdspark.so")

DSPARK_OK = 0
DSPARK_F32 = 0
DSPARK_BF16 = 1
OP_SCHEDULE, OP_VERIFY, OP_VERIFY_GREEDY, OP_MARKOV_DRAFT, OP_SCHEDULE_VERIFY = 0, 1, 2, 3, 4

DEV_BAD_TOKEN = 1
DEV_NONFINITE = 2
DEV_BAD_TEMP = 4
DEV_BAD_UNIFORM = 8
DEV_BAD_CONF = 16
DEV_BAD_LENGTH = 32
DEV_BAD_LOAD = 64
DEV_BAD_CURVE = 128
ERR_PARAM = 7

PHASE_STREAM = 1
PHASE_FINISH = 2
PHASE_ALL = PHASE_STREAM | PHASE_FINISH

EXPORTS = ("dspark_workspace_bytes", "dspark_status_string", "dspark_schedule",
           "dspark_schedule_load_aware", "dspark_calibrate", "dspark_calib_state_bytes",
           "dspark_calib_observe", "dspark_markov_draft", "dspark_verify", "dspark_verify_greedy",
           "dspark_schedule_verify", "dspark_verify_phase", "dspark_verify_greedy_phase",
           "dspark_schedule_verify_phase", "dspark_schedule_verify_noalloc")
ERR_SCRATCH = 8
SCRATCH_BYTES = 16 << 20


class DsparkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"dspark status {status}: {msg}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and type the C ABI.  Raises if the library is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run python -m draft_verification_dspark_amd.build")
    lib = ctypes.CDLL(path)
    vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    lib.dspark_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.dspark_workspace_bytes.restype = sz
    lib.dspark_status_string.argtypes = [i32]
    lib.dspark_status_string.restype = ctypes.c_char_p
    lib.dspark_schedule.argtypes = [vp, i32, i32, f32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.dspark_schedule.restype = i32
    lib.dspark_schedule_load_aware.argtypes = [vp, i32, i32, vp, f32, f32, f32, f32, vp, i32, f32,
                                               i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dspark_schedule_load_aware.restype = i32
    lib.dspark_calibrate.argtypes = [vp, vp, i32, i32, vp, vp, vp]
    lib.dspark_calibrate.restype = i32
    lib.dspark_calib_state_bytes.argtypes = [i32, i32]
    lib.dspark_calib_state_bytes.restype = sz
    lib.dspark_calib_observe.argtypes = [vp, vp, vp, i32, i32, vp, f32, f32, i32, i32, vp, sz, vp,
                                         vp, vp]
    lib.dspark_calib_observe.restype = i32
    lib.dspark_markov_draft.argtypes = [vp, i32, i32, i32, i32, vp, vp, i32, f32, vp, vp, vp, vp, vp,
                                        vp, vp, vp, sz, vp]
    lib.dspark_markov_draft.restype = i32
    lib.dspark_verify.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                  vp, sz, vp]
    lib.dspark_verify.restype = i32
    lib.dspark_verify_greedy.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dspark_verify_greedy.restype = i32
    lib.dspark_schedule_verify.argtypes = [vp, f32, i32, i32, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                           vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dspark_schedule_verify.restype = i32
    lib.dspark_verify_phase.argtypes = [i32] + lib.dspark_verify.argtypes
    lib.dspark_verify_phase.restype = i32
    lib.dspark_verify_greedy_phase.argtypes = [i32] + lib.dspark_verify_greedy.argtypes
    lib.dspark_verify_greedy_phase.restype = i32
    lib.dspark_schedule_verify_phase.argtypes = [i32] + lib.dspark_schedule_verify.argtypes
    lib.dspark_schedule_verify_phase.restype = i32
    lib.dspark_schedule_verify_noalloc.argtypes = lib.dspark_schedule_verify.argtypes[:-3] + [vp]
    lib.dspark_schedule_verify_noalloc.restype = i32
    _lib = lib
    return lib


def dspark_status_string(status: int) -> str:
    return load_library().dspark_status_string(int(status)).decode()


def dspark_workspace_bytes(op: int, B: int, K: int, V: int) -> int:
    return int(load_library().dspark_workspace_bytes(int(op), int(B), int(K), int(V)))


def _check(status: int):
    if status != DSPARK_OK:
        raise DsparkError(status, dspark_status_string(status))


# ---------------------------------------------------------------- torch glue

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _req(t, name, dtype, shape, device):
    torch = _torch()
    if t.device != device or t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)} on {device}, got "
                         f"{t.dtype} {tuple(t.shape)} on {t.device} contiguous={t.is_contiguous()}")
    return t


_ws_cache = {}


class Workspace:
    """Caller-owned workspace: a device byte buffer aligned to 256 bytes."""

    def __init__(self, nbytes: int, device):
        torch = _torch()
        self.buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        self.ptr = (self.buf.data_ptr() + 255) // 256 * 256
        self.nbytes = nbytes


def workspace(op: int, B: int, K: int, V: int, device, stream=None) -> Workspace:
    """Cached workspace for (device, op, B, K, V) and one stream (``None``: the
    device's current stream).  Calls that may run at the same time need
    distinct workspaces, so calls on different streams never share one."""
    torch = _torch()
    device = torch.device(device)
    if stream is None:
        stream = torch.cuda.current_stream(device)
    key = (device.index, op, B, K, V, int(stream.cuda_stream))
    ws = _ws_cache.get(key)
    if ws is None:
        nbytes = dspark_workspace_bytes(op, B, K, V)
        if nbytes == 0:
            raise DsparkError(2, "bad sizes for the workspace query")
        ws = Workspace(nbytes, device)
        _ws_cache[key] = ws
    return ws


def _stream(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _status(dev_status, dev):
    """The caller's device-status word (int32[1] on the device) or a new
    zeroed one."""
    torch = _torch()
    if dev_status is None:
        return torch.zeros(1, dtype=torch.int32, device=dev)
    return _req(dev_status, "dev_status", torch.int32, (1,), dev)


def _out(t, name, dtype, shape, dev):
    """A caller-supplied output checked against what the kernels write, or a
    new one."""
    torch = _torch()
    if t is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    return _req(t, name, dtype, shape, dev)


def _ws(ws, op, B, K, V, dev, stream):
    """The caller's workspace, checked against the size the call needs, or the
    cached one of this stream."""
    if ws is None:
        return workspace(op, B, K, V, dev, stream)
    need = dspark_workspace_bytes(op, B, K, V)
    if ws.nbytes < need:
        raise ValueError(f"workspace of {ws.nbytes} bytes, the call needs {need}")
    return ws


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return DSPARK_BF16
    if t.dtype == torch.float32:
        return DSPARK_F32
    raise ValueError(f"logits dtype {t.dtype} not supported (bf16 or fp32)")


def schedule(conf, threshold: float, budget: int, min_len: int = 1, *, lengths=None, mask=None,
             survival=None, dev_status=None, ws: Optional[Workspace] = None, stream=None):
    """dspark_schedule on torch tensors.  Returns (lengths, mask, survival, dev_status)."""
    torch = _torch()
    lib = load_library()
    dev = conf.device
    B, K = conf.shape
    _req(conf, "conf", torch.float32, (B, K), dev)
    lengths = _out(lengths, "lengths", torch.int32, (B,), dev)
    mask = _out(mask, "mask", torch.uint8, (B, K), dev)
    survival = _out(survival, "survival", torch.float32, (B, K), dev)
    dev_status = _status(dev_status, dev)
    ws = _ws(ws, OP_SCHEDULE, B, K, 1, dev, stream)
    st = lib.dspark_schedule(_ptr(conf), B, K, float(threshold), int(budget), int(min_len),
                             _ptr(lengths), _ptr(mask), _ptr(survival), _ptr(dev_status),
                             ws.ptr, ws.nbytes, _stream(stream, dev))
    _check(st)
    return lengths, mask, survival, dev_status


def schedule_load_aware(conf, load, q_max: float, m_max: float, tau_min: float, tau_max: float,
                        curve, slot_cost: float, min_len: int = 1, *, lengths=None, mask=None,
                        survival=None, tau_out=None, budget_out=None, dev_status=None,
                        ws: Optional[Workspace] = None, stream=None):
    """dspark_schedule_load_aware on torch tensors (``load`` float32[2] and
    ``curve`` float32[n, 2] on the device; ``curve=None`` for no budget).
    Returns (lengths, mask, survival, tau_out, budget_out, dev_status)."""
    torch = _torch()
    lib = load_library()
    dev = conf.device
    B, K = conf.shape
    _req(conf, "conf", torch.float32, (B, K), dev)
    _req(load, "load", torch.float32, (2,), dev)
    n_curve = 0
    if curve is not None:
        n_curve = curve.shape[0]
        _req(curve, "curve", torch.float32, (n_curve, 2), dev)
    lengths = _out(lengths, "lengths", torch.int32, (B,), dev)
    mask = _out(mask, "mask", torch.uint8, (B, K), dev)
    survival = _out(survival, "survival", torch.float32, (B, K), dev)
    tau_out = _out(tau_out, "tau_out", torch.float32, (1,), dev)
    budget_out = _out(budget_out, "budget_out", torch.int32, (1,), dev)
    dev_status = _status(dev_status, dev)
    ws = _ws(ws, OP_SCHEDULE, B, K, 1, dev, stream)
    st = lib.dspark_schedule_load_aware(
        _ptr(conf), B, K, _ptr(load), float(q_max), float(m_max), float(tau_min), float(tau_max),
        _ptr(curve) if curve is not None else None, n_curve, float(slot_cost), int(min_len),
        _ptr(lengths), _ptr(mask), _ptr(survival), _ptr(tau_out), _ptr(budget_out),
        _ptr(dev_status), ws.ptr, ws.nbytes, _stream(stream, dev))
    _check(st)
    return lengths, mask, survival, tau_out, budget_out, dev_status


def calibrate(raw, theta, *, out=None, dev_status=None, stream=None):
    """dspark_calibrate on torch tensors.  Returns (calibrated, dev_status)."""
    torch = _torch()
    lib = load_library()
    dev = raw.device
    B, K = raw.shape
    _req(raw, "raw", torch.float32, (B, K), dev)
    _req(theta, "theta", torch.float32, (K,), dev)
    out = _out(out, "out", torch.float32, (B, K), dev)
    dev_status = _status(dev_status, dev)
    _check(lib.dspark_calibrate(_ptr(raw), _ptr(theta), B, K, _ptr(out), _ptr(dev_status),
                                _stream(stream, dev)))
    return out, dev_status


def calib_state(K: int, n_bins: int, device):
    """Zero-filled calibration window state (dspark_calib_state_bytes)."""
    torch = _torch()
    nbytes = load_library().dspark_calib_state_bytes(int(K), int(n_bins))
    if nbytes == 0:
        raise DsparkError(2, "bad sizes for the calibration state")
    return torch.zeros(nbytes // 8, dtype=torch.int64, device=device)


def calib_observe(calibrated, lengths, accepted, theta, lr: float, theta_min: float, window: int,
                  n_bins: int, state, *, ece_out=None, dev_status=None, stream=None):
    """dspark_calib_observe on torch tensors (``theta`` is updated in place at
    each window's end).  Returns (ece_out, dev_status)."""
    torch = _torch()
    lib = load_library()
    dev = calibrated.device
    B, K = calibrated.shape
    _req(calibrated, "calibrated", torch.float32, (B, K), dev)
    if lengths is not None:
        _req(lengths, "lengths", torch.int32, (B,), dev)
    _req(accepted, "accepted", torch.int32, (B,), dev)
    _req(theta, "theta", torch.float32, (K,), dev)
    if state.device != dev or not state.is_contiguous():
        raise ValueError("state: expected a contiguous tensor on the same device")
    ece_out = torch.zeros(1, dtype=torch.float32, device=dev) if ece_out is None else \
        _req(ece_out, "ece_out", torch.float32, (1,), dev)
    dev_status = _status(dev_status, dev)
    _check(lib.dspark_calib_observe(_ptr(calibrated), _ptr(lengths), _ptr(accepted), B, K,
                                    _ptr(theta), float(lr), float(theta_min), int(window),
                                    int(n_bins), _ptr(state), state.numel() * state.element_size(),
                                    _ptr(ece_out), _ptr(dev_status), _stream(stream, dev)))
    return ece_out, dev_status


def markov_draft(base, U, Vm, scale: float, y0, temperature, uniforms, *, corrected=None,
                 drafted=None, q_tok=None, dev_status=None, ws: Optional[Workspace] = None,
                 stream=None):
    """dspark_markov_draft on torch tensors (``U``, ``Vm``: [V, r] bfloat16).
    Returns (corrected, drafted, q_tok, dev_status)."""
    torch = _torch()
    lib = load_library()
    dev = base.device
    B, K, V = base.shape
    code = _dtype_code(base)
    _req(base, "base", base.dtype, (B, K, V), dev)
    r = U.shape[1]
    _req(U, "U", torch.bfloat16, (V, r), dev)
    _req(Vm, "Vm", torch.bfloat16, (V, r), dev)
    _req(y0, "y0", torch.int32, (B,), dev)
    _req(temperature, "temperature", torch.float32, (B,), dev)
    _req(uniforms, "uniforms", torch.float32, (B, K), dev)
    corrected = _out(corrected, "corrected", base.dtype, (B, K, V), dev)
    drafted = _out(drafted, "drafted", torch.int32, (B, K), dev)
    q_tok = _out(q_tok, "q_tok", torch.float32, (B, K), dev)
    dev_status = _status(dev_status, dev)
    ws = _ws(ws, OP_MARKOV_DRAFT, B, K, V, dev, stream)
    _check(lib.dspark_markov_draft(_ptr(base), code, B, K, V, _ptr(U), _ptr(Vm), r, float(scale),
                                   _ptr(y0), _ptr(temperature), _ptr(uniforms), _ptr(corrected),
                                   _ptr(drafted), _ptr(q_tok), _ptr(dev_status), ws.ptr, ws.nbytes,
                                   _stream(stream, dev)))
    return corrected, drafted, q_tok, dev_status


def verify(target, draft, drafted, lengths, temperature, uniforms, *, accepted=None, tokens=None,
           p_tok=None, q_tok=None, dev_status=None, ws: Optional[Workspace] = None, stream=None,
           want_probs: bool = True, phases: int = PHASE_ALL):
    """dspark_verify on torch tensors (``phases`` other than PHASE_ALL:
    dspark_verify_phase).  ``lengths=None`` verifies all K.
    Returns dict(accepted, tokens, p_tok, q_tok, dev_status)."""
    torch = _torch()
    lib = load_library()
    dev = target.device
    B, K1, V = target.shape
    K = K1 - 1
    code = _dtype_code(target)
    _req(target, "target", target.dtype, (B, K + 1, V), dev)
    _req(draft, "draft", target.dtype, (B, K, V), dev)
    _req(drafted, "drafted", torch.int32, (B, K), dev)
    if lengths is not None:
        _req(lengths, "lengths", torch.int32, (B,), dev)
    _req(temperature, "temperature", torch.float32, (B,), dev)
    _req(uniforms, "uniforms", torch.float32, (B, K + 1), dev)
    accepted = _out(accepted, "accepted", torch.int32, (B,), dev)
    tokens = _out(tokens, "tokens", torch.int32, (B, K + 1), dev)
    if want_probs:
        p_tok = _out(p_tok, "p_tok", torch.float32, (B, K), dev)
        q_tok = _out(q_tok, "q_tok", torch.float32, (B, K), dev)
    else:
        p_tok = None if p_tok is None else _req(p_tok, "p_tok", torch.float32, (B, K), dev)
        q_tok = None if q_tok is None else _req(q_tok, "q_tok", torch.float32, (B, K), dev)
    dev_status = _status(dev_status, dev)
    ws = _ws(ws, OP_VERIFY, B, K, V, dev, stream)
    args = (_ptr(target), _ptr(draft), code, B, K, V, _ptr(drafted), _ptr(lengths),
            _ptr(temperature), _ptr(uniforms), _ptr(accepted), _ptr(tokens), _ptr(p_tok),
            _ptr(q_tok), _ptr(dev_status), ws.ptr, ws.nbytes, _stream(stream, dev))
    if phases == PHASE_ALL:
        _check(lib.dspark_verify(*args))
    else:
        _check(lib.dspark_verify_phase(int(phases), *args))
    return dict(accepted=accepted, tokens=tokens, p_tok=p_tok, q_tok=q_tok, dev_status=dev_status)


def schedule_verify(conf, threshold: float, budget: int, min_len: int, target, draft, drafted,
                    temperature, uniforms, *, lengths=None, mask=None, survival=None,
                    accepted=None, tokens=None, p_tok=None, q_tok=None, dev_status=None,
                    ws: Optional[Workspace] = None, stream=None, phases: int = PHASE_ALL):
    """dspark_schedule_verify on torch tensors (``phases`` other than
    PHASE_ALL: dspark_schedule_verify_phase): the schedule and the
    verification of one step in one call.  Returns dict(lengths, mask,
    survival, accepted, tokens, p_tok, q_tok, dev_status)."""
    torch = _torch()
    lib = load_library()
    dev = target.device
    B, K1, V = target.shape
    K = K1 - 1
    code = _dtype_code(target)
    _req(conf, "conf", torch.float32, (B, K), dev)
    _req(target, "target", target.dtype, (B, K + 1, V), dev)
    _req(draft, "draft", target.dtype, (B, K, V), dev)
    _req(drafted, "drafted", torch.int32, (B, K), dev)
    _req(temperature, "temperature", torch.float32, (B,), dev)
    _req(uniforms, "uniforms", torch.float32, (B, K + 1), dev)
    lengths = _out(lengths, "lengths", torch.int32, (B,), dev)
    mask = _out(mask, "mask", torch.uint8, (B, K), dev)
    survival = _out(survival, "survival", torch.float32, (B, K), dev)
    accepted = _out(accepted, "accepted", torch.int32, (B,), dev)
    tokens = _out(tokens, "tokens", torch.int32, (B, K + 1), dev)
    p_tok = _out(p_tok, "p_tok", torch.float32, (B, K), dev)
    q_tok = _out(q_tok, "q_tok", torch.float32, (B, K), dev)
    dev_status = _status(dev_status, dev)
    ws = _ws(ws, OP_SCHEDULE_VERIFY, B, K, V, dev, stream)
    args = (_ptr(conf), float(threshold), int(budget), int(min_len), _ptr(lengths), _ptr(mask),
            _ptr(survival), _ptr(target), _ptr(draft), code, B, K, V, _ptr(drafted),
            _ptr(temperature), _ptr(uniforms), _ptr(accepted), _ptr(tokens), _ptr(p_tok),
            _ptr(q_tok), _ptr(dev_status), ws.ptr, ws.nbytes, _stream(stream, dev))
    if phases == PHASE_ALL:
        _check(lib.dspark_schedule_verify(*args))
    else:
        _check(lib.dspark_schedule_verify_phase(int(phases), *args))
    return dict(lengths=lengths, mask=mask, survival=survival, accepted=accepted, tokens=tokens,
                p_tok=p_tok, q_tok=q_tok, dev_status=dev_status)


def schedule_verify_noalloc(conf, threshold: float, budget: int, min_len: int, target, draft,
                            drafted, temperature, uniforms, *, lengths=None, mask=None,
                            survival=None, accepted=None, tokens=None, p_tok=None, q_tok=None,
                            dev_status=None, stream=None):
    """dspark_schedule_verify_noalloc on torch tensors: the same step with the
    library's built-in device scratch instead of a workspace (outputs left to
    None are allocated here; pass them all for a call that allocates
    nothing).  Returns dict(lengths, mask, survival, accepted, tokens, p_tok,
    q_tok, dev_status)."""
    torch = _torch()
    lib = load_library()
    dev = target.device
    B, K1, V = target.shape
    K = K1 - 1
    code = _dtype_code(target)
    _req(conf, "conf", torch.float32, (B, K), dev)
    _req(target, "target", target.dtype, (B, K + 1, V), dev)
    _req(draft, "draft", target.dtype, (B, K, V), dev)
    _req(drafted, "drafted", torch.int32, (B, K), dev)
    _req(temperature, "temperature", torch.float32, (B,), dev)
    _req(uniforms, "uniforms", torch.float32, (B, K + 1), dev)
    lengths = _out(lengths, "lengths", torch.int32, (B,), dev)
    mask = _out(mask, "mask", torch.uint8, (B, K), dev)
    survival = _out(survival, "survival", torch.float32, (B, K), dev)
    accepted = _out(accepted, "accepted", torch.int32, (B,), dev)
    tokens = _out(tokens, "tokens", torch.int32, (B, K + 1), dev)
    p_tok = _out(p_tok, "p_tok", torch.float32, (B, K), dev)
    q_tok = _out(q_tok, "q_tok", torch.float32, (B, K), dev)
    dev_status = _status(dev_status, dev)
    _check(lib.dspark_schedule_verify_noalloc(
        _ptr(conf), float(threshold), int(budget), int(min_len), _ptr(lengths), _ptr(mask),
        _ptr(survival), _ptr(target), _ptr(draft), code, B, K, V, _ptr(drafted),
        _ptr(temperature), _ptr(uniforms), _ptr(accepted), _ptr(tokens), _ptr(p_tok),
        _ptr(q_tok), _ptr(dev_status), _stream(stream, dev)))
    return dict(lengths=lengths, mask=mask, survival=survival, accepted=accepted, tokens=tokens,
                p_tok=p_tok, q_tok=q_tok, dev_status=dev_status)


def verify_greedy(target, drafted, lengths, *, accepted=None, tokens=None, dev_status=None,
                  ws: Optional[Workspace] = None, stream=None, phases: int = PHASE_ALL):
    """dspark_verify_greedy on torch tensors (``phases`` other than PHASE_ALL:
    dspark_verify_greedy_phase).  Returns dict(accepted, tokens, dev_status)."""
    torch = _torch()
    lib = load_library()
    dev = target.device
    B, K1, V = target.shape
    K = K1 - 1
    code = _dtype_code(target)
    _req(target, "target", target.dtype, (B, K + 1, V), dev)
    _req(drafted, "drafted", torch.int32, (B, K), dev)
    if lengths is not None:
        _req(lengths, "lengths", torch.int32, (B,), dev)
    accepted = _out(accepted, "accepted", torch.int32, (B,), dev)
    tokens = _out(tokens, "tokens", torch.int32, (B, K + 1), dev)
    dev_status = _status(dev_status, dev)
    ws = _ws(ws, OP_VERIFY_GREEDY, B, K, V, dev, stream)
    args = (_ptr(target), code, B, K, V, _ptr(drafted), _ptr(lengths), _ptr(accepted),
            _ptr(tokens), _ptr(dev_status), ws.ptr, ws.nbytes, _stream(stream, dev))
    if phases == PHASE_ALL:
        _check(lib.dspark_verify_greedy(*args))
    else:
        _check(lib.dspark_verify_greedy_phase(int(phases), *args))
    return dict(accepted=accepted, tokens=tokens, dev_status=dev_status)
