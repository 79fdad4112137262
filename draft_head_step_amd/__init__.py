"""DSpark drafter hot path on MI355X: thin Python binding over libdspark.so.

The binding only marshals arguments: it checks tensor dtypes, devices and
shapes, allocates outputs and workspaces with PyTorch (device memory is all
PyTorch is used for), and calls the C ABI declared in include/dspark.h on the
current HIP stream.  Every step of the computation runs in the library's HIP
kernels.  If the library is missing or fails to load, every entry point
raises: there is no fallback path.

Entry points (same names as the C ABI):
  dspark_markov_draft, dspark_confidence, dspark_survival, dspark_schedule,
  dspark_schedule_ex, dspark_verify_pack, dspark_verify_greedy, dspark_accept_prob,
  dspark_markov_draft_workspace, dspark_schedule_workspace, dspark_w2_store_from_rv.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

__all__ = [
    "DsparkError", "GREEDY", "SAMPLE", "LAYOUT_RGV", "LAYOUT_TILED", "lib", "lib_path",
    "dspark_markov_draft", "dspark_markov_draft_noalloc", "dspark_draft_step",
    "dspark_draft_step_workspace", "dspark_draft_step_launches", "dspark_rnn_draft",
    "dspark_rnn_draft_workspace",
    "dspark_confidence", "dspark_survival", "dspark_schedule",
    "dspark_schedule_ex", "dspark_verify_pack", "dspark_verify_greedy", "dspark_accept_prob",
    "dspark_markov_draft_workspace", "dspark_schedule_workspace", "dspark_w2_store_from_rv",
    "ScheduleInfo", "SCHED_GLOBAL", "SCHED_EARLY_STOP", "SCHED_CAPACITY",
]

GREEDY = 0
SAMPLE = 1
LAYOUT_RGV = 0     # base / uniforms / bias_out as [R, gamma, V]
LAYOUT_TILED = 1   # [gamma, ceil(V/32), 32, R]
SCHED_GLOBAL = 0       # dspark_schedule_ex admission rules
SCHED_EARLY_STOP = 1
SCHED_CAPACITY = 2
_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def lib_path() -> str:
    return os.environ.get("DSPARK_LIB", os.path.join(_PKG, "libdspark.so"))


class DsparkError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({_status_name(status)}): {detail}")
        self.status = status


class StepEvents(ctypes.Structure):
    _fields_ = [("begin", ctypes.POINTER(ctypes.c_void_p)),
                ("end", ctypes.POINTER(ctypes.c_void_p)),
                ("count", ctypes.c_int)]


class ScheduleInfo(ctypes.Structure):
    """Host mirror of dspark_schedule_info (32 bytes)."""
    _fields_ = [("B_star", ctypes.c_int32), ("m_star", ctypes.c_int32),
                ("tau_fx", ctypes.c_uint64), ("tau", ctypes.c_double), ("theta", ctypes.c_double)]


def _status_name(s: int) -> str:
    try:
        return lib().dspark_status_string(s).decode()
    except Exception:  # noqa: BLE001 - only used to format an error
        return "?"


def _tree_hash() -> Optional[str]:
    """Source hash of the tree this package sits in (None where the sources are not
    shipped next to it, e.g. an installed copy)."""
    from . import build as _build
    if not os.path.isdir(_build.CSRC):
        return None
    return _build.source_hash()


def lib() -> ctypes.CDLL:
    """Load libdspark.so once; raise if it is not built, or built from other sources."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(f"libdspark.so not found at {path}; build it with "
                          "`python -m draft_head_step_amd.build`")
    L = ctypes.CDLL(path)
    L.dspark_source_hash.argtypes = []
    L.dspark_source_hash.restype = ctypes.c_char_p
    built = L.dspark_source_hash().decode()
    want = _tree_hash()
    if want is not None and built != want:
        raise ImportError(f"{path} was built from other sources (hash {built}, tree {want}); "
                          "rebuild it with `python -m draft_head_step_amd.build`")
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.dspark_status_string.argtypes = [i32]
    L.dspark_status_string.restype = ctypes.c_char_p
    L.dspark_last_error.argtypes = []
    L.dspark_last_error.restype = ctypes.c_char_p
    L.dspark_markov_draft_workspace.argtypes = [i32, i32, i32, i32]
    L.dspark_markov_draft_workspace.restype = sz
    L.dspark_markov_draft.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, vp, vp,
                                      vp, vp, sz, ctypes.POINTER(StepEvents), vp]
    L.dspark_markov_draft.restype = i32
    L.dspark_markov_draft_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32,
                                              vp, vp, vp]
    L.dspark_markov_draft_noalloc.restype = i32
    L.dspark_draft_step_workspace.argtypes = [i32, i32, i32, i32]
    L.dspark_draft_step_workspace.restype = sz
    L.dspark_draft_step_launches.argtypes = [i32, i32, i32, i32, i32, i32, f32,
                                             ctypes.POINTER(ctypes.c_int)]
    L.dspark_draft_step_launches.restype = i32
    L.dspark_draft_step.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, vp,
                                    vp, vp, vp, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, sz,
                                    ctypes.POINTER(StepEvents), vp]
    L.dspark_draft_step.restype = i32
    L.dspark_rnn_draft_workspace.argtypes = [i32, i32, i32, i32, i32]
    L.dspark_rnn_draft_workspace.restype = sz
    L.dspark_rnn_draft.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                   f32, vp, vp, vp, vp, sz, ctypes.POINTER(StepEvents), vp]
    L.dspark_rnn_draft.restype = i32
    L.dspark_confidence.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp]
    L.dspark_confidence.restype = i32
    L.dspark_survival.argtypes = [vp, i32, i32, vp, vp]
    L.dspark_survival.restype = i32
    L.dspark_schedule_workspace.argtypes = [i32, i32]
    L.dspark_schedule_workspace.restype = sz
    L.dspark_schedule.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    L.dspark_schedule.restype = i32
    L.dspark_schedule_ex.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    L.dspark_schedule_ex.restype = i32
    L.dspark_verify_pack.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp]
    L.dspark_verify_pack.restype = i32
    L.dspark_verify_greedy.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp, vp, vp]
    L.dspark_verify_greedy.restype = i32
    L.dspark_accept_prob.argtypes = [vp, vp, i32, i32, f32, vp, vp]
    L.dspark_accept_prob.restype = i32
    L.dspark_w2_store_from_rv.argtypes = [vp, i32, i32, vp, vp]
    L.dspark_w2_store_from_rv.restype = i32
    _LIB = L
    return L


def _check(status: int, where: str) -> None:
    if status != 0:
        raise DsparkError(status, where, lib().dspark_last_error().decode())


def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _on(stream):
    """Context for the binding's own allocations (default outputs, workspaces):
    they are made on the stream the call enqueues on, so the caching allocator
    only hands their memory to later work on that stream once it is released."""
    if stream is None:
        return contextlib.nullcontext()
    return _torch().cuda.stream(stream)


def _need(t, name, dtypes, shape, device):
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _bf16_types():
    torch = _torch()
    return (torch.bfloat16, torch.int16, torch.uint16)


def dspark_markov_draft_workspace(R: int, gamma: int, V: int, r: int) -> int:
    return int(lib().dspark_markov_draft_workspace(R, gamma, V, r))


def dspark_schedule_workspace(R: int, gamma: int) -> int:
    return int(lib().dspark_schedule_workspace(R, gamma))


def dspark_markov_draft(W1, W2, base, anchors, mode: int = GREEDY, temperature: float = 1.0,
                        uniforms=None, tokens=None, bias_out=None, workspace=None,
                        events=None, stream=None, layout: int = LAYOUT_RGV, gamma=None):
    """gamma-step Markov-head draft.  W1, W2 [V, r] bf16; anchors [R] int32; base (and
    uniforms, SAMPLE only; bias_out, optional) fp32 as [R, gamma, V] (LAYOUT_RGV) or
    [gamma, ceil(V/32), 32, R] (LAYOUT_TILED).  Returns tokens [R, gamma] int32.
    ``base=None`` (GREEDY only, ``gamma`` given) drafts from the Markov bias alone.

    ``events`` is an optional pair (begin, end) of sequences of hipEvent_t handles (ints)
    that receive the start and stop of each step's fused kernel."""
    torch = _torch()
    L = lib()
    V, r = W1.shape
    R = anchors.shape[0]
    dev = W1.device
    if gamma is None:
        if base is None:
            raise ValueError("gamma must be given when base is None")
        gamma = base.shape[0] if layout == LAYOUT_TILED else base.shape[1]
    if layout == LAYOUT_TILED:
        shape = (gamma, (V + 31) // 32, 32, R)
    else:
        shape = (R, gamma, V)
    _need(W1, "W1", _bf16_types(), (V, r), dev)
    _need(W2, "W2", _bf16_types(), (V, r), dev)
    if base is not None:
        _need(base, "base", (torch.float32,), shape, dev)
    _need(anchors, "anchors", (torch.int32,), (R,), dev)
    if uniforms is not None:
        _need(uniforms, "uniforms", (torch.float32,), shape, dev)
    need = int(L.dspark_markov_draft_workspace(R, gamma, V, r))
    with _on(stream):
        if tokens is None:
            tokens = torch.empty((R, gamma), dtype=torch.int32, device=dev)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(tokens, "tokens", (torch.int32,), (R, gamma), dev)
    if bias_out is not None:
        _need(bias_out, "bias_out", (torch.float32,), shape, dev)
    ev = None
    if events is not None:
        b, e = events
        ev = StepEvents((ctypes.c_void_p * len(b))(*b), (ctypes.c_void_p * len(e))(*e),
                        min(len(b), len(e)))
    st = L.dspark_markov_draft(_ptr(W1), _ptr(W2), _ptr(base), _ptr(anchors), R, gamma, V, r,
                               int(layout), int(mode), float(temperature), _ptr(uniforms),
                               _ptr(tokens), _ptr(bias_out), _ptr(workspace), workspace.numel(),
                               ctypes.byref(ev) if ev is not None else None, _stream(stream))
    _check(st, "dspark_markov_draft")
    return tokens


def dspark_draft_step_workspace(R: int, gamma: int, V: int, r: int) -> int:
    return int(lib().dspark_draft_step_workspace(R, gamma, V, r))


def dspark_draft_step_launches(R: int, gamma: int, V: int, r: int, layout: int = LAYOUT_RGV,
                               mode: int = SAMPLE, temperature: float = 1.0) -> int:
    """Kernel launches of one dspark_draft_step call at these sizes (aligned W1
    and w_conf); planning on the host for the current device."""
    n = ctypes.c_int(0)
    _check(lib().dspark_draft_step_launches(R, gamma, V, r, int(layout), int(mode),
                                            float(temperature), ctypes.byref(n)),
           "dspark_draft_step_launches")
    return n.value


def _events(events):
    if events is None:
        return None
    b, e = events
    return StepEvents((ctypes.c_void_p * len(b))(*b), (ctypes.c_void_p * len(e))(*e),
                      min(len(b), len(e)))


def dspark_draft_step(W1, W2, base, anchors, h, w_conf, sps, mode: int = GREEDY,
                      temperature: float = 1.0, uniforms=None, sts_temp=None, tokens=None,
                      conf=None, surv=None, lengths=None, order=None, want_order: bool = False,
                      info=None, want_info: bool = False, workspace=None, events=None,
                      stream=None, layout: int = LAYOUT_RGV):
    """The whole step in one call: draft, confidence + STS + survival, schedule.
    Arguments as for dspark_markov_draft, dspark_confidence and dspark_schedule.
    Returns (tokens, conf, surv, lengths, order or None, info or None)."""
    torch = _torch()
    L = lib()
    V, r = W1.shape
    R = anchors.shape[0]
    dev = W1.device
    _, gamma, d = h.shape
    shape = (gamma, (V + 31) // 32, 32, R) if layout == LAYOUT_TILED else (R, gamma, V)
    _need(W1, "W1", _bf16_types(), (V, r), dev)
    _need(W2, "W2", _bf16_types(), (V, r), dev)
    if base is not None:
        _need(base, "base", (torch.float32,), shape, dev)
    if uniforms is not None:
        _need(uniforms, "uniforms", (torch.float32,), shape, dev)
    _need(anchors, "anchors", (torch.int32,), (R,), dev)
    _need(h, "h", _bf16_types(), (R, gamma, d), dev)
    _need(w_conf, "w_conf", (torch.float32,), (d + r,), dev)
    if sts_temp is not None:
        _need(sts_temp, "sts_temp", (torch.float32,), (gamma,), dev)
    if sps.dim() != 1 or sps.dtype != torch.float32 or sps.device != dev or not sps.is_contiguous():
        raise ValueError("sps must be a contiguous 1-D float32 tensor on the same device")
    need = int(L.dspark_draft_step_workspace(R, gamma, V, r))
    with _on(stream):
        if tokens is None:
            tokens = torch.empty((R, gamma), dtype=torch.int32, device=dev)
        if conf is None:
            conf = torch.empty((R, gamma), dtype=torch.float32, device=dev)
        if surv is None:
            surv = torch.empty((R, gamma), dtype=torch.float32, device=dev)
        if lengths is None:
            lengths = torch.empty((R,), dtype=torch.int32, device=dev)
        if order is None and want_order:
            order = torch.empty((R * gamma,), dtype=torch.int32, device=dev)
        if info is None and want_info:
            info = torch.empty((32,), dtype=torch.uint8, device=dev)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    for t, name, dt, shp in ((tokens, "tokens", torch.int32, (R, gamma)),
                             (conf, "conf", torch.float32, (R, gamma)),
                             (surv, "surv", torch.float32, (R, gamma)),
                             (lengths, "lengths", torch.int32, (R,))):
        _need(t, name, (dt,), shp, dev)
    if order is not None:
        _need(order, "order", (torch.int32,), (R * gamma,), dev)
    ev = _events(events)
    st = L.dspark_draft_step(_ptr(W1), _ptr(W2), _ptr(base), _ptr(anchors), R, gamma, V, r,
                             int(layout), int(mode), float(temperature), _ptr(uniforms), _ptr(h),
                             _ptr(w_conf), _ptr(sts_temp), d, _ptr(sps), sps.numel(),
                             _ptr(tokens), _ptr(conf), _ptr(surv), _ptr(lengths), _ptr(order),
                             _ptr(info), _ptr(workspace), workspace.numel(),
                             ctypes.byref(ev) if ev is not None else None, _stream(stream))
    _check(st, "dspark_draft_step")
    return tokens, conf, surv, lengths, order, info


def dspark_rnn_draft_workspace(R: int, gamma: int, V: int, r: int, d: int) -> int:
    return int(lib().dspark_rnn_draft_workspace(R, gamma, V, r, d))


def dspark_rnn_draft(W1, W2, U, b_rnn, base, h, anchors, mode: int = GREEDY,
                     temperature: float = 1.0, uniforms=None, tokens=None, state_out=None,
                     workspace=None, events=None, stream=None, layout: int = LAYOUT_RGV):
    """gamma-step RNN-head draft.  U [2r, 2r + d] bf16, b_rnn [2r] fp32, h [R, gamma, d]
    bf16; the other arguments as for dspark_markov_draft; state_out (optional,
    [R, r] fp32) receives the last state.  Returns tokens [R, gamma]."""
    torch = _torch()
    L = lib()
    V, r = W1.shape
    R = anchors.shape[0]
    dev = W1.device
    _, gamma, d = h.shape
    shape = (gamma, (V + 31) // 32, 32, R) if layout == LAYOUT_TILED else (R, gamma, V)
    _need(W1, "W1", _bf16_types(), (V, r), dev)
    _need(W2, "W2", _bf16_types(), (V, r), dev)
    _need(U, "U", _bf16_types(), (2 * r, 2 * r + d), dev)
    _need(b_rnn, "b_rnn", (torch.float32,), (2 * r,), dev)
    _need(h, "h", _bf16_types(), (R, gamma, d), dev)
    if base is not None:
        _need(base, "base", (torch.float32,), shape, dev)
    if uniforms is not None:
        _need(uniforms, "uniforms", (torch.float32,), shape, dev)
    _need(anchors, "anchors", (torch.int32,), (R,), dev)
    need = int(L.dspark_rnn_draft_workspace(R, gamma, V, r, d))
    with _on(stream):
        if tokens is None:
            tokens = torch.empty((R, gamma), dtype=torch.int32, device=dev)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(tokens, "tokens", (torch.int32,), (R, gamma), dev)
    if state_out is not None:
        _need(state_out, "state_out", (torch.float32,), (R, r), dev)
    ev = _events(events)
    st = L.dspark_rnn_draft(_ptr(W1), _ptr(W2), _ptr(U), _ptr(b_rnn), _ptr(base), _ptr(h),
                            _ptr(anchors), R, gamma, V, r, d, int(layout), int(mode),
                            float(temperature), _ptr(uniforms), _ptr(tokens), _ptr(state_out),
                            _ptr(workspace),
                            workspace.numel(), ctypes.byref(ev) if ev is not None else None,
                            _stream(stream))
    _check(st, "dspark_rnn_draft")
    return tokens


def dspark_markov_draft_noalloc(W1, W2, base, anchors, tokens, mode: int = GREEDY,
                                temperature: float = 1.0, uniforms=None, stream=None,
                                layout: int = LAYOUT_RGV, gamma=None):
    """dspark_markov_draft without a workspace: the library's static scratch array
    serves instead (R * gamma <= 32768).  `tokens` [R, gamma] int32 is required, so
    the call allocates nothing, here or in the library."""
    torch = _torch()
    V, r = W1.shape
    R = anchors.shape[0]
    dev = W1.device
    if gamma is None:
        if base is None:
            raise ValueError("gamma must be given when base is None")
        gamma = base.shape[0] if layout == LAYOUT_TILED else base.shape[1]
    shape = (gamma, (V + 31) // 32, 32, R) if layout == LAYOUT_TILED else (R, gamma, V)
    _need(W1, "W1", _bf16_types(), (V, r), dev)
    _need(W2, "W2", _bf16_types(), (V, r), dev)
    if base is not None:
        _need(base, "base", (torch.float32,), shape, dev)
    if uniforms is not None:
        _need(uniforms, "uniforms", (torch.float32,), shape, dev)
    _need(anchors, "anchors", (torch.int32,), (R,), dev)
    _need(tokens, "tokens", (torch.int32,), (R, gamma), dev)
    st = lib().dspark_markov_draft_noalloc(_ptr(W1), _ptr(W2), _ptr(base), _ptr(anchors), R,
                                           gamma, V, r, int(layout), int(mode),
                                           float(temperature), _ptr(uniforms), _ptr(tokens),
                                           _stream(stream))
    _check(st, "dspark_markov_draft_noalloc")
    return tokens


def dspark_confidence(h, W1, anchors, tokens, w_conf, sts_temp=None, conf=None, surv=None,
                      want_surv: bool = True, stream=None):
    """Confidence head + STS (+ survival).  Returns (conf [R, gamma] fp32, surv or None)."""
    torch = _torch()
    L = lib()
    R, gamma, d = h.shape
    V, r = W1.shape
    dev = h.device
    _need(h, "h", _bf16_types(), (R, gamma, d), dev)
    _need(W1, "W1", _bf16_types(), (V, r), dev)
    _need(anchors, "anchors", (torch.int32,), (R,), dev)
    _need(tokens, "tokens", (torch.int32,), (R, gamma), dev)
    _need(w_conf, "w_conf", (torch.float32,), (d + r,), dev)
    if sts_temp is not None:
        _need(sts_temp, "sts_temp", (torch.float32,), (gamma,), dev)
    with _on(stream):
        if conf is None:
            conf = torch.empty((R, gamma), dtype=torch.float32, device=dev)
        if surv is None and want_surv:
            surv = torch.empty((R, gamma), dtype=torch.float32, device=dev)
    _need(conf, "conf", (torch.float32,), (R, gamma), dev)
    if surv is not None:
        _need(surv, "surv", (torch.float32,), (R, gamma), dev)
    st = L.dspark_confidence(_ptr(h), _ptr(W1), _ptr(anchors), _ptr(tokens), _ptr(w_conf),
                             _ptr(sts_temp), R, gamma, d, V, r, _ptr(conf), _ptr(surv),
                             _stream(stream))
    _check(st, "dspark_confidence")
    return conf, surv


def dspark_survival(conf, surv=None, stream=None):
    torch = _torch()
    R, gamma = conf.shape
    _need(conf, "conf", (torch.float32,), (R, gamma), conf.device)
    if surv is None:
        with _on(stream):
            surv = torch.empty_like(conf)
    _need(surv, "surv", (torch.float32,), (R, gamma), conf.device)
    _check(lib().dspark_survival(_ptr(conf), R, gamma, _ptr(surv), _stream(stream)),
           "dspark_survival")
    return surv


def dspark_w2_store_from_rv(w2_rv, out=None, stream=None):
    """W2 given row by row as [r, V] bf16 -> the [V, r] storage the draft calls take."""
    torch = _torch()
    r, V = w2_rv.shape
    _need(w2_rv, "w2_rv", _bf16_types(), (r, V), w2_rv.device)
    if out is None:
        with _on(stream):
            out = torch.empty((V, r), dtype=w2_rv.dtype, device=w2_rv.device)
    _need(out, "out", _bf16_types(), (V, r), w2_rv.device)
    _check(lib().dspark_w2_store_from_rv(_ptr(w2_rv), r, V, _ptr(out), _stream(stream)),
           "dspark_w2_store_from_rv")
    return out


def dspark_schedule(surv, sps, lengths=None, order=None, want_order: bool = False, info=None,
                    want_info: bool = False, workspace=None, stream=None):
    """Prefix scheduler.  Returns (lengths [R] int32, order [R*gamma] int32 or None,
    info uint8[32] device tensor or None; decode with schedule_info())."""
    torch = _torch()
    L = lib()
    R, gamma = surv.shape
    dev = surv.device
    _need(surv, "surv", (torch.float32,), (R, gamma), dev)
    if sps.dim() != 1 or sps.dtype != torch.float32 or sps.device != dev or not sps.is_contiguous():
        raise ValueError("sps must be a contiguous 1-D float32 tensor on the same device")
    need = int(L.dspark_schedule_workspace(R, gamma))
    with _on(stream):
        if lengths is None:
            lengths = torch.empty((R,), dtype=torch.int32, device=dev)
        if order is None and want_order:
            order = torch.empty((R * gamma,), dtype=torch.int32, device=dev)
        if info is None and want_info:   # every field is written by the call
            info = torch.empty((32,), dtype=torch.uint8, device=dev)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(lengths, "lengths", (torch.int32,), (R,), dev)
    if order is not None:
        _need(order, "order", (torch.int32,), (R * gamma,), dev)
    if info is not None:
        _need(info, "info", (torch.uint8,), (32,), dev)
    st = L.dspark_schedule(_ptr(surv), _ptr(sps), R, gamma, sps.numel(), _ptr(lengths),
                           _ptr(order), _ptr(info), _ptr(workspace), workspace.numel(),
                           _stream(stream))
    _check(st, "dspark_schedule")
    return lengths, order, info


def dspark_schedule_ex(surv, sps=None, mode: int = SCHED_GLOBAL, capacity: int = 0,
                       lengths=None, order=None, want_order: bool = False, info=None,
                       want_info: bool = False, workspace=None, stream=None):
    """Prefix scheduler with a choice of admission rule (SCHED_GLOBAL,
    SCHED_EARLY_STOP, SCHED_CAPACITY with `capacity` = predicted batch tokens;
    sps may be None for SCHED_CAPACITY).  Returns (lengths, order or None, info
    or None) like dspark_schedule."""
    torch = _torch()
    L = lib()
    R, gamma = surv.shape
    dev = surv.device
    _need(surv, "surv", (torch.float32,), (R, gamma), dev)
    if sps is not None and (sps.dim() != 1 or sps.dtype != torch.float32 or sps.device != dev
                            or not sps.is_contiguous()):
        raise ValueError("sps must be a contiguous 1-D float32 tensor on the same device")
    need = int(L.dspark_schedule_workspace(R, gamma))
    with _on(stream):
        if lengths is None:
            lengths = torch.empty((R,), dtype=torch.int32, device=dev)
        if order is None and want_order:
            order = torch.empty((R * gamma,), dtype=torch.int32, device=dev)
        if info is None and want_info:   # every field is written by the call
            info = torch.empty((32,), dtype=torch.uint8, device=dev)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(lengths, "lengths", (torch.int32,), (R,), dev)
    if order is not None:
        _need(order, "order", (torch.int32,), (R * gamma,), dev)
    if info is not None:
        _need(info, "info", (torch.uint8,), (32,), dev)
    st = L.dspark_schedule_ex(_ptr(surv), _ptr(sps), R, gamma,
                              0 if sps is None else sps.numel(), int(mode), int(capacity),
                              _ptr(lengths), _ptr(order), _ptr(info), _ptr(workspace),
                              workspace.numel(), _stream(stream))
    _check(st, "dspark_schedule_ex")
    return lengths, order, info


def schedule_info(info_tensor) -> ScheduleInfo:
    """Copy a device dspark_schedule_info to the host (synchronises)."""
    raw = bytes(info_tensor.cpu().numpy().tobytes())
    return ScheduleInfo.from_buffer_copy(raw)


def dspark_verify_pack(anchors, tokens, lengths, pos0=None, flat_tokens=None, flat_pos=None,
                       flat_req=None, cu_seqlens=None, want_pos: bool = True,
                       want_req: bool = True, stream=None):
    """Flattened verification batch.  Returns (flat_tokens, flat_pos or None,
    flat_req or None, cu_seqlens); arrays have room for R * (1 + gamma) elements,
    the first cu_seqlens[R] are written."""
    torch = _torch()
    L = lib()
    R, gamma = tokens.shape
    dev = tokens.device
    _need(tokens, "tokens", (torch.int32,), (R, gamma), dev)
    _need(anchors, "anchors", (torch.int32,), (R,), dev)
    _need(lengths, "lengths", (torch.int32,), (R,), dev)
    if pos0 is not None:
        _need(pos0, "pos0", (torch.int32,), (R,), dev)
    n = R * (1 + gamma)
    with _on(stream):
        if flat_tokens is None:
            flat_tokens = torch.empty((n,), dtype=torch.int32, device=dev)
        if flat_pos is None and want_pos:
            flat_pos = torch.empty((n,), dtype=torch.int32, device=dev)
        if flat_req is None and want_req:
            flat_req = torch.empty((n,), dtype=torch.int32, device=dev)
        if cu_seqlens is None:
            cu_seqlens = torch.empty((R + 1,), dtype=torch.int32, device=dev)
    _need(flat_tokens, "flat_tokens", (torch.int32,), (n,), dev)
    for t, name in ((flat_pos, "flat_pos"), (flat_req, "flat_req")):
        if t is not None:
            _need(t, name, (torch.int32,), (n,), dev)
    _need(cu_seqlens, "cu_seqlens", (torch.int32,), (R + 1,), dev)
    _check(L.dspark_verify_pack(_ptr(anchors), _ptr(tokens), _ptr(lengths), _ptr(pos0), R, gamma,
                                _ptr(flat_tokens), _ptr(flat_pos), _ptr(flat_req),
                                _ptr(cu_seqlens), _stream(stream)), "dspark_verify_pack")
    return flat_tokens, flat_pos, flat_req, cu_seqlens


def dspark_verify_greedy(target_logits, cu_seqlens, tokens, target_argmax=None, accepted=None,
                         next_token=None, stream=None):
    """Greedy accept / correct over a flattened batch.  Returns (accepted [R],
    next_token [R], target_argmax [R*(1+gamma)])."""
    torch = _torch()
    L = lib()
    R, gamma = tokens.shape
    dev = tokens.device
    _need(tokens, "tokens", (torch.int32,), (R, gamma), dev)
    _need(cu_seqlens, "cu_seqlens", (torch.int32,), (R + 1,), dev)
    if target_logits.dim() != 2 or target_logits.dtype != torch.float32 or \
            target_logits.device != dev or not target_logits.is_contiguous():
        raise ValueError("target_logits must be a contiguous [rows, V] float32 device tensor")
    V = target_logits.shape[1]
    n = R * (1 + gamma)
    with _on(stream):
        if target_argmax is None:
            target_argmax = torch.empty((n,), dtype=torch.int32, device=dev)
        if accepted is None:
            accepted = torch.empty((R,), dtype=torch.int32, device=dev)
        if next_token is None:
            next_token = torch.empty((R,), dtype=torch.int32, device=dev)
    _need(target_argmax, "target_argmax", (torch.int32,), (n,), dev)
    _need(accepted, "accepted", (torch.int32,), (R,), dev)
    _need(next_token, "next_token", (torch.int32,), (R,), dev)
    _check(L.dspark_verify_greedy(_ptr(target_logits), _ptr(cu_seqlens), _ptr(tokens), R, gamma,
                                  V, _ptr(target_argmax), _ptr(accepted), _ptr(next_token),
                                  _stream(stream)), "dspark_verify_greedy")
    return accepted, next_token, target_argmax


def dspark_accept_prob(draft_logits, target_logits, temperature: float = 1.0, out=None,
                       stream=None):
    """sum_v min(softmax(draft/T), softmax(target/T)) per row of two [n, V] tensors."""
    torch = _torch()
    L = lib()
    for t, name in ((draft_logits, "draft_logits"), (target_logits, "target_logits")):
        if t.dim() != 2 or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [n, V] float32 tensor")
    if draft_logits.shape != target_logits.shape or draft_logits.device != target_logits.device:
        raise ValueError("draft_logits and target_logits must match in shape and device")
    n, V = draft_logits.shape
    if out is None:
        with _on(stream):
            out = torch.empty((n,), dtype=torch.float32, device=draft_logits.device)
    _need(out, "out", (torch.float32,), (n,), draft_logits.device)
    _check(L.dspark_accept_prob(_ptr(draft_logits), _ptr(target_logits), n, V,
                                float(temperature), _ptr(out), _stream(stream)),
           "dspark_accept_prob")
    return out
