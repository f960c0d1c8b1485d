"""ctypes binding of libmsgla.so (include/msgla.h) — argument marshalling only.

Every function has the name of the C entry point it calls.  Device buffers
are torch tensors on a ROCm device (torch supplies the memory and the stream;
all computation happens in the library's HIP kernels).  A non-OK status
raises MsglaError.  Loading fails loudly when the library has not been built;
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

from .config import BF16, F32, MsglaConfig

MAX_BRANCHES = 8
N_STAGES = 6
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmsgla.so")

STATUS = {0: "MSGLA_OK", 1: "MSGLA_ERR_INVALID_ARG", 2: "MSGLA_ERR_UNSUPPORTED",
          3: "MSGLA_ERR_WORKSPACE", 4: "MSGLA_ERR_HIP"}

# exported symbols declared by include/msgla.h
SYMBOLS = (
    "msgla_status_str", "msgla_validate_config", "msgla_packed_weights_bytes",
    "msgla_pack_weights", "msgla_workspace_bytes", "msgla_state_bytes", "msgla_state_init",
    "msgla_forward", "msgla_forward_timed", "msgla_decode_workspace_bytes", "msgla_decode_step",
    "msgla_fusion_weights", "msgla_state_query", "msgla_forward_noalloc",
    "msgla_backward_workspace_bytes", "msgla_backward", "msgla_forward_train", "msgla_backward_saved",
)
NOALLOC_WORKSPACE_BYTES = 192 << 20  # MSGLA_NOALLOC_WORKSPACE_BYTES


class MsglaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


class CConfig(ctypes.Structure):
    _fields_ = [
        ("n_branches", ctypes.c_int32),
        ("scale", ctypes.c_int32 * MAX_BRANCHES),
        ("heads", ctypes.c_int32 * MAX_BRANCHES),
        ("d_model", ctypes.c_int32),
        ("d_k", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("gate_rank", ctypes.c_int32),
        ("chunk", ctypes.c_int32),
        ("gate_normalizer", ctypes.c_float),
        ("q_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("norm", ctypes.c_int32),
    ]


class CBranchWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("W_q", "W_k", "W_v", "W_g1", "W_g2", "b_g", "W_o",
                                               "norm_g")]


class CWeights(ctypes.Structure):
    _fields_ = [("br", CBranchWeights * MAX_BRANCHES), ("W_f", ctypes.c_void_p),
                ("b_f", ctypes.c_void_p)]


class CBranchGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("W_q", "W_k", "W_v", "W_g1", "W_g2", "b_g", "W_o",
                                               "norm_g")]


class CGrads(ctypes.Structure):
    _fields_ = [("br", CBranchGrads * MAX_BRANCHES), ("W_f", ctypes.c_void_p),
                ("b_f", ctypes.c_void_p)]


class CStateInfo(ctypes.Structure):
    _fields_ = [("status", ctypes.c_int32), ("B", ctypes.c_int32), ("m", ctypes.c_int32),
                ("position", ctypes.c_int64)]


class CStageEvents(ctypes.Structure):
    _fields_ = [("start", ctypes.c_void_p * N_STAGES), ("stop", ctypes.c_void_p * N_STAGES)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmsgla.so; raises if it is missing (build it with scale_gla_layer_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run `python -m scale_gla_layer_amd.build` first "
                           "(the MS-GLA layer has no non-HIP implementation)")
    lib = ctypes.CDLL(path)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    cfgp = ctypes.POINTER(CConfig)
    sig = {
        "msgla_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "msgla_validate_config": (ctypes.c_int, [cfgp]),
        "msgla_packed_weights_bytes": (sz, [cfgp]),
        "msgla_pack_weights": (ctypes.c_int, [cfgp, ctypes.POINTER(CWeights), vp, sz, vp]),
        "msgla_workspace_bytes": (sz, [cfgp, i64, i64]),
        "msgla_state_bytes": (sz, [cfgp, i64]),
        "msgla_state_init": (ctypes.c_int, [cfgp, i64, vp, sz, vp]),
        "msgla_forward": (ctypes.c_int, [cfgp, vp, vp, vp, i64, i64, vp, vp, vp, vp, sz, vp]),
        "msgla_forward_timed": (ctypes.c_int, [cfgp, vp, vp, vp, i64, i64, vp, vp, vp, vp, sz, vp,
                                               ctypes.POINTER(CStageEvents)]),
        "msgla_decode_workspace_bytes": (sz, [cfgp, i64]),
        "msgla_decode_step": (ctypes.c_int, [cfgp, vp, vp, i64, vp, vp, vp, sz, vp]),
        "msgla_fusion_weights": (ctypes.c_int, [cfgp, vp, vp, i64, i64, vp, vp]),
        "msgla_state_query": (ctypes.c_int, [vp, ctypes.POINTER(CStateInfo), vp]),
        "msgla_forward_noalloc": (ctypes.c_int, [cfgp, vp, vp, vp, i64, i64, vp, vp, vp, vp]),
        "msgla_backward_workspace_bytes": (sz, [cfgp, i64, i64]),
        "msgla_backward": (ctypes.c_int, [cfgp, vp, vp, vp, vp, i64, i64, vp, ctypes.POINTER(CGrads),
                                          vp, sz, vp]),
        "msgla_backward_saved": (ctypes.c_int, [cfgp, vp, vp, vp, vp, i64, i64, vp, ctypes.POINTER(CGrads),
                                                vp, sz, vp]),
        "msgla_forward_train": (ctypes.c_int, [cfgp, vp, vp, vp, i64, i64, vp, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


_CFG_CACHE: dict = {}


def c_config(cfg: MsglaConfig) -> CConfig:
    """The C struct of a configuration (built once per distinct configuration)."""
    c = _CFG_CACHE.get(cfg)
    if c is None:
        c = _CFG_CACHE[cfg] = _build_config(cfg)
    return c


def _build_config(cfg: MsglaConfig) -> CConfig:
    c = CConfig()
    c.n_branches = len(cfg.scales)
    for i, (s, h) in enumerate(zip(cfg.scales, cfg.heads)):
        if i >= MAX_BRANCHES:
            break
        c.scale[i] = s
        c.heads[i] = h
    c.d_model, c.d_k, c.d_v = cfg.d_model, cfg.d_k, cfg.d_v
    c.gate_rank, c.chunk = cfg.gate_rank, cfg.chunk
    c.gate_normalizer, c.q_scale = cfg.gate_normalizer, cfg.q_scale
    c.dtype = 1 if cfg.dtype == BF16 else 0
    c.norm = 1 if cfg.norm else 0
    return c


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(fn: str, st: int):
    if st != 0:
        raise MsglaError(fn, st)


def msgla_validate_config(cfg: MsglaConfig) -> int:
    return load_library().msgla_validate_config(ctypes.byref(c_config(cfg)))


def msgla_packed_weights_bytes(cfg: MsglaConfig) -> int:
    return load_library().msgla_packed_weights_bytes(ctypes.byref(c_config(cfg)))


def msgla_workspace_bytes(cfg: MsglaConfig, B: int, L: int) -> int:
    return load_library().msgla_workspace_bytes(ctypes.byref(c_config(cfg)), B, L)


def msgla_state_bytes(cfg: MsglaConfig, B: int) -> int:
    return load_library().msgla_state_bytes(ctypes.byref(c_config(cfg)), B)


def msgla_decode_workspace_bytes(cfg: MsglaConfig, B: int) -> int:
    return load_library().msgla_decode_workspace_bytes(ctypes.byref(c_config(cfg)), B)


def msgla_pack_weights(cfg: MsglaConfig, branches: Sequence[dict], W_f, b_f, packed, stream=None):
    """branches: per branch a dict of device tensors W_q, W_k, W_v, W_g1, W_g2, b_g, W_o
    and, for configurations with the normalisation, norm_g."""
    w = CWeights()
    for i, br in enumerate(branches):
        for name in ("W_q", "W_k", "W_v", "W_g1", "W_g2", "b_g", "W_o", "norm_g"):
            setattr(w.br[i], name, _ptr(br.get(name)))
    w.W_f, w.b_f = _ptr(W_f), _ptr(b_f)
    st = load_library().msgla_pack_weights(ctypes.byref(c_config(cfg)), ctypes.byref(w),
                                           _ptr(packed), packed.numel() * packed.element_size(),
                                           _stream(stream))
    _check("msgla_pack_weights", st)


def msgla_state_init(cfg: MsglaConfig, B: int, state, stream=None):
    st = load_library().msgla_state_init(ctypes.byref(c_config(cfg)), B, _ptr(state),
                                         state.numel() * state.element_size(), _stream(stream))
    _check("msgla_state_init", st)


def msgla_forward(cfg: MsglaConfig, packed, x, B: int, L: int, out, workspace,
                  state_out=None, mask=None, state_in=None, stream=None, events=None):
    """events: optional (start[N_STAGES], stop[N_STAGES]) lists of torch.cuda.Event (or None entries)."""
    lib = load_library()
    args = (ctypes.byref(c_config(cfg)), _ptr(packed), _ptr(x), _ptr(mask), B, L, _ptr(out),
            _ptr(state_in), _ptr(state_out), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    if events is None:
        st = lib.msgla_forward(*args)
        _check("msgla_forward", st)
        return
    ev = CStageEvents()
    for i in range(N_STAGES):
        for slot, lst in ((ev.start, events[0]), (ev.stop, events[1])):
            e = lst[i]
            slot[i] = None if e is None else e.cuda_event
    st = lib.msgla_forward_timed(*args, ctypes.byref(ev))
    _check("msgla_forward_timed", st)


def msgla_decode_step(cfg: MsglaConfig, packed, x_t, B: int, state, out_t, workspace, stream=None):
    st = load_library().msgla_decode_step(ctypes.byref(c_config(cfg)), _ptr(packed), _ptr(x_t), B,
                                          _ptr(state), _ptr(out_t), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(),
                                          _stream(stream))
    _check("msgla_decode_step", st)


def msgla_fusion_weights(cfg: MsglaConfig, packed, x, B: int, L: int, w_out, stream=None):
    st = load_library().msgla_fusion_weights(ctypes.byref(c_config(cfg)), _ptr(packed), _ptr(x), B, L,
                                             _ptr(w_out), _stream(stream))
    _check("msgla_fusion_weights", st)


def msgla_backward_workspace_bytes(cfg: MsglaConfig, B: int, L: int) -> int:
    return load_library().msgla_backward_workspace_bytes(ctypes.byref(c_config(cfg)), B, L)


def msgla_backward(cfg: MsglaConfig, packed, x, dout, B: int, L: int, dx, branch_grads: Sequence[dict],
                   W_f, b_f, workspace, mask=None, stream=None, saved=False):
    """branch_grads: per branch a dict of fp32 device tensors W_q, W_k, W_v, W_g1, W_g2, b_g, W_o
    and, for configurations with the normalisation, norm_g (written, in the layout of the
    weights); W_f, b_f: fp32 device tensors (None when m == 1);
    mask: the forward's [B, L] uint8 token mask, or None;
    saved: msgla_backward_saved (the workspace holds msgla_forward_train's intermediates)."""
    g = CGrads()
    for i, br in enumerate(branch_grads):
        for name in ("W_q", "W_k", "W_v", "W_g1", "W_g2", "b_g", "W_o", "norm_g"):
            setattr(g.br[i], name, _ptr(br.get(name)))
    g.W_f, g.b_f = _ptr(W_f), _ptr(b_f)
    name = "msgla_backward_saved" if saved else "msgla_backward"
    st = getattr(load_library(), name)(ctypes.byref(c_config(cfg)), _ptr(packed), _ptr(x), _ptr(dout),
                                       _ptr(mask), B, L, _ptr(dx), ctypes.byref(g), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(stream))
    _check(name, st)


def msgla_forward_train(cfg: MsglaConfig, packed, x, B: int, L: int, out, workspace, mask=None, stream=None):
    """The training forward: out as msgla_forward, the backward's intermediates kept in
    workspace (at least msgla_backward_workspace_bytes)."""
    st = load_library().msgla_forward_train(ctypes.byref(c_config(cfg)), _ptr(packed), _ptr(x), _ptr(mask), B, L,
                                            _ptr(out), _ptr(workspace),
                                            workspace.numel() * workspace.element_size(), _stream(stream))
    _check("msgla_forward_train", st)


def msgla_state_query(state, stream=None) -> dict:
    """The state's header: {"status", "B", "m", "position"} (waits for the stream)."""
    info = CStateInfo()
    st = load_library().msgla_state_query(_ptr(state), ctypes.byref(info), _stream(stream))
    _check("msgla_state_query", st)
    return {"status": int(info.status), "B": int(info.B), "m": int(info.m),
            "position": int(info.position)}


def msgla_forward_noalloc(cfg: MsglaConfig, packed, x, B: int, L: int, out, state_out=None,
                          state_in=None, mask=None, stream=None):
    """The forward with the library's own per-device workspace (no allocation)."""
    st = load_library().msgla_forward_noalloc(ctypes.byref(c_config(cfg)), _ptr(packed), _ptr(x),
                                              _ptr(mask), B, L, _ptr(out), _ptr(state_in),
                                              _ptr(state_out), _stream(stream))
    _check("msgla_forward_noalloc", st)
