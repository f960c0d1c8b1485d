"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/msgla.h declares, and validates its arguments
before enqueueing anything."""
import ctypes
import os
import re

import pytest

from scale_gla_layer_amd import binding
from scale_gla_layer_amd.config import MsglaConfig, F32, BF16, WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    with open(os.path.join(ROOT, "include", "msgla.h"), encoding="utf-8") as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(msgla_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = binding.load_library()
    declared = _declared_symbols()
    assert declared, "no declarations found"
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(binding.SYMBOLS)


def test_status_strings():
    lib = binding.load_library()
    for code in range(5):
        assert lib.msgla_status_str(code)
    assert lib.msgla_status_str(99) == b"unknown status"


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_workload_configs_are_valid(name):
    wl = WORKLOADS[name]
    assert binding.msgla_validate_config(wl.cfg) == 0
    assert binding.msgla_packed_weights_bytes(wl.cfg) > 0
    assert binding.msgla_workspace_bytes(wl.cfg, wl.batch, wl.seq_len) > 0


def test_state_bytes_hold_the_recurrent_budget():
    """Per sequence the blob holds sum_s h_s d_k d_v fp32 state elements (131,072 at d=1024, H=4)."""
    cfg = WORKLOADS["main"].cfg
    for B in (1, 3, 16):
        n = binding.msgla_state_bytes(cfg, B)
        assert n >= 4 * B * 131072
        assert n - 4 * B * 131072 < 4 * B * 3 * 2 * cfg.d_model + 4096


def _cfg(**kw):
    base = dict(scales=(1, 2, 4), heads=(2, 1, 1), d_model=128, d_k=32, d_v=64, gate_rank=16,
                chunk=64, gate_normalizer=16.0, q_scale=1.0, dtype=BF16)
    base.update(kw)
    return base


def _raw_cfg(**kw):
    c = _cfg(**kw)
    cc = binding.CConfig()
    cc.n_branches = len(c["scales"])
    for i, (s, h) in enumerate(zip(c["scales"], c["heads"])):
        cc.scale[i], cc.heads[i] = s, h
    cc.d_model, cc.d_k, cc.d_v = c["d_model"], c["d_k"], c["d_v"]
    cc.gate_rank, cc.chunk = c["gate_rank"], c["chunk"]
    cc.gate_normalizer, cc.q_scale = c["gate_normalizer"], c["q_scale"]
    cc.dtype = 1 if c["dtype"] == BF16 else 0
    return cc


@pytest.mark.parametrize("bad", [
    dict(scales=(1, 1), heads=(1, 1)),            # duplicate scale
    dict(scales=(0, 2), heads=(1, 1)),            # non-positive scale
    dict(scales=(1, 2), heads=(1, 0)),            # non-positive heads
    dict(d_model=96),                             # not a multiple of 64
    dict(d_k=48),                                 # d_k must be a power of two
    dict(d_k=96),
    dict(d_k=16),                                 # bf16 needs d_k >= 32
    dict(d_k=512),
    dict(d_v=96),                                 # bf16 needs d_v % 64 == 0
    dict(d_v=48, dtype=F32, chunk=16),            # d_v % 32
    dict(gate_rank=0),
    dict(gate_rank=65),
    dict(chunk=16),                               # bf16 chunk must be 32 or 64
    dict(chunk=48, dtype=F32),
    dict(gate_normalizer=0.0),
])
def test_invalid_configs_are_rejected(bad):
    lib = binding.load_library()
    cc = _raw_cfg(**bad)
    assert lib.msgla_validate_config(ctypes.byref(cc)) == 1
    assert lib.msgla_packed_weights_bytes(ctypes.byref(cc)) == 0
    assert lib.msgla_workspace_bytes(ctypes.byref(cc), 1, 8) == 0


@pytest.mark.parametrize("shape,status", [
    (dict(d_k=256, chunk=64), 2),                    # state stages beyond 160 KB of LDS
    (dict(d_k=256, chunk=32), 0),
    (dict(d_k=128, chunk=64), 0),
    (dict(d_k=128, chunk=64, dtype=F32, d_v=64), 2),
    (dict(d_k=128, chunk=32, dtype=F32, d_v=64), 0),
    (dict(d_k=256, chunk=32, dtype=F32, d_v=64), 2),
    (dict(d_k=256, chunk=16, dtype=F32, d_v=64), 0),
    (dict(d_k=64, chunk=64, dtype=F32, d_v=64), 0),
])
def test_state_kernel_lds_limit(shape, status):
    """Shapes the state kernel cannot stage in one CU's LDS are reported as
    unsupported by validation, not found out by a failed launch."""
    lib = binding.load_library()
    cc = _raw_cfg(**shape)
    assert lib.msgla_validate_config(ctypes.byref(cc)) == status
    assert (lib.msgla_packed_weights_bytes(ctypes.byref(cc)) == 0) == (status != 0)


def test_too_many_branches_rejected():
    lib = binding.load_library()
    cc = _raw_cfg()
    cc.n_branches = 9
    assert lib.msgla_validate_config(ctypes.byref(cc)) == 1
    cc.n_branches = 0
    assert lib.msgla_validate_config(ctypes.byref(cc)) == 1


def test_forward_argument_errors_need_no_gpu():
    """Argument errors are returned before any HIP call (fake aligned pointers)."""
    lib = binding.load_library()
    cc = _raw_cfg()
    fake = 1 << 20
    ws = lib.msgla_workspace_bytes(ctypes.byref(cc), 2, 64)
    f = lib.msgla_forward
    # NULL input
    assert f(ctypes.byref(cc), fake, None, None, 2, 64, fake, None, None, fake, ws, None) == 1
    # misaligned output
    assert f(ctypes.byref(cc), fake, fake, None, 2, 64, fake + 2, None, None, fake, ws, None) == 1
    # bad sizes
    assert f(ctypes.byref(cc), fake, fake, None, 0, 64, fake, None, None, fake, ws, None) == 1
    assert f(ctypes.byref(cc), fake, fake, None, 2, 0, fake, None, None, fake, ws, None) == 1
    # a masked call with a misaligned state_out
    assert f(ctypes.byref(cc), fake, fake, fake, 2, 64, fake, None, fake + 4, fake, ws, None) == 1
    # misaligned state_in (a valid one is read on the device: GPU tests)
    assert f(ctypes.byref(cc), fake, fake, None, 2, 64, fake, fake + 8, None, fake, ws, None) == 1
    # workspace too small
    assert f(ctypes.byref(cc), fake, fake, None, 2, 64, fake, None, None, fake, ws - 1, None) == 3
    # decode
    dws = lib.msgla_decode_workspace_bytes(ctypes.byref(cc), 2)
    d = lib.msgla_decode_step
    assert d(ctypes.byref(cc), fake, None, 2, fake, fake, fake, dws, None) == 1
    assert d(ctypes.byref(cc), fake, fake, 2, fake, fake, fake, dws - 1, None) == 3
    # normalisation flag out of range; normalisation without gains
    bad = _raw_cfg()
    bad.norm = 2
    assert lib.msgla_validate_config(ctypes.byref(bad)) == 1
    nc = _raw_cfg()
    nc.norm = 1
    wn = binding.CWeights()
    for i in range(nc.n_branches):
        for name in ("W_q", "W_k", "W_v", "W_g1", "W_g2", "b_g", "W_o"):
            setattr(wn.br[i], name, fake)
    wn.W_f = wn.b_f = fake
    assert lib.msgla_pack_weights(ctypes.byref(nc), ctypes.byref(wn), fake,
                                  lib.msgla_packed_weights_bytes(ctypes.byref(nc)), None) == 1
    assert lib.msgla_packed_weights_bytes(ctypes.byref(nc)) > lib.msgla_packed_weights_bytes(ctypes.byref(cc))
    # fusion weights: NULL output, one branch
    fw = lib.msgla_fusion_weights
    assert fw(ctypes.byref(cc), fake, fake, 2, 64, None, None) == 1
    one = _raw_cfg()
    one.n_branches = 1
    assert fw(ctypes.byref(one), fake, fake, 2, 64, fake, None) == 1
    # packing
    w = binding.CWeights()
    assert lib.msgla_pack_weights(ctypes.byref(cc), ctypes.byref(w), fake,
                                  lib.msgla_packed_weights_bytes(ctypes.byref(cc)), None) == 1
    st = lib.msgla_state_bytes(ctypes.byref(cc), 2)
    assert lib.msgla_state_init(ctypes.byref(cc), 2, fake, st - 1, None) == 3


def test_workspace_grows_with_batch_and_length():
    cfg = WORKLOADS["main"].cfg
    a = binding.msgla_workspace_bytes(cfg, 1, 2048)
    b = binding.msgla_workspace_bytes(cfg, 2, 2048)
    c = binding.msgla_workspace_bytes(cfg, 1, 4096)
    assert 0 < a < b and a < c


def test_state_query_argument_errors_need_no_gpu():
    """msgla_state_query rejects a NULL or misaligned state or a NULL result
    before touching the device."""
    lib = binding.load_library()
    info = binding.CStateInfo()
    assert lib.msgla_state_query(None, ctypes.byref(info), None) == 1
    assert lib.msgla_state_query(ctypes.c_void_p(8), ctypes.byref(info), None) == 1
    assert lib.msgla_state_query(ctypes.c_void_p(256), None, None) == 1


def test_backward_argument_errors_need_no_gpu():
    """The backward's argument errors are returned before any HIP or rocBLAS call."""
    lib = binding.load_library()
    cc = _raw_cfg()
    fake = 1 << 20
    ws = lib.msgla_backward_workspace_bytes(ctypes.byref(cc), 2, 64)
    assert ws > lib.msgla_workspace_bytes(ctypes.byref(cc), 2, 64)
    g = binding.CGrads()
    for i in range(cc.n_branches):
        for name in ("W_q", "W_k", "W_v", "W_g1", "W_g2", "b_g", "W_o"):
            setattr(g.br[i], name, fake)
    g.W_f = g.b_f = fake
    f = lib.msgla_backward
    cfgp = ctypes.byref(cc)
    gp = ctypes.byref(g)
    # NULL dout, misaligned dx, bad sizes, workspace too small
    assert f(cfgp, fake, fake, None, None, 2, 64, fake, gp, fake, ws, None) == 1
    assert f(cfgp, fake, fake, fake, None, 2, 64, fake + 4, gp, fake, ws, None) == 1
    assert f(cfgp, fake, fake, fake, None, 0, 64, fake, gp, fake, ws, None) == 1
    assert f(cfgp, fake, fake, fake, None, 2, 64, fake, gp, fake, ws - 1, None) == 3
    # a missing gradient pointer; a missing fusion gradient with several branches
    g2 = binding.CGrads()
    ctypes.memmove(ctypes.byref(g2), ctypes.byref(g), ctypes.sizeof(g))
    g2.br[1].W_o = None
    assert f(cfgp, fake, fake, fake, None, 2, 64, fake, ctypes.byref(g2), fake, ws, None) == 1
    g2.br[1].W_o = fake
    g2.b_f = None
    assert f(cfgp, fake, fake, fake, None, 2, 64, fake, ctypes.byref(g2), fake, ws, None) == 1
    # with the normalisation the gains' gradient is required
    nc = _raw_cfg()
    nc.norm = 1
    assert lib.msgla_backward_workspace_bytes(ctypes.byref(nc), 2, 64) > ws
    wsn = lib.msgla_backward_workspace_bytes(ctypes.byref(nc), 2, 64)
    assert f(ctypes.byref(nc), fake, fake, fake, None, 2, 64, fake, gp, fake, wsn, None) == 1
    # d_v not a multiple of 64 (an fp32 configuration): unsupported, no workspace size
    odd = _raw_cfg(dtype="f32", d_v=96)
    assert lib.msgla_validate_config(ctypes.byref(odd)) == 0
    assert lib.msgla_backward_workspace_bytes(ctypes.byref(odd), 2, 64) == 0
    assert f(ctypes.byref(odd), fake, fake, fake, None, 2, 64, fake, gp, fake, ws, None) == 2


def test_training_pair_argument_errors_need_no_gpu():
    """msgla_forward_train and msgla_backward_saved return their argument errors before
    any HIP or rocBLAS call: the training forward needs the backward's workspace size."""
    lib = binding.load_library()
    cc = _raw_cfg()
    cfgp = ctypes.byref(cc)
    fake = 1 << 20
    ws = lib.msgla_backward_workspace_bytes(cfgp, 2, 64)
    fwd_ws = lib.msgla_workspace_bytes(cfgp, 2, 64)
    ft = lib.msgla_forward_train
    # NULL output, bad sizes, misaligned input, the forward's (smaller) workspace size
    assert ft(cfgp, fake, fake, None, 2, 64, None, fake, ws, None) == 1
    assert ft(cfgp, fake, fake, None, 0, 64, fake, fake, ws, None) == 1
    assert ft(cfgp, fake, fake + 4, None, 2, 64, fake, fake, ws, None) == 1
    assert ft(cfgp, fake, fake, None, 2, 64, fake, fake, fwd_ws, None) == 3
    assert ft(cfgp, fake, fake, None, 2, 64, fake, fake, ws - 1, None) == 3
    odd = _raw_cfg(dtype="f32", d_v=96)
    assert ft(ctypes.byref(odd), fake, fake, None, 2, 64, fake, fake, ws, None) == 2
    g = binding.CGrads()
    for i in range(cc.n_branches):
        for name in ("W_q", "W_k", "W_v", "W_g1", "W_g2", "b_g", "W_o"):
            setattr(g.br[i], name, fake)
    g.W_f = g.b_f = fake
    bs = lib.msgla_backward_saved
    gp = ctypes.byref(g)
    assert bs(cfgp, fake, fake, None, None, 2, 64, fake, gp, fake, ws, None) == 1
    assert bs(cfgp, fake, fake, fake, None, 2, 64, fake, gp, fake, ws - 1, None) == 3
    assert bs(cfgp, fake, fake, fake, None, 2, 64, fake, None, fake, ws, None) == 1
    assert bs(ctypes.byref(odd), fake, fake, fake, None, 2, 64, fake, gp, fake, ws, None) == 2
