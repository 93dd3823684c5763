"""fp64 CPU oracle for the gated delta-rule decode step (test infrastructure).

Only tests/, the smoke check in __graft_entry__.py and the cpu_baseline leg of
bench.py may import this package. It wraps oracle/liboracle.so (plain C, fp64
scalar loops, see ssm_oracle.c for the citations of each function) through
ctypes, and shares nothing with the HIP library.

Inputs are decoded to float64 here (bf16/f16/f32 -> fp64 is exact); states are
float64 arrays the caller keeps across chained steps, so a chained run follows
the exact-arithmetic trajectory rather than the GPU's fp32 one.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

FMT_F32, FMT_BF16, FMT_F16, FMT_NONE = 0, 1, 2, 3
ACT_SILU, ACT_SIGMOID = 0, 1

_LIB = None
_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)
_i, _d, _l = ctypes.c_int, ctypes.c_double, ctypes.c_long


def configure(L: ctypes.CDLL) -> ctypes.CDLL:
    """Declare the C signatures of an oracle library handle."""
    L.orc_softplus.argtypes = [_d]
    L.orc_sigmoid.argtypes = [_d]
    L.orc_silu.argtypes = [_d]
    L.orc_round_fmt.argtypes = [_d, _i]
    L.orc_kda_gate.argtypes = [_d, _d]
    for f in ("orc_softplus", "orc_sigmoid", "orc_silu", "orc_round_fmt", "orc_kda_gate"):
        getattr(L, f).restype = _d
    L.orc_gdn_gates.argtypes = [_d, _d, _d, _d, _dp, _dp]
    L.orc_gdn_gates.restype = None
    gdn = [_i] * 6 + [_dp, _l, _dp, _dp, _dp, _dp, _dp, _ip, _dp, _d, _i, _d, _dp, _dp, _d, _i]
    L.orc_gdn_step.argtypes = gdn + [_i]
    L.orc_gdn_step_buffered.argtypes = gdn + [_dp, _dp, _dp, _ip, _i, _i]
    L.orc_conv1d_update.argtypes = [_i] * 4 + [_dp, _dp, _dp, _dp, _ip, _i, _dp, _i]
    L.orc_kda_step.argtypes = [_i] * 4 + [_dp, _dp, _dp, _d, _dp, _ip, _dp,
                                          _dp, _dp, _d, _d, _i, _d]
    L.orc_kda_decode.argtypes = [_i] * 5 + [_dp, _dp, _dp, _dp, _dp, _dp, _d,
                                            _dp, _ip, _dp, _dp, _dp, _d, _d, _i, _d, _dp]
    L.orc_mamba_step.argtypes = [_i] * 4 + [_dp] * 8 + [_ip, _dp]
    L.orc_gdn_multi.argtypes = [_i] * 7 + [_dp, ctypes.c_long] + [_dp] * 5 + [_ip, _ip, _dp, _d, _i, _d, _dp, _dp,
                                                                        _d, _i]
    L.orc_mamba_scan.argtypes = [_i] * 5 + [_dp] * 8 + [_ip, _ip, _i, _dp]
    L.orc_gdn_step_conv.argtypes = [_i] * 7 + [_dp] * 9 + [_ip, _dp, _d, _i, _d, _dp, _dp, _d, _i, _dp]
    _fp = ctypes.POINTER(ctypes.c_float)
    L.orc_gdn_step_f32.argtypes = [_i] * 6 + [_fp, _l, _fp, _fp, _fp, _fp, _fp, _ip, _fp, ctypes.c_float, _i,
                                              ctypes.c_float]
    L.orc_gdn_step_f32.restype = _i
    L.orc_set_threads.argtypes = [_i]
    L.orc_set_threads.restype = None
    for f in ("orc_gdn_step", "orc_gdn_step_buffered", "orc_conv1d_update", "orc_gdn_step_conv",
              "orc_kda_step", "orc_kda_decode", "orc_mamba_step", "orc_mamba_scan", "orc_gdn_multi", "orc_num_threads"):
        getattr(L, f).restype = _i
    return L


def lib():
    """Load liboracle.so, building it first only if it is not there."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _LIB = configure(ctypes.CDLL(_build.LIB))
    return _LIB


def f64(x) -> np.ndarray:
    """Exact decode of a torch tensor or array-like to a C-contiguous float64 array."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().cpu().double().numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def i32(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return np.ascontiguousarray(x.detach().cpu().numpy().astype(np.int32))
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    if a.dtype == np.float64:
        return a.ctypes.data_as(_dp)
    if a.dtype == np.int32:
        return a.ctypes.data_as(_ip)
    raise TypeError(a.dtype)


def _chk(rc):
    if rc != 0:
        raise ValueError("oracle rejected the shapes")


# ----------------------------------------------------------------- scalars
def softplus(x):
    return lib().orc_softplus(float(x))


def sigmoid(x):
    return lib().orc_sigmoid(float(x))


def silu(x):
    return lib().orc_silu(float(x))


def round_fmt(x, fmt):
    return lib().orc_round_fmt(float(x), int(fmt))


def gdn_gates(a, b, A_log, dt_bias):
    g, beta = ctypes.c_double(), ctypes.c_double()
    lib().orc_gdn_gates(float(a), float(b), float(A_log), float(dt_bias),
                        ctypes.byref(g), ctypes.byref(beta))
    return g.value, beta.value


def kda_gate(raw_g, lower_bound):
    return lib().orc_kda_gate(float(raw_g), float(lower_bound))


def num_threads() -> int:
    return lib().orc_num_threads()


def set_threads(n: int) -> None:
    """Thread count of the parallel loops (timing only; results do not depend on it)."""
    lib().orc_set_threads(int(n))


# ----------------------------------------------------------------- GDN
def gdn_step(qkv, a, b, A_log, dt_bias, state, idx, *, H, HV, K, V, scale=None,
             use_l2=True, l2eps=1e-6, norm_gate=None, norm_weight=None,
             norm_eps=1e-5, norm_act=ACT_SILU, state_fmt=FMT_NONE):
    """One packed GDN step. `state` is a float64 [num_slots, HV, V, K] array
    updated in place (rounded to state_fmt when stored). Returns out float64
    [B, HV, V] (NaN for padded rows)."""
    qkv, a, b = f64(qkv), f64(a), f64(b)
    A_log, dt_bias, idx = f64(A_log), f64(dt_bias), i32(idx)
    assert state.dtype == np.float64 and state.flags["C_CONTIGUOUS"]
    B = idx.shape[0]
    num_slots = state.shape[0]
    assert state.shape[1:] == (HV, V, K)
    out = np.full((B, HV, V), np.nan)
    ng = None if norm_gate is None else f64(norm_gate)
    nw = None if norm_weight is None else f64(norm_weight)
    scale = K ** -0.5 if scale is None else scale
    _chk(lib().orc_gdn_step(B, H, HV, K, V, num_slots, _p(qkv), qkv.shape[1], _p(a), _p(b),
                            _p(A_log), _p(dt_bias), _p(state), _p(idx), _p(out), scale,
                            int(use_l2), l2eps, _p(ng), _p(nw), norm_eps, norm_act, int(state_fmt)))
    return out


def gdn_step_f32(qkv, a, b, A_log, dt_bias, state, idx, *, H, HV, K, V, scale=None, use_l2=True, l2eps=1e-6):
    """The packed GDN step computed entirely in fp32 (the oracle's float
    build, no output norm). `state` is a float32 [num_slots, HV, V, K] array
    updated in place. Returns out float32 [B, HV, V] (NaN for padded rows)."""
    f32 = lambda x: np.ascontiguousarray(f64(x).astype(np.float32))  # noqa: E731
    qkv, a, b, A_log, dt_bias, idx = f32(qkv), f32(a), f32(b), f32(A_log), f32(dt_bias), i32(idx)
    assert state.dtype == np.float32 and state.flags["C_CONTIGUOUS"]
    assert state.shape[1:] == (HV, V, K)
    B = idx.shape[0]
    out = np.full((B, HV, V), np.nan, dtype=np.float32)
    fp = lambda x: x.ctypes.data_as(ctypes.POINTER(ctypes.c_float))  # noqa: E731
    scale = K ** -0.5 if scale is None else scale
    _chk(lib().orc_gdn_step_f32(B, H, HV, K, V, state.shape[0], fp(qkv), qkv.shape[1], fp(a), fp(b), fp(A_log),
                                fp(dt_bias), fp(state), _p(idx), fp(out), scale, int(use_l2), l2eps))
    return out


def gdn_step_buffered(qkv, a, b, A_log, dt_bias, state, idx, d_cache, k_cache, g_cache,
                      write_pos, L, *, H, HV, K, V, scale=None, use_l2=True, l2eps=1e-6,
                      norm_gate=None, norm_weight=None, norm_eps=1e-5, norm_act=ACT_SILU,
                      ring_fmt=FMT_BF16):
    """One buffered GDN step. state [num_slots, HV, V, K], d_cache [num_slots,
    HV, L, V], k_cache [num_slots, H, L, K], g_cache [num_slots, HV, L] are
    float64 arrays updated in place. Returns out [B, HV, V]."""
    qkv, a, b = f64(qkv), f64(a), f64(b)
    A_log, dt_bias, idx, wp = f64(A_log), f64(dt_bias), i32(idx), i32(write_pos)
    for arr in (state, d_cache, k_cache, g_cache):
        assert arr.dtype == np.float64 and arr.flags["C_CONTIGUOUS"]
    B = idx.shape[0]
    num_slots = state.shape[0]
    assert d_cache.shape == (num_slots, HV, L, V) and k_cache.shape == (num_slots, H, L, K)
    assert g_cache.shape == (num_slots, HV, L)
    out = np.full((B, HV, V), np.nan)
    ng = None if norm_gate is None else f64(norm_gate)
    nw = None if norm_weight is None else f64(norm_weight)
    scale = K ** -0.5 if scale is None else scale
    _chk(lib().orc_gdn_step_buffered(
        B, H, HV, K, V, num_slots, _p(qkv), qkv.shape[1], _p(a), _p(b), _p(A_log),
        _p(dt_bias), _p(state), _p(idx), _p(out), scale, int(use_l2), l2eps, _p(ng), _p(nw),
        norm_eps, norm_act, _p(d_cache), _p(k_cache), _p(g_cache), _p(wp), L, ring_fmt))
    return out


def gdn_multi(qkv, a, b, A_log, dt_bias, state, idx, *, H, HV, K, V, lengths=None, scale=None, use_l2=True,
              l2eps=1e-6, norm_gate=None, norm_weight=None, norm_eps=1e-5, norm_act=ACT_SILU):
    """GDN over T tokens per row: qkv [B, T, C], a, b [B, T, HV], norm_gate
    [B, T, HV, V]; state float64 [num_slots, HV, V, K] in place. Returns out
    [B, T, HV, V] (NaN where not written)."""
    qkv, a, b = f64(qkv), f64(a), f64(b)
    A_log, dt_bias, idx = f64(A_log), f64(dt_bias), i32(idx)
    B, T, C = qkv.shape
    assert C == 2 * H * K + HV * V and a.shape == (B, T, HV) and b.shape == (B, T, HV)
    ln = None if lengths is None else i32(lengths)
    ng = None if norm_gate is None else f64(norm_gate)
    nw = None if norm_weight is None else f64(norm_weight)
    out = np.full((B, T, HV, V), np.nan)
    scale = K ** -0.5 if scale is None else scale
    _chk(lib().orc_gdn_multi(B, T, H, HV, K, V, state.shape[0], _p(qkv), C, _p(a), _p(b), _p(A_log),
                             _p(dt_bias), _p(state), _p(idx), _p(ln), _p(out), scale, int(use_l2), l2eps, _p(ng),
                             _p(nw), norm_eps, norm_act))
    return out


def gdn_step_conv(x, conv_w, conv_bias, conv_state, a, b, A_log, dt_bias, state, idx, *, H, HV, K, V,
                  scale=None, use_l2=True, l2eps=1e-6, norm_gate=None, norm_weight=None,
                  norm_eps=1e-5, norm_act=ACT_SILU):
    """GDN step with the causal conv1d update (+SiLU) fused in front. x is the
    pre-conv [B, 2HK + HV V]; conv_state float64 logical [num_slots, C, W-1]
    and state float64 [num_slots, HV, V, K] are updated in place. Returns out
    [B, HV, V]."""
    x, conv_w, a, b = f64(x), f64(conv_w), f64(a), f64(b)
    A_log, dt_bias, idx = f64(A_log), f64(dt_bias), i32(idx)
    cb = None if conv_bias is None else f64(conv_bias)
    B = idx.shape[0]
    W = conv_w.shape[1]
    C = 2 * H * K + HV * V
    assert x.shape == (B, C) and conv_state.shape[1:] == (C, W - 1)
    out = np.full((B, HV, V), np.nan)
    ysc = np.zeros((B, C))
    ng = None if norm_gate is None else f64(norm_gate)
    nw = None if norm_weight is None else f64(norm_weight)
    scale = K ** -0.5 if scale is None else scale
    _chk(lib().orc_gdn_step_conv(B, H, HV, K, V, W, state.shape[0], _p(x), _p(conv_w), _p(cb),
                                 _p(conv_state), _p(a), _p(b), _p(A_log), _p(dt_bias), _p(state),
                                 _p(idx), _p(out), scale, int(use_l2), l2eps, _p(ng), _p(nw), norm_eps,
                                 norm_act, _p(ysc)))
    return out


# ----------------------------------------------------------------- KDA
def conv1d_update(x, w, bias, conv_state, idx, *, skip_slot0=True, silu_act=True):
    """conv_state: float64 logical [num_slots, C, W-1], updated in place.
    Returns y [T, C] (NaN for skipped rows)."""
    x, w, idx = f64(x), f64(w), i32(idx)
    bias = None if bias is None else f64(bias)
    T, C = x.shape
    W = w.shape[1]
    assert conv_state.shape[1:] == (C, W - 1) and conv_state.dtype == np.float64
    y = np.full((T, C), np.nan)
    _chk(lib().orc_conv1d_update(T, C, W, conv_state.shape[0], _p(x), _p(w), _p(bias),
                                 _p(conv_state), _p(idx), int(skip_slot0), _p(y),
                                 int(silu_act)))
    return y


def kda_step(y, raw_g, raw_beta, state, idx, *, H, D, lower_bound=-5.0, gate=None, norm_weight=None, norm_eps=1e-5, scale=None,
             use_l2=True, l2eps=1e-6):
    """KDA recurrent step on post-conv activations y [T, 3*H*D]; state float64
    [num_slots, H, D, D] in place. Returns out [T, H, D]."""
    y, raw_g, raw_beta, idx = f64(y), f64(raw_g), f64(raw_beta), i32(idx)
    T = idx.shape[0]
    out = np.full((T, H, D), np.nan)
    gt = None if gate is None else f64(gate)
    nw = None if norm_weight is None else f64(norm_weight)
    scale = D ** -0.5 if scale is None else scale
    _chk(lib().orc_kda_step(T, H, D, state.shape[0], _p(y), _p(raw_g), _p(raw_beta), lower_bound, _p(state), _p(idx), _p(out), _p(gt), _p(nw),
                            norm_eps, scale, int(use_l2), l2eps))
    return out


def kda_decode(x, conv_w, conv_bias, conv_state, raw_g, raw_beta, state, idx, *, H, D,
               lower_bound=-5.0, gate=None, norm_weight=None,
               norm_eps=1e-5, scale=None, use_l2=True, l2eps=1e-6):
    """Fused KDA decode: conv1d update (+SiLU) -> KDA step -> sigmoid-gated
    RMSNorm. conv_state float64 logical [num_slots, 3HD, W-1] and state float64
    [num_slots, H, D, D] are updated in place. Returns out [T, H, D]."""
    x, conv_w, raw_g, raw_beta, idx = f64(x), f64(conv_w), f64(raw_g), f64(raw_beta), i32(idx)
    cb = None if conv_bias is None else f64(conv_bias)
    T = idx.shape[0]
    W = conv_w.shape[1]
    out = np.full((T, H, D), np.nan)
    ysc = np.zeros((T, 3 * H * D))
    gt = None if gate is None else f64(gate)
    nw = None if norm_weight is None else f64(norm_weight)
    scale = D ** -0.5 if scale is None else scale
    _chk(lib().orc_kda_decode(T, H, D, W, state.shape[0], _p(x), _p(conv_w), _p(cb),
                              _p(conv_state), _p(raw_g), _p(raw_beta), lower_bound, _p(state), _p(idx), _p(out), _p(gt), _p(nw),
                              norm_eps, scale, int(use_l2), l2eps, _p(ysc)))
    return out


# ----------------------------------------------------------------- Mamba
def mamba_scan(x, dt, A, Bm, Cm, Dv, z, hpool, idx, lengths=None, zero_init=False):
    """Mamba-1 over T tokens per row (prefill); x, dt, z [B, T, D], Bm, Cm
    [B, T, N]; hpool float64 [num_slots, D, N] in place (read unless
    zero_init, written with the final state). Returns y [B, T, D] (NaN where
    not written)."""
    x, dt, A, Bm, Cm, idx = f64(x), f64(dt), f64(A), f64(Bm), f64(Cm), i32(idx)
    Dv = None if Dv is None else f64(Dv)
    z = None if z is None else f64(z)
    ln = None if lengths is None else i32(lengths)
    B, T, Dm = x.shape
    N = A.shape[1]
    y = np.full((B, T, Dm), np.nan)
    _chk(lib().orc_mamba_scan(B, T, Dm, N, hpool.shape[0], _p(x), _p(dt), _p(A), _p(Bm), _p(Cm), _p(Dv),
                              _p(z), _p(hpool), _p(idx), _p(ln), int(bool(zero_init)), _p(y)))
    return y


def mamba_step(x, dt, A, Bm, Cm, Dv, z, hpool, idx):
    """Mamba-1 selective-scan decode step; hpool float64 [num_slots, D, N] in
    place. Returns y [B, D]."""
    x, dt, A, Bm, Cm, idx = f64(x), f64(dt), f64(A), f64(Bm), f64(Cm), i32(idx)
    Dv = None if Dv is None else f64(Dv)
    z = None if z is None else f64(z)
    B, Dm = x.shape
    N = A.shape[1]
    y = np.full((B, Dm), np.nan)
    _chk(lib().orc_mamba_step(B, Dm, N, hpool.shape[0], _p(x), _p(dt), _p(A), _p(Bm), _p(Cm),
                              _p(Dv), _p(z), _p(hpool), _p(idx), _p(y)))
    return y
