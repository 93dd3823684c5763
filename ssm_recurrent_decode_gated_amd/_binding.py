"""ctypes binding of libssmdec.so (include/ssmdec.h).

Argument marshalling only: torch tensors are checked for device, dtype,
shape and layout, and their device pointers, sizes and torch's current HIP
stream are passed to the C entry points of the same name. Every step of the
decode runs in the library's HIP kernels; there is no other implementation,
and a missing library is an error, not a fallback.
"""
from __future__ import annotations

import ctypes
import functools
import os

import torch  # loads torch's HIP runtime first, so libssmdec.so binds to that one

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libssmdec.so")

SSMD_F32, SSMD_BF16, SSMD_F16 = 0, 1, 2
SSMD_ACT_SILU, SSMD_ACT_SIGMOID = 0, 1
DTYPE_CODE = {torch.float32: SSMD_F32, torch.bfloat16: SSMD_BF16, torch.float16: SSMD_F16}
ACT_CODE = {"silu": SSMD_ACT_SILU, "sigmoid": SSMD_ACT_SIGMOID}
EXPORTS = ("gdn_decode_step", "gdn_decode_step_state16", "gdn_decode_step_buffered", "gdn_decode_step_conv",
           "gdn_fused_recurrent", "gdn_chunk_prefill", "gdn_chunk_prefill_noalloc", "gdn_chunk_workspace_bytes",
           "kda_decode_step", "mamba_decode_step", "mamba_scan", "mamba_scan_workspace_bytes", "ssmd_last_error",
           "ssmd_stream_copy", "ssmd_check_slot_indices")


class SsmdError(RuntimeError):
    """A non-zero status from the library; .code holds it."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


_LIB = None
_p, _i32, _i64, _f = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
_GDN_ARGS = [_p, _i64, _p, _p, _p, _p, _p, _i32, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
             _f, _i32, _f, _p, _p, _f, _i32]


def load_library() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
                "at the repository root. There is no non-HIP fallback.")
        L = ctypes.CDLL(LIB_PATH)
        L.gdn_decode_step.argtypes = _GDN_ARGS + [_p]
        L.gdn_decode_step_buffered.argtypes = _GDN_ARGS + [_p, _p, _p, _p, _i32, _p]
        L.gdn_decode_step_state16.argtypes = _GDN_ARGS[:7] + [_i32] + _GDN_ARGS[7:] + [_p]
        L.gdn_fused_recurrent.argtypes = _GDN_ARGS[:9] + [_p] + _GDN_ARGS[9:11] + [_i32] + _GDN_ARGS[11:] + [_p]
        L.gdn_chunk_prefill.argtypes = L.gdn_fused_recurrent.argtypes[:-1] + [_p, _i64, _p]
        L.gdn_chunk_prefill_noalloc.argtypes = L.gdn_fused_recurrent.argtypes
        L.gdn_chunk_workspace_bytes.argtypes = [_i32] * 6
        L.gdn_decode_step_conv.argtypes = [_p, _i64, _p, _p, _p, _i64, _i64, _i64, _i32] + _GDN_ARGS[2:] + [_p]
        L.kda_decode_step.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _p, _p, _p, _p, _f, _p, _i32,
                                      _p, _p, _p, _p, _f, _i32, _i32, _i32, _i32, _i32, _i32, _f,
                                      _i32, _f, _p]
        L.mamba_decode_step.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _i32, _p, _p, _i32, _i32, _i32,
                                        _i32, _i32, _p]
        L.mamba_scan.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _i32, _p, _p, _i32, _p, _p, _i64, _i32, _i32,
                                 _i32, _i32, _i32, _i32, _p]
        L.mamba_scan_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32]
        L.ssmd_stream_copy.argtypes = [_p, _p, _i64, _p]
        L.ssmd_check_slot_indices.argtypes = [_p, _i32, _i32, _i32, _p, _p]
        for f in EXPORTS:
            if f == "ssmd_last_error":
                continue
            getattr(L, f).restype = ctypes.c_int
        L.mamba_scan_workspace_bytes.restype = ctypes.c_int64
        L.gdn_chunk_workspace_bytes.restype = ctypes.c_int64
        L.ssmd_last_error.argtypes = []
        L.ssmd_last_error.restype = ctypes.c_char_p
        _LIB = L
    return _LIB


def ssmd_last_error() -> str:
    return load_library().ssmd_last_error().decode()


def _check(rc: int, name: str):
    if rc != 0:
        raise SsmdError(rc, ssmd_last_error() or name)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None, contiguous=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (HIP) tensor, got {t.device}")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name}: dtype {t.dtype} not allowed")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(t: torch.Tensor, stream):
    if stream is None:
        return torch.cuda.current_stream(t.device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


_ACTS = (torch.float32, torch.bfloat16, torch.float16)


def _one_device(fn):
    """Entry-point wrapper: every tensor argument (and a torch stream, if
    given) must be on one HIP device, which is made current for the call
    (the library launches on the current device). Kept to integer device
    ids on the common path: it runs on every eager call."""
    @functools.wraps(fn)
    def call(*args, **kwargs):
        dev = None
        for t in (*args, *kwargs.values()) if kwargs else args:
            if isinstance(t, torch.Tensor):
                g = t.get_device()
                if g < 0:
                    g = t.device.type  # host or meta tensor: rejected by the call's checks if alone
                if dev is None:
                    dev = g
                elif g != dev:
                    raise ValueError(f"{fn.__name__}: arguments on several devices ({dev} and {g})")
        st = kwargs.get("stream")
        if st is not None and hasattr(st, "device") and dev is not None:
            sd = torch.device(st.device)
            if sd.type != "cuda" or sd.index != dev:
                raise ValueError(f"{fn.__name__}: stream on {sd}, tensors on {dev}")
        if type(dev) is int and dev != torch.cuda.current_device():
            with torch.cuda.device(dev):
                return fn(*args, **kwargs)
        return fn(*args, **kwargs)
    return call


def _gdn_common(mixed_qkv, a, b, A_log, dt_bias, state, ssm_state_indices, out, H, norm_gate,
                norm_weight, state_dtypes=(torch.float32,)):
    _dev(state, "state", state_dtypes)
    if state.dim() != 4:
        raise ValueError("state must be [num_slots, HV, V, K]")
    num_slots, HV, V, K = state.shape
    _dev(mixed_qkv, "mixed_qkv", _ACTS, contiguous=False)
    if mixed_qkv.dim() != 2 or mixed_qkv.stride(1) != 1:
        raise ValueError("mixed_qkv must be [B, 2*H*K + HV*V] with unit column stride")
    B = mixed_qkv.shape[0]
    if H is None:
        qk = mixed_qkv.shape[1] - HV * V
        if qk <= 0 or qk % (2 * K):
            raise ValueError("cannot infer H from mixed_qkv width; pass H=")
        H = qk // (2 * K)
    if mixed_qkv.shape[1] != 2 * H * K + HV * V:
        raise ValueError(f"mixed_qkv width {mixed_qkv.shape[1]} != 2*H*K + HV*V")
    act = mixed_qkv.dtype
    _dev(a, "a", act, (B, HV))
    _dev(b, "b", act, (B, HV))
    _dev(A_log, "A_log", torch.float32, (HV,))
    _dev(dt_bias, "dt_bias", torch.float32, (HV,))
    _dev(ssm_state_indices, "ssm_state_indices", torch.int32, (B,))
    _dev(out, "out", _ACTS)
    if out.numel() != B * HV * V or out.shape[0] != B or out.shape[-1] != V:
        raise ValueError("out must be [B, 1, HV, V] (or [B, HV, V])")
    if norm_gate is not None:
        _dev(norm_gate, "norm_gate", act, (B, HV, V))
    if norm_weight is not None:
        _dev(norm_weight, "norm_weight", torch.float32, (V,))
    return B, H, HV, K, V, num_slots, DTYPE_CODE[act], DTYPE_CODE[out.dtype]


@_one_device
def gdn_decode_step(mixed_qkv, a, b, A_log, dt_bias, state, ssm_state_indices, out, *, H=None,
                    scale=None, use_qk_l2norm=True, l2norm_eps=1e-6, norm_gate=None,
                    norm_weight=None, norm_eps=1e-5, norm_act="silu", stream=None):
    """One packed GDN decode step (state and out updated in place); see
    gdn_decode_step in include/ssmdec.h for the computation."""
    B, H, HV, K, V, num_slots, act, odt = _gdn_common(mixed_qkv, a, b, A_log, dt_bias, state,
                                                      ssm_state_indices, out, H, norm_gate, norm_weight)
    scale = K ** -0.5 if scale is None else scale
    L = load_library()
    rc = L.gdn_decode_step(_ptr(mixed_qkv), mixed_qkv.stride(0), _ptr(a), _ptr(b), _ptr(A_log),
                           _ptr(dt_bias), _ptr(state), num_slots, _ptr(ssm_state_indices), _ptr(out),
                           B, H, HV, K, V, act, odt, scale, int(bool(use_qk_l2norm)), l2norm_eps,
                           _ptr(norm_gate), _ptr(norm_weight), norm_eps, ACT_CODE[norm_act],
                           _stream(state, stream))
    _check(rc, "gdn_decode_step")
    return out


@_one_device
def gdn_decode_step_state16(mixed_qkv, a, b, A_log, dt_bias, state, ssm_state_indices, out, *, H=None,
                            scale=None, use_qk_l2norm=True, l2norm_eps=1e-6, norm_gate=None,
                            norm_weight=None, norm_eps=1e-5, norm_act="silu", stream=None):
    """The packed GDN step on a bf16 or f16 state pool (rounded once per step
    on store); see gdn_decode_step_state16 in include/ssmdec.h."""
    B, H, HV, K, V, num_slots, act, odt = _gdn_common(
        mixed_qkv, a, b, A_log, dt_bias, state, ssm_state_indices, out, H, norm_gate, norm_weight,
        state_dtypes=(torch.bfloat16, torch.float16))
    scale = K ** -0.5 if scale is None else scale
    L = load_library()
    rc = L.gdn_decode_step_state16(_ptr(mixed_qkv), mixed_qkv.stride(0), _ptr(a), _ptr(b), _ptr(A_log),
                                   _ptr(dt_bias), _ptr(state), DTYPE_CODE[state.dtype], num_slots,
                                   _ptr(ssm_state_indices), _ptr(out), B, H, HV, K, V, act, odt, scale,
                                   int(bool(use_qk_l2norm)), l2norm_eps, _ptr(norm_gate), _ptr(norm_weight),
                                   norm_eps, ACT_CODE[norm_act], _stream(state, stream))
    _check(rc, "gdn_decode_step_state16")
    return out


@_one_device
def gdn_decode_step_buffered(mixed_qkv, a, b, A_log, dt_bias, state, ssm_state_indices, out,
                             d_cache, k_cache, g_cache, write_pos, *, H=None, scale=None,
                             use_qk_l2norm=True, l2norm_eps=1e-6, norm_gate=None, norm_weight=None,
                             norm_eps=1e-5, norm_act="silu", stream=None):
    """One buffered GDN decode step; see gdn_decode_step_buffered in
    include/ssmdec.h. write_pos is read only (the caller advances it)."""
    B, H, HV, K, V, num_slots, act, odt = _gdn_common(mixed_qkv, a, b, A_log, dt_bias, state,
                                                      ssm_state_indices, out, H, norm_gate, norm_weight)
    _dev(d_cache, "d_cache", mixed_qkv.dtype)
    if d_cache.dim() != 4 or tuple(d_cache.shape[:2]) != (num_slots, HV) or d_cache.shape[3] != V:
        raise ValueError("d_cache must be [num_slots, HV, L, V]")
    L_ = d_cache.shape[2]
    _dev(k_cache, "k_cache", mixed_qkv.dtype, (num_slots, H, L_, K))
    _dev(g_cache, "g_cache", torch.float32, (num_slots, HV, L_))
    _dev(write_pos, "write_pos", torch.int32, (B,))
    scale = K ** -0.5 if scale is None else scale
    L = load_library()
    rc = L.gdn_decode_step_buffered(
        _ptr(mixed_qkv), mixed_qkv.stride(0), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
        _ptr(state), num_slots, _ptr(ssm_state_indices), _ptr(out), B, H, HV, K, V, act, odt, scale,
        int(bool(use_qk_l2norm)), l2norm_eps, _ptr(norm_gate), _ptr(norm_weight), norm_eps,
        ACT_CODE[norm_act], _ptr(d_cache), _ptr(k_cache), _ptr(g_cache), _ptr(write_pos), L_,
        _stream(state, stream))
    _check(rc, "gdn_decode_step_buffered")
    return out


def _gdn_multi_args(mixed_qkv, a, b, A_log, dt_bias, state, ssm_state_indices, out, lengths, H, norm_gate,
                    norm_weight):
    _dev(state, "state", torch.float32)
    if state.dim() != 4:
        raise ValueError("state must be [num_slots, HV, V, K]")
    num_slots, HV, V, K = state.shape
    _dev(mixed_qkv, "mixed_qkv", _ACTS, contiguous=False)
    if mixed_qkv.dim() != 3 or mixed_qkv.stride(2) != 1:
        raise ValueError("mixed_qkv must be [B, T, C] with unit column stride")
    B, T, C = mixed_qkv.shape
    row_stride = mixed_qkv.stride(1) if T > 1 else mixed_qkv.stride(0)
    if B > 1 and T > 1 and mixed_qkv.stride(0) != T * row_stride:
        raise ValueError("mixed_qkv rows must be evenly spaced over the flattened B*T tokens")
    if H is None:
        qk = C - HV * V
        if qk <= 0 or qk % (2 * K):
            raise ValueError("cannot infer H from mixed_qkv width; pass H=")
        H = qk // (2 * K)
    if C != 2 * H * K + HV * V:
        raise ValueError(f"mixed_qkv width {C} != 2*H*K + HV*V")
    act = mixed_qkv.dtype
    _dev(a, "a", act, (B, T, HV))
    _dev(b, "b", act, (B, T, HV))
    _dev(A_log, "A_log", torch.float32, (HV,))
    _dev(dt_bias, "dt_bias", torch.float32, (HV,))
    _dev(ssm_state_indices, "ssm_state_indices", torch.int32, (B,))
    if lengths is not None:
        _dev(lengths, "lengths", torch.int32, (B,))
    _dev(out, "out", _ACTS, (B, T, HV, V))
    if norm_gate is not None:
        _dev(norm_gate, "norm_gate", act, (B, T, HV, V))
    if norm_weight is not None:
        _dev(norm_weight, "norm_weight", torch.float32, (V,))
    return B, T, H, HV, K, V, num_slots, row_stride, act


@_one_device
def gdn_fused_recurrent(mixed_qkv, a, b, A_log, dt_bias, state, ssm_state_indices, out, *, lengths=None, H=None,
                        scale=None, use_qk_l2norm=True, l2norm_eps=1e-6, norm_gate=None, norm_weight=None,
                        norm_eps=1e-5, norm_act="silu", stream=None):
    """The GDN step over T tokens per row, state read and written once; see
    gdn_fused_recurrent in include/ssmdec.h. mixed_qkv [B, T, C] with unit
    column stride and its B*T rows evenly spaced (any row stride >= C);
    a, b [B, T, HV]; out and norm_gate [B, T, HV, V]."""
    B, T, H, HV, K, V, num_slots, row_stride, act = _gdn_multi_args(
        mixed_qkv, a, b, A_log, dt_bias, state, ssm_state_indices, out, lengths, H, norm_gate, norm_weight)
    scale = K ** -0.5 if scale is None else scale
    rc = load_library().gdn_fused_recurrent(
        _ptr(mixed_qkv), row_stride, _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), _ptr(state), num_slots,
        _ptr(ssm_state_indices), _ptr(lengths), _ptr(out), B, T, H, HV, K, V, DTYPE_CODE[act],
        DTYPE_CODE[out.dtype], scale, int(bool(use_qk_l2norm)), l2norm_eps, _ptr(norm_gate), _ptr(norm_weight),
        norm_eps, ACT_CODE[norm_act], _stream(state, stream))
    _check(rc, "gdn_fused_recurrent")
    return out


def gdn_chunk_workspace_bytes(B, T, HV, K, V, with_norm=False) -> int:
    n = load_library().gdn_chunk_workspace_bytes(B, T, HV, K, V, int(bool(with_norm)))
    if n < 0:
        raise SsmdError(n, ssmd_last_error())
    return n


@_one_device
def gdn_chunk_prefill(mixed_qkv, a, b, A_log, dt_bias, state, ssm_state_indices, out, *, workspace=None,
                      lengths=None, H=None, scale=None, use_qk_l2norm=True, l2norm_eps=1e-6, norm_gate=None,
                      norm_weight=None, norm_eps=1e-5, norm_act="silu", stream=None):
    """gdn_fused_recurrent's result in chunked form (long sequences); see
    gdn_chunk_prefill in include/ssmdec.h. workspace: a device tensor of at
    least gdn_chunk_workspace_bytes(...) bytes; when None, one is allocated
    with torch for this call."""
    B, T, H, HV, K, V, num_slots, row_stride, act = _gdn_multi_args(
        mixed_qkv, a, b, A_log, dt_bias, state, ssm_state_indices, out, lengths, H, norm_gate, norm_weight)
    need = gdn_chunk_workspace_bytes(B, T, HV, K, V, norm_gate is not None)
    if workspace is None:
        workspace = torch.empty(max(need // 4, 1), dtype=torch.float32, device=state.device)
    _dev(workspace, "workspace")
    scale = K ** -0.5 if scale is None else scale
    rc = load_library().gdn_chunk_prefill(
        _ptr(mixed_qkv), row_stride, _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), _ptr(state), num_slots,
        _ptr(ssm_state_indices), _ptr(lengths), _ptr(out), B, T, H, HV, K, V, DTYPE_CODE[act],
        DTYPE_CODE[out.dtype], scale, int(bool(use_qk_l2norm)), l2norm_eps, _ptr(norm_gate), _ptr(norm_weight),
        norm_eps, ACT_CODE[norm_act], _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(state, stream))
    _check(rc, "gdn_chunk_prefill")
    return out


# size of the library's static workspace behind gdn_chunk_prefill_noalloc (include/ssmdec.h)
SSMD_CHUNK_SCRATCH_BYTES = 128 << 20


@_one_device
def gdn_chunk_prefill_noalloc(mixed_qkv, a, b, A_log, dt_bias, state, ssm_state_indices, out, *, lengths=None,
                              H=None, scale=None, use_qk_l2norm=True, l2norm_eps=1e-6, norm_gate=None,
                              norm_weight=None, norm_eps=1e-5, norm_act="silu", stream=None):
    """gdn_chunk_prefill with the library's static workspace instead of a
    caller's (for callers that cannot allocate); see
    gdn_chunk_prefill_noalloc in include/ssmdec.h. Nothing is allocated,
    here or in the library."""
    B, T, H, HV, K, V, num_slots, row_stride, act = _gdn_multi_args(
        mixed_qkv, a, b, A_log, dt_bias, state, ssm_state_indices, out, lengths, H, norm_gate, norm_weight)
    scale = K ** -0.5 if scale is None else scale
    rc = load_library().gdn_chunk_prefill_noalloc(
        _ptr(mixed_qkv), row_stride, _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), _ptr(state), num_slots,
        _ptr(ssm_state_indices), _ptr(lengths), _ptr(out), B, T, H, HV, K, V, DTYPE_CODE[act],
        DTYPE_CODE[out.dtype], scale, int(bool(use_qk_l2norm)), l2norm_eps, _ptr(norm_gate), _ptr(norm_weight),
        norm_eps, ACT_CODE[norm_act], _stream(state, stream))
    _check(rc, "gdn_chunk_prefill_noalloc")
    return out


@_one_device
def gdn_decode_step_conv(x, conv_weight, conv_bias, conv_state, a, b, A_log, dt_bias, state,
                         ssm_state_indices, out, *, H=None, scale=None, use_qk_l2norm=True,
                         l2norm_eps=1e-6, norm_gate=None, norm_weight=None, norm_eps=1e-5,
                         norm_act="silu", stream=None):
    """The GDN step with its causal conv1d update + SiLU fused in front; see
    gdn_decode_step_conv in include/ssmdec.h. x is the pre-conv row (unit
    column stride, any row stride); conv_state is the logical
    [num_slots, C, W-1] view of either physical layout."""
    B, H, HV, K, V, num_slots, act, odt = _gdn_common(x, a, b, A_log, dt_bias, state,
                                                      ssm_state_indices, out, H, norm_gate, norm_weight)
    C = 2 * H * K + HV * V
    _dev(conv_weight, "conv_weight", torch.float32)
    if conv_weight.dim() != 2 or conv_weight.shape[0] != C:
        raise ValueError(f"conv_weight must be [{C}, W]")
    W = conv_weight.shape[1]
    if conv_bias is not None:
        _dev(conv_bias, "conv_bias", torch.float32, (C,))
    _dev(conv_state, "conv_state", x.dtype, (num_slots, C, W - 1), contiguous=False)
    scale = K ** -0.5 if scale is None else scale
    rc = load_library().gdn_decode_step_conv(
        _ptr(x), x.stride(0), _ptr(conv_weight), _ptr(conv_bias), _ptr(conv_state), conv_state.stride(0),
        conv_state.stride(1), conv_state.stride(2), W, _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
        _ptr(state), num_slots, _ptr(ssm_state_indices), _ptr(out), B, H, HV, K, V, act, odt, scale,
        int(bool(use_qk_l2norm)), l2norm_eps, _ptr(norm_gate), _ptr(norm_weight), norm_eps,
        ACT_CODE[norm_act], _stream(state, stream))
    _check(rc, "gdn_decode_step_conv")
    return out


@_one_device
def kda_decode_step(x, conv_weight, conv_bias, conv_state, raw_g, raw_beta, A_log, dt_bias, state,
                    state_indices, out, *, output_gate=None, norm_weight=None, lower_bound=-5.0,
                    norm_eps=1e-5, scale=None, use_qk_l2norm=True, l2norm_eps=1e-6, stream=None):
    """The fused KDA decode op (conv1d update + SiLU, KDA delta rule, sigmoid
    gated RMSNorm); see kda_decode_step in include/ssmdec.h. conv_state is the
    logical [num_slots, 3*H*D, W-1] view of either physical layout. A_log and
    dt_bias are passed through as the ABI takes them; the library refuses
    anything but None for them (no formula for them is defined)."""
    _dev(state, "state", torch.float32)
    if state.dim() != 4 or state.shape[2] != state.shape[3]:
        raise ValueError("state must be [num_slots, H, D, D]")
    num_slots, H, D, _ = state.shape
    _dev(x, "x", _ACTS)
    T = x.shape[0]
    C = 3 * H * D
    if tuple(x.shape) != (T, C):
        raise ValueError(f"x must be [T, {C}]")
    act = x.dtype
    _dev(conv_weight, "conv_weight", torch.float32)
    if conv_weight.dim() != 2 or conv_weight.shape[0] != C:
        raise ValueError(f"conv_weight must be [{C}, W]")
    W = conv_weight.shape[1]
    if conv_bias is not None:
        _dev(conv_bias, "conv_bias", torch.float32, (C,))
    _dev(conv_state, "conv_state", act, (num_slots, C, W - 1), contiguous=False)
    _dev(raw_g, "raw_g", act)
    if raw_g.numel() != T * H * D:
        raise ValueError("raw_g must hold T*H*D values ([T, H, D] or [1, T, H, D])")
    _dev(raw_beta, "raw_beta", act)
    if raw_beta.numel() != T * H:
        raise ValueError("raw_beta must hold T*H values")
    if A_log is not None:
        _dev(A_log, "A_log", torch.float32, (H,))
    if dt_bias is not None:
        _dev(dt_bias, "dt_bias", torch.float32, (H * D,))
    _dev(state_indices, "state_indices", torch.int32, (T,))
    _dev(out, "out", _ACTS)
    if out.numel() != T * H * D:
        raise ValueError("out must hold T*H*D values")
    if output_gate is not None:
        _dev(output_gate, "output_gate", act)
        if output_gate.numel() != T * H * D:
            raise ValueError("output_gate must hold T*H*D values")
    if norm_weight is not None:
        _dev(norm_weight, "norm_weight", torch.float32, (D,))
    scale = D ** -0.5 if scale is None else scale
    L = load_library()
    rc = L.kda_decode_step(
        _ptr(x), _ptr(conv_weight), _ptr(conv_bias), _ptr(conv_state), conv_state.stride(0),
        conv_state.stride(1), conv_state.stride(2), _ptr(raw_g), _ptr(raw_beta), _ptr(A_log),
        _ptr(dt_bias), lower_bound, _ptr(state), num_slots, _ptr(state_indices), _ptr(out),
        _ptr(output_gate), _ptr(norm_weight), norm_eps, T, H, D, W, DTYPE_CODE[act],
        DTYPE_CODE[out.dtype], scale, int(bool(use_qk_l2norm)), l2norm_eps, _stream(state, stream))
    _check(rc, "kda_decode_step")
    return out


@_one_device
def mamba_decode_step(x, dt, A, Bm, Cm, Dvec, z, state, state_indices, out, *, stream=None):
    """One Mamba-1 selective-scan decode step (state and out updated in
    place); see mamba_decode_step in include/ssmdec.h."""
    _dev(state, "state", torch.float32)
    if state.dim() != 3:
        raise ValueError("state must be [num_slots, D, N]")
    num_slots, Dm, N = state.shape
    _dev(x, "x", _ACTS)
    B = x.shape[0]
    act = x.dtype
    _dev(x, "x", act, (B, Dm))
    _dev(dt, "dt", act, (B, Dm))
    _dev(A, "A", torch.float32, (Dm, N))
    _dev(Bm, "Bm", act, (B, N))
    _dev(Cm, "Cm", act, (B, N))
    if Dvec is not None:
        _dev(Dvec, "Dvec", torch.float32, (Dm,))
    if z is not None:
        _dev(z, "z", act, (B, Dm))
    _dev(state_indices, "state_indices", torch.int32, (B,))
    _dev(out, "out", _ACTS, (B, Dm))
    rc = load_library().mamba_decode_step(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dvec), _ptr(z), _ptr(state), num_slots,
        _ptr(state_indices), _ptr(out), B, Dm, N, DTYPE_CODE[act], DTYPE_CODE[out.dtype], _stream(state, stream))
    _check(rc, "mamba_decode_step")
    return out


def mamba_scan_workspace_bytes(B, T, Dm, N) -> int:
    """Workspace bytes that let mamba_scan run fully chunk-parallel on the
    current device (0: one pass is already enough)."""
    n = load_library().mamba_scan_workspace_bytes(B, T, Dm, N)
    if n < 0:
        raise SsmdError(n, ssmd_last_error())
    return n


@_one_device
def mamba_scan(x, dt, A, Bm, Cm, Dvec, z, state, state_indices, out, *, lengths=None, zero_init=False,
               workspace=None, stream=None):
    """Mamba-1 over T tokens per row (prefill); see mamba_scan in
    include/ssmdec.h. workspace: an optional device tensor (any dtype) of
    scratch; mamba_scan_workspace_bytes() gives the size for full
    parallelism."""
    _dev(state, "state", torch.float32)
    if state.dim() != 3:
        raise ValueError("state must be [num_slots, D, N]")
    num_slots, Dm, N = state.shape
    _dev(x, "x", _ACTS)
    if x.dim() != 3 or x.shape[2] != Dm:
        raise ValueError("x must be [B, T, D]")
    B, T = x.shape[0], x.shape[1]
    act = x.dtype
    _dev(dt, "dt", act, (B, T, Dm))
    _dev(A, "A", torch.float32, (Dm, N))
    _dev(Bm, "Bm", act, (B, T, N))
    _dev(Cm, "Cm", act, (B, T, N))
    if Dvec is not None:
        _dev(Dvec, "Dvec", torch.float32, (Dm,))
    if z is not None:
        _dev(z, "z", act, (B, T, Dm))
    _dev(state_indices, "state_indices", torch.int32, (B,))
    if lengths is not None:
        _dev(lengths, "lengths", torch.int32, (B,))
    _dev(out, "out", _ACTS, (B, T, Dm))
    ws_bytes = 0
    if workspace is not None:
        _dev(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    rc = load_library().mamba_scan(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dvec), _ptr(z), _ptr(state), num_slots,
        _ptr(state_indices), _ptr(lengths), int(bool(zero_init)), _ptr(out), _ptr(workspace), ws_bytes, B, T, Dm,
        N, DTYPE_CODE[act], DTYPE_CODE[out.dtype], _stream(state, stream))
    _check(rc, "mamba_scan")
    return out


@_one_device
def ssmd_stream_copy(src: torch.Tensor, dst: torch.Tensor, stream=None):
    """Copy src to dst (same byte size) with the library's 128-bit stream kernel."""
    _dev(src, "src")
    _dev(dst, "dst")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst sizes differ")
    _check(load_library().ssmd_stream_copy(_ptr(src), _ptr(dst), nbytes, _stream(src, stream)),
           "ssmd_stream_copy")
    return dst


@_one_device
def ssmd_check_slot_indices(idx: torch.Tensor, num_slots: int, null_slot_zero: bool = False,
                            dup_count: torch.Tensor = None, stream=None) -> torch.Tensor:
    """Debug check: count the active rows of idx ([B] int32) whose slot an
    earlier active row already names, into dup_count ([1] int32 on the same
    device, allocated if None). Asynchronous; read the result after a sync."""
    _dev(idx, "idx", torch.int32)
    if dup_count is None:
        dup_count = torch.empty(1, dtype=torch.int32, device=idx.device)
    _dev(dup_count, "dup_count", torch.int32, (1,))
    _check(load_library().ssmd_check_slot_indices(_ptr(idx), idx.numel(), int(num_slots), int(bool(null_slot_zero)),
                                                  _ptr(dup_count), _stream(idx, stream)),
           "ssmd_check_slot_indices")
    return dup_count
