"""GPU parity of gdn_decode_step_conv (causal conv1d update + SiLU fused in
front of the GDN step) against the fp64 oracle: outputs and states to the
fp32 tolerance (16-bit outputs: the RNE of the exact value), the rolled conv
state bit for bit (it holds raw inputs), and padded rows touching nothing."""
import numpy as np
import pytest
import torch

import oracle as O
import ssm_recurrent_decode_gated_amd as S
import workloads as W
from tests._helpers import CHAIN_TOL, FP32_TOL, assert_out16, assert_mixed, need_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _gpu(w, st_d, cs_d, idx, x, P, cv, out_dtype, norm=False, norm_act="silu", sentinel=float("nan"),
         row_pad=0):
    out = torch.full((w.B, 1, w.HV, w.V), sentinel, dtype=TD[out_dtype], device=DEV)
    xin = x["qkv"].to(DEV)
    if row_pad:  # same values behind a wider row stride
        wide = torch.zeros((w.B, xin.shape[1] + row_pad), dtype=xin.dtype, device=DEV)
        wide[:, : xin.shape[1]] = xin
        xin = wide[:, : xin.shape[1]]
    kw = {}
    if norm:
        kw = dict(norm_gate=x["norm_gate"].to(DEV), norm_weight=x["norm_weight"].to(DEV), norm_act=norm_act)
    S.gdn_decode_step_conv(xin, cv["conv_weight"].to(DEV),
                           None if cv["conv_bias"] is None else cv["conv_bias"].to(DEV), cs_d,
                           x["a"].to(DEV), x["b"].to(DEV), P["A_log"].to(DEV), P["dt_bias"].to(DEV), st_d,
                           idx.to(DEV), out, **kw)
    return out


def _oracle(w, ref_state, ref_cs, idx, x, P, cv, norm=False, norm_act="silu"):
    kw = {}
    if norm:
        kw = dict(norm_gate=x["norm_gate"], norm_weight=x["norm_weight"],
                  norm_act=O.ACT_SIGMOID if norm_act == "sigmoid" else O.ACT_SILU)
    return O.gdn_step_conv(x["qkv"], cv["conv_weight"], cv["conv_bias"], ref_cs, x["a"], x["b"], P["A_log"],
                           P["dt_bias"], ref_state, idx, H=w.H, HV=w.HV, K=w.K, V=w.V, **kw)


def _check_out(out, ref, what):
    B, _, HV, V = out.shape
    if out.dtype == torch.float32:
        assert_mixed(out.reshape(B, HV, V), ref, FP32_TOL, what)
    else:
        assert_out16(out.reshape(B, HV, V), ref, FP32_TOL, what)


def _setup(w, Wd=4, layout="DS", bias=True):
    P, idx = W.gdn_params(w), W.slot_indices(w)
    cv = W.gdn_conv(w, Wd, layout=layout, bias=bias)
    st = W.gdn_state(w)
    cs_d = cv["conv_state"].to(DEV)
    assert cs_d.stride() == cv["conv_state"].stride()
    return P, idx, cv, st, cs_d


def test_gdn_conv_b256_of_264_full_size():
    """256 rows over a 264-slot pool with permuted indices, H=16, HV=32,
    K=V=128, conv width 4 over the 8192 channels, bf16 activations and conv
    state: every output, state and conv-state element is compared; the 8
    unnamed slots must be bit-identical to their initial contents."""
    need_gpu()
    w = W.GDN_B256
    P, idx, cv, st, cs_d = _setup(w)
    x = W.gdn_step_inputs(w)
    st_d = st.to(DEV)
    out = _gpu(w, st_d, cs_d, idx, x, P, cv, "bf16")
    ref = st.double().numpy()
    ref_cs = cv["conv_state"].double().numpy().copy()
    ro = _oracle(w, ref, ref_cs, idx, x, P, cv)
    got, got_cs = st_d.cpu(), cs_d.cpu()
    _check_out(out, ro, "output")
    np.testing.assert_array_equal(got_cs.double().numpy(), ref_cs)
    named = set(idx.tolist())
    for s in range(w.num_slots):
        if s in named:
            assert_mixed(got[s], ref[s], FP32_TOL, f"slot {s}")
        else:
            assert torch.equal(got[s], st[s]), f"unnamed slot {s} changed"
            assert torch.equal(got_cs[s], cv["conv_state"][s]), f"unnamed slot {s}: conv state changed"


def test_gdn_conv_padded_rows_touch_nothing():
    need_gpu()
    w = W.GDNWorkload("gdn_conv_pad", B=5, H=2, HV=4, K=128, V=128, num_slots=6)
    P, _, cv, st, cs_d = _setup(w, layout="SD")
    x = W.gdn_step_inputs(w)
    idx = torch.tensor([3, -1, 6, 0, 2**31 - 1], dtype=torch.int32)
    st_d = st.to(DEV)
    out = _gpu(w, st_d, cs_d, idx, x, P, cv, "bf16", sentinel=7.0)
    ref, ref_cs = st.double().numpy().copy(), cv["conv_state"].double().numpy().copy()
    ro = _oracle(w, ref, ref_cs, idx, x, P, cv)
    got, got_cs = st_d.cpu(), cs_d.cpu()
    for b in (1, 2, 4):
        assert (out[b].float().cpu() == 7.0).all(), f"padded row {b} output written"
    _check_out(out[[0, 3]], ro[[0, 3]], "active rows")
    np.testing.assert_array_equal(got_cs.double().numpy(), ref_cs)
    for s in (1, 2, 4, 5):
        assert torch.equal(got[s], st[s])
        assert torch.equal(got_cs[s], cv["conv_state"][s])
    assert_mixed(got[[0, 3]], ref[[0, 3]], FP32_TOL, "active slots")


CASES = [
    # name, B, H, HV, K, V, slots, act, out, conv W, layout, bias, norm, row pad
    ("k16_v7_gqa2_w2_f16", 9, 4, 8, 16, 7, 9, "f16", "f16", 2, "DS", True, None, 0),
    ("k32_v100_w3_f32_sd", 3, 2, 2, 32, 100, 4, "f32", "f32", 3, "SD", True, None, 8),
    ("k64_gqa4_v128_norm_silu", 6, 2, 8, 64, 128, 6, "bf16", "bf16", 4, "DS", False, "silu", 0),
    ("k256_v64_gqa4_norm_sigmoid", 2, 1, 4, 256, 64, 3, "bf16", "f32", 4, "SD", True, "sigmoid", 0),
    ("k128_v200_gqa2_w5_runtime_width", 3, 2, 4, 128, 200, 5, "bf16", "bf16", 5, "DS", True, None, 0),
    ("k128_gqa16_v128_conv_chunks", 2, 1, 16, 128, 128, 3, "bf16", "bf16", 4, "SD", True, "silu", 24),
    ("k128_v1_w8", 4, 1, 2, 128, 1, 4, "f32", "f32", 8, "DS", True, None, 0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gdn_conv_shapes_dtypes_options(case):
    """Every head size, GQA groups of 1 to 16 value heads (a group of 16
    needs several conv chunks per block), ragged row counts, conv widths
    2 to 8 (4 is compiled separately), both conv-state layouts, conv bias on
    and off, the gated RMSNorm with either gate activation, a row stride wider
    than the row, and every activation/output dtype."""
    need_gpu()
    name, B, H, HV, K, V, slots, act, outd, Wd, layout, bias, norm, pad = case
    w = W.GDNWorkload("gdn_conv_" + name, B=B, H=H, HV=HV, K=K, V=V, num_slots=slots, act=act, out=outd,
                      idx="perm")
    P, idx, cv, st, cs_d = _setup(w, Wd, layout, bias)
    x = W.gdn_step_inputs(w, norm=norm is not None)
    st_d = st.to(DEV)
    out = _gpu(w, st_d, cs_d, idx, x, P, cv, outd, norm=norm is not None, norm_act=norm or "silu",
               row_pad=pad)
    ref, ref_cs = st.double().numpy().copy(), cv["conv_state"].double().numpy().copy()
    ro = _oracle(w, ref, ref_cs, idx, x, P, cv, norm=norm is not None, norm_act=norm or "silu")
    _check_out(out, ro, "output")
    np.testing.assert_array_equal(cs_d.cpu().double().numpy(), ref_cs)
    named = idx.tolist()
    assert_mixed(st_d.cpu()[named], ref[named], FP32_TOL, "state")


def test_gdn_conv_chain_32_steps():
    """32 chained steps: the conv window and the state both carry over; after
    W - 1 steps the conv state holds only inputs of this chain."""
    need_gpu()
    w = W.GDNWorkload("gdn_conv_chain", B=8, H=4, HV=8, K=128, V=128, num_slots=10, idx="perm", out="f32")
    P, idx, cv, st, cs_d = _setup(w)
    st_d = st.to(DEV)
    ref, ref_cs = st.double().numpy().copy(), cv["conv_state"].double().numpy().copy()
    for t in range(32):
        x = W.gdn_step_inputs(w, t)
        out = _gpu(w, st_d, cs_d, idx, x, P, cv, "f32")
        ro = _oracle(w, ref, ref_cs, idx, x, P, cv)
        assert_mixed(out.reshape(w.B, w.HV, w.V), ro, CHAIN_TOL, f"step {t} output")
    np.testing.assert_array_equal(cs_d.cpu().double().numpy(), ref_cs)
    named = idx.tolist()
    assert_mixed(st_d.cpu()[named], ref[named], CHAIN_TOL, "state after 32 steps")


def test_gdn_conv_equals_conv_then_packed_step():
    """With the conv output rounded to the activation dtype by the caller,
    the unfused pair (oracle conv, then gdn_decode_step on the GPU) sees the
    same q, k, v up to that rounding: both agree with their oracles, and the
    fused call's conv state matches the oracle conv's bit for bit."""
    need_gpu()
    w = W.GDNWorkload("gdn_conv_vs_unfused", B=4, H=2, HV=4, K=128, V=128, num_slots=4, act="f32", out="f32")
    P, idx, cv, st, cs_d = _setup(w)
    x = W.gdn_step_inputs(w)
    cs_ref = cv["conv_state"].double().numpy().copy()
    y = O.conv1d_update(x["qkv"], cv["conv_weight"], cv["conv_bias"], cs_ref, idx, skip_slot0=False)
    st_a, st_b = st.to(DEV), st.to(DEV)
    out_f = _gpu(w, st_a, cs_d, idx, x, P, cv, "f32")
    out_u = torch.empty_like(out_f)
    S.gdn_decode_step(torch.from_numpy(y).float().to(DEV), x["a"].to(DEV), x["b"].to(DEV),
                      P["A_log"].to(DEV), P["dt_bias"].to(DEV), st_b, idx.to(DEV), out_u)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(cs_d.cpu().double().numpy(), cs_ref)
    assert_mixed(out_f.cpu(), out_u.cpu().double().numpy(), FP32_TOL, "fused vs unfused output")
    assert_mixed(st_a.cpu(), st_b.cpu().double().numpy(), FP32_TOL, "fused vs unfused state")


# Shapes the persistent kernel takes (conv width 4, no output norm, G V = 256 at
# K = 64 or 128, at least two (row, q/k head) groups per CU): the grid walks the
# groups with a stride, so these counts leave a ragged last walk, and padded
# rows, which the walk must skip while keeping its barriers, sit among them.
PF_CASES = [
    # name, B, H, HV, K, V, slots, act, out, layout, bias, pad every, row pad
    ("k128_b264_h2_bf16_pad7", 264, 2, 4, 128, 128, 270, "bf16", "bf16", "DS", True, 7, 0),
    ("k128_b300_h2_f32_sd", 300, 2, 4, 128, 128, 301, "f32", "f32", "SD", False, 0, 16),
    ("k64_b280_h2_gqa4_v64_f16", 280, 2, 8, 64, 64, 290, "f16", "f32", "DS", True, 5, 0),
    ("k128_b520_h1_pad3_f16_out", 520, 1, 2, 128, 128, 530, "bf16", "f16", "SD", True, 3, 0),
    ("k128_b1_h1_one_group", 1, 1, 2, 128, 128, 2, "bf16", "bf16", "DS", True, 0, 0),
    ("k128_b6_h2_all_padded", 6, 2, 4, 128, 128, 8, "bf16", "bf16", "DS", True, 1, 0),
]


@pytest.mark.parametrize("case", PF_CASES, ids=[c[0] for c in PF_CASES])
def test_gdn_conv_persistent_walk(case):
    """The persistent conv-fused kernel against the oracle element by element:
    outputs, states, the rolled conv state bit for bit, and padded rows and
    unnamed slots left untouched."""
    need_gpu()
    name, B, H, HV, K, V, slots, act, outd, layout, bias, pad_every, row_pad = case
    w = W.GDNWorkload("gdn_conv_pf_" + name, B=B, H=H, HV=HV, K=K, V=V, num_slots=slots, act=act, out=outd,
                      idx="perm")
    P, idx, cv, st, cs_d = _setup(w, 4, layout, bias)
    if pad_every:
        idx[::pad_every] = -1
    x = W.gdn_step_inputs(w)
    st_d = st.to(DEV)
    out = _gpu(w, st_d, cs_d, idx, x, P, cv, outd, sentinel=7.0, row_pad=row_pad)
    ref, ref_cs = st.double().numpy().copy(), cv["conv_state"].double().numpy().copy()
    ro = _oracle(w, ref, ref_cs, idx, x, P, cv)
    act_rows = [b for b in range(B) if idx[b] >= 0]
    pad_rows = [b for b in range(B) if idx[b] < 0]
    if act_rows:
        _check_out(out[act_rows], ro[act_rows], "output")
    if pad_rows:
        assert (out[pad_rows].float().cpu() == 7.0).all(), "padded row output written"
    got, got_cs = st_d.cpu(), cs_d.cpu()
    np.testing.assert_array_equal(got_cs.double().numpy(), ref_cs)
    named = set(idx[idx >= 0].tolist())
    if named:
        assert_mixed(got[sorted(named)], ref[sorted(named)], FP32_TOL, "state")
    for s in range(slots):
        if s not in named:
            assert torch.equal(got[s], st[s]), f"unnamed slot {s} changed"
            assert torch.equal(got_cs[s], cv["conv_state"][s]), f"unnamed slot {s}: conv state changed"


def test_gdn_conv_persistent_chain_8_steps():
    """Eight chained steps on the persistent kernel (512 groups): conv window
    and state carry over from step to step."""
    need_gpu()
    w = W.GDNWorkload("gdn_conv_pf_chain", B=256, H=2, HV=4, K=128, V=128, num_slots=260, idx="perm", out="f32")
    P, idx, cv, st, cs_d = _setup(w)
    st_d = st.to(DEV)
    ref, ref_cs = st.double().numpy().copy(), cv["conv_state"].double().numpy().copy()
    for t in range(8):
        x = W.gdn_step_inputs(w, t)
        out = _gpu(w, st_d, cs_d, idx, x, P, cv, "f32")
        ro = _oracle(w, ref, ref_cs, idx, x, P, cv)
        assert_mixed(out.reshape(w.B, w.HV, w.V), ro, CHAIN_TOL, f"step {t} output")
    np.testing.assert_array_equal(cs_d.cpu().double().numpy(), ref_cs)
    named = idx.tolist()
    assert_mixed(st_d.cpu()[named], ref[named], CHAIN_TOL, "state after 8 steps")
