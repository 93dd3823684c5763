"""GPU parity of kda_decode_step (fused conv1d update + KDA delta rule +
sigmoid-gated RMSNorm) against the fp64 oracle: outputs and states to the
fp32 tolerance (16-bit outputs: RNE of the exact value), the rolled conv state bit for bit
(it holds raw inputs), and skipped tokens (slot 0 = NULL block, out of range)
touching nothing."""
import numpy as np
import pytest
import torch

import oracle as O
import ssm_recurrent_decode_gated_amd as S
import workloads as W
from tests._helpers import FP32_TOL, assert_out16, assert_mixed, need_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run_both(w, d, *, with_norm=True, conv_bias=None, out_dtype=torch.bfloat16):
    H, D, T = w.H, w.D, w.T
    cs_d = d["conv_state"].to(DEV)
    assert cs_d.stride() == d["conv_state"].stride()
    st_d = d["state"].to(DEV)
    out = torch.full((T, H, D), 7.0, dtype=out_dtype, device=DEV)
    S.kda_decode_step(d["x"].to(DEV), d["conv_weight"].to(DEV),
                      None if conv_bias is None else conv_bias.to(DEV), cs_d, d["raw_g"].to(DEV),
                      d["raw_beta"].to(DEV), None, None, st_d, d["idx"].to(DEV), out,
                      output_gate=d["gate"].to(DEV) if with_norm else None,
                      norm_weight=d["norm_weight"].to(DEV) if with_norm else None,
                      lower_bound=w.lower_bound, norm_eps=w.norm_eps)
    cs_ref = d["conv_state"].double().numpy().copy()  # logical [slots, C, W-1], contiguous copy
    st_ref = d["state"].double().numpy().copy()
    ro = O.kda_decode(d["x"], d["conv_weight"], conv_bias, cs_ref, d["raw_g"], d["raw_beta"], st_ref, d["idx"],
                      H=H, D=D, lower_bound=w.lower_bound,
                      gate=d["gate"] if with_norm else None,
                      norm_weight=d["norm_weight"] if with_norm else None, norm_eps=w.norm_eps)
    torch.cuda.synchronize()
    return out, st_d.cpu(), cs_d.cpu(), ro, st_ref, cs_ref


def _active(idx, num_slots):
    return [t for t, s in enumerate(idx.tolist()) if 0 < s < num_slots]


@pytest.mark.parametrize("layout", ["SD", "DS"])
def test_kda_t64_h96_full_size(layout):
    """T=64 tokens, 96 heads x 128, conv width 4, slots 1..64 of 72, bf16
    activations, gate -5 sigmoid(a), sigmoid-gated RMSNorm with eps 1e-5."""
    need_gpu()
    w = W.KDA_T64
    d = W.kda_inputs(w, layout=layout)
    out, st, cs, ro, st_ref, cs_ref = _run_both(w, d)
    assert_out16(out, ro, FP32_TOL, "output")
    slots = d["idx"].tolist()
    assert_mixed(st[slots], st_ref[slots], FP32_TOL, "state of named slots")
    np.testing.assert_array_equal(cs.double().numpy(), cs_ref)
    for s in set(range(w.num_slots)) - set(slots):
        assert torch.equal(st[s], d["state"][s]), f"unnamed slot {s} changed"


def test_kda_skips_null_slot_and_out_of_range():
    need_gpu()
    w = W.KDAWorkload("kda_skip", T=5, H=3, D=128, num_slots=6)
    d = W.kda_inputs(w)
    d["idx"] = torch.tensor([2, 0, 5, 6, -3], dtype=torch.int32)
    out, st, cs, ro, st_ref, cs_ref = _run_both(w, d)
    for t in (1, 3, 4):
        assert (out[t].float().cpu() == 7.0).all(), f"skipped token {t} wrote output"
    act = _active(d["idx"], w.num_slots)
    assert_out16(out[act], ro[act], FP32_TOL, "active outputs")
    np.testing.assert_array_equal(cs.double().numpy(), cs_ref)
    for s in (0, 1, 3, 4):
        assert torch.equal(st[s], d["state"][s])


SMALL = [
    # name, T, H, D, W, act dtype, out dtype, norm, conv bias
    ("d64_w3_f32_bias", 6, 4, 64, 3, "f32", torch.float32, False, True),
    ("d32_w4_bf16_norm_bias", 5, 2, 32, 4, "bf16", torch.bfloat16, True, True),
    ("d16_w2_f16", 7, 3, 16, 2, "f16", torch.float16, True, False),
    ("d256_w4_bf16", 3, 2, 256, 4, "bf16", torch.float32, True, False),
    ("d128_w4_nonorm", 4, 5, 128, 4, "bf16", torch.bfloat16, False, False),
    ("d128_w4_norm_bias", 9, 3, 128, 4, "bf16", torch.bfloat16, True, True),
    ("d64_w4_f16", 6, 4, 64, 4, "f16", torch.float32, True, False),
    ("d64_w4_f32_nonorm", 5, 2, 64, 4, "f32", torch.float32, False, True),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_kda_shapes_dtypes_options(case):
    """Every head size, conv widths 2-4, fp32/f16 activations (the conv state
    then is that dtype too), conv bias, norm on/off; head sizes 64 and 128 at
    width 4 run the persistent kernel, the rest the per-unit one."""
    need_gpu()
    name, T, H, D, Wd, act, outd, norm, bias = case
    w = W.KDAWorkload("kda_" + name, T=T, H=H, D=D, W=Wd, num_slots=T + 3)
    d = W.kda_inputs(w, layout="DS" if T % 2 else "SD")
    if act != "bf16":
        for k in ("x", "raw_g", "raw_beta", "gate", "conv_state"):
            d[k] = d[k].to(W.DTYPES[act])
    g = W.generator(0, name, "extra")
    conv_bias = W.normal((3 * H * D,), 0.5, "f32", g) if bias else None
    out, st, cs, ro, st_ref, cs_ref = _run_both(w, d, with_norm=norm, conv_bias=conv_bias, out_dtype=outd)
    act_t = _active(d["idx"], w.num_slots)
    if outd == torch.float32:
        assert_mixed(out[act_t].cpu(), ro[act_t], FP32_TOL, "output")
    else:
        assert_out16(out[act_t], ro[act_t], FP32_TOL, "output")
    slots = d["idx"].tolist()
    assert_mixed(st[slots], st_ref[slots], FP32_TOL, "state")
    np.testing.assert_array_equal(cs.double().numpy(), cs_ref)


def test_kda_many_tokens_with_skips_interleaved():
    """More (token, head) units than persistent blocks, with NULL-slot and
    out-of-range tokens interleaved: every block walks several units and
    skips some between computed ones, and every computed output and state
    still matches the oracle."""
    need_gpu()
    w = W.KDAWorkload("kda_interleaved_skips", T=600, H=2, D=128, num_slots=460)
    d = W.kda_inputs(w)
    idx = torch.arange(1, w.T + 1, dtype=torch.int32)
    idx[::7] = 0                  # NULL block
    idx[3::11] = w.num_slots + 5  # out of range
    idx[idx > w.num_slots - 1] = -1
    d["idx"] = idx
    out, st, cs, ro, st_ref, cs_ref = _run_both(w, d)
    act = _active(d["idx"], w.num_slots)
    assert len(act) > 300 and len(act) < w.T
    assert_out16(out[act], ro[act], FP32_TOL, "active outputs")
    skipped = [t for t in range(w.T) if t not in set(act)]
    assert (out[skipped].float().cpu() == 7.0).all(), "a skipped token wrote output"
    slots = sorted(set(d["idx"][act].tolist()))
    assert_mixed(st[slots], st_ref[slots], FP32_TOL, "states of named slots")
    np.testing.assert_array_equal(cs.double().numpy(), cs_ref)


@pytest.mark.parametrize("which", ["A_log", "dt_bias", "both"])
def test_kda_refuses_A_log_and_dt_bias(which):
    """No page gives the formula by which A_log and dt_bias would enter the
    KDA gate, so the library refuses them: the call raises, and output,
    state and conv state are left exactly as they were (nothing launched)."""
    need_gpu()
    w = W.KDAWorkload("kda_refuse", T=4, H=2, D=128, num_slots=7)
    d = W.kda_inputs(w)
    g = W.generator(0, "kda_refuse", "extra")
    A_log = W.normal((w.H,), 0.3, "f32", g).to(DEV) if which != "dt_bias" else None
    dt_bias = W.normal((w.H * w.D,), 0.1, "f32", g).to(DEV) if which != "A_log" else None
    cs_d, st_d = d["conv_state"].to(DEV), d["state"].to(DEV)
    out = torch.full((w.T, w.H, w.D), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(RuntimeError, match="A_log"):
        S.kda_decode_step(d["x"].to(DEV), d["conv_weight"].to(DEV), None, cs_d, d["raw_g"].to(DEV),
                          d["raw_beta"].to(DEV), A_log, dt_bias, st_d, d["idx"].to(DEV), out,
                          output_gate=d["gate"].to(DEV), norm_weight=d["norm_weight"].to(DEV))
    torch.cuda.synchronize()
    assert (out.float().cpu() == 7.0).all()
    assert torch.equal(st_d.cpu(), d["state"])
    assert torch.equal(cs_d.cpu(), d["conv_state"])
