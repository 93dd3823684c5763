"""GPU parity of gdn_decode_step (through the C ABI) against the fp64 oracle.

Every case runs the same seeded inputs (workloads/) through the HIP kernel and
through oracle/, and compares element by element: fp32 outputs and states to
the mixed relative error 1e-4 (single step) or 2e-3 (chained), 16-bit outputs
to the RNE of the exact value (the other neighbour only where a rounding
midpoint lies within the fp32 bar), and slot placement / untouched memory bit
for bit.
"""
import pytest
import torch

import oracle as O
import ssm_recurrent_decode_gated_amd as S
import workloads as W
from tests._helpers import CHAIN_TOL, FP32_TOL, assert_out16, assert_mixed, need_gpu, to_np64

pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _run(w, state_d, idx, x, P, out_dtype, norm=False, norm_act="silu", sentinel=None):
    dev = state_d.device
    out = torch.full((w.B, 1, w.HV, w.V), float("nan") if sentinel is None else sentinel,
                     dtype=TD[out_dtype], device=dev)
    kw = {}
    if norm:
        kw = dict(norm_gate=x["norm_gate"].to(dev), norm_weight=x["norm_weight"].to(dev), norm_act=norm_act)
    S.gdn_decode_step(x["qkv"].to(dev), x["a"].to(dev), x["b"].to(dev), P["A_log"].to(dev),
                      P["dt_bias"].to(dev), state_d, idx.to(dev), out, **kw)
    return out


def _oracle(w, ref_state, idx, x, P, norm=False, norm_act="silu"):
    kw = {}
    if norm:
        kw = dict(norm_gate=x["norm_gate"], norm_weight=x["norm_weight"],
                  norm_act=O.ACT_SIGMOID if norm_act == "sigmoid" else O.ACT_SILU)
    return O.gdn_step(x["qkv"], x["a"], x["b"], P["A_log"], P["dt_bias"], ref_state, idx,
                      H=w.H, HV=w.HV, K=w.K, V=w.V, **kw)


def _check_out(out, ref, what):
    B, _, HV, V = out.shape
    if out.dtype == torch.float32:
        assert_mixed(out.reshape(B, HV, V), ref, FP32_TOL, what)
    else:
        assert_out16(out.reshape(B, HV, V), ref, FP32_TOL, what)


def test_gdn_tiny_fp32_chain_64_steps():
    """B=2, H=HV=2, K=V=16, fp32 everywhere, 64 chained steps; the oracle keeps
    its own fp64 trajectory."""
    need_gpu()
    w = W.GDN_TINY
    P, idx = W.gdn_params(w), W.slot_indices(w)
    st = W.gdn_state(w)
    st_d, ref = st.to(DEV), st.double().numpy().copy()
    for t in range(w.steps):
        x = W.gdn_step_inputs(w, t)
        out = _run(w, st_d, idx, x, P, "f32")
        ro = _oracle(w, ref, idx, x, P)
        _check_out(out, ro, f"step {t} output")
    assert_mixed(st_d, ref, FP32_TOL, "state after 64 steps")


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_gdn_b16_single_step(out_dtype):
    """B=16 slots (identity), H=16, HV=32, K=V=128, bf16 activations."""
    need_gpu()
    w = W.GDN_B16
    P, idx, x = W.gdn_params(w), W.slot_indices(w), W.gdn_step_inputs(w)
    st = W.gdn_state(w)
    st_d, ref = st.to(DEV), st.double().numpy().copy()
    out = _run(w, st_d, idx, x, P, out_dtype)
    ro = _oracle(w, ref, idx, x, P)
    torch.cuda.synchronize()
    _check_out(out, ro, "output")
    assert_mixed(st_d, ref, FP32_TOL, "state")


def test_gdn_b256_of_264_full_size():
    """The bandwidth workload at full size, in the launch configuration the
    benchmark times: 256 rows over a 264-slot pool with permuted indices.
    Every output and state element is compared; the 8 unnamed slots must be
    bit-identical to their initial contents."""
    need_gpu()
    w = W.GDN_B256
    P, idx, x = W.gdn_params(w), W.slot_indices(w), W.gdn_step_inputs(w)
    st = W.gdn_state(w)
    st_d = st.to(DEV)
    out = _run(w, st_d, idx, x, P, "bf16")
    ref = st.double().numpy()
    ro = _oracle(w, ref, idx, x, P)
    got = st_d.cpu()
    _check_out(out, ro, "output")
    named = set(idx.tolist())
    for s in range(w.num_slots):
        if s in named:
            assert_mixed(got[s], ref[s], FP32_TOL, f"slot {s}")
        else:
            assert torch.equal(got[s], st[s]), f"unnamed slot {s} changed"
    assert len(named) == w.B and w.num_slots - len(named) == 8


def test_gdn_padded_rows_touch_nothing():
    need_gpu()
    w = W.GDNWorkload("gdn_pad", B=5, H=2, HV=4, K=128, V=128, num_slots=6)
    P, x = W.gdn_params(w), W.gdn_step_inputs(w)
    idx = torch.tensor([3, -1, 6, 0, 2**31 - 1], dtype=torch.int32)
    st = W.gdn_state(w)
    st_d, ref = st.to(DEV), st.double().numpy().copy()
    out = _run(w, st_d, idx, x, P, "bf16", sentinel=7.0)
    ro = _oracle(w, ref, idx, x, P)
    got = st_d.cpu()
    for b in (1, 2, 4):
        assert (out[b].float().cpu() == 7.0).all(), f"padded row {b} output written"
    _check_out(out[[0, 3]], ro[[0, 3]], "active rows")
    for s in (1, 4, 5):
        assert torch.equal(got[s], st[s])
    assert_mixed(got[[0, 3]], ref[[0, 3]], FP32_TOL, "active slots")


RAGGED = [
    # name, B, H, HV, K, V, slots, act, out
    ("k64_v40_f16", 5, 3, 6, 64, 40, 7, "f16", "f16"),
    ("k32_v100_bf16_f32out", 3, 2, 2, 32, 100, 4, "bf16", "f32"),
    ("k256_v64_f32_bf16out", 2, 1, 4, 256, 64, 3, "f32", "bf16"),
    ("k16_v7_gqa2", 9, 4, 8, 16, 7, 9, "bf16", "bf16"),
    ("k128_v200_two_tiles", 3, 2, 4, 128, 200, 5, "bf16", "f32"),
    ("k128_v1", 4, 1, 2, 128, 1, 4, "f32", "f32"),
    ("k64_gqa4_v128", 6, 2, 8, 64, 128, 6, "bf16", "bf16"),
    ("k256_v1024_max", 2, 1, 2, 256, 1024, 3, "bf16", "f32"),  # largest head the ABI takes
]


@pytest.mark.parametrize("case", RAGGED, ids=[c[0] for c in RAGGED])
def test_gdn_shapes_and_dtypes(case):
    """Ragged row tails, every compiled head size, GQA ratios 1/2/4 and every
    activation/output dtype, with a permuted slot pool."""
    need_gpu()
    name, B, H, HV, K, V, slots, act, outd = case
    w = W.GDNWorkload(name, B=B, H=H, HV=HV, K=K, V=V, num_slots=slots, act=act, out=outd, idx="perm")
    P, idx, x = W.gdn_params(w), W.slot_indices(w), W.gdn_step_inputs(w)
    st = W.gdn_state(w)
    st_d, ref = st.to(DEV), st.double().numpy().copy()
    out = _run(w, st_d, idx, x, P, outd)
    ro = _oracle(w, ref, idx, x, P)
    _check_out(out, ro, "output")
    assert_mixed(st_d, ref, FP32_TOL, "state")


NORM = [("k128_v128_silu", 128, 128, "silu", "bf16"), ("k64_v96_sigmoid", 64, 96, "sigmoid", "f32"),
        ("k128_v300_silu_looped", 128, 300, "silu", "f32"), ("k16_v16_sigmoid", 16, 16, "sigmoid", "bf16"),
        ("k256_v1024_sigmoid_max", 256, 1024, "sigmoid", "f32")]


@pytest.mark.parametrize("case", NORM, ids=[c[0] for c in NORM])
def test_gdn_gated_rmsnorm_epilogue(case):
    need_gpu()
    name, K, V, act_fn, outd = case
    w = W.GDNWorkload("gdn_norm_" + name, B=4, H=2, HV=4, K=K, V=V, num_slots=5, out=outd, idx="perm")
    P, idx, x = W.gdn_params(w), W.slot_indices(w), W.gdn_step_inputs(w, norm=True)
    st = W.gdn_state(w)
    st_d, ref = st.to(DEV), st.double().numpy().copy()
    out = _run(w, st_d, idx, x, P, outd, norm=True, norm_act=act_fn)
    ro = _oracle(w, ref, idx, x, P, norm=True, norm_act=act_fn)
    _check_out(out, ro, "normed output")
    assert_mixed(st_d, ref, FP32_TOL, "state")


def test_gdn_no_l2norm_and_explicit_scale():
    need_gpu()
    w = W.GDNWorkload("gdn_nol2", B=3, H=2, HV=2, K=64, V=64, num_slots=3, act="f32", out="f32")
    P, idx, x = W.gdn_params(w), W.slot_indices(w), W.gdn_step_inputs(w)
    x = dict(x, qkv=x["qkv"] * 0.05)  # keep |k| small so the unnormalised rule stays tame
    st = W.gdn_state(w)
    st_d, ref = st.to(DEV), st.double().numpy().copy()
    out = torch.empty(w.B, 1, w.HV, w.V, device=DEV)
    S.gdn_decode_step(x["qkv"].to(DEV), x["a"].to(DEV), x["b"].to(DEV), P["A_log"].to(DEV),
                      P["dt_bias"].to(DEV), st_d, idx.to(DEV), out, scale=0.3, use_qk_l2norm=False)
    ro = O.gdn_step(x["qkv"], x["a"], x["b"], P["A_log"], P["dt_bias"], ref, idx, H=w.H, HV=w.HV, K=w.K,
                    V=w.V, scale=0.3, use_l2=False)
    _check_out(out, ro, "output")
    assert_mixed(st_d, ref, FP32_TOL, "state")


def test_gdn_strided_qkv_rows():
    """mixed_qkv rows with a padded row stride (a view into a wider buffer)."""
    need_gpu()
    w = W.GDNWorkload("gdn_stride", B=4, H=2, HV=4, K=128, V=128, num_slots=4)
    P, idx, x = W.gdn_params(w), W.slot_indices(w), W.gdn_step_inputs(w)
    wide = torch.zeros(w.B, x["qkv"].shape[1] + 64, dtype=x["qkv"].dtype, device=DEV)
    wide[:, 16:16 + x["qkv"].shape[1]] = x["qkv"].to(DEV)
    view = wide[:, 16:16 + x["qkv"].shape[1]]
    st = W.gdn_state(w)
    st_d, ref = st.to(DEV), st.double().numpy().copy()
    out = torch.empty(w.B, 1, w.HV, w.V, device=DEV)
    S.gdn_decode_step(view, x["a"].to(DEV), x["b"].to(DEV), P["A_log"].to(DEV), P["dt_bias"].to(DEV),
                      st_d, idx.to(DEV), out)
    ro = _oracle(w, ref, idx, x, P)
    _check_out(out, ro, "output")


@pytest.mark.slow
def test_gdn_b64_1000_step_drift():
    """1000 chained steps at B=64, H=16, HV=32, K=V=128 with fresh inputs per
    step. The oracle follows all 64 rows (2048 heads) on its own fp64
    trajectory; outputs at steps 1, 10, 100, 1000 and the final state of
    every row must stay within 2e-3 of it."""
    need_gpu()
    w = W.GDN_B64_CHAIN
    P, idx = W.gdn_params(w), W.slot_indices(w)
    st = W.gdn_state(w)
    st_d = st.to(DEV)
    ref = st.double().numpy().copy()
    Pd = {k: v.to(DEV) for k, v in P.items()}
    idx_d = idx.to(DEV)
    out = torch.empty(w.B, 1, w.HV, w.V, dtype=torch.bfloat16, device=DEV)
    out32 = torch.empty(w.B, 1, w.HV, w.V, dtype=torch.float32, device=DEV)
    checks = {1, 10, 100, 1000}
    for t in range(1, w.steps + 1):
        x = W.gdn_step_inputs(w, t)
        o = out32 if t in checks else out
        S.gdn_decode_step(x["qkv"].to(DEV), x["a"].to(DEV), x["b"].to(DEV), Pd["A_log"], Pd["dt_bias"],
                          st_d, idx_d, o)
        ro = O.gdn_step(x["qkv"], x["a"], x["b"], P["A_log"], P["dt_bias"], ref, idx, H=w.H, HV=w.HV, K=w.K,
                        V=w.V)
        if t in checks:
            assert_mixed(out32.reshape(w.B, w.HV, w.V), ro, CHAIN_TOL, f"output at step {t}")
    assert_mixed(st_d, ref, CHAIN_TOL, "state after 1000 steps")
