"""GPU parity of gdn_decode_step_state16 (the packed GDN step on a bf16 / f16
state pool) against the fp64 oracle run with the same storage format.

Single steps start both sides from the same 16-bit pool: outputs (formed from
the unrounded update) to the fp32 bar, stored rows equal to the RNE of the
exact update (the other neighbour only where the exact value sits at a
rounding midpoint, where both are correct roundings), untouched slots bit for
bit. Chained runs hold every step to the same bars: the oracle takes the
kernel's rounding choice at validated midpoints, so each step starts both
sides from the same stored state."""
import pytest
import torch

import oracle as O
import ssm_recurrent_decode_gated_amd as S
import workloads as W
from tests._helpers import (FP32_TOL, assert_mixed, assert_out16, assert_rounded16, need_gpu,
                            take_valid_roundings, to_np64)

pytestmark = pytest.mark.gpu
DEV = "cuda"
FMT = {torch.bfloat16: O.FMT_BF16, torch.float16: O.FMT_F16}


def _state16(w, sdt, slots=None):
    # draw the pool at the workload's scale, then store it in the 16-bit format
    return W.gdn_state(w, slots=slots).to(sdt)


def _assert_state16(got, ref, sdt, what, exact):
    """The stored row is the fp32 update rounded once: the RNE of a value
    within the fp32 bar of the exact update (an element near zero, where
    e^g S and delta k cancel, carries an fp32 error of the row's size), and
    different from the oracle's rounding only where the exact update sits at
    a rounding midpoint."""
    assert_out16(got, exact, FP32_TOL, what)
    assert_rounded16(to_np64(got), ref, what, exact, 7 if sdt == torch.bfloat16 else 10)


def _run(w, sdt, out_dtype, norm=False, norm_act="silu", x=None, st=None, idx=None):
    P = W.gdn_params(w)
    idx = W.slot_indices(w) if idx is None else idx
    x = W.gdn_step_inputs(w, norm=norm) if x is None else x
    st = _state16(w, sdt) if st is None else st
    st_d = st.to(DEV)
    out = torch.full((w.B, 1, w.HV, w.V), 7.0, dtype=out_dtype, device=DEV)
    kw = dict(norm_gate=x["norm_gate"].to(DEV), norm_weight=x["norm_weight"].to(DEV), norm_act=norm_act) if norm else {}
    S.gdn_decode_step_state16(x["qkv"].to(DEV), x["a"].to(DEV), x["b"].to(DEV), P["A_log"].to(DEV),
                              P["dt_bias"].to(DEV), st_d, idx.to(DEV), out, **kw)
    ref = st.double().numpy().copy()
    okw = dict(norm_gate=x["norm_gate"], norm_weight=x["norm_weight"],
               norm_act=O.ACT_SIGMOID if norm_act == "sigmoid" else O.ACT_SILU) if norm else {}
    ro = O.gdn_step(x["qkv"], x["a"], x["b"], P["A_log"], P["dt_bias"], ref, idx, H=w.H, HV=w.HV, K=w.K,
                    V=w.V, state_fmt=FMT[sdt], **okw)
    exact = st.double().numpy().copy()  # the same update, not rounded on store
    O.gdn_step(x["qkv"], x["a"], x["b"], P["A_log"], P["dt_bias"], exact, idx, H=w.H, HV=w.HV, K=w.K, V=w.V,
               state_fmt=O.FMT_NONE, **okw)
    torch.cuda.synchronize()
    return out, st_d.cpu(), st, ro, ref, idx, exact


def _check(w, sdt, out, got, st0, ro, ref, idx, exact):
    B, _, HV, V = out.shape
    if out.dtype == torch.float32:
        assert_mixed(out.reshape(B, HV, V).cpu(), ro, FP32_TOL, "output")
    else:
        assert_out16(out.reshape(B, HV, V), ro, FP32_TOL, "output")
    named = set(idx.tolist())
    for s in range(w.num_slots):
        if s in named:
            _assert_state16(got[s], ref[s], sdt, f"slot {s}", exact[s])
        else:
            assert torch.equal(got[s], st0[s]), f"unnamed slot {s} changed"


@pytest.mark.parametrize("sdt", [torch.bfloat16, torch.float16])
def test_state16_b256_of_264_full_size(sdt):
    need_gpu()
    w = W.GDN_B256
    out, got, st0, ro, ref, idx, exact = _run(w, sdt, torch.bfloat16)
    _check(w, sdt, out, got, st0, ro, ref, idx, exact)


CASES = [
    ("k128_b16_f32out", 16, 16, 32, 128, 128, 16, "bf16", torch.float32),
    ("k64_v40_f16act", 5, 3, 6, 64, 40, 7, "f16", torch.float16),
    ("k16_v7", 9, 4, 8, 16, 7, 9, "bf16", torch.bfloat16),
    ("k32_v100", 3, 2, 2, 32, 100, 4, "f32", torch.float32),
    ("k256_v64", 2, 1, 4, 256, 64, 3, "bf16", torch.float32),
    ("k128_v200", 3, 2, 4, 128, 200, 5, "bf16", torch.float32),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("sdt", [torch.bfloat16, torch.float16])
def test_state16_shapes(case, sdt):
    need_gpu()
    name, B, H, HV, K, V, slots, act, outd = case
    w = W.GDNWorkload("s16_" + name, B=B, H=H, HV=HV, K=K, V=V, num_slots=slots, act=act, idx="perm")
    out, got, st0, ro, ref, idx, exact = _run(w, sdt, outd)
    _check(w, sdt, out, got, st0, ro, ref, idx, exact)


# More row tiles than four per CU on a 256-CU part: these take the launch with
# one block per tile (no walk), over every head size, ragged V and GQA groups.
TILE_CASES = [
    ("k256_v100_gqa4_f16act", 40, 2, 8, 256, 100, 41, "f16", torch.float32),
    ("k128_v200_gqa2", 12, 4, 8, 128, 200, 13, "bf16", torch.bfloat16),
    ("k64_v40_gqa16", 70, 1, 16, 64, 40, 72, "bf16", torch.float32),
    ("k32_v200", 20, 16, 16, 32, 200, 21, "f32", torch.float16),
    ("k16_v7_gqa8", 130, 1, 8, 16, 7, 131, "bf16", torch.float32),
]


@pytest.mark.parametrize("case", TILE_CASES, ids=[c[0] for c in TILE_CASES])
@pytest.mark.parametrize("sdt", [torch.bfloat16, torch.float16])
def test_state16_one_block_per_tile(case, sdt):
    need_gpu()
    name, B, H, HV, K, V, slots, act, outd = case
    w = W.GDNWorkload("s16_tiles_" + name, B=B, H=H, HV=HV, K=K, V=V, num_slots=slots, act=act, idx="perm")
    out, got, st0, ro, ref, idx, exact = _run(w, sdt, outd)
    _check(w, sdt, out, got, st0, ro, ref, idx, exact)


@pytest.mark.parametrize("V,act_fn", [(128, "silu"), (300, "sigmoid")])
def test_state16_gated_norm(V, act_fn):
    need_gpu()
    w = W.GDNWorkload(f"s16_norm_v{V}", B=4, H=2, HV=4, K=128, V=V, num_slots=5, idx="perm")
    out, got, st0, ro, ref, idx, exact = _run(w, torch.bfloat16, torch.float32, norm=True, norm_act=act_fn)
    _check(w, torch.bfloat16, out, got, st0, ro, ref, idx, exact)


def test_state16_padding_many_units():
    """More units than blocks, with padded rows among them."""
    need_gpu()
    w = W.GDNWorkload("s16_pad", B=300, H=1, HV=2, K=128, V=128, num_slots=280)
    idx = torch.arange(300, dtype=torch.int32)
    idx[::7] = -1
    idx[idx >= 280] = 280  # out of range -> padded
    out, got, st0, ro, ref, _, exact = _run(w, torch.bfloat16, torch.float32, idx=idx)
    act = (idx >= 0) & (idx < 280)
    assert (out[~act].cpu() == 7.0).all()
    assert_mixed(out[act].reshape(-1, w.HV, w.V).cpu(), ro[act.numpy()], FP32_TOL, "active outputs")
    for s in range(w.num_slots):
        if s in set(idx[act].tolist()):
            _assert_state16(got[s], ref[s], torch.bfloat16, f"slot {s}", exact[s])
        else:
            assert torch.equal(got[s], st0[s])


def test_state16_chain_200_steps():
    """200 chained steps at B = 16 on a bf16 pool. After each step the
    kernel's stored rows are checked against the oracle's rounding of the
    exact update (equal, or the other neighbour where the exact value sits at
    a rounding midpoint) and the oracle continues from its own rounding with
    the kernel's choice taken at exactly those midpoints
    (take_valid_roundings): both sides then start every step from the same
    stored state, and every step's outputs (all rows) must meet the
    single-step fp32 bar."""
    need_gpu()
    w = W.GDN_B16
    P, idx = W.gdn_params(w), W.slot_indices(w)
    st = _state16(w, torch.bfloat16)
    st_d = st.to(DEV)
    ref = st.double().numpy().copy()
    out = torch.empty(w.B, 1, w.HV, w.V, device=DEV)
    Pd = {k: v.to(DEV) for k, v in P.items()}
    kw = dict(H=w.H, HV=w.HV, K=w.K, V=w.V)
    taken = 0
    for t in range(200):
        x = W.gdn_step_inputs(w, 7000 + t)
        S.gdn_decode_step_state16(x["qkv"].to(DEV), x["a"].to(DEV), x["b"].to(DEV), Pd["A_log"], Pd["dt_bias"],
                                  st_d, idx.to(DEV), out)
        args = (x["qkv"], x["a"], x["b"], P["A_log"], P["dt_bias"])
        exact = ref.copy()
        O.gdn_step(*args, exact, idx, state_fmt=O.FMT_NONE, **kw)
        ro = O.gdn_step(*args, ref, idx, state_fmt=O.FMT_BF16, **kw)
        assert_mixed(out.reshape(w.B, w.HV, w.V), ro, FP32_TOL, f"output at step {t + 1}")
        ref, n = take_valid_roundings(to_np64(st_d), ref, exact, 7, f"state after step {t + 1}")
        taken += n
    print(f"{taken} midpoint rounding choices taken from the kernel over 200 steps")
