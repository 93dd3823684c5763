"""GPU parity of gdn_chunk_prefill (the GDN step over T tokens in chunked
form) against the fp64 oracle's token-by-token steps: outputs and final
states, ragged last chunks and row lengths, padding, GQA, both head sizes,
the gated norm, and agreement with the sequential multi-token kernel."""
import numpy as np
import pytest
import torch

import oracle as O
import ssm_recurrent_decode_gated_amd as S
import workloads as W
from tests._helpers import CHAIN_TOL, FP32_TOL, assert_out16, assert_mixed, need_gpu
from tests.test_gdn_multi_gpu import _inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _run(w, T, d, P, st, idx, *, out_dtype="f32", lengths=None, norm=None):
    st_d = st.to(DEV)
    out = torch.full((w.B, T, w.HV, w.V), 7.0, dtype=TD[out_dtype], device=DEV)
    kw = {}
    if norm:
        kw = dict(norm_gate=d["norm_gate"].to(DEV), norm_weight=d["norm_weight"].to(DEV), norm_act=norm)
    S.gdn_chunk_prefill(d["qkv"].to(DEV), d["a"].to(DEV), d["b"].to(DEV), P["A_log"].to(DEV),
                        P["dt_bias"].to(DEV), st_d, idx.to(DEV), out,
                        lengths=None if lengths is None else lengths.to(DEV), **kw)
    ref = st.double().numpy().copy()
    okw = {}
    if norm:
        okw = dict(norm_gate=d["norm_gate"], norm_weight=d["norm_weight"],
                   norm_act=O.ACT_SIGMOID if norm == "sigmoid" else O.ACT_SILU)
    ro = O.gdn_multi(d["qkv"], d["a"], d["b"], P["A_log"], P["dt_bias"], ref, idx, H=w.H, HV=w.HV, K=w.K, V=w.V,
                     lengths=lengths, **okw)
    torch.cuda.synchronize()
    return out, st_d.cpu(), ro, ref


def _check(out, ro, tol, what):
    if out.dtype == torch.float32:
        assert_mixed(out.cpu(), ro, tol, what)
    else:
        assert_out16(out, ro, tol, what)


def test_gdn_chunk_prompt_2048():
    """One 2048-token prompt (32 chunks) at H=16, HV=32, K=V=128, bf16
    activations: every output and the final state. The chunked arithmetic
    stays within the single-step bar here (measured max 2.4e-5); the chained
    bar is what the method is held to over 2048 tokens."""
    need_gpu()
    w = W.GDNWorkload("gdn_chunk_prompt", B=1, H=16, HV=32, K=128, V=128, num_slots=2, out="f32")
    T = 2048
    P, st = W.gdn_params(w), W.gdn_state(w)
    idx = torch.tensor([1], dtype=torch.int32)
    d = _inputs(w, T)
    out, got, ro, ref = _run(w, T, d, P, st, idx)
    _check(out, ro, CHAIN_TOL, "outputs")
    assert_mixed(got[1], ref[1], CHAIN_TOL, "final state")
    assert torch.equal(got[0], st[0]), "unnamed slot changed"


def test_gdn_chunk_ragged_lengths_padding_gqa():
    """T = 150 (last chunk of 22 tokens), lengths 150, 64, 65, 1, 0 and a
    padded row, K = 64, V = 48, GQA 2, fp32."""
    need_gpu()
    w = W.GDNWorkload("gdn_chunk_ragged", B=6, H=2, HV=4, K=64, V=48, num_slots=8, act="f32", out="f32")
    T = 150
    P, st = W.gdn_params(w), W.gdn_state(w)
    d = _inputs(w, T)
    idx = torch.tensor([6, 0, 3, 7, 2, -1], dtype=torch.int32)
    lengths = torch.tensor([150, 64, 65, 1, 0, 150], dtype=torch.int32)
    out, got, ro, ref = _run(w, T, d, P, st, idx, lengths=lengths)
    o = out.cpu()
    for b in range(5):
        L = int(lengths[b])
        if L:
            assert_mixed(o[b, :L], ro[b, :L], FP32_TOL, f"row {b}")
        assert (o[b, L:] == 7.0).all(), f"row {b} wrote past its length"
    assert (o[5] == 7.0).all()
    for s in (6, 0, 3, 7):
        assert_mixed(got[s], ref[s], FP32_TOL, f"slot {s}")
    for s in (1, 2, 4, 5):
        assert torch.equal(got[s], st[s]), f"slot {s} changed"


CASES = [
    # name, B, H, HV, K, V, act, out, T, norm
    ("k128_v128_norm_silu_bf16", 2, 2, 4, 128, 128, "bf16", "bf16", 130, "silu"),
    ("k64_v256_norm_sigmoid_f16", 1, 1, 2, 64, 256, "f16", "f32", 100, "sigmoid"),
    ("k128_v64_gqa4_f32", 3, 1, 4, 128, 64, "f32", "f32", 64, None),
    ("k64_v16_bf16_short", 4, 2, 2, 64, 16, "bf16", "bf16", 5, None),
    ("k128_v128_f16_gqa2_ragged_tail", 2, 2, 4, 128, 128, "f16", "f16", 200, None),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gdn_chunk_shapes(case):
    need_gpu()
    name, B, H, HV, K, V, act, outd, T, norm = case
    w = W.GDNWorkload("gdn_chunk_" + name, B=B, H=H, HV=HV, K=K, V=V, num_slots=B + 1, act=act, out=outd,
                      idx="perm")
    P, idx, st = W.gdn_params(w), W.slot_indices(w), W.gdn_state(w)
    d = _inputs(w, T, norm=norm is not None)
    out, got, ro, ref = _run(w, T, d, P, st, idx, out_dtype=outd, norm=norm)
    _check(out, ro, FP32_TOL, "outputs")
    named = idx.tolist()
    assert_mixed(got[named], ref[named], FP32_TOL, "states")


def test_gdn_chunk_matches_fused_recurrent():
    """The chunked and the sequential multi-token kernels on the same 300
    tokens (5 chunks) agree to the fp32 bar."""
    need_gpu()
    w = W.GDNWorkload("gdn_chunk_vs_seq", B=2, H=4, HV=8, K=128, V=128, num_slots=2, out="f32")
    T = 300
    P, idx, st = W.gdn_params(w), W.slot_indices(w), W.gdn_state(w)
    d = {k: v.to(DEV) for k, v in _inputs(w, T).items()}
    outs, states = [], []
    for fn in (S.gdn_chunk_prefill, S.gdn_fused_recurrent):
        st_d = st.to(DEV)
        o = torch.empty(w.B, T, w.HV, w.V, device=DEV)
        fn(d["qkv"], d["a"], d["b"], P["A_log"].to(DEV), P["dt_bias"].to(DEV), st_d, idx.to(DEV), o)
        outs.append(o.cpu())
        states.append(st_d.cpu())
    torch.cuda.synchronize()
    assert_mixed(outs[0], outs[1].double().numpy(), FP32_TOL, "outputs")
    assert_mixed(states[0], states[1].double().numpy(), FP32_TOL, "states")


def _rows_per_block(B, HV, V, act):
    """The state pass's rows per block as the launcher picks them: the largest
    of 64 / 32 / 16 (32 / 16 for bf16 inputs, which take the split-product
    kernel) dividing V that still gives two blocks per CU."""
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    bh8 = (B * HV + 7) // 8 * 8
    for c in (64, 32):
        if (act != "bf16" or c < 64) and V % c == 0 and bh8 * (V // c) >= 2 * n_cu:
            return c
    return 16


ROW_TILE_CASES = [
    # name, B, H, HV, K, V, act, out, T, norm; sized so the launcher takes 64 or 32 state rows per block
    # (bf16: the split-product kernel at 32 rows; f16 / f32: the fp32-product kernel at 64 and 32)
    ("k128_v128_bf16", 8, 16, 32, 128, 128, "bf16", "f32", 130, None),
    ("k64_v128_f16_norm", 8, 16, 32, 64, 128, "f16", "f16", 70, "silu"),
    ("k128_v128_bf16_norm", 4, 16, 32, 128, 128, "bf16", "bf16", 100, "sigmoid"),
    ("k64_v64_f32", 8, 8, 32, 64, 64, "f32", "f32", 66, None),
]


@pytest.mark.parametrize("case", ROW_TILE_CASES, ids=[c[0] for c in ROW_TILE_CASES])
def test_gdn_chunk_row_tiles(case):
    """Batched prompts, where the state pass holds 32 or 64 state rows per
    block: every output and state, with ragged lengths (a zero-length row and
    a padded row among them)."""
    need_gpu()
    name, B, H, HV, K, V, act, outd, T, norm = case
    vt = _rows_per_block(B, HV, V, act)
    if vt == 16:
        pytest.skip(f"{torch.cuda.get_device_properties(0).multi_processor_count} CUs: 16 rows per block here")
    w = W.GDNWorkload("gdn_chunk_rows_" + name, B=B, H=H, HV=HV, K=K, V=V, num_slots=B + 2, act=act, out=outd,
                      idx="perm")
    P, st = W.gdn_params(w), W.gdn_state(w)
    idx = W.slot_indices(w).clone()
    idx[1] = -1
    lengths = torch.tensor([T - 3 * b if b != 2 else 0 for b in range(B)], dtype=torch.int32)
    d = _inputs(w, T, norm=norm is not None)
    out, got, ro, ref = _run(w, T, d, P, st, idx, out_dtype=outd, lengths=lengths, norm=norm)
    for b in range(B):
        L = int(lengths[b]) if b != 1 else 0
        if L:
            _check(out[b, :L], ro[b, :L], FP32_TOL, f"row {b} (rows per block {vt})")
        if b != 1 and L < T:
            assert (out[b, L:].float() == 7.0).all(), f"row {b} wrote past its length"
    assert (out[1].float() == 7.0).all(), "padded row wrote output"
    live = [int(idx[b]) for b in range(B) if b != 1]
    assert_mixed(got[live], ref[live], FP32_TOL, f"states (rows per block {vt})")
    for s in range(w.num_slots):
        if s not in live:
            assert torch.equal(got[s], st[s]), f"slot {s} changed"
