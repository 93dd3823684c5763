"""GPU parity of gdn_decode_step_buffered against the fp64 oracle.

Single calls take the ring as an input (seeded records), so each phase is
checked on its own, with rows at different phases in one launch: outputs to
1e-4, the appended record (delta and key rounded to bf16, g as fp32), the
folded state on flush rows, and untouched checkpoints and ring positions on
the others. Chained runs follow all rows over several cycles to the chained
bar 2e-3, the oracle keeping its own ring and fp64 checkpoint.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle as O
import ssm_recurrent_decode_gated_amd as S
import workloads as W
from tests._helpers import (CHAIN_TOL, FP32_TOL, assert_mixed, assert_rounded16, need_gpu,
                            take_valid_roundings, to_np64)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _call(w, x, P, st_d, idx, ring_d, wp, out, norm=False):
    kw = {}
    if norm:
        kw = dict(norm_gate=x["norm_gate"].to(DEV), norm_weight=x["norm_weight"].to(DEV))
    S.gdn_decode_step_buffered(x["qkv"].to(DEV), x["a"].to(DEV), x["b"].to(DEV), P["A_log"].to(DEV),
                               P["dt_bias"].to(DEV), st_d, idx.to(DEV), out, ring_d["d_cache"],
                               ring_d["k_cache"], ring_d["g_cache"], wp.to(DEV), **kw)


CASES = [
    # name, B, H, HV, K, V, L, phases, norm
    ("k128_L8_mixed_phases", 6, 2, 4, 128, 128, 8, [0, 3, 7, 5, 1, 6], False),
    ("k128_L16_norm", 4, 2, 4, 128, 128, 16, [15, 0, 9, 14], True),
    ("k64_v40_L5", 5, 1, 3, 64, 40, 5, [4, 2, 0, 1, 3], False),
    ("k16_v16_L3", 3, 2, 2, 16, 16, 3, [2, 1, 0], False),
    ("k128_L1", 3, 2, 4, 128, 128, 1, [0, 0, 0], False),
]


def _ring_on_device(ring, offset):
    """The ring on the GPU; with `offset`, the 16-bit records start `offset`
    elements into a larger allocation (not 8-byte aligned for offset 1)."""
    out = {}
    for k, v in ring.items():
        if offset and v.element_size() == 2:
            buf = torch.zeros(v.numel() + offset, dtype=v.dtype, device=DEV)
            out[k] = buf[offset:].view(v.shape)
            out[k].copy_(v.to(DEV))
        else:
            out[k] = v.to(DEV)
    return out


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_buffered_single_call_every_phase(case):
    _single_call_case(case)


def test_buffered_f16_ring_every_phase():
    """f16 activations and ring records (the other 16-bit format): outputs,
    flushed states and records against the oracle's f16 ring, with rows at
    every phase of L = 8 in one launch, aligned and unaligned ring bases."""
    _single_call_case(("k128_L8_f16", 8, 2, 4, 128, 128, 8, [0, 1, 2, 3, 4, 5, 6, 7], False), act="f16")
    _single_call_case(("k64_v40_L5_f16_unaligned", 5, 1, 3, 64, 40, 5, [4, 2, 0, 1, 3], False), ring_offset=1,
                      act="f16")


def test_buffered_long_and_unaligned_rings():
    """A 32-record ring (more records than the vector staging covers in one
    go) and 16-bit rings whose base is not 8-byte aligned (element loads)."""
    _single_call_case(("k128_L32_long", 3, 2, 4, 128, 128, 32, [31, 20, 3], False))
    _single_call_case(("k128_L8_unaligned", 4, 2, 4, 128, 128, 8, [0, 5, 7, 2], False), ring_offset=1)
    _single_call_case(("k64_v40_L16_unaligned_norm", 3, 1, 3, 64, 40, 16, [15, 9, 1], True), ring_offset=1)


def _exact_records(w, x, P, st, idx, ring, wp, L, kw):
    """The oracle's ring after the same call with records left unrounded."""
    ex_st = st.double().numpy().copy()
    ex = {k: v.double().numpy().copy() for k, v in ring.items()}
    O.gdn_step_buffered(x["qkv"], x["a"], x["b"], P["A_log"], P["dt_bias"], ex_st, idx, ex["d_cache"],
                        ex["k_cache"], ex["g_cache"], wp, L, H=w.H, HV=w.HV, K=w.K, V=w.V,
                        ring_fmt=O.FMT_NONE, **kw)
    return ex


def _single_call_case(case, ring_offset=0, act="bf16"):
    need_gpu()
    name, B, H, HV, K, V, L, phases, norm = case
    w = W.GDNWorkload("buf_" + name, B=B, H=H, HV=HV, K=K, V=V, num_slots=B + 2, out="f32", idx="perm", act=act)
    fmt, mant = {"bf16": (O.FMT_BF16, 7), "f16": (O.FMT_F16, 10)}[act]
    P, idx, x = W.gdn_params(w), W.slot_indices(w), W.gdn_step_inputs(w, norm=norm)
    st = W.gdn_state(w)
    ring = W.gdn_ring(w, L)
    wp = torch.tensor(phases, dtype=torch.int32)
    st_d = st.to(DEV)
    ring_d = _ring_on_device(ring, ring_offset)
    out = torch.full((B, 1, HV, V), float("nan"), device=DEV)
    _call(w, x, P, st_d, idx, ring_d, wp, out, norm)
    ref_st = st.double().numpy().copy()
    ref_ring = {k: v.double().numpy().copy() for k, v in ring.items()}
    kw = dict(norm_gate=x["norm_gate"], norm_weight=x["norm_weight"]) if norm else {}
    ro = O.gdn_step_buffered(x["qkv"], x["a"], x["b"], P["A_log"], P["dt_bias"], ref_st, idx,
                             ref_ring["d_cache"], ref_ring["k_cache"], ref_ring["g_cache"], wp, L,
                             H=H, HV=HV, K=K, V=V, ring_fmt=fmt, **kw)
    ex_ring = _exact_records(w, x, P, st, idx, ring, wp, L, kw)
    torch.cuda.synchronize()
    assert_mixed(out.reshape(B, HV, V), ro, FP32_TOL, "output")
    got_st = st_d.cpu()
    got = {k: to_np64(v) for k, v in ring_d.items()}
    ring0 = {k: v.double().numpy() for k, v in ring.items()}
    G = HV // H
    for b in range(B):
        s, p = int(idx[b]), phases[b]
        if p == L - 1:  # a flush writes the folded state and appends no record
            assert_mixed(got_st[s], ref_st[s], FP32_TOL, f"flushed state row {b}")
            for k in ring0:
                np.testing.assert_array_equal(got[k][s], ring0[k][s], err_msg=f"{k} row {b} (flush)")
            continue
        assert torch.equal(got_st[s], st[s]), f"non-flush row {b} wrote the checkpoint"
        assert_rounded16(got["d_cache"][s, :, p], ref_ring["d_cache"][s, :, p], f"delta record row {b}",
                       ex_ring["d_cache"][s, :, p], mant)
        assert_rounded16(got["k_cache"][s, :, p], ref_ring["k_cache"][s, :, p], f"key record row {b}",
                       ex_ring["k_cache"][s, :, p], mant)
        np.testing.assert_allclose(got["g_cache"][s, :, p], ref_ring["g_cache"][s, :, p], rtol=1e-5)
        others = [j for j in range(L) if j != p]
        for k in ring0:
            np.testing.assert_array_equal(got[k][s][:, others], ring0[k][s][:, others], err_msg=f"{k} row {b}")
    for s in set(range(w.num_slots)) - set(idx.tolist()):
        assert torch.equal(got_st[s], st[s])
        for k in ring0:
            np.testing.assert_array_equal(got[k][s], ring0[k][s])
    assert G >= 1


@pytest.mark.parametrize("L,act", [(1, "bf16"), (8, "f32"), (16, "f32"), (8, "bf16"), (16, "bf16")])
def test_buffered_chain_matches_oracle(L, act):
    """B=64, H=16, HV=32, K=V=128 (the long-horizon workload) for 3 full
    cycles from a zeroed ring at write_pos 0, the host advancing write_pos.
    The oracle follows all 64 rows with its own ring in the same format and
    its own fp64 checkpoint; every output, and every checkpoint after a
    flush, within the chained bar 2e-3. fp32 rings: the two trajectories are
    independent throughout. 16-bit rings: each step's stored records are
    checked against the oracle's rounding of its exact record (equal, or the
    other neighbour at a rounding midpoint), and the oracle's ring takes the
    kernel's choice at those midpoints (take_valid_roundings), so the chains
    compare the same ring contents and the same checkpoint arithmetic."""
    need_gpu()
    w = replace(W.GDN_B64_CHAIN, act=act, name=W.GDN_B64_CHAIN.name + "_" + act)
    tdt = W.DTYPES[act]
    P, idx = W.gdn_params(w), W.slot_indices(w)
    st = W.gdn_state(w)
    st_d = st.to(DEV)
    ring_d = {"d_cache": torch.zeros(w.num_slots, w.HV, L, w.V, dtype=tdt, device=DEV),
              "k_cache": torch.zeros(w.num_slots, w.H, L, w.K, dtype=tdt, device=DEV),
              "g_cache": torch.zeros(w.num_slots, w.HV, L, device=DEV)}
    ref = st.double().numpy().copy()
    rr = {"d": np.zeros((w.num_slots, w.HV, L, w.V)), "k": np.zeros((w.num_slots, w.H, L, w.K)),
          "g": np.zeros((w.num_slots, w.HV, L))}
    out = torch.empty(w.B, 1, w.HV, w.V, device=DEV)
    Pd = {k: v.to(DEV) for k, v in P.items()}
    fmt = O.FMT_F32 if act == "f32" else O.FMT_BF16
    taken = 0
    for t in range(3 * L if L > 1 else 8):
        x = W.gdn_step_inputs(w, 5000 + t)
        p = t % L
        wp = torch.full((w.B,), p, dtype=torch.int32)
        S.gdn_decode_step_buffered(x["qkv"].to(DEV), x["a"].to(DEV), x["b"].to(DEV), Pd["A_log"],
                                   Pd["dt_bias"], st_d, idx.to(DEV), out, ring_d["d_cache"],
                                   ring_d["k_cache"], ring_d["g_cache"], wp.to(DEV))
        args = (x["qkv"], x["a"], x["b"], P["A_log"], P["dt_bias"])
        kw = dict(H=w.H, HV=w.HV, K=w.K, V=w.V)
        if act != "f32":  # this step's exact (unrounded) records, from the same ring and checkpoint
            ex = {k: v.copy() for k, v in rr.items()}
            ex_st = ref.copy() if p == L - 1 else ref  # only a flush writes the checkpoint
            O.gdn_step_buffered(*args, ex_st, idx, ex["d"], ex["k"], ex["g"], wp, L, ring_fmt=O.FMT_NONE, **kw)
        ro = O.gdn_step_buffered(*args, ref, idx, rr["d"], rr["k"], rr["g"], wp, L, ring_fmt=fmt, **kw)
        assert_mixed(out.reshape(w.B, w.HV, w.V), ro, CHAIN_TOL, f"output step {t} (phase {p})")
        if p == L - 1:
            assert_mixed(st_d, ref, CHAIN_TOL, f"checkpoint after step {t}")
        if act != "f32" and p < L - 1:  # a flushed cycle's records are not read again
            for key, dkey in (("d", "d_cache"), ("k", "k_cache")):
                got = to_np64(ring_d[dkey][:, :, p])
                rr[key][:, :, p], n = take_valid_roundings(got, rr[key][:, :, p], ex[key][:, :, p], 7,
                                                           f"{key} records step {t}")
                taken += n
    if act != "f32":
        print(f"L={L} {act}: {taken} midpoint rounding choices taken from the kernel")


def test_buffered_L1_equals_packed_on_gpu():
    """With L = 1 every call is a flush of an empty ring: the buffered kernel
    must compute the packed step."""
    need_gpu()
    w = W.GDN_B16
    P, idx, x = W.gdn_params(w), W.slot_indices(w), W.gdn_step_inputs(w)
    st = W.gdn_state(w)
    s1, s2 = st.to(DEV), st.to(DEV)
    o1 = torch.empty(w.B, 1, w.HV, w.V, device=DEV)
    o2 = torch.empty_like(o1)
    S.gdn_decode_step(x["qkv"].to(DEV), x["a"].to(DEV), x["b"].to(DEV), P["A_log"].to(DEV),
                      P["dt_bias"].to(DEV), s1, idx.to(DEV), o1)
    ring_d = {"d_cache": torch.zeros(w.num_slots, w.HV, 1, w.V, dtype=torch.bfloat16, device=DEV),
              "k_cache": torch.zeros(w.num_slots, w.H, 1, w.K, dtype=torch.bfloat16, device=DEV),
              "g_cache": torch.zeros(w.num_slots, w.HV, 1, device=DEV)}
    _call(w, x, P, s2, idx, ring_d, torch.zeros(w.B, dtype=torch.int32), o2)
    torch.cuda.synchronize()
    ref = to_np64(s1)
    assert_mixed(s2, ref, 1e-6, "state")
    assert_mixed(o2, to_np64(o1), 1e-6, "output")


@pytest.mark.parametrize("K,V,HV,L", [(128, 128, 8, 8), (256, 64, 4, 4), (64, 40, 6, 16)])
def test_buffered_many_rows_with_padding(K, V, HV, L):
    """120 rows over every phase, with padded slots and out-of-range phases
    interleaved: live rows match the oracle (outputs, flushed states, ring
    records), padded rows touch neither output, state nor ring."""
    need_gpu()
    B, H = 120, 2 if HV % 2 == 0 else 1
    w = W.GDNWorkload(f"buf_walk_k{K}_v{V}_hv{HV}_L{L}", B=B, H=H, HV=HV, K=K, V=V, num_slots=B + 10,
                      out="f32", idx="perm")
    P, idx, x = W.gdn_params(w), W.slot_indices(w).clone(), W.gdn_step_inputs(w)
    phases = [b % L for b in range(B)]
    for b in range(B):
        if b % 11 == 4:
            idx[b] = -1 if b % 2 else w.num_slots
        elif b % 13 == 6:
            phases[b] = L if b % 2 else -1
    st = W.gdn_state(w)
    ring = W.gdn_ring(w, L)
    wp = torch.tensor(phases, dtype=torch.int32)
    st_d = st.to(DEV)
    ring_d = _ring_on_device(ring, 0)
    out = torch.full((B, 1, HV, V), float("nan"), device=DEV)
    _call(w, x, P, st_d, idx, ring_d, wp, out)
    ref_st = st.double().numpy().copy()
    ref_ring = {k: v.double().numpy().copy() for k, v in ring.items()}
    ro = O.gdn_step_buffered(x["qkv"], x["a"], x["b"], P["A_log"], P["dt_bias"], ref_st, idx,
                             ref_ring["d_cache"], ref_ring["k_cache"], ref_ring["g_cache"], wp, L,
                             H=H, HV=HV, K=K, V=V, ring_fmt=O.FMT_BF16)
    ex_ring = _exact_records(w, x, P, st, idx, ring, wp, L, {})
    torch.cuda.synchronize()
    live = [b for b in range(B) if 0 <= int(idx[b]) < w.num_slots and 0 <= phases[b] < L]
    dead = [b for b in range(B) if b not in live]
    assert len(dead) > 10
    o = out.reshape(B, HV, V)
    assert_mixed(o[live], ro[live], FP32_TOL, "output")
    assert torch.isnan(o[dead]).all(), "a padded row wrote its output"
    got_st = st_d.cpu()
    got = {k: to_np64(v) for k, v in ring_d.items()}
    ring0 = {k: v.double().numpy() for k, v in ring.items()}
    for b in live:
        s, p = int(idx[b]), phases[b]
        if p == L - 1:  # a flush writes the folded state and appends no record
            assert_mixed(got_st[s], ref_st[s], FP32_TOL, f"flushed state row {b}")
            for k in ring0:
                np.testing.assert_array_equal(got[k][s], ring0[k][s], err_msg=f"{k} row {b} (flush)")
            continue
        assert torch.equal(got_st[s], st[s]), f"non-flush row {b} wrote the checkpoint"
        assert_rounded16(got["d_cache"][s, :, p], ref_ring["d_cache"][s, :, p], f"delta record row {b}",
                       ex_ring["d_cache"][s, :, p])
        assert_rounded16(got["k_cache"][s, :, p], ref_ring["k_cache"][s, :, p], f"key record row {b}",
                       ex_ring["k_cache"][s, :, p])
        np.testing.assert_allclose(got["g_cache"][s, :, p], ref_ring["g_cache"][s, :, p], rtol=1e-5)
    touched = {int(idx[b]) for b in live}
    for s in set(range(w.num_slots)) - touched:
        assert torch.equal(got_st[s], st[s]), f"slot {s} (no live row) changed"
        for k in ring0:
            np.testing.assert_array_equal(got[k][s], ring0[k][s], err_msg=f"{k} slot {s}")


@pytest.mark.parametrize("V,act", [(100, "bf16"), (128, "f32"), (20, "f16")])
def test_buffered_l1_large_batch(V, act):
    """L = 1 at a large batch (1280 heads: at least four per CU of a 256-CU
    part), where the launch takes 1-wave blocks over 8-row tiles: ragged last
    tiles (V = 100, 20), padded slots and out-of-range phases interleaved.
    Every live row is a flush of an empty ring: outputs and written states
    match the oracle, padded rows and the ring stay untouched."""
    need_gpu()
    B, H, HV, K, L = 40, 16, 32, 128, 1
    w = W.GDNWorkload(f"buf_l1_large_v{V}_{act}", B=B, H=H, HV=HV, K=K, V=V, num_slots=B + 6, act=act,
                      out="f32", idx="perm")
    P, idx, x = W.gdn_params(w), W.slot_indices(w).clone(), W.gdn_step_inputs(w)
    phases = [0] * B
    for b in range(B):
        if b % 7 == 3:
            idx[b] = -1 if b % 2 else w.num_slots
        elif b % 9 == 5:
            phases[b] = 1 if b % 2 else -1
    st = W.gdn_state(w)
    ring = W.gdn_ring(w, L)
    wp = torch.tensor(phases, dtype=torch.int32)
    st_d = st.to(DEV)
    ring_d = _ring_on_device(ring, 0)
    out = torch.full((B, 1, HV, V), float("nan"), device=DEV)
    _call(w, x, P, st_d, idx, ring_d, wp, out)
    ref_st = st.double().numpy().copy()
    ref_ring = {k: v.double().numpy().copy() for k, v in ring.items()}
    fmt = {"f32": O.FMT_F32, "bf16": O.FMT_BF16, "f16": O.FMT_F16}[act]
    ro = O.gdn_step_buffered(x["qkv"], x["a"], x["b"], P["A_log"], P["dt_bias"], ref_st, idx,
                             ref_ring["d_cache"], ref_ring["k_cache"], ref_ring["g_cache"], wp, L,
                             H=H, HV=HV, K=K, V=V, ring_fmt=fmt)
    torch.cuda.synchronize()
    live = [b for b in range(B) if 0 <= int(idx[b]) < w.num_slots and phases[b] == 0]
    dead = [b for b in range(B) if b not in live]
    assert len(dead) >= 8
    o = out.reshape(B, HV, V)
    assert_mixed(o[live], ro[live], FP32_TOL, "output")
    assert torch.isnan(o[dead]).all(), "a padded row wrote its output"
    got_st = st_d.cpu()
    for b in live:
        s = int(idx[b])
        assert_mixed(got_st[s], ref_st[s], FP32_TOL, f"flushed state row {b}")
    touched = {int(idx[b]) for b in live}
    for s in set(range(w.num_slots)) - touched:
        assert torch.equal(got_st[s], st[s]), f"slot {s} (no live row) changed"
    for k, v in ring_d.items():
        assert torch.equal(v.cpu(), ring[k]), f"{k} changed: an L = 1 flush appends no record"
