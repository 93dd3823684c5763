"""Pins of the fp64 oracle against facts fixed by the pages and by the
mathematics, not by the oracle itself: hand-worked cases (tests/golden),
closed forms, invariants, special cases that reduce to library routines, and
brute-force equivalences. Each pin targets a plausible mistake (a dropped term,
a wrong sign, a transposed operand, a wrong index or GQA map).

Pages (by title): [REPLAY] the buffered-vs-packed GDN decode microbenchmark;
[KDA] the fused Kimi-K3 KDA decode microbenchmark; [LOG] "Optimization Log:
Qwen3.5-27B Dense on B200"; [MBU] "Triton decode kernel + MBU analysis".
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BIG = 200.0  # sigmoid(+-200) is 1 / e^-200 in fp64: beta = 1 or beta ~ 1e-87


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _qkv(q, k, v):
    """Pack [B, HQ, K] q, k and [B, HV, V] v into mixed_qkv rows q|k|v."""
    B = q.shape[0]
    return np.concatenate([q.reshape(B, -1), k.reshape(B, -1), v.reshape(B, -1)], axis=1)


# ------------------------------------------------------------ scalar helpers
def test_round_bf16_ties_to_even():
    # bf16 keeps 8 significant bits: 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7
    assert O.round_fmt(1 + 2 ** -8, O.FMT_BF16) == 1.0
    assert O.round_fmt(1 + 3 * 2 ** -8, O.FMT_BF16) == 1 + 2 ** -6
    assert O.round_fmt(1 + 2 ** -8 + 2 ** -30, O.FMT_BF16) == 1 + 2 ** -7
    assert O.round_fmt(-(1 + 3 * 2 ** -8), O.FMT_BF16) == -(1 + 2 ** -6)
    assert math.isinf(O.round_fmt(3.5e38, O.FMT_BF16))          # beyond bf16 max + half ulp
    assert O.round_fmt(2.0 ** -133, O.FMT_BF16) == 2.0 ** -133   # smallest bf16 subnormal
    assert O.round_fmt(1 + 2 ** -11, O.FMT_F16) == 1.0
    assert math.isinf(O.round_fmt(65520.0, O.FMT_F16))           # ties away into inf
    assert O.round_fmt(65519.0, O.FMT_F16) == 65504.0


def test_round_matches_library_conversions():
    rng = np.random.default_rng(1)
    x32 = np.concatenate([
        np.clip(rng.standard_normal(20000) * 10.0 ** rng.integers(-40, 38, 20000), -3e38, 3e38),
        rng.standard_normal(2000),
        (rng.integers(0, 1 << 16, 2000).astype(np.uint32) << 16 | 0x8000).view(np.float32),  # exact bf16 midpoints
    ]).astype(np.float32)
    x32 = x32[np.isfinite(x32)]
    ref_bf16 = torch.from_numpy(x32).to(torch.bfloat16).double().numpy()
    ours = np.array([O.round_fmt(float(v), O.FMT_BF16) for v in x32])
    np.testing.assert_array_equal(ours, ref_bf16)
    x64 = rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 5, 20000)
    ref_f16 = x64.astype(np.float16).astype(np.float64)
    ours16 = np.array([O.round_fmt(float(v), O.FMT_F16) for v in x64])
    np.testing.assert_array_equal(ours16, ref_f16)
    ref_f32 = x64.astype(np.float32).astype(np.float64)
    ours32 = np.array([O.round_fmt(float(v), O.FMT_F32) for v in x64])
    np.testing.assert_array_equal(ours32, ref_f32)


def test_activation_closed_forms():
    assert O.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-15)
    assert O.softplus(math.log(math.e - 1.0)) == pytest.approx(1.0, rel=1e-15)
    assert O.softplus(50.0) == 50.0
    for x in (-3.0, -0.5, 0.25, 4.0):  # softplus(x) - softplus(-x) = x
        assert O.softplus(x) - O.softplus(-x) == pytest.approx(x, rel=1e-14)
    assert O.sigmoid(0.0) == 0.5
    assert O.sigmoid(math.log(3.0)) == pytest.approx(0.75, rel=1e-15)
    assert O.silu(0.0) == 0.0
    assert O.silu(math.log(3.0)) == pytest.approx(0.75 * math.log(3.0), rel=1e-15)
    assert O.silu(-40.0) == pytest.approx(-40.0 * math.exp(-40.0), rel=1e-12)


def test_gdn_gates_closed_forms():
    g, beta = O.gdn_gates(0.0, 0.0, 0.0, 0.0)
    assert g == pytest.approx(-math.log(2.0), rel=1e-15) and beta == 0.5
    g, beta = O.gdn_gates(0.3, math.log(3.0), math.log(2.0), -0.3)  # softplus(0) = ln 2
    assert math.exp(g) == pytest.approx(0.25, rel=1e-14) and beta == pytest.approx(0.75, rel=1e-15)
    g, _ = O.gdn_gates(math.log(math.e - 1), 0.0, math.log(2.5), 0.0)
    assert g == pytest.approx(-2.5, rel=1e-14)
    g, _ = O.gdn_gates(30.0, 0.0, 0.0, 0.0)  # softplus(30) = 30 -> g = -30
    assert g == -30.0


def test_kda_gate_is_lower_bound_sigmoid():
    # the workload's gate lb * sigmoid(raw_g): sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4
    assert O.kda_gate(0.0, -5.0) == -2.5
    assert O.kda_gate(math.log(3.0), -5.0) == pytest.approx(-3.75, rel=1e-15)
    assert O.kda_gate(-math.log(3.0), -4.0) == pytest.approx(-1.0, rel=1e-15)
    assert O.kda_gate(-BIG, -5.0) == pytest.approx(0.0, abs=1e-80)
    assert O.kda_gate(BIG, -5.0) == -5.0


# ------------------------------------------------------------ GDN step
def test_gdn_hand_4x4():
    gd = _load("gdn_hand_4x4.json")
    i, e = gd["inputs"], gd["expected"]
    state = np.array(i["S0"], dtype=np.float64)[None, None]
    qkv = np.array([i["q"] + i["k"] + i["v"]], dtype=np.float64)
    out = O.gdn_step(qkv, [[i["a"]]], [[i["b"]]], [i["A_log"]], [i["dt_bias"]], state, [0],
                     H=1, HV=1, K=4, V=4, scale=i["scale"], use_l2=i["use_qk_l2norm"])
    np.testing.assert_allclose(state[0, 0], np.array(e["S1"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(out[0, 0], np.array(e["o"]), rtol=0, atol=1e-15)


def _rand_gdn(rng, B=3, H=2, HV=4, K=8, V=6, slots=5):
    qkv = rng.standard_normal((B, 2 * H * K + HV * V))
    a = rng.standard_normal((B, HV)) * 0.5
    b = rng.standard_normal((B, HV))
    A_log = rng.standard_normal(HV) * 0.3
    dt_bias = rng.standard_normal(HV) * 0.1
    state = rng.standard_normal((slots, HV, V, K))
    return qkv, a, b, A_log, dt_bias, state


def test_pin_identity_step():
    """exp(g) = 1 and beta = 0 leave S unchanged; o = S q (q L2-normed, scaled)."""
    rng = np.random.default_rng(2)
    B, H, HV, K, V = 3, 2, 4, 8, 6
    qkv, a, b, _, dt_bias, state = _rand_gdn(rng, B, H, HV, K, V)
    A_log = np.full(HV, -BIG)  # exp(A_log) = e^-200 -> g ~ -1e-87 -> exp(g) == 1.0
    b = np.full((B, HV), -BIG)  # beta = e^-200
    s0 = state.copy()
    idx = np.array([4, 0, 2], np.int32)
    out = O.gdn_step(qkv, a, b, A_log, dt_bias, state, idx, H=H, HV=HV, K=K, V=V)
    np.testing.assert_allclose(state, s0, rtol=1e-15, atol=1e-80)
    G = HV // H
    for bi in range(B):
        for hv in range(HV):
            h = hv // G
            q = qkv[bi, h * K:(h + 1) * K]
            q = q / np.sqrt((q * q).sum() + 1e-6) * K ** -0.5
            np.testing.assert_allclose(out[bi, hv], s0[idx[bi], hv] @ q, rtol=1e-13, atol=1e-15)


def test_pin_delta_rule_recovers_v():
    """Unit-norm k and beta = 1: after the update S k = v, for any g and S."""
    rng = np.random.default_rng(3)
    B, H, HV, K, V = 2, 2, 4, 16, 12
    qkv, a, _, A_log, dt_bias, state = _rand_gdn(rng, B, H, HV, K, V, slots=2)
    b = np.full((B, HV), BIG)  # beta = 1
    idx = np.array([1, 0], np.int32)
    O.gdn_step(qkv, a, b, A_log, dt_bias, state, idx, H=H, HV=HV, K=K, V=V, l2eps=0.0)
    G = HV // H
    for bi in range(B):
        for hv in range(HV):
            h = hv // G
            k = qkv[bi, H * K + h * K: H * K + (h + 1) * K]
            k = k / np.linalg.norm(k)
            v = qkv[bi, 2 * H * K + hv * V: 2 * H * K + (hv + 1) * V]
            np.testing.assert_allclose(state[idx[bi], hv] @ k, v, rtol=1e-12, atol=1e-12)


def test_pin_state_layout_columns_are_keys():
    """beta = 1, g = 0 and k_t = e_t over K steps: column t of S[V][K] ends as v_t
    whatever S0 was (a transposed layout would fill rows instead)."""
    rng = np.random.default_rng(4)
    K, V = 6, 5
    state = rng.standard_normal((1, 1, V, K))
    vs = []
    for t in range(K):
        q = rng.standard_normal(K)
        k = np.zeros(K)
        k[t] = 1.0
        v = rng.standard_normal(V)
        vs.append(v)
        O.gdn_step(_qkv(q[None], k[None], v[None]), [[0.3]], [[BIG]], [-BIG], [0.0], state, [0],
                   H=1, HV=1, K=K, V=V, use_l2=False, scale=1.0)
    np.testing.assert_allclose(state[0, 0], np.stack(vs, axis=1), rtol=0, atol=1e-15)


def test_pin_decay_accumulates():
    """beta = 0 over T steps: S_T = exp(sum g) S_0; here exp(g) = 1/4 per step."""
    rng = np.random.default_rng(5)
    K, V, T = 8, 8, 7
    state = rng.standard_normal((1, 2, V, K))
    s0 = state.copy()
    for _ in range(T):
        qkv = rng.standard_normal((1, 2 * K + 2 * V))
        # A_log = ln 2, a + dt_bias = 0: g = -2 ln 2
        O.gdn_step(qkv, [[0.1, -0.2]], [[-BIG, -BIG]], [math.log(2.0)] * 2, [-0.1, 0.2],
                   state, [0], H=1, HV=2, K=K, V=V)
    np.testing.assert_allclose(state, s0 * 4.0 ** -T, rtol=1e-13, atol=0)


def test_pin_gqa_map_contiguous_groups():
    """HV = 2H with shared q/k equals H' = HV with each q/k head repeated
    (value head hv reads q/k head hv // (HV/H))."""
    rng = np.random.default_rng(6)
    B, H, HV, K, V = 2, 2, 6, 8, 5
    qkv, a, b, A_log, dt_bias, state = _rand_gdn(rng, B, H, HV, K, V, slots=2)
    G = HV // H
    q = qkv[:, :H * K].reshape(B, H, K)
    k = qkv[:, H * K:2 * H * K].reshape(B, H, K)
    v = qkv[:, 2 * H * K:]
    rep = _qkv(np.repeat(q, G, axis=1), np.repeat(k, G, axis=1), v)
    s1, s2 = state.copy(), state.copy()
    idx = np.array([1, 0], np.int32)
    o1 = O.gdn_step(qkv, a, b, A_log, dt_bias, s1, idx, H=H, HV=HV, K=K, V=V)
    o2 = O.gdn_step(rep, a, b, A_log, dt_bias, s2, idx, H=HV, HV=HV, K=K, V=V)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_pin_placement_permutation_and_padding():
    """Permuting rows with their indices permutes outputs; padded rows (index
    < 0 or >= num_slots) and slots nobody names are untouched, bit for bit."""
    rng = np.random.default_rng(7)
    B, H, HV, K, V, slots = 5, 1, 2, 8, 4, 9
    qkv, a, b, A_log, dt_bias, state = _rand_gdn(rng, B, H, HV, K, V, slots)
    idx = np.array([7, -1, 2, 9, 0], np.int32)
    s1 = state.copy()
    o1 = O.gdn_step(qkv, a, b, A_log, dt_bias, s1, idx, H=H, HV=HV, K=K, V=V)
    perm = np.array([3, 0, 4, 2, 1])
    s2 = state.copy()
    o2 = O.gdn_step(qkv[perm], a[perm], b[perm], A_log, dt_bias, s2, idx[perm], H=H, HV=HV, K=K, V=V)
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(o1[perm], o2)
    touched = {7, 2, 0}
    for s in range(slots):
        if s not in touched:
            np.testing.assert_array_equal(s1[s], state[s])
        else:
            assert not np.array_equal(s1[s], state[s])
    assert np.isnan(o1[1]).all() and np.isnan(o1[3]).all()


def test_pin_non_expansion():
    """Unit-norm k, beta in [0, 1], g <= 0: the step is a contraction in the
    Frobenius norm, so two runs on the same inputs never drift apart."""
    rng = np.random.default_rng(8)
    K, V, T = 16, 16, 200
    s1 = rng.standard_normal((1, 1, V, K))
    s2 = s1 + rng.standard_normal(s1.shape) * 1e-3
    prev = np.linalg.norm(s1 - s2)
    for _ in range(T):
        qkv = rng.standard_normal((1, 2 * K + V))
        a, b = rng.standard_normal((1, 1)), rng.standard_normal((1, 1)) * 3
        O.gdn_step(qkv, a, b, [0.2], [0.0], s1, [0], H=1, HV=1, K=K, V=V, l2eps=0.0)
        O.gdn_step(qkv, a, b, [0.2], [0.0], s2, [0], H=1, HV=1, K=K, V=V, l2eps=0.0)
        cur = np.linalg.norm(s1 - s2)
        assert cur <= prev * (1 + 1e-12) + 1e-15 * np.linalg.norm(s1)
        prev = cur


def test_pin_gated_norm_constant_output():
    """Zero state, k = q = e0, beta = 1/2, v = 2: o = 1 on every row, so the
    gated RMSNorm gives 1/sqrt(1 + eps) * w * act(z) (mean, not sum, of o^2)."""
    V, K, eps = 6, 4, 1e-3
    state = np.zeros((1, 1, V, K))
    q = np.eye(K)[0]
    z = np.linspace(-2, 2, V)
    w = np.linspace(0.5, 1.5, V)
    qkv = _qkv(q[None], q[None], np.full((1, V), 2.0))
    for act, f in ((O.ACT_SILU, lambda x: x / (1 + np.exp(-x))), (O.ACT_SIGMOID, lambda x: 1 / (1 + np.exp(-x)))):
        s = state.copy()
        out = O.gdn_step(qkv, [[0.0]], [[0.0]], [0.0], [0.0], s, [0], H=1, HV=1, K=K, V=V,
                         use_l2=False, scale=1.0, norm_gate=z[None, None], norm_weight=w,
                         norm_eps=eps, norm_act=act)
        np.testing.assert_allclose(out[0, 0], w * f(z) / math.sqrt(1 + eps), rtol=1e-14)


@pytest.mark.parametrize("fmt", [O.FMT_BF16, O.FMT_F16])
def test_pin_16bit_state_rounds_on_store_only(fmt):
    """A 16-bit state pool ([LOG] "Kernel 4" sizes the state as 16-bit) stores
    round(S_new) while the step's output comes from the unrounded S_new: the
    output equals the fp64-state run exactly and the stored state is its
    elementwise rounding."""
    rng = np.random.default_rng(60 + fmt)
    B, H, HV, K, V = 3, 2, 4, 16, 8
    qkv, a, b, A_log, dt_bias, state = _rand_gdn(rng, B, H, HV, K, V, slots=4)
    state = np.vectorize(lambda x: O.round_fmt(x, fmt))(state)  # a pool that holds 16-bit values
    idx = np.array([3, 1, 0], np.int32)
    s64, s16 = state.copy(), state.copy()
    o64 = O.gdn_step(qkv, a, b, A_log, dt_bias, s64, idx, H=H, HV=HV, K=K, V=V)
    o16 = O.gdn_step(qkv, a, b, A_log, dt_bias, s16, idx, H=H, HV=HV, K=K, V=V, state_fmt=fmt)
    np.testing.assert_array_equal(o16, o64)
    np.testing.assert_array_equal(s16, np.vectorize(lambda x: O.round_fmt(x, fmt))(s64))
    assert not np.array_equal(s16[idx], s64[idx])
    np.testing.assert_array_equal(s16[2], state[2])


# ------------------------------------------------------------ buffered step
def _buffered_setup(rng, B=3, H=2, HV=4, K=8, V=6, L=4):
    qkv, a, b, A_log, dt_bias, state = _rand_gdn(rng, B, H, HV, K, V, slots=B)
    ring = (np.zeros((B, HV, L, V)), np.zeros((B, H, L, K)), np.zeros((B, HV, L)))
    return A_log, dt_bias, state, ring


@pytest.mark.parametrize("L", [1, 3, 8])
def test_pin_buffered_equals_packed(L):
    """With an unrounded ring the buffered chain reproduces the packed chain:
    outputs at every step, the checkpoint after each full cycle (g is stored
    as fp32, the only rounding left), and the checkpoint stays put between
    flushes."""
    rng = np.random.default_rng(10 + L)
    B, H, HV, K, V = 3, 2, 4, 8, 6
    A_log, dt_bias, state, (dc, kc, gc) = _buffered_setup(rng, B, H, HV, K, V, L)
    sp, sb = state.copy(), state.copy()
    idx = np.array([2, 0, 1], np.int32)
    for t in range(3 * L):
        qkv = rng.standard_normal((B, 2 * H * K + HV * V))
        a, b = rng.standard_normal((B, HV)) * 0.5, rng.standard_normal((B, HV))
        op = O.gdn_step(qkv, a, b, A_log, dt_bias, sp, idx, H=H, HV=HV, K=K, V=V)
        ck = sb.copy()
        wp = np.full(B, t % L, np.int32)
        ob = O.gdn_step_buffered(qkv, a, b, A_log, dt_bias, sb, idx, dc, kc, gc, wp, L,
                                 H=H, HV=HV, K=K, V=V, ring_fmt=O.FMT_NONE)
        if L == 1:
            np.testing.assert_array_equal(ob, op)
            np.testing.assert_array_equal(sb, sp)
            continue
        # the ring keeps g as fp32: exp(g) moves by ~|g| 2^-24, nothing else differs
        np.testing.assert_allclose(ob, op, rtol=1e-6, atol=1e-9)
        if t % L == L - 1:
            np.testing.assert_allclose(sb, sp, rtol=1e-6, atol=1e-9)
        else:
            np.testing.assert_array_equal(sb, ck)


def test_pin_buffered_ring_records():
    """The record at write_pos holds this step's delta (= v - S_new k ... via
    beta = 1 and unit k: delta = v - decayed S k), the normalised key and g,
    rounded to bf16 / bf16 / fp32; other positions are untouched."""
    rng = np.random.default_rng(20)
    B, H, HV, K, V, L = 2, 1, 2, 8, 4, 5
    A_log, dt_bias, state, (dc, kc, gc) = _buffered_setup(rng, B, H, HV, K, V, L)
    dc[:] = 7.0
    kc[:] = 7.0
    gc[:] = 7.0
    qkv = rng.standard_normal((B, 2 * H * K + HV * V))
    a = rng.standard_normal((B, HV))
    b = np.full((B, HV), BIG)
    wp = np.array([0, 0], np.int32)
    s0 = state.copy()
    O.gdn_step_buffered(qkv, a, b, A_log, dt_bias, state, np.array([0, 1], np.int32), dc, kc, gc,
                        wp, L, H=H, HV=HV, K=K, V=V, ring_fmt=O.FMT_BF16, l2eps=0.0)
    for bi in range(B):
        k = qkv[bi, H * K:2 * H * K]
        k = k / np.linalg.norm(k)
        np.testing.assert_array_equal(kc[bi, 0, 0], [O.round_fmt(x, O.FMT_BF16) for x in k])
        for hv in range(HV):
            g, _ = O.gdn_gates(a[bi, hv], BIG, A_log[hv], dt_bias[hv])
            assert gc[bi, hv, 0] == O.round_fmt(g, O.FMT_F32)
            v = qkv[bi, 2 * H * K + hv * V: 2 * H * K + (hv + 1) * V]
            delta = v - math.exp(g) * (s0[bi, hv] @ k)
            np.testing.assert_allclose(dc[bi, hv, 0], delta, rtol=2 ** -8, atol=1e-12)
            np.testing.assert_array_equal(dc[bi, hv, 0], [O.round_fmt(x, O.FMT_BF16) for x in dc[bi, hv, 0]])
        assert (dc[bi, :, 1:] == 7.0).all() and (kc[bi, :, 1:] == 7.0).all() and (gc[bi, :, 1:] == 7.0).all()
    np.testing.assert_array_equal(state, s0)  # phase 0 of L = 5 is not a flush


def test_pin_buffered_padding_and_phase_bounds():
    rng = np.random.default_rng(21)
    B, H, HV, K, V, L = 3, 1, 1, 4, 4, 2
    A_log, dt_bias, state, (dc, kc, gc) = _buffered_setup(rng, B, H, HV, K, V, L)
    s0, d0 = state.copy(), dc.copy()
    qkv = rng.standard_normal((B, 2 * H * K + HV * V))
    out = O.gdn_step_buffered(qkv, [[0.1]] * B, [[0.2]] * B, A_log, dt_bias, state,
                              np.array([-1, 1, 2], np.int32), dc, kc, gc,
                              np.array([0, L, -1], np.int32), L, H=H, HV=HV, K=K, V=V)
    assert np.isnan(out).all()
    np.testing.assert_array_equal(state, s0)
    np.testing.assert_array_equal(dc, d0)


# ------------------------------------------------------------ KDA
def test_conv_hand_case():
    gd = _load("conv1d_hand_w4.json")
    i, e = gd["inputs"], gd["expected"]
    for silu_act, key in ((False, "y_linear"), (True, "y_silu")):
        cs = np.array(i["state"], dtype=np.float64).reshape(1, 1, 3)
        cs = np.concatenate([np.zeros_like(cs), cs])  # slot 0 is the NULL block
        y = O.conv1d_update([[i["x"]]], [i["w"]], [i["bias"]], cs, [1], silu_act=silu_act)
        assert y[0, 0] == e[key]
        np.testing.assert_array_equal(cs[1, 0], e["state"])


def test_pin_conv_orientation():
    """w = e_{W-1} gives silu(x_t); w = e_0 gives silu(x_{t-3}); after three
    steps the conv state holds the last three raw inputs, oldest first."""
    rng = np.random.default_rng(30)
    C, W, T = 5, 4, 6
    xs = rng.standard_normal((T, C))
    for tap, lag in ((W - 1, 0), (0, 3), (1, 2)):
        w = np.zeros((C, W))
        w[:, tap] = 1.0
        cs = np.zeros((2, C, W - 1))
        for t in range(T):
            y = O.conv1d_update(xs[t:t + 1], w, None, cs, [1])
            src = xs[t - lag] if t - lag >= 0 else np.zeros(C)
            np.testing.assert_allclose(y[0], src / (1 + np.exp(-src)), rtol=1e-15, atol=0)
        np.testing.assert_array_equal(cs[1], xs[T - 3:].T)
        assert (cs[0] == 0).all()


def test_pin_conv_skips_null_and_out_of_range():
    rng = np.random.default_rng(31)
    cs = rng.standard_normal((3, 4, 3))
    c0 = cs.copy()
    y = O.conv1d_update(rng.standard_normal((3, 4)), rng.standard_normal((4, 4)), None, cs,
                        [0, 3, -2])
    assert np.isnan(y).all()
    np.testing.assert_array_equal(cs, c0)


def test_pin_kda_uniform_gate_equals_gdn():
    """A KDA step whose per-channel gates are all equal is a GDN step with that
    scalar gate: raw_g = 0 gives g = -5 sigmoid(0) = -2.5 on every channel;
    GDN reaches g = -2.5 with A_log = ln 2.5 and a + dt_bias = ln(e - 1)."""
    rng = np.random.default_rng(32)
    T, H, D = 3, 2, 8
    y = rng.standard_normal((T, 3 * H * D))
    raw_beta = rng.standard_normal((T, H))
    gate = rng.standard_normal((T, H, D))
    w = 1 + 0.1 * rng.standard_normal(D)
    st = rng.standard_normal((T + 1, H, D, D))
    s1, s2 = st.copy(), st.copy()
    idx = np.arange(1, T + 1, dtype=np.int32)
    o1 = O.kda_step(y, np.zeros((T, H, D)), raw_beta, s1, idx, H=H, D=D, gate=gate, norm_weight=w)
    o2 = O.gdn_step(y, np.full((T, H), math.log(math.e - 1)), raw_beta, [math.log(2.5)] * H,
                    [0.0] * H, s2, idx, H=H, HV=H, K=D, V=D, norm_gate=gate, norm_weight=w,
                    norm_act=O.ACT_SIGMOID)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(s1, s2, rtol=1e-13, atol=1e-15)


def test_pin_kda_decay_is_per_key_column():
    """beta = 0: S[v, c] <- S[v, c] exp(g_c), i.e. the decay scales key columns."""
    rng = np.random.default_rng(33)
    H, D = 2, 6
    y = rng.standard_normal((1, 3 * H * D))
    raw_g = rng.standard_normal((1, H, D))
    st = rng.standard_normal((2, H, D, D))
    s0 = st.copy()
    O.kda_step(y, raw_g, np.full((1, H), -BIG), st, [1], H=H, D=D)
    for h in range(H):
        dec = np.exp(-5.0 / (1.0 + np.exp(-raw_g[0, h])))  # e^{lb sigmoid(raw_g)}, lb = -5
        np.testing.assert_allclose(st[1, h], s0[1, h] * dec[None, :], rtol=1e-15)
    np.testing.assert_array_equal(st[0], s0[0])


def test_pin_kda_decode_is_conv_then_step():
    """The fused op equals the conv update followed by the KDA step on the fp64
    conv output, and skips slot 0."""
    rng = np.random.default_rng(34)
    T, H, D, W = 3, 2, 4, 4
    C = 3 * H * D
    x = rng.standard_normal((T, C))
    cw = rng.standard_normal((C, W))
    raw_g, raw_beta = rng.standard_normal((T, H, D)), rng.standard_normal((T, H))
    gate = rng.standard_normal((T, H, D))
    cs = rng.standard_normal((T + 2, C, W - 1))
    st = rng.standard_normal((T + 2, H, D, D))
    idx = np.array([1, 0, 3], np.int32)
    cs1, st1, cs2, st2 = cs.copy(), st.copy(), cs.copy(), st.copy()
    o1 = O.kda_decode(x, cw, None, cs1, raw_g, raw_beta, st1, idx, H=H, D=D, gate=gate)
    yy = O.conv1d_update(x, cw, None, cs2, idx)
    o2 = O.kda_step(np.nan_to_num(yy), raw_g, raw_beta, st2, idx, H=H, D=D, gate=gate)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(cs1, cs2)
    np.testing.assert_array_equal(st1, st2)
    np.testing.assert_array_equal(st1[0], st[0])
    assert np.isnan(o1[1]).all()


def test_pin_gdn_conv_is_conv_then_step():
    """The fused GDN conv step equals the conv update (SiLU) followed by the GDN
    step on the fp64 conv output; padded rows (GDN rule: < 0 or >= num_slots)
    touch neither the conv state nor the recurrent state."""
    rng = np.random.default_rng(50)
    B, H, HV, K, V, W = 3, 2, 4, 8, 6, 4
    C = 2 * H * K + HV * V
    x = rng.standard_normal((B, C))
    cw = rng.standard_normal((C, W)) * 0.5
    cb = rng.standard_normal(C) * 0.1
    a, b = rng.standard_normal((B, HV)), rng.standard_normal((B, HV))
    A_log, dt_bias = rng.standard_normal(HV) * 0.3, rng.standard_normal(HV) * 0.1
    cs = rng.standard_normal((4, C, W - 1))
    st = rng.standard_normal((4, HV, V, K))
    idx = np.array([2, -1, 0], np.int32)
    cs1, st1, cs2, st2 = cs.copy(), st.copy(), cs.copy(), st.copy()
    o1 = O.gdn_step_conv(x, cw, cb, cs1, a, b, A_log, dt_bias, st1, idx, H=H, HV=HV, K=K, V=V)
    y = O.conv1d_update(x, cw, cb, cs2, idx, skip_slot0=False)
    o2 = O.gdn_step(np.nan_to_num(y), a, b, A_log, dt_bias, st2, idx, H=H, HV=HV, K=K, V=V)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(cs1, cs2)
    np.testing.assert_array_equal(st1, st2)
    for s_ in (1, 3):
        np.testing.assert_array_equal(cs1[s_], cs[s_])
        np.testing.assert_array_equal(st1[s_], st[s_])
    assert not np.array_equal(cs1[0], cs[0])  # slot 0 is a real slot for GDN
    assert np.isnan(o1[1]).all()


# ------------------------------------------------------------ Mamba-1
def test_pin_mamba_scalar_recurrence():
    """N = 1 with constant inputs: h_T = a^T h0 + dB x (1 - a^T) / (1 - a) with
    a = exp(dt A), dB = dt B; y = C h + D x, times silu(z)."""
    dt, A, Bv, Cv, Dv, x, z, h0, T = 0.05, -3.0, 0.7, 1.3, 0.4, 0.9, 0.6, 2.0, 25
    h = np.array([[[h0]]])
    for t in range(1, T + 1):
        y = O.mamba_step([[x]], [[dt]], [[A]], [[Bv]], [[Cv]], [Dv], [[z]], h, [0])
        a = math.exp(dt * A)
        ht = a ** t * h0 + dt * Bv * x * (1 - a ** t) / (1 - a)
        assert h[0, 0, 0] == pytest.approx(ht, rel=1e-13)
        silu = z / (1 + math.exp(-z))
        assert y[0, 0] == pytest.approx((Cv * ht + Dv * x) * silu, rel=1e-13)


def test_pin_mamba_channels_independent_and_padding():
    """A channel's result depends only on its own (d, n) row; padded rows are
    untouched; N > 1 sums C[n] h[n]."""
    rng = np.random.default_rng(40)
    B, Dm, N = 2, 3, 4
    x, dt = rng.standard_normal((B, Dm)), np.full((B, Dm), 0.1)
    A = -np.abs(rng.standard_normal((Dm, N)))
    Bm, Cm = rng.standard_normal((B, N)), rng.standard_normal((B, N))
    h = rng.standard_normal((3, Dm, N))
    h0 = h.copy()
    y = O.mamba_step(x, dt, A, Bm, Cm, None, None, h, [2, -1])
    for d in range(Dm):
        hn = np.exp(0.1 * A[d]) * h0[2, d] + 0.1 * Bm[0] * x[0, d]
        np.testing.assert_allclose(h[2, d], hn, rtol=1e-15)
        assert y[0, d] == pytest.approx(float(Cm[0] @ hn), rel=1e-13)
    assert np.isnan(y[1]).all()
    np.testing.assert_array_equal(h[:2], h0[:2])


def test_pin_mamba_scan_scalar_closed_form():
    """The multi-token scan with N = 1 and constant inputs over T tokens:
    every y_t and the final state follow the geometric closed form, from a
    stored initial state and from zero."""
    dt, A, Bv, Cv, Dv, x, z, h0, T = 0.05, -3.0, 0.7, 1.3, 0.4, 0.9, 0.6, 2.0, 25
    a = math.exp(dt * A)
    silu = z / (1 + math.exp(-z))
    for zero_init, start in ((False, h0), (True, 0.0)):
        h = np.array([[[h0]]])
        y = O.mamba_scan(np.full((1, T, 1), x), np.full((1, T, 1), dt), [[A]], np.full((1, T, 1), Bv),
                         np.full((1, T, 1), Cv), [Dv], np.full((1, T, 1), z), h, [0], zero_init=zero_init)
        for t in range(1, T + 1):
            ht = a ** t * start + dt * Bv * x * (1 - a ** t) / (1 - a)
            assert y[0, t - 1, 0] == pytest.approx((Cv * ht + Dv * x) * silu, rel=1e-13)
        assert h[0, 0, 0] == pytest.approx(a ** T * start + dt * Bv * x * (1 - a ** T) / (1 - a), rel=1e-13)


def test_pin_mamba_scan_splits_and_lengths():
    """Scanning T1 tokens then T2 more from the stored state equals scanning
    T1 + T2 at once; a row of length L < T is the scan of its first L tokens
    and leaves y past L unwritten; padded rows touch nothing; T = 1 is the
    decode step."""
    rng = np.random.default_rng(41)
    B, T, Dm, N = 3, 9, 5, 4
    x, z = rng.standard_normal((B, T, Dm)), rng.standard_normal((B, T, Dm))
    dt = rng.uniform(0.01, 0.2, (B, T, Dm))
    A = -rng.uniform(0.5, 4.0, (Dm, N))
    Bm, Cm = rng.standard_normal((B, T, N)), rng.standard_normal((B, T, N))
    Dv = rng.standard_normal(Dm)
    h0 = rng.standard_normal((4, Dm, N))
    idx = [3, 0, 1]
    hw = h0.copy()
    yw = O.mamba_scan(x, dt, A, Bm, Cm, Dv, z, hw, idx)
    hs = h0.copy()
    y1 = O.mamba_scan(x[:, :4], dt[:, :4], A, Bm[:, :4], Cm[:, :4], Dv, z[:, :4], hs, idx)
    y2 = O.mamba_scan(x[:, 4:], dt[:, 4:], A, Bm[:, 4:], Cm[:, 4:], Dv, z[:, 4:], hs, idx)
    np.testing.assert_allclose(np.concatenate([y1, y2], axis=1), yw, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(hs, hw, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(hw[2], h0[2])  # slot 2 is not named
    hl = h0.copy()
    yl = O.mamba_scan(x, dt, A, Bm, Cm, Dv, z, hl, idx, lengths=[9, 4, 0])
    np.testing.assert_allclose(yl[0], yw[0], rtol=1e-12)
    np.testing.assert_allclose(yl[1, :4], y1[1], rtol=1e-12)
    assert np.isnan(yl[1, 4:]).all() and np.isnan(yl[2]).all()
    np.testing.assert_allclose(hl[0], _state_by_steps(x, dt, A, Bm, Cm, Dv, z, h0, b=1, slot=0, L=4),
                               rtol=1e-12)
    np.testing.assert_array_equal(hl[1], h0[1])  # length 0: state unchanged
    hp = h0.copy()
    yp = O.mamba_scan(x, dt, A, Bm, Cm, Dv, z, hp, [-1, 4, 2])
    assert np.isnan(yp[:2]).all()
    np.testing.assert_array_equal(hp[[0, 1, 3]], h0[[0, 1, 3]])
    h1, hstep = h0.copy(), h0.copy()
    ys = O.mamba_scan(x[:, :1], dt[:, :1], A, Bm[:, :1], Cm[:, :1], Dv, z[:, :1], h1, idx)
    yst = O.mamba_step(x[:, 0], dt[:, 0], A, Bm[:, 0], Cm[:, 0], Dv, z[:, 0], hstep, idx)
    np.testing.assert_allclose(ys[:, 0], yst, rtol=1e-14)
    np.testing.assert_allclose(h1, hstep, rtol=1e-14)


def _state_by_steps(x, dt, A, Bm, Cm, Dv, z, h0, *, b, slot, L):
    """State of row b (stored at slot) after its first L tokens, by L single
    decode steps."""
    h = h0.copy()
    for t in range(L):
        O.mamba_step(x[b:b + 1, t], dt[b:b + 1, t], A, Bm[b:b + 1, t], Cm[b:b + 1, t], Dv, z[b:b + 1, t], h, [slot])
    return h[slot]


def _gdn_multi_inputs(seed, B, T, H, HV, K, V, slots):
    rng = np.random.default_rng(seed)
    C = 2 * H * K + HV * V
    return dict(qkv=rng.standard_normal((B, T, C)), a=0.5 * rng.standard_normal((B, T, HV)),
                b=rng.standard_normal((B, T, HV)), A_log=0.3 * rng.standard_normal(HV),
                dt_bias=0.1 * rng.standard_normal(HV), gate=rng.standard_normal((B, T, HV, V)),
                w=1 + 0.1 * rng.standard_normal(V), state=rng.standard_normal((slots, HV, V, K)))


def test_pin_gdn_multi_is_token_by_token_steps():
    """T tokens in one call equal T single steps on each token's slice (GQA,
    gated norm, permuted slots), bit for bit."""
    B, T, H, HV, K, V = 3, 5, 2, 4, 8, 6
    d = _gdn_multi_inputs(50, B, T, H, HV, K, V, 4)
    idx = [2, 0, 3]
    st_m, st_s = d["state"].copy(), d["state"].copy()
    om = O.gdn_multi(d["qkv"], d["a"], d["b"], d["A_log"], d["dt_bias"], st_m, idx, H=H, HV=HV, K=K, V=V,
                     norm_gate=d["gate"], norm_weight=d["w"])
    for t in range(T):
        os_ = O.gdn_step(d["qkv"][:, t], d["a"][:, t], d["b"][:, t], d["A_log"], d["dt_bias"], st_s, idx,
                         H=H, HV=HV, K=K, V=V, norm_gate=d["gate"][:, t], norm_weight=d["w"])
        np.testing.assert_array_equal(om[:, t], os_)
    np.testing.assert_array_equal(st_m, st_s)


def test_pin_gdn_multi_lengths_padding_split():
    """A row of length L < T is the first L tokens and writes nothing after;
    a padded row touches nothing; T1 tokens then T2 more equal T1 + T2."""
    B, T, H, HV, K, V = 4, 6, 1, 2, 4, 3
    d = _gdn_multi_inputs(51, B, T, H, HV, K, V, 5)
    idx = [4, -1, 1, 2]
    lengths = [6, 6, 2, 0]
    st = d["state"].copy()
    o = O.gdn_multi(d["qkv"], d["a"], d["b"], d["A_log"], d["dt_bias"], st, idx, H=H, HV=HV, K=K, V=V,
                    lengths=lengths)
    assert np.isnan(o[1]).all() and np.isnan(o[2, 2:]).all() and np.isnan(o[3]).all()
    for s_ in (0, 2, 3):
        np.testing.assert_array_equal(st[s_], d["state"][s_])
    st2 = d["state"].copy()
    o2 = O.gdn_multi(d["qkv"][:, :2], d["a"][:, :2], d["b"][:, :2], d["A_log"], d["dt_bias"], st2, idx,
                     H=H, HV=HV, K=K, V=V)
    np.testing.assert_array_equal(o[2, :2], o2[2])
    np.testing.assert_array_equal(st[1], st2[1])  # row 2 (slot 1) stopped after 2 tokens
    st3 = d["state"].copy()
    o3a = O.gdn_multi(d["qkv"][:, :4], d["a"][:, :4], d["b"][:, :4], d["A_log"], d["dt_bias"], st3, idx,
                      H=H, HV=HV, K=K, V=V)
    o3b = O.gdn_multi(d["qkv"][:, 4:], d["a"][:, 4:], d["b"][:, 4:], d["A_log"], d["dt_bias"], st3, idx,
                      H=H, HV=HV, K=K, V=V)
    np.testing.assert_array_equal(np.concatenate([o3a, o3b], axis=1)[0], o[0])
    np.testing.assert_array_equal(st3[4], st[4])


# ------------------------------------------------------- fp32 build of the oracle
def test_fp32_build_matches_fp64_on_tiny_chain():
    """The oracle's fp32 build of the packed step against its fp64 one on the
    tiny workload (B = 2, H = HV = 2, K = V = 16, fp32 inputs, q/k L2-normed,
    a ~ N(0,1), S0 ~ N(0, 0.1^2)), 64 chained steps from the same fp32
    state, each side on its own trajectory: every output and the final state
    within 1e-5 (the fp32 tolerance of [MBU] "Correctness"). A mistake in
    either build (they share no code) separates them by far more."""
    import workloads as W
    from tests._helpers import mixed_err
    w = W.GDN_TINY
    P, idx = W.gdn_params(w), W.slot_indices(w)
    s0 = W.gdn_state(w)
    s64, s32 = s0.double().numpy().copy(), s0.numpy().copy()
    worst = 0.0
    for t in range(w.steps):
        x = W.gdn_step_inputs(w, t)
        o64 = O.gdn_step(x["qkv"], x["a"], x["b"], P["A_log"], P["dt_bias"], s64, idx, H=w.H, HV=w.HV, K=w.K,
                         V=w.V)
        o32 = O.gdn_step_f32(x["qkv"], x["a"], x["b"], P["A_log"], P["dt_bias"], s32, idx, H=w.H, HV=w.HV,
                             K=w.K, V=w.V)
        worst = max(worst, float(mixed_err(o32, o64).max()))
    worst = max(worst, float(mixed_err(s32, s64).max()))
    assert worst <= 1e-5, worst
    assert worst > 0.0  # the float build really rounds to fp32
