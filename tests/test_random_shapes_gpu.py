"""Seeded random-shape parity sweep of the decode entry points against the
fp64 oracle: head sizes, ragged value dims, GQA ratios, dtypes, gated norm
on/off, padded rows and (buffered) mixed and out-of-range phases drawn from a
fixed generator, so every run checks the same cases. Complements the
hand-picked cases of the per-entry-point tests with combinations nobody chose.
The `large` tests draw batches with more than four heads per CU of a 256-CU
part, so the launch shapes chosen for large batches (32-row tiles of the
packed step, one-unit tiles of the 16-bit-state step, 2-wave buffered blocks,
one block per conv group) meet ragged shapes too.
"""
import numpy as np
import pytest
import torch

import oracle as O
import ssm_recurrent_decode_gated_amd as S
import workloads as W
from tests._helpers import FP32_TOL, assert_out16, assert_mixed, assert_rounded16, need_gpu, to_np64

pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
FMT = {"f32": O.FMT_F32, "bf16": O.FMT_BF16, "f16": O.FMT_F16}
MANT = {"bf16": 7, "f16": 10}


def _draw(rng, i):
    K = int(rng.choice([16, 32, 64, 128, 256]))
    H = int(rng.integers(1, 4))
    G = int(rng.choice([1, 2, 4]))
    V = int(rng.choice([1, 3, 16, 40, 64, 100, 128, 200, 300]))
    B = int(rng.integers(1, 10))
    slots = B + int(rng.integers(0, 5))
    act = str(rng.choice(["f32", "bf16", "f16"]))
    out = str(rng.choice(["f32", "bf16", "f16"]))
    norm = str(rng.choice(["none", "silu", "sigmoid"]))
    w = W.GDNWorkload(f"rand{i}_k{K}_h{H}_g{G}_v{V}_b{B}_{act}", B=B, H=H, HV=G * H, K=K, V=V, num_slots=slots,
                      act=act, out=out, idx="perm")
    idx = W.slot_indices(w).clone()
    for b in range(B):  # about one row in five padded, both ways
        if rng.random() < 0.2:
            idx[b] = -1 if rng.random() < 0.5 else slots + int(rng.integers(0, 3))
    return w, idx, norm


def _draw_large(rng, i, K=None, G=None, V=None):
    """A large-batch case: B HV >= 1100 heads, state at most 40 M elements."""
    K = int(rng.choice([16, 32, 64, 128, 128, 256])) if K is None else K
    G = int(rng.choice([1, 2, 4])) if G is None else G
    H = int(rng.choice([2, 4, 8]))
    HV = G * H
    B = -(-1100 // HV) + int(rng.integers(0, 40))
    vs = [v for v in (16, 40, 64, 100, 128, 200) if B * HV * v * K <= 40_000_000]
    V = int(rng.choice(vs)) if V is None else V
    slots = B + int(rng.integers(0, 5))
    act = str(rng.choice(["f32", "bf16", "f16"]))
    out = str(rng.choice(["f32", "bf16", "f16"]))
    norm = str(rng.choice(["none", "none", "silu", "sigmoid"]))
    w = W.GDNWorkload(f"large{i}_k{K}_h{H}_g{G}_v{V}_b{B}_{act}", B=B, H=H, HV=HV, K=K, V=V, num_slots=slots,
                      act=act, out=out, idx="perm")
    idx = W.slot_indices(w).clone()
    for b in range(B):
        if rng.random() < 0.2:
            idx[b] = -1 if rng.random() < 0.5 else slots + int(rng.integers(0, 3))
    return w, idx, norm


def _check(out, ref, live, what):
    if not live:
        return
    o = out[live]
    if o.dtype == torch.float32:
        assert_mixed(o, ref[live], FP32_TOL, what)
    else:
        assert_out16(o, ref[live], FP32_TOL, what)


CASES = list(range(48))


@pytest.mark.parametrize("i", CASES)
def test_random_gdn_step(i):
    need_gpu()
    rng = np.random.default_rng(1000 + i)
    _case_gdn_step(i, *_draw(rng, i))


@pytest.mark.parametrize("i", range(12))
def test_random_large_gdn_step(i):
    need_gpu()
    rng = np.random.default_rng(11000 + i)
    _case_gdn_step(i, *_draw_large(rng, i))


def _case_gdn_step(i, w, idx, norm):
    P, x = W.gdn_params(w), W.gdn_step_inputs(w, norm=norm != "none")
    st = W.gdn_state(w)
    st_d = st.to(DEV)
    out = torch.full((w.B, 1, w.HV, w.V), float("nan"), dtype=TD[w.out], device=DEV)
    kw, okw = {}, {}
    if norm != "none":
        kw = dict(norm_gate=x["norm_gate"].to(DEV), norm_weight=x["norm_weight"].to(DEV), norm_act=norm)
        okw = dict(norm_gate=x["norm_gate"], norm_weight=x["norm_weight"],
                   norm_act=O.ACT_SIGMOID if norm == "sigmoid" else O.ACT_SILU)
    S.gdn_decode_step(x["qkv"].to(DEV), x["a"].to(DEV), x["b"].to(DEV), P["A_log"].to(DEV), P["dt_bias"].to(DEV),
                      st_d, idx.to(DEV), out, **kw)
    ref = st.double().numpy().copy()
    ro = O.gdn_step(x["qkv"], x["a"], x["b"], P["A_log"], P["dt_bias"], ref, idx, H=w.H, HV=w.HV, K=w.K, V=w.V,
                    **okw)
    torch.cuda.synchronize()
    live = [b for b in range(w.B) if 0 <= int(idx[b]) < w.num_slots]
    o = out.reshape(w.B, w.HV, w.V)
    _check(o, ro, live, f"case {i} ({w.name}, norm {norm}) output")
    dead = [b for b in range(w.B) if b not in live]
    if dead:
        assert torch.isnan(o[dead].float()).all(), f"case {i}: a padded row wrote its output"
    got = st_d.cpu()
    named = {int(idx[b]) for b in live}
    for s in range(w.num_slots):
        if s in named:
            assert_mixed(got[s], ref[s], FP32_TOL, f"case {i} slot {s}")
        else:
            assert torch.equal(got[s], st[s]), f"case {i}: slot {s} changed"


@pytest.mark.parametrize("i", CASES)
def test_random_gdn_buffered(i):
    need_gpu()
    rng = np.random.default_rng(2000 + i)
    w, idx, norm = _draw(rng, 100 + i)
    _case_gdn_buffered(i, rng, w, idx, norm)


@pytest.mark.parametrize("i", range(12))
def test_random_large_gdn_buffered(i):
    need_gpu()
    rng = np.random.default_rng(12000 + i)
    # K = 128 in half the cases: the head size whose large batches take 2-wave blocks
    w, idx, norm = _draw_large(rng, 100 + i, K=128 if i % 2 == 0 else None)
    _case_gdn_buffered(i, rng, w, idx, norm)


def _case_gdn_buffered(i, rng, w, idx, norm):
    L = int(rng.integers(1, 17))
    phases = [int(rng.integers(0, L)) if rng.random() > 0.1 else L for _ in range(w.B)]
    P, x = W.gdn_params(w), W.gdn_step_inputs(w, norm=norm != "none")
    st = W.gdn_state(w)
    ring = W.gdn_ring(w, L)
    st_d = st.to(DEV)
    ring_d = {k: v.to(DEV) for k, v in ring.items()}
    wp = torch.tensor(phases, dtype=torch.int32)
    out = torch.full((w.B, 1, w.HV, w.V), float("nan"), dtype=TD[w.out], device=DEV)
    kw, okw = {}, {}
    if norm != "none":
        kw = dict(norm_gate=x["norm_gate"].to(DEV), norm_weight=x["norm_weight"].to(DEV), norm_act=norm)
        okw = dict(norm_gate=x["norm_gate"], norm_weight=x["norm_weight"],
                   norm_act=O.ACT_SIGMOID if norm == "sigmoid" else O.ACT_SILU)
    S.gdn_decode_step_buffered(x["qkv"].to(DEV), x["a"].to(DEV), x["b"].to(DEV), P["A_log"].to(DEV),
                               P["dt_bias"].to(DEV), st_d, idx.to(DEV), out, ring_d["d_cache"], ring_d["k_cache"],
                               ring_d["g_cache"], wp.to(DEV), **kw)
    ref = st.double().numpy().copy()
    rr = {k: v.double().numpy().copy() for k, v in ring.items()}
    ro = O.gdn_step_buffered(x["qkv"], x["a"], x["b"], P["A_log"], P["dt_bias"], ref, idx, rr["d_cache"],
                             rr["k_cache"], rr["g_cache"], wp, L, H=w.H, HV=w.HV, K=w.K, V=w.V,
                             ring_fmt=FMT[w.act], **okw)
    ex = {k: v.double().numpy().copy() for k, v in ring.items()}
    O.gdn_step_buffered(x["qkv"], x["a"], x["b"], P["A_log"], P["dt_bias"], st.double().numpy().copy(), idx,
                        ex["d_cache"], ex["k_cache"], ex["g_cache"], wp, L, H=w.H, HV=w.HV, K=w.K, V=w.V,
                        ring_fmt=O.FMT_NONE, **okw)
    torch.cuda.synchronize()
    live = [b for b in range(w.B) if 0 <= int(idx[b]) < w.num_slots and 0 <= phases[b] < L]
    o = out.reshape(w.B, w.HV, w.V)
    _check(o, ro, live, f"case {i} ({w.name}, L {L}, norm {norm}) output")
    got_st = st_d.cpu()
    got = {k: to_np64(v) for k, v in ring_d.items()}
    ring0 = {k: to_np64(v) for k, v in ring.items()}
    for b in live:
        s, p = int(idx[b]), phases[b]
        if p == L - 1:  # a flush writes the folded state and appends no record
            assert_mixed(got_st[s], ref[s], FP32_TOL, f"case {i} flushed slot {s}")
            for k in ring0:
                np.testing.assert_array_equal(got[k][s], ring0[k][s], err_msg=f"case {i} {k} slot {s} (flush)")
            continue
        assert torch.equal(got_st[s], st[s]), f"case {i}: non-flush slot {s} written"
        for k in ("d_cache", "k_cache"):
            if w.act == "f32":
                assert_mixed(got[k][s][:, p], rr[k][s][:, p], FP32_TOL, f"case {i} {k} row {b}")
            else:
                assert_rounded16(got[k][s][:, p], rr[k][s][:, p], f"case {i} {k} row {b}", ex[k][s][:, p],
                              MANT[w.act])
        np.testing.assert_allclose(got["g_cache"][s][:, p], rr["g_cache"][s][:, p], rtol=1e-5)
    touched = {int(idx[b]) for b in live}
    for s in set(range(w.num_slots)) - touched:
        assert torch.equal(got_st[s], st[s]), f"case {i}: slot {s} changed"


@pytest.mark.parametrize("i", CASES[:24])
def test_random_kda(i):
    need_gpu()
    rng = np.random.default_rng(3000 + i)
    D = int(rng.choice([16, 32, 64, 128, 256]))
    H = int(rng.integers(1, 5))
    T = int(rng.integers(1, 9))
    Wd = int(rng.choice([2, 3, 4, 4]))
    w = W.KDAWorkload(f"kda_rand{i}_d{D}_h{H}_t{T}_w{Wd}", T=T, H=H, D=D, W=Wd, num_slots=T + 3)
    layout = str(rng.choice(["SD", "DS"]))
    d = W.kda_inputs(w, layout=layout)
    for t in range(T):  # about one token in five skipped: the NULL slot 0 or past the pool
        if rng.random() < 0.2:
            d["idx"][t] = 0 if rng.random() < 0.5 else w.num_slots
    norm = bool(rng.random() < 0.6)
    cs_d = d["conv_state"].to(DEV)
    st_d = d["state"].to(DEV)
    out = torch.full((T, H, D), 7.0, dtype=torch.float32, device=DEV)
    S.kda_decode_step(d["x"].to(DEV), d["conv_weight"].to(DEV), None, cs_d, d["raw_g"].to(DEV),
                      d["raw_beta"].to(DEV), None, None, st_d, d["idx"].to(DEV), out,
                      output_gate=d["gate"].to(DEV) if norm else None,
                      norm_weight=d["norm_weight"].to(DEV) if norm else None,
                      lower_bound=w.lower_bound, norm_eps=w.norm_eps)
    cs_ref = d["conv_state"].double().numpy().copy()
    st_ref = d["state"].double().numpy().copy()
    ro = O.kda_decode(d["x"], d["conv_weight"], None, cs_ref, d["raw_g"], d["raw_beta"], st_ref, d["idx"], H=H, D=D,
                      lower_bound=w.lower_bound, gate=d["gate"] if norm else None,
                      norm_weight=d["norm_weight"] if norm else None, norm_eps=w.norm_eps)
    torch.cuda.synchronize()
    live = [t for t, s in enumerate(d["idx"].tolist()) if 0 < s < w.num_slots]
    if live:
        assert_mixed(out[live], ro[live], FP32_TOL, f"case {i} ({w.name}, {layout}, norm {norm}) output")
    got = st_d.cpu()
    named = {int(d["idx"][t]) for t in live}
    for s in range(w.num_slots):
        if s in named:
            assert_mixed(got[s], st_ref[s], FP32_TOL, f"case {i} state slot {s}")
        else:
            assert torch.equal(got[s], d["state"][s]), f"case {i}: slot {s} changed"
    skipped = [t for t in range(T) if t not in live]
    if skipped:
        assert (out[skipped] == 7.0).all(), f"case {i}: a skipped token wrote its output"
    # the conv state holds raw inputs: bit for bit
    assert np.array_equal(to_np64(cs_d), cs_ref), f"case {i}: conv state differs"


def _norm_kw(x, norm):
    if norm == "none":
        return {}, {}
    return (dict(norm_gate=x["norm_gate"].to(DEV), norm_weight=x["norm_weight"].to(DEV), norm_act=norm),
            dict(norm_gate=x["norm_gate"], norm_weight=x["norm_weight"],
                 norm_act=O.ACT_SIGMOID if norm == "sigmoid" else O.ACT_SILU))


@pytest.mark.parametrize("i", CASES[:24])
def test_random_gdn_conv(i):
    need_gpu()
    rng = np.random.default_rng(4000 + i)
    w, idx, norm = _draw(rng, 200 + i)
    _case_gdn_conv(i, rng, w, idx, norm, int(rng.integers(2, 9)))


@pytest.mark.parametrize("i", range(8))
def test_random_large_gdn_conv(i):
    """Half the cases have the shape of the one-block-per-group kernel (width
    4, G V = 256, K = 64 or 128, no norm)."""
    need_gpu()
    rng = np.random.default_rng(14000 + i)
    if i % 2 == 0:
        G = int(rng.choice([2, 4]))
        w, idx, norm = _draw_large(rng, 200 + i, K=int(rng.choice([64, 128])), G=G, V=256 // G)
        _case_gdn_conv(i, rng, w, idx, "none", 4)
    else:
        w, idx, norm = _draw_large(rng, 200 + i)
        _case_gdn_conv(i, rng, w, idx, norm, int(rng.integers(2, 9)))


def _case_gdn_conv(i, rng, w, idx, norm, Wd):
    layout = str(rng.choice(["DS", "SD"]))
    P, x = W.gdn_params(w), W.gdn_step_inputs(w, norm=norm != "none")
    st, cv = W.gdn_state(w), W.gdn_conv(w, Wd, layout=layout, bias=bool(rng.random() < 0.5))
    st_d, cs_d = st.to(DEV), cv["conv_state"].to(DEV)
    out = torch.full((w.B, 1, w.HV, w.V), float("nan"), dtype=TD[w.out], device=DEV)
    kw, okw = _norm_kw(x, norm)
    cb = cv["conv_bias"]
    S.gdn_decode_step_conv(x["qkv"].to(DEV), cv["conv_weight"].to(DEV), None if cb is None else cb.to(DEV), cs_d,
                           x["a"].to(DEV), x["b"].to(DEV), P["A_log"].to(DEV), P["dt_bias"].to(DEV), st_d,
                           idx.to(DEV), out, **kw)
    ref, ref_cs = st.double().numpy().copy(), cv["conv_state"].double().numpy().copy()
    ro = O.gdn_step_conv(x["qkv"], cv["conv_weight"], cb, ref_cs, x["a"], x["b"], P["A_log"], P["dt_bias"], ref, idx,
                         H=w.H, HV=w.HV, K=w.K, V=w.V, **okw)
    torch.cuda.synchronize()
    live = [b for b in range(w.B) if 0 <= int(idx[b]) < w.num_slots]
    _check(out.reshape(w.B, w.HV, w.V), ro, live, f"case {i} ({w.name}, W {Wd}, {layout}, norm {norm}) output")
    got, got_cs = st_d.cpu(), cs_d.cpu()
    named = {int(idx[b]) for b in live}
    for s in range(w.num_slots):
        if s in named:
            assert_mixed(got[s], ref[s], FP32_TOL, f"case {i} slot {s}")
        else:
            assert torch.equal(got[s], st[s]), f"case {i}: slot {s} changed"
    # the conv state holds raw inputs: bit for bit, touched and untouched slots alike
    assert np.array_equal(to_np64(got_cs), ref_cs), f"case {i}: conv state differs"


@pytest.mark.parametrize("i", CASES[:24])
def test_random_gdn_state16(i):
    need_gpu()
    rng = np.random.default_rng(5000 + i)
    w, idx, norm = _draw(rng, 300 + i)
    _case_gdn_state16(i, rng, w, idx, norm)


@pytest.mark.parametrize("i", range(12))
def test_random_large_gdn_state16(i):
    need_gpu()
    rng = np.random.default_rng(15000 + i)
    w, idx, norm = _draw_large(rng, 300 + i)
    _case_gdn_state16(i, rng, w, idx, norm)


def _case_gdn_state16(i, rng, w, idx, norm):
    sdt = torch.bfloat16 if rng.random() < 0.5 else torch.float16
    P, x = W.gdn_params(w), W.gdn_step_inputs(w, norm=norm != "none")
    st = W.gdn_state(w).to(sdt)
    st_d = st.to(DEV)
    out = torch.full((w.B, 1, w.HV, w.V), float("nan"), dtype=TD[w.out], device=DEV)
    kw, okw = _norm_kw(x, norm)
    S.gdn_decode_step_state16(x["qkv"].to(DEV), x["a"].to(DEV), x["b"].to(DEV), P["A_log"].to(DEV),
                              P["dt_bias"].to(DEV), st_d, idx.to(DEV), out, **kw)
    fmt = O.FMT_BF16 if sdt == torch.bfloat16 else O.FMT_F16
    ref, exact = st.double().numpy().copy(), st.double().numpy().copy()
    ro = O.gdn_step(x["qkv"], x["a"], x["b"], P["A_log"], P["dt_bias"], ref, idx, H=w.H, HV=w.HV, K=w.K, V=w.V,
                    state_fmt=fmt, **okw)
    O.gdn_step(x["qkv"], x["a"], x["b"], P["A_log"], P["dt_bias"], exact, idx, H=w.H, HV=w.HV, K=w.K, V=w.V,
               state_fmt=O.FMT_NONE, **okw)
    torch.cuda.synchronize()
    live = [b for b in range(w.B) if 0 <= int(idx[b]) < w.num_slots]
    _check(out.reshape(w.B, w.HV, w.V), ro, live, f"case {i} ({w.name}, {sdt}, norm {norm}) output")
    got = st_d.cpu()
    named = {int(idx[b]) for b in live}
    for s in range(w.num_slots):
        if s in named:
            assert_rounded16(to_np64(got[s]), ref[s], f"case {i} slot {s}", exact[s],
                             7 if sdt == torch.bfloat16 else 10)
        else:
            assert torch.equal(got[s], st[s]), f"case {i}: slot {s} changed"


@pytest.mark.parametrize("i", CASES[:24])
def test_random_gdn_multi(i):
    need_gpu()
    rng = np.random.default_rng(6000 + i)
    w, idx, norm = _draw(rng, 400 + i)
    _case_gdn_multi(i, rng, w, idx, int(rng.integers(1, 12)))


@pytest.mark.parametrize("i", range(8))
def test_random_large_gdn_multi(i):
    need_gpu()
    rng = np.random.default_rng(16000 + i)
    w, idx, norm = _draw_large(rng, 400 + i)
    _case_gdn_multi(i, rng, w, idx, int(rng.integers(1, 5)))


def _case_gdn_multi(i, rng, w, idx, T):
    lengths = torch.tensor([int(rng.integers(0, T + 1)) for _ in range(w.B)], dtype=torch.int32)
    P = W.gdn_params(w)
    g = W.generator(0, w.name, "rand_multi", T)
    C = 2 * w.H * w.K + w.HV * w.V
    qkv = W.normal((w.B, T, C), 1.0, w.act, g)
    a = W.normal((w.B, T, w.HV), 0.5, w.act, g)
    b = W.normal((w.B, T, w.HV), 1.0, w.act, g)
    st = W.gdn_state(w)
    st_d = st.to(DEV)
    out = torch.full((w.B, T, w.HV, w.V), float("nan"), dtype=TD[w.out], device=DEV)
    S.gdn_fused_recurrent(qkv.to(DEV), a.to(DEV), b.to(DEV), P["A_log"].to(DEV), P["dt_bias"].to(DEV), st_d,
                          idx.to(DEV), out, lengths=lengths.to(DEV))
    ref = st.double().numpy().copy()
    ro = O.gdn_multi(qkv, a, b, P["A_log"], P["dt_bias"], ref, idx, H=w.H, HV=w.HV, K=w.K, V=w.V, lengths=lengths)
    torch.cuda.synchronize()
    for bi in range(w.B):
        n = int(lengths[bi])
        if not (0 <= int(idx[bi]) < w.num_slots) or n == 0:
            continue
        o, r = out[bi, :n], ro[bi, :n]
        if o.dtype == torch.float32:
            assert_mixed(o, r, CHAIN_TOL_T(n), f"case {i} ({w.name}, T {T}) row {bi} outputs")
        else:
            assert_out16(o, r, CHAIN_TOL_T(n), f"case {i} ({w.name}, T {T}) row {bi} outputs")
        assert torch.isnan(out[bi, n:].float()).all(), f"case {i}: outputs past row {bi}'s length written"
    got = st_d.cpu()
    for s in range(w.num_slots):
        rows = [bi for bi in range(w.B) if int(idx[bi]) == s and int(lengths[bi]) > 0]
        if rows:
            assert_mixed(got[s], ref[s], CHAIN_TOL_T(int(lengths[rows[0]])), f"case {i} slot {s}")
        else:
            assert torch.equal(got[s], st[s]), f"case {i}: slot {s} changed"


def CHAIN_TOL_T(n):
    """Bar for outputs and states after n chained tokens: the single-step bar
    for one token, the chained bar beyond."""
    return FP32_TOL if n <= 1 else 2e-3


@pytest.mark.parametrize("i", CASES[:24])
def test_random_mamba_decode(i):
    need_gpu()
    rng = np.random.default_rng(7000 + i)
    N = int(rng.choice([16, 32, 64, 128, 256]))
    Dm = int(rng.choice([1, 7, 64, 100, 300, 1536]))
    B = int(rng.integers(1, 9))
    act = str(rng.choice(["f32", "bf16", "f16"]))
    w = W.MambaWorkload(f"mamba_rand{i}_n{N}_d{Dm}_b{B}", B=B, Dm=Dm, N=N, num_slots=B + 2)
    d = W.mamba_inputs(w, act=act)
    use_D, use_z = bool(rng.random() < 0.5), bool(rng.random() < 0.5)
    idx = d["idx"].clone() if "idx" in d else torch.arange(B, dtype=torch.int32)
    for bi in range(B):
        if rng.random() < 0.2:
            idx[bi] = -1
    h_d = d["h"].to(DEV)
    out = torch.full((B, Dm), float("nan"), dtype=torch.float32, device=DEV)
    S.mamba_decode_step(d["x"].to(DEV), d["dt"].to(DEV), d["A"].to(DEV), d["Bm"].to(DEV), d["Cm"].to(DEV),
                        d["Dv"].to(DEV) if use_D else None, d["z"].to(DEV) if use_z else None, h_d, idx.to(DEV), out)
    ref = d["h"].double().numpy().copy()
    ro = O.mamba_step(d["x"], d["dt"], d["A"], d["Bm"], d["Cm"], d["Dv"] if use_D else None,
                      d["z"] if use_z else None, ref, idx)
    torch.cuda.synchronize()
    live = [bi for bi in range(B) if 0 <= int(idx[bi]) < w.num_slots]
    if live:
        assert_mixed(out[live], ro[live], FP32_TOL, f"case {i} ({w.name}, {act}, D {use_D}, z {use_z}) output")
    got = h_d.cpu()
    named = {int(idx[bi]) for bi in live}
    for s in range(w.num_slots):
        if s in named:
            assert_mixed(got[s], ref[s], FP32_TOL, f"case {i} slot {s}")
        else:
            assert torch.equal(got[s], d["h"][s]), f"case {i}: slot {s} changed"


def _tokens(w, T, seed_tag):
    g = W.generator(0, w.name, seed_tag, T)
    C = 2 * w.H * w.K + w.HV * w.V
    return (W.normal((w.B, T, C), 1.0, w.act, g), W.normal((w.B, T, w.HV), 0.5, w.act, g),
            W.normal((w.B, T, w.HV), 1.0, w.act, g), W.normal((w.B, T, w.HV, w.V), 1.0, w.act, g))


@pytest.mark.parametrize("i", CASES[:24])
def test_random_gdn_chunk_prefill(i):
    need_gpu()
    rng = np.random.default_rng(8000 + i)
    K = int(rng.choice([64, 128]))
    V = int(rng.choice([16, 48, 64, 128, 256]))
    H, G = int(rng.integers(1, 3)), int(rng.choice([1, 2, 4]))
    B = int(rng.integers(1, 5))
    T = int(rng.choice([1, 7, 63, 64, 65, 130, 200]))
    act, outd = str(rng.choice(["f32", "bf16", "f16"])), str(rng.choice(["f32", "bf16"]))
    norm = str(rng.choice(["none", "silu", "sigmoid"]))
    w = W.GDNWorkload(f"chunk_rand{i}_k{K}_v{V}_h{H}_g{G}_b{B}_t{T}_{act}", B=B, H=H, HV=G * H, K=K, V=V,
                      num_slots=B + 2, act=act, out=outd, idx="perm")
    idx = W.slot_indices(w).clone()
    if B > 1 and rng.random() < 0.5:
        idx[int(rng.integers(0, B))] = -1
    lengths = torch.tensor([int(rng.choice([T, int(rng.integers(0, T + 1))])) for _ in range(B)], dtype=torch.int32)
    P, st = W.gdn_params(w), W.gdn_state(w)
    qkv, a, b, z = _tokens(w, T, "rand_chunk")
    nw = torch.ones(V, dtype=torch.float32) * 0.75
    st_d = st.to(DEV)
    out = torch.full((B, T, w.HV, V), 7.0, dtype=TD[outd], device=DEV)
    kw = dict(norm_gate=z.to(DEV), norm_weight=nw.to(DEV), norm_act=norm) if norm != "none" else {}
    S.gdn_chunk_prefill(qkv.to(DEV), a.to(DEV), b.to(DEV), P["A_log"].to(DEV), P["dt_bias"].to(DEV), st_d,
                        idx.to(DEV), out, lengths=lengths.to(DEV), **kw)
    ref = st.double().numpy().copy()
    okw = dict(norm_gate=z, norm_weight=nw, norm_act=O.ACT_SIGMOID if norm == "sigmoid" else O.ACT_SILU) \
        if norm != "none" else {}
    ro = O.gdn_multi(qkv, a, b, P["A_log"], P["dt_bias"], ref, idx, H=H, HV=w.HV, K=K, V=V, lengths=lengths, **okw)
    torch.cuda.synchronize()
    o = out.cpu()
    for bi in range(B):
        n = int(lengths[bi])
        live = 0 <= int(idx[bi]) < w.num_slots
        if live and n:
            if o.dtype == torch.float32:
                assert_mixed(o[bi, :n], ro[bi, :n], CHAIN_TOL_T(n), f"case {i} ({w.name}, norm {norm}) row {bi}")
            else:
                assert_out16(o[bi, :n], ro[bi, :n], CHAIN_TOL_T(n), f"case {i} ({w.name}, norm {norm}) row {bi}")
        assert (o[bi, n if live else 0:].float() == 7.0).all(), f"case {i}: row {bi} wrote past its length"
    got = st_d.cpu()
    for s in range(w.num_slots):
        rows = [bi for bi in range(B) if int(idx[bi]) == s and int(lengths[bi]) > 0]
        if rows:
            assert_mixed(got[s], ref[s], CHAIN_TOL_T(int(lengths[rows[0]])), f"case {i} slot {s}")
        else:
            assert torch.equal(got[s], st[s]), f"case {i}: slot {s} changed"


@pytest.mark.parametrize("i", CASES[:24])
def test_random_mamba_scan(i):
    need_gpu()
    rng = np.random.default_rng(9000 + i)
    N = int(rng.choice([16, 32, 64, 128, 256]))
    Dm = int(rng.choice([7, 64, 100, 300, 1536]))
    B = int(rng.integers(1, 5))
    T = int(rng.choice([1, 5, 31, 64, 100, 257]))
    act = str(rng.choice(["f32", "bf16", "f16"]))
    w = W.MambaScanWorkload(f"scan_rand{i}_n{N}_d{Dm}_b{B}_t{T}_{act}", B=B, T=T, Dm=Dm, N=N, num_slots=B + 2)
    d = W.mamba_scan_inputs(w, act=act)
    lengths = torch.tensor([int(rng.choice([T, int(rng.integers(0, T + 1))])) for _ in range(B)], dtype=torch.int32)
    idx = d["idx"].clone()
    if B > 1 and rng.random() < 0.5:
        idx[int(rng.integers(0, B))] = -1
    use_D, use_z, zero = bool(rng.random() < 0.5), bool(rng.random() < 0.5), bool(rng.random() < 0.3)
    ws_mode = str(rng.choice(["full", "none", "small"]))
    nws = S.mamba_scan_workspace_bytes(B, T, Dm, N)
    ws = None if ws_mode == "none" else torch.empty(max((nws if ws_mode == "full" else nws // 3) // 4, 1),
                                                      device=DEV)
    h_d = d["h"].to(DEV)
    out = torch.full((B, T, Dm), 7.0, dtype=torch.float32, device=DEV)
    S.mamba_scan(d["x"].to(DEV), d["dt"].to(DEV), d["A"].to(DEV), d["Bm"].to(DEV), d["Cm"].to(DEV),
                 d["Dv"].to(DEV) if use_D else None, d["z"].to(DEV) if use_z else None, h_d, idx.to(DEV), out,
                 lengths=lengths.to(DEV), zero_init=zero, workspace=ws)
    ref = d["h"].double().numpy().copy()
    ro = O.mamba_scan(d["x"], d["dt"], d["A"], d["Bm"], d["Cm"], d["Dv"] if use_D else None,
                      d["z"] if use_z else None, ref, idx, lengths=lengths, zero_init=zero)
    torch.cuda.synchronize()
    o = out.cpu()
    what = f"case {i} ({w.name}, ws {ws_mode}, D {use_D}, z {use_z}, zero {zero})"
    for bi in range(B):
        n = int(lengths[bi])
        live = 0 <= int(idx[bi]) < w.num_slots
        if live and n:
            assert_mixed(o[bi, :n], ro[bi, :n], CHAIN_TOL_T(n), f"{what} row {bi}")
        assert (o[bi, n if live else 0:] == 7.0).all(), f"{what}: row {bi} wrote past its length"
    got = h_d.cpu()
    for s in range(w.num_slots):
        rows = [bi for bi in range(B) if int(idx[bi]) == s]
        if rows:  # whatever the row's length, the pool must hold what the oracle's does
            assert_mixed(got[s], ref[s], CHAIN_TOL_T(max(int(lengths[rows[0]]), 1)), f"{what} slot {s}")
        else:
            assert torch.equal(got[s], d["h"][s]), f"{what}: slot {s} changed"
