"""Slot pools past 2^31 state elements. Every entry point that indexes a slot
pool runs here on a pool of more than 2^31 state elements (over 8 GiB of
fp32, over 4 GiB of bf16), with the named slots on both sides of the 4 GiB
byte line and of the 2^31 element line and spread over the rest of the pool,
so an offset formed in 32 bits anywhere (slot times head stride, ring or
conv-state row) would land on another slot. The pool's other slots hold a
sentinel and must keep it, bit for bit; the named slots are compared with the
oracle run on a compact pool that holds the same slots in order (compact slot
c is pool slot far[c]), to the fp32 bar."""
import numpy as np
import pytest
import torch

import oracle as O
import ssm_recurrent_decode_gated_amd as S
import workloads as W
from tests._helpers import FP32_TOL, assert_mixed, assert_out16, need_gpu, to_np64

pytestmark = pytest.mark.gpu
DEV = "cuda"
SENT = -7.25
E31 = 2 ** 31


def _pool_slots(per_slot):
    """Slot count of a pool holding just over 2^31 elements of per_slot each."""
    return E31 // per_slot + 64


def _far(n, n_big, per_slot, elem_bytes, seed, keep_zero=False):
    """n distinct pool slots: the slots on either side of the 4 GiB byte line
    and of the 2^31 element line, the last slot, then seeded picks over the
    whole pool. keep_zero pins compact slot 0 to pool slot 0 (a null slot)."""
    lines = [(4 << 30) // (per_slot * elem_bytes), E31 // per_slot]
    first = [0] if keep_zero else []
    for s in lines:
        first += [s - 1, s]
    first.append(n_big - 1)
    first = list(dict.fromkeys(t for t in first if 0 <= t < n_big))
    g = torch.Generator().manual_seed(seed)
    taken = set(first)
    rest = [s for s in torch.randperm(n_big, generator=g).tolist() if s not in taken and s != 0]
    far = (first + rest)[:n]
    if not keep_zero:  # the line slots land on seeded compact positions
        perm = torch.randperm(n, generator=g).tolist()
        far = [far[i] for i in perm]
    assert len(set(far)) == n
    return torch.tensor(far, dtype=torch.int64)


def _embed(compact, far, n_big):
    """The compact pool (CPU) placed at slots `far` of a sentinel-filled
    device pool of n_big slots."""
    big = torch.full((n_big,) + tuple(compact.shape[1:]), SENT, dtype=compact.dtype, device=DEV)
    big[far.to(DEV)] = compact.to(DEV)
    return big


def _map_idx(idx_c, far):
    """Row indices of the compact pool mapped to the big pool; padding stays."""
    out = idx_c.clone()
    m = idx_c >= 0
    out[m] = far[idx_c[m].long()].to(torch.int32)
    return out


def _check_rest(big, far, what):
    """Everything outside the named slots still holds the sentinel."""
    big[far.to(DEV)] = SENT
    n_bad = int(torch.count_nonzero(big != SENT))
    assert n_bad == 0, f"{what}: {n_bad} elements outside the named slots changed"


def _check_named(got, ref, initial, idx_c, tol, what):
    """Named compact slots against the oracle, unnamed ones unchanged."""
    named = sorted({int(i) for i in idx_c.tolist() if 0 <= i < got.shape[0]})
    others = sorted(set(range(got.shape[0])) - set(named))
    assert_mixed(got[named], ref[named], tol, what)
    if others:
        assert torch.equal(got[others], initial[others]), f"{what}: an unnamed slot changed"


def _gdn(name, B, act="bf16", out="bf16"):
    w = W.GDNWorkload(name, B=B, H=16, HV=32, K=128, V=128, num_slots=B + 4, act=act, out=out, idx="perm")
    idx = W.slot_indices(w).clone()
    idx[B // 2] = -1  # one padded row
    return w, W.gdn_params(w), idx, W.gdn_state(w)


def _dev(d):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


GDN_PER_SLOT = 32 * 128 * 128


@pytest.mark.parametrize("B,norm", [(8, False), (256, False), (40, True)])
def test_packed_step_pool_past_2g_elements(B, norm):
    need_gpu()
    w, P, idx_c, st = _gdn(f"big_pool_packed_b{B}", B)
    n_big = _pool_slots(GDN_PER_SLOT)
    far = _far(w.num_slots, n_big, GDN_PER_SLOT, 4, seed=B)
    x = W.gdn_step_inputs(w, norm=norm)
    big = _embed(st, far, n_big)
    idx = _map_idx(idx_c, far)
    out = torch.full((B, 1, w.HV, w.V), 7.0, dtype=torch.bfloat16, device=DEV)
    kw = dict(norm_gate=x["norm_gate"].to(DEV), norm_weight=x["norm_weight"].to(DEV)) if norm else {}
    xd, Pd = _dev(x), _dev(P)
    S.gdn_decode_step(xd["qkv"], xd["a"], xd["b"], Pd["A_log"], Pd["dt_bias"], big, idx.to(DEV), out, **kw)
    ref = st.double().numpy().copy()
    okw = dict(norm_gate=x["norm_gate"], norm_weight=x["norm_weight"]) if norm else {}
    ro = O.gdn_step(x["qkv"], x["a"], x["b"], P["A_log"], P["dt_bias"], ref, idx_c, H=w.H, HV=w.HV, K=w.K, V=w.V,
                    **okw)
    torch.cuda.synchronize()
    live = [r for r in range(B) if idx_c[r] >= 0]
    assert_out16(out[live].reshape(len(live), w.HV, w.V), ro[live], FP32_TOL, "output")
    assert (out[B // 2].float() == 7.0).all(), "padded row written"
    _check_named(big[far.to(DEV)].cpu(), ref, st, idx_c, FP32_TOL, "state")
    _check_rest(big, far, "state pool")
    del big
    torch.cuda.empty_cache()


def test_state16_step_pool_past_2g_elements():
    need_gpu()
    B = 64
    w, P, idx_c, st = _gdn("big_pool_s16", B)
    st16 = st.to(torch.bfloat16)
    n_big = _pool_slots(GDN_PER_SLOT)
    far = _far(w.num_slots, n_big, GDN_PER_SLOT, 2, seed=16)
    x = W.gdn_step_inputs(w)
    big = _embed(st16, far, n_big)
    idx = _map_idx(idx_c, far)
    out = torch.zeros(B, 1, w.HV, w.V, device=DEV)
    xd, Pd = _dev(x), _dev(P)
    S.gdn_decode_step_state16(xd["qkv"], xd["a"], xd["b"], Pd["A_log"], Pd["dt_bias"], big, idx.to(DEV), out)
    ref = st16.double().numpy().copy()
    ro = O.gdn_step(x["qkv"], x["a"], x["b"], P["A_log"], P["dt_bias"], ref, idx_c, H=w.H, HV=w.HV, K=w.K, V=w.V)
    torch.cuda.synchronize()
    live = [r for r in range(B) if idx_c[r] >= 0]
    assert_mixed(out.cpu()[live].reshape(len(live), w.HV, w.V), ro[live], FP32_TOL, "output")
    got = to_np64(big[far.to(DEV)])
    named = sorted({int(i) for i in idx_c.tolist() if i >= 0})
    # each stored row is the exact update rounded once to bf16
    err = np.abs(got[named] - ref[named])
    assert (err <= 2.0 ** -8 * np.abs(ref[named]) + 1e-6).all(), "16-bit state beyond one rounding"
    others = sorted(set(range(w.num_slots)) - set(named))
    assert torch.equal(big[far[others].to(DEV)].cpu(), st16[others]), "an unnamed slot changed"
    _check_rest(big, far, "16-bit state pool")
    del big
    torch.cuda.empty_cache()


def test_buffered_step_pool_past_2g_elements():
    """Every phase of a 4-record fp32 ring in one launch; the rings are slot
    pools too and are embedded the same way."""
    need_gpu()
    B, L = 64, 4
    w, P, idx_c, st = _gdn("big_pool_buffered", B, act="f32", out="f32")
    n_big = _pool_slots(GDN_PER_SLOT)
    far = _far(w.num_slots, n_big, GDN_PER_SLOT, 4, seed=64)
    x = W.gdn_step_inputs(w)
    ring = W.gdn_ring(w, L)
    wp = torch.tensor([r % L for r in range(B)], dtype=torch.int32)
    big = _embed(st, far, n_big)
    rings = {k: _embed(v, far, n_big) for k, v in ring.items()}
    idx = _map_idx(idx_c, far)
    out = torch.zeros(B, 1, w.HV, w.V, device=DEV)
    xd, Pd = _dev(x), _dev(P)
    S.gdn_decode_step_buffered(xd["qkv"], xd["a"], xd["b"], Pd["A_log"], Pd["dt_bias"], big, idx.to(DEV), out,
                               rings["d_cache"], rings["k_cache"], rings["g_cache"], wp.to(DEV))
    ref = st.double().numpy().copy()
    rr = {k: v.double().numpy().copy() for k, v in ring.items()}
    ro = O.gdn_step_buffered(x["qkv"], x["a"], x["b"], P["A_log"], P["dt_bias"], ref, idx_c, rr["d_cache"],
                             rr["k_cache"], rr["g_cache"], wp, L, H=w.H, HV=w.HV, K=w.K, V=w.V, ring_fmt=O.FMT_F32)
    torch.cuda.synchronize()
    live = [r for r in range(B) if idx_c[r] >= 0]
    assert_mixed(out.cpu()[live].reshape(len(live), w.HV, w.V), ro[live], FP32_TOL, "output")
    _check_named(big[far.to(DEV)].cpu(), ref, st, idx_c, FP32_TOL, "state")
    flushed = [int(idx_c[r]) for r in range(B) if idx_c[r] >= 0 and wp[r] == L - 1]
    for k in ("d_cache", "k_cache", "g_cache"):
        got = rings[k][far.to(DEV)].cpu()
        want = rr[k].copy()
        want[flushed] = ring[k][flushed].double().numpy()  # a flush appends no record
        _check_named(got, want, ring[k], idx_c, FP32_TOL, k)
        _check_rest(rings[k], far, k)
    _check_rest(big, far, "state pool")
    del big, rings
    torch.cuda.empty_cache()


def test_conv_step_pool_past_2g_elements():
    need_gpu()
    B = 64
    w, P, idx_c, st = _gdn("big_pool_conv", B)
    cv = W.gdn_conv(w, W=4, layout="DS")
    n_big = _pool_slots(GDN_PER_SLOT)
    far = _far(w.num_slots, n_big, GDN_PER_SLOT, 4, seed=65)
    x = W.gdn_step_inputs(w)
    big = _embed(st, far, n_big)
    cs = _embed(cv["conv_state"], far, n_big)
    idx = _map_idx(idx_c, far)
    out = torch.zeros(B, 1, w.HV, w.V, device=DEV)
    xd, Pd = _dev(x), _dev(P)
    S.gdn_decode_step_conv(xd["qkv"], cv["conv_weight"].to(DEV), cv["conv_bias"].to(DEV), cs, xd["a"], xd["b"],
                           Pd["A_log"], Pd["dt_bias"], big, idx.to(DEV), out)
    ref = st.double().numpy().copy()
    ref_cs = cv["conv_state"].double().numpy().copy()
    ro = O.gdn_step_conv(x["qkv"], cv["conv_weight"], cv["conv_bias"], ref_cs, x["a"], x["b"], P["A_log"],
                         P["dt_bias"], ref, idx_c, H=w.H, HV=w.HV, K=w.K, V=w.V)
    torch.cuda.synchronize()
    live = [r for r in range(B) if idx_c[r] >= 0]
    assert_mixed(out.cpu()[live].reshape(len(live), w.HV, w.V), ro[live], FP32_TOL, "output")
    _check_named(big[far.to(DEV)].cpu(), ref, st, idx_c, FP32_TOL, "state")
    # the conv state is a shift of stored bf16 inputs: bit-exact
    got_cs = to_np64(cs[far.to(DEV)])
    np.testing.assert_array_equal(got_cs, ref_cs, err_msg="conv state")
    _check_rest(cs, far, "conv-state pool")
    _check_rest(big, far, "state pool")
    del big, cs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("path", ["fused_recurrent", "chunk_prefill", "chunk_prefill_noalloc"])
def test_multi_token_pool_past_2g_elements(path):
    need_gpu()
    B, T = (64, 4) if path == "fused_recurrent" else (3, 100)  # 100 tokens: chunks and a ragged tail
    w, P, idx_c, st = _gdn(f"big_pool_{path}", B, out="f32")
    n_big = _pool_slots(GDN_PER_SLOT)
    far = _far(w.num_slots, n_big, GDN_PER_SLOT, 4, seed=T)
    xs = [W.gdn_step_inputs(w, step=t) for t in range(T)]
    d = {k: torch.stack([s[k] for s in xs], dim=1).contiguous() for k in ("qkv", "a", "b")}
    big = _embed(st, far, n_big)
    idx = _map_idx(idx_c, far)
    out = torch.zeros(B, T, w.HV, w.V, device=DEV)
    fn = getattr(S, "gdn_" + path)
    dd, Pd = _dev(d), _dev(P)
    fn(dd["qkv"], dd["a"], dd["b"], Pd["A_log"], Pd["dt_bias"], big, idx.to(DEV), out)
    ref = st.double().numpy().copy()
    ro = O.gdn_multi(d["qkv"], d["a"], d["b"], P["A_log"], P["dt_bias"], ref, idx_c, H=w.H, HV=w.HV, K=w.K,
                     V=w.V)
    torch.cuda.synchronize()
    live = [r for r in range(B) if idx_c[r] >= 0]
    assert_mixed(out.cpu()[live], ro[live], FP32_TOL, "outputs")
    _check_named(big[far.to(DEV)].cpu(), ref, st, idx_c, FP32_TOL, "state")
    _check_rest(big, far, "state pool")
    del big
    torch.cuda.empty_cache()


def test_kda_step_pool_past_2g_elements():
    """64 tokens x 96 heads of 128 channels; slot 0 is the null slot and stays
    slot 0 of the big pool."""
    need_gpu()
    w = W.KDAWorkload("big_pool_kda", T=64, H=96, num_slots=68)
    d = W.kda_inputs(w, layout="DS")
    per = w.H * w.D * w.D
    n_big = _pool_slots(per)
    far = _far(w.num_slots, n_big, per, 4, seed=96, keep_zero=True)
    idx_c = d["idx"]
    big = _embed(d["state"], far, n_big)
    cs = _embed(d["conv_state"], far, n_big)
    idx = _map_idx(idx_c, far)
    out = torch.zeros(w.T, w.H, w.D, device=DEV)
    dd = _dev(d)
    S.kda_decode_step(dd["x"], dd["conv_weight"], None, cs, dd["raw_g"], dd["raw_beta"], None, None, big,
                      idx.to(DEV), out, output_gate=dd["gate"], norm_weight=dd["norm_weight"])
    st_ref = d["state"].double().numpy().copy()
    cs_ref = d["conv_state"].double().numpy().copy()
    ro = O.kda_decode(d["x"], d["conv_weight"], None, cs_ref, d["raw_g"], d["raw_beta"], st_ref, idx_c, H=w.H,
                      D=w.D, lower_bound=w.lower_bound, gate=d["gate"], norm_weight=d["norm_weight"],
                      norm_eps=w.norm_eps)
    torch.cuda.synchronize()
    assert_mixed(out.cpu(), ro, FP32_TOL, "output")
    _check_named(big[far.to(DEV)].cpu(), st_ref, d["state"], idx_c, FP32_TOL, "state")
    np.testing.assert_array_equal(to_np64(cs[far.to(DEV)]), cs_ref, err_msg="conv state")
    _check_rest(cs, far, "conv-state pool")
    _check_rest(big, far, "state pool")
    del big, cs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("path", ["decode", "scan"])
def test_mamba_pool_past_2g_elements(path):
    need_gpu()
    Dm, N = 4096, 16
    if path == "decode":
        w = W.MambaWorkload("big_pool_mamba", B=64, Dm=Dm, N=N, num_slots=68)
        d = W.mamba_inputs(w)
    else:
        w = W.MambaScanWorkload("big_pool_mamba_scan", B=3, T=64, Dm=Dm, N=N, num_slots=5)
        d = W.mamba_scan_inputs(w, act="f32")
    per = Dm * N
    n_big = _pool_slots(per)
    far = _far(w.num_slots, n_big, per, 4, seed=Dm)
    idx_c = d["idx"].clone()
    idx_c[w.B // 2] = -1
    big = _embed(d["h"], far, n_big)
    idx = _map_idx(idx_c, far)
    dd = _dev(d)
    ref = d["h"].double().numpy().copy()
    if path == "decode":
        out = torch.zeros(w.B, Dm, device=DEV)
        S.mamba_decode_step(dd["x"], dd["dt"], dd["A"], dd["Bm"], dd["Cm"], dd["Dv"], dd["z"], big, idx.to(DEV),
                            out)
        ro = O.mamba_step(d["x"], d["dt"], d["A"], d["Bm"], d["Cm"], d["Dv"], d["z"], ref, idx_c)
    else:
        out = torch.zeros(w.B, w.T, Dm, device=DEV)
        ws = torch.empty(S.mamba_scan_workspace_bytes(w.B, w.T, Dm, N) // 4 + 1, device=DEV)  # the chunked path
        S.mamba_scan(dd["x"], dd["dt"], dd["A"], dd["Bm"], dd["Cm"], dd["Dv"], dd["z"], big, idx.to(DEV), out,
                     workspace=ws)
        ro = O.mamba_scan(d["x"], d["dt"], d["A"], d["Bm"], d["Cm"], d["Dv"], d["z"], ref, idx_c)
    torch.cuda.synchronize()
    live = [r for r in range(w.B) if idx_c[r] >= 0]
    assert_mixed(out.cpu()[live], ro[live], FP32_TOL, "output")
    _check_named(big[far.to(DEV)].cpu(), ref, d["h"], idx_c, FP32_TOL, "state")
    _check_rest(big, far, "state pool")
    del big
    torch.cuda.empty_cache()
