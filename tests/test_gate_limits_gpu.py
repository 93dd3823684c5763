"""The gates at their limits, on the GPU against the fp64 oracle. Value heads
are split four ways: a decay that underflows to exactly 0 (A_log = 3,
a = 100: g = -e^3 softplus(100) ~ -2000, so the state is replaced by
delta k^T), beta = 0 (b = -200: the state only decays and the output is
e^g S q), a decay of exactly 1 with beta = 1 (A_log = -100, b = 200: the
delta rule overwrites S k with v), and ordinary gates. For KDA, whose decay
lies in [e^lb, 1], the per-channel gate is pushed to 1 (raw_g = -200) and to
e^lb (raw_g = 200), and beta to 0 and 1. Outputs and states to the fp32 bar,
for the packed step (both launch shapes), the buffered step (every phase),
the 16-bit-state step, the multi-token step and the fused KDA op."""
import pytest
import torch

import oracle as O
import ssm_recurrent_decode_gated_amd as S
import workloads as W
from tests._helpers import FP32_TOL, assert_mixed, need_gpu, to_np64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _limits(w, x, P):
    """Rewrite gates per value head hv % 4 (see the module docstring)."""
    a, b = x["a"].clone(), x["b"].clone()
    A_log, dt_bias = P["A_log"].clone(), P["dt_bias"].clone()
    for hv in range(w.HV):
        kind = hv % 4
        if kind == 0:
            A_log[hv], dt_bias[hv] = 3.0, 0.0
            a[:, hv] = 100.0
        elif kind == 1:
            b[:, hv] = -200.0
        elif kind == 2:
            A_log[hv] = -100.0
            b[:, hv] = 200.0
    return a, b, A_log, dt_bias


def _setup(B, act="bf16"):
    w = W.GDNWorkload(f"gate_limits_b{B}", B=B, H=16, HV=32, K=128, V=128, num_slots=B + 3, act=act, out="f32",
                      idx="perm")
    P, idx, x, st = W.gdn_params(w), W.slot_indices(w), W.gdn_step_inputs(w), W.gdn_state(w)
    a, b, A_log, dt_bias = _limits(w, x, P)
    return w, idx, x["qkv"], a, b, A_log, dt_bias, st


@pytest.mark.parametrize("B", [4, 40])
def test_packed_step_gate_limits(B):
    need_gpu()
    w, idx, qkv, a, b, A_log, dt_bias, st = _setup(B)
    sd = st.to(DEV)
    out = torch.zeros(B, 1, w.HV, w.V, device=DEV)
    S.gdn_decode_step(qkv.to(DEV), a.to(DEV), b.to(DEV), A_log.to(DEV), dt_bias.to(DEV), sd, idx.to(DEV), out)
    ref = st.double().numpy().copy()
    ro = O.gdn_step(qkv, a, b, A_log, dt_bias, ref, idx, H=w.H, HV=w.HV, K=w.K, V=w.V)
    torch.cuda.synchronize()
    assert_mixed(out.reshape(B, w.HV, w.V), ro, FP32_TOL, "output")
    assert_mixed(sd, ref, FP32_TOL, "state")
    # the limits themselves: decay 0 forgets the old state, beta 0 writes no delta
    s0 = int(idx[0])
    got = sd.cpu()
    kn = qkv[0, _k_slice(w, 0)].float()
    kn = kn / kn.norm()
    v0 = qkv[0, 2 * w.H * w.K: 2 * w.H * w.K + w.V].float()
    bet = torch.sigmoid(b[0, 0].float())
    assert torch.allclose(got[s0, 0], bet * torch.outer(v0, kn), rtol=1e-4, atol=1e-6), "decay 0 kept old state"
    assert torch.allclose(got[s0, 1], st[s0, 1] * torch.exp(_g(A_log[1], a[0, 1], dt_bias[1])), rtol=1e-5,
                          atol=1e-7), "beta 0 changed more than the decay"


def _k_slice(w, h):
    return slice((w.H + h) * w.K, (w.H + h + 1) * w.K)


def _g(A_log, a, dt_bias):
    return -torch.exp(A_log.float()) * torch.nn.functional.softplus(a.float() + dt_bias.float())


def test_buffered_step_gate_limits_every_phase():
    need_gpu()
    B, L = 40, 4
    w, idx, qkv, a, b, A_log, dt_bias, st = _setup(B)
    ring = W.gdn_ring(w, L)
    wp = torch.tensor([r % L for r in range(B)], dtype=torch.int32)
    sd = st.to(DEV)
    rd = {k: v.to(DEV) for k, v in ring.items()}
    out = torch.zeros(B, 1, w.HV, w.V, device=DEV)
    S.gdn_decode_step_buffered(qkv.to(DEV), a.to(DEV), b.to(DEV), A_log.to(DEV), dt_bias.to(DEV), sd, idx.to(DEV),
                               out, rd["d_cache"], rd["k_cache"], rd["g_cache"], wp.to(DEV))
    ref = st.double().numpy().copy()
    rr = {k: v.double().numpy().copy() for k, v in ring.items()}
    ro = O.gdn_step_buffered(qkv, a, b, A_log, dt_bias, ref, idx, rr["d_cache"], rr["k_cache"], rr["g_cache"], wp,
                             L, H=w.H, HV=w.HV, K=w.K, V=w.V, ring_fmt=O.FMT_BF16)
    torch.cuda.synchronize()
    assert_mixed(out.reshape(B, w.HV, w.V), ro, FP32_TOL, "output")
    flushed = sorted({int(idx[r]) for r in range(B) if wp[r] == L - 1})
    got = sd.cpu()
    for s in flushed:
        assert_mixed(got[s], ref[s], FP32_TOL, f"flushed slot {s}")
    gg = rd["g_cache"].cpu()
    for r in range(B):
        if wp[r] < L - 1:
            s, p = int(idx[r]), int(wp[r])
            # A_log = -100 makes g a subnormal fp32 value (or 0 where subnormals flush): atol covers it
            assert torch.allclose(gg[s, :, p].double(), torch.from_numpy(rr["g_cache"][s, :, p]), rtol=1e-5,
                                  atol=1e-30), f"g record row {r}"


def test_state16_step_gate_limits():
    need_gpu()
    B = 40
    w, idx, qkv, a, b, A_log, dt_bias, st = _setup(B)
    st16 = st.to(torch.bfloat16)
    sd = st16.to(DEV)
    out = torch.zeros(B, 1, w.HV, w.V, device=DEV)
    S.gdn_decode_step_state16(qkv.to(DEV), a.to(DEV), b.to(DEV), A_log.to(DEV), dt_bias.to(DEV), sd, idx.to(DEV),
                              out)
    ref = st16.double().numpy().copy()
    ro = O.gdn_step(qkv, a, b, A_log, dt_bias, ref, idx, H=w.H, HV=w.HV, K=w.K, V=w.V, state_fmt=O.FMT_NONE)
    torch.cuda.synchronize()
    assert_mixed(out.reshape(B, w.HV, w.V), ro, FP32_TOL, "output")
    # the stored rows are the exact state rounded once to bf16: within half a bf16 ulp, plus fp32 noise
    got = to_np64(sd)
    err = abs(got - ref)
    assert (err <= 2.0 ** -8 * abs(ref) + 1e-6).all(), "16-bit state beyond one rounding"


def test_multi_token_gate_limits():
    need_gpu()
    B, T = 8, 4
    w = W.GDNWorkload("gate_limits_multi", B=B, H=16, HV=32, K=128, V=128, num_slots=B + 2, out="f32", idx="perm")
    P, idx, st = W.gdn_params(w), W.slot_indices(w), W.gdn_state(w)
    xs = [W.gdn_step_inputs(w, step=t) for t in range(T)]
    lim = [_limits(w, x, P) for x in xs]
    qkv = torch.stack([x["qkv"] for x in xs], dim=1).contiguous()
    a = torch.stack([l[0] for l in lim], dim=1).contiguous()
    b = torch.stack([l[1] for l in lim], dim=1).contiguous()
    A_log, dt_bias = lim[0][2], lim[0][3]
    sd = st.to(DEV)
    out = torch.zeros(B, T, w.HV, w.V, device=DEV)
    S.gdn_fused_recurrent(qkv.to(DEV), a.to(DEV), b.to(DEV), A_log.to(DEV), dt_bias.to(DEV), sd, idx.to(DEV), out)
    ref = st.double().numpy().copy()
    ro = O.gdn_multi(qkv, a, b, A_log, dt_bias, ref, idx, H=w.H, HV=w.HV, K=w.K, V=w.V)
    torch.cuda.synchronize()
    assert_mixed(out.cpu(), ro, FP32_TOL, "outputs")
    assert_mixed(sd, ref, FP32_TOL, "state")


def test_kda_gate_limits():
    need_gpu()
    w = W.KDAWorkload("gate_limits_kda", T=8, H=4, num_slots=12)
    d = W.kda_inputs(w)
    raw_g, raw_beta = d["raw_g"].clone(), d["raw_beta"].clone()
    raw_g[:, 0, :] = -200.0          # decay 1 on every channel of head 0
    raw_g[:, 1, :64] = 200.0         # decay e^lb on half of head 1's channels
    raw_beta[:, 2] = -200.0          # beta 0 on head 2
    raw_beta[:, 3] = 200.0           # beta 1 on head 3
    cs = d["conv_state"].to(DEV)
    sd = d["state"].to(DEV)
    out = torch.zeros(w.T, w.H, w.D, device=DEV)
    S.kda_decode_step(d["x"].to(DEV), d["conv_weight"].to(DEV), None, cs, raw_g.to(DEV), raw_beta.to(DEV), None,
                      None, sd, d["idx"].to(DEV), out, output_gate=d["gate"].to(DEV),
                      norm_weight=d["norm_weight"].to(DEV))
    cs_ref = d["conv_state"].double().numpy().copy()
    st_ref = d["state"].double().numpy().copy()
    ro = O.kda_decode(d["x"], d["conv_weight"], None, cs_ref, raw_g, raw_beta, st_ref, d["idx"], H=w.H, D=w.D,
                      lower_bound=w.lower_bound, gate=d["gate"], norm_weight=d["norm_weight"], norm_eps=w.norm_eps)
    torch.cuda.synchronize()
    assert_mixed(out.cpu(), ro, FP32_TOL, "output")
    assert_mixed(sd, st_ref, FP32_TOL, "state")
