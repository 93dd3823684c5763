"""Non-finite inputs stay in their own row. NaN and Inf are not guarded
(they propagate, as any fp32 arithmetic propagates them), and every kernel
works on independent (row, head) units, so one row's NaN key or Inf state
must leave every other row's outputs and every other slot bit-for-bit as a
clean run of the same call leaves them. The poisoned row itself must come out
non-finite (the value is not masked). The sequential multi-token kernel is
also causal under poison: a row's tokens before the poisoned one are
unchanged. Each entry point runs twice on copies of the same inputs, clean
and poisoned; nothing here needs the oracle."""
import pytest
import torch

import ssm_recurrent_decode_gated_amd as S
import workloads as W
from tests._helpers import need_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"
NAN = float("nan")


def _gdn(B, HV=32, H=16, K=128, V=128, act="bf16", slots_extra=4):
    w = W.GDNWorkload(f"nonfinite_b{B}_hv{HV}", B=B, H=H, HV=HV, K=K, V=V, num_slots=B + slots_extra, act=act,
                      out="f32", idx="perm")
    return w, W.gdn_params(w), W.slot_indices(w), W.gdn_step_inputs(w), W.gdn_state(w)


def _k_col(w, h):
    """First column of q/k head h's key inside a mixed_qkv row."""
    return (w.H + h) * w.K


def _assert_isolated(clean, dirty, bad_rows, what):
    """Rows (dim 0) not in bad_rows are bit-identical; each bad row holds a
    non-finite value."""
    for b in range(clean.shape[0]):
        if b in bad_rows:
            assert not torch.isfinite(dirty[b]).all(), f"{what}: poisoned row {b} came out finite"
        else:
            assert torch.equal(clean[b], dirty[b]), f"{what}: row {b} changed by another row's poison"


def _slots_isolated(st_clean, st_dirty, bad_slots, what):
    for s in range(st_clean.shape[0]):
        if s in bad_slots:
            assert not torch.isfinite(st_dirty[s]).all(), f"{what}: poisoned slot {s} came out finite"
        else:
            assert torch.equal(st_clean[s], st_dirty[s]), f"{what}: slot {s} changed by another row's poison"


@pytest.mark.parametrize("B", [4, 40])
def test_packed_step_nan_key_and_inf_state(B):
    """B = 4 (one block per head) and B = 40 (1-wave 8-row tiles): a NaN in
    one row's key and an Inf in another row's state."""
    need_gpu()
    w, P, idx, x, st = _gdn(B)
    r_key, r_state = 1, B - 2
    qkv_bad = x["qkv"].clone()
    qkv_bad[r_key, _k_col(w, 3) + 5] = NAN
    st_bad = st.clone()
    st_bad[int(idx[r_state]), 7, 11, 13] = float("inf")
    outs, states = [], []
    for qkv, s0 in ((x["qkv"], st), (qkv_bad, st_bad)):
        sd = s0.to(DEV)
        out = torch.zeros(B, 1, w.HV, w.V, device=DEV)
        S.gdn_decode_step(qkv.to(DEV), x["a"].to(DEV), x["b"].to(DEV), P["A_log"].to(DEV), P["dt_bias"].to(DEV),
                          sd, idx.to(DEV), out)
        torch.cuda.synchronize()
        outs.append(out.cpu())
        states.append(sd.cpu())
    _assert_isolated(outs[0], outs[1], {r_key, r_state}, "output")
    _slots_isolated(states[0], states[1], {int(idx[r_key]), int(idx[r_state])}, "state")


def test_buffered_step_nan_key_every_phase():
    """L = 4, rows at every phase (flushes included): a NaN key in a flush row
    and in a non-flush row; the rings of other slots and other rows' outputs
    are unchanged."""
    need_gpu()
    B, L = 40, 4
    w, P, idx, x, st = _gdn(B)
    ring = W.gdn_ring(w, L)
    wp = torch.tensor([b % L for b in range(B)], dtype=torch.int32)
    bad = {3, 6}  # phase 3 (flush) and phase 2
    qkv_bad = x["qkv"].clone()
    for r in bad:
        qkv_bad[r, _k_col(w, 5) + 17] = NAN
    res = []
    for qkv in (x["qkv"], qkv_bad):
        sd = st.to(DEV)
        rd = {k: v.to(DEV) for k, v in ring.items()}
        out = torch.zeros(B, 1, w.HV, w.V, device=DEV)
        S.gdn_decode_step_buffered(qkv.to(DEV), x["a"].to(DEV), x["b"].to(DEV), P["A_log"].to(DEV),
                                   P["dt_bias"].to(DEV), sd, idx.to(DEV), out, rd["d_cache"], rd["k_cache"],
                                   rd["g_cache"], wp.to(DEV))
        torch.cuda.synchronize()
        res.append((out.cpu(), sd.cpu(), {k: v.cpu() for k, v in rd.items()}))
    _assert_isolated(res[0][0], res[1][0], bad, "output")
    # only the flush row writes its state; the non-flush row writes its record
    _slots_isolated(res[0][1], res[1][1], {int(idx[3])}, "state")
    bad_slots = {int(idx[r]) for r in bad}
    for k in ("d_cache", "k_cache"):
        for s in range(w.num_slots):
            if s not in bad_slots:
                assert torch.equal(res[0][2][k][s], res[1][2][k][s]), f"{k} of slot {s} changed"
    assert not torch.isfinite(res[1][2]["d_cache"][int(idx[6])]).all(), "the poisoned record came out finite"


def test_state16_step_nan_key():
    need_gpu()
    B = 40
    w, P, idx, x, st = _gdn(B)
    st16 = st.to(torch.bfloat16)
    qkv_bad = x["qkv"].clone()
    qkv_bad[9, _k_col(w, 0)] = NAN
    res = []
    for qkv in (x["qkv"], qkv_bad):
        sd = st16.to(DEV)
        out = torch.zeros(B, 1, w.HV, w.V, device=DEV)
        S.gdn_decode_step_state16(qkv.to(DEV), x["a"].to(DEV), x["b"].to(DEV), P["A_log"].to(DEV),
                                  P["dt_bias"].to(DEV), sd, idx.to(DEV), out)
        torch.cuda.synchronize()
        res.append((out.cpu(), sd.cpu()))
    _assert_isolated(res[0][0], res[1][0], {9}, "output")
    _slots_isolated(res[0][1], res[1][1], {int(idx[9])}, "state")


def test_conv_fused_step_nan_input():
    """B = 40 groups per q/k head run the persistent conv-fused kernel: a NaN
    in one row's raw key channel poisons that row's conv output, state and
    conv state only."""
    need_gpu()
    B = 40
    w, P, idx, x, st = _gdn(B)
    cv = W.gdn_conv(w, 4)
    qkv_bad = x["qkv"].clone()
    qkv_bad[12, _k_col(w, 2) + 40] = NAN
    res = []
    for qkv in (x["qkv"], qkv_bad):
        sd = st.to(DEV)
        cs = cv["conv_state"].to(DEV)
        out = torch.zeros(B, 1, w.HV, w.V, device=DEV)
        S.gdn_decode_step_conv(qkv.to(DEV), cv["conv_weight"].to(DEV),
                               None if cv["conv_bias"] is None else cv["conv_bias"].to(DEV), cs, x["a"].to(DEV),
                               x["b"].to(DEV), P["A_log"].to(DEV), P["dt_bias"].to(DEV), sd, idx.to(DEV), out)
        torch.cuda.synchronize()
        res.append((out.cpu(), sd.cpu(), cs.cpu()))
    _assert_isolated(res[0][0], res[1][0], {12}, "output")
    _slots_isolated(res[0][1], res[1][1], {int(idx[12])}, "state")
    _slots_isolated(res[0][2], res[1][2], {int(idx[12])}, "conv state")


def _tokens(w, T):
    xs = [W.gdn_step_inputs(w, step=t) for t in range(T)]
    return {k: torch.stack([x[k] for x in xs], dim=1).contiguous() for k in ("qkv", "a", "b")}


def test_multi_token_nan_is_causal_and_isolated():
    """Sequential kernel, 6 tokens: a NaN key at token 3 of one row leaves
    that row's tokens 0-2 unchanged and poisons its tokens 3-5."""
    need_gpu()
    B, T, t_bad, r = 16, 6, 3, 5
    w, P, idx, _, st = _gdn(B)
    d = _tokens(w, T)
    qkv_bad = d["qkv"].clone()
    qkv_bad[r, t_bad, _k_col(w, 1) + 2] = NAN
    res = []
    for qkv in (d["qkv"], qkv_bad):
        sd = st.to(DEV)
        out = torch.zeros(B, T, w.HV, w.V, device=DEV)
        S.gdn_fused_recurrent(qkv.to(DEV), d["a"].to(DEV), d["b"].to(DEV), P["A_log"].to(DEV),
                              P["dt_bias"].to(DEV), sd, idx.to(DEV), out)
        torch.cuda.synchronize()
        res.append((out.cpu(), sd.cpu()))
    _assert_isolated(res[0][0], res[1][0], {r}, "output")
    assert torch.equal(res[0][0][r, :t_bad], res[1][0][r, :t_bad]), "tokens before the poisoned one changed"
    for t in range(t_bad, T):
        assert not torch.isfinite(res[1][0][r, t]).all(), f"token {t} after the poison came out finite"
    _slots_isolated(res[0][1], res[1][1], {int(idx[r])}, "state")


def test_chunk_prefill_nan_stays_in_its_row():
    """Chunked form, 2 rows x 128 tokens: a NaN key in row 1's second chunk
    leaves row 0 unchanged. (Inside the poisoned row the chunk's matrix
    products may spread it to earlier tokens of that chunk: 0 x NaN is NaN.)"""
    need_gpu()
    B, T = 2, 128
    w, P, idx, _, st = _gdn(B, act="bf16")
    d = _tokens(w, T)
    qkv_bad = d["qkv"].clone()
    qkv_bad[1, 70, _k_col(w, 4) + 9] = NAN
    res = []
    for qkv in (d["qkv"], qkv_bad):
        sd = st.to(DEV)
        out = torch.zeros(B, T, w.HV, w.V, device=DEV)
        S.gdn_chunk_prefill(qkv.to(DEV), d["a"].to(DEV), d["b"].to(DEV), P["A_log"].to(DEV),
                            P["dt_bias"].to(DEV), sd, idx.to(DEV), out)
        torch.cuda.synchronize()
        res.append((out.cpu(), sd.cpu()))
    _assert_isolated(res[0][0], res[1][0], {1}, "output")
    assert torch.equal(res[0][0][1, :64], res[1][0][1, :64]), "an earlier chunk of the poisoned row changed"
    _slots_isolated(res[0][1], res[1][1], {int(idx[1])}, "state")


def test_kda_nan_input_token():
    """The fused KDA op over 8 tokens x 4 heads: a NaN raw key channel of
    token 2 poisons that token's output, state and conv state only."""
    need_gpu()
    w = W.KDAWorkload("nonfinite_kda_t8_h4", T=8, H=4, num_slots=12)
    d = W.kda_inputs(w)
    x_bad = d["x"].clone()
    x_bad[2, w.H * w.D + 1 * w.D + 3] = NAN  # k channel 3 of head 1
    res = []
    for x in (d["x"], x_bad):
        cs = d["conv_state"].to(DEV)
        sd = d["state"].to(DEV)
        out = torch.zeros(w.T, w.H, w.D, dtype=torch.bfloat16, device=DEV)
        S.kda_decode_step(x.to(DEV), d["conv_weight"].to(DEV), None, cs, d["raw_g"].to(DEV),
                          d["raw_beta"].to(DEV), None, None, sd, d["idx"].to(DEV), out,
                          output_gate=d["gate"].to(DEV), norm_weight=d["norm_weight"].to(DEV))
        torch.cuda.synchronize()
        res.append((out.cpu(), sd.cpu(), cs.cpu()))
    _assert_isolated(res[0][0], res[1][0], {2}, "output")
    _slots_isolated(res[0][1], res[1][1], {int(d["idx"][2])}, "state")
    _slots_isolated(res[0][2], res[1][2], {int(d["idx"][2])}, "conv state")


def test_mamba_nan_input_row():
    need_gpu()
    w = W.MambaWorkload("nonfinite_mamba", B=8, Dm=1536, N=16, num_slots=8)
    d = W.mamba_inputs(w)
    x_bad = d["x"].clone()
    x_bad[4, 100] = NAN
    res = []
    for x in (d["x"], x_bad):
        sd = d["h"].to(DEV)
        out = torch.zeros(w.B, w.Dm, device=DEV)
        S.mamba_decode_step(x.to(DEV), d["dt"].to(DEV), d["A"].to(DEV), d["Bm"].to(DEV), d["Cm"].to(DEV),
                            d["Dv"].to(DEV), d["z"].to(DEV), sd, d["idx"].to(DEV), out)
        torch.cuda.synchronize()
        res.append((out.cpu(), sd.cpu()))
    _assert_isolated(res[0][0], res[1][0], {4}, "output")
    _slots_isolated(res[0][1], res[1][1], {int(d["idx"][4])}, "state")
