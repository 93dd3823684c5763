"""gdn_chunk_prefill_noalloc (the chunked GDN prefill on the library's static
workspace, for callers that cannot allocate) against gdn_chunk_prefill (the
same computation on a caller's workspace), through the C ABI: two calls in a
row, the second smaller (it reuses the array the first one filled), and a
call too large for the static workspace, which must be refused before
anything runs."""
import pytest
import torch

import ssm_recurrent_decode_gated_amd as S
import workloads as W
from tests._helpers import FP32_TOL, assert_mixed, need_gpu, to_np64
from tests.test_gdn_multi_gpu import _inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _both(w, T, lengths, norm):
    P, st, idx = W.gdn_params(w), W.gdn_state(w), W.slot_indices(w)
    d = _inputs(w, T, norm=norm is not None)
    args = [d[k].to(DEV) for k in ("qkv", "a", "b")] + [P["A_log"].to(DEV), P["dt_bias"].to(DEV)]
    kw = dict(lengths=None if lengths is None else lengths.to(DEV))
    if norm:
        kw.update(norm_gate=d["norm_gate"].to(DEV), norm_weight=d["norm_weight"].to(DEV), norm_act=norm)
    res = []
    for fn in (S.gdn_chunk_prefill, S.gdn_chunk_prefill_noalloc):
        st_d = st.to(DEV)
        out = torch.full((w.B, T, w.HV, w.V), 7.0, dtype=TD[w.out], device=DEV)
        fn(*args, st_d, idx.to(DEV), out, **kw)
        torch.cuda.synchronize()
        res.append((out.cpu(), st_d.cpu()))
    (o_ws, s_ws), (o_na, s_na) = res
    live = [b for b in range(w.B) if lengths is None or int(lengths[b]) > 0]
    for b in live:
        n = T if lengths is None else int(lengths[b])
        assert_mixed(to_np64(o_na[b, :n]), to_np64(o_ws[b, :n]), FP32_TOL, f"row {b} outputs")
        assert (o_na[b, n:].float() == 7.0).all(), f"row {b}: outputs past its length written"
    assert_mixed(to_np64(s_na), to_np64(s_ws), FP32_TOL, "state pool")
    return o_ws, o_na


def test_noalloc_matches_workspace_entry_point_twice():
    """First call: 2 rows of 300 tokens (5 chunks, the last partial) with a
    ragged second row, K = V = 128, bf16. Second, smaller call: one row of
    70 tokens at K = 64, V = 32, fp32 activations, with the gated norm
    (its fp32 outputs also live in the static array)."""
    need_gpu()
    w1 = W.GDNWorkload("noalloc_first", B=2, H=2, HV=4, K=128, V=128, num_slots=3, idx="perm", out="f32")
    _both(w1, 300, torch.tensor([300, 170], dtype=torch.int32), None)
    w2 = W.GDNWorkload("noalloc_second", B=1, H=1, HV=2, K=64, V=32, num_slots=2, idx="perm", act="f32",
                       out="bf16")
    _both(w2, 70, None, "silu")


def test_noalloc_refuses_more_than_its_static_workspace():
    """4096 (row, value head, chunk) records need 138 MB of workspace, more
    than the 128 MiB array: refused with SSMD_ERR_BAD_SHAPE, nothing written."""
    need_gpu()
    w = W.GDNWorkload("noalloc_too_big", B=1, H=1, HV=32, K=64, V=64, num_slots=1, out="f32")
    T = 8192
    assert S.gdn_chunk_workspace_bytes(w.B, T, w.HV, w.K, w.V) > S.SSMD_CHUNK_SCRATCH_BYTES
    C = 2 * w.H * w.K + w.HV * w.V
    qkv = torch.zeros(w.B, T, C, dtype=torch.bfloat16, device=DEV)
    a = torch.zeros(w.B, T, w.HV, dtype=torch.bfloat16, device=DEV)
    P = {k: v.to(DEV) for k, v in W.gdn_params(w).items()}
    st = torch.ones(w.num_slots, w.HV, w.V, w.K, device=DEV)
    out = torch.full((w.B, T, w.HV, w.V), 7.0, device=DEV)
    with pytest.raises(S.SsmdError, match="static") as e:
        S.gdn_chunk_prefill_noalloc(qkv, a, a, P["A_log"], P["dt_bias"], st, torch.zeros(1, dtype=torch.int32,
                                                                                         device=DEV), out)
    assert e.value.code == -2
    torch.cuda.synchronize()
    assert (out == 7.0).all() and (st == 1.0).all()
