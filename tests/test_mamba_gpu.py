"""GPU parity of mamba_decode_step (Mamba-1 selective-scan decode) against the
fp64 oracle, over the shapes of the MBU write-up's decode table, its dtype
options, the optional D skip and z gate, ragged channel counts, padding and a
chained run."""
import numpy as np
import pytest
import torch

import oracle as O
import ssm_recurrent_decode_gated_amd as S
import workloads as W
from tests._helpers import CHAIN_TOL, FP32_TOL, assert_out16, assert_mixed, need_gpu, to_np64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(d, with_D, with_z, out_dtype, idx=None):
    idx = d["idx"] if idx is None else idx
    st = d["h"].to(DEV)
    B, Dm = d["x"].shape
    out = torch.full((B, Dm), 7.0, dtype=out_dtype, device=DEV)
    S.mamba_decode_step(d["x"].to(DEV), d["dt"].to(DEV), d["A"].to(DEV), d["Bm"].to(DEV), d["Cm"].to(DEV),
                        d["Dv"].to(DEV) if with_D else None, d["z"].to(DEV) if with_z else None, st,
                        idx.to(DEV), out)
    ref = d["h"].double().numpy().copy()
    ro = O.mamba_step(d["x"], d["dt"], d["A"], d["Bm"], d["Cm"], d["Dv"] if with_D else None,
                      d["z"] if with_z else None, ref, idx)
    torch.cuda.synchronize()
    return out, st.cpu(), ro, ref


CASES = [(B, Dm, N, act) for (B, Dm, N) in ((1, 1536, 16), (4, 1536, 16), (8, 1536, 16), (1, 3072, 16), (1, 1536, 64))
         for act in ("f32",)] + [(1, 1536, 16, "f16"), (1, 1536, 16, "bf16"), (3, 1000, 32, "bf16"),
                                 (2, 200, 128, "f32"), (2, 64, 256, "f16")]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}_D{c[1]}_N{c[2]}_{c[3]}" for c in CASES])
@pytest.mark.parametrize("with_D,with_z", [(True, True), (False, False), (True, False)])
def test_mamba_decode_step(case, with_D, with_z):
    need_gpu()
    B, Dm, N, act = case
    w = W.MambaWorkload(f"mamba_b{B}_d{Dm}_n{N}", B=B, Dm=Dm, N=N, num_slots=B + 2)
    d = W.mamba_inputs(w, act=act)
    d["idx"] = torch.randperm(w.num_slots, generator=W.generator(0, w.name, "idx"))[:B].to(torch.int32)
    outd = torch.float32 if act == "f32" else W.DTYPES[act]
    out, st, ro, ref = _run(d, with_D, with_z, outd)
    if outd == torch.float32:
        assert_mixed(out.cpu(), ro, FP32_TOL, "y")
    else:
        assert_out16(out, ro, FP32_TOL, "y")
    slots = d["idx"].tolist()
    assert_mixed(st[slots], ref[slots], FP32_TOL, "state")
    for s in set(range(w.num_slots)) - set(slots):
        assert torch.equal(st[s], d["h"][s])


def test_mamba_padded_rows():
    need_gpu()
    w = W.MambaWorkload("mamba_pad", B=4, Dm=512, N=16, num_slots=3)
    d = W.mamba_inputs(w)
    idx = torch.tensor([2, -1, 3, 0], dtype=torch.int32)
    out, st, ro, ref = _run(d, True, True, torch.float32, idx=idx)
    for b in (1, 2):
        assert (out[b].cpu() == 7.0).all()
    assert_mixed(out[[0, 3]].cpu(), ro[[0, 3]], FP32_TOL, "active rows")
    assert torch.equal(st[1], d["h"][1])
    assert_mixed(st[[0, 2]], ref[[0, 2]], FP32_TOL, "state")


def test_mamba_chain_100_steps():
    """100 chained steps, fresh inputs each step; the oracle keeps its fp64 state."""
    need_gpu()
    w = W.MambaWorkload("mamba_chain", B=4, Dm=1536, N=16, num_slots=4)
    d0 = W.mamba_inputs(w)
    st = d0["h"].to(DEV)
    ref = d0["h"].double().numpy().copy()
    A, Dv = d0["A"], d0["Dv"]
    out = torch.empty(w.B, w.Dm, device=DEV)
    for t in range(100):
        d = W.mamba_inputs(W.MambaWorkload(f"mamba_chain_{t}", B=4, Dm=1536, N=16, num_slots=4))
        S.mamba_decode_step(d["x"].to(DEV), d["dt"].to(DEV), A.to(DEV), d["Bm"].to(DEV), d["Cm"].to(DEV),
                            Dv.to(DEV), d["z"].to(DEV), st, d0["idx"].to(DEV), out)
        ro = O.mamba_step(d["x"], d["dt"], A, d["Bm"], d["Cm"], Dv, d["z"], ref, d0["idx"])
        if t in (0, 9, 99):
            assert_mixed(out.cpu(), ro, CHAIN_TOL, f"y at step {t + 1}")
    assert_mixed(st.cpu(), ref, CHAIN_TOL, "state after 100 steps")
