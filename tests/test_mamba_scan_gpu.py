"""GPU parity of mamba_scan (Mamba-1 over T tokens, prefill) against the fp64
oracle: every output and final state, for the chunk-parallel path (with a
workspace), the single-pass path (without), workspaces that fit only a few
chunks, ragged row lengths, zero starts, padding, every state width and
dtype, and a scan followed by decode steps."""
import numpy as np
import pytest
import torch

import oracle as O
import ssm_recurrent_decode_gated_amd as S
import workloads as W
from tests._helpers import FP32_TOL, assert_out16, assert_mixed, need_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _ws(w, frac=1.0):
    n = S.mamba_scan_workspace_bytes(w.B, w.T, w.Dm, w.N)
    n = int(n * frac) // 16 * 16
    return torch.empty(max(n // 4, 1), dtype=torch.float32, device=DEV) if n > 0 else None


def _run(w, d, *, ws=None, with_D=True, with_z=True, out_dtype=torch.bfloat16, lengths=None, zero_init=False,
         idx=None):
    idx = d["idx"] if idx is None else idx
    st = d["h"].to(DEV)
    out = torch.full((w.B, w.T, w.Dm), 7.0, dtype=out_dtype, device=DEV)
    S.mamba_scan(d["x"].to(DEV), d["dt"].to(DEV), d["A"].to(DEV), d["Bm"].to(DEV), d["Cm"].to(DEV),
                 d["Dv"].to(DEV) if with_D else None, d["z"].to(DEV) if with_z else None, st, idx.to(DEV), out,
                 lengths=None if lengths is None else lengths.to(DEV), zero_init=zero_init, workspace=ws)
    ref = d["h"].double().numpy().copy()
    ro = O.mamba_scan(d["x"], d["dt"], d["A"], d["Bm"], d["Cm"], d["Dv"] if with_D else None,
                      d["z"] if with_z else None, ref, idx, lengths=lengths, zero_init=zero_init)
    torch.cuda.synchronize()
    return out, st.cpu(), ro, ref


def _check_out(out, ro, what="y"):
    if out.dtype == torch.float32:
        assert_mixed(out.cpu(), ro, FP32_TOL, what)
    else:
        assert_out16(out, ro, FP32_TOL, what)


@pytest.mark.parametrize("path", ["chunked", "single_pass", "three_chunks"])
def test_mamba_scan_prefill_2048(path):
    """One 2048-token prompt at the page's model width (D = 1536, N = 16),
    bf16 activations: with the full workspace (chunk-parallel), none
    (one sequential pass), and a workspace for only three chunks."""
    need_gpu()
    w = W.MAMBA_PREFILL
    d = W.mamba_scan_inputs(w)
    ws = {"chunked": lambda: _ws(w), "single_pass": lambda: None,
          "three_chunks": lambda: torch.empty(3 * 2 * w.B * w.Dm * w.N, device=DEV)}[path]()
    if path == "chunked":
        assert ws is not None, "a single 2048-token row should want chunking"
    out, st, ro, ref = _run(w, d, ws=ws)
    _check_out(out, ro)
    assert_mixed(st, ref, FP32_TOL, "final state")


def test_mamba_scan_ragged_lengths_zero_start_and_padding():
    """Rows of lengths T, 37, 0, 100 and 1 (T = 130, not a multiple of the
    8-token groups), one padded row, from zero and from the stored state:
    outputs past a row's length and unnamed slots stay untouched."""
    need_gpu()
    w = W.MambaScanWorkload("mamba_scan_ragged", B=6, T=130, Dm=700, N=16, num_slots=8)
    d = W.mamba_scan_inputs(w, act="f32")
    idx = torch.tensor([5, 0, 7, 2, -1, 3], dtype=torch.int32)
    lengths = torch.tensor([130, 37, 0, 100, 50, 1], dtype=torch.int32)
    for zero_init in (False, True):
        for ws in (_ws(w), None):
            out, st, ro, ref = _run(w, d, ws=ws, out_dtype=torch.float32, lengths=lengths, zero_init=zero_init,
                                    idx=idx)
            live = [0, 1, 2, 3, 5]
            o = out.cpu()
            for b in live:
                L = int(lengths[b])
                if L:
                    assert_mixed(o[b, :L], ro[b, :L], FP32_TOL, f"row {b}")
                assert (o[b, L:] == 7.0).all(), f"row {b} wrote past its length"
            assert (o[4] == 7.0).all(), "padded row wrote output"
            slots = [5, 0, 7, 2, 3]
            assert_mixed(st[slots], ref[slots], FP32_TOL, "states")
            for s in (1, 4, 6):
                assert torch.equal(st[s], d["h"][s]), f"unnamed slot {s} changed"


CASES = [
    # B, T, D, N, act, out, D skip, z gate
    (2, 96, 512, 32, "bf16", "bf16", True, True),
    (1, 300, 256, 64, "f16", "f32", False, True),
    (3, 64, 200, 128, "f32", "f32", True, False),
    (1, 40, 96, 256, "bf16", "bf16", False, False),
    (4, 17, 1536, 16, "f16", "f16", True, True),
    (64, 33, 256, 16, "bf16", "bf16", True, True),
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}_T{c[1]}_D{c[2]}_N{c[3]}_{c[4]}" for c in CASES])
def test_mamba_scan_shapes(case):
    """Every state width (N = 16 ... 256, one to sixteen lanes per channel),
    ragged channel counts, every dtype, with and without the D skip and the z
    gate, chunked and single-pass."""
    need_gpu()
    B, T, Dm, N, act, outd, with_D, with_z = case
    w = W.MambaScanWorkload(f"mamba_scan_b{B}_t{T}_d{Dm}_n{N}", B=B, T=T, Dm=Dm, N=N, num_slots=B + 1)
    d = W.mamba_scan_inputs(w, act=act)
    for ws in (_ws(w), None):
        out, st, ro, ref = _run(w, d, ws=ws, with_D=with_D, with_z=with_z, out_dtype=W.DTYPES[outd])
        _check_out(out, ro)
        slots = d["idx"].tolist()
        assert_mixed(st[slots], ref[slots], FP32_TOL, "final state")


def test_mamba_scan_then_decode_steps():
    """A 256-token prefill then 16 decode steps on the same pool: the state
    the scan leaves is the one the decode step continues from."""
    need_gpu()
    w = W.MambaScanWorkload("mamba_scan_then_decode", B=2, T=256, Dm=1536, N=16, num_slots=3)
    d = W.mamba_scan_inputs(w, act="f32")
    st = d["h"].to(DEV)
    ref = d["h"].double().numpy().copy()
    out = torch.empty(w.B, w.T, w.Dm, device=DEV)
    S.mamba_scan(d["x"].to(DEV), d["dt"].to(DEV), d["A"].to(DEV), d["Bm"].to(DEV), d["Cm"].to(DEV),
                 d["Dv"].to(DEV), d["z"].to(DEV), st, d["idx"].to(DEV), out, workspace=_ws(w))
    ro = O.mamba_scan(d["x"], d["dt"], d["A"], d["Bm"], d["Cm"], d["Dv"], d["z"], ref, d["idx"])
    torch.cuda.synchronize()
    assert_mixed(out.cpu(), ro, FP32_TOL, "prefill y")
    dw = W.MambaWorkload("mamba_scan_then_decode_steps", B=2, Dm=1536, N=16, num_slots=3)
    y = torch.empty(w.B, w.Dm, device=DEV)
    for t in range(16):
        s = W.mamba_inputs(dw, seed=t, act="f32")
        S.mamba_decode_step(s["x"].to(DEV), s["dt"].to(DEV), d["A"].to(DEV), s["Bm"].to(DEV), s["Cm"].to(DEV),
                            d["Dv"].to(DEV), s["z"].to(DEV), st, d["idx"].to(DEV), y)
        ry = O.mamba_step(s["x"], s["dt"], d["A"], s["Bm"], s["Cm"], d["Dv"], s["z"], ref, d["idx"])
        torch.cuda.synchronize()
        assert_mixed(y.cpu(), ry, FP32_TOL, f"decode step {t}")
    slots = d["idx"].tolist()
    assert_mixed(st.cpu()[slots], ref[slots], FP32_TOL, "state")
