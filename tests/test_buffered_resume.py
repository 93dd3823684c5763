"""Resume of the buffered (L-step write-back) decode from persisted state.

The ReplaySSM page's buffered step keeps a checkpoint that is written only
once every L steps plus a ring of per-step records, with the caller's
write_pos saying where the cycle stands ("Microbenchmark: buffered
output-only GDN decode (ReplaySSM Part A) ...", module docstring and
`_bench_cfg`). Those three things are the whole state of a sequence: a run
persisted at any phase (checkpoint, ring, write_pos), restored into fresh
buffers and continued must follow the uninterrupted run exactly. The oracle
is checked on the CPU; the kernel on the GPU, against itself uninterrupted
(bit for bit: same kernel, same inputs) and against the oracle's
uninterrupted run (the parity bar).
"""
import io

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

L = 4
STEPS = 2 * L + 1  # two full cycles and one step into the third


def _persist(arrays):
    """Round trip through a byte stream, as a checkpoint file would."""
    buf = io.BytesIO()
    np.savez(buf, **arrays)
    buf.seek(0)
    with np.load(buf, allow_pickle=False) as z:
        return {k: z[k].copy() for k in z.files}


def _oracle_run(w, P, idx, steps_inputs, state, ring, wp0, stop=None, ring_fmt=O.FMT_BF16):
    """Runs the oracle's buffered steps; with `stop`, persists everything after
    `stop` steps and continues from the restored copies. Returns outputs."""
    st = state.copy()
    rr = {k: v.copy() for k, v in ring.items()}
    wp = wp0
    outs = []
    for t, x in enumerate(steps_inputs):
        if stop is not None and t == stop:
            saved = _persist({"state": st, "d": rr["d"], "k": rr["k"], "g": rr["g"], "wp": np.int32(wp)})
            del st, rr
            st = saved["state"]
            rr = {k: saved[k] for k in ("d", "k", "g")}
            wp = int(saved["wp"])
        o = O.gdn_step_buffered(x["qkv"], x["a"], x["b"], P["A_log"], P["dt_bias"], st, idx, rr["d"], rr["k"],
                                rr["g"], np.full(w.B, wp, np.int32), L, H=w.H, HV=w.HV, K=w.K, V=w.V,
                                ring_fmt=ring_fmt)
        outs.append(o)
        wp = (wp + 1) % L
    return outs, st


def _setup(act="bf16"):
    w = W.GDNWorkload("buffered_resume", B=3, H=2, HV=4, K=32, V=24, num_slots=5, idx="perm", act=act)
    P, idx = W.gdn_params(w), W.slot_indices(w)
    state = W.gdn_state(w).double().numpy()
    ring = {"d": np.zeros((w.num_slots, w.HV, L, w.V)), "k": np.zeros((w.num_slots, w.H, L, w.K)),
            "g": np.zeros((w.num_slots, w.HV, L))}
    xs = [W.gdn_step_inputs(w, 900 + t) for t in range(STEPS)]
    return w, P, idx, state, ring, xs


@pytest.mark.parametrize("stop", range(1, STEPS))
def test_oracle_resume_at_every_phase(stop):
    """Persisted after `stop` steps (every phase of the cycle, the flush
    included) and resumed: every later output and the final checkpoint are
    bit-identical to the uninterrupted run."""
    w, P, idx, state, ring, xs = _setup()
    ref_outs, ref_st = _oracle_run(w, P, idx, xs, state, ring, 0)
    outs, st = _oracle_run(w, P, idx, xs, state, ring, 0, stop=stop)
    for t in range(STEPS):
        np.testing.assert_array_equal(outs[t], ref_outs[t], err_msg=f"output at step {t}")
    np.testing.assert_array_equal(st, ref_st)


def test_oracle_resume_needs_the_ring():
    """The ring is part of the state: resuming mid-cycle with the ring
    cleared (checkpoint and write_pos alone) changes the outputs, so the
    resume test above does exercise the ring."""
    w, P, idx, state, ring, xs = _setup()
    ref_outs, _ = _oracle_run(w, P, idx, xs, state, ring, 0)
    st = state.copy()
    rr = {k: v.copy() for k, v in ring.items()}
    for t in range(2):
        O.gdn_step_buffered(xs[t]["qkv"], xs[t]["a"], xs[t]["b"], P["A_log"], P["dt_bias"], st, idx, rr["d"],
                            rr["k"], rr["g"], np.full(w.B, t, np.int32), L, H=w.H, HV=w.HV, K=w.K, V=w.V)
    rr = {k: np.zeros_like(v) for k, v in rr.items()}
    o = O.gdn_step_buffered(xs[2]["qkv"], xs[2]["a"], xs[2]["b"], P["A_log"], P["dt_bias"], st, idx, rr["d"],
                            rr["k"], rr["g"], np.full(w.B, 2, np.int32), L, H=w.H, HV=w.HV, K=w.K, V=w.V)
    assert np.abs(o - ref_outs[2]).max() > 1e-3


@pytest.mark.gpu
@pytest.mark.parametrize("act", ["bf16", "f32"])
@pytest.mark.parametrize("stop", range(1, STEPS))
def test_gpu_resume_at_every_phase(stop, act):
    """The kernel persisted at every phase (state, ring and write_pos copied
    to the host, through a byte stream, into freshly allocated device
    buffers) continues bit for bit as the uninterrupted kernel run. With an
    fp32 ring (fp32 activations) both also meet the oracle's uninterrupted
    run at the chained bar; a bf16 ring's records may round differently from
    the oracle's at midpoints, which the chained buffered tests handle."""
    from tests._helpers import CHAIN_TOL, assert_mixed, need_gpu
    need_gpu()
    import ssm_recurrent_decode_gated_amd as S
    w, P, idx, state, ring, xs = _setup(act)
    dev = "cuda"
    tdt = W.DTYPES[act]
    Pd = {k: v.to(dev) for k, v in P.items()}

    def to_host(t):
        return t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()

    def to_dev(a):
        t = torch.from_numpy(a).to(dev)
        return t.view(torch.bfloat16) if a.dtype == np.int16 else t

    def run(stop_at):
        st = torch.from_numpy(state.astype(np.float32)).to(dev)
        rg = {"d": torch.zeros(w.num_slots, w.HV, L, w.V, dtype=tdt, device=dev),
              "k": torch.zeros(w.num_slots, w.H, L, w.K, dtype=tdt, device=dev),
              "g": torch.zeros(w.num_slots, w.HV, L, device=dev)}
        wp = 0
        outs = []
        for t, x in enumerate(xs):
            if stop_at is not None and t == stop_at:
                torch.cuda.synchronize()
                saved = _persist({"state": st.cpu().numpy(), "d": to_host(rg["d"]), "k": to_host(rg["k"]),
                                  "g": rg["g"].cpu().numpy(), "wp": np.int32(wp)})
                del st, rg
                torch.cuda.empty_cache()
                st = to_dev(saved["state"])
                rg = {k: to_dev(saved[k]) for k in ("d", "k", "g")}
                wp = int(saved["wp"])
            out = torch.empty(w.B, 1, w.HV, w.V, device=dev)
            S.gdn_decode_step_buffered(x["qkv"].to(dev), x["a"].to(dev), x["b"].to(dev), Pd["A_log"],
                                       Pd["dt_bias"], st, idx.to(dev), out, rg["d"], rg["k"], rg["g"],
                                       torch.full((w.B,), wp, dtype=torch.int32, device=dev))
            outs.append(out.cpu())
            wp = (wp + 1) % L
        return outs, st.cpu()

    base_outs, base_st = run(None)
    outs, st = run(stop)
    for t in range(STEPS):
        assert torch.equal(outs[t], base_outs[t]), f"output at step {t} differs after resuming at {stop}"
    assert torch.equal(st, base_st)
    if act == "f32":
        ref_outs, ref_st = _oracle_run(w, P, idx, xs, state, ring, 0, ring_fmt=O.FMT_F32)
        for t in range(STEPS):
            assert_mixed(outs[t].reshape(w.B, w.HV, w.V), ref_outs[t], CHAIN_TOL, f"output at step {t}")
        named = idx.tolist()
        assert_mixed(st[named], ref_st[named], CHAIN_TOL, "final checkpoint")
