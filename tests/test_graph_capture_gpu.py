"""Every entry point enqueues work on the caller's stream only, with no
allocation, synchronisation or host read of device memory, so it can be
captured into a HIP graph. Each test captures calls, replays the graph
several times with eager work in between, and checks every replay against
the same calls made eagerly on identical copies of the inputs."""
import pytest
import torch

import ssm_recurrent_decode_gated_amd as S
import workloads as W
from tests.test_gdn_multi_gpu import _inputs
from tests._helpers import need_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _replay_matches_eager(make_state, call, outputs, replays=3):
    """make_state() -> dict of fresh device tensors; call(d) enqueues the op on
    the current stream; outputs(d) -> tensors to compare after each step."""
    eager, graph_d = make_state(), make_state()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call(graph_d)  # warm-up outside the capture (library load, first launch)
    torch.cuda.synchronize()
    graph_d.update(make_state())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(graph_d)
    for step in range(replays):
        call(eager)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outputs(eager), outputs(graph_d)):
            assert torch.equal(a, b), f"replay {step} differs from the eager call"


def _gdn_setup(w):
    P, idx, x = W.gdn_params(w), W.slot_indices(w), W.gdn_step_inputs(w)
    st = W.gdn_state(w)

    def make():
        return {"st": st.to(DEV), "out": torch.zeros(w.B, 1, w.HV, w.V, dtype=torch.bfloat16, device=DEV),
                "qkv": x["qkv"].to(DEV), "a": x["a"].to(DEV), "b": x["b"].to(DEV),
                "A_log": P["A_log"].to(DEV), "dt_bias": P["dt_bias"].to(DEV), "idx": idx.to(DEV)}
    return make


def test_graph_gdn_packed_and_state16():
    need_gpu()
    make = _gdn_setup(W.GDN_B16)
    _replay_matches_eager(make, lambda d: S.gdn_decode_step(d["qkv"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                                                            d["st"], d["idx"], d["out"]),
                          lambda d: (d["st"], d["out"]))

    def make16():
        d = make()
        d["st"] = d["st"].to(torch.bfloat16)
        return d
    _replay_matches_eager(make16, lambda d: S.gdn_decode_step_state16(d["qkv"], d["a"], d["b"], d["A_log"],
                                                                      d["dt_bias"], d["st"], d["idx"], d["out"]),
                          lambda d: (d["st"], d["out"]))


def test_graph_gdn_buffered_cycle():
    need_gpu()
    w = W.GDNWorkload("graph_buffered", B=8, H=2, HV=4, K=128, V=128, num_slots=8)
    make0 = _gdn_setup(w)
    L = 4

    def make():
        d = make0()
        d["d"] = torch.zeros(w.num_slots, w.HV, L, w.V, dtype=torch.bfloat16, device=DEV)
        d["k"] = torch.zeros(w.num_slots, w.H, L, w.K, dtype=torch.bfloat16, device=DEV)
        d["g"] = torch.zeros(w.num_slots, w.HV, L, device=DEV)
        d["wp"] = [torch.full((w.B,), p, dtype=torch.int32, device=DEV) for p in range(L)]
        return d

    def cycle(d):
        for p in range(L):
            S.gdn_decode_step_buffered(d["qkv"], d["a"], d["b"], d["A_log"], d["dt_bias"], d["st"], d["idx"],
                                       d["out"], d["d"], d["k"], d["g"], d["wp"][p])
    _replay_matches_eager(make, cycle, lambda d: (d["st"], d["out"], d["d"], d["k"], d["g"]))


def test_graph_kda_conv_and_mamba():
    need_gpu()
    w = W.KDAWorkload("graph_kda", T=12, H=4, D=128, num_slots=16)
    k = W.kda_inputs(w)

    def make_kda():
        return {n: v.to(DEV) for n, v in k.items()} | {"out": torch.zeros(w.T, w.H, w.D, dtype=torch.bfloat16,
                                                                          device=DEV)}
    _replay_matches_eager(make_kda, lambda d: S.kda_decode_step(d["x"], d["conv_weight"], None, d["conv_state"],
                                                                d["raw_g"], d["raw_beta"], None, None, d["state"],
                                                                d["idx"], d["out"], output_gate=d["gate"],
                                                                norm_weight=d["norm_weight"]),
                          lambda d: (d["state"], d["conv_state"], d["out"]))
    wg = W.GDNWorkload("graph_conv", B=4, H=2, HV=4, K=128, V=128, num_slots=4)
    make0 = _gdn_setup(wg)
    cv = W.gdn_conv(wg)

    def make_conv():
        d = make0()
        d.update(cw=cv["conv_weight"].to(DEV), cb=cv["conv_bias"].to(DEV), cs=cv["conv_state"].to(DEV))
        return d
    _replay_matches_eager(make_conv, lambda d: S.gdn_decode_step_conv(d["qkv"], d["cw"], d["cb"], d["cs"], d["a"],
                                                                      d["b"], d["A_log"], d["dt_bias"], d["st"],
                                                                      d["idx"], d["out"]),
                          lambda d: (d["st"], d["cs"], d["out"]))
    mw = W.MambaScanWorkload("graph_mamba_scan", B=2, T=200, Dm=256, N=16, num_slots=2)
    m = W.mamba_scan_inputs(mw)
    nws = S.mamba_scan_workspace_bytes(mw.B, mw.T, mw.Dm, mw.N)

    def make_scan():
        d = {n: v.to(DEV) for n, v in m.items()}
        d["out"] = torch.zeros(mw.B, mw.T, mw.Dm, dtype=torch.bfloat16, device=DEV)
        d["ws"] = torch.empty(max(nws // 4, 1), device=DEV)
        return d
    _replay_matches_eager(make_scan, lambda d: S.mamba_scan(d["x"], d["dt"], d["A"], d["Bm"], d["Cm"], d["Dv"],
                                                            d["z"], d["h"], d["idx"], d["out"], workspace=d["ws"]),
                          lambda d: (d["h"], d["out"]))


def test_graph_gdn_multi_and_chunked():
    need_gpu()
    w = W.GDNWorkload("graph_multi", B=2, H=2, HV=4, K=128, V=128, num_slots=2, out="f32")
    T = 100
    P, idx, st = W.gdn_params(w), W.slot_indices(w), W.gdn_state(w)
    x = _inputs(w, T)
    nws = S.gdn_chunk_workspace_bytes(w.B, T, w.HV, w.K, w.V)

    def make():
        return {"st": st.to(DEV), "out": torch.zeros(w.B, T, w.HV, w.V, device=DEV), "qkv": x["qkv"].to(DEV),
                "a": x["a"].to(DEV), "b": x["b"].to(DEV), "A_log": P["A_log"].to(DEV),
                "dt_bias": P["dt_bias"].to(DEV), "idx": idx.to(DEV), "ws": torch.empty(nws // 4, device=DEV)}
    _replay_matches_eager(make, lambda d: S.gdn_fused_recurrent(d["qkv"], d["a"], d["b"], d["A_log"],
                                                                d["dt_bias"], d["st"], d["idx"], d["out"]),
                          lambda d: (d["st"], d["out"]))
    _replay_matches_eager(make, lambda d: S.gdn_chunk_prefill(d["qkv"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                                                              d["st"], d["idx"], d["out"], workspace=d["ws"]),
                          lambda d: (d["st"], d["out"]))

    # the static-workspace form, for callers that cannot allocate under capture
    _replay_matches_eager(make, lambda d: S.gdn_chunk_prefill_noalloc(d["qkv"], d["a"], d["b"], d["A_log"],
                                                                      d["dt_bias"], d["st"], d["idx"], d["out"]),
                          lambda d: (d["st"], d["out"]))


def test_graph_mamba_decode():
    need_gpu()
    w = W.MambaWorkload("graph_mamba", B=8, Dm=1536, N=16, num_slots=8)
    m = W.mamba_inputs(w)

    def make():
        return {n: v.to(DEV) for n, v in m.items()} | {"out": torch.zeros(w.B, w.Dm, device=DEV)}
    _replay_matches_eager(make, lambda d: S.mamba_decode_step(d["x"], d["dt"], d["A"], d["Bm"], d["Cm"], d["Dv"],
                                                              d["z"], d["h"], d["idx"], d["out"]),
                          lambda d: (d["h"], d["out"]))

def test_graph_slot_index_check_and_stream_copy():
    """The two helper entry points captured too: the duplicate-slot count
    (into a result the graph overwrites each replay) and the stream copy."""
    need_gpu()

    def make():
        idx = W.slot_indices(W.GDN_B256).clone()
        idx[7] = idx[3]  # one planted duplicate
        return {"idx": idx.to(DEV), "dups": torch.full((1,), -1, dtype=torch.int32, device=DEV),
                "src": torch.arange(4096, dtype=torch.float32, device=DEV),
                "dst": torch.zeros(4096, dtype=torch.float32, device=DEV)}

    def call(d):
        S.ssmd_check_slot_indices(d["idx"], 264, dup_count=d["dups"])
        S.ssmd_stream_copy(d["src"], d["dst"])

    _replay_matches_eager(make, call, lambda d: (d["dups"], d["dst"]))
    d = make()
    call(d)
    torch.cuda.synchronize()
    assert int(d["dups"].item()) == 1
