"""Host threads calling the library at the same time. The entry points keep
no mutable state besides lazily filled caches (compute-unit count, launch
shape, the static workspace's device address) and the thread-local error
string, so four threads, each driving a different entry point on its own
stream (default priority), must produce bit for bit what the same calls
produce one after another on one stream. The threaded run comes first, so
in a fresh process the caches are filled under contention."""
import threading

import pytest
import torch

import ssm_recurrent_decode_gated_amd as S
import workloads as W
from tests._helpers import need_gpu
from tests.test_gdn_multi_gpu import _inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"
STEPS = 3


def _packed():
    w = W.GDNWorkload("threads_packed", B=40, H=16, HV=32, K=128, V=128, num_slots=44, out="f32", idx="perm")
    P, idx, st = W.gdn_params(w), W.slot_indices(w), W.gdn_state(w)
    xs = [W.gdn_step_inputs(w, 300 + t) for t in range(STEPS)]

    def make():
        return {"st": st.to(DEV), "out": torch.zeros(w.B, 1, w.HV, w.V, device=DEV)}

    def run(d, t, stream):
        x = xs[t]
        S.gdn_decode_step(x["qkv"].to(DEV), x["a"].to(DEV), x["b"].to(DEV), P["A_log"].to(DEV),
                          P["dt_bias"].to(DEV), d["st"], idx.to(DEV), d["out"], stream=stream)
    return make, run, ("st", "out")


def _buffered():
    w = W.GDNWorkload("threads_buffered", B=16, H=4, HV=8, K=128, V=128, num_slots=16, out="f32")
    P, idx, st = W.gdn_params(w), W.slot_indices(w), W.gdn_state(w)
    L = 4
    ring = W.gdn_ring(w, L)
    xs = [W.gdn_step_inputs(w, 400 + t) for t in range(STEPS)]

    def make():
        return {"st": st.to(DEV), "out": torch.zeros(w.B, 1, w.HV, w.V, device=DEV)} | \
               {k: v.to(DEV) for k, v in ring.items()}

    def run(d, t, stream):
        x = xs[t]
        wp = torch.full((w.B,), (t + 2) % L, dtype=torch.int32, device=DEV)  # phases 2, 3 (flush), 0
        S.gdn_decode_step_buffered(x["qkv"].to(DEV), x["a"].to(DEV), x["b"].to(DEV), P["A_log"].to(DEV),
                                   P["dt_bias"].to(DEV), d["st"], idx.to(DEV), d["out"], d["d_cache"],
                                   d["k_cache"], d["g_cache"], wp, stream=stream)
    return make, run, ("st", "out", "d_cache", "k_cache", "g_cache")


def _kda():
    w = W.KDAWorkload("threads_kda", T=8, H=4, num_slots=12)
    k = W.kda_inputs(w)

    def make():
        return {"st": k["state"].to(DEV), "cs": k["conv_state"].to(DEV),
                "out": torch.zeros(w.T, w.H, w.D, dtype=torch.bfloat16, device=DEV)}

    def run(d, t, stream):
        S.kda_decode_step(k["x"].to(DEV), k["conv_weight"].to(DEV), None, d["cs"], k["raw_g"].to(DEV),
                          k["raw_beta"].to(DEV), None, None, d["st"], k["idx"].to(DEV), d["out"],
                          output_gate=k["gate"].to(DEV), norm_weight=k["norm_weight"].to(DEV), stream=stream)
    return make, run, ("st", "cs", "out")


def _chunked():
    w = W.GDNWorkload("threads_chunk", B=2, H=2, HV=4, K=128, V=128, num_slots=2, out="f32")
    T = 100
    P, idx, st = W.gdn_params(w), W.slot_indices(w), W.gdn_state(w)
    x = _inputs(w, T)
    nws = S.gdn_chunk_workspace_bytes(w.B, T, w.HV, w.K, w.V)

    def make():
        return {"st": st.to(DEV), "out": torch.zeros(w.B, T, w.HV, w.V, device=DEV),
                "ws": torch.empty(nws // 4, device=DEV)}

    def run(d, t, stream):
        S.gdn_chunk_prefill(x["qkv"].to(DEV), x["a"].to(DEV), x["b"].to(DEV), P["A_log"].to(DEV),
                            P["dt_bias"].to(DEV), d["st"], idx.to(DEV), d["out"], workspace=d["ws"], stream=stream)
    return make, run, ("st", "out")


def test_four_host_threads_on_four_streams():
    need_gpu()
    jobs = [_packed(), _buffered(), _kda(), _chunked()]
    # the same calls from four threads at once, each on its own stream
    states = [make() for make, _, _ in jobs]
    torch.cuda.synchronize()
    barrier = threading.Barrier(len(jobs), timeout=60)  # a thread that fails early breaks it
    errors = []

    def worker(j):
        try:
            stream = torch.cuda.Stream()
            _, run, _ = jobs[j]
            barrier.wait()
            with torch.cuda.stream(stream):
                for t in range(STEPS):
                    run(states[j], t, stream)
            stream.synchronize()
        except Exception as e:  # reported in the main thread
            errors.append(f"job {j}: {e!r}")

    threads = [threading.Thread(target=worker, args=(j,)) for j in range(len(jobs))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    # the same calls one after another on the current stream
    seq = []
    for make, run, keys in jobs:
        d = make()
        torch.cuda.synchronize()
        for t in range(STEPS):
            run(d, t, None)
        torch.cuda.synchronize()
        seq.append({k: d[k].cpu() for k in keys})
    for j, (_, _, keys) in enumerate(jobs):
        for k in keys:
            assert torch.equal(seq[j][k], states[j][k].cpu()), f"job {j}: {k} differs from the sequential run"
