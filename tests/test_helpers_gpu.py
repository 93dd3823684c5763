"""GPU tests of the two helper entry points: ssmd_check_slot_indices, the
debug check that no two active rows of a call name one slot (the decode
steps' precondition; expected counts come from a plain host count over the
same vector), and the stream copy behind the benchmark's copy ceiling; and
calls on two streams at once (the library keeps no device state between
calls)."""
import numpy as np
import pytest
import torch

import ssm_recurrent_decode_gated_amd as S
import workloads as W
from tests._helpers import need_gpu

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _host_count(idx, num_slots, lo):
    seen, dups = set(), 0
    for s in idx:
        if lo <= s < num_slots:
            dups += s in seen
            seen.add(s)
    return dups


def _gpu_count(idx, num_slots, null_slot_zero=False):
    t = torch.tensor(idx, dtype=torch.int32, device=DEV)
    out = S.ssmd_check_slot_indices(t, num_slots, null_slot_zero)
    torch.cuda.synchronize()
    return int(out.item())


def test_benchmark_indices_are_valid():
    """The 256-of-264 permutation subset the bandwidth workload uses."""
    need_gpu()
    idx = W.slot_indices(W.GDN_B256).tolist()
    assert _gpu_count(idx, 264) == 0


@pytest.mark.parametrize("idx,num_slots,nz,want", [
    ([3, 1, 3], 4, False, 1),
    ([0, 0, 0, 2], 4, False, 2),
    ([0, 0, 0, 2], 4, True, 0),           # slot 0 is the NULL block under the KDA convention
    ([-1, -1, 5, 7, 7], 6, False, 0),     # padded rows (negative, past the pool) never count
    ([2, -1, 2, 9, 2], 6, False, 2),
    ([], 4, False, 0),
])
def test_small_vectors(idx, num_slots, nz, want):
    need_gpu()
    assert want == _host_count(idx, num_slots, 1 if nz else 0)
    assert _gpu_count(idx, num_slots, nz) == want


def test_large_vector_with_planted_duplicates():
    """4096 rows over a 5000-slot pool: a permutation with 37 rows redirected
    to slots earlier rows already hold, and 50 padded rows."""
    need_gpu()
    rng = np.random.default_rng(7)
    idx = rng.permutation(5000)[:4096].astype(np.int64)
    for i in rng.choice(np.arange(100, 4096), 37, replace=False):
        idx[i] = idx[rng.integers(0, 100)]
    idx[rng.choice(4096, 50, replace=False)] = -1
    want = _host_count(idx.tolist(), 5000, 0)
    assert want > 0
    assert _gpu_count(idx.tolist(), 5000) == want


def test_stream_copy_is_bit_exact():
    """The measurement aid the benchmark's copy ceiling uses: a 16-byte
    aligned copy of 33 MiB plus a 16-byte tail, compared bit for bit."""
    need_gpu()
    n = (33 * 2 ** 20 + 16) // 4
    src = torch.randn(n, device=DEV)
    dst = torch.zeros_like(src)
    S.ssmd_stream_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src.view(torch.int32), dst.view(torch.int32))


def test_two_streams_interleaved_calls():
    """Two independent workloads enqueued alternately on two streams (default
    priority) for several steps: each matches its own oracle run, so calls
    share no device state and take the stream they are given."""
    import oracle as O
    from tests._helpers import CHAIN_TOL, assert_mixed
    need_gpu()
    ws = [W.GDNWorkload(f"two_streams_{j}", B=6 + 4 * j, H=2, HV=4, K=128, V=64 + 64 * j, num_slots=12 + 4 * j,
                        out="f32", idx="perm") for j in range(2)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    setups = []
    for w in ws:
        P, idx, st = W.gdn_params(w), W.slot_indices(w), W.gdn_state(w)
        setups.append({"w": w, "P": P, "Pd": {k: v.to(DEV) for k, v in P.items()}, "idx": idx, "idx_d": idx.to(DEV),
                       "st_d": st.to(DEV), "ref": st.double().numpy().copy(),
                       "out": torch.empty(w.B, 1, w.HV, w.V, device=DEV)})
    torch.cuda.synchronize()
    steps = 6
    xs = [[W.gdn_step_inputs(s["w"], 100 + t) for t in range(steps)] for s in setups]
    xd = [[{k: v.to(DEV) for k, v in x.items()} for x in xl] for xl in xs]
    torch.cuda.synchronize()
    for t in range(steps):
        for j, s in enumerate(setups):
            with torch.cuda.stream(streams[j]):
                x = xd[j][t]
                S.gdn_decode_step(x["qkv"], x["a"], x["b"], s["Pd"]["A_log"], s["Pd"]["dt_bias"], s["st_d"],
                                  s["idx_d"], s["out"], stream=streams[j])
    torch.cuda.synchronize()
    for j, s in enumerate(setups):
        w = s["w"]
        for t in range(steps):
            x = xs[j][t]
            ro = O.gdn_step(x["qkv"], x["a"], x["b"], s["P"]["A_log"], s["P"]["dt_bias"], s["ref"], s["idx"],
                            H=w.H, HV=w.HV, K=w.K, V=w.V)
        assert_mixed(s["out"].reshape(w.B, w.HV, w.V), ro, CHAIN_TOL, f"workload {j}: last output")
        named = set(s["idx"].tolist())
        got = s["st_d"].cpu()
        for sl in named:
            assert_mixed(got[sl], s["ref"][sl], CHAIN_TOL, f"workload {j}: slot {sl}")
