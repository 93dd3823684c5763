"""Benchmark of the GDN single-token decode step on one MI355X.

Headline: state GB/s (and % of the 8 TB/s HBM peak) and us/step of
gdn_decode_step at B=256 rows over a 264-slot pool (H=16, HV=32, K=V=128,
bf16 activations, fp32 state), inputs resident in HBM. A step is one
gdn_decode_step call; consecutive steps rotate over several state pools so
the 256 MB Infinity Cache cannot hold the state between steps.

The same JSON line also carries the latency-to-bandwidth sweep (B = 1, 16,
64, 256 under HIP-graph replay of one call per pool), the buffered variant
against the packed step (B = 16, 64, 256; L = 1/8/16, exact cycle mean), the
fused KDA step (T=64, 96 heads, and one TP-8 rank's 12 heads),
the conv-fused GDN step, the 16-bit-state step, Mamba-1 decode and prefill
scan, the multi-token GDN call, the chunked and sequential GDN prefill, a
same-size stream-copy ceiling, the roofline entry of the dominant kernel and
the fp64 oracle's rate on the host cores.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle S] [--no-cpu-baseline]
                  [--batch-sizes 16 64 256] [--ls 1 8 16]     # the buffered legs
  python bench.py --replay-table [--batch-sizes 1 16 64 256] [--ls 1 8 16] [--hv 32] [--h 16] [--k 128]
                  [--v 128] [--dtype bf16|fp16|fp32]          # the ReplaySSM page's packed-vs-buffered table
  python bench.py --kda-table [--tokens 1 8 32 64 128] [--heads 12] [--layout SD|DS] [--graph]
                  [--layers N]                                # the fused-KDA page's table
  python bench.py --profile-pass [gdn|kda|chunk|buffered|conv|state16|multi]   # rocprofv3 counter passes
  python bench.py --summarize-counters FETCH_DIR WRITE_DIR --kernel gdn|kda --out profiles/X.txt
  python bench.py --summarize-trace TRACE_DIR --title T --command C --out profiles/X.md
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 * 2 ** 20
# What the headline kernel is built from: its source, the device header, and
# the two parameter structs it takes (other declarations in that header do
# not change it).
KERNEL_SOURCES = ["ssm_recurrent_decode_gated_amd/csrc/gdn_decode_pf.hip",
                  "ssm_recurrent_decode_gated_amd/csrc/ssmd_device.h"]
KERNEL_STRUCTS = ("ssm_recurrent_decode_gated_amd/csrc/ssmd_internal.h", ("GdnParams", "Launch"))
KERNEL_NAME = "gdn_decode_pf_kernel"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "gdn_b256_of264_hbm_counters.txt")
METRIC = "state GB/s (% of HBM peak) and µs/step, GDN decode HV=32 K=V=128, B=1/16/256"


def kernel_source_hash() -> str:
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    rel, names = KERNEL_STRUCTS
    text = open(os.path.join(ROOT, rel)).read()
    for name in names:
        m = re.search(r"^struct %s \{.*?^\};" % name, text, re.M | re.S)
        if m is None:
            raise SystemExit(f"struct {name} not found in {rel}")
        h.update(m.group(0).encode())
    return h.hexdigest()[:16]


# ------------------------------------------------------------ byte models
def gdn_state_bytes(B, HV, V, K):
    """State traffic of one packed step: each named head is read and written once."""
    return 2 * B * HV * V * K * 4


def gdn_alg_bytes(B, H, HV, K, V, act=2, outb=2):
    """All algorithmic bytes of one packed launch: state read+write, mixed_qkv,
    a, b, A_log, dt_bias, slot indices and the output."""
    return (gdn_state_bytes(B, HV, V, K) + B * (2 * H * K + HV * V) * act + 2 * B * HV * act
            + 2 * HV * 4 + B * 4 + B * HV * V * outb)


# ------------------------------------------------------------ helpers
def _events_ms(fn, reps, stream):
    import torch
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(reps):
        fn()
    e.record(stream)
    e.synchronize()
    return s.elapsed_time(e)


def _pools_for(pool_bytes, min_total=4 * MALL_BYTES, cap=64):
    return max(2, min(cap, -(-min_total // pool_bytes)))


class GDNSetup:
    """Device-resident inputs of one GDN workload, with M state pools."""

    def __init__(self, w, pools, dev, out_dtype="bf16"):
        import torch
        import workloads as W
        self.w = w
        self.P = W.gdn_params(w)
        self.x = W.gdn_step_inputs(w)
        self.idx = W.slot_indices(w)
        st = W.gdn_state(w)
        self.state_host = st
        d = {k: v.to(dev) for k, v in self.x.items()}
        self.qkv, self.a, self.b = d["qkv"], d["a"], d["b"]
        self.A_log, self.dt_bias = self.P["A_log"].to(dev), self.P["dt_bias"].to(dev)
        self.idx_d = self.idx.to(dev)
        first = st.to(dev)
        self.pools = [first] + [first.clone() for _ in range(pools - 1)]
        self.out = torch.empty(w.B, 1, w.HV, w.V, dtype=W.DTYPES[out_dtype], device=dev)

    def call(self, i):
        import ssm_recurrent_decode_gated_amd as S
        S.gdn_decode_step(self.qkv, self.a, self.b, self.A_log, self.dt_bias, self.pools[i % len(self.pools)],
                          self.idx_d, self.out)


GRAPH_MIN_CALLS = 64


def graph_time_us(calls, reps, stream, min_calls=GRAPH_MIN_CALLS):
    """us per call for a HIP graph holding `calls` (one launch each), replayed.
    The list is repeated in order until the graph holds at least `min_calls`
    launches, as a model step captures all its layers in one graph: a graph
    launch costs about 20 us on this runtime and does not overlap the previous
    replay, so a 2-call graph would charge 10 us to every call. Repeating the
    list keeps its pool rotation (and each pool's phase order). Five warm-up
    replays, then the median of at least 20 timed replays."""
    import torch
    for c in calls:  # warm (and first-touch) outside the capture
        c()
    torch.cuda.synchronize()
    calls = list(calls) * max(1, -(-min_calls // len(calls)))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    # one event pair per replay, median over the replays
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(max(reps, 20))]
    for a, b in ev:
        a.record(stream)
        g.replay()
        b.record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    n = len(ms)
    med = ms[n // 2] if n % 2 else 0.5 * (ms[n // 2 - 1] + ms[n // 2])
    return med * 1e3 / len(calls)


# ------------------------------------------------------------ legs
def _settle(call, seconds):
    """Runs call(0), call(1), ... untimed for `seconds` (synchronising every 64
    calls), past the clock ramp that follows any idle period; returns the
    number of calls."""
    import torch
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        call(n)
        n += 1
        if n % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def headline(dev, steps, warmup, settle_s=0.3):
    """The B=256-of-264 packed step, eager launches over rotated pools.

    After any idle period (here: the host-side input generation) the first
    ~60 launches run in a power-management transient: on MI355X launches
    10-40 after idle read 192-201 us against 185-186 us at steady state. So
    the W + K steps are first run straight after setup (reported as the cold
    sample), then the step runs untimed for `settle_s` seconds, then W
    warm-up steps and the K timed steps (the value)."""
    import torch
    import workloads as W
    w = W.GDN_B256
    pool_bytes = w.num_slots * w.HV * w.V * w.K * 4
    M = _pools_for(pool_bytes)
    su = GDNSetup(w, M, dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def sample():
        for i in range(warmup):
            su.call(i)
        torch.cuda.synchronize()
        it = iter(range(10 ** 9))
        ms = _events_ms(lambda: su.call(next(it)), steps, stream)
        torch.cuda.synchronize()
        return ms * 1e3 / steps
    cold = sample()
    n = _settle(su.call, settle_s)
    us = sample()
    sb = gdn_state_bytes(w.B, w.HV, w.V, w.K)
    ab = gdn_alg_bytes(w.B, w.H, w.HV, w.K, w.V)
    return {"w": w, "pools": M, "us": us, "state_gbs": sb / us / 1e3, "alg_gbs": ab / us / 1e3,
            "alg_bytes": ab, "state_bytes": sb, "setup": su, "cold_us": cold, "settle_steps": n}


def state16(dev, steps=200, warmup=10, settle_s=0.2):
    """The B=256-of-264 step on a bf16 state pool (gdn_decode_step_state16):
    half the state bytes of the fp32 step. Eager launches over rotated pools,
    timed after a settle period as the headline is."""
    import torch
    import ssm_recurrent_decode_gated_amd as S
    import workloads as W
    w = W.GDN_B256
    pool_bytes = w.num_slots * w.HV * w.V * w.K * 2
    M = _pools_for(pool_bytes)
    su = GDNSetup(w, 1, dev)
    first = su.pools[0].to(torch.bfloat16)
    su.pools = None
    torch.cuda.empty_cache()
    pools = [first] + [first.clone() for _ in range(M - 1)]

    def call(i):
        S.gdn_decode_step_state16(su.qkv, su.a, su.b, su.A_log, su.dt_bias, pools[i % M], su.idx_d, su.out)
    _settle(call, settle_s)
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    it = iter(range(10 ** 9))
    ms = _events_ms(lambda: call(next(it)), steps, torch.cuda.current_stream())
    us = ms * 1e3 / steps
    sb = w.B * w.HV * w.V * w.K * 2 * 2
    del pools, su
    torch.cuda.empty_cache()
    return {"workload": w.name + "_bf16_state", "us_per_step": round(us, 3), "state_GBps": round(sb / us / 1e3, 1),
            "pct_hbm_peak": round(100 * sb / us / 1e3 / HBM_PEAK_GBS, 2), "pools": M,
            "speedup_vs_fp32_state": None}


def sweep(dev, batches=(1, 16, 64, 256), reps=50):
    import workloads as W
    import torch
    res = {}
    for B in batches:
        w = W.gdn_sweep(B)
        pool_bytes = w.num_slots * w.HV * w.V * w.K * 4
        M = _pools_for(pool_bytes)
        su = GDNSetup(w, M, dev)
        us = graph_time_us([lambda i=i: su.call(i) for i in range(M)], reps, torch.cuda.current_stream())
        # the same M calls launched one by one from the host (a layer per pool):
        # what the graph replay amortises
        it = iter(range(10 ** 9))
        ms = _events_ms(lambda: su.call(next(it)), M * reps, torch.cuda.current_stream())
        eager = ms * 1e3 / (M * reps)
        sb = gdn_state_bytes(B, w.HV, w.V, w.K)
        res[f"B{B}"] = {"us_per_step": round(us, 3), "state_GBps": round(sb / us / 1e3, 1),
                        "pct_hbm_peak": round(100 * sb / us / 1e3 / HBM_PEAK_GBS, 2), "pools": M,
                        "eager_us_per_step": round(eager, 3)}
        if B == 1:
            # a graph holding one call, replayed: what one graph launch costs
            # when nothing amortises it (the page's one-call KDA graph)
            res["B1"]["one_call_graph_us"] = round(
                graph_time_us([lambda: su.call(0)], reps, torch.cuda.current_stream(), min_calls=1), 3)
        if pool_bytes <= MALL_BYTES // 2:
            # one pool stepped over and over: its state stays in the Infinity
            # Cache, so this is a cache rate, not an HBM one
            hot = graph_time_us([lambda: su.call(0)] * M, reps, torch.cuda.current_stream())
            res[f"B{B}"]["hot_single_pool_MALL_resident_us"] = round(hot, 3)
        del su
        torch.cuda.empty_cache()
    return res


def copy_ceiling(dev, nbytes=2 * 2 ** 30, reps=20):
    import torch
    import ssm_recurrent_decode_gated_amd as S
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).normal_()
    dst = torch.empty_like(src)
    S.ssmd_stream_copy(src, dst)
    torch.cuda.synchronize()
    ms = _events_ms(lambda: S.ssmd_stream_copy(src, dst), reps, torch.cuda.current_stream())
    gbs = 2 * nbytes * reps / (ms * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_moved_per_copy": 2 * nbytes, "GBps": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}


def buffered(dev, batches=(16, 64, 256), Ls=(1, 8, 16), reps=30, H=16, HV=32, K=128, V=128, act="bf16"):
    """The buffered step (gdn_decode_step_buffered) against the packed one at
    each batch size, the ReplaySSM page's comparison: per L, the exact mean
    of a full L-phase cycle (a graph holding phases 0..L-1 on every pool, so
    no cycle-mean estimate is needed), the non-flush phases 0 and (L-1)/2 and
    the flush phase L-1, the speed-up over the packed step (graph replay of
    the same pools) and the page's state-traffic ratio (1 + 1/L) / 2."""
    import torch
    import ssm_recurrent_decode_gated_amd as S
    import workloads as W
    tdt = W.DTYPES[act]
    out = {}
    for B in batches:
        w = W.GDNWorkload(f"gdn_b{B}_h{H}_hv{HV}_k{K}_v{V}_{act}", B=B, H=H, HV=HV, K=K, V=V, num_slots=B,
                          act=act)
        pool_bytes = w.num_slots * w.HV * w.V * w.K * 4
        M = _pools_for(pool_bytes)
        su = GDNSetup(w, M, dev)
        packed = graph_time_us([lambda i=i: su.call(i) for i in range(M)], reps, torch.cuda.current_stream())
        res = {"packed_us": round(packed, 3), "pools": M}
        for L in Ls:
            rings = [{"d": torch.zeros(w.num_slots, w.HV, L, w.V, dtype=tdt, device=dev),
                      "k": torch.zeros(w.num_slots, w.H, L, w.K, dtype=tdt, device=dev),
                      "g": torch.zeros(w.num_slots, w.HV, L, device=dev)} for _ in range(M)]
            wps = [torch.full((w.B,), p, dtype=torch.int32, device=dev) for p in range(L)]

            def call(i, p):
                r = rings[i]
                S.gdn_decode_step_buffered(su.qkv, su.a, su.b, su.A_log, su.dt_bias, su.pools[i], su.idx_d,
                                           su.out, r["d"], r["k"], r["g"], wps[p])
            # one cycle on every pool: L launches per pool, phases 0..L-1 in order
            calls = [lambda i=i, p=p: call(i, p) for p in range(L) for i in range(M)]
            us = graph_time_us(calls, reps, torch.cuda.current_stream())
            per_phase = {}
            for p in sorted({0, (L - 1) // 2, L - 1}):
                per_phase[p] = round(graph_time_us([lambda i=i, p=p: call(i, p) for i in range(M)], reps,
                                                   torch.cuda.current_stream()), 3)
            state_b = w.B * w.HV * w.V * w.K * 4 * (1 + 1.0 / L)
            res[f"L{L}"] = {"cycle_mean_us": round(us, 3), "phase_us": per_phase,
                            "speedup_vs_packed": round(packed / us, 3),
                            "state_GBps": round(state_b / us / 1e3, 1),
                            "state_bytes_ratio_vs_packed": round((1 + 1.0 / L) / 2, 5)}
            del rings
        out[f"B{B}"] = res
        del su
        torch.cuda.empty_cache()
    return out


def kda_time(dev, w, layout="SD", graph=True, layers=None, reps=30):
    """One fused KDA decode call (kda_decode_step) at workload w: graph replay
    of one call per layer (each layer its own state and conv-state buffers,
    `layers` of them, by default enough to exceed the Infinity Cache), or,
    without `graph`, the same calls launched one by one."""
    import torch
    import ssm_recurrent_decode_gated_amd as S
    import workloads as W
    d = W.kda_inputs(w, layout=layout)
    pool_bytes = w.num_slots * w.H * w.D * w.D * 4
    M = layers or _pools_for(pool_bytes)
    first = d["state"].to(dev)
    pools = [first] + [first.clone() for _ in range(M - 1)]
    cs = [d["conv_state"].to(dev) for _ in range(M)]
    dd = {k: d[k].to(dev) for k in ("x", "conv_weight", "raw_g", "raw_beta", "gate", "norm_weight", "idx")}
    out = torch.empty(w.T, w.H, w.D, dtype=torch.bfloat16, device=dev)

    def call(i):
        S.kda_decode_step(dd["x"], dd["conv_weight"], None, cs[i], dd["raw_g"], dd["raw_beta"], None, None,
                          pools[i], dd["idx"], out, output_gate=dd["gate"], norm_weight=dd["norm_weight"])
    if graph:
        us = graph_time_us([lambda i=i: call(i) for i in range(M)], reps, torch.cuda.current_stream())
    else:
        for i in range(M):
            call(i)
        it = iter(range(10 ** 9))
        us = _events_ms(lambda: call(next(it) % M), M * reps, torch.cuda.current_stream()) * 1e3 / (M * reps)
    sb = w.T * w.H * w.D * w.D * 4 * 2
    ab = kda_alg_bytes(w)
    del pools, cs
    torch.cuda.empty_cache()
    return {"workload": w.name, "us_per_step": round(us, 3), "state_GBps": round(sb / us / 1e3, 1),
            "pct_hbm_peak": round(100 * sb / us / 1e3 / HBM_PEAK_GBS, 2), "alg_GBps": round(ab / us / 1e3, 1),
            "pct_hbm_peak_alg": round(100 * ab / us / 1e3 / HBM_PEAK_GBS, 2), "layers": M,
            "timing": "graph replay" if graph else "eager dispatch", "layout": layout}


def kda(dev, reps=30):
    """The fused KDA op at T = 64 tokens x 96 heads, and one tensor-parallel
    rank's share (12 heads: the step has no exchange between heads)."""
    import workloads as W
    res = kda_time(dev, W.KDA_T64, reps=reps)
    res["tp8_rank_h12"] = kda_time(dev, W.KDAWorkload("kda_t64_h12_d128_w4", T=64, H=12, num_slots=72), reps=reps)
    return res


def gdn_conv_alg_bytes(w, Wd=4):
    """The packed step's algorithmic bytes plus the conv state read and
    written (16-bit) and the conv weights and bias read once (fp32)."""
    C = 2 * w.H * w.K + w.HV * w.V
    return gdn_alg_bytes(w.B, w.H, w.HV, w.K, w.V) + 2 * w.B * C * (Wd - 1) * 2 + C * (Wd + 1) * 4


def gdn_conv(dev, reps=30, Wd=4):
    """The B=256-of-264 GDN step with its causal conv1d update fused in front
    (gdn_decode_step_conv, conv width 4, bf16 conv state in the [slots, C,
    W-1] layout), graph replay of one call per pool. Algorithmic bytes: the
    packed step's plus the conv state read and written and the conv weights
    read once."""
    import torch
    import ssm_recurrent_decode_gated_amd as S
    import workloads as W
    w = W.GDN_B256
    pool_bytes = w.num_slots * w.HV * w.V * w.K * 4
    M = _pools_for(pool_bytes)
    su = GDNSetup(w, M, dev)
    cv = W.gdn_conv(w, Wd)
    cw, cb = cv["conv_weight"].to(dev), cv["conv_bias"].to(dev)
    cs = [cv["conv_state"].to(dev) for _ in range(M)]

    def call(i):
        S.gdn_decode_step_conv(su.qkv, cw, cb, cs[i], su.a, su.b, su.A_log, su.dt_bias, su.pools[i], su.idx_d,
                               su.out)
    us = graph_time_us([lambda i=i: call(i) for i in range(M)], reps, torch.cuda.current_stream())
    sb = gdn_state_bytes(w.B, w.HV, w.V, w.K)
    ab = gdn_conv_alg_bytes(w, Wd)
    del su, cs
    torch.cuda.empty_cache()
    return {"workload": w.name + f"_conv{Wd}", "us_per_step": round(us, 3), "state_GBps": round(sb / us / 1e3, 1),
            "alg_GBps": round(ab / us / 1e3, 1), "pct_hbm_peak_alg": round(100 * ab / us / 1e3 / HBM_PEAK_GBS, 2),
            "pools": M}


def mamba(dev, reps=30):
    """Mamba-1 decode (graph replay of one call per pool): the MBU write-up's
    table shapes, plus a bandwidth-sized batch. Byte counts: the write-up's
    model B*D*(20N+24), and the state traffic B*D*N*8."""
    import torch
    import ssm_recurrent_decode_gated_amd as S
    import workloads as W
    res = {}
    for (B, Dm, N) in ((1, 1536, 16), (8, 1536, 16), (1, 1536, 64), (256, 4096, 16)):
        w = W.MambaWorkload(f"mamba_b{B}_d{Dm}_n{N}", B=B, Dm=Dm, N=N, num_slots=B)
        d = W.mamba_inputs(w)
        pool_bytes = B * Dm * N * 4
        M = _pools_for(pool_bytes)
        dd = {k: v.to(dev) for k, v in d.items()}
        pools = [dd["h"]] + [dd["h"].clone() for _ in range(M - 1)]
        out = torch.empty(B, Dm, device=dev)

        def call(i):
            S.mamba_decode_step(dd["x"], dd["dt"], dd["A"], dd["Bm"], dd["Cm"], dd["Dv"], dd["z"], pools[i],
                                dd["idx"], out)
        us = graph_time_us([lambda i=i: call(i) for i in range(M)], reps, torch.cuda.current_stream())
        # launched one by one from Python, as the write-up's table times its calls
        it = iter(range(10 ** 9))
        eager = _events_ms(lambda: call(next(it) % M), M * reps, torch.cuda.current_stream()) * 1e3 / (M * reps)
        res[f"B{B}_D{Dm}_N{N}"] = {"us_per_step": round(us, 3), "eager_us_per_step": round(eager, 3),
                                   "page_model_GBps": round(B * Dm * (20 * N + 24) / us / 1e3, 1),
                                   "state_GBps": round(B * Dm * N * 8 / us / 1e3, 1), "pools": M}
        del pools, dd
        torch.cuda.empty_cache()
    return res


def gdn_multi(dev, reps=20):
    """The GDN step over T tokens per row (gdn_fused_recurrent), bf16, H=16,
    HV=32, K=V=128: verification of 4 and 8 speculative tokens at B=256 and
    64 (one state round trip for all T tokens; compared with T packed steps),
    and a 2048-token prompt at B=1. Pools rotated as in the sweep."""
    import torch
    import ssm_recurrent_decode_gated_amd as S
    import workloads as W
    res = {}
    for (B, T) in ((256, 4), (64, 8), (1, 2048)):
        w = W.gdn_sweep(B)
        pool_bytes = w.num_slots * w.HV * w.V * w.K * 4
        M = _pools_for(pool_bytes)
        su = GDNSetup(w, M, dev)
        g = W.generator(0, w.name, "multi", T)
        C = 2 * w.H * w.K + w.HV * w.V
        qkv = W.normal((B, T, C), 1.0, "bf16", g).to(dev)
        a = W.normal((B, T, w.HV), 0.5, "bf16", g).to(dev)
        b = W.normal((B, T, w.HV), 1.0, "bf16", g).to(dev)
        out = torch.empty(B, T, w.HV, w.V, dtype=torch.bfloat16, device=dev)

        def call(i):
            S.gdn_fused_recurrent(qkv, a, b, su.A_log, su.dt_bias, su.pools[i], su.idx_d, out)
        us = graph_time_us([lambda i=i: call(i) for i in range(M)], reps, torch.cuda.current_stream())
        sb = gdn_state_bytes(B, w.HV, w.V, w.K)
        res[f"B{B}_T{T}"] = {"us_per_call": round(us, 2), "tokens_per_s": round(B * T / us * 1e6),
                             "state_GBps": round(sb / us / 1e3, 1), "pools": M}
        del su, qkv, a, b, out
        torch.cuda.empty_cache()
    return res


def gdn_prefill(dev, reps=10):
    """GDN prompts (H=16, HV=32, K=V=128, bf16) through the chunked form
    (gdn_chunk_prefill, chunks of 64 tokens) and the sequential multi-token
    kernel (gdn_fused_recurrent): one 2048-token prompt and 8 at once."""
    import torch
    import ssm_recurrent_decode_gated_amd as S
    import workloads as W
    res = {}
    for (B, T) in ((1, 2048), (8, 2048)):
        w = W.gdn_sweep(B)
        su = GDNSetup(w, 2, dev)
        g = W.generator(0, w.name, "prefill", T)
        C = 2 * w.H * w.K + w.HV * w.V
        qkv = W.normal((B, T, C), 1.0, "bf16", g).to(dev)
        a = W.normal((B, T, w.HV), 0.5, "bf16", g).to(dev)
        b = W.normal((B, T, w.HV), 1.0, "bf16", g).to(dev)
        out = torch.empty(B, T, w.HV, w.V, dtype=torch.bfloat16, device=dev)
        ws = torch.empty(S.gdn_chunk_workspace_bytes(B, T, w.HV, w.K, w.V) // 4, device=dev)
        r = {}
        for name, fn, kw in (("chunked", S.gdn_chunk_prefill, {"workspace": ws}),
                             ("sequential", S.gdn_fused_recurrent, {})):
            def call(i, fn=fn, kw=kw):
                fn(qkv, a, b, su.A_log, su.dt_bias, su.pools[i], su.idx_d, out, **kw)
            us = graph_time_us([lambda i=i: call(i) for i in range(2)], reps, torch.cuda.current_stream())
            r[name] = {"us_per_call": round(us, 1), "tokens_per_s": round(B * T / us * 1e6)}
        r["workspace_bytes"] = ws.numel() * 4
        res[f"B{B}_T{T}"] = r
        del su, qkv, a, b, out, ws
        torch.cuda.empty_cache()
    return res


def mamba_prefill(dev, reps=20):
    """Mamba-1 multi-token scan (mamba_scan), bf16 activations: one 2048-token
    prompt at the page's model width (chunk-parallel with the workspace the
    library asks for, and one sequential pass without), and 8 prompts at
    once. Input sets are rotated so the replayed graph touches more than the
    Infinity Cache holds. Bytes: x, dt, z read and y written (2 B each per
    token and channel), B and C (2 B per token and state element), the state
    read and written once."""
    import torch
    import ssm_recurrent_decode_gated_amd as S
    import workloads as W
    res = {}
    for (B, T, Dm, N, chunked) in ((1, 2048, 1536, 16, True), (1, 2048, 1536, 16, False), (8, 2048, 1536, 16, True)):
        w = W.MambaScanWorkload(f"mamba_prefill_b{B}_t{T}_d{Dm}_n{N}", B=B, T=T, Dm=Dm, N=N, num_slots=B)
        d = W.mamba_scan_inputs(w)
        alg = B * T * Dm * 8 + B * T * N * 4 + 2 * B * Dm * N * 4
        M = _pools_for(alg)
        sets = [{k: v.to(dev) for k, v in d.items()} for _ in range(M)]
        out = torch.empty(B, T, Dm, dtype=torch.bfloat16, device=dev)
        nws = S.mamba_scan_workspace_bytes(B, T, Dm, N) if chunked else 0
        ws = torch.empty(max(nws // 4, 1), device=dev) if nws else None

        def call(i):
            s = sets[i]
            S.mamba_scan(s["x"], s["dt"], s["A"], s["Bm"], s["Cm"], s["Dv"], s["z"], s["h"], s["idx"], out,
                         workspace=ws)
        us = graph_time_us([lambda i=i: call(i) for i in range(M)], reps, torch.cuda.current_stream())
        key = f"B{B}_T{T}_D{Dm}_N{N}_" + ("chunked" if chunked else "single_pass")
        res[key] = {"us_per_call": round(us, 2), "tokens_per_s": round(B * T / us * 1e6),
                    "alg_GBps": round(alg / us / 1e3, 1), "workspace_bytes": nws, "sets": M,
                    "exp_per_s_T": round(B * T * Dm * N / us / 1e6, 2)}
        del sets, ws
        torch.cuda.empty_cache()
    return res


def cpu_baseline(su, target_s=10.0, single_s=5.0):
    """The fp64 oracle, as it stands, on the host cores: the full B=256 step
    repeated (state evolving) until about target_s seconds have passed on all
    threads, then single_s seconds on one thread."""
    import numpy as np
    import oracle as O
    w = su.w
    ref = su.state_host.double().numpy().copy()
    q, a, b = O.f64(su.x["qkv"]), O.f64(su.x["a"]), O.f64(su.x["b"])
    idx = su.idx.numpy().astype(np.int32)
    sb1 = gdn_state_bytes(w.B, w.HV, w.V, w.K)

    def run(limit):
        n, t0 = 0, time.perf_counter()
        while True:
            O.gdn_step(q, a, b, su.P["A_log"], su.P["dt_bias"], ref, idx, H=w.H, HV=w.HV, K=w.K, V=w.V)
            n += 1
            el = time.perf_counter() - t0
            if el >= limit:
                return n, el
    cores = O.num_threads()
    n, el = run(target_s)
    O.set_threads(1)
    n1, el1 = run(single_s)
    O.set_threads(cores)
    return {"value": round(sb1 * n / el / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "us_per_step": round(el / n * 1e6, 1),
            "single_thread": {"value": round(sb1 * n1 / el1 / 1e9, 3), "unit": "GB/s", "cores": 1,
                              "us_per_step": round(el1 / n1 * 1e6, 1), "steps": n1},
            "sample": f"full B=256-of-264 step (H=16, HV=32, K=V=128) repeated {n} times in {el:.1f} s on "
                      f"{cores} threads, then {n1} times in {el1:.1f} s on one; fp32-state byte model"}


TRACE_FILE = os.path.join(ROOT, "profiles", "gdn_b256_of264_kernel_trace.md")


def trace_kernel_avg_us():
    """The headline kernel's average duration in the committed rocprofv3
    kernel-trace summary, or None when the kernel source changed since."""
    if not os.path.exists(TRACE_FILE):
        return None
    text = open(TRACE_FILE).read()
    if f"kernel_source_sha256 = {kernel_source_hash()}" not in text:
        return None
    for line in text.splitlines():
        if line.startswith("|") and KERNEL_NAME in line:
            cells = [c.strip() for c in line.strip("|").split("|")]
            try:
                return round(float(cells[3]) / 1e3, 3)
            except (IndexError, ValueError):
                return None
    return None


def counters_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel source changed since it was taken."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    kv = {}
    for line in open(COUNTERS_FILE):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        copy_kib = float(kv["copy_bytes"]) / 1024
        ff = copy_kib / float(kv["copy_fetch_kib"])
        wf = copy_kib / float(kv["copy_write_kib"])
        return float(kv["gdn_fetch_kib"]) * 1024 * ff + float(kv["gdn_write_kib"]) * 1024 * wf
    except (KeyError, ValueError, ZeroDivisionError):
        return None


# ------------------------------------------------------------ rocprofv3 helpers
def kda_alg_bytes(w, out_bytes=2, act=2):
    """All algorithmic bytes of one fused KDA launch: state read + write, conv
    state read + write, x, raw_g, raw_beta, output gate, output, conv weights."""
    C = 3 * w.H * w.D
    return (2 * w.T * w.H * w.D * w.D * 4 + 2 * w.T * C * (w.W - 1) * act + w.T * C * act
            + w.T * w.H * w.D * act + w.T * w.H * act + w.T * w.H * w.D * act + w.T * w.H * w.D * out_bytes
            + C * w.W * 4)


BUF_PROF_L, BUF_PROF_P = 8, 3  # ring length and phase of the buffered counter pass
MULTI_PROF_T = 4  # tokens per row in the multi-token counter pass


def buffered_nonflush_alg_bytes(w, p, act=2, outb=2):
    """Bytes a non-flush buffered step at phase p must move: the checkpoint
    and the p ring records read; q/k/v, a, b, A_log, dt_bias, indices and
    phases read; the output and this step's record (delta, key, g) written."""
    state = w.B * w.HV * w.V * w.K * 4
    ring_rd = p * w.B * (w.HV * w.V * act + w.H * w.K * act + w.HV * 4)
    inputs = w.B * (2 * w.H * w.K + w.HV * w.V) * act + 2 * w.B * w.HV * act + 2 * w.HV * 4 + 2 * w.B * 4
    writes = w.B * w.HV * w.V * outb + w.B * (w.HV * w.V * act + w.H * w.K * act + w.HV * 4)
    return state + ring_rd + inputs + writes


def profile_pass(which="gdn"):
    """A few launches of one kernel (the headline GDN step, the fused KDA op at
    64 tokens x 96 heads, or the chunked GDN prefill of one and of eight
    2048-token prompts) and one copy of known size, for rocprofv3 counter
    passes."""
    import torch
    import ssm_recurrent_decode_gated_amd as S
    import workloads as W
    dev = torch.device("cuda:0")
    if which == "chunk":
        for B in (1, 8):
            w = W.gdn_sweep(B)
            su = GDNSetup(w, 1, dev)
            T = 2048
            g = W.generator(0, w.name, "prefill", T)
            C = 2 * w.H * w.K + w.HV * w.V
            qkv = W.normal((B, T, C), 1.0, "bf16", g).to(dev)
            a = W.normal((B, T, w.HV), 0.5, "bf16", g).to(dev)
            b = W.normal((B, T, w.HV), 1.0, "bf16", g).to(dev)
            out = torch.empty(B, T, w.HV, w.V, dtype=torch.bfloat16, device=dev)
            ws = torch.empty(S.gdn_chunk_workspace_bytes(B, T, w.HV, w.K, w.V) // 4, device=dev)
            for _ in range(3):
                S.gdn_chunk_prefill(qkv, a, b, su.A_log, su.dt_bias, su.pools[0], su.idx_d, out, workspace=ws)
            del su, qkv, a, b, out, ws
    elif which == "state16":
        w = W.GDN_B256
        su = GDNSetup(w, 1, dev)
        st16 = su.pools[0].to(torch.bfloat16)
        for _ in range(4):
            S.gdn_decode_step_state16(su.qkv, su.a, su.b, su.A_log, su.dt_bias, st16, su.idx_d, su.out)
        del su, st16
    elif which == "multi":
        w = W.GDN_B256
        su = GDNSetup(w, 1, dev)
        g = W.generator(0, w.name, "multi", MULTI_PROF_T)
        C = 2 * w.H * w.K + w.HV * w.V
        qkv = W.normal((w.B, MULTI_PROF_T, C), 1.0, "bf16", g).to(dev)
        a = W.normal((w.B, MULTI_PROF_T, w.HV), 0.5, "bf16", g).to(dev)
        b = W.normal((w.B, MULTI_PROF_T, w.HV), 1.0, "bf16", g).to(dev)
        out = torch.empty(w.B, MULTI_PROF_T, w.HV, w.V, dtype=torch.bfloat16, device=dev)
        for _ in range(4):
            S.gdn_fused_recurrent(qkv, a, b, su.A_log, su.dt_bias, su.pools[0], su.idx_d, out)
        del su, qkv, a, b, out
    elif which == "conv":
        w = W.GDN_B256
        su = GDNSetup(w, 1, dev)
        cv = {k: v.to(dev) for k, v in W.gdn_conv(w, 4).items()}
        for _ in range(4):
            S.gdn_decode_step_conv(su.qkv, cv["conv_weight"], cv["conv_bias"], cv["conv_state"], su.a, su.b,
                                   su.A_log, su.dt_bias, su.pools[0], su.idx_d, su.out)
        del su, cv
    elif which == "buffered":
        # non-flush steps of the buffered form: B = 64, phase 3 of an 8-record ring
        w = W.GDN_B64_CHAIN
        su = GDNSetup(w, 1, dev)
        ring = {k: v.to(dev) for k, v in W.gdn_ring(w, BUF_PROF_L).items()}
        wp = torch.full((w.B,), BUF_PROF_P, dtype=torch.int32, device=dev)
        for _ in range(4):
            S.gdn_decode_step_buffered(su.qkv, su.a, su.b, su.A_log, su.dt_bias, su.pools[0], su.idx_d, su.out,
                                       ring["d_cache"], ring["k_cache"], ring["g_cache"], wp)
        del su, ring
    elif which == "kda":
        w = W.KDA_T64
        d = {k: v.to(dev) for k, v in W.kda_inputs(w).items()}
        out = torch.empty(w.T, w.H, w.D, dtype=torch.bfloat16, device=dev)
        for i in range(4):
            S.kda_decode_step(d["x"], d["conv_weight"], None, d["conv_state"], d["raw_g"], d["raw_beta"], None, None,
                              d["state"], d["idx"], out, output_gate=d["gate"], norm_weight=d["norm_weight"])
    else:
        su = GDNSetup(W.GDN_B256, 2, dev)
        for i in range(6):
            su.call(i)
    n = 1 << 30
    src = torch.ones(n // 4, device=dev)
    dst = torch.empty_like(src)
    S.ssmd_stream_copy(src, dst)
    torch.cuda.synchronize()
    print(f"profile pass done: {which} launches, 1 x stream copy of {n} bytes", flush=True)


def _read_counter_csv(d, counter, kernel=KERNEL_NAME):
    import csv
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r.get("Counter_Name") != counter:
                continue
            name = r.get("Kernel_Name", "")
            key = "gdn" if kernel in name else ("copy" if "stream_copy_kernel" in name else None)
            if key:
                per.setdefault(key, {}).setdefault(r.get("Dispatch_Id"), 0.0)
                per[key][r.get("Dispatch_Id")] += float(r["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in per.items()}


def summarize_counters(fetch_dir, write_dir, out, command, which="gdn"):
    import workloads as W
    if which == "kda":
        kernel, wl = "kda_decode_pf_kernel", W.KDA_T64
        alg = kda_alg_bytes(wl)
        title = f"# rocprofv3 HBM counters, {kernel} at 64 tokens x 96 heads (D=128, conv width 4, bf16 act, norm)"
    elif which == "state16":
        kernel, wl = "gdn_decode_s16_kernel", W.GDN_B256
        alg = gdn_alg_bytes(wl.B, wl.H, wl.HV, wl.K, wl.V) - gdn_state_bytes(wl.B, wl.HV, wl.V, wl.K) // 2
        title = f"# rocprofv3 HBM counters, {kernel} at B=256 of 264 slots (H=16 HV=32 K=V=128, bf16 act, bf16 state)"
    elif which == "multi":
        kernel, wl = "gdn_multi_kernel", W.GDN_B256
        T = MULTI_PROF_T
        alg = (gdn_state_bytes(wl.B, wl.HV, wl.V, wl.K) + T * wl.B * (2 * wl.H * wl.K + wl.HV * wl.V) * 2
               + 2 * T * wl.B * wl.HV * 2 + T * wl.B * wl.HV * wl.V * 2 + 2 * wl.HV * 4 + wl.B * 4)
        title = f"# rocprofv3 HBM counters, {kernel} at B=256 of 264 slots x {T} tokens (H=16 HV=32 K=V=128, bf16)"
    elif which == "conv":
        kernel, wl = "gdn_conv_pf_kernel", W.GDN_B256
        alg = gdn_conv_alg_bytes(wl, 4)
        title = f"# rocprofv3 HBM counters, {kernel} at B=256 of 264 slots (H=16 HV=32 K=V=128, bf16 act, conv width 4)"
    elif which == "buffered":
        kernel, wl = "gdn_buffered_kernel", W.GDN_B64_CHAIN
        alg = buffered_nonflush_alg_bytes(wl, BUF_PROF_P)
        title = (f"# rocprofv3 HBM counters, {kernel} at B=64 (H=16 HV=32 K=V=128, bf16 act and ring), "
                 f"non-flush phase {BUF_PROF_P} of L={BUF_PROF_L}")
    else:
        kernel, wl = KERNEL_NAME, W.GDN_B256
        alg = gdn_alg_bytes(wl.B, wl.H, wl.HV, wl.K, wl.V)
        title = f"# rocprofv3 HBM counters, {kernel} at B=256 of 264 slots (H=16 HV=32 K=V=128, bf16 act)"
    f = _read_counter_csv(fetch_dir, "FETCH_SIZE", kernel)
    w = _read_counter_csv(write_dir, "WRITE_SIZE", kernel)
    copy_bytes = 1 << 30
    ff, wf = copy_bytes / 1024 / f["copy"], copy_bytes / 1024 / w["copy"]
    traffic = f["gdn"] * 1024 * ff + w["gdn"] * 1024 * wf
    lines = [
        title,
        f"# command: {command}",
        "# values are KiB per dispatch, averaged over dispatches; the copy kernel moves copy_bytes each way",
        f"kernel_source_sha256 = {kernel_source_hash()}" if which == "gdn" else f"kernel = {kernel}",
        f"gdn_fetch_kib = {f['gdn']:.1f}" if which == "gdn" else f"kernel_fetch_kib = {f['gdn']:.1f}",
        f"gdn_write_kib = {w['gdn']:.1f}" if which == "gdn" else f"kernel_write_kib = {w['gdn']:.1f}",
        f"copy_bytes = {copy_bytes}",
        f"copy_fetch_kib = {f['copy']:.1f}",
        f"copy_write_kib = {w['copy']:.1f}",
        f"# fetch scale {ff:.4f}, write scale {wf:.4f}",
        f"# scaled HBM traffic per launch = {traffic / 1e6:.2f} MB; algorithmic = {alg / 1e6:.2f} MB "
        f"(ratio {traffic / alg:.4f})",
    ]
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# ------------------------------------------------------------ main
def summarize_trace(trace_dir, out, command, title):
    """Markdown table of rocprofv3's kernel statistics (run_kernel_stats.csv)."""
    import csv
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    rows = list(csv.DictReader(open(files[0])))
    cols = ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"]
    lines = [f"# {title}", "", "Command (run from /tmp on the MI355X, `<repo>` = repository root):", "",
             f"    {command}", ""]
    if any(KERNEL_NAME in r["Name"] for r in rows):
        lines += [f"kernel_source_sha256 = {kernel_source_hash()} ({KERNEL_NAME} source at the time of the run)",
                  ""]
    lines += ["`run_kernel_stats.csv`:", "", "| " + " | ".join(cols) + " |", "|" + "---|" * len(cols)]
    for r in rows:
        name = r["Name"]
        if len(name) > 160:  # torch's generated template names; the head names the kernel
            name = name[:150] + " ..."
        vals = [f"`{name}`"] + [r.get(c, "") for c in cols[1:]]
        lines.append("| " + " | ".join(vals) + " |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def replay_table(dev, args):
    """The ReplaySSM page's table (its `main`): per batch size the packed
    step, then per L the buffered cycle mean split into its non-flush and
    flush steps, the speed-up and the state-traffic ratio. Times in ms, as
    the page prints them."""
    act = {"bf16": "bf16", "fp16": "f16", "fp32": "f32"}[args.dtype]
    print(f"GDN buffered decode HV={args.hv} H={args.h} K={args.k} V={args.v} dtype={args.dtype}\n"
          "replay = exact mean per-step latency over one L-phase cycle (ms; graph replay, pools rotated past "
          "the Infinity Cache); speedup = packed/replay; state-traffic = replay/packed", flush=True)
    for B in args.batch_sizes:
        r = buffered(dev, batches=(B,), Ls=tuple(args.ls), H=args.h, HV=args.hv, K=args.k, V=args.v,
                     act=act)[f"B{B}"]
        print(f"\nB={B:<4d} packed={r['packed_us'] / 1e3:.4f} ms")
        for L in args.ls:
            x = r[f"L{L}"]
            ph = x["phase_us"]
            split = "(flush only)" if L == 1 else \
                f"(non-flush {ph[(L - 1) // 2] / 1e3:.4f}, flush {ph[L - 1] / 1e3:.4f})"
            print(f"  L={L:<3d} replay={x['cycle_mean_us'] / 1e3:.4f} ms speedup={x['speedup_vs_packed']:5.2f}x "
                  f"state-traffic={x['state_bytes_ratio_vs_packed']:5.2f}x {split}", flush=True)


def kda_table(dev, args):
    """The fused-KDA page's table (its `main`): per head count and token
    count, the fused op's time and its state TB/s."""
    import workloads as W
    mode = "graph replay" if args.graph else "eager dispatch"
    print(f"device: {__import__('torch').cuda.get_device_name(0)} timing: {mode} layout: {args.layout}")
    print(f"{'heads':>6} {'tokens':>7} {'fused us':>9} {'state TB/s':>11} {'all TB/s':>9} {'layers':>7}", flush=True)
    for H in args.heads:
        for T in args.tokens:
            w = W.KDAWorkload(f"kda_t{T}_h{H}_d128_w4", T=T, H=H, num_slots=T + 8, layout=args.layout)
            r = kda_time(dev, w, layout=args.layout, graph=args.graph, layers=args.layers)
            print(f"{H:>6} {T:>7} {r['us_per_step']:>9.2f} {r['state_GBps'] / 1e3:>11.3f} "
                  f"{r['alg_GBps'] / 1e3:>9.3f} {r['layers']:>7}", flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds the headline step runs untimed before its warm-up (leaves the post-idle "
                         "power-management transient)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--replay-table", action="store_true", help="print the ReplaySSM page's table and exit")
    ap.add_argument("--kda-table", action="store_true", help="print the fused-KDA page's table and exit")
    ap.add_argument("--batch-sizes", type=int, nargs="+", default=None,
                    help="buffered legs (default 16 64 256) / --replay-table rows (default 1 16 64 256)")
    ap.add_argument("--ls", type=int, nargs="+", default=[1, 8, 16], help="buffered ring lengths")
    ap.add_argument("--hv", type=int, default=32)
    ap.add_argument("--h", type=int, default=16)
    ap.add_argument("--k", type=int, default=128)
    ap.add_argument("--v", type=int, default=128)
    ap.add_argument("--dtype", choices=("bf16", "fp16", "fp32"), default="bf16")
    ap.add_argument("--tokens", type=int, nargs="+", default=[1, 8, 32, 64, 128])
    ap.add_argument("--heads", type=int, nargs="+", default=[12])
    ap.add_argument("--layout", choices=("SD", "DS"), default="SD")
    ap.add_argument("--graph", action="store_true", help="--kda-table: graph replay instead of eager dispatch")
    ap.add_argument("--layers", type=int, default=None,
                    help="--kda-table: layers (state buffers) per graph; default: enough to exceed the "
                         "Infinity Cache")
    ap.add_argument("--no-extras", action="store_true", help="headline only (no sweep/buffered/KDA/conv/Mamba/copy)")
    ap.add_argument("--profile-pass", nargs="?", const="gdn",
                    choices=("gdn", "kda", "chunk", "buffered", "conv", "state16", "multi"))
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR")
    ap.add_argument("--title", default="")
    ap.add_argument("--kernel", default="gdn", choices=("gdn", "kda", "buffered", "conv", "state16", "multi"),
                    help="which kernel --summarize-counters covers")
    ap.add_argument("--out", default=COUNTERS_FILE)
    ap.add_argument("--command", default="")
    args = ap.parse_args()

    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.out, args.command, args.kernel)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.out, args.command, args.title)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the decode step has no cross-GPU exchange (each slot and "
              "head is independent), so the figure is one GPU's share; --gpus above 1 is not supported.",
              file=sys.stderr)
        sys.exit(1)
    if args.profile_pass:
        profile_pass(args.profile_pass)
        return

    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    import ssm_recurrent_decode_gated_amd as S
    S.load_library()
    if args.replay_table:
        args.batch_sizes = args.batch_sizes or [1, 16, 64, 256]
        replay_table(dev, args)
        return
    if args.kda_table:
        kda_table(dev, args)
        return

    torch.cuda.synchronize()
    h = headline(dev, args.steps, args.warmup, args.settle)
    torch.cuda.synchronize()
    print(f"[bench] headline done: {h['us']:.1f} us/step (cold sample {h['cold_us']:.1f})", file=sys.stderr,
          flush=True)
    extra = {"eager_us_per_step": round(h["us"], 3),
             "cold_start_us_per_step": round(h["cold_us"], 3),
             "settle_steps_before_warmup": h["settle_steps"]}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(h["setup"])
        print("[bench] cpu_baseline done", file=sys.stderr, flush=True)
    del h["setup"]
    torch.cuda.empty_cache()
    if not args.no_extras:
        bsz = tuple(args.batch_sizes or (16, 64, 256))
        for key, leg in (("graph_sweep", sweep), ("copy_ceiling", copy_ceiling),
                         ("buffered", lambda d: buffered(d, batches=bsz, Ls=tuple(args.ls))),
                         ("kda_t64_h96", kda), ("gdn_conv_b256", gdn_conv), ("mamba1", mamba), ("mamba1_prefill", mamba_prefill), ("gdn_multi_token", gdn_multi), ("gdn_prefill", gdn_prefill),
                         ("state16_b256", state16)):
            extra[key] = leg(dev)
            print(f"[bench] {key} done", file=sys.stderr, flush=True)
        extra["state16_b256"]["speedup_vs_fp32_state"] = round(h["us"] / extra["state16_b256"]["us_per_step"], 3)
        extra["pct_of_copy_ceiling"] = round(100 * h["state_gbs"] / extra["copy_ceiling"]["GBps"], 2)
        extra["graph_replay_us_per_step_B256"] = extra["graph_sweep"]["B256"]["us_per_step"]
    w = h["w"]
    traffic = counters_traffic()
    trace_us = trace_kernel_avg_us()
    line = {
        "metric": METRIC,
        "value": round(h["state_gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["us"] / 1e3, 6),
        "us_per_step": round(h["us"], 3),
        "pct_hbm_peak": round(100 * h["state_gbs"] / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded randn, the pages' distributions)",
        "config": {"workload": w.name, "B": w.B, "num_slots": w.num_slots, "H": w.H, "HV": w.HV, "K": w.K,
                   "V": w.V, "act_dtype": w.act, "out_dtype": w.out, "state_dtype": "f32",
                   "state_pools_rotated": h["pools"], "parallelism": "single GPU"},
        "timing": ("eager launches, one gdn_decode_step per step over rotated state pools; HIP events around "
                   "the K timed steps after a settle period and W warm-up steps (extra.cold_start_us_per_step: "
                   "the same K steps straight after setup); graph replay of the same calls in "
                   "extra.graph_replay_us_per_step_B256"),
        "roofline": {"bound": "hbm", "achieved": round(h["alg_gbs"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(h["alg_gbs"] / HBM_PEAK_GBS, 4),
                     "kernel_avg_us_rocprofv3": trace_us,
                     "frac_at_rocprofv3_kernel_avg": None if trace_us is None else
                     round(h["alg_bytes"] / trace_us / 1e3 / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "algorithmic_bytes_per_launch": h["alg_bytes"], "kernel": KERNEL_NAME},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
