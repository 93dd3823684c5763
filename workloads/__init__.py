"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This module only draws random tensors with the shapes, dtypes and value
distributions of the pages' workloads; it holds none of the decode method's
arithmetic. Everything is generated on the CPU with torch's seeded generator
(deterministic for a given seed and tag), rounded once to the storage dtype,
and handed unchanged to both sides.

Distributions follow the pages' own synthetic set-ups:
  * GDN ("Microbenchmark: buffered output-only GDN decode (ReplaySSM Part A)
    vs. the existing packed GDN decode kernel", `_make_static`/`_bench_cfg`):
    mixed_qkv ~ N(0,1); a ~ N(0, 0.5^2); b ~ N(0,1); A_log ~ N(0, 0.3^2) fp32;
    dt_bias ~ N(0, 0.1^2) fp32; state ~ N(0,1) fp32.
  * KDA ("Microbenchmark for the fused Kimi-K3 KDA decode kernel on ROCm",
    `Inputs`): all tensors ~ N(0,1), norm weight ones, slots 1..T of T+8.
  * Mamba-1 ("Triton decode kernel + MBU analysis"): shapes of its microbench
    table; dt drawn positive, A drawn negative.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field, replace

import torch

DTYPES = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def generator(seed: int, *tags) -> torch.Generator:
    """A CPU generator whose seed is a hash of (seed, tags)."""
    key = repr((int(seed),) + tuple(tags)).encode()
    g = torch.Generator(device="cpu")
    g.manual_seed(int.from_bytes(hashlib.sha256(key).digest()[:7], "little"))
    return g


def normal(shape, std, dtype, gen) -> torch.Tensor:
    x = torch.randn(tuple(shape), generator=gen, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(DTYPES[dtype] if isinstance(dtype, str) else dtype)


def uniform(shape, lo, hi, gen) -> torch.Tensor:
    return torch.rand(tuple(shape), generator=gen, dtype=torch.float32) * (hi - lo) + lo


# ----------------------------------------------------------------- GDN
@dataclass(frozen=True)
class GDNWorkload:
    name: str
    B: int
    H: int
    HV: int
    K: int
    V: int
    num_slots: int
    act: str = "bf16"          # dtype of mixed_qkv, a, b (and the ring)
    out: str = "bf16"          # dtype of the output
    a_std: float = 0.5
    b_std: float = 1.0
    state_std: float = 1.0
    idx: str = "identity"      # "identity" | "perm" (seeded permutation subset)
    steps: int = 1
    Ls: tuple = field(default_factory=tuple)


GDN_TINY = GDNWorkload("gdn_tiny_b2_h2_d16_fp32", B=2, H=2, HV=2, K=16, V=16, num_slots=2,
                       act="f32", out="f32", a_std=1.0, state_std=0.1, steps=64)
GDN_B16 = GDNWorkload("gdn_b16_h16_hv32_d128", B=16, H=16, HV=32, K=128, V=128, num_slots=16)
GDN_B256 = GDNWorkload("gdn_b256_of264_h16_hv32_d128", B=256, H=16, HV=32, K=128, V=128,
                       num_slots=264, idx="perm")
GDN_B64_CHAIN = GDNWorkload("gdn_b64_h16_hv32_d128_chain1000", B=64, H=16, HV=32, K=128,
                            V=128, num_slots=64, steps=1000, Ls=(1, 8, 16))


def gdn_sweep(B: int) -> GDNWorkload:
    """The B=256 math at another batch size, pool = B + 8, permuted slots."""
    return replace(GDN_B256, name=f"gdn_b{B}_of{B + 8}_h16_hv32_d128", B=B, num_slots=B + 8)


def slot_indices(w, seed=0) -> torch.Tensor:
    if w.idx == "identity":
        return torch.arange(w.B, dtype=torch.int32)
    perm = torch.randperm(w.num_slots, generator=generator(seed, w.name, "idx"))
    return perm[: w.B].to(torch.int32).contiguous()


def gdn_params(w: GDNWorkload, seed=0) -> dict:
    """Per-layer parameters: A_log, dt_bias [HV] fp32."""
    g = generator(seed, w.name, "params")
    return {"A_log": normal((w.HV,), 0.3, "f32", g), "dt_bias": normal((w.HV,), 0.1, "f32", g)}


def gdn_state(w: GDNWorkload, seed=0, slots=None) -> torch.Tensor:
    """fp32 state pool [num_slots, HV, V, K]. Each slot draws from its own
    stream, so a subset of slots can be regenerated on its own."""
    slots = range(w.num_slots) if slots is None else slots
    out = torch.empty((len(slots), w.HV, w.V, w.K), dtype=torch.float32)
    for i, s in enumerate(slots):
        out[i] = normal((w.HV, w.V, w.K), w.state_std, "f32", generator(seed, w.name, "state", int(s)))
    return out


def gdn_step_inputs(w: GDNWorkload, step=0, seed=0, norm=False) -> dict:
    """Fresh per-step activations: mixed_qkv [B, 2HK + HV V], a, b [B, HV]
    (activation dtype); with norm=True also norm_gate [B, HV, V] and an fp32
    norm_weight [V]."""
    g = generator(seed, w.name, "step", step)
    d = {
        "qkv": normal((w.B, 2 * w.H * w.K + w.HV * w.V), 1.0, w.act, g),
        "a": normal((w.B, w.HV), w.a_std, w.act, g),
        "b": normal((w.B, w.HV), w.b_std, w.act, g),
    }
    if norm:
        d["norm_gate"] = normal((w.B, w.HV, w.V), 1.0, w.act, g)
        d["norm_weight"] = (1.0 + normal((w.V,), 0.1, "f32", g)).contiguous()
    return d


def gdn_ring(w: GDNWorkload, L: int, seed=0) -> dict:
    """Ring contents for a buffered call: d [num_slots, HV, L, V] and k
    [num_slots, H, L, K] in the activation dtype, g [num_slots, HV, L] fp32.
    d ~ N(0, 0.5^2), k ~ N(0, 1/K) (about unit norm), g ~ -U(0.05, 2)."""
    g = generator(seed, w.name, "ring", L)
    return {
        "d_cache": normal((w.num_slots, w.HV, L, w.V), 0.5, w.act, g),
        "k_cache": normal((w.num_slots, w.H, L, w.K), w.K ** -0.5, w.act, g),
        "g_cache": -uniform((w.num_slots, w.HV, L), 0.05, 2.0, g),
    }


def gdn_conv(w: GDNWorkload, W: int = 4, seed=0, layout="DS", bias=True) -> dict:
    """Conv parameters and state of the conv-fused GDN step, over the
    C = 2HK + HV V channels of mixed_qkv: conv_weight [C, W] ~ N(0, 1/W),
    conv_bias [C] ~ N(0, 0.1^2) fp32, and conv_state, a logical
    [num_slots, C, W-1] view (activation dtype, ~N(0, 1)) over the physical
    layout `layout` ("DS" = [slots, C, W-1], "SD" = [slots, W-1, C])."""
    g = generator(seed, w.name, "conv", W)
    C = 2 * w.H * w.K + w.HV * w.V
    cs = normal((w.num_slots, C, W - 1), 1.0, w.act, g)
    d = {
        "conv_weight": normal((C, W), W ** -0.5, "f32", g),
        "conv_bias": normal((C,), 0.1, "f32", g) if bias else None,
        "conv_state": cs.transpose(1, 2).contiguous().transpose(1, 2) if layout == "SD" else cs.contiguous(),
    }
    return d


# ----------------------------------------------------------------- KDA
@dataclass(frozen=True)
class KDAWorkload:
    name: str
    T: int
    H: int
    D: int = 128
    W: int = 4
    num_slots: int = 0
    layout: str = "SD"         # conv-state physical layout: SD = [slots, W-1, C], DS = [slots, C, W-1]
    lower_bound: float = -5.0
    norm_eps: float = 1e-5


KDA_T64 = KDAWorkload("kda_t64_h96_d128_w4", T=64, H=96, num_slots=72)


def kda_inputs(w: KDAWorkload, seed=0, layout=None) -> dict:
    """The fused KDA op's inputs. conv_state is returned as a logical
    [num_slots, C, W-1] view over the physical layout `layout`."""
    layout = layout or w.layout
    g = generator(seed, w.name, "kda")
    C = 3 * w.H * w.D
    d = {
        "x": normal((w.T, C), 1.0, "bf16", g),
        "conv_weight": normal((C, w.W), 1.0, "f32", g),
        "raw_g": normal((w.T, w.H, w.D), 1.0, "bf16", g),
        "raw_beta": normal((w.T, w.H), 1.0, "bf16", g),
        "gate": normal((w.T, w.H, w.D), 1.0, "bf16", g),
        "norm_weight": torch.ones(w.D, dtype=torch.float32),
        "idx": torch.arange(1, w.T + 1, dtype=torch.int32),
    }
    cs = normal((w.num_slots, C, w.W - 1), 1.0, "bf16", g)
    if layout == "SD":
        d["conv_state"] = cs.transpose(1, 2).contiguous().transpose(1, 2)
    else:
        d["conv_state"] = cs.contiguous()
    d["state"] = normal((w.num_slots, w.H, w.D, w.D), 1.0, "f32", g)
    return d


# ----------------------------------------------------------------- Mamba-1
@dataclass(frozen=True)
class MambaWorkload:
    name: str
    B: int
    Dm: int
    N: int
    num_slots: int


MAMBA_SMALL = MambaWorkload("mamba_b8_d1536_n16", B=8, Dm=1536, N=16, num_slots=8)


def mamba_inputs(w: MambaWorkload, seed=0, act="f32") -> dict:
    g = generator(seed, w.name, "mamba")
    return {
        "x": normal((w.B, w.Dm), 1.0, act, g),
        "dt": uniform((w.B, w.Dm), 0.001, 0.1, g).to(DTYPES[act]),
        "A": -uniform((w.Dm, w.N), 0.5, 16.0, g),
        "Bm": normal((w.B, w.N), 1.0, act, g),
        "Cm": normal((w.B, w.N), 1.0, act, g),
        "Dv": normal((w.Dm,), 1.0, "f32", g),
        "z": normal((w.B, w.Dm), 1.0, act, g),
        "h": normal((w.num_slots, w.Dm, w.N), 1.0, "f32", g),
        "idx": torch.arange(w.B, dtype=torch.int32),
    }


@dataclass(frozen=True)
class MambaScanWorkload:
    name: str
    B: int
    T: int
    Dm: int
    N: int
    num_slots: int


# the page's model width (d_inner 1536, N 16) over a 2048-token prompt
MAMBA_PREFILL = MambaScanWorkload("mamba_prefill_b1_t2048_d1536_n16", B=1, T=2048, Dm=1536, N=16, num_slots=1)


def mamba_scan_inputs(w: MambaScanWorkload, seed=0, act="bf16") -> dict:
    """Prefill inputs: the decode recipe with a token axis (x, dt, z [B, T, D],
    B, C [B, T, N]); slots are a seeded permutation of the pool's first B."""
    g = generator(seed, w.name, "mamba_scan")
    return {
        "x": normal((w.B, w.T, w.Dm), 1.0, act, g),
        "dt": uniform((w.B, w.T, w.Dm), 0.001, 0.1, g).to(DTYPES[act]),
        "A": -uniform((w.Dm, w.N), 0.5, 16.0, g),
        "Bm": normal((w.B, w.T, w.N), 1.0, act, g),
        "Cm": normal((w.B, w.T, w.N), 1.0, act, g),
        "Dv": normal((w.Dm,), 1.0, "f32", g),
        "z": normal((w.B, w.T, w.Dm), 1.0, act, g),
        "h": normal((w.num_slots, w.Dm, w.N), 1.0, "f32", g),
        "idx": torch.randperm(w.num_slots, generator=g)[: w.B].to(torch.int32).contiguous(),
    }
