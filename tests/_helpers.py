"""Comparison helpers for the parity tests (no decode arithmetic here).

Acceptance metric for floating point (fp32 kernels against the fp64 oracle):
    err = |x - ref| / max(|ref|, rms(ref over its row), 1e-30)
where a row is the last axis (a head's V outputs, or a state row of K
columns). A plain relative error fails spuriously near zero, and a plain
absolute error is meaningless across magnitudes; the row rms is the natural
scale of each element.

Outputs stored in 16-bit types are checked against the exact value: the
kernel's fp32 result rounded once (RNE) lies within half a unit in the last
place of the exact value plus the fp32 error, so
    |x - ref| <= ulp(ref) + tol * max(|ref|, rms)
holds for a correct kernel and fails for any error of one 16-bit ulp or more
beyond rounding.
"""
from __future__ import annotations

import numpy as np
import torch

FP32_TOL = 1e-4        # single step, fp32 outputs and states
CHAIN_TOL = 2e-3       # after up to 1000 chained steps


def to_np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().double().numpy()


def mixed_err(x: np.ndarray, ref: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    den = np.maximum(np.maximum(np.abs(ref), rms), 1e-30)
    return np.abs(x - ref) / den


def assert_mixed(x, ref, tol, what=""):
    x = to_np64(x) if isinstance(x, torch.Tensor) else np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (what, x.shape, ref.shape)
    assert np.isfinite(ref).all(), f"{what}: reference not finite"
    err = mixed_err(x, ref)
    worst = np.unravel_index(int(np.argmax(err)), err.shape)
    assert err.max() <= tol, (f"{what}: max err {err.max():.3e} > {tol:.1e} at {worst}: "
                              f"got {x[worst]!r}, want {ref[worst]!r}")
    return float(err.max())


def ulp16(ref: np.ndarray, mant_bits: int) -> np.ndarray:
    """Spacing of a 16-bit float format at |ref|: bf16 (7 mantissa bits) or
    f16 (10). Below the format's smallest normal (2^-126 bf16, 2^-14 f16) the
    spacing stays that of the smallest normal binade (subnormals)."""
    a = np.maximum(np.abs(ref), 1e-30)
    emin = -14 if mant_bits == 10 else -126
    return np.exp2(np.maximum(np.floor(np.log2(a)), emin) - mant_bits)


def assert_16bit(x: torch.Tensor, ref, tol=FP32_TOL, what=""):
    mant = {torch.bfloat16: 7, torch.float16: 10}[x.dtype]
    xv = to_np64(x).reshape(np.shape(ref))
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    bound = ulp16(ref, mant) + tol * np.maximum(np.abs(ref), rms)
    bad = np.abs(xv - ref) > bound
    if bad.any():
        i = np.argwhere(bad)[0]
        i = tuple(int(v) for v in i)
        raise AssertionError(f"{what}: {int(bad.sum())} elements off by more than one ulp, first at {i}: "
                             f"got {xv[i]!r}, want {ref[i]!r}")


def need_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


MIDPOINT_REL = 2.0 ** -16  # far above fp32 rounding error, far below half a 16-bit ulp (2^-9 bf16, 2^-12 f16)


def assert_rounded16(got, ref, what, exact, mant_bits=7):
    """A stored 16-bit value (a ring record, a 16-bit state row) may differ
    from the oracle's rounding by one ulp
    only where the exact (unrounded) value sits at the rounding midpoint
    between the two neighbours, to within fp32 arithmetic error (2^-16 of
    max(|value|, rms of its record)): there both neighbours are correct
    roundings of what an fp32 kernel computes. Elements that share a mantissa
    flip together, so no count of flips is imposed."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    exact = np.asarray(exact, dtype=np.float64)
    diff = np.abs(got - ref)
    # fp32 error is measured against the record's scale, as in the fp32 parity
    # metric: delta = beta (v - S k) can cancel, so its error tracks the row, not itself
    scale = np.maximum(np.abs(exact), np.sqrt(np.mean(exact * exact, axis=-1, keepdims=True)))
    assert (diff <= ulp16(ref, mant_bits) * 1.0000001 + MIDPOINT_REL * scale).all(), \
        f"{what}: stored value off by more than one ulp"
    flip = diff != 0
    off_mid = np.abs(exact - 0.5 * (got + ref)) > MIDPOINT_REL * scale
    assert not (flip & off_mid).any(), \
        f"{what}: {(flip & off_mid).sum()} record(s) differ where the exact value is not at a midpoint"
