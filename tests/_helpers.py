"""Comparison helpers for the parity tests (no decode arithmetic here).

Acceptance metric for floating point (fp32 kernels against the fp64 oracle):
    err = |x - ref| / max(|ref|, rms(ref over its row), 1e-30)
where a row is the last axis (a head's V outputs, or a state row of K
columns). A plain relative error fails spuriously near zero, and a plain
absolute error is meaningless across magnitudes; the row rms is the natural
scale of each element. A row of fewer than MIN_ROW values has no meaningful
rms (at V = 1 it is the element itself, so an output produced by cancellation
would be held to a relative bar no fp32 evaluation meets): its scale is the
rms over the last two axes, the batch row's heads.

Outputs stored in 16-bit types are the kernel's fp32 result rounded once,
to nearest even. A kernel within the fp32 bar computes some y with
|y - exact| <= tol * max(|exact|, rms), and RNE is monotone, so its stored
value must lie between RNE(exact - tol*s) and RNE(exact + tol*s): it equals
RNE(exact) except where a rounding midpoint lies within the fp32 bar of the
exact value, where the other neighbour is a correct rounding too. A
truncating or one-ulp-off store fails this.
"""
from __future__ import annotations

import numpy as np
import torch

FP32_TOL = 1e-4        # single step, fp32 outputs and states
CHAIN_TOL = 2e-3       # after up to 1000 chained steps


def to_np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().double().numpy()


MIN_ROW = 8  # rows shorter than this take their scale over the last two axes


def row_rms(ref: np.ndarray) -> np.ndarray:
    """rms of ref over its row (the last axis), or over the last two axes
    where a row holds fewer than MIN_ROW values; broadcastable to ref."""
    ref = np.asarray(ref, dtype=np.float64)
    axes = (-2, -1) if ref.ndim >= 2 and ref.shape[-1] < MIN_ROW else -1
    return np.sqrt(np.mean(ref * ref, axis=axes, keepdims=True))


def mixed_err(x: np.ndarray, ref: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = row_rms(ref)
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


def rne16(x, mant_bits: int) -> np.ndarray:
    """Round-to-nearest-even of fp64 values to bf16 (7 mantissa bits) or f16
    (10), straight from fp64 (one rounding): subnormals at the format's fixed
    spacing, values past the largest finite one + half an ulp to +-inf."""
    x = np.asarray(x, dtype=np.float64)
    emin, emax = (-14, 15) if mant_bits == 10 else (-126, 127)
    _, e = np.frexp(x)
    lead = np.maximum(e - 1, emin)
    ulp = np.ldexp(1.0, lead - mant_bits)
    r = np.rint(x / ulp) * ulp  # numpy's rint rounds halves to even
    maxv = np.ldexp(2.0 - 2.0 ** -mant_bits, emax)
    r = np.where(np.abs(r) > maxv, np.copysign(np.inf, x), r)
    return np.where((x == 0) | ~np.isfinite(x), x, r)


def assert_out16(x: torch.Tensor, exact, tol=FP32_TOL, what=""):
    """16-bit outputs against the oracle's exact values: RNE of the exact
    value, or its neighbour only where a rounding midpoint lies within the
    fp32 bar `tol` (of max(|exact|, row rms)) of the exact value."""
    mant = {torch.bfloat16: 7, torch.float16: 10}[x.dtype]
    xv = to_np64(x).reshape(np.shape(exact))
    ex = np.asarray(exact, dtype=np.float64)
    assert np.isfinite(ex).all(), f"{what}: reference not finite"
    band = tol * np.maximum(np.abs(ex), row_rms(ex))
    lo, hi = rne16(ex - band, mant), rne16(ex + band, mant)
    bad = (xv < lo) | (xv > hi) | ~np.isfinite(xv)
    if bad.any():
        i = tuple(int(v) for v in np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} 16-bit outputs are not a rounding to "
                             f"nearest of a value within {tol:.0e} of the exact one; first at {i}: got "
                             f"{xv[i]!r}, RNE(exact) {rne16(ex[i], mant)!r}, exact {ex[i]!r}")


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
    scale = np.maximum(np.abs(exact), row_rms(exact))
    assert (diff <= ulp16(ref, mant_bits) * 1.0000001 + MIDPOINT_REL * scale).all(), \
        f"{what}: stored value off by more than one ulp"
    flip = diff != 0
    off_mid = np.abs(exact - 0.5 * (got + ref)) > MIDPOINT_REL * scale
    assert not (flip & off_mid).any(), \
        f"{what}: {(flip & off_mid).sum()} record(s) differ where the exact value is not at a midpoint"


def take_valid_roundings(got, ref, exact, mant_bits, what):
    """Chained runs that store 16-bit values (ring records, 16-bit state
    rows). Where a value's exact counterpart sits at a rounding midpoint, the
    kernel and the oracle may store different neighbours; both are correct
    roundings, but each trajectory then carries its own value forward and the
    two drift apart by up to one 16-bit ulp of that term. So after each step
    the kernel's stored values are checked against the oracle's rounding
    (assert_rounded16: equal, or the other neighbour where the exact value is
    at a midpoint), and the oracle continues from its own values with the
    kernel's choice taken at exactly those midpoints: it picks, between its
    own two candidate roundings, the one the kernel picked. Nothing the check
    rejects is ever taken. Returns (values for the oracle's next step, number
    of midpoint choices taken)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    exact = np.asarray(exact, dtype=np.float64)
    assert got.shape == ref.shape == exact.shape, (what, got.shape, ref.shape, exact.shape)
    flip = got != ref
    if not flip.any():
        return ref.copy(), 0
    rows = flip.any(axis=-1)  # the check needs each differing value's whole row (its rms)
    assert_rounded16(got[rows], ref[rows], what, exact[rows], mant_bits)
    return np.where(flip, got, ref), int(flip.sum())
