"""CPU checks of the comparison criteria themselves (no GPU): a criterion
that a plausible kernel mistake passes proves nothing, so each one is run
against correct and planted-wrong values built here from first principles."""
import numpy as np
import pytest
import torch

from tests._helpers import assert_rounded16, ulp16


def _bf16_rne(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).double().numpy()


def _bf16_trunc(x):
    u = np.asarray(x, np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    return u.view(np.float32).astype(np.float64)


def _records(seed=0):
    # 64 records of 256 values, exact values in fp64
    return np.random.default_rng(seed).standard_normal((64, 256))


def test_ring16_accepts_the_correct_rounding():
    ex = _records()
    ref = _bf16_rne(ex)
    assert_rounded16(ref, ref, "identical", ex)


def test_ring16_accepts_the_other_neighbour_at_a_midpoint():
    # exact values placed at bf16 rounding midpoints (plus fp32-sized noise):
    # either neighbour is a correct rounding of what an fp32 kernel computes
    lo = _bf16_rne(_records(1))
    ulp = 2.0 ** (np.floor(np.log2(np.abs(lo))) - 7)
    ex = lo + 0.5 * ulp * np.sign(lo) * (1 + 1e-7)
    ref = _bf16_rne(ex)
    other = np.where(ref == lo, lo + ulp * np.sign(lo), lo)
    assert_rounded16(other, ref, "midpoints", ex)


def test_ring16_rejects_truncation():
    ex = _records(2)
    with pytest.raises(AssertionError):
        assert_rounded16(_bf16_trunc(ex), _bf16_rne(ex), "truncated", ex)


def test_ring16_rejects_a_two_ulp_error():
    ex = _records(3)
    ref = _bf16_rne(ex)
    bad = ref.copy()
    bad[5, 7] += 2 * 2.0 ** (np.floor(np.log2(abs(ref[5, 7]))) - 7)
    with pytest.raises(AssertionError):
        assert_rounded16(bad, ref, "two ulp", ex)


def test_ulp16_spacing_including_subnormals():
    """The 16-bit spacings the checks allow, against the formats' own
    neighbours (torch's conversions): normal range and f16 subnormals."""
    def rnd(v, dt):
        return float(torch.tensor([v], dtype=torch.float64).to(dt).double().item())

    for x, mant, dt in ((1.0, 7, torch.bfloat16), (0.3, 7, torch.bfloat16), (1.0, 10, torch.float16),
                        (0.3, 10, torch.float16), (4.9e-6, 10, torch.float16), (2.0 ** -20, 10, torch.float16)):
        v = rnd(x, dt)  # a representable value
        u = float(ulp16(np.array([v]), mant)[0])
        assert rnd(v + u, dt) == v + u, (x, mant)  # one spacing up is the next representable value
        assert rnd(v + 0.49 * u, dt) == v, (x, mant)  # under half a spacing rounds back


def test_ring16_f16_subnormal_neighbour_accepted():
    """A tiny f16 record (subnormal) one spacing from the oracle's rounding,
    with its exact value at the midpoint: accepted."""
    ex = np.array([[1.0, -0.5, 4.9e-6 + 2.0 ** -25 * 1.0000001, 0.25]])
    ref = torch.from_numpy(ex).to(torch.float16).double().numpy()
    got = ref.copy()
    got[0, 2] = ref[0, 2] + 2.0 ** -24 if ref[0, 2] < ex[0, 2] else ref[0, 2] - 2.0 ** -24
    assert_rounded16(got, ref, "f16 subnormal", ex, 10)
