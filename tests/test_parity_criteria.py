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


# ------------------------------------------------ 16-bit outputs (assert_out16)
def test_rne16_matches_library_conversions():
    """The test-side RNE against torch's float32 -> bf16 / f16 conversions
    (each a single rounding): normal values, exact ties, tiny and subnormal
    values, overflow."""
    from tests._helpers import rne16
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-8, 5, 20000),
        (rng.integers(0, 1 << 16, 4000).astype(np.uint32) << 16 | 0x8000).view(np.float32),  # bf16 ties
        [0.0, -0.0, 65504.0, 65519.0, 65520.0, 1e5, 6.0e-8, 3.0e-8, 2.0 ** -25, 3.4e38],
    ]).astype(np.float32)
    x = x[np.isfinite(x)]
    t = torch.from_numpy(x)
    np.testing.assert_array_equal(rne16(x.astype(np.float64), 7), t.to(torch.bfloat16).double().numpy())
    np.testing.assert_array_equal(rne16(x.astype(np.float64), 10), t.to(torch.float16).double().numpy())


def _out16_case(seed=0, dtype=torch.bfloat16):
    ex = np.random.default_rng(seed).standard_normal((32, 128))
    return ex, torch.from_numpy(ex).to(torch.float32).to(dtype)  # fp64 -> fp32 (exact to 1e-8) -> RNE


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_out16_accepts_a_correct_rounding(dtype):
    from tests._helpers import assert_out16
    ex, got = _out16_case(0, dtype)
    assert_out16(got, ex, 1e-4, "rne")


def test_out16_accepts_the_other_neighbour_only_near_a_midpoint():
    from tests._helpers import assert_out16, rne16
    lo = rne16(np.random.default_rng(1).standard_normal((16, 64)), 7)
    ulp = np.ldexp(1.0, np.frexp(np.abs(lo))[1] - 1 - 7)
    up = lo + ulp * np.sign(lo)
    near = 0.5 * (lo + up) + 1e-7 * np.sign(lo) * np.abs(lo)  # just past the midpoint: RNE gives `up`
    assert_out16(torch.from_numpy(lo).to(torch.bfloat16), near, 1e-4, "other neighbour at a midpoint")
    far = lo + 0.8 * (up - lo)  # well past the midpoint: only `up` is a correct rounding
    with pytest.raises(AssertionError):
        assert_out16(torch.from_numpy(lo).to(torch.bfloat16), far, 1e-4, "one ulp off")


def test_out16_rejects_truncation():
    from tests._helpers import assert_out16
    ex, _ = _out16_case(2)
    with pytest.raises(AssertionError):
        assert_out16(torch.from_numpy(_bf16_trunc(ex)).to(torch.bfloat16), ex, 1e-4, "truncated")


def test_out16_rejects_an_error_above_the_fp32_bar():
    from tests._helpers import assert_out16
    ex, _ = _out16_case(3)
    bad = ex * (1 + 3e-3)  # a kernel 3e-3 off, rounded correctly
    with pytest.raises(AssertionError):
        assert_out16(torch.from_numpy(bad).to(torch.float32).to(torch.bfloat16), ex, 1e-4, "3e-3 off")


def test_short_rows_take_their_scale_over_the_heads():
    """A one-value row (V = 1) is scaled by the rms over the batch row's
    heads, not by itself: an output that cancellation made small keeps the
    absolute fp32 bar of its neighbours, while a wrong value still fails."""
    from tests._helpers import MIN_ROW, assert_mixed, mixed_err, row_rms
    ref = np.random.default_rng(3).standard_normal((4, 12, 1))
    ref[1, 1, 0] = 1.6e-6  # a cancellation-sized output among normal ones
    scale = row_rms(ref)[1, 0, 0]
    x = ref.copy()
    x[1, 1, 0] += 0.5e-4 * scale  # within the bar of the heads' scale
    assert_mixed(x, ref, 1e-4, "short row, fp32-sized error")
    x[1, 1, 0] = ref[1, 1, 0] + 3e-4 * scale
    with pytest.raises(AssertionError):
        assert_mixed(x, ref, 1e-4, "short row, wrong value")
    # rows of MIN_ROW values or more keep their own rms
    wide = np.random.default_rng(4).standard_normal((2, 3, MIN_ROW))
    np.testing.assert_allclose(row_rms(wide), np.sqrt(np.mean(wide * wide, axis=-1, keepdims=True)))
    assert mixed_err(wide, wide).max() == 0.0
