"""Pins of the parity rule (oracle/compare.py), CPU only.

The rule every float parity test uses: |y - y_ref| <= 1e-3 * max(|y_ref|, tau)
+ ulp_out(y_ref) / 2 with tau = 1e-3 * rms(y_ref). ``ulp`` is pinned to
hand-worked spacings of the IEEE binary16, bfloat16 and binary32 formats
(p-bit significand: spacing 2**(e - p + 1) in the binade [2**e, 2**(e+1)),
the subnormal quantum 2**(MIN_EXP - p + 1) at zero and below the normal
range) and to numpy's own ``spacing`` for the two IEEE formats; ``compare`` is
pinned to rows worked out by hand on both sides of the bound.
"""
import numpy as np
import pytest

from oracle import compare

F16_ROWS = [  # (value, spacing) worked from p = 11, MIN_EXP = -14
    (0.0, 2.0 ** -24), (2.0 ** -24, 2.0 ** -24), (2.0 ** -20, 2.0 ** -24), (2.0 ** -14, 2.0 ** -24),
    (2.0 ** -14 * 1.5, 2.0 ** -24), (2.0 ** -13, 2.0 ** -23), (0.999, 2.0 ** -11), (1.0, 2.0 ** -10),
    (1.5, 2.0 ** -10), (2.0, 2.0 ** -9), (-3.0, 2.0 ** -9), (2048.0, 2.0), (65504.0, 32.0)]
BF16_ROWS = [  # p = 8, MIN_EXP = -126
    (0.0, 2.0 ** -133), (2.0 ** -130, 2.0 ** -133), (2.0 ** -126, 2.0 ** -133), (1.0, 2.0 ** -7),
    (-1.0, 2.0 ** -7), (0.75, 2.0 ** -8), (255.0, 1.0), (256.0, 2.0), (3.0e38, 2.0 ** 120)]
F32_ROWS = [  # p = 24, MIN_EXP = -126
    (0.0, 2.0 ** -149), (2.0 ** -140, 2.0 ** -149), (2.0 ** -126, 2.0 ** -149), (1.0, 2.0 ** -23),
    (0.5, 2.0 ** -24), (-7.0, 2.0 ** -21), (16777216.0, 2.0)]


@pytest.mark.parametrize("dtype,rows", [("f16", F16_ROWS), ("bf16", BF16_ROWS), ("f32", F32_ROWS)])
def test_ulp_hand_worked_spacings(dtype, rows):
    v = np.array([r[0] for r in rows])
    want = np.array([r[1] for r in rows])
    np.testing.assert_array_equal(compare.ulp(v, dtype), want)


@pytest.mark.parametrize("dtype,np_t", [("f16", np.float16), ("f32", np.float32)])
def test_ulp_matches_numpy_spacing_for_ieee_formats(dtype, np_t):
    """At every representable non-negative value of a sample (zero, subnormals, binade
    edges, random normals) the spacing equals numpy's spacing toward +inf."""
    rng = np.random.default_rng(11)
    info = np.finfo(np_t)
    vals = np.concatenate([
        [0.0, float(info.smallest_subnormal), float(info.smallest_normal), 1.0, 2.0, 0.5],
        2.0 ** np.arange(-20, 14).astype(np.float64),
        np.abs(rng.standard_normal(500)) * 100.0,
        np.abs(rng.standard_normal(200)) * float(info.smallest_normal) * 4.0,
    ]).astype(np_t)
    vals = vals[np.isfinite(vals)]
    want = np.spacing(vals).astype(np.float64)
    np.testing.assert_array_equal(compare.ulp(vals.astype(np.float64), dtype), want)


def test_ulp_is_even_in_sign():
    v = np.array([1e-3, 0.7, 3.0, 1234.5])
    for d in ("f16", "bf16", "f32"):
        np.testing.assert_array_equal(compare.ulp(v, d), compare.ulp(-v, d))


def test_compare_zero_reference_takes_the_subnormal_quantum():
    # y_ref all zero: rms = 0, tau = 0, bound = ulp_f16(0) / 2 = 2**-25.
    assert not compare.compare([2e-4, 0.0], [0.0, 0.0], "f16")["ok"]
    assert not compare.compare([2.0 ** -24, 0.0], [0.0, 0.0], "f16")["ok"]
    assert compare.compare([2.0 ** -25, 0.0], [0.0, 0.0], "f16")["ok"]
    assert compare.compare([0.0, 0.0], [0.0, 0.0], "bf16")["ok"]


def test_compare_at_the_bound_one_reference():
    # y_ref = [1]: rms = 1, tau = 1e-3; bound = 1e-3 * 1 + ulp_f16(1) / 2 = 0.001 + 2**-11.
    bound = 1e-3 + 2.0 ** -11
    assert compare.compare([1.0 + 0.999 * bound], [1.0], "f16")["ok"]
    assert compare.compare([1.0 - 0.999 * bound], [1.0], "f16")["ok"]
    assert not compare.compare([1.0 + 1.001 * bound], [1.0], "f16")["ok"]
    assert not compare.compare([-1.0 - 1.001 * bound], [-1.0], "f16")["ok"]
    # bf16: ulp(1) = 2**-7, bound 1e-3 + 2**-8
    b16 = 1e-3 + 2.0 ** -8
    assert compare.compare([1.0 + 0.999 * b16], [1.0], "bf16")["ok"]
    assert not compare.compare([1.0 + 1.001 * b16], [1.0], "bf16")["ok"]


def test_compare_cancellation_floor():
    # y_ref = [1, 0]: rms = sqrt(1/2), tau = 1e-3 * sqrt(1/2). At the zero entry the
    # bound is 1e-3 * tau + 2**-25 (f16) = 7.0711e-7 + 2.98e-8 = 7.369e-7.
    tau = 1e-3 * np.sqrt(0.5)
    b0 = 1e-3 * tau + 2.0 ** -25
    assert compare.compare([1.0, 0.99 * b0], [1.0, 0.0], "f16")["ok"]
    assert not compare.compare([1.0, 1.01 * b0], [1.0, 0.0], "f16")["ok"]
    # an entry much smaller than tau is held to the floor, not to its own magnitude
    tiny = 1e-9
    floor = 1e-3 * tau + 0.5 * float(compare.ulp(tiny, "f32"))
    assert compare.compare([1.0, tiny + 0.5 * floor], [1.0, tiny], "f32")["ok"]
    assert not compare.compare([1.0, tiny + 1.01 * floor], [1.0, tiny], "f32")["ok"]


def test_compare_rejects_non_finite_and_shape_mismatch():
    assert not compare.compare([np.nan], [1.0], "f32")["ok"]
    assert not compare.compare([np.inf], [1.0], "f32")["ok"]
    with pytest.raises(ValueError):
        compare.compare([1.0, 2.0], [1.0], "f32")


def test_compare_reports_worst_ratio():
    # error exactly half the bound -> worst_ratio 0.5
    bound = 1e-3 * 4.0 + 0.5 * compare.ulp(4.0, "f32")
    r = compare.compare([4.0 + 0.5 * bound], [4.0], "f32")
    assert r["ok"] and abs(r["worst_ratio"] - 0.5) < 1e-9


def test_compare_fp32_accumulation_term():
    # y_ref = [1, 0]: at the zero entry the bound is 1e-3 * tau + 2**-25 (f16) without
    # the term; with abs_sum = 100 and K = 4096 it gains sqrt(4096) * 2**-24 * 100.
    tau = 1e-3 * np.sqrt(0.5)
    b0 = 1e-3 * tau + 2.0 ** -25
    extra = 64.0 * 2.0 ** -24 * 100.0
    y_ref = [1.0, 0.0]
    assert not compare.compare([1.0, 1.5 * b0], y_ref, "f16")["ok"]
    assert compare.compare([1.0, 0.99 * (b0 + extra)], y_ref, "f16", abs_sum=[1.0, 100.0], k=4096)["ok"]
    assert not compare.compare([1.0, 1.01 * (b0 + extra)], y_ref, "f16", abs_sum=[1.0, 100.0], k=4096)["ok"]
    # the term scales with sqrt(K) and with abs_sum, entry by entry
    assert not compare.compare([1.0, 0.99 * (b0 + extra)], y_ref, "f16", abs_sum=[1.0, 100.0], k=1024)["ok"]
    assert not compare.compare([1.0, 0.99 * (b0 + extra)], y_ref, "f16", abs_sum=[100.0, 1.0], k=4096)["ok"]
    with pytest.raises(ValueError):
        compare.compare([1.0], [1.0], "f16", abs_sum=[1.0, 2.0], k=4)
