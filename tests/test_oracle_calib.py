"""Pins of the calibration-statistics oracle against definitions it does not
share code with: exact rational ranks, numpy's textbook nearest-rank
quantile, pure-Python brute force with struct-rounded float32 quotients,
closed forms and the E4M3 thresholds.  No GPU."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import brute
from oracle import calib
from oracle import formats as ofmt


def test_nearest_rank_is_the_smallest_rank_reaching_the_fraction():
    for m in list(range(1, 2500)) + [9999, 10000, 10001, 123457, 2 ** 31 + 3]:
        for num, den in ((999, 1000), (9999, 10000)):
            k = calib.nearest_rank(m, num, den)
            assert Fraction(k, m) >= Fraction(num, den)
            assert k == 1 or Fraction(k - 1, m) < Fraction(num, den)


def test_percentiles_match_numpy_inverted_cdf():
    rng = np.random.default_rng(3)
    for m in (1, 7, 999, 1000, 1001, 20000, 54321):
        x = (rng.standard_t(4, size=m) * 0.5).astype(np.float32)
        st = calib.calib_stats(x, "fp32", 1.0)
        a = np.abs(x.astype(np.float64))
        assert st["p999"] == np.quantile(a, 0.999, method="inverted_cdf")
        assert st["p9999"] == np.quantile(a, 0.9999, method="inverted_cdf")
        assert st["max_abs"] == a.max()


def _brute(xs, scale):
    """Pure Python: sorted list, exact ranks, struct-rounded quotients."""
    vals = [v for v in xs if v == v]
    m = len(vals)
    s = sorted(abs(v) for v in vals)
    k1 = -((-999 * m) // 1000)
    k2 = -((-9999 * m) // 10000)
    sat = below = sub = nz = 0
    for v in vals:
        y = abs(brute.f32(v / scale)) if abs(v) != float("inf") else float("inf")
        if v != 0:
            nz += 1
            if y < 2.0 ** -9:
                below += 1
            elif y < 2.0 ** -6:
                sub += 1
        if y > 448.0:
            sat += 1
    return {"max_abs": s[-1], "p999": s[k1 - 1], "p9999": s[k2 - 1], "nonzero": nz,
            "saturated": sat, "below_min_subnormal": below, "subnormal": sub,
            "nan": len(xs) - m}


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_vs_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = 3001
    scale = float(np.float32(rng.uniform(0.01, 0.2)))
    x = (rng.standard_t(4, size=n) * 0.5).astype(np.float32)
    # magnitudes around every threshold of the quotient
    for i, t in enumerate([448.0, 2.0 ** -9, 2.0 ** -6]):
        for j, f in enumerate([0.999999, 1.0, 1.000001, 0.5, 2.0]):
            x[40 * i + j] = np.float32(t * scale * f) * (1 if j % 2 else -1)
    x[200:230] = 0.0
    x[230] = np.nan
    x[231] = np.inf
    x[232] = -np.inf
    st = calib.calib_stats(x, "fp32", scale)
    br = _brute([float(v) for v in x], scale)
    for k, v in br.items():
        assert st[k] == v, k


def test_closed_forms():
    x = np.arange(1, 10001, dtype=np.float32)
    st = calib.calib_stats(x, "fp32", float(np.float32(10000.0 / 448.0)))
    assert (st["max_abs"], st["p999"], st["p9999"]) == (10000.0, 9990.0, 9999.0)
    assert st["nonzero"] == 10000 and st["nan"] == 0
    # scale = 1: everything above 448 saturates, nothing is small
    st1 = calib.calib_stats(x, "fp32", 1.0)
    assert st1["saturated"] == 10000 - 448
    assert st1["below_min_subnormal"] == 0 and st1["subnormal"] == 0
    # all zeros: no nonzero elements, percentiles 0
    z = calib.calib_stats(np.zeros(100, np.float32), "fp32", 1.0)
    assert z["nonzero"] == 0 and z["max_abs"] == 0.0 and z["p9999"] == 0.0


def test_thresholds_are_strict_where_the_format_says():
    s = 1.0
    x = np.array([448.0, np.nextafter(np.float32(448.0), np.float32(1e9)),
                  2.0 ** -9, np.nextafter(np.float32(2.0 ** -9), np.float32(0)),
                  2.0 ** -6, np.nextafter(np.float32(2.0 ** -6), np.float32(0))], np.float32)
    st = calib.calib_stats(x, "fp32", s)
    assert st["saturated"] == 1                    # 448 itself is finite E4M3
    assert st["below_min_subnormal"] == 1          # just below 2^-9
    assert st["subnormal"] == 2                    # 2^-9 and just below 2^-6


def test_source_dtypes_agree_on_representable_values():
    rng = np.random.default_rng(9)
    v = rng.standard_normal(4000).astype(np.float16).astype(np.float32)
    v = ofmt.bf16_bits_to_f32(ofmt.f32_to_bf16_bits(v))   # representable in all three
    v = v[np.isfinite(v)]
    bits = ofmt.f32_to_bf16_bits(v)
    keep = v.astype(np.float16).astype(np.float32) == v
    v, bits = v[keep], bits[keep]
    a = calib.calib_stats(v, "fp32", 0.02)
    b = calib.calib_stats(v.astype(np.float16), "fp16", 0.02)
    c = calib.calib_stats(bits, "bf16", 0.02)
    assert a == b == c


def test_shares():
    st = {"finite_or_inf": 10, "nonzero": 8, "saturated": 1, "below_min_subnormal": 2,
          "subnormal": 4}
    assert calib.shares(st) == {"saturation": 0.1, "below_min_subnormal": 0.25,
                                "subnormal": 0.5}
