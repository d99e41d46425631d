"""Oracle for the per-tensor calibration statistics of an E4M3 KV cache
(test infrastructure only; see package docstring).

Page "[Model][SM70][FP8] Add calibrated E4M3 QSA KV cache" (section
"Implementation scope") reports, for every layer's K and V tensor, max-abs,
p99.9, p99.99 and saturation; its section "Why calibrated scale is part of
this contract" measures, at a given scale, the share of nonzero elements
below E4M3's minimum subnormal magnitude 2^-9 and the share in the
subnormal range [2^-9, 2^-6).  Page "Qwen3.8 Flash Next NVFP4 QSA FP8 E4M3
KV Scales" (section "Calibration") fixes the converter the statistics are
taken against: stored = e4m3fn(x / scale), scale = max envelope / 448.

Readings (the pages do not define these further):

* the element quotient is the converter's: y = fl32(x / scale), IEEE
  float32 division;
* NaN elements are counted apart and excluded from every other statistic;
* max-abs is max |x| over the remaining elements (infinities included);
* p99.9 / p99.99 are nearest-rank percentiles of |x| over the non-NaN
  elements, zeros included: the k-th smallest |x| with
  k = ceil(999 m / 1000) and ceil(9999 m / 10000) (exact integer
  arithmetic; m = number of non-NaN elements);
* saturated: non-NaN elements with |y| > 448 (the largest finite E4M3FN
  magnitude; infinities included);
* below_min_subnormal: nonzero elements with |y| < 2^-9;
* subnormal: nonzero elements with 2^-9 <= |y| < 2^-6;
* shares are counts over the nonzero (non-NaN) elements.

Everything here is a definition written out with numpy (a sort for the
percentiles, float32 division for the quotients, comparisons for the
counts).
"""

import numpy as np

from .formats import E4M3_MAX, E4M3_MIN_NORMAL, E4M3_MIN_SUBNORMAL, upcast_to_f32


def nearest_rank(m, num, den):
    """1-based rank ceil(num * m / den) in exact integer arithmetic."""
    return -((-num * m) // den)


def calib_stats(x, dtype, scale):
    """Statistics of one tensor ``x`` (any shape; fp16, fp32 or bf16 bit
    patterns as uint16) at the fp32 ``scale``.  Returns a dict of Python
    ints / floats (the float values are exact float32 values)."""
    a = upcast_to_f32(np.asarray(x).reshape(-1), dtype)
    nan = np.isnan(a)
    v = np.abs(a[~nan])
    m = int(v.size)
    out = {"count": int(a.size), "nan": int(nan.sum()), "finite_or_inf": m}
    if m == 0:
        out.update(max_abs=0.0, p999=0.0, p9999=0.0, nonzero=0, saturated=0,
                   below_min_subnormal=0, subnormal=0)
        return out
    srt = np.sort(v)
    out["max_abs"] = float(srt[-1])
    out["p999"] = float(srt[nearest_rank(m, 999, 1000) - 1])
    out["p9999"] = float(srt[nearest_rank(m, 9999, 10000) - 1])
    y = np.abs(a[~nan] / np.float32(scale))          # IEEE float32 quotient
    nz = v != 0
    out["nonzero"] = int(nz.sum())
    out["saturated"] = int((y > np.float32(E4M3_MAX)).sum())
    out["below_min_subnormal"] = int((nz & (y < np.float32(E4M3_MIN_SUBNORMAL))).sum())
    out["subnormal"] = int((nz & (y >= np.float32(E4M3_MIN_SUBNORMAL))
                            & (y < np.float32(E4M3_MIN_NORMAL))).sum())
    return out


def shares(stats):
    """The pages' fractions: saturated over all non-NaN elements; the two
    low-magnitude counts over the nonzero elements."""
    nz = max(stats["nonzero"], 1)
    m = max(stats["finite_or_inf"], 1)
    return {"saturation": stats["saturated"] / m,
            "below_min_subnormal": stats["below_min_subnormal"] / nz,
            "subnormal": stats["subnormal"] / nz}
