"""Pins of the top-k selection oracle against definitions it does not share
code with: a pure-Python rank count (candidate i is listed iff fewer than k
candidates beat it), numpy's argpartition on distinct scores, closed forms,
and the IEEE special values.  No GPU."""

import math
import random

import numpy as np
import pytest

from oracle import formats as ofmt
from oracle import topk as otopk


def _beats(vj, j, vi, i):
    """Candidate j ranks ahead of candidate i: numbers ahead of NaN, larger
    numbers ahead, equal scores (or two NaN) by lower position."""
    nj, ni = math.isnan(vj), math.isnan(vi)
    if nj != ni:
        return ni
    if not nj and vj != vi:
        return vj > vi
    return j < i


def _rank_select(vals, k):
    n = len(vals)
    sel = [i for i in range(n)
           if sum(1 for j in range(n) if j != i and _beats(vals[j], j, vals[i], i)) < k]
    return sel + [-1] * (k - len(sel))


@pytest.mark.parametrize("seed", range(6))
def test_vs_rank_count_with_ties_and_specials(seed):
    rnd = random.Random(seed)
    pool = [0.0, -0.0, 1.0, -1.0, 0.5, 2.0, float("inf"), float("-inf"), float("nan"), 3.0]
    R, stride = 7, 40
    s = np.array([[rnd.choice(pool) for _ in range(stride)] for _ in range(R)], np.float32)
    row_len = [0, 1, 5, 17, 33, 40, 39]
    for k in (1, 3, 16, 40):
        got = otopk.topk_select(s, "fp32", row_len, k)
        for r in range(R):
            want = _rank_select([float(x) for x in s[r, :row_len[r]]], k)
            assert got[r].tolist() == want, (seed, r, k)


def test_distinct_scores_match_argpartition():
    rng = np.random.default_rng(1)
    s = rng.standard_normal((5, 3000)).astype(np.float32)
    lens = [3000, 2999, 1500, 1025, 777]
    got = otopk.topk_select(s, "fp32", lens, 1024)
    for r in range(5):
        n = lens[r]
        if n <= 1024:
            want = np.arange(n)
        else:
            want = np.sort(np.argpartition(-s[r, :n].astype(np.float64), 1023)[:1024])
        assert got[r, :len(want)].tolist() == want.tolist()
        assert (got[r, len(want):] == -1).all()


def test_closed_forms():
    n, k = 1000, 100
    inc = np.arange(n, dtype=np.float32)[None, :]
    assert otopk.topk_select(inc, "fp32", [n], k)[0].tolist() == list(range(n - k, n))
    assert otopk.topk_select(-inc, "fp32", [n], k)[0].tolist() == list(range(k))
    const = np.full((1, n), 7.0, np.float32)
    assert otopk.topk_select(const, "fp32", [n], k)[0].tolist() == list(range(k))
    # fewer candidates than k: all of them, then padding; lengths clamp
    out = otopk.topk_select(np.zeros((3, 10), np.float32), "fp32", [4, -3, 99], 8)
    assert out[0].tolist() == [0, 1, 2, 3, -1, -1, -1, -1]
    assert out[1].tolist() == [-1] * 8
    assert out[2].tolist() == list(range(8))


def test_signed_zero_ties_and_nan_order():
    s = np.array([[-0.0, 0.0, -0.0, np.nan, -np.inf, np.nan]], np.float32)
    # numbers first (the three zeros tie, lowest positions first), then -inf, then NaN
    assert otopk.topk_select(s, "fp32", [6], 2)[0].tolist() == [0, 1]
    assert otopk.topk_select(s, "fp32", [6], 4)[0].tolist() == [0, 1, 2, 4]
    assert otopk.topk_select(s, "fp32", [6], 5)[0].tolist() == [0, 1, 2, 3, 4]
    # -0 does not rank below +0: ordered by bit pattern, position 2 would win
    z = np.array([[-0.0, -0.0, 0.0]], np.float32)
    assert otopk.topk_select(z, "fp32", [3], 2)[0].tolist() == [0, 1]


def test_source_dtypes_agree_on_representable_values():
    rng = np.random.default_rng(5)
    v = (rng.integers(-64, 64, size=(4, 512)) / 8.0).astype(np.float32)  # exact in all three
    v[0, :5] = [np.inf, -np.inf, np.nan, -0.0, 0.0]
    lens = [512, 400, 200, 37]
    a = otopk.topk_select(v, "fp32", lens, 64)
    b = otopk.topk_select(v.astype(np.float16), "fp16", lens, 64)
    c = otopk.topk_select(ofmt.f32_to_bf16_bits(v), "bf16", lens, 64)
    assert (a == b).all() and (a == c).all()


def test_rows_subset():
    rng = np.random.default_rng(2)
    s = rng.standard_normal((6, 300)).astype(np.float32)
    full = otopk.topk_select(s, "fp32", [300] * 6, 50)
    part = otopk.topk_select(s, "fp32", [300] * 6, 50, rows=[4, 1])
    assert (part == full[[4, 1]]).all()


def test_overlap_metrics():
    a = np.array([[0, 1, 2, 3], [4, 5, -1, -1], [-1, -1, -1, -1]])
    assert otopk.overlap(a, a) == {"row_jaccard": 1.0, "recall": 1.0, "exact_rows": 1.0,
                                   "micro_jaccard": 1.0}
    b = np.array([[0, 1, 6, 7], [8, 9, -1, -1], [-1, -1, -1, -1]])
    m = otopk.overlap(a, b)
    # row 0: 2 common of 6 -> 1/3; row 1: 0 of 4; row 2: both empty -> 1
    assert m["row_jaccard"] == pytest.approx((1 / 3 + 0 + 1) / 3)
    assert m["recall"] == pytest.approx((2 / 4 + 0 + 1) / 3)
    assert m["exact_rows"] == pytest.approx(1 / 3)
    assert m["micro_jaccard"] == pytest.approx(2 / 10)
