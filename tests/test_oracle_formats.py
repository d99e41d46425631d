"""Pins of the oracle's number formats against the pages and the mathematics.

No GPU.  Each test pins the oracle to something other than itself: the
constants the pages print, an independent bit-level route, brute force, or a
library routine.
"""

import json
import os
import struct

import numpy as np
import pytest
import torch

from oracle import brute, formats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# E4M3
# ---------------------------------------------------------------------------

def test_e4m3_constants_from_pages():
    g = _golden("e4m3_format.json")
    dec = formats.e4m3_decode(np.arange(256, dtype=np.uint8))
    finite = dec[np.isfinite(dec)]
    assert np.max(finite) == g["max_finite"] == dec[0x7E]
    assert -np.min(finite) == g["max_finite"] == -dec[0xFE]
    pos = finite[finite > 0]
    assert np.min(pos) == 2.0 ** g["min_subnormal_log2"] == dec[0x01]
    # subnormals (exponent field 0) are exactly the non-zero values below 2^-6
    sub = dec[1:8]
    assert np.all(sub < 2.0 ** g["subnormal_upper_bound_log2"])
    assert dec[0x08] == 2.0 ** g["subnormal_upper_bound_log2"]
    # NaN is S.1111.111 only; no infinities
    nan_codes = [c for c in range(256) if np.isnan(dec[c])]
    assert nan_codes == [0x7F, 0xFF]
    assert not np.any(np.isinf(dec))


def test_e4m3_decode_all_256_via_fp16_bits():
    """Independent route: an E4M3FN code's bits placed into an fp16 word (sign
    to bit 15, exponent+mantissa shifted left by 7) give value / 2^8 for every
    finite code, normal or subnormal (fp16 bias 15 = E4M3 bias 7 + 8)."""
    c = np.arange(256, dtype=np.uint16)
    bits = ((c & 0x80) << 8) | ((c & 0x7F) << 7)
    via_fp16 = bits.astype(np.uint16).view(np.float16).astype(np.float64) * 256.0
    dec = formats.e4m3_decode(c.astype(np.uint8))
    finite = (c & 0x7F) != 0x7F
    np.testing.assert_array_equal(dec[finite], via_fp16[finite])
    # every E4M3 value is exact in fp16 and in bf16
    assert np.all(dec[finite].astype(np.float16).astype(np.float64) == dec[finite])
    bf = torch.tensor(dec[finite], dtype=torch.float64).to(torch.bfloat16).double().numpy()
    assert np.all(bf == dec[finite])


def test_e4m3_monotone_and_roundtrip():
    dec = formats.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(dec) > 0)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = formats.e4m3_decode(codes).astype(np.float32)
    vals = np.where(codes == 0x80, np.float32(-0.0), vals)
    np.testing.assert_array_equal(formats.e4m3_encode(vals), codes)


def test_e4m3_ties_go_to_even_code():
    dec = formats.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    for c in range(0x7E):
        mid = np.float32((dec[c] + dec[c + 1]) / 2)        # exact in fp32
        assert float(mid) == (dec[c] + dec[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        assert formats.e4m3_encode(mid) == even, (c, mid)
        assert formats.e4m3_encode(-mid) == 0x80 | even
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(1e9))
        assert formats.e4m3_encode(below) == c
        assert formats.e4m3_encode(above) == c + 1
    # the example the format makes easy to check by hand: 1.0625 lies halfway
    # between 1.0 (0x38) and 1.125 (0x39) and goes to the even mantissa
    assert formats.e4m3_encode(np.float32(1.0625)) == 0x38


def test_e4m3_saturation_nan_and_signed_zero():
    big = np.array([448, 449, 463.99, 464, 479.9, 480, 1e6, 3e38, np.inf], np.float32)
    assert np.all(formats.e4m3_encode(big) == 0x7E)
    assert np.all(formats.e4m3_encode(-big) == 0xFE)
    assert formats.e4m3_encode(np.float32(np.nan)) == 0x7F
    assert formats.e4m3_encode(-np.float32(np.nan)) == 0xFF
    assert formats.e4m3_encode(np.float32(0.0)) == 0x00
    assert formats.e4m3_encode(np.float32(-0.0)) == 0x80
    assert formats.e4m3_encode(np.float32(-1e-30)) == 0x80
    # half the smallest subnormal is a tie between 0 and 2^-9 -> 0
    assert formats.e4m3_encode(np.float32(2.0 ** -10)) == 0x00
    assert formats.e4m3_encode(np.nextafter(np.float32(2.0 ** -10), np.float32(1))) == 0x01


def test_e4m3_encode_vs_brute_force():
    rng = np.random.default_rng(11)
    mags = np.exp2(rng.uniform(-14, 10, 4000)).astype(np.float32)
    sgn = np.where(rng.random(4000) < 0.5, -1, 1).astype(np.float32)
    vals = np.concatenate([mags * sgn, rng.standard_normal(1000).astype(np.float32)])
    got = formats.e4m3_encode(vals)
    want = np.array([brute.e4m3_encode_scalar(float(v)) for v in vals], dtype=np.uint8)
    np.testing.assert_array_equal(got, want)


def test_e4m3_encode_bit_sweep_vs_brute_force():
    """Every sign/exponent pattern of fp32 with the top 5 mantissa bits and a
    set of low patterns that exercise rounding and stickiness."""
    exps = np.arange(256, dtype=np.uint32)
    top = np.arange(32, dtype=np.uint32) << np.uint32(18)
    low = np.array([0, 1, 0x1FFFF, 0x20000, 0x20001, 0x3FFFF], dtype=np.uint32)
    u = (exps[:, None, None] << np.uint32(23)) | top[None, :, None] | low[None, None, :]
    u = u.ravel()
    u = np.concatenate([u, u | np.uint32(0x80000000)])
    vals = u.view(np.float32)
    got = formats.e4m3_encode(vals)
    want = np.array([brute.e4m3_encode_scalar(float(v)) for v in vals], dtype=np.uint8)
    np.testing.assert_array_equal(got, want)


def test_e4m3_calibrated_envelope_maps_to_top_code():
    """scale = max/448 (converter contract): the envelope element lands on
    +-448 and nothing saturates beyond it; reconstruction is code * scale."""
    rng = np.random.default_rng(12)
    for _ in range(50):
        x = (rng.standard_t(4, size=4096) * 0.5).astype(np.float16).astype(np.float32)
        s = formats.e4m3_calibrate_scale(x)
        codes = formats.e4m3_quantize(x, s)
        i = np.argmax(np.abs(x))
        assert codes[i] & 0x7F == 0x7E
        rec = formats.e4m3_decode(codes) * np.float64(s)
        assert np.max(np.abs(rec)) == pytest.approx(448.0 * float(s), rel=0)


def test_e4m3_quotient_is_fp32():
    """The quotient x/scale is formed in float32 before encoding (the reading
    of the converter contract); compare with the brute-force route."""
    rng = np.random.default_rng(13)
    x = rng.standard_normal(2000).astype(np.float32)
    s = np.float32(0.0171247218)
    got = formats.e4m3_quantize(x, s)
    want = [brute.e4m3_encode_scalar(brute.f32(float(a) / float(s))) for a in x]
    np.testing.assert_array_equal(got, np.array(want, dtype=np.uint8))


# ---------------------------------------------------------------------------
# int8
# ---------------------------------------------------------------------------

def test_int8_closed_forms():
    D = 256
    for c in [1.0, -3.5, 1e-3, 7e4]:
        x = np.zeros(D, np.float32)
        x[17] = c
        q, s = formats.int8_quantize(x[None])
        assert s[0] == np.float32(np.float32(abs(c)) / np.float32(127))
        assert q[0, 17] == (127 if c > 0 else -127)
        assert np.count_nonzero(q) == 1
    x = np.where(np.arange(D) % 3 == 0, 2.5, -2.5).astype(np.float32)
    q, s = formats.int8_quantize(x[None])
    np.testing.assert_array_equal(q[0], np.where(np.arange(D) % 3 == 0, 127, -127))
    q, s = formats.int8_quantize(np.zeros((2, D), np.float32))
    assert np.all(q == 0) and np.all(s == 0)


def test_int8_bounds_and_error():
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((500, 128)) * np.exp2(rng.uniform(-20, 20, (500, 1)))).astype(np.float32)
    q, s = formats.int8_quantize(x)
    assert q.min() >= -127 and q.max() <= 127
    err = np.abs(x.astype(np.float64) - formats.int8_dequantize(q, s))
    assert np.all(err <= 0.5 * s[:, None].astype(np.float64) * (1 + 1e-6))
    # the largest element always reaches the end of the range
    i = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(q[np.arange(500), i]) == 127)


def test_int8_vs_brute_force():
    rng = np.random.default_rng(22)
    cases = [rng.standard_normal(64).astype(np.float32) for _ in range(40)]
    # near-ties: elements placed at (k + 1/2) * s give quotients on .5 boundaries
    for _ in range(40):
        a = np.float32(rng.uniform(0.5, 50))
        s = np.float32(a / np.float32(127))
        k = rng.integers(-126, 126, 63)
        xs = ((k + 0.5) * np.float64(s)).astype(np.float32)
        cases.append(np.concatenate([[a], xs]).astype(np.float32))
    for x in cases:
        q, s = formats.int8_quantize(x[None])
        bq, bs = brute.int8_quantize_vec([float(v) for v in x])
        assert float(s[0]) == bs
        assert q[0].tolist() == bq


def test_int8_quotient_rounding_is_fp32_not_fp64():
    """Find inputs whose fp64 quotient lies just off a .5 boundary that the
    fp32 quotient rounds onto; the oracle must follow the fp32 quotient."""
    rng = np.random.default_rng(23)
    found = 0
    for _ in range(200):
        a = np.float32(rng.uniform(1, 100))
        s = np.float32(a / np.float32(127))
        k = rng.integers(-126, 126, 4096)
        base = (k + 0.5) * np.float64(s)
        x = np.nextafter(base.astype(np.float32), np.float32(np.inf) * np.sign(base).astype(np.float32))
        y32 = (x / s).astype(np.float32)
        y64 = x.astype(np.float64) / np.float64(s)
        differ = np.rint(y32) != np.rint(y64)
        if not differ.any():
            continue
        j = int(np.argmax(differ))
        vec = np.zeros(8, np.float32)
        vec[0] = a
        vec[1] = x[j]
        q, _ = formats.int8_quantize(vec[None])
        assert q[0, 1] == np.clip(np.rint(y32[j]), -127, 127)
        assert q[0, 1] != np.clip(np.rint(y64[j]), -127, 127)
        found += 1
        if found >= 5:
            break
    assert found >= 1


# ---------------------------------------------------------------------------
# bf16 / source upcasts
# ---------------------------------------------------------------------------

def test_bf16_round_and_upcast_vs_torch():
    rng = np.random.default_rng(31)
    x = np.concatenate([
        (rng.standard_normal(20000) * np.exp2(rng.uniform(-30, 30, 20000))).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 3.4e38, -3.4e38, 1e-40, -1e-45, np.inf, -np.inf], np.float32),
        rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    x = x[np.isfinite(x) | np.isinf(x)]
    ours = formats.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    up = formats.bf16_bits_to_f32(ref)
    tref = torch.from_numpy(ref.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(up.view(np.uint32), tref.view(np.uint32))


def test_fp16_upcast_exact():
    h = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    f = formats.upcast_to_f32(h, "fp16")
    fin = np.isfinite(h)
    assert np.all(f[fin].astype(np.float16).view(np.uint16) == h[fin].view(np.uint16))


def test_brute_f32_rounding_matches_struct_semantics():
    # struct packing rounds to nearest even: 1 + 2^-24 is a tie -> 1.0
    assert brute.f32(1.0 + 2.0 ** -24) == 1.0
    assert brute.f32(1.0 + 3 * 2.0 ** -24) == 1.0 + 2.0 ** -22
    assert struct.unpack("<f", struct.pack("<f", 0.1))[0] == float(np.float32(0.1))
