"""Pins of the NVFP4 oracle (E2M1 codes, E4M3 block scales, a float32 layer
scale) against definitions it does not share code with: the E2M1 value
table written out, a pure-Python nearest-value search with ties to the even
code, brute-force block quantization with struct-rounded float32
arithmetic, closed forms and the byte layout.  No GPU."""

import struct

import numpy as np
import pytest

from oracle import brute
from oracle import cache as ocache
from oracle import formats as ofmt

# E2M1 magnitudes by code 0..7 (sign in bit 3)
TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_table():
    got = ofmt.e2m1_decode(np.arange(16))
    want = TABLE + [-v for v in TABLE]
    assert [float(v) for v in got] == want
    assert np.signbit(got[8])                        # code 0x8 is -0


def _nearest(v):
    """Pure Python: nearest table magnitude, ties to the even code,
    saturating; sign from v; NaN -> 0."""
    if v != v:
        return 0
    a = abs(v)
    if a >= 6.0:
        c = 7
    else:
        best = None
        for i, t in enumerate(TABLE):
            d = abs(a - t)
            if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
                best = (d, i)
        c = best[1]
    neg = struct.unpack("<I", struct.pack("<f", v))[0] >> 31
    return c | (8 if neg else 0)


def test_e2m1_encode_vs_nearest_search():
    vals = [k / 64.0 for k in range(-512, 513)] + [0.2499, 0.2501, 5.0, 5.0001, 4.9999, 1e-30,
                                                   -1e-30, 1e9, float("inf"), float("-inf"),
                                                   float("nan"), -0.0]
    y = np.array(vals, dtype=np.float32)
    got = ofmt.e2m1_encode(y)
    for v, g in zip(y.tolist(), got.tolist()):
        assert g == _nearest(v), (v, g, _nearest(v))


def test_e2m1_round_trip():
    codes = np.arange(16, dtype=np.uint8)
    assert (ofmt.e2m1_encode(ofmt.e2m1_decode(codes).astype(np.float32)) == codes).all()


def _brute_block(xs, g):
    """One block of 16 floats, struct-rounded float32 steps."""
    f = brute.f32
    a = 0.0
    for v in xs:
        if v == v:
            a = max(a, abs(v))
    s = f(a / 6.0)
    sc = int(ofmt.e4m3_encode(np.array([f(s / g)], np.float32))[0])
    S = float(ofmt.e4m3_decode(np.array([sc], np.uint8))[0])
    eff = f(S * g)
    q = [0 if eff == 0 else _nearest(f(v / eff)) for v in xs]
    return q, sc


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_block_quantization_vs_brute_force(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_t(3, size=(6, 64)) * 0.7).astype(np.float32)
    x[0, :16] = 0.0                                   # a zero block
    x[1, 16:32] *= np.float32(1e-12)                  # a block whose scale underflows
    x[2, 3] = np.nan                                  # NaN ignored by the block max
    x[3, 40] = np.inf                                 # saturating block
    g = float(np.float32(0.0021))
    q, sc = ofmt.nvfp4_quantize(x, g)
    for r in range(6):
        for b in range(4):
            qb, scb = _brute_block([float(v) for v in x[r, 16 * b:16 * b + 16]], g)
            assert sc[r, b] == scb, (r, b)
            assert q[r, 16 * b:16 * b + 16].tolist() == qb, (r, b)


def test_closed_forms():
    g = np.float32(2.0 ** -5)
    # a block whose max is 6 * 448 * g: scale code 448 (0x7E), the max -> 6
    x = np.zeros((1, 16), np.float32)
    x[0, 0] = 6 * 448 * g
    x[0, 1] = -x[0, 0]
    x[0, 2] = 448 * g                                 # exactly 1.0 after scaling
    q, sc = ofmt.nvfp4_quantize(x, g)
    assert sc[0, 0] == 0x7E
    assert q[0, :3].tolist() == [7, 15, 2]
    # grid values times a representable scale come back exactly
    S = 0.8125                                        # E4M3 1.101 x 2^-1
    vals = np.array(TABLE * 2, np.float32)
    vals[8:] *= -1
    x2 = (vals * np.float32(S) * g).astype(np.float32)[None, :]
    q2, sc2 = ofmt.nvfp4_quantize(x2, g)
    back = ofmt.nvfp4_dequantize(q2, sc2, g)
    assert np.array_equal(back, x2.astype(np.float64))
    # all-zero rows: zero codes and zero scales
    qz, sz = ofmt.nvfp4_quantize(np.zeros((2, 32), np.float32), g)
    assert not qz.any() and not sz.any()


def test_pack_layout_and_sizes():
    q = np.arange(16, dtype=np.uint8)[None, :]
    b = ofmt.nvfp4_pack(q)
    assert b.tolist() == [[0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]]
    assert (ofmt.nvfp4_unpack(b) == q).all()
    # K + V per token: codes D/2 and block scales D/16 per row
    assert ocache.bytes_per_token("nvfp4", 2, 256) == 2 * 2 * (128 + 16)
    assert ocache.bytes_per_token("nvfp4", 1, 128) == 2 * (64 + 8)


def test_calibrated_scale_puts_the_tensor_max_on_448():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((8, 4, 128)).astype(np.float32)
    g = ofmt.nvfp4_calibrate_scale(x)
    _, sc = ofmt.nvfp4_quantize(x, g)
    assert sc.max() == 0x7E and (sc & 0x80).max() == 0   # 448, never negative
    assert np.abs(x).max() / 6 / g == pytest.approx(448, rel=1e-6)


def test_cache_write_and_dequant_round_trip():
    rng = np.random.default_rng(5)
    T, H, D = 12, 2, 128
    k = rng.standard_normal((T, H, D)).astype(np.float32)
    v = rng.standard_normal((T, H, D)).astype(np.float32)
    ks, vs = ofmt.nvfp4_calibrate_scale(k), ofmt.nvfp4_calibrate_scale(v)
    c = ocache.OracleCache("nvfp4", 4, 4, H, D, k_scale=ks, v_scale=vs)
    slots = rng.permutation(16)[:T]
    c.write(k, v, "fp32", slots)
    qk, sk = ofmt.nvfp4_quantize(k, ks)
    assert (c.k[slots] == ofmt.nvfp4_pack(qk)).all() and (c.kv_scale[slots, :, 0] == sk).all()
    kh = c.dequant(slots, "k")
    assert np.array_equal(kh, ofmt.nvfp4_dequantize(qk, sk, ks))
    # the quantization error of a block is at most one E2M1 step times the
    # block's effective scale (no saturation at the calibrated scale)
    assert np.abs(kh - k).max() <= 2.0 * (np.abs(k).max() / 6) * 1.01
