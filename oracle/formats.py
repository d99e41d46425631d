"""Oracle number formats (test infrastructure only; see package docstring).

All quantization decisions are taken in IEEE binary32, exactly as the method
states them: the scale is a float32 quotient and the element quotient
``x / scale`` is a float32 quotient, both correctly rounded.  numpy's float32
division is IEEE correctly rounded, and ``np.rint`` rounds half to even.
"""

import numpy as np

E4M3_MAX = 448.0            # largest finite OCP E4M3FN magnitude
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_MIN_SUBNORMAL = 2.0 ** -9
INT8_QMAX = 127


# --------------------------------------------------------------------------
# Source upcasts (bf16 bit patterns are carried as uint16: numpy has no bf16)
# --------------------------------------------------------------------------

def bf16_bits_to_f32(bits):
    """bf16 -> fp32 is exact: the 16 bits become the high half of the word."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def upcast_to_f32(src, dtype):
    """Source element -> float32, exactly.  ``dtype`` in {'fp32','bf16','fp16'}."""
    if dtype == "fp32":
        return np.asarray(src, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_to_f32(src)
    if dtype == "fp16":
        return np.asarray(src, dtype=np.float16).astype(np.float32)
    raise ValueError(dtype)


def f32_to_bf16_bits(x):
    """float32 -> bf16 bit pattern, round to nearest, ties to even.

    NaN maps to the quiet NaN 0x7FC0 with the input's sign bit.  Used for the
    bf16 comparison arm of the cache and for bf16 inputs made by tests.
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint32)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    sign = ((u >> np.uint64(16)) & np.uint64(0x8000)).astype(np.uint32)
    r = np.where(nan, sign | np.uint32(0x7FC0), r)
    return r.astype(np.uint16)


# --------------------------------------------------------------------------
# int8 per-(token, KV head) symmetric quantization
# --------------------------------------------------------------------------

def int8_quantize(x):
    """Quantize each vector along the last axis to int8 with one fp32 scale.

    Page "int8 per-(token,head) KV cache for the Qwen3.8-Flash-Next QSA path"
    (sections "Headline result", "The finding worth upstreaming"): one fp32
    scale per (token, KV head) for K and V separately.  The arithmetic:

        a   = max_d |x_d|                       (float32, exact)
        s   = fl32(a / 127)                     (correctly rounded)
        q_d = clamp(rne(fl32(x_d / s)), -127, 127)

    Reading for the degenerate case: if s == 0 (an all-zero vector, or a
    magnitude so small that a/127 underflows to zero) every q_d is 0 and the
    stored scale is 0.  -128 is never produced.  Inputs must be finite.

    Returns (q int8 [..., D], s float32 [...]).
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.max(np.abs(x), axis=-1)
    s = (a / np.float32(INT8_QMAX)).astype(np.float32)
    zero = s == np.float32(0)
    safe = np.where(zero, np.float32(1), s).astype(np.float32)
    y = (x / safe[..., None]).astype(np.float32)
    q = np.clip(np.rint(y), -INT8_QMAX, INT8_QMAX)
    q = np.where(zero[..., None], 0.0, q).astype(np.int8)
    return q, s


def int8_dequantize(q, s):
    """Exact reconstruction q * s in float64."""
    return np.asarray(q, dtype=np.float64) * np.asarray(s, dtype=np.float64)[..., None]


# --------------------------------------------------------------------------
# OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits,
# no infinities, NaN = S.1111.111, largest finite 448.
# --------------------------------------------------------------------------

def e4m3_decode(codes):
    """Decode E4M3FN byte codes to float64 (exact).

    E >= 1: (-1)^S * 2^(E-7) * (1 + M/8);  E == 0: (-1)^S * M * 2^-9;
    S.1111.111 is NaN.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * E4M3_MIN_SUBNORMAL,
                   np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64)))
    val = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def e4m3_encode(y):
    """Encode float32 values to E4M3FN codes: round to nearest even, saturate.

    Converter contract of page "Qwen3.8 Flash Next NVFP4 QSA FP8 E4M3 KV
    Scales", section "Calibration" (stored = e4m3fn(x / scale)); the format's
    boundaries follow page "[Model][SM70][FP8] Add calibrated E4M3 QSA KV
    cache", section "Why calibrated scale is part of this contract".

    * NaN            -> S.1111.111 (sign kept)
    * |y| >= 448, inf -> S.1111.110 (= +-448, saturation)
    * otherwise the nearest representable magnitude, ties to the even
      mantissa; below 2^-6 the quantum is the subnormal step 2^-9.
    * the sign of zero is kept (-0 -> 0x80).
    """
    y = np.asarray(y, dtype=np.float32)
    with np.errstate(invalid="ignore"):          # signalling NaN payloads
        a = np.abs(y.astype(np.float64))
    sign = np.signbit(y).astype(np.uint8) << np.uint8(7)
    nan = np.isnan(y)
    a = np.where(nan, 0.0, a)
    _, ex = np.frexp(a)                      # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex.astype(np.int64) - 1, -6)   # floor(log2 a), floored at -6
    quantum = np.ldexp(1.0, e - 3)
    r = np.rint(a / quantum)                 # exact scaling, half-even rounding
    v = np.minimum(r * quantum, E4M3_MAX)    # saturate
    # magnitude value -> code
    _, ev = np.frexp(v)
    ev = ev.astype(np.int64) - 1
    normal = v >= E4M3_MIN_NORMAL
    evn = np.where(normal, ev, 0)
    mant = np.where(normal, np.rint(np.ldexp(v, -evn) * 8.0 - 8.0), 0.0)
    code_norm = ((evn + 7) << 3) + mant.astype(np.int64)
    code_sub = np.rint(v / E4M3_MIN_SUBNORMAL).astype(np.int64)
    code = np.where(normal, code_norm, code_sub).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code) | sign
    return code.astype(np.uint8)


def e4m3_quantize(x, scale):
    """stored = e4m3fn(fl32(x / scale)) with a per-tensor float32 scale."""
    x = np.asarray(x, dtype=np.float32)
    y = (x / np.float32(scale)).astype(np.float32)
    return e4m3_encode(y)


def e4m3_calibrate_scale(x):
    """scale = fl32(max|x| / 448) for one tensor (the converter contract)."""
    a = np.max(np.abs(np.asarray(x, dtype=np.float32)))
    return np.float32(a / np.float32(E4M3_MAX))


# --------------------------------------------------------------------------
# NVFP4 rows (a reading; the pages name NVFP4 KV storage as a variant outside
# the calibrated-E4M3 contract of page "[Model][SM70][FP8] Add calibrated
# E4M3 QSA KV cache", section "Relationship to vLLM #54846", without its
# layout): FP4 E2M1 element codes, one E4M3 scale per block of 16
# consecutive elements of a (token, KV head) row, and one float32 scale per
# layer and tensor, as the E4M3 cache keeps one per layer.
#
# E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; magnitudes 0, 0.5, 1,
# 1.5, 2, 3, 4, 6; no infinities or NaN.
# --------------------------------------------------------------------------
E2M1_MAX = 6.0
NVFP4_BLOCK = 16


def e2m1_decode(codes):
    """4-bit E2M1 codes (low nibble of each value) -> float64, exactly.

    E >= 1: (-1)^S * 2^(E-1) * (1 + M/2);  E == 0: (-1)^S * M / 2.
    """
    c = np.asarray(codes).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(e == 0, m * 0.5, np.ldexp(1.0 + m / 2.0, (e - 1).astype(np.int64)))
    return sign * mag


def e2m1_encode(y):
    """float32 -> 4-bit E2M1 codes: nearest magnitude, ties to the even
    code (mantissa bit 0), saturating at 6 (infinities included); the sign
    bit is the sign of y (so -0 and small negatives give 0x8); NaN -> 0."""
    y = np.asarray(y, dtype=np.float32)
    nan = np.isnan(y)
    a = np.where(nan, 0.0, np.abs(y.astype(np.float64)))
    grid = e2m1_decode(np.arange(8))
    lo = np.clip(np.searchsorted(grid, a, side="right") - 1, 0, 7)
    hi = np.minimum(lo + 1, 7)
    dlo = a - grid[lo]
    dhi = grid[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(a >= E2M1_MAX, 7, np.where(pick_hi, hi, lo)).astype(np.uint8)
    sign = (np.signbit(y) & ~nan).astype(np.uint8) << np.uint8(3)
    return code | sign


def nvfp4_quantize(x, scale):
    """Rows of float32 x [..., D] (D a multiple of 16) with the layer's
    float32 scale g -> (element codes [..., D] 4-bit, block scale codes
    [..., D/16] E4M3).  Per block of 16: a = max |x| (NaN ignored),
    s = fl32(a / 6), code = e4m3fn(fl32(s / g)) (round to nearest even,
    saturating), S = its value; the elements are e2m1(fl32(x / fl32(S g))),
    or 0 when S g is 0.  Divisions are IEEE float32, as the E4M3 converter's.
    """
    x = np.asarray(x, dtype=np.float32)
    shp = x.shape
    D = shp[-1]
    xb = x.reshape(shp[:-1] + (D // NVFP4_BLOCK, NVFP4_BLOCK))
    with np.errstate(invalid="ignore"):
        a = np.max(np.where(np.isnan(xb), np.float32(0), np.abs(xb)), axis=-1).astype(np.float32)
    s = (a / np.float32(E2M1_MAX)).astype(np.float32)
    with np.errstate(over="ignore"):
        sc = e4m3_encode((s / np.float32(scale)).astype(np.float32))
        eff = (e4m3_decode(sc).astype(np.float32) * np.float32(scale)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = (xb / eff[..., None]).astype(np.float32)
    q = np.where(eff[..., None] > 0, e2m1_encode(y), np.uint8(0))
    return q.reshape(shp).astype(np.uint8), sc


def nvfp4_pack(q):
    """4-bit codes [..., D] -> bytes [..., D/2]: element 2j in the low nibble
    of byte j, element 2j + 1 in the high nibble."""
    q = np.asarray(q, dtype=np.uint8)
    return (q[..., 0::2] & 0xF) | ((q[..., 1::2] & 0xF) << 4)


def nvfp4_unpack(b):
    b = np.asarray(b, dtype=np.uint8)
    q = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    q[..., 0::2] = b & 0xF
    q[..., 1::2] = b >> 4
    return q


def nvfp4_dequantize(q, sc, scale):
    """Exact float64 values: e2m1(q) * e4m3(block scale) * g."""
    v = e2m1_decode(q)
    S = e4m3_decode(sc)
    shp = v.shape
    vb = v.reshape(shp[:-1] + (shp[-1] // NVFP4_BLOCK, NVFP4_BLOCK))
    return (vb * S[..., None] * np.float64(np.float32(scale))).reshape(shp)


def nvfp4_calibrate_scale(x):
    """g = fl32(max|x| / 2688) for one tensor: the largest block scale,
    max|x| / 6 / g, lands on E4M3's 448."""
    a = np.max(np.abs(np.asarray(x, dtype=np.float32)))
    return np.float32(a / np.float32(E2M1_MAX * E4M3_MAX))
