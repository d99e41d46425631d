"""Pure-Python brute-force versions of the oracle's steps, for tiny inputs.

Test infrastructure only.  These take a different route to the same
definitions so that a slip in the vectorized oracle (a wrong rounding, a
transposed operand, a dropped term) shows up as a disagreement:

* float32 rounding is done with ``struct`` packing of Python doubles; a
  float32 quotient is the float32 rounding of the double quotient, which is
  the correctly rounded float32 quotient because 53 >= 2*24 + 2 (double
  rounding is innocuous for division at these precisions);
* E4M3 encoding is a nearest-neighbour search over the table of the 127
  finite non-negative E4M3 values, ties to the even code;
* attention uses ``math.exp`` / ``math.log`` and explicit loops.
"""

import math
import struct


def f32(x):
    """Round a Python float to the nearest float32 (ties to even)."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def rne(x):
    """Round half to even for a Python float."""
    return float(round(x))   # Python's round() on floats is half-to-even


def int8_quantize_vec(xs):
    """One vector -> (list of int codes, float32 scale), by the definition."""
    a = 0.0
    for x in xs:
        a = max(a, abs(x))
    s = f32(a / 127.0)
    if s == 0.0:
        return [0] * len(xs), 0.0
    out = []
    for x in xs:
        y = f32(x / s)
        q = rne(y)
        q = max(-127.0, min(127.0, q))
        out.append(int(q))
    return out, s


def e4m3_table():
    """The 127 finite non-negative E4M3FN magnitudes by code 0x00..0x7E."""
    vals = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        vals.append(m * 2.0 ** -9 if e == 0 else 2.0 ** (e - 7) * (1 + m / 8))
    return vals


_TABLE = e4m3_table()


def e4m3_encode_scalar(y):
    """Nearest finite E4M3 value (ties to even code), saturating at 448."""
    if math.isnan(y):
        return 0x7F | (0x80 if math.copysign(1.0, y) < 0 else 0)
    sign = 0x80 if math.copysign(1.0, y) < 0 else 0
    a = abs(y)
    if a >= _TABLE[-1]:
        return sign | 0x7E
    best = 0
    for c in range(0x7F):
        d, db = abs(_TABLE[c] - a), abs(_TABLE[best] - a)
        if d < db or (d == db and (c & 1) == 0 and (best & 1) == 1):
            best = c
    return sign | best


def attend_row(q, k_hat, v_hat, sm_scale):
    """q: [Hq][D] lists; k_hat, v_hat: [n][Hkv][D] lists -> (out, lse) lists."""
    Hq = len(q)
    D = len(q[0])
    n = len(k_hat)
    if n == 0:
        return [[0.0] * D for _ in range(Hq)], [-math.inf] * Hq
    Hkv = len(k_hat[0])
    G = Hq // Hkv
    out, lse = [], []
    for h in range(Hq):
        g = h // G
        s = []
        for j in range(n):
            acc = 0.0
            for d in range(D):
                acc += q[h][d] * k_hat[j][g][d]
            s.append(sm_scale * acc)
        m = max(s)
        w = [math.exp(x - m) for x in s]
        l = sum(w)
        o = []
        for d in range(D):
            acc = 0.0
            for j in range(n):
                acc += w[j] * v_hat[j][g][d]
            o.append(acc / l)
        out.append(o)
        lse.append(m + math.log(l))
    return out, lse
