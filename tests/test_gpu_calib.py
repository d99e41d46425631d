"""GPU parity of the calibration statistics (kv_calib_stats) against the
oracle: every field exact, for fp16 / bf16 / fp32 sources with NaN, +-inf,
zeros and values at every threshold, ragged sizes, a garbage workspace, and
a full-size E4M3-workload layer tensor."""

import numpy as np
import pytest
import torch

from oracle import calib as ocalib
from oracle import formats as ofmt
from quantized_kv_top_amd import qsakv
from quantized_kv_top_amd import workloads as wl

from parity_util import say

pytestmark = pytest.mark.gpu

FIELDS = ("count", "nan", "nonzero", "saturated", "below_min_subnormal", "subnormal",
          "max_abs", "p999", "p9999")


def _gpu(x, scale, ws_fill=None):
    out = torch.zeros(64, dtype=torch.uint8, device="cuda")
    ws = torch.empty(qsakv.calib_workspace_bytes(), dtype=torch.uint8, device="cuda")
    ws.fill_(0xA5 if ws_fill is None else ws_fill)
    qsakv.kv_calib_stats(x, scale, out, ws)
    torch.cuda.synchronize()
    return qsakv.calib_result(out)


def _oracle(x, scale):
    xs = wl.to_numpy_src(x)
    dt = {torch.float16: "fp16", torch.bfloat16: "bf16", torch.float32: "fp32"}[x.dtype]
    return ocalib.calib_stats(xs, dt, scale)


def _check(x, scale, what):
    g = _gpu(x, scale)
    r = _oracle(x, scale)
    for f in FIELDS:
        assert g[f] == r[f], "%s: %s gpu %r oracle %r" % (what, f, g[f], r[f])


def _specials(n, scale, dtype, seed):
    """Student-t values with zeros, NaN, +-inf and values at the E4M3
    thresholds of the quotient (and their neighbours) sprinkled in."""
    rng = np.random.default_rng(seed)
    v = (rng.standard_t(4, size=n) * 0.5).astype(np.float32)
    if n >= 64:
        pos = rng.choice(n, size=48, replace=False)
        t = [448.0, 2.0 ** -9, 2.0 ** -6]
        vals = []
        for th in t:
            c = np.float32(th * scale)
            vals += [c, np.nextafter(c, np.float32(0)), np.nextafter(c, np.float32(1e30))]
        vals += [0.0, -0.0, np.nan, np.inf, -np.inf, 1e-30, -1e-30]
        for i, p in enumerate(pos):
            v[p] = np.float32(vals[i % len(vals)]) * (1 if i % 2 else -1)
    x = torch.from_numpy(v)
    if dtype == torch.bfloat16:
        return torch.from_numpy(ofmt.f32_to_bf16_bits(v).view(np.int16)).view(torch.bfloat16)
    return x.to(dtype)


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16, torch.float32])
@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 1000, 100003, (1 << 20) + 5])
def test_small_and_ragged(dtype, n):
    scale = 0.0171247218 if n % 2 else 1.0
    x = _specials(n, scale, dtype, seed=n).cuda()
    say("calib", dtype, n)
    _check(x, scale, "calib %s n=%d" % (dtype, n))


def test_fp32_ties_in_selected_bins():
    """Many fp32 values sharing the high 16 bits of the percentile bins, so
    the second pass decides the low bits."""
    rng = np.random.default_rng(11)
    base = np.float32(3.0)
    u = base.view(np.uint32) + rng.integers(0, 1 << 16, size=3_000_000).astype(np.uint32)
    v = u.view(np.float32) * np.where(rng.random(u.size) < 0.5, -1, 1).astype(np.float32)
    v[:2_000_000] *= np.float32(0.25)      # the bulk below the percentile bins
    x = torch.from_numpy(v).cuda()
    _check(x, 0.01, "fp32 ties")


def test_all_nan_and_all_zero():
    x = torch.full((1001,), float("nan"), dtype=torch.float16, device="cuda")
    _check(x, 1.0, "all nan")
    x = torch.zeros(4099, dtype=torch.bfloat16, device="cuda")
    _check(x, 1.0, "all zero")


def test_workspace_contents_ignored():
    x = _specials(50001, 0.05, torch.float16, seed=3).cuda()
    a = _gpu(x, 0.05, ws_fill=0x00)
    b = _gpu(x, 0.05, ws_fill=0xFF)
    assert a == b


@pytest.mark.parametrize("which", ["k", "v"])
def test_full_size_layer_tensor(which):
    """One layer's K or V source of the E4M3 workload (4 x 65536 tokens x
    4 heads x 128, fp16): at its calibrated envelope scale (K) and at the
    unit scale (V)."""
    w = wl.e4m3_layer(5, device="cuda")
    x = (w.k_src if which == "k" else w.v_src).reshape(-1)
    if which == "k":
        amax = float(x.abs().max().float().item())
        scale = float(np.float32(amax) / np.float32(448))
    else:
        scale = 1.0
    say("calib full size", which, x.numel(), scale)
    _check(x, scale, "full %s" % which)
