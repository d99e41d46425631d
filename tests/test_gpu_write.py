"""GPU parity of quantize-on-write (kv_quant_write): cache bytes and scales
must equal the oracle's bit for bit."""

import zlib

import numpy as np
import pytest
import torch

from oracle import formats as ofmt
from quantized_kv_top_amd import qsakv
from quantized_kv_top_amd import workloads as wl

from parity_util import assert_rows_equal, dev, gpu_write, layer_scales, oracle_write, say

pytestmark = pytest.mark.gpu

KINDS = ["int8", "int8_inline", "e4m3", "bf16", "nvfp4"]


def _scales(kind, w):
    return layer_scales(kind, w)


@pytest.mark.parametrize("kind", KINDS)
def test_write_tiny(kind):
    w = wl.tiny()
    ks, vs = _scales(kind, w)
    say("write tiny", kind, ks, vs)
    c = gpu_write(kind, w, ks or 1.0, vs or 1.0)
    oc = oracle_write(kind, w, ks, vs)
    assert_rows_equal(c, oc, np.arange(oc.num_slots))


def _special_rows(D, H, rng):
    """Rows that stress the quantizers: zero, one-hot, constant, tiny
    (subnormal scale), huge, near-ties, ordinary."""
    rows = []
    rows.append(np.zeros(D))
    oh = np.zeros(D)
    oh[5] = -3.25
    rows.append(oh)
    rows.append(np.full(D, 2.5))
    rows.append(rng.standard_normal(D) * 1e-38)            # scale underflows
    rows.append(rng.standard_normal(D) * 1e-41)            # subnormal sources
    rows.append(rng.standard_normal(D) * 1e30)
    a = np.float32(37.0)
    s = np.float32(a / np.float32(127))
    k = rng.integers(-126, 126, D)
    ties = ((k + 0.5) * np.float64(s)).astype(np.float32)
    ties[0] = a
    rows.append(ties)
    rows.append(np.nextafter(ties, np.float32(np.inf)))
    while len(rows) % H:
        rows.append(rng.standard_normal(D))
    return np.stack(rows).astype(np.float32)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("src", ["fp32", "bf16", "fp16"])
def test_write_dtypes_and_special_rows(kind, D, src):
    rng = np.random.default_rng(zlib.crc32((kind + str(D) + src).encode()))
    H, BS, NB = 2, 16, 64
    special = _special_rows(D, H, rng)
    T = 300
    x = (rng.standard_normal((T, H, D)) * np.exp2(rng.uniform(-8, 8, (T, H, 1)))).astype(np.float32)
    sp = special.reshape(-1, H, D)
    x[:sp.shape[0]] = sp
    y = np.roll(x, 7, axis=0)
    tdt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[src]
    kt = torch.from_numpy(x).to(tdt)
    vt = torch.from_numpy(y).to(tdt)
    if src == "fp16":       # keep fp16 sources finite
        kt = torch.nan_to_num(kt, posinf=60000.0, neginf=-60000.0)
        vt = torch.nan_to_num(vt, posinf=60000.0, neginf=-60000.0)
    slots = rng.permutation(NB * BS)[:T].astype(np.int64)
    slots[::17] = -1                                   # skipped tokens
    slots[5] = NB * BS + 3                             # out of range: skipped
    w = wl.Workload("t", 2 * H, H, D, BS, NB, "bf16", "fp32", src, kt, vt, slots,
                    torch.zeros(1, 2 * H, D, dtype=torch.bfloat16), np.zeros(1, np.int32),
                    np.zeros((1, 1), np.int32), np.zeros((1, 1), np.int32), 0.1)
    ks, vs = {"e4m3": (0.0171247218, 0.0841238871),
              "nvfp4": (0.0021, 0.0000317)}.get(kind, (None, None))
    say("write", kind, D, src)
    c = gpu_write(kind, w, ks or 1.0, vs or 1.0)
    good = (slots >= 0) & (slots < NB * BS)
    w.slot_mapping = np.where(good, slots, -1)
    oc = oracle_write(kind, w, ks, vs)
    assert_rows_equal(c, oc, np.arange(NB * BS))


@pytest.mark.parametrize("src", ["fp32", "bf16"])
def test_int8_quotients_at_rounding_ties(src):
    """Rows whose quotients x / s land on, and within a few ulps of, the
    half-integers where the int8 rounding decides (ties to even), at
    non-power-of-two scales: the codes must equal the oracle's fp32
    quotient-then-round."""
    rng = np.random.default_rng(77 if src == "fp32" else 78)
    H, D, T = 2, 128, 96
    x = np.zeros((T, H, D), np.float32)
    for t in range(T):
        for h in range(H):
            amax = np.float32(rng.uniform(0.3, 3.0) * np.exp2(rng.integers(-20, 20)))
            if src == "bf16":
                amax = (torch.tensor([float(amax)]).to(torch.bfloat16).float().numpy()[0])
            s = np.float32(amax / np.float32(127))
            k = rng.integers(0, 127, size=D - 1)
            v = ((k + np.float32(0.5)) * s).astype(np.float32)     # ~ on a tie
            off = rng.integers(-3, 4, size=D - 1).astype(np.int32)  # a few ulps off
            v = (v.view(np.int32) + off).view(np.float32)
            v = np.minimum(v, amax) * rng.choice(np.array([-1, 1], np.float32), size=D - 1)
            x[t, h, 0] = amax
            x[t, h, 1:] = v
    tdt = {"fp32": torch.float32, "bf16": torch.bfloat16}[src]
    kt = torch.from_numpy(x).to(tdt)
    vt = torch.from_numpy(-x[::-1].copy()).to(tdt)
    BS, NB = 16, 8
    slots = rng.permutation(NB * BS)[:T].astype(np.int64)
    w = wl.Workload("t", 2 * H, H, D, BS, NB, "bf16", "fp32", src, kt, vt, slots,
                    torch.zeros(1, 2 * H, D, dtype=torch.bfloat16), np.zeros(1, np.int32),
                    np.zeros((1, 1), np.int32), np.zeros((1, 1), np.int32), 0.1)
    say("int8 ties", src)
    for kind in ("int8", "int8_inline"):
        c = gpu_write(kind, w)
        oc = oracle_write(kind, w, None, None)
        assert_rows_equal(c, oc, np.arange(NB * BS))


def _sweep_values():
    exps = np.arange(256, dtype=np.uint32)
    top = np.arange(64, dtype=np.uint32) << np.uint32(17)
    low = np.array([0, 1, 0xFFFF, 0x10000, 0x10001, 0x1FFFF], dtype=np.uint32)
    u = (exps[:, None, None] << np.uint32(23)) | top[None, :, None] | low[None, None, :]
    u = u.ravel()
    u = np.concatenate([u, u | np.uint32(0x80000000)])
    return u.view(np.float32)


@pytest.mark.parametrize("scale", [1.0, 0.0171247218, 3.0])
def test_e4m3_encoder_bit_sweep(scale):
    """Every fp32 sign/exponent with the top 6 mantissa bits and rounding /
    sticky patterns below them (196,608 values, NaN and inf included) through
    kv_quant_write; finite results must equal the oracle's codes, NaN
    sources must give a NaN code."""
    vals = _sweep_values()
    D, H = 256, 1
    T = vals.size // D
    x = vals[:T * D].reshape(T, H, D)
    kt = torch.from_numpy(x.copy())
    slots = np.arange(T, dtype=np.int64)
    BS = 64
    NB = -(-T // BS)
    w = wl.Workload("sweep", 1, 1, D, BS, NB, "bf16", "fp32", "fp32", kt, kt, slots,
                    torch.zeros(1, 1, D, dtype=torch.bfloat16), np.zeros(1, np.int32),
                    np.zeros((1, 1), np.int32), np.zeros((1, 1), np.int32), 0.1)
    say("e4m3 sweep scale", scale, "values", x.size)
    c = gpu_write("e4m3", w, scale, scale)
    got = c.k.view(NB * BS, H, D)[:T].cpu().numpy().ravel()
    want = ofmt.e4m3_quantize(x.ravel(), np.float32(scale))
    nan = np.isnan(x.ravel())
    np.testing.assert_array_equal(got[~nan], want[~nan])
    assert np.all(got[nan] & 0x7F == 0x7F)


def test_e4m3_encoder_exhaustive():
    """Every fp32 bit pattern -- 2^32 values: both signs, every exponent and
    mantissa, subnormals, +-inf and every NaN payload -- written through
    kv_quant_write into an E4M3 cache at scale 1.0, each code equal to the
    oracle's encoding of the same pattern (the converter contract
    stored = e4m3fn(x / scale) of page "Qwen3.8 Flash Next NVFP4 QSA FP8 E4M3
    KV Scales", section "Calibration"; NaN sources keep their sign).  Each
    call writes 2^28 patterns as K rows and the next 2^28 as V rows; the
    oracle side runs in chunks on a pool of host threads."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    D, H, BS = 256, 1, 64
    half = 1 << 28
    T = half // D
    c = qsakv.Cache("e4m3", T // BS, BS, H, D, k_scale=1.0, v_scale=1.0, zero=False)
    slots = torch.arange(T, dtype=torch.int64, device="cuda")
    CH = 1 << 22
    nthreads = max(1, min(16, int(os.environ.get("OMP_NUM_THREADS", 0)) or (os.cpu_count() or 1)))

    def patterns(start):             # int32 tensor of the bit patterns start .. start + half
        lo = start - (1 << 32) if start >= (1 << 31) else start
        return torch.arange(lo, lo + half, dtype=torch.int32, device="cuda")

    def check(got, start, off):
        with np.errstate(all="ignore"):
            x = np.arange(start + off, start + off + CH, dtype=np.uint64).astype(np.uint32)
            want = ofmt.e4m3_quantize(x.view(np.float32), np.float32(1.0))
        bad = np.flatnonzero(got[off:off + CH] != want)
        return int(bad.size), [hex(start + off + int(b)) for b in bad[:4]]

    total = 0
    with ThreadPoolExecutor(nthreads) as pool:
        for base in range(0, 1 << 32, 2 * half):
            k = patterns(base).view(torch.float32).reshape(T, H, D)
            v = patterns(base + half).view(torch.float32).reshape(T, H, D)
            qsakv.kv_quant_write(c, k, v, slots)
            got_k = c.k.cpu().numpy()
            got_v = c.v.cpu().numpy()
            del k, v
            futs = [pool.submit(check, got, start, off)
                    for got, start in ((got_k, base), (got_v, base + half))
                    for off in range(0, half, CH)]
            res = [f.result() for f in futs]
            bad = sum(r[0] for r in res)
            first = [h for r in res for h in r[1]][:4]
            total += 2 * half
            say("e4m3 exhaustive: patterns 0x%08x..0x%08x checked (%d threads), mismatches %d %s"
                % (base, base + 2 * half - 1, nthreads, bad, first))
            assert bad == 0, "codes differ from the oracle at fp32 patterns %s" % first
    assert total == 1 << 32


@pytest.mark.parametrize("g", [1.0, 0.0021, 3.0e-6])
def test_nvfp4_blocks_sweep(g):
    """NVFP4 rows whose blocks hold the fp32 sweep values (NaN, +-inf,
    subnormals, every exponent) and blocks built on the E2M1 midpoints of a
    representable block scale (ties): element codes and block-scale codes
    must equal the oracle's."""
    vals = _sweep_values()
    D, H = 256, 1
    rng = np.random.default_rng(17)
    T0 = vals.size // D
    x = vals[:T0 * D].reshape(T0, D).copy()
    # tie rows: midpoints between E2M1 values times S g, with S = 2.5 (E4M3
    # exact) and the block max 6 S g so that the block scale is exactly S
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    tie = np.empty((64, D), np.float32)
    for r in range(64):
        m = rng.choice(mids, size=D) * np.where(rng.random(D) < 0.5, -1, 1)
        m[::16] = 6.0
        tie[r] = (m * np.float32(2.5) * np.float32(g)).astype(np.float32)
    x = np.concatenate([x, tie])
    T = x.shape[0]
    kt = torch.from_numpy(x.reshape(T, H, D).copy())
    BS = 64
    NB = -(-T // BS)
    slots = np.arange(T, dtype=np.int64)
    w = wl.Workload("nvfp4 sweep", 1, 1, D, BS, NB, "bf16", "fp32", "fp32", kt, kt, slots,
                    torch.zeros(1, 1, D, dtype=torch.bfloat16), np.zeros(1, np.int32),
                    np.zeros((1, 1), np.int32), np.zeros((1, 1), np.int32), 0.1)
    say("nvfp4 sweep g", g, "rows", T)
    c = gpu_write("nvfp4", w, g, g)
    oc = oracle_write("nvfp4", w, g, g)
    assert_rows_equal(c, oc, np.arange(T))


def test_write_is_deterministic_and_launch_independent():
    w = wl.prefill(num_rows=4, topk=64, ctx=4096, pool_blocks=80)
    a = gpu_write("int8", w)
    b = gpu_write("int8", w)
    assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v) and torch.equal(a.kv_scale, b.kv_scale)
    # writing the tokens in two calls of different sizes gives the same cache
    c = qsakv.Cache("int8", w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    sm = dev(w.slot_mapping, torch.int64)
    ks, vs = w.k_src.cuda(), w.v_src.cuda()
    qsakv.kv_quant_write(c, ks[:1000].contiguous(), vs[:1000].contiguous(), sm[:1000])
    qsakv.kv_quant_write(c, ks[1000:].contiguous(), vs[1000:].contiguous(), sm[1000:])
    torch.cuda.synchronize()
    assert torch.equal(a.k, c.k) and torch.equal(a.kv_scale, c.kv_scale)


@pytest.mark.parametrize("seed", list(range(500, 540)))
def test_random_writes(seed):
    """A seeded random write: cache kind, D, Hkv, block size, pool size,
    token count, source dtype, magnitudes over many octaves, layer scales,
    and slots with skipped (-1) and out-of-range entries; every slot's bytes
    against the oracle."""
    rng = np.random.default_rng(seed)
    kind = KINDS[rng.integers(len(KINDS))]
    D = int(rng.choice([128, 256]))
    H = int(rng.integers(1, 5))
    BS = int(2 ** rng.integers(0, 8))
    NB = int(rng.integers(1, 2048 // BS + 2))
    T = int(rng.integers(1, NB * BS + 1))
    src = str(rng.choice(["fp32", "bf16", "fp16"]))
    x = (rng.standard_normal((T, H, D)) *
         np.exp2(rng.uniform(-10, 6, (T, H, 1)))).astype(np.float32)
    y = (rng.standard_normal((T, H, D)) *
         np.exp2(rng.uniform(-10, 6, (T, H, 1)))).astype(np.float32)
    tdt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[src]
    slots = rng.permutation(NB * BS)[:T].astype(np.int64)
    drop = rng.random(T)
    slots[drop < 0.05] = -1
    slots[(drop >= 0.05) & (drop < 0.07)] = NB * BS + 5
    w = wl.Workload("t", H, H, D, BS, NB, "bf16", "fp32", src, torch.from_numpy(x).to(tdt),
                    torch.from_numpy(y).to(tdt), slots,
                    torch.zeros(1, H, D, dtype=torch.bfloat16), np.zeros(1, np.int32),
                    np.zeros((1, 1), np.int32), np.zeros((1, 1), np.int32), 0.1)
    ks = vs = None
    if kind == "e4m3":
        ks, vs = float(np.exp2(rng.uniform(-8, 2))), float(np.exp2(rng.uniform(-8, 2)))
    elif kind == "nvfp4":
        ks, vs = float(np.exp2(rng.uniform(-14, -2))), float(np.exp2(rng.uniform(-14, -2)))
    say("random write", seed, kind, "D", D, "H", H, "BS", BS, "NB", NB, "T", T, src)
    c = gpu_write(kind, w, ks or 1.0, vs or 1.0)
    good = (slots >= 0) & (slots < NB * BS)
    w.slot_mapping = np.where(good, slots, -1)
    oc = oracle_write(kind, w, ks, vs)
    assert_rows_equal(c, oc, np.arange(NB * BS))
