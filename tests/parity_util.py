"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and the oracle on the same seeded inputs, and compare."""

import sys

import numpy as np
import torch

from oracle import attention as oatt
from oracle import cache as ocache
from oracle import formats as ofmt
from quantized_kv_top_amd import qsakv
from quantized_kv_top_amd import workloads as wl

ATOL, RTOL = 2e-3, 1e-2       # outputs vs the fp64 oracle, elementwise
LSE_ATOL = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x, dtype=None):
    t = torch.as_tensor(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def e4m3_scales(w):
    """Per-layer K and V scales: the oracle's calibration rule applied to the
    layer's max |x| (found on the device; max of |x| is exact)."""
    ka = np.float32(w.k_src.abs().max().float().item())
    va = np.float32(w.v_src.abs().max().float().item())
    return (float(ofmt.e4m3_calibrate_scale(np.array([ka], np.float32))),
            float(ofmt.e4m3_calibrate_scale(np.array([va], np.float32))))


def nvfp4_scales(w):
    """Per-layer K and V scales of an NVFP4 cache: max|x| / (6 * 448)."""
    ka = np.float32(w.k_src.abs().max().float().item())
    va = np.float32(w.v_src.abs().max().float().item())
    return (float(ofmt.nvfp4_calibrate_scale(np.array([ka], np.float32))),
            float(ofmt.nvfp4_calibrate_scale(np.array([va], np.float32))))


def layer_scales(kind, w):
    """(k_scale, v_scale) for kinds with per-layer scales, else (None, None)."""
    if kind == "e4m3":
        return e4m3_scales(w)
    if kind == "nvfp4":
        return nvfp4_scales(w)
    return None, None


def gpu_write(kind, w, k_scale=1.0, v_scale=1.0, num_blocks=None):
    c = qsakv.Cache(kind, num_blocks or w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim,
                    k_scale=k_scale, v_scale=v_scale)
    ks = w.k_src.cuda().contiguous()
    vs = w.v_src.cuda().contiguous()
    qsakv.kv_quant_write(c, ks, vs, dev(w.slot_mapping, torch.int64))
    return c


def oracle_write(kind, w, k_scale=None, v_scale=None, tokens=None, num_blocks=None):
    """Oracle cache with the workload's tokens (or the subset ``tokens``)."""
    oc = ocache.OracleCache(kind, num_blocks or w.num_blocks, w.block_size, w.num_kv_heads,
                            w.head_dim, k_scale, v_scale)
    if tokens is None:
        ks, vs, sm = wl.to_numpy_src(w.k_src), wl.to_numpy_src(w.v_src), w.slot_mapping
    else:
        ti = torch.as_tensor(np.asarray(tokens, np.int64))
        ks = wl.to_numpy_src(w.k_src[ti.to(w.k_src.device)])
        vs = wl.to_numpy_src(w.v_src[ti.to(w.v_src.device)])
        sm = w.slot_mapping[np.asarray(tokens)]
    oc.write(ks, vs, w.src_dtype, sm)
    return oc


def gpu_rows(c, slots):
    """Raw cache bytes of the given slots from the device: (k, v, kv_scale)."""
    H = c.num_kv_heads
    rb = c.k.numel() // (c.num_slots * H)
    s = dev(np.asarray(slots, np.int64))
    k = c.k.view(c.num_slots, H, rb)[s].cpu().numpy()
    v = c.v.view(c.num_slots, H, rb)[s].cpu().numpy()
    sc = None
    if c.kv_scale is not None:
        per = c.kv_scale.numel() // (c.num_slots * H)
        sc = c.kv_scale.view(c.num_slots, H, per)[s].cpu().numpy()
    return k, v, sc


def assert_rows_equal(c, oc, slots):
    k, v, sc = gpu_rows(c, slots)
    slots = np.asarray(slots, np.int64)
    np.testing.assert_array_equal(k, oc.k[slots])
    np.testing.assert_array_equal(v, oc.v[slots])
    if sc is not None:
        want = oc.kv_scale[slots]
        if want.dtype == np.float32:
            np.testing.assert_array_equal(sc.view(np.uint32), want.view(np.uint32))
        else:                                   # block-scale bytes [n][H][2][D/16]
            np.testing.assert_array_equal(sc, want.reshape(sc.shape))


def run_attention(c, w, num_splits=1, out_dtype=None, lse=True, decode=None, topk_idx=None,
                  row_seq=None, q=None, sm_scale=None):
    """HIP sparse attention through the C ABI -> (out float64, lse float64)."""
    q = (w.q if q is None else q).cuda().contiguous()
    R, Hq, D = q.shape
    odt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[
        out_dtype or w.out_dtype]
    out = torch.full((R, Hq, D), float("nan"), dtype=odt, device="cuda")
    lse_t = torch.full((R, Hq), float("nan"), dtype=torch.float32, device="cuda") if lse else None
    idx = dev(w.topk_idx if topk_idx is None else topk_idx, torch.int32)
    rs = dev(w.row_seq if row_seq is None else row_seq, torch.int32)
    bt = dev(w.block_table, torch.int32)
    sm = w.sm_scale if sm_scale is None else sm_scale
    use_decode = (num_splits != 1) if decode is None else decode
    if use_decode:
        nb = qsakv.qsa_decode_workspace_bytes(R, Hq, D, num_splits)
        ws = torch.zeros(max(nb, 1), dtype=torch.uint8, device="cuda")
        qsakv.qsa_sparse_attn_decode(c, q, rs, bt, idx, sm, out, num_splits, ws, lse=lse_t)
    else:
        qsakv.qsa_sparse_attn_prefill(c, q, rs, bt, idx, sm, out, lse=lse_t)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    l = None if lse_t is None else lse_t.cpu().numpy().astype(np.float64)
    return o, l


def oracle_attention(oc, w, rows=None, topk_idx=None, row_seq=None, q=None, sm_scale=None):
    q = w.q if q is None else q
    return oatt.sparse_attention(
        oc, wl.to_numpy_src(q), w.q_dtype, w.row_seq if row_seq is None else row_seq,
        w.block_table, w.topk_idx if topk_idx is None else topk_idx,
        w.sm_scale if sm_scale is None else sm_scale, rows=rows)


def check(got_o, got_l, ref_o, ref_l, what=""):
    ok = oatt.within_tolerance(got_o, ref_o, ATOL, RTOL)
    m = oatt.metrics(got_o, ref_o)
    if not ok.all():
        bad = np.argwhere(~ok)[:5]
        raise AssertionError("%s: %d/%d outside tolerance; first %s got %s ref %s; %s" % (
            what, int((~ok).sum()), ok.size, bad.tolist(),
            [got_o[tuple(b)] for b in bad], [ref_o[tuple(b)] for b in bad], m))
    if got_l is not None:
        fin = np.isfinite(ref_l)
        assert np.array_equal(np.isfinite(got_l), fin), what + ": lse finiteness differs"
        assert np.all(got_l[~fin] == ref_l[~fin]), what + ": empty-row lse"
        if fin.any():
            d = np.max(np.abs(got_l[fin] - ref_l[fin]))
            assert d <= LSE_ATOL, "%s: lse max |diff| %g" % (what, d)
    return m


def needed_tokens(w, rows):
    """Token indices (into k_src) that the listed rows attend to, for
    workloads whose slot_mapping covers every position they list."""
    inv = np.full(int(w.slot_mapping.max()) + 1, -1, np.int64)
    inv[w.slot_mapping] = np.arange(w.slot_mapping.size)
    want = []
    for r in rows:
        b = int(w.row_seq[r])
        pos = w.topk_idx[r].astype(np.int64)
        pos = pos[pos >= 0]
        want.append(w.block_table[b][pos // w.block_size].astype(np.int64) * w.block_size
                    + pos % w.block_size)
    toks = inv[np.unique(np.concatenate(want))]
    assert np.all(toks >= 0)
    return toks
