"""GPU parity of qsa_sparse_attn_decode_noalloc (split-K partials in the
library's static per-GPU scratch) with qsa_sparse_attn_decode (a caller
workspace): the same kernels, so the outputs must be bitwise equal -- on
calls in a row that reuse the scratch, the later ones smaller, and on a
call that fills the scratch almost to its limit."""

import numpy as np
import pytest
import torch

from quantized_kv_top_amd import qsakv
from quantized_kv_top_amd import workloads as wl

from parity_util import check, dev, gpu_write, layer_scales, oracle_attention, oracle_write, say

pytestmark = pytest.mark.gpu


def _case(seed, kind, rows, Hq, Hkv, D, topk, ctx=3000, BS=64):
    rng = np.random.default_rng(seed)
    nb = -(-ctx // BS)
    bt = wl.scattered_block_table(rng, 2, nb, 2 * nb + 5).astype(np.int32)
    slots = np.concatenate([wl.slot_mapping_for(bt, b, np.arange(ctx), BS) for b in range(2)])
    src = torch.float16 if kind == "e4m3" else torch.bfloat16
    k = wl.normal((2 * ctx, Hkv, D), seed + 1, "cpu", src)
    v = wl.normal((2 * ctx, Hkv, D), seed + 2, "cpu", src)
    qdt = torch.float16 if kind == "e4m3" else torch.bfloat16
    q = wl.normal((rows, Hq, D), seed + 3, "cpu", qdt)
    row_seq = (np.arange(rows) % 2).astype(np.int32)
    idx = np.full((rows, topk), -1, np.int32)
    for r in range(rows):
        n = topk - (r % 7)                       # ragged lists, -1 padded
        idx[r, :n] = wl.draw_sorted_distinct(rng, n, 0, ctx - 1 - (r % 5))
    return wl.Workload("noalloc", Hq, Hkv, D, BS, 2 * nb + 5, "fp16" if kind == "e4m3" else "bf16",
                       "bf16", "fp16" if kind == "e4m3" else "bf16", k, v, slots, q, row_seq, bt,
                       idx, wl.sm_scale_for(D))


def _both(c, w, P):
    """(workspace result, no-alloc result) as (out, lse) device tensors."""
    q = w.q.cuda().contiguous()
    R, Hq, D = q.shape
    rs, bt, idx = dev(w.row_seq, torch.int32), dev(w.block_table, torch.int32), \
        dev(w.topk_idx, torch.int32)
    res = []
    for noalloc in (False, True):
        out = torch.full((R, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((R, Hq), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            qsakv.qsa_sparse_attn_decode_noalloc(c, q, rs, bt, idx, w.sm_scale, out, P, lse=lse)
        else:
            nb = qsakv.qsa_decode_workspace_bytes(R, Hq, D, P)
            ws = torch.full((max(nb, 256),), 0x5A, dtype=torch.uint8, device="cuda")
            qsakv.qsa_sparse_attn_decode(c, q, rs, bt, idx, w.sm_scale, out, P, ws, lse=lse)
        torch.cuda.synchronize()
        res.append((out, lse))
    return res


@pytest.mark.parametrize("kind", ["int8", "e4m3"])
def test_noalloc_decode_matches_workspace_decode(kind):
    D, Hq, Hkv = (256, 16, 2) if kind == "int8" else (128, 32, 4)
    # the first call nearly fills the scratch (127 rows x 16 heads x 8 splits
    # at D = 256 is 16,776,192 of 16,777,216 bytes); the next ones are smaller
    calls = [(127, 8, 300), (9, 5, 200), (3, 8, 150), (40, 1, 100)] if kind == "int8" else \
        [(60, 16, 257), (4, 8, 2051 // 8), (1, 3, 64)]
    w0 = _case(61, kind, max(r for r, _, _ in calls), Hq, Hkv, D, max(t for _, _, t in calls))
    ks, vs = layer_scales(kind, w0)
    c = gpu_write(kind, w0, ks or 1.0, vs or 1.0)
    oc = oracle_write(kind, w0, ks, vs)
    for i, (rows, P, topk) in enumerate(calls):
        w = _case(61, kind, rows, Hq, Hkv, D, topk)
        need = qsakv.qsa_decode_workspace_bytes(rows, Hq, D, P)
        assert need <= qsakv.NOALLOC_SCRATCH_BYTES
        say("noalloc", kind, "call", i, "rows", rows, "P", P, "topk", topk, "scratch bytes", need)
        (o1, l1), (o2, l2) = _both(c, w, P)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "outputs differ"
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), "lse differs"
        pick = sorted({0, rows - 1, rows // 2})
        ro, rl = oracle_attention(oc, w, rows=pick)
        check(o2.float().cpu().numpy().astype(np.float64)[pick],
              l2.cpu().numpy().astype(np.float64)[pick], ro, rl, "noalloc %s call %d" % (kind, i))


def test_noalloc_decode_refuses_oversize_calls():
    """A call beyond the scratch fails with QKV_ERR_SCRATCH and leaves the
    output untouched."""
    w = _case(67, "int8", 128, 16, 2, 256, 64)
    c = gpu_write("int8", w)
    q = w.q.cuda().contiguous()
    out = torch.zeros(q.shape, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(qsakv.QsakvError) as e:
        qsakv.qsa_sparse_attn_decode_noalloc(c, q, dev(w.row_seq, torch.int32),
                                             dev(w.block_table, torch.int32),
                                             dev(w.topk_idx, torch.int32), w.sm_scale, out, 8)
    assert e.value.status == qsakv.ERR_SCRATCH
    torch.cuda.synchronize()
    assert int(out.view(torch.int16).abs().max()) == 0
