"""GPU parity of the sparse-attention entry points against the fp64 oracle:
every cache kind, prefill and split-K decode, layouts, edge cases."""

import numpy as np
import pytest
import torch

from oracle import formats as ofmt
from quantized_kv_top_amd import qsakv
from quantized_kv_top_amd import workloads as wl

from parity_util import (check, dev, e4m3_scales, gpu_write, layer_scales, oracle_attention,
                         oracle_write, run_attention, say)

pytestmark = pytest.mark.gpu

KINDS = ["int8", "int8_inline", "e4m3", "bf16", "nvfp4"]


def _setup(kind, w):
    ks, vs = layer_scales(kind, w)
    c = gpu_write(kind, w, ks or 1.0, vs or 1.0)
    oc = oracle_write(kind, w, ks, vs)
    return c, oc


def small_workload(seed=7, Hq=8, Hkv=2, D=256, BS=16, ctx=700, rows=12, topk=100,
                   q_dtype="bf16", src="bf16", pad=0):
    """A multi-tile case with a ragged tail: ``topk`` positions per row drawn
    from each row's causal prefix, in random order, plus ``pad`` -1 entries."""
    rng = np.random.default_rng(seed)
    nb = -(-ctx // BS)
    pool = nb + 7
    bt = wl.scattered_block_table(rng, 2, nb, 2 * nb + 11).astype(np.int32)
    pool = 2 * nb + 11
    T = 2 * ctx
    slots = np.concatenate([wl.slot_mapping_for(bt, b, np.arange(ctx), BS) for b in range(2)])
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[src]
    k = wl.normal((T, Hkv, D), seed + 1, "cpu", tdt)
    v = wl.normal((T, Hkv, D), seed + 2, "cpu", tdt)
    qdt = torch.bfloat16 if q_dtype == "bf16" else torch.float16
    q = wl.normal((rows, Hq, D), seed + 3, "cpu", qdt)
    row_seq = (np.arange(rows) % 2).astype(np.int32)
    idx = np.full((rows, topk + pad), -1, np.int32)
    for r in range(rows):
        p = ctx - 1 - r
        sel = rng.permutation(wl.draw_sorted_distinct(rng, min(topk, p + 1), 0, p))
        idx[r, :sel.size] = sel
        idx[r] = rng.permutation(idx[r])
    return wl.Workload("small", Hq, Hkv, D, BS, pool, q_dtype, "fp32", src, k, v, slots, q,
                       row_seq, bt, idx, wl.sm_scale_for(D))


@pytest.mark.parametrize("kind", KINDS)
def test_tiny_prefill(kind):
    w = wl.tiny()
    c, oc = _setup(kind, w)
    say("tiny prefill", kind)
    o, l = run_attention(c, w)
    ro, rl = oracle_attention(oc, w)
    check(o, l, ro, rl, "tiny " + kind)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("D", [128, 256])
def test_small_multitile(kind, D):
    w = small_workload(D=D, q_dtype="bf16", pad=9)
    c, oc = _setup(kind, w)
    ro, rl = oracle_attention(oc, w)
    for od in ["fp32", "bf16", "fp16"]:
        say("small", kind, D, od)
        o, l = run_attention(c, w, out_dtype=od)
        check(o, l, ro, rl, "small %s D%d %s" % (kind, D, od))


@pytest.mark.parametrize("kind", ["int8", "int8_inline", "e4m3", "nvfp4"])
def test_fp16_queries(kind):
    w = small_workload(seed=11, q_dtype="fp16", src="fp16", D=128, Hq=32, Hkv=4, topk=77)
    c, oc = _setup(kind, w)
    say("fp16 q", kind)
    o, l = run_attention(c, w, out_dtype="fp16")
    ro, rl = oracle_attention(oc, w)
    check(o, l, ro, rl, "fp16 q " + kind)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("P", [1, 2, 3, 8, 16, 64])
def test_decode_splits(kind, P):
    w = small_workload(seed=5, topk=150, rows=6)
    c, oc = _setup(kind, w)
    ro, rl = oracle_attention(oc, w)
    say("decode", kind, "P", P)
    o, l = run_attention(c, w, num_splits=P, decode=True)
    check(o, l, ro, rl, "decode %s P%d" % (kind, P))


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("D", [128, 256])
def test_workgroup_shapes(kind, D):
    """40 rows x 2 KV heads x P partitions = 80 .. 2560 workgroup items: the
    launch spreads an item over 8, 4, 2 or 1 waves by item count, and every
    shape must give the oracle's result."""
    w = small_workload(seed=23, D=D, rows=40, topk=150)
    c, oc = _setup(kind, w)
    ro, rl = oracle_attention(oc, w)
    for P in [1, 4, 8, 16, 32]:
        say("wg shapes", kind, D, "P", P)
        o, l = run_attention(c, w, num_splits=P, decode=P > 1)
        check(o, l, ro, rl, "wg shapes %s D%d P%d" % (kind, D, P))


# (waves per workgroup, rows, positions one workgroup resolves per LDS batch):
# with 8 KV heads the rows give 32, 520, 1040 and 2056 workgroup items, one
# for each wave count the launch picks by item count.
_SHAPES = [(8, 4, 1024), (2, 65, 512), (1, 130, 256), (4, 257, 1024)]


@pytest.mark.parametrize("nw,rows,batch", _SHAPES, ids=["nw%d" % s[0] for s in _SHAPES])
@pytest.mark.parametrize("extra", [0, 1, "2x"])
def test_list_length_at_lds_batch_edges(nw, rows, batch, extra):
    """A row's list exactly one LDS batch of positions long, one position
    longer, and a little over two batches: the single-batch and the batched
    tile loops meet at these lengths, for every workgroup shape.  The list
    carries 3 padding entries; large launches are checked on sampled rows."""
    width = batch + (batch + 37 if extra == "2x" else extra)
    kinds = ["int8", "nvfp4"] if extra == 1 else ["int8"]
    w = small_workload(seed=41 + nw, Hq=8, Hkv=8, D=128, ctx=width + rows + 3, rows=rows,
                       topk=width - 3, pad=3)
    assert w.topk_idx.shape[1] == width
    rng = np.random.default_rng(nw)
    pick = np.unique(np.concatenate([[0, rows - 1], rng.integers(0, rows, 10)]))
    for kind in kinds:
        c, oc = _setup(kind, w)
        ro, rl = oracle_attention(oc, w, rows=pick)
        say("lds batch edge", kind, "nw", nw, "rows", rows, "width", width)
        o, l = run_attention(c, w)
        check(o[pick], l[pick], ro, rl, "batch edge %s nw%d width %d" % (kind, nw, width))


@pytest.mark.parametrize("G", [1, 4, 16])
def test_group_sizes(G):
    w = small_workload(seed=13, Hq=2 * G, Hkv=2, D=128, topk=40)
    c, oc = _setup("int8", w)
    say("group", G)
    o, l = run_attention(c, w)
    ro, rl = oracle_attention(oc, w)
    check(o, l, ro, rl, "G%d" % G)


def test_layouts_give_identical_bits():
    """The aligned side-tensor and inline-260 layouts hold the same values, so
    the attention outputs must be bitwise equal."""
    w = small_workload(seed=17, topk=300, rows=8)
    a = gpu_write("int8", w)
    b = gpu_write("int8_inline", w)
    oa, la = run_attention(a, w, out_dtype="fp32")
    ob, lb = run_attention(b, w, out_dtype="fp32")
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_permuted_block_table_same_bits():
    w = small_workload(seed=19, topk=120, rows=6)
    a = gpu_write("int8", w)
    oa, la = run_attention(a, w, out_dtype="fp32")
    # move every block to a different physical block
    rng = np.random.default_rng(3)
    perm = rng.permutation(w.num_blocks).astype(np.int32)
    w2 = small_workload(seed=19, topk=120, rows=6)
    w2.block_table = perm[w2.block_table]
    w2.slot_mapping = (perm[w2.slot_mapping // w2.block_size].astype(np.int64) * w2.block_size
                       + w2.slot_mapping % w2.block_size)
    b = gpu_write("int8", w2)
    ob, lb = run_attention(b, w2, out_dtype="fp32")
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_deterministic():
    w = small_workload(seed=23, topk=200)
    c = gpu_write("int8", w)
    o1, l1 = run_attention(c, w, out_dtype="fp32")
    o2, l2 = run_attention(c, w, out_dtype="fp32")
    o3, l3 = run_attention(c, w, num_splits=8, out_dtype="fp32")
    o4, l4 = run_attention(c, w, num_splits=8, out_dtype="fp32")
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.array_equal(o3, o4) and np.array_equal(l3, l4)


def test_edge_cases():
    """topk = 1, all-padding rows, invalid sequence ids, out-of-range
    positions, out-of-range block-table entries, duplicates."""
    w = small_workload(seed=29, topk=40, rows=8)
    c, oc = _setup("int8", w)
    idx = w.topk_idx.copy()
    idx[0] = -1                                   # empty row
    idx[1, 1:] = -1                               # a single position
    idx[2, :5] = 10 ** 6                          # beyond the block table
    idx[3, 3] = idx[3, 2]                         # a duplicate (counts twice)
    row_seq = w.row_seq.copy()
    row_seq[4] = 7                                # no such sequence
    ref_idx = idx.copy()
    ref_idx[2, :5] = -1
    ref_rs = row_seq.copy()
    ref_rs[4] = 0
    ref_idx[4] = -1
    for P in (1, 4):
        say("edge P", P)
        o, l = run_attention(c, w, num_splits=P, decode=P > 1, topk_idx=idx, row_seq=row_seq)
        ro, rl = oracle_attention(oc, w, topk_idx=ref_idx, row_seq=ref_rs)
        check(o, l, ro, rl, "edge P%d" % P)
        assert np.all(o[0] == 0) and np.all(np.isneginf(l[0]))
        assert np.all(o[4] == 0) and np.all(np.isneginf(l[4]))
    # block-table entries outside the cache are padding too
    bt = w.block_table.copy()
    bt[0, 0] = w.num_blocks + 5
    bt[1, 1] = -3
    w2 = small_workload(seed=29, topk=40, rows=8)
    w2.block_table = bt
    o, l = run_attention(c, w2)
    ref_idx = w2.topk_idx.copy()
    for r in range(w2.num_rows):
        b = w2.row_seq[r]
        lb = ref_idx[r] // w2.block_size
        bad = ((b == 0) & (lb == 0)) | ((b == 1) & (lb == 1))
        ref_idx[r][bad & (ref_idx[r] >= 0)] = -1
    ro, rl = oracle_attention(oc, w, topk_idx=ref_idx)
    check(o, l, ro, rl, "bad block table")


def _without_block0(w):
    """Move whatever uses physical block 0 to an unused block, so that slot 0
    (the row every padding token reads) is never attended."""
    used = set(np.unique(w.block_table).tolist())
    spare = next(b for b in range(1, w.num_blocks) if b not in used)
    bt = w.block_table.copy()
    bt[bt == 0] = spare
    blk = w.slot_mapping // w.block_size
    w.slot_mapping = np.where(blk == 0, spare, blk) * w.block_size + w.slot_mapping % w.block_size
    w.block_table = bt
    return w


def _poison_slot0(c):
    """NaN / inf in everything slot 0 holds: int8 scales (side tensor and
    inline slot), E4M3 NaN codes, bf16 NaNs, NVFP4 NaN block-scale codes."""
    H, D = c.num_kv_heads, c.head_dim
    bad = np.array([np.nan, np.inf, -np.inf, np.nan][:H] + [np.nan] * max(0, H - 4), np.float32)
    if c.kind == "int8":
        c.kv_scale.view(c.num_slots, H, 2)[0] = dev(np.stack([bad, bad[::-1]], axis=1))
    elif c.kind == "int8_inline":
        for t in (c.k, c.v):
            t.view(c.num_slots, H, D + 4)[0, :, D:] = dev(bad.view(np.uint8).reshape(H, 4))
    elif c.kind == "e4m3":
        c.k.view(c.num_slots, H, D)[0] = 0x7F
        c.v.view(c.num_slots, H, D)[0] = 0xFF
    elif c.kind == "bf16":
        nan = np.tile(np.array([0xC0, 0x7F], np.uint8), (H, D))   # bf16 NaN 0x7FC0
        c.k.view(c.num_slots, H, 2 * D)[0] = dev(nan)
        c.v.view(c.num_slots, H, 2 * D)[0] = dev(nan)
    elif c.kind == "nvfp4":
        c.kv_scale.view(c.num_slots, H, 2 * (D // 16))[0] = 0x7F


@pytest.mark.parametrize("kind", KINDS)
def test_padding_never_reads_slot0_values(kind):
    """Padding entries (-1, positions past the block table, rows of an
    invalid sequence) and the padded tail of the last tile read slot 0 as a
    stand-in; NaN / inf stored there must not reach any output, for lists of
    every tile phase, at P = 1 and P = 8."""
    w = _without_block0(small_workload(seed=47, topk=133, rows=10, pad=15))
    c, oc = _setup(kind, w)
    _poison_slot0(c)
    idx = w.topk_idx.copy()
    idx[0] = -1                                   # an empty row
    idx[1, 1:] = -1                               # one position, 15 pads in its tile
    idx[2, :7] = 10 ** 6                          # beyond the block table
    ref_idx = idx.copy()
    ref_idx[2, :7] = -1
    for P in (1, 8):
        say("padding vs poisoned slot 0", kind, "P", P)
        o, l = run_attention(c, w, num_splits=P, decode=P > 1, topk_idx=idx)
        assert np.isfinite(o).all(), "non-finite output"
        ro, rl = oracle_attention(oc, w, topk_idx=ref_idx)
        check(o, l, ro, rl, "poisoned slot 0 %s P%d" % (kind, P))


def test_equal_keys_give_uniform_softmax():
    """Closed form through the whole HIP path: identical keys -> the output is
    the mean of the selected values."""
    w = small_workload(seed=31, topk=64, rows=4, D=128)
    key = w.k_src[:1].clone()
    w.k_src = key.expand_as(w.k_src).contiguous()
    c, oc = _setup("int8", w)
    o, l = run_attention(c, w, out_dtype="fp32")
    ro, rl = oracle_attention(oc, w)
    check(o, l, ro, rl, "equal keys")
    slots = [w.block_table[w.row_seq[r]][p // w.block_size] * w.block_size + p % w.block_size
             for r in range(4) for p in [w.topk_idx[r][w.topk_idx[r] >= 0]]]
    for r in range(4):
        vh = oc.dequant(np.asarray(slots[r], np.int64), "v")
        G = w.num_q_heads // w.num_kv_heads
        for h in range(w.num_q_heads):
            mean = vh[:, h // G, :].mean(axis=0)
            assert np.allclose(o[r, h], mean, atol=2e-3, rtol=1e-2)


def test_zero_value_rows_and_large_queries():
    """Zero V rows (scale 0) and bf16 queries far from unit magnitude (the
    fp16 prescale path)."""
    w = small_workload(seed=37, topk=90, rows=6)
    v = w.v_src.clone()
    v[::3] = 0
    w.v_src = v
    q = w.q.float()
    q[0] *= 3e4
    q[1] *= 1e-5
    q[2, :, ::2] *= 1e-20
    w.q = q.to(torch.bfloat16)
    c, oc = _setup("int8", w)
    o, l = run_attention(c, w, out_dtype="fp32", sm_scale=w.sm_scale * 1e-3)
    ro, rl = oracle_attention(oc, w, sm_scale=w.sm_scale * 1e-3)
    check(o, l, ro, rl, "zero V / large q")


def outlier_logit_workload(seed, rows=48, topk=1024, ctx=4096, q_mean=0.75, q_out=5.0,
                           k_out=30.0):
    """The prefill layer shape (Hq 16 / Hkv 2, D 256, block 64) with K rows
    dominated by 4 outlier channels (N(0,1) x ``k_out``) and queries of mean
    ``q_mean`` whose outlier channels carry +-``q_out``: per-head logits that
    reach 20-80, set mostly by one or two channels of each key, with a large
    sum of the query over the head dimension."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, BS = 16, 2, 256, 64
    nb = ctx // BS
    bt = wl.scattered_block_table(rng, 1, nb, nb + 13).astype(np.int32)
    slots = wl.slot_mapping_for(bt, 0, np.arange(ctx), BS)
    chans = np.sort(rng.permutation(D)[:4])
    k = wl.normal((ctx, Hkv, D), seed + 1, "cpu")
    k[:, :, chans] *= k_out
    v = wl.normal((ctx, Hkv, D), seed + 2, "cpu")
    q = wl.normal((rows, Hq, D), seed + 3, "cpu") + q_mean
    sign = torch.from_numpy(rng.choice([-1.0, 1.0], size=(rows, Hq, 4)).astype(np.float32))
    q[:, :, chans] = q_out * sign
    idx = np.stack([wl.draw_sorted_distinct(rng, topk, 0, ctx - rows + r)
                    for r in range(rows)]).astype(np.int32)
    return wl.Workload("outlier-logits", Hq, Hkv, D, BS, nb + 13, "bf16", "bf16", "bf16",
                       k.to(torch.bfloat16), v.to(torch.bfloat16), slots, q.to(torch.bfloat16),
                       np.zeros(rows, np.int32), bt, idx, wl.sm_scale_for(D))


@pytest.mark.parametrize("kind", ["int8", "int8_inline"])
def test_int8_large_logits_outlier_keys(kind):
    """Large logits from outlier-dominated int8 keys and nonzero-mean
    queries: each logit must keep the accuracy of its own products (a
    constant offset on the codes, times the query's sum over the head
    dimension, must not set the rounding error).  Prefill and split-K 8, at
    the stated tolerance; the workload's logits are checked to reach the
    20-80 range so that the case is the one meant."""
    w = outlier_logit_workload(53)
    c, oc = _setup(kind, w)
    # the oracle's logits of a few rows: the case must reach 20-80
    qn = w.q.float().numpy().astype(np.float64)
    top = []
    for r in range(0, w.num_rows, 8):
        sl = w.block_table[0][w.topk_idx[r] // 64].astype(np.int64) * 64 + w.topk_idx[r] % 64
        kh = oc.dequant(sl, "k")                                  # [topk][Hkv][D]
        lg = np.einsum("hd,thd->ht", qn[r], np.repeat(kh, 8, axis=1)) * w.sm_scale
        top.append(lg.max(axis=1))
    top = np.concatenate(top)
    say("outlier logits: per-head max logit %.1f .. %.1f" % (top.min(), top.max()))
    assert top.max() >= 60 and np.median(top) >= 20
    ro, rl = oracle_attention(oc, w)
    for P in (1, 8):
        o, l = run_attention(c, w, num_splits=P, decode=P > 1)
        m = check(o, l, ro, rl, "outlier logits %s P%d" % (kind, P))
        say("outlier logits", kind, "P", P, m)


def test_every_e4m3_code_decodes_exactly():
    """Write all 254 finite E4M3 codes as V rows directly into the cache and
    read each back with top-k = 1: out = decode(code) * v_scale exactly."""
    D, Hkv, BS = 128, 1, 16
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    n = codes.size
    NB = -(-n // BS)
    c = qsakv.Cache("e4m3", NB, BS, Hkv, D, k_scale=1.0, v_scale=0.75)
    vrows = np.repeat(codes[:, None], D, axis=1)
    c.v.view(NB * BS, D)[:n] = dev(vrows)
    q = torch.zeros(n, 1, D, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(n, 1, D, dtype=torch.float32, device="cuda")
    lse = torch.empty(n, 1, dtype=torch.float32, device="cuda")
    bt = dev(np.arange(NB, dtype=np.int32)[None], torch.int32)
    idx = dev(np.arange(n, dtype=np.int32)[:, None], torch.int32)
    rs = torch.zeros(n, dtype=torch.int32, device="cuda")
    qsakv.qsa_sparse_attn_prefill(c, q, rs, bt, idx, 0.1, out, lse=lse)
    torch.cuda.synchronize()
    want = ofmt.e4m3_decode(codes) * 0.75
    got = out.cpu().numpy()
    assert np.array_equal(got, np.repeat(want[:, None, None], D, axis=2).astype(np.float32))
    assert np.all(lse.cpu().numpy() == 0)


@pytest.mark.parametrize("D", [128, 256])
def test_every_fp4_byte_decodes_exactly(D):
    """V rows holding every byte value (two E2M1 codes) with every V block
    scaled by a different E4M3 code; read back with top-k = 1: out =
    e2m1(code) * block scale * v_scale exactly (element 2j from the low
    nibble of byte j)."""
    Hkv, BS = 1, 16
    n = 256
    NB = -(-n // BS)
    c = qsakv.Cache("nvfp4", NB, BS, Hkv, D, k_scale=1.0, v_scale=0.375)
    rng = np.random.default_rng(3)
    vbytes = np.stack([np.roll(np.arange(256, dtype=np.uint8), r)[:D // 2] for r in range(n)])
    c.v.view(NB * BS, D // 2)[:n] = dev(vbytes)
    nb = D // 16
    scodes = rng.integers(1, 0x7F, size=(n, nb)).astype(np.uint8)      # finite, positive
    sc = np.zeros((NB * BS, 2, nb), np.uint8)
    sc[:n, 1] = scodes
    sc[:n, 0] = 0x38                                                     # K blocks: 1.0
    c.kv_scale.copy_(dev(sc.reshape(-1)))
    q = torch.zeros(n, 1, D, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(n, 1, D, dtype=torch.float32, device="cuda")
    bt = dev(np.arange(NB, dtype=np.int32)[None], torch.int32)
    idx = dev(np.arange(n, dtype=np.int32)[:, None], torch.int32)
    rs = torch.zeros(n, dtype=torch.int32, device="cuda")
    qsakv.qsa_sparse_attn_prefill(c, q, rs, bt, idx, 0.1, out)
    torch.cuda.synchronize()
    want = ofmt.nvfp4_dequantize(ofmt.nvfp4_unpack(vbytes), scodes, 0.375)
    np.testing.assert_array_equal(out.cpu().numpy()[:, 0], want.astype(np.float32))


def test_every_int8_code_decodes_exactly():
    D, Hkv, BS = 256, 1, 16
    codes = np.arange(-127, 128, dtype=np.int8)
    n = codes.size
    NB = -(-n // BS)
    c = qsakv.Cache("int8", NB, BS, Hkv, D)
    c.v.view(NB * BS, D)[:n] = dev(np.repeat(codes.view(np.uint8)[:, None], D, axis=1))
    s = np.float32(0.0371)
    c.kv_scale.view(NB * BS, 2)[:n, 1] = float(s)
    c.kv_scale.view(NB * BS, 2)[:n, 0] = 1.0
    q = torch.zeros(n, 1, D, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(n, 1, D, dtype=torch.float32, device="cuda")
    bt = dev(np.arange(NB, dtype=np.int32)[None], torch.int32)
    idx = dev(np.arange(n, dtype=np.int32)[:, None], torch.int32)
    rs = torch.zeros(n, dtype=torch.int32, device="cuda")
    qsakv.qsa_sparse_attn_prefill(c, q, rs, bt, idx, 0.1, out)
    torch.cuda.synchronize()
    want = codes.astype(np.float64) * np.float64(s)
    got = out.cpu().numpy()[:, 0, 0].astype(np.float64)
    np.testing.assert_allclose(got, want, rtol=2e-7, atol=0)


def test_e4m3_scale_folding():
    """k_scale = c equals k_scale = 1 with sm_scale * c; v_scale = c scales
    the output by c -- on the same stored codes."""
    w = small_workload(seed=41, D=128, topk=120, rows=6)
    ks, vs = e4m3_scales(w)
    a = gpu_write("e4m3", w, ks, vs)
    b = qsakv.Cache("e4m3", w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim,
                    k_scale=1.0, v_scale=1.0)
    b.k.copy_(a.k)
    b.v.copy_(a.v)
    oa, la = run_attention(a, w, out_dtype="fp32")
    ob, lb = run_attention(b, w, out_dtype="fp32", sm_scale=w.sm_scale * ks)
    np.testing.assert_allclose(oa, vs * ob, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(la, lb, rtol=1e-5, atol=1e-5)


def test_decode_workspace_reuse():
    """One workspace (contents arbitrary) serves repeated split-K calls, also
    with fewer rows."""
    w = small_workload(seed=43, topk=150, rows=6)
    c, oc = _setup("int8", w)
    ro, rl = oracle_attention(oc, w)
    R, Hq, D = w.q.shape
    nb = qsakv.qsa_decode_workspace_bytes(R, Hq, D, 8)
    ws = torch.full((nb,), 0xA5, dtype=torch.uint8, device="cuda")
    q = w.q.cuda()
    rs = dev(w.row_seq, torch.int32)
    bt = dev(w.block_table, torch.int32)
    idx = dev(w.topk_idx, torch.int32)
    for rows in (R, R, 3, R):
        say("workspace reuse, rows", rows)
        out = torch.full((rows, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((rows, Hq), float("nan"), dtype=torch.float32, device="cuda")
        qsakv.qsa_sparse_attn_decode(c, q[:rows].contiguous(), rs[:rows].contiguous(), bt,
                                     idx[:rows].contiguous(), w.sm_scale, out, 8, ws, lse=lse)
        torch.cuda.synchronize()
        check(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
              ro[:rows], rl[:rows], "reuse rows %d" % rows)


def test_graph_replays_match_eager():
    """Write, prefill, split-K decode and calibration statistics captured in
    one HIP graph: every replay (with eager work and synchronizations in
    between) reproduces the eager results bit for bit."""
    w = small_workload(seed=41, topk=200, rows=10)
    c = qsakv.Cache("int8", w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, "cuda")
    ks, vs = w.k_src.cuda(), w.v_src.cuda()
    sm = dev(w.slot_mapping, torch.int64)
    q = w.q.cuda().contiguous()
    rs, bt, idx = dev(w.row_seq, torch.int32), dev(w.block_table, torch.int32), \
        dev(w.topk_idx, torch.int32)
    R, Hq, D = q.shape
    out1 = torch.empty((R, Hq, D), dtype=torch.bfloat16, device="cuda")
    out2 = torch.empty_like(out1)
    lse = torch.empty((R, Hq), dtype=torch.float32, device="cuda")
    ws = torch.zeros(qsakv.qsa_decode_workspace_bytes(R, Hq, D, 8), dtype=torch.uint8,
                     device="cuda")
    cres = torch.zeros(64, dtype=torch.uint8, device="cuda")
    cws = torch.zeros(qsakv.calib_workspace_bytes(), dtype=torch.uint8, device="cuda")
    xs = ks.reshape(-1)

    def step(stream):
        qsakv.kv_quant_write(c, ks, vs, sm, stream=stream)
        qsakv.qsa_sparse_attn_prefill(c, q, rs, bt, idx, w.sm_scale, out1, lse=lse,
                                      stream=stream)
        qsakv.qsa_sparse_attn_decode(c, q, rs, bt, idx, w.sm_scale, out2, 8, ws, stream=stream)
        qsakv.kv_calib_stats(xs, 0.05, cres, cws, stream=stream)

    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [t.clone() for t in (c.k, c.kv_scale, out1, lse, out2, cres)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step(s)
    for i in range(3):
        for t in (c.k, c.kv_scale, out1, lse, out2, cres, ws, cws):
            t.zero_()                    # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say("graph replay", i)
        for a, b in zip((c.k, c.kv_scale, out1, lse, out2, cres), ref):
            assert torch.equal(a, b)


def _random_case(seed):
    """A seeded random configuration: block size 1..1024, G 1..16, D 128 or
    256, cache kind, query / output dtypes, list length (up to several LDS
    chunks of 1024 positions, with padding and duplicates), split count."""
    rng = np.random.default_rng(seed)
    kind = KINDS[rng.integers(len(KINDS))]
    D = int(rng.choice([128, 256]))
    BS = int(2 ** rng.integers(0, 11))
    G = int(rng.choice([1, 2, 3, 4, 8, 16]))
    Hkv = int(rng.integers(1, 4))
    ctx = int(rng.integers(64, 3000))
    topk = int(rng.integers(1, min(ctx, 2600) + 1))
    rows = int(rng.integers(1, 7))
    q_dtype = "bf16" if kind == "bf16" else str(rng.choice(["bf16", "fp16"]))
    src = "fp16" if q_dtype == "fp16" else "bf16"
    w = small_workload(seed=seed, Hq=G * Hkv, Hkv=Hkv, D=D, BS=BS, ctx=ctx, rows=rows,
                       topk=topk, q_dtype=q_dtype, src=src, pad=int(rng.integers(0, 5)))
    idx = w.topk_idx.copy()
    if topk > 2:                         # a duplicated position in some rows
        idx[0, 1] = idx[0, 0]
    w.topk_idx = idx
    P = int(rng.choice([1, 1, 2, 5, 8, 33]))
    od = str(rng.choice(["fp32", "bf16", "fp16"]))
    return kind, w, P, od


@pytest.mark.parametrize("seed", list(range(100, 260)))
def test_random_configurations(seed):
    kind, w, P, od = _random_case(seed)
    say("random", seed, kind, "D", w.head_dim, "BS", w.block_size, "G",
        w.num_q_heads // w.num_kv_heads, "Hkv", w.num_kv_heads, "topk", w.topk, "P", P, od)
    c, oc = _setup(kind, w)
    ro, rl = oracle_attention(oc, w)
    o, l = run_attention(c, w, num_splits=P, out_dtype=od, decode=P > 1)
    check(o, l, ro, rl, "random seed %d" % seed)
