"""Seeded synthetic inputs for the five workloads (shared by tests and bench).

This module only draws inputs: it holds none of the method's arithmetic (no
quantization, no scale rule, no attention).  Float tensors are drawn with a
seeded ``torch.Generator`` on the requested device; integer structure (block
tables, slot mappings, top-k lists) with ``numpy.random.default_rng(seed)``
on the host, in a fixed draw order.  The same seed on the same device type
gives the same inputs.

The shapes and distributions follow the workloads the pages measure
(shapes only: the pages' data are real model activations):

* tiny      1 seq, Hq 4 / Hkv 1, D 128, ctx 64 in 4 blocks of 16 (physical
            order a seeded permutation), K/V fp32 ~ N(0,1), 4 rows at
            positions 60..63, top-k 16 distinct uniform causal, fp32 out.
* prefill   1 seq, Hq 16 / Hkv 2, D 256, ctx 32768 in blocks of 64 scattered
            over a larger pool, K/V bf16 ~ N(0,1) with 4 outlier channels x10
            per tensor, 2048 rows at 30720..32767, top-k 1024 distinct
            uniform causal, bf16 Q/out (2048 rows / top-k 1024 as on page
            "int8 per-(token,head) KV cache for the Qwen3.8-Flash-Next QSA
            path", section "The finding worth upstreaming").
* decode    8 seqs x ctx 131072, Hq 16 / Hkv 2, D 256, BS 64, K/V bf16 ~
            N(0,1); 5 query rows per seq (1 + 4 speculative) at ctx-5..ctx-1;
            top-k 2048 = 1434 distinct from the last 4096 positions + 614
            distinct from before them, sorted; 8 split-K partitions.
* e4m3      12 layers, 4 seqs x ctx 65536, Hq 32 / Hkv 4, D 128, BS 64
            (one block table for all layers), K/V fp16(0.5 * t_4)
            (Student-t, nu = 4); 1 row per seq at 65535;
            top-k 2051 distinct uniform causal; fp16 Q/out (top-k 2051 as on
            page "[Perf][SM70][FP8] Hoist QSA E4M3 KV scales", section "Test
            plan").
* scores    indexer scores for the top-k selection: the prefill rows
            (2048 x 32768, N(0,1)) and the decode rows (40 x 131072, N(0,1)
            plus 2.2 over each row's last 4096 positions).
* e2e       1 seq, Hq 16 / Hkv 2, D 256, BS 64: 122880 existing tokens, a
            chunk of 8192 new tokens whose rows attend with top-k 1024, then
            8 decode steps (one new token each) with top-k 2048 in the decode
            scheme; blocks spread at random over a fixed 13.75 GiB pool.
"""

from dataclasses import dataclass, field

import numpy as np
import torch

GiB = 1 << 30
E2E_POOL_BYTES = int(13.75 * GiB)     # 14,763,950,080 bytes


# ---------------------------------------------------------------------------
# integer structure
# ---------------------------------------------------------------------------

def draw_sorted_distinct(rng, n, lo, hi):
    """n distinct integers drawn uniformly from [lo, hi], returned sorted.

    Draws with replacement, keeps the distinct values and, if more than n
    remain, keeps a uniformly chosen n of them; every n-subset is equally
    likely.  Small ranges use a permutation instead.
    """
    span = hi - lo + 1
    if n > span:
        raise ValueError("cannot draw %d distinct values from %d" % (n, span))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    if span <= 4 * n:
        return np.sort(rng.permutation(span)[:n] + lo).astype(np.int64)
    while True:
        cand = np.unique(rng.integers(lo, hi + 1, size=n + n // 4 + 16))
        if cand.size >= n:
            pick = rng.permutation(cand.size)[:n]
            return np.sort(cand[pick]).astype(np.int64)


def scattered_block_table(rng, num_seqs, blocks_per_seq, pool_blocks):
    """Each sequence's logical blocks mapped to distinct physical blocks drawn
    at random from a pool of ``pool_blocks``."""
    need = num_seqs * blocks_per_seq
    if need > pool_blocks:
        raise ValueError("pool too small")
    phys = rng.permutation(pool_blocks)[:need].astype(np.int64)
    return phys.reshape(num_seqs, blocks_per_seq)


def slot_mapping_for(block_table, seq, positions, block_size):
    """Slots of the given logical positions of one sequence."""
    pos = np.asarray(positions, dtype=np.int64)
    return block_table[seq][pos // block_size] * block_size + pos % block_size


def decode_topk(rng, pos, topk, window=4096, recent_frac=0.7):
    """top-k list of a decode row: rint(0.7 * topk) distinct positions from the
    last ``window`` positions (pos - window + 1 .. pos) and the rest distinct
    from before them; sorted."""
    n_recent = int(np.rint(recent_frac * topk))
    n_far = topk - n_recent
    lo_recent = max(0, pos - window + 1)
    recent = draw_sorted_distinct(rng, n_recent, lo_recent, pos)
    far = draw_sorted_distinct(rng, n_far, 0, lo_recent - 1) if n_far else np.zeros(0, np.int64)
    return np.sort(np.concatenate([far, recent]))


# ---------------------------------------------------------------------------
# float data
# ---------------------------------------------------------------------------

def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, seed, device, dtype=torch.float32):
    """N(0,1) drawn in float32 and rounded (RNE) to ``dtype``."""
    x = torch.randn(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    return x.to(dtype)


def normal_with_outliers(shape, seed, device, channels, factor=10.0, dtype=torch.bfloat16):
    """N(0,1) with the listed last-axis channels multiplied by ``factor``."""
    x = torch.randn(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    x[..., torch.as_tensor(channels, device=device)] *= factor
    return x.to(dtype)


def student_t4(shape, seed, device, scale=0.5, dtype=torch.float16):
    """scale * T with T ~ Student-t(4): T = Z / sqrt(C / 4), C ~ chi^2_4 drawn as
    -2 ln(U1 U2); rounded (RNE) to ``dtype``."""
    g = _gen(seed, device)
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    u = torch.rand((2,) + tuple(shape), generator=g, device=device, dtype=torch.float32)
    u = u.clamp_min(torch.finfo(torch.float32).tiny)
    chi2 = -2.0 * (torch.log(u[0]) + torch.log(u[1]))
    return (scale * z / torch.sqrt(chi2 / 4.0)).to(dtype)


def sm_scale_for(head_dim):
    """The workloads' softmax scale 1/sqrt(D), as the float32 value both the
    library and the oracle receive."""
    return float(np.float32(1.0 / np.sqrt(head_dim)))


# ---------------------------------------------------------------------------
# workload descriptions
# ---------------------------------------------------------------------------

@dataclass
class Workload:
    """One attention call's inputs plus the tokens written before it."""
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int                  # physical blocks in the layer's cache
    q_dtype: str                     # 'bf16' | 'fp16'
    out_dtype: str                   # 'bf16' | 'fp16' | 'fp32'
    src_dtype: str                   # 'fp32' | 'bf16' | 'fp16'
    k_src: torch.Tensor              # [T][Hkv][D]
    v_src: torch.Tensor
    slot_mapping: np.ndarray         # [T] int64
    q: torch.Tensor                  # [R][Hq][D]
    row_seq: np.ndarray              # [R] int32
    block_table: np.ndarray          # [B][max_blocks] int32
    topk_idx: np.ndarray             # [R][topk] int32
    sm_scale: float
    num_splits: int = 1
    extra: dict = field(default_factory=dict)

    @property
    def num_rows(self):
        return int(self.topk_idx.shape[0])

    @property
    def topk(self):
        return int(self.topk_idx.shape[1])


def tiny(device="cpu", seed=1):
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, BS, ctx = 4, 1, 128, 16, 64
    bt = rng.permutation(ctx // BS).astype(np.int64).reshape(1, -1)
    pos = np.arange(ctx)
    slots = slot_mapping_for(bt, 0, pos, BS)
    rows = np.arange(60, 64)
    topk = np.stack([draw_sorted_distinct(rng, 16, 0, p) for p in rows])
    k = normal((ctx, Hkv, D), seed * 1000 + 1, device)
    v = normal((ctx, Hkv, D), seed * 1000 + 2, device)
    q = normal((len(rows), Hq, D), seed * 1000 + 3, device, torch.bfloat16)
    return Workload("tiny", Hq, Hkv, D, BS, ctx // BS, "bf16", "fp32", "fp32",
                    k, v, slots, q, np.zeros(len(rows), np.int32),
                    bt.astype(np.int32), topk.astype(np.int32), sm_scale_for(D),
                    extra={"positions": rows})


def prefill(device="cpu", seed=2, num_rows=2048, topk=1024, ctx=32768, pool_blocks=640):
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, BS = 16, 2, 256, 64
    nb = ctx // BS
    bt = scattered_block_table(rng, 1, nb, pool_blocks)
    k_out = np.sort(rng.permutation(D)[:4])
    v_out = np.sort(rng.permutation(D)[:4])
    rows = np.arange(ctx - num_rows, ctx)
    topk_idx = np.stack([draw_sorted_distinct(rng, topk, 0, p) for p in rows])
    slots = slot_mapping_for(bt, 0, np.arange(ctx), BS)
    k = normal_with_outliers((ctx, Hkv, D), seed * 1000 + 1, device, k_out)
    v = normal_with_outliers((ctx, Hkv, D), seed * 1000 + 2, device, v_out)
    q = normal((num_rows, Hq, D), seed * 1000 + 3, device, torch.bfloat16)
    return Workload("prefill", Hq, Hkv, D, BS, pool_blocks, "bf16", "bf16", "bf16",
                    k, v, slots, q, np.zeros(num_rows, np.int32), bt.astype(np.int32),
                    topk_idx.astype(np.int32), sm_scale_for(D),
                    extra={"positions": rows, "k_outlier_channels": k_out,
                           "v_outlier_channels": v_out})


def decode(device="cpu", seed=3, num_seqs=8, ctx=131072, rows_per_seq=5, topk=2048,
           pool_blocks=None, num_splits=8, layer=None):
    """The decode workload; ``layer`` = i draws layer i of a model over the
    same sequences: the block table is the model's (drawn from ``seed``
    alone, shared by every layer, as one paged cache serves all layers),
    the lists, queries and K/V are the layer's own."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, BS = 16, 2, 256, 64
    nb = ctx // BS
    pool_blocks = pool_blocks or (num_seqs * nb + num_seqs * nb // 8)
    bt = scattered_block_table(rng, num_seqs, nb, pool_blocks)
    if layer is not None:
        rng = np.random.default_rng([seed, layer])
        seed = seed * 100 + layer
    row_seq, idx, positions = [], [], []
    for b in range(num_seqs):
        for p in range(ctx - rows_per_seq, ctx):
            row_seq.append(b)
            positions.append(p)
            idx.append(decode_topk(rng, p, topk))
    T = num_seqs * ctx
    slots = np.concatenate([slot_mapping_for(bt, b, np.arange(ctx), BS)
                            for b in range(num_seqs)])
    k = normal((T, Hkv, D), seed * 1000 + 1, device, torch.bfloat16)
    v = normal((T, Hkv, D), seed * 1000 + 2, device, torch.bfloat16)
    R = len(row_seq)
    q = normal((R, Hq, D), seed * 1000 + 3, device, torch.bfloat16)
    return Workload("decode", Hq, Hkv, D, BS, pool_blocks, "bf16", "bf16", "bf16",
                    k, v, slots, q, np.asarray(row_seq, np.int32), bt.astype(np.int32),
                    np.stack(idx).astype(np.int32), sm_scale_for(D), num_splits,
                    extra={"positions": np.asarray(positions)})


def e4m3_layer(layer, device="cpu", seed=4, num_seqs=4, ctx=65536, topk=2051,
               pool_blocks=None, num_splits=8):
    """Layer ``layer`` (0..11) of the E4M3 workload; K/V are fp16 sources.
    The block table is the model's (drawn from ``seed`` alone: every layer
    pages the same sequences the same way); lists and data are per layer."""
    Hq, Hkv, D, BS = 32, 4, 128, 64
    nb = ctx // BS
    pool_blocks = pool_blocks or num_seqs * nb
    bt = scattered_block_table(np.random.default_rng(seed), num_seqs, nb, pool_blocks)
    rng = np.random.default_rng([seed, layer])
    row_seq = np.arange(num_seqs, dtype=np.int32)
    idx = np.stack([draw_sorted_distinct(rng, topk, 0, ctx - 1) for _ in range(num_seqs)])
    T = num_seqs * ctx
    slots = np.concatenate([slot_mapping_for(bt, b, np.arange(ctx), BS)
                            for b in range(num_seqs)])
    base = seed * 100000 + layer * 10
    k = student_t4((T, Hkv, D), base + 1, device)
    v = student_t4((T, Hkv, D), base + 2, device)
    q = normal((num_seqs, Hq, D), base + 3, device, torch.float16)
    return Workload("e4m3", Hq, Hkv, D, BS, pool_blocks, "fp16", "fp16", "fp16",
                    k, v, slots, q, row_seq, bt.astype(np.int32), idx.astype(np.int32),
                    sm_scale_for(D), num_splits,
                    extra={"layer": layer, "positions": np.full(num_seqs, ctx - 1)})


def mixed_layer(layer, device="cpu", seed=6, ctx=65536, topk=2051, catch_up=46, decode_rows=3,
                short_topk=1500):
    """One E4M3 layer (the ``e4m3_layer`` cache and shapes) read by a mixed
    batch in one launch: ``catch_up`` consecutive rows of sequence 0 ending
    at its last position, then one decode row for each of the next
    ``decode_rows`` sequences -- 46 + 1 + 1 + 1 = 49 rows by default.  Rows
    have top-k ``topk`` except the last decode row, which lists only
    ``short_topk`` positions followed by -1 padding (varlen lists)."""
    w = e4m3_layer(layer, device=device, seed=seed, num_seqs=1 + decode_rows, ctx=ctx, topk=topk)
    rng = np.random.default_rng([seed, layer, 7])
    positions = np.concatenate([np.arange(ctx - catch_up, ctx), np.full(decode_rows, ctx - 1)])
    row_seq = np.concatenate([np.zeros(catch_up, np.int32),
                              np.arange(1, 1 + decode_rows, dtype=np.int32)])
    R = positions.size
    idx = np.full((R, topk), -1, np.int32)
    for r in range(R):
        n = short_topk if r == R - 1 else topk
        idx[r, :n] = draw_sorted_distinct(rng, n, 0, int(positions[r]))
    q = normal((R, w.num_q_heads, w.head_dim), seed * 100000 + layer * 10 + 5, device,
               torch.float16)
    w.name = "mixed"
    w.q = q
    w.row_seq = row_seq
    w.topk_idx = idx
    w.extra = {"layer": layer, "positions": positions}
    return w


@dataclass
class E2EWorkload:
    """The end-to-end layer step: existing context, one prefill chunk, then
    ``steps`` decode steps, in one sequence."""
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    pool_blocks: int
    block_table: np.ndarray          # [1][max_blocks]
    ctx_k: torch.Tensor              # existing tokens [T0][Hkv][D] bf16
    ctx_v: torch.Tensor
    ctx_slots: np.ndarray
    chunk_k: torch.Tensor            # [C][Hkv][D]
    chunk_v: torch.Tensor
    chunk_slots: np.ndarray
    chunk_q: torch.Tensor            # [C][Hq][D]
    chunk_topk: np.ndarray           # [C][1024]
    step_k: torch.Tensor             # [S][Hkv][D]
    step_v: torch.Tensor
    step_slots: np.ndarray
    step_q: torch.Tensor             # [S][Hq][D]
    step_topk: np.ndarray            # [S][2048]
    sm_scale: float
    num_splits: int = 8


def e2e(pool_blocks, device="cpu", seed=5, ctx0=122880, chunk=8192, steps=8,
        prefill_topk=1024, decode_topk_n=2048):
    """``pool_blocks`` = whole blocks that fit the 13.75 GiB pool for the cache
    kind under test (the caller computes it from the kind's bytes per token)."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, BS = 16, 2, 256, 64
    total = ctx0 + chunk + steps
    nb = -(-total // BS)
    bt = scattered_block_table(rng, 1, nb, pool_blocks)
    chunk_pos = np.arange(ctx0, ctx0 + chunk)
    chunk_topk = np.stack([draw_sorted_distinct(rng, prefill_topk, 0, p) for p in chunk_pos])
    step_pos = np.arange(ctx0 + chunk, total)
    step_topk = np.stack([decode_topk(rng, p, decode_topk_n) for p in step_pos])
    s = seed * 1000
    return E2EWorkload(
        Hq, Hkv, D, BS, pool_blocks, bt.astype(np.int32),
        normal((ctx0, Hkv, D), s + 1, device, torch.bfloat16),
        normal((ctx0, Hkv, D), s + 2, device, torch.bfloat16),
        slot_mapping_for(bt, 0, np.arange(ctx0), BS),
        normal((chunk, Hkv, D), s + 3, device, torch.bfloat16),
        normal((chunk, Hkv, D), s + 4, device, torch.bfloat16),
        slot_mapping_for(bt, 0, chunk_pos, BS),
        normal((chunk, Hq, D), s + 5, device, torch.bfloat16),
        chunk_topk.astype(np.int32),
        normal((steps, Hkv, D), s + 6, device, torch.bfloat16),
        normal((steps, Hkv, D), s + 7, device, torch.bfloat16),
        slot_mapping_for(bt, 0, step_pos, BS),
        normal((steps, Hq, D), s + 8, device, torch.bfloat16),
        step_topk.astype(np.int32), sm_scale_for(D))


# ---------------------------------------------------------------------------
# host views for the oracle (numpy; bf16 as uint16 bit patterns)
# ---------------------------------------------------------------------------

# ---------------------------------------------------------------------------
# indexer scores (inputs of the top-k selection)
# ---------------------------------------------------------------------------

@dataclass
class ScoreSet:
    name: str
    scores: torch.Tensor     # [R][stride] fp32 / fp16 / bf16
    row_len: np.ndarray      # int32 [R]: candidates per row (its position + 1)
    topk: int


def prefill_scores(device="cpu", seed=12, num_rows=2048, ctx=32768, topk=1024,
                   dtype=torch.float32):
    """Scores of the prefill rows (positions ctx-2048 .. ctx-1) over their
    causal prefixes, N(0,1): the top-k of iid scores is a uniform causal
    subset, as the prefill workload's lists are."""
    pos = np.arange(ctx - num_rows, ctx)
    return ScoreSet("prefill", normal((num_rows, ctx), seed, device, dtype),
                    (pos + 1).astype(np.int32), topk)


def decode_scores(device="cpu", seed=13, num_seqs=8, ctx=131072, rows_per_seq=5, topk=2048,
                  window=4096, boost=2.2, dtype=torch.float32):
    """Scores of the decode rows (rows_per_seq per sequence at ctx-5 .. ctx-1):
    N(0,1) plus ``boost`` over each row's last ``window`` positions, so that
    the top-2048 holds about 1434 recent and 614 earlier positions, the mix
    of the decode workload's lists."""
    R = num_seqs * rows_per_seq
    pos = np.tile(np.arange(ctx - rows_per_seq, ctx), num_seqs)
    x = normal((R, ctx), seed, device, torch.float32)
    cols = torch.arange(ctx, device=device)[None, :]
    p = torch.as_tensor(pos, device=device)[:, None]
    x += boost * ((cols > p - window) & (cols <= p)).to(torch.float32)
    return ScoreSet("decode", x.to(dtype), (pos + 1).astype(np.int32), topk)


def to_numpy_src(t):
    """A torch tensor -> numpy array the oracle accepts (bf16 -> uint16 bits)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def dtype_name(t):
    return {torch.float32: "fp32", torch.bfloat16: "bf16", torch.float16: "fp16"}[t.dtype]
