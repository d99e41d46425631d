"""Oracle top-k sparse attention in float64 (test infrastructure only).

For each query row r (one query token with all its heads) and query head h:

    g      = h // (Hq / Hkv)                    (contiguous GQA groups)
    slot_j = block_table[row_seq[r]][j // BS] * BS + j % BS   for each listed
             logical position j >= 0 of the row (j < 0 is padding)
    s_j    = sm_scale * <q[r,h], k_hat[slot_j, g]>
    m = max s_j,  w_j = exp(s_j - m),  l = sum w_j
    out[r,h] = sum_j w_j v_hat[slot_j, g] / l,    lse[r,h] = m + ln l

k_hat / v_hat are the exact dequantized cache rows.  A row whose list holds
no valid position gives out = 0 and lse = -inf.

This is the plain definition of the attention the pages' QSA path computes
over the selected tokens (page "int8 per-(token,head) KV cache for the
Qwen3.8-Flash-Next QSA path", section "The finding worth upstreaming": the
path gathers the scattered rows of a row's top-k list).  Folding the E4M3 K
scale into the softmax factor and applying the V scale after normalization or
after the split-K merge (page "[Perf][SM70][FP8] Hoist QSA E4M3 KV scales",
section "Changes") are rearrangements of the same arithmetic, so the oracle
applies the scales during dequantization and needs no split.
"""

import numpy as np


def resolve_slots(block_table_row, positions, block_size):
    """Logical positions -> physical slots; positions < 0 are dropped."""
    pos = np.asarray(positions, dtype=np.int64)
    pos = pos[pos >= 0]
    bt = np.asarray(block_table_row, dtype=np.int64)
    return bt[pos // block_size] * block_size + pos % block_size


def attend(q, k_hat, v_hat, sm_scale):
    """Dense fp64 softmax attention of one row over its gathered tokens.

    q: [Hq][D]; k_hat, v_hat: [n][Hkv][D] (float64).  Returns (out [Hq][D],
    lse [Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    Hq, D = q.shape
    n = k_hat.shape[0]
    if n == 0:
        return np.zeros((Hq, D)), np.full(Hq, -np.inf)
    Hkv = k_hat.shape[1]
    G = Hq // Hkv
    out = np.empty((Hq, D))
    lse = np.empty(Hq)
    for g in range(Hkv):
        qg = q[g * G:(g + 1) * G]                         # [G][D]
        s = float(sm_scale) * (qg @ k_hat[:, g, :].T)     # [G][n]
        m = s.max(axis=1, keepdims=True)
        w = np.exp(s - m)
        l = w.sum(axis=1, keepdims=True)
        out[g * G:(g + 1) * G] = (w @ v_hat[:, g, :]) / l
        lse[g * G:(g + 1) * G] = (m + np.log(l))[:, 0]
    return out, lse


def query_to_f64(q, q_dtype):
    """bf16 (uint16 bit patterns) or fp16 queries -> exact float64."""
    from .formats import upcast_to_f32
    return upcast_to_f32(q, q_dtype).astype(np.float64)


def sparse_attention(cache, q, q_dtype, row_seq, block_table, topk_idx, sm_scale,
                     rows=None):
    """Run ``attend`` for the selected rows (all rows by default).

    cache: an ``oracle.cache.OracleCache``.  Returns (out [n][Hq][D],
    lse [n][Hq]) in float64 for the rows in ``rows`` order.
    """
    R = np.asarray(topk_idx).shape[0]
    rows = np.arange(R) if rows is None else np.asarray(rows)
    qf = query_to_f64(np.asarray(q)[rows], q_dtype)
    outs, lses = [], []
    for i, r in enumerate(rows):
        slots = resolve_slots(block_table[int(row_seq[r])], topk_idx[r],
                              cache.block_size)
        k_hat = cache.dequant(slots, "k")
        v_hat = cache.dequant(slots, "v")
        o, l = attend(qf[i], k_hat, v_hat, sm_scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


# --------------------------------------------------------------------------
# Split-K partitions (white-box checks of the merge)
# --------------------------------------------------------------------------

def partition_bounds(topk, num_splits):
    """Contiguous partitions of the top-k list: chunk C = ceil(topk / P);
    partition p covers list positions [p*C, min((p+1)*C, topk)), possibly
    empty."""
    C = -(-topk // num_splits)
    return [(min(p * C, topk), min((p + 1) * C, topk)) for p in range(num_splits)]


def merge_partials(outs, lses):
    """Log-sum-exp merge of normalized partials (o_p, lse_p) -> (out, lse).

    out = sum_p exp(lse_p - lse) o_p with lse = log sum_p exp(lse_p); empty
    partitions carry lse_p = -inf and weigh nothing.
    """
    lses = np.asarray(lses, dtype=np.float64)
    outs = np.asarray(outs, dtype=np.float64)
    m = np.max(lses, axis=0)
    if np.all(np.isneginf(m)):
        return np.zeros(outs.shape[1:]), m
    w = np.exp(lses - m)
    lse = m + np.log(w.sum(axis=0))
    wn = np.exp(lses - lse)
    return np.einsum("p...,p...d->...d", wn, outs), lse


def metrics(got, ref):
    """max-abs, max-rel, relative L2 and cosine of got vs ref (flattened)."""
    g = np.asarray(got, dtype=np.float64).ravel()
    r = np.asarray(ref, dtype=np.float64).ravel()
    d = g - r
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    denom = np.maximum(np.abs(r), 1e-30)
    max_rel = float(np.max(np.abs(d) / denom)) if d.size else 0.0
    nr = float(np.linalg.norm(r))
    rel_l2 = float(np.linalg.norm(d) / nr) if nr > 0 else 0.0
    ng = float(np.linalg.norm(g))
    cos = float(g @ r / (ng * nr)) if ng > 0 and nr > 0 else 1.0
    return {"max_abs": max_abs, "max_rel": max_rel, "rel_l2": rel_l2,
            "cosine": cos, "n": int(d.size)}


def within_tolerance(got, ref, atol=2e-3, rtol=1e-2):
    """Elementwise |got - ref| <= atol + rtol * |ref| against the fp64 ref."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    return np.abs(g - r) <= atol + rtol * np.abs(r)

