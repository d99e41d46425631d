"""Oracle for the top-k selection that produces the sparse-attention index
lists (test infrastructure only; see package docstring).

Page "[Model][SM70][FP8] Add calibrated E4M3 QSA KV cache" (section listing
the validated contract, and "Non-obvious design decisions") describes the
step before the attention: FP16 raw and compressed indexer caches score the
candidates of each query row and a block/position selection picks the row's
list; its validation section compares those selections between cache modes
by row Jaccard, recall and exact-row ratio.  The pages give neither the
scoring formula nor the selection rule in detail, so the selection is taken
in its plainest reading, on scores that are inputs here:

* a row r has row_len[r] candidates, positions 0 .. row_len[r] - 1 (its
  causal prefix); row_len is clamped to [0, row_stride];
* the row's list is the k candidates with the largest scores, compared as
  numbers (so -0 == +0); NaN ranks below every number, -inf included;
* equal scores are taken in increasing position order (the lower position
  wins a tie at the cut);
* the list is returned in increasing position order (the order the attention
  path reads), padded with -1 when the row has fewer than k candidates
  (then every candidate is listed).

Scores are fp32, fp16 or bf16 (bf16 as its 16-bit patterns); every such
value is exact in float64, where the comparisons are made.  The selection is
one numpy lexsort per row (primary key: is-NaN, then the negated score, then
the position) followed by a sort of the chosen positions.
"""

import numpy as np

from .formats import upcast_to_f32


def scores_f64(scores, dtype):
    """Score array (any shape) -> float64, exactly."""
    return upcast_to_f32(scores, dtype).astype(np.float64)


def select_row(vals, k):
    """Positions of the k largest of ``vals`` (float64, the row's
    candidates), ties and NaN as in the module docstring, increasing."""
    n = vals.shape[0]
    if n <= k:
        return np.arange(n, dtype=np.int64)
    nan = np.isnan(vals)
    neg = np.where(nan, 0.0, -vals)
    order = np.lexsort((np.arange(n), neg, nan))
    return np.sort(order[:k])


def topk_select(scores, dtype, row_len, k, rows=None):
    """[R][row_stride] scores -> int32 [len(rows)][k] lists, -1 padded."""
    scores = np.asarray(scores)
    R, stride = scores.shape
    rows = range(R) if rows is None else rows
    out = np.full((len(rows), k), -1, dtype=np.int32)
    for i, r in enumerate(rows):
        n = int(min(max(int(row_len[r]), 0), stride))
        sel = select_row(scores_f64(scores[r, :n], dtype), k)
        out[i, :sel.shape[0]] = sel
    return out


def overlap(a, b):
    """Selection overlap of two lists per row (-1 entries ignored), the
    metrics of the validation section: mean row Jaccard |A & B| / |A | B|
    (1 for two empty rows), mean recall |A & B| / |A| of reference A (1 for
    an empty A), the ratio of rows with A == B, and the micro Jaccard
    sum |A & B| / sum |A | B| over all rows."""
    jac, rec, exact, inter_t, union_t = [], [], 0, 0, 0
    for ra, rb in zip(a, b):
        sa, sb = set(int(x) for x in ra if x >= 0), set(int(x) for x in rb if x >= 0)
        inter, union = len(sa & sb), len(sa | sb)
        jac.append(inter / union if union else 1.0)
        rec.append(inter / len(sa) if sa else 1.0)
        exact += sa == sb
        inter_t += inter
        union_t += union
    n = len(jac)
    return {"row_jaccard": float(np.mean(jac)) if n else 1.0,
            "recall": float(np.mean(rec)) if n else 1.0,
            "exact_rows": exact / n if n else 1.0,
            "micro_jaccard": inter_t / union_t if union_t else 1.0}
