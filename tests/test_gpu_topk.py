"""GPU parity of the top-k selection (qsa_topk_select) against the oracle:
bit-exact lists for fp32 / fp16 / bf16 scores, ragged and clamped row
lengths, heavy ties, NaN / +-inf / +-0, monotone and constant rows, and the
full-size prefill and decode score sets."""

import numpy as np
import pytest
import torch

from oracle import topk as otopk
from quantized_kv_top_amd import qsakv
from quantized_kv_top_amd import workloads as wl

from parity_util import dev, say

pytestmark = pytest.mark.gpu

DTYPES = [torch.float32, torch.float16, torch.bfloat16]


def _gpu(scores, row_len, k):
    R, stride = scores.shape[0], scores.stride(0)
    out = torch.full((R, k), -7, dtype=torch.int32, device="cuda")
    nb = qsakv.qsa_topk_workspace_bytes(R, stride, k)
    ws = torch.full((nb,), 0xA5, dtype=torch.uint8, device="cuda") if nb else None
    qsakv.qsa_topk_select(scores, dev(row_len, torch.int32), k, out, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check(scores, row_len, k, what, rows=None):
    say("topk", what, tuple(scores.shape), scores.dtype, "k", k)
    g = _gpu(scores, row_len, k)
    src = wl.to_numpy_src(scores)
    want = otopk.topk_select(src, wl.dtype_name(scores), row_len, k, rows=rows)
    got = g if rows is None else g[list(rows)]
    bad = np.nonzero((got != want).any(axis=1))[0]
    assert bad.size == 0, "%s: %d rows differ, first %d: gpu %s oracle %s" % (
        what, bad.size, bad[0], got[bad[0]][:12], want[bad[0]][:12])


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("k", [1, 64, 1024])
def test_random_scores_ragged_lengths(dtype, k):
    stride = 4096
    lens = [0, 1, k - 1, k, k + 1, 2 * k + 3, stride - 1, stride, 777, 3001, 4095, 100]
    lens = [max(v, 0) for v in lens]
    x = wl.normal((len(lens), stride), seed=k, device="cuda", dtype=dtype)
    _check(x, np.array(lens, np.int32), k, "random")


@pytest.mark.parametrize("dtype", DTYPES)
def test_ties_and_special_values(dtype):
    """Scores from a small pool (NaN, +-inf, +-0, a few numbers): every cut
    falls inside a run of equal scores."""
    rng = np.random.default_rng(8)
    pool = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 1.0, -1.0, 0.5, 2.0, -3.0], np.float32)
    R, stride = 24, 2048
    v = pool[rng.integers(0, pool.size, size=(R, stride))]
    x = torch.from_numpy(v).to(dtype).cuda()
    lens = rng.integers(0, stride + 1, size=R).astype(np.int32)
    lens[:4] = [stride, stride - 1, 1000, 2]
    for k in (1, 100, 1000, 2047):
        _check(x, lens, k, "ties k=%d" % k)


def test_monotone_constant_and_clamped_rows():
    stride = 8192
    inc = torch.arange(stride, dtype=torch.float32)
    rows = torch.stack([inc, -inc, torch.zeros(stride), torch.full((stride,), 5.0),
                        inc, inc]).cuda()
    lens = np.array([stride, stride, stride, 5000, -5, 1 << 20], np.int32)
    for k in (1, 333, 4096):
        _check(rows, lens, k, "monotone k=%d" % k)


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_long_16bit_rows(dtype):
    """16-bit rows of up to 65536 scores (the widest register-held rows)."""
    x = wl.normal((6, 65536), seed=9, device="cuda", dtype=dtype)
    lens = np.array([65536, 65535, 40000, 32769, 2049, 65536], np.int32)
    _check(x, lens, 2048, "long 16-bit rows")


@pytest.mark.parametrize("dtype", DTYPES)
def test_bin_overflow_falls_back_to_streaming(dtype):
    """More candidates share the k-th score's top digit than LDS holds
    (scores drawn from 3 values): the remaining digits re-read the row."""
    rng = np.random.default_rng(10)
    v = np.array([0.25, 0.5, 0.75], np.float32)[rng.integers(0, 3, size=(5, 30000))]
    x = torch.from_numpy(v).to(dtype).cuda()
    lens = np.array([30000, 29999, 20000, 12000, 9000], np.int32)
    for k in (1, 1000, 5000):
        _check(x, lens, k, "bin overflow k=%d" % k)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("stride,k", [(65536, 2051), (131072, 2048), (40960, 1024)])
def test_split_rows_ragged(dtype, stride, k):
    """Rows longer than one workgroup holds: segments select their own top k,
    then a merge; lengths that end inside, at and before segment edges, and
    rows with at most k candidates."""
    lens = [stride, stride - 1, 32768, 32769, 32767, 3 * k + 1, k, k + 1, 100, 0,
            stride // 2 + 7, 24575, min(stride, 65536 + 5)]
    x = wl.normal((len(lens), stride), seed=stride + k, device="cuda", dtype=dtype)
    _check(x, np.array(lens, np.int32), k, "split ragged")


@pytest.mark.parametrize("dtype", DTYPES)
def test_split_rows_ties_and_specials(dtype):
    """Long rows of a few values with NaN / +-inf / +-0: the cut falls inside
    runs of equal scores that cross segment edges (and overflow the
    candidate capacity in places)."""
    rng = np.random.default_rng(21)
    pool = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 1.0, -1.0, 2.0], np.float32)
    stride = 65536
    v = pool[rng.integers(0, pool.size, size=(6, stride))]
    v[3] = np.nan                     # all NaN
    v[4, :] = 1.0                     # all equal
    x = torch.from_numpy(v).to(dtype).cuda()
    lens = np.array([stride, 60000, 33000, stride, 50001, 40000], np.int32)
    for k in (1, 2048, 4096):
        _check(x, lens, k, "split ties k=%d" % k)


def test_strided_rows():
    """Rows of a wider buffer (row stride above the row length)."""
    base = wl.normal((9, 3000), seed=4, device="cuda", dtype=torch.float16)
    x = base[:, :2992]          # stride 3000 (6000 B, a multiple of 16)
    lens = np.array([2992, 2000, 1500, 100, 2992, 0, 7, 2991, 1024], np.int32)
    say("topk strided")
    g = _gpu(x, lens, 128)
    want = otopk.topk_select(wl.to_numpy_src(x.contiguous()), "fp16", lens, 128)
    assert (g == want).all()


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16])
def test_full_size_prefill_scores(dtype):
    """The prefill rows: 2048 x 32768 scores, top-1024, every row."""
    s = wl.prefill_scores(device="cuda", dtype=dtype)
    _check(s.scores, s.row_len, s.topk, "prefill full size")


def test_full_size_decode_scores():
    """The decode rows: 40 x 131072 scores (recent window boosted), top-2048."""
    s = wl.decode_scores(device="cuda")
    _check(s.scores, s.row_len, s.topk, "decode full size")


def test_lists_drive_the_attention():
    """The selected lists are valid top-k input of the sparse attention:
    increasing, in range, -1 padded."""
    s = wl.prefill_scores(device="cuda", num_rows=64, ctx=4096, topk=1024)
    g = _gpu(s.scores, s.row_len, s.topk)
    for r in range(64):
        n = min(int(s.row_len[r]), s.topk)
        assert (np.diff(g[r, :n]) > 0).all() and g[r, 0] >= 0 and g[r, n - 1] < s.row_len[r]
        assert (g[r, n:] == -1).all()


def _random_topk_case(seed):
    """A seeded random selection: dtype, rows, row stride (a multiple of 8
    up to 160K, so that long rows take the segmented path), k, row lengths
    (including 0, <= k, the stride and clamped values beyond it) and a score
    distribution (normal, a few distinct values, or normal with NaN / +-inf
    sprinkled in)."""
    rng = np.random.default_rng(seed)
    dtype = DTYPES[rng.integers(len(DTYPES))]
    R = int(rng.integers(1, 9))
    stride = int(rng.choice([8, 64, 1000, 4096, 32768, 40000, 70000, 131072, 163840]))
    stride = -(-stride // 8) * 8
    k = int(rng.integers(1, min(stride, 4096) + 1))
    lens = rng.integers(0, stride + 1, size=R).astype(np.int64)
    picks = [0, 1, k, k + 1, stride, stride + 100]
    for i in range(min(R, 2)):
        lens[i] = picks[rng.integers(len(picks))]
    mode = int(rng.integers(3))
    v = rng.standard_normal((R, stride)).astype(np.float32)
    if mode == 1:
        pool = np.array([0.0, -0.0, 1.0, -1.0, 0.25, 3.0], np.float32)
        v = pool[rng.integers(0, pool.size, size=(R, stride))]
    elif mode == 2:
        m = rng.random((R, stride))
        v[m < 0.01] = np.nan
        v[(m >= 0.01) & (m < 0.015)] = np.inf
        v[(m >= 0.015) & (m < 0.02)] = -np.inf
    return torch.from_numpy(v).to(dtype).cuda(), lens.astype(np.int32), k, mode


@pytest.mark.parametrize("seed", list(range(300, 360)))
def test_random_selections(seed):
    x, lens, k, mode = _random_topk_case(seed)
    _check(x, lens, k, "random seed %d mode %d" % (seed, mode))
