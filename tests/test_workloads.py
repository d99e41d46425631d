"""Host checks of the seeded input generators (no method arithmetic).  No GPU."""

import numpy as np
import torch

from quantized_kv_top_amd import workloads as wl


def test_draw_sorted_distinct():
    rng = np.random.default_rng(0)
    for n, lo, hi in [(16, 0, 60), (1024, 0, 30719), (614, 0, 126975), (5, 3, 7)]:
        x = wl.draw_sorted_distinct(rng, n, lo, hi)
        assert x.size == n and np.all(np.diff(x) > 0)
        assert x.min() >= lo and x.max() <= hi


def test_decode_topk_mix():
    rng = np.random.default_rng(1)
    pos = 131071
    x = wl.decode_topk(rng, pos, 2048)
    assert x.size == 2048 and np.all(np.diff(x) > 0)
    recent = np.sum(x >= pos - 4095)
    assert recent == 1434
    assert x.max() <= pos


def test_tiny_shapes_and_causality():
    w = wl.tiny()
    assert w.k_src.shape == (64, 1, 128) and w.k_src.dtype == torch.float32
    assert w.q.dtype == torch.bfloat16 and w.q.shape == (4, 4, 128)
    assert sorted(w.block_table[0].tolist()) == [0, 1, 2, 3]
    for r, p in enumerate(w.extra["positions"]):
        assert w.topk_idx[r].max() <= p and np.unique(w.topk_idx[r]).size == 16
    assert np.unique(w.slot_mapping).size == 64


def test_prefill_small_structure():
    w = wl.prefill(num_rows=8, topk=64, ctx=4096, pool_blocks=96)
    assert w.block_table.shape == (1, 64)
    assert np.unique(w.block_table).size == 64 and w.block_table.max() < 96
    k = w.k_src.float()
    # the outlier channels carry ~10x the spread of the others
    ch = w.extra["k_outlier_channels"]
    other = np.setdiff1d(np.arange(256), ch)
    assert k[..., ch].std() > 5 * k[..., other].std()


def test_student_t_heavy_tail():
    x = wl.student_t4((200000,), 7, "cpu").float()
    # t(4) has excess kurtosis (infinite in theory); sample kurtosis >> 3
    z = (x - x.mean()) / x.std()
    assert float((z ** 4).mean()) > 5.0
    assert abs(float(x.std()) - 0.5 * np.sqrt(2.0)) < 0.1


def test_mixed_layer_structure():
    w = wl.mixed_layer(0, ctx=4096, topk=300, short_topk=100)
    assert w.num_rows == 49 and w.topk == 300
    assert list(w.row_seq) == [0] * 46 + [1, 2, 3]
    pos = w.extra["positions"]
    assert list(pos[:46]) == list(range(4096 - 46, 4096)) and list(pos[46:]) == [4095] * 3
    for r in range(49):
        valid = w.topk_idx[r][w.topk_idx[r] >= 0]
        assert valid.size == (100 if r == 48 else 300)
        assert np.all(valid <= pos[r]) and np.unique(valid).size == valid.size
    assert np.all(w.topk_idx[48, 100:] == -1)
