"""The Python binding rejects what the C ABI cannot see (tensor dtypes,
shapes, contiguity, device) before any call into the library.  CPU only:
every case here fails validation, so nothing reaches a kernel."""

import pytest
import torch

from quantized_kv_top_amd import qsakv

H, D, BS, NB = 1, 128, 16, 4


@pytest.fixture(scope="module")
def cache():
    return qsakv.Cache("int8", NB, BS, H, D, device="cpu")


def _write_args(T=5):
    return (torch.zeros(T, H, D), torch.zeros(T, H, D), torch.zeros(T, dtype=torch.int64))


def test_write_checks(cache):
    k, v, sm = _write_args()
    with pytest.raises(TypeError, match="slot_mapping"):
        qsakv.kv_quant_write(cache, k, v, sm.int())
    with pytest.raises(TypeError, match="k_src"):
        qsakv.kv_quant_write(cache, k.double(), v, sm)
    with pytest.raises(TypeError, match="v_src"):
        qsakv.kv_quant_write(cache, k, v.half(), sm)
    with pytest.raises(ValueError, match="v_src"):
        qsakv.kv_quant_write(cache, k, v[:4], sm)
    with pytest.raises(ValueError, match="k_src"):
        qsakv.kv_quant_write(cache, torch.zeros(5, H, 2 * D)[:, :, ::2], v, sm)
    with pytest.raises(ValueError, match="k_src"):
        qsakv.kv_quant_write(cache, torch.zeros(5, H + 1, D), v, sm)
    with pytest.raises(ValueError, match="slot_mapping"):
        qsakv.kv_quant_write(cache, k, v, sm[:3])
    with pytest.raises(ValueError, match="CUDA"):
        qsakv.kv_quant_write(cache, k, v, sm)


def _attn_args(R=3, Hq=4, topk=7):
    return dict(q=torch.zeros(R, Hq, D, dtype=torch.bfloat16),
                row_seq=torch.zeros(R, dtype=torch.int32),
                block_table=torch.zeros(2, NB, dtype=torch.int32),
                topk_idx=torch.zeros(R, topk, dtype=torch.int32),
                sm_scale=0.1, out=torch.zeros(R, Hq, D), lse=torch.zeros(R, Hq))


@pytest.mark.parametrize("field,bad,exc", [
    ("q", torch.zeros(3, 4, D), TypeError),
    ("q", torch.zeros(3, 4 * D, dtype=torch.bfloat16), ValueError),
    ("out", torch.zeros(3, 4, D, dtype=torch.float64), TypeError),
    ("out", torch.zeros(3, 5, D), ValueError),
    ("row_seq", torch.zeros(3, dtype=torch.int64), TypeError),
    ("row_seq", torch.zeros(2, dtype=torch.int32), ValueError),
    ("block_table", torch.zeros(2 * NB, dtype=torch.int32), ValueError),
    ("topk_idx", torch.zeros(4, 7, dtype=torch.int32), ValueError),
    ("topk_idx", torch.zeros(7, 3, dtype=torch.int32).t(), ValueError),
    ("lse", torch.zeros(3, 5), ValueError),
    ("lse", torch.zeros(3, 4, dtype=torch.float16), TypeError),
])
def test_attention_checks(cache, field, bad, exc):
    a = _attn_args()
    a[field] = bad
    with pytest.raises(exc, match=field):
        qsakv.qsa_sparse_attn_prefill(cache, **a)
    ws = torch.zeros(1024, dtype=torch.uint8)
    with pytest.raises(exc, match=field):
        qsakv.qsa_sparse_attn_decode(cache, a["q"], a["row_seq"], a["block_table"],
                                     a["topk_idx"], a["sm_scale"], a["out"], 2, ws,
                                     lse=a["lse"])


def test_attention_valid_host_tensors_are_refused(cache):
    with pytest.raises(ValueError, match="CUDA"):
        qsakv.qsa_sparse_attn_prefill(cache, **_attn_args())
    a = _attn_args()
    with pytest.raises(TypeError, match="workspace"):
        qsakv.qsa_sparse_attn_decode(cache, a["q"], a["row_seq"], a["block_table"],
                                     a["topk_idx"], a["sm_scale"], a["out"], 2,
                                     torch.zeros(16, dtype=torch.int32))


def test_topk_and_calib_checks():
    s = torch.zeros(4, 64)
    lens = torch.full((4,), 64, dtype=torch.int32)
    out = torch.zeros(4, 8, dtype=torch.int32)
    with pytest.raises(ValueError, match="scores"):
        qsakv.qsa_topk_select(s.t(), lens, 8, out)
    with pytest.raises(TypeError, match="scores"):
        qsakv.qsa_topk_select(s.double(), lens, 8, out)
    s_dev_like = torch.zeros(4, 64)
    with pytest.raises(ValueError, match="scores"):      # host tensor
        qsakv.qsa_topk_select(s_dev_like, lens, 8, out)
    x = torch.zeros(100, dtype=torch.float16)
    ws = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="out"):
        qsakv.kv_calib_stats(x, 1.0, torch.zeros(8, dtype=torch.uint8), ws)
    with pytest.raises(TypeError, match="x"):
        qsakv.kv_calib_stats(x.double(), 1.0, torch.zeros(64, dtype=torch.uint8), ws)
