"""Host-side checks of the C ABI: the library loads, exports what the header
declares, sizes caches and workspaces by the closed forms, and rejects bad
arguments before any HIP call.  No GPU: every call here returns from host
validation (dummy device pointers are never dereferenced)."""

import ctypes
import os
import re

import pytest

from oracle import cache as ocache
from quantized_kv_top_amd import qsakv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsakv.h")

pytestmark = pytest.mark.skipif(not os.path.exists(qsakv.LIB_PATH),
                                reason="libqsakv.so not built")

DUMMY = 0x10000          # 64 KiB: 256-byte aligned, never dereferenced on these paths


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*QSAKV_API\s+(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


def test_exports_every_declared_function():
    names = header_functions()
    assert set(names) == set(qsakv.EXPORTED)
    L = qsakv.lib()
    for n in names:
        assert hasattr(L, n), n
    assert L.qkv_abi_version() == 1


def test_struct_layouts():
    # int32 x 6, then pointers: offsets follow the C ABI
    assert qsakv.QkvCache.k.offset == 24
    assert qsakv.QkvCache.k_scale.offset == 48
    assert ctypes.sizeof(qsakv.QkvCache) == 56
    assert qsakv.QsaArgs.row_seq.offset == 24
    assert ctypes.sizeof(qsakv.QsaArgs) == 80


@pytest.mark.parametrize("kind", ocache.KINDS)
@pytest.mark.parametrize("D", [128, 256])
def test_cache_bytes_match_oracle_layout(kind, D):
    NB, BS, H = 37, 64, 2
    kb, vb, sb = qsakv.cache_bytes(kind, NB, BS, H, D)
    assert kb == vb == NB * BS * H * ocache.row_bytes(kind, D)
    per_token = (kb + vb + sb) // (NB * BS)
    assert per_token == ocache.bytes_per_token(kind, H, D)


def test_workspace_bytes():
    L = qsakv.lib()
    n = 40 * 16 * 8
    # the partials (padded to 256 B), then (max, sum) pairs
    assert L.qsa_decode_workspace_bytes(40, 16, 256, 8) == n * 256 * 4 + n * 8
    assert L.qsa_decode_workspace_bytes(3, 4, 128, 2) == 24 * 512 + 24 * 8
    assert L.qsa_decode_workspace_bytes(40, 16, 256, 1) == 0
    assert L.qsa_decode_workspace_bytes(40, 16, 64, 8) == 0
    assert L.qsa_decode_workspace_bytes(40, 16, 256, 65) == 0


def _cache(kind="int8", NB=8, BS=16, H=1, D=128, ks=1.0, vs=1.0, scale_ptr=DUMMY):
    return qsakv.QkvCache(qsakv.KIND_BY_NAME[kind], NB, BS, H, D, 0, DUMMY, DUMMY,
                          scale_ptr, ks, vs)


def _args(R=4, Hq=4, topk=16, q_dtype=qsakv.BF16, out_dtype=qsakv.FP32, sm=0.125, q=DUMMY):
    return qsakv.QsaArgs(q, q_dtype, R, Hq, 1, DUMMY, DUMMY, 4, topk, DUMMY, sm, out_dtype,
                         DUMMY, None)


def _prefill(c, a):
    return qsakv.lib().qsa_sparse_attn_prefill(ctypes.byref(c), ctypes.byref(a), None)


def _decode(c, a, P=8, ws=DUMMY, wsb=1 << 30):
    return qsakv.lib().qsa_sparse_attn_decode(ctypes.byref(c), ctypes.byref(a), P, ws, wsb, None)


def _write(c, T=4, dt=qsakv.FP32, k=DUMMY):
    return qsakv.lib().kv_quant_write(ctypes.byref(c), k, DUMMY, dt, T, DUMMY, None)


def test_null_pointers():
    L = qsakv.lib()
    assert L.qsa_sparse_attn_prefill(None, ctypes.byref(_args()), None) == qsakv.ERR_NULL
    assert L.qsa_sparse_attn_prefill(ctypes.byref(_cache()), None, None) == qsakv.ERR_NULL
    assert _write(_cache(), k=None) == qsakv.ERR_NULL
    assert _prefill(_cache(scale_ptr=None), _args()) == qsakv.ERR_NULL
    assert _prefill(_cache(), _args(q=None)) == qsakv.ERR_NULL


def test_shapes_and_supported_set():
    assert _prefill(_cache(D=64), _args()) == qsakv.ERR_UNSUPPORTED
    assert _prefill(_cache(BS=48), _args()) == qsakv.ERR_BAD_SHAPE
    assert _prefill(_cache(BS=2048), _args()) == qsakv.ERR_BAD_SHAPE
    assert _prefill(_cache(H=3), _args(Hq=4)) == qsakv.ERR_BAD_SHAPE
    assert _prefill(_cache(H=1), _args(Hq=32)) == qsakv.ERR_UNSUPPORTED
    assert _prefill(_cache(), _args(topk=0)) == qsakv.ERR_BAD_SHAPE
    assert _prefill(_cache(), _args(R=1, topk=(1 << 30) + 1)) == qsakv.ERR_BAD_SHAPE
    assert _decode(_cache(), _args(R=1, topk=(1 << 31) - 1)) == qsakv.ERR_BAD_SHAPE
    assert _prefill(_cache(), _args(R=-1)) == qsakv.ERR_BAD_SHAPE
    assert _prefill(_cache(), _args(q_dtype=qsakv.FP32)) == qsakv.ERR_UNSUPPORTED
    assert _prefill(_cache(kind="bf16"), _args(q_dtype=qsakv.FP16)) == qsakv.ERR_UNSUPPORTED
    assert _prefill(_cache(), _args(out_dtype=7)) == qsakv.ERR_UNSUPPORTED
    bad = _cache()
    bad.kind = 9
    assert _prefill(bad, _args()) == qsakv.ERR_UNSUPPORTED
    assert _write(_cache(), T=-1) == qsakv.ERR_BAD_SHAPE
    assert _write(_cache(), dt=5) == qsakv.ERR_UNSUPPORTED


def test_fail_closed_scales():
    """E4M3 scales must be explicit, finite and positive; 1.0 is legal."""
    for ks in [float("nan"), float("inf"), 0.0, -1.0, 1e-40]:
        assert _prefill(_cache("e4m3", ks=ks), _args()) == qsakv.ERR_BAD_SCALE
        assert _prefill(_cache("e4m3", vs=ks), _args()) == qsakv.ERR_BAD_SCALE
        assert _write(_cache("e4m3", ks=ks)) == qsakv.ERR_BAD_SCALE
    # the softmax scale: finite and positive (a zero, negative or -0 scale fails)
    for sm in [float("nan"), float("inf"), -float("inf"), 0.0, -0.0, -0.0625]:
        assert _prefill(_cache(), _args(sm=sm)) == qsakv.ERR_BAD_SCALE
        assert _decode(_cache(), _args(sm=sm)) == qsakv.ERR_BAD_SCALE
    assert _prefill(_cache(), _args(R=0, sm=1e-30)) == qsakv.OK
    # unit scale passes validation (checked with a zero-row call: no launch)
    assert _prefill(_cache("e4m3", ks=1.0, vs=1.0), _args(R=0)) == qsakv.OK
    # int8 caches ignore k_scale / v_scale entirely
    assert _prefill(_cache("int8", ks=float("nan")), _args(R=0)) == qsakv.OK


def test_alignment():
    assert _prefill(_cache(), _args(q=DUMMY + 4)) == qsakv.ERR_ALIGNMENT
    c = _cache()
    c.k = DUMMY + 8
    assert _prefill(c, _args()) == qsakv.ERR_ALIGNMENT
    c = _cache("int8_inline")
    c.k = DUMMY + 4          # inline rows are 4-byte aligned by construction
    assert _prefill(c, _args(R=0)) == qsakv.OK
    assert _decode(_cache(), _args(), ws=DUMMY + 16) == qsakv.ERR_WORKSPACE


def test_decode_splits_and_workspace():
    assert _decode(_cache(), _args(), P=0) == qsakv.ERR_UNSUPPORTED
    assert _decode(_cache(), _args(), P=65) == qsakv.ERR_UNSUPPORTED
    assert _decode(_cache(), _args(), ws=None) == qsakv.ERR_WORKSPACE
    need = qsakv.lib().qsa_decode_workspace_bytes(4, 4, 128, 8)
    assert _decode(_cache(), _args(), wsb=need - 1) == qsakv.ERR_WORKSPACE


def test_empty_calls_are_noops():
    assert _write(_cache(), T=0) == qsakv.OK
    assert _prefill(_cache(), _args(R=0)) == qsakv.OK
    assert _decode(_cache(), _args(R=0)) == qsakv.OK


def test_status_strings():
    L = qsakv.lib()
    for s in range(8):
        assert L.qkv_status_str(s).decode().startswith("QKV_")
    assert b"unknown" in L.qkv_status_str(99)


def _calib(x=DUMMY, dt=qsakv.FP16, n=1000, scale=1.0, out=DUMMY, ws=DUMMY, wsb=None):
    L = qsakv.lib()
    wsb = L.qkv_calib_workspace_bytes() if wsb is None else wsb
    return L.kv_calib_stats(x, dt, n, scale, out, ws, wsb, None)


def test_calib_struct_and_validation():
    """qkv_calib_result layout, and every rejection happens before a launch."""
    assert ctypes.sizeof(qsakv.QkvCalibResult) == 64
    assert qsakv.QkvCalibResult.max_abs.offset == 48
    L = qsakv.lib()
    # uint64: a 32K-bin and two 64K-bin histograms, selection state, 256
    # per-workgroup and 128 per-reduction-block counter sets; then 256
    # uint32 32K-bin per-workgroup histograms
    assert L.qkv_calib_workspace_bytes() == (32768 + 2 * 65536 + 8 + 256 * 8 + 128 * 8) * 8 \
        + 256 * 32768 * 4
    assert _calib(dt=3) == qsakv.ERR_UNSUPPORTED
    assert _calib(n=-1) == qsakv.ERR_BAD_SHAPE
    assert _calib(x=None) == qsakv.ERR_NULL
    assert _calib(out=None) == qsakv.ERR_NULL
    for s in [float("nan"), float("inf"), 0.0, -1.0, 1e-40]:
        assert _calib(scale=s) == qsakv.ERR_BAD_SCALE
    assert _calib(x=DUMMY + 8) == qsakv.ERR_ALIGNMENT
    assert _calib(out=DUMMY + 4) == qsakv.ERR_ALIGNMENT
    assert _calib(ws=None) == qsakv.ERR_WORKSPACE
    assert _calib(ws=DUMMY + 128) == qsakv.ERR_WORKSPACE
    assert _calib(wsb=L.qkv_calib_workspace_bytes() - 1) == qsakv.ERR_WORKSPACE


def _topk(sc=DUMMY, dt=qsakv.FP32, R=4, stride=1024, rl=DUMMY, k=16, out=DUMMY, ws=None, wsb=0):
    return qsakv.lib().qsa_topk_select(sc, dt, R, stride, rl, k, out, ws, wsb, None)


def test_topk_validation():
    """Every rejection of qsa_topk_select happens before a launch; no rows is
    a no-op."""
    assert _topk(dt=3) == qsakv.ERR_UNSUPPORTED
    assert _topk(R=-1) == qsakv.ERR_BAD_SHAPE
    assert _topk(stride=-4) == qsakv.ERR_BAD_SHAPE
    assert _topk(stride=(1 << 30) + 4) == qsakv.ERR_BAD_SHAPE
    assert _topk(k=0) == qsakv.ERR_BAD_SHAPE
    assert _topk(R=1 << 20, k=4096) == qsakv.ERR_BAD_SHAPE      # R * k >= 2^31
    assert _topk(R=0, sc=None, rl=None, out=None) == qsakv.OK
    assert _topk(sc=None) == qsakv.ERR_NULL
    assert _topk(rl=None) == qsakv.ERR_NULL
    assert _topk(out=None) == qsakv.ERR_NULL
    assert _topk(sc=DUMMY + 8) == qsakv.ERR_ALIGNMENT
    assert _topk(stride=1022) == qsakv.ERR_ALIGNMENT            # 4088 B rows
    assert _topk(dt=qsakv.FP16, stride=1020) == qsakv.ERR_ALIGNMENT
    assert _topk(rl=DUMMY + 2) == qsakv.ERR_ALIGNMENT
    assert _topk(out=DUMMY + 2) == qsakv.ERR_ALIGNMENT
    # long rows need the segment workspace
    need = qsakv.lib().qsa_topk_workspace_bytes(40, 131072, 2048)
    assert _topk(R=40, stride=131072, k=2048) == qsakv.ERR_WORKSPACE
    assert _topk(R=40, stride=131072, k=2048, ws=DUMMY, wsb=need - 1) == qsakv.ERR_WORKSPACE
    assert _topk(R=40, stride=131072, k=2048, ws=DUMMY + 128, wsb=need) == qsakv.ERR_WORKSPACE


def test_topk_workspace_bytes():
    """Rows of up to 32768 scores need none; longer rows are cut into the
    largest of 32K / 16K / 8K-score segments that is at least 4 k and keeps
    segments x k within 32768: keys and positions, [rows][segments * k
    rounded up to 4] each, 256-B aligned."""
    L = qsakv.lib()
    assert L.qsa_topk_workspace_bytes(2048, 32768, 1024) == 0
    # 131072 / 32768 = 4 segments x 2048
    assert L.qsa_topk_workspace_bytes(40, 131072, 2048) == 2 * 40 * 4 * 2048 * 4
    # 65536 / 32768 = 2 segments x 2051 -> 4102 slots, rounded up to 4104
    assert L.qsa_topk_workspace_bytes(4, 65536, 2051) == 2 * ((4 * 4104 * 4 + 255) // 256 * 256)
    # 1M-score rows, k 512: 32K segments (32 x 512 = 16384)
    assert L.qsa_topk_workspace_bytes(2, 1 << 20, 512) == 2 * 2 * 32 * 512 * 4
    # 1M-score rows, k 2048: 32 x 2048 > 32768, and shorter segments only
    # make more lists: streamed, no workspace
    assert L.qsa_topk_workspace_bytes(4, 1 << 20, 2048) == 0
    # k too large for segments: streamed, no workspace
    assert L.qsa_topk_workspace_bytes(4, 1 << 20, 8192) == 0


def _decode_noalloc(c, a, P=8):
    return qsakv.lib().qsa_sparse_attn_decode_noalloc(ctypes.byref(c), ctypes.byref(a), P, None)


def test_noalloc_decode_host_checks():
    """The no-alloc decode validates like qsa_sparse_attn_decode and refuses,
    before any HIP call, a call whose split-K partials exceed its static
    scratch (QSA_NOALLOC_SCRATCH_BYTES)."""
    L = qsakv.lib()
    assert qsakv.NOALLOC_SCRATCH_BYTES == 16 << 20
    # 127 rows x 16 heads x 8 splits at D = 256 fit; 128 rows do not
    assert L.qsa_decode_workspace_bytes(127, 16, 256, 8) <= qsakv.NOALLOC_SCRATCH_BYTES
    assert L.qsa_decode_workspace_bytes(128, 16, 256, 8) > qsakv.NOALLOC_SCRATCH_BYTES
    big = _cache(D=256, H=2)
    assert _decode_noalloc(big, _args(R=128, Hq=16)) == qsakv.ERR_SCRATCH
    assert _decode_noalloc(big, _args(R=4000, Hq=16), P=64) == qsakv.ERR_SCRATCH
    assert "QSA_NOALLOC_SCRATCH_BYTES" in L.qkv_status_str(qsakv.ERR_SCRATCH).decode()
    # the same argument checks as the workspace variant
    assert _decode_noalloc(_cache(), _args(sm=0.0)) == qsakv.ERR_BAD_SCALE
    assert _decode_noalloc(_cache(), _args(), P=0) == qsakv.ERR_UNSUPPORTED
    assert _decode_noalloc(_cache(), _args(), P=65) == qsakv.ERR_UNSUPPORTED
    assert _decode_noalloc(_cache(D=64), _args()) == qsakv.ERR_UNSUPPORTED
    assert _decode_noalloc(_cache(), _args(q=DUMMY + 4)) == qsakv.ERR_ALIGNMENT
    assert _decode_noalloc(_cache("e4m3", ks=0.0), _args()) == qsakv.ERR_BAD_SCALE
    assert _decode_noalloc(_cache(), _args(R=0)) == qsakv.OK
