"""Thin ctypes binding of the qsakv C ABI (``include/qsakv.h``).

Argument marshalling only: every step of the path runs in the HIP library.
PyTorch supplies device memory and streams.  The library must be built
(``python -m quantized_kv_top_amd.build``); loading fails loudly otherwise.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqsakv.so")

# status codes (qkv_status)
OK, ERR_NULL, ERR_BAD_SHAPE, ERR_UNSUPPORTED, ERR_BAD_SCALE, ERR_WORKSPACE, ERR_HIP, \
    ERR_ALIGNMENT, ERR_SCRATCH = range(9)
# QSA_NOALLOC_SCRATCH_BYTES: split-K scratch of qsa_sparse_attn_decode_noalloc
NOALLOC_SCRATCH_BYTES = 16 << 20
# dtypes (qkv_dtype)
BF16, FP16, FP32 = 0, 1, 2
# cache kinds (qkv_cache_kind)
CACHE_INT8, CACHE_INT8_INLINE, CACHE_E4M3, CACHE_BF16, CACHE_NVFP4 = 0, 1, 2, 3, 4
KIND_BY_NAME = {"int8": CACHE_INT8, "int8_inline": CACHE_INT8_INLINE,
                "e4m3": CACHE_E4M3, "bf16": CACHE_BF16, "nvfp4": CACHE_NVFP4}

EXPORTED = ("kv_quant_write", "qsa_sparse_attn_prefill", "qsa_decode_workspace_bytes",
            "qsa_sparse_attn_decode", "qsa_sparse_attn_decode_noalloc",
            "qkv_calib_workspace_bytes", "kv_calib_stats",
            "qsa_topk_workspace_bytes", "qsa_topk_select", "qkv_cache_bytes",
            "qkv_status_str", "qkv_last_hip_error", "qkv_abi_version")


class QkvCache(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("kv_scale", ctypes.c_void_p), ("k_scale", ctypes.c_float),
                ("v_scale", ctypes.c_float)]


class QsaArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("q_dtype", ctypes.c_int32),
                ("num_rows", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_seqs", ctypes.c_int32), ("row_seq", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("block_table_stride", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("topk_idx", ctypes.c_void_p),
                ("sm_scale", ctypes.c_float), ("out_dtype", ctypes.c_int32),
                ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p)]


class QkvCalibResult(ctypes.Structure):
    _fields_ = [("count", ctypes.c_uint64), ("nan", ctypes.c_uint64),
                ("nonzero", ctypes.c_uint64), ("saturated", ctypes.c_uint64),
                ("below_min_subnormal", ctypes.c_uint64), ("subnormal", ctypes.c_uint64),
                ("max_abs", ctypes.c_float), ("p999", ctypes.c_float),
                ("p9999", ctypes.c_float), ("reserved", ctypes.c_uint32)]


_lib = None


def lib():
    """Load libqsakv.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("qsakv: %s is not built; run `python -m quantized_kv_top_amd.build`"
                           % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    c_i32, c_i64, c_sz, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
    P = ctypes.POINTER
    L.kv_quant_write.argtypes = [P(QkvCache), c_vp, c_vp, c_i32, c_i64, c_vp, c_vp]
    L.kv_quant_write.restype = c_i32
    L.qsa_sparse_attn_prefill.argtypes = [P(QkvCache), P(QsaArgs), c_vp]
    L.qsa_sparse_attn_prefill.restype = c_i32
    L.qsa_decode_workspace_bytes.argtypes = [c_i32, c_i32, c_i32, c_i32]
    L.qsa_decode_workspace_bytes.restype = c_sz
    L.qsa_sparse_attn_decode.argtypes = [P(QkvCache), P(QsaArgs), c_i32, c_vp, c_sz, c_vp]
    L.qsa_sparse_attn_decode.restype = c_i32
    L.qsa_sparse_attn_decode_noalloc.argtypes = [P(QkvCache), P(QsaArgs), c_i32, c_vp]
    L.qsa_sparse_attn_decode_noalloc.restype = c_i32
    L.qkv_calib_workspace_bytes.argtypes = []
    L.qkv_calib_workspace_bytes.restype = c_sz
    L.kv_calib_stats.argtypes = [c_vp, c_i32, c_i64, ctypes.c_float, c_vp, c_vp, c_sz, c_vp]
    L.kv_calib_stats.restype = c_i32
    L.qsa_topk_workspace_bytes.argtypes = [c_i32, c_i32, c_i32]
    L.qsa_topk_workspace_bytes.restype = c_sz
    L.qsa_topk_select.argtypes = [c_vp, c_i32, c_i32, c_i32, c_vp, c_i32, c_vp, c_vp, c_sz, c_vp]
    L.qsa_topk_select.restype = c_i32
    L.qkv_cache_bytes.argtypes = [c_i32, c_i32, c_i32, c_i32, c_i32, P(c_sz), P(c_sz), P(c_sz)]
    L.qkv_cache_bytes.restype = c_i32
    L.qkv_status_str.argtypes = [c_i32]
    L.qkv_status_str.restype = ctypes.c_char_p
    L.qkv_last_hip_error.argtypes = []
    L.qkv_last_hip_error.restype = c_i32
    L.qkv_abi_version.argtypes = []
    L.qkv_abi_version.restype = c_i32
    _lib = L
    return L


class QsakvError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = lib().qkv_status_str(status).decode()
        if status == ERR_HIP:
            msg += " (hipError %d)" % lib().qkv_last_hip_error()
        super().__init__("%s: %s" % (where, msg))


def _check(status, where):
    if status != OK:
        raise QsakvError(status, where)


_DT = {torch.bfloat16: BF16, torch.float16: FP16, torch.float32: FP32}


def dtype_code(t):
    return _DT[t.dtype]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def cache_bytes(kind, num_blocks, block_size, num_kv_heads, head_dim):
    """(k_bytes, v_bytes, scale_bytes) of a cache, from the library."""
    kb, vb, sb = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().qkv_cache_bytes(KIND_BY_NAME.get(kind, kind), num_blocks, block_size,
                                 num_kv_heads, head_dim, ctypes.byref(kb), ctypes.byref(vb),
                                 ctypes.byref(sb)), "qkv_cache_bytes")
    return kb.value, vb.value, sb.value


class Cache:
    """One layer's paged cache: device tensors plus the descriptor.

    ``k``/``v`` are uint8 tensors of the layout's bytes; ``kv_scale`` is the
    side tensor -- float32 row scales (int8), uint8 block-scale codes
    (nvfp4) -- or None; ``k_scale``/``v_scale`` are the per-layer E4M3 /
    NVFP4 scales (host floats).
    """

    def __init__(self, kind, num_blocks, block_size, num_kv_heads, head_dim, device="cuda",
                 k_scale=1.0, v_scale=1.0, zero=True):
        self.kind = kind
        self.kind_code = KIND_BY_NAME[kind]
        self.num_blocks, self.block_size = num_blocks, block_size
        self.num_kv_heads, self.head_dim = num_kv_heads, head_dim
        kb, vb, sb = cache_bytes(kind, num_blocks, block_size, num_kv_heads, head_dim)
        alloc = torch.zeros if zero else torch.empty
        self.k = alloc(kb, dtype=torch.uint8, device=device)
        self.v = alloc(vb, dtype=torch.uint8, device=device)
        if not sb:
            self.kv_scale = None
        elif kind == "nvfp4":
            self.kv_scale = alloc(sb, dtype=torch.uint8, device=device)
        else:
            self.kv_scale = alloc(sb // 4, dtype=torch.float32, device=device)
        self.k_scale = float(k_scale)
        self.v_scale = float(v_scale)

    @property
    def num_slots(self):
        return self.num_blocks * self.block_size

    def desc(self):
        return QkvCache(self.kind_code, self.num_blocks, self.block_size, self.num_kv_heads,
                        self.head_dim, 0, self.k.data_ptr(), self.v.data_ptr(),
                        None if self.kv_scale is None else self.kv_scale.data_ptr(),
                        self.k_scale, self.v_scale)

    def nbytes(self):
        return self.k.numel() + self.v.numel() + (0 if self.kv_scale is None else
                                                  self.kv_scale.numel() *
                                                  self.kv_scale.element_size())


def _tensor(name, t, dtypes, shape=None, ndim=None):
    """Check what the C ABI cannot see: a dense (contiguous) tensor of an
    accepted dtype and shape (None in ``shape`` = any size).  The device is
    checked by ``_on_device`` once every argument's metadata has passed."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s: expected a torch.Tensor, got %s" % (name, type(t).__name__))
    if t.dtype not in dtypes:
        raise TypeError("%s: dtype %s, expected one of %s" % (name, t.dtype, list(dtypes)))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s: %d dimensions, expected %d" % (name, t.dim(), ndim))
    if shape is not None and (t.dim() != len(shape) or
                              any(w is not None and g != w for g, w in zip(t.shape, shape))):
        raise ValueError("%s: shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise ValueError("%s: must be contiguous" % name)


def _on_device(**tensors):
    """After the metadata checks: every tensor given must be on the GPU."""
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError("%s: must be a CUDA (HIP) device tensor" % name)


_QDT = (torch.bfloat16, torch.float16)
_ODT = (torch.bfloat16, torch.float16, torch.float32)


def kv_quant_write(cache, k_src, v_src, slot_mapping, stream=None):
    """Quantize-on-write ``k_src``/``v_src`` [T][Hkv][D] into ``cache`` at
    ``slot_mapping`` [T] (int64; < 0 skips)."""
    shape = (None, cache.num_kv_heads, cache.head_dim)
    _tensor("k_src", k_src, _ODT, shape)
    T = k_src.shape[0]
    _tensor("v_src", v_src, (k_src.dtype,), (T,) + shape[1:])
    _tensor("slot_mapping", slot_mapping, (torch.int64,), (T,))
    _on_device(k_src=k_src, v_src=v_src, slot_mapping=slot_mapping)
    d = cache.desc()
    _check(lib().kv_quant_write(ctypes.byref(d), _ptr(k_src), _ptr(v_src), dtype_code(k_src), T,
                                _ptr(slot_mapping), _stream(stream)), "kv_quant_write")


def _check_attn(q, row_seq, block_table, topk_idx, out, lse):
    _tensor("q", q, _QDT, ndim=3)
    R, Hq, D = q.shape
    _tensor("out", out, _ODT, (R, Hq, D))
    _tensor("row_seq", row_seq, (torch.int32,), (R,))
    _tensor("block_table", block_table, (torch.int32,), ndim=2)
    _tensor("topk_idx", topk_idx, (torch.int32,), (R, None))
    if lse is not None:
        _tensor("lse", lse, (torch.float32,), (R, Hq))


def _qsa_args(q, row_seq, block_table, topk_idx, sm_scale, out, lse):
    R, Hq = q.shape[0], q.shape[1]
    return QsaArgs(q.data_ptr(), dtype_code(q), R, Hq, block_table.shape[0], row_seq.data_ptr(),
                   block_table.data_ptr(), block_table.shape[1], topk_idx.shape[1],
                   topk_idx.data_ptr(), float(sm_scale), dtype_code(out), out.data_ptr(),
                   None if lse is None else lse.data_ptr())


def qsa_sparse_attn_prefill(cache, q, row_seq, block_table, topk_idx, sm_scale, out, lse=None,
                            stream=None):
    """Single-pass sparse attention; writes ``out`` [R][Hq][D] and ``lse`` [R][Hq]."""
    _check_attn(q, row_seq, block_table, topk_idx, out, lse)
    _on_device(q=q, out=out, row_seq=row_seq, block_table=block_table, topk_idx=topk_idx,
               lse=lse)
    a = _qsa_args(q, row_seq, block_table, topk_idx, sm_scale, out, lse)
    d = cache.desc()
    _check(lib().qsa_sparse_attn_prefill(ctypes.byref(d), ctypes.byref(a), _stream(stream)),
           "qsa_sparse_attn_prefill")


def qsa_decode_workspace_bytes(num_rows, num_q_heads, head_dim, num_splits):
    return lib().qsa_decode_workspace_bytes(num_rows, num_q_heads, head_dim, num_splits)


def qsa_sparse_attn_decode(cache, q, row_seq, block_table, topk_idx, sm_scale, out, num_splits,
                           workspace, lse=None, stream=None):
    """Split-K sparse attention with log-sum-exp merge; ``workspace`` is a
    uint8 device tensor of at least qsa_decode_workspace_bytes(...) bytes."""
    _check_attn(q, row_seq, block_table, topk_idx, out, lse)
    if workspace is not None:
        _tensor("workspace", workspace, (torch.uint8,), ndim=1)
    _on_device(q=q, out=out, row_seq=row_seq, block_table=block_table, topk_idx=topk_idx,
               lse=lse, workspace=workspace)
    a = _qsa_args(q, row_seq, block_table, topk_idx, sm_scale, out, lse)
    d = cache.desc()
    wp = None if workspace is None else ctypes.c_void_p(workspace.data_ptr())
    wb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().qsa_sparse_attn_decode(ctypes.byref(d), ctypes.byref(a), num_splits, wp, wb,
                                        _stream(stream)), "qsa_sparse_attn_decode")


def qsa_sparse_attn_decode_noalloc(cache, q, row_seq, block_table, topk_idx, sm_scale, out,
                                   num_splits, lse=None, stream=None):
    """Split-K sparse attention with the partials in the library's static
    per-GPU scratch (no workspace argument, nothing allocated); calls that
    overlap in time on one GPU race."""
    _check_attn(q, row_seq, block_table, topk_idx, out, lse)
    _on_device(q=q, out=out, row_seq=row_seq, block_table=block_table, topk_idx=topk_idx,
               lse=lse)
    a = _qsa_args(q, row_seq, block_table, topk_idx, sm_scale, out, lse)
    d = cache.desc()
    _check(lib().qsa_sparse_attn_decode_noalloc(ctypes.byref(d), ctypes.byref(a), num_splits,
                                                _stream(stream)),
           "qsa_sparse_attn_decode_noalloc")


def calib_workspace_bytes():
    return int(lib().qkv_calib_workspace_bytes())


def kv_calib_stats(x, scale, out, workspace, stream=None):
    """Calibration statistics of the device tensor ``x`` (fp16 / bf16 / fp32,
    contiguous) at the E4M3 ``scale``, written by the library into ``out``
    (a device uint8 tensor of at least sizeof(qkv_calib_result) bytes)."""
    _tensor("x", x, _ODT)
    _tensor("out", out, (torch.uint8,), ndim=1)
    if out.numel() < ctypes.sizeof(QkvCalibResult):
        raise ValueError("out: %d bytes, need %d" % (out.numel(), ctypes.sizeof(QkvCalibResult)))
    _tensor("workspace", workspace, (torch.uint8,), ndim=1)
    _on_device(x=x, out=out, workspace=workspace)
    _check(lib().kv_calib_stats(_ptr(x), dtype_code(x), x.numel(), float(scale), _ptr(out),
                                _ptr(workspace), workspace.numel(), _stream(stream)),
           "kv_calib_stats")


def qsa_topk_workspace_bytes(num_rows, row_stride, topk):
    return int(lib().qsa_topk_workspace_bytes(num_rows, row_stride, topk))


def qsa_topk_select(scores, row_len, topk, out, workspace=None, stream=None):
    """Top-k positions of each row of the device tensor ``scores``
    ([R][row_stride], fp32 / fp16 / bf16, rows contiguous) among the first
    ``row_len[r]`` (device int32 [R]); the library writes the increasing,
    -1 padded lists into ``out`` (device int32 [R][topk]).  ``workspace``: a
    device uint8 tensor of qsa_topk_workspace_bytes(...) bytes when that is
    not 0."""
    if not isinstance(scores, torch.Tensor) or scores.dtype not in _ODT:
        raise TypeError("scores: expected an fp32 / fp16 / bf16 torch.Tensor")
    if scores.dim() != 2 or scores.stride(1) != 1:
        raise ValueError("scores: expected a 2-D tensor with contiguous rows")
    R = scores.shape[0]
    _tensor("row_len", row_len, (torch.int32,), (R,))
    _tensor("out", out, (torch.int32,), (R, topk))
    if workspace is not None:
        _tensor("workspace", workspace, (torch.uint8,), ndim=1)
    _on_device(scores=scores, row_len=row_len, out=out, workspace=workspace)
    wb = 0 if workspace is None else workspace.numel()
    _check(lib().qsa_topk_select(_ptr(scores), dtype_code(scores), R, scores.stride(0),
                                 _ptr(row_len), topk, _ptr(out), _ptr(workspace), wb,
                                 _stream(stream)),
           "qsa_topk_select")


def calib_result(out):
    """Read a qkv_calib_result from ``out`` (device or host uint8 tensor)."""
    raw = bytes(out[:ctypes.sizeof(QkvCalibResult)].cpu().numpy().tobytes())
    r = QkvCalibResult.from_buffer_copy(raw)
    return {k: getattr(r, k) for k, _ in QkvCalibResult._fields_ if k != "reserved"}
