"""Oracle paged KV cache: byte layouts and quantize-on-write.

Test infrastructure only (see package docstring).

Layouts (per layer; a "slot" is block * block_size + offset):

* ``int8``        K and V: int8 ``[slots][Hkv][D]``; scales in a separate
  float32 tensor ``[slots][Hkv][2]`` holding (K scale, V scale).  This is the
  aligned side-tensor layout of page "int8 per-(token,head) KV cache for the
  Qwen3.8-Flash-Next QSA path", section "The finding worth upstreaming": the
  int8 rows keep their natural alignment and the scales move out of the slot
  at identical memory cost.
* ``int8_inline`` K and V: ``[slots][Hkv][D + 4]`` bytes, the D int8 codes
  followed by the row's float32 scale (little endian) -- the 260-byte slot the
  same section measures against (D = 256).
* ``e4m3``        K and V: E4M3FN codes ``[slots][Hkv][D]``; one float32 scale
  per layer for K and one for V (page "[Model][SM70][FP8] Add calibrated E4M3
  QSA KV cache", section "Purpose").
* ``bf16``        K and V: bf16 ``[slots][Hkv][D]`` (comparison arm).
* ``nvfp4``       K and V: E2M1 codes packed two per byte ``[slots][Hkv][D/2]``
  (element 2j in the low nibble of byte j); E4M3 block scales in a side
  tensor of bytes ``[slots][Hkv][2][D/16]`` (K's blocks, then V's); one
  float32 scale per layer for K and one for V.  A reading (see
  ``formats.nvfp4_quantize``): the pages name NVFP4 KV storage only as a
  variant outside the E4M3 contract.

Each row is held here as raw bytes so that it can be compared bit for bit.
"""

import numpy as np

from . import formats

KINDS = ("int8", "int8_inline", "e4m3", "bf16", "nvfp4")


def row_bytes(kind, head_dim):
    """Bytes of one (token, KV head) row of K (or of V) in the cache tensor."""
    if kind == "int8":
        return head_dim
    if kind == "int8_inline":
        return head_dim + 4
    if kind == "e4m3":
        return head_dim
    if kind == "bf16":
        return 2 * head_dim
    if kind == "nvfp4":
        return head_dim // 2
    raise ValueError(kind)


def bytes_per_token(kind, num_kv_heads, head_dim):
    """K + V bytes one token occupies, scales included.

    Page "Qwen3.8-Flash-Next -- INT8 KV build (int8_per_token_head)", section
    "What it buys you": 1024 (bf16) vs 520 (int8) bytes per token per GPU.
    Per-layer E4M3 scales are per tensor, not per token, and add nothing.
    """
    per_row = row_bytes(kind, head_dim)
    if kind == "int8":
        per_row += 4                      # the row's fp32 scale in the side tensor
    if kind == "nvfp4":
        per_row += head_dim // formats.NVFP4_BLOCK   # the row's block scales
    return 2 * num_kv_heads * per_row


def pool_tokens(pool_bytes, kind, num_kv_heads, head_dim, block_size):
    """Tokens held by a pool of ``pool_bytes`` bytes, counting whole blocks."""
    per_block = bytes_per_token(kind, num_kv_heads, head_dim) * block_size
    return (int(pool_bytes) // per_block) * block_size


class OracleCache:
    """A zero-initialised paged cache written by the oracle."""

    def __init__(self, kind, num_blocks, block_size, num_kv_heads, head_dim,
                 k_scale=None, v_scale=None):
        if kind not in KINDS:
            raise ValueError(kind)
        self.kind = kind
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.num_kv_heads = num_kv_heads
        self.head_dim = head_dim
        n = num_blocks * block_size
        rb = row_bytes(kind, head_dim)
        self.k = np.zeros((n, num_kv_heads, rb), dtype=np.uint8)
        self.v = np.zeros((n, num_kv_heads, rb), dtype=np.uint8)
        self.kv_scale = (np.zeros((n, num_kv_heads, 2), dtype=np.float32)
                         if kind == "int8" else None)
        if kind == "nvfp4":
            self.kv_scale = np.zeros((n, num_kv_heads, 2, head_dim // formats.NVFP4_BLOCK),
                                     dtype=np.uint8)
        self.k_scale = None if k_scale is None else np.float32(k_scale)
        self.v_scale = None if v_scale is None else np.float32(v_scale)
        if kind in ("e4m3", "nvfp4") and (self.k_scale is None or self.v_scale is None):
            raise ValueError("%s cache needs per-layer k_scale and v_scale" % kind)

    @property
    def num_slots(self):
        return self.num_blocks * self.block_size

    # ------------------------------------------------------------------
    # quantize-on-write
    # ------------------------------------------------------------------
    def _encode_rows(self, x32, which):
        """x32: float32 [T][Hkv][D] -> (row bytes [T][Hkv][rb], scales or None)."""
        kind = self.kind
        if kind in ("int8", "int8_inline"):
            q, s = formats.int8_quantize(x32)
            qb = q.view(np.uint8)
            if kind == "int8":
                return qb, s
            sb = s.astype("<f4").view(np.uint8).reshape(s.shape + (4,))
            return np.concatenate([qb, sb], axis=-1), None
        if kind == "e4m3":
            scale = self.k_scale if which == "k" else self.v_scale
            return formats.e4m3_quantize(x32, scale), None
        if kind == "nvfp4":
            scale = self.k_scale if which == "k" else self.v_scale
            q, sc = formats.nvfp4_quantize(x32, scale)
            return formats.nvfp4_pack(q), sc
        if kind == "bf16":
            b = formats.f32_to_bf16_bits(x32)
            return b.astype("<u2").view(np.uint8).reshape(b.shape[:-1] + (2 * b.shape[-1],)), None
        raise ValueError(kind)

    def write(self, k_src, v_src, src_dtype, slot_mapping):
        """Quantize tokens and store them at their slots; slot < 0 is skipped.

        k_src, v_src: [T][Hkv][D] in ``src_dtype`` ('fp32', 'bf16' bit
        patterns as uint16, or 'fp16').  When a slot repeats, the later token
        wins (the tests never repeat a slot).
        """
        slots = np.asarray(slot_mapping, dtype=np.int64)
        keep = slots >= 0
        if not keep.any():
            return
        sl = slots[keep]
        for which, src in (("k", k_src), ("v", v_src)):
            x32 = formats.upcast_to_f32(np.asarray(src)[keep], src_dtype)
            rows, s = self._encode_rows(x32, which)
            getattr(self, which)[sl] = rows
            if s is not None:
                self.kv_scale[sl, :, 0 if which == "k" else 1] = s

    # ------------------------------------------------------------------
    # exact dequantization of stored rows
    # ------------------------------------------------------------------
    def dequant(self, slots, which):
        """Exact float64 values of stored rows: [n][Hkv][D]."""
        slots = np.asarray(slots, dtype=np.int64)
        raw = getattr(self, which)[slots]
        D = self.head_dim
        kind = self.kind
        if kind == "int8":
            q = raw.view(np.int8)
            s = self.kv_scale[slots, :, 0 if which == "k" else 1]
            return formats.int8_dequantize(q, s)
        if kind == "int8_inline":
            q = raw[..., :D].view(np.int8)
            s = np.ascontiguousarray(raw[..., D:D + 4]).view("<f4")[..., 0]
            return formats.int8_dequantize(q, s)
        if kind == "e4m3":
            scale = self.k_scale if which == "k" else self.v_scale
            return formats.e4m3_decode(raw) * np.float64(scale)
        if kind == "nvfp4":
            scale = self.k_scale if which == "k" else self.v_scale
            sc = self.kv_scale[slots, :, 0 if which == "k" else 1]
            return formats.nvfp4_dequantize(formats.nvfp4_unpack(raw), sc, scale)
        if kind == "bf16":
            bits = np.ascontiguousarray(raw).view("<u2")
            return formats.bf16_bits_to_f32(bits).astype(np.float64)
        raise ValueError(kind)
