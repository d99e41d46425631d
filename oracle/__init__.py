"""CPU oracle for top-k sparse attention over a paged, quantized KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code, table or
constant generator with the HIP library under ``quantized_kv_top_amd/``.

What it computes, and where the pages define it (page titles are those of the
five web pages the method is taken from):

* ``formats``   -- source upcasts; int8 per-(token, KV-head) symmetric
  quantization (page "int8 per-(token,head) KV cache for the Qwen3.8-Flash-Next
  QSA path", sections "Headline result" and "The finding worth upstreaming");
  OCP FP8 E4M3 ("e4m3fn") encode/decode with saturation (page "Qwen3.8 Flash
  Next NVFP4 QSA FP8 E4M3 KV Scales", section "Calibration", converter
  contract; page "[Model][SM70][FP8] Add calibrated E4M3 QSA KV cache",
  section "Why calibrated scale is part of this contract" for the 2^-9 / 2^-6
  boundaries); bf16 round-to-nearest-even for the bf16 comparison arm.
* ``cache``     -- the paged cache layouts (aligned side-tensor scales and the
  inline 260-byte slot) and quantize-on-write into them.
* ``attention`` -- index -> slot resolution through the block table, exact
  fp64 dequantization, dense fp64 softmax attention over each row's top-k list,
  and the split-K partition rule (page "[Perf][SM70][FP8] Hoist QSA E4M3 KV
  scales", section "Changes").
* ``calib``     -- per-tensor calibration statistics of an E4M3 cache source
  (max-abs, nearest-rank percentiles, saturation and low-magnitude counts at
  a scale; page "[Model][SM70][FP8] Add calibrated E4M3 QSA KV cache").
* ``topk``      -- top-k selection of each row's positions from indexer
  scores, and the selection-overlap metrics (same page, validated contract
  and validation sections).
* ``brute``     -- pure-Python-loop versions of the same steps for tiny
  inputs; used only to pin the vectorized oracle.

Every function here is pinned by a ``-m "not gpu"`` test against closed forms,
the pages' printed constants, library special cases or brute force; nothing is
"parity unpinned".
"""

from . import formats, cache, attention, brute, calib, topk  # noqa: F401
