"""Benchmark of the top-k sparse-attention hot path on one MI355X.

Default (the default line): the prefill workload -- 2048 query rows x top-k
1024 over a 32K-token paged int8 cache (Hq 16 / Hkv 2, D 256, BS 64, fp32
scales in the aligned side tensor), one ``qsa_sparse_attn_prefill`` call per
step, rotating over independent layer caches (each with its own top-k lists)
so that more than twice the 256 MB last-level cache passes between two
visits of the same cache.  Prints ONE JSON line, whose "sub" object also
times the tiny workload, the decode workload (split-K 8), the 12-layer E4M3
step (split-K 16) and the end-to-end chunk prefills in their 13.75 GiB pools
(whose gathers miss the L2), each against the 8 TB/s HBM peak (--no-sub
skips them).

Other workloads (``--config``) print their own line for the record:
decode (8 x 128K, 40 rows, top-k 2048, split-K 8), e4m3 (12 layers, 4 rows,
top-k 2051, split-K 8 or 1), mixed (12 E4M3 layers x a 46 + 1 + 1 + 1 row
batch in one launch), e2e (chunk write + prefill + 8 decode steps), calib
(E4M3 calibration statistics of 24 K/V tensors), write (quantize-on-write
throughput), topk (top-k selection of the lists from indexer scores).
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from quantized_kv_top_amd import qsakv                       # noqa: E402
from quantized_kv_top_amd import workloads as wl              # noqa: E402

METRIC = "top-k sparse-attn query rows/s + gathered-KV HBM GB/s (% of peak), int8/E4M3"
HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# the sources the attention kernels are built from (their launch parameters
# included): a change to any of them invalidates the committed counters
ATTN_SOURCES = ("attn.hip", "qsakv_device.h", "qsakv_internal.h", "qsakv_api.hip")


def source_sha():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_kv_top_amd", "csrc")
    for f in ATTN_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def gathered_bytes_per_row(kind, topk, hkv, d):
    """Algorithmic gathered-KV bytes per query row: every listed token's K and
    V row of every KV head, plus its int8 scales (4 B each) or NVFP4 block
    scales (1 B per 16 elements)."""
    per = {"int8": 2 * (d + 4), "int8_inline": 2 * (d + 4), "e4m3": 2 * d, "bf16": 4 * d,
           "nvfp4": 2 * (d // 2 + d // 16)}[kind]
    return topk * hkv * per


def traffic_from_profile(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel sources."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get("%s|%s" % (kernel, workload))
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != source_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


class Timer:
    """hipEvent pairs around every step on the stream the kernels run on."""

    def __init__(self, stream):
        self.stream = stream
        self.pairs = []

    def step(self, fn):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record(self.stream)
        fn()
        e.record(self.stream)
        self.pairs.append((s, e))

    def ms(self):
        torch.cuda.synchronize()
        return [s.elapsed_time(e) for s, e in self.pairs]


def timed_loop(fn, steps, warmup, stream):
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t = Timer(stream)
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        t.step(lambda: fn(warmup + i))
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = t.ms()
    return start.elapsed_time(end), per, wall


# ---------------------------------------------------------------------------
# prefill (default)
# ---------------------------------------------------------------------------

class PrefillLayer:
    def __init__(self, kind, seed, rows, topk):
        w = wl.prefill(device="cuda", seed=seed, num_rows=rows, topk=topk)
        self.w = w
        self.c = qsakv.Cache(kind, w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
        qsakv.kv_quant_write(self.c, w.k_src, w.v_src,
                             torch.from_numpy(w.slot_mapping).cuda())
        self.q = w.q
        self.rs = torch.from_numpy(w.row_seq).cuda()
        self.bt = torch.from_numpy(w.block_table).cuda()
        self.idx = torch.from_numpy(w.topk_idx).cuda()
        self.out = torch.empty(w.q.shape, dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty(w.q.shape[:2], dtype=torch.float32, device="cuda")
        w.k_src = w.v_src = None      # free the sources

    def __call__(self, stream):
        w = self.w
        qsakv.qsa_sparse_attn_prefill(self.c, self.q, self.rs, self.bt, self.idx, w.sm_scale,
                                      self.out, lse=self.lse, stream=stream)


def cpu_baseline_prefill(seed, budget_s, rows_cap):
    """The oracle, as it stands, on the first rows of one prefill layer: with
    all BLAS threads (the reported value) and again on one thread."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import attention as oatt
    from oracle import cache as ocache

    w = wl.prefill(device="cpu", seed=seed)
    oc = ocache.OracleCache("int8", w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    t0 = time.perf_counter()
    oc.write(wl.to_numpy_src(w.k_src), wl.to_numpy_src(w.v_src), "bf16", w.slot_mapping)
    write_s = time.perf_counter() - t0
    qn = wl.to_numpy_src(w.q)

    def rate(budget):
        done = 0
        t0 = time.perf_counter()
        while done < rows_cap and time.perf_counter() - t0 < budget:
            oatt.sparse_attention(oc, qn, "bf16", w.row_seq, w.block_table, w.topk_idx,
                                  w.sm_scale, rows=[done % w.num_rows])
            done += 1
        return done, time.perf_counter() - t0

    done, el = rate(budget_s)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    with threadpool_limits(limits=1):
        done1, el1 = rate(budget_s / 3)
    per_row = gathered_bytes_per_row("int8", w.topk, w.num_kv_heads, w.head_dim)
    return {"value": done / el, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": "%d prefill rows (rows 0.. of %d, cycled; top-k %d, fp64 numpy) in "
                      "%.1f s with %d BLAS threads; oracle quantize-on-write of all %d tokens "
                      "took %.1f s" % (done, w.num_rows, w.topk, el, threads,
                                       w.slot_mapping.size, write_s),
            "gathered_GBps": done / el * per_row / 1e9,
            "one_thread_rows_per_s": done1 / el1,
            "one_thread_gathered_GBps": done1 / el1 * per_row / 1e9}


def cpu_baseline_rows(make_workloads, kind, budget_s, what):
    """The oracle, as it stands, on whole small launches: each workload's
    listed tokens (only those) quantized into an oracle cache, then its rows'
    attention, timed with all BLAS threads (the reported value) and again on
    one thread."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import attention as oatt
    from oracle import cache as ocache

    jobs = []
    per_row = 0
    for w in make_workloads():
        ks, vs = layer_scales(kind, w.k_src, w.v_src)
        oc = ocache.OracleCache(kind, w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim,
                                k_scale=ks, v_scale=vs)
        ctx = w.slot_mapping.size // (int(w.row_seq.max()) + 1)
        tok = np.unique((w.row_seq.astype(np.int64)[:, None] * ctx + w.topk_idx).ravel())
        oc.write(wl.to_numpy_src(w.k_src)[tok], wl.to_numpy_src(w.v_src)[tok], w.src_dtype,
                 w.slot_mapping[tok])
        jobs.append((oc, wl.to_numpy_src(w.q), w))
        per_row = gathered_bytes_per_row(kind, w.topk, w.num_kv_heads, w.head_dim)
    nrows = sum(j[2].num_rows for j in jobs)

    def rate(budget):
        # the rows in order, cycled until the budget is spent
        done, t0 = 0, time.perf_counter()
        while True:
            for oc, qn, w in jobs:
                for r in range(w.num_rows):
                    if time.perf_counter() - t0 >= budget:
                        return done, time.perf_counter() - t0
                    oatt.sparse_attention(oc, qn, w.q_dtype, w.row_seq, w.block_table,
                                          w.topk_idx, w.sm_scale, rows=[r])
                    done += 1

    done, el = rate(budget_s)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    with threadpool_limits(limits=1):
        done1, el1 = rate(budget_s / 3)
    return {"value": done / el, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": "%d rows (%s, %d rows cycled; %s cache, fp64 numpy) in %.1f s with %d "
                      "BLAS threads" % (done, what, nrows, kind, el, threads),
            "gathered_GBps": done / el * per_row / 1e9,
            "one_thread_rows_per_s": done1 / el1,
            "one_thread_gathered_GBps": done1 / el1 * per_row / 1e9}


def bench_prefill(args):
    stream = torch.cuda.current_stream()
    rows, topk = 2048, 1024
    L = args.layers or 16
    res = {}
    for kind in ("int8", "int8_inline"):
        log("building %d %s prefill layers" % (L, kind))
        layers = [PrefillLayer(kind, 100 + i, rows, topk) for i in range(L)]
        torch.cuda.synchronize()
        total_ms, per, wall = timed_loop(lambda i: layers[i % L](stream), args.steps,
                                         args.warmup, stream)
        res[kind] = (total_ms, per, wall)
        log("%s: %.3f ms/step (events), per-step median %.3f ms" % (
            kind, total_ms / args.steps, float(np.median(per))))
        del layers
        torch.cuda.empty_cache()
    total_ms, per, wall = res["int8"]
    ms = total_ms / args.steps
    value = rows * args.steps / (total_ms / 1e3)
    bytes_launch = rows * gathered_bytes_per_row("int8", topk, 2, 256)
    kern_ms = float(np.mean(per))
    achieved = bytes_launch / (kern_ms / 1e3) / 1e9
    traffic = traffic_from_profile("qsa_attn16_kernel<int8,256,4>", "prefill")
    inl_ms = res["int8_inline"][0] / args.steps
    line = {
        "metric": METRIC, "value": value, "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8", "data": "synthetic",
        "config": {"workload": "prefill: 2048 query rows x top-k 1024 over a 32768-token paged "
                               "int8 cache (aligned side-tensor scales), Hq 16 / Hkv 2, D 256, "
                               "block 64, bf16 Q/out; %d independent layer caches rotated" % L,
                   "rows": rows, "topk": topk, "num_q_heads": 16, "num_kv_heads": 2,
                   "head_dim": 256, "block_size": 64, "context": 32768, "layers_rotated": L,
                   "gathered_kv_bytes_per_step": bytes_launch,
                   "gathered_kv_GBps": achieved,
                   "inline260_ms_per_step": inl_ms,
                   "inline260_over_aligned": inl_ms / ms},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": "qsa_attn16_kernel<int8,256,4>",
                     "kernel_ms": kern_ms,
                     "timing": "achieved and frac: mean of the per-launch hipEvent pairs on "
                               "the kernel's stream; value and frac_step_span: the span of "
                               "all timed steps",
                     "frac_step_span": bytes_launch / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS,
                     "cache_resident": "last-level cache: each 34 MB layer cache is re-read "
                                       "~64x within one launch, so most gathers are served "
                                       "by the 256 MB MALL; the e2e_chunk_prefill "
                                       "sub-records gather from 13.75 GiB pools whose reads "
                                       "miss the L2 (L2-to-fabric traffic 0.98-1.08x the "
                                       "gathered bytes)",
                     "traffic_over_algorithmic": None if traffic is None
                     else traffic / bytes_launch},
    }
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        line["cpu_baseline"] = cpu_baseline_prefill(100, args.cpu_budget, 1 << 30)
    if not args.no_sub:
        log("sub-records: tiny, decode, e4m3, e2e chunk prefills")
        e2e = sub_e2e_prefill(args)
        line["sub"] = {"tiny": sub_tiny(args), "decode": sub_decode(args),
                       "e4m3_12_layers": sub_e4m3(args),
                       "e2e_chunk_prefill_int8": e2e["int8"],
                       "e2e_chunk_prefill_e4m3": e2e["e4m3"],
                       "e2e_chunk_prefill_bf16": e2e["bf16"]}
    return line


# ---------------------------------------------------------------------------
# decode / e4m3 (small launches: timed as captured graphs of L calls)
# ---------------------------------------------------------------------------

class DecodeLayer:
    """One layer's cache and decode call.  ``bt``: the model's block-table
    tensor when the layers of a model share it (its contents must be the
    workload's)."""

    def __init__(self, w, kind, ks=1.0, vs=1.0, splits=8, bt=None):
        self.w = w
        self.splits = splits
        self.c = qsakv.Cache(kind, w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim,
                             k_scale=ks, v_scale=vs, zero=False)
        qsakv.kv_quant_write(self.c, w.k_src, w.v_src, torch.from_numpy(w.slot_mapping).cuda())
        self.q = w.q.contiguous()
        self.rs = torch.from_numpy(w.row_seq).cuda()
        if bt is not None:
            assert np.array_equal(bt.cpu().numpy(), w.block_table)
            self.bt = bt
        else:
            self.bt = torch.from_numpy(w.block_table).cuda()
        self.idx = torch.from_numpy(w.topk_idx).cuda()
        R, Hq, D = w.q.shape
        odt = torch.float16 if w.out_dtype == "fp16" else torch.bfloat16
        self.out = torch.empty((R, Hq, D), dtype=odt, device="cuda")
        self.lse = torch.empty((R, Hq), dtype=torch.float32, device="cuda")
        nb = qsakv.qsa_decode_workspace_bytes(R, Hq, D, splits)
        self.ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device="cuda")
        w.k_src = w.v_src = None

    def __call__(self, stream):
        w = self.w
        qsakv.qsa_sparse_attn_decode(self.c, self.q, self.rs, self.bt, self.idx, w.sm_scale,
                                     self.out, self.splits, self.ws, lse=self.lse, stream=stream)


def graph_loop(layers, steps, warmup, reps):
    """Capture one pass over all layers into a graph; time ``steps`` replays."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            for lay in layers:
                lay(s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(reps):
            for lay in layers:
                lay(s)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    total, per, wall = timed_loop(lambda i: g.replay(), steps, 0, st)
    return total, per


def layer_scales(kind, k_src, v_src):
    """Per-layer (k_scale, v_scale): max|x| / 448 (E4M3), max|x| / (6 * 448)
    (NVFP4), 1 otherwise."""
    if kind not in ("e4m3", "nvfp4"):
        return 1.0, 1.0
    d = np.float32(448.0 if kind == "e4m3" else 6.0 * 448.0)
    return tuple(float(np.float32(t.abs().max().float().item()) / d) for t in (k_src, v_src))


def run_decode(kind, L, splits, steps, warmup):
    """The decode workload's layers (8 x 128K tokens each; one block table)
    as one graph: (ms per call, rows per call, gathered bytes per call)."""
    log("building %d decode layers (8 x 128K tokens each, %s)" % (L, kind))
    layers = []
    for i in range(L):
        # layers of one model: one block table (shared tensor), own lists and data
        w = wl.decode(device="cuda", seed=200, layer=i)
        layers.append(DecodeLayer(w, kind, *layer_scales(kind, w.k_src, w.v_src), splits,
                                  bt=layers[0].bt if layers else None))
    torch.cuda.synchronize()
    total, per = graph_loop(layers, steps, warmup, 1)
    w = layers[0].w
    rows = w.num_rows
    b = rows * gathered_bytes_per_row(kind, w.topk, 2, 256)
    del layers
    torch.cuda.empty_cache()
    return total / (steps * L), rows, b


def bench_decode(args):
    L = args.layers or 8
    kind = args.kind or "int8"
    ms_call, rows, b = run_decode(kind, L, args.splits, args.steps, args.warmup)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_rows(lambda: [wl.decode(device="cpu", seed=200, layer=0)], kind,
                                args.cpu_budget, "all 40 decode rows of one layer, top-k 2048")
    return {"metric": METRIC, "value": rows / (ms_call / 1e3), "unit": "rows/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_call,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": kind,
            "data": "synthetic",
            "config": {"workload": "decode: 8 seqs x 128K ctx, 5 rows each (40), top-k 2048 "
                                   "(70%% recent window), split-K %d + merge, %s cache; "
                                   "%d layers rotated, graph-captured" % (args.splits, kind, L),
                       "gathered_kv_bytes_per_call": b,
                       "gathered_kv_GBps": b / (ms_call / 1e3) / 1e9,
                       "hbm_frac": b / (ms_call / 1e3) / 1e9 / HBM_PEAK_GBPS},
            "cpu_baseline": cpu}


def run_e4m3(kind, sets, splits, steps, warmup):
    """``sets`` independent 12-layer models of the E4M3 workload (each with
    one block table) as one graph: (ms per 12-layer step, rows per layer,
    gathered bytes per 12-layer step)."""
    L = 12
    log("building %d x %d %s layers" % (L, sets, kind))
    layers = []
    for s in range(sets):
        for layer in range(L):
            # the 12 layers of a set are one model: one block-table tensor
            w = wl.e4m3_layer(layer, device="cuda", seed=4 + 1000 * s)
            layers.append(DecodeLayer(w, kind, *layer_scales(kind, w.k_src, w.v_src), splits,
                                      bt=layers[-layer].bt if layer else None))
    torch.cuda.synchronize()
    total, per = graph_loop(layers, steps, warmup, 1)
    w = layers[0].w
    rows = w.num_rows
    b = L * rows * gathered_bytes_per_row(kind, w.topk, 4, 128)
    del layers
    torch.cuda.empty_cache()
    return total / steps / sets, rows, b


def bench_e4m3(args):
    L = 12
    sets = args.layers or 4        # independent caches per layer position
    splits = args.splits
    kind = args.kind or "e4m3"     # nvfp4: the same 12-layer shape in NVFP4 caches
    ms_step, rows, b = run_e4m3(kind, sets, splits, args.steps, args.warmup)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_rows(lambda: [wl.e4m3_layer(i, device="cpu", seed=4) for i in range(3)],
                                kind, args.cpu_budget, "the 4 rows of layers 0-2 of 12")
    return {"metric": METRIC, "value": L * rows / (ms_step / 1e3),
            "unit": "layer-rows/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": kind, "data": "synthetic",
            "config": {"workload": "%s: 12 layers x 4 rows, top-k 2051, Hq 32 / Hkv 4, D 128, "
                                   "split-K %d; %d independent 12-layer sets rotated, "
                                   "graph-captured" % (kind, splits, sets),
                       "gathered_kv_bytes_per_step": b,
                       "gathered_kv_GBps": b / (ms_step / 1e3) / 1e9,
                       "hbm_frac": b / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBPS},
            "cpu_baseline": cpu}


class MixedLayer:
    """An E4M3 layer attended by 49 rows (46 + 1 + 1 + 1) either in one
    launch or, as the row-routing reference, in two launches (rows 0-45,
    then rows 46-48)."""

    def __init__(self, layer, seed, splits):
        w = wl.mixed_layer(layer, device="cuda", seed=seed)
        ks = float(np.float32(w.k_src.abs().max().float().item()) / np.float32(448))
        vs = float(np.float32(w.v_src.abs().max().float().item()) / np.float32(448))
        self.w, self.splits = w, splits
        self.c = qsakv.Cache("e4m3", w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim,
                             k_scale=ks, v_scale=vs, zero=False)
        qsakv.kv_quant_write(self.c, w.k_src, w.v_src, torch.from_numpy(w.slot_mapping).cuda())
        w.k_src = w.v_src = None
        self.bt = torch.from_numpy(w.block_table).cuda()
        R, Hq, D = w.q.shape
        self.parts = []
        for lo, hi in ((0, R), (0, 46), (46, R)):
            q = w.q[lo:hi].contiguous()
            rs = torch.from_numpy(w.row_seq[lo:hi].copy()).cuda()
            idx = torch.from_numpy(w.topk_idx[lo:hi].copy()).cuda()
            out = torch.empty((hi - lo, Hq, D), dtype=torch.float16, device="cuda")
            ws = torch.zeros(max(qsakv.qsa_decode_workspace_bytes(hi - lo, Hq, D, splits), 256),
                             dtype=torch.uint8, device="cuda")
            self.parts.append((q, rs, idx, out, ws))

    def _call(self, i, stream):
        q, rs, idx, out, ws = self.parts[i]
        qsakv.qsa_sparse_attn_decode(self.c, q, rs, self.bt, idx, self.w.sm_scale, out,
                                     self.splits, ws, stream=stream)

    def one_launch(self, stream):
        self._call(0, stream)

    def two_launches(self, stream):
        self._call(1, stream)
        self._call(2, stream)


class _Fn:
    def __init__(self, fn):
        self.fn = fn

    def __call__(self, stream):
        self.fn(stream)


def bench_mixed(args):
    """12 E4M3 layers; each layer is attended by one batch of 49 rows (46 rows
    of one sequence's chunk, then one row from each of three other
    sequences, the last with a shorter list), split-K ``--splits``; the
    batch as one launch per layer against the same rows routed as two
    launches."""
    L = 12
    sets = args.layers or 2
    log("building %d x %d mixed-batch layers" % (L, sets))
    layers = [MixedLayer(layer, 6 + 1000 * s, args.splits) for s in range(sets)
              for layer in range(L)]
    torch.cuda.synchronize()
    one, _ = graph_loop([_Fn(x.one_launch) for x in layers], args.steps, args.warmup, 1)
    two, _ = graph_loop([_Fn(x.two_launches) for x in layers], args.steps, args.warmup, 1)
    w = layers[0].w
    valid = int((w.topk_idx >= 0).sum())
    b = L * valid * w.num_kv_heads * 2 * w.head_dim
    ms1 = one / args.steps / sets
    ms2 = two / args.steps / sets
    return {"metric": METRIC, "value": L * w.num_rows / (ms1 / 1e3), "unit": "layer-rows/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms1,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "e4m3",
            "data": "synthetic",
            "config": {"workload": "mixed: 12 E4M3 layers (Hq 32 / Hkv 4, D 128, 64K ctx) x a "
                                   "49-row batch = 46 catch-up rows + 3 decode rows (top-k 2051, "
                                   "the last row 1500), split-K %d, one launch per layer; %d "
                                   "independent 12-layer sets rotated, graph-captured"
                                   % (args.splits, sets),
                       "gathered_kv_bytes_per_step": b,
                       "gathered_kv_GBps": b / (ms1 / 1e3) / 1e9,
                       "two_launch_routing_ms_per_step": ms2,
                       "two_launch_over_one": ms2 / ms1}}


def bench_calib(args):
    """Calibration statistics of the E4M3 workload's 24 K/V source tensors
    (12 layers x K, V; fp16 [4 x 65536][4][128] each, 268 MB) at their
    envelope scales max|x| / 448: one kv_calib_stats call per tensor."""
    stream = torch.cuda.current_stream()
    tensors = []
    log("building 12 E4M3 layers' K/V sources")
    for layer in range(12):
        w = wl.e4m3_layer(layer, device="cuda", seed=4)
        for t in (w.k_src, w.v_src):
            x = t.reshape(-1)
            amax = float(x.abs().max().float().item())
            tensors.append((x, float(np.float32(amax) / np.float32(448))))
    out = torch.zeros(64, dtype=torch.uint8, device="cuda")
    ws = torch.zeros(qsakv.calib_workspace_bytes(), dtype=torch.uint8, device="cuda")
    n = len(tensors)
    total, per, _ = timed_loop(lambda i: qsakv.kv_calib_stats(tensors[i % n][0], tensors[i % n][1],
                                                              out, ws, stream=stream),
                               args.steps, args.warmup, stream)
    ms = total / args.steps
    b = tensors[0][0].numel() * 2
    res = []
    for x, sc in tensors[:2]:
        qsakv.kv_calib_stats(x, sc, out, ws, stream=stream)
        torch.cuda.synchronize()
        res.append(qsakv.calib_result(out))
    return {"metric": "calibration statistics GB/s (E4M3 K/V sources)", "value": b / (ms / 1e3) / 1e9,
            "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "fp16", "data": "synthetic",
            "config": {"workload": "kv_calib_stats over 24 fp16 tensors of 134,217,728 "
                                   "elements (12 layers x K, V), one call per tensor, rotated",
                       "bytes_per_call": b, "hbm_frac": b / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS,
                       "layer0_k": res[0], "layer0_v": res[1]}}


def bench_topk(args):
    """Top-k selection from indexer scores: the prefill rows (2048 x 32768
    fp32 scores, top-1024; the value), the same in fp16 (two score sets
    rotated) and the decode rows (40 x 131072 fp32, top-2048; 16 sets
    rotated).  Algorithmic bytes: the candidates' scores read once plus the
    lists written."""
    stream = torch.cuda.current_stream()
    arms = {}
    for name, sets in (("prefill_fp32", [wl.prefill_scores("cuda", seed=12)]),
                       ("prefill_fp16", [wl.prefill_scores("cuda", seed=12 + i, dtype=torch.float16)
                                         for i in range(2)]),
                       ("decode_fp32", [wl.decode_scores("cuda", seed=13 + i) for i in range(16)])):
        s0 = sets[0]
        R, k = s0.scores.shape[0], s0.topk
        lens = [torch.from_numpy(s.row_len).cuda() for s in sets]
        outs = [torch.empty((R, k), dtype=torch.int32, device="cuda") for _ in sets]
        nb = qsakv.qsa_topk_workspace_bytes(R, s0.scores.shape[1], k)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda") if nb else None
        n = len(sets)
        total, per, _ = timed_loop(lambda i: qsakv.qsa_topk_select(sets[i % n].scores, lens[i % n], k,
                                                                   outs[i % n], workspace=ws,
                                                                   stream=stream),
                                   args.steps, args.warmup, stream)
        ms = total / args.steps
        b = int(s0.row_len.astype(np.int64).sum()) * s0.scores.element_size() + R * k * 4
        arms[name] = {"rows": R, "row_stride": s0.scores.shape[1], "topk": k, "ms": ms,
                      "rows_per_s": R / (ms / 1e3), "GBps": b / (ms / 1e3) / 1e9,
                      "bytes_per_call": b, "hbm_frac": b / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS}
        log("topk", name, "%.4f ms" % ms)
        del sets, lens, outs
    a = arms["prefill_fp32"]
    return {"metric": "top-k selection rows/s (indexer scores -> sparse-attention lists)",
            "value": a["rows_per_s"], "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": a["ms"], "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
            "config": {"workload": "qsa_topk_select: 2048 prefill rows x 32768 fp32 scores "
                                   "(row r scores its causal prefix), top-1024",
                       "arms": arms},
            "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_topk()}


def cpu_baseline_topk(rows=2048):
    """The selection oracle, as it stands (numpy, one process), on the first
    prefill rows' fp32 scores."""
    from oracle import topk as otopk
    s = wl.prefill_scores("cpu", seed=12)
    src = s.scores[:rows].numpy()
    t0 = time.perf_counter()
    otopk.topk_select(src, "fp32", s.row_len[:rows], s.topk)
    el = time.perf_counter() - t0
    return {"value": rows / el, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": "%d prefill rows (32K fp32 scores each, top-1024) in %.1f s" % (rows, el)}


class E2ELayer:
    """One layer of the end-to-end step in its own 13.75 GiB pool: the
    existing context written once; the chunk, its prefill and the decode
    steps are what the timed loops run."""

    def __init__(self, kind, seed):
        per_block = sum(qsakv.cache_bytes(kind, 1, 64, 2, 256))
        self.pool_blocks = wl.E2E_POOL_BYTES // per_block
        e = wl.e2e(self.pool_blocks, device="cuda", seed=seed)
        # per-layer scales (E4M3, NVFP4) over everything the layer holds
        ks, vs = layer_scales(kind, torch.cat([e.ctx_k, e.chunk_k, e.step_k]),
                              torch.cat([e.ctx_v, e.chunk_v, e.step_v]))
        self.c = qsakv.Cache(kind, self.pool_blocks, 64, 2, 256, k_scale=ks, v_scale=vs,
                             zero=False)
        qsakv.kv_quant_write(self.c, e.ctx_k, e.ctx_v, torch.from_numpy(e.ctx_slots).cuda())
        self.e = e
        self.chunk_slots = torch.from_numpy(e.chunk_slots).cuda()
        self.step_slots = torch.from_numpy(e.step_slots).cuda()
        self.bt = torch.from_numpy(e.block_table).cuda()
        self.rs_chunk = torch.zeros(e.chunk_q.shape[0], dtype=torch.int32, device="cuda")
        self.rs_one = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.chunk_idx = torch.from_numpy(e.chunk_topk).cuda()
        self.step_idx = [torch.from_numpy(e.step_topk[i:i + 1]).cuda()
                         for i in range(e.step_topk.shape[0])]
        self.chunk_out = torch.empty(e.chunk_q.shape, dtype=torch.bfloat16, device="cuda")
        self.step_out = torch.empty((1,) + tuple(e.step_q.shape[1:]), dtype=torch.bfloat16,
                                    device="cuda")
        self.ws = torch.zeros(qsakv.qsa_decode_workspace_bytes(1, 16, 256, 8),
                              dtype=torch.uint8, device="cuda")
        e.ctx_k = e.ctx_v = None

    def write_chunk(self, stream):
        qsakv.kv_quant_write(self.c, self.e.chunk_k, self.e.chunk_v, self.chunk_slots,
                             stream=stream)

    def prefill(self, stream):
        e = self.e
        qsakv.qsa_sparse_attn_prefill(self.c, e.chunk_q, self.rs_chunk, self.bt, self.chunk_idx,
                                      e.sm_scale, self.chunk_out, stream=stream)

    def decode_steps(self, stream):
        e = self.e
        for i in range(len(self.step_idx)):
            qsakv.kv_quant_write(self.c, e.step_k[i:i + 1], e.step_v[i:i + 1],
                                 self.step_slots[i:i + 1], stream=stream)
            qsakv.qsa_sparse_attn_decode(self.c, e.step_q[i:i + 1], self.rs_one, self.bt,
                                         self.step_idx[i], e.sm_scale, self.step_out, 8,
                                         self.ws, stream=stream)


def bench_e2e(args):
    """The end-to-end layer step of one 131K-token sequence in a 13.75 GiB
    pool per cache kind: write an 8192-token chunk (quantize-on-write),
    prefill its 8192 rows with top-k 1024, then 8 decode steps of [write one
    token, attend with top-k 2048, split-K 8] (graph-captured).  Each arm
    cycles over ``--layers`` (default 2) independent layers, each with its
    own pool."""
    stream = torch.cuda.current_stream()
    L = args.layers or 2
    arms = {}
    for kind in ("int8", "int8_inline", "bf16", "e4m3", "nvfp4"):
        log("building %d e2e layers (%s)" % (L, kind))
        layers = [E2ELayer(kind, 5 + 100 * i) for i in range(L)]
        for lay in layers:       # the step's inputs are device-resident before timing
            lay.e.step_k, lay.e.step_v = lay.e.step_k.contiguous(), lay.e.step_v.contiguous()
        e = layers[0].e
        R, topk = e.chunk_q.shape[0], e.chunk_topk.shape[1]
        torch.cuda.synchronize()
        wr, _, _ = timed_loop(lambda i: layers[i % L].write_chunk(stream), args.steps,
                              args.warmup, stream)
        pf, _, _ = timed_loop(lambda i: layers[i % L].prefill(stream), args.steps,
                              args.warmup, stream)
        # the decode steps (16 small launches) as one captured graph per layer,
        # so that host launch overhead stays out of their time
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for lay in layers:
                lay.decode_steps(side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for lay in layers:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                lay.decode_steps(side)
            graphs.append(g)
        dc, _, _ = timed_loop(lambda i: graphs[i % L].replay(), args.steps, args.warmup, stream)
        pf_ms, wr_ms, dc_ms = pf / args.steps, wr / args.steps, dc / args.steps
        pb = R * gathered_bytes_per_row(kind, topk, 2, 256)
        per_tok = sum(qsakv.cache_bytes(kind, 1, 64, 2, 256)) // 64
        arms[kind] = {
            "pool_blocks": int(layers[0].pool_blocks),
            "pool_tokens": int(layers[0].pool_blocks) * 64,
            "cache_bytes_per_token": int(per_tok),
            "chunk_write_ms": wr_ms,
            "chunk_prefill_ms": pf_ms,
            "chunk_prefill_rows_per_s": R / (pf_ms / 1e3),
            "chunk_prefill_gathered_GBps": pb / (pf_ms / 1e3) / 1e9,
            "decode_8_steps_ms": dc_ms,
            "layer_step_ms": wr_ms + pf_ms + dc_ms,
        }
        log("%s: write %.3f ms, prefill %.3f ms (%.0f GB/s), 8 decode steps %.3f ms" % (
            kind, wr_ms, pf_ms, arms[kind]["chunk_prefill_gathered_GBps"], dc_ms))
        del graphs, layers
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    for kind in arms:
        arms[kind]["pool_tokens_vs_bf16"] = arms[kind]["pool_tokens"] / arms["bf16"]["pool_tokens"]
    a = arms["int8"]
    return {"metric": METRIC, "value": a["chunk_prefill_rows_per_s"], "unit": "rows/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": a["chunk_prefill_ms"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "int8", "data": "synthetic",
            "config": {"workload": "e2e: one 131K-token sequence per layer in a 13.75 GiB pool "
                                   "(Hq 16 / Hkv 2, D 256, block 64, bf16 Q/out); 8192-token "
                                   "chunk write + prefill (top-k 1024) + 8 x [write 1 token, "
                                   "decode top-k 2048, split-K 8] (one graph); %d layers rotated; "
                                   "value = "
                                   "int8 chunk-prefill rows/s" % L,
                       "arms": arms,
                       "inline260_over_aligned_prefill": arms["int8_inline"]["chunk_prefill_ms"]
                       / a["chunk_prefill_ms"],
                       "hbm_frac_int8_prefill": a["chunk_prefill_gathered_GBps"] / HBM_PEAK_GBPS}}


def bench_write(args):
    """Quantize-on-write of 262,144 tokens (Hkv 2, D 256, bf16 sources) into
    int8 and E4M3 caches, beside a plain device copy of the same source
    bytes as the read+write reference."""
    stream = torch.cuda.current_stream()
    w = wl.decode(device="cuda", seed=300, num_seqs=2)
    sm = torch.from_numpy(w.slot_mapping).cuda()
    T = w.slot_mapping.size
    arms = {}
    for kind in ("int8", "e4m3", "nvfp4"):
        c = qsakv.Cache(kind, w.num_blocks, w.block_size, 2, 256, k_scale=0.05, v_scale=0.05,
                        zero=False)
        total, _, _ = timed_loop(lambda i: qsakv.kv_quant_write(c, w.k_src, w.v_src, sm,
                                                                stream=stream),
                                 args.steps, args.warmup, stream)
        ms = total / args.steps
        per_tok = 2 * 2 * (2 * 256 + {"int8": 256 + 4, "e4m3": 256, "nvfp4": 128 + 16}[kind])
        arms[kind] = {"ms": ms, "tokens_per_s": T / (ms / 1e3),
                      "GBps": T * per_tok / (ms / 1e3) / 1e9, "bytes_per_token": per_tok}
        del c
    src = torch.cat([w.k_src.reshape(-1), w.v_src.reshape(-1)])
    dst = torch.empty_like(src)
    total, _, _ = timed_loop(lambda i: dst.copy_(src), args.steps, args.warmup, stream)
    cms = total / args.steps
    a = arms["int8"]
    return {"metric": "quantize-on-write tokens/s", "value": a["tokens_per_s"], "unit": "tokens/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": a["ms"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
            "data": "synthetic",
            "config": {"workload": "kv_quant_write: %d tokens, Hkv 2, D 256, bf16 src; value = "
                                   "int8 (side scales)" % T,
                       "bytes_per_call": T * a["bytes_per_token"], "GBps": a["GBps"],
                       "arms": arms,
                       "device_copy_of_sources_GBps": 2 * src.numel() * 2 / (cms / 1e3) / 1e9}}


# ---------------------------------------------------------------------------
# sub-records of the default line: the other workloads the method is judged
# on, each timed on the device as the standalone configs time it
# ---------------------------------------------------------------------------

def sub_record(workload, ms, rows, bytes_call, timing, **extra):
    gbps = bytes_call / (ms / 1e3) / 1e9
    rec = {"workload": workload, "ms_per_call": ms, "rows_per_s": rows / (ms / 1e3),
           "gathered_kv_bytes_per_call": bytes_call, "gathered_kv_GBps": gbps,
           "frac_of_hbm_peak": gbps / HBM_PEAK_GBPS, "timing": timing}
    rec.update(extra)
    return rec


class TinyCall:
    """The tiny workload's 4 rows (top-k 16 over 64 tokens, int8) in one
    prefill call."""

    def __init__(self):
        w = wl.tiny(device="cuda")
        self.w = w
        self.c = qsakv.Cache("int8", w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
        qsakv.kv_quant_write(self.c, w.k_src, w.v_src, torch.from_numpy(w.slot_mapping).cuda())
        self.q = w.q.contiguous()
        self.rs = torch.from_numpy(w.row_seq).cuda()
        self.bt = torch.from_numpy(w.block_table).cuda()
        self.idx = torch.from_numpy(w.topk_idx).cuda()
        self.out = torch.empty(w.q.shape, dtype=torch.float32, device="cuda")

    def __call__(self, stream):
        qsakv.qsa_sparse_attn_prefill(self.c, self.q, self.rs, self.bt, self.idx,
                                      self.w.sm_scale, self.out, stream=stream)


def sub_tiny(args):
    t = TinyCall()
    torch.cuda.synchronize()
    reps = 32
    total, _ = graph_loop([t], args.steps, args.warmup, reps)
    ms = total / (args.steps * reps)
    w = t.w
    b = w.num_rows * gathered_bytes_per_row("int8", w.topk, w.num_kv_heads, w.head_dim)
    rec = sub_record("tiny: 4 rows x top-k 16 over a 64-token int8 cache (4 blocks of 16), "
                     "Hq 4 / Hkv 1, D 128, one prefill call; latency-bound (reported, not "
                     "judged)", ms, w.num_rows, b,
                     "graph of %d calls replayed %d times, hipEvents" % (reps, args.steps))
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_rows(lambda: [wl.tiny()], "int8",
                                                min(args.cpu_budget, 3.0), "all 4 tiny rows")
    return rec


# oracle seconds per sub-record baseline (the main line's takes --cpu-budget)
SUB_CPU_BUDGET = 8.0


def sub_decode(args):
    ms, rows, b = run_decode("int8", 8, 8, args.steps, args.warmup)
    rec = sub_record("decode: 8 seqs x 128K ctx, 40 rows (5 per seq), top-k 2048 (70% "
                     "recent window), Hq 16 / Hkv 2, D 256, int8, split-K 8 + merge; 8 layers "
                     "(one block table) rotated", ms, rows, b,
                     "graph of the 8 layers' calls, per call", num_splits=8)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_rows(
            lambda: [wl.decode(device="cpu", seed=200, layer=0)], "int8",
            min(args.cpu_budget, SUB_CPU_BUDGET), "all 40 decode rows of one layer, top-k 2048")
    return rec


C4_SPLITS = 16


def sub_e4m3(args):
    ms, rows, b = run_e4m3("e4m3", 4, C4_SPLITS, args.steps, args.warmup)
    rec = sub_record("e4m3: 12 layers x 4 rows, top-k 2051, Hq 32 / Hkv 4, D 128, calibrated "
                     "E4M3 caches, split-K %d + merge; 4 independent 12-layer models rotated; "
                     "per 12-layer step" % C4_SPLITS, ms, 12 * rows, b,
                     "graph of 4 x 12 layer calls, per 12-layer step",
                     num_splits=C4_SPLITS, unit_rows="layer-rows")
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_rows(
            lambda: [wl.e4m3_layer(i, device="cpu", seed=4) for i in range(3)], "e4m3",
            min(args.cpu_budget, SUB_CPU_BUDGET), "the 4 rows of layers 0-2 of 12 (layer-rows)")
    return rec


def e2e_chunk_oracle_workload(rows=512):
    """The first ``rows`` rows of the end-to-end chunk prefill for the oracle:
    the sequence's 131,072 existing and chunk tokens in a cache of exactly
    its 2049 blocks (where the blocks sit in a pool does not change the
    oracle's arithmetic, only the size of the host arrays)."""
    e = wl.e2e(2049, device="cpu", seed=5)
    return wl.Workload("e2e chunk", e.num_q_heads, e.num_kv_heads, e.head_dim, e.block_size,
                       2049, "bf16", "bf16", "bf16", torch.cat([e.ctx_k, e.chunk_k]),
                       torch.cat([e.ctx_v, e.chunk_v]),
                       np.concatenate([e.ctx_slots, e.chunk_slots]), e.chunk_q[:rows],
                       np.zeros(rows, np.int32), e.block_table, e.chunk_topk[:rows], e.sm_scale)


def sub_e2e_prefill(args, kinds=("int8", "e4m3", "bf16")):
    stream = torch.cuda.current_stream()
    recs = {}
    for kind in kinds:
        log("building 2 e2e layers (%s, 13.75 GiB pool each)" % kind)
        layers = [E2ELayer(kind, 5 + 100 * i) for i in range(2)]
        e = layers[0].e
        R, topk = e.chunk_q.shape[0], e.chunk_topk.shape[1]
        torch.cuda.synchronize()
        total, per, _ = timed_loop(lambda i: layers[i % 2].prefill(stream), args.steps,
                                   args.warmup, stream)
        b = R * gathered_bytes_per_row(kind, topk, 2, 256)
        recs[kind] = sub_record(
            "e2e chunk prefill: 8192 rows x top-k 1024 over one 131K-token sequence whose "
            "blocks are spread over a 13.75 GiB %s pool (gathers miss the L2), Hq 16 / Hkv 2, "
            "D 256; 2 layers rotated" % kind, total / args.steps, R, b,
            "hipEvents around the steps", pool_tokens=int(layers[0].pool_blocks) * 64)
        if kind == "int8" and not args.no_cpu_baseline:
            recs[kind]["cpu_baseline"] = cpu_baseline_rows(
                lambda: [e2e_chunk_oracle_workload()], "int8",
                min(args.cpu_budget, SUB_CPU_BUDGET),
                "the first 512 of the 8192 chunk rows, top-k 1024")
        del layers, e
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return recs


def bench_copy(args):
    """A plain 1 GiB device copy: the known-size kernel that calibrates the
    FETCH_SIZE / WRITE_SIZE counters."""
    x = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    for _ in range(args.steps):
        y.copy_(x)
    torch.cuda.synchronize()
    return {"metric": "copy", "value": 1 << 30, "unit": "bytes", "n_gpus": 1}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="prefill",
                    choices=["prefill", "decode", "e4m3", "mixed", "e2e", "calib", "write",
                             "topk", "copy"])
    ap.add_argument("--layers", type=int, default=0)
    ap.add_argument("--splits", type=int, default=8)
    ap.add_argument("--kind", default=None, choices=["int8", "e4m3", "bf16", "nvfp4"],
                    help="cache kind of the decode / e4m3 configs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sub", action="store_true",
                    help="prefill line only: skip the other workloads' sub-records")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the per-GPU share is the single-GPU workload); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    qsakv.lib()
    fn = {"prefill": bench_prefill, "decode": bench_decode, "e4m3": bench_e4m3,
          "mixed": bench_mixed, "e2e": bench_e2e, "calib": bench_calib, "write": bench_write,
          "topk": bench_topk, "copy": bench_copy}[args.config]
    print(json.dumps(fn(args)), flush=True)


if __name__ == "__main__":
    main()
