"""Host-side logic of bench.py that needs no GPU: the one-GPU refusal, the
algorithmic byte counts behind the roofline, and the rule that stored HBM
traffic is reported only for the kernel sources it was measured on."""

import json
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.skipif(torch.cuda.is_available(), reason="a GPU is present: bench.py would run")
def test_no_gpu_is_refused():
    r = _run("--steps", "1")
    assert r.returncode == 2
    assert "needs a GPU" in r.stderr and r.stdout == ""


def test_gathered_bytes_per_row():
    # 2048 rows x top-k 1024 x 2 KV heads x K and V rows of 256 int8 codes
    # plus a 4-B scale each
    assert 2048 * bench.gathered_bytes_per_row("int8", 1024, 2, 256) == 2_181_038_080
    assert bench.gathered_bytes_per_row("int8_inline", 1, 1, 256) == 2 * 260
    assert bench.gathered_bytes_per_row("e4m3", 1, 1, 128) == 2 * 128
    assert bench.gathered_bytes_per_row("bf16", 1, 1, 256) == 2 * 512
    # NVFP4: 128 code bytes and 16 E4M3 block scales per 256-element row
    assert bench.gathered_bytes_per_row("nvfp4", 1, 1, 256) == 2 * (128 + 16)


def test_traffic_reported_only_for_the_measured_sources(monkeypatch):
    path = os.path.join(bench.PROFILES, "traffic.json")
    rec = json.load(open(path))
    key, entry = next(iter(rec.items()))
    kernel, workload = key.split("|")
    monkeypatch.setattr(bench, "source_sha", lambda: entry["source_sha"])
    assert bench.traffic_from_profile(kernel, workload) == entry["hbm_bytes_per_launch"]
    assert bench.traffic_from_profile(kernel, "no-such-workload") is None
    monkeypatch.setattr(bench, "source_sha", lambda: "0" * 16)
    assert bench.traffic_from_profile(kernel, workload) is None


def test_source_sha_covers_the_attention_sources():
    a = bench.source_sha()
    assert len(a) == 16 and a == bench.source_sha()
    assert "attn.hip" in bench.ATTN_SOURCES


def test_bench_lines_use_only_assigned_names():
    """Every name a bench_* function returns is assigned on every path
    (at its top level, or in a with-block, which always runs) -- a config's
    JSON line must not depend on a branch such as the CPU-baseline one."""
    import ast
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    bad = []
    for fn in (n for n in tree.body if isinstance(n, ast.FunctionDef) and n.name.startswith("bench_")):
        sure, maybe = {a.arg for a in fn.args.args}, set()
        for st in fn.body:
            blocks = st.body if isinstance(st, ast.With) else [st]
            for b in blocks:
                target = maybe if isinstance(b, (ast.If, ast.For, ast.While, ast.Try)) else sure
                for n in ast.walk(b):
                    if isinstance(n, ast.Name) and isinstance(n.ctx, ast.Store):
                        target.add(n.id)
        for st in fn.body:
            if isinstance(st, ast.Return) and st.value is not None:
                for n in ast.walk(st.value):
                    if isinstance(n, ast.Name) and n.id in maybe and n.id not in sure:
                        bad.append((fn.name, n.id))
    assert not bad, bad
