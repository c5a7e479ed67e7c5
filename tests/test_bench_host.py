"""The bench's own arithmetic on the CPU: the algorithmic-byte formulas the
reported GB/s divide by (pinned to hand counts), the HBM counter summary it
reads, and the one-GPU refusal."""
import json
import os
import subprocess
import sys
import types

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from paged_kv_cache_43_amd import inputs  # noqa: E402


def _w(n, hq, hkv, d, es, block=16):
    return types.SimpleNamespace(n=n, hq=hq, hkv=hkv, d=d, es=es, block=block)


def test_attention_bytes_by_hand():
    # two sequences of 1 and 17 tokens, 2 query heads on 1 kv head, d 16, 2-byte elements:
    # K+V 18 tokens * 1 head * 16 dims * 2 (K, V) * 2 B = 1152; q and out 2 seqs * 2 heads * 16 * (2 + 2) = 256;
    # table entries 1 + 2 pages * 4 B = 12; lengths 2 * 4 = 8
    assert bench.alg_bytes_attention([1, 17], _w(2, 2, 1, 16, 2), 2) == 1152 + 256 + 12 + 8
    # fp32 out: q 2 B + out 4 B per element
    assert bench.alg_bytes_attention([1, 17], _w(2, 2, 1, 16, 2), 4) == 1152 + 2 * 2 * 16 * 6 + 12 + 8
    # 8-token pages: 1 + 3 table entries
    assert bench.alg_bytes_attention([1, 17], _w(2, 2, 1, 16, 2, block=8), 2) == 1152 + 256 + 16 + 8


def test_workload_per_token_bytes():
    # 13B-style: 40 heads * 128 dims * 2 (K, V) * 2 B = 20480 B per context token
    w = inputs.Workload("13b", frames="shuffled")
    one = bench.alg_bytes_attention(w.ctx, w, w.es)
    two = bench.alg_bytes_attention(w.ctx + 1, w, w.es)
    extra_pages = int(((w.ctx + 16) // 16 - (w.ctx + 15) // 16).sum())
    assert two - one == w.n * 20480 + 4 * extra_pages
    # GQA: 2 kv heads * 64 dims * 2 * 2 B = 512 B per context token
    g = inputs.Workload("gqa", frames="shuffled")
    assert bench.alg_bytes_attention(g.ctx + 1, g, g.es) - bench.alg_bytes_attention(g.ctx, g, g.es) == \
        g.n * 512 + 4 * int(((g.ctx + 16) // 16 - (g.ctx + 15) // 16).sum())


def test_scatter_bytes_by_hand():
    w = inputs.Workload("13b", frames="shuffled")
    # read k and v, write both: 64 seqs * 40 heads * 128 * 2 (K, V) * 2 B * 2; plus tok_seq, tok_pos, table entry
    assert bench.alg_bytes_scatter(w) == 64 * 40 * 128 * 2 * 2 * 2 + 64 * 12 == 2622208


def test_traffic_summary_is_read_only_for_its_source_hash(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "hbm_traffic.txt").write_text(
        "# comment\nsource_hash: abc123\n13b: 1500 1400\ngqa: 300\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abc123")
    assert bench.measured_traffic("13b") == (1500, 1400)
    assert bench.measured_traffic("gqa") == (300, None)
    assert bench.measured_traffic("mixed") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "other")
    assert bench.measured_traffic("13b") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], stdout=subprocess.PIPE,
                       stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _fake_workload(name):
    w = inputs.Workload(name, frames="shuffled")
    w.drop_values = lambda: None
    return w


def _fake_run(name, frames):
    w = _fake_workload(name)
    attention = {"what": "x" * 150, "launches": 50, "median_us": 250.0, "mean_us": 251.0, "sd_us": 1.0,
                 "min_us": 249.0, "kv_GBps": 6000.0, "pct_hbm_peak": 75.0, "seqs_per_ms": 250.0}
    scatter = {"what": "y" * 150, "launches": 50, "median_us": 5.5, "min_us": 5.0, "alg_bytes": 1, "GBps": 1.0}
    return dict(w=w, name=name, frames=frames, ms_step=0.25, ms_step_wall=0.26, ms_step_events=0.25,
                value=6100.0, seqs_per_ms=w.n / 0.25, part_avg_us=245.0, part_med_us=244.0, part_min_us=240.0,
                part_sd_us=2.0, attn_bytes=1.5e9, achieved=6400.0, split=0, waves=2048, mfma=False,
                whole=False, kernel_seqs_per_ms=1.0, attention=attention, scatter=scatter)


def _fake_cpu(name, budget):
    one = {"value": 1.1, "cores": 1, "seqs_per_ms": 0.05, "seconds": 12.0, "sample": "z" * 200}
    return {"value": 15.0, "unit": "GB/s", "cores": 16, "kind": "oracle", "seqs_per_ms": 0.67,
            "seconds": 24.0, "sample": "s" * 300, "sample_short": "13b layer 0, 800 sequence-attentions",
            "one_core": one, "host": {"cpu_model": "m" * 60, "os_cpu_count": 256, "affinity_cpus": 16}}


REQUIRED = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "dtype", "config",
            "pct_hbm_peak", "seqs_per_ms", "roofline", "cpu_baseline", "higher_is_better", "scaling",
            "vs_baseline", "data")


def test_headline_is_compact_and_printed_last(monkeypatch, capsys):
    """Every printed line stays under 4 KB and the last one is the headline
    with the keys a reader of a short stdout tail needs (the GPU legs are
    replaced by fixtures; only the printing is under test)."""
    import torch
    monkeypatch.setattr(torch.cuda, "is_available", lambda: True)
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a, **k: None)
    monkeypatch.setattr(bench, "run_gpu", lambda args, name, frames, *a, **k: _fake_run(name, frames))
    monkeypatch.setattr(bench, "run_twin", lambda name, frames, reps: {"paged_us": 1.0, "what": "t" * 100})
    monkeypatch.setattr(bench, "run_cow", lambda *a: {"shared_pages": 1})
    monkeypatch.setattr(bench, "run_swap", lambda *a: {"out_ms": 6.4})
    monkeypatch.setattr(bench, "run_fused", lambda names, steps: {n: {"speedup": 1.0} for n in names})
    monkeypatch.setattr(bench, "run_block_sweep", lambda names, blocks, reps: {
        n: {str(b): {"partition_us": 1.0, "kernel": "valu"} for b in blocks} for n in names})
    monkeypatch.setattr(bench, "cpu_baseline", _fake_cpu)
    monkeypatch.setattr(bench, "measured_traffic", lambda config: (1540000000, 1528000000))
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    bench.main()
    lines = [l for l in capsys.readouterr().out.splitlines() if l.strip()]
    assert len(lines) > 10
    parsed = [json.loads(l) for l in lines]
    assert all(len(l.encode()) < 4096 for l in lines)
    head = parsed[-1]
    for k in REQUIRED:
        assert k in head, k
    assert "leg" not in head and all("leg" in p for p in parsed[:-1])
    assert head["config"]["workload"].startswith("13B-style")
    assert head["n_gpus"] == 1 and head["unit"] == "GB/s" and head["dtype"] == "f16"
    for k in ("frac", "traffic", "traffic_over_alg", "avg_launch_us", "alg_bytes_per_launch", "bound", "peak"):
        assert k in head["roofline"], k
    assert head["roofline"]["traffic"] == 1540000000
    for k in ("value", "unit", "cores", "kind", "sample"):
        assert k in head["cpu_baseline"], k
    assert len(json.dumps(head)) < 4000
    # every other workload and frame order reported on a line of its own
    names = {p["name"] for p in parsed if p.get("leg") == "workload"}
    assert {"13b_shuffled", "13b_ordered", "gqa_shuffled", "gqa_ordered", "gqa_32k_ordered"} <= names
