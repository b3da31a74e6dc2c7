"""Host-side logic of bench.py (no GPU): byte and flop accounting per workload form, the
parity summary on partial CPU-baseline samples, and the single-GPU guard."""

from __future__ import annotations

import os
import subprocess
import sys

import numpy as np

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_and_flops():
    w = workloads.custom(8, 32, [3, 5], seed=1)
    assert bench.algorithmic_bytes(w) == 8 * 64 + 2 * 12 + 8 * 32 * 2
    assert bench.algorithmic_flops(w) == 2.0 * 8 * 32 * 8
    workloads.to_fp8(w)
    assert bench.algorithmic_bytes(w) == 8 * 32 + 2 * 12 + 8 * 32 * 2
    p = workloads.custom_pairs([2, 3], 16, [1, 2], np.array([4, 5, 6]), seed=2)
    assert bench.algorithmic_bytes(p) == 15 * 32 + 3 * 16 + 5 * 16 * 2 + 2 * 8
    assert bench.algorithmic_flops(p) == 2.0 * 16 * (2 * 4 + 3 * 5 + 3 * 6)
    m = workloads.custom_multi([2, 3], 16, np.array([4, 5]), seed=3)
    assert bench.algorithmic_bytes(m) == 9 * 32 + 2 * (8 + 4 * 2) + 5 * 16 * 2
    assert bench.algorithmic_flops(m) == 2.0 * 16 * 5 * 9


def test_parity_summary_partial_samples():
    rng = np.random.default_rng(0)
    w = workloads.custom(4, 16, np.full(30, 5), seed=1)
    ref = rng.random(20) * 10
    gpu = np.concatenate([ref + 1e-6, np.zeros(10)])
    out = bench.parity_summary(gpu, ref, w)
    assert out["docs_checked"] == 20 and out["violations"] == 0 and out["top10_ok"] is None
    out = bench.parity_summary(ref + 1e-6, ref, workloads.custom(4, 16, np.full(20, 5), seed=1))
    assert out["top10_ok"] is True
    bad = ref.copy()
    bad[3] += 1.0
    assert bench.parity_summary(bad, ref, workloads.custom(4, 16, np.full(20, 5), seed=1))["violations"] == 1
    m = workloads.custom_multi([2, 2], 16, np.full(30, 5), seed=3)
    refm = rng.random((2, 17))
    gm = np.concatenate([refm, np.zeros((2, 13))], axis=1)
    out = bench.parity_summary(gm, refm, m)
    assert out["docs_checked"] == 17 and out["queries"] == 2 and out["violations"] == 0
    p = workloads.custom_pairs([2, 2], 16, [12, 12], np.full(24, 5), seed=4)
    refp = rng.random(14)
    out = bench.parity_summary(np.concatenate([refp, np.zeros(10)]), refp, p)
    assert out["violations"] == 0 and out["top10_queries_checked"] == 1


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_score_launches_mirror_the_pass_rule():
    m = workloads.custom_multi([32] * 8, 128, np.full(3, 5), seed=1)
    assert bench.score_launches(m) == 2          # 4 queries of 2 tiles per 8-tile pass
    m = workloads.custom_multi([32] * 8, 256, np.full(3, 5), seed=1)
    assert bench.score_launches(m) == 4          # d = 256: 4 tiles per pass
    m = workloads.custom_multi([200, 0, 5], 128, np.full(3, 5), seed=1)
    assert bench.score_launches(m) == 2          # a 13-tile query alone, then the 1-tile one
    assert bench.score_launches(workloads.custom(8, 32, [3], seed=1)) == 1


def test_percentiles():
    p = bench.percentiles(list(range(1, 102)))
    assert p["median"] == 51 and p["p10"] == 11 and p["p90"] == 91 and p["n"] == 101
    assert p["min"] == 1 and p["max"] == 101


def test_host_threads_respect_affinity_and_share(monkeypatch):
    n_aff = len(os.sched_getaffinity(0))
    monkeypatch.delenv("OMP_NUM_THREADS", raising=False)
    monkeypatch.setattr(bench, "cgroup_cpu_quota", lambda: None)
    assert bench.host_threads() == n_aff
    monkeypatch.setenv("OMP_NUM_THREADS", "1")
    assert bench.host_threads() == 1
    monkeypatch.delenv("OMP_NUM_THREADS")
    monkeypatch.setattr(bench, "cgroup_cpu_quota", lambda: 2.5)
    assert bench.host_threads() == min(n_aff, 2)
    info = bench.cpu_info()
    assert info["affinity_cpus"] == n_aff and isinstance(info["model_name"], str)


def test_fp8_quality_against_the_fp16_oracle():
    """The quality report on a small workload, with the FP8 oracle's scores standing in
    for the GPU's: quantised scores stay near the fp16 ones, the report's rank and
    overlap figures are consistent, and the unquantised scores themselves score perfectly."""
    import oracle

    w = workloads.custom(32, 128, np.random.default_rng(3).integers(16, 200, size=400), seed=3)
    workloads.to_fp8(w, keep_x=True)
    ref16 = oracle.maxsim(w.dtype, w.Q, w.X, w.offsets, w.lengths, d=w.d)
    q8 = oracle.maxsim_fp8(w.dtype, w.Q, w.X8, w.offsets, w.lengths, w.doc_scale, d=w.d)
    out = bench.fp8_quality(q8, w)
    assert out["docs"] == 400
    assert 0 < out["max_scaled_err"] < 0.05
    assert 0 <= out["top10_overlap"] <= 10 and out["top100_overlap"] <= 100
    assert out["spearman"] > 0.9
    same = bench.fp8_quality(ref16, w)
    assert same["max_scaled_err"] == 0.0 and same["top10_overlap"] == 10
    assert same["top10_max_rank_displacement"] == 0 and abs(same["spearman"] - 1.0) < 1e-12
