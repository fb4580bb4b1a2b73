"""Host-side logic of bench.py, without a GPU: the shapes and algorithmic
bytes of the 197-matvec step (inferno.rs, "One command buffer": 7
projections per layer for 28 layers, then the lm_head with its argmax), and
the refusal of more than one GPU."""
import os
import subprocess
import sys

import numpy as np

import bench
import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# q, k, v, o, gate, up, down of one Qwen3-0.6B layer as (n, p): x width, rows
LAYER = [(1024, 2048), (1024, 1024), (1024, 1024), (2048, 1024), (1024, 3072),
         (1024, 3072), (3072, 1024)]


def test_step_shapes():
    shapes = gen.step_shapes()
    assert len(shapes) == 197
    assert [(n, p) for _, n, p in shapes[:-1]] == LAYER * 28
    assert shapes[-1][1:] == (1024, 151936)


def test_step_algorithmic_bytes():
    """Weight blocks (p rows of n/32 blocks of 34 bytes), each x once, every
    y but the lm_head's (its argmax is fused: one int32 instead)."""
    weights = 28 * sum(p * (n // 32) * 34 for n, p in LAYER) + 151936 * (1024 // 32) * 34
    xs = 28 * sum(4 * n for n, _ in LAYER) + 4 * 1024
    ys = 28 * sum(4 * p for _, p in LAYER)
    assert (weights, xs, ys) == (633_233_408, 1_150_976, 1_376_256)
    shapes = gen.step_shapes()
    last = len(shapes) - 1
    total = sum(bench.alg_bytes(n, p, 1, i < last, i == last)
                for i, (_, n, p) in enumerate(shapes))
    assert total == weights + xs + ys + 4 == 635_760_644
    # batched rows scale x and y, not the weights
    m8 = sum(bench.alg_bytes(n, p, 8, i < last, i == last)
             for i, (_, n, p) in enumerate(shapes))
    assert m8 == weights + 8 * (xs + ys + 4)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_trace_summary(tmp_path):
    """Durations and gaps from a hand-made rocprofv3 kernel trace: two graph
    launches of three nodes (1 us kernels, 0.5 us apart inside a launch, 4
    us between launches), one foreign kernel filtered out."""
    rows = ["Kind,Kernel_Name,Start_Timestamp,End_Timestamp"]
    t = 10_000
    for g in range(2):
        for k in range(3):
            rows.append(f"KERNEL_DISPATCH,q8::step_kernel,{t},{t + 1000}")
            t += 1500
        t += 3500
    rows.append(f"KERNEL_DISPATCH,at::fill,{t},{t + 700}")
    path = tmp_path / "kt.csv"
    path.write_text("\n".join(rows) + "\n")
    out = bench.trace_summary(str(path), "q8", group=3)
    assert out["dispatches"] == 6
    assert out["duration_us"]["q8::step_kernel"]["median"] == 1.0
    assert out["gap_in_graph_us"]["median"] == 0.5 and out["gap_in_graph_us"]["count"] == 4
    assert out["gap_between_graphs_us"]["median"] == 4.0
    assert out["graph_span_us"]["median"] == 4.0 and out["graph_busy_us"]["median"] == 3.0
    skipped = bench.trace_summary(str(path), "q8", group=3, skip_groups=1)
    assert skipped["dispatches"] == 3 and skipped["gap_between_graphs_us"] is None
    flat = bench.trace_summary(str(path), "", group=0)
    assert flat["dispatches"] == 7 and flat["gap_us"]["count"] == 6


def test_cpu_configs_use_the_gpu_byte_counts(monkeypatch):
    """The CPU leg's rates divide the same algorithmic bytes as the GPU
    figures: config 4 is the whole step's 635,760,644 bytes, config 5 the
    m = 8 step's (its single-thread run on layer 0 + lm_head); timing is
    replaced by a fixed 1 s so only the bytes are checked."""
    import oracle

    class Fake:
        def matvec_mt(self, w, x, th):
            return None, None, th

        def matvec_batched(self, w, x):
            return None, None

    monkeypatch.setattr(oracle, "get", lambda: Fake())
    monkeypatch.setattr(bench, "_median_time", lambda fn, runs: (fn(), 1.0)[1])
    shapes = gen.step_shapes()
    m_host = {"w": [None] * len(shapes), "x": [np.zeros((1, n), np.float32) for _, n, _ in shapes]}
    m8 = [np.zeros((8, n), np.float32) for _, n, _ in shapes]
    out = bench.cpu_configs(m_host, m8, 4, runs=1)
    assert out["4_full_step_m1"]["all_cores_GBps"] == round(635_760_644 / 1e9, 3)
    assert out["3_lm_head_argmax"]["single_thread_GBps"] == round(
        bench.alg_bytes(1024, 151936, 1, False, True) / 1e9, 3)
    assert out["1_matvec_1024x2048"]["all_cores_GBps"] == round(
        bench.alg_bytes(1024, 2048, 1, True, False) / 1e9, 3)
    last = len(shapes) - 1
    m8_step = sum(bench.alg_bytes(n, p, 8, i < last, i == last)
                  for i, (_, n, p) in enumerate(shapes))
    assert out["5_full_step_m8"]["all_cores_GBps"] == round(m8_step / 1e9, 3)
    assert "single_thread_sample" in out["5_full_step_m8"]
