"""Host-side logic of bench.py, without a GPU: the shapes and algorithmic
bytes of the 197-matvec step (inferno.rs, "One command buffer": 7
projections per layer for 28 layers, then the lm_head with its argmax), and
the refusal of more than one GPU."""
import os
import subprocess
import sys

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
