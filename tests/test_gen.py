"""The seeded input generator (CPU only): rounding, determinism, slicing and
the workload distributions."""
import numpy as np

import gen


def test_f16_rne_matches_numpy():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 5, 20000),
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6,
                  2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26,
                  2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1.0 + 2.0 ** -11,
                  1.0 + 3 * 2.0 ** -11, 1e-30, np.inf, -np.inf]),
    ])
    got = np.array([gen.f16_rne(v) for v in vals], dtype=np.uint16)
    with np.errstate(over="ignore"):
        want = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_weights_deterministic_and_sliceable():
    w1 = gen.weights(64, 1024, seed=0, index=3)
    w2 = gen.weights(64, 1024, seed=0, index=3)
    assert np.array_equal(w1, w2)
    assert not np.array_equal(w1, gen.weights(64, 1024, seed=0, index=4))
    key = gen.stream_key(0, gen.ROLE_W, 3)
    part = gen.blocks(key, 100, 900)
    assert np.array_equal(part.ravel(), w1.reshape(-1, 34)[100:1000].ravel())


def test_activations_deterministic_and_sliceable():
    x = gen.activations(2, 3000, seed=5, index=9)
    assert np.array_equal(x, gen.activations(2, 3000, seed=5, index=9))
    assert not np.array_equal(x[0], x[1])
    key = gen.stream_key(5, gen.ROLE_X, 9, 1)
    assert np.array_equal(gen.normals(key, 1234, 500), x[1, 1234:1734])


def test_distributions():
    w = gen.weights(2048, 1024, seed=0, index=0)
    blk = w.reshape(-1, 34)
    q = blk[:, 2:].view(np.int8).astype(np.int64).ravel()
    assert q.min() == -127 and q.max() == 127
    hist = np.bincount(q + 127, minlength=255)
    assert hist.min() > 0.9 * q.size / 255 and hist.max() < 1.1 * q.size / 255
    scale = np.ascontiguousarray(blk[:, 0:2]).view("<f2")[:, 0].astype(np.float64)
    assert np.all(scale >= 0)
    # |N(0, 0.02)| / 127 has mean 0.02 * sqrt(2/pi) / 127
    assert abs(scale.mean() / (0.02 * np.sqrt(2 / np.pi) / 127) - 1) < 0.02
    # about 30 % of the scales are binary16 subnormals
    sub = np.mean(scale < 2.0 ** -14)
    assert 0.25 < sub < 0.35
    x = gen.activations(1, 200000, seed=0, index=0)[0].astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01


def test_step_shapes():
    s = gen.step_shapes()
    assert len(s) == 197
    assert s[-1] == ("lm_head", 1024, 151936)
    blocks = sum(p * n // 32 for _, n, p in s)
    assert blocks == 18_624_512
    assert blocks * 34 == 633_233_408
