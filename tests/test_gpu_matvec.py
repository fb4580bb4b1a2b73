"""GPU parity of q8_matvec and q8_matvec_batched against the oracle.

Every output is compared with the oracle's exact value under the bar
|y - y_ref| <= 1e-4 * sum|scale*q*x| + 1e-6; where the arithmetic makes the
GPU result exact (one-hot x, power-of-two scales with integer x, scaling x by
a power of two) the comparison is bit for bit."""
import numpy as np
import pytest

import gen
import oracle
from tests import pagegen
from tests.gpu_helpers import (assert_parity, cuda, gpu_batched, gpu_matvec,  # noqa: F401
                               say, to_dev)
from tests.oracle_pins import make_blocks, rich_case

pytestmark = pytest.mark.gpu

SHAPES = [  # (p, n): tiny, ragged, the model's widths, odd widths, max width
    (1, 32), (3, 96), (50, 96), (7, 128), (2, 1024), (129, 1024), (4097, 1024),
    (1, 2048), (33, 2048), (65, 3072), (257, 3072), (100, 4096), (17, 1056),
    (1000, 64), (3, 65536),
]


@pytest.mark.parametrize("p,n", SHAPES)
def test_matvec_matches_oracle(cuda, p, n):
    say(f"matvec p={p} n={n}")
    w, x = rich_case(p, n, seed=p * 7 + n)
    y = gpu_matvec(w, x, cuda)
    ref, tol = oracle.matvec(w, x)
    assert_parity(y, ref, tol, f"p={p} n={n}")


def test_page_matvec_case(cuda):
    """The page's kernel test inputs; also its own 5e-4 absolute bound."""
    w = pagegen.fabricated_q8(50, 96, 7)
    x = pagegen.lcg_f32(42, 96)
    y = gpu_matvec(w, x, cuda)
    ref, tol = oracle.matvec(w, x)
    assert_parity(y, ref, tol, "page case")
    assert np.max(np.abs(y - ref)) < 5e-4


def test_single_matvec_workload(cuda):
    """1024 -> 2048, seeded weights and x, every output."""
    w = gen.weights(2048, 1024, seed=0, index=0)
    x = gen.activations(1, 1024, seed=0, index=0)[0]
    y = gpu_matvec(w, x, cuda)
    ref, tol = oracle.matvec(w, x)
    assert_parity(y, ref, tol, "1024->2048")


def test_layer_workload(cuda):
    """One layer's seven projections, x reseeded per projection."""
    for i, (name, n, p) in enumerate(gen.LAYER_SHAPES):
        say(f"layer {name} {n}->{p}")
        w = gen.weights(p, n, seed=0, index=i)
        x = gen.activations(1, n, seed=0, index=i)[0]
        y = gpu_matvec(w, x, cuda)
        ref, tol = oracle.matvec(w, x)
        assert_parity(y, ref, tol, name)


def test_empty_shapes(cuda):
    import torch
    import q8_block_quantized_amd as q8
    x = torch.ones(64, dtype=torch.float32, device=cuda)
    y = torch.empty(0, dtype=torch.float32, device=cuda)
    w = torch.empty(0, dtype=torch.uint8, device=cuda)
    q8.q8_matvec(w, x, y)  # p == 0: nothing to do
    x0 = torch.empty(0, dtype=torch.float32, device=cuda)
    y5 = torch.full((5,), 7.0, dtype=torch.float32, device=cuda)
    q8.q8_matvec(w, x0, y5)  # n == 0: every output is the empty sum
    torch.cuda.synchronize()
    assert torch.all(y5 == 0).item()


@pytest.mark.parametrize("p,n", [(64, 1024), (5, 96), (9, 2048), (4, 3072)])
def test_one_hot_is_exact(cuda, p, n):
    w, _ = rich_case(p, n, seed=5)
    blk = w.reshape(p, n // 32, 34)
    scale = np.ascontiguousarray(blk[:, :, 0:2]).view("<f2")[..., 0].astype(np.float32)
    q = np.ascontiguousarray(blk[:, :, 2:]).view(np.int8).astype(np.float32)
    for k in [0, 1, 33, n - 1]:
        x = np.zeros(n, dtype=np.float32)
        x[k] = 1.0
        y = gpu_matvec(w, x, cuda)
        want = scale[:, k // 32] * q[:, k // 32, k % 32]
        assert np.array_equal(y, want), k


@pytest.mark.parametrize("p,n", [(40, 1024), (11, 160), (6, 3072)])
def test_pow2_scales_integer_x_exact(cuda, p, n):
    # |partial sums| < 2^21 on a 2^-3 grid: exact in f32 in any order
    rng = np.random.default_rng(p + n)
    quants = rng.integers(-128, 128, size=(p, n // 32, 32))
    expo = rng.integers(-3, 1, size=(p, n // 32))
    w = make_blocks(((15 + expo).astype(np.uint16) << 10), quants)
    x = rng.integers(-4, 5, size=n).astype(np.float32)
    y = gpu_matvec(w, x, cuda)
    ref, _ = oracle.matvec(w, x)
    assert np.array_equal(y.astype(np.float64), ref)


def test_homogeneity_and_determinism(cuda):
    w, x = rich_case(300, 1024, seed=9)
    y1 = gpu_matvec(w, x, cuda)
    y2 = gpu_matvec(w, x, cuda)
    assert np.array_equal(y1, y2)
    y4 = gpu_matvec(w, x * np.float32(4.0), cuda)
    assert np.array_equal(y4, y1 * np.float32(4.0))
    yn = gpu_matvec(w, -x, cuda)
    assert np.array_equal(yn, -y1)


def test_subnormal_scales(cuda):
    """Every scale a binary16 subnormal: a flush to zero would show at once."""
    p, n = 64, 1024
    rng = np.random.default_rng(3)
    quants = rng.integers(-127, 128, size=(p, n // 32, 32))
    sb = rng.integers(1, 0x400, size=(p, n // 32)).astype(np.uint16)
    w = make_blocks(sb, quants)
    x = gen.activations(1, n, seed=3, index=3)[0]
    y = gpu_matvec(w, x, cuda)
    ref, tol = oracle.matvec(w, x)
    assert_parity(y, ref, tol, "subnormal scales")
    assert np.all(np.abs(y) > 0)


def test_nan_scale_propagates(cuda):
    p, n = 8, 1024
    w, x = rich_case(p, n, seed=4)
    blk = w.reshape(p, n // 32, 34)
    blk[3, 5, 0], blk[3, 5, 1] = 0x00, 0x7E  # NaN scale in row 3
    y = gpu_matvec(w, x, cuda)
    ref, tol = oracle.matvec(w, x)
    assert np.isnan(y[3]) and np.isnan(ref[3])
    assert_parity(y, ref, tol, "nan scale")


@pytest.mark.parametrize("m", [2, 5, 8])
@pytest.mark.parametrize("p,n", [(50, 96), (129, 1024), (65, 3072), (31, 2048)])
def test_batched_matches_oracle(cuda, m, p, n):
    say(f"batched m={m} p={p} n={n}")
    w, _ = rich_case(p, n, seed=m * 100 + p)
    x = gen.activations(m, n, seed=m, index=p)
    y = gpu_batched(w, x, cuda)
    ref, tol = oracle.matvec_batched(w, x)
    assert_parity(y, ref, tol, f"m={m} p={p} n={n}")


def test_batched_m1_equals_matvec(cuda):
    w, x = rich_case(77, 1056, seed=1)
    yb = gpu_batched(w, x[None, :], cuda)[0]
    y = gpu_matvec(w, x, cuda)
    assert np.array_equal(yb, y)


# ---- batched (1 < m <= 8) -----------------------------------------------------
# Widths 1024, 2048 and 3072 take the matrix-core path (x split into two
# bf16 parts); other widths the direct or generic paths.

@pytest.mark.parametrize("m", [2, 7, 8])
@pytest.mark.parametrize("p,n", [(1000, 1024), (333, 2048), (170, 3072),
                                 (40, 4096), (21, 1056), (37, 256)])
def test_batched_tiles_and_paths(cuda, m, p, n):
    say(f"batched tiles m={m} p={p} n={n}")
    w, _ = rich_case(p, n, seed=m + p)
    x = gen.activations(m, n, seed=p, index=m)
    y = gpu_batched(w, x, cuda)
    ref, tol = oracle.matvec_batched(w, x)
    assert_parity(y, ref, tol, f"m={m} p={p} n={n}")


def test_batched_many_tiles(cuda):
    """Enough rows that each workgroup takes several 48-row tiles, ragged end."""
    m, p, n = 8, 30011, 1024
    w = gen.weights(p, n, seed=4, index=4)
    x = gen.activations(m, n, seed=4, index=4)
    y = gpu_batched(w, x, cuda)
    ref, tol = oracle.matvec_batched(w, x)
    assert_parity(y, ref, tol, "m=8 p=30011")


@pytest.mark.parametrize("p,n", [(40, 1024), (17, 2048), (6, 3072), (11, 160)])
def test_batched_pow2_scales_integer_x_exact(cuda, p, n):
    # integers in [-4, 4] are exact in the high bf16 part, so the products,
    # block sums and the 2^-3-grid row sums are all exact
    m = 8
    rng = np.random.default_rng(p * n)
    quants = rng.integers(-128, 128, size=(p, n // 32, 32))
    expo = rng.integers(-3, 1, size=(p, n // 32))
    w = make_blocks(((15 + expo).astype(np.uint16) << 10), quants)
    x = rng.integers(-4, 5, size=(m, n)).astype(np.float32)
    y = gpu_batched(w, x, cuda)
    ref, _ = oracle.matvec_batched(w, x)
    assert np.array_equal(y.astype(np.float64), ref)


@pytest.mark.parametrize("n", [1024, 2048, 3072])
def test_batched_one_hot_is_exact(cuda, n):
    p, m = 48, 8
    w, _ = rich_case(p, n, seed=n)
    blk = w.reshape(p, n // 32, 34)
    scale = np.ascontiguousarray(blk[:, :, 0:2]).view("<f2")[..., 0].astype(np.float32)
    q = np.ascontiguousarray(blk[:, :, 2:]).view(np.int8).astype(np.float32)
    ks = [0, 1, 33, 100, n // 2 + 7, n - 33, n - 2, n - 1]
    x = np.zeros((m, n), dtype=np.float32)
    for r, k in enumerate(ks):
        x[r, k] = 1.0
    y = gpu_batched(w, x, cuda)
    for r, k in enumerate(ks):
        assert np.array_equal(y[r], scale[:, k // 32] * q[:, k // 32, k % 32]), (r, k)


@pytest.mark.parametrize("n", [1024, 3072])
def test_batched_rows_independent_and_homogeneous(cuda, n):
    """Each output row depends on its own x row only (bit for bit), and
    scaling x by 4 scales y exactly.  Negating x negates y to the oracle's
    bound only: the matrix cores' block sums are not rounded symmetrically
    about zero, so -x may differ from x in the last bits."""
    p = 200
    w, _ = rich_case(p, n, seed=11)
    x = gen.activations(8, n, seed=11, index=n)
    y8 = gpu_batched(w, x, cuda)
    y3 = gpu_batched(w, x[[5, 0, 2]], cuda)
    assert np.array_equal(y3, y8[[5, 0, 2]])
    y4 = gpu_batched(w, x * np.float32(4.0), cuda)
    assert np.array_equal(y4, y8 * np.float32(4.0))
    yn = gpu_batched(w, -x, cuda)
    ref, tol = oracle.matvec_batched(w, -x)
    assert_parity(yn, ref, tol, "-x")
    assert np.all(np.abs(yn + y8) <= tol)


def test_batched_wide_dynamic_range(cuda):
    """x spread over twelve decades: the two bf16 parts still carry each
    value to the f32 bound."""
    m, p, n = 8, 96, 2048
    w, _ = rich_case(p, n, seed=12)
    rng = np.random.default_rng(12)
    mag = 10.0 ** rng.uniform(-6, 6, size=(m, n))
    x = (mag * rng.choice([-1.0, 1.0], size=(m, n))).astype(np.float32)
    y = gpu_batched(w, x, cuda)
    ref, tol = oracle.matvec_batched(w, x)
    assert_parity(y, ref, tol, "wide range")


def test_batched_special_scales(cuda):
    """Subnormal scales everywhere, one NaN scale in row 3 of x row 0's
    matrix: NaN reaches every x row of output row 3 only."""
    m, p, n = 4, 64, 1024
    rng = np.random.default_rng(13)
    quants = rng.integers(-127, 128, size=(p, n // 32, 32))
    sb = rng.integers(1, 0x400, size=(p, n // 32)).astype(np.uint16)
    w = make_blocks(sb, quants)
    x = gen.activations(m, n, seed=13, index=13)
    y = gpu_batched(w, x, cuda)
    ref, tol = oracle.matvec_batched(w, x)
    assert_parity(y, ref, tol, "subnormal scales")
    assert np.all(np.abs(y) > 0)
    blk = w.reshape(p, n // 32, 34)
    blk[3, 7, 0], blk[3, 7, 1] = 0x00, 0x7E
    y = gpu_batched(w, x, cuda)
    ref, tol = oracle.matvec_batched(w, x)
    assert np.all(np.isnan(y[:, 3])) and np.all(np.isnan(ref[:, 3]))
    assert_parity(y, ref, tol, "nan scale")
