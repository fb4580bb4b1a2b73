"""GPU parity of wide batches (8 < m <= 32 activation rows sharing one
weight sweep, on the matrix cores with x staged per 256-column chunk):
every output within the oracle's bar, the argmax per row, and the
persistent step over all 197 shapes at m = 32."""
import numpy as np
import pytest

import gen
import oracle
from tests.gpu_helpers import assert_parity, cuda, gpu_batched, oracle_rows, say, to_dev  # noqa: F401
from tests.oracle_pins import make_blocks, rich_case
from tests.test_gpu_step import device_step, run_graph, step_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("m", [9, 16, 17, 24, 32])
@pytest.mark.parametrize("p,n", [(2048, 1024), (1024, 3072), (1000, 2048), (300, 256),
                                 (64, 8192), (129, 512)])
def test_wide_matches_oracle(cuda, m, p, n):
    """Chunk counts 1..32, tiles of 128 rows with ragged ends, partial column
    groups (m not a multiple of 8), planted -128 quants and special scales."""
    say(f"wide m={m} p={p} n={n}")
    w, _ = rich_case(p, n, seed=m * 7 + p)
    x = gen.activations(m, n, seed=m, index=p + 1)
    y = gpu_batched(w, x, cuda)
    ref, tol = oracle.matvec_batched(w, x)
    assert_parity(y, ref, tol, f"wide m={m} p={p} n={n}")


def test_wide_rows_independent(cuda):
    """Row i of a 32-row batch equals the same x row alone in a 9-row batch
    (padded with other rows) to the bar, and permuting x rows permutes y
    exactly (each row's arithmetic does not depend on the others)."""
    p, n = 700, 1024
    w = gen.weights(p, n, seed=3, index=3)
    x = gen.activations(32, n, seed=3, index=3)
    y = gpu_batched(w, x, cuda)
    perm = np.random.default_rng(3).permutation(32)
    yp = gpu_batched(w, x[perm], cuda)
    assert np.array_equal(yp, y[perm])
    y9 = gpu_batched(w, x[:9], cuda)
    ref, tol = oracle.matvec_batched(w, x[:9])
    assert_parity(y9, ref, tol, "9 rows")
    assert_parity(y[:9], ref, tol, "first 9 of 32")


@pytest.mark.parametrize("p,n", [(96, 1024), (40, 2048)])
def test_wide_pow2_scales_integer_x_exact(cuda, p, n):
    """Integers in [-4, 4] are exact in the high bf16 part and power-of-two
    scales keep every block and row sum on a grid: the results are exact."""
    m = 32
    rng = np.random.default_rng(p + n)
    quants = rng.integers(-128, 128, size=(p, n // 32, 32))
    expo = rng.integers(-3, 1, size=(p, n // 32))
    w = make_blocks(((15 + expo).astype(np.uint16) << 10), quants)
    x = rng.integers(-4, 5, size=(m, n)).astype(np.float32)
    y = gpu_batched(w, x, cuda)
    ref, _ = oracle.matvec_batched(w, x)
    assert np.array_equal(y.astype(np.float64), ref)


@pytest.mark.parametrize("m", [12, 32])
def test_wide_fused_argmax(cuda, m):
    """q8_matvec_argmax with m rows of a 40,000-row head (ties and NaN rules
    as the narrow paths): each index accepted against the oracle's logits and
    equal to the argmax of the GPU's own logits."""
    import torch
    import q8_block_quantized_amd as q8
    p, n = 40000, 1024
    w = gen.weights(p, n, seed=m, index=9)
    x = gen.activations(m, n, seed=m, index=9)
    wd = to_dev(w.reshape(-1), cuda)
    xd = to_dev(x, cuda)
    yd = torch.empty((m, p), dtype=torch.float32, device=cuda)
    idx = torch.full((m,), -7, dtype=torch.int32, device=cuda)
    q8.q8_matvec_argmax(wd, xd, idx, p, y=yd)
    idx2 = torch.full((m,), -7, dtype=torch.int32, device=cuda)
    q8.q8_matvec_argmax(wd, xd, idx2, p)
    torch.cuda.synchronize()
    y = yd.cpu().numpy()
    ref, tol = oracle.matvec_batched(w, x)
    assert_parity(y, ref, tol, f"wide head m={m}")
    for r in range(m):
        g = int(idx[r])
        assert oracle.argmax_accepted(g, ref[r], tol[r])
        assert g == oracle.argmax_f32(y[r]) == int(idx2[r])


def test_wide_argmax_standalone(cuda):
    """q8_argmax over 32 rows of f32 logits with planted ties and NaN."""
    import torch
    import q8_block_quantized_amd as q8
    m, p = 32, 5000
    rng = np.random.default_rng(5)
    lg = rng.standard_normal((m, p)).astype(np.float32)
    lg[3, 100] = lg[3, 4000] = 50.0   # tie: lower index
    lg[7, :] = np.nan                 # all NaN: -1
    lg[9, 10] = np.nan
    ld = to_dev(lg, cuda)
    idx = torch.full((m,), -7, dtype=torch.int32, device=cuda)
    q8.q8_argmax(ld, idx)
    torch.cuda.synchronize()
    for r in range(m):
        assert int(idx[r]) == oracle.argmax_f32(lg[r])
    assert int(idx[3]) == 100 and int(idx[7]) == -1


def test_wide_step_every_output(cuda):
    """m = 32 through all 197 shapes of a step in the persistent launch:
    every output of every matvec for all 32 x rows against the oracle, and
    the lm_head's 32 tokens (host tokens from the kernel)."""
    import torch
    m = 32
    say("wide step m=32: generating 197 matvecs")
    shapes, ws, xs = step_inputs(28, 151936, m, seed=5)
    descs = device_step(shapes, ws, xs, m, cuda)
    g, host = run_graph(descs, m, 1, cuda)
    assert g.info() == (1, 0)
    g.launch()
    torch.cuda.synchronize()
    say("wide step m=32: checking every output")
    for i, (name, n, p) in enumerate(shapes):
        y = descs[i]["y"].cpu().numpy()
        ref, tol = oracle_rows(ws[i], xs[i])
        assert_parity(y, ref, tol, f"m=32 {name}")
        if i == len(shapes) - 1:
            for r in range(m):
                assert oracle.argmax_accepted(int(host[r]), ref[r], tol[r])
                assert int(host[r]) == oracle.argmax_f32(y[r])
    g.close()


def test_wide_levels_and_chain(cuda):
    """A 2-layer step at m = 20 as a chain graph, a persistent graph and a
    levels graph: the same outputs bit for bit, within the bar."""
    import torch
    import q8_block_quantized_amd as q8
    m = 20
    shapes, ws, xs = step_inputs(2, 3000, m, seed=6)
    outs = []
    for mode in ("chain", "persistent", "levels"):
        descs = device_step(shapes, ws, xs, m, cuda)
        host = torch.zeros(m, dtype=torch.int32).pin_memory()
        if mode == "levels":
            lv = [0, 0, 0, 1, 2, 2, 3] * 2
            lv = [v + 4 * (i // 7) for i, v in enumerate(lv)] + [8]
            g = q8.StepGraph(descs, m, host_idx=host, levels=lv)
        else:
            g = q8.StepGraph(descs, m, host_idx=host,
                             mode=q8.Q8_GRAPH_CHAIN if mode == "chain" else q8.Q8_GRAPH_PERSISTENT)
        g.launch()
        torch.cuda.synchronize()
        outs.append(([d["y"].cpu().numpy() for d in descs], host.clone().numpy()))
        g.close()
    for ys, h in outs[1:]:
        for a, b in zip(outs[0][0], ys):
            assert np.array_equal(a, b)
        assert np.array_equal(outs[0][1], h)
    for i, (name, n, p) in enumerate(shapes):
        ref, tol = oracle.matvec_batched(ws[i], xs[i])
        assert_parity(outs[0][0][i], ref, tol, f"m=20 {name}")
