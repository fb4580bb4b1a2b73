"""GPU parity of the int8-activation variant (q8_matvec_i8x,
q8_matvec_argmax_i8x, Q8_GRAPH_PERSISTENT_I8X) against the oracle's
quantised product.  Both sides quantise x by the same binary32 rule, so the
GPU is held to the f32 bar against the oracle's quantised result; separately
it must stay within the quantisation bound of the exact-x result."""
import numpy as np
import pytest

import gen
import oracle
import q8_block_quantized_amd as q8
from tests.gpu_helpers import assert_parity, cuda, say, to_dev  # noqa: F401
from tests.oracle_pins import make_blocks, rich_case

pytestmark = pytest.mark.gpu


def gpu_i8x(w, x, device):
    import torch
    x2 = np.atleast_2d(x).astype(np.float32)
    m, p = x2.shape[0], w.shape[0]
    wd = to_dev(w.reshape(-1), device)
    xd = to_dev(x2, device)
    yd = torch.full((m, p), float("nan"), dtype=torch.float32, device=device)
    q8.q8_matvec_i8x(wd, xd, yd)
    torch.cuda.synchronize()
    return yd.cpu().numpy()


def quant_bound(w, x):
    """sum_b |scale| * d_b / 2 * sum_j |q|: what quantising x may change."""
    p = w.shape[0]
    n = x.size
    d, _ = oracle.quantize_x(x)
    blk = np.ascontiguousarray(w).reshape(p, n // 32, 34)
    scale = np.ascontiguousarray(blk[:, :, 0:2]).view("<f2")[..., 0].astype(np.float64)
    qabs = np.abs(np.ascontiguousarray(blk[:, :, 2:]).view(np.int8).astype(np.float64)).sum(axis=2)
    return (np.abs(scale) * (d.astype(np.float64) / 2)[None, :] * qabs).sum(axis=1)


@pytest.mark.parametrize("m", [1, 3, 8])
@pytest.mark.parametrize("p,n", [(1000, 1024), (333, 2048), (170, 3072),
                                 (7, 256), (64, 512)])
def test_i8x_matches_oracle(cuda, m, p, n):
    say(f"i8x m={m} p={p} n={n}")
    w, _ = rich_case(p, n, seed=p + n + m)
    x = gen.activations(m, n, seed=m, index=n)
    y = gpu_i8x(w, x, cuda)
    ref, tol = oracle.matvec_i8x(w, x)
    assert_parity(y, ref, tol, f"i8x m={m} p={p} n={n}")
    for i in range(m):
        exact, etol = oracle.matvec(w, x[i])
        assert np.all(np.abs(y[i] - exact) <= quant_bound(w, x[i]) + etol)


def test_i8x_lm_head_many_tiles(cuda):
    w = gen.weights(151936, 1024, seed=0, index=196)
    x = gen.activations(1, 1024, seed=0, index=196)
    y = gpu_i8x(w, x, cuda)
    ref, tol = oracle.matvec_i8x(w, x)
    assert_parity(y, ref, tol, "i8x lm_head")


def test_i8x_special_blocks(cuda):
    """A zero block adds nothing; a block of x holding a NaN (or an
    infinity) makes every output NaN, as in the oracle; subnormal scales."""
    p, n = 40, 1024
    rng = np.random.default_rng(8)
    quants = rng.integers(-127, 128, size=(p, n // 32, 32))
    sb = rng.integers(1, 0x400, size=(p, n // 32)).astype(np.uint16)
    w = make_blocks(sb, quants)
    x = gen.activations(2, n, seed=8, index=8)
    x[0, 64:96] = 0.0
    y = gpu_i8x(w, x, cuda)
    ref, tol = oracle.matvec_i8x(w, x)
    assert_parity(y, ref, tol, "zero block, subnormal scales")
    x[1, 300] = np.nan
    x[0, 900] = np.inf
    y = gpu_i8x(w, x, cuda)
    ref, tol = oracle.matvec_i8x(w, x)
    assert np.all(np.isnan(y)) and np.all(np.isnan(ref))


@pytest.mark.parametrize("m,n", [(3, 1024), (5, 3072), (8, 2048)])
def test_i8x_bad_block_stays_in_its_row(cuda, m, n):
    """A NaN (or infinity) block in one x row makes that row's outputs NaN
    and leaves every other row at the oracle's bar (each x row keeps its own
    steps and sums, also on the matrix-core tile); a zero block in another
    row adds nothing."""
    p = 70
    w, _ = rich_case(p, n, seed=n + m)
    x = gen.activations(m, n, seed=m, index=n + 1)
    bad = m // 2
    x[bad, 37] = np.nan if m % 2 else np.inf
    x[0, 0:32] = 0.0
    y = gpu_i8x(w, x, cuda)
    ref, tol = oracle.matvec_i8x(w, x)
    assert np.all(np.isnan(y[bad])) and np.all(np.isnan(ref[bad]))
    keep = [r for r in range(m) if r != bad]
    assert_parity(y[keep], ref[keep], tol[keep], f"rows beside the bad one, m={m} n={n}")


def test_i8x_exact_on_grid(cuda):
    """x already on its grid (power-of-two steps, one code 127 per block):
    quantising changes nothing and the result meets the f32 oracle's bar."""
    rng = np.random.default_rng(9)
    p, n = 77, 2048
    w, _ = rich_case(p, n, seed=9)
    codes = rng.integers(-127, 128, size=n)
    codes[::32] = 127
    x = (codes * np.repeat(2.0 ** rng.integers(-9, -2, size=n // 32), 32)).astype(np.float32)
    y = gpu_i8x(w, x, cuda)[0]
    ref, tol = oracle.matvec(w, x)
    assert_parity(y, ref, tol, "on grid")


def test_i8x_widths(cuda):
    """Widths other than multiples of 256 up to 3072 are refused before any
    GPU work; n = 0 writes zeros."""
    import torch
    for n in (96, 1056, 4096):
        w, _ = rich_case(4, n, seed=1)
        with pytest.raises(q8.Q8Error) as e:
            gpu_i8x(w, np.ones(n, dtype=np.float32), cuda)
        assert e.value.name == "q8_err_shape"
    x = torch.empty((1, 0), dtype=torch.float32, device=cuda)
    y = torch.full((1, 5), float("nan"), dtype=torch.float32, device=cuda)
    q8.q8_matvec_i8x(torch.empty(0, dtype=torch.uint8, device=cuda), x, y)
    torch.cuda.synchronize()
    assert torch.all(y == 0).item()


@pytest.mark.parametrize("m,p,n", [(1, 151936, 1024), (2, 4097, 1024), (5, 999, 3072)])
def test_i8x_fused_argmax(cuda, m, p, n):
    import torch
    w = gen.weights(p, n, seed=m, index=p) if p > 10000 else rich_case(p, n, seed=p)[0]
    x = gen.activations(m, n, seed=m, index=n)
    wd = to_dev(w.reshape(-1), cuda)
    xd = to_dev(x, cuda)
    idx = torch.full((m,), -5, dtype=torch.int32, device=cuda)
    y = torch.empty((m, p), dtype=torch.float32, device=cuda)
    q8.q8_matvec_argmax_i8x(wd, xd, idx, p, y=y)
    torch.cuda.synchronize()
    ref, tol = oracle.matvec_i8x(w, x)
    yh = y.cpu().numpy()
    assert_parity(yh, ref, tol, f"fused i8x m={m}")
    for r in range(m):
        g = int(idx[r])
        assert g == oracle.argmax_f32(yh[r])
        assert oracle.argmax_accepted(g, ref[r], tol[r])
    idx2 = torch.full((m,), -5, dtype=torch.int32, device=cuda)
    q8.q8_matvec_argmax_i8x(wd, xd, idx2, p)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)


def _step(layers, lm_p, m, seed, device):
    import torch
    shapes = [(f"L{l}.{name}", n, p) for l in range(layers)
              for name, n, p in gen.LAYER_SHAPES] + [("lm_head", 1024, lm_p)]
    ws, xs, descs = [], [], []
    for i, (_, n, p) in enumerate(shapes):
        ws.append(gen.weights(p, n, seed=seed, index=i))
        xs.append(gen.activations(m, n, seed=seed, index=i))
        last = i == len(shapes) - 1
        descs.append(dict(n=n, p=p, w=to_dev(ws[i].reshape(-1), device),
                          x=to_dev(xs[i], device),
                          y=torch.full((m, p), float("nan"), dtype=torch.float32,
                                       device=device),
                          idx=torch.full((m,), -7, dtype=torch.int32, device=device)
                          if last else None))
    return shapes, ws, xs, descs


@pytest.mark.parametrize("m", [1, 8])
def test_i8x_step_equals_standalone(cuda, m):
    """The int8-activation persistent step gives, bit for bit, what
    q8_matvec_i8x gives for each descriptor, through the graph and through
    the kernel launch, on three launches.  At m = 8 the step runs in column
    slices (a second node adds the o and down slices' partials): those two
    round as the slices' sum does, so they are held to the oracle's bar
    instead, and to their own first launch."""
    import torch
    shapes, ws, xs, descs = _step(2, 20000, m, 4, cuda)
    host = torch.full((m,), -5, dtype=torch.int32).pin_memory()
    g = q8.StepGraph(descs, m, host_idx=host, mode=q8.Q8_GRAPH_PERSISTENT_I8X, device=cuda)
    assert g.info() == ((1, 0) if m == 1 else (2, 0))
    want = []
    for d in descs:
        y = torch.empty_like(d["y"])
        q8.q8_matvec_i8x(d["w"], d["x"], y)
        want.append(y)
    torch.cuda.synchronize()
    first = None
    for k in range(3):
        for d in descs:
            d["y"].fill_(float("nan"))
        (g.launch if k != 1 else g.launch_kernel)()
        torch.cuda.synchronize()
        for i, (d, w_) in enumerate(zip(descs, want)):
            name, n, p = shapes[i]
            if m == 1 or n == 1024:
                assert torch.equal(d["y"], w_), name
            else:
                ref, tol = oracle.matvec_i8x(ws[i], xs[i])
                assert_parity(d["y"].cpu().numpy(), ref, tol, f"{name} launch {k}")
        outs = [d["y"].clone() for d in descs]
        if first is None:
            first = outs
        for a, b in zip(first, outs):
            assert torch.equal(a, b)
        yl = descs[-1]["y"].cpu().numpy()
        for r in range(m):
            assert int(host[r]) == oracle.argmax_f32(yl[r])
    g.close()


@pytest.mark.parametrize("m", [2, 3, 5, 7])
def test_i8x_sliced_batched_step(cuda, m):
    """The int8-activation persistent step in column slices (every width
    1024, 2048 or 3072): ragged wide matvecs, an odd m, an empty matvec and
    an argmax on a 1024-wide one; every output against the oracle's
    quantised product over three launches with the outputs poisoned in
    between, the kernel launch equal to the graph launch."""
    import torch
    shapes = [("a", 2048, 77), ("b", 1024, 100), ("c", 3072, 33), ("empty", 3072, 0),
              ("d", 2048, 1), ("e", 3072, 200), ("lm", 1024, 5000)]
    ws = [gen.weights(p, n, seed=13, index=i) for i, (_, n, p) in enumerate(shapes)]
    xs = [gen.activations(m, n, seed=13, index=i) for i, (_, n, p) in enumerate(shapes)]
    descs = []
    for i, (name, n, p) in enumerate(shapes):
        descs.append(dict(n=n, p=p, w=to_dev(ws[i].reshape(-1), cuda), x=to_dev(xs[i], cuda),
                          y=torch.full((m, p), float("nan"), dtype=torch.float32, device=cuda),
                          idx=torch.full((m,), -7, dtype=torch.int32, device=cuda)
                          if name == "lm" else None))
    host = torch.full((m,), -5, dtype=torch.int32).pin_memory()
    g = q8.StepGraph(descs, m, host_idx=host, mode=q8.Q8_GRAPH_PERSISTENT_I8X, device=cuda)
    assert g.info() == (2, 0)  # the sliced step, then the slices' sums
    refs = [oracle.matvec_i8x(ws[i], xs[i]) if p else None for i, (_, n, p) in enumerate(shapes)]
    first = None
    for rep in range(3):
        for d in descs:
            d["y"].fill_(float("nan"))
        host[:] = -9
        (g.launch if rep != 2 else g.launch_kernel)()
        torch.cuda.synchronize()
        for i, (name, n, p) in enumerate(shapes):
            if p:
                assert_parity(descs[i]["y"].cpu().numpy(), refs[i][0], refs[i][1],
                              f"m={m} {name} rep {rep}")
        ref, tol = refs[-1]
        for r in range(m):
            assert oracle.argmax_accepted(int(host[r]), ref[r], tol[r])
        outs = [d["y"].clone() for d in descs]
        if first is None:
            first = outs
        for a, b in zip(first, outs):
            assert torch.equal(a, b)
    g.close()


def test_i8x_full_step_against_oracle(cuda):
    """All 197 matvecs of a step with int8 activations, every output."""
    import torch
    shapes, ws, xs, descs = _step(28, 151936, 1, 0, cuda)
    host = torch.full((1,), -5, dtype=torch.int32).pin_memory()
    g = q8.StepGraph(descs, 1, host_idx=host, mode=q8.Q8_GRAPH_PERSISTENT_I8X, device=cuda)
    g.launch()
    torch.cuda.synchronize()
    for i, (name, n, p) in enumerate(shapes):
        ref, tol = oracle.matvec_i8x(ws[i], xs[i])
        assert_parity(descs[i]["y"].cpu().numpy(), ref, tol, name)
    ref, tol = oracle.matvec_i8x(ws[-1], xs[-1])
    assert oracle.argmax_accepted(int(host[0]), ref[0], tol[0])
    g.close()


@pytest.mark.parametrize("m", [2, 4])
def test_i8x_mixed_width_batched_step(cuda, m):
    """A batched int8 step whose widths mix the matrix-core ones with others
    (256, 512: the VALU tile, with x's packed codes in LDS after the steps),
    one launch (not sliced), an argmax on a 1024-wide matvec: every output
    against the oracle, over two launches."""
    import torch
    shapes = [("a", 512, 100), ("b", 1024, 77), ("c", 2048, 40), ("d", 256, 33),
              ("e", 3072, 50), ("lm", 1024, 3000)]
    ws = [rich_case(p, n, seed=20 + i)[0] for i, (_, n, p) in enumerate(shapes)]
    xs = [gen.activations(m, n, seed=20, index=i) for i, (_, n, p) in enumerate(shapes)]
    descs = []
    for i, (name, n, p) in enumerate(shapes):
        descs.append(dict(n=n, p=p, w=to_dev(ws[i].reshape(-1), cuda), x=to_dev(xs[i], cuda),
                          y=torch.full((m, p), float("nan"), dtype=torch.float32, device=cuda),
                          idx=torch.full((m,), -7, dtype=torch.int32, device=cuda)
                          if name == "lm" else None))
    host = torch.full((m,), -5, dtype=torch.int32).pin_memory()
    g = q8.StepGraph(descs, m, host_idx=host, mode=q8.Q8_GRAPH_PERSISTENT_I8X, device=cuda)
    assert g.info() == (1, 0)
    refs = [oracle.matvec_i8x(ws[i], xs[i]) for i in range(len(shapes))]
    for rep in range(2):
        for d in descs:
            d["y"].fill_(float("nan"))
        g.launch()
        torch.cuda.synchronize()
        for i, (name, n, p) in enumerate(shapes):
            assert_parity(descs[i]["y"].cpu().numpy(), refs[i][0], refs[i][1],
                          f"m={m} {name} rep {rep}")
        ref, tol = refs[-1]
        for r in range(m):
            assert oracle.argmax_accepted(int(host[r]), ref[r], tol[r])
    g.close()


def test_i8x_full_batched_step_every_output(cuda):
    """m = 8 through all 197 matvecs of a step with int8 activations, in the
    persistent launch the benchmark times (column slices and their sums):
    every output of every matvec for all 8 x rows against the oracle's
    quantised product, and the lm_head's 8 tokens."""
    import torch
    m = 8
    say("full int8 m=8 step: generating 197 matvecs")
    shapes, ws, xs, descs = _step(28, 151936, m, 2, cuda)
    host = torch.full((m,), -5, dtype=torch.int32).pin_memory()
    g = q8.StepGraph(descs, m, host_idx=host, mode=q8.Q8_GRAPH_PERSISTENT_I8X, device=cuda)
    assert g.info() == (2, 0)
    g.launch()
    torch.cuda.synchronize()
    say("full int8 m=8 step: checking every output against the oracle")
    for i, (name, n, p) in enumerate(shapes):
        y = descs[i]["y"].cpu().numpy()
        ref, tol = oracle.matvec_i8x(ws[i], xs[i])
        assert_parity(y, ref, tol, f"i8x m=8 {name}")
        if i == len(shapes) - 1:
            for r in range(m):
                assert oracle.argmax_accepted(int(host[r]), ref[r], tol[r])
                assert int(host[r]) == oracle.argmax_f32(y[r])
    g.close()


def test_i8x_step_refuses_other_widths(cuda):
    import torch
    shapes, ws, xs, descs = _step(0, 64, 1, 5, cuda)
    descs.append(dict(n=96, p=8, w=to_dev(rich_case(8, 96, 1)[0].reshape(-1), cuda),
                      x=to_dev(np.ones((1, 96), np.float32), cuda),
                      y=torch.empty((1, 8), dtype=torch.float32, device=cuda), idx=None))
    with pytest.raises(q8.Q8Error) as e:
        q8.StepGraph(descs, 1, mode=q8.Q8_GRAPH_PERSISTENT_I8X, device=cuda)
    assert e.value.name == "q8_err_shape"
