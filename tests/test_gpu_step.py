"""GPU tests of the recorded decode step (q8_step_graph_*).

A step is the model-order sequence of matvecs (q, k, v, o, gate, up, down per
layer, then the lm_head with its fused argmax), each with its own seeded x,
recorded once and launched as one graph; one int32 per activation row comes
back to pinned host memory."""
import numpy as np
import pytest

import gen
import oracle
from tests.gpu_helpers import assert_parity, cuda, oracle_rows, say, to_dev  # noqa: F401

pytestmark = pytest.mark.gpu


def step_inputs(layers: int, lm_p: int, m: int, seed: int = 0):
    shapes = [(f"L{l}.{name}", n, p) for l in range(layers)
              for name, n, p in gen.LAYER_SHAPES]
    shapes.append(("lm_head", 1024, lm_p))
    ws, xs = [], []
    for i, (_, n, p) in enumerate(shapes):
        ws.append(gen.weights(p, n, seed=seed, index=i))
        xs.append(gen.activations(m, n, seed=seed, index=i))
    return shapes, ws, xs


def device_step(shapes, ws, xs, m, device, lm_logits=True):
    import torch
    descs = []
    for i, (name, n, p) in enumerate(shapes):
        last = i == len(shapes) - 1
        d = dict(n=n, p=p, w=to_dev(ws[i].reshape(-1), device),
                 x=to_dev(xs[i], device), idx=None,
                 y=torch.full((m, p), float("nan"), dtype=torch.float32, device=device))
        if last:
            d["idx"] = torch.full((m,), -7, dtype=torch.int32, device=device)
            if not lm_logits:
                d["y"] = None
        descs.append(d)
    return descs


def run_graph(descs, m, mode, device):
    import torch
    import q8_block_quantized_amd as q8
    host = torch.full((m,), -5, dtype=torch.int32).pin_memory()
    g = q8.StepGraph(descs, m, host_idx=host, mode=mode, device=device)
    return g, host


@pytest.mark.parametrize("mode", [0, 1], ids=["chain", "persistent"])
def test_small_step_matches_standalone_calls(cuda, mode):
    """Graph outputs equal the standalone calls bit for bit, on every replay,
    with eager work between replays; node counts match the descriptors."""
    import torch
    import q8_block_quantized_amd as q8
    m = 1
    shapes, ws, xs = step_inputs(2, 20000, m, seed=3)
    descs = device_step(shapes, ws, xs, m, cuda)
    g, host = run_graph(descs, m, mode, cuda)
    k, c = g.info()
    assert (k, c) == ((len(shapes), 0) if mode == 0 else (1, 0))
    # standalone results
    want = []
    for d in descs[:-1]:
        y = torch.empty_like(d["y"])
        q8.q8_matvec(d["w"], d["x"].view(-1), y.view(-1))
        want.append(y)
    lm = descs[-1]
    idx_ref = torch.empty(m, dtype=torch.int32, device=cuda)
    y_lm = torch.empty_like(lm["y"])
    q8.q8_matvec_argmax(lm["w"], lm["x"], idx_ref, lm["p"], y=y_lm)
    torch.cuda.synchronize()
    for rep in range(3):
        for d in descs:
            d["y"].fill_(float("nan"))
        lm["idx"].fill_(-9)
        torch.cuda.synchronize()
        g.launch()
        torch.cuda.synchronize()
        for i, d in enumerate(descs[:-1]):
            assert torch.equal(d["y"], want[i]), f"rep {rep} desc {i}"
        assert torch.equal(lm["y"], y_lm), f"rep {rep} lm logits"
        assert lm["idx"].item() == idx_ref.item() == host[0].item(), f"rep {rep}"
    g.close()


@pytest.mark.parametrize("mode", [0, 1], ids=["chain", "persistent"])
def test_full_step_against_oracle(cuda, mode):
    """All 197 matvecs of a step (28 layers + lm_head), every output."""
    import torch
    m = 1
    say("full step: generating 197 matvecs")
    shapes, ws, xs = step_inputs(28, 151936, m, seed=0)
    descs = device_step(shapes, ws, xs, m, cuda)
    g, host = run_graph(descs, m, mode, cuda)
    assert g.info() == ((197, 0) if mode == 0 else (1, 0))
    g.launch()
    torch.cuda.synchronize()
    say("full step: checking against the oracle")
    for i, (name, n, p) in enumerate(shapes):
        ref, tol = oracle.get().matvec_mt(ws[i], xs[i][0], 16)[:2]
        y = descs[i]["y"].cpu().numpy()[0]
        assert_parity(y, ref, tol, name)
        if i == len(shapes) - 1:
            assert oracle.argmax_accepted(int(host[0]), ref, tol)
            assert int(host[0]) == oracle.argmax_f32(y)
    g.close()


@pytest.mark.parametrize("mode", [0, 1], ids=["chain", "persistent"])
def test_batched_step(cuda, mode):
    """m = 8 rows through every shape of a step (4 layers + lm_head here, the
    full 28 layers in the benchmark), argmax per row."""
    import torch
    m = 8
    shapes, ws, xs = step_inputs(4, 151936, m, seed=1)
    descs = device_step(shapes, ws, xs, m, cuda)
    g, host = run_graph(descs, m, mode, cuda)
    g.launch()
    torch.cuda.synchronize()
    for i, (name, n, p) in enumerate(shapes):
        ref, tol = oracle.matvec_batched(ws[i], xs[i])
        y = descs[i]["y"].cpu().numpy()
        assert_parity(y, ref, tol, f"m=8 {name}")
        if i == len(shapes) - 1:
            for r in range(m):
                assert oracle.argmax_accepted(int(host[r]), ref[r], tol[r])
                assert int(host[r]) == oracle.argmax_f32(y[r])
    g.close()


def test_full_batched_step_every_output(cuda):
    """m = 8 through all 197 shapes of a step (28 layers + lm_head), in the
    persistent launch the benchmark times: every output of every matvec for
    all 8 x rows against the oracle, and the lm_head's 8 tokens."""
    import torch
    m = 8
    say("full m=8 step: generating 197 matvecs")
    shapes, ws, xs = step_inputs(28, 151936, m, seed=2)
    descs = device_step(shapes, ws, xs, m, cuda)
    g, host = run_graph(descs, m, 1, cuda)
    # the step kernel over column slices of 1024, then the slices' sums (o
    # and down are 2048 and 3072 wide)
    assert g.info() == (2, 0)
    g.launch()
    torch.cuda.synchronize()
    say("full m=8 step: checking every output against the oracle")
    for i, (name, n, p) in enumerate(shapes):
        y = descs[i]["y"].cpu().numpy()
        ref, tol = oracle_rows(ws[i], xs[i])
        assert_parity(y, ref, tol, f"m=8 {name}")
        if i == len(shapes) - 1:
            for r in range(m):
                assert oracle.argmax_accepted(int(host[r]), ref[r], tol[r])
                assert int(host[r]) == oracle.argmax_f32(y[r])
    g.close()


@pytest.mark.parametrize("m", [2, 3, 5, 7])
def test_sliced_batched_step(cuda, m):
    """The batched persistent step in column slices (every width 1024, 2048
    or 3072): wide matvecs with ragged row counts (not a multiple of the
    32-row tile), an odd m (m * p not a multiple of four: the sums' scalar
    path), one empty matvec and an argmax on a 1024-wide one; every output
    against the oracle, over three launches with the outputs poisoned in
    between, and the kernel launch equal to the graph launch."""
    import torch
    shapes = [("a", 2048, 77), ("b", 1024, 100), ("c", 3072, 33), ("empty", 3072, 0),
              ("d", 2048, 1), ("e", 3072, 200), ("lm", 1024, 5000)]
    ws = [gen.weights(p, n, seed=11, index=i) for i, (_, n, p) in enumerate(shapes)]
    xs = [gen.activations(m, n, seed=11, index=i) for i, (_, n, p) in enumerate(shapes)]
    descs = device_step(shapes, ws, xs, m, cuda)
    g, host = run_graph(descs, m, 1, cuda)
    assert g.info() == (2, 0)  # the sliced step, then the slices' sums
    refs = [oracle_rows(ws[i], xs[i]) if p else None for i, (_, n, p) in enumerate(shapes)]
    first = None
    for rep in range(3):
        for d in descs:
            d["y"].fill_(float("nan"))
        host[:] = -9
        (g.launch if rep != 2 else g.launch_kernel)()
        torch.cuda.synchronize()
        for i, (name, n, p) in enumerate(shapes):
            if not p:
                continue
            y = descs[i]["y"].cpu().numpy()
            assert_parity(y, refs[i][0], refs[i][1], f"m={m} {name} rep {rep}")
        ref, tol = refs[-1]
        for r in range(m):
            assert oracle.argmax_accepted(int(host[r]), ref[r], tol[r])
        outs = [d["y"].clone() for d in descs]
        if first is None:
            first = outs
        else:
            for a, b in zip(first, outs):
                assert torch.equal(a, b)
    g.close()


def test_wide_argmax_keeps_the_unsliced_step(cuda):
    """An argmax on a matvec wider than 1024 keeps the whole-row step (one
    node): its outputs and token against the oracle."""
    import torch
    m = 4
    shapes = [("a", 1024, 64), ("lm", 2048, 3000)]
    ws = [gen.weights(p, n, seed=12, index=i) for i, (_, n, p) in enumerate(shapes)]
    xs = [gen.activations(m, n, seed=12, index=i) for i, (_, n, p) in enumerate(shapes)]
    descs = device_step(shapes, ws, xs, m, cuda)
    g, host = run_graph(descs, m, 1, cuda)
    assert g.info() == (1, 0)
    g.launch()
    torch.cuda.synchronize()
    for i, (name, n, p) in enumerate(shapes):
        ref, tol = oracle_rows(ws[i], xs[i])
        assert_parity(descs[i]["y"].cpu().numpy(), ref, tol, name)
    for r in range(m):
        assert oracle.argmax_accepted(int(host[r]), ref[r], tol[r])
    g.close()


@pytest.mark.parametrize("m", [1, 8])
def test_kernel_launch_equals_graph_launch(cuda, m):
    """q8_step_graph_launch_kernel enqueues the recorded persistent step with
    one kernel launch: every output and the host tokens equal the graph
    launch's bit for bit; a chain graph refuses it (Q8_ERR_MODE)."""
    import torch
    import q8_block_quantized_amd as q8
    shapes, ws, xs = step_inputs(2, 20000, m, seed=7)
    descs = device_step(shapes, ws, xs, m, cuda)
    g, host = run_graph(descs, m, 1, cuda)
    g.launch()
    torch.cuda.synchronize()
    want = [d["y"].clone() for d in descs]
    want_tok = host.clone()
    for _ in range(3):
        for d in descs:
            d["y"].fill_(float("nan"))
        host[:] = -9
        g.launch_kernel()
        torch.cuda.synchronize()
        for d, w in zip(descs, want):
            assert torch.equal(d["y"], w)
        assert torch.equal(host, want_tok)
    g.close()
    gc, _ = run_graph(descs, m, 0, cuda)
    assert q8.load().q8_step_graph_launch_kernel(gc._h, None) == 11
    gc.close()


def layer_levels(layers):
    """Dependency levels of a decoder step in model order: q, k, v together,
    then o, then gate and up together, then down, per layer; the lm_head
    last."""
    lv = []
    for l in range(layers):
        base = 4 * l
        lv += [base, base, base, base + 1, base + 2, base + 2, base + 3]
    return lv + [4 * layers]


@pytest.mark.parametrize("m", [1, 8])
def test_levels_step_equals_standalone(cuda, m):
    """q8_step_graph_build_levels: one persistent node per level (9 for two
    layers and the lm_head); every output and token equals the standalone
    calls' bit for bit, through the graph and through the kernel launches."""
    import torch
    import q8_block_quantized_amd as q8
    shapes, ws, xs = step_inputs(2, 20000, m, seed=8)
    descs = device_step(shapes, ws, xs, m, cuda)
    host = torch.full((m,), -5, dtype=torch.int32).pin_memory()
    g = q8.StepGraph(descs, m, host_idx=host, device=cuda, levels=layer_levels(2))
    assert g.info() == (9, 0)
    want = []
    for d in descs[:-1]:
        y = torch.empty_like(d["y"])
        q8.q8_matvec_batched(d["w"], d["x"], y)
        want.append(y)
    lm = descs[-1]
    ylm = torch.empty_like(lm["y"])
    idx = torch.empty_like(lm["idx"])
    q8.q8_matvec_argmax(lm["w"], lm["x"], idx, lm["p"], y=ylm)
    want.append(ylm)
    torch.cuda.synchronize()
    for k in range(3):
        for d in descs:
            d["y"].fill_(float("nan"))
        host[:] = -9
        (g.launch if k != 1 else g.launch_kernel)()
        torch.cuda.synchronize()
        for d, w_ in zip(descs, want):
            assert torch.equal(d["y"], w_)
        assert torch.equal(host, idx.cpu())
    g.close()


@pytest.mark.parametrize("m", [1, 8])
def test_levels_step_against_oracle(cuda, m):
    """The levels graph (one persistent node per dependency level: q|k|v, o,
    gate|up, down per layer, then the lm_head) against the oracle itself:
    two layers and a 20,000-row lm_head, every output of every matvec for
    every x row, the tokens accepted by the oracle and equal to the argmax
    of the logits the graph wrote."""
    import torch
    import q8_block_quantized_amd as q8
    shapes, ws, xs = step_inputs(2, 20000, m, seed=10 + m)
    descs = device_step(shapes, ws, xs, m, cuda)
    host = torch.full((m,), -5, dtype=torch.int32).pin_memory()
    g = q8.StepGraph(descs, m, host_idx=host, device=cuda, levels=layer_levels(2))
    assert g.info() == (9, 0)
    for launch in (g.launch, g.launch_kernel):
        for d in descs:
            d["y"].fill_(float("nan"))
        host[:] = -9
        torch.cuda.synchronize()
        launch()
        torch.cuda.synchronize()
        for i, (name, n, p) in enumerate(shapes):
            y = descs[i]["y"].cpu().numpy()
            ref, tol = oracle.matvec_batched(ws[i], xs[i])
            assert_parity(y, ref, tol, f"levels m={m} {name}")
            if i == len(shapes) - 1:
                for r in range(m):
                    assert oracle.argmax_accepted(int(host[r]), ref[r], tol[r])
                    assert int(host[r]) == oracle.argmax_f32(y[r])
    g.close()


@pytest.mark.parametrize("mode", [1, 2], ids=["persistent", "persistent-i8x"])
def test_step_with_empty_descriptors(cuda, mode):
    """Descriptors with p = 0 own no tiles; placed first, between others and
    last-but-one, the tile lookup skips them and every other output equals
    its standalone call bit for bit."""
    import torch
    import q8_block_quantized_amd as q8
    shapes, ws, xs = step_inputs(1, 3000, 1, seed=9)
    descs = device_step(shapes, ws, xs, 1, cuda)
    empty = lambda: dict(n=1024, p=0, w=torch.empty(0, dtype=torch.uint8, device=cuda),  # noqa: E731
                         x=to_dev(np.ones((1, 1024), np.float32), cuda), idx=None,
                         y=torch.empty((1, 0), dtype=torch.float32, device=cuda))
    mixed = [empty(), descs[0], descs[1], empty(), empty(), *descs[2:-1], empty(), descs[-1]]
    g, host = run_graph(mixed, 1, mode, cuda)
    g.launch()
    torch.cuda.synchronize()
    fn = q8.q8_matvec_i8x if mode == 2 else q8.q8_matvec_batched
    for d in descs[:-1]:
        y = torch.empty_like(d["y"])
        fn(d["w"], d["x"], y)
        torch.cuda.synchronize()
        assert torch.equal(d["y"], y)
    g.close()


def test_destroyed_handle_is_refused(cuda):
    import q8_block_quantized_amd as q8
    shapes, ws, xs = step_inputs(0, 64, 1, seed=4)
    descs = device_step(shapes, ws, xs, 1, cuda)
    g, _ = run_graph(descs, 1, 0, cuda)
    h = g._h
    g.close()
    assert q8.load().q8_step_graph_launch(h, None) == 9
    assert q8.load().q8_step_graph_destroy(h) == 9


def test_unpinned_host_idx_is_refused(cuda):
    """The token is stored by the kernel into host_idx, so host_idx must be
    pinned host memory; ordinary pageable memory is refused before any GPU
    work (Q8_ERR_HIP), straight through the C ABI."""
    import ctypes
    import q8_block_quantized_amd as q8
    shapes, ws, xs = step_inputs(0, 64, 1, seed=5)
    descs = device_step(shapes, ws, xs, 1, cuda)
    d = descs[0]
    arr = (q8.MatvecDesc * 1)()
    arr[0] = q8.MatvecDesc(d["w"].data_ptr(), d["x"].data_ptr(), d["y"].data_ptr(),
                           d["idx"].data_ptr(), d["n"], d["p"])
    pageable = (ctypes.c_int32 * 4)()
    out = ctypes.c_void_p()
    st = q8.load().q8_step_graph_build(arr, 1, 1, ctypes.addressof(pageable), 1, None,
                                       ctypes.byref(out))
    assert st == 7 and not out.value


@pytest.mark.parametrize("mode", [0, 1], ids=["chain", "persistent"])
def test_token_reaches_host_without_copy(cuda, mode):
    """The argmax's last arrival stores each row's token into pinned host
    memory itself: the graph has no copy node, and the host value equals the
    device idx after the stream is synchronised, for every launch."""
    import torch
    m = 3
    shapes, ws, xs = step_inputs(1, 5000, m, seed=6)
    descs = device_step(shapes, ws, xs, m, cuda)
    g, host = run_graph(descs, m, mode, cuda)
    assert g.info()[1] == 0
    for k in range(3):
        host[:] = -9
        g.launch()
        torch.cuda.synchronize()
        dev_idx = descs[-1]["idx"].cpu()
        assert torch.equal(host, dev_idx), (k, host, dev_idx)
    ref, tol = oracle.matvec_batched(ws[-1], xs[-1])
    for r in range(m):
        assert oracle.argmax_accepted(int(host[r]), ref[r], tol[r])
    g.close()
