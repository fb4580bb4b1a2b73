"""Split-K: one activation row of a matrix wider than the staged path (n a
multiple of 256 above 3072) is cut into column slices of at most 3072
columns, each slice's partial sums written apart and added in slice order
(the rvllm page's K-split for matrices whose output alone gives too few
work items, "The matmul pain story").  Every output against the oracle at
its bar, the argmax on the summed logits, bit-identical repeats, and the
per-stream partial-sum buffer growing between calls."""
import numpy as np
import pytest

import gen
import oracle
from tests.gpu_helpers import assert_parity, cuda, oracle_rows, say, to_dev  # noqa: F401
from tests.oracle_pins import rich_case

pytestmark = pytest.mark.gpu

NAN = float("nan")


def slices_of(n):
    """Slice count and width in blocks, by the rule the library states."""
    bpr = n // 32
    s = -(-bpr // 96)
    b = -(-bpr // s)
    b = (b + 7) // 8 * 8
    return -(-bpr // b), b


def test_slice_rule():
    assert slices_of(3328) == (2, 56)
    assert slices_of(4096) == (2, 64)
    assert slices_of(8192) == (3, 88)
    assert slices_of(12288) == (4, 96)
    assert slices_of(65536) == (22, 96)


SHAPES = [(1, 3328), (7, 4096), (300, 4096), (4099, 8192), (65, 12288), (2, 65536),
          (513, 65536), (33, 5120)]


@pytest.mark.parametrize("p,n", SHAPES)
def test_split_matvec_matches_oracle(cuda, p, n):
    """Planted -128 quants, subnormal, zero, negative and large scales."""
    import torch
    import q8_block_quantized_amd as q8
    say(f"split matvec p={p} n={n}")
    w, x = rich_case(p, n, seed=p + n)
    wd, xd = to_dev(w.reshape(-1), cuda), to_dev(x.astype(np.float32), cuda)
    y = torch.full((p,), NAN, dtype=torch.float32, device=cuda)
    q8.q8_matvec(wd, xd, y)
    y2 = torch.full((1, p), NAN, dtype=torch.float32, device=cuda)
    q8.q8_matvec_batched(wd, xd.view(1, -1), y2)
    torch.cuda.synchronize()
    ref, tol = oracle.get().matvec_mt(w, x, 16)[:2]
    assert_parity(y.cpu().numpy(), ref, tol, f"p={p} n={n}")
    assert torch.equal(y, y2.view(-1)), "batched m = 1 and q8_matvec differ"
    # repeats are bit-identical
    y3 = torch.full_like(y, NAN)
    q8.q8_matvec(wd, xd, y3)
    torch.cuda.synchronize()
    assert torch.equal(y, y3)


@pytest.mark.parametrize("p,n", [(151936, 4096), (20000, 8192), (9, 65536)])
def test_split_fused_argmax(cuda, p, n):
    """The fused argmax over the summed logits: accepted by the oracle and
    equal to the argmax of the logits it wrote; the same index without
    logits; ties planted across slices' rows go to the lowest index."""
    import torch
    import q8_block_quantized_amd as q8
    say(f"split fused argmax p={p} n={n}")
    w = gen.weights(p, n, seed=60, index=n)
    x = gen.activations(1, n, seed=60, index=n + 1)
    wd, xd = to_dev(w.reshape(-1), cuda), to_dev(x, cuda)
    idx = torch.full((1,), -7, dtype=torch.int32, device=cuda)
    y = torch.full((1, p), NAN, dtype=torch.float32, device=cuda)
    q8.q8_matvec_argmax(wd, xd, idx, p, y=y)
    idx2 = torch.full((1,), -7, dtype=torch.int32, device=cuda)
    q8.q8_matvec_argmax(wd, xd, idx2, p)
    torch.cuda.synchronize()
    ref, tol = oracle.get().matvec_mt(w, x[0], 16)[:2]
    yh = y.cpu().numpy()[0]
    assert_parity(yh, ref, tol, f"logits p={p} n={n}")
    g = int(idx.item())
    assert oracle.argmax_accepted(g, ref, tol)
    assert g == oracle.argmax_f32(yh) == int(idx2.item())
    # rows equal to the winner's, further down: the lowest index stays
    if p > 2:
        w2 = w.reshape(p, -1).copy()
        w2[p - 1] = w2[g]
        w2[p // 2] = w2[g]
        wd2 = to_dev(w2.reshape(-1), cuda)
        q8.q8_matvec_argmax(wd2, xd, idx, p)
        torch.cuda.synchronize()
        assert int(idx.item()) == min(g, p // 2)


def test_split_streams_and_growing_buffer(cuda):
    """Small then large outputs on one stream (the partial-sum buffer grows
    and its old contents are never read), and four streams at once, each
    with its own buffer: every result equals the default stream's."""
    import torch
    import q8_block_quantized_amd as q8
    n = 8192
    cases = [(64, 70), (20000, 71), (500, 72), (30000, 73)]
    data = []
    for p, seed in cases:
        w = gen.weights(p, n, seed=seed, index=0)
        x = gen.activations(1, n, seed=seed, index=1)
        data.append((p, to_dev(w.reshape(-1), cuda), to_dev(x, cuda), w, x))
    want = []
    for p, wd, xd, w, x in data:
        y = torch.empty(p, dtype=torch.float32, device=cuda)
        q8.q8_matvec(wd, xd.view(-1), y)
        torch.cuda.synchronize()
        ref, tol = oracle.get().matvec_mt(w, x[0], 16)[:2]
        assert_parity(y.cpu().numpy(), ref, tol, f"p={p}")
        want.append(y)
    streams = [torch.cuda.Stream(device=cuda) for _ in cases]
    outs = [torch.full((p,), NAN, dtype=torch.float32, device=cuda) for p, *_ in data]
    torch.cuda.synchronize()
    for rep in range(5):
        for (p, wd, xd, _, _), st, o in zip(data, streams, outs):
            q8.q8_matvec(wd, xd.view(-1), o, stream=st)
    torch.cuda.synchronize()
    for o, w_ in zip(outs, want):
        assert torch.equal(o, w_)


def test_split_nan_scale_and_one_hot(cuda):
    """A NaN scale in the second slice reaches its row only; one-hot x picks
    scale * q exactly from any slice."""
    import torch
    import q8_block_quantized_amd as q8
    p, n = 40, 8192
    w = gen.weights(p, n, seed=74, index=0).reshape(p, n // 32, 34).copy()
    w[5, 100, 0], w[5, 100, 1] = 0x00, 0x7E  # NaN scale (block 100: second slice)
    wd = to_dev(w.reshape(-1), cuda)
    for col in (3, 2816 + 40, 8191):
        x = np.zeros(n, np.float32)
        x[col] = 1.0
        y = torch.full((p,), NAN, dtype=torch.float32, device=cuda)
        q8.q8_matvec(wd, to_dev(x, cuda), y)
        torch.cuda.synchronize()
        ref, tol = oracle.matvec(w.reshape(p, -1), x)
        yh = y.cpu().numpy()
        assert np.isnan(yh[5]) and np.isnan(ref[5])
        keep = np.arange(p) != 5
        assert np.array_equal(yh[keep], ref[keep].astype(np.float32)), col
