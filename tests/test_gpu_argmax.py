"""GPU parity of q8_argmax and of the fused lm_head q8_matvec_argmax.

On the same float32 logits the GPU and the oracle take the argmax decision in
the same precision, so the index must match exactly.  For the fused kernel
the GPU decides on its own float32 logits: the index must equal the argmax of
the logits it wrote, and must be a correct argmax of the exact logits (equal
to the oracle's, or within the bound of it)."""
import numpy as np
import pytest

import gen
import oracle
from tests import pagegen
from tests.gpu_helpers import assert_parity, cuda, say, to_dev  # noqa: F401
from tests.oracle_pins import rich_case

pytestmark = pytest.mark.gpu

NAN, INF = float("nan"), float("inf")


def gpu_argmax(logits: np.ndarray, device) -> np.ndarray:
    import torch
    import q8_block_quantized_amd as q8
    lg = to_dev(logits.astype(np.float32), device)
    m = 1 if logits.ndim == 1 else logits.shape[0]
    idx = torch.full((m,), -7, dtype=torch.int32, device=device)
    q8.q8_argmax(lg, idx)
    torch.cuda.synchronize()
    return idx.cpu().numpy()


def gpu_fused(w, x, device, write_y: bool):
    import torch
    import q8_block_quantized_amd as q8
    x = np.atleast_2d(x)
    m = x.shape[0]
    p = w.shape[0]
    wd = to_dev(w.reshape(-1), device)
    xd = to_dev(x.astype(np.float32), device)
    idx = torch.full((m,), -7, dtype=torch.int32, device=device)
    y = torch.full((m, p), NAN, dtype=torch.float32, device=device) if write_y else None
    q8.q8_matvec_argmax(wd, xd, idx, p, y=y)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), (y.cpu().numpy() if write_y else None)


def test_page_argmax_example(cuda):
    """151,936 logits, 9.5 at 140011 and 140012: the lower index wins."""
    kv = pagegen.read_kv(pagegen.__file__.replace("pagegen.py", "golden/argmax_tie.txt"))
    v = pagegen.lcg_f32(int(kv["seed"][0][0]), int(kv["n"][0][0]))
    for i, val in kv["plant"]:
        v[int(i)] = np.float32(float(val))
    got = gpu_argmax(v, cuda)
    assert got[0] == int(kv["expect"][0][0]) == oracle.argmax_f32(v)


def test_argmax_rules(cuda):
    rows = [
        [1.0, 3.0, 3.0, 2.0], [5.0, 1.0, 5.0, 0.0], [NAN, 1.0, 0.5, NAN],
        [NAN, NAN, NAN, NAN], [-0.0, 0.0, -1.0, -2.0], [0.0, -0.0, -1.0, -3.0],
        [-INF, -INF, -INF, -INF], [1.0, INF, INF, NAN],
    ]
    v = np.array(rows, dtype=np.float32)
    got = gpu_argmax(v, cuda)
    want = [oracle.argmax_f32(r) for r in v]
    assert list(got) == want == [1, 0, 1, -1, 0, 0, 0, 1]


@pytest.mark.parametrize("m,p", [(1, 1), (1, 7), (3, 151936), (8, 5000), (2, 1 << 20)])
def test_argmax_random_exact(cuda, m, p):
    rng = np.random.default_rng(m * p)
    v = rng.standard_normal((m, p)).astype(np.float32)
    if p > 10:  # a tie at the top of row 0, a NaN in row m-1
        top = np.float32(v[0].max() + 1)
        v[0, p // 3] = top
        v[0, p // 2] = top
        v[m - 1, p - 1] = NAN
    got = gpu_argmax(v, cuda)
    assert list(got) == [oracle.argmax_f32(r) for r in v]


def test_argmax_repeated_calls(cuda):
    """The workspace is cleared by each launch: repeated calls stay right."""
    rng = np.random.default_rng(5)
    for t in range(5):
        v = rng.standard_normal((2, 3001 + t)).astype(np.float32)
        assert list(gpu_argmax(v, cuda)) == [oracle.argmax_f32(r) for r in v]


def check_fused(w, x, device, label):
    x2 = np.atleast_2d(x)
    idx_y, y = gpu_fused(w, x2, device, True)
    idx_n, _ = gpu_fused(w, x2, device, False)
    ref, tol = oracle.matvec_batched(w, x2)
    assert_parity(y, ref, tol, label)
    for i in range(x2.shape[0]):
        assert idx_y[i] == idx_n[i], f"{label} row {i}: with/without logits differ"
        assert idx_y[i] == oracle.argmax_f32(y[i]), f"{label} row {i}: not argmax of own logits"
        assert oracle.argmax_accepted(int(idx_y[i]), ref[i], tol[i]), \
            f"{label} row {i}: {idx_y[i]} vs oracle {oracle.argmax_f64(ref[i])}"
    return idx_y


def test_lm_head_fused(cuda):
    """The lm_head: 1024 -> 151,936 with the fused argmax, every logit."""
    say("lm_head fused 1024->151936")
    w = gen.weights(151936, 1024, seed=0, index=196)
    x = gen.activations(1, 1024, seed=0, index=196)
    check_fused(w, x, cuda, "lm_head")


@pytest.mark.parametrize("m,p,n", [(1, 1, 1024), (1, 3, 96), (2, 4097, 1024),
                                   (8, 20000, 1024), (3, 999, 3072), (5, 130, 160)])
def test_fused_shapes(cuda, m, p, n):
    w, _ = rich_case(p, n, seed=p + n)
    x = gen.activations(m, n, seed=m, index=n)
    check_fused(w, x, cuda, f"m={m} p={p} n={n}")


@pytest.mark.parametrize("m,n", [(1, 1024), (2, 1024), (1, 96)])
def test_fused_tie_goes_low(cuda, m, n):
    """Two identical weight rows that hold the largest logit: the page's tie
    example at the lm_head's size, through the fused kernel."""
    p = 151936 if (m, n) == (1, 1024) else 5000
    lo = 140011 if p == 151936 else 3001
    w = gen.weights(p, n, seed=1, index=1)
    x = gen.activations(m, n, seed=1, index=1)
    w[lo] = w[lo + 1]
    # make that row dominant: copy x's sign pattern into its quants
    blk = w.reshape(p, n // 32, 34)
    s = np.sign(x[0]).reshape(n // 32, 32)
    blk[lo, :, 2:] = (s * 127).astype(np.int8).view(np.uint8)
    blk[lo + 1] = blk[lo]
    idx = check_fused(w, x, cuda, f"tie m={m} n={n}")
    assert idx[0] == lo


def test_fused_all_nan_row_is_minus_one(cuda):
    p, n = 300, 1024
    w, x = rich_case(p, n, seed=2)
    blk = w.reshape(p, n // 32, 34)
    blk[:, :, 0], blk[:, :, 1] = 0x00, 0x7E  # every scale NaN
    idx, _ = gpu_fused(w, x, cuda, False)
    assert idx[0] == -1


def test_streams_have_their_own_workspace(cuda):
    """Fused lm_head argmax calls on four streams at once, interleaved over
    many rounds: each stream's argmax workspace is its own, so every call
    returns its own input's token (checked against the oracle) and the
    standalone argmax on the same streams agrees."""
    import torch
    import q8_block_quantized_amd as q8
    p, n, S = 151936, 1024, 4
    w = gen.weights(p, n, seed=40, index=0)
    wd = to_dev(w.reshape(-1), cuda)
    xs = gen.activations(S, n, seed=40, index=1)
    xd = [to_dev(xs[i:i + 1], cuda) for i in range(S)]
    streams = [torch.cuda.Stream(device=cuda) for _ in range(S)]
    want = []
    for i in range(S):
        ref, tol = oracle.get().matvec_mt(w, xs[i], 16)[:2]
        y = torch.empty((1, p), dtype=torch.float32, device=cuda)
        idx = torch.empty(1, dtype=torch.int32, device=cuda)
        q8.q8_matvec_argmax(wd, xd[i], idx, p, y=y)
        torch.cuda.synchronize()
        assert oracle.argmax_accepted(int(idx.item()), ref, tol)
        want.append((int(idx.item()), y))
    torch.cuda.synchronize()
    outs = [torch.full((20,), -7, dtype=torch.int32, device=cuda) for _ in range(S)]
    outs2 = [torch.full((20,), -7, dtype=torch.int32, device=cuda) for _ in range(S)]
    torch.cuda.synchronize()  # the fills above ran on the default stream
    for k in range(20):
        for i in range(S):
            q8.q8_matvec_argmax(wd, xd[i], outs[i][k:k + 1], p, stream=streams[i])
            q8.q8_argmax(want[i][1], outs2[i][k:k + 1], stream=streams[i])
    torch.cuda.synchronize()
    for i in range(S):
        assert torch.all(outs[i] == want[i][0]), (i, outs[i])
        assert torch.all(outs2[i] == want[i][0]), (i, outs2[i])


def test_first_call_on_a_capturing_stream_is_refused(cuda):
    """A stream's argmax workspace is allocated and cleared on its first
    argmax call; made while the stream is capturing, that call is refused
    with Q8_ERR_GRAPH (8) before any GPU work, and the same call outside the
    capture then runs normally."""
    import ctypes
    import torch
    import q8_block_quantized_amd as q8
    hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch has loaded
    p, n = 5000, 1024
    w = gen.weights(p, n, seed=41, index=0)
    x = gen.activations(1, n, seed=41, index=1)
    wd, xd = to_dev(w.reshape(-1), cuda), to_dev(x, cuda)
    idx = torch.full((1,), -7, dtype=torch.int32, device=cuda)
    torch.cuda.synchronize()
    s = ctypes.c_void_p()
    assert hip.hipStreamCreate(ctypes.byref(s)) == 0
    assert hip.hipStreamBeginCapture(s, 2) == 0  # relaxed mode
    st = q8.load().q8_matvec_argmax(wd.data_ptr(), xd.data_ptr(), None, idx.data_ptr(),
                                    1, n, p, s)
    graph = ctypes.c_void_p()
    assert hip.hipStreamEndCapture(s, ctypes.byref(graph)) == 0
    if graph.value:
        hip.hipGraphDestroy(graph)
    assert st == 8, q8.q8_status_name(st)
    st = q8.load().q8_matvec_argmax(wd.data_ptr(), xd.data_ptr(), None, idx.data_ptr(),
                                    1, n, p, s)
    assert st == 0
    assert hip.hipStreamSynchronize(s) == 0
    assert hip.hipStreamDestroy(s) == 0
    ref, tol = oracle.matvec(w, x[0])
    assert oracle.argmax_accepted(int(idx.item()), ref, tol)
