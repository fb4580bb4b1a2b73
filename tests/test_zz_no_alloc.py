"""q8_matvec_argmax_noalloc, the fused lm_head argmax for callers that
cannot allocate, through the C ABI: on two calls in a row (the second with
a smaller input) its logits and indices equal q8_matvec_argmax's bit for
bit and meet the oracle's bar; rows beyond the workspace's limit are
refused."""
import numpy as np
import pytest

import gen
import oracle
from tests.gpu_helpers import assert_parity, cuda, oracle_rows, say, to_dev  # noqa: F401

pytestmark = pytest.mark.gpu


def _case(cuda, m, n, p, seed, logits=True):
    import torch
    import q8_block_quantized_amd as q8
    say(f"noalloc case m={m} n={n} p={p} seed={seed} logits={logits}")
    w = gen.weights(p, n, seed=seed, index=0)
    x = gen.activations(m, n, seed=seed, index=1)
    wd, xd = to_dev(w.reshape(-1), cuda), to_dev(x, cuda)
    idx_a = torch.full((m,), -7, dtype=torch.int32, device=cuda)
    idx_b = torch.full((m,), -9, dtype=torch.int32, device=cuda)
    y_a = torch.full((m, p), float("nan"), dtype=torch.float32, device=cuda)
    y_b = torch.full((m, p), float("nan"), dtype=torch.float32, device=cuda) if logits else None
    torch.cuda.synchronize()
    q8.q8_matvec_argmax(wd, xd, idx_a, p, y=y_a)
    lib = q8.load()
    st = lib.q8_matvec_argmax_noalloc(wd.data_ptr(), xd.data_ptr(),
                                      y_b.data_ptr() if logits else None,
                                      idx_b.data_ptr(), m, n, p,
                                      torch.cuda.current_stream(cuda).cuda_stream)
    assert st == 0, q8.q8_status_name(st)
    torch.cuda.synchronize()
    assert torch.equal(idx_a, idx_b), (idx_a, idx_b)
    ya = y_a.cpu().numpy()
    if logits:
        assert torch.equal(y_a, y_b)
    ref, tol = oracle_rows(w, x)
    assert_parity(ya, ref, tol, f"noalloc m={m} p={p}")
    for r in range(m):
        g = int(idx_b[r])
        assert oracle.argmax_accepted(g, ref[r], tol[r]), (r, g)
        assert g == oracle.argmax_f32(ya[r])


def test_noalloc_matches_allocating_entry_point(cuda):
    """Two calls in a row, the second smaller (fewer rows, fewer logits,
    another width), then one without logits: the shared workspace is left
    clean by each call, so every result equals the allocating entry
    point's."""
    _case(cuda, 4, 1024, 151936, 50)
    _case(cuda, 2, 2048, 5000, 51)
    _case(cuda, 1, 1024, 20000, 52, logits=False)


def test_noalloc_refuses_rows_beyond_the_workspace(cuda):
    """The workspace holds the keys of at most 32 activation rows: m = 33 is
    refused with Q8_ERR_SHAPE before any GPU work; a null idx with
    Q8_ERR_NULL."""
    import torch
    import q8_block_quantized_amd as q8
    n, p = 256, 64
    w = torch.zeros(q8.weight_bytes(n, p), dtype=torch.uint8, device=cuda)
    x = torch.zeros((33, n), dtype=torch.float32, device=cuda)
    idx = torch.zeros(33, dtype=torch.int32, device=cuda)
    lib = q8.load()
    assert lib.q8_matvec_argmax_noalloc(w.data_ptr(), x.data_ptr(), None, idx.data_ptr(),
                                        33, n, p, None) == 2
    assert lib.q8_matvec_argmax_noalloc(w.data_ptr(), x.data_ptr(), None, None,
                                        1, n, p, None) == 1
