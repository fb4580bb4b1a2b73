"""GPU tests of the whole decode step (q8_decode_graph_build): norms, the
q/k/v projections, QK-norm, RoPE, the KV append, attention, the o
projection and residual add, SwiGLU, the down projection and residual add,
the final norm and the lm_head argmax, recorded as one graph.

Parity is checked stage by stage: every stage's GPU output is compared with
the oracle applied to that stage's GPU inputs (read back from the step's
buffers), within a bound derived from binary32 arithmetic for that stage
(u = 2^-24):
  * rms_norm_row over n values: |d| <= (n + 16) u |ref|  (the sum of
    squares in any order, the root, the quotient and two products);
  * QK-norm then RoPE of a pair (a, b) of a head of 128: |d| <= 256 u
    (|a| + |b|) of the reference pair (the norm's bound plus 2-ulp sine and
    cosine; both sides use the same binary32 angle);
  * attention: with p the reference softmax weights and dq the bound on the
    GPU query, each score is off by at most
      ds_t = (sum_j dq_j |k_tj| + 130 u sum_j |q_j k_tj|) / sqrt(128) + u |s_t|,
    so |d out_j| <= 1.5 (2 max_t ds_t + (3 (64 + nc) + 20) u) sum_t p_t |v_tj|
    (64 rows per partial, nc partials merged);
  * silu_hadamard: |d| <= 16 u |ref| + 1e-30;
  * the matvecs: the oracle's own bar, 1e-4 sum|scale q x| + 1e-6;
  * residual adds: bit-exact (one binary32 addition);
  * cache rows other than pos: untouched, bit-exact.
The whole 28-layer step is also run against the oracle's binary64 chain from
the same inputs: the final normed state within 1e-3 relative (the stage
bounds compound over 28 layers; this is the loose end-to-end check), and the
token accepted when its exact logit is within the propagated bound of the
maximum."""
import math

import numpy as np
import pytest

import gen
import oracle
import q8_block_quantized_amd as q8
from tests.gpu_helpers import assert_parity, cuda, say, to_dev  # noqa: F401

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
BUF_F32 = ("x", "xn", "q", "k", "v", "attn", "attn_out", "xn2", "gate", "up", "h",
           "ffn_out", "xf", "logits")


def oracle_layer(L):
    return dict(wq=L["wq"], wk=L["wk"], wv=L["wv"], wo=L["wo"], wg=L["w_gate"],
                wu=L["w_up"], wd=L["w_down"], attn_norm=L["attn_norm"],
                q_norm=L["q_norm"], k_norm=L["k_norm"], ffn_norm=L["ffn_norm"])


class DeviceModel:
    """The model's tensors on the GPU, the step's buffers and its graph."""

    def __init__(self, model, device, logits=True, form=None):
        import torch
        self.model = model
        self.dims = model["dims"]
        self.device = device
        self.layers = []
        for L in model["layers"]:
            d = {}
            for f in q8.LAYER_FIELDS:
                a = L[f]
                d[f] = to_dev(a.reshape(-1), device)
            self.layers.append(d)
        self.out_norm = to_dev(model["out_norm"], device)
        self.lm_head = to_dev(model["lm_head"].reshape(-1), device)
        self.bufs = q8.decode_buffers(self.dims, device, logits=logits)
        self.bufs["x_in"].copy_(to_dev(model["x_in"], device))
        self.host = torch.full((1,), -7, dtype=torch.int32).pin_memory()
        self.graph = q8.DecodeGraph(self.dims, self.layers, self.out_norm, self.lm_head,
                                    self.bufs, host_token=self.host, form=form)

    def run(self, pos, kernel=False, x_in=None):
        import torch
        if x_in is not None:
            self.bufs["x_in"].copy_(to_dev(x_in, self.device))
        self.bufs["pos"].fill_(pos)
        self.host.fill_(-7)
        for k in BUF_F32:
            if self.bufs.get(k) is not None:
                self.bufs[k].fill_(float("nan"))
        self.bufs["token"].fill_(-9)
        if kernel:
            self.graph.launch_kernel()
        else:
            self.graph.launch()
        torch.cuda.synchronize()
        out = {k: self.bufs[k].cpu().numpy() for k in BUF_F32 if self.bufs.get(k) is not None}
        out["token"] = int(self.bufs["token"].item())
        out["host_token"] = int(self.host[0])
        kvw = self.dims["n_kv_heads"] * self.dims["head_dim"]
        out["kc"] = [L["k_cache"].cpu().numpy().reshape(-1, kvw) for L in self.layers]
        out["vc"] = [L["v_cache"].cpu().numpy().reshape(-1, kvw) for L in self.layers]
        return out

    def close(self):
        self.graph.close()


def norm_bound(ref, n):
    return (n + 16) * U * np.abs(ref) + 1e-37


def assert_within(got, ref, bound, label):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    ok = err <= bound
    if not ok.all():
        i = int(np.argmax(err / bound))
        raise AssertionError(f"{label}: index {i}: gpu {got[i]!r} ref {ref[i]!r} "
                             f"err {err[i]:.3e} bound {bound[i]:.3e}")
    say(f"  {label}: worst err/bound {float(np.max(err / bound)):.3f}")


def qk_prep(x, w, hd, pos, dims):
    """QK-norm then RoPE (oracle) of heads x, and the per-element bound."""
    xn = oracle.rms_norm(np.asarray(x, np.float64).reshape(-1, hd), w, dims["eps"]).ravel()
    r = oracle.rope(xn, hd, pos, dims["theta"])
    half = hd // 2
    rr = r.reshape(-1, 2, half)
    pair = np.abs(rr[:, 0, :]) + np.abs(rr[:, 1, :])
    bound = 256 * U * np.repeat(pair[:, None, :], 2, axis=1).ravel() + 1e-37
    return r, bound


def attention_bound(qref, dq, kc, vc, probs, seq, dims):
    H, KV, hd = dims["n_heads"], dims["n_kv_heads"], dims["head_dim"]
    G = H // KV
    nc = (seq + 63) // 64
    out = np.empty(H * hd)
    for h in range(H):
        g = h // G
        kh = kc[:seq, g * hd:(g + 1) * hd]
        vh = vc[:seq, g * hd:(g + 1) * hd]
        qh, dqh = qref[h * hd:(h + 1) * hd], dq[h * hd:(h + 1) * hd]
        s = kh @ qh / math.sqrt(hd)
        ds = (np.abs(kh) @ dqh + 130 * U * (np.abs(kh) @ np.abs(qh))) / math.sqrt(hd) \
            + U * np.abs(s)
        mag = probs[h, :seq] @ np.abs(vh)
        out[h * hd:(h + 1) * hd] = 1.5 * (2 * ds.max() + (3 * (64 + nc) + 20) * U) * mag
    return out + 1e-37


def check_stages(res, model, pos, x_in=None):
    """Stage-by-stage parity of the last layer of a step (and the head)."""
    dims = model["dims"]
    L = model["layers"][-1]
    H, hd = dims["hidden"], dims["head_dim"]
    KV = dims["n_kv_heads"]
    eps = dims["eps"]
    if x_in is not None:  # one-layer model: the layer's input is x_in
        ref = oracle.rms_norm(x_in, L["attn_norm"], eps)
        assert_within(res["xn"], ref, norm_bound(ref, H), "attention norm")
    for name, w in (("q", L["wq"]), ("k", L["wk"]), ("v", L["wv"])):
        y, tol = oracle.matvec(w, res["xn"])
        assert_parity(res[name], y, tol, f"{name} projection")
    kref, kb = qk_prep(res["k"], L["k_norm"], hd, pos, dims)
    assert_within(res["kc"][-1][pos], kref, kb, "appended key (QK-norm, RoPE)")
    assert np.array_equal(res["vc"][-1][pos], res["v"]), "appended value"
    qref, qb = qk_prep(res["q"], L["q_norm"], hd, pos, dims)
    kc = res["kc"][-1].astype(np.float64)
    vc = res["vc"][-1].astype(np.float64)
    aref, probs = oracle.attention(qref, kc, vc, pos + 1, dims["n_heads"], KV, hd)
    ab = attention_bound(qref, qb, kc, vc, probs, pos + 1, dims)
    assert_within(res["attn"], aref, ab, "attention")
    y, tol = oracle.matvec(L["wo"], res["attn"])
    assert_parity(res["attn_out"], y, tol, "o projection")
    for name, w in (("gate", L["w_gate"]), ("up", L["w_up"])):
        y, tol = oracle.matvec(w, res["xn2"])
        assert_parity(res[name], y, tol, f"{name} projection")
    href = oracle.silu_mul(res["gate"], res["up"])
    assert_within(res["h"], href, 16 * U * np.abs(href) + 1e-30, "silu_hadamard")
    y, tol = oracle.matvec(L["w_down"], res["h"])
    assert_parity(res["ffn_out"], y, tol, "down projection")
    if x_in is not None:
        x_mid = (x_in.astype(np.float32) + res["attn_out"]).astype(np.float32)
        ref = oracle.rms_norm(x_mid, L["ffn_norm"], eps)
        assert_within(res["xn2"], ref, norm_bound(ref, H), "ffn norm")
        x_fin = (x_mid + res["ffn_out"]).astype(np.float32)
        assert np.array_equal(res["x"], x_fin), "residual adds"
    ref = oracle.rms_norm(res["x"], model["out_norm"], eps)
    assert_within(res["xf"], ref, norm_bound(ref, H), "final norm")
    y, tol = oracle.matvec(model["lm_head"], res["xf"])
    if "logits" in res:
        assert_parity(res["logits"], y, tol, "lm_head")
    assert oracle.argmax_accepted(res["token"], y, tol), "token"
    assert res["host_token"] == res["token"]


def check_untouched(res, model, pos):
    for l, L in enumerate(model["layers"]):
        for name in ("kc", "vc"):
            src = L["k_cache" if name == "kc" else "v_cache"]
            got = res[name][l]
            keep = np.ones(got.shape[0], dtype=bool)
            if 0 <= pos < got.shape[0]:
                keep[pos] = False
            assert np.array_equal(got[keep], src[keep]), f"layer {l} {name} rows besides pos"


QWEN1 = dict(gen.QWEN3_DIMS, n_layers=1)


@pytest.mark.parametrize("pos", [0, 1, 63, 64, 65, 300, 1023])
def test_one_layer_stages(cuda, pos):
    model = gen.decode_model(QWEN1, cache_rows=1024, seed=pos + 1)
    say(f"one Qwen3-shaped layer, pos {pos}, cache 1024 rows")
    dm = DeviceModel(model, cuda)
    try:
        res = dm.run(pos)
    finally:
        dm.close()
    check_stages(res, model, pos, x_in=model["x_in"])
    check_untouched(res, model, pos)


SMALL = [
    # (label, dims, cache rows, pos): G = 1, 2, 4 query heads per kv head,
    # a cache that is not a multiple of 64, the widest hidden (4096)
    ("g1", dict(n_layers=1, hidden=256, n_heads=2, n_kv_heads=2, head_dim=128, inter=512,
                vocab=300, eps=1e-6, theta=1e4), 100, 99),
    ("g2-ragged", dict(n_layers=1, hidden=256, n_heads=2, n_kv_heads=1, head_dim=128,
                       inter=512, vocab=300, eps=1e-5, theta=1e6), 100, 70),
    ("g4", dict(n_layers=1, hidden=512, n_heads=4, n_kv_heads=1, head_dim=128, inter=96,
                vocab=1000, eps=1e-6, theta=1e6), 200, 130),
    ("g3-odd", dict(n_layers=1, hidden=384, n_heads=3, n_kv_heads=1, head_dim=128, inter=160,
                    vocab=77, eps=1e-6, theta=5e5), 64, 63),
    ("wide", dict(n_layers=1, hidden=4096, n_heads=4, n_kv_heads=2, head_dim=128, inter=128,
                  vocab=500, eps=1e-6, theta=1e6), 130, 129),
    # long caches: the merge of the chunk partials takes two rounds (64
    # chunks per round for G <= 2, 32 for G = 3, 4), the second ragged
    ("g2-long", dict(n_layers=1, hidden=256, n_heads=2, n_kv_heads=1, head_dim=128,
                     inter=256, vocab=300, eps=1e-6, theta=1e6), 5000, 4700),
    ("g3-long", dict(n_layers=1, hidden=384, n_heads=3, n_kv_heads=1, head_dim=128,
                     inter=160, vocab=77, eps=1e-6, theta=5e5), 2200, 2100),
    ("g4-long", dict(n_layers=1, hidden=512, n_heads=4, n_kv_heads=2, head_dim=128,
                     inter=96, vocab=1000, eps=1e-6, theta=1e6), 2600, 2500),
]


@pytest.mark.parametrize("label,dims,rows,pos", SMALL, ids=[c[0] for c in SMALL])
def test_small_shapes(cuda, label, dims, rows, pos):
    model = gen.decode_model(dims, cache_rows=rows, seed=7)
    say(f"{label}: {dims}, cache {rows}, pos {pos}")
    dm = DeviceModel(model, cuda)
    try:
        res = dm.run(pos)
        res2 = dm.run(pos, kernel=True)
    finally:
        dm.close()
    check_stages(res, model, pos, x_in=model["x_in"])
    check_untouched(res, model, pos)
    for k in BUF_F32:
        if k in res:
            assert np.array_equal(res[k], res2[k], equal_nan=True), f"kernel launch: {k}"
    assert res2["token"] == res["token"]


def test_repeat_and_launch_kinds(cuda):
    """Two graph launches and one kernel launch at one position give
    bit-identical buffers (the step reads x_in, rewrites row pos with the same
    values); the host token equals the device token; a two-layer step checks
    the last layer's stages."""
    dims = dict(gen.QWEN3_DIMS, n_layers=2)
    model = gen.decode_model(dims, cache_rows=256, seed=3)
    dm = DeviceModel(model, cuda, logits=False)
    try:
        a = dm.run(200)
        b = dm.run(200)
        c = dm.run(200, kernel=True)
        k, mc = dm.graph.info()
    finally:
        dm.close()
    assert (k, mc) == (5 * 2 + 2, 0)
    for k_ in BUF_F32:
        if k_ in a:
            assert np.array_equal(a[k_], b[k_]) and np.array_equal(a[k_], c[k_]), k_
    for l in range(2):
        assert np.array_equal(a["kc"][l], c["kc"][l]) and np.array_equal(a["vc"][l], c["vc"][l])
    assert a["token"] == b["token"] == c["token"] == a["host_token"]
    check_stages(a, model, 200)
    check_untouched(a, model, 200)


def test_bad_position(cuda):
    """pos outside [0, cache_rows): no cache row written, attention NaN, token -1."""
    dims = dict(n_layers=1, hidden=256, n_heads=2, n_kv_heads=1, head_dim=128, inter=512,
                vocab=300, eps=1e-6, theta=1e6)
    model = gen.decode_model(dims, cache_rows=64, seed=9)
    dm = DeviceModel(model, cuda)
    try:
        for pos in (64, -1):
            res = dm.run(pos)
            assert np.isnan(res["attn"]).all()
            assert res["token"] == -1 and res["host_token"] == -1
            check_untouched(res, model, -5)
        res = dm.run(5)  # a good position still works afterwards
    finally:
        dm.close()
    check_stages(res, model, 5, x_in=model["x_in"])


def test_full_step_against_oracle(cuda):
    """The 28-layer Qwen3-shaped step at position 777 (cache 1024 rows) against
    the oracle's binary64 chain from the same inputs."""
    import torch
    dims = gen.QWEN3_DIMS
    pos = 777
    model = gen.decode_model(dims, cache_rows=1024, seed=11)
    say("full 28-layer step, pos 777")
    dm = DeviceModel(model, cuda)
    try:
        res = dm.run(pos)
    finally:
        dm.close()
        torch.cuda.empty_cache()
    check_stages(res, model, pos)
    check_untouched(res, model, pos)
    kcs = [L["k_cache"].astype(np.float64) for L in model["layers"]]
    vcs = [L["v_cache"].astype(np.float64) for L in model["layers"]]
    ref = oracle.decode_step(dict(dims=dims, layers=[oracle_layer(L) for L in model["layers"]],
                                  out_norm=model["out_norm"], lm_head=model["lm_head"]),
                             model["x_in"], pos, kcs, vcs)
    rel = np.linalg.norm(res["xf"] - ref["xf"]) / np.linalg.norm(ref["xf"])
    say(f"  end to end: |xf - ref| / |ref| = {rel:.3e}")
    assert rel <= 1e-3
    for l in range(dims["n_layers"]):
        r = np.linalg.norm(res["kc"][l][pos] - kcs[l][pos]) / np.linalg.norm(kcs[l][pos])
        assert r <= 1e-3, f"layer {l} appended key: {r:.3e}"
    # the token: logits of the GPU's xf differ from the exact ones by at most
    # |W| |xf_gpu - xf_ref| plus the matvec bar
    y_ref, tol = oracle.matvec_f64(model["lm_head"], ref["xf"])
    # |W| |dx| without forming W: a matvec of |W| (sign bits cleared) with |dx|
    w = model["lm_head"].reshape(dims["vocab"], -1, 34).copy()
    w[:, :, 1] &= 0x7F  # |scale|
    q = w[:, :, 2:].view(np.int8)
    assert not (q == -128).any()
    q[:] = np.abs(q)
    dense_abs, _ = oracle.matvec_f64(w.reshape(dims["vocab"], -1),
                                     np.abs(res["xf"].astype(np.float64) - ref["xf"]))
    slack = 1e-4 * tol + 1e-6 + dense_abs
    assert oracle.argmax_accepted(res["token"], y_ref, slack), "token"


# ---- the persistent form: one launch, a grid-wide barrier between phases ----

PERSIST = [
    # (label, dims, cache rows, pos): G = 1, 2, 3, 4; the widest shapes the
    # form takes (hidden and inter 3072); ragged and two-round merges
    ("p-g1", dict(n_layers=2, hidden=256, n_heads=2, n_kv_heads=2, head_dim=128, inter=512,
                  vocab=300, eps=1e-6, theta=1e4), 100, 99),
    ("p-g2-ragged", dict(n_layers=1, hidden=256, n_heads=2, n_kv_heads=1, head_dim=128,
                         inter=512, vocab=300, eps=1e-5, theta=1e6), 100, 70),
    ("p-g3", dict(n_layers=3, hidden=768, n_heads=6, n_kv_heads=2, head_dim=128, inter=512,
                  vocab=1000, eps=1e-6, theta=5e5), 200, 150),
    ("p-g4-long", dict(n_layers=1, hidden=512, n_heads=4, n_kv_heads=1, head_dim=128,
                       inter=256, vocab=1000, eps=1e-6, theta=1e6), 2600, 2500),
    ("p-g2-long", dict(n_layers=1, hidden=256, n_heads=2, n_kv_heads=1, head_dim=128,
                       inter=256, vocab=300, eps=1e-6, theta=1e6), 5000, 4700),
    ("p-widest", dict(n_layers=2, hidden=3072, n_heads=8, n_kv_heads=4, head_dim=128,
                      inter=3072, vocab=5000, eps=1e-6, theta=1e6), 130, 129),
]


def run_both(model, device, pos, logits=True, seq=()):
    """The node form's and the persistent form's results at one position,
    then (both forms) at each (position, input) of seq in order: launches
    that read other values than the launch before (a stale cached copy of
    the previous launch's activations would show as a difference)."""
    res = {}
    for form in (q8.Q8_DECODE_NODES, q8.Q8_DECODE_PERSISTENT):
        dm = DeviceModel(model, device, logits=logits, form=form)
        try:
            res[form] = dm.run(pos)
            if form == q8.Q8_DECODE_PERSISTENT:  # the same inputs (row pos rewritten alike)
                res["kernel"] = dm.run(pos, kernel=True)
                res["again"] = dm.run(pos)
                res["info"] = dm.graph.info()
            res[(form, "seq")] = [dm.run(p, x_in=x) for p, x in seq]
        finally:
            dm.close()
    for i, (a, b) in enumerate(zip(res[(q8.Q8_DECODE_NODES, "seq")],
                                   res[(q8.Q8_DECODE_PERSISTENT, "seq")])):
        assert_same(a, b, f"node form against persistent form, launch {i + 2}")
    return res[q8.Q8_DECODE_NODES], res[q8.Q8_DECODE_PERSISTENT], res


def assert_same(a, b, label):
    for k in BUF_F32:
        if k in a:
            assert np.array_equal(a[k], b[k], equal_nan=True), f"{label}: {k}"
    for l in range(len(a["kc"])):
        assert np.array_equal(a["kc"][l], b["kc"][l]), f"{label}: layer {l} key cache"
        assert np.array_equal(a["vc"][l], b["vc"][l]), f"{label}: layer {l} value cache"
    assert a["token"] == b["token"] and a["host_token"] == b["host_token"], label


@pytest.mark.parametrize("label,dims,rows,pos", PERSIST, ids=[c[0] for c in PERSIST])
def test_persistent_shapes(cuda, label, dims, rows, pos):
    """Each stage against the oracle; the node form's buffers bit for bit
    (every output row is computed by one workgroup in the same order in both
    forms, the attention rotation from the same binary32 angle); a kernel
    launch and a second graph launch the same again; one kernel node."""
    model = gen.decode_model(dims, cache_rows=rows, seed=17)
    say(f"persistent {label}: {dims}, cache {rows}, pos {pos}")
    x2 = np.ascontiguousarray(model["x_in"][::-1] * np.float32(0.5))
    seq = [(pos - 1, x2), (pos, x2), (pos - 1, model["x_in"])]
    nodes, pers, extra = run_both(model, cuda, pos, seq=seq)
    assert pers["token"] >= 0, f"token {pers['token']} (-2: the grid barrier gave up)"
    check_stages(pers, model, pos, x_in=model["x_in"] if dims["n_layers"] == 1 else None)
    check_untouched(pers, model, pos)
    assert_same(nodes, pers, "node form against persistent form")
    assert_same(pers, extra["kernel"], "kernel launch")
    assert_same(pers, extra["again"], "second graph launch")
    assert extra["info"] == (1, 0)


@pytest.mark.parametrize("pos", [0, 64, 1023])
def test_persistent_one_layer(cuda, pos):
    model = gen.decode_model(QWEN1, cache_rows=1024, seed=pos + 5)
    say(f"persistent, one Qwen3-shaped layer, pos {pos}")
    nodes, pers, _ = run_both(model, cuda, pos)
    check_stages(pers, model, pos, x_in=model["x_in"])
    check_untouched(pers, model, pos)
    assert_same(nodes, pers, "node form against persistent form")


def test_persistent_bad_position(cuda):
    """pos outside [0, cache_rows) in the persistent form: as the node form."""
    dims = dict(n_layers=2, hidden=256, n_heads=2, n_kv_heads=1, head_dim=128, inter=512,
                vocab=300, eps=1e-6, theta=1e6)
    model = gen.decode_model(dims, cache_rows=64, seed=9)
    dm = DeviceModel(model, cuda, form=q8.Q8_DECODE_PERSISTENT)
    try:
        for pos in (64, -1):
            res = dm.run(pos)
            assert np.isnan(res["attn"]).all()
            assert res["token"] == -1 and res["host_token"] == -1
            check_untouched(res, model, -5)
        res = dm.run(5)
    finally:
        dm.close()
    check_stages(res, model, 5)


def test_persistent_full_step(cuda):
    """The 28-layer Qwen3-shaped step at position 1023 (cache 1024 rows) in
    both forms: bit-identical buffers, and the last layer's stages against
    the oracle."""
    import torch
    pos = 1023
    model = gen.decode_model(gen.QWEN3_DIMS, cache_rows=1024, seed=23)
    say("persistent, full 28-layer step, pos 1023")
    try:
        nodes, pers, extra = run_both(model, cuda, pos, logits=False)
    finally:
        torch.cuda.empty_cache()
    assert_same(nodes, pers, "node form against persistent form")
    assert_same(pers, extra["kernel"], "kernel launch")
    check_stages(pers, model, pos)
    check_untouched(pers, model, pos)


def test_persistent_refuses_unstaged_shapes(cuda):
    """Widths the staged tiles do not take (inter 96) or wider than 3072:
    Q8_ERR_SHAPE for the persistent form; the node form still builds."""
    for dims in (dict(n_layers=1, hidden=512, n_heads=4, n_kv_heads=1, head_dim=128,
                      inter=96, vocab=100, eps=1e-6, theta=1e6),
                 dict(n_layers=1, hidden=4096, n_heads=4, n_kv_heads=2, head_dim=128,
                      inter=128, vocab=100, eps=1e-6, theta=1e6)):
        model = gen.decode_model(dims, cache_rows=64, seed=1)
        with pytest.raises(q8.Q8Error, match="shape"):
            DeviceModel(model, cuda, form=q8.Q8_DECODE_PERSISTENT)
        DeviceModel(model, cuda).close()
