"""Pins that tie the oracle to facts outside itself.

Each pin takes an ``oracle.Oracle`` and raises AssertionError when the oracle
disagrees with something the pages or the mathematics fix:
  * printed values (golden fixtures with citations),
  * the IEEE-754 binary16 format as decoded by numpy (an independent routine),
  * brute force: a dense binary64 dequantised matrix built with numpy and
    multiplied with numpy, on tiny inputs,
  * closed forms: all-ones x, one-hot x, a single nonzero quant,
    power-of-two scales with small-integer x (exact dyadic sums),
  * invariants: exact homogeneity in powers of two, odd symmetry, row
    permutation, batched == per-row, threaded == single-threaded,
  * the argmax rule: lowest index on ties, NaN skipped, -0 == +0.
The mutation tests compile deliberately broken copies of the oracle and
require every one of them to fail at least one pin.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

import gen
from tests import pagegen

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---- independent helpers (numpy, not the oracle) ---------------------------

def dense_dequant(w: np.ndarray, n: int) -> np.ndarray:
    """W as a dense float64 [p, n] matrix, decoded by numpy's float16."""
    p = w.shape[0]
    bpr = n // 32
    blk = np.ascontiguousarray(w).reshape(p, bpr, 34)
    scale = np.ascontiguousarray(blk[:, :, 0:2]).view("<f2")[..., 0]
    q = np.ascontiguousarray(blk[:, :, 2:]).view(np.int8)
    return (scale.astype(np.float64)[:, :, None] * q.astype(np.float64)).reshape(p, n)


def make_blocks(scale_bits: np.ndarray, quants: np.ndarray) -> np.ndarray:
    """Assemble uint8 [p, bpr*34] from scale bits [p, bpr] and int8 [p, bpr, 32]."""
    p, bpr = scale_bits.shape
    out = np.empty((p, bpr, 34), dtype=np.uint8)
    sb = scale_bits.astype(np.uint16)
    out[:, :, 0] = (sb & 0xFF).astype(np.uint8)
    out[:, :, 1] = (sb >> 8).astype(np.uint8)
    out[:, :, 2:] = quants.astype(np.int8).view(np.uint8)
    return out.reshape(p, bpr * 34)


def rich_case(p: int, n: int, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """Generator weights with planted extremes: -128 quants, subnormal, zero,
    negative and large scales."""
    w = gen.weights(p, n, seed=seed, index=seed)
    x = gen.activations(1, n, seed=seed, index=seed)[0]
    bpr = n // 32
    blk = w.reshape(p, bpr, 34)
    rng = np.random.default_rng(seed)
    specials = [0x0001, 0x03FF, 0x0000, 0x8000, 0xAC00, 0x7BFF, 0x0400, 0x8001]
    for i, bits in enumerate(specials):
        r, b = i % p, (i * 7) % bpr
        blk[r, b, 0] = bits & 0xFF
        blk[r, b, 1] = bits >> 8
    flat = blk[:, :, 2:].reshape(-1)
    idx = rng.choice(flat.size, size=max(1, flat.size // 50), replace=False)
    flat[idx] = 0x80  # int8 -128
    blk[:, :, 2:] = flat.reshape(p, bpr, 32)
    return blk.reshape(p, bpr * 34), x


def sum_bound(w: np.ndarray, x: np.ndarray) -> np.ndarray:
    """n * 2^-52 * sum|scale*q*x| per row: a rounding bound for any order."""
    d = np.abs(dense_dequant(w, x.size))
    return x.size * 2.0 ** -52 * (d @ np.abs(x.astype(np.float64))) + 1e-300


# ---- pins -------------------------------------------------------------------

def pin_f16_golden(orc):
    """Printed and format-defined binary16 values."""
    kv = pagegen.read_kv(os.path.join(GOLDEN, "f16_values.txt"))
    assert kv, "empty fixture"
    for key, vals in kv.items():
        bits = int(key, 16)
        want = float(vals[0][0])
        got = float(orc.half_to_double([bits])[0])
        if math.isnan(want):
            assert math.isnan(got), f"{key}: {got} != nan"
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), \
                f"{key}: {got!r} != {want!r}"


def pin_f16_exhaustive(orc):
    """All 65,536 binary16 patterns against numpy's own float16 decoder."""
    bits = np.arange(65536, dtype=np.uint16)
    got = orc.half_to_double(bits)
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), "NaN patterns differ"
    assert np.array_equal(got[~nan], want[~nan]), "values differ"
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan])), "signs differ"


def pin_bruteforce_dense(orc):
    """Tiny shapes vs a dense numpy float64 dequantised matmul."""
    for p, n, seed in [(1, 32, 1), (3, 96, 2), (50, 96, 3), (7, 128, 4),
                       (5, 1024, 5), (9, 64, 6)]:
        w, x = rich_case(p, n, seed)
        y, tol = orc.matvec(w, x)
        d = dense_dequant(w, n)
        ref = d @ x.astype(np.float64)
        bound = sum_bound(w, x)
        assert np.all(np.abs(y - ref) <= bound), f"p={p} n={n}: y differs"
        mag = np.abs(d) @ np.abs(x.astype(np.float64))
        want_tol = 1e-4 * mag + 1e-6
        assert np.allclose(tol, want_tol, rtol=1e-12, atol=0), f"p={p} n={n}: tol"


def pin_page_matvec_case(orc):
    """The page's matvec test inputs (p=50, n=96, seeds 7/42) vs brute force
    and the page's own 5e-4 absolute bound against a float32 sequential sum."""
    kv = pagegen.read_kv(os.path.join(GOLDEN, "page_matvec_case.txt"))
    p, n = int(kv["p"][0][0]), int(kv["n"][0][0])
    w = pagegen.fabricated_q8(p, n, int(kv["weight_seed"][0][0]),
                              int(kv["scale_bits"][0][0], 16))
    x = pagegen.lcg_f32(int(kv["x_seed"][0][0]), n)
    y, _ = orc.matvec(w, x)
    ref = dense_dequant(w, n) @ x.astype(np.float64)
    assert np.all(np.abs(y - ref) <= sum_bound(w, x))
    # the page's expected value: a sequential f32 sum with the scale inside
    blk = w.reshape(p, n // 32, 34)
    q = np.ascontiguousarray(blk[:, :, 2:]).view(np.int8).reshape(p, n)
    scale = np.float32(1.0 / 16.0)
    seq = np.zeros(p, dtype=np.float32)
    for c in range(n):
        seq = seq + scale * q[:, c].astype(np.float32) * x[c]
    assert np.max(np.abs(y - seq.astype(np.float64))) < float(kv["abs_tol"][0][0])


def pin_closed_form_ones(orc):
    """x = 1: y[r] = sum_b scale_b * sum_j q_bj, computed with exact rationals."""
    p, n = 6, 256
    w, _ = rich_case(p, n, 11)
    blk = w.reshape(p, n // 32, 34)
    scale = np.ascontiguousarray(blk[:, :, 0:2]).view("<f2")[..., 0]
    qsum = np.ascontiguousarray(blk[:, :, 2:]).view(np.int8).astype(np.int64).sum(axis=2)
    y, _ = orc.matvec(w, np.ones(n, dtype=np.float32))
    for r in range(p):
        exact = sum((Fraction(float(scale[r, b])) * int(qsum[r, b])
                     for b in range(n // 32)), Fraction(0))
        mag = sum((abs(Fraction(float(scale[r, b]))) * int(abs(qsum[r, b]))
                   for b in range(n // 32)), Fraction(0))
        assert abs(Fraction(float(y[r])) - exact) <= mag * Fraction(n, 2 ** 52), r


def pin_closed_form_one_hot(orc):
    """x = e_k: y[r] = scale[r, k/32] * q[r, k/32, k%32] exactly."""
    p, n = 5, 128
    w, _ = rich_case(p, n, 12)
    d = dense_dequant(w, n)
    for k in [0, 1, 31, 32, 33, 77, 127]:
        x = np.zeros(n, dtype=np.float32)
        x[k] = 1.0
        y, _ = orc.matvec(w, x)
        assert np.array_equal(y, d[:, k]), f"k={k}"


def pin_single_nonzero_quant(orc):
    """One nonzero weight isolates one term: y = scale*q*x[c] at its row only."""
    p, n = 4, 96
    x = gen.activations(1, n, seed=13, index=13)[0]
    for (r, c, qv, sbits) in [(0, 0, 5, 0x3C00), (3, 95, -128, 0x2C00),
                              (2, 40, 127, 0x0003), (1, 63, -1, 0xC200)]:
        quants = np.zeros((p, n // 32, 32), dtype=np.int8)
        quants[r, c // 32, c % 32] = qv
        sb = np.full((p, n // 32), sbits, dtype=np.uint16)
        w = make_blocks(sb, quants)
        y, _ = orc.matvec(w, x)
        s = float(np.array([sbits], dtype=np.uint16).view(np.float16)[0])
        want = np.zeros(p)
        want[r] = s * qv * float(x[c])
        assert np.array_equal(y, want), (r, c)


def pin_pow2_integer_exact(orc):
    """Power-of-two scales and small-integer x: every partial sum is an exact
    dyadic, so y equals the integer arithmetic exactly."""
    p, n = 8, 512
    rng = np.random.default_rng(14)
    quants = rng.integers(-128, 128, size=(p, n // 32, 32), dtype=np.int64)
    expo = rng.integers(-6, 3, size=(p, n // 32))
    sb = (15 + expo).astype(np.uint16) << 10  # 2^expo
    w = make_blocks(sb, quants)
    xi = rng.integers(-8, 9, size=n)
    y, _ = orc.matvec(w, xi.astype(np.float32))
    for r in range(p):
        exact = Fraction(0)
        for b in range(n // 32):
            dot = int(np.dot(quants[r, b], xi[32 * b:32 * b + 32]))
            exact += Fraction(2) ** int(expo[r, b]) * dot
        assert Fraction(float(y[r])) == exact, r


def pin_homogeneity_and_sign(orc):
    """y(2^k x) == 2^k y(x) and y(-x) == -y(x), bit for bit."""
    w, x = rich_case(7, 160, 15)
    y, _ = orc.matvec(w, x)
    for k in (-3, 1, 5):
        yk, _ = orc.matvec(w, (x * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(yk, y * 2.0 ** k), k
    yn, _ = orc.matvec(w, -x)
    assert np.array_equal(yn, -y)


def pin_row_permutation(orc):
    """Permuting weight rows permutes y (rows are independent)."""
    w, x = rich_case(9, 96, 16)
    y, _ = orc.matvec(w, x)
    perm = np.random.default_rng(16).permutation(9)
    yp, _ = orc.matvec(w[perm], x)
    assert np.array_equal(yp, y[perm])


def pin_batched_and_threads(orc):
    """Batched row i == single matvec on row i; threaded == single, bitwise."""
    p, n, m = 33, 256, 5
    w = gen.weights(p, n, seed=17, index=17)
    xs = gen.activations(m, n, seed=17, index=17)
    yb, tb = orc.matvec_batched(w, xs)
    for i in range(m):
        y, t = orc.matvec(w, xs[i])
        assert np.array_equal(yb[i], y) and np.array_equal(tb[i], t), i
    y, t = orc.matvec(w, xs[0])
    for threads in (1, 3, 8):
        ym, tm, used = orc.matvec_mt(w, xs[0], threads)
        assert used == threads
        assert np.array_equal(ym, y) and np.array_equal(tm, t), threads


def pin_tolerance_hand_case(orc):
    """tol = 1e-4 * sum|scale*q*x| + 1e-6 on a hand-worked block: scale 1,
    q = (1, -2, 0, ...), x = (3, 5, 7, ...) gives y = -7 and sum|t| = 13."""
    quants = np.zeros((1, 1, 32), dtype=np.int8)
    quants[0, 0, 0], quants[0, 0, 1] = 1, -2
    w = make_blocks(np.array([[0x3C00]], dtype=np.uint16), quants)
    x = np.arange(3, 3 + 2 * 32, 2).astype(np.float32)
    y, tol = orc.matvec(w, x)
    assert y[0] == -7.0
    assert abs(tol[0] - (1e-4 * 13 + 1e-6)) < 1e-18


def pin_argmax_page_tie(orc):
    """The page's argmax example: ties at 140011/140012 go to 140011."""
    kv = pagegen.read_kv(os.path.join(GOLDEN, "argmax_tie.txt"))
    n, seed = int(kv["n"][0][0]), int(kv["seed"][0][0])
    v = pagegen.lcg_f32(seed, n)
    for idx, val in kv["plant"]:
        v[int(idx)] = np.float32(float(val))
    want = int(kv["expect"][0][0])
    assert orc.argmax_f32(v) == want
    assert orc.argmax_f64(v.astype(np.float64)) == want


def pin_argmax_rules(orc):
    """Lowest index on ties; NaN never wins (even at index 0); -0 == +0."""
    nan, inf = float("nan"), float("inf")
    cases = [
        ([1.0, 3.0, 3.0, 2.0], 1),
        ([5.0, 1.0, 5.0], 0),
        ([1.0, 2.0, 9.0], 2),
        ([2.0, 2.0, 2.0, 2.0], 0),
        ([nan, 1.0, 0.5], 1),
        ([0.5, nan, 7.0, nan], 2),
        ([nan, nan], -1),
        ([], -1),
        ([-0.0, 0.0], 0),
        ([0.0, -0.0], 0),
        ([-1.0, -0.0, 0.0, -2.0], 1),
        ([-inf, -inf], 0),
        ([1.0, inf, inf], 1),
        ([nan, -inf], 1),
    ]
    for vals, want in cases:
        assert orc.argmax_f64(np.array(vals, dtype=np.float64)) == want, vals
        assert orc.argmax_f32(np.array(vals, dtype=np.float32)) == want, vals


# ---- int8-activation variant -----------------------------------------------

def _golden_q8x():
    d, rows = None, []
    for line in open(os.path.join(GOLDEN, "q8x_quantize.txt")):
        line = line.split("#")[0].split()
        if not line:
            continue
        if line[0] == "d":
            d = float(line[1])
        else:
            rows.append((int(line[0]), int(line[1])))
    return d, rows


def pin_q8x_quantize_golden(orc):
    """A block whose exact quantisation follows by hand: ties go to even."""
    d_want, rows = _golden_q8x()
    x = np.zeros(32, dtype=np.float32)
    for j, (k, _) in enumerate(rows):
        x[j] = k * 2.0 ** -7
    d, q = orc.quantize_x(x)
    assert float(d[0]) == d_want
    for j, (_, qw) in enumerate(rows):
        assert int(q[j]) == qw, (j, int(q[j]), qw)
    assert np.all(q[len(rows):] == 0)


def pin_q8x_quantize_properties(orc):
    """Every code lies within half a step of x/d, |q| <= 127, the largest |x|
    of a block maps to +-127, and d * 127 is amax to binary32 rounding."""
    rng = np.random.default_rng(21)
    for scale in (1.0, 1e-3, 1e4):
        x = (rng.standard_normal(32 * 40) * scale).astype(np.float32)
        x[::97] *= 50.0  # outliers
        d, q = orc.quantize_x(x)
        xb = x.reshape(-1, 32).astype(np.float64)
        qb = q.reshape(-1, 32).astype(np.float64)
        dd = d.astype(np.float64)[:, None]
        assert np.all(np.abs(qb) <= 127)
        assert np.all(np.abs(xb - dd * qb) <= dd * (0.5 + 1e-6))
        top = np.argmax(np.abs(xb), axis=1)
        assert np.all(np.abs(qb[np.arange(len(top)), top]) == 127)
        amax = np.abs(xb).max(axis=1)
        assert np.all(np.abs(dd[:, 0] * 127 - amax) <= amax * 2.0 ** -22)


def pin_q8x_quantize_special(orc):
    """A zero block quantises to d = 0, q = 0; a block holding a NaN or an
    infinity to d = NaN, q = 0, and its neighbours are unaffected."""
    x = np.ones(32 * 4, dtype=np.float32)
    x[32:64] = 0.0
    x[64 + 5] = np.nan
    x[96 + 31] = -np.inf
    d, q = orc.quantize_x(x)
    assert d[1] == 0.0 and np.all(q[32:64] == 0)
    assert np.isnan(d[2]) and np.all(q[64:96] == 0)
    assert np.isnan(d[3]) and np.all(q[96:] == 0)
    assert d[0] == np.float32(1.0) / np.float32(127.0) and np.all(q[:32] == 127)


def _dense_i8x(w, x, orc_quant):
    d, q = orc_quant
    xd = np.repeat(d.astype(np.float64), 32) * q.astype(np.float64)
    return dense_dequant(w, x.size) @ xd


def pin_q8x_bruteforce_dense(orc):
    """The int8-activation product against numpy: the dequantised weights
    times the dequantised activations, in binary64."""
    for p, n, seed in [(5, 64, 1), (7, 96, 2), (3, 256, 3)]:
        w, x = rich_case(p, n, seed)
        y, _ = orc.matvec_i8x(w, x)
        want = _dense_i8x(w, x, orc.quantize_x(x))
        assert np.allclose(y, want, rtol=1e-12, atol=1e-300), (p, n)


def pin_q8x_exact_on_grid(orc):
    """When x already sits on its quantisation grid (d = 2^-k, integer codes,
    one code of each block at 127) the quantisation is exact and the product
    equals the f32-activation oracle's."""
    rng = np.random.default_rng(5)
    p, n = 9, 128
    w, _ = rich_case(p, n, 5)
    codes = rng.integers(-127, 128, size=n)
    codes[::32] = 127
    expo = rng.integers(-9, -2, size=n // 32)
    x = (codes * np.repeat(2.0 ** expo, 32)).astype(np.float32)
    y, _ = orc.matvec_i8x(w, x)
    ref, _ = orc.matvec(w, x)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-300)


def pin_q8x_quantization_bound(orc):
    """|y_int8x - y_exact| <= sum_b |scale| * d/2 * sum_j |q_w|: the error
    quantising x may add, with y_exact from the f32-activation oracle."""
    for seed in (11, 12):
        w, x = rich_case(40, 512, seed)
        d, _ = orc.quantize_x(x)
        y, _ = orc.matvec_i8x(w, x)
        ref, _ = orc.matvec(w, x)
        blk = np.ascontiguousarray(w).reshape(40, 16, 34)
        scale = np.ascontiguousarray(blk[:, :, 0:2]).view("<f2")[..., 0].astype(np.float64)
        qabs = np.abs(np.ascontiguousarray(blk[:, :, 2:]).view(np.int8).astype(np.float64)).sum(axis=2)
        bound = (np.abs(scale) * (d.astype(np.float64) / 2)[None, :] * qabs).sum(axis=1)
        assert np.all(np.abs(y - ref) <= bound * (1 + 1e-9) + 1e-12)


def pin_q8x_tolerance_hand_case(orc):
    """One block by hand: scale 1, weight codes 1 and -2, activation codes
    127 and 127 (x = 1 and 1), so y = d*(127 - 254), tolerance
    1e-4 * d * 381 + 1e-6 with d = 1/127 in binary32."""
    w = make_blocks(np.array([[0x3C00]]), np.array([[[1, -2] + [0] * 30]]))
    x = np.zeros(32, dtype=np.float32)
    x[0] = x[1] = 1.0
    y, tol = orc.matvec_i8x(w, x)
    d = float(np.float32(1.0) / np.float32(127.0))
    assert y[0] == d * (127 - 254)
    assert abs(tol[0] - (1e-4 * d * 381 + 1e-6)) <= 1e-18


# ---- the rest of the decode step ----------------------------------------------

def selector(p: int, n: int, col) -> np.ndarray:
    """Q8_0 rows that pick one input: row r has scale 1.0 and quant 1 at
    column col(r), zero elsewhere (zero scales on the other blocks)."""
    bpr = n // 32
    bits = np.zeros((p, bpr), dtype=np.uint16)
    q = np.zeros((p, bpr, 32), dtype=np.int8)
    for r in range(p):
        c = col(r)
        bits[r, c // 32] = 0x3C00
        q[r, c // 32, c % 32] = 1
    return make_blocks(bits, q)


def zero_q8(p: int, n: int) -> np.ndarray:
    return np.zeros((p, n // 32 * 34), dtype=np.uint8)


def np_rms(x, w, eps):
    """rms_norm_row with numpy, rows of the last axis."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def np_silu_mul(g, u):
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g)) * u


TINY = dict(hidden=64, n_heads=4, n_kv_heads=2, head_dim=16, inter=96,
            eps=1e-6, theta=10000.0)


def tiny_layer(rng, **over):
    """A layer of the tiny shapes: random weights unless replaced."""
    H, hd, inter = TINY["hidden"], TINY["head_dim"], TINY["inter"]
    qw, kvw = TINY["n_heads"] * hd, TINY["n_kv_heads"] * hd

    def rnd(p, n):
        bits = np.full((p, n // 32), 0x2000, dtype=np.uint16)  # 2^-7
        q = rng.integers(-127, 128, size=(p, n // 32, 32)).astype(np.int8)
        return make_blocks(bits, q)
    layer = dict(wq=rnd(qw, H), wk=rnd(kvw, H), wv=rnd(kvw, H), wo=rnd(H, qw),
                 wg=rnd(inter, H), wu=rnd(inter, H), wd=rnd(H, inter),
                 attn_norm=rng.uniform(0.5, 1.5, H), q_norm=rng.uniform(0.5, 1.5, hd),
                 k_norm=rng.uniform(0.5, 1.5, hd), ffn_norm=rng.uniform(0.5, 1.5, H))
    layer.update(over)
    return layer


def pin_rms_norm_closed_forms(orc):
    """rms_norm_row: (3, 4) with eps 0 is (3, 4)/sqrt(12.5); a constant row
    c with eps e is c/sqrt(c^2 + e) times the weight; with eps 0 and unit
    weight the mean square of the output is 1; scaling x by 8 changes
    nothing (exact in binary64); rows are independent; the weight is applied
    element-wise."""
    out = orc.rms_norm(np.array([3.0, 4.0]), np.ones(2), 0.0)
    assert np.allclose(out, [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=1e-15, atol=0)
    w = np.arange(1.0, 9.0)
    out = orc.rms_norm(np.full(8, 2.0), w, 0.5)
    assert np.allclose(out, 2.0 / math.sqrt(4.5) * w, rtol=1e-15, atol=0)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, 128))
    out = orc.rms_norm(x, np.ones(128), 0.0)
    assert np.allclose(np.mean(out * out, axis=1), 1.0, rtol=1e-13, atol=0)
    assert np.array_equal(orc.rms_norm(8.0 * x, np.ones(128), 0.0), out)
    for r in range(3):
        assert np.array_equal(orc.rms_norm(x[r], np.ones(128), 0.0), out[r])
    e = np.zeros(128)
    e[17] = 5.0
    o2 = orc.rms_norm(x[0], e, 1e-6)
    assert np.count_nonzero(o2) == 1 and o2[17] != 0.0
    assert np.allclose(orc.rms_norm(x, np.ones(128), 1e-6), np_rms(x, 1.0, 1e-6),
                       rtol=1e-13, atol=0)


def pin_rope_closed_forms(orc):
    """rope_row: pair 0 turns by exactly pos radians (its frequency is 1);
    pair i's angle at position 1 is theta^(-i/half) to binary32 accuracy;
    position 0 is the identity; a unit vector on element 0 goes to
    (cos pos, sin pos) on elements 0 and half, one on element half to
    (-sin pos, cos pos); every pair keeps its length; every head turns the
    same way; pair 0's dot products depend only on the difference of the
    positions."""
    for pos in (0, 1, 7, 513, 4095):
        assert orc.rope_angle(pos, 0, 64, 1e6) == np.float32(pos)
    for i in range(64):
        a = float(orc.rope_angle(1, i, 64, 1e6))
        ref = 1e6 ** (-i / 64)
        assert abs(a - ref) <= 2 * 2.0 ** -23 * ref
    rng = np.random.default_rng(5)
    x = rng.standard_normal(3 * 8)
    assert np.array_equal(orc.rope(x, 8, 0, 1e4), x)
    for pos in (1, 3, 100):
        e0 = np.zeros(8)
        e0[0] = 1.0
        out = orc.rope(e0, 8, pos, 1e4)
        ref = np.zeros(8)
        ref[0], ref[4] = math.cos(pos), math.sin(pos)
        assert np.allclose(out, ref, rtol=0, atol=1e-15)
        e4 = np.zeros(8)
        e4[4] = 1.0
        out = orc.rope(e4, 8, pos, 1e4)
        ref = np.zeros(8)
        ref[0], ref[4] = -math.sin(pos), math.cos(pos)
        assert np.allclose(out, ref, rtol=0, atol=1e-15)
        e1 = np.zeros(8)
        e1[1] = 1.0
        out = orc.rope(e1, 8, pos, 1e4)
        ang = float(np.float32(pos) * (np.float32(1.0) / np.float32(1e4 ** 0.25)))
        ref = np.zeros(8)
        ref[1], ref[5] = math.cos(ang), math.sin(ang)
        assert np.allclose(out, ref, rtol=0, atol=1e-15)
    out = orc.rope(x, 8, 37, 1e4).reshape(3, 8)
    xr = x.reshape(3, 8)
    assert np.allclose(np.hypot(out[:, :4], out[:, 4:]), np.hypot(xr[:, :4], xr[:, 4:]),
                       rtol=1e-14, atol=0)
    same = orc.rope(np.concatenate([xr[0], xr[0]]), 8, 37, 1e4).reshape(2, 8)
    assert np.array_equal(same[0], same[1]) and np.array_equal(same[0], out[0])
    q, k = rng.standard_normal(8), rng.standard_normal(8)

    def dot0(a, b):
        return a[0] * b[0] + a[4] * b[4]
    d1 = dot0(orc.rope(q, 8, 5, 1e4), orc.rope(k, 8, 3, 1e4))
    d2 = dot0(orc.rope(q, 8, 2, 1e4), orc.rope(k, 8, 0, 1e4))
    assert abs(d1 - d2) <= 1e-13


def pin_attention_closed_forms(orc):
    """attention_decode (4 query heads, 2 key/value heads of width 4): one
    cached row gives that row's values; equal keys give the mean of the
    values; query head h reads key/value head h // 2; two rows with scores
    s/2 and 0 (the 1/sqrt(4) scale) weigh the first by 1/(1 + e^(-s/2));
    scores of +-1000 (beyond exp's binary64 range) stay finite and pick the top row; permuting the cached
    rows changes nothing; the weights sum to one."""
    rng = np.random.default_rng(11)
    H, KV, hd = 4, 2, 4
    kvw = KV * hd
    q = rng.standard_normal(H * hd)
    kc = rng.standard_normal((5, kvw))
    vc = rng.standard_normal((5, kvw))
    out, pr = orc.attention(q, kc, vc, 1, H, KV, hd)
    for h in range(H):
        assert np.array_equal(out[h * hd:(h + 1) * hd], vc[0, (h // 2) * hd:(h // 2 + 1) * hd])
    kce = np.tile(kc[:1], (5, 1))
    out, pr = orc.attention(q, kce, vc, 5, H, KV, hd)
    for h in range(H):
        g = h // 2
        assert np.allclose(out[h * hd:(h + 1) * hd], vc[:, g * hd:(g + 1) * hd].mean(axis=0),
                           rtol=1e-13, atol=1e-15)
    vcg = np.empty_like(vc)
    vcg[:, :hd], vcg[:, hd:] = 1.0, 2.0
    out, pr = orc.attention(q, kc, vcg, 5, H, KV, hd)
    assert np.allclose(out, np.repeat([1.0, 1.0, 2.0, 2.0], hd), rtol=1e-14, atol=0)
    assert np.allclose(pr.sum(axis=1), 1.0, rtol=1e-14, atol=0)
    s = 3.0
    q2 = np.zeros(H * hd)
    q2[0] = s
    k2 = np.zeros((2, kvw))
    k2[0, 0] = 1.0
    v2 = np.zeros((2, kvw))
    v2[0, :] = 1.0
    out, pr = orc.attention(q2, k2, v2, 2, H, KV, hd)
    p0 = 1.0 / (1.0 + math.exp(-s / 2))
    assert abs(out[0] - p0) <= 1e-15 and abs(pr[0, 0] - p0) <= 1e-15
    q3 = np.zeros(H * hd)
    q3[0] = 2000.0
    k3 = np.zeros((3, kvw))
    k3[0, 0], k3[1, 0], k3[2, 0] = 1.0, -1.0, 0.5
    v3 = np.arange(3 * kvw, dtype=np.float64).reshape(3, kvw)
    out, pr = orc.attention(q3, k3, v3, 3, H, KV, hd)
    assert np.all(np.isfinite(out))
    assert np.allclose(out[:hd], v3[0, :hd], rtol=1e-15, atol=1e-100)
    perm = [3, 0, 4, 1, 2]
    o1, _ = orc.attention(q, kc, vc, 5, H, KV, hd)
    o2, _ = orc.attention(q, kc[perm], vc[perm], 5, H, KV, hd)
    assert np.allclose(o1, o2, rtol=1e-13, atol=1e-15)


def pin_silu_closed_forms(orc):
    """silu_hadamard: silu(0) = 0; silu(1) = 1/(1 + e^-1); silu(-1000) = -0;
    silu(40) = 40 to binary64 rounding; the up factor multiplies."""
    out = orc.silu_mul([0.0, 1.0, -1000.0, 40.0, 2.0, 1.0], [5.0, 1.0, 1.0, 1.0, 3.0, 2.0])
    assert out[0] == 0.0
    assert abs(out[1] - 0.7310585786300049) <= 1e-16
    assert out[2] == 0.0 and math.copysign(1.0, out[2]) == -1.0
    assert abs(out[3] - 40.0) <= 40.0 * 2.0 ** -52 * 4
    assert abs(out[4] - 6.0 / (1.0 + math.exp(-2.0))) <= 1e-15
    assert abs(out[5] - 2.0 * 0.7310585786300049) <= 2e-16


def pin_matvec_f64_is_matvec(orc):
    """With binary32-representable activations the binary64-activation matvec
    gives the pinned matvec's values and magnitudes, bit for bit."""
    w, x = rich_case(40, 256, seed=21)
    y, tol = orc.matvec(w, x)
    y2, mag = orc.matvec_f64(w, x.astype(np.float64))
    assert np.array_equal(y, y2)
    assert np.array_equal(tol, 1e-4 * mag + 1e-6)


def _tiny_run(orc, layer, x, pos, kc, vc):
    kc, vc = kc.copy(), vc.copy()
    xo, acts = orc.decode_layer(TINY, layer, x, kc, vc, pos)
    return xo, acts, kc, vc


def pin_decode_layer_attention_branch(orc):
    """A layer whose value and o projections pick inputs one to one and whose
    MLP is zero: at position 0 attention returns the value row, so x gains
    xn[kv slice of the head]; the cache receives v = xn[:32] and the QK-normed
    key (RoPE is the identity at 0).  With a zero query projection at
    position 3 every score is 0, so attention is the mean of the 3 cached
    value rows and the appended one: the step attends over pos + 1 rows and
    appends at row pos; the appended key is RoPE(QK-norm(k)) at 3."""
    rng = np.random.default_rng(17)
    H, hd = TINY["hidden"], TINY["head_dim"]
    qw, kvw, inter = 4 * hd, 2 * hd, TINY["inter"]
    eps = TINY["eps"]
    layer = tiny_layer(rng, wv=selector(kvw, H, lambda r: r), wo=selector(H, qw, lambda r: r),
                       wg=zero_q8(inter, H), wu=zero_q8(inter, H), wd=zero_q8(H, inter))
    x = rng.standard_normal(H)
    kc0 = rng.standard_normal((8, kvw))
    vc0 = rng.standard_normal((8, kvw))
    xo, acts, kc, vc = _tiny_run(orc, layer, x, 0, kc0, vc0)
    xn = np_rms(x, layer["attn_norm"], eps)
    gidx = np.array([((r // hd) // 2) * hd + r % hd for r in range(H)])
    assert np.allclose(xo, x + xn[gidx], rtol=1e-14, atol=1e-15)
    assert np.allclose(vc[0], xn[:kvw], rtol=1e-15, atol=0)
    k = dense_dequant(layer["wk"], H) @ xn
    kn = np_rms(k.reshape(2, hd), layer["k_norm"], eps).ravel()
    assert np.allclose(kc[0], kn, rtol=1e-12, atol=1e-14)
    assert np.array_equal(kc[1:], kc0[1:]) and np.array_equal(vc[1:], vc0[1:])
    layer["wq"] = zero_q8(qw, H)
    xo, acts, kc, vc = _tiny_run(orc, layer, x, 3, kc0, vc0)
    vmean = (vc0[:3].sum(axis=0) + xn[:kvw]) / 4.0
    assert np.allclose(xo, x + vmean[gidx], rtol=1e-13, atol=1e-14)
    assert np.allclose(kc[3], orc.rope(kn, hd, 3, TINY["theta"]), rtol=1e-12, atol=1e-14)
    assert np.array_equal(kc[4:], kc0[4:]) and np.array_equal(kc[:3], kc0[:3])


def pin_decode_layer_mlp_branch(orc):
    """A layer whose o projection is zero and whose gate/up pick xn2[r % 64]
    and down picks h[r]: x gains silu(xn2) * xn2, with xn2 the ffn-normed x."""
    rng = np.random.default_rng(19)
    H, hd = TINY["hidden"], TINY["head_dim"]
    qw, inter = 4 * hd, TINY["inter"]
    layer = tiny_layer(rng, wo=zero_q8(H, qw), wg=selector(inter, H, lambda r: r % H),
                       wu=selector(inter, H, lambda r: r % H),
                       wd=selector(H, inter, lambda r: r))
    x = rng.standard_normal(H)
    kc0 = rng.standard_normal((4, 2 * hd))
    xo, acts, _, _ = _tiny_run(orc, layer, x, 1, kc0, kc0)
    xn2 = np_rms(x, layer["ffn_norm"], TINY["eps"])
    assert np.allclose(xo, x + np_silu_mul(xn2, xn2), rtol=1e-14, atol=1e-15)
    assert np.allclose(acts["h"][:H], np_silu_mul(xn2, xn2), rtol=1e-14, atol=1e-15)


def pin_decode_step_head(orc):
    """Two layers with zero o and down projections leave x unchanged, so the
    step's logits are the lm_head applied to out_norm(x) (dense numpy product)
    and its token is their argmax."""
    rng = np.random.default_rng(23)
    H, hd, inter = TINY["hidden"], TINY["head_dim"], TINY["inter"]
    layers = [tiny_layer(rng, wo=zero_q8(H, 4 * hd), wd=zero_q8(H, inter)) for _ in range(2)]
    vocab = 50
    lm = gen.weights(vocab, H, seed=5, index=1)
    model = dict(dims=dict(TINY, vocab=vocab), layers=layers,
                 out_norm=rng.uniform(0.5, 1.5, H), lm_head=lm)
    x = rng.standard_normal(H)
    kcs = [rng.standard_normal((4, 2 * hd)) for _ in range(2)]
    vcs = [rng.standard_normal((4, 2 * hd)) for _ in range(2)]
    r = orc.decode_step(model, x, 2, kcs, vcs)
    assert np.array_equal(r["x"], x)
    xf = np_rms(x, model["out_norm"], TINY["eps"])
    assert np.allclose(r["xf"], xf, rtol=1e-14, atol=0)
    ref = dense_dequant(lm, H) @ xf
    assert np.allclose(r["logits"], ref, rtol=1e-12, atol=1e-14)
    assert r["token"] == int(np.argmax(ref))


ALL_PINS = [
    pin_f16_golden,
    pin_f16_exhaustive,
    pin_bruteforce_dense,
    pin_page_matvec_case,
    pin_closed_form_ones,
    pin_closed_form_one_hot,
    pin_single_nonzero_quant,
    pin_pow2_integer_exact,
    pin_homogeneity_and_sign,
    pin_row_permutation,
    pin_batched_and_threads,
    pin_tolerance_hand_case,
    pin_argmax_page_tie,
    pin_argmax_rules,
    pin_q8x_quantize_golden,
    pin_q8x_quantize_properties,
    pin_q8x_quantize_special,
    pin_q8x_bruteforce_dense,
    pin_q8x_exact_on_grid,
    pin_q8x_quantization_bound,
    pin_q8x_tolerance_hand_case,
    pin_rms_norm_closed_forms,
    pin_rope_closed_forms,
    pin_attention_closed_forms,
    pin_silu_closed_forms,
    pin_matvec_f64_is_matvec,
    pin_decode_layer_attention_branch,
    pin_decode_layer_mlp_branch,
    pin_decode_step_head,
]


# ---- the parity bar (oracle.matvec_errors, oracle.argmax_accepted) ----------
#
# These two helpers turn the oracle's values into pass/fail for every GPU
# test, so a slip in them would loosen every parity claim at once.  The
# pins below are hand cases whose answers follow from the bar's definition
# (inferno.rs "IV.4", "The correctness ladder": an assert_close bar per
# output and the tie rule of the argmax; the bound itself is
# |err| <= 1e-4 * sum|scale*q*x| + 1e-6 per output, and an argmax is correct
# when it is the oracle's index or the two logits lie within the sum of
# their bounds).  All values are dyadic, so every comparison is exact.
# Each pin takes the module that holds the two helpers.

def bar_pin_matvec_errors(bar):
    """err = |y - y_ref| / tol, exactly 1 at the bound and above it past it;
    equal values (infinities included) and NaN against NaN are 0; NaN
    against a number, or a finite value against an infinity, is inf."""
    nan, inf = float("nan"), float("inf")
    eps = 2.0 ** -40
    y_ref = np.array([1.0, 1.0, 1.0, -2.0, 0.0, inf, -inf, nan, nan, 3.0, inf, 5.0,
                      1.0, 1.0])
    tol = np.array([0.25, 0.25, 0.25, 0.5, 0.125, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0,
                    0.25, 4.0])
    y = np.array([1.0, 1.25, 1.25 + eps, -2.5, -0.0625, inf, -inf, nan, 1.0, nan, 7.0,
                  -inf, 0.75, 9.0])
    want = np.array([0.0, 1.0, 1.0 + eps / 0.25, 1.0, 0.5, 0.0, 0.0, 0.0, inf, inf, inf,
                     inf, 1.0, 2.0])
    got = bar.matvec_errors(y, y_ref, tol)
    assert got.shape == y.shape
    assert np.array_equal(got, want), (got, want)
    assert got[1] <= 1.0 and got[2] > 1.0  # at the bound passes, just past it fails
    assert got[12] <= 1.0 and bar.matvec_errors([0.75 - eps], [1.0], [0.25])[0] > 1.0
    # per-output tolerance: each output is divided by its own bound
    got2 = bar.matvec_errors([2.0, 2.0], [1.0, 1.0], [1.0, 0.5])
    assert np.array_equal(got2, [1.0, 2.0]), got2
    # +inf against -inf, and a sign error, fail
    assert bar.matvec_errors([inf], [-inf], [1.0])[0] == inf
    assert bar.matvec_errors([-1.0], [1.0], [1.0])[0] == 2.0
    # batched shapes keep their layout
    g3 = bar.matvec_errors(np.ones((2, 3)), np.zeros((2, 3)), np.full((2, 3), 0.5))
    assert g3.shape == (2, 3) and np.all(g3 == 2.0)


def bar_pin_argmax_accepted(bar):
    """The oracle's index is always accepted; another index only when its
    logit lies within tol[best] + tol[g] of the best (the sum of the two
    bounds, not one of them, not twice it); -1, out-of-range indices and
    NaN logits never."""
    nan = float("nan")
    eps = 2.0 ** -40
    y = np.array([0.5, 1.0, 0.75, 0.75 - eps, 0.875])
    tol = np.array([0.0, 0.0625, 0.1875, 0.1875, 0.0])
    assert bar.argmax_accepted(1, y, tol)                 # the oracle's index
    assert bar.argmax_accepted(2, y, tol)                 # 0.25 == 0.0625 + 0.1875
    assert not bar.argmax_accepted(3, y, tol)             # just outside the band
    assert not bar.argmax_accepted(0, y, tol)             # far outside
    # index 4 lies within tol[best] = 0.0625 * 2 but not within tol[best] + tol[4]
    assert not bar.argmax_accepted(4, y, tol)
    # asymmetric bounds: only their sum accepts index 2 (0.25 = 0.0625 + 0.1875)
    y2 = np.array([1.0, 0.75])
    assert bar.argmax_accepted(1, y2, np.array([0.0625, 0.1875]))
    assert bar.argmax_accepted(1, y2, np.array([0.1875, 0.0625]))
    assert not bar.argmax_accepted(1, y2, np.array([0.0625, 0.0625]))
    assert not bar.argmax_accepted(1, y2, np.array([0.0, 0.125]))
    # -1 and out of range: rejected even when the wrapped index would be close
    y3 = np.array([0.0, 1.0, 1.0 - eps])
    t3 = np.array([0.5, 0.5, 0.5])
    assert bar.argmax_accepted(2, y3, t3)
    assert not bar.argmax_accepted(-1, y3, t3)
    assert not bar.argmax_accepted(3, y3, t3)
    assert not bar.argmax_accepted(-2, y3, t3)
    # NaN logits: never the answer; all-NaN rows accept exactly -1
    y4 = np.array([nan, 1.0, 0.999])
    t4 = np.array([1.0, 0.5, 0.5])
    assert bar.argmax_accepted(1, y4, t4)
    assert not bar.argmax_accepted(0, y4, t4)
    yn = np.array([nan, nan])
    assert bar.argmax_accepted(-1, yn, np.ones(2))
    assert not bar.argmax_accepted(0, yn, np.ones(2))
    # ties: the lowest index is the oracle's, the other one is in the band
    y5 = np.array([2.0, 2.0])
    assert bar.argmax_accepted(0, y5, np.zeros(2))
    assert bar.argmax_accepted(1, y5, np.zeros(2))


BAR_PINS = [bar_pin_matvec_errors, bar_pin_argmax_accepted]
