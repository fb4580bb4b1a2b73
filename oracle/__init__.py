"""CPU oracle for the Q8_0 decode matvec -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (``libq8dec``) never
does, and the two share no code.  The arithmetic lives in ``q8_oracle.c``
(plain C11, binary64, no fast-math); this module only marshals numpy arrays.

Parity bar (the acceptance rule these helpers implement):
  * every output:  |y_gpu - y_ref| <= 1e-4 * sum|scale*q*x| + 1e-6;
  * argmax: the GPU index g is accepted when it equals the oracle's index i*,
    or when y_ref[i*] - y_ref[g] <= tol[i*] + tol[g] (the two logits lie
    within the bound, so either index is a correct answer).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q8_oracle.c")
_LIB = os.path.join(_HERE, "libq8oracle.so")
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
          "-shared", "-Wall"]

REL_TOL = 1e-4
ABS_TOL = 1e-6


def build(src: str = _SRC, out: str = _LIB, cc: str = "gcc", extra=()) -> str:
    """Compile the oracle (optionally another source, for mutation tests, or
    with another compiler and extra flags, for the sanitizer test)."""
    subprocess.run([cc, *CFLAGS, *extra, src, "-o", out, "-lm", "-lpthread"],
                   check=True)
    return out


def _bind(lib):
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.q8o_half_to_double.restype = ctypes.c_double
    lib.q8o_half_to_double.argtypes = [ctypes.c_uint16]
    lib.q8o_matvec.restype = None
    lib.q8o_matvec.argtypes = [vp, vp, i64, i64, vp, vp]
    lib.q8o_matvec_batched.restype = None
    lib.q8o_matvec_batched.argtypes = [vp, vp, i64, i64, i64, vp, vp]
    lib.q8o_matvec_mt.restype = ctypes.c_int
    lib.q8o_matvec_mt.argtypes = [vp, vp, i64, i64, vp, vp, ctypes.c_int]
    lib.q8o_argmax_f64.restype = i64
    lib.q8o_argmax_f64.argtypes = [vp, i64]
    lib.q8o_argmax_f32.restype = i64
    lib.q8o_argmax_f32.argtypes = [vp, i64]
    lib.q8o_quantize_x.argtypes = [vp, i64, vp, vp]
    lib.q8o_quantize_x.restype = None
    lib.q8o_matvec_i8x.argtypes = [vp, vp, vp, i64, i64, vp, vp]
    lib.q8o_matvec_i8x.restype = None
    lib.q8o_matvec_f64.argtypes = [vp, vp, i64, i64, vp, vp]
    lib.q8o_matvec_f64.restype = None
    lib.q8o_rms_norm.argtypes = [vp, vp, vp, i64, i64, ctypes.c_double]
    lib.q8o_rms_norm.restype = None
    lib.q8o_rope_angle.argtypes = [i64, i64, i64, ctypes.c_float]
    lib.q8o_rope_angle.restype = ctypes.c_float
    lib.q8o_rope.argtypes = [vp, i64, i64, i64, ctypes.c_float]
    lib.q8o_rope.restype = None
    lib.q8o_attention.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64]
    lib.q8o_attention.restype = None
    lib.q8o_silu_mul.argtypes = [vp, vp, vp, i64]
    lib.q8o_silu_mul.restype = None
    lib.q8o_decode_layer.argtypes = [vp, vp, vp, vp, vp, i64, vp]
    lib.q8o_decode_layer.restype = None
    return lib


class _Dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int64), ("n_heads", ctypes.c_int64),
                ("n_kv_heads", ctypes.c_int64), ("head_dim", ctypes.c_int64),
                ("inter", ctypes.c_int64), ("eps", ctypes.c_double),
                ("theta", ctypes.c_float)]


class _Layer(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in
                ("wq", "wk", "wv", "wo", "wg", "wu", "wd",
                 "attn_norm", "q_norm", "k_norm", "ffn_norm")]


ACT_NAMES = ("xn", "q", "k", "v", "attn", "attn_out", "xn2", "gate", "up", "h",
             "ffn_out")


class _Acts(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in ACT_NAMES]


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: str):
        self.lib = _bind(ctypes.CDLL(path))

    def half_to_double(self, bits) -> np.ndarray:
        bits = np.asarray(bits, dtype=np.uint16).ravel()
        f = self.lib.q8o_half_to_double
        return np.array([f(int(b)) for b in bits], dtype=np.float64)

    @staticmethod
    def _check_w(w: np.ndarray, n: int, p: int | None) -> tuple[np.ndarray, int]:
        """Weights as uint8 [p, n/32*34]; p from the first axis if not given."""
        if n % 32:
            raise ValueError("n must be a multiple of 32")
        w = np.ascontiguousarray(w, dtype=np.uint8)
        if p is None:
            p = w.shape[0]
        if w.size != p * (n // 32) * 34:
            raise ValueError("weight bytes do not match (p, n)")
        return w, p

    def matvec(self, w: np.ndarray, x: np.ndarray, p: int | None = None):
        """y, tol (float64 [p]) for w = p rows of Q8_0 blocks and x[n]."""
        x = np.ascontiguousarray(x, dtype=np.float32).ravel()
        n = x.size
        w, p = self._check_w(w, n, p)
        y = np.empty(p, dtype=np.float64)
        tol = np.empty(p, dtype=np.float64)
        self.lib.q8o_matvec(w.ctypes.data, x.ctypes.data, n, p, y.ctypes.data,
                            tol.ctypes.data)
        return y, tol

    def matvec_batched(self, w: np.ndarray, x: np.ndarray, p: int | None = None):
        """y, tol (float64 [m, p]) for x [m, n]."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        m, n = x.shape
        w, p = self._check_w(w, n, p)
        y = np.empty((m, p), dtype=np.float64)
        tol = np.empty((m, p), dtype=np.float64)
        self.lib.q8o_matvec_batched(w.ctypes.data, x.ctypes.data, m, n, p,
                                    y.ctypes.data, tol.ctypes.data)
        return y, tol

    def matvec_mt(self, w: np.ndarray, x: np.ndarray, threads: int):
        """Row-parallel matvec; returns y, tol and the thread count used."""
        x = np.ascontiguousarray(x, dtype=np.float32).ravel()
        n = x.size
        w, p = self._check_w(w, n, None)
        y = np.empty(p, dtype=np.float64)
        tol = np.empty(p, dtype=np.float64)
        used = self.lib.q8o_matvec_mt(w.ctypes.data, x.ctypes.data, n, p,
                                      y.ctypes.data, tol.ctypes.data, threads)
        return y, tol, used

    def quantize_x(self, x: np.ndarray):
        """Q8_0 activation blocks of x[n]: d (float32 [n/32]), q (int8 [n])."""
        x = np.ascontiguousarray(x, dtype=np.float32).ravel()
        n = x.size
        if n % 32:
            raise ValueError("n must be a multiple of 32")
        d = np.empty(n // 32, dtype=np.float32)
        q = np.empty(n, dtype=np.int8)
        self.lib.q8o_quantize_x(x.ctypes.data, n, d.ctypes.data, q.ctypes.data)
        return d, q

    def matvec_i8x(self, w: np.ndarray, x: np.ndarray, p: int | None = None):
        """y, tol (float64 [m, p]) of the int8-activation product, x [m, n]
        (or [n]: then [p]); each x row is quantised by quantize_x."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        flat = x.ndim == 1
        x2 = x.reshape(1, -1) if flat else x
        m, n = x2.shape
        w, p = self._check_w(w, n, p)
        y = np.empty((m, p), dtype=np.float64)
        tol = np.empty((m, p), dtype=np.float64)
        for i in range(m):
            d, q = self.quantize_x(x2[i])
            self.lib.q8o_matvec_i8x(w.ctypes.data, d.ctypes.data, q.ctypes.data, n, p,
                                    y[i].ctypes.data, tol[i].ctypes.data)
        return (y[0], tol[0]) if flat else (y, tol)

    # ---- the rest of the decode step (binary64) ---------------------------

    def matvec_f64(self, w: np.ndarray, x, p: int | None = None):
        """y and mag = sum|scale*q*x| (float64 [p]) for binary64 x[n]."""
        x = _f64(x).ravel()
        n = x.size
        w, p = self._check_w(w, n, p)
        y = np.empty(p, dtype=np.float64)
        mag = np.empty(p, dtype=np.float64)
        self.lib.q8o_matvec_f64(w.ctypes.data, x.ctypes.data, n, p, y.ctypes.data,
                                mag.ctypes.data)
        return y, mag

    def rms_norm(self, x, w, eps: float):
        """rms_norm_row over the rows of x ([rows, dim] or [dim])."""
        x = _f64(x)
        dim = x.shape[-1]
        w = _f64(w).ravel()
        if w.size != dim:
            raise ValueError("norm weight length must equal dim")
        out = np.empty_like(x)
        self.lib.q8o_rms_norm(x.ctypes.data, w.ctypes.data, out.ctypes.data,
                              x.size // dim if dim else 0, dim, float(eps))
        return out

    def rope_angle(self, pos: int, i: int, half: int, theta: float) -> np.float32:
        return np.float32(self.lib.q8o_rope_angle(pos, i, half, float(theta)))

    def rope(self, x, head_dim: int, pos: int, theta: float):
        """rope_row over every head of x (heads * head_dim values)."""
        out = _f64(x).copy()
        self.lib.q8o_rope(out.ctypes.data, out.size // head_dim, head_dim, pos,
                          float(theta))
        return out

    def attention(self, q, kc, vc, seq: int, n_heads: int, n_kv_heads: int,
                  head_dim: int):
        """attention_decode: out [n_heads*head_dim] and the softmax weights
        [n_heads, seq]; kc, vc are [>= seq, n_kv_heads*head_dim]."""
        q = _f64(q).ravel()
        kvw = n_kv_heads * head_dim
        kc = _f64(kc).reshape(-1, kvw)
        vc = _f64(vc).reshape(-1, kvw)
        if kc.shape[0] < seq or vc.shape[0] < seq or q.size != n_heads * head_dim:
            raise ValueError("attention shapes")
        out = np.empty(n_heads * head_dim, dtype=np.float64)
        probs = np.empty((n_heads, max(seq, 0)), dtype=np.float64)
        self.lib.q8o_attention(q.ctypes.data, kc.ctypes.data, vc.ctypes.data,
                               out.ctypes.data, probs.ctypes.data, seq, kvw, head_dim,
                               n_heads // n_kv_heads, n_heads)
        return out, probs

    def silu_mul(self, g, u):
        g = _f64(g).ravel()
        u = _f64(u).ravel()
        out = np.empty_like(g)
        self.lib.q8o_silu_mul(g.ctypes.data, u.ctypes.data, out.ctypes.data, g.size)
        return out

    def decode_layer(self, dims: dict, layer: dict, x, kc, vc, pos: int):
        """One decode layer at position pos: returns (x after the layer, the
        layer's intermediates); kc and vc (float64 [rows, kv_width], C order)
        receive row pos in place."""
        d = _Dims(dims["hidden"], dims["n_heads"], dims["n_kv_heads"],
                  dims["head_dim"], dims["inter"], float(dims["eps"]),
                  float(dims["theta"]))
        keep = {}
        for k in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
            keep[k] = np.ascontiguousarray(layer[k], dtype=np.uint8)
        for k in ("attn_norm", "q_norm", "k_norm", "ffn_norm"):
            keep[k] = _f64(layer[k]).ravel()
        L = _Layer(*[keep[k].ctypes.data for k, _ in _Layer._fields_])
        H, hd = dims["hidden"], dims["head_dim"]
        qw, kvw, inter = dims["n_heads"] * hd, dims["n_kv_heads"] * hd, dims["inter"]
        sizes = dict(xn=H, q=qw, k=kvw, v=kvw, attn=qw, attn_out=H, xn2=H,
                     gate=inter, up=inter, h=inter, ffn_out=H)
        acts = {k: np.zeros(sizes[k], dtype=np.float64) for k in ACT_NAMES}
        A = _Acts(*[acts[k].ctypes.data for k in ACT_NAMES])
        x = _f64(x).ravel().copy()
        for c in (kc, vc):
            if c.dtype != np.float64 or not c.flags.c_contiguous or c.shape[1] != kvw \
                    or c.shape[0] <= pos:
                raise ValueError("caches must be float64 C-ordered [> pos, kv_width]")
        self.lib.q8o_decode_layer(ctypes.byref(d), ctypes.byref(L), x.ctypes.data,
                                  kc.ctypes.data, vc.ctypes.data, pos, ctypes.byref(A))
        return x, acts

    def decode_step(self, model: dict, x_in, pos: int, kcaches, vcaches):
        """The whole step at position pos: every layer in order, the final
        norm, the lm_head and its argmax.  kcaches/vcaches: one float64
        [rows, kv_width] array per layer, updated in place.  Returns a dict
        with x (after the last layer), xf (its norm), logits, mag (sum of
        |terms| per logit), token and the last layer's intermediates."""
        dims = model["dims"]
        x = _f64(x_in).ravel().copy()
        acts = None
        for li, layer in enumerate(model["layers"]):
            x, acts = self.decode_layer(dims, layer, x, kcaches[li], vcaches[li], pos)
        xf = self.rms_norm(x, model["out_norm"], dims["eps"])
        logits, mag = self.matvec_f64(model["lm_head"], xf)
        return dict(x=x, xf=xf, logits=logits, mag=mag, token=self.argmax_f64(logits),
                    acts=acts)

    def argmax_f64(self, v) -> int:
        v = np.ascontiguousarray(v, dtype=np.float64).ravel()
        return int(self.lib.q8o_argmax_f64(v.ctypes.data, v.size))

    def argmax_f32(self, v) -> int:
        v = np.ascontiguousarray(v, dtype=np.float32).ravel()
        return int(self.lib.q8o_argmax_f32(v.ctypes.data, v.size))


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from ``q8_oracle.c`` (compiled on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB):
            build()
        _default = Oracle(_LIB)
    return _default


def matvec(w, x, p=None):
    return get().matvec(w, x, p)


def matvec_batched(w, x, p=None):
    return get().matvec_batched(w, x, p)


def quantize_x(x):
    return get().quantize_x(x)


def matvec_i8x(w, x, p=None):
    return get().matvec_i8x(w, x, p)


def argmax_f64(v) -> int:
    return get().argmax_f64(v)


def matvec_f64(w, x, p=None):
    return get().matvec_f64(w, x, p)


def rms_norm(x, w, eps):
    return get().rms_norm(x, w, eps)


def rope_angle(pos, i, half, theta):
    return get().rope_angle(pos, i, half, theta)


def rope(x, head_dim, pos, theta):
    return get().rope(x, head_dim, pos, theta)


def attention(q, kc, vc, seq, n_heads, n_kv_heads, head_dim):
    return get().attention(q, kc, vc, seq, n_heads, n_kv_heads, head_dim)


def silu_mul(g, u):
    return get().silu_mul(g, u)


def decode_layer(dims, layer, x, kc, vc, pos):
    return get().decode_layer(dims, layer, x, kc, vc, pos)


def decode_step(model, x_in, pos, kcaches, vcaches):
    return get().decode_step(model, x_in, pos, kcaches, vcaches)


def argmax_f32(v) -> int:
    return get().argmax_f32(v)


# ---- the parity bar --------------------------------------------------------

def matvec_errors(y_gpu, y_ref, tol) -> np.ndarray:
    """|y_gpu - y_ref| / tol per output (<= 1 passes).

    Equal values (infinities included) and NaN against NaN count as zero
    error; any other NaN fails."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    err = np.abs(y_gpu - y_ref) / np.asarray(tol, dtype=np.float64)
    same = (np.isnan(y_gpu) & np.isnan(y_ref)) | (y_gpu == y_ref)
    err[same] = 0.0
    err[np.isnan(err)] = np.inf
    return err


def argmax_accepted(g: int, y_ref, tol) -> bool:
    """True when index g is a correct argmax of the exact logits y_ref."""
    y_ref = np.asarray(y_ref, dtype=np.float64)
    tol = np.asarray(tol, dtype=np.float64)
    best = argmax_f64(y_ref)
    if g == best:
        return True
    if best < 0 or g < 0 or g >= y_ref.size or np.isnan(y_ref[g]):
        return False
    return bool(y_ref[best] - y_ref[g] <= tol[best] + tol[g])
