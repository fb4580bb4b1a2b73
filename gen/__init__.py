"""Seeded synthetic inputs for the Q8_0 decode-matvec workloads.

A pure data source shared by the HIP path's tests and benchmark and by the
oracle's tests.  It holds none of the matvec's arithmetic: it only draws
weight bytes and activations (see ``q8_gen.c`` for the generator and the
distributions).  The shapes are those of a Qwen3-0.6B decode step, the model
the inferno.rs page ("IV.4: One command buffer per token") decodes: hidden
1024, query width 2048, key/value width 1024, MLP width 3072, vocabulary
151,936, 28 layers, seven projections per layer plus the lm_head.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q8_gen.c")
_LIB = os.path.join(_HERE, "libq8gen.so")
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-Wall"]

BLOCK = 32          # quants per Q8_0 block
BLOCK_BYTES = 34    # f16 scale + 32 int8 quants

ROLE_W = 1
ROLE_X = 2

# (name, n_in, p_out) of the seven projections of one layer, in model order.
LAYER_SHAPES = (
    ("q", 1024, 2048),
    ("k", 1024, 1024),
    ("v", 1024, 1024),
    ("o", 2048, 1024),
    ("gate", 1024, 3072),
    ("up", 1024, 3072),
    ("down", 3072, 1024),
)
N_LAYERS = 28
LM_HEAD = ("lm_head", 1024, 151936)


def step_shapes():
    """The 197 (name, n, p) matvecs of one decode step, in launch order."""
    out = []
    for layer in range(N_LAYERS):
        for name, n, p in LAYER_SHAPES:
            out.append((f"L{layer}.{name}", n, p))
    out.append(LM_HEAD)
    return out


def build(out: str = _LIB, cc: str = "gcc", extra=()) -> str:
    """Compile the generator (optionally elsewhere, with another compiler
    and extra flags: the sanitizer test builds an instrumented copy)."""
    subprocess.run([cc, *CFLAGS, *extra, _SRC, "-o", out, "-lm", "-lpthread"],
                   check=True)
    return out


_lib = None


def load(path: str = _LIB):
    """Loads the generator library (builds the default one if absent); a
    later call with another path is ignored once one is loaded."""
    return _load(path)


def _load(path: str = _LIB):
    global _lib
    if _lib is None:
        if path == _LIB and not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(path)
        u64, i64, u32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_uint32
        lib.q8g_stream_key.restype = u64
        lib.q8g_stream_key.argtypes = [u64, u32, u32, u32]
        lib.q8g_draw.restype = u64
        lib.q8g_draw.argtypes = [u64, u64]
        lib.q8g_f16_rne.restype = ctypes.c_uint16
        lib.q8g_f16_rne.argtypes = [ctypes.c_double]
        lib.q8g_blocks.restype = None
        lib.q8g_blocks.argtypes = [u64, i64, i64, ctypes.c_void_p, ctypes.c_int]
        lib.q8g_normals.restype = None
        lib.q8g_normals.argtypes = [u64, i64, i64, ctypes.c_void_p, ctypes.c_int]
        _lib = lib
    return _lib


def _threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return 1


def stream_key(seed: int, role: int, index: int, row: int = 0) -> int:
    return int(_load().q8g_stream_key(seed, role, index, row))


def draw(key: int, i: int) -> int:
    return int(_load().q8g_draw(key, i))


def f16_rne(v: float) -> int:
    """Bits of the binary16 nearest (ties to even) to the double v."""
    return int(_load().q8g_f16_rne(float(v)))


def blocks(key: int, first: int, count: int) -> np.ndarray:
    """Blocks first..first+count-1 of a weight stream, as uint8 [count, 34]."""
    out = np.empty((count, BLOCK_BYTES), dtype=np.uint8)
    if count:
        _load().q8g_blocks(key, first, count, out.ctypes.data, _threads())
    return out


def normals(key: int, first: int, count: int) -> np.ndarray:
    """Normals first..first+count-1 of a stream, as float32 [count]."""
    out = np.empty(count, dtype=np.float32)
    if count:
        _load().q8g_normals(key, first, count, out.ctypes.data, _threads())
    return out


def weights(p: int, n: int, seed: int = 0, index: int = 0) -> np.ndarray:
    """Q8_0 weight matrix of p rows and n columns as uint8 [p, n/32*34]."""
    if n % BLOCK:
        raise ValueError("n must be a multiple of 32")
    bpr = n // BLOCK
    key = stream_key(seed, ROLE_W, index)
    return blocks(key, 0, p * bpr).reshape(p, bpr * BLOCK_BYTES)


def activations(m: int, n: int, seed: int = 0, index: int = 0) -> np.ndarray:
    """m independent N(0,1) activation rows of length n, float32 [m, n]."""
    out = np.empty((m, n), dtype=np.float32)
    for r in range(m):
        out[r] = normals(stream_key(seed, ROLE_X, index, r), 0, n)
    return out


# ---- a whole synthetic decoder ------------------------------------------------

ROLE_MODEL = 3  # the decode model's weights, norms, caches and input row

# Qwen3-0.6B's shapes (the model the inferno.rs page decodes; its eps and
# RoPE base are the ones that model's configuration states).
QWEN3_DIMS = dict(n_layers=N_LAYERS, hidden=1024, n_heads=16, n_kv_heads=8, head_dim=128,
                  inter=3072, vocab=151936, eps=1e-6, theta=1e6)

DECODE_WEIGHTS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")


def decode_weight_shapes(dims: dict) -> dict:
    """(n_in, p_out) of each projection of a layer."""
    H, hd, inter = dims["hidden"], dims["head_dim"], dims["inter"]
    qw, kvw = dims["n_heads"] * hd, dims["n_kv_heads"] * hd
    return dict(wq=(H, qw), wk=(H, kvw), wv=(H, kvw), wo=(qw, H), w_gate=(H, inter),
                w_up=(H, inter), w_down=(inter, H))


def decode_model(dims: dict, cache_rows: int, seed: int = 0) -> dict:
    """Seeded synthetic decoder of the given shapes: per layer the seven Q8_0
    projections (generator weights), norm weights 1 + N(0, 0.1^2), a key
    cache of N(0, 1) rows and a value cache of N(0, 0.4^2) rows
    ([cache_rows, n_kv*head_dim], standing in for earlier tokens); the final
    norm, the lm_head, and an N(0, 1) input row x_in."""
    H, hd = dims["hidden"], dims["head_dim"]
    kvw = dims["n_kv_heads"] * hd
    shapes = decode_weight_shapes(dims)

    def nrm(index, count, sd=1.0, mean=0.0):
        v = normals(stream_key(seed, ROLE_MODEL, index), 0, count)
        return (mean + np.float32(sd) * v).astype(np.float32)
    layers = []
    for l in range(dims["n_layers"]):
        base = 64 * (l + 1)
        L = {}
        for j, name in enumerate(DECODE_WEIGHTS):
            n, p = shapes[name]
            L[name] = weights(p, n, seed=seed, index=base + j)
        L["attn_norm"] = nrm(base + 10, H, 0.1, 1.0)
        L["ffn_norm"] = nrm(base + 11, H, 0.1, 1.0)
        L["q_norm"] = nrm(base + 12, hd, 0.1, 1.0)
        L["k_norm"] = nrm(base + 13, hd, 0.1, 1.0)
        L["k_cache"] = nrm(base + 14, cache_rows * kvw).reshape(cache_rows, kvw)
        L["v_cache"] = nrm(base + 15, cache_rows * kvw, 0.4).reshape(cache_rows, kvw)
        layers.append(L)
    return dict(dims=dict(dims, cache_rows=cache_rows), layers=layers,
                out_norm=nrm(1, H, 0.1, 1.0),
                lm_head=weights(dims["vocab"], H, seed=seed, index=2),
                x_in=nrm(3, H))
