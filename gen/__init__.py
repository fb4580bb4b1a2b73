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


def build() -> None:
    subprocess.run(["gcc", *CFLAGS, _SRC, "-o", _LIB, "-lm", "-lpthread"],
                   check=True)


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
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
