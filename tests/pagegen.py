"""Inputs of the worked examples printed on the inferno.rs page.

inferno.rs "IV.4: One command buffer per token", "The correctness ladder":
the kernel tests draw from a 64-bit linear congruential generator
(state <- state * 6364136223846793005 + 1442695040888963407 mod 2^64) and map
each state to the f32 value (state >> 33) / 2^31 - 1.  Because state >> 33 is
below 2^31 the values lie in [-1, 0]; the weight fabricator stores the scale
bits 0x2C00 and the quant (int8)(value * 127), truncated toward zero.  These
helpers restate that generator so the page's examples can be rebuilt here.
"""
from __future__ import annotations

import numpy as np

_MUL = 6364136223846793005
_INC = 1442695040888963407
_MASK = (1 << 64) - 1


def lcg_f32(seed: int, count: int) -> np.ndarray:
    """`count` successive values of the page's test generator, as float32."""
    state = seed & _MASK
    hi = np.empty(count, dtype=np.float64)
    for i in range(count):
        state = (state * _MUL + _INC) & _MASK
        hi[i] = state >> 33
    # u32 -> f32 rounds to nearest; /2^31 is exact; the -1 is an f32 add.
    return (hi.astype(np.float32) / np.float32(2.0 ** 31)) - np.float32(1.0)


def fabricated_q8(rows: int, cols: int, seed: int,
                  scale_bits: int = 0x2C00) -> np.ndarray:
    """The page's Q8 weight fabricator: uint8 [rows, cols/32*34]."""
    bpr = cols // 32
    vals = lcg_f32(seed, rows * bpr * 32).reshape(rows, bpr, 32)
    q = np.trunc(vals * np.float32(127.0)).astype(np.int8)  # f32 product
    out = np.empty((rows, bpr, 34), dtype=np.uint8)
    out[:, :, 0] = scale_bits & 0xFF
    out[:, :, 1] = scale_bits >> 8
    out[:, :, 2:] = q.view(np.uint8)
    return out.reshape(rows, bpr * 34)


def read_kv(path: str) -> dict:
    """Parse a golden fixture: '#' comments, then 'key value...' lines."""
    out: dict = {}
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            out.setdefault(key, []).append(vals)
    return out
