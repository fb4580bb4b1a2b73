"""Mutation tests: a plausible mistake planted in a copy of the oracle (on the
CPU, never on the GPU path) must make at least one pin fail.  This is what
shows the pins are strong enough to trust the oracle."""
import os

import pytest

import oracle
from tests.oracle_pins import ALL_PINS

MUTANTS = [
    ("scale dropped",
     "double t = scale * q * (double)x[32 * b + j];",
     "double t = q * (double)x[32 * b + j];"),
    ("quant read unsigned",
     "(double)(int8_t)blk[2 + j]", "(double)blk[2 + j]"),
    ("quant offset off by one",
     "(int8_t)blk[2 + j]", "(int8_t)blk[1 + j]"),
    ("x index rotated",
     "x[32 * b + j]", "x[32 * b + (j + 1) % 32]"),
    ("block stride 32 bytes",
     "row + (size_t)b * 34u", "row + (size_t)b * 32u"),
    ("row stride 32 bytes per block",
     "(size_t)r * (size_t)blocks * 34u", "(size_t)r * (size_t)blocks * 32u"),
    ("scale bytes big-endian",
     "(blk[0] | (blk[1] << 8))", "(blk[1] | (blk[0] << 8))"),
    ("exponent bias off by one",
     "expo - 25", "expo - 24"),
    ("subnormal decoded as normal",
     "v = ldexp((double)frac, -24);", "v = ldexp((double)(1024 + frac), -25);"),
    ("hidden bit dropped",
     "ldexp((double)(1024 + frac), expo - 25)", "ldexp((double)(frac), expo - 25)"),
    ("sign bit ignored",
     "return sign ? -v : v;", "return v;"),
    ("product rounded to f32",
     "double t = scale * q * (double)x[32 * b + j];",
     "double t = (float)(scale * q) * x[32 * b + j];"),
    ("row sum in f32",
     "double sum = 0.0, mag = 0.0;", "float sum = 0.0f; double mag = 0.0;"),
    ("last block skipped",
     "for (int64_t b = 0; b < blocks; b++)", "for (int64_t b = 0; b + 1 < blocks; b++)"),
    ("tolerance uses signed terms",
     "mag += fabs(t);", "mag += t;"),
    ("tolerance constant",
     "1e-4 * mag + 1e-6", "1e-3 * mag + 1e-6"),
    ("argmax ties to the higher index",
     "v[i] > bv", "v[i] >= bv"),
    ("argmax keeps NaN",
     "if (isnan(v[i])) continue;", ""),
    ("argmax never updates the best value",
     "bv = v[i];", ""),
    ("activation codes truncated",
     "rintf(xb[j] * inv)", "truncf(xb[j] * inv)"),
    ("activation codes rounded half away from zero",
     "rintf(xb[j] * inv)", "roundf(xb[j] * inv)"),
    ("activation step amax / 128",
     "amax / 127.0f", "amax / 128.0f"),
    ("non-finite activations quantised",
     "if (!isfinite(a)) bad = 1;\n      else if (a > amax) amax = a;",
     "if (a > amax) amax = a;"),
    ("activation step dropped from the product",
     " * (double)d[b];", ";"),
    ("activation codes read unsigned",
     "(int64_t)q[32 * b + j]", "(int64_t)(uint8_t)q[32 * b + j]"),
    ("int8-activation tolerance uses signed products",
     "iabs += prod < 0 ? -prod : prod;", "iabs += prod;"),
    ("rms eps outside the root",
     "sqrt(ss / (double)dim + eps)", "(sqrt(ss / (double)dim) + eps)"),
    ("rms mean over dim - 1",
     "ss / (double)dim", "ss / (double)(dim - 1)"),
    ("rms weight dropped",
     "out[r * dim + i] = xr[i] * inv * w[i];", "out[r * dim + i] = xr[i] * inv;"),
    ("rope rotates the wrong way",
     "xh[i] = a * c - b * s;", "xh[i] = a * c + b * s;"),
    ("rope second element sign",
     "xh[i + half] = a * s + b * c;", "xh[i + half] = b * c - a * s;"),
    ("rope frequency exponent over head_dim",
     "(float)i / (float)half", "(float)i / (float)(2 * half)"),
    ("rope pairs adjacent elements",
     "const double a = xh[i], b = xh[i + half];", "const double a = xh[i], b = xh[(i + 1) % half];"),
    ("attention without the scale",
     "sc[t] = d * scale;", "sc[t] = d;"),
    ("attention scaled by head_dim",
     "1.0 / sqrt((double)head_dim)", "1.0 / (double)head_dim"),
    ("attention kv head by modulo",
     "(h / kv_group) * head_dim", "(h % kv_group) * head_dim"),
    ("attention without the max",
     "sc[t] = exp(sc[t] - mx);", "sc[t] = exp(sc[t]);"),
    ("attention not normalised",
     "for (int64_t t = 0; t < seq; t++) sc[t] /= sum;", ""),
    ("attention over pos rows",
     "a->attn, 0, pos + 1,", "a->attn, 0, pos,"),
    ("silu of the negated gate",
     "exp(-g[i])", "exp(g[i])"),
    ("silu without the up factor",
     "(1.0 + exp(-g[i])) * u[i];", "(1.0 + exp(-g[i]));"),
    ("attention residual replaces x",
     "x[i] += a->attn_out[i];", "x[i] = a->attn_out[i];"),
    ("mlp residual dropped",
     "x[i] += a->ffn_out[i];", "x[i] += 0.0 * a->ffn_out[i];"),
    ("ffn norm with the attention weight",
     "L->ffn_norm, a->xn2", "L->attn_norm, a->xn2"),
    ("k norm with the q weight",
     "L->k_norm, a->k", "L->q_norm, a->k"),
    ("rope skipped on k",
     "q8o_rope(a->k, dm->n_kv_heads, hd, pos, dm->theta);", ""),
    ("value cache gets the key",
     "vc[pos * kvw + i] = a->v[i];", "vc[pos * kvw + i] = a->k[i];"),
    ("mlp reads the attention norm output",
     "q8o_matvec_f64(L->wg, a->xn2,", "q8o_matvec_f64(L->wg, a->xn,"),
    ("f64 matvec drops the scale",
     "double t = scale * (double)(int8_t)blk[2 + j] * x[32 * b + j];",
     "double t = (double)(int8_t)blk[2 + j] * x[32 * b + j];"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_fails_a_pin(tmp_path, name, old, new):
    with open(oracle._SRC) as f:
        src = f.read()
    assert old in src, f"mutation site for '{name}' no longer in the oracle"
    src_path = tmp_path / "mutant.c"
    src_path.write_text(src.replace(old, new))
    lib = oracle.build(str(src_path), str(tmp_path / "libmutant.so"))
    orc = oracle.Oracle(lib)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except Exception:  # a wrong value, or a NaN where none belongs
            failed.append(pin.__name__)
    assert failed, f"mutant '{name}' passed every pin"
