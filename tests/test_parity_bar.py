"""The parity bar itself (oracle.matvec_errors, oracle.argmax_accepted)
against hand cases, and mutants of it that each must fail one (CPU only).

A mutant is a copy of oracle/__init__.py with one plausible slip planted,
loaded as a module of its own; its C library is the real oracle's."""
import importlib.util

import numpy as np
import pytest

import oracle
from tests.oracle_pins import BAR_PINS


@pytest.mark.parametrize("pin", BAR_PINS, ids=[p.__name__ for p in BAR_PINS])
def test_bar_pin(pin):
    with np.errstate(invalid="ignore"):
        pin(oracle)


BAR_MUTANTS = [
    ("error divided by twice the bound",
     "err = np.abs(y_gpu - y_ref) / np.asarray(tol, dtype=np.float64)",
     "err = np.abs(y_gpu - y_ref) / (2.0 * np.asarray(tol, dtype=np.float64))"),
    ("bound dropped from the error",
     "err = np.abs(y_gpu - y_ref) / np.asarray(tol, dtype=np.float64)",
     "err = np.abs(y_gpu - y_ref) + 0.0 * np.asarray(tol, dtype=np.float64)"),
    ("signed error",
     "err = np.abs(y_gpu - y_ref) /", "err = (y_gpu - y_ref) /"),
    ("NaN error mapped to zero",
     "err[np.isnan(err)] = np.inf", "err[np.isnan(err)] = 0.0"),
    ("NaN against NaN fails",
     "same = (np.isnan(y_gpu) & np.isnan(y_ref)) | (y_gpu == y_ref)",
     "same = (y_gpu == y_ref)"),
    ("NaN against anything passes",
     "same = (np.isnan(y_gpu) & np.isnan(y_ref)) | (y_gpu == y_ref)",
     "same = (np.isnan(y_gpu) | np.isnan(y_ref)) | (y_gpu == y_ref)"),
    ("equal infinities fail",
     "same = (np.isnan(y_gpu) & np.isnan(y_ref)) | (y_gpu == y_ref)",
     "same = (np.isnan(y_gpu) & np.isnan(y_ref))"),
    ("bound reversed per output",
     "/ np.asarray(tol, dtype=np.float64)", "/ np.asarray(tol, dtype=np.float64)[::-1]"),
    ("argmax band strict",
     "return bool(y_ref[best] - y_ref[g] <= tol[best] + tol[g])",
     "return bool(y_ref[best] - y_ref[g] < tol[best] + tol[g])"),
    ("argmax band of the best only",
     "return bool(y_ref[best] - y_ref[g] <= tol[best] + tol[g])",
     "return bool(y_ref[best] - y_ref[g] <= tol[best])"),
    ("argmax band of g only",
     "return bool(y_ref[best] - y_ref[g] <= tol[best] + tol[g])",
     "return bool(y_ref[best] - y_ref[g] <= tol[g])"),
    ("argmax band doubled",
     "return bool(y_ref[best] - y_ref[g] <= tol[best] + tol[g])",
     "return bool(y_ref[best] - y_ref[g] <= 2.0 * (tol[best] + tol[g]))"),
    ("argmax band on absolute difference",
     "return bool(y_ref[best] - y_ref[g] <= tol[best] + tol[g])",
     "return bool(abs(y_ref[best] - y_ref[g]) <= 2.0 * tol[g] + tol[best])"),
    ("argmax accepts -1",
     "if best < 0 or g < 0 or g >= y_ref.size", "if best < 0 or g >= y_ref.size"),
    ("argmax accepts negative indices that wrap",
     "if best < 0 or g < 0 or g >= y_ref.size", "if best < 0 or g < -1 or g >= y_ref.size"),
    ("argmax accepts any index on an all-NaN row",
     "if g == best:\n        return True", "if g == best or best < 0:\n        return True"),
    ("argmax accepts everything",
     "if g == best:\n        return True", "if True:\n        return True"),
]


def _load_mutant(tmp_path, old, new):
    with open(oracle.__file__) as f:
        src = f.read()
    assert old in src, f"mutation site no longer in the oracle: {old!r}"
    path = tmp_path / "oracle_mutant.py"
    path.write_text(src.replace(old, new, 1))
    spec = importlib.util.spec_from_file_location("oracle_mutant", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod._default = oracle.get()  # the real C library behind the mutated helpers
    return mod


@pytest.mark.parametrize("name,old,new", BAR_MUTANTS, ids=[m[0] for m in BAR_MUTANTS])
def test_bar_mutant_fails_a_pin(tmp_path, name, old, new):
    mod = _load_mutant(tmp_path, old, new)
    failed = []
    for pin in BAR_PINS:
        try:
            with np.errstate(invalid="ignore"):
                pin(mod)
        except Exception:  # a wrong verdict, or an index error on a bad g
            failed.append(pin.__name__)
    assert failed, f"mutant '{name}' passed every parity-bar pin"
