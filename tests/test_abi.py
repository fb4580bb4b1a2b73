"""The C ABI on the CPU: the library loads, exports every function that
include/q8dec.h declares, names its status codes, and refuses bad arguments
before any GPU work.  Every call here carries an invalid argument, so it can
never reach a kernel launch, with or without a device."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import q8_block_quantized_amd as q8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, NULL, SHAPE, ALIGN, NODEV = 0, 1, 2, 3, 4
BAD_HANDLE, COUNT, MODE = 9, 10, 11

# fake device addresses: aligned, never dereferenced (each call below fails
# validation first)
W, X, Y, I = 0x10000, 0x20000, 0x30000, 0x40000


@pytest.fixture(scope="module")
def lib():
    return q8.load()


def declared_functions():
    with open(q8.HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q8_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) >= 12
    for name in names:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", q8.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (q8_[a-z0-9_]+)", out))
    assert set(names) <= exported


def test_bench_helper_exports_its_header():
    """libq8bench.so (the benchmark's read-stream helper) exports every
    function include/q8bench.h declares, and refuses bad arguments before
    launching anything."""
    path = os.path.join(ROOT, "q8_block_quantized_amd", "libq8bench.so")
    with open(os.path.join(ROOT, "include", "q8bench.h")) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(q8bench_[a-z0-9_]+)\s*\(", text)))
    assert names == ["q8bench_read_stream"]
    out = subprocess.run(["nm", "-D", "--defined-only", path],
                         capture_output=True, text=True, check=True).stdout
    assert set(names) <= set(re.findall(r"\bT (q8bench_[a-z0-9_]+)", out))
    b = ctypes.CDLL(path)
    b.q8bench_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    assert b.q8bench_read_stream(None, 16, X, 1, 4, None) == 1
    assert b.q8bench_read_stream(W, 16, None, 1, 4, None) == 1
    assert b.q8bench_read_stream(W, 17, X, 1, 4, None) == 2
    assert b.q8bench_read_stream(W + 4, 16, X, 1, 4, None) == 2
    assert b.q8bench_read_stream(W, 16, X, 0, 4, None) == 2
    assert b.q8bench_read_stream(W, 16, X, 1, 5, None) == 2


def test_status_names(lib):
    want = {0: "q8_ok", 1: "q8_err_null", 2: "q8_err_shape", 3: "q8_err_align",
            4: "q8_err_no_device", 5: "q8_err_arch", 6: "q8_err_code_object",
            7: "q8_err_hip", 8: "q8_err_graph", 9: "q8_err_bad_handle",
            10: "q8_err_count", 11: "q8_err_mode", 12: "q8_err_levels"}
    for code, name in want.items():
        assert q8.q8_status_name(code) == name
    for code in (-1, 13, 99, 1 << 30):
        assert q8.q8_status_name(code) == "q8_code_out_of_range"


@pytest.mark.parametrize("args,want", [
    ((None, X, Y, 32, 1), NULL),
    ((W, None, Y, 32, 1), NULL),
    ((W, X, None, 32, 1), NULL),
    ((W, X, Y, 33, 1), SHAPE),
    ((W, X, Y, -32, 1), SHAPE),
    ((W, X, Y, 65536 + 32, 1), SHAPE),
    ((W, X, Y, 32, -1), SHAPE),
    ((W + 2, X, Y, 32, 1), ALIGN),
    ((W + 8, X, Y, 32, 1), ALIGN),
    ((W, X + 4, Y, 32, 1), ALIGN),
    ((W, X, Y + 2, 32, 1), ALIGN),
])
def test_matvec_refusals(lib, args, want):
    assert lib.q8_matvec(*args, None) == want


@pytest.mark.parametrize("m,n,p,want", [
    (0, 32, 1, SHAPE), (33, 256, 1, SHAPE), (-1, 32, 1, SHAPE),
    (2, 31, 1, SHAPE), (2, 32, -5, SHAPE),
    # more than 8 rows: n a positive multiple of 256
    (9, 32, 1, SHAPE), (9, 0, 1, SHAPE), (32, 1000, 1, SHAPE), (16, 288, 4, SHAPE),
])
def test_batched_refusals(lib, m, n, p, want):
    assert lib.q8_matvec_batched(W, X, Y, m, n, p, None) == want


def test_argmax_refusals(lib):
    assert lib.q8_argmax(X, 1, 0, I, None) == SHAPE
    assert lib.q8_argmax(X, 0, 5, I, None) == SHAPE
    assert lib.q8_argmax(X, 33, 5, I, None) == SHAPE
    assert lib.q8_argmax(None, 1, 5, I, None) == NULL
    assert lib.q8_argmax(X, 1, 5, None, None) == NULL
    assert lib.q8_argmax(X + 2, 1, 5, I, None) == ALIGN
    assert lib.q8_argmax(X, 1, 5, I + 1, None) == ALIGN


def test_matvec_argmax_refusals(lib):
    assert lib.q8_matvec_argmax(W, X, None, None, 1, 32, 4, None) == NULL
    assert lib.q8_matvec_argmax(W, X, None, I, 1, 32, 0, None) == SHAPE
    assert lib.q8_matvec_argmax(W, X, None, I, 33, 256, 4, None) == SHAPE
    assert lib.q8_matvec_argmax(W, X, None, I, 9, 32, 4, None) == SHAPE
    assert lib.q8_matvec_argmax(None, X, None, I, 1, 32, 4, None) == NULL
    assert lib.q8_matvec_argmax(W, X, Y + 1, I, 1, 32, 4, None) == ALIGN


def _descs(k, **over):
    arr = (q8.MatvecDesc * k)()
    for i in range(k):
        d = dict(w=W, x=X, y=Y, idx=None, n=32, p=4)
        d.update(over)
        arr[i] = q8.MatvecDesc(d["w"], d["x"], d["y"], d["idx"], d["n"], d["p"])
    return arr


def test_step_graph_levels_refusals(lib):
    """Levels are checked before any GPU work: NULL, negative or decreasing
    levels are refused, and the plain builder refuses the levels mode."""
    h = ctypes.c_void_p(None)
    b = lib.q8_step_graph_build_levels
    keep = []

    def lv(*v):
        a = (ctypes.c_int32 * len(v))(*v)
        keep.append(a)
        return ctypes.addressof(a)
    assert b(_descs(2), None, 2, 1, None, None, ctypes.byref(h)) == NULL
    assert b(_descs(2), lv(1, 0), 2, 1, None, None, ctypes.byref(h)) == 12
    assert b(_descs(2), lv(-1, 0), 2, 1, None, None, ctypes.byref(h)) == 12
    assert b(_descs(2), lv(0, 0), 2, 0, None, None, ctypes.byref(h)) == SHAPE
    assert b(_descs(2, n=40), lv(0, 1), 2, 1, None, None, ctypes.byref(h)) == SHAPE
    assert lib.q8_step_graph_build(_descs(1), 1, 1, None, 3, None, ctypes.byref(h)) == MODE
    assert not h.value


def test_step_graph_refusals(lib):
    h = ctypes.c_void_p(None)
    b = lib.q8_step_graph_build
    assert b(_descs(1), 1, 1, None, 0, None, None) == NULL
    assert b(None, 1, 1, None, 0, None, ctypes.byref(h)) == NULL
    assert b(_descs(1), 0, 1, None, 0, None, ctypes.byref(h)) == COUNT
    assert b(_descs(1), 4097, 1, None, 0, None, ctypes.byref(h)) == COUNT
    assert b(_descs(1), 1, 1, None, 7, None, ctypes.byref(h)) == MODE
    assert b(_descs(1), 1, 0, None, 0, None, ctypes.byref(h)) == SHAPE
    assert b(_descs(1), 1, 9, None, 0, None, ctypes.byref(h)) == SHAPE
    assert b(_descs(2, n=40), 2, 1, None, 0, None, ctypes.byref(h)) == SHAPE
    assert b(_descs(2, y=None), 2, 1, None, 0, None, ctypes.byref(h)) == NULL
    assert b(_descs(2, w=W + 4), 2, 1, None, 0, None, ctypes.byref(h)) == ALIGN
    assert b(_descs(65, idx=I), 65, 1, None, 0, None, ctypes.byref(h)) == COUNT
    assert b(_descs(1), 1, 1, I + 2, 0, None, ctypes.byref(h)) == ALIGN
    assert h.value is None


def test_graph_handle_refusals(lib):
    fake = ctypes.c_void_p(0x12345678)
    k = ctypes.c_int32(0)
    assert lib.q8_step_graph_launch(None, None) == BAD_HANDLE
    assert lib.q8_step_graph_launch_kernel(None, None) == BAD_HANDLE
    assert lib.q8_step_graph_launch_kernel(fake, None) == BAD_HANDLE
    assert lib.q8_step_graph_launch(fake, None) == BAD_HANDLE
    assert lib.q8_step_graph_info(None, ctypes.byref(k), None) == BAD_HANDLE
    assert lib.q8_step_graph_info(fake, ctypes.byref(k), None) == BAD_HANDLE
    assert lib.q8_step_graph_destroy(None) == BAD_HANDLE
    assert lib.q8_step_graph_destroy(fake) == BAD_HANDLE


_NO_DEVICE_SCRIPT = r"""
import ctypes, sys
sys.path.insert(0, sys.argv[1])
import q8_block_quantized_amd as q8
lib = q8.load()
c = ctypes.c_int32(-1)
assert lib.q8_device_count(ctypes.byref(c)) == 0
if c.value != 0:
    print("SKIP device visible")
    sys.exit(0)
W, X, Y, I = 0x10000, 0x20000, 0x30000, 0x40000
codes = [lib.q8_init(),
         lib.q8_matvec(W, X, Y, 32, 1, None),
         lib.q8_matvec_batched(W, X, Y, 2, 32, 1, None),
         lib.q8_argmax(X, 1, 4, I, None),
         lib.q8_matvec_argmax(W, X, None, I, 1, 32, 4, None)]
print("CODES", codes)
"""


def test_no_device_is_reported():
    """With no visible device every valid call returns Q8_ERR_NO_DEVICE.
    Runs in a child process with the devices hidden, and only proceeds past
    the device count when that count is zero."""
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    out = subprocess.run([sys.executable, "-c", _NO_DEVICE_SCRIPT, ROOT],
                         capture_output=True, text=True, env=env, timeout=120)
    assert out.returncode == 0, out.stderr
    if "SKIP" in out.stdout:
        pytest.skip("a device stayed visible")
    assert f"CODES {[NODEV] * 5}" in out.stdout, out.stdout


def _decode_args(n_layers=1, layer_over=None, buf_over=None, **over):
    """A decode model and buffers of fake aligned device addresses."""
    keep = []
    layers = (q8.DecodeLayer * n_layers)()
    for i in range(n_layers):
        vals = {f: 0x100000 * (j + 1) for j, f in enumerate(q8.LAYER_FIELDS)}
        vals.update(layer_over or {})
        layers[i] = q8.DecodeLayer(*[vals[f] for f in q8.LAYER_FIELDS])
    keep.append(layers)
    dims = dict(n_layers=n_layers, hidden=1024, n_heads=16, n_kv_heads=8, head_dim=128,
                inter=3072, vocab=151936, cache_rows=1024, eps=1e-6, theta=1e6, form=0)
    dims.update(over)
    model = q8.DecodeModel(dims["n_layers"], dims["hidden"], dims["n_heads"],
                           dims["n_kv_heads"], dims["head_dim"], dims["inter"], dims["vocab"],
                           dims["cache_rows"], dims["eps"], dims["theta"],
                           ctypes.addressof(layers), 0x7000000, 0x7100000, dims["form"])
    bvals = {f: 0x8000000 + 0x100000 * j for j, f in enumerate(q8.BUFFER_FIELDS)}
    bvals.update(buf_over or {})
    bufs = q8.DecodeBuffers(*[bvals[f] for f in q8.BUFFER_FIELDS])
    keep += [model, bufs]
    return model, bufs, keep


def test_decode_graph_refusals(lib):
    """The whole-step builder checks shapes, pointers and alignment before any
    GPU work."""
    h = ctypes.c_void_p(None)
    b = lib.q8_decode_graph_build

    def call(**kw):
        model, bufs, keep = _decode_args(**kw)
        return b(ctypes.byref(model), ctypes.byref(bufs), None, None, ctypes.byref(h))
    model, bufs, keep = _decode_args()
    assert b(None, ctypes.byref(bufs), None, None, ctypes.byref(h)) == NULL
    assert b(ctypes.byref(model), None, None, None, ctypes.byref(h)) == NULL
    assert b(ctypes.byref(model), ctypes.byref(bufs), None, None, None) == NULL
    assert call(head_dim=64) == SHAPE
    assert call(n_kv_heads=3) == SHAPE          # 16 heads not a multiple of 3
    assert call(n_heads=40, n_kv_heads=8) == SHAPE  # 5 query heads per kv head
    assert call(n_kv_heads=0) == SHAPE
    assert call(hidden=8192) == SHAPE
    assert call(hidden=1000) == SHAPE
    assert call(inter=100) == SHAPE
    assert call(vocab=0) == SHAPE
    assert call(cache_rows=0) == SHAPE
    assert call(cache_rows=65537) == SHAPE
    assert call(n_layers=0) == SHAPE
    assert call(eps=-1.0) == SHAPE
    assert call(eps=float("nan")) == SHAPE
    assert call(theta=0.0) == SHAPE
    assert call(form=2) == MODE and call(form=-1) == MODE
    assert call(layer_over=dict(wq=0)) == NULL
    assert call(layer_over=dict(k_cache=0)) == NULL
    assert call(layer_over=dict(wo=0x100004)) == ALIGN
    assert call(buf_over=dict(xn=0)) == NULL
    assert call(buf_over=dict(pos=0)) == NULL
    assert call(buf_over=dict(token=0)) == NULL
    assert call(buf_over=dict(q=0x8000008)) == ALIGN
    assert call(buf_over=dict(logits=0x8000004)) == ALIGN
    assert h.value is None


def test_wide_batch_int8_refusals(lib):
    """The int8-activation entry points take at most 8 rows."""
    assert lib.q8_matvec_i8x(W, X, Y, 9, 256, 4, None) == SHAPE
    assert lib.q8_matvec_argmax_i8x(W, X, None, I, 9, 256, 4, None) == SHAPE
