"""Python binding of libq8dec, the gfx950 Q8_0 decode matvec.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of ``include/q8dec.h``.  The functions carry the C
names and take torch tensors (device memory and streams come from PyTorch);
sizes are checked here because the C ABI receives bare pointers.  There is
no fallback: if ``libq8dec.so`` is missing or a call fails, a ``Q8Error``
is raised.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libq8dec.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "q8dec.h")

Q8_OK = 0
Q8_MAX_M = 32
Q8_MAX_M_NARROW = 8
Q8_MAX_N = 65536
Q8_GRAPH_CHAIN = 0
Q8_GRAPH_PERSISTENT = 1
Q8_GRAPH_PERSISTENT_I8X = 2
Q8_GRAPH_LEVELS = 3
Q8_GRAPH_DECODE = 4
Q8_DECODE_NODES = 0
Q8_DECODE_PERSISTENT = 1
BLOCK = 32
BLOCK_BYTES = 34


class Q8Error(RuntimeError):
    """A libq8dec call returned a nonzero status (or the library is absent)."""

    def __init__(self, status: int, name: str, detail: str = ""):
        self.status = status
        self.name = name
        super().__init__(f"{name} ({status}){': ' + detail if detail else ''}")


class MatvecDesc(ctypes.Structure):
    """q8_matvec_desc of include/q8dec.h."""
    _fields_ = [("w", ctypes.c_void_p), ("x", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("idx", ctypes.c_void_p),
                ("n", ctypes.c_int32), ("p", ctypes.c_int32)]


LAYER_FIELDS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down", "attn_norm",
                "ffn_norm", "q_norm", "k_norm", "k_cache", "v_cache")
BUFFER_FIELDS = ("x_in", "pos", "x", "xn", "q", "k", "v", "attn", "attn_out", "xn2",
                 "gate", "up", "h", "ffn_out", "xf", "logits", "token")


class DecodeLayer(ctypes.Structure):
    """q8_decode_layer of include/q8dec.h."""
    _fields_ = [(f, ctypes.c_void_p) for f in LAYER_FIELDS]


class DecodeModel(ctypes.Structure):
    """q8_decode_model of include/q8dec.h."""
    _fields_ = [(f, ctypes.c_int32) for f in
                ("n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim", "inter",
                 "vocab", "cache_rows")] + [
                ("eps", ctypes.c_float), ("theta", ctypes.c_float),
                ("layers", ctypes.c_void_p), ("out_norm", ctypes.c_void_p),
                ("lm_head", ctypes.c_void_p), ("form", ctypes.c_int32)]


class DecodeBuffers(ctypes.Structure):
    """q8_decode_buffers of include/q8dec.h."""
    _fields_ = [(f, ctypes.c_void_p) for f in BUFFER_FIELDS]


_lib = None


def load(path: str = LIB_PATH):
    """Loads libq8dec.so (raises Q8Error if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise Q8Error(-1, "q8_library_missing",
                      f"{path} not built; run python -m q8_block_quantized_amd._build")
    lib = ctypes.CDLL(path)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    pi32 = ctypes.POINTER(ctypes.c_int32)
    sig = {
        "q8_status_name": (ctypes.c_char_p, [ctypes.c_int]),
        "q8_last_hip_error": (ctypes.c_int, []),
        "q8_device_count": (ctypes.c_int, [pi32]),
        "q8_init": (ctypes.c_int, []),
        "q8_matvec": (ctypes.c_int, [vp, vp, vp, i32, i32, vp]),
        "q8_matvec_batched": (ctypes.c_int, [vp, vp, vp, i32, i32, i32, vp]),
        "q8_argmax": (ctypes.c_int, [vp, i32, i32, vp, vp]),
        "q8_matvec_argmax": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i32, vp]),
        "q8_matvec_argmax_noalloc": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i32, vp]),
        "q8_matvec_i8x": (ctypes.c_int, [vp, vp, vp, i32, i32, i32, vp]),
        "q8_matvec_argmax_i8x": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i32, vp]),
        "q8_step_graph_build": (ctypes.c_int, [ctypes.POINTER(MatvecDesc), i32,
                                               i32, vp, i32, vp,
                                               ctypes.POINTER(vp)]),
        "q8_step_graph_build_levels": (ctypes.c_int, [ctypes.POINTER(MatvecDesc), vp,
                                                      i32, i32, vp, vp,
                                                      ctypes.POINTER(vp)]),
        "q8_step_graph_launch": (ctypes.c_int, [vp, vp]),
        "q8_step_graph_launch_kernel": (ctypes.c_int, [vp, vp]),
        "q8_step_graph_info": (ctypes.c_int, [vp, pi32, pi32]),
        "q8_step_graph_destroy": (ctypes.c_int, [vp]),
        "q8_decode_graph_build": (ctypes.c_int, [ctypes.POINTER(DecodeModel),
                                                 ctypes.POINTER(DecodeBuffers), vp, vp,
                                                 ctypes.POINTER(vp)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def q8_status_name(status: int) -> str:
    return load().q8_status_name(status).decode()


def _check(status: int) -> None:
    if status != Q8_OK:
        lib = load()
        detail = ""
        if status == 7:  # Q8_ERR_HIP
            detail = f"hipError {lib.q8_last_hip_error()}"
        raise Q8Error(status, q8_status_name(status), detail)


def q8_device_count() -> int:
    c = ctypes.c_int32(0)
    _check(load().q8_device_count(ctypes.byref(c)))
    return c.value


def q8_init() -> None:
    _check(load().q8_init())


# ---- torch marshalling ------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t) -> int | None:
    return t.data_ptr() if t is not None and t.numel() > 0 else None


def _stream(stream, device) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _need(t, dtype, what: str, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if t.device.type != "cuda":
        raise ValueError(f"{what} must be on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{what} is on {t.device}, expected {device}")


def weight_bytes(n: int, p: int) -> int:
    return p * (n // BLOCK) * BLOCK_BYTES


def _check_w(w, n: int, p: int, device) -> None:
    torch = _torch()
    _need(w, torch.uint8, "w", device)
    if w.numel() != weight_bytes(n, p):
        raise ValueError(f"w holds {w.numel()} bytes; n={n}, p={p} need "
                         f"{weight_bytes(n, p)}")


def q8_matvec(w, x, y, stream=None) -> None:
    """y[p] = W x[n] (m = 1)."""
    torch = _torch()
    _need(x, torch.float32, "x")
    _need(y, torch.float32, "y", x.device)
    n, p = x.numel(), y.numel()
    _check_w(w, n, p, x.device)
    _check(load().q8_matvec(_ptr(w), _ptr(x), _ptr(y), n, p,
                            _stream(stream, x.device)))


def q8_matvec_batched(w, x, y, stream=None) -> None:
    """y[m, p] = x[m, n] W^T, 1 <= m <= 32 (m > 8: n a multiple of 256)."""
    torch = _torch()
    _need(x, torch.float32, "x")
    _need(y, torch.float32, "y", x.device)
    if x.dim() != 2 or y.dim() != 2 or x.shape[0] != y.shape[0]:
        raise ValueError("x must be [m, n] and y [m, p]")
    m, n = x.shape
    p = y.shape[1]
    _check_w(w, n, p, x.device)
    _check(load().q8_matvec_batched(_ptr(w), _ptr(x), _ptr(y), m, n, p,
                                    _stream(stream, x.device)))


def q8_argmax(logits, idx, stream=None) -> None:
    """idx[m] = argmax of each row of logits[m, p] (ties to the lower index)."""
    torch = _torch()
    _need(logits, torch.float32, "logits")
    _need(idx, torch.int32, "idx", logits.device)
    if logits.dim() == 1:
        m, p = 1, logits.numel()
    else:
        m, p = logits.shape
    if idx.numel() != m:
        raise ValueError("idx must hold one int32 per row")
    _check(load().q8_argmax(_ptr(logits), m, p, _ptr(idx),
                            _stream(stream, logits.device)))


def q8_matvec_argmax(w, x, idx, p: int, y=None, stream=None) -> None:
    """Fused lm_head: idx[m] = argmax(x[m, n] W^T); y [m, p] optional."""
    torch = _torch()
    _need(x, torch.float32, "x")
    _need(idx, torch.int32, "idx", x.device)
    x2 = x if x.dim() == 2 else x.view(1, -1)
    m, n = x2.shape
    if idx.numel() != m:
        raise ValueError("idx must hold one int32 per row")
    if y is not None:
        _need(y, torch.float32, "y", x.device)
        if y.numel() != m * p:
            raise ValueError("y must hold m * p floats")
    _check_w(w, n, p, x.device)
    _check(load().q8_matvec_argmax(_ptr(w), _ptr(x2), _ptr(y), _ptr(idx),
                                   m, n, p, _stream(stream, x.device)))


def q8_matvec_argmax_noalloc(w, x, idx, p: int, y=None, stream=None) -> None:
    """q8_matvec_argmax with the library's fixed per-device workspace (no
    allocation; calls that overlap on one device race)."""
    torch = _torch()
    _need(x, torch.float32, "x")
    _need(idx, torch.int32, "idx", x.device)
    x2 = x if x.dim() == 2 else x.view(1, -1)
    m, n = x2.shape
    if idx.numel() != m:
        raise ValueError("idx must hold one int32 per row")
    if y is not None:
        _need(y, torch.float32, "y", x.device)
        if y.numel() != m * p:
            raise ValueError("y must hold m * p floats")
    _check_w(w, n, p, x.device)
    _check(load().q8_matvec_argmax_noalloc(_ptr(w), _ptr(x2), _ptr(y), _ptr(idx),
                                           m, n, p, _stream(stream, x.device)))


def q8_matvec_i8x(w, x, y, stream=None) -> None:
    """y[m, p] = x[m, n] W^T with x quantised per 32-block to int8 (the
    int8-activation variant; n a multiple of 256, n <= 3072)."""
    torch = _torch()
    _need(x, torch.float32, "x")
    _need(y, torch.float32, "y", x.device)
    x2 = x if x.dim() == 2 else x.view(1, -1)
    m, n = x2.shape
    p = y.numel() // m if m else 0
    if y.numel() != m * p:
        raise ValueError("y must be [m, p]")
    _check_w(w, n, p, x.device)
    _check(load().q8_matvec_i8x(_ptr(w), _ptr(x2), _ptr(y), m, n, p,
                                _stream(stream, x.device)))


def q8_matvec_argmax_i8x(w, x, idx, p: int, y=None, stream=None) -> None:
    """q8_matvec_i8x with the argmax of each row; y [m, p] optional."""
    torch = _torch()
    _need(x, torch.float32, "x")
    _need(idx, torch.int32, "idx", x.device)
    x2 = x if x.dim() == 2 else x.view(1, -1)
    m, n = x2.shape
    if idx.numel() != m:
        raise ValueError("idx must hold one int32 per row")
    if y is not None:
        _need(y, torch.float32, "y", x.device)
        if y.numel() != m * p:
            raise ValueError("y must hold m * p floats")
    _check_w(w, n, p, x.device)
    _check(load().q8_matvec_argmax_i8x(_ptr(w), _ptr(x2), _ptr(y), _ptr(idx),
                                       m, n, p, _stream(stream, x.device)))


class StepGraph:
    """A recorded decode step (q8_step_graph_*): build once, launch per step.

    ``descs`` is a list of dicts with keys w, x, y, idx (tensors or None),
    n and p.  The tensors must stay alive while the graph exists; this object
    keeps references to them.  ``host_idx`` is a pinned int32 CPU tensor
    that receives m ints per argmax descriptor after each launch.
    """

    def __init__(self, descs, m: int, host_idx=None,
                 mode: int = Q8_GRAPH_CHAIN, device=None, levels=None):
        torch = _torch()
        self._keep = []
        arr = (MatvecDesc * len(descs))()
        for i, d in enumerate(descs):
            n, p = int(d["n"]), int(d["p"])
            x = d["x"]
            _need(x, torch.float32, f"descs[{i}].x")
            if x.numel() != m * n:
                raise ValueError(f"descs[{i}].x must hold m * n floats")
            _check_w(d["w"], n, p, x.device)
            if d.get("y") is not None:
                _need(d["y"], torch.float32, f"descs[{i}].y", x.device)
                if d["y"].numel() != m * p:
                    raise ValueError(f"descs[{i}].y must hold m * p floats")
            if d.get("idx") is not None:
                _need(d["idx"], torch.int32, f"descs[{i}].idx", x.device)
                if d["idx"].numel() != m:
                    raise ValueError(f"descs[{i}].idx must hold m ints")
            arr[i] = MatvecDesc(_ptr(d["w"]), _ptr(x), _ptr(d.get("y")),
                                _ptr(d.get("idx")), n, p)
            self._keep.append(d)
        nargmax = sum(1 for d in descs if d.get("idx") is not None)
        if host_idx is not None:
            if host_idx.dtype != torch.int32 or host_idx.device.type != "cpu" \
                    or not host_idx.is_pinned():
                raise ValueError("host_idx must be a pinned int32 CPU tensor")
            if host_idx.numel() < nargmax * m:
                raise ValueError("host_idx too small")
        self._keep.append(host_idx)
        self.host_idx = host_idx
        self.m = m
        self.mode = mode
        dev = device if device is not None else descs[0]["x"].device
        handle = ctypes.c_void_p(None)
        hptr = host_idx.data_ptr() if host_idx is not None else None
        with torch.cuda.device(dev):
            if levels is not None:  # one persistent node per run of a level
                lv = (ctypes.c_int32 * len(descs))(*[int(v) for v in levels])
                if len(levels) != len(descs):
                    raise ValueError("one level per descriptor")
                self._keep.append(lv)
                _check(load().q8_step_graph_build_levels(
                    arr, ctypes.addressof(lv), len(descs), m, hptr,
                    _stream(None, dev), ctypes.byref(handle)))
                self.mode = Q8_GRAPH_LEVELS
            else:
                _check(load().q8_step_graph_build(
                    arr, len(descs), m, hptr, mode, _stream(None, dev),
                    ctypes.byref(handle)))
        self._h = handle
        self.device = dev

    def launch(self, stream=None) -> None:
        _check(load().q8_step_graph_launch(self._h, _stream(stream, self.device)))

    def launch_kernel(self, stream=None) -> None:
        """The same recorded step as one kernel launch (persistent mode)."""
        _check(load().q8_step_graph_launch_kernel(self._h, _stream(stream, self.device)))

    def info(self) -> tuple[int, int]:
        k, c = ctypes.c_int32(0), ctypes.c_int32(0)
        _check(load().q8_step_graph_info(self._h, ctypes.byref(k), ctypes.byref(c)))
        return k.value, c.value

    def close(self) -> None:
        if self._h is not None and self._h.value:
            _check(load().q8_step_graph_destroy(self._h))
        self._h = None

    def __del__(self):  # pragma: no cover - best effort
        try:
            self.close()
        except Exception:
            pass


# ---- the whole decode step --------------------------------------------------

def decode_buffer_sizes(dims: dict) -> dict:
    """Element counts of every q8_decode_buffers entry for the given shapes."""
    H, hd, inter = dims["hidden"], dims["head_dim"], dims["inter"]
    qw, kvw = dims["n_heads"] * hd, dims["n_kv_heads"] * hd
    return dict(x_in=H, pos=1, x=H, xn=H, q=qw, k=kvw, v=kvw, attn=qw, attn_out=H, xn2=H,
                gate=inter, up=inter, h=inter, ffn_out=H, xf=H, logits=dims["vocab"],
                token=1)


def decode_buffers(dims: dict, device, logits: bool = True) -> dict:
    """Allocates (with torch) the activation buffers of one decode step."""
    torch = _torch()
    out = {}
    for k, n in decode_buffer_sizes(dims).items():
        if k == "logits" and not logits:
            out[k] = None
            continue
        dt = torch.int32 if k in ("pos", "token") else torch.float32
        out[k] = torch.zeros(n, dtype=dt, device=device)
    return out


class DecodeGraph(StepGraph):
    """The whole decode step (q8_decode_graph_build), launched like a StepGraph.

    ``dims``: n_layers, hidden, n_heads, n_kv_heads, head_dim, inter, vocab,
    cache_rows, eps, theta.  ``layers``: one dict per layer with the tensors
    of LAYER_FIELDS (uint8 Q8_0 weights, float32 norms and caches).
    ``bufs``: the tensors of BUFFER_FIELDS (decode_buffers makes them;
    logits may be None).  Every tensor must stay alive while the graph
    exists; this object keeps references to them.  ``form``:
    Q8_DECODE_NODES (a kernel node per stage) or Q8_DECODE_PERSISTENT (one
    launch with a grid-wide barrier between phases).
    """

    def __init__(self, dims: dict, layers, out_norm, lm_head, bufs: dict,
                 host_token=None, device=None, form=None):
        torch = _torch()
        dev = device if device is not None else bufs["x"].device
        H, hd = int(dims["hidden"]), int(dims["head_dim"])
        qw, kvw = int(dims["n_heads"]) * hd, int(dims["n_kv_heads"]) * hd
        inter, rows = int(dims["inter"]), int(dims["cache_rows"])
        if len(layers) != int(dims["n_layers"]):
            raise ValueError("one layer dict per layer")
        wshape = dict(wq=(H, qw), wk=(H, kvw), wv=(H, kvw), wo=(qw, H), w_gate=(H, inter),
                      w_up=(H, inter), w_down=(inter, H))
        fsize = dict(attn_norm=H, ffn_norm=H, q_norm=hd, k_norm=hd, k_cache=rows * kvw,
                     v_cache=rows * kvw)
        self._keep = [layers, out_norm, lm_head, bufs, host_token]
        arr = (DecodeLayer * len(layers))()
        for i, L in enumerate(layers):
            vals = []
            for f in LAYER_FIELDS:
                t = L[f]
                if f in wshape:
                    _check_w(t, *wshape[f], dev)
                else:
                    _need(t, torch.float32, f"layers[{i}].{f}", dev)
                    if t.numel() != fsize[f]:
                        raise ValueError(f"layers[{i}].{f} must hold {fsize[f]} floats")
                vals.append(t.data_ptr())
            arr[i] = DecodeLayer(*vals)
        _need(out_norm, torch.float32, "out_norm", dev)
        _check_w(lm_head, H, int(dims["vocab"]), dev)
        sizes = decode_buffer_sizes(dims)
        bvals = []
        for f in BUFFER_FIELDS:
            t = bufs.get(f)
            if t is None and f == "logits":
                bvals.append(None)
                continue
            _need(t, torch.int32 if f in ("pos", "token") else torch.float32, f, dev)
            if t.numel() != sizes[f]:
                raise ValueError(f"bufs[{f}] must hold {sizes[f]} elements")
            bvals.append(t.data_ptr())
        if host_token is not None:
            if host_token.dtype != torch.int32 or host_token.device.type != "cpu" \
                    or not host_token.is_pinned() or host_token.numel() < 1:
                raise ValueError("host_token must be a pinned int32 CPU tensor")
        model = DecodeModel(int(dims["n_layers"]), H, int(dims["n_heads"]),
                            int(dims["n_kv_heads"]), hd, inter, int(dims["vocab"]), rows,
                            float(dims["eps"]), float(dims["theta"]),
                            ctypes.addressof(arr), out_norm.data_ptr(), lm_head.data_ptr(),
                            Q8_DECODE_NODES if form is None else int(form))
        cb = DecodeBuffers(*bvals)
        self._keep += [arr, model, cb]
        self.host_idx = host_token
        self.m = 1
        self.mode = Q8_GRAPH_DECODE
        self.form = Q8_DECODE_NODES if form is None else int(form)
        self.dims = dict(dims)
        handle = ctypes.c_void_p(None)
        hptr = host_token.data_ptr() if host_token is not None else None
        with torch.cuda.device(dev):
            _check(load().q8_decode_graph_build(ctypes.byref(model), ctypes.byref(cb), hptr,
                                                _stream(None, dev), ctypes.byref(handle)))
        self._h = handle
        self.device = dev
