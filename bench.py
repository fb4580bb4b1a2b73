"""Benchmark of the Q8_0 decode matvec path on one MI355X.

A step is one full decode step's matvecs: 28 layers x (q, k, v, o, gate, up,
down) plus the lm_head 1024 -> 151,936 with its fused argmax = 197 Q8_0
matvecs, recorded once as a hipGraph and launched once; the kernel stores the
one int32 token straight into pinned host memory.  Inputs are seeded synthetic stand-ins for the
Qwen3-0.6B weights (see gen/): two full weight sets (1.27 GB, beyond the
256 MB Infinity Cache) are alternated step by step, so every step streams
its weights from HBM.

Prints one JSON line on stdout (progress goes to stderr).  The timed region
is exactly --steps steps, bracketed by device synchronisation, after an
untimed settling run (~0.3 s of the same work: the clocks' steady state) and
--warmup steps.  Each step is
one graph launch followed by a wait for the token: a spin on the pinned
host slot that the kernel stores last (headline), and in a second timed run
a full stream synchronisation (every output of the step complete).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import gen  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
METRIC = ("Q8_0 matvec HBM GB/s (% of peak) + 197-matvec decode-step "
          "latency (µs)")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


KERNEL_SOURCES = ["q8dec_api.hip", "q8dec_internal.h", "q8dec_kernels.hip",
                  "q8dec_decode_dev.h"]
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "step_kernel_decode_step_hbm_bytes.md")


def kernel_source_hash() -> str:
    """sha256 of the library sources with comments and white space removed
    (a comment edit does not change the kernel the counters describe)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "q8_block_quantized_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update("".join(text.split()).encode())
    return h.hexdigest()


def profiled_traffic():
    """HBM bytes per step-kernel launch from the committed rocprofv3 counter
    summary, or None when the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_PROFILE) as f:
            kv = dict(line.split(": ", 1) for line in f.read().splitlines()
                      if line.startswith(("traffic_bytes_per_launch:",
                                          "kernel_source_sha256:")))
    except OSError:
        return None
    if kv.get("kernel_source_sha256", "").strip() != kernel_source_hash():
        return None
    return int(kv["traffic_bytes_per_launch"])


def alg_bytes(n: int, p: int, m: int, logits: bool, argmax: bool) -> int:
    """Algorithmic bytes of one matvec: weight blocks + x + outputs."""
    return (p * (n // 32) * 34 + m * n * 4 + (m * p * 4 if logits else 0)
            + (m * 4 if argmax else 0))


class StepSet:
    """Device buffers of one decode step's 197 matvecs (one weight set)."""

    def __init__(self, torch, dev, seed: int, base: int, m: int, lm_logits: bool,
                 weights=None):
        self.shapes = gen.step_shapes()
        self.descs = []
        self.w = weights if weights is not None else []
        for i, (name, n, p) in enumerate(self.shapes):
            if weights is None:
                w = gen.weights(p, n, seed=seed, index=base + i)
                self.w.append(torch.from_numpy(w.reshape(-1)).to(dev))
            x = torch.from_numpy(gen.activations(m, n, seed=seed, index=base + i)).to(dev)
            last = i == len(self.shapes) - 1
            y = None
            if not last or lm_logits:
                y = torch.empty((m, p), dtype=torch.float32, device=dev)
            idx = torch.full((m,), -1, dtype=torch.int32, device=dev) if last else None
            self.descs.append(dict(w=self.w[i], x=x, y=y, idx=idx, n=n, p=p))
        self.bytes = sum(alg_bytes(d["n"], d["p"], m, d["y"] is not None,
                                   d["idx"] is not None) for d in self.descs)
        self.weight_bytes = sum(p * (n // 32) * 34 for _, n, p in self.shapes)


class _KernelLaunch:
    """A step graph whose launch() submits its recorded kernel directly."""

    def __init__(self, g):
        self.g = g

    def launch(self):
        self.g.launch_kernel()


SETTLE_S = 0.3  # untimed load before each timed section


def settle(torch, fn, seconds: float = SETTLE_S) -> None:
    """Runs fn(k) back to back (untimed) for about `seconds`: the GPU's
    clocks take tens of milliseconds of load to reach their steady state, and
    a decode loop runs at that state.  Measured on MI355X: the polled step
    right after 20 warmup steps takes ~121 us, ~115.5 us once settled."""
    t_end = time.perf_counter() + seconds
    k = 0
    while time.perf_counter() < t_end:
        for _ in range(16):
            fn(k)
            k += 1
        torch.cuda.synchronize()


def time_graph_steps(torch, graphs, host, steps: int, warmup: int,
                     poll: bool = False, spread: dict = None):
    """Wall seconds per step of: launch the step graph, wait, read the token.
    The wait is a stream synchronisation (every output complete), or with
    poll=True a spin on the pinned token slot, which the kernel writes last
    (the token is on the host; the kernel may still be retiring).  The
    timed steps follow a settling run (see settle) and `warmup` steps."""
    stream = torch.cuda.current_stream()
    hv = host.numpy()
    sentinel = -2  # never an argmax result

    def one(k):
        if poll:
            hv[:] = sentinel
            graphs[k % len(graphs)].launch()
            if hv.size == 1:
                while hv[0] == sentinel:
                    pass
            else:
                while (hv == sentinel).any():
                    pass
        else:
            graphs[k % len(graphs)].launch()
            stream.synchronize()
        return int(hv[0])

    settle(torch, one)
    for k in range(warmup):
        one(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    toks = []
    stamps = [t0]
    for k in range(steps):
        toks.append(one(k))
        stamps.append(time.perf_counter())
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    if spread is not None:  # per-step wall times: p10, median, p90 (us)
        per = sorted(b - a for a, b in zip(stamps, stamps[1:]))
        spread.update(p10=round(per[len(per) // 10] * 1e6, 2),
                      median=round(statistics.median(per) * 1e6, 2),
                      p90=round(per[(9 * len(per)) // 10] * 1e6, 2))
    return sec, toks


def event_time(torch, fn, count: int, warmup: int = 3) -> float:
    """Average HIP-event time (s) per call of fn(k), k = 0..count-1, issued
    back to back on torch's current stream between one pair of events (the
    GPU never waits on the host inside the bracket), after a settling run
    (see settle)."""
    settle(torch, fn)
    for k in range(warmup):
        fn(k)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for k in range(count):
        fn(k)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e-3 / count


def cpu_baseline(sets, m_host, threads_req: int, budget_s: float):
    """The oracle on the host cores over the first weight set's step, and a
    parity check of the GPU outputs of that step against it."""
    import oracle
    orc = oracle.get()
    s0 = sets
    ws = [w for w in m_host["w"]]
    xs = m_host["x"]
    times = []
    used = 1
    worst = 0.0
    ok_idx = True
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        ys = []
        for i, (name, n, p) in enumerate(s0.shapes):
            y, tol, used = orc.matvec_mt(ws[i], xs[i][0], threads_req)
            ys.append((y, tol))
        times.append(time.perf_counter() - t0)
        if len(times) >= 3 or time.perf_counter() - t_start > budget_s:
            break
    # parity of the GPU step outputs (written by the last launch of set 0)
    for i, d in enumerate(s0.descs):
        y, tol = ys[i]
        if d["y"] is not None:
            g = d["y"].cpu().numpy()[0]
            worst = max(worst, float(oracle.matvec_errors(g, y, tol).max()))
        if d["idx"] is not None:
            ok_idx = ok_idx and oracle.argmax_accepted(int(d["idx"][0].item()), y, tol)
    return statistics.median(times), used, worst, ok_idx


def decode_step(torch, q8, dev, pos: int, rows: int, steps: int, warmup: int,
                seed: int = 0) -> dict:
    """The whole Qwen3-0.6B-shaped decode step (q8_decode_graph_build) at
    position pos with a cache of `rows` rows: token latency of the graph
    launch (and of its kernels launched directly), waiting on the token the
    kernel stores into pinned memory.  Algorithmic bytes: the weights, the
    norm weights, the pos + 1 key and value rows each layer reads, and the
    activations (x, caches written: one row per layer)."""
    model = gen.decode_model(gen.QWEN3_DIMS, cache_rows=rows, seed=seed)
    dims = model["dims"]
    layers = [{f: torch.from_numpy(L[f].reshape(-1)).to(dev) for f in q8.LAYER_FIELDS}
              for L in model["layers"]]
    out_norm = torch.from_numpy(model["out_norm"]).to(dev)
    lm_head = torch.from_numpy(model["lm_head"].reshape(-1)).to(dev)
    bufs = q8.decode_buffers(dims, dev, logits=False)
    bufs["x_in"].copy_(torch.from_numpy(model["x_in"]))
    bufs["pos"].fill_(pos)
    host = torch.zeros(1, dtype=torch.int32).pin_memory()
    g = q8.DecodeGraph(dims, layers, out_norm, lm_head, bufs, host_token=host)
    nodes = g.info()
    sec, toks = time_graph_steps(torch, [g], host, steps, warmup, poll=True)
    ksec, ktoks = time_graph_steps(torch, [_KernelLaunch(g)], host, steps, warmup, poll=True)
    assert ktoks == toks, "decode token differs between graph and kernel launches"
    H, L = dims["hidden"], dims["n_layers"]
    kvw = dims["n_kv_heads"] * dims["head_dim"]
    wb = sum(model["layers"][0][k].size for k in gen.DECODE_WEIGHTS) * L \
        + model["lm_head"].size
    kvb = 2 * (pos + 1) * kvw * 4 * L
    normb = (2 * H + 2 * dims["head_dim"]) * 4 * L + 4 * H
    alg = wb + kvb + normb
    g.close()
    del layers, lm_head, bufs
    torch.cuda.empty_cache()
    return {
        "pos": pos, "cache_rows": rows, "token": toks[-1],
        "token_latency_us": round(sec * 1e6, 2),
        "kernel_launches_token_latency_us": round(ksec * 1e6, 2),
        "tokens_per_s": round(1.0 / sec, 1),
        "GBps": round(alg / sec / 1e9, 1),
        "alg_bytes": alg, "weight_bytes": wb, "kv_bytes": kvb,
        "graph_nodes": {"kernel": nodes[0], "memcpy": nodes[1]},
    }


def only_workload(args, torch, q8, dev) -> int:
    """One configuration alone, for a kernel trace or counters of its kernel."""
    out = {"workload": args.only, "steps": args.steps}
    if args.only == "lm_head":
        # 4 weight copies (661 MB, beyond the Infinity Cache) rotated
        ws = [torch.from_numpy(gen.weights(151936, 1024, seed=0, index=3000 + c)
                               .reshape(-1)).to(dev) for c in range(4)]
        x = torch.from_numpy(gen.activations(1, 1024, seed=0, index=3000)).to(dev)
        idx = torch.empty(1, dtype=torch.int32, device=dev)
        t = event_time(torch, lambda k: q8.q8_matvec_argmax(ws[k % 4], x, idx, 151936),
                       args.steps, args.warmup)
        b = alg_bytes(1024, 151936, 1, False, True)
        out.update(avg_us=round(t * 1e6, 2), GBps=round(b / t / 1e9, 1), alg_bytes=b)
    elif args.only == "wide":
        m = 32
        sets32 = [StepSet(torch, dev, 0, 7000 + 1000 * j, m, False) for j in range(2)]
        host32 = torch.zeros(m, dtype=torch.int32).pin_memory()
        gw = [q8.StepGraph(s.descs, m, host_idx=host32, mode=q8.Q8_GRAPH_PERSISTENT)
              for s in sets32]
        sw, _ = time_graph_steps(torch, gw, host32, args.steps, args.warmup, poll=True)
        bw = sets32[0].bytes
        out.update(step_latency_us=round(sw * 1e6, 2), GBps=round(bw / sw / 1e9, 1),
                   per_row_us=round(sw * 1e6 / m, 2), alg_bytes=bw)
        for g in gw:
            g.close()
    elif args.only == "decode":
        out.update(decode_step(torch, q8, dev, 1023, 4096, args.steps, args.warmup))
    elif args.only == "i8x_step":
        sets1 = [StepSet(torch, dev, 0, 1000 * j, 1, False) for j in range(2)]
        host = torch.zeros(1, dtype=torch.int32).pin_memory()
        gs = [q8.StepGraph(s.descs, 1, host_idx=host, mode=q8.Q8_GRAPH_PERSISTENT_I8X)
              for s in sets1]
        sec, _ = time_graph_steps(torch, gs, host, args.steps, args.warmup, poll=True)
        b = sets1[0].bytes
        out.update(step_latency_us=round(sec * 1e6, 2), GBps=round(b / sec / 1e9, 1),
                   alg_bytes=b)
        for g in gs:
            g.close()
    else:
        sets8 = [StepSet(torch, dev, 0, 5000 + 1000 * j, 8, False) for j in range(2)]
        host8 = torch.zeros(8, dtype=torch.int32).pin_memory()
        p8 = [q8.StepGraph(s.descs, 8, host_idx=host8, mode=q8.Q8_GRAPH_PERSISTENT)
              for s in sets8]
        s8, _ = time_graph_steps(torch, p8, host8, args.steps, args.warmup, poll=True)
        b8 = sets8[0].bytes
        out.update(step_latency_us=round(s8 * 1e6, 2), GBps=round(b8 / s8 / 1e9, 1),
                   alg_bytes=b8)
        for g in p8:
            g.close()
    print(json.dumps(out))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true",
                    help="only the headline step (for profiling runs)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle leg")
    ap.add_argument("--only", choices=["lm_head", "batched", "i8x_step", "decode", "wide"],
                    default=None,
                    help="only time one other configuration (for profiling runs): "
                         "the fused lm_head (1024 -> 151,936 + argmax, m = 1), "
                         "the m = 8 step, the int8-activation step, the whole "
                         "decode step at position 1023, or the m = 32 step; prints "
                         "one JSON line")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 5 times "
                         "(reference for the HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build runs on a single MI355X "
              "and has no multi-GPU path; use --gpus 1", file=sys.stderr)
        return 2

    import torch
    import q8_block_quantized_amd as q8

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5}))
        return 0
    q8.q8_init()
    if args.only:
        return only_workload(args, torch, q8, dev)
    log("generating two weight sets of a decode step (2 x 633 MB)")
    sets = [StepSet(torch, dev, 0, 0, 1, False), StepSet(torch, dev, 0, 1000, 1, False)]
    host = torch.zeros(1, dtype=torch.int32).pin_memory()
    pers = [q8.StepGraph(s.descs, 1, host_idx=host, mode=q8.Q8_GRAPH_PERSISTENT)
            for s in sets]
    bare = [q8.StepGraph(s.descs, 1, mode=q8.Q8_GRAPH_PERSISTENT) for s in sets]
    assert pers[0].info() == (1, 0)
    step_bytes = sets[0].bytes

    log(f"headline: {args.steps} persistent-graph steps")
    # the headline waits for the token the way a decode loop does: spinning
    # on the pinned slot the kernel writes last; the fully synchronised
    # figure (every output of the step complete) is reported beside it
    spread = {}
    sec, toks = time_graph_steps(torch, pers, host, args.steps, args.warmup,
                                 poll=True, spread=spread)
    ssec, stoks = time_graph_steps(torch, pers, host, args.steps, args.warmup)
    assert stoks == toks, "token differs between the two waits"
    # the same recorded step submitted as one kernel launch instead of a
    # hipGraphLaunch (reported beside the headline, never as it)
    ksec, ktoks = time_graph_steps(torch, [_KernelLaunch(g) for g in pers], host,
                                   args.steps, args.warmup, poll=True)
    assert ktoks == toks, "token differs between graph and kernel launches"
    # dominant kernel: the step kernel's duration, from back-to-back launches
    # of the recorded kernel (graph without the host token, submitted
    # directly).  Back-to-back hipGraphLaunches leave ~4.5 us idle between
    # executions (a kernel trace shows the same kernel duration either way),
    # so that figure is reported beside it, not as it.
    k_avg = event_time(torch, lambda k: bare[k % 2].launch_kernel(), args.steps)
    g_avg = event_time(torch, lambda k: bare[k % 2].launch(), args.steps)
    achieved = step_bytes / k_avg / 1e9

    result = {
        "metric": METRIC,
        "value": round(step_bytes / sec / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": ("full decode step: 197 Q8_0 matvecs (28 layers x q,k,v,"
                         "o,gate,up,down + lm_head 1024->151936 with fused argmax), "
                         "m=1, one persistent-kernel hipGraph launch per step, the "
                         "int32 token stored by the kernel into pinned host memory, "
                         "2 weight sets alternated (1.27 GB)"),
            "matvecs": 197,
            "m": 1,
            "weight_bytes_per_step": sets[0].weight_bytes,
            "alg_bytes_per_step": step_bytes,
            "graph_nodes": {"kernel": 1, "memcpy": 0},
        },
        "step_latency_us": round(sec * 1e6, 2),
        "step_latency_spread_us": spread,
        "step_latency_synchronized_us": round(ssec * 1e6, 2),
        "step_latency_kernel_launch_us": round(ksec * 1e6, 2),
        "pct_of_hbm_peak": round(100 * step_bytes / sec / 1e9 / HBM_PEAK_GBS, 2),
        "roofline": {
            "bound": "hbm",
            "kernel": "step_kernel (persistent, 197 matvecs)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": profiled_traffic(),
            "avg_launch_us": round(k_avg * 1e6, 2),
            "timing": ("HIP events around back-to-back launches of the recorded "
                       "step kernel on torch's current stream"),
            "graph_back_to_back_us": round(g_avg * 1e6, 2),
        },
    }

    extra = {}
    if not args.no_extra:
        steps2 = max(5, min(args.steps, 50))
        log("chain graph (197 kernel nodes)")
        chain = [q8.StepGraph(s.descs, 1, host_idx=host, mode=q8.Q8_GRAPH_CHAIN)
                 for s in sets]
        assert chain[0].info() == (197, 0)
        csec, ctoks = time_graph_steps(torch, chain, host, steps2, 3, poll=True)
        extra["chain_graph_197_nodes"] = {
            "step_latency_us": round(csec * 1e6, 2),
            "GBps": round(step_bytes / csec / 1e9, 1),
            "per_node_us": round(csec * 1e6 / 197, 3),
        }
        for g in chain:
            g.close()

        log("levels graph (q|k|v, o, gate|up, down per layer: 113 nodes)")
        lv = []
        for l in range(28):
            lv += [4 * l] * 3 + [4 * l + 1] + [4 * l + 2] * 2 + [4 * l + 3]
        lv.append(4 * 28)
        lvg = [q8.StepGraph(s.descs, 1, host_idx=host, levels=lv) for s in sets]
        assert lvg[0].info() == (113, 0)
        lsec, ltoks = time_graph_steps(torch, lvg, host, steps2, 3, poll=True)
        lksec, _ = time_graph_steps(torch, [_KernelLaunch(g) for g in lvg], host,
                                    steps2, 3, poll=True)
        assert ltoks == toks[:len(ltoks)], "levels graph token differs"
        extra["levels_graph_113_nodes"] = {
            "step_latency_us": round(lsec * 1e6, 2),
            "GBps": round(step_bytes / lsec / 1e9, 1),
            "per_node_us": round(lsec * 1e6 / 113, 3),
            "kernel_launches_step_latency_us": round(lksec * 1e6, 2),
        }
        for g in lvg:
            g.close()

        log("lm_head fused (4 copies rotated)")
        lm_extra = [torch.from_numpy(gen.weights(151936, 1024, seed=0, index=2000 + c)
                                     .reshape(-1)).to(dev) for c in range(2)]
        lm_w = [sets[0].w[-1], sets[1].w[-1]] + lm_extra
        lm_x = sets[0].descs[-1]["x"]
        lm_idx = torch.empty(1, dtype=torch.int32, device=dev)
        lt = event_time(torch, lambda k: q8.q8_matvec_argmax(
            lm_w[k % 4], lm_x, lm_idx, 151936), 40)
        lb = alg_bytes(1024, 151936, 1, False, True)
        extra["lm_head_fused"] = {
            "avg_us": round(lt * 1e6, 2),
            "GBps": round(lb / lt / 1e9, 1),
            "pct_of_peak": round(100 * lb / lt / 1e9 / HBM_PEAK_GBS, 2),
            "alg_bytes": lb,
        }
        lm_y = torch.empty(151936, dtype=torch.float32, device=dev)
        lt0 = event_time(torch, lambda k: q8.q8_matvec(
            lm_w[k % 4], lm_x.view(-1), lm_y), 40)
        lb0 = alg_bytes(1024, 151936, 1, True, False)
        extra["lm_head_matvec_only"] = {
            "avg_us": round(lt0 * 1e6, 2),
            "GBps": round(lb0 / lt0 / 1e9, 1),
        }

        log("single matvec 1024->2048 (rotating 240 copies, 535 MB)")
        qs = [d["w"] for s in sets for d in s.descs if d["p"] == 2048 and d["n"] == 1024]
        qs += [torch.from_numpy(gen.weights(2048, 1024, seed=0, index=4000 + c)
                                .reshape(-1)).to(dev) for c in range(240 - len(qs))]
        qx = sets[0].descs[0]["x"].view(-1)
        qy = torch.empty(2048, dtype=torch.float32, device=dev)
        st = event_time(torch, lambda k: q8.q8_matvec(qs[k % len(qs)], qx, qy), 240)
        hot = event_time(torch, lambda k: q8.q8_matvec(qs[0], qx, qy), 240)
        sb = alg_bytes(1024, 2048, 1, True, False)
        extra["single_matvec_1024x2048"] = {
            "avg_us": round(st * 1e6, 2),
            "GBps": round(sb / st / 1e9, 1),
            "matvecs_per_s": round(1.0 / st, 1),
            "hot_avg_us": round(hot * 1e6, 2),
            "note": ("back-to-back launches over 240 distinct weight copies (535 MB, "
                     "beyond the 256 MB Infinity Cache); hot: one copy, cached"),
        }
        del qs

        log("one layer: 7 matvecs back to back (56 layers rotated)")
        layers = [s.descs[7 * l:7 * l + 7] for s in sets for l in range(28)]

        def run_layer(k):
            for d in layers[k % len(layers)]:
                q8.q8_matvec(d["w"], d["x"].view(-1), d["y"].view(-1))
        lt2 = event_time(torch, run_layer, 56)
        lyb = sum(alg_bytes(n, p, 1, True, False) for _, n, p in gen.LAYER_SHAPES)
        extra["layer_7_matvecs_stream"] = {
            "avg_us": round(lt2 * 1e6, 2),
            "GBps": round(lyb / lt2 / 1e9, 1),
        }

        log("int8-activation step (persistent graph, x quantised per 32-block)")
        pi8 = [q8.StepGraph(s.descs, 1, host_idx=host, mode=q8.Q8_GRAPH_PERSISTENT_I8X)
               for s in sets]
        isec, _ = time_graph_steps(torch, pi8, host, steps2, 3, poll=True)
        ik = event_time(torch, lambda k: pi8[k % 2].launch_kernel(), steps2)
        extra["i8x_step"] = {
            "step_latency_us": round(isec * 1e6, 2),
            "GBps": round(step_bytes / isec / 1e9, 1),
            "kernel_avg_us": round(ik * 1e6, 2),
            "kernel_GBps": round(step_bytes / ik / 1e9, 1),
            "note": "int8 activations: a separate operation with its own bound, "
                    "not the headline",
        }
        for g in pi8:
            g.close()
        li = event_time(torch, lambda k: q8.q8_matvec_argmax_i8x(
            lm_w[k % 4], lm_x, lm_idx, 151936), 40)
        extra["lm_head_fused_i8x"] = {
            "avg_us": round(li * 1e6, 2),
            "GBps": round(lb / li / 1e9, 1),
            "pct_of_peak": round(100 * lb / li / 1e9 / HBM_PEAK_GBS, 2),
        }

        log("batched m=8 step (persistent graph)")
        sets8 = [StepSet(torch, dev, 0, 5000 + 1000 * j, 8, False, weights=s.w)
                 for j, s in enumerate(sets)]
        host8 = torch.zeros(8, dtype=torch.int32).pin_memory()
        p8 = [q8.StepGraph(s.descs, 8, host_idx=host8, mode=q8.Q8_GRAPH_PERSISTENT)
              for s in sets8]
        s8, _ = time_graph_steps(torch, p8, host8, steps2, 3, poll=True)
        b8 = sets8[0].bytes
        extra["batched_m8_step"] = {
            "step_latency_us": round(s8 * 1e6, 2),
            "GBps": round(b8 / s8 / 1e9, 1),
            "per_row_us": round(s8 * 1e6 / 8, 2),
            "per_row_vs_m1": round((s8 / 8) / sec, 3),
        }
        for g in p8:
            g.close()
        del sets8, p8

        log("batched m=32 step (wide batch, persistent graph)")
        sets32 = [StepSet(torch, dev, 0, 7000 + 1000 * j, 32, False, weights=s.w)
                  for j, s in enumerate(sets)]
        host32 = torch.zeros(32, dtype=torch.int32).pin_memory()
        p32 = [q8.StepGraph(s.descs, 32, host_idx=host32, mode=q8.Q8_GRAPH_PERSISTENT)
               for s in sets32]
        s32, _ = time_graph_steps(torch, p32, host32, steps2, 3, poll=True)
        b32 = sets32[0].bytes
        extra["batched_m32_step"] = {
            "step_latency_us": round(s32 * 1e6, 2),
            "GBps": round(b32 / s32 / 1e9, 1),
            "per_row_us": round(s32 * 1e6 / 32, 2),
            "per_row_vs_m1": round((s32 / 32) / sec, 3),
        }
        for g in p32:
            g.close()
        del sets32, p32

        for dpos in (1023, 4095):
            log(f"whole decode step (norms, attention, SwiGLU; 142 nodes), pos {dpos}")
            extra[f"decode_step_pos{dpos}"] = decode_step(torch, q8, dev, dpos, 4096,
                                                           steps2, 3)
    if extra:
        result["extra"] = extra

    if not args.no_cpu:
        log("cpu baseline: the oracle on the host cores")
        try:
            ncpu = len(os.sched_getaffinity(0))
        except AttributeError:  # pragma: no cover
            ncpu = os.cpu_count() or 1
        m_host = {"w": [], "x": []}
        for i, (name, n, p) in enumerate(sets[0].shapes):
            m_host["w"].append(gen.weights(p, n, seed=0, index=i))
            m_host["x"].append(gen.activations(1, n, seed=0, index=i))
        # the GPU outputs compared below come from one launch of set 0
        pers[0].launch()
        torch.cuda.synchronize()
        csec_, used, worst, ok_idx = cpu_baseline(sets[0], m_host, ncpu, 20.0)
        result["cpu_baseline"] = {
            "value": round(step_bytes / csec_ / 1e9, 3),
            "unit": "GB/s",
            "cores": used,
            "kind": "oracle",
            "sample": ("the full 197-matvec step (set 0) computed by the oracle, "
                       "rows split over the host cores; median of up to 3 runs"),
            "step_latency_us": round(csec_ * 1e6, 1),
            "gpu_parity_max_err_over_tol": round(worst, 5),
            "gpu_argmax_accepted": bool(ok_idx),
        }
    print(json.dumps(result), flush=True)
    for g in pers + bare:
        g.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
