"""Benchmark of the SNACK COO layer's hot path on one MI355X.

A step is one forward (Y = X W^T + b), one input gradient (dX = dY W) and one
weight gradient (dW on the stored entries) of one sparse layer, inputs already
resident in HBM.  Default workload: a 10000 x 10000 layer at 95 % sparsity
(5,000,000 stored entries, uniform positions), batch 64, fp32.

Prints one JSON line: the metric (microseconds per fwd+dX+dW step), the
roofline of the dominant kernel (algorithmic HBM bytes per launch over its
average duration, timed with HIP events that bracket exactly that kernel), and
the fp64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
COLD_CALLS = 50        # flushed launches behind each cold median

# The values of a layer's weight are kept in the order that makes its step fastest: column-view
# order ("col": the one-pass tiled backward reads them and writes dW in place, the forward reads
# them through a permutation) at batches of one 64-column tile, triple order ("row") elsewhere.
WORKLOADS = {
    # name: (layer, batch, dtype, value order)
    "target95_b64": ("target95", 64, "f32", "col"),
    "target95_b64_bf16": ("target95", 64, "bf16", "col"),
    "target95_b1": ("target95", 1, "f32", "row"),
    "llm90_b64": ("llm90", 64, "f32", "col"),
    "llm90_b16": ("llm90", 16, "f32", "col"),
    "llm90_b1": ("llm90", 1, "f32", "row"),
    "mid_b32": ("mid", 32, "f32", "row"),
    "xs99_b1": ("xs99", 1, "f32", "row"),
    "xs999_b1": ("xs999", 1, "f32", "row"),
    "xs99_zipf_b1": ("xs99_zipf", 1, "f32", "row"),
    "gpt2_fc_b1024": ("gpt2_fc", 1024, "f32", "row"),
    "gpt2_fc_b1024_bf16": ("gpt2_fc", 1024, "bf16", "row"),
    # bf16 activations and bf16 weights on the matrix cores (SNACK_BF16_HW)
    "target95_b64_bf16hw": ("target95", 64, "bf16hw", "col"),
    "gpt2_fc_b1024_bf16hw": ("gpt2_fc", 1024, "bf16hw", "row"),
    "gamlp90_b4096_bf16": ("gamlp90", 4096, "bf16", "row"),
    "gamlp90_b4096_bf16hw": ("gamlp90", 4096, "bf16hw", "row"),
    "gamlp90_b1": ("gamlp90", 1, "f32", "row"),
    "gamlp90_b4096": ("gamlp90", 4096, "f32", "row"),
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(op, nnz, O, I, B, s):
    """Bytes the method itself must move per launch (HBM), s = activation bytes."""
    if op == "fwd":
        return 12 * nnz + s * B * I + s * B * O + 4 * O
    if op == "dx":
        return 12 * nnz + s * B * O + s * B * I
    if op == "bwd":  # both gradients: the triple once, dW written; dY and X read, dX written
        return 16 * nnz + s * B * O + 2 * s * B * I
    return 12 * nnz + s * B * I + s * B * O  # dw: rows, cols, write dW; read X and dY


def dtype_code(dtype):
    import coo_spmm_row_amd as snk
    return {"f32": snk.SNACK_F32, "bf16": snk.SNACK_BF16, "bf16hw": snk.SNACK_BF16_HW}[dtype]


def bwd_fused(layer):
    """Whether snack_coo_bwd runs its single column-view pass for this layer and batch (the
    library's own choice, snack_coo_bwd_is_fused); otherwise it runs the two gradients as separate
    passes and the step's dominant kernel is one of the three products.  Labels timings only."""
    import coo_spmm_row_amd as snk
    return snk.snack_coo_bwd_is_fused(layer.W, layer.B, dtype_code(layer.dtype))


def other_order_step(layer, K):
    """The same step on the same layer with its values kept in the other order (triple order for a
    layer in column-view order, and the reverse): graph-replayed step time and per-kernel times.
    The layer is restored."""
    import torch
    import coo_spmm_row_amd as snk
    W0, ws0 = layer.W, layer.ws
    layer.W = W0.to_row_order() if W0.column_order else W0.to_column_order()
    code = dtype_code(layer.dtype)
    need = max(snk.snack_coo_workspace_bytes(op, layer.W, layer.B, code) for op in (0, 1, 2, 3))
    layer.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=ws0.device)
    try:
        for _ in range(3):
            layer.step()
        torch.cuda.synchronize()
        e = plain_steps(layer, K)
        g = graph_steps(layer, K)
        _, kern = timed_steps(layer, K)
        return {"us_per_step_eager": round(e, 2), "us_per_step_graph": None if g is None else round(g, 2),
                "kernel_us": {op: round(float(np.mean(v)) * 1000.0, 2) for op, v in kern.items()}}
    finally:
        layer.W, layer.ws = W0, ws0


def half_weights_step(dev, K):
    """The headline layer (10k x 10k, 95 %, batch 64, values in column order) with bf16
    activations, once through the bf16 kernels (fp32 weights) and once through the half-precision
    path (weights rounded to bf16, forward and input gradient on the matrix cores): eager step and
    kernel times of the forward, the input gradient and the weight gradient."""
    import torch
    out = {}
    for dt in ("bf16", "bf16hw"):
        lay = Layer("target95", 64, dt, dev, "col")
        for _ in range(20):
            lay.step()
        torch.cuda.synchronize()
        e = plain_steps(lay, K)
        _, kern = timed_steps(lay, K, ("fwd", "dx", "dw"))
        out["half_weights" if dt == "bf16hw" else "bf16_weights_fp32"] = {
            "us_per_step_eager": round(e, 2),
            "kernel_us": {op: round(float(np.mean(v)) * 1000.0, 2) for op, v in kern.items()}}
        del lay
        torch.cuda.empty_cache()
    return out


def kernel_source_sha():
    """sha256[:16] over the library's device sources (csrc/*.hip and csrc/*.h, by name)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "coo_spmm_row_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode() + b"\0")
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


class Layer:
    def __init__(self, name, B, dtype, dev, order="row"):
        import torch
        import coo_spmm_row_amd as snk
        import synth
        spec = synth.LAYERS[name]
        t0 = time.time()
        L = synth.make_layer(spec)
        built = snk.snack_coo_build(L["out_features"], L["in_features"], L["rows"], L["cols"], L["vals"])
        self.host_build_s = time.time() - t0
        self.spec, self.L, self.built, self.B, self.dtype = spec, L, built, B, dtype
        self.O, self.I, self.nnz = L["out_features"], L["in_features"], L["nnz"]
        self.W = snk.SnackCOO.from_built(built, dev)
        if order == "col":  # values (and dW) in column-view order
            self.W = self.W.to_column_order()
        self.order = order
        seeds = synth.seeds_for(spec.config_id, spec.variant)
        self.x = synth.make_acts(seeds["X"](0), B, self.I)
        self.dy = synth.make_acts(seeds["dY"](0), B, self.O)
        tdt = torch.float32 if dtype == "f32" else torch.bfloat16
        self.X = torch.from_numpy(self.x).to(dev).to(tdt)
        self.dY = torch.from_numpy(self.dy).to(dev).to(tdt)
        self.bias = torch.from_numpy(L["bias"]).to(dev)
        self.Y = torch.empty((B, self.O), dtype=tdt, device=dev)
        self.dX = torch.empty((B, self.I), dtype=tdt, device=dev)
        self.dW = torch.empty(self.nnz, dtype=torch.float32, device=dev)
        code = dtype_code(dtype)
        need = max(snk.snack_coo_workspace_bytes(op, self.W, B, code) for op in (0, 1, 2, 3))
        self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        self.s = 4 if dtype == "f32" else 2
        self.hw = dtype == "bf16hw"  # weights rounded to bf16, products on the matrix cores

    def op(self, name):
        import coo_spmm_row_amd as snk
        hw = self.hw
        if name == "fwd":
            snk.snack_coo_fwd(self.W, self.X, self.bias, out=self.Y, workspace=self.ws, half_weights=hw)
        elif name == "dx":
            snk.snack_coo_bwd_input(self.W, self.dY, out=self.dX, workspace=self.ws, half_weights=hw)
        elif name == "dw":
            snk.snack_coo_grad_weight(self.W, self.X, self.dY, out=self.dW, workspace=self.ws, half_weights=hw)
        else:  # both gradients in one call
            snk.snack_coo_bwd(self.W, self.X, self.dY, dx_out=self.dX, dw_out=self.dW, workspace=self.ws,
                              half_weights=hw)

    def step(self):
        """One layer step: the forward and both gradients (snack_coo_bwd)."""
        self.op("fwd")
        self.op("bwd")


STEP_OPS = ("fwd", "bwd")          # what a step runs
SPLIT_OPS = ("fwd", "dx", "dw")    # the three products as separate calls (reported beside)


def make_events(n):
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()  # creates the underlying HIP event
    return evs


def plain_steps(layer, K):
    """K back-to-back steps, eager, with events only around the whole region: us per step."""
    import torch
    start, stop = make_events(2)
    torch.cuda.synchronize()
    start.record()
    for _ in range(K):
        layer.step()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / K * 1000.0


def timed_steps(layer, K, ops=STEP_OPS):
    """K back-to-back passes over `ops`; the probe brackets each op's main kernel.
    Returns (total ms, {op: [kernel ms per launch]}).  The events between the kernels make each
    step slower than plain_steps (each event write-back releases the caches): step times come
    from plain_steps or graph_steps, kernel times from here."""
    import torch
    import coo_spmm_row_amd as snk
    pairs = {op: [(a, b) for a, b in zip(make_events(K), make_events(K))] for op in ops}
    start, stop = make_events(2)
    torch.cuda.synchronize()
    start.record()
    for i in range(K):
        for op in ops:
            a, b = pairs[op][i]
            snk.snack_coo_set_probe(a, b)
            layer.op(op)
    snk.snack_coo_set_probe()
    stop.record()
    torch.cuda.synchronize()
    total = start.elapsed_time(stop)
    kern = {op: [a.elapsed_time(b) for a, b in pairs[op]] for op in ops}
    return total, kern


def graph_steps(layer, K, reps=3, ops=None):
    """The step (or just `ops`) captured once as a HIP graph and replayed K times (no host launch
    cost).  Returns microseconds per replay (median over reps), or None if capture fails."""
    import torch

    def run():
        if ops is None:
            layer.step()
        else:
            for op in ops:
                layer.op(op)
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        graph.replay()
        torch.cuda.synchronize()
    except RuntimeError as exc:  # capture unsupported: report eager only
        log(f"graph capture failed: {exc}")
        return None
    times = []
    for _ in range(reps):
        a, b = make_events(2)
        torch.cuda.synchronize()
        a.record()
        for _ in range(K):
            graph.replay()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) / K * 1000.0)
    return float(np.median(times))


def op_times(layer, K, ops=STEP_OPS + ("dx", "dw")):
    """Per-op wall time on the stream (all kernels of the op), back to back."""
    import torch
    out = {}
    for op in ops:
        a, b = make_events(2)
        torch.cuda.synchronize()
        a.record()
        for _ in range(K):
            layer.op(op)
        b.record()
        torch.cuda.synchronize()
        out[op] = a.elapsed_time(b) / K * 1000.0
    return out


def cold_kernel_times(layer, K, ops, flush_bytes=1 << 30, write_flush=False):
    """Main-kernel time per op with L2 and the 256 MB last-level cache flushed before each launch
    by reading flush_bytes.  A read stream leaves clean lines behind; a write stream
    (write_flush=True) leaves dirty ones, whose write-back the measured kernel then pays for as
    it brings its own data in (about 14 us more on the 10k x 10k / 95 % / batch 64 backward)."""
    import torch
    import coo_spmm_row_amd as snk
    scratch = torch.zeros(flush_bytes // 4, dtype=torch.float32, device=layer.X.device)
    res = {}
    for op in ops:
        evs = [(a, b) for a, b in zip(make_events(K), make_events(K))]
        for i in range(K):
            if write_flush:
                scratch.add_(1.0)  # reads and writes flush_bytes
            else:
                scratch.sum()  # reads flush_bytes
            snk.snack_coo_set_probe(*evs[i])
            layer.op(op)
            snk.snack_coo_set_probe()
        torch.cuda.synchronize()
        res[op] = float(np.median([a.elapsed_time(b) for a, b in evs])) * 1000.0
    del scratch
    return res


def profile_op(layer, op, K, W, flush):
    """Counter runs (rocprofv3 --pmc): W warm-up steps, then K calls of one op (or of the step),
    each after a 1 GiB read when flush == "read".  Prints one JSON line."""
    import torch
    scratch = torch.zeros((1 << 30) // 4, dtype=torch.float32, device=layer.X.device) if flush == "read" else None
    for _ in range(W):
        layer.step()
    torch.cuda.synchronize()
    for _ in range(K):
        if scratch is not None:
            scratch.sum()
        if op == "step":
            layer.step()
        else:
            layer.op(op)
    torch.cuda.synchronize()
    print(json.dumps({"profile_op": op, "calls": K, "warmup_steps": W, "flush": flush}), flush=True)


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(layer, budget_s=15.0, single_budget_s=10.0):
    """The fp64 oracle on the first Bs batch rows of the same inputs, scaled to the full batch: on
    the host threads this process may use (at most 16, the CPU share of one GPU), and on one."""
    import oracle
    nthreads = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity")
                          else (os.cpu_count() or 1)))
    b = layer.built
    r, c, v = b["rows"], b["cols"], b["vals"]
    O, I, B = layer.O, layer.I, layer.B
    x = layer.x.astype(np.float64)
    dy = layer.dy.astype(np.float64)

    def run(bs, nt):
        t0 = time.perf_counter()
        oracle.fwd(O, I, r, c, v, x[:bs], layer.L["bias"], nthreads=nt)
        oracle.bwd_input(O, I, r, c, v, dy[:bs], nthreads=nt)
        oracle.grad_weight(O, I, r, c, x[:bs], dy[:bs], nthreads=nt)
        return time.perf_counter() - t0

    def measure(nt, budget):
        # grow the batch sample until one pass costs >= budget/8, then repeat passes to ~budget
        bs = 1
        t = run(bs, nt)
        while bs < B and t * 8 < budget:
            bs = min(B, bs * 2)
            t = run(bs, nt)
        reps, total = 1, t
        while total < budget and reps < 2000:
            total += run(bs, nt)
            reps += 1
        return total / reps * 1e6 * (B / bs), bs, reps, total

    us, bs, reps, total = measure(nthreads, budget_s)
    us1, bs1, reps1, total1 = measure(1, single_budget_s)
    model = cpu_model()
    return {"value": round(us, 1), "unit": "us/step (fwd+dX+dW)", "cores": nthreads,
            "kind": "oracle",
            "sample": f"fp64 oracle fwd+dX+dW on the first {bs} of {B} batch rows of the same layer, "
                      f"{reps} passes ({total:.1f} s), scaled by {B}/{bs}; {nthreads} threads of a {model}",
            "cpu_model": model,
            "single_core": {"value": round(us1, 1), "cores": 1,
                            "sample": f"the same on one thread: first {bs1} of {B} rows, {reps1} passes "
                                      f"({total1:.1f} s), scaled by {B}/{bs1}"}}


def traffic_for(workload, kernel):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(workload, {})
    except (OSError, ValueError):
        return None
    if rec.get("kernel") != kernel or rec.get("source_sha") != kernel_source_sha():
        return None  # counters were taken on another kernel version
    return rec.get("traffic_bytes")


def batch_sweep(dev, K, batches=(16, 32)):
    """The step (eager and graph-replayed, us) at small batches on the 10k x 10k layers at 90 and 95 %: the
    metric's batch range below 64, values in column order as in the headline workload, with the
    backward's form and the per-op kernel times."""
    out = {}
    for name, label in (("llm90", "90%"), ("target95", "95%")):
        for B in batches:
            layer = Layer(name, B, "f32", dev, "col")
            for _ in range(3):
                layer.step()
            e = plain_steps(layer, K)
            g = graph_steps(layer, K)
            _, kern = timed_steps(layer, K)
            out[f"{label} B={B}"] = {"us_per_step_eager": round(e, 2),
                                     "us_per_step_graph": None if g is None else round(g, 2),
                                     "backward_fused": bwd_fused(layer),
                                     "kernel_us": {op: round(float(np.mean(kern[op])) * 1000.0, 2)
                                                   for op in STEP_OPS}}
            del layer
    return out


def batch1_sweep(dev, K):
    """Batch-1 fwd+dX+dW latency at every sparsity level of the 10k x 10k layer."""
    out = {}
    for name, label in (("llm90", "90%"), ("target95", "95%"), ("xs99", "99%"), ("xs999", "99.9%")):
        layer = Layer(name, 1, "f32", dev)
        for _ in range(3):
            layer.step()
        eager = plain_steps(layer, K)
        g = graph_steps(layer, K)
        _, kern = timed_steps(layer, K, SPLIT_OPS)  # at batch 1 the gradients run as two kernels
        out[label] = {"us_per_step_eager": round(eager, 2),
                      "us_per_step_graph": None if g is None else round(g, 2),
                      "kernel_us": {op: round(float(np.mean(kern[op])) * 1000.0, 2) for op in SPLIT_OPS}}
        del layer
    return out


def module_step_us(layer, K):
    """The same layer step through the PyTorch drop-in (SnackLinear: autograd forward and
    backward, plus the bias gradient the raw step does not take), eager, us per step."""
    import torch
    from coo_spmm_row_amd.layer import SnackLinear
    m = SnackLinear.from_triple(layer.O, layer.I, layer.built["rows"], layer.built["cols"], layer.built["vals"],
                                layer.L["bias"], device=layer.X.device)
    X = layer.X.detach().clone().requires_grad_(True)
    G = layer.dY
    for _ in range(3):
        m(X).backward(G)
    start, stop = make_events(2)
    torch.cuda.synchronize()
    start.record()
    for _ in range(K):
        m.zero_grad(set_to_none=True)
        X.grad = None
        m(X).backward(G)
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / K * 1000.0


def topology_times(layer, frac=0.1, reps=3):
    """Prune-and-regrow of the layer (floor(frac * nnz) entries) with its column view: on the
    device (snack_coo_topology_update_device, which synchronizes; wall clock) and on the host
    (snack_coo_topology_update + snack_coo_build, host arrays; copies not included). ms, best of reps."""
    import torch
    import coo_spmm_row_amd as snk
    p = int(frac * layer.nnz)
    r, c, v = layer.built["rows"], layer.built["cols"], layer.built["vals"]
    W = layer.W.to_row_order()  # the update works on the triple with its values in row order
    snk.snack_coo_topology_update_device(W, p, 7)  # warm-up (first launch of the sort kernels)
    dev_ms, host_ms = [], []
    for i in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        Wn, trials = snk.snack_coo_topology_update_device(W, p, 100 + i)
        torch.cuda.synchronize()
        dev_ms.append((time.perf_counter() - t0) * 1e3)
        del Wn
        t0 = time.perf_counter()
        out = snk.snack_coo_topology_update(layer.O, layer.I, r, c, v, p, 100 + i)
        snk.snack_coo_build(layer.O, layer.I, out["rows"], out["cols"], out["vals"])
        host_ms.append((time.perf_counter() - t0) * 1e3)
    return {"n_prune": p, "device_ms": round(min(dev_ms), 2), "host_ms": round(min(host_ms), 1)}


def gamlp_inference(dev, K):
    """Batch-1 forward of the 5000 x 5000 GAMLP-shaped projection at 90 / 95 / 99 % sparsity: us
    per call replayed as a one-call HIP graph (includes the graph launch), and the main kernel's
    time from the probe events."""
    out = {}
    for name, label in (("gamlp90", "90%"), ("gamlp95", "95%"), ("gamlp99", "99%")):
        layer = Layer(name, 1, "f32", dev)
        for _ in range(3):
            layer.op("fwd")
        g = graph_steps(layer, K, ops=("fwd",))
        _, kern = timed_steps(layer, K, ("fwd",))
        out[label] = {"graph_us": None if g is None else round(g, 2),
                      "kernel_us": round(float(np.mean(kern["fwd"])) * 1000.0, 2)}
        del layer
    return out


def copy_peak_gbs(dev, nbytes=1 << 30, reps=20):
    """A plain device copy of nbytes (read nbytes, write nbytes), median over reps: the box's own
    streaming rate, GB/s of reads plus writes."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ts = []
    for _ in range(reps):
        a, b = make_events(2)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3)
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / float(np.median(ts)) / 1e9


def calibrate_copy(dev, nbytes, reps):
    """A plain elementwise kernel of known size (reads nbytes, writes nbytes), for
    scaling the HBM byte counters."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.mul(src, 2.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the default warm-up (about 0.1 s at the headline shape) lets the host and the GPU reach their
    # steady clocks after the layer build: with 10 steps the eager step measured 109 us, with 1000
    # steps 96.5 us, the kernels themselves unchanged
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default="target95_b64", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip cold-cache and batch-1 sweeps")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES")
    ap.add_argument("--profile-op", choices=("fwd", "bwd", "dx", "dw", "step"),
                    help="for counter runs: only --steps calls of this op after --warmup steps")
    ap.add_argument("--flush", choices=("none", "read"), default="none",
                    help="with --profile-op: a 1 GiB read before each call (the cold-cache runs)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(each GPU would own a range of the weight's rows balanced by entries); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import coo_spmm_row_amd as snk  # noqa: F401  (fails loudly if the library is missing)
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        calibrate_copy(dev, args.calibrate_copy, max(1, args.steps))
        return

    name, B, dtype, order = WORKLOADS[args.workload]
    log(f"workload {args.workload}: building layer")
    layer = Layer(name, B, dtype, dev, order)
    if args.profile_op:
        profile_op(layer, args.profile_op, args.steps, args.warmup, args.flush)
        return
    log(f"layer {layer.O}x{layer.I} nnz={layer.nnz} B={B} {dtype} (host build {layer.host_build_s:.1f} s)")
    for _ in range(args.warmup):
        layer.step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    eager_us = plain_steps(layer, args.steps)
    log("timing the step as a replayed HIP graph")
    graph_us = graph_steps(layer, args.steps)
    # the step as launched eagerly or as one replayed graph, whichever is faster (both reported)
    step_us = eager_us if graph_us is None else min(eager_us, graph_us)
    step_timing = "eager" if step_us == eager_us else "graph"
    ms_per_step = step_us / 1000.0
    log("kernel times (probe events around each op's main kernels)")
    _, kern = timed_steps(layer, args.steps)
    _, kern_split = timed_steps(layer, args.steps, ("dx", "dw"))
    kern.update(kern_split)
    all_ops = STEP_OPS + ("dx", "dw")
    kernel_us = {op: float(np.mean(kern[op])) * 1000.0 for op in all_ops}
    kernel_pct = {op: {f"p{q}": round(float(np.percentile(kern[op], q)) * 1000.0, 2) for q in (10, 50, 90)}
                  for op in all_ops}
    # the dominant kernel of the step (the fused backward pass when the batch allows it)
    cand = STEP_OPS if bwd_fused(layer) else SPLIT_OPS
    dom = max(cand, key=lambda o: kernel_us[o])
    kname = {"fwd": "forward gather-reduce", "dx": "input-gradient gather-reduce",
             "dw": "weight-gradient sampled product", "bwd": "backward pass (dX and dW in one pass)"}[dom]
    nbytes = {op: algorithmic_bytes(op, layer.nnz, layer.O, layer.I, B, layer.s) for op in all_ops}
    # the roofline of the dominant kernel from its cold median (L2 and the 256 MB last-level cache
    # flushed by a read stream before each of COLD_CALLS launches), the warm back-to-back mean
    # beside it
    log(f"cold-cache timing of the dominant kernel ({COLD_CALLS} flushed calls)")
    cold_dom = cold_kernel_times(layer, COLD_CALLS, (dom,))[dom]
    achieved = nbytes[dom] / (cold_dom * 1e-6) / 1e9
    achieved_warm = nbytes[dom] / (kernel_us[dom] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic_for(args.workload, dom),
                "kernel": kname, "kernel_us": round(cold_dom, 2), "timing": f"cold median of {COLD_CALLS} calls (caches flushed by a 1 GiB read)",
                "warm": {"achieved": round(achieved_warm, 1), "frac": round(achieved_warm / HBM_PEAK_GBS, 4),
                         "kernel_us": round(kernel_us[dom], 2), "timing": f"mean of {args.steps} back-to-back calls"},
                "algorithmic_bytes": nbytes[dom]}
    log("stream-copy rate of the box (1 GiB device copy)")
    cp = copy_peak_gbs(dev)
    roofline["copy_peak"] = {"achieved_gbs": round(cp, 1), "frac": round(achieved / cp, 4),
                             "note": "cold achieved GB/s against a plain 1 GiB device copy on this box"}
    extras = {"us_per_step_eager": round(eager_us, 2),
              "us_per_step_graph": None if graph_us is None else round(graph_us, 2),
              "step_timing": step_timing,
              "backward_fused": bwd_fused(layer),
              "kernel_us": {op: round(v, 2) for op, v in kernel_us.items()},
              "kernel_us_percentiles": kernel_pct,
              "kernel_frac_hbm": {op: round(nbytes[op] / (kernel_us[op] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                                  for op in all_ops}}
    if not args.no_extras:
        log("op-level and cold-cache timings")
        extras["op_us"] = {op: round(v, 2) for op, v in op_times(layer, args.steps).items()}
        cold = cold_kernel_times(layer, COLD_CALLS, cand)
        extras["kernel_us_cold"] = {op: round(v, 2) for op, v in cold.items()}
        extras["kernel_frac_hbm_cold"] = {op: round(nbytes[op] / (cold[op] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                                          for op in cand}
        coldw = cold_kernel_times(layer, COLD_CALLS, (dom,), write_flush=True)
        extras["kernel_us_cold_write_flush"] = {dom: round(coldw[dom], 2)}
        log("the step through the PyTorch drop-in layer")
        extras["module_us_per_step_eager"] = round(module_step_us(layer, args.steps), 2)
        log("topology update (prune 10 %, regrow, column view): device and host")
        extras["topology_update"] = topology_times(layer)
        other = "row_order_values" if order == "col" else "column_order_values"
        log(f"the step with the values in the other order ({other})")
        extras[other] = other_order_step(layer, args.steps)
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(layer)
    if not args.no_extras and B != 1:
        log("batch-1 sweep over sparsity")
        del layer
        torch.cuda.empty_cache()
        extras["batch1_us_per_step"] = batch1_sweep(dev, max(10, args.steps // 2))
        log("batch 16 and 32 steps")
        extras["small_batch_us_per_step"] = batch_sweep(dev, max(10, args.steps // 2))
        log("GAMLP-shaped batch-1 inference")
        extras["gamlp_5000_b1_fwd_us"] = gamlp_inference(dev, max(20, args.steps))
        log("bf16 activations with fp32 and with half-precision weights")
        extras["bf16_step_weights"] = half_weights_step(dev, max(10, args.steps // 2))
    line = {
        "metric": "COO SpMM fwd+dX+dW us/call (one layer step)",
        "value": round(step_us, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if dtype == "bf16hw" else dtype,
        "data": "synthetic (seeded uniform positions, N(0,1) activations)",
        "config": {},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extras": extras,
    }
    import synth
    spec = synth.LAYERS[name]
    line["config"] = {"workload": f"{spec.out_features}x{spec.in_features} sparse layer, "
                                  f"{100 * (1 - spec.density):.1f}% sparsity, batch {B}",
                      "out_features": spec.out_features, "in_features": spec.in_features,
                      "nnz": spec.nnz, "batch": B, "structure": spec.structure,
                      "value_order": {"col": "column view", "row": "triple (row)"}[order]}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
