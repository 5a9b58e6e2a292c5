#!/usr/bin/env python3
"""Throughput of the fused equivariant convolution on one MI355X.

Default workload: the training step of the MACE-scale graph (N=20000 nodes,
~596k directed edges from a radius graph, 128x0e+128x1o features, spherical
harmonics to lmax 3, output 128x(0e+1o+2e+3o), fp32): one step is the fused
forward plus the fused reverse pass (grad x, grad y, grad s) over the whole
graph.  Inputs are seeded synthetic data, resident in HBM before timing; the
plan and the receiver CSR are built once per graph, outside the timed region
(reported separately).

Prints one JSON line: edges/s of whole steps, plus the roofline of the
dominant kernel (algorithmic bytes / average duration from HIP events on the
launch stream, against HBM; algorithmic flops against the vector-ALU peak
when the kernel's arithmetic intensity is above the ridge point), the CPU
oracle timed on the whole workload over the host cores with the full-output
parity of the GPU result against it, and the forwards of the MACE-scale and
large bf16 workloads against both roofs.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0   # MI355X HBM3E, AMD published
PEAK_FP32_MFMA_TFLOPS = 157.3   # MI355X dense fp32 matrix, AMD published
PEAK_FP16_MFMA_TFLOPS = 2500.0   # MI355X dense fp16/bf16 matrix, AMD published
# Vector fp32 FMA without packed math: 256 CUs x 4 SIMDs x 16 lanes x 2 flops x
# 2.4 GHz (a wave-64 instruction occupies its SIMD for four cycles).  The
# published 157.3 TFLOP/s counts packed FP32, which this build does not emit.
PEAK_FP32_VALU_TFLOPS = 78.6
METRIC = "edges/sec + achieved HBM GB/s (% of peak) for fused TP conv fwd/bwd, 1 MI355X"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=4, help="0..4; 4 = training step (fwd+bwd)")
    ap.add_argument("--fwd-variant", type=int, default=0)
    ap.add_argument("--bwd-variant", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-order", action="store_true",
                    help="process receivers in index order (no locality schedule)")
    ap.add_argument("--cluster", type=int, default=512, help="receivers per locality cluster")
    ap.add_argument("--cpu-sample-edges", type=int, default=12000,
                    help="edges of the single-threaded oracle sample of the --mode variants")
    ap.add_argument("--no-extra", action="store_true",
                    help="default run: skip the extra forward figures of workloads 2 and 3")
    ap.add_argument("--eager", action="store_true",
                    help="time the training step as eager launches only (default: the step "
                         "captured once in a HIP graph and replayed is the headline, eager figures "
                         "beside it; a forward-only step is one kernel launch and always eager)")
    ap.add_argument("--sweep", action="store_true",
                    help="time every compiled kernel variant (one JSON line each) and exit")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="run a plain device copy of MIB MiB (counter calibration) and exit")
    ap.add_argument("--mode", default="conv",
                    choices=("conv", "sender", "jvp", "second", "linear", "radial", "pairs"),
                    help="conv: the hot path (default); sender: SENDER graph ordering; "
                         "jvp: fused forward-mode pass; second: second derivatives of the "
                         "training step; linear: output linear; radial: edge scalars from "
                         "edge lengths in the kernel (gate-points workload); pairs: reverse pass "
                         "with y and s stored once per undirected pair against the directed "
                         "reverse pass on the same symmetric graph (one line each)")
    return ap.parse_args()


def calibrate_copy(mib, reps=5):
    """A plain device-to-device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE.

    Also reports the streaming rates this device attains outside the
    convolution: the copy (read + write) and a read-only reduction.
    """
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    from equivariant_gnn_message_amd import e3conv as E
    for _ in range(reps):
        E.e3conv_stream_reference(a, b)
        E.e3conv_stream_reference(a)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ev[0].record()
    for _ in range(reps):
        b.copy_(a)
    ev[1].record()
    for _ in range(reps):
        E.e3conv_stream_reference(a, b)
    ev[2].record()
    for _ in range(reps):
        E.e3conv_stream_reference(a)
    ev[3].record()
    torch.cuda.synchronize()
    ms = [ev[i].elapsed_time(ev[i + 1]) / reps for i in range(3)]
    print(json.dumps({"calibrate_copy_bytes": n * 4, "reps": reps,
                      "runtime_copy_GBps": 2 * n * 4 / ms[0] / 1e6,
                      "stream_copy_GBps": 2 * n * 4 / ms[1] / 1e6,
                      "stream_read_GBps": n * 4 / ms[2] / 1e6}), flush=True)


def sweep(plan, w, run_fwd, run_bwd, nbytes, orders, reps=10):
    """Average HIP-event time of every compiled variant, with each receiver order."""
    import numpy as np
    import torch
    from equivariant_gnn_message_amd import e3conv as E
    dt = E.E3CONV_BF16 if w.dtype == "bf16" else E.E3CONV_F32
    nf, nb = plan.num_variants(dt)
    for kind, n, run, by in (("fwd", nf, run_fwd, nbytes[0]), ("bwd", nb if w.backward else 0, run_bwd, nbytes[1])):
        for v in range(n):
            for oname, order in orders:
                plan.set_variant(v if kind == "fwd" else 0, v if kind == "bwd" else 0)
                run(order)
                torch.cuda.synchronize()
                ts = []
                for _ in range(reps):
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record()
                    run(order)
                    b.record()
                    ts.append((a, b))
                torch.cuda.synchronize()
                ms = float(np.mean([a.elapsed_time(b) for a, b in ts]))
                print(json.dumps({"workload": w.idx, "kernel": kind, "variant": v, "order": oname,
                                  "ms": ms, "GBps": by / ms / 1e6,
                                  "frac": by / ms / 1e6 / PEAK_HBM_GBPS}), flush=True)


def alg_bytes(w, N, E, b_in):
    """Compulsory bytes: every input read once, every output written once."""
    C, nx, ny, no, P = w.channels, w.num_x, (w.lmax + 1) ** 2, w.num_out, w.num_paths
    fwd = N * nx * C * b_in + E * (ny * b_in + P * C * b_in + 4) + 4 * (N + 1) + N * no * C * 4
    bwd = 4 * (2 * N * nx * C + N * no * C + (N + 1) + E * (2 * ny + 2 * P * C + 1))
    return fwd, bwd


def _conv_counts(plan):
    import numpy as np
    ix, iy, ip, io, v = (np.asarray(a) for a in plan.coefficients())
    nz = v != 0
    nnz = int(nz.sum())
    nnz_k = len(set(zip(ip[nz].tolist(), ix[nz].tolist(), io[nz].tolist())))
    smul = sum(min(2 * q["l1"] + 1, 2 * q["l3"] + 1) for q in plan.paths())
    return nnz, nnz_k, smul


def forward_flops_per_edge(plan):
    """Arithmetic the forward needs per edge with K^p(y) built once per edge:
    2 flops per CG term for K, then per channel one product per nonzero of
    each K^p and min(2 l1 + 1, 2 l3 + 1) products for the scalar s (applied
    before or after K, whichever is smaller)."""
    nnz, nnz_k, smul = _conv_counts(plan)
    return 2 * nnz + 2 * plan.channels * (nnz_k + smul)


def jvp_flops_per_edge(plan):
    """Forward mode: K(y) and K(dy) per edge; per channel K(y)(s x),
    K(y)(s dx + ds x) and K(dy)(s x)."""
    nnz, nnz_k, smul = _conv_counts(plan)
    return 4 * nnz + 6 * plan.channels * (nnz_k + smul)


def roofline(kernel, ms, nbytes, flops=None, traffic=None):
    """The roof of a kernel is HBM unless its arithmetic at the vector-ALU
    peak takes longer than its bytes at the HBM peak (above the ridge)."""
    gbps = nbytes / (ms * 1e-3) / 1e9
    r = {"bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
         "frac": gbps / PEAK_HBM_GBPS, "traffic": traffic, "kernel": kernel, "algorithmic_bytes": nbytes}
    if flops and flops / PEAK_FP32_VALU_TFLOPS / 1e12 > nbytes / PEAK_HBM_GBPS / 1e9:
        tf = flops / (ms * 1e-3) / 1e12
        r.update({"bound": "alu", "achieved": tf, "peak": PEAK_FP32_VALU_TFLOPS, "unit": "TFLOP/s",
                  "frac": tf / PEAK_FP32_VALU_TFLOPS, "algorithmic_flops": flops,
                  "hbm_GBps": gbps, "hbm_frac": gbps / PEAK_HBM_GBPS})
    return r


def kernel_source_files():
    """Every device source: the .hip files and every header except the host builder's."""
    csrc = os.path.join(ROOT, "equivariant_gnn_message_amd", "csrc")
    return sorted(f for f in os.listdir(csrc)
                  if f.endswith(".hip") or (f.endswith(".h") and f != "host_core.h"))


def strip_comments(src):
    """C/C++ source without comments and with whitespace runs collapsed (code only)."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash():
    """sha256[:16] of the code of the device sources (every .hip file and the kernel
    headers), comments and layout whitespace excluded: an edit of the comments
    leaves the counter records of unchanged kernels valid."""
    h = hashlib.sha256()
    for f in kernel_source_files():
        with open(os.path.join(ROOT, "equivariant_gnn_message_amd", "csrc", f)) as fh:
            h.update(strip_comments(fh.read()).encode())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if still current."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_w{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def host_cores():
    """Cores this process may use: its affinity set, capped by OMP_NUM_THREADS and by 16 (the
    host share of one GPU on the MI355X boxes)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, min(16, n))


_POOL = {}   # operands and shared result buffers inherited by the forked oracle workers


def _shared_f64(shape):
    """A float64 array in an anonymous shared mapping (written by forked workers)."""
    import mmap
    import numpy as np
    n = int(np.prod(shape)) * 8
    buf = mmap.mmap(-1, max(n, 8))
    return np.frombuffer(buf, dtype=np.float64, count=int(np.prod(shape))).reshape(shape)


def _oracle_chunk(k):
    """Worker: oracle forward (and reverse) on the receiver-aligned edge range k."""
    from threadpoolctl import threadpool_limits

    from oracle import conv
    P = _POOL
    e0, e1 = P["bounds"][k], P["bounds"][k + 1]
    b0, b1 = P["rows"][k], P["rows"][k + 1]
    with threadpool_limits(1):
        if e1 > e0:
            rcv = P["receivers"][e0:e1] - b0
            P["out"][b0:b1] = conv.forward(P["lay"], P["x"], P["y"][e0:e1], P["s"][e0:e1],
                                           P["senders"][e0:e1], rcv, b1 - b0)
            if P["backward"]:
                dx, dy, ds = conv.backward(P["lay"], P["x"], P["y"][e0:e1], P["s"][e0:e1], P["g"],
                                           P["senders"][e0:e1], P["receivers"][e0:e1], P["num_nodes"])
                P["dx"][k] = dx
                P["dy"][e0:e1] = dy
                P["ds"][e0:e1] = ds
    return e1 - e0


def cpu_baseline(inp, with_backward, workers):
    """The oracle, as it stands, on the whole workload: the receivers are cut into `workers`
    ranges of about equal edge counts, each run by one single-threaded process (forked before
    the GPU is touched, so no worker holds a device).  Returns the baseline record and the
    oracle's outputs (out, and dx, dy, ds with the reverse pass) for the parity check."""
    import multiprocessing as mp
    import numpy as np

    from oracle import conv, so3

    w = inp.workload
    lay = conv.make_layout(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    for q in lay.paths:                       # CG tables built once, outside the timed region
        so3.real_cg(q.l1, q.l2, q.l3)
    N, E = inp.num_nodes, inp.num_edges
    ptr = np.searchsorted(inp.receivers, np.arange(N + 1))
    cuts = np.searchsorted(ptr, np.linspace(0, E, workers + 1), side="left")
    cuts[0], cuts[-1] = 0, N
    rows = np.maximum.accumulate(cuts)
    _POOL.clear()
    _POOL.update(lay=lay, x=inp.as_f32("x"), y=inp.as_f32("y"), s=inp.as_f32("s"), g=inp.g,
                 senders=inp.senders, receivers=inp.receivers, num_nodes=N, backward=with_backward,
                 rows=rows, bounds=ptr[rows], out=_shared_f64((N, lay.num_out, lay.channels)))
    if with_backward:
        _POOL.update(dx=_shared_f64((workers, N, lay.num_x, lay.channels)),
                     dy=_shared_f64((E, lay.num_y)), ds=_shared_f64((E, lay.num_paths, lay.channels)))
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(workers) as pool:
        done = sum(pool.map(_oracle_chunk, range(workers), chunksize=1))
    dt = time.perf_counter() - t0
    assert done == E
    res = {"out": _POOL["out"]}
    if with_backward:
        res.update(dx=_POOL["dx"].sum(axis=0), dy=_POOL["dy"], ds=_POOL["ds"])
    what = "forward + reverse" if with_backward else "forward"
    base = {"value": E / dt, "unit": "edges/s", "cores": workers, "kind": "oracle",
            "sample": (f"the whole workload ({E} edges, {N} receivers): {what}, fp64 numpy, "
                       f"{workers} single-threaded processes over receiver-aligned edge ranges"),
            "wall_s": dt, "edges_per_s_per_core": E / dt / workers}
    _POOL.clear()
    return base, res


def oracle_forward_threads(inp, threads):
    """The oracle's forward over the whole workload: receiver-aligned ranges run on a thread
    pool (numpy releases the interpreter lock in its array loops); bf16 operands decoded per
    range.  Returns (out fp64, seconds)."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits

    from oracle import conv
    from equivariant_gnn_message_amd import synth
    w = inp.workload
    lay = conv.make_layout(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    N = inp.num_nodes
    ptr = np.searchsorted(inp.receivers, np.arange(N + 1))
    x = inp.as_f32("x")
    dec = (lambda a: synth.bf16_to_f32(a).reshape(a.shape)) if w.dtype == "bf16" else (lambda a: a)
    out = np.empty((N, w.num_out, w.channels))
    parts = max(1, 8 * threads)

    def run(k):
        b0, b1 = N * k // parts, N * (k + 1) // parts
        e0, e1 = int(ptr[b0]), int(ptr[b1])
        out[b0:b1] = conv.forward(lay, x, dec(inp.y[e0:e1]), dec(inp.s[e0:e1]), inp.senders[e0:e1],
                                  inp.receivers[e0:e1] - b0, b1 - b0)

    t0 = time.perf_counter()
    with threadpool_limits(1), ThreadPoolExecutor(threads) as ex:
        list(ex.map(run, range(parts)))
    return out, time.perf_counter() - t0


def parity_full(got, ref):
    """max|got - ref| / RMS(ref) over whole tensors (chunked to bound host memory)."""
    import numpy as np
    g = got.reshape(-1)
    r = ref.reshape(-1)
    step = 1 << 24
    err = 0.0
    ss = 0.0
    for i in range(0, r.size, step):
        rr = r[i:i + step]
        err = max(err, float(np.max(np.abs(g[i:i + step].astype(np.float64) - rr))) if rr.size else 0.0)
        ss += float(np.dot(rr, rr))
    rms = math.sqrt(ss / max(r.size, 1))
    return err / rms if rms > 0 else err


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: e3conv runs on one GPU per process; --gpus {args.gpus} is not supported "
              f"(multi-GPU sharding is not implemented)", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    import numpy as np

    from equivariant_gnn_message_amd import synth

    if args.mode != "conv":
        bench_mode(args)
        return

    w = synth.WORKLOADS[args.workload]
    t0 = time.perf_counter()
    inp = synth.make_inputs(args.workload)
    t_gen = time.perf_counter() - t0
    N, Ecount = inp.num_nodes, inp.num_edges

    # The oracle runs first: its worker processes are forked before this process touches the
    # GPU, so none of them holds the device.  Its outputs are kept for the parity check.
    base = ref = None
    if not args.no_cpu_baseline:
        base, ref = cpu_baseline(inp, w.backward, host_cores())

    import torch

    from equivariant_gnn_message_amd import e3conv as E
    dev = torch.device("cuda:0")

    def t(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    x, y, s, g = t(inp.x), t(inp.y), t(inp.s), t(inp.g)
    src, dst = t(inp.senders), t(inp.receivers)
    torch.cuda.synchronize()

    tp = time.perf_counter()
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    plan.set_variant(args.fwd_variant, args.bwd_variant)
    plan_ms = (time.perf_counter() - tp) * 1e3
    E.e3conv_csr_from_receivers(dst, N)          # first launch loads the code object
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    row_ptr = E.e3conv_csr_from_receivers(dst, N)
    ev1.record()
    torch.cuda.synchronize()
    csr_ms = ev0.elapsed_time(ev1)
    to = time.perf_counter()
    order_np = E.e3conv_receiver_order(row_ptr.cpu().numpy(), inp.senders, N, Ecount, args.cluster)
    order_ms = (time.perf_counter() - to) * 1e3
    order_dev = torch.from_numpy(order_np).to(dev)
    order = None if args.no_order else order_dev

    out = torch.empty((N, w.num_out, w.channels), dtype=torch.float32, device=dev)
    grads = None
    if w.backward:
        grads = (torch.empty_like(x), torch.empty_like(y), torch.empty_like(s))

    fwd_ev, bwd_ev = [], []

    def step(record):
        if record:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
        plan.forward(x, y, s, src, row_ptr, out=out, order=order)
        if record:
            b.record()
            fwd_ev.append((a, b))
        if w.backward:
            if record:
                c, d = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                c.record()
            plan.backward(x, y, s, src, row_ptr, g, grads=grads, order=order)
            if record:
                d.record()
                bwd_ev.append((c, d))

    if args.sweep:
        b_in = 2 if w.dtype == "bf16" else 4
        sweep(plan, w, lambda o: plan.forward(x, y, s, src, row_ptr, out=out, order=o),
              lambda o: plan.backward(x, y, s, src, row_ptr, g, grads=grads, order=o),
              alg_bytes(w, N, Ecount, b_in), [("index", None), ("clustered", order_dev)])
        return

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t1

    eager_ms_per_step = wall / args.steps * 1e3
    ms_per_step, graph_ms = eager_ms_per_step, None
    if w.backward and not args.eager:
        # The headline training step: the same step (every kernel of it) captured once in a
        # HIP graph and replayed, W untimed replays, then K replays bracketed by
        # synchronisations, timed by the host clock like the eager loop.  (A graph removes the
        # gaps between a step's kernel launches; a forward-only step is one launch, which a
        # graph replay only makes slower, so it stays eager.)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(False)
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(False)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        tg = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - tg) / args.steps * 1e3
        ms_per_step = graph_ms
        del graph
    fwd_times = [a.elapsed_time(b) for a, b in fwd_ev]
    fwd_ms = float(np.mean(fwd_times))
    b_in = 2 if w.dtype == "bf16" else 4
    fwd_bytes, bwd_bytes = alg_bytes(w, N, Ecount, b_in)
    res = {
        "metric": METRIC,
        "value": Ecount / (ms_per_step * 1e-3),
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "execution": "eager launches" if graph_ms is None else "HIP graph replay of the captured step",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"{w.name}: {'forward + reverse' if w.backward else 'forward'} convolution, "
                         f"radius graph N={N} E={Ecount}, {w.irreps_in} (x) SH lmax {w.lmax} -> "
                         f"{w.irreps_out}, avg_num_neighbors {w.avg_num_neighbors:g}, "
                         f"{'bf16 storage / fp32 accumulation' if w.dtype == 'bf16' else 'fp32'}"),
            "num_nodes": N, "num_edges": Ecount, "channels": w.channels, "num_paths": w.num_paths,
            "parallelism": "single GPU",
        },
        "fwd_ms": fwd_ms,
        "fwd_hbm_GBps": fwd_bytes / (fwd_ms * 1e-3) / 1e9,
        "fwd_hbm_frac": fwd_bytes / (fwd_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "csr_ms": csr_ms,
        "order_ms": order_ms,
        "receiver_order": "index" if args.no_order else f"clustered {args.cluster}",
        "plan_ms": plan_ms,
        "variants": [args.fwd_variant, args.bwd_variant],
        "fwd_ms_stats": time_stats(fwd_times),
    }
    res["eager_ms_per_step"] = eager_ms_per_step
    res["eager_value"] = Ecount / (eager_ms_per_step * 1e-3)
    res["eager_step_hbm_frac"] = ((fwd_bytes + (bwd_bytes if w.backward else 0)) / (eager_ms_per_step * 1e-3)
                                  / 1e9 / PEAK_HBM_GBPS)
    if N * w.num_out * w.channels * 4 < (64 << 20):
        # small problems fit the 256 MB MALL: also report cold-cache forwards
        res["fwd_ms_cold"] = cold_forward_ms(lambda: plan.forward(x, y, s, src, row_ptr, out=out,
                                                                  order=order), reps=10)
    kernel, kbytes, kms = "conv_fwd", fwd_bytes, fwd_ms
    if w.backward:
        bwd_times = [a.elapsed_time(b) for a, b in bwd_ev]
        bwd_ms = float(np.mean(bwd_times))
        res["bwd_ms"] = bwd_ms
        res["bwd_ms_stats"] = time_stats(bwd_times)
        res["bwd_hbm_GBps"] = bwd_bytes / (bwd_ms * 1e-3) / 1e9
        res["bwd_hbm_frac"] = res["bwd_hbm_GBps"] / PEAK_HBM_GBPS
        res["step_hbm_frac"] = (fwd_bytes + bwd_bytes) / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBPS
        kernel, kbytes, kms = "conv_bwd", bwd_bytes, bwd_ms
    fwd_flops = forward_flops_per_edge(plan) * Ecount
    res["fwd_alg_flops"] = fwd_flops
    res["fwd_valu_TFLOPs"] = fwd_flops / (fwd_ms * 1e-3) / 1e12
    res["roofline"] = roofline(kernel, kms, kbytes, fwd_flops if kernel == "conv_fwd" else None,
                               traffic_from_profiles(kernel, args.workload))
    res["cpu_baseline"] = base
    if ref is not None:
        # the GPU outputs of the last timed step against the oracle, element by element
        tol = 2e-2 if w.dtype == "bf16" else 1e-5
        par = {"out": parity_full(out.cpu().numpy(), ref["out"])}
        if w.backward:
            for name, t_gpu, key in (("grad_x", grads[0], "dx"), ("grad_y", grads[1], "dy"),
                                     ("grad_s", grads[2], "ds")):
                par[name] = parity_full(t_gpu.cpu().numpy(), ref[key])
        res["parity_full"] = {"max_abs_err_over_rms": par, "tolerance": tol,
                              "pass": all(v <= tol for v in par.values())}
    del ref
    res["input_gen_s"] = t_gen
    if w.backward and w.idx == 4 and not args.no_extra:
        # workload 2 (MACE-scale forward) is the forward of this step: same graph and operands
        res["w2_forward"] = forward_block(plan, w, fwd_times, fwd_bytes, N, Ecount)
        del x, y, s, g, grads, out, order, order_dev, src, dst, row_ptr
        torch.cuda.empty_cache()
        # beside the default kernel: the matrix-core form (bf16 operands, variant 6)
        res["w3_forward"] = bench_forward_workload(3, args, parity=not args.no_cpu_baseline,
                                                   variants=((6, "matrix_core_variant"),))
        res["pairs_reverse"] = pairs_block(plan, w, inp, res["fwd_ms"], res["bwd_ms"], args)
        res["relabeled_step"] = relabeled_block(plan, w, inp, fwd_bytes, bwd_bytes, args)
        # the small configurations' forwards (latency-bound: far from either roof)
        res["w0_forward"] = bench_forward_workload(0, args, parity=not args.no_cpu_baseline)
        res["w1_forward"] = bench_forward_workload(1, args, parity=not args.no_cpu_baseline)
        res["bar_60pct_hbm"] = {
            "w2_forward": res["w2_forward"]["hbm_frac"] >= 0.6,
            "w3_forward": res["w3_forward"]["hbm_frac"] >= 0.6,
            "w4_step": res["step_hbm_frac"] >= 0.6,
            "w4_step_relabeled_graph": res["relabeled_step"]["step_hbm_frac"] >= 0.6}
    print(json.dumps(res), flush=True)


def alg_forward_flops(plan):
    """Algorithmic forward flops per edge: 2 per CG term for K^p(y), then per channel one
    product per nonzero of each K^p and one mixing product per output component of each path
    (sum over paths of 2 l3 + 1), whatever order a kernel applies them in."""
    nnz, nnz_k, _ = _conv_counts(plan)
    mix = sum(2 * q["l3"] + 1 for q in plan.paths())
    return 2 * nnz + 2 * plan.channels * (nnz_k + mix)


def forward_block(plan, w, times, nbytes, N, Ecount):
    """One forward's figures against both roofs: HBM bytes and vector-ALU flops."""
    import numpy as np
    ms = float(np.mean(times))
    flops = alg_forward_flops(plan) * Ecount
    gbps = nbytes / (ms * 1e-3) / 1e9
    tf = flops / (ms * 1e-3) / 1e12
    return {"workload": f"{w.name}: forward, N={N} E={Ecount}, {w.irreps_in} (x) SH lmax {w.lmax} -> "
                        f"{w.irreps_out}, {'bf16 storage / fp32 accumulation' if w.dtype == 'bf16' else 'fp32'}",
            "ms": ms, "ms_stats": time_stats(times), "edges_per_s": Ecount / (ms * 1e-3),
            "algorithmic_bytes": nbytes, "hbm_GBps": gbps, "hbm_frac": gbps / PEAK_HBM_GBPS,
            "algorithmic_flops": flops, "valu_TFLOPs": tf, "valu_frac": tf / PEAK_FP32_VALU_TFLOPS,
            "bound": "alu" if flops / PEAK_FP32_VALU_TFLOPS / 1e12 > nbytes / PEAK_HBM_GBPS / 1e9 else "hbm"}


def bench_forward_workload(idx, args, parity=False, variants=()):
    """Forward of workload idx (full size, default kernel, clustered receiver order), timed
    per call with HIP events on the launch stream.  variants: (index, key) pairs of other
    forward variants timed the same way, each reported under its key with its own parity
    against the same oracle output."""
    import numpy as np
    import torch

    from equivariant_gnn_message_amd import e3conv as E
    from equivariant_gnn_message_amd import synth

    w = synth.WORKLOADS[idx]
    inp = synth.make_inputs(idx)
    N, Ec = inp.num_nodes, inp.num_edges
    b_in = 2 if w.dtype == "bf16" else 4

    def t(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    x, y, s = t(inp.x), t(inp.y), t(inp.s)
    src = t(inp.senders)
    row_ptr = E.e3conv_csr_from_receivers(t(inp.receivers), N)
    order = torch.from_numpy(E.e3conv_receiver_order(row_ptr.cpu().numpy(), inp.senders, N, Ec,
                                                     args.cluster)).cuda()
    if not parity:
        del inp
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    out = torch.empty((N, w.num_out, w.channels), dtype=torch.float32, device="cuda")

    def timed():
        for _ in range(args.warmup):
            plan.forward(x, y, s, src, row_ptr, out=out, order=order)
        torch.cuda.synchronize()
        ev = []
        for _ in range(args.steps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            plan.forward(x, y, s, src, row_ptr, out=out, order=order)
            b.record()
            ev.append((a, b))
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    nbytes = alg_bytes(w, N, Ec, b_in)[0]
    blk = forward_block(plan, w, timed(), nbytes, N, Ec)
    outs = {None: out.cpu().numpy()} if parity else {}
    nf, _ = plan.num_variants(E.E3CONV_BF16 if w.dtype == "bf16" else E.E3CONV_F32)
    for v, key in variants:
        if v >= nf:
            continue
        plan.set_variant(v, 0)
        blk[key] = forward_block(plan, w, timed(), nbytes, N, Ec)
        blk[key]["variant"] = v
        if parity:
            outs[key] = out.cpu().numpy()
    plan.set_variant(0, 0)
    if parity:
        # every output element against the oracle (fp64, over the host cores)
        del x, y, s, src, row_ptr, order, out
        torch.cuda.empty_cache()
        threads = host_cores()
        ref, secs = oracle_forward_threads(inp, threads)
        tol = 2e-2 if w.dtype == "bf16" else 1e-5
        for key, got in outs.items():
            err = parity_full(got, ref)
            par = {"max_abs_err_over_rms": err, "tolerance": tol, "pass": err <= tol}
            if key is None:
                par.update(oracle_s=secs, oracle_threads=threads)
                blk["parity_full"] = par
            else:
                blk[key]["parity_full"] = par
        del outs, ref
    else:
        del x, y, s, src, row_ptr, order, out
        torch.cuda.empty_cache()
    return blk


def time_stats(times):
    """Median, min and 90th percentile of per-call HIP-event times (ms)."""
    import numpy as np
    a = np.asarray(times, dtype=np.float64)
    return {"median": float(np.median(a)), "min": float(a.min()), "p90": float(np.percentile(a, 90))}


def cold_forward_ms(run, reps=10, flush_mib=512):
    """Forward time after overwriting a 512 MiB buffer (evicts the 256 MB MALL and the L2s)."""
    import numpy as np
    import torch

    from equivariant_gnn_message_amd import e3conv as E
    a = torch.ones(flush_mib << 18, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    times = []
    for _ in range(reps):
        E.e3conv_stream_reference(a, b)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del a, b
    return time_stats(times)


def _timed(fn, steps, warmup):
    """Mean time (ms) per call of fn() over `steps` back-to-back calls, from one HIP-event pair
    on torch's current stream (the launch stream); one pair per region keeps the event records'
    own cost (a few microseconds each) out of short kernels' times."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def bench_mode(args):
    """One JSON line for a variant of the path: SENDER ordering, forward mode, second order."""
    import numpy as np
    import torch

    from equivariant_gnn_message_amd import e3conv as E
    from equivariant_gnn_message_amd import synth

    if args.mode == "linear":
        bench_linear(args)
        return
    if args.mode == "radial":
        bench_radial(args)
        return
    if args.mode == "pairs":
        bench_pairs(args)
        return
    w = synth.WORKLOADS[args.workload]
    inp = synth.make_inputs(args.workload)
    N, Ec = inp.num_nodes, inp.num_edges
    b_in = 2 if w.dtype == "bf16" else 4
    C, nx, ny, no, P = w.channels, w.num_x, (w.lmax + 1) ** 2, w.num_out, w.num_paths

    def dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    src_np, dst_np = inp.senders, inp.receivers
    ordering = E.E3CONV_RECEIVER
    y_np, s_np = inp.y, inp.s
    if args.mode == "sender":
        perm = synth.sender_sorted(src_np, dst_np)
        src_np, dst_np, y_np, s_np = src_np[perm], dst_np[perm], y_np[perm], s_np[perm]
        ordering = E.E3CONV_SENDER
    gather_np, seg_np = (dst_np, src_np) if args.mode == "sender" else (src_np, dst_np)
    x, y, s, g = dev(inp.x), dev(y_np), dev(s_np), dev(inp.g)
    gather = dev(gather_np.astype(np.int32))
    row_ptr = E.e3conv_csr_from_receivers(dev(seg_np.astype(np.int32)), N)
    order = dev(E.e3conv_receiver_order(row_ptr.cpu().numpy(), gather_np.astype(np.int32), N, Ec,
                                        args.cluster))
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors, ordering=ordering)
    fwd_bytes, bwd_bytes = alg_bytes(w, N, Ec, b_in)
    node_x, node_o = N * nx * C, N * no * C
    res = {"metric": None, "value": None, "unit": "edges/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic",
           "config": {"workload": f"{w.name}, N={N} E={Ec}, {w.irreps_in} (x) SH lmax {w.lmax} -> "
                                  f"{w.irreps_out}", "mode": args.mode}}
    kernels = {}
    if args.mode == "sender":
        out = torch.empty((N, no, C), dtype=torch.float32, device="cuda")
        kernels["forward"] = (_timed(lambda: plan.forward(x, y, s, gather, row_ptr, out=out, order=order),
                                     args.steps, args.warmup), fwd_bytes)
        if w.backward:
            grads = (torch.empty_like(x), torch.empty_like(y), torch.empty_like(s))
            kernels["reverse"] = (_timed(lambda: plan.backward(x, y, s, gather, row_ptr, g, grads=grads,
                                                               order=order), args.steps, args.warmup),
                                  bwd_bytes)
        res["metric"] = "edges/sec, SENDER graph ordering (edges grouped by sender), 1 MI355X"
    elif args.mode == "jvp":
        dx, dy, ds = (dev(a) for a in synth.make_tangents(inp))
        out = torch.empty((N, no, C), dtype=torch.float32, device="cuda")
        out_dot = torch.empty_like(out)
        jvp_bytes = (2 * node_x * b_in + Ec * (2 * ny * b_in + 2 * P * C * b_in + 4) + 4 * (N + 1)
                     + 2 * node_o * 4)
        kernels["jvp"] = (_timed(lambda: plan.jvp(x, y, s, dx, dy, ds, gather, row_ptr, out=out,
                                                  out_dot=out_dot, order=order),
                                 args.steps, args.warmup), jvp_bytes)
        res["metric"] = "edges/sec, fused forward-mode pass (out and its tangent), 1 MI355X"
    else:
        if not w.backward:
            raise SystemExit("--mode second needs a workload with a reverse pass (4)")
        Gx, Gy, Gs = (dev(a) for a in synth.make_tangents(inp))
        dx, dy, ds = torch.empty_like(x), torch.empty_like(y), torch.empty_like(s)
        dg = torch.empty_like(g)
        e_in = Ec * (ny + P * C) * 4 + Ec * 4 + 4 * (N + 1)

        def second():
            plan.backward(Gx, y, s, gather, row_ptr, g, grads=(None, dy, ds), order=order)
            plan.backward(x, Gy, s, gather, row_ptr, g, grads=(dx, None, ds), order=order,
                          accumulate=(False, False, True))
            plan.backward(x, y, Gs, gather, row_ptr, g, grads=(dx, dy, None), order=order,
                          accumulate=(True, True, False))
            plan.jvp(x, y, s, Gx, Gy, Gs, gather, row_ptr, out_dot=dg, order=order, want_out=False)

        # per call: operands read once, outputs written once, accumulated outputs read once more
        second_bytes = ((node_x + e_in + node_o + Ec * (ny + P * C) * 4)
                        + (2 * node_x + e_in + node_o + 2 * Ec * P * C * 4)
                        + (2 * node_x + e_in + node_o + 2 * Ec * ny * 4)
                        + (2 * node_x + e_in + Ec * (ny + P * C) * 4 + node_o))
        kernels["second_order"] = (_timed(second, args.steps, args.warmup), second_bytes)
        res["metric"] = "edges/sec, second derivatives of the training step (gradient of <G, grad>), 1 MI355X"
    total_ms = sum(ms for ms, _ in kernels.values())
    res["value"] = Ec / (total_ms * 1e-3)
    res["ms_per_step"] = total_ms
    for k, (ms, by) in kernels.items():
        res[f"{k}_ms"] = ms
        res[f"{k}_hbm_GBps"] = by / (ms * 1e-3) / 1e9
        res[f"{k}_hbm_frac"] = by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS
    k, (ms, by) = max(kernels.items(), key=lambda kv: kv[1][0])
    flops = {"forward": forward_flops_per_edge(plan) * Ec, "jvp": jvp_flops_per_edge(plan) * Ec}
    res["roofline"] = roofline(k, ms, by, flops.get(k))
    res["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_mode(args.mode, inp, args.cpu_sample_edges)
    print(json.dumps(res), flush=True)


def pair_bytes(w, N, Ep):
    """Compulsory bytes of the pair-stored reverse pass: x and g read, grad_x
    written once; per stored edge y, s, src, dst read and grad_y, grad_s written."""
    C, nx, ny, no, P = w.channels, w.num_x, (w.lmax + 1) ** 2, w.num_out, w.num_paths
    return 4 * (2 * N * nx * C + N * no * C + Ep * (2 * ny + 2 * P * C + 2))


def pair_inputs(inp, cluster=512):
    """Pair storage of a workload's symmetric radius graph (e3conv_pair_layout: one
    stored edge per pair, receivers in the locality order, runs of one receiver),
    one seeded N(0,1) row of s per pair, and for each directed edge its pair."""
    import numpy as np

    from equivariant_gnn_message_amd import e3conv as E
    from equivariant_gnn_message_amd import synth
    w = inp.workload
    N, Ec = inp.num_nodes, inp.num_edges
    row_ptr = np.searchsorted(inp.receivers, np.arange(N + 1)).astype(np.int32)
    t0 = time.perf_counter()
    stored, pair_of = E.e3conv_pair_layout(row_ptr, inp.senders, N, Ec, cluster)
    layout_ms = (time.perf_counter() - t0) * 1e3
    s_pair = synth.normal_f32(w.idx, synth.T_S_PAIR, (len(stored), w.num_paths, w.channels))
    return stored, pair_of, s_pair, layout_ms


def time_pairs(plan, w, inp, stored, pmap, s_pair, args):
    """HIP-event times (ms) of the pair-stored forward (directed receiver CSR, receiver
    order, rows through the pair map) and of the pair-stored reverse pass."""
    import numpy as np
    import torch

    from equivariant_gnn_message_amd import e3conv as E
    N, Ec, Ep = inp.num_nodes, inp.num_edges, len(stored)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    x, g = t(inp.x), t(inp.g)
    y, s = t(inp.y[stored]), t(s_pair)
    src, dst = t(inp.senders[stored].astype(np.int32)), t(inp.receivers[stored].astype(np.int32))
    dsrc, d_map = t(inp.senders.astype(np.int32)), t(pmap.astype(np.int32))
    row_ptr = E.e3conv_csr_from_receivers(t(inp.receivers.astype(np.int32)), N)
    order = t(E.e3conv_receiver_order(row_ptr.cpu().numpy(), inp.senders, N, Ec, args.cluster))
    out = torch.empty((N, w.num_out, w.channels), dtype=torch.float32, device="cuda")
    gx, gy, gs = torch.empty_like(x), torch.empty_like(y), torch.empty_like(s)
    fwd_ms = _timed(lambda: E.e3conv_forward_pairs(plan.handle, x, y, s, dsrc, row_ptr, d_map, N, Ec, Ep,
                                                   out, order=order), args.steps, args.warmup)
    bwd_ms = _timed(lambda: E.e3conv_backward_pairs(plan.handle, x, y, s, src, dst, N, Ep, g, gx, gy, gs),
                    args.steps, args.warmup)
    del x, g, y, s, src, dst, dsrc, d_map, row_ptr, order, out, gx, gy, gs
    torch.cuda.empty_cache()
    return fwd_ms, bwd_ms


def relabeled_block(plan, w, inp, fwd_bytes, bwd_bytes, args):
    """The training step on the same graph with its nodes renamed by e3conv_relabel_nodes
    (index order = the receiver-cluster order; a permutation of the inputs computed once
    per graph on the host, outside the timed region like the CSR): forward, reverse pass
    and step timed as in the headline, and the output checked against the relabeled
    output of the graph as generated."""
    import numpy as np
    import torch

    from equivariant_gnn_message_amd import e3conv as E

    N, Ec = inp.num_nodes, inp.num_edges
    row_ptr_h = np.searchsorted(inp.receivers, np.arange(N + 1)).astype(np.int32)
    t0 = time.perf_counter()
    node_new, perm = E.e3conv_relabel_nodes(row_ptr_h, inp.senders, N, Ec, args.cluster)
    relabel_ms = (time.perf_counter() - t0) * 1e3
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    inv = t(np.argsort(node_new).astype(np.int64))      # old id of each new node
    p = t(perm.astype(np.int64))
    x0, g0 = t(inp.x), t(inp.g)
    x, g = x0[inv].contiguous(), g0[inv].contiguous()
    y, s = t(inp.y)[p].contiguous(), t(inp.s)[p].contiguous()
    src = t(node_new[inp.senders[perm]].astype(np.int32))
    row_ptr = E.e3conv_csr_from_receivers(t(node_new[inp.receivers[perm]].astype(np.int32)), N)
    out = torch.empty((N, w.num_out, w.channels), dtype=torch.float32, device="cuda")
    grads = (torch.empty_like(x), torch.empty_like(y), torch.empty_like(s))
    fwd = lambda: plan.forward(x, y, s, src, row_ptr, out=out)
    bwd = lambda: plan.backward(x, y, s, src, row_ptr, g, grads=grads)
    fwd_ms = _timed(fwd, args.steps, args.warmup)
    bwd_ms = _timed(bwd, args.steps, args.warmup)
    eager_step_ms = step_ms = _timed(lambda: (fwd(), bwd()), args.steps, args.warmup)
    if not args.eager:
        # the step captured in a HIP graph and replayed, as the headline step
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fwd()
            bwd()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fwd()
            bwd()
        step_ms = _timed(graph.replay, args.steps, args.warmup)
        del graph
    # the same forward on the generated ids, relabeled, against this one
    src0 = t(inp.senders.astype(np.int32))
    rp0 = E.e3conv_csr_from_receivers(t(inp.receivers.astype(np.int32)), N)
    ref = plan.forward(x0, t(inp.y), t(inp.s), src0, rp0)[inv]
    fwd()
    torch.cuda.synchronize()
    diff = float((out - ref).abs().max() / ref.pow(2).mean().sqrt())
    blk = {"workload": f"{w.name}: training step on the same graph, nodes renamed in receiver-cluster "
                       f"order (cluster {args.cluster}), N={N} E={Ec}",
           "relabel_host_ms": relabel_ms, "fwd_ms": fwd_ms, "bwd_ms": bwd_ms, "step_ms": step_ms,
           "eager_step_ms": eager_step_ms,
           "edges_per_s": Ec / (step_ms * 1e-3),
           "fwd_hbm_frac": fwd_bytes / (fwd_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
           "bwd_hbm_frac": bwd_bytes / (bwd_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
           "step_hbm_frac": (fwd_bytes + bwd_bytes) / (step_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
           "out_vs_generated_ids_max_err_over_rms": diff}
    del x0, g0, x, g, y, s, src, row_ptr, out, grads, src0, rp0, ref, inv, p
    torch.cuda.empty_cache()
    return blk


def pairs_block(plan, w, inp, directed_fwd_ms, directed_ms, args):
    """The pair-stored forward and reverse pass on the training graph (one y and s row per
    pair) next to the directed passes of the same graph (their times do not depend on the
    values)."""
    stored, pmap, s_pair, layout_ms = pair_inputs(inp, args.cluster)
    N, Ec, Ep = inp.num_nodes, inp.num_edges, len(stored)
    fwd_ms, ms = time_pairs(plan, w, inp, stored, pmap, s_pair, args)
    nbytes = pair_bytes(w, N, Ep)
    dir_bytes = alg_bytes(w, N, Ec, 4)[1]
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"workload": f"{w.name}: reverse pass, y and s stored once per undirected pair, N={N}, "
                        f"{Ep} pairs ({Ec} directed edges)",
            "ms": ms, "directed_edges_per_s": Ec / (ms * 1e-3), "algorithmic_bytes": nbytes,
            "hbm_GBps": gbps, "hbm_frac": gbps / PEAK_HBM_GBPS,
            "directed_reverse_ms": directed_ms, "directed_algorithmic_bytes": dir_bytes,
            "speedup_vs_directed": directed_ms / ms, "pair_layout_ms": layout_ms,
            "pair_order": f"clustered {args.cluster}",
            "forward_ms": fwd_ms, "directed_forward_ms": directed_fwd_ms,
            "step_ms": fwd_ms + ms, "directed_step_ms": directed_fwd_ms + directed_ms,
            "step_speedup_vs_directed": (directed_fwd_ms + directed_ms) / (fwd_ms + ms)}


def bench_pairs(args):
    """Reverse pass of the training graph with symmetric scalars: directed storage
    (every edge its own y and s rows) against pair storage (one row per pair)."""
    import numpy as np
    import torch

    from equivariant_gnn_message_amd import e3conv as E
    from equivariant_gnn_message_amd import synth

    w = synth.WORKLOADS[args.workload]
    if not w.backward or w.dtype != "f32":
        raise SystemExit("--mode pairs needs the fp32 training workload (4)")
    inp = synth.make_inputs(args.workload)
    N, Ec = inp.num_nodes, inp.num_edges
    stored, pair_of, s_pair, layout_ms = pair_inputs(inp, args.cluster)
    Ep = len(stored)
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    # directed: the same graph with s expanded to both directions of each pair
    x, y, g = t(inp.x), t(inp.y), t(inp.g)
    s = t(s_pair)[t(np.where(pair_of >= 0, pair_of, ~pair_of))]
    src = t(inp.senders)
    row_ptr = E.e3conv_csr_from_receivers(t(inp.receivers), N)
    grads = (torch.empty_like(x), torch.empty_like(y), torch.empty_like(s))
    order = t(E.e3conv_receiver_order(row_ptr.cpu().numpy(), inp.senders, N, Ec, args.cluster))
    out = torch.empty((N, w.num_out, w.channels), dtype=torch.float32, device="cuda")
    dir_fwd_ms = _timed(lambda: plan.forward(x, y, s, src, row_ptr, out=out, order=order), args.steps,
                        args.warmup)
    dir_ms = _timed(lambda: plan.backward(x, y, s, src, row_ptr, g, grads=grads), args.steps, args.warmup)
    del x, y, g, s, src, row_ptr, grads, order, out
    torch.cuda.empty_cache()
    pair_fwd_ms, pair_ms = time_pairs(plan, w, inp, stored, pair_of, s_pair, args)
    pb, db = pair_bytes(w, N, Ep), alg_bytes(w, N, Ec, 4)[1]
    res = {"metric": "directed edges/sec of the reverse pass, y and s stored once per undirected pair, "
                     "1 MI355X",
           "value": Ec / (pair_ms * 1e-3), "unit": "edges/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": pair_ms, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": f"{w.name}: reverse pass on the radius graph N={N} E={Ec} "
                                  f"({Ep} undirected pairs), one N(0,1) row of s per pair",
                      "mode": "pairs"},
           "pairs_ms": pair_ms, "pairs_algorithmic_bytes": pb,
           "pairs_hbm_GBps": pb / (pair_ms * 1e-3) / 1e9,
           "directed_ms": dir_ms, "directed_algorithmic_bytes": db,
           "directed_hbm_GBps": db / (dir_ms * 1e-3) / 1e9,
           "speedup_vs_directed": dir_ms / pair_ms, "pair_layout_ms": layout_ms,
           "pair_order": f"clustered {args.cluster}",
           "pairs_forward_ms": pair_fwd_ms, "directed_forward_ms": dir_fwd_ms,
           "pairs_step_ms": pair_fwd_ms + pair_ms, "directed_step_ms": dir_fwd_ms + dir_ms,
           "step_speedup_vs_directed": (dir_fwd_ms + dir_ms) / (pair_fwd_ms + pair_ms),
           "roofline": roofline("conv_bwd_pairs", pair_ms, pb,
                                traffic=traffic_from_profiles("conv_bwd_pairs", args.workload))}
    res["cpu_baseline"] = None
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits

        from oracle import conv, variants
        lay = conv.make_layout(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
        k = min(args.cpu_sample_edges // 8, Ep)
        with threadpool_limits(1):
            t0 = time.perf_counter()
            variants.backward_pairs(lay, inp.x, inp.y[stored[:k]], s_pair[:k], inp.g,
                                    inp.senders[stored[:k]], inp.receivers[stored[:k]], N)
            dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": 2 * k / dt, "unit": "edges/s", "cores": 1, "kind": "oracle",
                               "sample": f"first {k} pairs ({2 * k} directed edges), pair-stored "
                                         f"reverse pass, fp64 numpy, {dt:.1f} s"}
    print(json.dumps(res), flush=True)


def bench_linear(args):
    """The output linear on the convolution output of a workload (C_out = C)."""
    import numpy as np
    import torch

    from equivariant_gnn_message_amd import e3conv as E
    from equivariant_gnn_message_amd import synth

    w = synth.WORKLOADS[args.workload]
    inp = synth.make_inputs(args.workload)
    N, C, NO = inp.num_nodes, w.channels, w.num_out
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    nb = plan.num_out_blocks()
    rng = np.random.default_rng(5)
    x = torch.from_numpy(rng.standard_normal((N, NO, C)).astype(np.float32)).cuda()
    W = torch.from_numpy(rng.standard_normal((nb, C, C)).astype(np.float32)).cuda()
    g = torch.from_numpy(rng.standard_normal((N, NO, C)).astype(np.float32)).cuda()
    out, gi, gw = torch.empty_like(x), torch.empty_like(x), torch.empty_like(W)
    fwd_ms = _timed(lambda: plan.linear(x, W, C, out=out), args.steps, args.warmup)
    bwd_ms = _timed(lambda: E.e3conv_linear_backward(plan.handle, C, 1.0, W, x, N, g, gi, gw),
                    args.steps, args.warmup)
    flops = 2.0 * N * NO * C * C
    tf_f, tf_b = flops / (fwd_ms * 1e-3) / 1e12, 2 * flops / (bwd_ms * 1e-3) / 1e12
    byt = 4.0 * (2 * N * NO * C + nb * C * C)
    # the forward streams in and out once; its fp32 products run as six bf16 matrix products
    # (three-part operands), which take less time than the bytes
    gbps = byt / (fwd_ms * 1e-3) / 1e9
    res = {"metric": "node rows/sec, output linear (channel mixing per irrep block), fp32 products on the "
                     "matrix cores, 1 MI355X",
           "value": N / ((fwd_ms + bwd_ms) * 1e-3), "unit": "nodes/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": fwd_ms + bwd_ms, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": f"output linear on {w.name} output: N={N}, {w.irreps_out} -> same irreps",
                      "mode": "linear"},
           "forward_ms": fwd_ms, "forward_TFLOPs": tf_f, "forward_hbm_GBps": gbps,
           "reverse_ms": bwd_ms, "reverse_TFLOPs": tf_b,
           "roofline": {"bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                        "frac": gbps / PEAK_HBM_GBPS, "traffic": None,
                        "kernel": "linear_rows (forward): reads in and W, writes out once",
                        "algorithmic_bytes": byt, "fp32_equivalent_TFLOPs": tf_f,
                        "bf16_issued_TFLOPs": 6 * tf_f, "bf16_peak_TFLOPs": PEAK_FP16_MFMA_TFLOPS}}
    if plan.kernels_fused_linear():
        res["fused_epilogue"] = fused_linear_block(plan, w, inp, W, args)
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits
        from oracle import conv, linear
        lay = conv.make_layout(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
        n1 = min(N, 4000)
        xs, gs = x[:n1].cpu().numpy(), g[:n1].cpu().numpy()
        Wn = W.cpu().numpy()
        with threadpool_limits(1):
            t0 = time.perf_counter()
            linear.linear(lay, Wn, 1.0, xs)
            linear.linear_backward(lay, Wn, 1.0, xs, gs)
            dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": n1 / dt, "unit": "nodes/s", "cores": 1, "kind": "oracle",
                               "sample": f"first {n1} node rows, forward + reverse, fp64 numpy, {dt:.1f} s"}
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def fused_linear_block(plan, w, inp, W, args):
    """The convolution then the output linear (C_out = C) of a workload: two calls
    (e3conv_forward, e3conv_linear) against one with the linear in the epilogue
    (e3conv_forward_linear), same graph, operands, receiver order and weights."""
    import numpy as np
    import torch

    from equivariant_gnn_message_amd import e3conv as E

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    N, Ec, C, NO = inp.num_nodes, inp.num_edges, w.channels, w.num_out
    x, y, s, src = dev(inp.x), dev(inp.y), dev(inp.s), dev(inp.senders)
    row_ptr = E.e3conv_csr_from_receivers(dev(inp.receivers), N)
    order = torch.from_numpy(E.e3conv_receiver_order(row_ptr.cpu().numpy(), inp.senders, N, Ec,
                                                     args.cluster)).cuda()
    m = torch.empty((N, NO, C), dtype=torch.float32, device="cuda")
    o_sep, o_fus = torch.empty_like(m), torch.empty_like(m)

    def separate():
        plan.forward(x, y, s, src, row_ptr, out=m, order=order)
        plan.linear(m, W, C, out=o_sep)

    fused = lambda: E.e3conv_forward_linear(plan.handle, x, y, s, src, row_ptr, N, Ec, 1.0, W, o_fus,
                                            order=order)
    sep_ms = _timed(separate, args.steps, args.warmup)
    conv_ms = _timed(lambda: plan.forward(x, y, s, src, row_ptr, out=m, order=order), args.steps,
                     args.warmup)
    fus_ms = _timed(fused, args.steps, args.warmup)
    torch.cuda.synchronize()
    diff = float((o_sep - o_fus).abs().max() / o_sep.pow(2).mean().sqrt())
    b_in = 2 if w.dtype == "bf16" else 4
    fwd_bytes = alg_bytes(w, N, Ec, b_in)[0]
    fused_bytes = fwd_bytes + 4 * W.numel()
    return {"workload": f"{w.name}: forward, then the output linear, N={N} E={Ec}, {w.irreps_out}, "
                        f"C_out = C, {'bf16' if w.dtype == 'bf16' else 'fp32'} operands",
            "separate_ms": sep_ms, "forward_only_ms": conv_ms, "fused_ms": fus_ms,
            "speedup_vs_separate": sep_ms / fus_ms,
            "fused_algorithmic_bytes": fused_bytes,
            "fused_hbm_GBps": fused_bytes / (fus_ms * 1e-3) / 1e9,
            "separate_algorithmic_bytes": fused_bytes + 2 * 4 * N * NO * C,
            "max_abs_diff_over_rms_fused_vs_separate": diff}


def bench_radial(args):
    """Forward with the edge scalars formed in the kernel from the edge lengths (gate-points)."""
    import numpy as np
    import torch

    from equivariant_gnn_message_amd import e3conv as E
    from equivariant_gnn_message_amd import synth

    w = synth.WORKLOADS[1]
    inp = synth.make_inputs(1)
    N, Ec, C, P = inp.num_nodes, inp.num_edges, w.channels, w.num_paths
    r, w1, w2 = synth.radial_inputs(inp)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    x, y, rr, W1, W2 = dev(inp.x), dev(inp.y), dev(r), dev(w1), dev(w2)
    src = dev(inp.senders.astype(np.int32))
    row_ptr = E.e3conv_csr_from_receivers(dev(inp.receivers.astype(np.int32)), N)
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    out = torch.empty((N, w.num_out, C), dtype=torch.float32, device="cuda")
    fused_ms = _timed(lambda: plan.forward_radial(x, y, rr, W1, W2, src, row_ptr, w.radius, 0.5, out=out),
                      args.steps, args.warmup)
    # the same convolution reading precomputed scalars (E, P, C) from memory
    s = dev(inp.s)
    plain_ms = _timed(lambda: plan.forward(x, y, s, src, row_ptr, out=out), args.steps, args.warmup)
    # the unfused composition for comparison: the network as torch (hipBLAS) GEMMs writing s, then
    # the plain forward reading it
    nb_, hid_ = w1.shape
    centers = torch.arange(nb_, device="cuda", dtype=torch.float32) * (w.radius / (nb_ - 1))

    def unfused():
        f = torch.exp(-((rr[:, None] - centers[None, :]) / 0.5) ** 2) * \
            (0.5 * (1.0 + torch.cos(math.pi * rr / w.radius)))[:, None]
        h = f @ W1
        s_ = (h * torch.sigmoid(h)) @ W2
        return plan.forward(x, y, s_.view(Ec, P, C), src, row_ptr, out=out)
    unfused_ms = _timed(unfused, args.steps, args.warmup)
    nb, hid = w1.shape
    flops = 2.0 * Ec * (nb * hid + hid * P * C)
    # second-layer matrix work as issued: tiles of four quads (up to four edges of one receiver;
    # per-work-group rounding of the tile count ignored), hidden units padded to steps of 32,
    # three fp16 products per fp32 product
    deg = np.bincount(inp.receivers, minlength=N)
    issued = 3 * 2.0 * 16 * (-(-hid // 32) * 32) * P * C * float(np.sum((deg + 3) // 4)) / 4
    tf = flops / (fused_ms * 1e-3) / 1e12
    # compulsory bytes: per edge y, r and the sender index; per node x, out and row_ptr
    byt = 4.0 * (Ec * ((w.lmax + 1) ** 2 + 2) + N * (w.num_x + w.num_out) * C + N + 1)
    res = {"metric": "edges/sec, convolution with edge scalars computed in the kernel from edge "
                     "lengths (radial basis + 2-layer network), fp32, 1 MI355X",
           "value": Ec / (fused_ms * 1e-3), "unit": "edges/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": fused_ms, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": (f"{w.name}: radial graph N={N} E={Ec}, {w.irreps_in} (x) SH lmax {w.lmax} "
                                   f"-> {w.irreps_out}, s = silu(rbf({nb}) x cutoff @ W1[{nb}x{hid}]) "
                                   f"@ W2[{hid}x{P * C}] per edge"),
                      "mode": "radial"},
           "fused_ms": fused_ms, "fused_TFLOPs_network": tf,
           "fused_hbm_GBps": byt / (fused_ms * 1e-3) / 1e9,
           "plain_forward_ms_with_precomputed_s": plain_ms,
           "unfused_ms_torch_network_then_forward": unfused_ms,
           "scalar_bytes_not_moved": 2.0 * Ec * P * C * 4,
           "roofline": {"bound": "mfma", "achieved": issued / (fused_ms * 1e-3) / 1e12,
                        "peak": PEAK_FP16_MFMA_TFLOPS, "unit": "TFLOP/s",
                        "frac": issued / (fused_ms * 1e-3) / 1e12 / PEAK_FP16_MFMA_TFLOPS, "traffic": None,
                        "kernel": ("conv_fwd_radial: the fp16 matrix work its network's second layer issues "
                                   "(three fp16 products per fp32 product of two-part operands, tiles of four "
                                   "quads, hidden units padded to 32) against the dense fp16 matrix peak; the "
                                   "tensor product runs on the VALU"),
                        "issued_fp16_flops": issued,
                        "algorithmic_flops": flops,
                        "fp32_equivalent_TFLOPs": tf,
                        "fp32_equivalent_frac_of_fp32_matrix_peak": tf / PEAK_FP32_MFMA_TFLOPS}}
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits
        from oracle import conv, radial
        lay = conv.make_layout(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
        e1 = min(args.cpu_sample_edges, Ec)
        with threadpool_limits(1):
            t0 = time.perf_counter()
            radial.forward_radial(lay, inp.x, inp.y[:e1], r[:e1], w1, w2, w.radius, 0.5,
                                  inp.senders[:e1], inp.receivers[:e1], N)
            dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": e1 / dt, "unit": "edges/s", "cores": 1, "kind": "oracle",
                               "sample": f"first {e1} edges (receiver order), fp64 numpy, {dt:.1f} s"}
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def cpu_baseline_mode(mode, inp, sample_edges):
    """The oracle's variant on the edges of the first receivers (single thread)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import conv, variants
    from equivariant_gnn_message_amd import synth

    w = inp.workload
    lay = conv.make_layout(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    # these passes cost several plain forwards each: a smaller sample keeps ~10-30 s
    e1 = min(sample_edges // (8 if w.dtype == "bf16" else 4), inp.num_edges)
    x = inp.as_f32("x")
    y, s = inp.as_f32("y")[:e1], inp.as_f32("s")[:e1]
    src, dst, N = inp.senders[:e1], inp.receivers[:e1], inp.num_nodes
    with threadpool_limits(1):
        t0 = time.perf_counter()
        if mode == "sender":
            variants.forward_sender(lay, x, y, s, src, dst, N)
            if w.backward:
                variants.backward_sender(lay, x, y, s, inp.g, src, dst, N)
            what = "SENDER forward" + (" + reverse" if w.backward else "")
        elif mode == "jvp":
            dx, dy, ds = (synth.bf16_to_f32(a).reshape(a.shape) if a.dtype == np.uint16 else a
                          for a in synth.make_tangents(inp))
            variants.jvp(lay, x, y, s, dx, dy[:e1], ds[:e1], src, dst, N)
            what = "forward-mode pass"
        else:
            Gx, Gy, Gs = synth.make_tangents(inp)
            variants.double_backward(lay, x, y, s, inp.g, Gx, Gy[:e1], Gs[:e1], src, dst, N)
            what = "second derivatives"
        dt = time.perf_counter() - t0
    return {"value": e1 / dt, "unit": "edges/s", "cores": 1, "kind": "oracle",
            "sample": f"first {e1} edges of the same graph, {what}, fp64 numpy, {dt:.1f} s"}


if __name__ == "__main__":
    main()
