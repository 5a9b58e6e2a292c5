"""Helpers for the GPU tests: move seeded inputs to the device, call the library."""

import math
import sys

import numpy as np

from equivariant_gnn_message_amd import e3conv as E
from equivariant_gnn_message_amd import synth


def say(*msg):
    print(*msg, flush=True)
    sys.stdout.flush()


def device_inputs(inp):
    """torch device tensors for x, y, s (f32 or bf16), src, receivers, g."""
    import torch
    dev = torch.device("cuda:0")

    def t(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    d = {k: t(getattr(inp, k)) for k in ("x", "y", "s", "g")}
    d["src"] = t(inp.senders.astype(np.int32))
    d["dst"] = t(inp.receivers.astype(np.int32))
    d["row_ptr"] = E.e3conv_csr_from_receivers(d["dst"], inp.num_nodes)
    return d


def plan_for(inp):
    w = inp.workload
    return E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = math.sqrt(float(np.mean(ref ** 2)))
    err = float(np.max(np.abs(got - ref)))
    return err / rms if rms > 0 else err


def tolerance(inp):
    return 2e-2 if inp.workload.dtype == "bf16" else 1e-5


def oracle_inputs(inp):
    return inp.as_f32("x"), inp.as_f32("y"), inp.as_f32("s")


def sample_rows(inp, k=96, seed=0):
    """Receivers for sampled checks: random ones plus extremes of the degree range."""
    deg = np.diff(np.searchsorted(inp.receivers, np.arange(inp.num_nodes + 1)))
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(inp.num_nodes, size=min(k, inp.num_nodes), replace=False).tolist())
    rows |= {0, inp.num_nodes - 1, int(np.argmax(deg)), int(np.argmin(deg))}
    return np.array(sorted(rows), dtype=np.int64)


def edges_of_rows(inp, rows):
    ptr = np.searchsorted(inp.receivers, np.arange(inp.num_nodes + 1))
    return np.concatenate([np.arange(ptr[b], ptr[b + 1]) for b in rows]) if len(rows) else np.zeros(0, np.int64)
