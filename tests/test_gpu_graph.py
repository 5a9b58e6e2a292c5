"""The library's calls captured in a HIP graph (through torch.cuda.CUDAGraph).

Every compute call enqueues kernels on the caller's stream, allocates nothing
and records no memset (grad_x is cleared by a fill kernel), so a training
step can be captured once and replayed. Each case replays the graph several
times, with eager work on the same buffers between the replays, and checks
every replay against the eager result: bit for bit, except grad_x, whose
fp32 atomics may add in another order (within the 1e-5 RMS bar).
"""

import numpy as np
import pytest

from equivariant_gnn_message_amd import e3conv as E
from equivariant_gnn_message_amd import synth

from ._gpu import rel_err, say

pytestmark = pytest.mark.gpu


def _dev(a, dtype=None):
    import torch
    a = np.ascontiguousarray(a if dtype is None else a.astype(dtype))
    return torch.from_numpy(a).cuda()


def test_training_step_graph_replays():
    import torch
    inp = synth.make_inputs(4, num_nodes=601)
    w, N = inp.workload, inp.num_nodes
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    x, y, s, g = _dev(inp.x), _dev(inp.y), _dev(inp.s), _dev(inp.g)
    src = _dev(inp.senders, np.int32)
    row_ptr = E.e3conv_csr_from_receivers(_dev(inp.receivers, np.int32), N)
    order = _dev(E.e3conv_receiver_order(row_ptr.cpu().numpy(), inp.senders, N, inp.num_edges, 64))
    out = torch.empty((N, w.num_out, w.channels), device="cuda")
    grads = (torch.empty_like(x), torch.empty_like(y), torch.empty_like(s))

    def step():
        plan.forward(x, y, s, src, row_ptr, out=out, order=order)
        plan.backward(x, y, s, src, row_ptr, g, grads=grads, order=order)

    step()
    torch.cuda.synchronize()
    ref = [out.clone()] + [t.clone() for t in grads]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # warm-up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    say(f"[graph] training step captured, N={N} E={inp.num_edges}")
    for r in range(4):
        # eager work on the same buffers between replays
        out.fill_(3.0)
        for t in grads:
            t.fill_(-1.0)
        E.e3conv_forward(plan.handle, x, y, s, src, row_ptr, N, inp.num_edges, out)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [out] + list(grads)
        assert torch.equal(got[0], ref[0]), r
        assert torch.equal(got[2], ref[2]) and torch.equal(got[3], ref[3]), r
        err = rel_err(got[1].cpu().numpy(), ref[1].cpu().numpy())
        say(f"  replay {r}: out, grad_y, grad_s bitwise; grad_x max|err|/RMS {err:.2e}")
        assert err <= 1e-5


def test_pair_step_graph_replays():
    import torch
    inp = synth.make_inputs(4, num_nodes=601)
    w, N, Ec = inp.workload, inp.num_nodes, inp.num_edges
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    rp = np.searchsorted(inp.receivers, np.arange(N + 1)).astype(np.int32)
    stored, pmap = E.e3conv_pair_layout(rp, inp.senders, N, Ec, 64)
    Ep = len(stored)
    s_p = synth.normal_f32(w.idx, synth.T_S_PAIR, (Ep, w.num_paths, w.channels))
    x, g, y, s = _dev(inp.x), _dev(inp.g), _dev(inp.y[stored]), _dev(s_p)
    dsrc, m = _dev(inp.senders, np.int32), _dev(pmap)
    psrc, pdst = _dev(inp.senders[stored], np.int32), _dev(inp.receivers[stored], np.int32)
    row_ptr = E.e3conv_csr_from_receivers(_dev(inp.receivers, np.int32), N)
    out = torch.empty((N, w.num_out, w.channels), device="cuda")
    gx, gy, gs = torch.empty_like(x), torch.empty_like(y), torch.empty_like(s)

    def step():
        E.e3conv_forward_pairs(plan.handle, x, y, s, dsrc, row_ptr, m, N, Ec, Ep, out)
        E.e3conv_backward_pairs(plan.handle, x, y, s, psrc, pdst, N, Ep, g, gx, gy, gs)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, gx, gy, gs)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    say(f"[graph] pair-stored step captured, N={N} pairs={Ep}")
    for r in range(3):
        for t in (out, gx, gy, gs):
            t.fill_(5.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(gy, ref[2]) and torch.equal(gs, ref[3]), r
        assert rel_err(gx.cpu().numpy(), ref[1].cpu().numpy()) <= 1e-5, r
