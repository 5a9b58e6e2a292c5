"""GPU parity of the bf16 layout's forward kernels at a tight bar (through the C ABI).

The layout 64x(0e+1o+2e), SH lmax 3 -> 64x(0e+1o+2e+3o) with bf16 storage is
held to far less than the 2e-2 RMS bar of bf16 storage: the stored values are
exact bf16 numbers, every product and sum is fp32 (relative rounding 2^-24
per operation), so the kernels agree with the fp64 oracle on the decoded
values to ~1e-6 RMS.  A bar of 2e-4 RMS holds that arithmetic to account: a
kernel that rounded any intermediate (K, a product, a partial sum) to bf16
(2^-9) would be off by ~1e-2 RMS and fail it.  Every compiled bf16 variant of
the layout runs, in both graph orderings, with padding receivers and with
receivers that have no edges.

The exception is the matrix-core form (RECEIVER variants 6 and 7): its
operands are bf16 by design (u = s x rounded once; K rounded once, or split
into two bf16 parts in variant 7), so it is held to the 2e-2 bar of bf16
storage, and to at least 2e-3 (it must show the rounding it is built on, so
that a silent fall back to the fp32 arithmetic would be noticed).
"""

import numpy as np
import pytest

from oracle import conv, variants
from equivariant_gnn_message_amd import e3conv as E
from equivariant_gnn_message_amd import synth

from ._gpu import rel_err, say

pytestmark = pytest.mark.gpu

TIGHT = 2e-4
BF16_BAR = 2e-2
MATRIX_CORE = (6, 7)        # RECEIVER bf16 variants of this layout on the matrix cores
N_RECEIVER_BF16 = 9         # variants compiled for the layout (a change of the list fails here)


def lay_of(w):
    return conv.make_layout(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)


def bf(a):
    """float array -> bf16 device tensor (round to nearest even) and the decoded values."""
    import torch
    bits = synth.bf16_bits(np.asarray(a, np.float32))
    t = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    return t, synth.bf16_to_f32(bits).reshape(bits.shape)


def i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def run_all_variants(plan, x, y, s, src, row_ptr, ref, label, **kw):
    import torch
    nf, _ = plan.num_variants(E.E3CONV_BF16)
    assert nf >= 1
    receiver = plan.ordering == E.E3CONV_RECEIVER
    if receiver:
        assert nf == N_RECEIVER_BF16, nf
    outs = []
    for v in range(nf):
        plan.set_variant(v, 0)
        say(f"[{label}] bf16 variant {v}")
        out = plan.forward(x, y, s, src, row_ptr, **kw)
        torch.cuda.synchronize()
        err = rel_err(out.cpu().numpy(), ref)
        say(f"  max|err|/RMS = {err:.3e}")
        if receiver and v in MATRIX_CORE:
            assert err <= BF16_BAR, (v, err)
            if np.abs(ref).max() > 0:
                assert err >= 2e-3, (v, err)
        else:
            assert err <= TIGHT, (v, err)
        outs.append(out)
    plan.set_variant(0, 0)
    return outs


@pytest.mark.parametrize("n", [37, 601, 2000])
def test_receiver_all_variants_tight(n):
    inp = synth.make_inputs(3, num_nodes=n)
    w = inp.workload
    x, y, s = (inp.as_f32(k) for k in ("x", "y", "s"))
    ref = conv.forward(lay_of(w), x, y, s, inp.senders, inp.receivers, inp.num_nodes)
    d = {k: bf(a)[0] for k, a in (("x", x), ("y", y), ("s", s))}
    src = i32(inp.senders)
    row_ptr = E.e3conv_csr_from_receivers(i32(inp.receivers), inp.num_nodes)
    say(f"[receiver] N={inp.num_nodes} E={inp.num_edges}")
    run_all_variants(E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors),
                     d["x"], d["y"], d["s"], src, row_ptr, ref, f"receiver N={n}")


def test_empty_receivers_and_empty_graph():
    """Receivers without edges get exact zero rows; a graph without edges is all zeros."""
    import torch
    inp = synth.make_inputs(3, num_nodes=400)
    w = inp.workload
    keep = (inp.receivers % 5 != 0) & (inp.receivers < 380)     # every 5th receiver and the tail: empty
    src, dst = inp.senders[keep], inp.receivers[keep]
    x, y, s = inp.as_f32("x"), inp.as_f32("y")[keep], inp.as_f32("s")[keep]
    N = inp.num_nodes
    ref = conv.forward(lay_of(w), x, y, s, src, dst, N)
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    row_ptr = E.e3conv_csr_from_receivers(i32(dst), N)
    outs = run_all_variants(plan, bf(x)[0], bf(y)[0], bf(s)[0], i32(src), row_ptr, ref, "empty rows",
                            out=None)
    empty = np.setdiff1d(np.arange(N), dst)
    assert len(empty) > 60
    for out in outs:
        assert torch.all(out[torch.from_numpy(empty).cuda()] == 0)
    # no edges at all
    zs = np.zeros((0,) + s.shape[1:], np.float32)
    zy = np.zeros((0,) + y.shape[1:], np.float32)
    row_ptr0 = E.e3conv_csr_from_receivers(i32(np.zeros(0)), N)
    nf, _ = plan.num_variants(E.E3CONV_BF16)
    for v in range(nf):
        plan.set_variant(v, 0)
        out = torch.full((N, 16, 64), 3.0, device="cuda")
        plan.forward(bf(x)[0], bf(zy)[0], bf(zs)[0], i32(np.zeros(0)), row_ptr0, out=out)
        torch.cuda.synchronize()
        assert torch.all(out == 0), v


@pytest.mark.parametrize("use_order", [False, True], ids=["index", "clustered"])
def test_padding_receivers_all_variants(use_order):
    import torch
    inp = synth.make_inputs(3, num_nodes=301)
    w = inp.workload
    lay = lay_of(w)
    rng = np.random.default_rng(17)
    n_pad, e_pad = 29, 120
    N = inp.num_nodes + n_pad
    src = np.concatenate([inp.senders, rng.integers(inp.num_nodes, N, e_pad)])
    dst = np.concatenate([inp.receivers, np.sort(rng.integers(inp.num_nodes, N, e_pad))])
    x = np.concatenate([inp.as_f32("x"), rng.standard_normal((n_pad, lay.num_x, 64)).astype(np.float32)])
    y = np.concatenate([inp.as_f32("y"), synth.spherical_harmonics(3, rng.standard_normal((e_pad, 3))).astype(np.float32)])
    s = np.concatenate([inp.as_f32("s"), rng.standard_normal((e_pad, lay.num_paths, 64)).astype(np.float32)])
    (xt, xd), (yt, yd), (st, sd) = bf(x), bf(y), bf(s)
    ref = variants.forward_masked(lay, xd, yd, sd, src, dst, N, inp.num_nodes)
    row_ptr = E.e3conv_csr_from_receivers(i32(dst), N)
    order = None
    if use_order:
        order = i32(E.e3conv_receiver_order(row_ptr.cpu().numpy(), src.astype(np.int32), N, len(src), 64))
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    outs = run_all_variants(plan, xt, yt, st, i32(src), row_ptr, ref, f"padding order={use_order}",
                            order=order, num_real_nodes=inp.num_nodes)
    for out in outs:
        assert torch.all(out[inp.num_nodes:] == 0)


def test_sender_ordering_all_variants_tight():
    inp = synth.make_inputs(3, num_nodes=401)
    w = inp.workload
    perm = synth.sender_sorted(inp.senders, inp.receivers)
    src, dst = inp.senders[perm], inp.receivers[perm]
    x, y, s = inp.as_f32("x"), inp.as_f32("y")[perm], inp.as_f32("s")[perm]
    ref = variants.forward_sender(lay_of(w), x, y, s, src, dst, inp.num_nodes)
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors, ordering=E.E3CONV_SENDER)
    row_ptr = E.e3conv_csr_from_receivers(i32(src), inp.num_nodes)
    run_all_variants(plan, bf(x)[0], bf(y)[0], bf(s)[0], i32(dst), row_ptr, ref, "sender")
