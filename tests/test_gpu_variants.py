"""GPU parity of the SENDER ordering, node-mask padding and forward-mode kernels.

Each case compares the library (through the C ABI) with ``oracle.variants``
element by element; bar 1e-5 RMS for fp32 operands, 2e-2 RMS for bf16.
"""

import numpy as np
import pytest

from oracle import conv, variants
from equivariant_gnn_message_amd import e3conv as E
from equivariant_gnn_message_amd import synth

from ._gpu import rel_err, say, tolerance

pytestmark = pytest.mark.gpu


def lay_of(inp):
    w = inp.workload
    return conv.make_layout(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)


def dev(a, bf16=False):
    import torch
    if bf16:
        return torch.from_numpy(synth.bf16_bits(np.asarray(a, np.float32)).view(np.int16)).cuda().view(torch.bfloat16)
    if a.dtype == np.float64:
        a = a.astype(np.float32)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def decoded(a, bf16):
    a = np.asarray(a, np.float32)
    return synth.bf16_to_f32(synth.bf16_bits(a)).reshape(a.shape) if bf16 else a


def sender_sorted_inputs(idx, n, symmetric_s=False):
    """Operands of workload idx on n nodes, edges re-sorted by sender (fp32 arrays)."""
    inp = synth.make_inputs(idx, num_nodes=n, with_cotangent=True)
    x, y, s = inp.as_f32("x"), inp.as_f32("y"), inp.as_f32("s")
    src, dst = inp.senders, inp.receivers
    if symmetric_s:
        s = synth.symmetric_normal(src, dst, s.shape[1:], 99).astype(np.float32)
    perm = synth.sender_sorted(src, dst)
    return inp, x, y[perm], s[perm], src[perm], dst[perm], inp.g


@pytest.mark.parametrize("idx,n", [(0, None), (2, 601), (3, 601)], ids=["w0", "w2-n601", "w3bf16-n601"])
def test_sender_forward_parity(idx, n):
    import torch
    inp, x, y, s, src, dst, _ = sender_sorted_inputs(idx, n)
    bf = inp.workload.dtype == "bf16"
    x, y, s = decoded(x, bf), decoded(y, bf), decoded(s, bf)
    N = inp.num_nodes
    say(f"[sender fwd] workload {idx} N={N} E={len(src)}")
    ref = variants.forward_sender(lay_of(inp), x, y, s, src, dst, N)
    w = inp.workload
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors, ordering=E.E3CONV_SENDER)
    assert plan.ordering == E.E3CONV_SENDER
    srt = dev(src.astype(np.int32))
    row_ptr = E.e3conv_csr_from_receivers(srt, N)
    out = plan.forward(dev(x, bf), dev(y, bf), dev(s, bf), dev(dst.astype(np.int32)), row_ptr)
    torch.cuda.synchronize()
    err = rel_err(out.cpu().numpy(), ref)
    say(f"  max|err|/RMS {err:.3e}")
    assert err <= tolerance(inp)


def test_sender_equals_receiver_on_symmetric_graph():
    """The e3j page's SENDER assumptions hold: both orderings give the same output."""
    import torch
    inp, x, y, s, src, dst, _ = sender_sorted_inputs(2, 601, symmetric_s=True)
    w, N = inp.workload, inp.num_nodes
    # RECEIVER order of the same edges
    rperm = np.lexsort((src, dst))
    recv = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    send = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors, ordering=E.E3CONV_SENDER)
    out_r = recv.forward(dev(x), dev(y[rperm]), dev(s[rperm]), dev(src[rperm].astype(np.int32)),
                         E.e3conv_csr_from_receivers(dev(dst[rperm].astype(np.int32)), N))
    out_s = send.forward(dev(x), dev(y), dev(s), dev(dst.astype(np.int32)),
                         E.e3conv_csr_from_receivers(dev(src.astype(np.int32)), N))
    torch.cuda.synchronize()
    err = rel_err(out_s.cpu().numpy(), out_r.cpu().numpy())
    say(f"[sender = receiver] N={N} E={len(src)} max|diff|/RMS {err:.3e}")
    assert err <= 1e-5


@pytest.mark.parametrize("idx,n", [(0, None), (4, 401)], ids=["w0", "w4-n401"])
def test_sender_backward_parity(idx, n):
    import torch
    inp, x, y, s, src, dst, g = sender_sorted_inputs(idx, n)
    N = inp.num_nodes
    say(f"[sender bwd] workload {idx} N={N} E={len(src)}")
    rx, ry, rs = variants.backward_sender(lay_of(inp), x, y, s, g, src, dst, N)
    w = inp.workload
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors, ordering=E.E3CONV_SENDER)
    row_ptr = E.e3conv_csr_from_receivers(dev(src.astype(np.int32)), N)
    gx, gy, gs = plan.backward(dev(x), dev(y), dev(s), dev(dst.astype(np.int32)), row_ptr, dev(g))
    torch.cuda.synchronize()
    errs = [rel_err(a.cpu().numpy(), b) for a, b in ((gx, rx), (gy, ry), (gs, rs))]
    say(f"  max|err|/RMS dx {errs[0]:.3e} dy {errs[1]:.3e} ds {errs[2]:.3e}")
    assert max(errs) <= 1e-5


def padded_inputs(idx, n_real, n_pad=37, e_pad=150, seed=3):
    """Workload idx on n_real nodes plus padding nodes and edges among them (receiver sorted)."""
    inp = synth.make_inputs(idx, num_nodes=n_real, with_cotangent=True)
    rng = np.random.default_rng(seed)
    N = inp.num_nodes + n_pad
    lay = lay_of(inp)
    C = lay.channels
    ps = rng.integers(inp.num_nodes, N, e_pad)
    pd = np.sort(rng.integers(inp.num_nodes, N, e_pad))
    src = np.concatenate([inp.senders, ps])
    dst = np.concatenate([inp.receivers, pd])
    x = np.concatenate([inp.as_f32("x"), rng.standard_normal((n_pad, lay.num_x, C)).astype(np.float32)])
    y = np.concatenate([inp.as_f32("y"),
                        synth.spherical_harmonics(lay.lmax, rng.standard_normal((e_pad, 3))).astype(np.float32)])
    s = np.concatenate([inp.as_f32("s"), rng.standard_normal((e_pad, lay.num_paths, C)).astype(np.float32)])
    g = np.concatenate([inp.g, rng.standard_normal((n_pad, lay.num_out, C)).astype(np.float32)])
    return inp, lay, x, y, s, g, src, dst, N, inp.num_nodes


@pytest.mark.parametrize("use_order", [False, True], ids=["index", "clustered"])
def test_masked_forward_and_backward_parity(use_order):
    import torch
    inp, lay, x, y, s, g, src, dst, N, n_real = padded_inputs(4, 301)
    say(f"[masked] N={N} real={n_real} E={len(src)} order={use_order}")
    ref = variants.forward_masked(lay, x, y, s, src, dst, N, n_real)
    rx, ry, rs = variants.backward_masked(lay, x, y, s, g, src, dst, N, n_real)
    w = inp.workload
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    row_ptr = E.e3conv_csr_from_receivers(dev(dst.astype(np.int32)), N)
    order = None
    if use_order:
        order = dev(E.e3conv_receiver_order(row_ptr.cpu().numpy(), src.astype(np.int32), N, len(src), 64))
    out = torch.full((N, lay.num_out, lay.channels), 7.0, device="cuda")
    plan.forward(dev(x), dev(y), dev(s), dev(src.astype(np.int32)), row_ptr, out=out, order=order,
                 num_real_nodes=n_real)
    grads = tuple(torch.full_like(dev(a), 7.0) for a in (x, y, s))
    gx, gy, gs = plan.backward(dev(x), dev(y), dev(s), dev(src.astype(np.int32)), row_ptr, dev(g),
                               grads=grads, order=order, num_real_nodes=n_real)
    torch.cuda.synchronize()
    errs = [rel_err(a.cpu().numpy(), b) for a, b in ((out, ref), (gx, rx), (gy, ry), (gs, rs))]
    say(f"  max|err|/RMS out {errs[0]:.3e} dx {errs[1]:.3e} dy {errs[2]:.3e} ds {errs[3]:.3e}")
    assert max(errs) <= 1e-5
    assert torch.all(out[n_real:] == 0) and torch.all(gy[len(inp.senders):] == 0)
    assert torch.all(gs[len(inp.senders):] == 0)


def test_masked_rejects_bad_count():
    inp = synth.make_inputs(0)
    w = inp.workload
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    x, y, s = dev(inp.x), dev(inp.y), dev(inp.s)
    src = dev(inp.senders.astype(np.int32))
    row_ptr = E.e3conv_csr_from_receivers(dev(inp.receivers.astype(np.int32)), inp.num_nodes)
    with pytest.raises(E.E3ConvError):
        plan.forward(x, y, s, src, row_ptr, num_real_nodes=inp.num_nodes + 1)
    with pytest.raises(E.E3ConvError):
        plan.forward(x, y, s, src, row_ptr, num_real_nodes=-1)


@pytest.mark.parametrize("idx,n,ordering,force_bf", [(0, None, 0, False), (1, None, 0, False),
                                                     (2, 601, 0, False), (3, 601, 0, False),
                                                     (2, 401, 1, False), (2, 501, 0, True),
                                                     (3, 401, 1, False)],
                         ids=["w0", "w1", "w2-n601", "w3bf16-n601", "w2-n401-sender", "w2bf16-n501",
                              "w3bf16-n401-sender"])
def test_jvp_parity(idx, n, ordering, force_bf):
    import torch
    inp = synth.make_inputs(idx, num_nodes=n) if n else synth.make_inputs(idx)
    bf = inp.workload.dtype == "bf16" or force_bf
    lay = lay_of(inp)
    x, y, s = inp.as_f32("x"), inp.as_f32("y"), inp.as_f32("s")
    src, dst, N = inp.senders, inp.receivers, inp.num_nodes
    if ordering == E.E3CONV_SENDER:
        perm = synth.sender_sorted(src, dst)
        y, s, src, dst = y[perm], s[perm], src[perm], dst[perm]
    rng = np.random.default_rng(idx + 40)
    dx, dy, ds = (decoded(rng.standard_normal(a.shape), bf) for a in (x, y, s))
    x, y, s = decoded(x, bf), decoded(y, bf), decoded(s, bf)
    say(f"[jvp] workload {idx} N={N} E={len(src)} ordering={ordering}")
    if ordering == E.E3CONV_SENDER:
        sign = variants.parity_sign(lay)
        ref, ref_dot = variants.jvp(lay, x, y * sign, s, dx, dy * sign, ds, dst, src, N)
        gather, seg = dst, src
    else:
        ref, ref_dot = variants.jvp(lay, x, y, s, dx, dy, ds, src, dst, N)
        gather, seg = src, dst
    w = inp.workload
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors, ordering=ordering)
    row_ptr = E.e3conv_csr_from_receivers(dev(seg.astype(np.int32)), N)
    out, out_dot = plan.jvp(dev(x, bf), dev(y, bf), dev(s, bf), dev(dx, bf), dev(dy, bf), dev(ds, bf),
                            dev(gather.astype(np.int32)), row_ptr)
    _, only_dot = plan.jvp(dev(x, bf), dev(y, bf), dev(s, bf), dev(dx, bf), dev(dy, bf), dev(ds, bf),
                           dev(gather.astype(np.int32)), row_ptr, want_out=False)
    torch.cuda.synchronize()
    errs = [rel_err(out.cpu().numpy(), ref), rel_err(out_dot.cpu().numpy(), ref_dot),
            rel_err(only_dot.cpu().numpy(), ref_dot)]
    say(f"  max|err|/RMS out {errs[0]:.3e} out_dot {errs[1]:.3e} (tangent only {errs[2]:.3e})")
    # operands rounded to bf16 on both sides: the kernel adds fp32 rounding only (the
    # tight bf16 bar of test_gpu_bf16_tight)
    assert max(errs) <= (2e-4 if force_bf else tolerance(inp))


def test_backward_ex_optional_outputs_and_accumulation():
    import torch
    inp = synth.make_inputs(4, num_nodes=301, with_cotangent=True)
    lay = lay_of(inp)
    say(f"[reverse, general] N={inp.num_nodes} E={inp.num_edges}")
    rx, ry, rs = conv.backward(lay, inp.x, inp.y, inp.s, inp.g, inp.senders, inp.receivers,
                               inp.num_nodes)
    w = inp.workload
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    x, y, s, g = dev(inp.x), dev(inp.y), dev(inp.s), dev(inp.g)
    src = dev(inp.senders.astype(np.int32))
    row_ptr = E.e3conv_csr_from_receivers(dev(inp.receivers.astype(np.int32)), inp.num_nodes)
    gy, gs = torch.empty_like(y), torch.empty_like(s)
    plan.backward(x, y, s, src, row_ptr, g, grads=(None, gy, gs))
    gx = torch.empty_like(x)
    plan.backward(x, y, s, src, row_ptr, g, grads=(gx, None, None))
    rng = np.random.default_rng(4)
    pre = [rng.standard_normal(a.shape).astype(np.float32) for a in (rx, ry, rs)]
    acc = tuple(dev(a) for a in pre)
    plan.backward(x, y, s, src, row_ptr, g, grads=acc, accumulate=(True, True, True))
    torch.cuda.synchronize()
    errs = [rel_err(gx.cpu().numpy(), rx), rel_err(gy.cpu().numpy(), ry), rel_err(gs.cpu().numpy(), rs)]
    errs += [rel_err(a.cpu().numpy() - p, r) for a, p, r in zip(acc, pre, (rx, ry, rs))]
    say("  max|err|/RMS " + " ".join(f"{e:.3e}" for e in errs))
    assert max(errs) <= 1e-5


@pytest.mark.parametrize("idx,n", [(0, None), (4, 201)], ids=["w0", "w4-n201"])
def test_second_derivatives(idx, n):
    """Reverse over reverse through E3ConvFunction against the oracle."""
    import torch
    inp = synth.make_inputs(idx, num_nodes=n, with_cotangent=True) if n else \
        synth.make_inputs(idx, with_cotangent=True)
    lay = lay_of(inp)
    N = inp.num_nodes
    rng = np.random.default_rng(idx + 70)
    G = [rng.standard_normal(a.shape).astype(np.float32) for a in (inp.x, inp.y, inp.s)]
    say(f"[second derivatives] workload {idx} N={N} E={inp.num_edges}")
    ref = variants.double_backward(lay, inp.x, inp.y, inp.s, inp.g, *G, inp.senders,
                                   inp.receivers, N)
    w = inp.workload
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    x, y, s, g = (dev(a).requires_grad_(True) for a in (inp.x, inp.y, inp.s, inp.g))
    src = dev(inp.senders.astype(np.int32))
    row_ptr = E.e3conv_csr_from_receivers(dev(inp.receivers.astype(np.int32)), N)
    out = E.E3ConvFunction.apply(plan, x, y, s, src, row_ptr)
    first = torch.autograd.grad(out, (x, y, s), g, create_graph=True)
    second = torch.autograd.grad(first, (x, y, s, g), tuple(dev(a) for a in G))
    torch.cuda.synchronize()
    errs = [rel_err(a.detach().cpu().numpy(), b) for a, b in zip(second, ref)]
    say("  max|err|/RMS dx {:.3e} dy {:.3e} ds {:.3e} dg {:.3e}".format(*errs))
    assert max(errs) <= 1e-5


def _rows_and_edges(seg, N, k=48, seed=0):
    """Sampled segment nodes (random plus the heaviest) and the edges of each."""
    ptr = np.searchsorted(seg, np.arange(N + 1))
    deg = np.diff(ptr)
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([rng.choice(N, k, replace=False), [int(np.argmax(deg)), 0, N - 1]]))
    edges = np.concatenate([np.arange(ptr[b], ptr[b + 1]) for b in rows])
    return rows, edges, ptr


def test_sender_full_size_sampled():
    """SENDER ordering at the full training-workload size, sampled rows against the oracle."""
    import torch
    inp, x, y, s, src, dst, g = sender_sorted_inputs(4, None)
    N, E_ = inp.num_nodes, len(src)
    say(f"[sender full] N={N} E={E_}")
    w = inp.workload
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors, ordering=E.E3CONV_SENDER)
    row_ptr = E.e3conv_csr_from_receivers(dev(src.astype(np.int32)), N)
    order = dev(E.e3conv_receiver_order(row_ptr.cpu().numpy(), dst.astype(np.int32), N, E_, 512))
    out = plan.forward(dev(x), dev(y), dev(s), dev(dst.astype(np.int32)), row_ptr, order=order)
    torch.cuda.synchronize()
    rows, edges, _ = _rows_and_edges(src, N)
    ref = variants.forward_sender(lay_of(inp), x, y[edges], s[edges], src[edges], dst[edges], N)[rows]
    err = rel_err(out.cpu().numpy()[rows], ref)
    say(f"  {len(rows)} rows, max|err|/RMS {err:.3e}")
    assert err <= 1e-5


def test_jvp_full_size_sampled():
    """Forward mode at the full MACE-scale size, sampled receivers against the oracle."""
    import torch
    inp = synth.make_inputs(2)
    N = inp.num_nodes
    say(f"[jvp full] N={N} E={inp.num_edges}")
    dx, dy, ds = synth.make_tangents(inp)
    w = inp.workload
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    row_ptr = E.e3conv_csr_from_receivers(dev(inp.receivers.astype(np.int32)), N)
    out, out_dot = plan.jvp(dev(inp.x), dev(inp.y), dev(inp.s), dev(dx), dev(dy), dev(ds),
                            dev(inp.senders.astype(np.int32)), row_ptr)
    torch.cuda.synchronize()
    rows, edges, _ = _rows_and_edges(inp.receivers, N, seed=1)
    r, rd = variants.jvp(lay_of(inp), inp.x, inp.y[edges], inp.s[edges], dx, dy[edges], ds[edges],
                         inp.senders[edges], inp.receivers[edges], N)
    errs = [rel_err(out.cpu().numpy()[rows], r[rows]), rel_err(out_dot.cpu().numpy()[rows], rd[rows])]
    say(f"  {len(rows)} rows, max|err|/RMS out {errs[0]:.3e} out_dot {errs[1]:.3e}")
    assert max(errs) <= 1e-5
