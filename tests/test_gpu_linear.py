"""GPU parity of the output linear (fp32 MFMA GEMMs) against oracle.linear.

Bar: max|gpu - oracle| <= 1e-5 RMS(oracle) for out, grad_in and grad_weights.
"""

import numpy as np
import pytest

from oracle import conv, linear
from equivariant_gnn_message_amd import e3conv as E
from equivariant_gnn_message_amd import synth

from ._gpu import rel_err, say

pytestmark = pytest.mark.gpu


def cuda(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def icuda(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


@pytest.mark.parametrize("idx,C,Co,N", [(2, 128, 128, 301), (2, 128, 64, 1000), (0, 8, 16, 64),
                                        (3, 64, 32, 257), (1, 32, 48, 5), (2, 128, 128, 20000),
                                        (0, 20, 24, 33), (1, 12, 136, 77), (3, 64, 64, 300),
                                        (1, 32, 32, 1000)],
                         ids=["mace-301", "mace-64out-1000", "tiny-64", "big-257", "gate-5",
                              "mace-full", "k20-unaligned", "wide-136", "big-64x64", "gate-32x32"])
def test_linear_parity(idx, C, Co, N):
    import torch
    w = synth.WORKLOADS[idx]
    irin = w.irreps_in.replace(f"{w.channels}x", f"{C}x")
    irout = w.irreps_out.replace(f"{w.channels}x", f"{C}x")
    lay = conv.make_layout(irin, w.lmax, irout)
    plan = E.Plan(irin, w.lmax, irout)
    nb = plan.num_out_blocks()
    rng = np.random.default_rng(N + Co)
    x = rng.standard_normal((N, lay.num_out, C)).astype(np.float32)
    W = rng.standard_normal((nb, C, Co)).astype(np.float32)
    g = rng.standard_normal((N, lay.num_out, Co)).astype(np.float32)
    scale = 0.8
    say(f"[linear] {irout} C={C} C_out={Co} N={N}")
    ref = linear.linear(lay, W, scale, x)
    rdx, rdw = linear.linear_backward(lay, W, scale, x, g)
    out = plan.linear(cuda(x), cuda(W), Co, scale)
    gi, gw = plan.linear_backward(cuda(x), cuda(W), Co, cuda(g), scale)
    torch.cuda.synchronize()
    errs = [rel_err(out.cpu().numpy(), ref), rel_err(gi.cpu().numpy(), rdx), rel_err(gw.cpu().numpy(), rdw)]
    say("  max|err|/RMS out {:.3e} grad_in {:.3e} grad_w {:.3e}".format(*errs))
    assert max(errs) <= 1e-5


def test_conv_then_linear():
    """The step after the convolution: conv output fed to the linear, end to end."""
    import torch
    inp = synth.make_inputs(2, num_nodes=401)
    w = inp.workload
    lay = conv.make_layout(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    rng = np.random.default_rng(8)
    W = rng.standard_normal((plan.num_out_blocks(), w.channels, 96)).astype(np.float32)
    ref = linear.linear(lay, W, 1.0, conv.forward(lay, inp.x, inp.y, inp.s, inp.senders,
                                                  inp.receivers, inp.num_nodes))
    row_ptr = E.e3conv_csr_from_receivers(icuda(inp.receivers), inp.num_nodes)
    m = plan.forward(cuda(inp.x), cuda(inp.y), cuda(inp.s), icuda(inp.senders), row_ptr)
    out = plan.linear(m, cuda(W), 96)
    torch.cuda.synchronize()
    err = rel_err(out.cpu().numpy(), ref)
    say(f"[conv -> linear] N={inp.num_nodes} max|err|/RMS {err:.3e}")
    assert err <= 1e-5


def _bf16_dev(a):
    import torch
    return torch.from_numpy(synth.bf16_bits(np.asarray(a, np.float32)).view(np.int16)).cuda().view(torch.bfloat16)


@pytest.mark.parametrize("idx,kw,bf16", [(0, {}, False), (1, {"num_graphs": 6}, False),
                                         (3, {"num_nodes": 501}, True), (3, {"num_nodes": 301}, False),
                                         (0, {}, True), (1, {"num_graphs": 2}, True)],
                         ids=["tiny", "gate", "big-bf16", "big-f32", "tiny-bf16", "gate-bf16"])
def test_forward_linear_fused_parity(idx, kw, bf16):
    """e3conv_forward_linear against oracle.linear(oracle.conv(...)) on the layouts of
    up to 64 channels, and against the two separate calls on the device."""
    import torch
    inp = synth.make_inputs(idx, **kw)
    w = inp.workload
    lay = conv.make_layout(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    x, y, s = inp.as_f32("x"), inp.as_f32("y"), inp.as_f32("s")
    if bf16:        # the values the kernel reads
        x, y, s = (synth.bf16_to_f32(synth.bf16_bits(a.astype(np.float32))).reshape(a.shape) for a in (x, y, s))
    rng = np.random.default_rng(idx + 70)
    W = rng.standard_normal((plan.num_out_blocks(), w.channels, w.channels)).astype(np.float32)
    scale = 0.7
    N, Ec = inp.num_nodes, inp.num_edges
    ref = linear.linear(lay, W, scale, conv.forward(lay, x, y, s, inp.senders, inp.receivers, N))
    dev = _bf16_dev if bf16 else cuda
    dx, dy, ds = dev(x), dev(y), dev(s)
    src = icuda(inp.senders)
    row_ptr = E.e3conv_csr_from_receivers(icuda(inp.receivers), N)
    out = torch.full((N, lay.num_out, w.channels), 3.0, device="cuda")
    E.e3conv_forward_linear(plan.handle, dx, dy, ds, src, row_ptr, N, Ec, scale, cuda(W), out)
    sep = plan.linear(plan.forward(dx, dy, ds, src, row_ptr), cuda(W), w.channels, scale)
    torch.cuda.synchronize()
    err, err_sep = rel_err(out.cpu().numpy(), ref), rel_err(sep.cpu().numpy(), ref)
    say(f"[forward+linear fused] {w.name} bf16={bf16} N={N} E={Ec} max|err|/RMS {err:.3e} "
        f"(separate calls {err_sep:.3e})")
    assert err <= 1e-5 and err_sep <= 1e-5


def test_forward_linear_edge_cases():
    """Receivers without edges, a graph without edges, a receiver order, and the
    128-channel layout (not compiled: the separate calls serve it)."""
    import torch
    w = synth.WORKLOADS[1]
    lay = conv.make_layout(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    rng = np.random.default_rng(3)
    N, Ec = 90, 400
    dst = np.sort(rng.integers(0, 60, Ec))            # receivers 60..89 take no edges
    src = rng.integers(0, N, Ec)
    x = rng.standard_normal((N, lay.num_x, w.channels)).astype(np.float32)
    y = synth.spherical_harmonics(w.lmax, rng.standard_normal((Ec, 3))).astype(np.float32)
    s = rng.standard_normal((Ec, lay.num_paths, w.channels)).astype(np.float32)
    W = rng.standard_normal((plan.num_out_blocks(), w.channels, w.channels)).astype(np.float32)
    ref = linear.linear(lay, W, 1.3, conv.forward(lay, x, y, s, src, dst, N))
    row_ptr = E.e3conv_csr_from_receivers(icuda(dst), N)
    order = icuda(rng.permutation(N))
    out = torch.full((N, lay.num_out, w.channels), 3.0, device="cuda")
    E.e3conv_forward_linear(plan.handle, cuda(x), cuda(y), cuda(s), icuda(src), row_ptr, N, Ec, 1.3,
                            cuda(W), out, order=order)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert rel_err(got, ref) <= 1e-5 and np.all(got[60:] == 0.0)
    # no edges at all: zero rows
    e0 = torch.zeros(0, dtype=torch.int32, device="cuda")
    out0 = torch.full((N, lay.num_out, w.channels), 3.0, device="cuda")
    E.e3conv_forward_linear(plan.handle, cuda(x), torch.zeros(0, lay.num_y, device="cuda"),
                            torch.zeros(0, lay.num_paths, w.channels, device="cuda"), e0,
                            E.e3conv_csr_from_receivers(e0, N), N, 0, 1.0, cuda(W), out0)
    torch.cuda.synchronize()
    assert float(out0.abs().max()) == 0.0
    w2 = synth.WORKLOADS[2]
    big = E.Plan(w2.irreps_in, w2.lmax, w2.irreps_out, w2.avg_num_neighbors)
    with pytest.raises(E.E3ConvError) as err:
        E.e3conv_forward_linear(big.handle, cuda(np.zeros((2, 4, 128))), cuda(np.zeros((1, 16))),
                                cuda(np.zeros((1, 10, 128))), icuda([0]), icuda([0, 1, 1]), 2, 1, 1.0,
                                cuda(np.zeros((4, 128, 128))), torch.empty(2, 16, 128, device="cuda"))
    assert err.value.status == E.E3CONV_ERR_UNSUPPORTED
