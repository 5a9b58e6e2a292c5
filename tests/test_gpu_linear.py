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
