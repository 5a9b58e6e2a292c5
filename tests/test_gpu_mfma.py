"""GPU parity of the matrix-core forward of the bf16 layout (through the C ABI).

64x(0e+1o+2e), SH lmax 3 -> 64x(0e+1o+2e+3o), bf16 storage, RECEIVER variants
6 (K and u = s x rounded once to bf16) and 7 (K split into two bf16 parts),
against the fp64 oracle.  Bars: element by element, the rounding bound of the
form (u and K rounded to bf16, relative error at most 2^-8 each, products
exact, sums in fp32): |out - oracle| <= (2^-7 + 1e-3) * B with
B = (1/N) sum over edges and CG terms of |C| |y| |s| |x|; and on graphs of the
workload's degree (about 32) the 2e-2 RMS bar of bf16 storage.  On graphs of
low degree the RMS-relative error of the form exceeds 2e-2 (2.7e-2 at degree
1 to 7, the same number from a numpy model of the rounding), which is why it
is not the default kernel.  The kernel takes
a receiver's edges four at a time and walks every T-th receiver of the
processing order in a persistent grid, so the cases cover every remainder of
a receiver's degree modulo four (0 to 11 edges), more receivers than waves,
both graph orderings of the receivers, and the full 100k-node workload on
sampled rows.  Padding receivers and empty graphs run in the tight-bar test
file with every variant.
"""

import numpy as np
import pytest

from oracle import conv
from oracle.so3 import real_cg
from equivariant_gnn_message_amd import e3conv as E
from equivariant_gnn_message_amd import synth

from ._gpu import device_inputs, edges_of_rows, rel_err, sample_rows, say

pytestmark = pytest.mark.gpu

MATRIX_CORE = (6, 7)
BAR = 2e-2
ROUND = 2.0 ** -7 + 1e-3


def abs_bound(lay, x, y, s, src, dst, N):
    """B[b] = (1/N) sum_{e into b} sum_p sum_(m1,m2,m3) |C| |x_a| |y_e| |s_e| (fp64)."""
    out = np.zeros((N, lay.num_out, lay.channels))
    xa = np.abs(x[src])
    for p, P in enumerate(lay.paths):
        cg = np.abs(real_cg(P.l1, P.l2, P.l3))
        t = np.einsum("ijk,eic,ej->ekc", cg, xa[:, P.o1:P.o1 + 2 * P.l1 + 1],
                      np.abs(y[:, P.o2:P.o2 + 2 * P.l2 + 1]))
        np.add.at(out[:, P.o3:P.o3 + 2 * P.l3 + 1], dst, np.abs(s[:, p, None, :]) * t)
    return out / lay.avg_num_neighbors


def check_bound(got, ref, bound, label):
    excess = np.abs(got - ref) - ROUND * bound
    ratio = float(np.max(np.abs(got - ref) / np.maximum(bound, 1e-30)))
    say(f"  {label}: max |err| / B = {ratio:.3e} (bound {ROUND:.3e})")
    assert np.all(excess <= 0), (label, ratio)


def _w():
    return synth.WORKLOADS[3]


def _plan():
    w = _w()
    return E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)


def _lay():
    w = _w()
    return conv.make_layout(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)


def _bf(a):
    import torch
    bits = synth.bf16_bits(np.asarray(a, np.float32))
    return (torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16),
            synth.bf16_to_f32(bits).reshape(bits.shape).astype(np.float64))


def _i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _graph(degrees, num_senders, seed):
    """Receivers 0..len(degrees)-1 with the given in-degrees, senders uniform."""
    rng = np.random.default_rng(seed)
    dst = np.repeat(np.arange(len(degrees)), degrees)
    src = rng.integers(0, num_senders, len(dst))
    return src, dst


def _run(plan, v, x, y, s, src, row_ptr, order=None):
    import torch
    plan.set_variant(v, 0)
    out = plan.forward(x, y, s, src, row_ptr, order=order)
    torch.cuda.synchronize()
    plan.set_variant(0, 0)
    return out.cpu().numpy()


@pytest.mark.parametrize("use_order", [False, True], ids=["index", "clustered"])
def test_every_degree_remainder(use_order):
    """Receivers with 0..11 edges (every quad remainder, empty rows included)."""
    lay = _lay()
    degrees = np.tile(np.arange(12), 9)
    N = len(degrees)
    src, dst = _graph(degrees, N, 3)
    rng = np.random.default_rng(4)
    x, xd = _bf(rng.standard_normal((N, lay.num_x, 64)))
    y, yd = _bf(synth.spherical_harmonics(3, rng.standard_normal((len(src), 3))))
    s, sd = _bf(rng.standard_normal((len(src), lay.num_paths, 64)))
    ref = conv.forward(lay, xd, yd, sd, src, dst, N)
    bound = abs_bound(lay, xd, yd, sd, src, dst, N)
    row_ptr = E.e3conv_csr_from_receivers(_i32(dst), N)
    order = None
    if use_order:
        order = _i32(E.e3conv_receiver_order(row_ptr.cpu().numpy(), src.astype(np.int32), N, len(src), 64))
    plan = _plan()
    for v in MATRIX_CORE:
        got = _run(plan, v, x, y, s, _i32(src), row_ptr, order)
        say(f"[degrees 0..11, order={use_order}] variant {v}: max|err|/RMS {rel_err(got, ref):.3e}")
        check_bound(got, ref, bound, f"variant {v}")
        assert np.all(got[degrees == 0] == 0)


def test_more_receivers_than_waves():
    """7000 receivers of degree 1..7: each wave of the persistent grid takes several."""
    lay = _lay()
    rng = np.random.default_rng(8)
    degrees = rng.integers(1, 8, 7000)
    N = len(degrees)
    src, dst = _graph(degrees, N, 9)
    x, xd = _bf(rng.standard_normal((N, lay.num_x, 64)))
    y, yd = _bf(synth.spherical_harmonics(3, rng.standard_normal((len(src), 3))))
    s, sd = _bf(rng.standard_normal((len(src), lay.num_paths, 64)))
    ref = conv.forward(lay, xd, yd, sd, src, dst, N)
    bound = abs_bound(lay, xd, yd, sd, src, dst, N)
    row_ptr = E.e3conv_csr_from_receivers(_i32(dst), N)
    plan = _plan()
    for v in MATRIX_CORE:
        got = _run(plan, v, x, y, s, _i32(src), row_ptr)
        say(f"[N={N} E={len(src)}] variant {v}: max|err|/RMS {rel_err(got, ref):.3e}")
        check_bound(got, ref, bound, f"variant {v}")


def test_workload_graph_and_register_form():
    """A 1500-node graph of the workload's recipe: the oracle at the 2e-2 RMS bar and
    the rounding bound, and variant 0 (fp32 arithmetic) within the same distance."""
    inp = synth.make_inputs(3, num_nodes=1500)
    d = device_inputs(inp)
    lay = _lay()
    x, y, s = inp.as_f32("x"), inp.as_f32("y"), inp.as_f32("s")
    ref = conv.forward(lay, x, y, s, inp.senders, inp.receivers, inp.num_nodes)
    bound = abs_bound(lay, x, y, s, inp.senders, inp.receivers, inp.num_nodes)
    plan = _plan()
    reg = _run(plan, 0, d["x"], d["y"], d["s"], d["src"], d["row_ptr"]).astype(np.float64)
    for v in MATRIX_CORE:
        got = _run(plan, v, d["x"], d["y"], d["s"], d["src"], d["row_ptr"])
        err, err0 = rel_err(got, ref), rel_err(got, reg)
        say(f"[N=1500] variant {v}: max|err|/RMS {err:.3e}, against variant 0 {err0:.3e}")
        assert err <= BAR and err0 <= BAR, (v, err, err0)
        assert err >= 1e-3, (v, err)       # the bf16 operands show (no silent fp32 path)
        check_bound(got, ref, bound, f"variant {v}")


def test_full_size_sampled_rows():
    """The 100k-node, 3.2M-edge bf16 workload in the clustered receiver order; about a
    hundred receiver rows against the oracle computed for those rows alone."""
    inp = synth.make_inputs(3)
    d = device_inputs(inp)
    N, Ec = inp.num_nodes, inp.num_edges
    order = _i32(E.e3conv_receiver_order(d["row_ptr"].cpu().numpy(), inp.senders, N, Ec, 64))
    rows = sample_rows(inp, k=96, seed=11)
    e = edges_of_rows(inp, rows)
    lay = _lay()
    x = inp.as_f32("x")
    y = synth.bf16_to_f32(inp.y[e]).reshape(len(e), inp.y.shape[1])
    s = synth.bf16_to_f32(inp.s[e]).reshape((len(e),) + inp.s.shape[1:])
    ref = conv.forward_rows(lay, x, y, s, inp.senders[e], inp.receivers[e], rows)
    plan = _plan()
    for v in MATRIX_CORE:
        got = _run(plan, v, d["x"], d["y"], d["s"], d["src"], d["row_ptr"], order)[rows]
        err = rel_err(got, ref)
        say(f"[full N={N} E={Ec}] variant {v} sampled rows: max|err|/RMS {err:.3e}")
        assert err <= BAR, (v, err)
