"""GPU parity of the fused forward kernels against the CPU oracle (through the C ABI).

Bar: max|gpu - oracle| <= 1e-5 RMS(oracle) for fp32 inputs, 2e-2 RMS for bf16
storage with fp32 accumulation; bit-exact for the integer CSR.
"""

import numpy as np
import pytest

from oracle import conv, so3
from equivariant_gnn_message_amd import e3conv as E
from equivariant_gnn_message_amd import synth

from ._gpu import (device_inputs, edges_of_rows, oracle_inputs, plan_for, rel_err, sample_rows, say,
                   tolerance)

pytestmark = pytest.mark.gpu

# workload, scaled size (None = full size); scaled graphs span hundreds of
# waves and end in a ragged tail (N not a multiple of the receivers per block)
SMALL = [(0, None), (1, None), (2, 601), (3, 601)]


def make(idx, n):
    if n is None:
        return synth.make_inputs(idx)
    return synth.make_inputs(idx, num_nodes=n)


def oracle_layout(inp):
    w = inp.workload
    return conv.make_layout(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)


@pytest.fixture(scope="module", params=SMALL, ids=lambda p: f"w{p[0]}-n{p[1]}")
def small(request):
    idx, n = request.param
    inp = make(idx, n)
    say(f"[setup] workload {idx} N={inp.num_nodes} E={inp.num_edges} dtype={inp.workload.dtype}")
    x, y, s = oracle_inputs(inp)
    ref = conv.forward(oracle_layout(inp), x, y, s, inp.senders, inp.receivers, inp.num_nodes)
    return inp, device_inputs(inp), ref


def test_csr_bit_exact(small):
    inp, d, _ = small
    want = np.searchsorted(inp.receivers, np.arange(inp.num_nodes + 1)).astype(np.int32)
    np.testing.assert_array_equal(d["row_ptr"].cpu().numpy(), want)
    E.e3conv_validate_graph(d["src"], d["row_ptr"], inp.num_nodes, inp.num_edges)


def test_forward_parity_all_variants(small):
    import torch
    inp, d, ref = small
    plan = plan_for(inp)
    dt = E.E3CONV_BF16 if inp.workload.dtype == "bf16" else E.E3CONV_F32
    nf, _ = plan.num_variants(dt)
    for v in range(nf):
        plan.set_variant(v, 0)
        say(f"[forward] workload {inp.workload.idx} N={inp.num_nodes} variant {v}")
        out = plan.forward(d["x"], d["y"], d["s"], d["src"], d["row_ptr"])
        torch.cuda.synchronize()
        err = rel_err(out.cpu().numpy(), ref)
        say(f"  max|err|/RMS = {err:.3e}")
        assert err <= tolerance(inp), (v, err)


def test_forward_f32_kernels_on_decoded_bf16_inputs():
    """The bf16 layout's fp32 kernels, fed the decoded values, meet the fp32 bar."""
    import torch
    inp = make(3, 301)
    x, y, s = oracle_inputs(inp)
    ref = conv.forward(oracle_layout(inp), x, y, s, inp.senders, inp.receivers, inp.num_nodes)
    d = device_inputs(inp)
    xf, yf, sf = (torch.from_numpy(a).cuda() for a in (x, y, s))
    plan = plan_for(inp)
    nf, _ = plan.num_variants(E.E3CONV_F32)
    for v in range(nf):
        plan.set_variant(v, 0)
        say(f"[forward f32 on layout 3] variant {v}")
        out = plan.forward(xf, yf, sf, d["src"], d["row_ptr"])
        torch.cuda.synchronize()
        assert rel_err(out.cpu().numpy(), ref) <= 1e-5


def test_forward_bf16_kernels_on_fp32_layouts():
    """bf16 storage on the fp32 layouts (oracle on the rounded values), 2e-2 bar."""
    import torch
    for idx, n in ((0, None), (1, None), (2, 301)):
        inp = make(idx, n)
        xb, yb, sb = (synth.bf16_bits(a) for a in (inp.x, inp.y, inp.s))
        x, y, s = (synth.bf16_to_f32(a).reshape(a.shape) for a in (xb, yb, sb))
        ref = conv.forward(oracle_layout(inp), x, y, s, inp.senders, inp.receivers, inp.num_nodes)
        d = device_inputs(inp)
        to_bf = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        plan = plan_for(inp)
        nf, _ = plan.num_variants(E.E3CONV_BF16)
        for v in range(nf):
            plan.set_variant(v, 0)
            say(f"[forward bf16 on layout {idx}] variant {v}")
            out = plan.forward(to_bf(xb), to_bf(yb), to_bf(sb), d["src"], d["row_ptr"])
            torch.cuda.synchronize()
            assert rel_err(out.cpu().numpy(), ref) <= 2e-2


def test_forward_deterministic(small):
    import torch
    inp, d, _ = small
    plan = plan_for(inp)
    a = plan.forward(d["x"], d["y"], d["s"], d["src"], d["row_ptr"])
    b = plan.forward(d["x"], d["y"], d["s"], d["src"], d["row_ptr"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_forward_receiver_order_bitwise(small):
    """Processing receivers in another order changes nothing, bit for bit."""
    import torch
    inp, d, _ = small
    plan = plan_for(inp)
    dt = E.E3CONV_BF16 if inp.workload.dtype == "bf16" else E.E3CONV_F32
    order = E.e3conv_receiver_order(d["row_ptr"].cpu().numpy(), inp.senders, inp.num_nodes,
                                    inp.num_edges, 64)
    perm = torch.from_numpy(order).cuda()
    rev = torch.flip(torch.arange(inp.num_nodes, dtype=torch.int32, device="cuda"), [0])
    nf, _ = plan.num_variants(dt)
    for v in range(nf):
        plan.set_variant(v, 0)
        a = plan.forward(d["x"], d["y"], d["s"], d["src"], d["row_ptr"])
        b = plan.forward(d["x"], d["y"], d["s"], d["src"], d["row_ptr"], order=perm)
        c = plan.forward(d["x"], d["y"], d["s"], d["src"], d["row_ptr"], order=rev.contiguous())
        torch.cuda.synchronize()
        assert torch.equal(a, b) and torch.equal(a, c), v


def test_forward_on_side_stream(small):
    import torch
    inp, d, _ = small
    plan = plan_for(inp)
    ref = plan.forward(d["x"], d["y"], d["s"], d["src"], d["row_ptr"])
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        out = plan.forward(d["x"], d["y"], d["s"], d["src"], d["row_ptr"])
    st.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(ref, out)


def test_forward_equivariance_on_gpu():
    """GPU out(D x, D y) equals D GPU out(x, y) for a rotation and an inversion."""
    import torch
    inp = make(2, 301)
    d = device_inputs(inp)
    lay = oracle_layout(inp)
    plan = plan_for(inp)
    out = plan.forward(d["x"], d["y"], d["s"], d["src"], d["row_ptr"]).double().cpu().numpy()
    rng = np.random.default_rng(3)
    for improper in (False, True):
        axis = rng.standard_normal(3)
        ang = float(rng.uniform(0.2, 3.0))
        Dx = so3.block_D([(1, l, p) for (l, p) in lay.x_blocks], axis, ang, improper)
        Dy = so3.block_D([(1, l, (-1) ** l) for l in range(lay.lmax + 1)], axis, ang, improper)
        Do = so3.block_D([(1, l, p) for (l, p) in lay.out_blocks], axis, ang, improper)
        xr = np.einsum("ij,njc->nic", Dx, inp.x.astype(np.float64)).astype(np.float32)
        yr = (inp.y.astype(np.float64) @ Dy.T).astype(np.float32)
        out_r = plan.forward(torch.from_numpy(xr).cuda(), torch.from_numpy(yr).cuda(), d["s"],
                             d["src"], d["row_ptr"]).double().cpu().numpy()
        assert rel_err(out_r, np.einsum("ij,njc->nic", Do, out)) <= 1e-5


def test_forward_edge_order_within_receivers():
    import torch
    inp = make(3, 301)
    d = device_inputs(inp)
    plan = plan_for(inp)
    base = plan.forward(d["x"], d["y"], d["s"], d["src"], d["row_ptr"]).double().cpu().numpy()
    rng = np.random.default_rng(5)
    key = inp.receivers.astype(np.float64) + rng.uniform(0, 0.5, inp.num_edges)
    perm = np.argsort(key, kind="stable")          # shuffles edges inside each receiver segment
    assert np.all(np.diff(inp.receivers[perm]) >= 0) and not np.array_equal(perm, np.arange(len(perm)))
    p = torch.from_numpy(perm).cuda()
    out = plan.forward(d["x"], d["y"][p].contiguous(), d["s"][p].contiguous(), d["src"][p].contiguous(),
                       d["row_ptr"]).double().cpu().numpy()
    assert rel_err(out, base) <= 1e-5


def test_forward_zero_edges_and_isolated_receivers():
    import torch
    inp = make(2, 301)
    lay = oracle_layout(inp)
    plan = plan_for(inp)
    # no edges at all
    N = 37
    z = lambda *s: torch.zeros(s, dtype=torch.float32, device="cuda")
    dst = torch.zeros(0, dtype=torch.int32, device="cuda")
    row_ptr = E.e3conv_csr_from_receivers(dst, N)
    assert int(row_ptr.abs().sum()) == 0
    out = torch.full((N, lay.num_out, lay.channels), 7.0, device="cuda")
    plan.forward(z(N, lay.num_x, lay.channels), z(0, lay.num_y), z(0, lay.num_paths, lay.channels),
                 dst, row_ptr, out=out)
    torch.cuda.synchronize()
    assert float(out.abs().max()) == 0.0
    # drop the edges of a few receivers, incl. the first and the last
    drop = {0, 5, 6, 7, inp.num_nodes - 1}
    keep = np.array([r not in drop for r in inp.receivers])
    src, dst_np = inp.senders[keep], inp.receivers[keep]
    x, y, s = oracle_inputs(inp)
    ref = conv.forward(lay, x, y[keep], s[keep], src, dst_np, inp.num_nodes)
    dd = torch.from_numpy(dst_np).cuda()
    out = plan.forward(torch.from_numpy(x).cuda(), torch.from_numpy(y[keep]).cuda(),
                       torch.from_numpy(s[keep]).cuda(), torch.from_numpy(src).cuda(), E.e3conv_csr_from_receivers(dd, inp.num_nodes))
    got = out.cpu().numpy()
    for b in drop:
        assert not got[b].any()
    assert rel_err(got, ref) <= 1e-5


def test_forward_single_node_self_loops():
    import torch
    inp = make(0, None)
    lay = oracle_layout(inp)
    plan = plan_for(inp)
    rng = np.random.default_rng(9)
    E_ = 5
    x = rng.standard_normal((1, lay.num_x, lay.channels)).astype(np.float32)
    y = synth.spherical_harmonics(lay.lmax, rng.standard_normal((E_, 3))).astype(np.float32)
    s = rng.standard_normal((E_, lay.num_paths, lay.channels)).astype(np.float32)
    src = np.zeros(E_, np.int32)
    ref = conv.forward(lay, x, y, s, src, src, 1)
    t = lambda a: torch.from_numpy(a).cuda()
    out = plan.forward(t(x), t(y), t(s), t(src), E.e3conv_csr_from_receivers(t(src), 1))
    assert rel_err(out.cpu().numpy(), ref) <= 1e-5


@pytest.mark.parametrize("idx", [2, 3])
def test_forward_full_size_sampled_rows(idx):
    """Full-size graph in the benchmark's launch configuration; oracle on sampled receivers."""
    import torch
    inp = synth.make_inputs(idx)
    say(f"[full size] workload {idx} N={inp.num_nodes} E={inp.num_edges}")
    d = device_inputs(inp)
    plan = plan_for(inp)
    out = plan.forward(d["x"], d["y"], d["s"], d["src"], d["row_ptr"])
    torch.cuda.synchronize()
    rows = sample_rows(inp)
    eids = edges_of_rows(inp, rows)
    x = inp.as_f32("x")
    y = synth.bf16_to_f32(inp.y[eids]).reshape(-1, inp.y.shape[1]) if inp.y.dtype == np.uint16 else inp.y[eids]
    s = synth.bf16_to_f32(inp.s[eids]).reshape((-1,) + inp.s.shape[1:]) if inp.s.dtype == np.uint16 else inp.s[eids]
    ref = conv.forward_rows(oracle_layout(inp), x, y, s, inp.senders[eids], inp.receivers[eids], rows)
    got = out[torch.from_numpy(rows).cuda()].cpu().numpy()
    err = rel_err(got, ref)
    say(f"  sampled rows {len(rows)} max|err|/RMS = {err:.3e}")
    assert err <= tolerance(inp)
    # every row of the output is finite and rows of receivers without edges are zero
    assert bool(torch.isfinite(out).all())
    deg = np.diff(np.searchsorted(inp.receivers, np.arange(inp.num_nodes + 1)))
    if (deg == 0).any():
        assert float(out[torch.from_numpy(np.flatnonzero(deg == 0)).cuda()].abs().max()) == 0.0


@pytest.mark.parametrize("idx", [2, 3])
def test_forward_on_relabeled_graph(idx):
    """e3conv_relabel_nodes: the forward of the relabeled graph, as index order, is the
    relabeled forward of the graph as generated (up to the order of the fp32 sums within a
    receiver), and matches the oracle of the relabeled graph."""
    import torch
    inp = make(idx, 1500)
    N, Ec = inp.num_nodes, inp.num_edges
    row_ptr_h = np.searchsorted(inp.receivers, np.arange(N + 1)).astype(np.int32)
    node_new, perm = E.e3conv_relabel_nodes(row_ptr_h, inp.senders, N, Ec, 512)
    d = device_inputs(inp)
    plan = plan_for(inp)
    out = plan.forward(d["x"], d["y"], d["s"], d["src"], d["row_ptr"]).cpu().numpy()
    x2 = torch.empty_like(d["x"])
    x2[torch.from_numpy(node_new.astype(np.int64)).cuda()] = d["x"]
    p = torch.from_numpy(perm.astype(np.int64)).cuda()
    src2 = torch.from_numpy(node_new[inp.senders[perm]].astype(np.int32)).cuda()
    dst2 = torch.from_numpy(node_new[inp.receivers[perm]].astype(np.int32)).cuda()
    rp2 = E.e3conv_csr_from_receivers(dst2, N)
    out2 = plan.forward(x2, d["y"][p].contiguous(), d["s"][p].contiguous(), src2, rp2).cpu().numpy()
    torch.cuda.synchronize()
    err = rel_err(out2[node_new], out)
    say(f"[w{idx} relabeled] max|diff|/RMS against the generated ids: {err:.3e}")
    assert err <= 1e-5
    x, y, s = oracle_inputs(inp)
    xo = np.empty_like(x)
    xo[node_new] = x
    ref = conv.forward(oracle_layout(inp), xo, y[perm], s[perm], node_new[inp.senders[perm]],
                       node_new[inp.receivers[perm]], N)
    assert rel_err(out2, ref) <= tolerance(inp)
