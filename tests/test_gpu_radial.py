"""GPU parity of the convolution with in-kernel radial edge scalars (through the C ABI).

``e3conv_forward_radial`` against ``oracle.radial`` on the gate-points layout:
whole outputs on scaled graphs and on hand-built graphs whose receivers take
0, 1, 15, 16, 17 and 40 edges (edge tiles of 16), sampled rows at the full
workload size, padding receivers and a receiver processing order, and the
range limits of the network shape.  Bar: 1e-5 RMS (fp32 operands).
"""

import math

import numpy as np
import pytest

from oracle import conv, radial
from equivariant_gnn_message_amd import e3conv as E
from equivariant_gnn_message_amd import synth

from ._gpu import rel_err, sample_rows, say

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS[1]


def lay():
    return conv.make_layout(W.irreps_in, W.lmax, W.irreps_out, W.avg_num_neighbors)


def plan():
    return E.Plan(W.irreps_in, W.lmax, W.irreps_out, W.avg_num_neighbors)


def dev(a, dtype=None):
    import torch
    a = np.ascontiguousarray(a)
    if dtype is not None:
        a = a.astype(dtype)
    elif a.dtype == np.float64:
        a = a.astype(np.float32)
    return torch.from_numpy(a).cuda()


def run(x, y, r, w1, w2, src, dst, N, sigma=0.5, r_max=2.0, order=None, num_real=None):
    import torch
    row_ptr = E.e3conv_csr_from_receivers(dev(dst, np.int32), N)
    out = torch.full((N, lay().num_out, lay().channels), 5.0, device="cuda")
    plan().forward_radial(dev(x), dev(y), dev(r), dev(w1), dev(w2), dev(src, np.int32), row_ptr, r_max,
                          sigma, out=out, order=None if order is None else dev(order, np.int32),
                          num_real_nodes=num_real)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("graphs", [1, 8])
def test_radial_parity_scaled_graphs(graphs):
    inp = synth.make_inputs(1, num_graphs=graphs)
    r, w1, w2 = synth.radial_inputs(inp)
    N = inp.num_nodes
    say(f"[radial] graphs={graphs} N={N} E={inp.num_edges}")
    ref = radial.forward_radial(lay(), inp.x, inp.y, r, w1, w2, W.radius, 0.5, inp.senders, inp.receivers, N)
    got = run(inp.x, inp.y, r, w1, w2, inp.senders, inp.receivers, N)
    err = rel_err(got, ref)
    say(f"  max|err|/RMS = {err:.3e}")
    assert err <= 1e-5


def handmade(degrees, seed=3, n_extra=5):
    """Receiver-sorted graph whose receivers have the given in-degrees."""
    rng = np.random.default_rng(seed)
    N = len(degrees) + n_extra
    dst = np.repeat(np.arange(len(degrees)), degrees)
    src = rng.integers(0, N, len(dst))
    L = lay()
    x = rng.standard_normal((N, L.num_x, L.channels)).astype(np.float32)
    y = synth.spherical_harmonics(L.lmax, rng.standard_normal((len(dst), 3))).astype(np.float32)
    r = rng.uniform(0.0, 2.0, len(dst)).astype(np.float32)
    return x, y, r, src, dst, N


def test_radial_tile_boundaries():
    degrees = [0, 1, 15, 16, 17, 40, 3, 0, 32, 33]
    x, y, r, src, dst, N = handmade(degrees)
    _, w1, w2 = synth.radial_inputs(synth.make_inputs(1, num_graphs=1))
    ref = radial.forward_radial(lay(), x, y, r, w1, w2, 2.0, 0.5, src, dst, N)
    got = run(x, y, r, w1, w2, src, dst, N)
    err = rel_err(got, ref)
    say(f"[radial tiles] degrees {degrees}: max|err|/RMS = {err:.3e}")
    assert err <= 1e-5
    empty = [b for b in range(N) if b >= len(degrees) or degrees[b] == 0]
    assert np.all(got[empty] == 0.0)


@pytest.mark.parametrize("degrees", [
    [5, 700, 0, 0, 3, 250, 17, 0, 1, 64, 2],   # receivers spread over several waves of a work-group
    [0] * 40 + [3, 0, 0, 9] + [0] * 30,        # receivers without edges around a few tiles
    [1, 2, 1, 0, 3, 1, 1, 2] * 30,             # many one-tile receivers
], ids=["long", "sparse", "short"])
def test_radial_receivers_shared_between_waves(degrees):
    x, y, r, src, dst, N = handmade(degrees, seed=len(degrees))
    _, w1, w2 = synth.radial_inputs(synth.make_inputs(1, num_graphs=1))
    ref = radial.forward_radial(lay(), x, y, r, w1, w2, 2.0, 0.5, src, dst, N)
    got = run(x, y, r, w1, w2, src, dst, N)
    err = rel_err(got, ref)
    say(f"[radial shared] {len(degrees)} receivers, {len(dst)} edges: max|err|/RMS = {err:.3e}")
    assert err <= 1e-5
    empty = [b for b in range(N) if b >= len(degrees) or degrees[b] == 0]
    assert np.all(got[empty] == 0.0)


@pytest.mark.parametrize("use_order", [False, True], ids=["index", "clustered"])
def test_radial_heavy_tailed_degrees(use_order):
    """Degrees 0 .. 600 over 3 000 receivers: work-groups and waves cut inside receivers."""
    rng = np.random.default_rng(21)
    deg = rng.geometric(1 / 12, 3000) - 1
    deg[rng.choice(3000, 12, replace=False)] = rng.integers(100, 600, 12)
    x, y, r, src, dst, N = handmade(list(deg), seed=22, n_extra=0)
    _, w1, w2 = synth.radial_inputs(synth.make_inputs(1, num_graphs=1))
    ref = radial.forward_radial(lay(), x, y, r, w1, w2, 2.0, 0.5, src, dst, N)
    order = None
    if use_order:
        ptr = np.searchsorted(dst, np.arange(N + 1)).astype(np.int32)
        order = E.e3conv_receiver_order(ptr, src.astype(np.int32), N, len(src), 64)
    got = run(x, y, r, w1, w2, src, dst, N, order=order)
    err = rel_err(got, ref)
    # context: the plain forward reading the oracle's scalars rounded to fp32
    import torch
    s = radial.scalars(lay(), r, w1, w2, 2.0, 0.5).astype(np.float32)
    row_ptr = E.e3conv_csr_from_receivers(dev(dst, np.int32), N)
    plain = plan().forward(dev(x), dev(y), dev(s), dev(src, np.int32), row_ptr)
    torch.cuda.synchronize()
    say(f"[radial heavy] order={use_order} E={len(dst)}: max|err|/RMS = {err:.3e} "
        f"(plain forward on fp32 scalars: {rel_err(plain.cpu().numpy(), ref):.3e})")
    assert err <= 1e-5
    assert np.all(got[deg == 0] == 0.0)


@pytest.mark.parametrize("nb,hidden,sigma", [(2, 4, 0.8), (8, 128, 0.3), (5, 36, 0.5)])
def test_radial_network_shapes(nb, hidden, sigma):
    x, y, r, src, dst, N = handmade([5, 20, 0, 16, 9], seed=nb)
    rng = np.random.default_rng(hidden)
    L = lay()
    w1 = (rng.standard_normal((nb, hidden)) / math.sqrt(nb)).astype(np.float32)
    w2 = (rng.standard_normal((hidden, L.num_paths * L.channels)) / math.sqrt(hidden)).astype(np.float32)
    ref = radial.forward_radial(L, x, y, r, w1, w2, 2.0, sigma, src, dst, N)
    got = run(x, y, r, w1, w2, src, dst, N, sigma=sigma)
    err = rel_err(got, ref)
    say(f"[radial shape] nb={nb} hidden={hidden}: max|err|/RMS = {err:.3e}")
    assert err <= 1e-5


def test_radial_edges_beyond_the_cutoff():
    """Edge lengths past r_max carry no message (the cutoff is zero there), also where the
    cosine alone would not vanish (r = 1.5 r_max, 2 r_max)."""
    x, y, r, src, dst, N = handmade([7, 30, 0, 18, 4], seed=21)
    rng = np.random.default_rng(22)
    far = rng.random(len(r)) < 0.4
    r = np.where(far, rng.choice([2.0, 2.5, 3.0, 4.0], size=len(r)), r).astype(np.float32)
    _, w1, w2 = synth.radial_inputs(synth.make_inputs(1, num_graphs=1))
    ref = radial.forward_radial(lay(), x, y, r, w1, w2, 2.0, 0.5, src, dst, N)
    got = run(x, y, r, w1, w2, src, dst, N)
    err = rel_err(got, ref)
    # the same graph without the far edges gives the same result
    near = ~far
    ref_near = radial.forward_radial(lay(), x, y[near], r[near], w1, w2, 2.0, 0.5, src[near], dst[near], N)
    say(f"[radial beyond cutoff] {int(far.sum())} of {len(r)} edges past r_max: {err:.3e}")
    assert err <= 1e-5
    np.testing.assert_allclose(ref, ref_near, rtol=0, atol=1e-12 * max(1.0, float(np.abs(ref).max())))


def test_radial_graph_without_edges():
    """No edges at all: every output row is zero (receivers and padding alike)."""
    import torch
    L = lay()
    N = 37
    rng = np.random.default_rng(4)
    x = rng.standard_normal((N, L.num_x, L.channels)).astype(np.float32)
    _, w1, w2 = synth.radial_inputs(synth.make_inputs(1, num_graphs=1))
    empty_i = np.zeros(0, np.int32)
    y = np.zeros((0, L.num_y), np.float32)
    r = np.zeros(0, np.float32)
    got = run(x, y, r, w1, w2, empty_i, empty_i, N)
    say(f"[radial empty] N={N}: max|out| = {np.abs(got).max():.1e}")
    assert np.all(got == 0.0)


@pytest.mark.parametrize("s1,s2,spread", [(1e-3, 1e5, 0), (30.0, 1e-6, 0), (1.0, 1.0, 6)],
                         ids=["small-w1-large-w2", "large-w1-small-w2", "channel-spread"])
def test_radial_weight_scales(s1, s2, spread):
    """Weights far outside the fp16 range, and channels whose magnitudes differ by up to 1e6:
    the kernel's power-of-two operand scales must keep fp32-level accuracy."""
    x, y, r, src, dst, N = handmade([5, 20, 0, 16, 9, 33], seed=11)
    _, w1, w2 = synth.radial_inputs(synth.make_inputs(1, num_graphs=1))
    L = lay()
    w1 = (w1 * s1).astype(np.float32)
    w2 = (w2 * s2).astype(np.float32)
    if spread:
        # channel c of every path scaled by 10^(-spread c / (C - 1))
        ch = 10.0 ** (-spread * np.arange(L.channels) / (L.channels - 1))
        w2 = (w2.reshape(w2.shape[0], L.num_paths, L.channels) * ch).reshape(w2.shape).astype(np.float32)
    ref = radial.forward_radial(L, x, y, r, w1, w2, 2.0, 0.5, src, dst, N)
    got = run(x, y, r, w1, w2, src, dst, N)
    err = rel_err(got, ref)
    say(f"[radial scales] w1 x{s1:g}, w2 x{s2:g}, spread {spread}: max|err|/RMS = {err:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= 1e-5
    if spread:
        # the smallest channel keeps its own relative accuracy, not just the global one
        c = L.channels - 1
        rms_c = math.sqrt(float(np.mean(ref[..., c] ** 2)))
        err_c = float(np.abs(got[..., c] - ref[..., c]).max()) / rms_c
        say(f"  channel {c}: max|err|/RMS = {err_c:.3e}")
        assert err_c <= 1e-5


@pytest.mark.parametrize("use_order", [False, True], ids=["index", "clustered"])
def test_radial_padding_and_order(use_order):
    inp = synth.make_inputs(1, num_graphs=4)
    r, w1, w2 = synth.radial_inputs(inp)
    n_real = inp.num_nodes
    rng = np.random.default_rng(8)
    n_pad, e_pad = 19, 60
    N = n_real + n_pad
    L = lay()
    src = np.concatenate([inp.senders, rng.integers(n_real, N, e_pad)])
    dst = np.concatenate([inp.receivers, np.sort(rng.integers(n_real, N, e_pad))])
    x = np.concatenate([inp.x, rng.standard_normal((n_pad, L.num_x, L.channels)).astype(np.float32)])
    y = np.concatenate([inp.y, synth.spherical_harmonics(L.lmax, rng.standard_normal((e_pad, 3))).astype(np.float32)])
    rr = np.concatenate([r, rng.uniform(0.0, 2.0, e_pad).astype(np.float32)])
    real = dst < n_real
    ref = radial.forward_radial(L, x[:n_real], y[real], rr[real], w1, w2, 2.0, 0.5, src[real], dst[real], n_real)
    order = None
    if use_order:
        ptr = np.searchsorted(dst, np.arange(N + 1)).astype(np.int32)
        order = E.e3conv_receiver_order(ptr, src.astype(np.int32), N, len(src), 64)
    got = run(x, y, rr, w1, w2, src, dst, N, order=order, num_real=n_real)
    err = rel_err(got[:n_real], ref)
    say(f"[radial padding] order={use_order}: max|err|/RMS = {err:.3e}")
    assert err <= 1e-5
    assert np.all(got[n_real:] == 0.0)


def test_radial_full_size_sampled_rows():
    inp = synth.make_inputs(1)
    r, w1, w2 = synth.radial_inputs(inp)
    say(f"[radial full] N={inp.num_nodes} E={inp.num_edges}")
    got = run(inp.x, inp.y, r, w1, w2, inp.senders, inp.receivers, inp.num_nodes)
    rows = sample_rows(inp, k=200)
    ref = radial.forward_radial_rows(lay(), inp.x, inp.y, r, w1, w2, W.radius, 0.5, inp.senders,
                                     inp.receivers, rows)
    full = radial.forward_radial(lay(), inp.x, inp.y, r, w1, w2, W.radius, 0.5, inp.senders,
                                 inp.receivers, inp.num_nodes)
    rms = math.sqrt(float(np.mean(full ** 2)))
    err = float(np.abs(got[rows] - ref).max()) / rms
    say(f"  sampled {len(rows)} rows: max|err|/RMS = {err:.3e}")
    assert err <= 1e-5
    # the same s through the plain forward: the fused scalars equal the network's
    s = radial.scalars(lay(), r, w1, w2, W.radius, 0.5).astype(np.float32)
    import torch
    row_ptr = E.e3conv_csr_from_receivers(dev(inp.receivers, np.int32), inp.num_nodes)
    plain = plan().forward(dev(inp.x), dev(inp.y), dev(s), dev(inp.senders, np.int32), row_ptr)
    torch.cuda.synchronize()
    assert rel_err(got, plain.cpu().numpy()) <= 1e-5
