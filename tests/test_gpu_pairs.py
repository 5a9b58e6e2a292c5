"""GPU parity of the pair-stored reverse pass (e3conv_backward_pairs).

Each stored edge (a -> b) stands for itself and its reverse (b -> a) with the
odd-l blocks of y negated and the same s (e3j Convolution page, the note on
SENDER ordering).  The library is compared with ``oracle.variants.backward_pairs``
element by element (bar 1e-5 RMS, fp32), on symmetric radius graphs with
distance-based scalars (the gate-points recipe), on the training layout with
symmetric random scalars, on arbitrary stored lists (any order, self loops,
duplicates), at tile edges and ragged tails, and at the full training size on
sampled rows.  The directed reverse pass of the expanded graph is a second,
independent check.
"""

import numpy as np
import pytest

from oracle import conv, variants
from equivariant_gnn_message_amd import e3conv as E
from equivariant_gnn_message_amd import synth

from ._gpu import rel_err, say

pytestmark = pytest.mark.gpu

TOL = 1e-5


def lay_of(w):
    return conv.make_layout(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)


def dev(a, dtype=None):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.float64:
        a = a.astype(np.float32)
    if dtype is not None:
        a = a.astype(dtype)
    return torch.from_numpy(a).cuda()


def plan_of(w):
    return E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)


def run_pairs(w, x, y, s, g, src, dst, N, grads=None):
    """The library's pair-stored reverse pass on host arrays; returns host grads."""
    import torch
    plan = plan_of(w)
    E_ = len(src)
    dx, dy, ds = dev(x), dev(y), dev(s)
    gx = torch.full((N, plan.num_x, plan.channels), 7.0, device="cuda")   # must be overwritten
    gy = torch.empty((E_, plan.num_y), device="cuda")
    gs = torch.empty((E_, plan.num_paths, plan.channels), device="cuda")
    E.e3conv_backward_pairs(plan.handle, dx, dy, ds, dev(src, np.int32), dev(dst, np.int32), N, E_,
                            dev(g), gx, gy, gs)
    torch.cuda.synchronize()
    return gx.cpu().numpy(), gy.cpu().numpy(), gs.cpu().numpy()


def check(got, ref, what):
    for name, a, b in zip(("grad_x", "grad_y", "grad_s"), got, ref):
        err = rel_err(a, b)
        say(f"  {what} {name} max|err|/RMS {err:.3e}")
        assert err <= TOL, (what, name, err)


def symmetric_inputs(idx, **kw):
    """Workload idx (fp32 operands) on a radius graph, cut to pair storage.
    Workload 1's scalars come from edge lengths and are symmetric already;
    the others get one seeded N(0,1) row per pair."""
    inp = synth.make_inputs(idx, with_cotangent=True, **kw)
    w = inp.workload
    x, y, s = inp.as_f32("x"), inp.as_f32("y"), inp.as_f32("s")
    src, dst = inp.senders, inp.receivers
    stored, pair_of = synth.pair_index(src, dst)
    if idx == 1:
        s_pair = s[stored]
        assert np.array_equal(s, s_pair[pair_of])          # symmetric by construction
    else:
        s_pair = synth.normal_f32(w.idx, synth.T_S_PAIR, (len(stored),) + s.shape[1:])
    return inp, x, y, s_pair, stored, pair_of


@pytest.mark.parametrize("idx,kw", [(1, {"num_graphs": 3}), (2, {"num_nodes": 601}),
                                    (3, {"num_nodes": 401})], ids=["w1-gate", "w2-n601", "w3-n401"])
def test_pairs_parity_on_radius_graphs(idx, kw):
    inp, x, y, s_p, stored, _ = symmetric_inputs(idx, **kw)
    w, N = inp.workload, inp.num_nodes
    src, dst, y_p = inp.senders[stored], inp.receivers[stored], y[stored]
    say(f"[pairs] workload {idx} N={N} pairs={len(stored)}")
    ref = variants.backward_pairs(lay_of(w), x, y_p, s_p, inp.g, src, dst, N)
    got = run_pairs(w, x, y_p, s_p, inp.g, src, dst, N)
    check(got, ref, f"w{idx}")


def test_pairs_equal_directed_backward_on_device():
    """grad_x of the pairs equals the directed pass's; grad_s[e] is the sum of
    the two directed rows of its pair (directed y from the geometry of both
    directions, directed s expanded from the pairs)."""
    import torch
    inp, x, y, s_p, stored, pair_of = symmetric_inputs(2, num_nodes=801)
    w, N = inp.workload, inp.num_nodes
    s_dir = s_p[pair_of]
    plan = plan_of(w)
    d_dst = dev(inp.receivers, np.int32)
    row_ptr = E.e3conv_csr_from_receivers(d_dst, N)
    gx_d, gy_d, gs_d = plan.backward(dev(x), dev(y), dev(s_dir), dev(inp.senders, np.int32), row_ptr,
                                     dev(inp.g))
    torch.cuda.synchronize()
    gx_d, gs_d = gx_d.cpu().numpy(), gs_d.cpu().numpy()
    got = run_pairs(w, x, y[stored], s_p, inp.g, inp.senders[stored], inp.receivers[stored], N)
    gs_sum = np.zeros_like(got[2])
    np.add.at(gs_sum, pair_of, gs_d)
    say(f"[pairs vs directed] N={N} pairs={len(stored)}")
    assert rel_err(got[0], gx_d) <= TOL
    assert rel_err(got[2], gs_sum) <= TOL


@pytest.mark.parametrize("idx", [0, 1, 2, 3])
def test_pairs_any_stored_list(idx):
    """Arbitrary stored edges in random order: self loops, duplicate pairs,
    both orientations, nodes without edges."""
    w = synth.WORKLOADS[idx]
    lay = lay_of(w)
    rng = np.random.default_rng(idx + 40)
    N, E_ = 37, 211
    src = rng.integers(0, N - 3, E_)
    dst = rng.integers(0, N - 3, E_)
    src[:3] = dst[:3]                                   # self loops
    src[3:6], dst[3:6] = src[6:9], dst[6:9]             # duplicates
    x = rng.standard_normal((N, lay.num_x, lay.channels)).astype(np.float32)
    y = synth.spherical_harmonics(lay.lmax, rng.standard_normal((E_, 3))).astype(np.float32)
    s = rng.standard_normal((E_, lay.num_paths, lay.channels)).astype(np.float32)
    g = rng.standard_normal((N, lay.num_out, lay.channels)).astype(np.float32)
    say(f"[pairs any list] layout of workload {idx} C={lay.channels} E={E_}")
    ref = variants.backward_pairs(lay, x, y, s, g, src, dst, N)
    check(run_pairs(w, x, y, s, g, src, dst, N), ref, f"list-w{idx}")
    # sorted by dst (runs of one receiver): the same values
    perm = np.argsort(dst, kind="stable")
    got = run_pairs(w, x, y[perm], s[perm], g, src[perm], dst[perm], N)
    check((got[0], got[1], got[2]), (ref[0], ref[1][perm], ref[2][perm]), f"sorted-w{idx}")


@pytest.mark.parametrize("E_", [1, 2, 15, 16, 17, 33, 250])
def test_pairs_tile_edges_and_tails(E_):
    """Stored-edge counts around the tile size (16) on the training layout."""
    w = synth.WORKLOADS[2]
    lay = lay_of(w)
    rng = np.random.default_rng(E_)
    N = 29
    dst = np.sort(rng.integers(0, N, E_))
    src = rng.integers(0, N, E_)
    x = rng.standard_normal((N, lay.num_x, lay.channels)).astype(np.float32)
    y = synth.spherical_harmonics(lay.lmax, rng.standard_normal((E_, 3))).astype(np.float32)
    s = rng.standard_normal((E_, lay.num_paths, lay.channels)).astype(np.float32)
    g = rng.standard_normal((N, lay.num_out, lay.channels)).astype(np.float32)
    say(f"[pairs tail] E={E_}")
    check(run_pairs(w, x, y, s, g, src, dst, N),
          variants.backward_pairs(lay, x, y, s, g, src, dst, N), f"E={E_}")


def test_pairs_without_edges_zero_grad_x():
    w = synth.WORKLOADS[2]
    lay = lay_of(w)
    N = 11
    x = np.ones((N, lay.num_x, lay.channels), np.float32)
    g = np.ones((N, lay.num_out, lay.channels), np.float32)
    gx, gy, gs = run_pairs(w, x, np.zeros((0, lay.num_y), np.float32),
                           np.zeros((0, lay.num_paths, lay.channels), np.float32), g,
                           np.zeros(0, np.int64), np.zeros(0, np.int64), N)
    assert gx.shape == x.shape and np.all(gx == 0.0) and gy.size == 0 and gs.size == 0


def test_pairs_reject_sender_plans_and_null_pointers():
    import torch
    w = synth.WORKLOADS[2]
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors, ordering=E.E3CONV_SENDER)
    lay = lay_of(w)
    N, E_ = 4, 2
    t = lambda *sh: torch.zeros(*sh, device="cuda")
    i = torch.zeros(E_, dtype=torch.int32, device="cuda")
    args = (t(N, lay.num_x, lay.channels), t(E_, lay.num_y), t(E_, lay.num_paths, lay.channels), i, i,
            N, E_, t(N, lay.num_out, lay.channels), t(N, lay.num_x, lay.channels), t(E_, lay.num_y),
            t(E_, lay.num_paths, lay.channels))
    with pytest.raises(E.E3ConvError) as err:
        E.e3conv_backward_pairs(plan.handle, *args)
    assert err.value.status == E.E3CONV_ERR_UNSUPPORTED
    rplan = plan_of(w)
    lib = E.load_library()
    st = lib.e3conv_backward_pairs(rplan.handle, None, None, None, None, None, N, E_, None, None,
                                   None, None, None)
    assert st == E.E3CONV_ERR_INVALID_ARGUMENT


def test_pairs_full_training_size_sampled():
    """The training graph at full size (N = 20000, 298061 pairs) in the pair
    layout and launch configuration the benchmark times: sampled grad_s / grad_y rows (each
    depends on its own edge only) and sampled grad_x rows (every stored edge
    touching the node), plus the trilinear identity <g, out> = <grad_s, s>."""
    import torch
    inp = synth.make_inputs(4)
    w, N = inp.workload, inp.num_nodes
    lay = lay_of(w)
    row_ptr = np.searchsorted(inp.receivers, np.arange(N + 1)).astype(np.int32)
    stored, _ = E.e3conv_pair_layout(row_ptr, inp.senders, N, inp.num_edges, 512)
    src, dst = inp.senders[stored], inp.receivers[stored]
    y = inp.y[stored]
    s = synth.normal_f32(w.idx, synth.T_S_PAIR, (len(stored), lay.num_paths, lay.channels))
    say(f"[pairs full size] N={N} pairs={len(stored)}")
    gx, gy, gs = run_pairs(w, inp.x, y, s, inp.g, src, dst, N)
    rng = np.random.default_rng(5)
    eids = np.sort(rng.choice(len(stored), size=384, replace=False))
    _, ry, rs = variants.backward_pairs(lay, inp.x, y[eids], s[eids], inp.g, src[eids], dst[eids], N)
    assert rel_err(gs[eids], rs) <= TOL
    assert rel_err(gy[eids], ry) <= TOL
    nodes = np.sort(rng.choice(N, size=32, replace=False))
    sel = np.flatnonzero(np.isin(src, nodes) | np.isin(dst, nodes))
    rx, _, _ = variants.backward_pairs(lay, inp.x, y[sel], s[sel], inp.g, src[sel], dst[sel], N)
    err = rel_err(gx[nodes], rx[nodes])
    say(f"  sampled grad_x rows max|err|/RMS {err:.3e}")
    assert err <= TOL
    # <g, out> = <grad_s, s> (out trilinear in s), with out = the pair forward
    # computed by the directed forward pass of the expanded graph on the device
    P = variants.parity_sign(lay).astype(np.float32)
    order = np.argsort(np.concatenate([dst, src]), kind="stable")
    a2 = np.concatenate([src, dst])[order]
    b2 = np.concatenate([dst, src])[order]
    y2 = np.concatenate([y, y * P])[order]
    s2 = np.concatenate([s, s])[order]
    plan = plan_of(w)
    d_b2 = dev(b2, np.int32)
    out = plan.forward(dev(inp.x), dev(y2), dev(s2), dev(a2, np.int32), E.e3conv_csr_from_receivers(d_b2, N))
    torch.cuda.synchronize()
    L = float(np.vdot(inp.g.astype(np.float64), out.cpu().numpy().astype(np.float64)))
    val = float(np.vdot(gs.astype(np.float64), s.astype(np.float64)))
    say(f"  <g,out> {L:.6e} vs <grad_s,s> {val:.6e}")
    assert abs(val - L) <= 1e-5 * abs(L)


# ------------------------------------------------------- pair-stored forward -----

def pair_layout(inp):
    """e3conv_pair_layout of a workload's radius graph: stored edges and the signed map."""
    N, Ec = inp.num_nodes, inp.num_edges
    row_ptr = np.searchsorted(inp.receivers, np.arange(N + 1)).astype(np.int32)
    return E.e3conv_pair_layout(row_ptr, inp.senders, N, Ec, 64)


# The directed forward variant with the pair forward's lane layout (on the 128-channel
# layout, one 64-lane group per receiver: variant 2; elsewhere the default), whose
# summation order the pair forward shares, so the two agree bit for bit.
DIRECTED_TWIN = {"mace": 2, "training": 2}


def directed_twin(plan, w):
    plan.set_variant(DIRECTED_TWIN.get(w.name, 0), 0)
    return plan


def run_forward_pairs(w, x, y_p, s_p, inp, pmap, order=None):
    import torch
    plan = plan_of(w)
    N, Ec = inp.num_nodes, inp.num_edges
    d_dst = dev(inp.receivers, np.int32)
    row_ptr = E.e3conv_csr_from_receivers(d_dst, N)
    out = torch.full((N, plan.num_out, plan.channels), 5.0, device="cuda")
    E.e3conv_forward_pairs(plan.handle, dev(x), dev(y_p), dev(s_p), dev(inp.senders, np.int32), row_ptr,
                           dev(pmap, np.int32), N, Ec, len(y_p), out,
                           order=None if order is None else dev(order, np.int32))
    torch.cuda.synchronize()
    return out.cpu().numpy(), plan, row_ptr


@pytest.mark.parametrize("idx,kw", [(1, {"num_graphs": 3}), (2, {"num_nodes": 601}),
                                    (3, {"num_nodes": 401})], ids=["w1-gate", "w2-n601", "w3-n401"])
def test_forward_pairs_parity(idx, kw):
    """Against oracle.variants.forward_pairs, and bitwise against the directed forward of the
    expanded rows (s_pair[k], and y_pair[k] with the odd-l blocks negated for reverses)."""
    import torch
    inp = synth.make_inputs(idx, with_cotangent=True, **kw)
    w = inp.workload
    x, y = inp.as_f32("x"), inp.as_f32("y")
    stored, pmap = pair_layout(inp)
    k = np.where(pmap >= 0, pmap, ~pmap)
    y_p = y[stored]
    if idx == 1:
        s_p = inp.as_f32("s")[stored]
    else:
        s_p = synth.normal_f32(w.idx, synth.T_S_PAIR, (len(stored),) + inp.s.shape[1:])
    N = inp.num_nodes
    say(f"[forward pairs] workload {idx} N={N} pairs={len(stored)}")
    got, plan, row_ptr = run_forward_pairs(w, x, y_p, s_p, inp, pmap)
    ref = variants.forward_pairs(lay_of(w), x, y_p, s_p, inp.senders[stored], inp.receivers[stored], N)
    err = rel_err(got, ref)
    say(f"  max|err|/RMS {err:.3e}")
    assert err <= TOL
    P = variants.parity_sign(lay_of(w)).astype(np.float32)
    y_dir = np.where((pmap >= 0)[:, None], y_p[k], y_p[k] * P)
    dirc = directed_twin(plan, w).forward(dev(x), dev(y_dir), dev(s_p[k]), dev(inp.senders, np.int32),
                                          row_ptr)
    torch.cuda.synchronize()
    assert np.array_equal(got, dirc.cpu().numpy())


def test_forward_pairs_order_and_full_size():
    """The training graph at full size with the receiver order the benchmark uses:
    bitwise equal to the directed forward of the expanded rows, sampled rows against
    the oracle."""
    import torch
    inp = synth.make_inputs(4)
    w, N = inp.workload, inp.num_nodes
    stored, pmap = pair_layout(inp)
    k = np.where(pmap >= 0, pmap, ~pmap)
    y_p = inp.y[stored]
    s_p = synth.normal_f32(w.idx, synth.T_S_PAIR, (len(stored), w.num_paths, w.channels))
    row_ptr_h = np.searchsorted(inp.receivers, np.arange(N + 1)).astype(np.int32)
    order = E.e3conv_receiver_order(row_ptr_h, inp.senders, N, inp.num_edges, 512)
    say(f"[forward pairs full size] N={N} pairs={len(stored)}")
    got, plan, row_ptr = run_forward_pairs(w, inp.x, y_p, s_p, inp, pmap, order=order)
    P = variants.parity_sign(lay_of(w)).astype(np.float32)
    y_dir = np.where((pmap >= 0)[:, None], y_p[k], y_p[k] * P)
    dirc = directed_twin(plan, w).forward(dev(inp.x), dev(y_dir), dev(s_p[k]),
                                          dev(inp.senders, np.int32), row_ptr, order=dev(order, np.int32))
    torch.cuda.synchronize()
    assert np.array_equal(got, dirc.cpu().numpy())
    rows = np.sort(np.random.default_rng(2).choice(N, size=64, replace=False))
    sel = np.flatnonzero(np.isin(inp.receivers[stored], rows) | np.isin(inp.senders[stored], rows))
    ref = variants.forward_pairs(lay_of(w), inp.x, y_p[sel], s_p[sel], inp.senders[stored][sel],
                                 inp.receivers[stored][sel], N)
    err = rel_err(got[rows], ref[rows])
    say(f"  sampled rows max|err|/RMS {err:.3e}")
    assert err <= TOL
