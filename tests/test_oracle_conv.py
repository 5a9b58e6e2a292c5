"""Pins for the oracle convolution (forward and backward), CPU only.

The properties come from the pages: the definition and plain algorithm on the
e3j Convolution page; O(3) equivariance over rotations and inversion, results
independent of the edge order, graphs without edges, repeated indices and
empty inputs for the scatter, isolated nodes, input gradients (e3nn_mlx
gate-points page, verification evidence); explicit edgewise summation and
finite differences (cuEquivariance skill page, examples).  Hand-worked values
are in tests/golden/worked_convolution.json.
"""

import math

import numpy as np
import pytest

from oracle import conv, so3
from equivariant_gnn_message_amd import synth

from ._util import eval_array, load_golden, random_rotation, rel_max_err


def small_case(idx, seed=0, num_nodes=12, num_edges=40, channels=None):
    """A small random graph with the layout of workload ``idx`` (fp64 operands)."""
    w = synth.WORKLOADS[idx]
    C = channels or min(w.channels, 4)
    irin = w.irreps_in.replace(f"{w.channels}x", f"{C}x")
    irout = w.irreps_out.replace(f"{w.channels}x", f"{C}x")
    lay = conv.make_layout(irin, w.lmax, irout, w.avg_num_neighbors)
    rng = np.random.default_rng(seed)
    src = rng.integers(0, num_nodes, num_edges)
    dst = rng.integers(0, num_nodes, num_edges)
    x = rng.standard_normal((num_nodes, lay.num_x, C))
    vec = rng.standard_normal((num_edges, 3))
    y = synth.spherical_harmonics(w.lmax, vec)
    s = rng.standard_normal((num_edges, lay.num_paths, C))
    g = rng.standard_normal((num_nodes, lay.num_out, C))
    return lay, x, y, s, g, src, dst, num_nodes, vec


# ------------------------------------------------------------------ layout ---

@pytest.mark.parametrize("idx", range(5))
def test_path_counts_match_workload_table(idx):
    w = synth.WORKLOADS[idx]
    lay = conv.make_layout(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    assert lay.num_paths == w.num_paths
    assert (lay.channels, lay.num_x, lay.num_out) == (w.channels, w.num_x, w.num_out)
    assert lay.num_y == (w.lmax + 1) ** 2


def test_path_order_workload2():
    lay = conv.make_layout("1x0e+1x1o", 3, "1x0e+1x1o+1x2e+1x3o")
    got = [(p.l1, p.l2, p.l3) for p in lay.paths]
    assert got == [(0, 0, 0), (0, 1, 1), (0, 2, 2), (0, 3, 3), (1, 0, 1), (1, 1, 0),
                   (1, 1, 2), (1, 2, 1), (1, 2, 3), (1, 3, 2)]


def test_bad_layouts_rejected():
    with pytest.raises(ValueError):
        conv.make_layout("8x0e+4x1o", 2, "8x0e")
    with pytest.raises(ValueError):
        conv.make_layout("8x0e+8x0e", 2, "8x0e")
    with pytest.raises(ValueError):
        conv.make_layout("8x0e", 1, "8x1e")       # no path reaches 1e
    with pytest.raises(ValueError):
        conv.make_layout("8x0e", -1, "8x0e")


def test_irreps_sugar():
    from oracle import irreps
    assert irreps.parse("64x(0e+1o+2e)") == [(64, 0, 1), (64, 1, -1), (64, 2, 1)]
    assert irreps.parse("0e + 2x1o") == [(1, 0, 1), (2, 1, -1)]
    with pytest.raises(ValueError):
        irreps.parse("8x1q")


# ----------------------------------------------------------------- forward ---

def test_golden_worked_examples():
    gold = load_golden("worked_convolution.json")
    for case in gold["cases"]:
        lay = conv.make_layout(case["irreps_in"], case["lmax"], case["irreps_out"],
                               eval_array(case["avg_num_neighbors"]))
        assert lay.num_paths == len(case["paths"])
        x = eval_array(case["x"])[:, :, None]
        y = eval_array(case["y"])
        s = eval_array(case["s"])[:, :, None]
        want = eval_array(case["out"])[:, :, None]
        for fn in (conv.forward, conv.forward_bruteforce):
            got = fn(lay, x, y, s, np.array(case["senders"]), np.array(case["receivers"]),
                     case["num_nodes"])
            np.testing.assert_allclose(got, want, atol=1e-13, err_msg=case["name"])


@pytest.mark.parametrize("idx", range(4))
def test_bruteforce_equals_vectorised(idx):
    lay, x, y, s, g, src, dst, N, _ = small_case(idx, seed=idx)
    a = conv.forward_bruteforce(lay, x, y, s, src, dst, N)
    b = conv.forward(lay, x, y, s, src, dst, N, chunk=7)
    np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-12)
    rows = [0, 3, N - 1]
    np.testing.assert_allclose(conv.forward_rows(lay, x, y, s, src, dst, rows), a[rows],
                               rtol=1e-12, atol=1e-12)


def test_one_hot_paths_are_textbook_products():
    """With s one-hot on a path the result is a textbook product of x and y."""
    lay = conv.make_layout("1x0e+1x1o", 2, "1x0e+1x1o+1x2e")
    rng = np.random.default_rng(7)
    x = rng.standard_normal((1, 4, 1))
    y = rng.standard_normal((1, 9))
    names = [(p.l1, p.l2, p.l3) for p in lay.paths]
    for p, (l1, l2, l3) in enumerate(names):
        s = np.zeros((1, lay.num_paths, 1))
        s[0, p, 0] = 1.0
        out = conv.forward(lay, x, y, s, np.array([0]), np.array([0]), 1)[0, :, 0]
        P = lay.paths[p]
        got = out[P.o3:P.o3 + 2 * l3 + 1]
        xv = x[0, P.o1:P.o1 + 2 * l1 + 1, 0]
        yv = y[0, P.o2:P.o2 + 2 * l2 + 1]
        if l1 == 0:
            np.testing.assert_allclose(got, xv[0] * yv, atol=1e-14)
        elif l2 == 0:
            np.testing.assert_allclose(got, yv[0] * xv, atol=1e-14)
        elif (l1, l2, l3) == (1, 1, 0):
            np.testing.assert_allclose(got, [np.dot(xv, yv) / math.sqrt(3)], atol=1e-14)
        # every other output block of this path is exactly zero
        mask = np.ones(lay.num_out, bool)
        mask[P.o3:P.o3 + 2 * l3 + 1] = False
        assert not out[mask].any()


def test_cross_product_path():
    lay = conv.make_layout("1x1o", 1, "1x1e")
    rng = np.random.default_rng(8)
    v = rng.standard_normal(3)    # (x, y, z)
    u = rng.standard_normal(3)
    perm = [1, 2, 0]               # (x,y,z) -> (y,z,x)
    x = v[perm][None, :, None]
    y = np.concatenate([[0.3], u[perm]])[None, :]
    s = np.ones((1, 1, 1))
    out = conv.forward(lay, x, y, s, np.array([0]), np.array([0]), 1)[0, :, 0]
    np.testing.assert_allclose(out, np.cross(v, u)[perm] / math.sqrt(2), atol=1e-14)


@pytest.mark.parametrize("idx", range(4))
@pytest.mark.parametrize("improper", [False, True])
def test_equivariance(idx, improper):
    """out(D_x x, D_y y, s) = D_out out(x, y, s) for rotations and inversion."""
    lay, x, y, s, g, src, dst, N, _ = small_case(idx, seed=10 + idx)
    rng = np.random.default_rng(20 + idx)
    axis, ang = random_rotation(rng)
    xb = [(1, l, p) for (l, p) in lay.x_blocks]
    ob = [(1, l, p) for (l, p) in lay.out_blocks]
    yb = [(1, l, (-1) ** l) for l in range(lay.lmax + 1)]
    Dx = so3.block_D(xb, axis, ang, improper)
    Dy = so3.block_D(yb, axis, ang, improper)
    Do = so3.block_D(ob, axis, ang, improper)
    out = conv.forward(lay, x, y, s, src, dst, N)
    out_rot = conv.forward(lay, np.einsum("ij,njc->nic", Dx, x), y @ Dy.T, s, src, dst, N)
    err = rel_max_err(out_rot, np.einsum("ij,njc->nic", Do, out))
    assert err < 1e-12


def test_equivariance_with_rotated_positions():
    """Rotating the edge vectors (then taking harmonics) rotates the output."""
    lay, x, y, s, g, src, dst, N, vec = small_case(2, seed=31)
    rng = np.random.default_rng(32)
    axis, ang = random_rotation(rng)
    R = so3.rotation_matrix(axis, ang)
    y2 = synth.spherical_harmonics(lay.lmax, vec @ R.T)
    xb = [(1, l, p) for (l, p) in lay.x_blocks]
    ob = [(1, l, p) for (l, p) in lay.out_blocks]
    Dx = so3.block_D(xb, axis, ang)
    Do = so3.block_D(ob, axis, ang)
    out = conv.forward(lay, x, y, s, src, dst, N)
    out2 = conv.forward(lay, np.einsum("ij,njc->nic", Dx, x), y2, s, src, dst, N)
    assert rel_max_err(out2, np.einsum("ij,njc->nic", Do, out)) < 1e-12


def test_edge_order_invariance():
    lay, x, y, s, g, src, dst, N, _ = small_case(3, seed=40)
    perm = np.random.default_rng(41).permutation(len(src))
    a = conv.forward(lay, x, y, s, src, dst, N)
    b = conv.forward(lay, x, y[perm], s[perm], src[perm], dst[perm], N)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_zero_edges_and_isolated_nodes():
    lay, x, y, s, g, src, dst, N, _ = small_case(2, seed=50)
    out = conv.forward(lay, x, y[:0], s[:0], src[:0], dst[:0], N)
    assert out.shape == (N, lay.num_out, lay.channels) and not out.any()
    keep = dst != 5
    out = conv.forward(lay, x, y[keep], s[keep], src[keep], dst[keep], N)
    assert not out[5].any()
    assert out.any()


def test_repeated_edges_sum():
    lay, x, y, s, g, src, dst, N, _ = small_case(1, seed=60)
    rep = np.concatenate([np.arange(len(src)), [3, 3, 7]])
    a = conv.forward(lay, x, y[rep], s[rep], src[rep], dst[rep], N)
    s2 = s.copy()
    s2[3] *= 3.0
    s2[7] *= 2.0
    b = conv.forward(lay, x, y, s2, src, dst, N)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_linearity_and_scaling():
    lay, x, y, s, g, src, dst, N, _ = small_case(2, seed=70)
    rng = np.random.default_rng(71)
    f = lambda x_, y_, s_: conv.forward(lay, x_, y_, s_, src, dst, N)
    base = f(x, y, s)
    x2, y2, s2 = rng.standard_normal(x.shape), rng.standard_normal(y.shape), rng.standard_normal(s.shape)
    np.testing.assert_allclose(f(2 * x + x2, y, s), 2 * base + f(x2, y, s), atol=1e-12)
    np.testing.assert_allclose(f(x, -3 * y + y2, s), -3 * base + f(x, y2, s), atol=1e-12)
    np.testing.assert_allclose(f(x, y, 0.5 * s + s2), 0.5 * base + f(x, y, s2), atol=1e-12)
    lay4 = conv.make_layout("4x0e+4x1o", 3, "4x0e+4x1o+4x2e+4x3o", 4 * lay.avg_num_neighbors)
    np.testing.assert_allclose(conv.forward(lay4, x, y, s, src, dst, N), base / 4, atol=1e-13)


def test_channels_are_independent():
    """Channelwise product: channel c of the output only sees channel c of x and s."""
    lay, x, y, s, g, src, dst, N, _ = small_case(2, seed=80)
    out = conv.forward(lay, x, y, s, src, dst, N)
    x2, s2 = x.copy(), s.copy()
    x2[:, :, 1] += 5.0
    s2[:, :, 1] -= 2.0
    out2 = conv.forward(lay, x2, y, s2, src, dst, N)
    keep = [c for c in range(lay.channels) if c != 1]
    np.testing.assert_array_equal(out[:, :, keep], out2[:, :, keep])


# ---------------------------------------------------------------- backward ---

@pytest.mark.parametrize("idx", range(4))
def test_backward_bruteforce_equals_vectorised(idx):
    lay, x, y, s, g, src, dst, N, _ = small_case(idx, seed=90 + idx, num_edges=25)
    a = conv.backward_bruteforce(lay, x, y, s, g, src, dst, N)
    b = conv.backward(lay, x, y, s, g, src, dst, N, chunk=6)
    for u, v in zip(a, b):
        np.testing.assert_allclose(v, u, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("idx", range(4))
def test_backward_trilinear_identity(idx):
    """out is linear in each operand, so <g,out> = <dx,x> = <dy,y> = <ds,s>."""
    lay, x, y, s, g, src, dst, N, _ = small_case(idx, seed=100 + idx)
    L = float(np.sum(g * conv.forward(lay, x, y, s, src, dst, N)))
    dx, dy, ds = conv.backward(lay, x, y, s, g, src, dst, N)
    for val in (np.sum(dx * x), np.sum(dy * y), np.sum(ds * s)):
        assert abs(val - L) <= 1e-11 * max(1.0, abs(L))


def test_backward_finite_differences_subgraph():
    """Central differences on the 16-node subgraph of the training workload.

    L is linear in each operand, so a difference quotient with any step is
    exact up to rounding; step 1 is used.  The product is channelwise, so the
    first 16 channels form a complete sub-problem of the same layout.
    """
    inp = synth.make_inputs(4, num_nodes=3000)
    nodes, eids, src, dst = synth.subgraph16(inp)
    w = inp.workload
    C = 16
    lay = conv.make_layout(w.irreps_in.replace("128x", f"{C}x"), w.lmax,
                           w.irreps_out.replace("128x", f"{C}x"), w.avg_num_neighbors)
    x = inp.x[nodes][:, :, :C].astype(np.float64)
    y = inp.y[eids].astype(np.float64)
    s = inp.s[eids][:, :, :C].astype(np.float64)
    g = inp.g[nodes][:, :, :C].astype(np.float64)
    N = len(nodes)
    assert N == 16 and len(eids) > 16
    Lf = lambda x_, y_, s_: float(np.sum(g * conv.forward(lay, x_, y_, s_, src, dst, N)))
    dx, dy, ds = conv.backward(lay, x, y, s, g, src, dst, N)
    rng = np.random.default_rng(110)

    def check(which, idx):
        args_p, args_m = [x, y, s], [x, y, s]
        d = np.zeros_like(args_p[which])
        d[idx] = 1.0
        args_p[which] = args_p[which] + d
        args_m[which] = args_m[which] - d
        fd = (Lf(*args_p) - Lf(*args_m)) / 2
        grad = (dx, dy, ds)[which]
        assert abs(fd - grad[idx]) <= 1e-10 * max(1.0, abs(grad).max()), (which, idx)

    for i in range(16):                      # every coordinate of y on 16 edges
        for j in range(y.shape[1]):
            check(1, (i, j))
    for _ in range(64):
        check(0, tuple(int(rng.integers(0, n)) for n in x.shape))
        check(2, tuple(int(rng.integers(0, n)) for n in s.shape))
    for _ in range(8):                       # random directions
        for (arr, grad, which) in ((x, dx, 0), (y, dy, 1), (s, ds, 2)):
            d = rng.standard_normal(arr.shape)
            args_p, args_m = [x, y, s], [x, y, s]
            args_p[which] = arr + d
            args_m[which] = arr - d
            fd = (Lf(*args_p) - Lf(*args_m)) / 2
            assert abs(fd - np.sum(grad * d)) <= 1e-10 * max(1.0, abs(fd))


def test_backward_gradient_equivariance():
    """dx rotates like x, dy like y, ds is invariant (g rotated like out)."""
    lay, x, y, s, g, src, dst, N, _ = small_case(2, seed=120)
    rng = np.random.default_rng(121)
    for improper in (False, True):
        axis, ang = random_rotation(rng)
        Dx = so3.block_D([(1, l, p) for (l, p) in lay.x_blocks], axis, ang, improper)
        Dy = so3.block_D([(1, l, (-1) ** l) for l in range(lay.lmax + 1)], axis, ang, improper)
        Do = so3.block_D([(1, l, p) for (l, p) in lay.out_blocks], axis, ang, improper)
        rot = lambda D, a: np.einsum("ij,njc->nic", D, a)
        dx, dy, ds = conv.backward(lay, x, y, s, g, src, dst, N)
        dx2, dy2, ds2 = conv.backward(lay, rot(Dx, x), y @ Dy.T, s, rot(Do, g), src, dst, N)
        assert rel_max_err(dx2, rot(Dx, dx)) < 1e-12
        assert rel_max_err(dy2, dy @ Dy.T) < 1e-12
        assert rel_max_err(ds2, ds) < 1e-12


def test_backward_zero_edges():
    lay, x, y, s, g, src, dst, N, _ = small_case(2, seed=130)
    dx, dy, ds = conv.backward(lay, x, y[:0], s[:0], g, src[:0], dst[:0], N)
    assert dx.shape == x.shape and not dx.any()
    assert dy.shape == (0, lay.num_y) and ds.shape == (0, lay.num_paths, lay.channels)
