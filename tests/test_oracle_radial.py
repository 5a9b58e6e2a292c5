"""Pins for the radial edge scalars and the convolution they feed (CPU only).

The definitions (gate-points page, radial embedding and fully connected
network; reading R11) fix closed-form values: the cutoff is 1 at r = 0, 1/2
at r_max / 2 and 0 at r_max; each Gaussian is 1 at its center and e^-1 one
sigma away; silu(z) - silu(-z) = z for every z; the network is linear in its
last weight matrix; its vectorised route must agree with pure-Python loops.
Those are the pins.  A further consistency check (not a pin: both sides are
this project's code) compares the oracle's scalars with the ones the input
generator stores for the gate-points workload.
"""

import math

import numpy as np
import pytest

from oracle import conv, radial
from equivariant_gnn_message_amd import synth

from ._util import rel_max_err


def test_cutoff_closed_forms():
    assert radial.cutoff(0.0, 2.0) == 1.0
    assert radial.cutoff(2.0, 2.0) == 0.0
    assert abs(radial.cutoff(1.0, 2.0) - 0.5) < 1e-15


def test_cutoff_vanishes_beyond_the_radius():
    # a cutoff function is zero outside its radius; the cosine alone would rise again
    # (to 1 at 2 r_max), so this pins the clamp
    r = np.array([2.0, 2.5, 3.0, 4.0, 7.3])
    assert np.all(radial.cutoff(r, 2.0) == 0.0)
    assert np.all(radial.basis(r, 5, 2.0, 0.5) == 0.0)
    assert radial.cutoff(1.999, 2.0) > 0.0
    r = np.linspace(0.0, 2.0, 101)
    assert np.all(np.diff(radial.cutoff(r, 2.0)) < 0)


@pytest.mark.parametrize("nb,r_max,sigma", [(5, 2.0, 0.5), (8, 3.0, 0.3)])
def test_gaussians_at_their_centers_and_one_sigma_away(nb, r_max, sigma):
    centers = np.array([k * r_max / (nb - 1) for k in range(nb)])
    f = radial.basis(centers, nb, r_max, sigma)
    cut = radial.cutoff(centers, r_max)
    np.testing.assert_allclose(np.diag(f), cut, rtol=1e-15, atol=0)
    inner = centers[1:-1]
    up = radial.basis(inner + sigma, nb, r_max, sigma)[np.arange(len(inner)), np.arange(1, nb - 1)]
    down = radial.basis(inner - sigma, nb, r_max, sigma)[np.arange(len(inner)), np.arange(1, nb - 1)]
    np.testing.assert_allclose(up, math.exp(-1.0) * radial.cutoff(inner + sigma, r_max), rtol=1e-14)
    np.testing.assert_allclose(down, math.exp(-1.0) * radial.cutoff(inner - sigma, r_max), rtol=1e-14)


def test_silu_identities():
    z = np.linspace(-30.0, 30.0, 241)
    np.testing.assert_allclose(radial.silu(z) - radial.silu(-z), z, rtol=0, atol=1e-13)
    assert radial.silu(0.0) == 0.0
    assert abs(radial.silu(40.0) - 40.0) < 1e-12
    assert abs(radial.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16


def test_network_linear_in_last_layer_and_zero_without_first():
    rng = np.random.default_rng(4)
    f = rng.standard_normal((20, 5))
    w1, w2 = rng.standard_normal((5, 12)), rng.standard_normal((12, 7))
    np.testing.assert_allclose(radial.mlp(f, w1, 3.0 * w2), 3.0 * radial.mlp(f, w1, w2), rtol=1e-13)
    assert np.all(radial.mlp(f, 0.0 * w1, w2) == 0.0)


def gate_layout(C=None):
    w = synth.WORKLOADS[1]
    irin, irout = w.irreps_in, w.irreps_out
    if C is not None:
        irin = irin.replace(f"{w.channels}x", f"{C}x")
        irout = irout.replace(f"{w.channels}x", f"{C}x")
    return conv.make_layout(irin, w.lmax, irout, w.avg_num_neighbors)


def test_scalars_match_the_workload_recipe():
    """Consistency, not a pin: the gate-points workload's stored s (written by the
    input generator's own code) equals the oracle's scalars of the same inputs."""
    inp = synth.make_inputs(1, num_graphs=3)
    r, w1, w2 = synth.radial_inputs(inp)
    w1d, w2d = synth.radial_mlp_weights(w2.shape[1])
    s = radial.scalars(gate_layout(), r.astype(np.float64), w1d, w2d, inp.workload.radius, 0.5)
    assert rel_max_err(s.astype(np.float32), inp.s) < 1e-6


def test_vectorised_equals_bruteforce():
    lay = gate_layout(C=3)
    rng = np.random.default_rng(9)
    n, E = 9, 30
    src, dst = rng.integers(0, n, E), rng.integers(0, n, E)
    x = rng.standard_normal((n, lay.num_x, lay.channels))
    y = synth.spherical_harmonics(lay.lmax, rng.standard_normal((E, 3)))
    r = rng.uniform(0.05, 1.95, E)
    w1 = rng.standard_normal((5, 16)) / math.sqrt(5)
    w2 = rng.standard_normal((16, lay.num_paths * lay.channels)) / 4.0
    got = radial.forward_radial(lay, x, y, r, w1, w2, 2.0, 0.5, src, dst, n)
    ref = radial.forward_radial_bruteforce(lay, x, y, r, w1, w2, 2.0, 0.5, src, dst, n)
    assert rel_max_err(got, ref) < 1e-12
    rows = np.array([0, 3, 8])
    part = radial.forward_radial_rows(lay, x, y, r, w1, w2, 2.0, 0.5, src, dst, rows)
    assert rel_max_err(part, got[rows]) < 1e-12


def test_edges_at_the_cutoff_radius_carry_no_message():
    lay = gate_layout(C=3)
    rng = np.random.default_rng(2)
    n, E = 5, 12
    src, dst = rng.integers(0, n, E), rng.integers(0, n, E)
    x = rng.standard_normal((n, lay.num_x, lay.channels))
    y = synth.spherical_harmonics(lay.lmax, rng.standard_normal((E, 3)))
    w1 = rng.standard_normal((5, 8))
    w2 = rng.standard_normal((8, lay.num_paths * lay.channels))
    out = radial.forward_radial(lay, x, y, np.full(E, 2.0), w1, w2, 2.0, 0.5, src, dst, n)
    assert np.all(out == 0.0)
