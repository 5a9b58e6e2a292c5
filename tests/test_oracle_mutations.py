"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case patches one plausible error into the oracle (a sign, a dropped term,
a reversed index, a parity-violating path, a missing 1/N) and checks that at
least one of the pins used in test_oracle_conv / test_oracle_so3 fails.
"""

import numpy as np
import pytest

import oracle.conv as conv
from oracle import so3
from oracle.conv import Layout, Path

from ._util import eval_array, load_golden, random_rotation, rel_max_err
from .test_oracle_conv import small_case


def golden_ok():
    gold = load_golden("worked_convolution.json")
    for case in gold["cases"]:
        lay = conv.make_layout(case["irreps_in"], case["lmax"], case["irreps_out"],
                               eval_array(case["avg_num_neighbors"]))
        got = conv.forward(lay, eval_array(case["x"])[:, :, None], eval_array(case["y"]),
                           eval_array(case["s"])[:, :, None], np.array(case["senders"]),
                           np.array(case["receivers"]), case["num_nodes"])
        if not np.allclose(got, eval_array(case["out"])[:, :, None], atol=1e-12):
            return False
    return True


def equivariance_ok(lay=None, improper=False, idx=3):
    base_lay, x, y, s, g, src, dst, N, _ = small_case(idx, seed=5)
    lay = lay or base_lay
    if lay.num_paths != s.shape[1]:
        s = np.random.default_rng(6).standard_normal((s.shape[0], lay.num_paths, s.shape[2]))
    axis, ang = random_rotation(np.random.default_rng(7))
    Dx = so3.block_D([(1, l, p) for (l, p) in lay.x_blocks], axis, ang, improper)
    Dy = so3.block_D([(1, l, (-1) ** l) for l in range(lay.lmax + 1)], axis, ang, improper)
    Do = so3.block_D([(1, l, p) for (l, p) in lay.out_blocks], axis, ang, improper)
    out = conv.forward(lay, x, y, s, src, dst, N)
    out2 = conv.forward(lay, np.einsum("ij,njc->nic", Dx, x), y @ Dy.T, s, src, dst, N)
    return rel_max_err(out2, np.einsum("ij,njc->nic", Do, out)) < 1e-10


def trilinear_ok(idx=2):
    lay, x, y, s, g, src, dst, N, _ = small_case(idx, seed=9)
    L = float(np.sum(g * conv.forward(lay, x, y, s, src, dst, N)))
    dx, dy, ds = conv.backward(lay, x, y, s, g, src, dst, N)
    return all(abs(v - L) <= 1e-9 * max(1, abs(L)) for v in (np.sum(dx * x), np.sum(dy * y), np.sum(ds * s)))


def all_pins_ok():
    return (golden_ok() and equivariance_ok() and equivariance_ok(improper=True)
            and trilinear_ok())


def test_unpatched_oracle_passes_the_pins():
    assert all_pins_ok()


def _patched_cg(fn):
    orig = so3.real_cg

    def patched(l1, l2, l3):
        return fn(l1, l2, l3, orig(l1, l2, l3))
    return patched


MUTATIONS = {
    # sign flip of the quadrupole path
    "sign_112": lambda l1, l2, l3, C: -C if (l1, l2, l3) == (1, 1, 2) else C,
    # one CG term dropped
    "drop_term_123": lambda l1, l2, l3, C: (lambda D: (D.__setitem__(tuple(np.argwhere(D)[0]), 0.0), D)[1])(C.copy())
    if (l1, l2, l3) == (1, 2, 3) else C,
    # output index reversed
    "reverse_m3_213": lambda l1, l2, l3, C: C[:, :, ::-1] if (l1, l2, l3) == (2, 1, 3) else C,
    # x and y operands swapped on the antisymmetric (cross-product) path
    "transpose_111": lambda l1, l2, l3, C: C.transpose(1, 0, 2) if (l1, l2, l3) == (1, 1, 1) else C,
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_cg_mistakes_are_caught(monkeypatch, name):
    monkeypatch.setattr(conv, "real_cg", _patched_cg(MUTATIONS[name]))
    results = {"golden": golden_ok(), "rot": equivariance_ok(), "inv": equivariance_ok(improper=True),
               "sign_rule": all(np.flatnonzero(conv.real_cg(*t).reshape(-1)).size == 0
                                or conv.real_cg(*t).reshape(-1)[np.flatnonzero(conv.real_cg(*t).reshape(-1))[0]] > 0
                                for t in [(1, 1, 2), (1, 2, 3), (2, 1, 3), (1, 1, 1)])}
    assert not all(results.values()), results


def test_parity_violating_path_is_caught():
    """Adding 1o x 1 -> 1o (parity-forbidden) breaks inversion equivariance only."""
    lay = conv.make_layout("4x0e+4x1o", 2, "4x0e+4x1o+4x2e", 8.0)
    extra = Path(1, 1, -1, 1, 1, 1, 1, 1, -1, 1)
    bad = Layout(lay.channels, lay.x_blocks, lay.lmax, lay.out_blocks, lay.paths + (extra,),
                 lay.num_x, lay.num_y, lay.num_out, lay.avg_num_neighbors)
    assert equivariance_ok(bad, improper=False, idx=0)
    assert not equivariance_ok(bad, improper=True, idx=0)


def test_missing_average_is_caught(monkeypatch):
    orig = conv.forward

    def no_avg(lay, *a, **k):
        return orig(lay, *a, **k) * lay.avg_num_neighbors
    monkeypatch.setattr(conv, "forward", no_avg)
    assert not golden_ok()
    assert not trilinear_ok()


# ------------------------------------------------------- radial scalars -----

def radial_pins_ok():
    """The closed-form pins of tests/test_oracle_radial.py, as one predicate."""
    from . import test_oracle_radial as T
    try:
        T.test_cutoff_closed_forms()
        T.test_gaussians_at_their_centers_and_one_sigma_away(5, 2.0, 0.5)
        T.test_silu_identities()
        T.test_network_linear_in_last_layer_and_zero_without_first()
        T.test_scalars_match_the_workload_recipe()
    except AssertionError:
        return False
    return True


def test_unpatched_radial_oracle_passes_its_pins():
    assert radial_pins_ok()


@pytest.mark.parametrize("name", ["centers", "no_cutoff", "sigma_squared", "sigmoid", "half_period"])
def test_radial_mistakes_are_caught(monkeypatch, name):
    import math as _m
    from oracle import radial
    orig_basis, orig_cut, orig_silu = radial.basis, radial.cutoff, radial.silu
    if name == "centers":            # centers at k r_max / num_basis
        def basis(r, nb, r_max, sigma):
            r = np.asarray(r, np.float64)
            c = np.array([k * r_max / nb for k in range(nb)])
            return np.exp(-(((r[:, None] - c[None, :]) / sigma) ** 2)) * orig_cut(r, r_max)[:, None]
        monkeypatch.setattr(radial, "basis", basis)
    elif name == "no_cutoff":
        monkeypatch.setattr(radial, "basis", lambda r, nb, r_max, sigma:
                            orig_basis(r, nb, r_max, sigma) / orig_cut(r, r_max)[:, None])
    elif name == "sigma_squared":     # exp(-(r - mu)^2 / sigma)
        def basis(r, nb, r_max, sigma):
            return orig_basis(r, nb, r_max, _m.sqrt(sigma))
        monkeypatch.setattr(radial, "basis", basis)
    elif name == "sigmoid":
        monkeypatch.setattr(radial, "silu", lambda z: 1.0 / (1.0 + np.exp(-np.asarray(z, np.float64))))
    elif name == "half_period":       # cos(pi r / (2 r_max))
        monkeypatch.setattr(radial, "cutoff", lambda r, r_max: orig_cut(r, 2.0 * r_max))
    assert not radial_pins_ok()


# ---------------------------------------------- pair storage (variants) -----

def pair_pins_ok():
    from .test_oracle_variants import pairs_backward_is_derivative, pairs_equal_receiver
    return pairs_equal_receiver(2) and pairs_backward_is_derivative(2)


def test_unpatched_pair_oracle_passes_its_pins():
    assert pair_pins_ok()


@pytest.mark.parametrize("name", ["reverse_y_unflipped", "reverse_edges_dropped",
                                  "grad_y_fold_unflipped", "grad_s_one_direction",
                                  "grad_x_one_direction"])
def test_pair_mistakes_are_caught(monkeypatch, name):
    from oracle import variants
    expand = variants.expand_pairs

    def fold(dy_sign, both_s, both_x):
        def backward_pairs(lay, x, y, s, g, senders, receivers, num_nodes):
            y2, s2, a2, b2 = expand(lay, y, s, senders, receivers)
            m = len(senders)
            dx, dy2, ds2 = conv.backward(lay, x, y2, s2, g, a2, b2, num_nodes)
            if not both_x:
                dx = conv.backward(lay, x, y2[:m], s2[:m], g, a2[:m], b2[:m], num_nodes)[0]
            sign = variants.parity_sign(lay) if dy_sign else 1.0
            return dx, dy2[:m] + dy2[m:] * sign, ds2[:m] + (ds2[m:] if both_s else 0.0)
        return backward_pairs

    if name == "reverse_y_unflipped":
        def expand_bad(lay, y, s, senders, receivers):
            y2, s2, a2, b2 = expand(lay, y, s, senders, receivers)
            m = len(senders)
            y2[m:] = y2[:m]
            return y2, s2, a2, b2
        monkeypatch.setattr(variants, "expand_pairs", expand_bad)
    elif name == "reverse_edges_dropped":
        monkeypatch.setattr(variants, "forward_pairs",
                            lambda lay, x, y, s, a, b, n: conv.forward(lay, x, y, s, a, b, n))
    elif name == "grad_y_fold_unflipped":
        monkeypatch.setattr(variants, "backward_pairs", fold(False, True, True))
    elif name == "grad_s_one_direction":
        monkeypatch.setattr(variants, "backward_pairs", fold(True, False, True))
    else:
        monkeypatch.setattr(variants, "backward_pairs", fold(True, True, False))
    assert not pair_pins_ok()
