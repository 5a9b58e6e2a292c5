"""Pins for the oracle's output linear (cuEquivariance page, IrrepsLinear), CPU only.

The page states the layer's properties: channel mixing within matching
irreps with scale / sqrt(mul_in) normalization, and rotation equivariance
(rotating each input irrep rotates the output the same way).  Pinned here by
a hand-worked value, the identity closed form, block independence, the
rotation property with the oracle's Wigner matrices, and exact central
differences for the gradients (the map is bilinear in (w, x)).
"""

import math

import numpy as np
import pytest

from oracle import conv, linear, so3
from equivariant_gnn_message_amd import synth

from ._util import random_rotation, rel_max_err


def layout_of(idx, C):
    w = synth.WORKLOADS[idx]
    return conv.make_layout(w.irreps_in.replace(f"{w.channels}x", f"{C}x"), w.lmax,
                            w.irreps_out.replace(f"{w.channels}x", f"{C}x"))


def test_hand_worked_value():
    lay = conv.make_layout("2x0e", 0, "2x0e")
    x = np.array([[[3.0, -1.0]]])                    # one node, one scalar component, C = 2
    w = np.array([[[1.0], [2.0]]])                   # (blocks, C, C_out=1)
    out = linear.linear(lay, w, math.sqrt(2.0), x)   # factor sqrt(2)/sqrt(2) = 1
    assert out.shape == (1, 1, 1) and out[0, 0, 0] == pytest.approx(3.0 - 2.0)


@pytest.mark.parametrize("idx,C", [(0, 4), (2, 8), (3, 4)])
def test_identity_weights(idx, C):
    lay = layout_of(idx, C)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, lay.num_out, C))
    nb = len(lay.out_blocks)
    scale = 0.7
    w = np.broadcast_to(np.eye(C) * math.sqrt(C) / scale, (nb, C, C))
    assert rel_max_err(linear.linear(lay, w, scale, x), x) < 1e-14


def test_blocks_are_independent():
    lay = layout_of(2, 4)
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, lay.num_out, 4))
    w = np.zeros((len(lay.out_blocks), 4, 6))
    w[2] = rng.standard_normal((4, 6))
    out = linear.linear(lay, w, 1.0, x)
    for k, (o, d) in enumerate(linear.blocks(lay)):
        part = out[:, o:o + d, :]
        assert (np.abs(part).max() > 0) == (k == 2)


@pytest.mark.parametrize("idx", [2, 3])
def test_rotation_equivariance(idx):
    lay = layout_of(idx, 3)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, lay.num_out, 3))
    w = rng.standard_normal((len(lay.out_blocks), 3, 5))
    axis, angle = random_rotation(rng)
    D = so3.block_D([(1, l, p) for l, p in lay.out_blocks], axis, angle, improper=True)
    rotate = lambda a: np.einsum("ij,njc->nic", D, a)
    lhs = linear.linear(lay, w, 0.9, rotate(x))
    rhs = rotate(linear.linear(lay, w, 0.9, x))
    assert rel_max_err(lhs, rhs) < 1e-12


@pytest.mark.parametrize("idx,C,Co", [(0, 3, 5), (2, 4, 2)])
def test_gradients_central_differences(idx, C, Co):
    lay = layout_of(idx, C)
    rng = np.random.default_rng(4)
    x = rng.standard_normal((6, lay.num_out, C))
    w = rng.standard_normal((len(lay.out_blocks), C, Co))
    g = rng.standard_normal((6, lay.num_out, Co))
    dx, dw = rng.standard_normal(x.shape), rng.standard_normal(w.shape)
    L = lambda ww, xx: np.vdot(g, linear.linear(lay, ww, 1.3, xx))
    # bilinear: the central difference at h = 1 is the exact directional derivative
    deriv = (L(w + dw, x + dx) - L(w - dw, x - dx)) / 2
    gx, gw = linear.linear_backward(lay, w, 1.3, x, g)
    assert abs(np.vdot(gx, dx) + np.vdot(gw, dw) - deriv) <= 1e-10 * (abs(deriv) + 1.0)
