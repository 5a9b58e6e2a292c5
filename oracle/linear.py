"""Oracle for the output linear (test infrastructure, fp64).

cuEquivariance page, Flax NNX layers, ``IrrepsLinear``: within each irrep
block, output[..., v, i] = scale / sqrt(mul_in) * sum_u w[u, v] input[..., u, i],
u and v running over the input and output channels, i over the components.  Applied
to the convolution output (N, num_out, C) -- trailing channels -- each output
block of the layout is one ``ir`` with mul_in = C.
"""

import numpy as np


def blocks(lay):
    """(offset, dim) of each output block of a convolution layout."""
    out, o = [], 0
    for (l, _p) in lay.out_blocks:
        out.append((o, 2 * l + 1))
        o += 2 * l + 1
    return out


def linear(lay, w, scale, x):
    """w (num_blocks, C, C_out); x (N, num_out, C) -> (N, num_out, C_out)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    N, _, C = x.shape
    out = np.zeros((N, lay.num_out, w.shape[2]))
    factor = scale / np.sqrt(C)
    for k, (o, d) in enumerate(blocks(lay)):
        # trailing channels: x[n, component, u]; out[n, component, v]
        out[:, o:o + d, :] = factor * np.einsum("niu,uv->niv", x[:, o:o + d, :], w[k])
    return out


def linear_backward(lay, w, scale, x, g):
    """Gradients (d x, d w) of <g, linear(w, x)>."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    C = x.shape[2]
    factor = scale / np.sqrt(C)
    dx = np.zeros_like(x)
    dw = np.zeros_like(w)
    for k, (o, d) in enumerate(blocks(lay)):
        xs, gs = x[:, o:o + d, :], g[:, o:o + d, :]
        dx[:, o:o + d, :] = factor * np.einsum("uv,niv->niu", w[k], gs)
        dw[k] = factor * np.einsum("niu,niv->uv", xs, gs)
    return dx, dw
