"""Oracle for the convolution fed by radial edge scalars (test infrastructure, fp64).

The edge scalars of the gate-points model are not an input there: each edge
computes its own from its length (e3nn_mlx gate-points page: the network
embeds the edge length in a radial basis with a smooth cutoff and maps it
through a fully connected network to the per-path, per-channel weights of
the convolution; the workload fixes the plain reading R11):

    f_k(r) = exp(-((r - mu_k) / sigma)^2) * (1 + cos(pi r / r_max)) / 2,
             mu_k = k r_max / (num_basis - 1),  k = 0 .. num_basis - 1,
    h      = silu(f(r) W1),     silu(z) = z / (1 + exp(-z)),
    s[e]   = h W2,  reshaped to (num_paths, C)  (path-major, as the s axis).

``forward_radial`` is the e3j convolution of ``oracle.conv`` with those
scalars.  The oracle is written from these definitions only; it shares no
code with the library's kernels or with the input generator.
"""

import math

import numpy as np

from . import conv


def cutoff(r, r_max):
    """Cosine cutoff: (1 + cos(pi r / r_max)) / 2 for r < r_max, 0 from r_max on (a cutoff
    function vanishes beyond its radius; e3nn_mlx gate-points page, Scope: cosine cutoff)."""
    r = np.asarray(r, dtype=np.float64)
    return np.where(r < r_max, 0.5 * (1.0 + np.cos(math.pi * r / r_max)), 0.0)


def basis(r, num_basis, r_max, sigma):
    """Gaussian radial basis times the cutoff: (E, num_basis)."""
    r = np.asarray(r, dtype=np.float64)
    centers = np.array([k * r_max / (num_basis - 1) for k in range(num_basis)])
    g = np.exp(-(((r[:, None] - centers[None, :]) / sigma) ** 2))
    return g * cutoff(r, r_max)[:, None]


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def mlp(feat, w1, w2):
    """silu(feat W1) W2 in fp64."""
    return silu(np.asarray(feat, np.float64) @ np.asarray(w1, np.float64)) @ np.asarray(w2, np.float64)


def scalars(lay, r, w1, w2, r_max, sigma):
    """Edge scalars (E, num_paths, C) of the layout from edge lengths."""
    w1 = np.asarray(w1, np.float64)
    s = mlp(basis(r, w1.shape[0], r_max, sigma), w1, w2)
    return s.reshape(len(s), lay.num_paths, lay.channels)


def forward_radial(lay, x, y, r, w1, w2, r_max, sigma, senders, receivers, num_nodes):
    """The convolution with s computed per edge from r."""
    s = scalars(lay, r, w1, w2, r_max, sigma)
    return conv.forward(lay, x, y, s, senders, receivers, num_nodes)


def forward_radial_rows(lay, x, y, r, w1, w2, r_max, sigma, senders, receivers, rows):
    """Output rows of the selected receivers only (sampled full-size checks)."""
    rows = np.asarray(rows, dtype=np.int64)
    receivers = np.asarray(receivers)
    pick = np.flatnonzero(np.isin(receivers, rows))
    s = scalars(lay, np.asarray(r)[pick], w1, w2, r_max, sigma)
    return conv.forward_rows(lay, x, np.asarray(y)[pick], s, np.asarray(senders)[pick], receivers[pick], rows)


def forward_radial_bruteforce(lay, x, y, r, w1, w2, r_max, sigma, senders, receivers, num_nodes):
    """Pure-Python loops for the scalars (math.exp, math.cos), then the brute-force convolution."""
    w1 = np.asarray(w1, np.float64)
    w2 = np.asarray(w2, np.float64)
    nb, hid = w1.shape
    E = len(senders)
    s = np.zeros((E, lay.num_paths * lay.channels))
    for e in range(E):
        re = float(r[e])
        cut = 0.5 * (1.0 + math.cos(math.pi * re / r_max)) if re < r_max else 0.0
        f = [math.exp(-(((re - k * r_max / (nb - 1)) / sigma) ** 2)) * cut for k in range(nb)]
        for j in range(hid):
            z = sum(f[k] * w1[k, j] for k in range(nb))
            hj = z / (1.0 + math.exp(-z))
            for q in range(s.shape[1]):
                s[e, q] += hj * w2[j, q]
    s = s.reshape(E, lay.num_paths, lay.channels)
    return conv.forward_bruteforce(lay, x, y, s, senders, receivers, num_nodes)
