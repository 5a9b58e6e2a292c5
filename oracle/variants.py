"""Oracle for the convolution's variants (test infrastructure, fp64).

Built from ``oracle.conv`` without new arithmetic of its own:

* SENDER graph ordering (e3j ``Convolution`` page, the note on
  ``graph_ordering`` for the fused kernels): edges are grouped by sender and
  the message of node b is assembled from b's outgoing edges, using the
  reverse edge's features under the page's symmetry assumptions
  (y_ab = (-1)^l y_ba per l block, s_ab = s_ba).  Read plainly: every edge
  e = (b -> a) is reversed to (a -> b) with its y blocks of odd l negated and
  its s unchanged, and the RECEIVER convolution is applied to the reversed
  edges.  The gradients are those of that function.
* node_mask padding (same page, ``__call__`` argument ``node_mask``): True for
  real nodes, False for padding nodes at the tail; padding edges only connect
  padding nodes.  Read plainly: the messages of edges into padding receivers
  are dropped and the rows of padding nodes are zero; the reverse pass is the
  derivative of that function.
* pair storage (same page, same note: every edge a -> b has its reverse
  b -> a, y_ba = (-1)^l y_ab per l block, s_ba = s_ab).  Read plainly, those
  assumptions let a symmetric graph keep one row of y and s per undirected
  pair: a stored edge e = (a -> b) stands for itself and for its reverse
  (b -> a) with features P y[e] (odd-l blocks negated) and scalars s[e].  The
  function of the stored arrays is the RECEIVER convolution of those 2 E
  directed edges (a stored self loop a -> a therefore counts twice); its
  reverse pass follows by the chain rule: grad_y[e] = dy(a -> b) +
  P dy(b -> a) and grad_s[e] = ds(a -> b) + ds(b -> a).
* forward-mode derivative and second derivatives (e3nn_mlx page, "JVP and
  generated-kernel boundary"): the convolution is trilinear in (x, y, s), so
  by the product rule its derivative along (dx, dy, ds) is
  conv(dx, y, s) + conv(x, dy, s) + conv(x, y, ds).
"""

import numpy as np

from . import conv


def parity_sign(lay):
    """(-1)^l of each edge-feature component (blocks l = 0..lmax)."""
    sign = np.empty(lay.num_y)
    for l in range(lay.lmax + 1):
        sign[l * l:(l + 1) * (l + 1)] = (-1.0) ** l
    return sign


def forward_sender(lay, x, y, s, senders, receivers, num_nodes):
    """SENDER ordering: node b sums its outgoing edges, reversed."""
    y_rev = np.asarray(y, dtype=np.float64) * parity_sign(lay)
    return conv.forward(lay, x, y_rev, s, receivers, senders, num_nodes)


def backward_sender(lay, x, y, s, g, senders, receivers, num_nodes):
    """Gradients of ``forward_sender`` (chain rule through the sign flip)."""
    sign = parity_sign(lay)
    y_rev = np.asarray(y, dtype=np.float64) * sign
    dx, dy_rev, ds = conv.backward(lay, x, y_rev, s, g, receivers, senders, num_nodes)
    return dx, dy_rev * sign, ds


def expand_pairs(lay, y, s, senders, receivers):
    """The directed edges that the stored pairs stand for: the stored edges
    (a -> b) with y and s, then their reverses (b -> a) with P y and s.
    Returns (y2, s2, senders2, receivers2) of length 2 E."""
    y = np.asarray(y, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    a = np.asarray(senders)
    b = np.asarray(receivers)
    return (np.concatenate([y, y * parity_sign(lay)]), np.concatenate([s, s]),
            np.concatenate([a, b]), np.concatenate([b, a]))


def forward_pairs(lay, x, y, s, senders, receivers, num_nodes):
    """Pair storage: the RECEIVER convolution of every stored edge and its reverse."""
    y2, s2, a2, b2 = expand_pairs(lay, y, s, senders, receivers)
    return conv.forward(lay, x, y2, s2, a2, b2, num_nodes)


def backward_pairs(lay, x, y, s, g, senders, receivers, num_nodes):
    """Gradients of ``forward_pairs``: each stored row collects the gradients
    of both directed edges it stands for (the reverse one through P)."""
    y2, s2, a2, b2 = expand_pairs(lay, y, s, senders, receivers)
    dx, dy2, ds2 = conv.backward(lay, x, y2, s2, g, a2, b2, num_nodes)
    m = len(senders)
    return dx, dy2[:m] + dy2[m:] * parity_sign(lay), ds2[:m] + ds2[m:]


def edges_into_real(receivers, num_real):
    return np.asarray(receivers) < num_real


def forward_masked(lay, x, y, s, senders, receivers, num_nodes, num_real):
    """node_mask padding: messages into padding receivers dropped, their rows zero."""
    keep = edges_into_real(receivers, num_real)
    out = conv.forward(lay, x, np.asarray(y)[keep], np.asarray(s)[keep],
                       np.asarray(senders)[keep], np.asarray(receivers)[keep], num_nodes)
    out[num_real:] = 0.0
    return out


def backward_masked(lay, x, y, s, g, senders, receivers, num_nodes, num_real):
    """Gradients of ``forward_masked``: zero for the dropped edges."""
    keep = edges_into_real(receivers, num_real)
    dx, dyk, dsk = conv.backward(lay, x, np.asarray(y)[keep], np.asarray(s)[keep], g,
                                 np.asarray(senders)[keep], np.asarray(receivers)[keep], num_nodes)
    dy = np.zeros((len(keep), lay.num_y))
    ds = np.zeros((len(keep), lay.num_paths, lay.channels))
    dy[keep] = dyk
    ds[keep] = dsk
    return dx, dy, ds


def jvp(lay, x, y, s, dx, dy, ds, senders, receivers, num_nodes):
    """(out, out_dot): the convolution and its derivative along (dx, dy, ds)."""
    f = lambda a, b, c: conv.forward(lay, a, b, c, senders, receivers, num_nodes)
    out = f(x, y, s)
    out_dot = f(dx, y, s) + f(x, dy, s) + f(x, y, ds)
    return out, out_dot


def double_backward(lay, x, y, s, g, Gx, Gy, Gs, senders, receivers, num_nodes):
    """Second derivatives (reverse over reverse; e3nn_mlx page, JVP section).

    With (gx, gy, gs) the gradients of <g, conv(x, y, s)>, returns the
    gradients of L2 = <Gx, gx> + <Gy, gy> + <Gs, gs> with respect to
    (x, y, s, g).  L2 = <g, D conv(x, y, s)[Gx, Gy, Gs]>, so by the product
    rule dL2/dg is the JVP along (Gx, Gy, Gs) and each operand's gradient sums
    the reverse passes in which another operand is replaced by its cotangent.
    """
    bw = lambda a, b, c: conv.backward(lay, a, b, c, g, senders, receivers, num_nodes)
    _, dy_a, ds_a = bw(Gx, y, s)
    dx_b, _, ds_b = bw(x, Gy, s)
    dx_c, dy_c, _ = bw(x, y, Gs)
    _, dg = jvp(lay, x, y, s, Gx, Gy, Gs, senders, receivers, num_nodes)
    return dx_b + dx_c, dy_a + dy_c, ds_a + ds_b, dg
