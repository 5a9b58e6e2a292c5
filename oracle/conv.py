"""Oracle convolution: paths, forward and backward in fp64 (test infrastructure).

Definition (e3j ``Convolution`` page, class formula):

    m_b = (1/N) sum_{a -> b} (x_a (x) y_ab) (.) s_ab

computed in the order of the unfused JAX implementation that the same
page describes, step by step over all edges:
  1. each edge takes its sender's row of x,
  2. that row meets the edge's harmonics y in the channelwise CG product,
  3. every (path, channel) of the product is weighted by the edge scalar s,
  4. each edge's message is added into its receiver's row,
and the sums are scaled by 1/N, N = ``avg_num_neighbors``.

Shapes follow the same page's ``__call__``: node_features (num_nodes, num_x, C),
edge_features (num_edges, num_y) broadcast over channels, edge_scalars
(num_edges, num_scalars, C), senders / receivers index vectors in
[0, num_nodes).  The oracle accepts edges in any order.

Readings where the page is silent:
* the tensor product is channelwise ("weighted"): channel c of x meets the
  channel-less y, every allowed (x block, l2, out block) triple is one path,
  and the mixing scalars carry one value per (path, channel): the page derives
  this third operand's space from the spaces of x and y;
* a path exists iff |l1-l2| <= l3 <= l1+l2 and p3 = p1 * (-1)^l2 (y are
  spherical harmonics, parity (-1)^l2); paths are enumerated x block, then
  l2 = 0..L, then output block; this order is the scalar axis;
* paths into the same output block add up;
* an output block no path reaches is an error (the target argument filters
  output blocks, it does not create them);
* CG tensors are the real, orthonormal ones of ``oracle.so3.real_cg``.
"""

from dataclasses import dataclass

import numpy as np

from . import irreps as _irreps
from .so3 import real_cg


@dataclass(frozen=True)
class Path:
    i1: int   # x block index
    l1: int
    p1: int
    o1: int   # component offset of the x block
    l2: int
    o2: int   # component offset of the y block (= l2^2)
    i3: int   # output block index
    l3: int
    p3: int
    o3: int   # component offset of the output block


@dataclass(frozen=True)
class Layout:
    channels: int
    x_blocks: tuple      # ((l, p), ...)
    lmax: int
    out_blocks: tuple
    paths: tuple
    num_x: int
    num_y: int
    num_out: int
    avg_num_neighbors: float

    @property
    def num_paths(self):
        return len(self.paths)


def make_layout(irreps_in, sh_lmax, irreps_out, avg_num_neighbors=1.0):
    """Parse, check and enumerate paths (raises ValueError on a bad layout)."""
    xin = _irreps.parse(irreps_in)
    xout = _irreps.parse(irreps_out)
    if sh_lmax < 0:
        raise ValueError("sh_lmax must be >= 0")
    muls = {m for (m, _, _) in xin + xout}
    if len(muls) != 1:
        raise ValueError("the convolution needs one multiplicity across all blocks")
    C = muls.pop()
    if C <= 0:
        raise ValueError("multiplicity must be positive")
    xb = tuple((l, p) for (_, l, p) in xin)
    ob = tuple((l, p) for (_, l, p) in xout)
    if len(set(xb)) != len(xb) or len(set(ob)) != len(ob):
        raise ValueError("duplicate irreps in a block list")
    offs_x = np.cumsum([0] + [2 * l + 1 for (l, _) in xb])
    offs_o = np.cumsum([0] + [2 * l + 1 for (l, _) in ob])
    paths = []
    for i1, (l1, p1) in enumerate(xb):
        for l2 in range(sh_lmax + 1):
            for i3, (l3, p3) in enumerate(ob):
                if abs(l1 - l2) <= l3 <= l1 + l2 and p3 == p1 * (-1) ** l2:
                    paths.append(Path(i1, l1, p1, int(offs_x[i1]), l2, l2 * l2,
                                      i3, l3, p3, int(offs_o[i3])))
    reached = {p.i3 for p in paths}
    for i3 in range(len(ob)):
        if i3 not in reached:
            raise ValueError(f"output block {ob[i3]} is reached by no path")
    return Layout(C, xb, sh_lmax, ob, tuple(paths), int(offs_x[-1]),
                  (sh_lmax + 1) ** 2, int(offs_o[-1]), float(avg_num_neighbors))


def _as64(a):
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------- forward ---

def forward_bruteforce(lay, x, y, s, senders, receivers, num_nodes):
    """Pure-Python loops: per edge, per path, per (m1, m2, m3), per channel."""
    x, y, s = _as64(x), _as64(y), _as64(s)
    C = lay.channels
    out = [[[0.0] * C for _ in range(lay.num_out)] for _ in range(num_nodes)]
    for e in range(len(senders)):
        a, b = int(senders[e]), int(receivers[e])
        for p, P in enumerate(lay.paths):
            cg = real_cg(P.l1, P.l2, P.l3)
            for m1 in range(2 * P.l1 + 1):
                for m2 in range(2 * P.l2 + 1):
                    for m3 in range(2 * P.l3 + 1):
                        w = cg[m1, m2, m3]
                        if w == 0.0:
                            continue
                        for c in range(C):
                            out[b][P.o3 + m3][c] += (
                                w * x[a, P.o1 + m1, c] * y[e, P.o2 + m2] * s[e, p, c])
    return np.array(out, dtype=np.float64).reshape(num_nodes, lay.num_out, C) / lay.avg_num_neighbors


def messages(lay, x, y, s, senders):
    """Steps 1-3 for a chunk of edges: per-edge messages (E, num_out, C)."""
    y, s = _as64(y), _as64(s)
    E = len(senders)
    msg = np.zeros((E, lay.num_out, lay.channels))
    xa = _as64(x[np.asarray(senders, dtype=np.int64)])                # step 1: gather
    for p, P in enumerate(lay.paths):
        cg = real_cg(P.l1, P.l2, P.l3)
        t = np.einsum("ijk,eic,ej->ekc", cg,                         # step 2: TP
                      xa[:, P.o1:P.o1 + 2 * P.l1 + 1, :],
                      y[:, P.o2:P.o2 + 2 * P.l2 + 1])
        msg[:, P.o3:P.o3 + 2 * P.l3 + 1, :] += s[:, p, None, :] * t  # step 3: mix
    return msg


def forward(lay, x, y, s, senders, receivers, num_nodes, chunk=8192):
    """Vectorised oracle forward (any edge order), fp64 result."""
    out = np.zeros((num_nodes, lay.num_out, lay.channels))
    E = len(senders)
    for e0 in range(0, E, chunk):
        e1 = min(E, e0 + chunk)
        msg = messages(lay, x, y[e0:e1], s[e0:e1], senders[e0:e1])
        np.add.at(out, np.asarray(receivers[e0:e1], dtype=np.int64), msg)  # step 4
    return out / lay.avg_num_neighbors


def forward_rows(lay, x, y, s, senders, receivers, rows):
    """Oracle output for selected receiver rows only (for sampled checks)."""
    rows = np.asarray(rows, dtype=np.int64)
    receivers = np.asarray(receivers)
    out = np.zeros((len(rows), lay.num_out, lay.channels))
    for k, b in enumerate(rows):
        sel = np.flatnonzero(receivers == b)
        if len(sel):
            msg = messages(lay, x, y[sel], s[sel], np.asarray(senders)[sel])
            out[k] = msg.sum(axis=0)
    return out / lay.avg_num_neighbors


# --------------------------------------------------------------- backward ---

def edge_grads(lay, x, y, s, g, senders, receivers):
    """Per-edge pieces of the reverse pass for a chunk of edges.

    With t^p = CG^p(x_a, y_e) and h^p = s^p * g_b (per channel), the output is
    linear in each of x, y, s, so for L = <g, out>:
      dL/ds[e,p,c]      = (1/N) sum_m3 g[b,o3+m3,c] t^p[m3,c]
      dL/dy[e,o2+m2]    = (1/N) sum_p sum_c sum_{m1,m3} C[m1,m2,m3] x[a,o1+m1,c] h^p[m3,c]
      contribution to dL/dx[a,o1+m1,c] = (1/N) sum_p sum_{m2,m3} C[m1,m2,m3] y[e,o2+m2] h^p[m3,c]
    Returns (ds, dy, dx_edge) with dx_edge (E, num_x, C) still to be summed by sender.
    """
    y, s = _as64(y), _as64(s)
    inv = 1.0 / lay.avg_num_neighbors
    snd = np.asarray(senders, dtype=np.int64)
    rcv = np.asarray(receivers, dtype=np.int64)
    E = len(snd)
    xa, gb = _as64(x[snd]), _as64(g[rcv])
    ds = np.zeros((E, lay.num_paths, lay.channels))
    dy = np.zeros((E, lay.num_y))
    dxe = np.zeros((E, lay.num_x, lay.channels))
    for p, P in enumerate(lay.paths):
        cg = real_cg(P.l1, P.l2, P.l3)
        xs = xa[:, P.o1:P.o1 + 2 * P.l1 + 1, :]
        ys = y[:, P.o2:P.o2 + 2 * P.l2 + 1]
        gs = gb[:, P.o3:P.o3 + 2 * P.l3 + 1, :]
        t = np.einsum("ijk,eic,ej->ekc", cg, xs, ys)
        ds[:, p, :] = np.einsum("ekc,ekc->ec", gs, t) * inv
        h = s[:, p, None, :] * gs
        dy[:, P.o2:P.o2 + 2 * P.l2 + 1] += np.einsum("ijk,eic,ekc->ej", cg, xs, h) * inv
        dxe[:, P.o1:P.o1 + 2 * P.l1 + 1, :] += np.einsum("ijk,ej,ekc->eic", cg, ys, h) * inv
    return ds, dy, dxe


def backward(lay, x, y, s, g, senders, receivers, num_nodes, chunk=8192):
    """Vectorised oracle gradients (dx, dy, ds) of L = <g, out> (fp64)."""
    E = len(senders)
    dx = np.zeros((num_nodes, lay.num_x, lay.channels))
    dy = np.zeros((E, lay.num_y))
    ds = np.zeros((E, lay.num_paths, lay.channels))
    for e0 in range(0, E, chunk):
        e1 = min(E, e0 + chunk)
        dsc, dyc, dxe = edge_grads(lay, x, y[e0:e1], s[e0:e1], g,
                                   senders[e0:e1], receivers[e0:e1])
        ds[e0:e1] = dsc
        dy[e0:e1] = dyc
        np.add.at(dx, np.asarray(senders[e0:e1], dtype=np.int64), dxe)
    return dx, dy, ds


def backward_bruteforce(lay, x, y, s, g, senders, receivers, num_nodes):
    """Pure-Python loops over the same closed forms as ``edge_grads``."""
    x, y, s, g = _as64(x), _as64(y), _as64(s), _as64(g)
    C = lay.channels
    inv = 1.0 / lay.avg_num_neighbors
    E = len(senders)
    dx = np.zeros((num_nodes, lay.num_x, C))
    dy = np.zeros((E, lay.num_y))
    ds = np.zeros((E, lay.num_paths, C))
    for e in range(E):
        a, b = int(senders[e]), int(receivers[e])
        for p, P in enumerate(lay.paths):
            cg = real_cg(P.l1, P.l2, P.l3)
            for m1 in range(2 * P.l1 + 1):
                for m2 in range(2 * P.l2 + 1):
                    for m3 in range(2 * P.l3 + 1):
                        w = cg[m1, m2, m3]
                        if w == 0.0:
                            continue
                        for c in range(C):
                            xv = x[a, P.o1 + m1, c]
                            yv = y[e, P.o2 + m2]
                            gv = g[b, P.o3 + m3, c]
                            sv = s[e, p, c]
                            ds[e, p, c] += w * xv * yv * gv * inv
                            dy[e, P.o2 + m2] += w * xv * sv * gv * inv
                            dx[a, P.o1 + m1, c] += w * yv * sv * gv * inv
    return dx, dy, ds
