"""Seeded synthetic inputs for the convolution (shared by tests, bench and smoke).

This module holds none of the convolution's arithmetic: it draws graphs and
operands.  Both the CPU oracle and the HIP path consume what it returns.

Workloads (a radius graph of random points stands in for the point clouds the
e3nn_mlx gate-points page builds with its radius graph; no dataset is named on
the pages):

  0 tiny       N=64, E=512, senders/receivers independent uniform draws
               (self loops and duplicates kept), 8x0e+8x1o, SH lmax 2,
               s ~ N(0,1), out 8x0e+8x1o+8x2e, avg_num_neighbors 8
  1 gatepoints 64 graphs x 64 nodes in a cube of side 4.17 (mean degree ~16
               within r=2.0), 32x0e+32x1o, SH lmax 3, s = radial MLP of 5
               Gaussian RBFs x cosine cutoff (Linear 5->100, silu,
               Linear 100->P*C, fan-in normalised), out 32x(0e+1o+2e), avg 16
  2 mace       N=20000 in a cube of side 27.40, r=2.0 (~598k edges),
               128x0e+128x1o, SH lmax 3, s ~ N(0,1), out 128x(0e+1o+2e+3o),
               avg 30
  3 large_bf16 N=100000 in a cube of side 46.38, r=2.0 (~3.2M edges),
               64x(0e+1o+2e), SH lmax 3, x/y/s rounded to bf16, out fp32
               64x(0e+1o+2e+3o), avg 32
  4 training   graph and operands of 2, plus a cotangent g ~ N(0,1) on the output

Graphs are directed, loop-free, strict ``|p_a - p_b| < r``, and edges are
sorted by (receiver, sender).  Edge features are real spherical harmonics
(component normalisation, |Y^l|^2 = 2l+1) of the unit vector from sender to
receiver.  Every random tensor comes from
``numpy.random.SeedSequence([20261203, workload, tensor_id, chunk])`` with
tensor ids: positions/graph 0, x 1, edge directions 2, s 3, MLP weights 4,
cotangent 5.
"""

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

ROOT_SEED = 20261203
_CHUNK = 1 << 22


@dataclass(frozen=True)
class Workload:
    idx: int
    name: str
    irreps_in: str
    lmax: int
    irreps_out: str
    avg_num_neighbors: float
    dtype: str           # "f32" or "bf16" (storage of x, y, s)
    channels: int
    num_x: int           # components per channel of x
    num_out: int         # components per channel of the output
    num_paths: int       # size of the scalar axis of s (paths of the layout)
    num_nodes: int
    cube_side: float = 0.0
    radius: float = 2.0
    num_graphs: int = 1
    num_edges: int = 0   # for the uniform-random tiny graph
    backward: bool = False


# Sizes are data here (the path count of each layout is stated, not derived;
# tests check it against both the oracle's and the library's enumeration).
WORKLOADS = {
    0: Workload(0, "tiny", "8x0e+8x1o", 2, "8x0e+8x1o+8x2e", 8.0, "f32",
                8, 4, 9, 7, 64, num_edges=512),
    1: Workload(1, "gatepoints", "32x0e+32x1o", 3, "32x0e+32x1o+32x2e", 16.0, "f32",
                32, 4, 9, 8, 64, cube_side=4.17, num_graphs=64),
    2: Workload(2, "mace", "128x0e+128x1o", 3, "128x0e+128x1o+128x2e+128x3o", 30.0, "f32",
                128, 4, 16, 10, 20000, cube_side=27.40),
    3: Workload(3, "large_bf16", "64x0e+64x1o+64x2e", 3, "64x0e+64x1o+64x2e+64x3o", 32.0,
                "bf16", 64, 9, 16, 17, 100000, cube_side=46.38),
    4: Workload(4, "training", "128x0e+128x1o", 3, "128x0e+128x1o+128x2e+128x3o", 30.0, "f32",
                128, 4, 16, 10, 20000, cube_side=27.40, backward=True),
}

# tensor ids
T_GRAPH, T_X, T_DIR, T_S, T_MLP, T_G = 0, 1, 2, 3, 4, 5
T_DX, T_DY, T_DS = 6, 7, 8   # tangents / second-order cotangents
T_S_PAIR = 9                  # edge scalars, one row per undirected pair


def rng(workload, tensor_id, chunk=0):
    return np.random.default_rng(np.random.SeedSequence([ROOT_SEED, workload, tensor_id, chunk]))


def _threads():
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:
        return max(1, min(16, os.cpu_count() or 1))


def normal_f32(workload, tensor_id, shape):
    """N(0,1) float32 draws filled chunk by chunk (chunk k has its own seed)."""
    out = np.empty(int(np.prod(shape)), dtype=np.float32)
    n = out.size
    starts = list(range(0, n, _CHUNK))

    def fill(k):
        a = starts[k]
        b = min(n, a + _CHUNK)
        out[a:b] = rng(workload, tensor_id, k).standard_normal(b - a, dtype=np.float32)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(len(starts))))
    return out.reshape(shape)


# -------------------------------------------------------------------- bf16 ---

def bf16_bits(a):
    """Round float32 values to bfloat16 (round-to-nearest-even), as uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits):
    """Exact decode of bfloat16 bits (uint16) to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(workload, tensor_id, shape):
    """N(0,1) draws as in ``normal_f32``, rounded to bf16 (uint16 bits)."""
    out = np.empty(int(np.prod(shape)), dtype=np.uint16)
    n = out.size
    starts = list(range(0, n, _CHUNK))

    def fill(k):
        a = starts[k]
        b = min(n, a + _CHUNK)
        out[a:b] = bf16_bits(rng(workload, tensor_id, k).standard_normal(b - a, dtype=np.float32))

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(len(starts))))
    return out.reshape(shape)


# ------------------------------------------------------ spherical harmonics ---

def spherical_harmonics(lmax, vec):
    """Real spherical harmonics l = 0..lmax of the directions ``vec``.

    Component normalisation (|Y^l(v)|^2 = 2l+1), m = -l..l, z polar axis, so
    l=1 is sqrt(3) (y, z, x).  Textbook closed forms of the orthonormal real
    harmonics times sqrt(4 pi) for l <= 3; the associated Legendre recursion
    (``sh_by_recursion``) from l = 4 on.  Vectors are normalised first.
    Returns (n, (lmax+1)^2) float64.
    """
    if lmax < 0:
        raise ValueError("lmax must be non-negative")
    if lmax > 3:
        low = spherical_harmonics(3, vec)
        high = sh_by_recursion(lmax, vec)[..., 16:]
        return np.concatenate([low, high], axis=-1)
    v = np.asarray(vec, dtype=np.float64)
    v = v / np.linalg.norm(v, axis=-1, keepdims=True)
    x, y, z = v[..., 0], v[..., 1], v[..., 2]
    cols = [np.ones_like(x)]
    if lmax >= 1:
        s3 = math.sqrt(3.0)
        cols += [s3 * y, s3 * z, s3 * x]
    if lmax >= 2:
        s15 = math.sqrt(15.0)
        cols += [s15 * x * y, s15 * y * z, math.sqrt(5.0) / 2 * (3 * z * z - 1),
                 s15 * x * z, s15 / 2 * (x * x - y * y)]
    if lmax >= 3:
        a = math.sqrt(35.0 / 8.0)
        b = math.sqrt(105.0)
        c = math.sqrt(21.0 / 8.0)
        d = math.sqrt(7.0) / 2
        cols += [a * (3 * x * x - y * y) * y, b * x * y * z, c * y * (5 * z * z - 1),
                 d * (5 * z ** 3 - 3 * z), c * x * (5 * z * z - 1),
                 b / 2 * (x * x - y * y) * z, a * (x * x - 3 * y * y) * x]
    return np.stack(cols, axis=-1)


def sh_by_recursion(lmax, vec):
    """The same harmonics for any lmax from the associated Legendre recursion.

    Y_l^m = sqrt(2l+1) sqrt((l-|m|)! / (l+|m|)!) Q_l^|m|(z) A_m(x, y), with
    Q_l^m the polynomial part of P_l^m (no Condon-Shortley phase):
    Q_m^m = (2m-1)!!, Q_{m+1}^m = (2m+1) z Q_m^m,
    (l-m) Q_l^m = (2l-1) z Q_{l-1}^m - (l+m-1) Q_{l-2}^m;
    and A_0 = 1, A_m = sqrt(2) Re (x + i y)^m, A_-m = sqrt(2) Im (x + i y)^m.
    """
    v = np.asarray(vec, dtype=np.float64)
    v = v / np.linalg.norm(v, axis=-1, keepdims=True)
    x, y, z = v[..., 0], v[..., 1], v[..., 2]
    w = x + 1j * y
    out = np.empty(v.shape[:-1] + ((lmax + 1) ** 2,))
    for m in range(lmax + 1):
        q_prev = None
        q = np.full(z.shape, float(np.prod(np.arange(2 * m - 1, 0, -2, dtype=np.float64))))
        a = w ** m
        for l in range(m, lmax + 1):
            if l == m + 1:
                q_prev, q = q, (2 * m + 1) * z * q
            elif l > m + 1:
                q_prev, q = q, ((2 * l - 1) * z * q - (l + m - 1) * q_prev) / (l - m)
            norm = math.sqrt((2 * l + 1) * math.factorial(l - m) / math.factorial(l + m))
            if m == 0:
                out[..., l * l + l] = norm * q
            else:
                out[..., l * l + l + m] = math.sqrt(2.0) * norm * q * a.real
                out[..., l * l + l - m] = math.sqrt(2.0) * norm * q * a.imag
    return out


# ------------------------------------------------------------------ graphs ---

def radius_graph(pos, r, batch=None):
    """Directed, loop-free radius graph with a strict boundary |p_a - p_b| < r.

    Returns (senders, receivers) as int64, sorted by (receiver, sender).
    Points in different ``batch`` entries are never connected.
    """
    from scipy.spatial import cKDTree

    pos = np.asarray(pos, dtype=np.float64)
    if batch is None:
        batch = np.zeros(len(pos), dtype=np.int64)
    src_all, dst_all = [], []
    for gid in np.unique(batch):
        idx = np.flatnonzero(batch == gid)
        if len(idx) < 2:
            continue
        tree = cKDTree(pos[idx])
        pairs = tree.query_pairs(r, output_type="ndarray")
        if len(pairs) == 0:
            continue
        d = np.linalg.norm(pos[idx[pairs[:, 0]]] - pos[idx[pairs[:, 1]]], axis=1)
        pairs = pairs[d < r]
        i, j = idx[pairs[:, 0]], idx[pairs[:, 1]]
        src_all += [i, j]
        dst_all += [j, i]
    if not src_all:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    src = np.concatenate(src_all)
    dst = np.concatenate(dst_all)
    order = np.lexsort((src, dst))
    return src[order], dst[order]


# ----------------------------------------------------------------- inputs ---

@dataclass
class Inputs:
    workload: Workload
    num_nodes: int
    senders: np.ndarray          # int32, sorted by receiver
    receivers: np.ndarray        # int32, non-decreasing
    x: np.ndarray                # float32 or uint16 (bf16 bits), (N, num_x, C)
    y: np.ndarray                # float32 or uint16, (E, num_y)
    s: np.ndarray                # float32 or uint16, (E, P, C)
    g: np.ndarray = None         # float32 (N, num_out, C) for the reverse pass
    extra: dict = field(default_factory=dict)

    @property
    def num_edges(self):
        return len(self.senders)

    def as_f32(self, name):
        a = getattr(self, name)
        return bf16_to_f32(a).reshape(a.shape) if a.dtype == np.uint16 else a


def make_inputs(idx, num_nodes=None, num_graphs=None, with_cotangent=None):
    """Build the seeded inputs of workload ``idx``.

    ``num_nodes`` (workloads 2-4) or ``num_graphs`` (workload 1) shrink the
    graph at the same point density, for parity runs the oracle can finish.
    """
    w = WORKLOADS[idx]
    C, num_x, num_out, P = w.channels, w.num_x, w.num_out, w.num_paths
    extra = {}
    if idx == 0:
        N = w.num_nodes
        gr = rng(idx, T_GRAPH)
        src = gr.integers(0, N, size=w.num_edges)
        dst = gr.integers(0, N, size=w.num_edges)
        order = np.argsort(dst, kind="stable")
        src, dst = src[order], dst[order]
        dirs = rng(idx, T_DIR).standard_normal((w.num_edges, 3))
        y = spherical_harmonics(w.lmax, dirs)
    elif idx == 1:
        G = num_graphs or w.num_graphs
        N = G * w.num_nodes
        pos = rng(idx, T_GRAPH).uniform(0.0, w.cube_side, size=(N, 3))
        batch = np.repeat(np.arange(G), w.num_nodes)
        src, dst = radius_graph(pos, w.radius, batch)
        vec = pos[dst] - pos[src]
        y = spherical_harmonics(w.lmax, vec)
        extra["pos"] = pos
        extra["batch"] = batch
    else:
        N = num_nodes or w.num_nodes
        side = w.cube_side * (N / w.num_nodes) ** (1.0 / 3.0)
        pos = rng(idx if idx != 4 else 2, T_GRAPH).uniform(0.0, side, size=(N, 3))
        src, dst = radius_graph(pos, w.radius)
        vec = pos[dst] - pos[src]
        y = spherical_harmonics(w.lmax, vec)
        extra["pos"] = pos
    E = len(src)
    # workload 4 reuses the operands of workload 2
    key = 2 if idx == 4 else idx
    if w.dtype == "bf16":
        x = normal_bf16(key, T_X, (N, num_x, C))
        yv = bf16_bits(y.astype(np.float32))
        s = normal_bf16(key, T_S, (E, P, C))
    else:
        x = normal_f32(key, T_X, (N, num_x, C))
        yv = y.astype(np.float32)
        if idx == 1:
            s = radial_mlp_scalars(np.linalg.norm(vec, axis=1), P * C, w.radius, idx).reshape(E, P, C)
        else:
            s = normal_f32(key, T_S, (E, P, C))
    g = None
    if with_cotangent or (with_cotangent is None and w.backward):
        g = normal_f32(idx, T_G, (N, num_out, C))
    return Inputs(w, N, src.astype(np.int32), dst.astype(np.int32), x, yv, s, g, extra)


def radial_mlp_scalars(r, width, rmax, idx=1, num_basis=5, hidden=100):
    """Edge scalars from lengths: Gaussian RBFs x cosine cutoff -> 2-layer MLP.

    RBF_k(r) = exp(-((r - mu_k) / sigma)^2), mu = linspace(0, rmax, 5),
    sigma = 0.5; cutoff(r) = (1 + cos(pi r / rmax)) / 2; MLP = Linear(5, 100)
    (no bias), silu, Linear(100, width) (no bias); weights N(0, 1) / sqrt(fan_in).
    """
    r = np.asarray(r, dtype=np.float64)
    mu = np.linspace(0.0, rmax, num_basis)
    sigma = 0.5
    rbf = np.exp(-(((r[:, None] - mu[None, :]) / sigma) ** 2))
    cut = 0.5 * (1.0 + np.cos(np.pi * r / rmax))
    feat = rbf * cut[:, None]
    W1, W2 = radial_mlp_weights(width, idx, num_basis, hidden)
    h = feat @ W1
    h = h / (1.0 + np.exp(-h))
    return (h @ W2).astype(np.float32)


def radial_mlp_weights(width, idx=1, num_basis=5, hidden=100):
    """The two weight matrices of the radial MLP, N(0, 1) / sqrt(fan_in), float64."""
    wr = rng(idx, T_MLP)
    W1 = wr.standard_normal((num_basis, hidden)) / math.sqrt(num_basis)
    W2 = wr.standard_normal((hidden, width)) / math.sqrt(hidden)
    return W1, W2


def radial_inputs(inp):
    """Edge lengths and float32 MLP weights of a gate-points workload's edges.

    The lengths are |pos[receiver] - pos[sender]|; the weights are the draws
    that generate the workload's s, so the MLP of these inputs reproduces s.
    """
    w = inp.workload
    pos = inp.extra["pos"]
    r = np.linalg.norm(pos[inp.receivers] - pos[inp.senders], axis=1).astype(np.float32)
    W1, W2 = radial_mlp_weights(w.num_paths * w.channels, w.idx)
    return r, W1.astype(np.float32), W2.astype(np.float32)


def subgraph16(inp):
    """16-node subgraph of workload 4 for finite differences.

    Receiver node 0 plus its first 15 distinct in-neighbours in CSR order; the
    induced edges (both endpoints in the set), relabelled by ascending original
    id, keeping the receiver-sorted order.  Returns (nodes, edge_ids, src, dst).
    """
    dst = inp.receivers
    src = inp.senders
    first = np.flatnonzero(dst == 0)
    nodes = [0]
    for e in first:
        a = int(src[e])
        if a not in nodes:
            nodes.append(a)
        if len(nodes) == 16:
            break
    nodes = np.array(sorted(nodes), dtype=np.int64)
    inset = np.zeros(inp.num_nodes, dtype=bool)
    inset[nodes] = True
    eids = np.flatnonzero(inset[src] & inset[dst])
    relabel = -np.ones(inp.num_nodes, dtype=np.int64)
    relabel[nodes] = np.arange(len(nodes))
    return nodes, eids, relabel[src[eids]].astype(np.int32), relabel[dst[eids]].astype(np.int32)


# ------------------------------------------------ graph-ordering helpers ----

def sender_sorted(senders, receivers):
    """Permutation that sorts edges by (sender, receiver)."""
    return np.lexsort((np.asarray(receivers), np.asarray(senders)))


def symmetric_normal(senders, receivers, shape_tail, seed):
    """Per-edge N(0,1) arrays that agree on an edge and its reverse.

    One draw per unordered node pair {a, b}; both directed edges get it (the
    symmetric edge scalars s_ab = s_ba of the e3j SENDER ordering).
    """
    a = np.asarray(senders, dtype=np.int64)
    b = np.asarray(receivers, dtype=np.int64)
    lo, hi = np.minimum(a, b), np.maximum(a, b)
    n = int(max(hi.max(initial=0), 0)) + 1
    key = lo * n + hi
    uniq, inv = np.unique(key, return_inverse=True)
    draw = np.random.default_rng(seed).standard_normal((len(uniq),) + tuple(shape_tail))
    return draw[inv]


def pair_index(senders, receivers):
    """Pair storage of a symmetric graph without self loops (it holds b -> a
    whenever it holds a -> b).

    Returns (stored, pair_of): ``stored`` are the indices of the edges with
    sender < receiver, in input order (one per undirected pair, so an input
    sorted by receiver stays grouped by receiver); ``pair_of[e]`` is the
    position among them of directed edge e's pair.  Raises ValueError if an
    edge's reverse is missing or an edge is a self loop.
    """
    a = np.asarray(senders, dtype=np.int64)
    b = np.asarray(receivers, dtype=np.int64)
    stored = np.flatnonzero(a < b)
    n = int(max(a.max(initial=-1), b.max(initial=-1))) + 1
    key_stored = a[stored] * n + b[stored]
    key_all = np.minimum(a, b) * n + np.maximum(a, b)
    order = np.argsort(key_stored, kind="stable")
    pos = np.searchsorted(key_stored[order], key_all)
    pos = np.minimum(pos, max(len(order) - 1, 0))
    pair_of = order[pos] if len(order) else np.zeros(len(a), np.int64)
    if len(a) and (len(order) == 0 or not np.array_equal(key_stored[pair_of], key_all)
                   or np.any(a == b) or 2 * len(stored) != len(a)):
        raise ValueError("not a symmetric graph without self loops")
    return stored, pair_of


def edge_vectors(pos, senders, receivers):
    """Receiver minus sender position of each edge."""
    pos = np.asarray(pos, dtype=np.float64)
    return pos[np.asarray(receivers)] - pos[np.asarray(senders)]


def make_tangents(inp):
    """Seeded N(0,1) arrays shaped like x, y, s, in the workload's storage type."""
    w = inp.workload
    draw = normal_bf16 if w.dtype == "bf16" else normal_f32
    return tuple(draw(w.idx, tid, a.shape) for tid, a in ((T_DX, inp.x), (T_DY, inp.y), (T_DS, inp.s)))
