"""CPU tests of libe3conv.so: exports, host CG tables and paths vs the oracle, errors.

No compute is launched here (no GPU in CPU CI): plans, coefficient export,
host-side graph validation and argument checking run on the host only.
"""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from oracle import conv, so3
from equivariant_gnn_message_amd import e3conv as E
from equivariant_gnn_message_amd import synth

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "e3conv.h")


@pytest.fixture(scope="module")
def lib():
    return E.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(e3conv_[a-z_]+)\s*\(", text)))


def test_header_declares_what_binding_lists():
    assert declared_functions() == sorted(E.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", E.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (e3conv_\w+)", out))
    assert set(declared_functions()) <= exported


def test_status_strings(lib):
    for code in range(9):
        assert E.e3conv_status_string(code) not in ("", "unknown status")
    assert E.e3conv_status_string(99) == "unknown status"


def _oracle_layout(irin, lmax, irout):
    return conv.make_layout(irin, lmax, irout)


LAYOUTS = [(w.irreps_in, w.lmax, w.irreps_out) for w in synth.WORKLOADS.values()] + [
    ("4x1o", 1, "4x1e+4x2e"),
    ("4x2e+4x0e+4x1o", 2, "4x1o+4x0e"),          # blocks not in ascending l
    ("2x0o+2x1e+2x3o", 3, "2x0e+2x1o+2x2e+2x3e"),
    ("1x4e+1x5o+1x6e", 2, "1x4e+1x5o+1x6e+1x3o"),
]


@pytest.mark.parametrize("irin,lmax,irout", LAYOUTS)
def test_paths_match_oracle(irin, lmax, irout):
    p = E.Plan(irin, lmax, irout)
    lay = _oracle_layout(irin, lmax, irout)
    got = [(d["l1"], d["p1"], d["l2"], d["l3"], d["p3"], d["o1"], d["o2"], d["o3"]) for d in p.paths()]
    want = [(q.l1, q.p1, q.l2, q.l3, q.p3, q.o1, q.o2, q.o3) for q in lay.paths]
    assert got == want
    assert (p.channels, p.num_x, p.num_y, p.num_paths, p.num_out) == (
        lay.channels, lay.num_x, lay.num_y, lay.num_paths, lay.num_out)


@pytest.mark.parametrize("irin,lmax,irout", LAYOUTS)
def test_coefficients_match_oracle_cg(irin, lmax, irout):
    """The C++ Racah/real-basis tables equal the oracle's to 1e-12 (sparse export)."""
    p = E.Plan(irin, lmax, irout)
    lay = _oracle_layout(irin, lmax, irout)
    ix, iy, ip, io, val = p.coefficients()
    dense = np.zeros((lay.num_paths, lay.num_x, lay.num_y, lay.num_out))
    dense[ip, ix, iy, io] = val
    want = np.zeros_like(dense)
    for k, q in enumerate(lay.paths):
        C = so3.real_cg(q.l1, q.l2, q.l3)
        want[k, q.o1:q.o1 + 2 * q.l1 + 1, q.o2:q.o2 + 2 * q.l2 + 1, q.o3:q.o3 + 2 * q.l3 + 1] = C
    np.testing.assert_allclose(dense, want, atol=1e-12, rtol=0)
    assert len(val) == int(np.count_nonzero(want))


def test_all_cg_tables_to_l6_match_oracle():
    """Every real CG with l1, l2 <= 6, l3 <= 6, through single-path plans."""
    for l1 in range(7):
        for l2 in range(7):
            for l3 in range(abs(l1 - l2), min(l1 + l2, 6) + 1):
                p3 = "e" if l2 % 2 == 0 else "o"     # x block is even; y block has parity (-1)^l2
                # lmax = l2 also enumerates l2' < l2; keep only the (l1, l2, l3) path
                plan = E.Plan(f"1x{l1}e", l2, f"1x{l3}{p3}")
                ix, iy, ip, io, val = plan.coefficients()
                paths = plan.paths()
                k = [i for i, d in enumerate(paths) if d["l2"] == l2][0]
                D = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
                for a, b, c, d, v in zip(ix, iy, ip, io, val):
                    if c == k:
                        D[a, b - l2 * l2, d] = v
                np.testing.assert_allclose(D, so3.real_cg(l1, l2, l3), atol=1e-12, rtol=0)


def test_workload_layouts_have_kernels():
    for w in synth.WORKLOADS.values():
        p = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
        f32, bf16, bwd = p.supported()
        assert f32 and bf16 and bwd, w.name
        assert p.num_paths == w.num_paths


def test_layout_without_kernel_is_a_valid_plan():
    p = E.Plan("4x2e+4x0e+4x1o", 2, "4x1o+4x0e")
    assert p.supported() == (False, False, False)
    fake = ctypes.c_void_p(0x1000)    # never dereferenced: the call fails before any launch
    st = E.load_library().e3conv_forward(p.handle, 0, fake, fake, fake, fake, fake, None, 4, 4, fake, None)
    assert st == 3  # E3CONV_ERR_UNSUPPORTED


@pytest.mark.parametrize("args,code", [
    (("8x0e+8x1q", 2, "8x0e"), 2),            # parse error
    (("8x0e+(8x1o", 2, "8x0e"), 2),
    (("", 2, "8x0e"), 2),
    (("8x0e+4x1o", 2, "8x0e"), 1),            # mixed multiplicity
    (("8x0e+8x0e", 2, "8x0e"), 1),            # duplicate irreps
    (("8x0e", 1, "8x1e"), 4),                 # output reached by no path
    (("8x0e", 7, "8x0e"), 1),                 # sh_lmax out of range
    (("8x0e", -1, "8x0e"), 1),
    (("8x7e", 0, "8x7e"), 3),                 # l > 6
])
def test_plan_errors(args, code):
    with pytest.raises(E.E3ConvError) as ei:
        E.e3conv_plan(*args)
    assert ei.value.status == code
    assert ei.value.detail


def test_plan_rejects_bad_average_and_null(lib):
    h = ctypes.c_void_p()
    assert lib.e3conv_plan(b"8x0e", 0, b"8x0e", 0.0, ctypes.byref(h)) == 1
    assert lib.e3conv_plan(b"8x0e", 0, b"8x0e", float("nan"), ctypes.byref(h)) == 1
    assert lib.e3conv_plan(None, 0, b"8x0e", 1.0, ctypes.byref(h)) == 1
    assert lib.e3conv_plan(b"8x0e", 0, b"8x0e", 1.0, None) == 1


def test_forward_backward_argument_errors(lib):
    w = synth.WORKLOADS[2]
    p = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    f = ctypes.c_void_p(0x1000)
    n = ctypes.c_void_p(0)
    h = p.handle
    assert lib.e3conv_forward(None, 0, f, f, f, f, f, None, 4, 4, f, None) == 1
    assert lib.e3conv_forward(h, 5, f, f, f, f, f, None, 4, 4, f, None) == 1       # bad dtype
    assert lib.e3conv_forward(h, 0, f, f, f, f, f, None, -1, 4, f, None) == 1      # negative size
    assert lib.e3conv_forward(h, 0, f, f, f, f, f, None, 4, -4, f, None) == 1
    assert lib.e3conv_forward(h, 0, f, f, f, f, f, None, 4, 1 << 31, f, None) == 1
    assert lib.e3conv_forward(h, 0, n, f, f, f, f, None, 4, 4, f, None) == 1       # null x
    assert lib.e3conv_forward(h, 0, f, f, f, f, n, None, 4, 4, f, None) == 1       # null row_ptr
    assert lib.e3conv_forward(h, 0, n, n, n, n, n, None, 0, 0, n, None) == 0       # num_nodes = 0: no-op
    assert lib.e3conv_backward(h, 1, f, f, f, f, f, None, 4, 4, f, f, f, f, n, 0, None) == 3   # bf16 reverse
    assert lib.e3conv_backward(h, 0, f, f, f, f, f, None, 4, 4, f, n, f, f, n, 0, None) == 1   # partial outputs
    assert lib.e3conv_backward(h, 0, f, f, f, f, f, None, 4, 4, f, n, n, n, n, 0, None) == 0   # nothing to do
    # general reverse pass: unknown flag bits, mask count out of range, bf16, nothing to do
    assert lib.e3conv_backward_ex(h, 0, f, f, f, f, f, None, 4, 4, 4, f, f, f, f, 8, n, 0, None) == 1
    assert lib.e3conv_backward_ex(h, 0, f, f, f, f, f, None, 4, 4, 5, f, f, f, f, 0, n, 0, None) == 1
    assert lib.e3conv_backward_ex(h, 0, f, f, f, f, f, None, 4, 4, -1, f, f, f, f, 0, n, 0, None) == 1
    assert lib.e3conv_backward_ex(h, 1, f, f, f, f, f, None, 4, 4, 4, f, f, f, f, 0, n, 0, None) == 3
    assert lib.e3conv_backward_ex(h, 0, f, f, f, f, f, None, 4, 4, 4, f, n, n, n, 7, n, 0, None) == 0
    assert lib.e3conv_backward_ex(h, 0, f, f, f, f, n, None, 4, 4, 4, f, n, f, n, 0, n, 0, None) == 1
    # masked forward and forward-mode: count out of range, null tangent, bad dtype
    assert lib.e3conv_forward_masked(h, 0, f, f, f, f, f, None, 4, 4, 5, f, None) == 1
    assert lib.e3conv_forward_masked(h, 0, f, f, f, f, f, None, 4, 4, -1, f, None) == 1
    assert lib.e3conv_jvp(h, 0, f, f, f, f, n, f, f, f, None, 4, 4, 4, f, f, None) == 1
    assert lib.e3conv_jvp(h, 0, f, f, f, f, f, f, f, f, None, 4, 4, 4, f, n, None) == 1
    assert lib.e3conv_jvp(h, 2, f, f, f, f, f, f, f, f, None, 4, 4, 4, f, f, None) == 1
    assert lib.e3conv_jvp(h, 0, f, f, f, f, f, f, f, f, None, 4, 4, 9, f, f, None) == 1
    sz = ctypes.c_size_t(123)
    assert lib.e3conv_backward_workspace_size(h, 10, 10, ctypes.byref(sz)) == 0 and sz.value == 0
    assert lib.e3conv_csr_from_receivers(f, -1, 4, f, None) == 1
    assert lib.e3conv_csr_from_receivers(n, 4, 4, f, None) == 1


def test_variants(lib):
    w = synth.WORKLOADS[3]
    p = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    nf, nb = p.num_variants(E.E3CONV_BF16)
    assert nf >= 1 and nb == 0
    p.set_variant(nf - 1, 0)
    with pytest.raises(E.E3ConvError):
        p.set_variant(99, 0)


def test_validate_graph_host():
    src = np.array([1, 2, 0, 1], np.int32)
    E.e3conv_validate_graph(src, np.array([0, 1, 3, 4], np.int32), 3, 4)
    for bad_src, bad_ptr in [
        (src, np.array([0, 3, 1, 4], np.int32)),       # decreasing
        (src, np.array([1, 1, 3, 4], np.int32)),       # row_ptr[0] != 0
        (src, np.array([0, 1, 3, 3], np.int32)),       # row_ptr[N] != E
        (np.array([1, 2, 3, 1], np.int32), np.array([0, 1, 3, 4], np.int32)),   # sender out of range
        (np.array([1, -1, 0, 1], np.int32), np.array([0, 1, 3, 4], np.int32)),
    ]:
        with pytest.raises(E.E3ConvError) as ei:
            E.e3conv_validate_graph(bad_src, bad_ptr, 3, 4)
        assert ei.value.status == 5


def test_validate_graph_workload_csr():
    inp = synth.make_inputs(1)
    row_ptr = np.searchsorted(inp.receivers, np.arange(inp.num_nodes + 1)).astype(np.int32)
    E.e3conv_validate_graph(inp.senders, row_ptr, inp.num_nodes, inp.num_edges)


def test_receiver_order_is_a_permutation():
    for idx, n in ((1, None), (2, 1500)):
        inp = synth.make_inputs(idx, num_nodes=n) if n else synth.make_inputs(idx)
        row_ptr = np.searchsorted(inp.receivers, np.arange(inp.num_nodes + 1)).astype(np.int32)
        for cluster in (1, 64, 512, 10 ** 6):
            order = E.e3conv_receiver_order(row_ptr, inp.senders, inp.num_nodes, inp.num_edges, cluster)
            np.testing.assert_array_equal(np.sort(order), np.arange(inp.num_nodes))
    with pytest.raises(E.E3ConvError) as ei:
        E.e3conv_receiver_order(np.array([0, 2, 1], np.int32), np.array([0, 1], np.int32), 2, 2, 8)
    assert ei.value.status == 5
    with pytest.raises(E.E3ConvError) as ei:
        E.e3conv_receiver_order(np.array([0, 1], np.int32), np.array([0], np.int32), 1, 1, 0)
    assert ei.value.status == 1


def test_receiver_order_clusters_are_connected():
    """Each cluster of the order is grown breadth-first: a member after the seed has an
    in-neighbour earlier in the same cluster (when the graph is connected there)."""
    inp = synth.make_inputs(2, num_nodes=1500)
    row_ptr = np.searchsorted(inp.receivers, np.arange(inp.num_nodes + 1)).astype(np.int32)
    cluster = 64
    order = E.e3conv_receiver_order(row_ptr, inp.senders, inp.num_nodes, inp.num_edges, cluster)
    pos = np.empty_like(order)
    pos[order] = np.arange(len(order))
    first = order[:cluster]
    for v in first[1:]:
        nbrs = inp.senders[row_ptr[v]:row_ptr[v + 1]]
        assert np.any(pos[nbrs] < pos[v])    # the radius graph is symmetric


@pytest.mark.parametrize("cluster", [1, 64, 512])
def test_relabel_nodes(cluster):
    """Node ids renamed to their rank in the receiver order; the relabeled edges are the
    same directed edges, sorted by new receiver then new sender; and the oracle's
    output of the relabeled graph is the relabeled output (the sum does not see ids)."""
    from oracle import conv
    inp = synth.make_inputs(0)
    N, Ec = inp.num_nodes, inp.num_edges
    row_ptr = np.searchsorted(inp.receivers, np.arange(N + 1)).astype(np.int32)
    node_new, edge_perm = E.e3conv_relabel_nodes(row_ptr, inp.senders, N, Ec, cluster)
    order = E.e3conv_receiver_order(row_ptr, inp.senders, N, Ec, cluster)
    assert np.array_equal(node_new[order], np.arange(N))
    assert np.array_equal(np.sort(edge_perm), np.arange(Ec))
    s2, d2 = node_new[inp.senders[edge_perm]], node_new[inp.receivers[edge_perm]]
    key = d2.astype(np.int64) * N + s2
    assert np.all(np.diff(key) >= 0)
    old = np.sort(node_new[inp.receivers].astype(np.int64) * N + node_new[inp.senders])
    assert np.array_equal(np.sort(key), old)
    w = inp.workload
    lay = conv.make_layout(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    x, y, s = inp.as_f32("x"), inp.as_f32("y"), inp.as_f32("s")
    ref = conv.forward(lay, x, y, s, inp.senders, inp.receivers, N)
    x2 = np.empty_like(x)
    x2[node_new] = x
    got = conv.forward(lay, x2, y[edge_perm], s[edge_perm], s2, d2, N)
    np.testing.assert_allclose(got[node_new], ref, rtol=1e-12, atol=1e-12)


def test_relabel_nodes_edge_cases():
    node_new, edge_perm = E.e3conv_relabel_nodes(np.zeros(4, np.int32), np.zeros(0, np.int32), 3, 0, 8)
    assert np.array_equal(np.sort(node_new), np.arange(3)) and len(edge_perm) == 0
    with pytest.raises(E.E3ConvError) as ei:
        E.e3conv_relabel_nodes(np.array([0, 2, 1], np.int32), np.array([0, 1], np.int32), 2, 2, 8)
    assert ei.value.status == 5
    with pytest.raises(E.E3ConvError) as ei:
        E.e3conv_relabel_nodes(np.array([0, 1], np.int32), np.array([0], np.int32), 1, 1, 0)
    assert ei.value.status == 1
    with pytest.raises(E.E3ConvError) as ei:
        E.e3conv_relabel_nodes(np.array([0, 1], np.int32), np.array([3], np.int32), 1, 1, 8)
    assert ei.value.status == 5


def test_ordered_plans(lib):
    w = synth.WORKLOADS[2]
    h = ctypes.c_void_p()
    args = (w.irreps_in.encode(), w.lmax, w.irreps_out.encode(), w.avg_num_neighbors)
    assert lib.e3conv_plan_ordered(*args, 2, ctypes.byref(h)) == 1          # unknown ordering
    assert lib.e3conv_plan_ordered(*args, -1, ctypes.byref(h)) == 1
    for ordering in (E.E3CONV_RECEIVER, E.E3CONV_SENDER):
        p = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors, ordering=ordering)
        assert p.ordering == ordering
        assert p.supported() == (True, True, True)
        nf, nb = p.num_variants(E.E3CONV_F32)
        assert nf >= 1 and nb >= 1
    plain = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    assert plain.ordering == E.E3CONV_RECEIVER
    v = ctypes.c_int(5)
    assert lib.e3conv_plan_ordering(None, ctypes.byref(v)) == 1


def test_linear_argument_errors(lib):
    w = synth.WORKLOADS[2]
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out)
    assert plan.num_out_blocks() == 4
    f = ctypes.c_void_p(0x1000)
    h = plan.handle
    assert lib.e3conv_linear(None, 8, 1.0, f, f, 4, f, None) == 1
    assert lib.e3conv_linear(h, 0, 1.0, f, f, 4, f, None) == 1               # channels_out
    assert lib.e3conv_linear(h, 8, float("inf"), f, f, 4, f, None) == 1      # scale
    assert lib.e3conv_linear(h, 8, 1.0, None, f, 4, f, None) == 1            # weights
    assert lib.e3conv_linear(h, 8, 1.0, f, f, -1, f, None) == 1              # num_nodes
    assert lib.e3conv_linear(h, 8, 1.0, f, f, 0, f, None) == 0               # empty: no-op
    assert lib.e3conv_linear_backward(h, 8, 1.0, f, f, 4, f, None, None, None) == 0   # nothing asked
    assert lib.e3conv_linear_backward(h, 8, 1.0, f, f, 4, None, f, None, None) == 1   # grad_out


def test_radial_argument_errors(lib):
    """e3conv_forward_radial rejects bad network shapes, radii and layouts before any launch."""
    w = synth.WORKLOADS[1]
    gate = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    w2 = synth.WORKLOADS[2]
    mace = E.Plan(w2.irreps_in, w2.lmax, w2.irreps_out, w2.avg_num_neighbors)
    sender = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors, ordering=E.E3CONV_SENDER)
    f = ctypes.c_void_p(0x1000)
    call = lambda h, nb=5, hid=100, rmax=2.0, sig=0.5, N=4, Ecount=8, nr=4, x=f, w1=f: \
        lib.e3conv_forward_radial(h, x, f, f, w1, f, nb, hid, rmax, sig, f, f, None, N, Ecount, nr, f, None)
    assert call(None) == 1
    assert call(gate.handle, nb=1) == 1
    assert call(gate.handle, nb=9) == 1
    assert call(gate.handle, hid=102) == 1
    assert call(gate.handle, hid=132) == 1
    assert call(gate.handle, rmax=0.0) == 1
    assert call(gate.handle, sig=float("nan")) == 1
    assert call(gate.handle, nr=5) == 1
    assert call(gate.handle, x=None) == 1
    assert call(gate.handle, w1=None) == 1
    assert call(mace.handle) == 3        # E3CONV_ERR_UNSUPPORTED: 128 channels
    assert call(sender.handle) == 3      # RECEIVER ordering only
    assert call(gate.handle, N=0, Ecount=0, nr=0) == 0


def test_backward_pairs_argument_errors(lib):
    w = synth.WORKLOADS[2]
    p = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    ps = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors, ordering=E.E3CONV_SENDER)
    f = ctypes.c_void_p(0x1000)
    n = ctypes.c_void_p(0)
    h = p.handle
    assert lib.e3conv_backward_pairs(None, f, f, f, f, f, 4, 4, f, f, f, f, None) == 1
    assert lib.e3conv_backward_pairs(h, f, f, f, f, f, -1, 4, f, f, f, f, None) == 1    # negative size
    assert lib.e3conv_backward_pairs(h, f, f, f, f, f, 4, 1 << 31, f, f, f, f, None) == 1
    assert lib.e3conv_backward_pairs(h, f, f, f, f, n, 4, 4, f, f, f, f, None) == 1     # null dst
    assert lib.e3conv_backward_pairs(h, f, f, f, f, f, 4, 4, f, f, n, f, None) == 1     # null grad_y
    assert lib.e3conv_backward_pairs(h, f, f, f, f, f, 0, 4, f, f, f, f, None) == 1     # edges, no nodes
    assert lib.e3conv_backward_pairs(h, n, n, n, n, n, 0, 0, n, n, n, n, None) == 0     # empty: no-op
    assert lib.e3conv_backward_pairs(ps.handle, f, f, f, f, f, 4, 4, f, f, f, f, None) == 3


def _csr(src, dst, n):
    order = np.lexsort((src, dst))
    src, dst = np.asarray(src)[order], np.asarray(dst)[order]
    return np.searchsorted(dst, np.arange(n + 1)).astype(np.int32), src.astype(np.int32), dst


@pytest.mark.parametrize("cluster", [1, 16, 512])
def test_pair_layout_of_radius_graphs(cluster):
    """One stored edge per pair, both directions mapped to it, the stored edges of a
    receiver consecutive, receivers in the receiver order, each pair stored as its edge
    into the endpoint the order visits first; the pair set equals the plain selection."""
    pos = np.random.default_rng(cluster).uniform(0.0, 4.0, (300, 3))
    src, dst = synth.radius_graph(pos, 1.0)
    N, Ec = len(pos), len(src)
    row_ptr = np.searchsorted(dst, np.arange(N + 1)).astype(np.int32)
    stored, pmap = E.e3conv_pair_layout(row_ptr, src, N, Ec, cluster)
    pair_of = np.where(pmap >= 0, pmap, ~pmap)
    assert len(stored) * 2 == Ec
    assert np.array_equal(np.bincount(pair_of, minlength=len(stored)), np.full(len(stored), 2))
    assert np.array_equal(pmap[stored], np.arange(len(stored)))      # stored edges: non-negative
    assert np.count_nonzero(pmap < 0) == len(stored)                # their reverses: ~pair
    lo, hi = np.minimum(src, dst), np.maximum(src, dst)
    assert np.array_equal(lo[stored][pair_of], lo) and np.array_equal(hi[stored][pair_of], hi)
    rev = pmap < 0
    assert np.array_equal(src[rev], dst[stored][pair_of[rev]])      # a reverse runs the other way
    order = E.e3conv_receiver_order(row_ptr, src, N, Ec, cluster)
    rank = np.empty(N, np.int64)
    rank[order] = np.arange(N)
    b, a = dst[stored], src[stored]
    assert np.all(np.diff(rank[b]) >= 0)                 # receivers in order, runs consecutive
    assert np.all(rank[a] > rank[b])                     # stored into the earlier endpoint
    plain, _ = synth.pair_index(src, dst)
    key = lambda e: set(zip(lo[e].tolist(), hi[e].tolist()))
    assert key(stored) == key(plain)


def test_pair_layout_rejects_graphs_that_are_not_symmetric():
    def call(src, dst, n):
        row_ptr, s, _ = _csr(np.array(src), np.array(dst), n)
        return E.e3conv_pair_layout(row_ptr, s, n, len(s))
    call([0, 1, 1, 2], [1, 0, 2, 1], 3)                              # symmetric: accepted
    stored, pair_of = E.e3conv_pair_layout(np.zeros(1, np.int32), np.zeros(0, np.int32), 0, 0)
    assert len(stored) == 0 and len(pair_of) == 0                    # empty graph
    with pytest.raises(E.E3ConvError):
        E.e3conv_pair_layout(np.zeros(1, np.int32), np.zeros(2, np.int32), 0, 2)   # edges, no nodes
    for src, dst in (([0, 1, 2], [1, 0, 0]),                         # odd edge count
                     ([0, 1, 0, 1], [1, 0, 2, 2]),                   # reverses missing
                     ([0, 1, 1, 1], [1, 0, 1, 1]),                   # self loops
                     ([0, 0, 1, 1], [1, 1, 0, 0])):                  # repeated edges
        with pytest.raises(E.E3ConvError) as err:
            call(src, dst, 3)
        assert err.value.status == E.E3CONV_ERR_GRAPH


def test_forward_linear_argument_errors(lib):
    f = ctypes.c_void_p(0x1000)
    n = ctypes.c_void_p(0)
    w = synth.WORKLOADS[1]
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)   # kept alive: owns h
    h = plan.handle
    assert lib.e3conv_forward_linear(None, 0, f, f, f, f, f, None, 4, 4, 1.0, f, f, None) == 1
    assert lib.e3conv_forward_linear(h, 3, f, f, f, f, f, None, 4, 4, 1.0, f, f, None) == 1     # dtype
    assert lib.e3conv_forward_linear(h, 0, f, f, f, f, f, None, 4, 4, float("inf"), f, f, None) == 1
    assert lib.e3conv_forward_linear(h, 0, f, f, f, f, f, None, 4, 4, 1.0, n, f, None) == 1     # weights
    assert lib.e3conv_forward_linear(h, 0, n, n, n, n, n, None, 0, 0, 1.0, n, n, None) == 0     # no-op
    w2 = synth.WORKLOADS[2]                                                                      # 128 ch.
    plan2 = E.Plan(w2.irreps_in, w2.lmax, w2.irreps_out, w2.avg_num_neighbors)
    h2 = plan2.handle
    assert lib.e3conv_forward_linear(h2, 0, f, f, f, f, f, None, 4, 4, 1.0, f, f, None) == 3


def test_forward_pairs_argument_errors(lib):
    f = ctypes.c_void_p(0x1000)
    n = ctypes.c_void_p(0)
    w = synth.WORKLOADS[2]
    plan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors)
    splan = E.Plan(w.irreps_in, w.lmax, w.irreps_out, w.avg_num_neighbors, ordering=E.E3CONV_SENDER)
    h = plan.handle
    assert lib.e3conv_forward_pairs(None, f, f, f, f, f, f, None, 4, 4, 2, f, None) == 1
    assert lib.e3conv_forward_pairs(h, f, f, f, f, f, f, None, 4, 4, 5, f, None) == 1     # pairs > edges
    assert lib.e3conv_forward_pairs(h, f, f, f, f, f, n, None, 4, 4, 2, f, None) == 1     # null map
    assert lib.e3conv_forward_pairs(h, n, n, n, n, n, n, None, 0, 0, 0, n, None) == 0     # no-op
    assert lib.e3conv_forward_pairs(splan.handle, f, f, f, f, f, f, None, 4, 4, 2, f, None) == 3
