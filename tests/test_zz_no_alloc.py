"""The allocation-free graph check (e3conv_validate_graph_noalloc) against the allocating one
(e3conv_validate_graph with on_device = 1), through the C ABI: same status and detail on valid and
invalid graphs, on two calls in a row (the second with a smaller graph), and on a side stream."""

import numpy as np
import pytest

from equivariant_gnn_message_amd import e3conv as E
from equivariant_gnn_message_amd import synth

pytestmark = pytest.mark.gpu


def _outcome(fn):
    try:
        fn()
        return (0, "")
    except E.E3ConvError as err:
        return (err.status, err.detail)


def _check_pair(src, row_ptr, n, e, stream=None):
    want = _outcome(lambda: E.e3conv_validate_graph(src, row_ptr, n, e))
    got = _outcome(lambda: E.e3conv_validate_graph_noalloc(src, row_ptr, n, e, stream=stream))
    assert got == want, (got, want)
    return got


def test_noalloc_matches_allocating_check():
    import torch
    big = synth.make_inputs(2, num_nodes=3000)
    small = synth.make_inputs(2, num_nodes=300)
    for inp in (big, small):                      # two calls, the second smaller
        src = torch.from_numpy(inp.senders).cuda()
        row_ptr = torch.from_numpy(np.searchsorted(inp.receivers, np.arange(inp.num_nodes + 1))
                                   .astype(np.int32)).cuda()
        assert _check_pair(src, row_ptr, inp.num_nodes, inp.num_edges) == (0, "")
        bad_src = src.clone()
        bad_src[inp.num_edges // 3] = inp.num_nodes       # out of range
        bad_src[inp.num_edges // 2] = -1
        status, detail = _check_pair(bad_src, row_ptr, inp.num_nodes, inp.num_edges)
        assert status == 5 and f"edge {inp.num_edges // 3}" in detail
        bad_ptr = row_ptr.clone()
        bad_ptr[inp.num_nodes // 2] = inp.num_edges + 1    # beyond num_edges and decreasing after
        status, detail = _check_pair(src, bad_ptr, inp.num_nodes, inp.num_edges)
        assert status == 5 and f"row_ptr index {inp.num_nodes // 2}" in detail
    # a valid graph after the failing ones: the shared scratch starts clean on every call
    assert _check_pair(src, row_ptr, small.num_nodes, small.num_edges) == (0, "")


def test_noalloc_on_a_side_stream():
    import torch
    inp = synth.make_inputs(2, num_nodes=500)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        src = torch.from_numpy(inp.senders).cuda()
        row_ptr = torch.from_numpy(np.searchsorted(inp.receivers, np.arange(inp.num_nodes + 1))
                                   .astype(np.int32)).cuda()
        bad = src.clone()
        bad[7] = inp.num_nodes + 5
    st.synchronize()
    assert _check_pair(src, row_ptr, inp.num_nodes, inp.num_edges, stream=st) == (0, "")
    assert _check_pair(bad, row_ptr, inp.num_nodes, inp.num_edges, stream=st)[0] == 5


def test_noalloc_rejects_bad_arguments():
    import torch
    src = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(E.E3ConvError) as ei:
        E.e3conv_validate_graph_noalloc(src, src, -1, 4)
    assert ei.value.status == 1
    with pytest.raises(E.E3ConvError) as ei:
        E.e3conv_validate_graph_noalloc(src, src, 3, 1 << 31)
    assert ei.value.status == 1
