"""Checks of the seeded input generators (CPU only)."""

import numpy as np
import pytest

from equivariant_gnn_message_amd import synth


def test_bf16_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(10000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 1e-30], np.float32)])
    ours = synth.bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = synth.bf16_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_radius_graph_brute_force():
    rng = np.random.default_rng(1)
    pos = rng.uniform(0, 3, (60, 3))
    pos[5] = pos[6]                      # coincident points are neighbours (distance 0 < r)
    pos[7] = pos[8] + np.array([2.0, 0, 0])   # exactly at r: strict boundary excludes it
    src, dst = synth.radius_graph(pos, 2.0)
    d = np.linalg.norm(pos[:, None] - pos[None], axis=-1)
    want = {(a, b) for a in range(60) for b in range(60) if a != b and d[a, b] < 2.0}
    assert set(zip(src.tolist(), dst.tolist())) == want
    assert (5, 6) in want and (7, 8) not in want
    assert np.all(np.diff(dst) >= 0)
    order = np.lexsort((src, dst))
    np.testing.assert_array_equal(order, np.arange(len(src)))


def test_radius_graph_batches_and_empty():
    pos = np.zeros((4, 3))
    src, dst = synth.radius_graph(pos, 1.0, batch=np.array([0, 0, 1, 2]))
    assert sorted(zip(src.tolist(), dst.tolist())) == [(0, 1), (1, 0)]
    src, dst = synth.radius_graph(np.zeros((1, 3)), 1.0)
    assert len(src) == 0


@pytest.mark.parametrize("idx", [0, 1])
def test_small_workloads_shapes(idx):
    inp = synth.make_inputs(idx)
    w = inp.workload
    E = inp.num_edges
    assert inp.x.shape == (inp.num_nodes, w.num_x, w.channels)
    assert inp.y.shape == (E, (w.lmax + 1) ** 2)
    assert inp.s.shape == (E, w.num_paths, w.channels)
    assert inp.senders.dtype == np.int32 and inp.receivers.dtype == np.int32
    assert np.all(np.diff(inp.receivers) >= 0)
    assert inp.senders.min() >= 0 and inp.senders.max() < inp.num_nodes
    if idx == 1:
        assert np.all(inp.senders != inp.receivers)
        deg = np.bincount(inp.receivers, minlength=inp.num_nodes)
        assert 14.0 < deg.mean() < 18.0
    # seeded: same call, same bytes
    again = synth.make_inputs(idx)
    np.testing.assert_array_equal(inp.s, again.s)
    np.testing.assert_array_equal(inp.senders, again.senders)


def test_scaled_workload3_is_bf16_and_dense():
    inp = synth.make_inputs(3, num_nodes=4000)
    assert inp.x.dtype == np.uint16 and inp.s.dtype == np.uint16 and inp.y.dtype == np.uint16
    deg = np.bincount(inp.receivers, minlength=inp.num_nodes)
    assert 25 < deg.mean() < 34
    x = inp.as_f32("x")
    assert abs(float(x.std()) - 1.0) < 0.02


def test_subgraph16():
    inp = synth.make_inputs(4, num_nodes=2000)
    nodes, eids, src, dst = synth.subgraph16(inp)
    assert len(nodes) == 16 and 0 in nodes
    assert np.all(np.diff(dst) >= 0)
    np.testing.assert_array_equal(nodes[src], inp.senders[eids])
    np.testing.assert_array_equal(nodes[dst], inp.receivers[eids])


def test_pair_index_of_a_radius_graph():
    pos = np.random.default_rng(3).uniform(0.0, 3.0, (60, 3))
    src, dst = synth.radius_graph(pos, 1.2)
    stored, pair_of = synth.pair_index(src, dst)
    assert 2 * len(stored) == len(src)
    assert np.all(src[stored] < dst[stored])
    assert np.all(np.diff(dst[stored]) >= 0)            # still grouped by receiver
    # every directed edge maps to the stored edge of its pair, both directions covered
    assert np.array_equal(np.minimum(src, dst), src[stored][pair_of])
    assert np.array_equal(np.maximum(src, dst), dst[stored][pair_of])
    assert np.array_equal(np.bincount(pair_of, minlength=len(stored)), np.full(len(stored), 2))


def test_pair_index_rejects_asymmetric_graphs():
    with pytest.raises(ValueError):
        synth.pair_index(np.array([0, 1, 2]), np.array([1, 0, 0]))
    with pytest.raises(ValueError):
        synth.pair_index(np.array([0, 1, 1]), np.array([1, 0, 1]))     # self loop
