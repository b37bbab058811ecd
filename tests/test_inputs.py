"""The seeded synthetic inputs (block_sparse_taylor_amd/inputs.py): shapes and
dtypes of every workload, per-head streams (any head regenerates alone), and
the head-sharded share of the Wan2.1-14B shape equal to its first heads."""

import numpy as np
import pytest

from block_sparse_taylor_amd import inputs as I


@pytest.mark.parametrize("name", ["tiny", "flux"])
def test_shapes_and_dtypes(name):
    w = I.WORKLOADS[name]
    arrs = I.make_inputs(w, heads=[0])
    for a in arrs:
        assert a.shape == (w.batch, 1, w.seq_len, w.head_dim)
        assert a.dtype == (np.uint16 if w.dtype == "bf16" else np.float32)


def test_heads_regenerate_alone():
    w = I.WORKLOADS["flux"]
    both = I.make_inputs(w, heads=[0, 3])
    one = I.make_inputs(w, heads=[3])
    for a, b in zip(both, one):
        assert np.array_equal(a[:, 1], b[:, 0])


def test_shard_is_the_first_heads_of_the_headline_shape():
    """wan14_shard8 (5 heads: one GPU's share of 40 heads over 8 GPUs) holds
    exactly heads 0..4 of the Wan2.1-14B inputs."""
    w, s = I.WORKLOADS["wan14"], I.WORKLOADS["wan14_shard8"]
    assert s.heads == w.heads // 8 and (s.seq_len, s.head_dim, s.dtype, s.density) == (
        w.seq_len, w.head_dim, w.dtype, w.density)
    for a, b in zip(I.make_inputs(w, heads=[4]), I.make_inputs(s, heads=[4])):
        assert np.array_equal(a, b)
