"""Pins of the oracle's video-block selection (sparse forward).

The block score is stated in fp32 with a fixed order of operations; these
tests pin it to cases whose arithmetic is exact and whose ranking can be read
off by hand, to the always-kept rule for text tiles, and to the dense result
when every block is kept."""
import numpy as np
import pytest

import oracle
from oracle import sparse
from segment_causal_masked_amd import workloads as wl
from test_oracle_mask import random_tiny_layout


def one_segment(frames=4):
    """256 video queries (4 frames x 64 tokens): one query pair, 4 video key tiles."""
    return [wl.Segment(0, 0, frames, 64, 0, [])]


def tile_scaled(cs, heads=1, dim=0):
    """Q rows all e_dim; the rows of key tile t all c_t e_dim (exact in fp32)."""
    segs = one_segment(len(cs))
    n = 64 * len(cs)
    q = np.zeros((n, heads, 128))
    q[:, :, dim] = 1.0
    k = np.zeros((n, heads, 128))
    for t, c in enumerate(cs):
        k[64 * t:64 * (t + 1), :, dim] = c
    return segs, q, k


@pytest.mark.parametrize("keep,want", [(25, [2]), (50, [0, 2]), (75, [0, 2, 3]), (100, [0, 1, 2, 3])])
def test_integer_scores_rank_by_hand(keep, want):
    # scores 256 * 64 * c_t, exact: c = 3, 1, 4, 2 ranks tiles 2, 0, 3, 1
    segs, q, k = tile_scaled([3.0, 1.0, 4.0, 2.0])
    t = oracle.expand(segs)
    np.testing.assert_array_equal(sparse.block_scores(q, k)[0, 0], [49152, 16384, 65536, 32768])
    kept = sparse.select_tiles(q, k, t, t, keep)
    assert sorted(np.flatnonzero(kept[0, 0])) == want


def test_ties_go_to_the_lower_tile():
    segs, q, k = tile_scaled([2.0, 2.0, 1.0, 1.0])
    t = oracle.expand(segs)
    assert list(np.flatnonzero(sparse.select_tiles(q, k, t, t, 25)[0, 0])) == [0]
    assert list(np.flatnonzero(sparse.select_tiles(q, k, t, t, 75)[0, 0])) == [0, 1, 2]


def test_negative_scores_and_heads_rank_independently():
    segs, q, k = tile_scaled([-1.0, -3.0, -2.0, 0.5], heads=2)
    k[:, 1] *= -1.0     # head 1 sees the opposite order
    t = oracle.expand(segs)
    kept = sparse.select_tiles(q, k, t, t, 50)
    assert list(np.flatnonzero(kept[0, 0])) == [0, 3]
    assert list(np.flatnonzero(kept[1, 0])) == [1, 2]


def test_text_tiles_always_kept_and_counts():
    g = np.random.default_rng(31)
    for _ in range(20):
        segs = [wl.Segment(0, j, int(g.integers(1, 5)), 64, int(g.integers(0, 70)),
                           [(int(g.integers(1, 40)), 0, 1)]) for j in range(int(g.integers(1, 4)))]
        t = oracle.expand(segs)
        n = len(t)
        q = wl.randn((n, 2, 128), int(g.integers(1 << 30)))
        k = wl.randn((n, 2, 128), int(g.integers(1 << 30)))
        keep = int(g.integers(1, 100))
        kept = sparse.select_tiles(q, k, t, t, keep)
        vid = sparse.video_tiles(t)
        cls = oracle.tile_classes(t, t, 128, 64)
        for u in range(kept.shape[1]):
            seen = (cls[2 * u] != 0) | ((cls[2 * u + 1] != 0) if 2 * u + 1 < cls.shape[0] else False)
            for h in range(2):
                assert kept[h, u, ~vid].all()
                assert kept[h, u, vid & seen].sum() == -(-int((vid & seen).sum()) * keep // 100)


def test_keep_all_is_the_dense_forward():
    g = np.random.default_rng(5)
    segs = random_tiny_layout(g, n_videos=2)
    t = oracle.expand(segs)
    n = len(t)
    q, k, v = (wl.randn((n, 2, 128), 40 + i) for i in range(3))
    kept = sparse.select_tiles(q, k, t, t, 100)
    o1, l1 = oracle.forward(q, k, v, t, t, 128 ** -0.5)
    o2, l2 = oracle.forward(q, k, v, t, t, 128 ** -0.5, tile_keep=kept)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_dropped_tiles_are_hidden():
    """A query pair's output over kept tiles only equals the dense softmax
    over the same keys with the dropped ones removed from the layout's K/V
    (checked by zeroing their attention weight via a -inf copy)."""
    segs, q, k = tile_scaled([3.0, 1.0, 4.0, 2.0])
    t = oracle.expand(segs)
    v = wl.randn((q.shape[0], 1, 128), 9)
    kept = sparse.select_tiles(q, k, t, t, 50)        # tiles 0 and 2
    o, _ = oracle.forward(q, k, v, t, t, 1.0, tile_keep=kept)
    keys = np.r_[0:64, 128:192]
    o_ref, _ = oracle.forward(q, k[keys], v[keys], t, t.take(keys), 1.0)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
