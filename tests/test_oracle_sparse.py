"""Pins of the oracle's video-block selection (sparse forward).

The block score is the exact dot product of a query unit's sum and a key
tile's sum; these tests pin it to hand-ranked cases with exact integer
scores, to its equality with the sum of all the unit's logits over the tile
(a different expression of the same quantity), to the candidate rule (tiles
no query of the unit sees do not count), to the always-kept rule for tiles
holding text or padding keys (video_tiles on hand-built layouts with head,
tail, padding and segment-straddling tiles), and to the dense result when
every block is kept."""
import numpy as np
import pytest

import oracle
from oracle import sparse
from segment_causal_masked_amd import workloads as wl
from test_oracle_mask import random_tiny_layout

UNIT, TILE = 256, 64


def one_segment(frames=4):
    """256 video queries (4 frames x 64 tokens): one query unit, 4 video key tiles."""
    return [wl.Segment(0, 0, frames, 64, 0, [])]


def tile_scaled(cs, heads=1, dim=0):
    """Q rows all e_dim; the rows of key tile t all c_t e_dim (exact)."""
    segs = one_segment(len(cs))
    n = 64 * len(cs)
    q = np.zeros((n, heads, 128))
    q[:, :, dim] = 1.0
    k = np.zeros((n, heads, 128))
    for t, c in enumerate(cs):
        k[64 * t:64 * (t + 1), :, dim] = c
    return segs, q, k


def select(q, k, t, keep, **kw):
    return sparse.select_tiles(q, k, t, t, keep, unit_rows=UNIT, tile_keys=TILE, **kw)


@pytest.mark.parametrize("keep,want", [(25, [2]), (50, [0, 2]), (75, [0, 2, 3]), (100, [0, 1, 2, 3])])
def test_integer_scores_rank_by_hand(keep, want):
    # scores 256 * 64 * c_t: c = 3, 1, 4, 2 ranks tiles 2, 0, 3, 1
    segs, q, k = tile_scaled([3.0, 1.0, 4.0, 2.0])
    t = oracle.expand(segs)
    np.testing.assert_array_equal(sparse.block_scores(q, k, UNIT, TILE)[0, 0],
                                  [49152, 16384, 65536, 32768])
    assert sorted(np.flatnonzero(select(q, k, t, keep)[0, 0])) == want


def test_ties_go_to_the_lower_tile():
    segs, q, k = tile_scaled([2.0, 2.0, 1.0, 1.0])
    t = oracle.expand(segs)
    assert list(np.flatnonzero(select(q, k, t, 25)[0, 0])) == [0]
    assert list(np.flatnonzero(select(q, k, t, 75)[0, 0])) == [0, 1, 2]


def test_negative_scores_and_heads_rank_independently():
    segs, q, k = tile_scaled([-1.0, -3.0, -2.0, 0.5], heads=2)
    k[:, 1] *= -1.0     # head 1 sees the opposite order
    t = oracle.expand(segs)
    kept = select(q, k, t, 50)
    assert list(np.flatnonzero(kept[0, 0])) == [0, 3]
    assert list(np.flatnonzero(kept[1, 0])) == [1, 2]


def test_score_is_the_sum_of_the_units_logits_over_the_tile():
    """s(h, u, t) = sum over q in u, k in t of Q_q . K_k, evaluated pair by
    pair in a double loop (bilinearity of the pooled score), ragged edges
    included (a short last unit and a short last tile)."""
    g = np.random.default_rng(11)
    nq, nk, unit, tile = 23, 29, 8, 6
    q = wl.round_to_bf16(g.standard_normal((nq, 2, 128), np.float32))
    k = wl.round_to_bf16(g.standard_normal((nk, 2, 128), np.float32))
    s = sparse.block_scores(q, k, unit, tile)
    assert s.shape == (2, 3, 5)
    for h in range(2):
        for u in range(3):
            for t in range(5):
                want = 0.0
                for i in range(u * unit, min(nq, (u + 1) * unit)):
                    for j in range(t * tile, min(nk, (t + 1) * tile)):
                        want += float(np.dot(q[i, h].astype(np.float64), k[j, h].astype(np.float64)))
                assert abs(s[h, u, t] - want) <= 1e-9 * (1 + abs(want)), (h, u, t)


def test_video_tiles_with_head_tail_padding_and_straddling_tiles():
    # [2 frames x 40 video | 30 head | 10 tail | 8 pad] + [3 frames x 64 video]:
    # tile 1 holds video, head, tail and padding keys; tiles 2-4 are video
    a = [wl.Segment(0, 0, 2, 40, 30, [(10, 0, 1)], n_pad=8), wl.Segment(0, 1, 3, 64, 0, [])]
    ta = oracle.expand(a)
    assert len(ta) == 320
    assert list(sparse.video_tiles(ta, 64)) == [True, False, True, True, True]
    assert list(sparse.video_tiles(ta, 32)) == [True, True, False, False] + [True] * 6
    # a tile of video keys from two segments is a video tile; the head and
    # tail of the second segment make the last (short) tile a text tile
    b = [wl.Segment(0, 0, 2, 50, 0, []), wl.Segment(0, 1, 1, 28, 4, [(2, 0, 1)])]
    tb = oracle.expand(b)
    assert len(tb) == 134
    assert list(sparse.video_tiles(tb, 64)) == [True, True, False]
    # padding alone makes a tile a text tile
    c = [wl.Segment(0, 0, 1, 64, 0, [], n_pad=64)]
    assert list(sparse.video_tiles(oracle.expand(c), 64)) == [True, False]


def test_text_tile_kept_whatever_its_score():
    """A key tile holding head tokens scores lowest but is kept; the video
    tiles are ranked among themselves."""
    segs = [wl.Segment(0, 0, 3, 64, 64, [])]            # tiles 0-2 video, tile 3 head
    t = oracle.expand(segs)
    n = len(t)
    q = np.zeros((n, 1, 128))
    q[:, 0, 0] = 1.0
    k = np.zeros((n, 1, 128))
    for tile, c in enumerate([2.0, 5.0, 1.0, -100.0]):
        k[64 * tile:64 * (tile + 1), 0, 0] = c
    kept = select(q, k, t, 34)                           # ceil(0.34 * 3) = 2 video tiles
    assert list(np.flatnonzero(kept[0, 0])) == [0, 1, 3]


def test_candidates_are_the_tiles_a_unit_sees():
    """Two segments of 256 video tokens: unit 0 (segment 0) sees tiles 0-3
    only, unit 1 sees tiles 0-7; at 50% they keep 2 and 4 video tiles."""
    segs = [wl.Segment(0, j, 4, 64, 0, []) for j in range(2)]
    t = oracle.expand(segs)
    seen = sparse.candidates(t, t, UNIT, TILE)
    assert seen.tolist() == [[True] * 4 + [False] * 4, [True] * 8]
    g = np.random.default_rng(3)
    q = wl.round_to_bf16(g.standard_normal((512, 1, 128), np.float32))
    k = wl.round_to_bf16(g.standard_normal((512, 1, 128), np.float32))
    kept = select(q, k, t, 50)
    assert int((kept[0, 0] & seen[0]).sum()) == 2 and int(kept[0, 1].sum()) == 4
    # of unit 0's own candidates the two best scores are kept
    s = sparse.block_scores(q, k, UNIT, TILE)[0, 0, :4]
    assert set(np.flatnonzero(kept[0, 0, :4])) == set(np.argsort(-s)[:2])


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
        kept = select(q, k, t, keep)
        vid = sparse.video_tiles(t, TILE)
        seen = sparse.candidates(t, t, UNIT, TILE)
        for u in range(kept.shape[1]):
            for h in range(2):
                assert kept[h, u, ~vid].all()
                assert kept[h, u, vid & seen[u]].sum() == -(-int((vid & seen[u]).sum()) * keep // 100)


def test_keep_all_is_the_dense_forward():
    g = np.random.default_rng(5)
    segs = random_tiny_layout(g, n_videos=2)
    t = oracle.expand(segs)
    n = len(t)
    q, k, v = (wl.randn((n, 2, 128), 40 + i) for i in range(3))
    kept = select(q, k, t, 100)
    o1, l1 = oracle.forward(q, k, v, t, t, 128 ** -0.5)
    o2, l2 = oracle.forward(q, k, v, t, t, 128 ** -0.5, tile_keep=kept, unit_rows=UNIT,
                            tile_keys=TILE)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_dropped_tiles_are_hidden():
    """A query unit's output over kept tiles only equals the dense softmax over
    the same keys with the dropped ones removed from the layout's K/V."""
    segs, q, k = tile_scaled([3.0, 1.0, 4.0, 2.0])
    t = oracle.expand(segs)
    v = wl.randn((q.shape[0], 1, 128), 9)
    kept = select(q, k, t, 50)        # tiles 0 and 2
    o, _ = oracle.forward(q, k, v, t, t, 1.0, tile_keep=kept, unit_rows=UNIT, tile_keys=TILE)
    keys = np.r_[0:64, 128:192]
    o_ref, _ = oracle.forward(q, k[keys], v[keys], t, t.take(keys), 1.0)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)


def test_tile_keep_requires_the_geometry():
    segs, q, k = tile_scaled([1.0, 2.0])
    t = oracle.expand(segs)
    kept = select(q, k, t, 50)
    with pytest.raises(ValueError):
        oracle.forward(q, k, q, t, t, 1.0, tile_keep=kept)
