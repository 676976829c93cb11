"""Pins of the camera cross-attention oracle (oracle/camera.py).

Each pin is fixed from outside the oracle's own code: visibility counted by
hand from the reading of "Summary (Overview)", Camera-Trajectory Conditioning
(one camera token per latent frame, own segment, frame radius); softmax over
one key (the value row itself); two keys (a logistic weight computed with
scalar math); identical keys (the plain mean of the visible values); and
perturbations of camera tokens a query cannot see.
"""
import math

import numpy as np
import pytest

from oracle.camera import camera_forward, camera_layout, camera_mask
from segment_causal_masked_amd.workloads import Segment, randn

SCALE = 128 ** -0.5


def hand_layout():
    # segment A: 3 latent frames x 2 tokens, a 1-token head, one 1-token
    # action tail, 1 pad; segment B (another video): 2 frames x 3 tokens
    return [Segment(0, 0, 3, 2, 1, [(1, 0, 2)], 1), Segment(1, 0, 2, 3, 0, [])]


# (token -> visible camera tokens), written out by hand: camera tokens 0..2 are
# A's frames 0..2, 3..4 are B's frames 0..1; tokens 0..5 are A's video (two
# per frame), 6..8 A's head, tail and pad, 9..14 B's video (three per frame)
HAND = {
    -1: {0: [0, 1, 2], 1: [0, 1, 2], 2: [0, 1, 2], 3: [0, 1, 2], 4: [0, 1, 2], 5: [0, 1, 2],
         9: [3, 4], 10: [3, 4], 11: [3, 4], 12: [3, 4], 13: [3, 4], 14: [3, 4]},
    0: {0: [0], 1: [0], 2: [1], 3: [1], 4: [2], 5: [2],
        9: [3], 10: [3], 11: [3], 12: [4], 13: [4], 14: [4]},
    1: {0: [0, 1], 1: [0, 1], 2: [0, 1, 2], 3: [0, 1, 2], 4: [1, 2], 5: [1, 2],
        9: [3, 4], 10: [3, 4], 11: [3, 4], 12: [3, 4], 13: [3, 4], 14: [3, 4]},
}
HAND_COUNT = {-1: 30, 0: 12, 1: 26, 2: 30}


@pytest.mark.parametrize("radius", [-1, 0, 1])
def test_hand_built_visibility(radius):
    m = camera_mask(hand_layout(), radius)
    assert m.shape == (15, 5)
    want = np.zeros((15, 5), bool)
    for t, cams in HAND[radius].items():
        want[t, cams] = True
    np.testing.assert_array_equal(m, want)


@pytest.mark.parametrize("radius", sorted(HAND_COUNT))
def test_hand_counts(radius):
    assert int(camera_mask(hand_layout(), radius).sum()) == HAND_COUNT[radius]


def test_layout_counts():
    q_seg, q_frame, c_seg, c_frame = camera_layout(hand_layout())
    assert list(q_seg) == [0] * 6 + [-1] * 3 + [1] * 6
    assert list(q_frame) == [0, 0, 1, 1, 2, 2, -1, -1, -1, 0, 0, 0, 1, 1, 1]
    assert list(c_seg) == [0, 0, 0, 1, 1] and list(c_frame) == [0, 1, 2, 0, 1]


def _inputs(n_tok, n_cam, heads=2, seed=7):
    q = randn((n_tok, heads, 128), seed)
    kc = randn((n_cam, heads, 128), seed + 1)
    vc = randn((n_cam, heads, 128), seed + 2)
    return q, kc, vc


def test_one_key_returns_its_value():
    # radius 0: a single visible key, softmax weight exactly 1
    segs = hand_layout()
    q, kc, vc = _inputs(15, 5)
    o = camera_forward(q, kc, vc, segs, SCALE, 0)
    for t, cams in HAND[0].items():
        np.testing.assert_array_equal(o[t], vc[cams[0]].astype(np.float64))


def test_two_keys_logistic_weight():
    segs = [Segment(0, 0, 2, 3, 0, [])]
    q, kc, vc = _inputs(6, 2, heads=3, seed=11)
    o = camera_forward(q, kc, vc, segs, SCALE, -1)
    for t in range(6):
        for h in range(3):
            d = SCALE * (sum(float(a) * float(b) for a, b in zip(q[t, h], kc[1, h]))
                         - sum(float(a) * float(b) for a, b in zip(q[t, h], kc[0, h])))
            w0 = 1.0 / (1.0 + math.exp(d))
            want = [w0 * float(x) + (1.0 - w0) * float(y) for x, y in zip(vc[0, h], vc[1, h])]
            np.testing.assert_allclose(o[t, h], want, rtol=0, atol=1e-12)


def test_equal_keys_give_the_mean_of_visible_values():
    segs = [Segment(0, 0, 5, 2, 2, [(3, 1, 4)])]
    q, kc, vc = _inputs(15, 5, seed=21)
    kc[:] = kc[0]
    o = camera_forward(q, kc, vc, segs, SCALE, 1)
    for f in range(5):
        g = [x for x in (f - 1, f, f + 1) if 0 <= x < 5]
        want = vc[g].astype(np.float64).mean(axis=0)
        for t in (2 * f, 2 * f + 1):
            np.testing.assert_allclose(o[t], want, rtol=0, atol=1e-12)


def test_text_and_pad_rows_are_zero():
    segs = hand_layout()
    q, kc, vc = _inputs(15, 5)
    for r in (-1, 0, 1):
        o = camera_forward(q, kc, vc, segs, SCALE, r)
        assert not o[6:9].any()
        assert o[[0, 9]].any()


def test_hidden_camera_tokens_do_not_matter():
    segs = [Segment(0, 0, 6, 3, 1, []), Segment(0, 1, 4, 2, 0, [(2, 0, 1)])]
    q, kc, vc = _inputs(18 + 1 + 8 + 2, 10, seed=31)
    o = camera_forward(q, kc, vc, segs, SCALE, 1)
    kc2, vc2 = kc.copy(), vc.copy()
    # frame 5 of segment 0 (camera 5) is hidden from frames 0..3 of segment 0;
    # segment 1's camera tokens (6..9) from all of segment 0
    kc2[5] += 3.0
    vc2[5] -= 2.0
    kc2[6:] *= -1.5
    vc2[6:] += 1.0
    o2 = camera_forward(q, kc2, vc2, segs, SCALE, 1)
    np.testing.assert_array_equal(o[:12], o2[:12])
    assert not np.array_equal(o[12:18], o2[12:18])
    assert not np.array_equal(o[19:27], o2[19:27])


def test_row_subset_and_head_subset_agree_with_full():
    segs = hand_layout()
    q, kc, vc = _inputs(15, 5, heads=3)
    full = camera_forward(q, kc, vc, segs, SCALE, 1)
    part = camera_forward(q, kc, vc, segs, SCALE, 1, rows=[3, 10, 7], heads=[2, 0])
    np.testing.assert_array_equal(part, full[[3, 10, 7]][:, [2, 0]])
