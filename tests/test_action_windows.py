"""Action windows in latent frames (CPU): the oracle's enumeration of Eq. 1's
frame groups against the pages' count and hand-worked cases, and the
library's closed form (nomas_action_latent_window) against the oracle on
every window of segments up to 41 pixel frames."""
import pytest

import oracle.tokens as tk
import segment_causal_masked_amd as nm


@pytest.mark.parametrize("n_frames", range(1, 61))
def test_groups_match_the_latent_frame_count_of_eq1(n_frames):
    """[Summary] Theoretical Foundation, Eq. 1: F_z = floor((F - 1) / 4) + 1;
    the groups cover pixel frames 0 .. 4 (F_z - 1) once each, in order."""
    g = tk.latent_groups(n_frames)
    assert len(g) == (n_frames - 1) // 4 + 1
    flat = [t for grp in g for t in grp]
    assert flat == list(range(4 * (len(g) - 1) + 1))
    assert g[0] == [0] and all(len(grp) == 4 for grp in g[1:])


@pytest.mark.parametrize("first,end,n,want", [
    (0, 1, 17, (0, 1)),     # the first frame is a latent frame of its own
    (1, 5, 17, (1, 2)),     # frames 1-4: one latent frame
    (4, 9, 17, (1, 3)),     # straddles two groups
    (16, 17, 17, (4, 5)),   # the last complete group
    (0, 17, 17, (0, 5)),    # the whole segment
    (17, 18, 18, (5, 5)),   # only a frame of the dropped trailing group
    (16, 18, 18, (4, 5)),   # partly in it
    (0, 3, 3, (0, 1)),      # F = 3: one latent frame, frames 1-2 dropped
])
def test_hand_worked_windows(first, end, n, want):
    assert tk.action_latent_window(first, end, n) == want


def test_library_equals_oracle_on_every_window():
    nm.load()
    for n in range(1, 42):
        for first in range(n):
            for end in range(first + 1, n + 1):
                assert nm.nomas_action_latent_window(first, end, n) == \
                    tk.action_latent_window(first, end, n), (first, end, n)


@pytest.mark.parametrize("first,end,n", [(-1, 2, 9), (3, 3, 9), (4, 2, 9), (0, 10, 9), (0, 1, 0)])
def test_library_rejects_bad_spans(first, end, n):
    nm.load()
    with pytest.raises(nm.NomasError) as e:
        nm.nomas_action_latent_window(first, end, n)
    assert e.value.status == 1
