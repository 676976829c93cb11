"""Expand segment records into per-token attributes (oracle side).

[Summary] Model Architecture, Action-Aware Causal Attention: a segment's text
is a descriptive head plus action tails a_0..a_n, each tail carrying a
temporal window.  [Summary] Theoretical Foundation, Eq. 1: video tokens live
on a latent grid of F_z frames x (H_z * W_z) positions.

Token order inside a segment (the pages do not fix it; any order gives the
same attention because visibility depends on attributes only):
    video tokens frame by frame, then the head, then a_0, a_1, ..., then pad.

A segment record is any object with the attributes
    video, index, n_frames, tokens_per_frame, n_head, actions, n_pad
where actions is a sequence of (n_tokens, frame_lo, frame_hi), window
half-open in latent frames.
"""
from __future__ import annotations

import dataclasses

import numpy as np

V, H, A, PAD = 0, 1, 2, 3


@dataclasses.dataclass
class TokenAttrs:
    video: np.ndarray     # int64 [n]
    seg: np.ndarray       # int64 [n] segment index within its video
    kind: np.ndarray      # int8  [n] V / H / A / PAD
    frame: np.ndarray     # int64 [n] latent frame (video tokens), else -1
    act: np.ndarray       # int64 [n] action number (tail tokens), else -1
    win_lo: np.ndarray    # int64 [n] window of the tail's action, else 0
    win_hi: np.ndarray    # int64 [n] (half-open), else 0

    def __len__(self):
        return int(self.kind.shape[0])

    def take(self, idx) -> "TokenAttrs":
        return TokenAttrs(*(getattr(self, f.name)[idx]
                            for f in dataclasses.fields(self)))


def expand(segments) -> TokenAttrs:
    cols = {k: [] for k in ("video", "seg", "kind", "frame", "act", "win_lo", "win_hi")}

    def push(n, video, seg, kind, frame, act, lo, hi):
        cols["video"].append(np.full(n, video, np.int64))
        cols["seg"].append(np.full(n, seg, np.int64))
        cols["kind"].append(np.full(n, kind, np.int8))
        cols["frame"].append(np.asarray(frame, np.int64) if np.ndim(frame)
                             else np.full(n, frame, np.int64))
        cols["act"].append(np.full(n, act, np.int64))
        cols["win_lo"].append(np.full(n, lo, np.int64))
        cols["win_hi"].append(np.full(n, hi, np.int64))

    for s in segments:
        nv = s.n_frames * s.tokens_per_frame
        if nv:
            push(nv, s.video, s.index, V,
                 np.repeat(np.arange(s.n_frames), s.tokens_per_frame), -1, 0, 0)
        if s.n_head:
            push(s.n_head, s.video, s.index, H, -1, -1, 0, 0)
        for j, (n, lo, hi) in enumerate(s.actions):
            push(n, s.video, s.index, A, -1, j, lo, hi)
        if s.n_pad:
            push(s.n_pad, s.video, s.index, PAD, -1, -1, 0, 0)
    if not cols["kind"]:
        e = np.zeros(0, np.int64)
        return TokenAttrs(e, e, e.astype(np.int8), e, e, e, e)
    return TokenAttrs(*(np.concatenate(cols[k]) for k in
                        ("video", "seg", "kind", "frame", "act", "win_lo", "win_hi")))


def latent_groups(n_pixel_frames: int) -> list:
    """[Summary] Theoretical Foundation, Eq. 1: F pixel frames compress into
    floor((F - 1) / 4) + 1 latent frames.  The grouping taken is the causal
    one that count implies: the first latent frame is pixel frame 0 alone,
    every later one the next four pixel frames; a trailing incomplete group
    is dropped.  Returns the list of pixel-frame lists, one per latent frame."""
    groups = [[0]] if n_pixel_frames >= 1 else []
    t = 1
    while t + 4 <= n_pixel_frames:
        groups.append(list(range(t, t + 4)))
        t += 4
    return groups


def action_latent_window(first: int, end: int, n_pixel_frames: int):
    """Latent window [lo, hi) of an action over pixel frames [first, end):
    the latent frames holding any of its frames (lo == hi, at the number of
    latent frames, when none does)."""
    groups = latent_groups(n_pixel_frames)
    hit = [i for i, g in enumerate(groups) if any(first <= t < end for t in g)]
    if not hit:
        return len(groups), len(groups)
    return min(hit), max(hit) + 1
