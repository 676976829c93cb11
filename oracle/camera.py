"""Camera cross-attention in float64 (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

[Summary] Model Architecture, Camera-Trajectory Conditioning (Eq. 3): the
video tokens are the queries of a cross-attention whose keys and values are
camera tokens, and its result is added to the video tokens.  Each camera token
stands for a group of four consecutive frames ([Summary], same passage: four
4x4 relative poses flattened into one 64-dim vector; [News] "Inside the
Architecture: Dual Stream, Language Encoder, and Explicit Camera Math": the
poses are grouped over four video frames and fed to every double-stream block
through cross-attention).  Four frames are one latent frame ([Summary]
Theoretical Foundation, Eq. 1, 4x temporal compression), so a segment of F_z
latent frames has F_z camera tokens.

Readings taken where the pages are silent:
  * camera tokens: one per latent frame of each segment, in frame order; the
    camera tokens of a layout are its segments' tokens concatenated in
    segment order;
  * a video query of latent frame f in segment i sees the camera tokens
    (i, g) of its own segment with |f - g| <= radius; radius < 0 means every
    camera token of segment i (cross-attention with no stated mask), radius
    0 the time-aligned reading (its own latent frame only);
  * text and padding tokens are not queries of this attention: their output
    rows are 0 (nothing is added to them);
  * the projections of the 64-dim camera vectors to heads x 128 and of the
    output are outside: K_c, V_c come per head.

O = softmax(scale * Q K_c^T + M_c) V_c per head, rows with no visible camera
token are 0.  Parity pins: tests/test_oracle_camera.py (hand-counted
visibility, the one-key and two-key closed forms, the equal-key mean, masked
perturbations).
"""
from __future__ import annotations

import numpy as np


def camera_layout(segments):
    """Per query token: (segment number in the layout or -1 for a non-video
    token, latent frame or -1); per camera token: (segment number, frame)."""
    q_seg, q_frame, c_seg, c_frame = [], [], [], []
    for i, s in enumerate(segments):
        nv = s.n_frames * s.tokens_per_frame
        q_seg.append(np.full(nv, i, np.int64))
        q_frame.append(np.repeat(np.arange(s.n_frames, dtype=np.int64), s.tokens_per_frame))
        n_text = s.n_head + sum(int(a[0]) for a in s.actions) + getattr(s, "n_pad", 0)
        q_seg.append(np.full(n_text, -1, np.int64))
        q_frame.append(np.full(n_text, -1, np.int64))
        c_seg.append(np.full(s.n_frames, i, np.int64))
        c_frame.append(np.arange(s.n_frames, dtype=np.int64))
    cat = lambda xs: np.concatenate(xs) if xs else np.zeros(0, np.int64)  # noqa: E731
    return cat(q_seg), cat(q_frame), cat(c_seg), cat(c_frame)


def camera_mask(segments, radius: int) -> np.ndarray:
    """bool [tokens, camera tokens]: query token sees camera token."""
    q_seg, q_frame, c_seg, c_frame = camera_layout(segments)
    same = (q_seg[:, None] == c_seg[None, :]) & (q_seg[:, None] >= 0)
    if radius < 0:
        return same
    return same & (np.abs(q_frame[:, None] - c_frame[None, :]) <= radius)


def camera_forward(q, kc, vc, segments, scale: float, radius: int, rows=None, heads=None):
    """O [len(rows), Hs, D] in float64; q [tokens, H, D], kc / vc [camera, H, D]."""
    q = np.asarray(q, np.float64)
    kc = np.asarray(kc, np.float64)
    vc = np.asarray(vc, np.float64)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    heads = list(range(q.shape[1])) if heads is None else list(heads)
    m = camera_mask(segments, radius)[rows]
    any_vis = m.any(axis=1)
    o = np.zeros((len(rows), len(heads), q.shape[2]))
    for hi, h in enumerate(heads):
        s = scale * (q[rows, h, :] @ kc[:, h, :].T)
        s = np.where(m, s, -np.inf)
        mx = np.where(any_vis, s.max(axis=1, initial=-np.inf), 0.0)
        mx = np.where(np.isfinite(mx), mx, 0.0)
        p = np.exp(s - mx[:, None])
        l = p.sum(axis=1)
        o[:, hi, :] = np.where(any_vis[:, None], (p @ vc[:, h, :]) / np.where(any_vis, l, 1.0)[:, None], 0.0)
    return o
