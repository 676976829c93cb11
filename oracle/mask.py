"""The visibility mask M[q, k] of action-aware causal attention (oracle side).

Rules, each restated from the pages:

  (1) Segment-wise causality -- [Summary] Model Architecture, Segment-wise
      Causal Attention; [Guide] "Eyleme Duyarlı Nedensel Dikkat": a query of
      segment j sees tokens of segments 0..j and nothing later; inside a
      segment attention runs both ways.
  (2) Packing -- [Summary] Training Infrastructure; [Guide] "Dağıtık Paketleme
      FLOP Tahmini": independent videos packed into one sequence never see one
      another (block-diagonal), so (1) applies within a video only.
  (3) Heads persist -- [Summary] Action-Aware Causal Attention; [Review]
      "무엇과 다른가": a segment's descriptive head stays visible to later
      segments.  With (1), every head of segments <= j is visible.
  (4) Tails stay home -- same passages: an action tail is visible only inside
      the segment that owns it.
  (5) Windows -- same passages: a video query whose latent frame lies inside
      action a_k's window sees a_k's text; outside every window a video query
      sees no tail (it still sees the heads and all visible video).
  (6) Text queries (pages silent; see the package docstring): mode R -- a
      query of a_k sees a_k's own tokens, a head query sees no tail; mode K --
      no text query sees a tail; mode H -- head queries also see every tail of
      their own segment.
  (7) Padding is never visible and sees nothing.
  (8) Sliding window (optional) -- [Summary] Inference lists sliding-window
      attention among the single-GPU optimisations without saying over what;
      read as whole segments: with a window of W >= 1 segments a query of
      segment j sees only segments j - W + 1 .. j of its video (older heads
      included in what is dropped).  window = 0 means no window.
"""
from __future__ import annotations

import numpy as np

from .tokens import A, H, PAD, V, TokenAttrs

MODES = ("R", "K", "H")


def visible_mask(tq: TokenAttrs, tk: TokenAttrs, mode: str = "R", window: int = 0) -> np.ndarray:
    """Boolean M[q, k] for the given query and key tokens (vectorised)."""
    assert mode in MODES and window >= 0
    qv = tq.video[:, None]
    qs = tq.seg[:, None]
    kv = tk.video[None, :]
    ks = tk.seg[None, :]
    qkind = tq.kind[:, None]
    kkind = tk.kind[None, :]

    live = (qkind != PAD) & (kkind != PAD)                 # rule (7)
    earlier_or_same = (qv == kv) & (ks <= qs)              # rules (1), (2)
    if window:
        earlier_or_same &= qs - ks < window                # rule (8)
    video_or_head_key = (kkind == V) | (kkind == H)        # rule (3) + video
    same_segment = (qv == kv) & (qs == ks)                 # rule (4)

    in_window = ((qkind == V)
                 & (tk.win_lo[None, :] <= tq.frame[:, None])
                 & (tq.frame[:, None] < tk.win_hi[None, :]))  # rule (5)
    if mode == "R":
        text_q = (qkind == A) & (tq.act[:, None] == tk.act[None, :])
    elif mode == "K":
        text_q = np.zeros_like(in_window)
    else:
        text_q = ((qkind == A) & (tq.act[:, None] == tk.act[None, :])) | (qkind == H)
    tail_key = (kkind == A) & same_segment & (in_window | text_q)

    return live & earlier_or_same & (video_or_head_key | tail_key)


# ----------------------------------------------------------------------------
# independent per-pair statement of the same rules (used on tiny layouts)
# ----------------------------------------------------------------------------

def _locate(segments, t):
    """Token number t of a layout -> (segment record, role, detail).

    role: 'video' (detail = latent frame), 'head', ('tail', j), or 'pad'.
    Decoded from the record's counts directly, not from expand().
    """
    for s in segments:
        n_video = s.n_frames * s.tokens_per_frame
        if t < n_video:
            return s, "video", t // s.tokens_per_frame
        t -= n_video
        if t < s.n_head:
            return s, "head", None
        t -= s.n_head
        for j, act in enumerate(s.actions):
            if t < act[0]:
                return s, "tail", j
            t -= act[0]
        if t < s.n_pad:
            return s, "pad", None
        t -= s.n_pad
    raise IndexError("token outside layout")


def visible_pair(q_seg, q_role, q_detail, k_seg, k_role, k_detail, mode="R", window=0) -> bool:
    """One (query, key) decision written as nested cases, for brute force."""
    if q_role == "pad" or k_role == "pad":
        return False
    if q_seg.video != k_seg.video:
        return False                     # different videos of a pack
    if k_seg.index > q_seg.index:
        return False                     # future segment
    if window and q_seg.index - k_seg.index >= window:
        return False                     # outside the sliding window
    if k_role in ("video", "head"):
        return True
    # key is a tail token of action k_detail
    if k_seg.index != q_seg.index:
        return False                     # tails never leave their segment
    if q_role == "video":
        lo, hi = k_seg.actions[k_detail][1], k_seg.actions[k_detail][2]
        return lo <= q_detail < hi
    if q_role == "tail":
        return mode in ("R", "H") and q_detail == k_detail
    # q_role == "head"
    return mode == "H"


def brute_force_mask(q_segments, k_segments, mode="R", window=0) -> np.ndarray:
    """M from visible_pair over every pair: O(nq*nk) Python calls; tiny only."""
    nq = sum(s.n_frames * s.tokens_per_frame + s.n_head +
             sum(a[0] for a in s.actions) + s.n_pad for s in q_segments)
    nk = sum(s.n_frames * s.tokens_per_frame + s.n_head +
             sum(a[0] for a in s.actions) + s.n_pad for s in k_segments)
    kloc = [_locate(k_segments, j) for j in range(nk)]
    m = np.zeros((nq, nk), dtype=bool)
    for i in range(nq):
        qs, qr, qd = _locate(q_segments, i)
        for j in range(nk):
            ks, kr, kd = kloc[j]
            m[i, j] = visible_pair(qs, qr, qd, ks, kr, kd, mode, window)
    return m
