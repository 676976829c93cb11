"""Video-block sparse attention (oracle side).

[Summary] Inference: after the first two denoising steps only a quarter of
the video blocks are retained.  The pages leave the selection open; the
reading followed (the same one the library states at its boundary):

  * blocks are 64-key tiles; a video block is a key tile whose keys are all
    video tokens; tiles holding any head, tail or padding key are always
    kept;
  * per (head h, query-tile pair u) -- queries 256 u .. 256 u + 255 -- the
    candidates are the video tiles that some query of u can see at all, and
    the ceil(P% of them) with the highest block score are kept;
  * block score, in float32 with every product and add rounded on its own:
        qsum[d] = sum over rows r = 0..255 of Q[256 u + r, h, d],
        ksum[d] = sum over rows r = 0..63 of K[64 t + r, h, d],
        s       = sum over d = 0..127 of qsum[d] * ksum[d], ascending d,
    where a row sum is taken in groups of 16 consecutive rows -- each group
    added in ascending row order, then the group sums in ascending group
    order, every sum starting from +0.0 -- and rows past the end enter as
    +0.0;
  * ties go to the lower tile index.

The selection is a decision taken in floating point, so it is stated in the
precision the device takes it in (fp32) and in a fixed order of operations.
The attention itself is then the plain masked softmax of attention.forward
with the dropped tiles hidden (tile_keep).
"""
from __future__ import annotations

import numpy as np

from .tiles import tile_classes
from .tokens import V, TokenAttrs

BQ_PAIR, BK = 256, 64


def video_tiles(tk: TokenAttrs, bk: int = BK) -> np.ndarray:
    """bool per key tile: every key in it is a video token."""
    nk = len(tk)
    nkt = -(-nk // bk)
    out = np.zeros(nkt, bool)
    for t in range(nkt):
        out[t] = bool((tk.kind[t * bk:(t + 1) * bk] == V).all())
    return out


GROUP = 16


def _f32_block_sums(x: np.ndarray, rows: int) -> np.ndarray:
    """x [n, H, D] -> float32 [ceil(n / rows), H, D]: the sum of each block of
    `rows` consecutive rows in the stated order -- groups of GROUP rows, each
    added in ascending row order, then the group sums in ascending order,
    every sum from +0.0 with one rounding per add; rows past the end enter
    as +0.0."""
    n = x.shape[0]
    nb = -(-n // rows)
    xp = np.zeros((nb * rows,) + x.shape[1:], np.float32)
    xp[:n] = np.asarray(x, np.float32)
    xp = xp.reshape((nb, rows // GROUP, GROUP) + x.shape[1:])
    part = np.zeros((nb, rows // GROUP) + x.shape[1:], np.float32)
    for r in range(GROUP):
        part = (part + xp[:, :, r]).astype(np.float32)
    acc = np.zeros((nb,) + x.shape[1:], np.float32)
    for g in range(rows // GROUP):
        acc = (acc + part[:, g]).astype(np.float32)
    return acc


def block_scores(q, k) -> np.ndarray:
    """float32 s[h, u, t] for every head, query pair u and key tile t."""
    qsum = _f32_block_sums(q, BQ_PAIR)        # [n_pairs, H, D]
    ksum = _f32_block_sums(k, BK)             # [nkt, H, D]
    qs = np.transpose(qsum, (1, 0, 2))        # [H, n_pairs, D]
    ks = np.transpose(ksum, (1, 0, 2))        # [H, nkt, D]
    s = np.zeros((qs.shape[0], qs.shape[1], ks.shape[1]), np.float32)
    for d in range(qs.shape[2]):
        prod = (qs[:, :, None, d] * ks[:, None, :, d]).astype(np.float32)
        s = (s + prod).astype(np.float32)
    return s


def select_tiles(q, k, tq: TokenAttrs, tk: TokenAttrs, keep_percent: int, mode="R",
                 heads=None, window=0) -> np.ndarray:
    """bool keep[h, u, t]: key tile t is attended by query pair u in head h.

    Non-video tiles are always True; of each pair's candidate video tiles the
    ceil(keep_percent% of them) best-scoring ones are True.
    """
    nq, nk = len(tq), len(tk)
    n_pairs = -(-nq // BQ_PAIR)
    nkt = -(-nk // BK)
    heads = list(range(q.shape[1])) if heads is None else list(heads)
    vid = video_tiles(tk)
    cls = tile_classes(tq, tk, 128, BK, mode, window=window)
    scores = block_scores(q, k)
    keep = np.ones((q.shape[1], n_pairs, nkt), bool)
    for u in range(n_pairs):
        seen = (cls[2 * u] != 0) | ((cls[2 * u + 1] != 0) if 2 * u + 1 < cls.shape[0] else False)
        cand = [t for t in range(nkt) if seen[t] and vid[t]]
        n_keep = -(-len(cand) * keep_percent // 100)
        for h in heads:
            keep[h, u, vid] = False
            order = sorted(cand, key=lambda t: (-float(scores[h, u, t]), t))
            keep[h, u, order[:n_keep]] = True
    return keep
