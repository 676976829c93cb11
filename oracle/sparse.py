"""Video-block sparse attention (oracle side).  TEST INFRASTRUCTURE ONLY.

[Summary] Inference: after the first two denoising steps only a quarter of
the video blocks are retained.  The pages leave the selection open; the
reading followed (the same one the library states at its boundary):

  * a block is a key tile of `tile_keys` consecutive keys; a video block is a
    tile whose keys are all video tokens; a tile holding any head, tail or
    padding key is always kept;
  * selection is made per (head h, query unit u), a unit being `unit_rows`
    consecutive queries; u's candidates are the video tiles that some query
    of u can see at all, and the ceil(P% of them) with the highest block
    score are kept;
  * block score: the dot product of the unit's query sum and the tile's key
    sum,
        s(h, u, t) = sum_d (sum_{q in u} Q[q, h, d]) * (sum_{k in t} K[k, h, d]),
    which equals the sum of all the unit's query-key logits over the tile
    (bilinearity);
  * ties go to the lower tile index.

Here the score is evaluated exactly (fp64, whose sums of bf16 values are exact
at these sizes).  The attention itself is the plain masked softmax of
attention.forward with the dropped tiles hidden (its tile_keep argument).
"""
from __future__ import annotations

import numpy as np

from .mask import visible_mask
from .tokens import V, TokenAttrs


def video_tiles(tk: TokenAttrs, tile_keys: int) -> np.ndarray:
    """bool per key tile: every key in it is a video token."""
    nk = len(tk)
    nkt = -(-nk // tile_keys)
    out = np.zeros(nkt, bool)
    for t in range(nkt):
        out[t] = bool((tk.kind[t * tile_keys:(t + 1) * tile_keys] == V).all())
    return out


def block_sums(x, rows: int) -> np.ndarray:
    """x [n, H, D] -> fp64 [ceil(n / rows), H, D]: sums of consecutive blocks
    of `rows` rows (the last block may be short)."""
    n = x.shape[0]
    nb = -(-n // rows)
    out = np.zeros((nb,) + x.shape[1:])
    for b in range(nb):
        out[b] = np.asarray(x[b * rows:(b + 1) * rows], np.float64).sum(axis=0)
    return out


def block_scores(q, k, unit_rows: int, tile_keys: int) -> np.ndarray:
    """fp64 s[h, u, t] for every head, query unit u and key tile t."""
    qs = block_sums(q, unit_rows)     # [n_units, H, D]
    ks = block_sums(k, tile_keys)     # [n_tiles, H, D]
    return np.einsum("uhd,thd->hut", qs, ks)


def candidates(tq: TokenAttrs, tk: TokenAttrs, unit_rows: int, tile_keys: int, mode="R",
               window=0) -> np.ndarray:
    """bool seen[u, t]: some query of unit u sees some key of tile t."""
    nq, nk = len(tq), len(tk)
    n_units, nkt = -(-nq // unit_rows), -(-nk // tile_keys)
    seen = np.zeros((n_units, nkt), bool)
    for u in range(n_units):
        m = visible_mask(tq.take(np.arange(u * unit_rows, min(nq, (u + 1) * unit_rows))), tk,
                         mode, window)
        cols = m.any(axis=0)
        seen[u] = np.logical_or.reduceat(cols, np.arange(0, nk, tile_keys)) if nk else seen[u]
    return seen


def select_tiles(q, k, tq: TokenAttrs, tk: TokenAttrs, keep_percent: int, unit_rows: int,
                 tile_keys: int, mode="R", heads=None, window=0) -> np.ndarray:
    """bool keep[h, u, t]: key tile t is attended by query unit u in head h.

    Tiles that are not video tiles are always True; of each unit's candidate
    video tiles the ceil(keep_percent% of them) best-scoring are True (ties:
    lower tile first); the other video tiles are False.
    """
    nq, nk = len(tq), len(tk)
    n_units, nkt = -(-nq // unit_rows), -(-nk // tile_keys)
    heads = list(range(q.shape[1])) if heads is None else list(heads)
    vid = video_tiles(tk, tile_keys)
    seen = candidates(tq, tk, unit_rows, tile_keys, mode, window)
    scores = block_scores(q, k, unit_rows, tile_keys)
    keep = np.ones((q.shape[1], n_units, nkt), bool)
    for u in range(n_units):
        cand = [t for t in range(nkt) if seen[u, t] and vid[t]]
        n_keep = -(-len(cand) * keep_percent // 100)
        for h in heads:
            keep[h, u, vid] = False
            order = sorted(cand, key=lambda t: (-scores[h, u, t], t))
            keep[h, u, order[:n_keep]] = True
    return keep
