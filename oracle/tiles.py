"""Unmasked-pair count A and the BQ x BK tile classes, from the mask (oracle).

A: [Guide] "Dağıtık Paketleme FLOP Tahmini" and [Summary] Training
Infrastructure, Eq. 6 -- A_i sums, over a sample's queries p, the number of
keys q with M[p,q] != -inf, i.e. the number of unmasked query-key pairs.  The
effective attention FLOP count of a call is 4 * D * heads * A (QK^T and PV
over unmasked pairs only).

Tile class of the tile (query rows [i*BQ, (i+1)*BQ) x key columns
[j*BK, (j+1)*BK)), clipped to the real rows and columns:
    EMPTY   no visible pair,
    FULL    every in-range pair visible,
    PARTIAL anything else.
"""
from __future__ import annotations

import numpy as np

from .mask import visible_mask
from .tokens import TokenAttrs

EMPTY, FULL, PARTIAL = 0, 1, 2


def unmasked_pairs(tq: TokenAttrs, tk: TokenAttrs, mode="R", block=256, window=0) -> int:
    total = 0
    for r0 in range(0, len(tq), block):
        total += int(visible_mask(tq.take(np.arange(r0, min(len(tq), r0 + block))),
                                  tk, mode, window).sum())
    return total


def tile_classes(tq: TokenAttrs, tk: TokenAttrs, bq: int, bk: int, mode="R",
                 q_tiles=None, window=0) -> np.ndarray:
    """uint8 [n_q_tiles (or len(q_tiles)), n_k_tiles] of EMPTY/FULL/PARTIAL."""
    nq, nk = len(tq), len(tk)
    nqt = -(-nq // bq)
    nkt = -(-nk // bk)
    q_tiles = range(nqt) if q_tiles is None else q_tiles
    out = []
    col_tile = np.arange(nk) // bk
    col_area = np.bincount(col_tile, minlength=nkt)
    for i in q_tiles:
        r = np.arange(i * bq, min(nq, (i + 1) * bq))
        m = visible_mask(tq.take(r), tk, mode, window)
        counts = np.add.reduceat(m.sum(axis=0), np.arange(0, nk, bk)) if nk else np.zeros(0, int)
        area = col_area * len(r)
        cls = np.full(nkt, PARTIAL, np.uint8)
        cls[counts == 0] = EMPTY
        cls[counts == area] = FULL
        out.append(cls)
    return np.stack(out) if out else np.zeros((0, nkt), np.uint8)
