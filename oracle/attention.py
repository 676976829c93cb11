"""Exact masked softmax attention and its gradient in float64 (oracle side).

Definition ([Guide] "Dağıtık Paketleme FLOP Tahmini" writes the mask as an
additive M with -inf on hidden pairs; [Summary] Theoretical Foundation gives
16 heads of 128 dims):

    S = scale * Q K^T,  S[q,k] = -inf where M[q,k] is false
    P = softmax_rows(S),  O = P V,  LSE = log sum_k exp(S[q,k])

A row with no visible key (padding) has O = 0 and LSE = -inf.

Gradient of O with respect to Q, K, V for an upstream dO (plain calculus of
the expression above):

    dV = P^T dO,  dP = dO V^T,  Dr = rowsum(dO * O),  dS = P * (dP - Dr)
    dQ = scale * dS K,  dK = scale * dS^T Q

Arrays are token-major [tokens, heads, dim] like the library's buffers; LSE is
[heads, queries].  Work is done per head on blocks of query rows so memory
stays bounded; the blocking only splits independent rows, it changes no sum.
"""
from __future__ import annotations

import numpy as np

from .mask import visible_mask
from .tokens import TokenAttrs


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def forward(q, k, v, tq: TokenAttrs, tk: TokenAttrs, scale: float, mode="R",
            rows=None, heads=None, block=512, window=0, tile_keep=None, unit_rows=None,
            tile_keys=None):
    """O [len(rows), Hs, D] and LSE [Hs, len(rows)] (natural log), fp64.

    rows: query indices to evaluate (default all); heads: head indices.
    tile_keep: optional bool [H, query units, key tiles] (sparse.select_tiles,
    with the same unit_rows and tile_keys): key tile t (keys tile_keys * t
    onward) is hidden from the queries of unit u (rows unit_rows * u onward)
    in head h where False.
    """
    if tile_keep is not None and (unit_rows is None or tile_keys is None):
        raise ValueError("tile_keep needs unit_rows and tile_keys")
    q, k, v = _f64(q), _f64(k), _f64(v)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    heads = list(range(q.shape[1])) if heads is None else list(heads)
    o = np.zeros((len(rows), len(heads), q.shape[2]))
    lse = np.full((len(heads), len(rows)), -np.inf)
    for r0 in range(0, len(rows), block):
        ridx = rows[r0:r0 + block]
        m0 = visible_mask(tq.take(ridx), tk, mode, window)
        for hi, h in enumerate(heads):
            m = m0 if tile_keep is None else \
                m0 & tile_keep[h][ridx // unit_rows][:, np.arange(k.shape[0]) // tile_keys]
            any_vis = m.any(axis=1)
            s = scale * (q[ridx, h, :] @ k[:, h, :].T)
            s = np.where(m, s, -np.inf)
            mx = np.where(any_vis, s.max(axis=1), 0.0)
            p = np.exp(s - mx[:, None])            # exp(-inf) = 0 exactly
            l = p.sum(axis=1)
            safe_l = np.where(any_vis, l, 1.0)
            o[r0:r0 + len(ridx), hi, :] = (p @ v[:, h, :]) / safe_l[:, None]
            lse[hi, r0:r0 + len(ridx)] = np.where(any_vis, mx + np.log(safe_l), -np.inf)
    return o, lse


def backward(q, k, v, d_o, tq: TokenAttrs, tk: TokenAttrs, scale: float,
             mode="R", heads=None, q_rows=None, k_rows=None, block=512, window=0):
    """dQ [len(q_rows), Hs, D], dK and dV [len(k_rows), Hs, D], fp64.

    Every query contributes to dK/dV; q_rows / k_rows only select which rows
    of dQ and dK/dV are returned (default: all).  The full row of P is formed
    for every query so the softmax normalisation is exact.
    """
    q, k, v, d_o = _f64(q), _f64(k), _f64(v), _f64(d_o)
    nq = q.shape[0]
    heads = list(range(q.shape[1])) if heads is None else list(heads)
    q_rows = np.arange(nq) if q_rows is None else np.asarray(q_rows)
    k_rows = np.arange(k.shape[0]) if k_rows is None else np.asarray(k_rows)
    want_q = np.zeros(nq, bool)
    want_q[q_rows] = True
    pos_q = np.full(nq, -1)
    pos_q[q_rows] = np.arange(len(q_rows))

    dq = np.zeros((len(q_rows), len(heads), q.shape[2]))
    dk = np.zeros((len(k_rows), len(heads), q.shape[2]))
    dv = np.zeros((len(k_rows), len(heads), q.shape[2]))
    for r0 in range(0, nq, block):
        ridx = np.arange(r0, min(nq, r0 + block))
        m = visible_mask(tq.take(ridx), tk, mode, window)
        any_vis = m.any(axis=1)
        sel = want_q[ridx]
        for hi, h in enumerate(heads):
            s = scale * (q[ridx, h, :] @ k[:, h, :].T)
            s = np.where(m, s, -np.inf)
            mx = np.where(any_vis, s.max(axis=1), 0.0)
            p = np.exp(s - mx[:, None])
            l = np.where(any_vis, p.sum(axis=1), 1.0)
            p = p / l[:, None]                       # normalised P
            o = p @ v[:, h, :]
            dob = d_o[ridx, h, :]
            dp = dob @ v[:, h, :].T
            dr = (dob * o).sum(axis=1)
            ds = p * (dp - dr[:, None])
            pk = p[:, k_rows]
            dsk = ds[:, k_rows]
            dv[:, hi, :] += pk.T @ dob
            dk[:, hi, :] += scale * (dsk.T @ q[ridx, h, :])
            if sel.any():
                dq[pos_q[ridx[sel]], hi, :] = scale * (ds[sel] @ k[:, h, :])
    return dq, dk, dv
