"""Error bounds and error models of the device arithmetic, for the GPU gates.

These are tolerances, not reference values: every expected value a GPU test
compares against comes from the oracle.  What is computed here says how far a
correct device result may lie from the oracle's exact one, given the
roundings the device performs:

  * the forward multiplies Q by scale * log2(e) in fp32 and rounds it to bf16
    (relative error at most U = 2^-8 per element) before its products, and
    accumulates in fp32;
  * the backward forms P = exp(scale * (Q K^T) - lse) from Q and K as given
    (fp32 scores) against the forward's lse, and rounds P and
    dS = P * (dP - delta) to bf16 (relative U) as MFMA operands;
  * delta = rowsum(dO * O) uses the forward's bf16 O.

LSE (a rigorous bound, natural-log units).  With Q' = bf16(Q c), c =
scale log2(e), the score of pair (q, k) moves by
    d_k = scale * sum_d eta_d q_d k_d,   |eta_d| <= U
(eta_d is the relative rounding of Q's element d, shared by all keys of the
row), and the LSE by  ln sum_k p_k exp(d_k)  with p the exact softmax row.
Jensen gives a lower bound E_p[d] and Hoeffding's lemma the upper bound
E_p[d] + (max d - min d)^2 / 8, and |E_p[d]| = |scale sum_d eta_d q_d kbar_d|
<= U scale sum_d |q_d kbar_d| with kbar = sum_k p_k k_k, so
    |dLSE| <= B1 + B2,  B1 = U scale sum_d |q_d kbar_d|,
                        B2 = (U scale max_k sum_d |q_d k_kd|)^2 / 2,
plus the fp32 terms: score accumulation (gamma_132 times twice the largest
|score|), exp2 (2^-21 relative), the row sum (gamma of a summation tree of
depth ceil(n_keys / 64) + 24: a few levels per 64-key tile, one per tile, and
the merges of split pieces) and the final log / scaling (4e-6 (1 + |lse|)).
gamma_n = n u / (1 - n u), u = 2^-24.

Gradients (an error model, standard deviations per element).  Each bf16
operand rounding is a relative error of at most U; modelled as independent
and uniform, variance U^2 / 3 (an overestimate: relative rounding errors of
values spread over binades have a smaller second moment).  P's row scale
error is the forward's LSE error, modelled by its first-order standard
deviation Bs = U / sqrt(3) scale ||q * kbar||_2 plus the bound's remaining
terms; delta's error from the forward's O is modelled as a per-element O
error of 1e-3 (the forward's mean-abs gate).  Then, with T = dS^2 (U^2/3 +
Bs^2) + P^2 var(delta):
    var dV[k,d] = sum_q P_qk^2 dO_qd^2 (U^2/3 + Bs_q^2)
    var dK[k,d] = scale^2 sum_q T_qk Q_qd^2
    var dQ[q,d] = scale^2 sum_k T_qk K_kd^2
and bf16 outputs add U^2/3 g^2 for their own rounding.  The gate on
z = |err| / sigma: mean(z) <= sqrt(2/pi) (the mean of |N(0,1)|: the model's
overestimate keeps a correct kernel below it, anything noisier than the model
fails) and max(z) <= 6.
"""
from __future__ import annotations

import numpy as np

import oracle

U_BF16 = 2.0 ** -8 * (1.0 + 2.0 ** -14)   # bf16 rounding after an fp32 product
U_F32 = 2.0 ** -24
Z_MEAN, Z_MAX = float(np.sqrt(2.0 / np.pi)), 6.0
O_ERR_STD = 1e-3


def gamma(n):
    return n * U_F32 / (1.0 - n * U_F32)


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _softmax_rows(qh, kh, m, scale):
    """Exact P (rows with no visible key: zeros), fp64."""
    s = scale * (qh @ kh.T)
    s = np.where(m, s, -np.inf)
    any_vis = m.any(axis=1)
    mx = np.where(any_vis, s.max(axis=1), 0.0)
    e = np.exp(s - mx[:, None])
    l = np.where(any_vis, e.sum(axis=1), 1.0)
    return e / l[:, None], np.where(any_vis, mx + np.log(l), 0.0), any_vis


def _row_terms(qh, kh, p, m, lse, scale, nk, u_inputs=0.0):
    """(B: rigorous LSE bound, Bs: first-order std of the LSE shift) per row.

    u_inputs > 0: the device also saw Q and K rounded (relative u_inputs per
    element) from the values the oracle used; the shifts then differ per key
    and the first-order term takes sum_d |q_d| sum_k p_k |k_kd|."""
    kbar = p @ kh
    a = np.abs(qh) @ np.abs(kh).T
    a_max = np.where(m, a, 0.0).max(axis=1) if a.shape[1] else np.zeros(len(qh))
    if u_inputs > 0:
        u = (1.0 + U_BF16) * (1.0 + u_inputs) ** 2 - 1.0
        b1 = u * scale * (np.abs(qh) * (p @ np.abs(kh))).sum(axis=1)
    else:
        u = U_BF16
        b1 = u * scale * np.abs(qh * kbar).sum(axis=1)
    e_max = u * scale * a_max
    b2 = e_max ** 2 / 2
    fp32 = (gamma(132) * 2.0 * scale * (1.0 + U_BF16) * a_max + 2.0 ** -21
            + gamma(-(-nk // 64) + 24) + 4e-6 * (1.0 + np.abs(lse)))
    bs = U_BF16 / np.sqrt(3.0) * scale * np.sqrt(((qh * kbar) ** 2).sum(axis=1)) + b2 + fp32
    return b1 + b2 + fp32, bs


def _keep_mask(tile_keep, h, ridx, nk, unit_rows, tile_keys):
    return tile_keep[h][ridx // unit_rows][:, np.arange(nk) // tile_keys]


def lse_bound(q, k, tq, tk, scale, mode="R", rows=None, heads=None, window=0, block=512,
              tile_keep=None, unit_rows=256, tile_keys=64, u_inputs=0.0):
    """Rigorous bound on |LSE_device - LSE_exact| per (head, row), natural log.
    tile_keep / unit_rows / tile_keys: as oracle.forward (sparse plans)."""
    q, k = _f64(q), _f64(k)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    heads = list(range(q.shape[1])) if heads is None else list(heads)
    out = np.zeros((len(heads), len(rows)))
    nk = k.shape[0]
    for r0 in range(0, len(rows), block):
        ridx = rows[r0:r0 + block]
        m0 = oracle.visible_mask(tq.take(ridx), tk, mode, window)
        for hi, h in enumerate(heads):
            m = m0 if tile_keep is None else m0 & _keep_mask(tile_keep, h, ridx, nk, unit_rows,
                                                             tile_keys)
            p, lse, _ = _softmax_rows(q[ridx, h], k[:, h], m, scale)
            out[hi, r0:r0 + len(ridx)] = _row_terms(q[ridx, h], k[:, h], p, m, lse, scale, nk,
                                                    u_inputs)[0]
    return out


def softmax_abs_v(q, k, v, tq, tk, scale, mode="R", rows=None, heads=None, block=512):
    """sum_k P_qk |V_kd| per (row, head, dim) with P the exact softmax rows:
    what a relative perturbation of P (at most r per element) can move O by
    is at most r times this."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    heads = list(range(q.shape[1])) if heads is None else list(heads)
    out = np.zeros((len(rows), len(heads), v.shape[2]))
    for r0 in range(0, len(rows), block):
        ridx = rows[r0:r0 + block]
        m = oracle.visible_mask(tq.take(ridx), tk, mode)
        for hi, h in enumerate(heads):
            p, _, _ = _softmax_rows(q[ridx, h], k[:, h], m, scale)
            out[r0:r0 + len(ridx), hi] = p @ np.abs(v[:, h])
    return out


def grad_sigma(q, k, v, d_o, tq, tk, scale, mode="R", heads=None, q_rows=None, k_rows=None,
               window=0, block=512):
    """Model standard deviations of the device dQ [len(q_rows), Hs, D] and
    dK, dV [len(k_rows), Hs, D] against the exact gradients (fp32 outputs)."""
    q, k, v, d_o = _f64(q), _f64(k), _f64(v), _f64(d_o)
    nq, nk = q.shape[0], k.shape[0]
    heads = list(range(q.shape[1])) if heads is None else list(heads)
    q_rows = np.arange(nq) if q_rows is None else np.asarray(q_rows)
    k_rows = np.arange(nk) if k_rows is None else np.asarray(k_rows)
    want_q = np.zeros(nq, bool)
    want_q[q_rows] = True
    pos_q = np.full(nq, -1)
    pos_q[q_rows] = np.arange(len(q_rows))
    var_q = np.zeros((len(q_rows), len(heads), q.shape[2]))
    var_k = np.zeros((len(k_rows), len(heads), q.shape[2]))
    var_v = np.zeros_like(var_k)
    u2 = U_BF16 ** 2 / 3.0
    for r0 in range(0, nq, block):
        ridx = np.arange(r0, min(nq, r0 + block))
        m = oracle.visible_mask(tq.take(ridx), tk, mode, window)
        sel = want_q[ridx]
        for hi, h in enumerate(heads):
            qh, kh, vh, doh = q[ridx, h], k[:, h], v[:, h], d_o[ridx, h]
            p, lse, _ = _softmax_rows(qh, kh, m, scale)
            _, bs = _row_terms(qh, kh, p, m, lse, scale, nk)
            o = p @ vh
            dp = doh @ vh.T
            ds = p * (dp - (doh * o).sum(axis=1)[:, None])
            vdelta = O_ERR_STD ** 2 * (doh ** 2).sum(axis=1)
            r = u2 + bs ** 2
            t = ds ** 2 * r[:, None] + p ** 2 * vdelta[:, None]
            var_v[:, hi] += (p[:, k_rows] ** 2 * r[:, None]).T @ doh ** 2
            var_k[:, hi] += scale ** 2 * (t[:, k_rows].T @ qh ** 2)
            if sel.any():
                var_q[pos_q[ridx[sel]], hi] = scale ** 2 * (t[sel] @ kh ** 2)
    return np.sqrt(var_q), np.sqrt(var_k), np.sqrt(var_v)


def grad_z(g_dev, g_ref, sigma, bf16_out):
    """z = |err| / sigma per element; bf16 outputs add their own rounding."""
    g_ref = _f64(g_ref)
    rms = float(np.sqrt(np.mean(g_ref ** 2))) if g_ref.size else 1.0
    var = sigma ** 2 + (U_BF16 ** 2 / 3.0 * g_ref ** 2 if bf16_out else 0.0) + (1e-6 * rms) ** 2
    return np.abs(_f64(g_dev) - g_ref) / np.sqrt(var)


# ---------------------------------------------------------------------------
# Video-block selection: the device's fp32 block score
# ---------------------------------------------------------------------------
#
# The device evaluates the block score s = sum_d qsum_d ksum_d of the
# selection in fp32 (sums of the bf16 rows, products, the dot over d), so its
# ranking may differ from the exact one between tiles whose scores are
# closer than the fp32 error.  Bound (standard error analysis, any
# summation order): a sum of n values in fp32 is off by at most gamma_n times
# the sum of their magnitudes, so with A_d = sum_q |Q_qd|, B_d = sum_k |K_kd|
#   |qsum_d' - qsum_d| <= eq_d = gamma_nq A_d,  |ksum_d' - ksum_d| <= ek_d = gamma_nk B_d,
#   |qsum' ksum' - qsum ksum| <= |qsum| ek + |ksum| eq + eq ek   (per d),
# and the fp32 dot adds at most gamma_128 sum_d |qsum'| |ksum'|.

def score_bound(q, k, unit_rows, tile_keys):
    """eps[h, u, t] >= |fp32 score - exact score| for every head, query unit
    and key tile (units of unit_rows queries, tiles of tile_keys keys)."""
    from oracle import sparse
    qs = sparse.block_sums(q, unit_rows)                  # [U, H, D]
    ks = sparse.block_sums(k, tile_keys)                  # [T, H, D]
    qa = sparse.block_sums(np.abs(q), unit_rows)
    ka = sparse.block_sums(np.abs(k), tile_keys)
    eq = gamma(unit_rows + 1) * qa
    ek = gamma(tile_keys + 1) * ka
    aq, ak = np.abs(qs), np.abs(ks)
    mix = (np.einsum("uhd,thd->hut", aq, ek) + np.einsum("uhd,thd->hut", eq, ak)
           + np.einsum("uhd,thd->hut", eq, ek))
    dot = gamma(128) * np.einsum("uhd,thd->hut", aq + eq, ak + ek)
    return (mix + dot) * (1.0 + 1e-12)
