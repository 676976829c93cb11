"""CPU checks of the GPU gates in tolerance.py.

The gates say how far a correct device result may lie from the oracle.  Here
the device's roundings are replayed in numpy (bf16 rounding of Q * scale *
log2(e) in the forward, of P and dS in the backward, bf16 O and outputs; sums
in fp64, which only makes the replay more exact than the device) on small
packs, and the gates are checked to (a) hold for that replay and (b) fail for
replays with a planted mistake of the size a faulty kernel would make.  They
also bound the mismatch between the backward's P (from Q and K as given) and
the forward's lse (from the rounded Q): the rows of that P sum to
exp(-dLSE), within [exp(-B), exp(B)] for the row's LSE bound B."""
import numpy as np
import pytest

import oracle
from segment_causal_masked_amd import workloads as wl
import tolerance as tol

SCALE = 128 ** -0.5
C32 = float(np.float32(np.float32(SCALE) * np.float32(1.4426950408889634)))


def r16(x):
    return wl.round_to_bf16(np.asarray(x, np.float32)).astype(np.float64)


def round_bits(x, bits):
    """Round to `bits` significant bits, ties away (a coarser rounding)."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.round(m * 2.0 ** bits) / 2.0 ** bits, e)


def replay(q, k, v, d_o, m, lse_shift=0.0, ds_bits=None):
    """One head: (lse, dq, dk, dv) as the kernels round them (fp32 gradients)."""
    q, k, v, d_o = (np.asarray(x, np.float64) for x in (q, k, v, d_o))
    av = m.any(axis=1)
    s2 = r16(q * C32) @ k.T                       # forward scores, log2 units
    s2 = np.where(m, s2, -np.inf)
    mx = np.where(av, s2.max(axis=1), 0.0)
    e = np.exp2(s2 - mx[:, None])
    l = np.where(av, e.sum(axis=1), 1.0)
    lse2 = np.where(av, mx + np.log2(l), 0.0)
    o = r16((r16(e) @ v) / l[:, None])            # P rounded for P.V, O stored bf16
    lse = np.where(av, lse2 / np.log2(np.e), -np.inf)
    lse2b = lse2 + lse_shift / np.log(2.0)
    sb = np.where(m, (q @ k.T) * C32, -np.inf)    # backward scores: Q, K as given
    p = np.exp2(sb - lse2b[:, None])
    delta = (d_o * o).sum(axis=1)
    ds = p * (d_o @ v.T - delta[:, None])
    ds = r16(ds) if ds_bits is None else round_bits(ds, ds_bits)
    dv = r16(p).T @ d_o
    return lse, SCALE * (ds @ k), SCALE * (ds.T @ q), dv, p


@pytest.fixture(scope="module")
def case():
    w = wl.small_pack(3, tokens_per_video=1024, heads=2)
    t = oracle.expand(w.q_layout)
    q, k, v, d_o = w.q(), w.k_new(), w.v_new(), w.d_o()
    m = oracle.visible_mask(t, t)
    ref = oracle.backward(q, k, v, d_o, t, t, SCALE)
    _, l_ref = oracle.forward(q, k, v, t, t, SCALE)
    sig = tol.grad_sigma(q, k, v, d_o, t, t, SCALE)
    bound = tol.lse_bound(q, k, t, t, SCALE)
    return dict(t=t, q=q, k=k, v=v, d_o=d_o, m=m, ref=ref, l_ref=l_ref, sig=sig, bound=bound)


def gate_stats(c, **planted):
    zs = []
    for h in range(2):
        _, dq, dk, dv, _ = replay(c["q"][:, h], c["k"][:, h], c["v"][:, h], c["d_o"][:, h], c["m"],
                                  **planted)
        for got, ref, sig in zip((dq, dk, dv), c["ref"], c["sig"]):
            for bf16_out in (False, True):
                g = r16(got) if bf16_out else got
                z = tol.grad_z(g, ref[:, h], sig[:, h], bf16_out)
                zs.append((float(z.mean()), float(z.max())))
    return zs


def test_lse_bound_holds_and_bounds_the_backward_row_sums(case):
    c = case
    for h in range(2):
        lse, _, _, _, p = replay(c["q"][:, h], c["k"][:, h], c["v"][:, h], c["d_o"][:, h], c["m"])
        fin = np.isfinite(c["l_ref"][h])
        err = np.abs(lse[fin] - c["l_ref"][h][fin])
        b = c["bound"][h][fin]
        assert (err <= b).all(), float((err / b).max())
        assert err.max() > 0.02 * b.max()          # not vacuous: the bound is within 50x
        rs = p.sum(axis=1)[fin]
        assert (rs <= np.exp(b)).all() and (rs >= np.exp(-b)).all()
        assert np.abs(rs - 1).max() > 1e-5          # the mismatch is real, and bounded


def test_gradient_gate_passes_the_replayed_kernel(case):
    for zmean, zmax in gate_stats(case):
        assert zmean <= tol.Z_MEAN and zmax <= tol.Z_MAX, (zmean, zmax)


@pytest.mark.parametrize("planted", [dict(ds_bits=6), dict(lse_shift=4e-3)])
def test_gradient_gate_fails_planted_mistakes(case, planted):
    """dS rounded to 6 instead of 8 significant bits, or P formed against an
    lse off by 4e-3 (stale or wrong row statistics): the gate must fail."""
    stats = gate_stats(case, **planted)
    assert any(zmean > tol.Z_MEAN or zmax > tol.Z_MAX for zmean, zmax in stats), stats


def _f32_rowsum(x, rows, order):
    """fp32 sums of blocks of `rows` rows of bf16 values, in a given order."""
    n = x.shape[0]
    nb = -(-n // rows)
    xp = np.zeros((nb * rows,) + x.shape[1:], np.float32)
    xp[:n] = x
    xp = xp.reshape((nb, rows) + x.shape[1:])
    if order == "pairwise":
        while xp.shape[1] > 1:
            xp = (xp[:, 0::2] + xp[:, 1::2]).astype(np.float32)
        return xp[:, 0]
    if order == "groups16":
        part = np.zeros((nb, rows // 16) + x.shape[1:], np.float32)
        g = xp.reshape((nb, rows // 16, 16) + x.shape[1:])
        for r in range(16):
            part = (part + g[:, :, r]).astype(np.float32)
        xp, rows = part, rows // 16
    acc = np.zeros((nb,) + x.shape[1:], np.float32)
    idx = range(rows - 1, -1, -1) if order == "reversed" else range(rows)
    for r in idx:
        acc = (acc + xp[:, r]).astype(np.float32)
    return acc


@pytest.mark.parametrize("order", ["sequential", "reversed", "groups16", "pairwise"])
def test_block_score_bound_covers_fp32_evaluations(order):
    """score_bound >= |fp32 score - exact score| for fp32 evaluations of the
    block score in several summation orders (the device's among them), on
    480p-step rows of two heads; and it is far below the spread of scores."""
    from oracle import sparse
    w = wl.cached_step_480p()
    kc, _ = w.cache_kv()
    q = w.q(2)[:, :2]
    k = np.concatenate([kc, w.k_new(2)])[:, :2]
    exact = sparse.block_scores(q, k, 256, 64)
    eps = tol.score_bound(q, k, 256, 64)
    qs = np.transpose(_f32_rowsum(q, 256, order), (1, 0, 2))
    ks = np.transpose(_f32_rowsum(k, 64, order), (1, 0, 2))
    s = np.zeros(exact.shape, np.float32)
    ds = range(127, -1, -1) if order == "reversed" else range(128)
    for d in ds:
        s = (s + (qs[:, :, None, d] * ks[:, None, :, d]).astype(np.float32)).astype(np.float32)
    err = np.abs(s.astype(np.float64) - exact)
    assert (err <= eps).all(), float((err / eps).max())
    assert err.max() > 0 and eps.max() < 1e-2 * exact.std()
