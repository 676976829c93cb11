"""Pins of the oracle's fp64 attention forward and backward.

Outside references: scipy's softmax / logsumexp, torch's CPU
scaled_dot_product_attention and autograd in float64, central finite
differences, and the invariants the method must satisfy.
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

import oracle
from segment_causal_masked_amd import workloads as wl
from test_oracle_mask import random_tiny_layout

SCALE = 1.0 / np.sqrt(128.0)


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_one_hot_values_reveal_softmax_rows():
    w = wl.tiny_two_segments()
    t = oracle.expand(w.q_layout)
    n = len(t)
    q, k = w.q(), w.k_new()
    v = np.zeros((n, 1, 128))
    v[np.arange(n), 0, np.arange(n)] = 1.0          # O[q] == P[q, :]
    o, lse = oracle.forward(q, k, v, t, t, SCALE)
    p = o[:, 0, :n]
    m = oracle.visible_mask(t, t)
    assert np.all(p[~m] == 0.0)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    s = SCALE * (q[:, 0, :].astype(np.float64) @ k[:, 0, :].astype(np.float64).T)
    for r in range(n):
        vis = np.flatnonzero(m[r])
        np.testing.assert_allclose(p[r, vis], softmax(s[r, vis]), rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(lse[0, r], logsumexp(s[r, vis]), rtol=1e-13)


def _sdpa(q, k, v, mask=None, causal=False):
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2))).double()
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2))).double()
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2))).double()
    am = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=am, is_causal=causal, scale=SCALE)
    return o.numpy().transpose(1, 0, 2)


def test_unmasked_case_matches_sdpa():
    segs = [wl.Segment(0, 0, 4, 9, 0, [])]
    t = oracle.expand(segs)
    q, k, v = rand((36, 3, 128), 1), rand((36, 3, 128), 2), rand((36, 3, 128), 3)
    o, _ = oracle.forward(q, k, v, t, t, SCALE)
    np.testing.assert_allclose(o, _sdpa(q, k, v), rtol=1e-12, atol=1e-12)


def test_one_token_segments_match_causal_sdpa():
    segs = [wl.Segment(0, j, 1, 1, 0, []) for j in range(40)]
    t = oracle.expand(segs)
    q, k, v = rand((40, 2, 128), 4), rand((40, 2, 128), 5), rand((40, 2, 128), 6)
    o, _ = oracle.forward(q, k, v, t, t, SCALE)
    np.testing.assert_allclose(o, _sdpa(q, k, v, causal=True), rtol=1e-12, atol=1e-12)


def test_general_mask_matches_sdpa_with_boolean_mask():
    g = np.random.default_rng(11)
    for trial in range(10):
        segs = random_tiny_layout(g, with_pad=False)
        t = oracle.expand(segs)
        n = len(t)
        q, k, v = rand((n, 2, 128), 10 + trial), rand((n, 2, 128), 40 + trial), rand((n, 2, 128), 70 + trial)
        o, _ = oracle.forward(q, k, v, t, t, SCALE, mode="R")
        np.testing.assert_allclose(o, _sdpa(q, k, v, mask=oracle.visible_mask(t, t)),
                                   rtol=1e-11, atol=1e-12)


def test_padding_rows_are_zero_with_minus_inf_lse():
    segs, *_ = __import__("golden_io").load_mask_fixture("pack2_mask.txt")
    t = oracle.expand(segs)
    n = len(t)
    q, k, v = rand((n, 1, 128), 1), rand((n, 1, 128), 2), rand((n, 1, 128), 3)
    o, lse = oracle.forward(q, k, v, t, t, SCALE)
    assert np.all(o[8] == 0.0) and lse[0, 8] == -np.inf
    assert np.isfinite(lse[0, np.arange(n) != 8]).all()


def test_output_is_linear_in_values():
    w = wl.tiny_two_segments()
    t = oracle.expand(w.q_layout)
    q, k, v = w.q(), w.k_new(), w.v_new()
    o1, _ = oracle.forward(q, k, v, t, t, SCALE)
    o2, _ = oracle.forward(q, k, 3.0 * v.astype(np.float64), t, t, SCALE)
    np.testing.assert_allclose(o2, 3.0 * o1, rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------------------
# backward
# ----------------------------------------------------------------------------

def _loss(q, k, v, do, t):
    o, _ = oracle.forward(q, k, v, t, t, SCALE)
    return float((o * do).sum())


def test_backward_central_differences():
    g = np.random.default_rng(3)
    segs = random_tiny_layout(g, n_videos=2)
    t = oracle.expand(segs)
    n = len(t)
    q, k, v, do = (rand((n, 1, 128), s) for s in (21, 22, 23, 24))
    dq, dk, dv = oracle.backward(q, k, v, do, t, t, SCALE)
    h = 1e-5
    pick = np.random.default_rng(0)
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            i, d = int(pick.integers(0, n)), int(pick.integers(0, 128))
            xp, xm = x.copy(), x.copy()
            xp[i, 0, d] += h
            xm[i, 0, d] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            fd = (_loss(args_p["q"], args_p["k"], args_p["v"], do, t)
                  - _loss(args_m["q"], args_m["k"], args_m["v"], do, t)) / (2 * h)
            assert abs(fd - grad[i, 0, d]) <= 1e-6 * max(1.0, abs(fd)), (name, i, d)


def test_backward_matches_torch_autograd_fp64():
    g = np.random.default_rng(8)
    segs = random_tiny_layout(g, n_videos=2, with_pad=False)
    t = oracle.expand(segs)
    n = len(t)
    q, k, v, do = (rand((n, 2, 128), s) for s in (31, 32, 33, 34))
    dq, dk, dv = oracle.backward(q, k, v, do, t, t, SCALE)
    m = torch.from_numpy(oracle.visible_mask(t, t))
    add = torch.zeros(m.shape, dtype=torch.float64).masked_fill(~m, float("-inf"))
    qt, kt, vt = (torch.tensor(x.transpose(1, 0, 2), requires_grad=True) for x in (q, k, v))
    s = SCALE * qt @ kt.transpose(1, 2) + add
    o = torch.softmax(s, dim=-1) @ vt
    o.backward(torch.from_numpy(np.ascontiguousarray(do.transpose(1, 0, 2))))
    for mine, ref in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
        np.testing.assert_allclose(mine, ref.numpy().transpose(1, 0, 2), rtol=1e-10, atol=1e-12)


def test_backward_row_subsets_match_full():
    w = wl.small_pack(seed=1, heads=2)
    t = oracle.expand(w.q_layout)
    q, k, v, do = w.q(), w.k_new(), w.v_new(), w.d_o()
    full = oracle.backward(q, k, v, do, t, t, SCALE, block=700)
    qr = np.arange(1000, 1500)
    kr = np.arange(1800, 2300)
    sub = oracle.backward(q, k, v, do, t, t, SCALE, q_rows=qr, k_rows=kr, heads=[1])
    np.testing.assert_allclose(sub[0][:, 0], full[0][qr, 1], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sub[1][:, 0], full[1][kr, 1], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sub[2][:, 0], full[2][kr, 1], rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------
# invariants of the method
# ----------------------------------------------------------------------------

def test_invariant_masked_kv_perturbation_changes_nothing():
    w = wl.tiny_two_segments()
    t = oracle.expand(w.q_layout)
    m = oracle.visible_mask(t, t)
    q, k, v = w.q(), w.k_new().astype(np.float64), w.v_new().astype(np.float64)
    o0, l0 = oracle.forward(q, k, v, t, t, SCALE)
    for r in (0, 20, 35, 41, 50, 70, 85, 93):
        hidden = ~m[r]
        k2, v2 = k.copy(), v.copy()
        k2[hidden] += 7.0
        v2[hidden] -= 5.0
        o1, l1 = oracle.forward(q, k2, v2, t, t, SCALE)   # same shapes: same BLAS path
        assert np.array_equal(o1[r], o0[r]) and l1[0, r] == l0[0, r]
        assert not np.array_equal(o1, o0)                  # the perturbation is seen elsewhere


def test_invariant_segment_unaffected_by_next_segment():
    w = wl.tiny_two_segments()
    t = oracle.expand(w.q_layout)
    q, k, v = w.q(), w.k_new().astype(np.float64), w.v_new().astype(np.float64)
    o0, _ = oracle.forward(q, k, v, t, t, SCALE)
    k[48:] = rand((48, 1, 128), 9)
    v[48:] = rand((48, 1, 128), 10)
    o1, _ = oracle.forward(q, k, v, t, t, SCALE)
    assert np.array_equal(o0[:48], o1[:48])


def test_invariant_cached_decoding_equals_full_sequence():
    w = wl.cached_step_480p()
    w.cached = w.cached[:2]                    # keep it quick: 2 cached + new
    full = w.cached + w.new
    tf = oracle.expand(full)
    nq = w.n_q
    g = np.random.default_rng(4)
    kk, vv = g.standard_normal((len(tf), 2, 128)), g.standard_normal((len(tf), 2, 128))
    qq = g.standard_normal((len(tf), 2, 128))
    rows = np.arange(len(tf) - nq, len(tf))[::7]
    o_full, l_full = oracle.forward(qq, kk, vv, tf, tf, SCALE, rows=rows)
    tq = oracle.expand(w.q_layout)
    o_c, l_c = oracle.forward(qq[len(tf) - nq:], kk, vv, tq, tf, SCALE,
                              rows=rows - (len(tf) - nq))
    np.testing.assert_allclose(o_c, o_full, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l_c, l_full, rtol=0, atol=1e-12)


def test_invariant_action_tail_locality_and_non_vacuity():
    w = wl.tiny_two_segments()
    t = oracle.expand(w.q_layout)
    q, k, v = w.q(), w.k_new().astype(np.float64), w.v_new().astype(np.float64)
    o0, _ = oracle.forward(q, k, v, t, t, SCALE)
    # tail a_1 of segment 0 = tokens 44..47, window [1,2) -> frame-1 video rows
    # 16..31 plus its own rows 44..47 may change; nothing else may.
    k2, v2 = k.copy(), v.copy()
    k2[44:48] += 3.0
    v2[44:48] += 3.0
    o1, _ = oracle.forward(q, k2, v2, t, t, SCALE)
    changed = np.any(o1 != o0, axis=(1, 2))
    expect = np.zeros(96, bool)
    expect[16:32] = True
    expect[44:48] = True
    np.testing.assert_array_equal(changed, expect)
