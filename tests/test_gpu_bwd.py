"""GPU parity of the backward kernels (dQ, dK, dV) against the fp64 oracle,
through the C ABI.  The forward output and log-sum-exp that the backward
consumes come from the GPU forward of the same inputs."""
import numpy as np
import pytest
import torch

import oracle
import segment_causal_masked_amd as nm
from segment_causal_masked_amd import workloads as wl
from gpu_util import SCALE, check_lse, check_o, dev, host, need_gpu, run_fwd, say

pytestmark = pytest.mark.gpu

# Gradient gate, in units of the oracle tensor's RMS (gradients are not unit
# scale).  Derived from the arithmetic, not taken from the forward's gate:
# storing a gradient in bf16 alone costs up to 2^-9 |g| per element, and
# gradients are heavy-tailed (max |g| ~ 6-10 RMS), so even exact arithmetic
# rounded to bf16 shows max-abs ~1.5e-2 RMS and mean-abs ~1.1e-3 RMS; rounding
# P and dS to bf16 as MFMA operands (relative 2^-9 per term) adds up to
# ~2.3e-2 RMS above 2^-8 |g| and brings the mean-abs to ~1.8e-3 RMS.  These
# figures come from replaying exactly that rounding in fp64 numpy on the tiny
# two-segment case and on the 4096-token packs.  Bound, with margin:
# |err| <= 2^-8 |g| + 4e-2 RMS per element and mean-abs <= 2.5e-3 RMS.  A
# wrong index, sign or dropped term gives errors of order the RMS itself.
G_ELEM_REL, G_ELEM_RMS, G_MEAN_RMS = 2.0 ** -8, 4e-2, 2.5e-3


def check_grad(g_gpu, g_ref, what):
    rms = float(np.sqrt(np.mean(g_ref ** 2)))
    err = np.abs(g_gpu.astype(np.float64) - g_ref)
    excess = float(((err - G_ELEM_REL * np.abs(g_ref)) / rms).max())
    mx, mean = float(err.max()) / rms, float(err.mean()) / rms
    say(f"  {what}: rms {rms:.3e}  max-abs/rms {mx:.3e}  mean-abs/rms {mean:.3e}  "
        f"max (err - 2^-8|g|)/rms {excess:.3e}")
    assert np.isfinite(g_gpu).all(), what
    assert excess <= G_ELEM_RMS and mean <= G_MEAN_RMS, (what, excess, mean)


def run_bwd(plan, q, k, v, o, d_o, lse, heads):
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    n = nm.nomas_attn_bwd_workspace_size(plan)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")
    nm.nomas_attn_bwd(plan, q, k, v, o, d_o, lse, dq, dk, dv, SCALE, workspace=ws)
    torch.cuda.synchronize()
    return dq, dk, dv


def full_case(segs, heads, seed, mode="R", check_heads=None, fp32=False, window=0):
    """Whole-tensor comparison on a dense (no cache) layout."""
    n = wl.layout_tokens(segs)
    q = wl.randn((n, heads, 128), seed + 1, bf16=not fp32)
    k = wl.randn((n, heads, 128), seed + 2, bf16=not fp32)
    v = wl.randn((n, heads, 128), seed + 3, bf16=not fp32)
    d_o = wl.randn((n, heads, 128), seed + 4, bf16=not fp32)
    qb, kb, vb, dob = (wl.round_to_bf16(x) for x in (q, k, v, d_o))
    plan = nm.nomas_attn_plan(segs, segs, heads=heads, mode=mode, window=window)
    qd, kd, vd, dod = dev(qb), dev(kb), dev(vb), dev(dob)
    o, lse = run_fwd(plan, None, qd, kd, vd, heads)
    dq, dk, dv = run_bwd(plan, qd, kd, vd, o, dod, lse, heads)
    tq = oracle.expand(segs)
    hs = list(range(heads)) if check_heads is None else list(check_heads)
    o_ref, l_ref = oracle.forward(qb, kb, vb, tq, tq, SCALE, mode=mode, heads=hs, window=window)
    check_o(host(o)[:, hs], o_ref, "O")
    check_lse(host(lse)[hs], l_ref, "LSE")
    dq_ref, dk_ref, dv_ref = oracle.backward(qb, kb, vb, dob, tq, tq, SCALE, mode=mode, heads=hs,
                                             window=window)
    check_grad(host(dq)[:, hs], dq_ref, "dQ")
    check_grad(host(dk)[:, hs], dk_ref, "dK")
    check_grad(host(dv)[:, hs], dv_ref, "dV")
    return host(dq), host(dk), host(dv)


def test_tiny_two_segments_backward():
    need_gpu()
    w = wl.tiny_two_segments()
    say("tiny two segments: 96 tokens, 1 head, backward")
    full_case(w.q_layout, 1, 8100)


def test_pack_4096_tokens_backward():
    need_gpu()
    w = wl.small_pack(0)
    say(f"self-contained pack: {w.n_q} tokens, 2 videos, 16 heads, backward")
    full_case(w.q_layout, 16, 8200, check_heads=[0, 5, 15])


@pytest.mark.parametrize("mode", ["K", "H"])
def test_pack_backward_text_query_modes(mode):
    need_gpu()
    w = wl.small_pack(1)
    say(f"pack, mode {mode}, 2 heads")
    full_case(w.q_layout, 2, 8300, mode=mode)


@pytest.mark.parametrize("window", [1, 2])
def test_pack_backward_sliding_window(window):
    need_gpu()
    w = wl.small_pack(2)
    say(f"pack, window of {window} segment(s), 2 heads, backward")
    full_case(w.q_layout, 2, 8600 + window, window=window)


def test_thirty_two_actions_backward():
    """A segment with the largest action count (32) after a short history, as
    a dense pack: all three gradients against the oracle."""
    need_gpu()
    g = np.random.default_rng(33)
    acts = []
    for a in range(32):
        lo = int(g.integers(0, 4))
        acts.append((int(g.integers(1, 4)), lo, int(g.integers(lo + 1, 5))))
    segs = [wl.Segment(0, j, 1, 16, 2, [(1, 0, 1)]) for j in range(6)]
    segs.append(wl.Segment(0, 6, 4, 16, 6, acts, n_pad=5))
    say("32 actions, backward")
    full_case(segs, 2, 8700)


def test_ragged_pack_backward():
    """Token counts that are not multiples of the tile sizes, padding tokens,
    an odd number of 64-key tiles (last key-tile pair half missing)."""
    need_gpu()
    segs = [wl.Segment(0, 0, 3, 37, 11, [(5, 0, 2), (7, 1, 3)], n_pad=3),
            wl.Segment(0, 1, 2, 37, 11, [(6, 0, 1)]),
            wl.Segment(1, 0, 4, 29, 9, [(4, 2, 4), (3, 0, 1), (8, 1, 2)], n_pad=53)]
    n = wl.layout_tokens(segs)
    say(f"ragged pack: {n} tokens ({n % 128} rows in the last q-tile, {(n + 63) // 64} key tiles)")
    assert n % 128 and ((n + 63) // 64) % 2 == 1
    full_case(segs, 3, 8400)


def test_backward_ignores_masked_upstream_rows_bitwise():
    """Padding tokens see nothing and are seen by nobody: changing dO on
    padding rows and K / V on padding keys leaves every gradient bit-identical
    (their P is exactly 0, so they add exact zeros)."""
    need_gpu()
    segs = [wl.Segment(0, 0, 2, 64, 16, [(16, 0, 1)], n_pad=40),
            wl.Segment(0, 1, 2, 64, 16, [(16, 1, 2)], n_pad=24)]
    n = wl.layout_tokens(segs)
    heads = 2
    q, k, v, d_o = (dev(wl.randn((n, heads, 128), 8500 + i)) for i in range(4))
    plan = nm.nomas_attn_plan(segs, segs, heads=heads)
    o, lse = run_fwd(plan, None, q, k, v, heads)
    g1 = run_bwd(plan, q, k, v, o, d_o, lse, heads)
    pad = oracle.expand(segs).kind == oracle.tokens.PAD
    assert pad.sum() == 64
    d_o2 = d_o.clone()
    d_o2[torch.from_numpy(pad).cuda()] += 3.0
    k2, v2 = k.clone(), v.clone()
    k2[torch.from_numpy(pad).cuda()] -= 2.0
    v2[torch.from_numpy(pad).cuda()] *= -1.5
    g2 = run_bwd(plan, q, k2, v2, o, d_o2, lse, heads)
    for a, b, name in zip(g1, g2, ("dQ", "dK", "dV")):
        a, b = host(a), host(b)
        assert np.array_equal(a, b), name
        assert not a[pad].any() and np.abs(a[~pad]).sum() > 0, name


@pytest.mark.timeout(600)
def test_training_pack_131k_backward_slice():
    """Full 131072-token pack on the GPU; the oracle checks the 4096-token slice
    that starts 2048 tokens before video 1's third segment: O, LSE and dQ rows
    of those queries, dK and dV rows of those keys (two heads).  The pack is
    block-diagonal over videos, so the oracle runs on video 1 alone."""
    need_gpu()
    w = wl.training_pack_131k()
    segs = w.q_layout
    starts = np.cumsum([0] + [s.n_tokens for s in segs])
    v1 = [i for i, s in enumerate(segs) if s.video == 1]
    t_seg2 = int(starts[v1[2]])
    t0 = t_seg2 - 2048
    v_lo, v_hi = int(starts[v1[0]]), int(starts[v1[-1] + 1])
    say(f"training pack: {w.n_q} tokens; slice [{t0}, {t0 + 4096}) inside video 1 [{v_lo}, {v_hi})")
    assert v_lo <= t0 and t0 + 4096 <= v_hi
    plan = nm.nomas_attn_plan(segs, segs, heads=16)
    q, k, v, d_o = w.q(), w.k_new(), w.v_new(), w.d_o()
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(d_o)
    o, lse = run_fwd(plan, None, qd, kd, vd, 16)
    dq, dk, dv = run_bwd(plan, qd, kd, vd, o, dod, lse, 16)
    del qd, kd, vd, dod
    heads = [2, 11]
    sl = np.arange(t0, t0 + 4096)
    sub = segs[v1[0]:v1[-1] + 1]
    tq = oracle.expand(sub)
    vs = slice(v_lo, v_hi)
    rows = sl - v_lo
    o_ref, l_ref = oracle.forward(q[vs], k[vs], v[vs], tq, tq, SCALE, rows=rows, heads=heads)
    check_o(host(o)[sl][:, heads], o_ref, "training pack O slice")
    check_lse(host(lse)[heads][:, sl], l_ref, "training pack LSE slice")
    dq_ref, dk_ref, dv_ref = oracle.backward(q[vs], k[vs], v[vs], d_o[vs], tq, tq, SCALE,
                                             heads=heads, q_rows=rows, k_rows=rows)
    check_grad(host(dq)[sl][:, heads], dq_ref, "training pack dQ slice")
    check_grad(host(dk)[sl][:, heads], dk_ref, "training pack dK slice")
    check_grad(host(dv)[sl][:, heads], dv_ref, "training pack dV slice")
