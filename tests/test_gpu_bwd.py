"""GPU parity of the backward kernels (dQ, dK, dV) against the fp64 oracle,
through the C ABI.  The forward output and log-sum-exp that the backward
consumes come from the GPU forward of the same inputs."""
import numpy as np
import pytest
import torch

import oracle
import tolerance as tol
import segment_causal_masked_amd as nm
from segment_causal_masked_amd import workloads as wl
from gpu_util import SCALE, check_lse, oracle_forward, check_o, dev, host, need_gpu, run_fwd, say

pytestmark = pytest.mark.gpu

# Gradient gate (tolerance.py): per element, z = |err| / sigma with sigma the
# standard deviation that the kernels' bf16 roundings (P and dS as MFMA
# operands, the forward's rounded Q through its lse, bf16 outputs) give around
# the exact gradient; mean(z) <= sqrt(2/pi) and max(z) <= 6.  Calibrated on a
# replay of those roundings (tests/test_tolerance_model.py), where it holds
# with margin and fails planted mistakes.  The mean-abs error over the RMS is
# printed beside it.


def check_grad(g_gpu, g_ref, sigma, what, bf16_out=True):
    rms = float(np.sqrt(np.mean(g_ref ** 2)))
    err = np.abs(g_gpu.astype(np.float64) - g_ref)
    z = tol.grad_z(g_gpu, g_ref, sigma, bf16_out)
    zmean, zmax = float(z.mean()), float(z.max())
    say(f"  {what} ({'bf16' if bf16_out else 'fp32'}): rms {rms:.3e}  max-abs/rms "
        f"{float(err.max()) / rms:.3e}  mean-abs/rms {float(err.mean()) / rms:.3e}  "
        f"z mean {zmean:.3f} max {zmax:.2f}")
    assert np.isfinite(g_gpu).all(), what
    assert zmean <= tol.Z_MEAN and zmax <= tol.Z_MAX, (what, zmean, zmax)


def run_bwd(plan, q, k, v, o, d_o, lse, heads):
    gd = torch.float32 if plan.grad_f32 else torch.bfloat16
    dq = torch.empty(q.shape, dtype=gd, device="cuda")
    dk = torch.empty(k.shape, dtype=gd, device="cuda")
    dv = torch.empty(v.shape, dtype=gd, device="cuda")
    n = nm.nomas_attn_bwd_workspace_size(plan)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")
    nm.nomas_attn_bwd(plan, q, k, v, o, d_o, lse, dq, dk, dv, SCALE, workspace=ws)
    torch.cuda.synchronize()
    return dq, dk, dv


def full_case(segs, heads, seed, mode="R", check_heads=None, fp32=False, window=0, grad_f32=False):
    """Whole-tensor comparison on a dense (no cache) layout; grad_f32: the
    plan asks for fp32 gradients."""
    n = wl.layout_tokens(segs)
    q = wl.randn((n, heads, 128), seed + 1, bf16=not fp32)
    k = wl.randn((n, heads, 128), seed + 2, bf16=not fp32)
    v = wl.randn((n, heads, 128), seed + 3, bf16=not fp32)
    d_o = wl.randn((n, heads, 128), seed + 4, bf16=not fp32)
    qb, kb, vb, dob = (wl.round_to_bf16(x) for x in (q, k, v, d_o))
    plan = nm.nomas_attn_plan(segs, segs, heads=heads, mode=mode, window=window, grad_f32=grad_f32)
    qd, kd, vd, dod = dev(qb), dev(kb), dev(vb), dev(dob)
    o, lse = run_fwd(plan, None, qd, kd, vd, heads)
    dq, dk, dv = run_bwd(plan, qd, kd, vd, o, dod, lse, heads)
    tq = oracle.expand(segs)
    hs = list(range(heads)) if check_heads is None else list(check_heads)
    o_ref, l_ref, l_bnd = oracle_forward(qb, kb, vb, tq, tq, SCALE, mode=mode, heads=hs, window=window)
    check_o(host(o)[:, hs], o_ref, "O")
    check_lse(host(lse)[hs], l_ref, "LSE", l_bnd)
    dq_ref, dk_ref, dv_ref = oracle.backward(qb, kb, vb, dob, tq, tq, SCALE, mode=mode, heads=hs,
                                             window=window)
    sq, sk, sv = tol.grad_sigma(qb, kb, vb, dob, tq, tq, SCALE, mode=mode, heads=hs, window=window)
    bf = not grad_f32
    check_grad(host(dq)[:, hs], dq_ref, sq, "dQ", bf)
    check_grad(host(dk)[:, hs], dk_ref, sk, "dK", bf)
    check_grad(host(dv)[:, hs], dv_ref, sv, "dV", bf)
    return host(dq), host(dk), host(dv)


@pytest.mark.parametrize("grad_f32", [False, True])
def test_tiny_two_segments_backward(grad_f32):
    need_gpu()
    w = wl.tiny_two_segments()
    say(f"tiny two segments: 96 tokens, 1 head, backward, {'fp32' if grad_f32 else 'bf16'} gradients")
    full_case(w.q_layout, 1, 8100, grad_f32=grad_f32)


@pytest.mark.parametrize("grad_f32", [False, True])
def test_pack_4096_tokens_backward(grad_f32):
    need_gpu()
    w = wl.small_pack(0)
    say(f"self-contained pack: {w.n_q} tokens, 2 videos, 16 heads, backward, "
        f"{'fp32' if grad_f32 else 'bf16'} gradients")
    full_case(w.q_layout, 16, 8200, check_heads=[0, 5, 15], grad_f32=grad_f32)


def test_fp32_gradients_round_to_the_bf16_ones():
    """The same backward with fp32 outputs: rounding them to bf16 gives the
    bf16 outputs bit for bit (one kernel, two epilogues)."""
    need_gpu()
    w = wl.small_pack(4)
    segs = w.q_layout
    n, heads = wl.layout_tokens(segs), 2
    q, k, v, d_o = (dev(wl.randn((n, heads, 128), 8800 + i)) for i in range(4))
    p16 = nm.nomas_attn_plan(segs, segs, heads=heads)
    p32 = nm.nomas_attn_plan(segs, segs, heads=heads, grad_f32=True)
    o, lse = run_fwd(p16, None, q, k, v, heads)
    g16 = run_bwd(p16, q, k, v, o, d_o, lse, heads)
    g32 = run_bwd(p32, q, k, v, o, d_o, lse, heads)
    for a, b, name in zip(g16, g32, ("dQ", "dK", "dV")):
        assert b.dtype == torch.float32 and a.dtype == torch.bfloat16
        assert torch.equal(b.to(torch.bfloat16), a), name
        assert not torch.equal(b, a.float()), name      # the fp32 outputs carry more bits


def test_backward_repeats_bitwise():
    """Which workgroup takes which unit varies from run to run (work queues),
    but each unit is summed by one workgroup in a fixed order: runs of the
    training-shape backward on the same inputs give bit-identical gradients
    (a race between waves or workgroups would show as a difference)."""
    need_gpu()
    w = wl.small_pack(5)
    segs = w.q_layout
    n, heads = wl.layout_tokens(segs), 16
    q, k, v, d_o = (dev(wl.randn((n, heads, 128), 8900 + i)) for i in range(4))
    plan = nm.nomas_attn_plan(segs, segs, heads=heads)
    o, lse = run_fwd(plan, None, q, k, v, heads)
    o2, lse2 = run_fwd(plan, None, q, k, v, heads)
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    g1 = run_bwd(plan, q, k, v, o, d_o, lse, heads)
    for _ in range(3):
        g2 = run_bwd(plan, q, k, v, o, d_o, lse, heads)
        for a, b, name in zip(g1, g2, ("dQ", "dK", "dV")):
            assert torch.equal(a, b), name


def test_backward_degenerate_layouts_and_workspace_reuse():
    """No queries (dK = dV = 0), no keys (dQ = 0) and a pack of padding only
    (all three zero), all through one workspace; then a real pack through the
    same workspace equals the same pack through a fresh one bit for bit (the
    work-queue counters in the workspace are reset by every call)."""
    need_gpu()
    heads = 2
    segs = wl.small_pack(2).q_layout
    n = wl.layout_tokens(segs)
    ws = torch.full((1 << 22,), 0xAB, dtype=torch.uint8, device="cuda")  # dirty on purpose

    def bwd(plan, q, k, v, o, d_o, lse):
        gs = [torch.full(x.shape, 7.0, dtype=torch.bfloat16, device="cuda") for x in (q, k, v)]
        need = nm.nomas_attn_bwd_workspace_size(plan)
        assert need <= ws.numel()
        nm.nomas_attn_bwd(plan, q, k, v, o, d_o, lse, *gs, SCALE, workspace=ws[:need])
        torch.cuda.synchronize()
        return gs

    k, v = (dev(wl.randn((n, heads, 128), 9300 + i)) for i in range(2))
    # no queries
    p0 = nm.nomas_attn_plan([], segs, heads=heads)
    e = torch.empty((0, heads, 128), dtype=torch.bfloat16, device="cuda")
    le = torch.empty((heads, 0), dtype=torch.float32, device="cuda")
    _, dk, dv = bwd(p0, e, k, v, e, e, le)
    assert (dk == 0).all() and (dv == 0).all()
    # no keys: the queries see nothing
    q, d_o = (dev(wl.randn((n, heads, 128), 9310 + i)) for i in range(2))
    p1 = nm.nomas_attn_plan(segs, [], heads=heads)
    o1, l1 = run_fwd(p1, None, q, e, e, heads)
    assert (o1 == 0).all() and torch.isinf(l1).all()
    dq, _, _ = bwd(p1, q, e, e, o1, d_o, l1)
    assert (dq == 0).all()
    # padding only
    sp = [wl.Segment(0, 0, 0, 0, 0, [], n_pad=300)]
    qp, kp, vp, dop = (dev(wl.randn((300, heads, 128), 9320 + i)) for i in range(4))
    p2 = nm.nomas_attn_plan(sp, sp, heads=heads)
    o2, l2 = run_fwd(p2, None, qp, kp, vp, heads)
    for g in bwd(p2, qp, kp, vp, o2, dop, l2):
        assert (g == 0).all()
    # a real pack through the reused workspace and through a fresh one
    p3 = nm.nomas_attn_plan(segs, segs, heads=heads)
    o3, l3 = run_fwd(p3, None, q, k, v, heads)
    g_reused = bwd(p3, q, k, v, o3, d_o, l3)
    g_fresh = run_bwd(p3, q, k, v, o3, d_o, l3, heads)
    for a, b, name in zip(g_reused, g_fresh, ("dQ", "dK", "dV")):
        assert torch.equal(a, b), name


def test_pack_backward_with_padding_only_tile_pairs():
    """640 padding tokens between the two videos of a pack: two query-tile
    pairs see no key at all (units without entries in the dQ kernel's loop of
    claims, between units with work), and the key tiles they would form are
    seen by nobody; whole tensors against the oracle."""
    need_gpu()
    segs = wl.small_pack(3).q_layout
    pad = wl.Segment(9, 0, 0, 0, 0, [], n_pad=640)
    full_case(segs[:3] + [pad] + segs[3:], 2, 9400)


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


@pytest.mark.timeout(900)
def test_training_pack_131k_backward_slice():
    """Full 131072-token pack on the GPU; the oracle checks the 4096-token slice
    that starts 2048 tokens before video 1's third segment: O, LSE and dQ rows
    of those queries, dK and dV rows of those keys (two heads), for bf16 and
    for fp32 gradient outputs.  The pack is block-diagonal over videos, so the
    oracle runs on video 1 alone."""
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
    plan16 = nm.nomas_attn_plan(segs, segs, heads=16)
    plan32 = nm.nomas_attn_plan(segs, segs, heads=16, grad_f32=True)
    q, k, v, d_o = w.q(), w.k_new(), w.v_new(), w.d_o()
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(d_o)
    o, lse = run_fwd(plan16, None, qd, kd, vd, 16)
    heads = [2, 11]
    sl = np.arange(t0, t0 + 4096)
    grads = {}
    for name, plan in (("bf16", plan16), ("fp32", plan32)):
        g = run_bwd(plan, qd, kd, vd, o, dod, lse, 16)
        grads[name] = [host(x)[sl][:, heads] for x in g]
        del g
    o_h, lse_h = host(o), host(lse)
    del qd, kd, vd, dod, o, lse
    sub = segs[v1[0]:v1[-1] + 1]
    tq = oracle.expand(sub)
    vs = slice(v_lo, v_hi)
    rows = sl - v_lo
    o_ref, l_ref, l_bnd = oracle_forward(q[vs], k[vs], v[vs], tq, tq, SCALE, rows=rows, heads=heads)
    check_o(o_h[sl][:, heads], o_ref, "training pack O slice")
    check_lse(lse_h[heads][:, sl], l_ref, "training pack LSE slice", l_bnd)
    say("  oracle backward over video 1 ...")
    dq_ref, dk_ref, dv_ref = oracle.backward(q[vs], k[vs], v[vs], d_o[vs], tq, tq, SCALE,
                                             heads=heads, q_rows=rows, k_rows=rows)
    say("  gate model over video 1 ...")
    sq, sk, sv = tol.grad_sigma(q[vs], k[vs], v[vs], d_o[vs], tq, tq, SCALE, heads=heads,
                                q_rows=rows, k_rows=rows)
    for name, (dq, dk, dv) in grads.items():
        bf = name == "bf16"
        check_grad(dq, dq_ref, sq, "training pack dQ slice", bf)
        check_grad(dk, dk_ref, sk, "training pack dK slice", bf)
        check_grad(dv, dv_ref, sv, "training pack dV slice", bf)
