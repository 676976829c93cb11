"""GPU parity of the forward kernel and the cache append against the fp64
oracle, through the C ABI, plus the method's invariants checked bitwise."""
import numpy as np
import pytest
import torch

import oracle
import tolerance as tol
import segment_causal_masked_amd as nm
from segment_causal_masked_amd import workloads as wl
from gpu_util import (SCALE, check_lse, oracle_forward, check_o, dev, fill_cache, host, need_gpu, new_cache,
                      run_fwd, say, stored_rows)

pytestmark = pytest.mark.gpu


def dense_case(w, mode="R", nfe=0):
    """Plan + inputs for a workload whose keys are all passed with the call."""
    keys = w.cached + w.new
    q = w.q(nfe)
    if w.cached:
        kc, vc = w.cache_kv()
        k = np.concatenate([kc, w.k_new(nfe)])
        v = np.concatenate([vc, w.v_new(nfe)])
    else:
        k, v = w.k_new(nfe), w.v_new(nfe)
    plan = nm.nomas_attn_plan(w.q_layout, keys, heads=w.heads, mode=mode)
    return plan, q, k, v, keys


def oracle_fwd(w, q, k, v, keys, mode="R", rows=None, heads=None, window=0, u_inputs=0.0):
    """(O, LSE) of the oracle and the LSE bound of the device for those rows."""
    tq, tk = oracle.expand(w.q_layout), oracle.expand(keys)
    return oracle_forward(q, k, v, tq, tk, SCALE, mode=mode, rows=rows, heads=heads, window=window,
                          u_inputs=u_inputs)


def test_tiny_two_segments_fp32_inputs():
    need_gpu()
    w = wl.tiny_two_segments()
    say("tiny two segments: 96 tokens, 1 head, fp32 inputs rounded to bf16 for the kernel")
    plan, q, k, v, keys = dense_case(w)
    o, l = run_fwd(plan, None, dev(q), dev(k), dev(v), 1)
    # oracle on the fp32 inputs: the LSE bound adds the kernel's bf16 rounding of Q and K
    o_ref, l_ref, l_bnd = oracle_fwd(w, q, k, v, keys, u_inputs=2.0 ** -8)
    check_o(host(o), o_ref, "vs fp32 inputs")
    check_lse(host(l), l_ref, "vs fp32 inputs", l_bnd)
    qb, kb, vb = (wl.round_to_bf16(x) for x in (q, k, v))
    o_ref_b, l_ref_b, l_bnd_b = oracle_fwd(w, qb, kb, vb, keys)     # same bf16 values
    check_o(host(o), o_ref_b, "vs bf16 inputs")
    check_lse(host(l), l_ref_b, "vs bf16 inputs", l_bnd_b)


@pytest.mark.parametrize("mode", ["R", "K", "H"])
def test_single_segment_480p(mode):
    need_gpu()
    w = wl.single_segment_480p()
    say(f"single 480p segment, 3280 tokens x 16 heads, mode {mode}")
    plan, q, k, v, keys = dense_case(w, mode)
    o, l = run_fwd(plan, None, dev(q), dev(k), dev(v), 16)
    heads = None if mode == "R" else [0, 7, 15]
    o_ref, l_ref, l_bnd = oracle_fwd(w, q, k, v, keys, mode=mode, heads=heads)
    hsel = slice(None) if heads is None else heads
    check_o(host(o)[:, hsel], o_ref, f"single segment {mode}")
    check_lse(host(l)[hsel], l_ref, f"single segment {mode}", l_bnd)


def test_single_segment_480p_sorted_windows():
    need_gpu()
    w = wl.single_segment_480p(seed_set=1)
    plan, q, k, v, keys = dense_case(w)
    o, l = run_fwd(plan, None, dev(q), dev(k), dev(v), 16)
    o_ref, l_ref, l_bnd = oracle_fwd(w, q, k, v, keys, heads=[3, 12])
    check_o(host(o)[:, [3, 12]], o_ref, "single segment, sorted windows")
    check_lse(host(l)[[3, 12]], l_ref, "single segment, sorted windows", l_bnd)


def build_cached(w, layer=0):
    kc, vc = w.cache_kv(layer)
    cap = w.n_cached + w.n_new
    cache = new_cache(w.heads, cap)
    kd, vd = dev(kc), dev(vc)
    fill_cache(cache, w.cached, kd, vd)
    torch.cuda.synchronize()
    return cache, kc, vc


def test_cached_step_480p_and_append_layout():
    need_gpu()
    w = wl.cached_step_480p()
    say("480p cached step: 4 cached segments (13120 tokens, 12736 stored rows) + 3280 new, 16 heads")
    cache, kc, vc = build_cached(w)
    # the append wrote the video + head rows of each segment (token-major) into
    # the head-major cache, bit for bit; action tails are not kept
    rows = stored_rows(w.cached)
    n = len(rows)
    assert n == w.n_cached - 4 * 96
    kb = cache.k_buf[:, :n].permute(1, 0, 2).contiguous()
    vb = cache.v_buf[:, :n].permute(1, 0, 2).contiguous()
    assert torch.equal(kb, dev(kc[rows])) and torch.equal(vb, dev(vc[rows]))
    assert nm.nomas_kvcache_len(cache) == (n, 4)
    plan = nm.nomas_attn_plan(w.q_layout, w.new, cache, heads=16)
    q, kn, vn = w.q(), w.k_new(), w.v_new()
    o, l = run_fwd(plan, cache, dev(q), dev(kn), dev(vn), 16)
    keys = w.cached + w.new
    o_ref, l_ref, l_bnd = oracle_fwd(w, q, np.concatenate([kc, kn]), np.concatenate([vc, vn]), keys)
    check_o(host(o), o_ref, "480p cached step")
    check_lse(host(l), l_ref, "480p cached step", l_bnd)


def test_cached_step_matches_full_sequence():
    """Cached decoding of the last segment against its rows of the
    full-sequence run.  Both round the same Q * scale * log2(e) and form the
    same scores; they differ in the grouping of keys into tiles, hence in the
    reference each exponential is taken against and the fp32 summation
    order: P then differs by fp32 rounding (relative ~1e-7), which can flip
    its bf16 rounding (one bf16 step, 2^-8 relative) for the P.V product.
    So every O element lies within 2^-8 * sum_k P |V| (P exact) plus one bf16
    step of O and 1e-6, and the LSE within the two runs' summation bound.
    And segment j does not depend on segment j + 1 (bitwise)."""
    need_gpu()
    w = wl.cached_step_480p()
    cache, kc, vc = build_cached(w)
    q, kn, vn = w.q(), w.k_new(), w.v_new()
    plan = nm.nomas_attn_plan(w.q_layout, w.new, cache, heads=16)
    o_c, l_c = run_fwd(plan, cache, dev(q), dev(kn), dev(vn), 16)
    full = w.cached + w.new
    g = np.random.default_rng(0)
    q_full = np.concatenate([wl.round_to_bf16(g.standard_normal((w.n_cached, 16, 128), np.float32)), q])
    k_full, v_full = np.concatenate([kc, kn]), np.concatenate([vc, vn])
    plan_f = nm.nomas_attn_plan(full, full, heads=16)
    o_f, l_f = run_fwd(plan_f, None, dev(q_full), dev(k_full), dev(v_full), 16)
    a, b = host(o_c).astype(np.float64), host(o_f[w.n_cached:]).astype(np.float64)
    d = np.abs(a - b)
    # one bf16 step of the larger magnitude: 2^(floor(log2|x|) - 7)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.maximum(np.abs(a), np.abs(b)), 1e-30))) - 7)
    keys = w.cached + w.new
    pv = tol.softmax_abs_v(q, k_full, v_full, oracle.expand(w.q_layout), oracle.expand(keys), SCALE)
    bound = 2.0 ** -8 * pv * (1 + 1e-3) + ulp + 1e-6
    say(f"  cached vs full rows: bitwise equal {torch.equal(o_c, o_f[w.n_cached:])}, "
        f"max-abs {float(d.max()):.3e}, elements differing {int((d > 0).sum())} of {d.size}, "
        f"max diff/bound {float((d / bound).max()):.3f}")
    assert bool((d <= bound).all())
    # LSE: the row sums of the two runs differ by at most their fp32 summation
    # error, gamma of the depth (tiles visited + 24) each, plus the final log
    lc, lf = l_c.double(), l_f[:, w.n_cached:].double()
    depth = (w.n_keys + 63) // 64 + 24
    bound = 2 * (tol.gamma(depth) + 4e-6 * (1 + lf.abs()))
    assert bool(((lc - lf).abs() <= bound).all()), float((lc - lf).abs().max())
    # segment j is unchanged by the contents of segment j+1 (bitwise)
    k2, v2 = k_full.copy(), v_full.copy()
    k2[w.n_cached:] += 1.0
    v2[w.n_cached:] -= 1.0
    o_p, _ = run_fwd(plan_f, None, dev(q_full), dev(k2), dev(v2), 16)
    assert torch.equal(o_p[:w.n_cached], o_f[:w.n_cached])
    assert not torch.equal(o_p[w.n_cached:], o_f[w.n_cached:])


def test_masked_kv_perturbation_is_invisible_bitwise():
    need_gpu()
    w = wl.single_segment_480p()
    plan, q, k, v, keys = dense_case(w)
    o0, l0 = run_fwd(plan, None, dev(q), dev(k), dev(v), 16)
    s = w.q_layout[0]
    n_video = s.n_frames * s.tokens_per_frame
    start = n_video + s.n_head                     # a_0's tokens
    n0, lo, hi = s.actions[0]
    k2, v2 = k.copy(), v.copy()
    k2[start:start + n0] = 5.0
    v2[start:start + n0] = -3.0
    o1, _ = run_fwd(plan, None, dev(q), dev(k2), dev(v2), 16)
    changed = (o1 != o0).any(dim=2).any(dim=1).cpu().numpy()
    t = oracle.expand(w.q_layout)
    m = oracle.visible_mask(t, t)
    sees_a0 = m[:, start:start + n0].any(axis=1)
    say(f"  rows seeing a_0: {int(sees_a0.sum())}, rows changed: {int(changed.sum())}")
    assert not changed[~sees_a0].any()             # invisible everywhere else, bit for bit
    assert changed[sees_a0].all()                  # and visible where it should be
    frames = np.flatnonzero(sees_a0[:n_video]) // s.tokens_per_frame
    assert frames.min() >= lo and frames.max() < hi


def test_padding_rows_and_ragged_shapes():
    need_gpu()
    segs = [wl.Segment(0, 0, 3, 7, 5, [(3, 0, 2), (2, 2, 3)], n_pad=9),
            wl.Segment(1, 0, 2, 50, 4, [(6, 1, 2)], n_pad=1),
            wl.Segment(1, 1, 5, 33, 17, [(1, 0, 5), (4, 3, 4), (2, 1, 3)], n_pad=3)]
    n = sum(s.n_tokens for s in segs)
    say(f"ragged pack: {n} tokens, 3 heads, padding rows")
    g = np.random.default_rng(1)
    q, k, v = (wl.round_to_bf16(g.standard_normal((n, 3, 128), np.float32)) for _ in range(3))
    plan = nm.nomas_attn_plan(segs, segs, heads=3)
    o, l = run_fwd(plan, None, dev(q), dev(k), dev(v), 3)
    t = oracle.expand(segs)
    o_ref, l_ref, l_bnd = oracle_forward(q, k, v, t, t, SCALE)
    check_o(host(o), o_ref, "ragged pack")
    check_lse(host(l), l_ref, "ragged pack", l_bnd)
    pad = t.kind == oracle.PAD
    assert (host(o)[pad] == 0).all()


def test_padding_rows_have_no_influence_bitwise():
    """Rows that see no key (padding) are computed unmasked on tiles where
    every other row of the tile sees every key, and written as exact zeros.
    So whatever the padding rows of Q hold -- large values, NaN -- the live
    rows' O and LSE stay bit-identical and the padding rows stay O = 0,
    LSE = -inf; in the backward, finite garbage in the padding rows of Q and
    dO changes no bit of dK, dV or the live rows of dQ, and their own dQ rows
    are 0."""
    need_gpu()
    segs = [wl.Segment(0, 0, 4, 40, 8, [(6, 0, 2)], n_pad=70),
            wl.Segment(0, 1, 4, 40, 8, [(5, 1, 3)], n_pad=90),
            wl.Segment(1, 0, 5, 37, 6, [(4, 0, 5)], n_pad=45)]
    n, heads = wl.layout_tokens(segs), 2
    t = oracle.expand(segs)
    pad = torch.from_numpy(t.kind == oracle.PAD).to("cuda")
    say(f"padding rows: {n} tokens, {int(pad.sum())} of them padding, {heads} heads")
    plan = nm.nomas_attn_plan(segs, segs, heads=heads)
    q, k, v, d_o = (dev(wl.randn((n, heads, 128), 7400 + i)) for i in range(4))
    o0, l0 = run_fwd(plan, None, q, k, v, heads)
    assert (o0[pad] == 0).all() and torch.isinf(l0[:, pad]).all() and (l0[:, pad] < 0).all()
    for what, fill in (("large", 3.0e4), ("NaN", float("nan"))):
        qg = q.clone()
        qg[pad] = fill
        o1, l1 = run_fwd(plan, None, qg, k, v, heads)
        assert torch.equal(o1.view(torch.int16), o0.view(torch.int16)), what
        assert torch.equal(l1, l0), what
    # backward: finite garbage in the padding rows of Q and dO
    gd = torch.bfloat16
    def bwd(qx, dox):
        dq, dk, dv = (torch.empty((n, heads, 128), dtype=gd, device="cuda") for _ in range(3))
        ws = torch.empty(max(nm.nomas_attn_bwd_workspace_size(plan), 16), dtype=torch.uint8, device="cuda")
        nm.nomas_attn_bwd(plan, qx, k, v, o0, dox, l0, dq, dk, dv, SCALE, workspace=ws)
        torch.cuda.synchronize()
        return dq, dk, dv
    base = bwd(q, d_o)
    qg, dog = q.clone(), d_o.clone()
    qg[pad] = 1.0e3
    dog[pad] = -2.0e3
    got = bwd(qg, dog)
    for b, g2, name in zip(base, got, ("dQ", "dK", "dV")):
        assert torch.equal(b.view(torch.int16), g2.view(torch.int16)), name
    assert (got[0][pad] == 0).all()


def test_thirty_two_actions_and_many_cached_segments():
    """The largest action count a segment may carry (32: every bit of the
    descriptors' tail masks in use) and a cache of 40 small segments, as a
    cached step, against the oracle."""
    need_gpu()
    g = np.random.default_rng(32)
    acts = []
    for a in range(32):
        lo = int(g.integers(0, 4))
        acts.append((int(g.integers(1, 4)), lo, int(g.integers(lo + 1, 5))))
    big = wl.Segment(0, 40, 4, 16, 6, acts, n_pad=5)
    cached = [wl.Segment(0, j, 1, 16, 2, [(1, 0, 1)]) for j in range(40)]
    say(f"32 actions in one segment ({big.n_tokens} tokens) over 40 cached segments")
    cache = new_cache(2, 40 * 19 + big.n_tokens)
    kc = wl.randn((40 * 19, 2, 128), 3201)
    vc = wl.randn((40 * 19, 2, 128), 3202)
    fill_cache(cache, cached, dev(kc), dev(vc))
    q, kn, vn = (wl.randn((big.n_tokens, 2, 128), 3203 + i) for i in range(3))
    plan = nm.nomas_attn_plan([big], [big], cache, heads=2)
    o, l = run_fwd(plan, cache, dev(q), dev(kn), dev(vn), 2)
    keys = cached + [big]
    tq, tk = oracle.expand([big]), oracle.expand(keys)
    o_ref, l_ref, l_bnd = oracle_forward(q, np.concatenate([kc, kn]), np.concatenate([vc, vn]), tq, tk, SCALE)
    check_o(host(o), o_ref, "32 actions, 40 cached segments")
    check_lse(host(l), l_ref, "32 actions, 40 cached segments", l_bnd)


def test_single_token_and_empty_query():
    need_gpu()
    s1 = [wl.Segment(0, 0, 1, 1, 0, [])]
    q = dev(wl.randn((1, 2, 128), 5))
    plan = nm.nomas_attn_plan(s1, s1, heads=2)
    o, l = run_fwd(plan, None, q, q, q, 2)
    assert torch.allclose(o.float(), q.float(), atol=0, rtol=2 ** -8)   # softmax over one key
    # no queries: a no-op that still validates arguments
    plan0 = nm.nomas_attn_plan([], s1, heads=2)
    o0 = torch.empty((0, 2, 128), dtype=torch.bfloat16, device="cuda")
    nm.nomas_attn_fwd(plan0, None, o0, q, q, o0, None, SCALE)
    # a plan whose queries see nothing at all (padding only): zeros and -inf
    sp = [wl.Segment(0, 0, 0, 0, 0, [], n_pad=200)]
    qp = dev(wl.randn((200, 2, 128), 6))
    o_p, l_p = run_fwd(nm.nomas_attn_plan(sp, sp, heads=2), None, qp, qp, qp, 2)
    assert (o_p == 0).all() and torch.isinf(l_p).all() and (l_p < 0).all()
    torch.cuda.synchronize()


def test_stale_plan_after_append_and_truncate():
    need_gpu()
    w = wl.cached_step_480p(n_cached=2)
    cache, kc, vc = build_cached(w)
    plan = nm.nomas_attn_plan(w.q_layout, w.new, cache, heads=16)
    q, kn, vn = dev(w.q()), dev(w.k_new()), dev(w.v_new())
    o_a, _ = run_fwd(plan, cache, q, kn, vn, 16)
    nm.nomas_kvcache_append(cache, w.new[0], kn, vn)
    with pytest.raises(nm.NomasError) as e:
        run_fwd(plan, cache, q, kn, vn, 16)
    assert e.value.status == 5
    nm.nomas_kvcache_truncate(cache, 2)          # back to the contents the plan saw
    o_b, _ = run_fwd(plan, cache, q, kn, vn, 16)
    assert torch.equal(o_a, o_b)
    # capacity: nothing written, nothing recorded
    small = new_cache(16, 100)
    before = small.k_buf.clone()
    with pytest.raises(nm.NomasError) as e:
        nm.nomas_kvcache_append(small, w.new[0], kn, vn)
    assert e.value.status == 4 and nm.nomas_kvcache_len(small) == (0, 0)
    torch.cuda.synchronize()
    assert torch.equal(before, small.k_buf)


def test_long_session_720p_sampled_rows():
    """Full 720p session shape (16 cached segments, 113664 stored rows), 4 denoising
    calls, then the append; outputs checked on sampled rows and heads."""
    need_gpu()
    w = wl.long_session_720p()
    say("720p long session: 16 cached x 7104 stored rows + 7232 new = 120896 keys, 4 calls")
    cache, kc, vc = build_cached(w)
    plan = nm.nomas_attn_plan(w.q_layout, w.new, cache, heads=16)
    keys = w.cached + w.new
    g = np.random.default_rng(44)
    rows = np.sort(np.concatenate([g.choice(w.n_q, 40, replace=False),
                                   np.arange(w.n_q - 300, w.n_q, 37)]))
    heads = [2, 9]
    for nfe in range(4):
        q, kn, vn = w.q(nfe), w.k_new(nfe), w.v_new(nfe)
        o, l = run_fwd(plan, cache, dev(q), dev(kn), dev(vn), 16)
        o_ref, l_ref, l_bnd = oracle_fwd(w, q, np.concatenate([kc, kn]), np.concatenate([vc, vn]), keys,
                                  rows=rows, heads=heads)
        check_o(host(o)[rows][:, heads], o_ref, f"720p long session call {nfe}")
        check_lse(host(l)[heads][:, rows], l_ref, f"720p long session call {nfe}", l_bnd)
    nm.nomas_kvcache_append(cache, w.new[0], dev(kn), dev(vn))   # K/V of the last call
    torch.cuda.synchronize()
    n_old, n_add = len(stored_rows(w.cached)), len(stored_rows(w.new))
    assert nm.nomas_kvcache_len(cache) == (n_old + n_add, 17)
    got = cache.k_buf[:, n_old:n_old + n_add].permute(1, 0, 2)
    assert torch.equal(got, dev(kn[stored_rows(w.new)]))


@pytest.mark.timeout(900)
def test_long_session_720p_two_heads_split_units():
    """One GPU's share of the 720p session when 16 heads are sharded over 8
    GPUs: 2 heads, 29 query-tile pairs each, i.e. 58 units on 256 persistent
    workgroups, so every unit is cut into several pieces and merged; every
    row of the call (all 7,232 queries, both heads) against the oracle."""
    need_gpu()
    w = wl.long_session_720p()
    H = 2
    say("720p long session at 2 heads: 58 units split over 256 workgroups")
    kc, vc = w.cache_kv()
    kc, vc = np.ascontiguousarray(kc[:, :H]), np.ascontiguousarray(vc[:, :H])
    cache = new_cache(H, w.n_cached + w.n_new)
    fill_cache(cache, w.cached, dev(kc), dev(vc))
    plan = nm.nomas_attn_plan(w.q_layout, w.new, cache, heads=H)
    q = np.ascontiguousarray(w.q(0)[:, :H])
    kn = np.ascontiguousarray(w.k_new(0)[:, :H])
    vn = np.ascontiguousarray(w.v_new(0)[:, :H])
    o, l = run_fwd(plan, cache, dev(q), dev(kn), dev(vn), H)
    rows = np.arange(w.n_q)
    keys = w.cached + w.new
    o_ref, l_ref, l_bnd = oracle_fwd(w, q, np.concatenate([kc, kn]), np.concatenate([vc, vn]), keys,
                              rows=rows)
    check_o(host(o)[rows], o_ref, "720p, 2 heads")
    check_lse(host(l)[:, rows], l_ref, "720p, 2 heads", l_bnd)


@pytest.mark.parametrize("window", [1, 2])
def test_cached_step_480p_sliding_window(window):
    """Sliding window over whole segments: the new segment sees only itself
    (window 1) or itself and the last cached segment (window 2); the older
    cached tiles are EMPTY and never loaded."""
    need_gpu()
    w = wl.cached_step_480p()
    say(f"480p cached step, window of {window} segment(s)")
    cache, kc, vc = build_cached(w)
    plan = nm.nomas_attn_plan(w.q_layout, w.new, cache, heads=16, window=window)
    q, kn, vn = w.q(), w.k_new(), w.v_new()
    o, l = run_fwd(plan, cache, dev(q), dev(kn), dev(vn), 16)
    keys = w.cached + w.new
    o_ref, l_ref, l_bnd = oracle_fwd(w, q, np.concatenate([kc, kn]), np.concatenate([vc, vn]), keys,
                              heads=[1, 14], window=window)
    check_o(host(o)[:, [1, 14]], o_ref, f"window {window}")
    check_lse(host(l)[[1, 14]], l_ref, f"window {window}", l_bnd)


def test_training_pack_131k_forward_sampled():
    need_gpu()
    w = wl.training_pack_131k()
    say("training pack: 131072 tokens, 4 videos, forward on sampled rows")
    plan, q, k, v, keys = dense_case(w)
    o, l = run_fwd(plan, None, dev(q), dev(k), dev(v), 16)
    g = np.random.default_rng(55)
    rows = np.sort(g.choice(w.n_q, 48, replace=False))
    o_ref, l_ref, l_bnd = oracle_fwd(w, q, k, v, keys, rows=rows, heads=[0, 13])
    check_o(host(o)[rows][:, [0, 13]], o_ref, "training pack fwd")
    check_lse(host(l)[[0, 13]][:, rows], l_ref, "training pack fwd", l_bnd)


@pytest.mark.timeout(900)
def test_training_pack_131k_forward_whole_video():
    """Every query row of one whole video of the 131072-token pack (video 2,
    32,768 rows: all its segments, heads, tails and padding), two heads,
    against the oracle run on that video alone (the pack is block-diagonal
    over videos), rows in blocks of 512."""
    need_gpu()
    w = wl.training_pack_131k()
    segs = w.q_layout
    plan, q, k, v, keys = dense_case(w)
    o, l = run_fwd(plan, None, dev(q), dev(k), dev(v), 16)
    starts = np.cumsum([0] + [s.n_tokens for s in segs])
    v2 = [i for i, s in enumerate(segs) if s.video == 2]
    lo, hi = int(starts[v2[0]]), int(starts[v2[-1] + 1])
    say(f"training pack: video 2 = rows [{lo}, {hi}), {len(v2)} segments, heads 5 and 10")
    t = oracle.expand(segs[v2[0]:v2[-1] + 1])
    heads = [5, 10]
    o_ref, l_ref, l_bnd = oracle_forward(q[lo:hi], k[lo:hi], v[lo:hi], t, t, SCALE, heads=heads)
    check_o(host(o)[lo:hi][:, heads], o_ref, "training pack, whole video 2")
    check_lse(host(l)[heads][:, lo:hi], l_ref, "training pack, whole video 2", l_bnd)


def test_cache_resume_by_adopt_bitwise():
    """A second handle over the same K/V buffers adopts the cached segments
    (as a new process would after restoring them): plans of either handle
    run on either, bit-identical to the forward over the cache that was
    filled by appends."""
    need_gpu()
    w = wl.cached_step_480p()
    cache, kc, vc = build_cached(w)
    resumed = nm.nomas_kvcache_create(16, w.n_cached + w.n_new, cache.k_buf, cache.v_buf)
    nm.nomas_kvcache_adopt(resumed, w.cached)
    assert nm.nomas_kvcache_len(resumed) == nm.nomas_kvcache_len(cache)
    q, kn, vn = dev(w.q(1)), dev(w.k_new(1)), dev(w.v_new(1))
    plan = nm.nomas_attn_plan(w.q_layout, w.new, cache, heads=16)
    plan_r = nm.nomas_attn_plan(w.q_layout, w.new, resumed, heads=16)
    o1, l1 = run_fwd(plan, cache, q, kn, vn, 16)
    o2, l2 = run_fwd(plan, resumed, q, kn, vn, 16)
    o3, l3 = run_fwd(plan_r, resumed, q, kn, vn, 16)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    # the resumed cache keeps growing like the original
    nm.nomas_kvcache_append(resumed, w.new[0], kn, vn)
    assert nm.nomas_kvcache_len(resumed)[1] == len(w.cached) + 1
    with pytest.raises(nm.NomasError) as e:
        nm.nomas_attn_fwd(plan_r, resumed, q, kn, vn, torch.empty_like(q), None, SCALE,
                          workspace=torch.empty(max(nm.nomas_attn_fwd_workspace_size(plan_r), 16),
                                                dtype=torch.uint8, device="cuda"))
    assert e.value.status == 5  # stale plan


def test_int8_cache_resume_by_adopt_bitwise():
    """The same for an INT8 cache: a handle over the same codes adopts the
    segments, and its expansion equals the original's bit for bit."""
    need_gpu()
    w = wl.cached_step_480p()
    kc, vc = w.cache_kv()
    cap = w.n_cached + w.n_new
    c8 = nm.nomas_kvcache_int8_create(16, cap)
    off = 0
    kd, vd = dev(kc), dev(vc)
    for s in w.cached:
        nm.nomas_kvcache_int8_append(c8, s, kd[off:off + s.n_tokens], vd[off:off + s.n_tokens])
        off += s.n_tokens
    r8 = nm.nomas_kvcache_int8_create(16, cap, buffers=(c8.k_codes, c8.v_codes, c8.k_exp, c8.v_exp))
    nm.nomas_kvcache_int8_adopt(r8, w.cached)
    works = []
    for c in (c8, r8):
        wk = new_cache(16, cap)
        nm.nomas_kvcache_int8_expand(c, wk)
        works.append(wk)
    torch.cuda.synchronize()
    n = nm.nomas_kvcache_len(works[0])[0]
    assert nm.nomas_kvcache_len(works[1])[0] == n > 0
    assert torch.equal(works[0].k_buf[:, :n], works[1].k_buf[:, :n])
    assert torch.equal(works[0].v_buf[:, :n], works[1].v_buf[:, :n])
