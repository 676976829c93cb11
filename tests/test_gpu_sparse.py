"""GPU parity of the video-block sparse forward through the C ABI.

The kept key-tile lists are checked against the oracle's exact selection
(block score = the exact dot product of a unit's query sum and a tile's key
sum).  The device evaluates that score in fp32, so its ranking can differ
only between tiles whose exact scores lie within the fp32 error bound
(tolerance.score_bound) of each other: every (head, unit) list must hold the
unit's text tiles, the right number of video tiles, and no dropped candidate
whose score exceeds a kept one's by more than their two bounds; where the
exact selection is separated from the rest by more than the bounds, the list
must equal it entry for entry.  The attention over the lists is compared with
the oracle's on the rows of units whose selection is unambiguous; plus the
dense equality at 100% and the invisibility of dropped tiles."""
import numpy as np
import pytest
import torch

import oracle
from oracle import sparse
import segment_causal_masked_amd as nm
from segment_causal_masked_amd import workloads as wl
import tolerance as tol
from gpu_util import (SCALE, check_lse, oracle_forward, check_o, dev, fill_cache, host, need_gpu,
                      new_cache, say, stored_rows)

pytestmark = pytest.mark.gpu

# The library's selection unit (a pair of 128-query tiles) and block (a
# 64-key tile): the reading stated at the boundary (video_keep_percent).
UNIT, TILE = 256, 64


def as_stored(segments):
    """Cached segments as the cache keeps them: video and head rows only."""
    return [wl.Segment(s.video, s.index, s.n_frames, s.tokens_per_frame, s.n_head, [], 0)
            for s in segments]


def setup(keep, nfe=2):
    w = wl.cached_step_480p()
    kc, vc = w.cache_kv()
    cache = new_cache(16, w.n_cached + w.n_new)
    fill_cache(cache, w.cached, dev(kc), dev(vc))
    rows = stored_rows(w.cached)
    keys = as_stored(w.cached) + w.new          # the key rows the call reads, in order
    q, kn, vn = w.q(nfe), w.k_new(nfe), w.v_new(nfe)
    k = np.concatenate([kc[rows], kn])
    v = np.concatenate([vc[rows], vn])
    plan = nm.nomas_attn_plan(w.q_layout, w.new, cache, heads=16, video_keep_percent=keep)
    return w, cache, plan, keys, q, k, v, kn, vn


def run(plan, cache, q, kn, vn):
    n = nm.nomas_attn_fwd_workspace_size(plan)
    ws = torch.zeros(max(n, 16), dtype=torch.uint8, device="cuda")
    o = torch.empty((q.shape[0], 16, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((16, q.shape[0]), dtype=torch.float32, device="cuda")
    nm.nomas_attn_fwd(plan, cache, q, kn, vn, o, lse, SCALE, workspace=ws)
    torch.cuda.synchronize()
    return o, lse, ws


def device_lists(plan, ws):
    info = plan.info()
    lists = ws[:16 * info.sparse_list_entries * 4].view(torch.int32).cpu().numpy()
    return lists.reshape(16, info.sparse_list_entries), info.sparse_list_entries


class Selection:
    """Exact selection of a layout, its fp32 error bounds and the unit lists."""

    def __init__(self, q, k, tq, tk, keep, window=0):
        self.s = sparse.block_scores(q, k, UNIT, TILE)
        self.eps = tol.score_bound(q, k, UNIT, TILE)
        self.vid = sparse.video_tiles(tk, TILE)
        self.exact = sparse.select_tiles(q, k, tq, tk, keep, UNIT, TILE, window=window)
        self.keep = keep
        cls = oracle.tile_classes(tq, tk, 128, TILE, window=window)
        seen = sparse.candidates(tq, tk, UNIT, TILE, window=window)
        self.in_list = []
        for u in range(self.exact.shape[1]):
            lst = (cls[2 * u] != 0) | ((cls[2 * u + 1] != 0) if 2 * u + 1 < cls.shape[0] else False)
            assert np.array_equal(lst & self.vid, seen[u] & self.vid)
            self.in_list.append(lst)

    def separated(self, h, u, kept, dropped):
        s, e = self.s[h, u], self.eps[h, u]
        return not len(kept) or not len(dropped) or (s[kept] - e[kept]).min() > (s[dropped] + e[dropped]).max()

    def check(self, lists, total):
        """Assert the device lists; return the ambiguous (head, unit) pairs."""
        off, n_exact, ambiguous = 0, 0, set()
        heads = self.exact.shape[0]
        for u, lst in enumerate(self.in_list):
            text = np.flatnonzero(lst & ~self.vid)
            cand = np.flatnonzero(lst & self.vid)
            n_keep = -(-len(cand) * self.keep // 100)
            n = len(text) + n_keep
            for h in range(heads):
                got = lists[h, off:off + n] >> 4
                assert (np.diff(got) > 0).all() and lst[got].all(), (h, u)
                assert np.isin(text, got).all(), (h, u)
                kept = got[self.vid[got]]
                assert len(kept) == n_keep, (h, u)
                dropped = np.setdiff1d(cand, kept)
                s, e = self.s[h, u], self.eps[h, u]
                if len(kept) and len(dropped):
                    assert (s[dropped] - e[dropped]).max() <= (s[kept] + e[kept]).min(), (h, u)
                ex_kept = np.flatnonzero(self.exact[h, u] & lst & self.vid)
                if self.separated(h, u, ex_kept, np.setdiff1d(cand, ex_kept)):
                    np.testing.assert_array_equal(got, np.flatnonzero(self.exact[h, u] & lst),
                                                  err_msg=f"head {h} unit {u}")
                    n_exact += 1
                else:
                    ambiguous.add((h, u))
            off += n
        assert off == total
        say(f"  lists: {n_exact} (head, unit) lists equal the exact selection, {len(ambiguous)} "
            f"within the fp32 bound of it")
        assert n_exact > 0
        return ambiguous

    def certainly_dropped(self, h):
        """Video tiles that no unit of head h can keep under any fp32 ranking."""
        out = np.ones(len(self.vid), bool)
        for u, lst in enumerate(self.in_list):
            cand = np.flatnonzero(lst & self.vid)
            n_keep = -(-len(cand) * self.keep // 100)
            s, e = self.s[h, u], self.eps[h, u]
            for t in cand:
                better = ((s[cand] - e[cand]) > s[t] + e[t]).sum()
                if better < n_keep:
                    out[t] = False
        return np.flatnonzero(out & self.vid)


def parity_on_clear_units(o, lse, sel, ambiguous, q, k, v, tq, tk, heads, what, window=0):
    for h in heads:
        units = [u for u in range(sel.exact.shape[1]) if (h, u) not in ambiguous]
        rows = np.concatenate([np.arange(u * UNIT, min(q.shape[0], (u + 1) * UNIT)) for u in units])
        o_ref, l_ref, l_bnd = oracle_forward(q, k, v, tq, tk, SCALE, rows=rows, heads=[h],
                                             window=window, tile_keep=sel.exact, unit_rows=UNIT,
                                             tile_keys=TILE)
        check_o(host(o)[rows][:, [h]], o_ref, f"{what}, head {h}, {len(units)} units")
        check_lse(host(lse)[[h]][:, rows], l_ref, f"{what}, head {h}", l_bnd)


def test_sparse_lists_480p_cached_step():
    need_gpu()
    w, cache, plan, keys, q, k, v, kn, vn = setup(25)
    _, _, ws = run(plan, cache, dev(q), dev(kn), dev(vn))
    lists, total = device_lists(plan, ws)
    say(f"480p cached step, 25% of video tiles: {total} entries per head")
    tq, tk = oracle.expand(w.q_layout), oracle.expand(keys)
    Selection(q, k, tq, tk, 25).check(lists, total)


def test_sparse_forward_480p_cached_step():
    need_gpu()
    w, cache, plan, keys, q, k, v, kn, vn = setup(25)
    o, lse, ws = run(plan, cache, dev(q), dev(kn), dev(vn))
    tq, tk = oracle.expand(w.q_layout), oracle.expand(keys)
    sel = Selection(q, k, tq, tk, 25)
    ambiguous = sel.check(*device_lists(plan, ws))
    parity_on_clear_units(o, lse, sel, ambiguous, q, k, v, tq, tk, [0, 6, 13], "sparse 25%")
    # not the dense result: a real subset of the keys was used
    o_dense, _ = oracle.forward(q, k, v, tq, tk, SCALE, heads=[0])
    assert np.abs(host(o)[:, 0] - o_dense[:, 0]).max() > 5e-2


def test_sparse_keep_all_equals_dense_bitwise():
    need_gpu()
    w, cache, plan, keys, q, k, v, kn, vn = setup(100)
    o_s, l_s, _ = run(plan, cache, dev(q), dev(kn), dev(vn))
    dense = nm.nomas_attn_plan(w.q_layout, w.new, cache, heads=16)
    o_d, l_d, _ = run(dense, cache, dev(q), dev(kn), dev(vn))
    assert torch.equal(o_s, o_d) and torch.equal(l_s, l_d)


def test_dropped_tiles_invisible_bitwise():
    """Changing V (in the cache) on key tiles that head 5 cannot keep in any
    unit (exact score below the keep cut by more than the fp32 bounds) leaves
    the whole output bit-identical."""
    need_gpu()
    w, cache, plan, keys, q, k, v, kn, vn = setup(25)
    tq, tk = oracle.expand(w.q_layout), oracle.expand(keys)
    sel = Selection(q, k, tq, tk, 25)
    n_cached_tiles = len(stored_rows(w.cached)) // 64
    dropped = [t for t in sel.certainly_dropped(5) if t < n_cached_tiles]
    say(f"head 5 drops {len(dropped)} cached tiles for every query unit")
    assert len(dropped) > 0
    o1, l1, _ = run(plan, cache, dev(q), dev(kn), dev(vn))
    for t in dropped:
        cache.v_buf[5, 64 * t:64 * t + 64, :] += 3.0
    o2, l2, _ = run(plan, cache, dev(q), dev(kn), dev(vn))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_sparse_rejected_by_backward():
    need_gpu()
    segs = wl.small_pack(0).q_layout
    plan = nm.nomas_attn_plan(segs, segs, heads=2, video_keep_percent=25)
    t = torch.zeros((wl.layout_tokens(segs), 2, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((2, t.shape[0]), dtype=torch.float32, device="cuda")
    with pytest.raises(nm.NomasError) as e:
        nm.nomas_attn_bwd(plan, t, t, t, t, t, lse, t, t, t, SCALE, workspace=None)
    assert e.value.status == 3


def test_sparse_with_window_480p_cached_step():
    """Both options at once: a 2-segment window, then 25% of the remaining
    video tiles; lists against the exact selection and the attention against
    the oracle."""
    need_gpu()
    w = wl.cached_step_480p()
    kc, vc = w.cache_kv()
    cache = new_cache(16, w.n_cached + w.n_new)
    fill_cache(cache, w.cached, dev(kc), dev(vc))
    rows = stored_rows(w.cached)
    keys = as_stored(w.cached) + w.new
    q, kn, vn = w.q(3), w.k_new(3), w.v_new(3)
    k, v = np.concatenate([kc[rows], kn]), np.concatenate([vc[rows], vn])
    plan = nm.nomas_attn_plan(w.q_layout, w.new, cache, heads=16, window=2, video_keep_percent=25)
    o, lse, ws = run(plan, cache, dev(q), dev(kn), dev(vn))
    tq, tk = oracle.expand(w.q_layout), oracle.expand(keys)
    sel = Selection(q, k, tq, tk, 25, window=2)
    ambiguous = sel.check(*device_lists(plan, ws))
    parity_on_clear_units(o, lse, sel, ambiguous, q, k, v, tq, tk, [2, 9], "window 2 + sparse 25%",
                          window=2)


@pytest.mark.timeout(600)
def test_sparse_lists_720p_long_session():
    """Long lists (about 1,900 key tiles per query unit): the bitonic sort at
    2,048 entries, all heads, against the exact selection."""
    need_gpu()
    w = wl.long_session_720p()
    kc, _ = w.cache_kv()
    cache = new_cache(16, w.n_cached + w.n_new)
    vz = np.zeros_like(kc)
    fill_cache(cache, w.cached, dev(kc), dev(vz))
    rows = stored_rows(w.cached)
    keys = as_stored(w.cached) + w.new
    q, kn = w.q(2), w.k_new(2)
    k = np.concatenate([kc[rows], kn])
    plan = nm.nomas_attn_plan(w.q_layout, w.new, cache, heads=16, video_keep_percent=25)
    _, _, ws = run(plan, cache, dev(q), dev(kn), dev(np.zeros_like(kn)))
    lists, total = device_lists(plan, ws)
    say(f"720p session, 25% of video tiles: {total} entries per head")
    tq, tk = oracle.expand(w.q_layout), oracle.expand(keys)
    Selection(q, k, tq, tk, 25).check(lists, total)


@pytest.mark.timeout(900)
def test_sparse_lists_long_session_past_the_lds_sort():
    """A 720p session of 40 cached segments (291,392 keys: about 4,550 key
    tiles per query unit, past the 4,096 entries the in-LDS sort ranks): the
    radix-select path, all heads, against the exact selection; and the
    attention over its lists on sampled rows of units whose selection is
    unambiguous."""
    need_gpu()
    w = wl.long_session_720p(n_cached=40)
    kc, vc = w.cache_kv()
    cache = new_cache(16, w.n_cached + w.n_new)
    fill_cache(cache, w.cached, dev(kc), dev(vc))
    rows = stored_rows(w.cached)
    keys = as_stored(w.cached) + w.new
    q, kn, vn = w.q(3), w.k_new(3), w.v_new(3)
    plan = nm.nomas_attn_plan(w.q_layout, w.new, cache, heads=16, video_keep_percent=25)
    o, lse, ws = run(plan, cache, dev(q), dev(kn), dev(vn))
    lists, total = device_lists(plan, ws)
    k = np.concatenate([kc[rows], kn])
    del kc
    tq, tk = oracle.expand(w.q_layout), oracle.expand(keys)
    say(f"720p session, 40 cached segments: {len(tk)} keys, {total} entries per head")
    assert (len(tk) + 63) // 64 > 4096
    sel = Selection(q, k, tq, tk, 25)
    ambiguous = sel.check(lists, total)
    v = np.concatenate([vc[rows], vn])
    del vc
    # the ~4,550-tile lists have scores so close together that few units'
    # selections are separated from the rest by the fp32 bound: the attention
    # is compared on those units (every head that has one)
    clear = sorted((h, u) for h in range(16) for u in range(sel.exact.shape[1])
                   if (h, u) not in ambiguous)
    say(f"  units with an unambiguous selection: {clear}")
    assert clear
    g = np.random.default_rng(17)
    for h, u in clear[:4]:
        rows_q = np.sort(g.choice(np.arange(u * UNIT, min(w.n_q, (u + 1) * UNIT)), 16, replace=False))
        o_ref, l_ref, l_bnd = oracle_forward(q, k, v, tq, tk, SCALE, rows=rows_q, heads=[h],
                                             tile_keep=sel.exact, unit_rows=UNIT, tile_keys=TILE)
        check_o(host(o)[rows_q][:, [h]], o_ref, f"long sparse session, head {h} unit {u}")
        check_lse(host(lse)[[h]][:, rows_q], l_ref, f"long sparse session, head {h} unit {u}", l_bnd)


def test_sparse_training_pack_phased_schedule():
    """A pack of two 16,384-token videos (64 query-tile pairs per (head,
    video): its plans take the phased schedule, each XCD on one head's video
    at a time).  Keeping every video tile equals the dense call bit for bit
    (both plans get the same cuts); at 25% the lists are checked against the
    exact selection and the attention against the oracle on sampled rows of
    units whose selection is unambiguous."""
    need_gpu()
    segs = wl.pack_layout(wl.rng(8080), 2, 16384)
    n = wl.layout_tokens(segs)
    say(f"sparse training pack: {n} tokens, 2 videos, 16 heads")
    q, k, v = (wl.randn((n, 16, 128), 8100 + i) for i in range(3))
    qd, kd, vd = dev(q), dev(k), dev(v)
    o_d, l_d, _ = run(nm.nomas_attn_plan(segs, segs, heads=16), None, qd, kd, vd)
    o_a, l_a, _ = run(nm.nomas_attn_plan(segs, segs, heads=16, video_keep_percent=100), None, qd, kd, vd)
    assert torch.equal(o_a.view(torch.int16), o_d.view(torch.int16)) and torch.equal(l_a, l_d)
    plan = nm.nomas_attn_plan(segs, segs, heads=16, video_keep_percent=25)
    o, lse, ws = run(plan, None, qd, kd, vd)
    lists, total = device_lists(plan, ws)
    t = oracle.expand(segs)
    sel = Selection(q, k, t, t, 25)
    ambiguous = sel.check(lists, total)
    clear = sorted((h, u) for h in range(16) for u in range(sel.exact.shape[1]) if (h, u) not in ambiguous)
    g = np.random.default_rng(81)
    picks = [clear[i] for i in sorted(g.choice(len(clear), min(6, len(clear)), replace=False))]
    for h, u in picks:
        rows_q = np.sort(g.choice(np.arange(u * UNIT, min(n, (u + 1) * UNIT)), 16, replace=False))
        o_ref, l_ref, l_bnd = oracle_forward(q, k, v, t, t, SCALE, rows=rows_q, heads=[h],
                                             tile_keep=sel.exact, unit_rows=UNIT, tile_keys=TILE)
        check_o(host(o)[rows_q][:, [h]], o_ref, f"sparse pack, head {h} unit {u}")
        check_lse(host(lse)[[h]][:, rows_q], l_ref, f"sparse pack, head {h} unit {u}", l_bnd)
