"""GPU parity of the video-block sparse forward through the C ABI: the kept
key-tile lists against the oracle's selection, bit for bit, and the attention
over them against the fp64 oracle; plus the dense equality at 100% and the
invisibility of dropped tiles."""
import numpy as np
import pytest
import torch

import oracle
from oracle import sparse
import segment_causal_masked_amd as nm
from segment_causal_masked_amd import workloads as wl
from gpu_util import (SCALE, check_lse, check_o, dev, fill_cache, host, need_gpu, new_cache,
                      say, stored_rows)

pytestmark = pytest.mark.gpu


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


def test_sparse_lists_bit_exact_480p_cached_step():
    need_gpu()
    w, cache, plan, keys, q, k, v, kn, vn = setup(25)
    info = plan.info()
    say(f"480p cached step, 25% of video tiles: {info.sparse_list_entries} entries per head")
    _, _, ws = run(plan, cache, dev(q), dev(kn), dev(vn))
    lists = ws[:16 * info.sparse_list_entries * 4].view(torch.int32).cpu().numpy()
    lists = lists.reshape(16, info.sparse_list_entries)
    tq, tk = oracle.expand(w.q_layout), oracle.expand(keys)
    kept = sparse.select_tiles(wl.round_to_bf16(q), wl.round_to_bf16(k), tq, tk, 25)
    cls = oracle.tile_classes(tq, tk, 128, 64)
    off = 0
    for u in range(kept.shape[1]):
        seen = (cls[2 * u] != 0) | ((cls[2 * u + 1] != 0) if 2 * u + 1 < cls.shape[0] else False)
        want = np.flatnonzero(kept[0, u] & seen)
        n = len(want)
        for h in range(16):
            want_h = np.flatnonzero(kept[h, u] & seen)
            got = lists[h, off:off + n] >> 4
            np.testing.assert_array_equal(got, want_h, err_msg=f"head {h} pair {u}")
        off += n
    assert off == info.sparse_list_entries


def test_sparse_forward_480p_cached_step():
    need_gpu()
    w, cache, plan, keys, q, k, v, kn, vn = setup(25)
    o, lse, _ = run(plan, cache, dev(q), dev(kn), dev(vn))
    tq, tk = oracle.expand(w.q_layout), oracle.expand(keys)
    kept = sparse.select_tiles(wl.round_to_bf16(q), wl.round_to_bf16(k), tq, tk, 25)
    heads = [0, 6, 13]
    o_ref, l_ref = oracle.forward(q, k, v, tq, tk, SCALE, heads=heads, tile_keep=kept)
    check_o(host(o)[:, heads], o_ref, "sparse 25%")
    check_lse(host(lse)[heads], l_ref, "sparse 25%")
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
    """Changing V (in the cache) on key tiles that head 5 drops for every
    query pair leaves the whole output bit-identical."""
    need_gpu()
    w, cache, plan, keys, q, k, v, kn, vn = setup(25)
    tq, tk = oracle.expand(w.q_layout), oracle.expand(keys)
    kept = sparse.select_tiles(wl.round_to_bf16(q), wl.round_to_bf16(k), tq, tk, 25)
    n_cached_tiles = len(stored_rows(w.cached)) // 64
    dropped = [t for t in np.flatnonzero(~kept[5].any(axis=0)) if t < n_cached_tiles]
    say(f"head 5 drops {len(dropped)} cached tiles for every query pair")
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
    video tiles; lists bit-exact and the attention against the oracle."""
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
    info = plan.info()
    o, lse, ws = run(plan, cache, dev(q), dev(kn), dev(vn))
    tq, tk = oracle.expand(w.q_layout), oracle.expand(keys)
    kept = sparse.select_tiles(q, k, tq, tk, 25, window=2)
    cls = oracle.tile_classes(tq, tk, 128, 64, window=2)
    lists = ws[:16 * info.sparse_list_entries * 4].view(torch.int32).cpu().numpy()
    lists = lists.reshape(16, info.sparse_list_entries)
    off = 0
    for u in range(kept.shape[1]):
        seen = (cls[2 * u] != 0) | ((cls[2 * u + 1] != 0) if 2 * u + 1 < cls.shape[0] else False)
        n = int((kept[0, u] & seen).sum())
        for h in range(16):
            np.testing.assert_array_equal(lists[h, off:off + n] >> 4, np.flatnonzero(kept[h, u] & seen))
        off += n
    heads = [2, 9]
    o_ref, l_ref = oracle.forward(q, k, v, tq, tk, SCALE, heads=heads, window=2, tile_keep=kept)
    check_o(host(o)[:, heads], o_ref, "window 2 + sparse 25%")
    check_lse(host(lse)[heads], l_ref, "window 2 + sparse 25%")


@pytest.mark.timeout(600)
def test_sparse_lists_bit_exact_720p_long_session():
    """Long lists (about 1,900 key tiles per query pair): the bitonic sort at
    2,048 entries, all heads, against the oracle's selection."""
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
    info = plan.info()
    say(f"720p session, 25% of video tiles: {info.sparse_list_entries} entries per head")
    _, _, ws = run(plan, cache, dev(q), dev(kn), dev(np.zeros_like(kn)))
    lists = ws[:16 * info.sparse_list_entries * 4].view(torch.int32).cpu().numpy()
    lists = lists.reshape(16, info.sparse_list_entries)
    tq, tk = oracle.expand(w.q_layout), oracle.expand(keys)
    kept = sparse.select_tiles(q, k, tq, tk, 25)
    cls = oracle.tile_classes(tq, tk, 128, 64)
    off = 0
    for u in range(kept.shape[1]):
        seen = (cls[2 * u] != 0) | ((cls[2 * u + 1] != 0) if 2 * u + 1 < cls.shape[0] else False)
        n = int((kept[0, u] & seen).sum())
        for h in range(16):
            np.testing.assert_array_equal(lists[h, off:off + n] >> 4, np.flatnonzero(kept[h, u] & seen),
                                          err_msg=f"head {h} pair {u}")
        off += n
    assert off == info.sparse_list_entries
