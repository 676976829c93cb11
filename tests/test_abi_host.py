"""Host side of the C ABI, on the CPU: the library loads, exports every
function the header declares, and its plan (descriptors, tile classes, A)
agrees bit for bit with the oracle.  No kernel is launched here."""
import ctypes as C

import numpy as np
import pytest

import oracle
import segment_causal_masked_amd as nm
from segment_causal_masked_amd import _lib
from segment_causal_masked_amd import workloads as wl
from golden_io import load_mask_fixture
from test_oracle_mask import random_tiny_layout


def test_library_exports_every_header_function():
    lib = nm.load()
    names = _lib.header_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(lib, n), n


def host_plan(q, kv, heads=1, mode="R", bq=0, bk=0):
    return nm.nomas_attn_plan(q, kv, heads=heads, mode=mode, host_only=True, block_q=bq, block_k=bk)


@pytest.mark.parametrize("name", ["tiny_two_segments_mask.txt", "pack2_mask.txt"])
def test_plan_matches_hand_built_fixtures(name):
    segs, mask, A, (bq, bk), tmap = load_mask_fixture(name)
    for mode in ("R", "K", "H"):
        p = host_plan(segs, segs, mode=mode, bq=bq, bk=bk)
        assert p.info().unmasked_pairs == A[mode]
        if mode == "R":
            np.testing.assert_array_equal(nm.nomas_plan_export_classes(p), tmap)


def test_plan_classes_random_layouts_and_tiles():
    g = np.random.default_rng(2024)
    for trial in range(150):
        segs = random_tiny_layout(g, n_videos=int(g.integers(1, 4)))
        mode = "RKH"[trial % 3]
        bq, bk = int(g.integers(1, 9)), int(g.integers(1, 9))
        # queries: a random sub-list of the segments; keys: all of them
        nq = int(g.integers(1, len(segs) + 1))
        qsegs = [segs[i] for i in sorted(g.choice(len(segs), nq, replace=False))]
        p = host_plan(qsegs, segs, mode=mode, bq=bq, bk=bk)
        tq, tk = oracle.expand(qsegs), oracle.expand(segs)
        np.testing.assert_array_equal(nm.nomas_plan_export_classes(p),
                                      oracle.tile_classes(tq, tk, bq, bk, mode))
        assert p.info().unmasked_pairs == oracle.unmasked_pairs(tq, tk, mode)


@pytest.mark.parametrize("name,mode", [("tiny_two_segments", "R"), ("single_segment_480p", "R"),
                                       ("single_segment_480p", "K"), ("single_segment_480p", "H"),
                                       ("cached_step_480p", "R"), ("cached_step_480p", "H")])
def test_plan_classes_workloads(name, mode):
    w = wl.WORKLOADS[name]()
    keys = w.cached + w.new
    p = host_plan(w.q_layout, keys, heads=w.heads, mode=mode)
    info = p.info()
    tq, tk = oracle.expand(w.q_layout), oracle.expand(keys)
    cls = nm.nomas_plan_export_classes(p)
    np.testing.assert_array_equal(cls, oracle.tile_classes(tq, tk, 128, 64, mode))
    assert info.unmasked_pairs == oracle.unmasked_pairs(tq, tk, mode)
    assert info.n_full_tiles == int((cls == 1).sum())
    assert info.effective_flop == 4.0 * 128 * w.heads * info.unmasked_pairs


@pytest.mark.slow
def test_plan_classes_long_session_720p_full():
    w = wl.long_session_720p()
    keys = w.cached + w.new
    p = host_plan(w.q_layout, keys, heads=16)
    tq, tk = oracle.expand(w.q_layout), oracle.expand(keys)
    np.testing.assert_array_equal(nm.nomas_plan_export_classes(p),
                                  oracle.tile_classes(tq, tk, 128, 64))
    assert p.info().unmasked_pairs == oracle.unmasked_pairs(tq, tk)


def test_plan_classes_training_pack_sampled_tiles():
    w = wl.training_pack_131k()
    p = host_plan(w.q_layout, w.new, heads=16)
    t = oracle.expand(w.q_layout)
    cls = nm.nomas_plan_export_classes(p)
    assert cls.shape == (1024, 2048)
    rows = list(range(0, 1024, 67)) + [1023]
    np.testing.assert_array_equal(cls[rows], oracle.tile_classes(t, t, 128, 64, q_tiles=rows))
    # A by the hand-derived closed form (all videos, all segments)
    from test_oracle_mask import closed_form_A
    assert p.info().unmasked_pairs == closed_form_A(w.q_layout)
    dens = p.info().unmasked_pairs / float(131072) ** 2
    assert 0.05 < dens < 0.25


# ----------------------------------------------------------------------------
# error paths (all caught on the host before any device work)
# ----------------------------------------------------------------------------

def seg(**kw):
    base = dict(video=0, index=0, n_frames=2, tokens_per_frame=4, n_head=2,
                actions=[(2, 0, 1)], n_pad=0)
    base.update(kw)
    return wl.Segment(**base)


@pytest.mark.parametrize("bad", [
    seg(actions=[(2, 1, 1)]),            # lo == hi
    seg(actions=[(2, 0, 3)]),            # hi > n_frames
    seg(actions=[(0, 0, 1)]),            # tail without tokens
    seg(actions=[(1, 0, 1)] * 33),       # more than 32 actions
    seg(n_frames=0, tokens_per_frame=0, n_head=0, actions=[]),  # empty segment
    seg(video=-1),
])
def test_layout_errors(bad):
    with pytest.raises(nm.NomasError) as e:
        host_plan([bad], [bad])
    assert e.value.status == _lib.ERR_LAYOUT


def test_duplicate_and_mismatched_segments():
    a, b = seg(), seg(n_head=3)
    with pytest.raises(nm.NomasError) as e:
        host_plan([a], [a, a])
    assert e.value.status == _lib.ERR_LAYOUT
    with pytest.raises(nm.NomasError) as e:
        host_plan([a], [b])
    assert e.value.status == _lib.ERR_LAYOUT


def test_unsupported_options():
    a = seg()
    lib = nm.load()
    lay = _lib._Layout([a])
    out = C.c_void_p()
    for hd, bq, bk, want in ((64, 0, 0, _lib.ERR_UNSUPPORTED), (128, 64, 64, _lib.ERR_UNSUPPORTED),
                             (128, 0, 0, _lib.OK)):
        opts = _lib.nomas_plan_opts(1, hd, bq, bk, 0, 0, 0, 0)
        st = lib.nomas_attn_plan(C.byref(lay.c), C.byref(lay.c), None, C.byref(opts), C.byref(out))
        if want == _lib.OK:
            # a device plan needs a device; without one the upload fails with a HIP error
            assert st in (_lib.OK, _lib.ERR_HIP)
            if st == _lib.OK:
                lib.nomas_plan_destroy(out)
        else:
            assert st == want, nm.nomas_last_error()
    opts = _lib.nomas_plan_opts(1, 128, 0, 0, 7, 1, 0, 0)
    assert lib.nomas_attn_plan(C.byref(lay.c), C.byref(lay.c), None, C.byref(opts),
                               C.byref(out)) == _lib.ERR_INVALID_ARGUMENT
    assert lib.nomas_attn_plan(None, C.byref(lay.c), None, C.byref(opts),
                               C.byref(out)) == _lib.ERR_INVALID_ARGUMENT


def test_host_only_plan_cannot_run_and_cache_checks():
    a = seg()
    p = host_plan([a], [a])
    lib = nm.load()
    st = lib.nomas_attn_fwd(p.handle, None, C.c_void_p(256), 128, C.c_void_p(256), C.c_void_p(256),
                            128, C.c_void_p(256), 128, None, 0.1, None, 0, None)
    assert st == _lib.ERR_INVALID_ARGUMENT
    assert "host-only" in nm.nomas_last_error()
    # cache bookkeeping on fake, aligned addresses (never dereferenced here)
    c = C.c_void_p()
    assert lib.nomas_kvcache_create(1, 128, 10, C.c_void_p(256), C.c_void_p(512), C.byref(c)) == 0
    assert lib.nomas_kvcache_create(1, 128, 10, C.c_void_p(258), C.c_void_p(512),
                                    C.byref(C.c_void_p())) == _lib.ERR_ALIGNMENT
    # token strides above 2^24 elements are refused before any device work
    fits = _lib.to_c_segment(seg(actions=[]))  # 10 cached rows: fits
    st = lib.nomas_kvcache_append(c, C.byref(fits), C.c_void_p(256), C.c_void_p(256), (1 << 24) + 8, None)
    assert st == _lib.ERR_INVALID_ARGUMENT and "2^24" in nm.nomas_last_error()
    big = _lib.to_c_segment(seg(n_frames=3, tokens_per_frame=4, actions=[]))  # 14 tokens > 10
    st = lib.nomas_kvcache_append(c, C.byref(big), C.c_void_p(256), C.c_void_p(256), 128, None)
    assert st == _lib.ERR_CAPACITY
    n, s = C.c_int64(-1), C.c_int32(-1)
    assert lib.nomas_kvcache_len(c, C.byref(n), C.byref(s)) == 0 and (n.value, s.value) == (0, 0)
    assert lib.nomas_kvcache_truncate(c, 1) == _lib.ERR_INVALID_ARGUMENT
    lib.nomas_kvcache_destroy(c)
    assert nm.nomas_status_string(_lib.ERR_STALE_PLAN).startswith("stale")


def test_backward_entry_checks_on_host_plans():
    """The backward refuses host-only plans and reports its workspace: two fp32
    row statistics (-delta, -lse * log2 e) per head and padded query row, then
    256 bytes of work-queue counters."""
    a = seg()
    b = seg(index=1)
    p = host_plan([a, b], [a, b], heads=3)
    lib = nm.load()
    n = C.c_size_t()
    assert lib.nomas_attn_bwd_workspace_size(p.handle, C.byref(n)) == 0
    nq = a.n_tokens + b.n_tokens
    assert n.value == 2 * 3 * (-(-nq // 128) * 128) * 4 + 256
    fake = C.c_void_p(256)
    st = lib.nomas_attn_bwd(p.handle, fake, fake, fake, fake, fake, C.c_void_p(512), 3 * 128, 3 * 128,
                            fake, fake, fake, 0.1, fake, n.value, None)
    assert st == _lib.ERR_INVALID_ARGUMENT and "host-only" in nm.nomas_last_error()
    assert lib.nomas_attn_bwd_workspace_size(None, C.byref(n)) == _lib.ERR_INVALID_ARGUMENT


def test_plan_window_matches_oracle_with_gaps():
    """Sliding window: plan A and classes against the oracle, on layouts whose
    key set skips segments (the window counts segment indices, not the
    segments present)."""
    g = np.random.default_rng(4242)
    for trial in range(120):
        segs = random_tiny_layout(g, n_videos=int(g.integers(1, 3)))
        keys = [s for s in segs if g.random() < 0.75] or segs[-1:]
        qsegs = [s for s in segs if g.random() < 0.6] or segs[:1]
        keys = sorted({(s.video, s.index): s for s in keys + qsegs}.values(),
                      key=lambda s: (s.video, s.index))
        window = int(g.integers(1, 4))
        mode = "RKH"[trial % 3]
        bq, bk = int(g.integers(1, 7)), int(g.integers(1, 7))
        p = nm.nomas_attn_plan(qsegs, keys, heads=1, mode=mode, host_only=True, block_q=bq,
                               block_k=bk, window=window)
        tq, tk = oracle.expand(qsegs), oracle.expand(keys)
        np.testing.assert_array_equal(nm.nomas_plan_export_classes(p),
                                      oracle.tile_classes(tq, tk, bq, bk, mode, window=window))
        assert p.info().unmasked_pairs == oracle.unmasked_pairs(tq, tk, mode, window=window)


@pytest.mark.parametrize("window", [1, 2])
def test_plan_window_cached_step_480p(window):
    w = wl.cached_step_480p()
    keys = w.cached + w.new
    p = host_plan(w.q_layout, keys, heads=16)
    pw = nm.nomas_attn_plan(w.q_layout, keys, heads=16, host_only=True, window=window)
    tq, tk = oracle.expand(w.q_layout), oracle.expand(keys)
    cls = nm.nomas_plan_export_classes(pw)
    np.testing.assert_array_equal(cls, oracle.tile_classes(tq, tk, 128, 64, window=window))
    assert pw.info().unmasked_pairs == oracle.unmasked_pairs(tq, tk, window=window)
    assert pw.info().unmasked_pairs < p.info().unmasked_pairs


def test_plan_window_rejects_negative():
    segs = wl.tiny_two_segments().q_layout
    with pytest.raises(nm.NomasError):
        nm.nomas_attn_plan(segs, segs, heads=1, host_only=True, window=-1)


@pytest.mark.parametrize("keep", [1, 25, 60, 100])
def test_plan_sparse_list_lengths_match_oracle(keep):
    """The plan sizes each (head, pair) list as its text tiles plus
    ceil(keep% of its video tiles); the oracle's selection kept exactly that."""
    from oracle import sparse
    w = wl.cached_step_480p()
    keys = w.cached + w.new
    p = nm.nomas_attn_plan(w.q_layout, keys, heads=16, host_only=True, video_keep_percent=keep)
    info = p.info()
    assert info.video_keep_percent == keep
    tq, tk = oracle.expand(w.q_layout), oracle.expand(keys)
    q = w.q()[:, :1]
    kc, _ = w.cache_kv()
    k = np.concatenate([kc, w.k_new()])[:, :1]
    kept = sparse.select_tiles(q, k, tq, tk, keep, unit_rows=256, tile_keys=64)
    seen = sparse.candidates(tq, tk, 256, 64) | ~sparse.video_tiles(tk, 64)[None, :]
    cls = oracle.tile_classes(tq, tk, 128, 64)
    total = 0
    for u in range(kept.shape[1]):
        in_list = (cls[2 * u] != 0) | ((cls[2 * u + 1] != 0) if 2 * u + 1 < cls.shape[0] else False)
        assert not (in_list & ~seen[u]).any()
        total += int((kept[0, u] & in_list).sum())
    assert info.sparse_list_entries == total


def test_plan_sparse_rejects_out_of_range():
    segs = wl.tiny_two_segments().q_layout
    for bad in (-1, 101):
        with pytest.raises(nm.NomasError):
            nm.nomas_attn_plan(segs, segs, heads=1, host_only=True, video_keep_percent=bad)


# ---------------------------------------------------------------------------
# camera cross-attention plan
# ---------------------------------------------------------------------------

def _ranges_to_mask(r, n_cam):
    cols = np.arange(n_cam)
    return (cols[None, :] >= r[:, :1]) & (cols[None, :] < r[:, 1:])


@pytest.mark.parametrize("radius", [-1, 0, 1, 2, 5])
def test_camera_plan_matches_oracle_random_layouts(radius):
    from oracle.camera import camera_mask
    g = np.random.default_rng(77 + radius)
    for _ in range(60):
        segs = random_tiny_layout(g, n_videos=int(g.integers(1, 4)))
        p = nm.nomas_camera_attn_plan(segs, heads=2, radius=radius, host_only=True)
        info = p.info()
        m = camera_mask(segs, radius)
        assert info.n_queries == m.shape[0] and info.n_camera_tokens == m.shape[1]
        assert info.visible_pairs == int(m.sum())
        assert info.radius_frames == (radius if radius >= 0 else -1)
        r = nm.nomas_camera_plan_export_ranges(p)
        np.testing.assert_array_equal(_ranges_to_mask(r, m.shape[1]), m)
        assert np.all((r[:, 0] == r[:, 1]) | m.any(axis=1))


@pytest.mark.parametrize("name", ["single_segment_480p", "training_pack_131k"])
def test_camera_plan_workloads(name):
    from oracle.camera import camera_layout
    w = wl.WORKLOADS[name]()
    p = nm.nomas_camera_attn_plan(w.q_layout, heads=16, radius=-1, host_only=True)
    info = p.info()
    q_seg, q_frame, c_seg, c_frame = camera_layout(w.q_layout)
    assert info.n_queries == len(q_seg) and info.n_camera_tokens == len(c_seg)
    assert info.n_video_queries == int((q_seg >= 0).sum())
    per_seg = np.bincount(c_seg, minlength=len(w.q_layout))
    assert info.visible_pairs == int(per_seg[q_seg[q_seg >= 0]].sum())
    assert info.effective_flop == 4 * 128 * 16 * info.visible_pairs
    r = nm.nomas_camera_plan_export_ranges(p)
    vid = q_seg >= 0
    starts = np.concatenate([[0], np.cumsum(per_seg)[:-1]])
    np.testing.assert_array_equal(r[vid, 0], starts[q_seg[vid]])
    np.testing.assert_array_equal(r[vid, 1], starts[q_seg[vid]] + per_seg[q_seg[vid]])
    assert not r[~vid].any()


def test_camera_plan_rejects_bad_arguments():
    segs = [wl.Segment(0, 0, 2, 4, 1, [])]
    with pytest.raises(nm.NomasError) as e:
        nm.nomas_camera_attn_plan(segs, heads=0, host_only=True)
    assert e.value.status == _lib.ERR_INVALID_ARGUMENT
    bad = [wl.Segment(0, 0, 2, 4, 1, [(3, 1, 5)])]  # window past the last frame
    with pytest.raises(nm.NomasError) as e:
        nm.nomas_camera_attn_plan(bad, heads=1, host_only=True)
    assert e.value.status == _lib.ERR_LAYOUT
    p = nm.nomas_camera_attn_plan(segs, heads=1, host_only=True)
    lib = nm.load()
    assert lib.nomas_camera_attn_fwd(p.handle, None, 128, None, None, 128, None, 128,
                                     C.c_float(0.1), None) == _lib.ERR_INVALID_ARGUMENT
    assert "host-only" in nm.nomas_last_error()
    buf = np.zeros(3, np.int32)
    assert lib.nomas_camera_plan_export_ranges(p.handle, buf.ctypes.data_as(C.c_void_p),
                                               buf.size) == _lib.ERR_INVALID_ARGUMENT


def test_int8_cache_create_rejects_bad_arguments():
    lib = nm.load()
    out = C.c_void_p()
    fake = C.c_void_p(0x10000)     # aligned, never dereferenced by create
    odd = C.c_void_p(0x10001)
    assert lib.nomas_kvcache_int8_create(0, 128, 16, fake, fake, fake, fake, C.byref(out)) == _lib.ERR_INVALID_ARGUMENT
    assert lib.nomas_kvcache_int8_create(2, 64, 16, fake, fake, fake, fake, C.byref(out)) == _lib.ERR_UNSUPPORTED
    assert lib.nomas_kvcache_int8_create(2, 128, 16, fake, odd, fake, fake, C.byref(out)) == _lib.ERR_ALIGNMENT
    assert lib.nomas_kvcache_int8_create(2, 128, 16, fake, fake, None, fake, C.byref(out)) == _lib.ERR_INVALID_ARGUMENT
    assert lib.nomas_kvcache_int8_create(2, 128, 16, fake, fake, fake, fake, None) == _lib.ERR_INVALID_ARGUMENT
    assert lib.nomas_kvcache_int8_create(2, 128, 16, fake, fake, fake, fake, C.byref(out)) == _lib.OK
    n, s = C.c_int64(-1), C.c_int32(-1)
    assert lib.nomas_kvcache_int8_len(out, C.byref(n), C.byref(s)) == _lib.OK and (n.value, s.value) == (0, 0)
    assert lib.nomas_kvcache_int8_truncate(out, 1) == _lib.ERR_INVALID_ARGUMENT
    assert lib.nomas_kvcache_int8_destroy(out) == _lib.OK


def test_kvcache_adopt_records_existing_rows():
    """Resume: an empty handle over buffers that already hold rows takes on
    the segments' records (no copy); errors leave it empty."""
    lib = _lib.load()
    segs = wl.cached_step_480p().cached[:2]
    stored = sum(s.n_frames * s.tokens_per_frame + s.n_head for s in segs)
    c = C.c_void_p()
    assert lib.nomas_kvcache_create(2, 128, stored, C.c_void_p(256), C.c_void_p(512), C.byref(c)) == 0
    cache = nm.KVCache(c.value, None, None, 2, stored)
    arr = (_lib.nomas_segment * 3)(*[_lib.to_c_segment(s) for s in segs + segs[:1]])
    # too many rows: CAPACITY, nothing recorded
    assert lib.nomas_kvcache_adopt(c, arr, 3) in (_lib.ERR_CAPACITY, _lib.ERR_LAYOUT)
    assert nm.nomas_kvcache_len(cache) == (0, 0)
    big = (_lib.nomas_segment * 3)(*[_lib.to_c_segment(s) for s in wl.cached_step_480p().cached[:3]])
    assert lib.nomas_kvcache_adopt(c, big, 3) == _lib.ERR_CAPACITY
    # a segment listed twice, a malformed record
    assert lib.nomas_kvcache_adopt(c, (_lib.nomas_segment * 2)(arr[0], arr[0]), 2) == _lib.ERR_LAYOUT
    broken = _lib.to_c_segment(wl.Segment(0, 5, 2, 16, 8, [(4, 1, 1)]))
    assert lib.nomas_kvcache_adopt(c, (_lib.nomas_segment * 1)(broken), 1) == _lib.ERR_LAYOUT
    assert nm.nomas_kvcache_len(cache) == (0, 0)
    nm.nomas_kvcache_adopt(cache, segs)
    assert nm.nomas_kvcache_len(cache) == (stored, 2)
    # not empty any more
    assert lib.nomas_kvcache_adopt(c, arr, 1) == _lib.ERR_INVALID_ARGUMENT
    nm.nomas_kvcache_reset(cache)
    assert lib.nomas_kvcache_adopt(c, arr, 1) == _lib.OK
    assert lib.nomas_kvcache_adopt(None, arr, 1) == _lib.ERR_INVALID_ARGUMENT


@pytest.mark.slow
def test_plan_classes_training_pack_full_map():
    """The whole 1,024 x 2,048 tile-class map of the 131072-token pack, bit
    for bit against the oracle's (slow: every q-tile's mask is materialised)."""
    w = wl.training_pack_131k()
    t = oracle.expand(w.q_layout)
    p = nm.nomas_attn_plan(w.q_layout, w.q_layout, heads=16, host_only=True)
    cls = nm.nomas_plan_export_classes(p)
    assert cls.shape == (1024, 2048)
    np.testing.assert_array_equal(cls, oracle.tile_classes(t, t, 128, 64))
