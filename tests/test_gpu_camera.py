"""GPU parity of the camera cross-attention kernel against the fp64 oracle
(oracle/camera.py), through the C ABI, plus exact cases checked bitwise."""
import numpy as np
import pytest
import torch

import segment_causal_masked_amd as nm
from oracle.camera import camera_forward, camera_mask
from segment_causal_masked_amd import workloads as wl
from gpu_util import O_MAX_ABS, O_MEAN_ABS, SCALE, dev, host, need_gpu, say

pytestmark = pytest.mark.gpu


def check_o(o_gpu, o_ref, what=""):
    """Gate of the camera cross-attention.  Its outputs average a handful of
    camera values, so they are not the unit-scale averages of the main
    attention: |O| reaches the largest |V| (about 4 for N(0,1) inputs), where
    one bf16 rounding of O alone is up to 2^-9 |O| ~ 8e-3 .. 1.6e-2.  The
    kernel's error is that rounding plus ~1e-5 relative (fp32 scores and
    sums, P to ~16 bits), so: every element within 2^-8 |O_ref| + 2e-4 (one
    bf16 ulp), max-abs 1e-2 on the unit-scale entries (|O_ref| < 2) and
    mean-abs 1e-3 overall."""
    o = o_gpu.astype(np.float64)
    err = np.abs(o - o_ref)
    if not err.size:
        return
    unit = np.abs(o_ref) < 2.0
    mx = float(err[unit].max()) if unit.any() else 0.0
    mean = float(err.mean())
    worst = float((err - 2.0 ** -8 * np.abs(o_ref)).max())
    say(f"  {what}: max-abs (|O|<2) {mx:.3e}, max-abs {float(err.max()):.3e}, mean-abs {mean:.3e}, "
        f"max(err - 2^-8|O|) {worst:.3e}")
    assert np.isfinite(o_gpu).all()
    assert mx <= O_MAX_ABS and mean <= O_MEAN_ABS, (what, mx, mean)
    assert worst <= 2e-4, (what, worst)


def run_camera(segs, q, kc, vc, heads, radius, q_stride=None, o_stride=None):
    plan = nm.nomas_camera_attn_plan(segs, heads=heads, radius=radius)
    n = q.shape[0]

    def strided(x, stride):
        if stride is None:
            return dev(x) if x is not None else torch.empty((n, heads, 128), dtype=torch.bfloat16, device="cuda")
        base = torch.full((n * stride + 64,), 7.0, dtype=torch.bfloat16, device="cuda")
        t = torch.as_strided(base, (n, heads, 128), (stride, 128, 1))
        if x is not None:
            t.copy_(dev(x))
        return t

    qd = strided(q, q_stride)
    o = strided(None, o_stride)
    o.fill_(3.0)  # every row must be written
    kd = dev(kc) if kc.shape[0] else None
    vd = dev(vc) if vc.shape[0] else None
    nm.nomas_camera_attn_fwd(plan, qd, kd, vd, o, SCALE)
    torch.cuda.synchronize()
    return host(o), plan


def inputs(segs, heads, seed):
    n = wl.layout_tokens(segs)
    n_cam = sum(s.n_frames for s in segs)
    return (wl.randn((n, heads, 128), seed), wl.randn((n_cam, heads, 128), seed + 1),
            wl.randn((n_cam, heads, 128), seed + 2))


@pytest.mark.parametrize("radius", [-1, 0, 1])
def test_camera_480p_segment(radius):
    need_gpu()
    w = wl.single_segment_480p()
    say(f"camera cross-attention, 480p segment (3280 tokens, 8 camera tokens, 16 heads), radius {radius}")
    q = w.q()
    kc, vc = w.camera_kv()
    o, plan = run_camera(w.q_layout, q, kc, vc, 16, radius)
    ref = camera_forward(q, kc, vc, w.q_layout, SCALE, radius)
    check_o(o, ref, f"480p camera r={radius}")
    assert plan.info().visible_pairs == int(camera_mask(w.q_layout, radius).sum())


def test_camera_radius0_copies_the_frame_value_exactly():
    need_gpu()
    w = wl.single_segment_480p()
    q = w.q()
    kc, vc = w.camera_kv()
    o, _ = run_camera(w.q_layout, q, kc, vc, 16, 0)
    s = w.q_layout[0]
    frames = np.repeat(np.arange(s.n_frames), s.tokens_per_frame)
    np.testing.assert_array_equal(o[:len(frames)], vc[frames])
    assert not o[len(frames):].any()


def test_camera_training_pack_sampled_rows():
    need_gpu()
    w = wl.training_pack_131k()
    say(f"camera cross-attention, 131072-token pack ({w.n_camera} camera tokens), sampled rows")
    q = w.q()
    kc, vc = w.camera_kv()
    o, _ = run_camera(w.q_layout, q, kc, vc, 16, -1)
    # 4096 rows across the boundary between video 1's segments 1 and 2, plus
    # 2048 random rows of the whole pack
    start = 0
    for s in w.q_layout:
        if s.video == 1 and s.index == 2:
            break
        start += s.n_tokens
    g = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(start - 2048, start + 2048),
                                     g.choice(w.n_q, 2048, replace=False)]))
    ref = camera_forward(q, kc, vc, w.q_layout, SCALE, -1, rows=rows)
    check_o(o[rows], ref, "pack camera, sampled rows")


@pytest.mark.parametrize("radius", [-1, 1])
def test_camera_many_small_segments_per_block(radius):
    need_gpu()
    # 2 frames x 3 tokens + 2 head + 1 tail token: a 32-token block spans
    # several segments (of two videos); 5 heads leave a partial head group
    segs = [wl.Segment(v, j, 2 + (j % 2), 3, 2, [(1, 0, 1)]) for v in range(2) for j in range(9)]
    q, kc, vc = inputs(segs, 5, 900)
    say(f"camera: {len(segs)} small segments, {q.shape[0]} tokens, 5 heads, radius {radius}")
    o, _ = run_camera(segs, q, kc, vc, 5, radius)
    check_o(o, camera_forward(q, kc, vc, segs, SCALE, radius), f"small segments r={radius}")


@pytest.mark.parametrize("radius", [-1, 20])
def test_camera_long_segment_several_chunks(radius):
    need_gpu()
    # 70 latent frames: 70 camera tokens, three 32-key chunks (online softmax
    # across chunks); 4 tokens per frame, 37 text tokens, ragged last block
    segs = [wl.Segment(0, 0, 70, 4, 5, [(32, 3, 60)]), wl.Segment(0, 1, 3, 5, 0, [])]
    q, kc, vc = inputs(segs, 2, 910)
    say(f"camera: a 70-frame segment, {q.shape[0]} tokens, radius {radius}")
    o, _ = run_camera(segs, q, kc, vc, 2, radius)
    check_o(o, camera_forward(q, kc, vc, segs, SCALE, radius), f"long segment r={radius}")


def test_camera_strided_rows_and_text_only_segments():
    need_gpu()
    segs = [wl.Segment(0, 0, 0, 0, 16, []),
            wl.Segment(0, 1, 4, 9, 3, [(2, 1, 3)], 5), wl.Segment(1, 0, 0, 0, 7, [])]
    q, kc, vc = inputs(segs, 3, 920)
    o, _ = run_camera(segs, q, kc, vc, 3, 1, q_stride=3 * 128 + 24, o_stride=3 * 128 + 8)
    check_o(o, camera_forward(q, kc, vc, segs, SCALE, 1), "strided rows")
    assert not o[:16].any() and not o[-7:].any()


def test_camera_layout_without_camera_tokens():
    need_gpu()
    segs = [wl.Segment(0, 0, 0, 0, 40, [])]
    q = wl.randn((40, 2, 128), 930)
    empty = np.zeros((0, 2, 128), np.float32)
    o, plan = run_camera(segs, q, empty, empty, 2, -1)
    assert plan.info().n_camera_tokens == 0
    assert not o.any()


def test_camera_hidden_tokens_do_not_change_outputs():
    need_gpu()
    w = wl.single_segment_480p()
    segs = w.q_layout + [wl.Segment(0, 1, 8, wl.TPF_480P, 64, [(32, 2, 5)])]
    q, kc, vc = inputs(segs, 4, 940)
    o1, _ = run_camera(segs, q, kc, vc, 4, 2)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[7] = wl.round_to_bf16(kc2[7] * -3.0)   # frame 7 of segment 0: hidden from frames 0..4
    vc2[7] = wl.round_to_bf16(vc2[7] + 5.0)
    kc2[8:] = wl.round_to_bf16(kc2[8:] * 2.0)  # segment 1's tokens: hidden from segment 0
    o2, _ = run_camera(segs, q, kc2, vc2, 4, 2)
    tpf = wl.TPF_480P
    np.testing.assert_array_equal(o1[:5 * tpf], o2[:5 * tpf])
    assert not np.array_equal(o1[5 * tpf:8 * tpf], o2[5 * tpf:8 * tpf])
    n0 = segs[0].n_tokens
    np.testing.assert_array_equal(o1[8 * tpf:n0], o2[8 * tpf:n0])  # text rows: zeros
