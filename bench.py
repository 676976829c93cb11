#!/usr/bin/env python3
"""Benchmark: effective TFLOP/s of the action-aware causal attention forward.

Workload (default): the 480p segment-autoregressive step -- 4 cached segments
(3120 video + 64 head + 3 x 32 tail tokens each) plus the new segment as
queries, 16 heads x 128, bf16.  One timed *step* is one segment step of the
denoising loop over L layers: for each of the 4 denoising calls, the forward
of every layer (each layer reads its own cache, so no call finds its K/V warm
in the last-level cache), then the append of the new segment's K/V to every
layer's cache.  The host plan is built once per segment step and shared by all
layers and calls; its time is reported separately.

value = 4 * 128 * 16 * A * (4 calls * L layers) / step time, A = unmasked pairs.
roofline = one forward call (the persistent forward kernel plus the small
kernel that merges split query tiles, back to back on one stream): the same
effective FLOPs per call / the call's average duration (HIP events on the
launch stream), against the bf16 dense MFMA peak of MI355X.
cpu_baseline = the fp64 oracle on one forward call of the same workload.
long_session (extra) = the 720p long session: 4 forward calls over 16 cached
segments + the new one (120,896 keys read: the cache keeps video and head
rows), then the append.
training_pack (extra, not the headline) = forward and backward times on the
131072-token training pack; backward effective TFLOP/s counts 8 D H A flops
(four products) and, beside it, the FlashAttention convention 10 D H A;
training_pack_kv_head_major: the same with K, V, dK, dV head-major.
sparse_step (extra) = the 480p step with its last two denoising calls keeping
25% of the video key tiles (video-block sparsity) and the first two dense.
long_session_window4 (extra) = the same session with a sliding window of 4
segments (whole segments; older ones, heads included, are not visible).
sp8_share (extra) = both rows again at 2 heads, one GPU's share when the 16
heads are sharded over 8 GPUs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0


# Every source the forward launch is compiled from or scheduled by: the
# kernels, their shared device helpers and interface, the C ABI that fills the
# launch parameters, and the host plan that builds the schedule.
FWD_SOURCES = ("attn_fwd.hip", "tile_common.h", "kernels.h", "abi.cpp", "plan.cpp", "plan.h")
TRAFFIC_PROFILE = os.path.join("profiles", "attn_fwd_480p_cached_step_traffic.json")


def kernel_hash():
    """Hash of the sources that decide the forward's HBM traffic."""
    h = hashlib.sha256()
    for f in FWD_SOURCES:
        h.update(open(os.path.join(ROOT, "segment_causal_masked_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload):
    """(HBM bytes per forward launch, source) from the committed counter
    summary if it was taken on the current forward sources; else (None, None)."""
    try:
        d = json.load(open(os.path.join(ROOT, TRAFFIC_PROFILE)))
    except (OSError, ValueError):
        return None, None
    if d.get("kernel_sha") != kernel_hash() or d.get("workload") != workload:
        return None, None
    return d.get("hbm_bytes_per_launch"), "profile:" + TRAFFIC_PROFILE


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, runs=3, full=True):
    """The fp64 oracle (numpy, BLAS threads = this process's cores) on one full
    forward call of the same workload -- all 16 heads, every query of the new
    segment against all cached + new keys -- median of `runs` runs."""
    import oracle
    cores, blas = len(os.sched_getaffinity(0)), "unknown"
    try:
        from threadpoolctl import threadpool_info
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if infos:
            cores = max(i.get("num_threads", 1) for i in infos)
            blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in infos}))
    except Exception:
        pass
    keys = w.cached + w.new
    kc, vc = w.cache_kv()
    q = w.q()
    k = np.concatenate([kc, w.k_new()])
    v = np.concatenate([vc, w.v_new()])
    tq, tk = oracle.expand(w.q_layout), oracle.expand(keys)
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        oracle.forward(q, k, v, tq, tk, 128 ** -0.5)
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    a = oracle.unmasked_pairs(tq, tk)
    flop = 4.0 * 128 * w.heads * a
    return {"value": round(flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"one forward call of {w.name} ({w.heads} heads, {w.n_q} queries x "
                      f"{w.n_keys} keys), fp64 numpy, median of {runs} runs: {dt:.2f} s",
            "cpu": cpu_model(), "blas": blas, "other_workloads": cpu_other_workloads(full)}


def cpu_other_workloads(full=True):
    """The oracle on the other shapes, for context: the single 480p segment in
    full (one run); one 720p long-session call in full (one run, all 16 heads,
    rows in blocks of 512; with full=False a 256-query sample scaled by its
    share of the unmasked pairs); and the training pack's forward and
    backward for the 4,096-token slice the GPU tests check (every query of
    its video that sees those keys, 2 heads, one run)."""
    import oracle
    from segment_causal_masked_amd import workloads as wl
    out = {}
    w = wl.single_segment_480p()
    tq = tk = oracle.expand(w.q_layout)
    t0 = time.perf_counter()
    oracle.forward(w.q(), w.k_new(), w.v_new(), tq, tk, 128 ** -0.5)
    dt = time.perf_counter() - t0
    a = oracle.unmasked_pairs(tq, tk)
    out["single_segment_480p"] = {"seconds": round(dt, 3), "tflops": round(4.0 * 128 * w.heads * a / dt / 1e12, 6),
                                  "sample": "whole call, one run"}
    w = wl.long_session_720p()
    keys = w.cached + w.new
    tq, tk = oracle.expand(w.q_layout), oracle.expand(keys)
    kc, vc = w.cache_kv()
    k = np.concatenate([kc, w.k_new()])
    v = np.concatenate([vc, w.v_new()])
    a_all = oracle.unmasked_pairs(tq, tk)
    if full:
        t0 = time.perf_counter()
        oracle.forward(w.q(), k, v, tq, tk, 128 ** -0.5)
        dt = time.perf_counter() - t0
        out["long_session_720p"] = {"seconds": round(dt, 2),
                                    "tflops": round(4.0 * 128 * w.heads * a_all / dt / 1e12, 6),
                                    "sample": "one whole call (7,232 queries x 122,944 keys, 16 heads), "
                                              "rows in blocks of 512, one run"}
    else:
        rows = np.arange(w.n_q - 256, w.n_q)  # the last 256 queries (video, head and tail tokens)
        t0 = time.perf_counter()
        oracle.forward(w.q(), k, v, tq, tk, 128 ** -0.5, rows=rows)
        dt = time.perf_counter() - t0
        a_rows = oracle.unmasked_pairs(tq.take(rows), tk)
        out["long_session_720p"] = {"seconds_sample": round(dt, 3),
                                    "seconds_per_call_scaled": round(dt * a_all / a_rows, 1),
                                    "tflops": round(4.0 * 128 * w.heads * a_rows / dt / 1e12, 6),
                                    "sample": "256 of 7,232 queries, all keys and heads, one run"}
    # training pack: the 4,096-token slice starting 2,048 tokens before video
    # 1's third segment; forward for its rows, backward for its dQ rows and
    # dK / dV rows (which needs every query of video 1)
    w = wl.training_pack_131k()
    segs = w.q_layout
    starts = np.cumsum([0] + [s.n_tokens for s in segs])
    v1 = [i for i, s in enumerate(segs) if s.video == 1]
    t_lo, t_hi = int(starts[v1[0]]), int(starts[v1[-1] + 1])
    rows = np.arange(int(starts[v1[2]]) - 2048, int(starts[v1[2]]) + 2048) - t_lo
    t = oracle.expand(segs[v1[0]:v1[-1] + 1])
    heads = [2, 11]
    vs = slice(t_lo, t_hi)
    q, k, v, d_o = w.q()[vs], w.k_new()[vs], w.v_new()[vs], w.d_o()[vs]
    t0 = time.perf_counter()
    oracle.forward(q, k, v, t, t, 128 ** -0.5, rows=rows, heads=heads)
    t1 = time.perf_counter()
    oracle.backward(q, k, v, d_o, t, t, 128 ** -0.5, heads=heads, q_rows=rows, k_rows=rows)
    t2 = time.perf_counter()
    a_video = oracle.unmasked_pairs(t, t)
    out["training_pack_slice"] = {"fwd_seconds": round(t1 - t0, 2), "bwd_seconds": round(t2 - t1, 2),
                                  "video_tokens": int(t_hi - t_lo), "heads": len(heads),
                                  "bwd_tflops_8DHA": round(8.0 * 128 * len(heads) * a_video / (t2 - t1) / 1e12, 6),
                                  "sample": "4,096-token slice of video 1 (forward rows; backward over "
                                            "every query of video 1), 2 heads, one run"}
    return out


def mfma_probe(torch, iters=20000):
    """The MFMA throughput probe (segment_causal_masked_amd/probe): dense bf16
    TFLOP/s of back-to-back v_mfma_f32_32x32x16_bf16 with no memory traffic
    and the shader clock meanwhile (the practical ceiling of the roofline)."""
    import ctypes as C
    lib = C.CDLL(os.path.join(ROOT, "segment_causal_masked_amd", "libnomas_probe.so"))
    lib.nomas_probe_mfma.restype = C.c_int
    lib.nomas_probe_mfma.argtypes = [C.c_int] + [C.POINTER(C.c_double)] * 3
    tf, mhz, ms = C.c_double(), C.c_double(), C.c_double()
    rc = lib.nomas_probe_mfma(iters, C.byref(tf), C.byref(mhz), C.byref(ms))
    if rc != 0:
        return {"error": f"hip error {rc}"}
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    at_clock = cus * mhz.value * 1e6 * 4096 / 1e12
    return {"tflops": round(tf.value, 1), "clock_mhz": round(mhz.value, 1), "ms": round(ms.value, 3),
            "cus": cus, "peak_at_clock_tflops": round(at_clock, 1),
            "frac_of_published_peak": round(tf.value / PEAK_BF16_TFLOPS, 4)}


def bench_training(nm, wl, torch, iters=5, warmup=2, heads=None, kv_head_major=False):
    """Forward + backward on the 131072-token training pack (4 videos, 16 heads,
    or `heads` of them: one GPU's share when heads are sharded): mean time of
    each over `iters` calls after `warmup`, HIP events on the launch stream.
    kv_head_major: K, V, dK, dV in head-major [H][tokens][128] buffers.
    Inputs are drawn on the device (timing only)."""
    w = wl.training_pack_131k()
    H, D = heads or w.heads, 128
    t0 = time.perf_counter()
    plan = nm.nomas_attn_plan(w.q_layout, w.q_layout, heads=H, kv_head_major=kv_head_major)
    plan_ms = (time.perf_counter() - t0) * 1e3
    info = plan.info()
    A = info.unmasked_pairs
    g = torch.Generator(device="cuda")
    g.manual_seed(5000)
    mk = lambda: torch.randn((w.n_q, H, D), generator=g, device="cuda").to(torch.bfloat16)
    q, k, v, d_o = mk(), mk(), mk(), mk()
    if kv_head_major:
        k, v = k.permute(1, 0, 2).contiguous(), v.permute(1, 0, 2).contiguous()
    o = torch.empty_like(q)
    lse = torch.empty((H, w.n_q), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    fws = torch.empty(max(nm.nomas_attn_fwd_workspace_size(plan), 16), dtype=torch.uint8, device="cuda")
    bws = torch.empty(max(nm.nomas_attn_bwd_workspace_size(plan), 16), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    fwd_ms, bwd_ms = [], []
    for it in range(warmup + iters):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        nm.nomas_attn_fwd(plan, None, q, k, v, o, lse, D ** -0.5, workspace=fws)
        e[1].record(stream)
        nm.nomas_attn_bwd(plan, q, k, v, o, d_o, lse, dq, dk, dv, D ** -0.5, workspace=bws)
        e[2].record(stream)
        torch.cuda.synchronize()
        if it >= warmup:
            fwd_ms.append(e[0].elapsed_time(e[1]))
            bwd_ms.append(e[1].elapsed_time(e[2]))
    f, b = float(np.mean(fwd_ms)), float(np.mean(bwd_ms))
    return {"workload": w.name, "tokens": w.n_q, "heads": H, "unmasked_pairs": A,
            "kv_layout": "head-major" if kv_head_major else "token-major",
            "plan_host_ms": round(plan_ms, 2),
            "fwd_ms": round(f, 3), "fwd_tflops": round(4.0 * D * H * A / (f * 1e-3) / 1e12, 2),
            "bwd_ms": round(b, 3),
            "bwd_tflops_8DHA": round(8.0 * D * H * A / (b * 1e-3) / 1e12, 2),
            "bwd_tflops_10DHA": round(10.0 * D * H * A / (b * 1e-3) / 1e12, 2),
            "iters": iters}


def bench_long_session(nm, wl, torch, sessions=3, warmup=1, heads=None, n_caches=1, window=0):
    """720p long session: 16 cached segments (7,232 tokens each) + the new
    segment; per session 4 forward calls with fresh Q / K_new / V_new, then the
    append of the new segment (rolled back after each session).  With `heads`
    below 16 (one GPU's share when heads are sharded) the caches are small
    enough to stay in the last-level cache, so `n_caches` identical caches
    are rotated, one per call.  Inputs are drawn on the device (timing only)."""
    w = wl.long_session_720p()
    H, D = heads or w.heads, 128
    g = torch.Generator(device="cuda")
    g.manual_seed(4000)
    rnd = lambda n: torch.randn((n, H, D), generator=g, device="cuda").to(torch.bfloat16)
    cap = w.n_cached + w.n_new
    caches = []
    for _ in range(n_caches):
        kb = torch.empty((H, cap, D), dtype=torch.bfloat16, device="cuda")
        vb = torch.empty_like(kb)
        c = nm.nomas_kvcache_create(H, cap, kb, vb)
        for s in w.cached:
            nm.nomas_kvcache_append(c, s, rnd(s.n_tokens), rnd(s.n_tokens))
        caches.append(c)
    cache = caches[0]
    t0 = time.perf_counter()
    plan = nm.nomas_attn_plan(w.q_layout, w.new, cache, heads=H, window=window)
    plan_ms = (time.perf_counter() - t0) * 1e3
    plans = [plan] + [nm.nomas_attn_plan(w.q_layout, w.new, c, heads=H, window=window)
                      for c in caches[1:]]
    pinfo = plan.info()
    A = pinfo.unmasked_pairs
    qs = [rnd(w.n_q) for _ in range(4)]
    ks = [rnd(w.n_new) for _ in range(4)]
    vs = [rnd(w.n_new) for _ in range(4)]
    o = torch.empty((w.n_q, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, w.n_q), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(nm.nomas_attn_fwd_workspace_size(plan), 16), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    call_ms, app_ms, sess_ms = [], [], []
    n_seg = len(w.cached)
    for it in range(warmup + sessions):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        ev[0].record(stream)
        for n in range(4):
            nm.nomas_attn_fwd(plans[n % n_caches], caches[n % n_caches], qs[n], ks[n], vs[n], o, lse,
                              D ** -0.5, workspace=ws)
            ev[n + 1].record(stream)
        nm.nomas_kvcache_append(cache, w.new[0], ks[3], vs[3])
        ev[5].record(stream)
        torch.cuda.synchronize()
        nm.nomas_kvcache_truncate(cache, n_seg)   # back to the contents plans[0] was built on
        if it >= warmup:
            call_ms += [ev[n].elapsed_time(ev[n + 1]) for n in range(4)]
            app_ms.append(ev[4].elapsed_time(ev[5]))
            sess_ms.append(ev[0].elapsed_time(ev[5]))
    c, a = float(np.mean(call_ms)), float(np.mean(app_ms))
    app_bytes = 2 * 2 * w.n_new * H * D * 2
    # keys the call reads: every key tile some query tile sees (all cached rows
    # and new tokens without a window)
    read_tiles = int((nm.nomas_plan_export_classes(plan) != 0).any(axis=0).sum())
    keys_read = min(read_tiles * 64, int(pinfo.n_keys))
    kv_bytes = 2 * keys_read * H * D * 2
    return {"workload": w.name, "queries": w.n_q, "keys": int(pinfo.n_keys), "keys_read": keys_read,
            "heads": H,
            "unmasked_pairs": A, "plan_host_ms": round(plan_ms, 2),
            "fwd_ms_per_call": round(c, 3),
            "fwd_tflops": round(4.0 * D * H * A / (c * 1e-3) / 1e12, 2),
            "kv_stream_gbs": round(kv_bytes / (c * 1e-3) / 1e9, 1),
            "append_ms": round(a, 4), "append_gbs": round(app_bytes / (a * 1e-3) / 1e9, 1),
            "session_ms": round(float(np.mean(sess_ms)), 3), "sessions": sessions,
            "caches_rotated": n_caches, "window_segments": window}


def bench_int8_session(nm, wl, torch, sessions=3, warmup=1):
    """720p long session over an INT8 cache: per session the INT8 cache (16
    cached segments) is expanded into a bf16 working cache, the 4 denoising
    calls run on it, and the new segment is appended to the INT8 cache
    (rolled back after each session).  In a model each layer keeps its own
    INT8 cache and the working cache is shared by the layers: one expansion
    per (layer, segment step).  Inputs are drawn on the device (timing only)."""
    w = wl.long_session_720p()
    H, D = w.heads, 128
    g = torch.Generator(device="cuda")
    g.manual_seed(4100)
    rnd = lambda n: torch.randn((n, H, D), generator=g, device="cuda").to(torch.bfloat16)
    cap = w.n_cached + w.n_new
    c8 = nm.nomas_kvcache_int8_create(H, cap)
    for s in w.cached:
        nm.nomas_kvcache_int8_append(c8, s, rnd(s.n_tokens), rnd(s.n_tokens))
    kb = torch.empty((H, cap, D), dtype=torch.bfloat16, device="cuda")
    work = nm.nomas_kvcache_create(H, cap, kb, torch.empty_like(kb))
    nm.nomas_kvcache_int8_expand(c8, work)
    plan = nm.nomas_attn_plan(w.q_layout, w.new, work, heads=H)
    A = plan.info().unmasked_pairs
    rows, n_seg = nm.nomas_kvcache_int8_len(c8)
    qs = [rnd(w.n_q) for _ in range(4)]
    ks = [rnd(w.n_new) for _ in range(4)]
    vs = [rnd(w.n_new) for _ in range(4)]
    o = torch.empty((w.n_q, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, w.n_q), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(nm.nomas_attn_fwd_workspace_size(plan), 16), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    exp_ms, call_ms, app_ms, sess_ms = [], [], [], []
    for it in range(warmup + sessions):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(7)]
        ev[0].record(stream)
        nm.nomas_kvcache_int8_expand(c8, work)
        ev[1].record(stream)
        for n in range(4):
            nm.nomas_attn_fwd(plan, work, qs[n], ks[n], vs[n], o, lse, D ** -0.5, workspace=ws)
            ev[n + 2].record(stream)
        nm.nomas_kvcache_int8_append(c8, w.new[0], ks[3], vs[3])
        ev[6].record(stream)
        torch.cuda.synchronize()
        nm.nomas_kvcache_int8_truncate(c8, n_seg)
        if it >= warmup:
            exp_ms.append(ev[0].elapsed_time(ev[1]))
            call_ms += [ev[n + 1].elapsed_time(ev[n + 2]) for n in range(4)]
            app_ms.append(ev[5].elapsed_time(ev[6]))
            sess_ms.append(ev[0].elapsed_time(ev[6]))
    e, c, a = float(np.mean(exp_ms)), float(np.mean(call_ms)), float(np.mean(app_ms))
    exp_bytes = 2 * rows * H * (129 + 256)      # K and V: codes + exponent read, bf16 row written
    app_rows = w.new[0].n_frames * w.new[0].tokens_per_frame + w.new[0].n_head
    app_bytes = 2 * app_rows * H * (256 + 129)  # bf16 row read, codes + exponent written
    return {"workload": w.name, "heads": H, "cached_rows": rows, "unmasked_pairs": A,
            "int8_cache_mb": round(2 * cap * H * 129 / 1e6, 1),
            "bf16_cache_mb": round(2 * cap * H * 256 / 1e6, 1),
            "expand_ms": round(e, 4), "expand_gbs": round(exp_bytes / (e * 1e-3) / 1e9, 1),
            "fwd_ms_per_call": round(c, 3),
            "fwd_tflops": round(4.0 * D * H * A / (c * 1e-3) / 1e12, 2),
            "int8_append_ms": round(a, 4), "int8_append_gbs": round(app_bytes / (a * 1e-3) / 1e9, 1),
            "session_ms": round(float(np.mean(sess_ms)), 3), "sessions": sessions}


def bench_camera(nm, wl, torch, iters=20, warmup=3):
    """Camera cross-attention (Eq. 3) with every camera token of a segment
    visible (radius -1) and with the time-aligned reading (radius 0: each
    video token sees its own latent frame's camera token): a 480p segment
    (3,280 tokens, 8 camera tokens) and the 131072-token training pack.  HBM-bound: the figure of merit is the
    algorithmic bytes (Q and O rows, camera K and V) per call time.  `iters`
    back-to-back calls between two HIP events on the launch stream; the 480p
    case rotates 12 query / output buffer pairs (322 MB, more than the 256 MB
    last-level cache) so that rows come from HBM.  Inputs are drawn on the
    device (timing only)."""
    out = {}
    for key, w, n_buf, radius in (("segment_480p", wl.single_segment_480p(), 12, -1),
                                  ("training_pack", wl.training_pack_131k(), 1, -1),
                                  ("segment_480p_radius0", wl.single_segment_480p(), 12, 0),
                                  ("training_pack_radius0", wl.training_pack_131k(), 1, 0)):
        H, D = w.heads, 128
        plan = nm.nomas_camera_attn_plan(w.q_layout, heads=H, radius=radius)
        info = plan.info()
        g = torch.Generator(device="cuda")
        g.manual_seed(7000)
        rnd = lambda n: torch.randn((n, H, D), generator=g, device="cuda").to(torch.bfloat16)
        qs = [rnd(w.n_q) for _ in range(n_buf)]
        outs = [torch.empty_like(qs[0]) for _ in range(n_buf)]
        kc, vc = rnd(w.n_camera), rnd(w.n_camera)
        stream = torch.cuda.current_stream()
        for i in range(warmup):
            nm.nomas_camera_attn_fwd(plan, qs[i % n_buf], kc, vc, outs[i % n_buf], D ** -0.5)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(iters):
            nm.nomas_camera_attn_fwd(plan, qs[i % n_buf], kc, vc, outs[i % n_buf], D ** -0.5)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        gbs = info.algorithmic_bytes / (ms * 1e-3) / 1e9
        out[key] = {"workload": w.name, "tokens": w.n_q, "video_tokens": int(info.n_video_queries),
                    "camera_tokens": int(info.n_camera_tokens), "heads": H, "radius_frames": radius,
                    "ms_per_call": round(ms, 4), "algorithmic_mb": round(info.algorithmic_bytes / 1e6, 2),
                    "gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                    "effective_tflops": round(info.effective_flop / (ms * 1e-3) / 1e12, 3),
                    "buffers_rotated": n_buf, "calls_timed": iters}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-quick", action="store_true",
                    help="oracle context rows on samples only (a 256-query part of the 720p "
                         "call instead of the whole call)")
    ap.add_argument("--no-training", action="store_true",
                    help="skip the extra forward + backward row on the 131072-token pack")
    ap.add_argument("--no-long-session", action="store_true",
                    help="skip the extra 720p long-session row")
    ap.add_argument("--no-sparse", action="store_true",
                    help="skip the extra 480p step whose last two denoising calls are sparse")
    ap.add_argument("--no-sp8-share", action="store_true",
                    help="skip the extra rows at one GPU's share of 16 heads sharded over 8")
    ap.add_argument("--no-int8", action="store_true",
                    help="skip the INT8-cache long-session row")
    ap.add_argument("--no-camera", action="store_true",
                    help="skip the camera cross-attention rows")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this size first (untimed), as a known "
                         "quantity for calibrating HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the attention is sharded by heads across GPUs outside this library).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import segment_causal_masked_amd as nm
    from segment_causal_masked_amd import workloads as wl

    nm.load()
    torch.cuda.set_device(0)
    w = wl.cached_step_480p()
    H, D, L, NFE = w.heads, 128, args.layers, 4
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(torch.bfloat16)

    kc, vc = w.cache_kv()
    kc_d, vc_d = dev(kc), dev(vc)
    caches = []
    for layer in range(L):
        kb = torch.empty((H, w.n_cached + w.n_new, D), dtype=torch.bfloat16, device="cuda")
        vb = torch.empty_like(kb)
        c = nm.nomas_kvcache_create(H, w.n_cached + w.n_new, kb, vb)
        off = 0
        for s in w.cached:
            nm.nomas_kvcache_append(c, s, kc_d[off:off + s.n_tokens], vc_d[off:off + s.n_tokens])
            off += s.n_tokens
        caches.append(c)
    del kc_d, vc_d
    t0 = time.perf_counter()
    plans = [nm.nomas_attn_plan(w.q_layout, w.new, c, heads=H) for c in caches]
    plan_ms = (time.perf_counter() - t0) * 1e3 / L
    info = plans[0].info()
    A = info.unmasked_pairs
    flop_call = 4.0 * D * H * A

    qs = [dev(w.q(n)) for n in range(NFE)]
    ks = [dev(w.k_new(n)) for n in range(NFE)]
    vs = [dev(w.v_new(n)) for n in range(NFE)]
    outs = [torch.empty((w.n_q, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    lses = [torch.empty((H, w.n_q), dtype=torch.float32, device="cuda") for _ in range(L)]
    ws_bytes = nm.nomas_attn_fwd_workspace_size(plans[0])
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    n_cached_segs = len(w.cached)

    # video-block sparse plans for the last two denoising calls (extra row)
    KEEP = 25
    sp_plans = [] if args.no_sparse else \
        [nm.nomas_attn_plan(w.q_layout, w.new, c, heads=H, video_keep_percent=KEEP) for c in caches]
    ws_sparse = torch.empty(max(nm.nomas_attn_fwd_workspace_size(sp_plans[0]), 16), dtype=torch.uint8,
                            device="cuda") if sp_plans else None

    def step(fwd_events=None, app_events=None, sparse=False):
        for n in range(NFE):
            for layer in range(L):
                if fwd_events is not None:
                    e0, e1 = ev(), ev()
                    e0.record(stream)
                if sparse and n >= 2:
                    nm.nomas_attn_fwd(sp_plans[layer], caches[layer], qs[n], ks[n], vs[n], outs[layer],
                                      lses[layer], D ** -0.5, workspace=ws_sparse)
                else:
                    nm.nomas_attn_fwd(plans[layer], caches[layer], qs[n], ks[n], vs[n], outs[layer],
                                      lses[layer], D ** -0.5, workspace=ws)
                if fwd_events is not None:
                    e1.record(stream)
                    fwd_events.append((e0, e1))
        for layer in range(L):
            if app_events is not None:
                a0, a1 = ev(), ev()
                a0.record(stream)
            nm.nomas_kvcache_append(caches[layer], w.new[0], ks[NFE - 1], vs[NFE - 1])
            if app_events is not None:
                a1.record(stream)
                app_events.append((a0, a1))
        # roll the caches back to the segment step's starting contents (host
        # bookkeeping only); the plans built for those contents stay valid
        for c in caches:
            nm.nomas_kvcache_truncate(c, n_cached_segs)

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    probe = mfma_probe(torch)       # untimed: the chip's MFMA ceiling and clock

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region 1: whole steps
    t_start, t_end = ev(), ev()
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps

    # timed region 2: the same steps with per-launch events
    fwd_ev, app_ev = [], []
    for _ in range(args.steps):
        step(fwd_ev, app_ev)
    torch.cuda.synchronize()

    # extra: the step with the last two denoising calls video-block sparse
    sparse_row = None
    if sp_plans:
        for _ in range(args.warmup):
            step(sparse=True)
        s0, s1 = ev(), ev()
        torch.cuda.synchronize()
        s0.record(stream)
        for _ in range(args.steps):
            step(sparse=True)
        s1.record(stream)
        torch.cuda.synchronize()
        ms_sparse_step = s0.elapsed_time(s1) / args.steps
        sp_ev = []
        for _ in range(args.steps):
            step(sp_ev, sparse=True)
        torch.cuda.synchronize()
        per_call = [a.elapsed_time(b) for a, b in sp_ev]
        sparse_calls = [t for i, t in enumerate(per_call) if (i // L) % NFE >= 2]
        dense_entries = nm.nomas_attn_plan(w.q_layout, w.new, caches[0], heads=H, host_only=True,
                                           video_keep_percent=100).info().sparse_list_entries
        kept = sp_plans[0].info().sparse_list_entries
        sparse_row = {"video_keep_percent": KEEP, "dense_calls": 2, "sparse_calls": 2,
                      "step_ms": round(ms_sparse_step, 4),
                      "speedup_vs_dense_step": round(ms_step / ms_sparse_step, 3),
                      "sparse_fwd_ms_per_call": round(float(np.mean(sparse_calls)), 4),
                      "kept_tile_fraction": round(kept / dense_entries, 4)}
    fwd_ms = np.array([a.elapsed_time(b) for a, b in fwd_ev])
    app_ms = np.array([a.elapsed_time(b) for a, b in app_ev])

    value = flop_call * NFE * L / (ms_step * 1e-3) / 1e12
    fwd_avg = float(fwd_ms.mean())
    achieved = flop_call / (fwd_avg * 1e-3) / 1e12
    traffic, traffic_source = traffic_from_profiles(w.name)
    app_bytes = 2 * 2 * w.n_new * H * D * 2  # K and V, read + write
    line = {
        "metric": "effective TFLOP/s of action-aware causal attn fwd; % of bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "queries": w.n_q, "keys": w.n_keys,
                   "keys_read": int(info.n_keys), "heads": H,
                   "head_dim": D, "cached_segments": n_cached_segs, "denoising_calls": NFE,
                   "layers_per_step": L, "unmasked_pairs": A,
                   "tiles": {"full": info.n_full_tiles, "partial": info.n_partial_tiles,
                             "empty": info.n_empty_tiles}},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     # counters cannot be read inside this run (they need the
                     # profiler): the figure, when present, is the committed one
                     # taken on the same forward sources
                     "traffic_source": traffic_source},
        "fwd_ms_per_call": round(fwd_avg, 4),
        "fwd_ms_median": round(float(np.median(fwd_ms)), 4),
        "fwd_calls_timed": int(fwd_ms.size),
        "fwd_ms_min": round(float(fwd_ms.min()), 4),
        "executed_over_effective": round(info.executed_pairs / A, 4),
        "append_ms": round(float(app_ms.mean()), 4),
        "append_gbs": round(app_bytes / (float(app_ms.mean()) * 1e-3) / 1e9, 1),
        "plan_host_ms": round(plan_ms, 3),
        "kernel_sha": kernel_hash(),
        "mfma_probe": probe,
    }
    if sparse_row is not None:
        line["sparse_step"] = sparse_row
    if not args.no_long_session:
        line["long_session"] = bench_long_session(nm, wl, torch)
        # the same session with a sliding window of 4 segments (the new one and
        # the 3 most recent cached ones): cost bounded whatever the session length
        line["long_session_window4"] = bench_long_session(nm, wl, torch, window=4)
    if not args.no_training:
        line["training_pack"] = bench_training(nm, wl, torch)
        line["training_pack_kv_head_major"] = bench_training(nm, wl, torch, kv_head_major=True)
    if not args.no_sp8_share:
        # one GPU's share when the 16 heads are sharded over 8 GPUs (2 heads at
        # full sequence length): 58 query-tile units on 256 CUs, so every unit
        # is split and merged; the four rotated caches exceed the 256 MB
        # last-level cache, as the layers of a real loop would
        share = {"heads": 2}
        if not args.no_long_session:
            share["long_session"] = bench_long_session(nm, wl, torch, heads=2, n_caches=4)
        if not args.no_training:
            share["training_pack"] = bench_training(nm, wl, torch, heads=2)
        line["sp8_share"] = share
    if not args.no_int8 and not args.no_long_session:
        line["long_session_int8_cache"] = bench_int8_session(nm, wl, torch)
    if not args.no_camera:
        line["camera_xattn"] = bench_camera(nm, wl, torch)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, full=not args.cpu_quick)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
