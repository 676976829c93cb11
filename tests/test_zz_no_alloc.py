"""The allocation-free forward, nomas_attn_fwd_noalloc, through the C ABI.

Its workspace is the library's fixed device array instead of caller memory;
the kernels are those of nomas_attn_fwd, so its outputs must equal that entry
point's bit for bit.  Two calls in a row on the shared array, the second with
a smaller input (and a sparse plan, whose selection also lives in the
array), then an oversized plan, which must be refused before anything runs."""
import numpy as np
import pytest
import torch

import segment_causal_masked_amd as nm
from segment_causal_masked_amd import workloads as wl
from gpu_util import SCALE, dev, fill_cache, need_gpu, new_cache, run_fwd, say

pytestmark = pytest.mark.gpu


def noalloc(plan, cache, q, kn, vn, heads):
    o = torch.empty((q.shape[0], heads, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((heads, q.shape[0]), dtype=torch.float32, device="cuda")
    nm.nomas_attn_fwd_noalloc(plan, cache, q, kn, vn, o, lse, SCALE)
    torch.cuda.synchronize()
    return o, lse


def test_noalloc_forward_equals_the_workspace_forward():
    need_gpu()
    # call 1: the 480p cached step, 16 heads (split units: partials in the array)
    w = wl.cached_step_480p()
    kc, vc = w.cache_kv()
    cache = new_cache(16, w.n_cached + w.n_new)
    fill_cache(cache, w.cached, dev(kc), dev(vc))
    plan = nm.nomas_attn_plan(w.q_layout, w.new, cache, heads=16)
    need = nm.nomas_attn_fwd_workspace_size(plan)
    say(f"480p cached step: workspace {need / 2 ** 20:.1f} MiB in the fixed array")
    assert 0 < need <= 64 << 20
    q, kn, vn = dev(w.q()), dev(w.k_new()), dev(w.v_new())
    o1, l1 = noalloc(plan, cache, q, kn, vn, 16)
    o2, l2 = run_fwd(plan, cache, q, kn, vn, 16)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert np.isfinite(o1.float().cpu().numpy()).all()

    # call 2: a smaller input on the same array (a 4096-token pack, 2 heads)
    w2 = wl.small_pack(0, heads=2)
    segs = w2.q_layout
    plan2 = nm.nomas_attn_plan(segs, segs, heads=2)
    assert nm.nomas_attn_fwd_workspace_size(plan2) < need
    q2, k2, v2 = dev(w2.q()), dev(w2.k_new()), dev(w2.v_new())
    o3, l3 = noalloc(plan2, None, q2, k2, v2, 2)
    o4, l4 = run_fwd(plan2, None, q2, k2, v2, 2)
    say(f"4096-token pack, 2 heads: workspace {nm.nomas_attn_fwd_workspace_size(plan2) / 2 ** 20:.1f} MiB")
    assert torch.equal(o3, o4) and torch.equal(l3, l4)

    # call 3: a sparse plan (selection sums and lists in the array too)
    sp = nm.nomas_attn_plan(w.q_layout, w.new, cache, heads=16, video_keep_percent=25)
    o5, l5 = noalloc(sp, cache, q, kn, vn, 16)
    o6, l6 = run_fwd(sp, cache, q, kn, vn, 16)
    assert torch.equal(o5, o6) and torch.equal(l5, l6)
    assert not torch.equal(o5, o1)


def test_noalloc_refuses_a_plan_above_the_array():
    """A plan whose workspace exceeds 64 MiB (the selection's per-head key-tile
    sums of a long sparse layout at 64 heads) is refused with UNSUPPORTED."""
    need_gpu()
    segs = [wl.Segment(0, j, 8, 880, 64, [], 0) for j in range(20)]
    plan = nm.nomas_attn_plan(segs, segs, heads=64, video_keep_percent=25)
    assert nm.nomas_attn_fwd_workspace_size(plan) > 64 << 20
    t = torch.zeros((8, 64, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(nm.NomasError) as e:
        nm.nomas_attn_fwd_noalloc(plan, None, t, t, t, t, None, SCALE)
    assert e.value.status == 3 and "64" in str(e.value)
