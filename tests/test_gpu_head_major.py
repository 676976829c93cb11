"""Head-major new-token keys and values (plans built with kv_head_major):
the same kernels read K / V (and write dK / dV) through a head stride instead
of a token stride, with the same arithmetic in the same order.  So every
output must equal, bit for bit, the token-major call on the same values, whose
parity with the oracle the other GPU tests establish.  Head strides are padded
past the rows (a caller's [H][capacity][128] buffer) to catch a kernel that
assumes a packed layout."""
import pytest
import torch

import segment_causal_masked_amd as nm
from segment_causal_masked_amd import workloads as wl
from gpu_util import SCALE, dev, need_gpu, say

pytestmark = pytest.mark.gpu


def head_major(t, pad_rows):
    """[n, H, 128] -> a [H, n, 128] view into a [H, n + pad_rows, 128] buffer
    (head stride (n + pad_rows) * 128) holding the same values."""
    n, h, d = t.shape
    buf = torch.full((h, n + pad_rows, d), float("nan"), dtype=t.dtype, device=t.device)
    view = buf[:, :n]
    view.copy_(t.permute(1, 0, 2))
    return view


def token_major(t):
    """[H, n, 128] -> contiguous [n, H, 128]."""
    return t.permute(1, 0, 2).contiguous()


def fwd(plan, cache, q, k, v, n_q, heads):
    o = torch.empty((n_q, heads, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((heads, n_q), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(nm.nomas_attn_fwd_workspace_size(plan), 16), dtype=torch.uint8, device="cuda")
    nm.nomas_attn_fwd(plan, cache, q, k, v, o, lse, SCALE, workspace=ws)
    torch.cuda.synchronize()
    return o, lse


def same_bits(a, b, what):
    assert a.shape == b.shape, (what, a.shape, b.shape)
    eq = bool(torch.equal(a.contiguous().view(torch.int16 if a.element_size() == 2 else torch.int32),
                          b.contiguous().view(torch.int16 if b.element_size() == 2 else torch.int32)))
    say(f"  {what}: bitwise equal {eq}")
    assert eq, what


@pytest.mark.parametrize("grad_f32", [False, True])
def test_pack_forward_and_backward_equal_token_major_bitwise(grad_f32):
    need_gpu()
    w = wl.small_pack(1)
    segs, heads, n = w.q_layout, w.heads, w.n_q
    say(f"head-major pack: {n} tokens, {heads} heads, {'fp32' if grad_f32 else 'bf16'} gradients")
    q, k, v, d_o = (dev(wl.randn((n, heads, 128), 9300 + i)) for i in range(4))
    pt = nm.nomas_attn_plan(segs, segs, heads=heads, grad_f32=grad_f32)
    ph = nm.nomas_attn_plan(segs, segs, heads=heads, grad_f32=grad_f32, kv_head_major=True)
    kh, vh = head_major(k, 37), head_major(v, 37)
    o_t, l_t = fwd(pt, None, q, k, v, n, heads)
    o_h, l_h = fwd(ph, None, q, kh, vh, n, heads)
    same_bits(o_h, o_t, "O")
    same_bits(l_h, l_t, "LSE")

    gd = torch.float32 if grad_f32 else torch.bfloat16
    nb = max(nm.nomas_attn_bwd_workspace_size(pt), 16)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    dq_t, dk_t, dv_t = (torch.empty((n, heads, 128), dtype=gd, device="cuda") for _ in range(3))
    nm.nomas_attn_bwd(pt, q, k, v, o_t, d_o, l_t, dq_t, dk_t, dv_t, SCALE, workspace=ws)
    dq_h = torch.empty((n, heads, 128), dtype=gd, device="cuda")
    # dK / dV share k's head stride: the same padding
    dkb, dvb = (torch.full((heads, n + 37, 128), float("nan"), dtype=gd, device="cuda") for _ in range(2))
    dk_h, dv_h = dkb[:, :n], dvb[:, :n]
    nm.nomas_attn_bwd(ph, q, kh, vh, o_h, d_o, l_h, dq_h, dk_h, dv_h, SCALE, workspace=ws)
    torch.cuda.synchronize()
    same_bits(dq_h, dq_t, "dQ")
    same_bits(token_major(dk_h), dk_t, "dK")
    same_bits(token_major(dv_h), dv_t, "dV")
    # the padding rows of the head-major gradient buffers stay untouched
    assert torch.isnan(dkb[:, n:].float()).all() and torch.isnan(dvb[:, n:].float()).all()


@pytest.mark.parametrize("keep", [0, 25])
def test_cached_step_new_keys_head_major_bitwise(keep):
    """480p cached step: the new segment's K / V head-major; dense and
    video-block sparse plans (the selection reads the new keys too)."""
    need_gpu()
    w = wl.cached_step_480p()
    H = w.heads
    say(f"480p step, new keys head-major, keep {keep or 100}%")
    kc, vc = w.cache_kv()
    kcd, vcd = dev(kc), dev(vc)
    kb = torch.empty((H, w.n_cached + w.n_new, 128), dtype=torch.bfloat16, device="cuda")
    vb = torch.empty_like(kb)
    cache = nm.nomas_kvcache_create(H, w.n_cached + w.n_new, kb, vb)
    off = 0
    for s in w.cached:
        nm.nomas_kvcache_append(cache, s, kcd[off:off + s.n_tokens], vcd[off:off + s.n_tokens])
        off += s.n_tokens
    q, k, v = dev(w.q(0)), dev(w.k_new(0)), dev(w.v_new(0))
    pt = nm.nomas_attn_plan(w.q_layout, w.new, cache, heads=H, video_keep_percent=keep)
    ph = nm.nomas_attn_plan(w.q_layout, w.new, cache, heads=H, video_keep_percent=keep,
                            kv_head_major=True)
    o_t, l_t = fwd(pt, cache, q, k, v, w.n_q, H)
    o_h, l_h = fwd(ph, cache, q, head_major(k, 5), head_major(v, 5), w.n_q, H)
    same_bits(o_h, o_t, "O")
    same_bits(l_h, l_t, "LSE")


def test_head_stride_below_the_rows_is_rejected():
    need_gpu()
    w = wl.small_pack(1)
    segs, heads, n = w.q_layout, 2, w.n_q
    plan = nm.nomas_attn_plan(segs, segs, heads=heads, kv_head_major=True)
    q = torch.zeros((n, heads, 128), dtype=torch.bfloat16, device="cuda")
    buf = torch.zeros((heads * n * 128,), dtype=torch.bfloat16, device="cuda")
    # head stride of n - 1 rows: heads would overlap
    k = torch.as_strided(buf, (heads, n, 128), ((n - 1) * 128, 128, 1))
    o = torch.empty_like(q)
    ws = torch.empty(max(nm.nomas_attn_fwd_workspace_size(plan), 16), dtype=torch.uint8, device="cuda")
    with pytest.raises(nm.NomasError) as e:
        nm.nomas_attn_fwd(plan, None, q, k, k, o, None, SCALE, workspace=ws)
    assert e.value.status == 1  # INVALID_ARGUMENT
    # a token-major tensor handed to a head-major plan is refused by the binding
    with pytest.raises(ValueError):
        nm.nomas_attn_fwd(plan, None, q, q, q, o, None, SCALE, workspace=ws)
