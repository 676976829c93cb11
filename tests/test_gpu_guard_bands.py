"""Guard bands around every buffer the kernels write (GPU, through the C ABI).

Each output lives inside a larger allocation filled with a canary pattern:
rows before and after it, the unused columns of a padded token stride, the
cache rows past its current length and the bytes past the workspace size
the library asked for.  After the call every canary must be bit-identical:
a kernel that writes out of its bounds (an off-by-one tile, a ragged row, a
wrong stride) shows up here even where the parity checks would not."""
import pytest
import torch

import segment_causal_masked_amd as nm
from segment_causal_masked_amd import workloads as wl
from gpu_util import SCALE, dev, need_gpu, say

pytestmark = pytest.mark.gpu

G = 64            # guard rows before and after
PAD = 64          # extra columns per token row (padded token stride)
CANARY16 = 0x7FC1  # a bf16 NaN pattern no kernel produces by arithmetic
CANARY32 = 0x7FC00001


def guarded(rows, heads, dtype):
    """(buffer, view): view = [rows, heads, 128] inside a canary-filled buffer
    with G guard rows on each side and PAD unused columns per row."""
    width = heads * 128 + PAD
    itype = torch.int16 if dtype == torch.bfloat16 else torch.int32
    canary = CANARY16 if dtype == torch.bfloat16 else CANARY32
    buf = torch.full((rows + 2 * G, width), canary, dtype=itype, device="cuda").view(dtype)
    view = buf[G:G + rows, :heads * 128].view(rows, heads, 128)
    return buf, view


def untouched(buf, rows, heads, what):
    itype = torch.int16 if buf.dtype == torch.bfloat16 else torch.int32
    canary = CANARY16 if buf.dtype == torch.bfloat16 else CANARY32
    raw = buf.view(itype)
    assert (raw[:G] == canary).all(), f"{what}: guard rows before written"
    assert (raw[G + rows:] == canary).all(), f"{what}: guard rows after written"
    assert (raw[G:G + rows, heads * 128:] == canary).all(), f"{what}: padding columns written"


def guarded_flat(n, dtype=torch.float32):
    buf = torch.full((n + 2 * 256,), CANARY32, dtype=torch.int32, device="cuda").view(dtype)
    return buf, buf[256:256 + n]


def flat_untouched(buf, n, what):
    raw = buf.view(torch.int32)
    assert (raw[:256] == CANARY32).all() and (raw[256 + n:] == CANARY32).all(), what


@pytest.mark.parametrize("grad_f32", [False, True])
def test_forward_and_backward_write_inside_their_buffers(grad_f32):
    need_gpu()
    segs = [wl.Segment(0, 0, 3, 37, 11, [(5, 0, 2), (7, 1, 3)], n_pad=3),
            wl.Segment(0, 1, 2, 37, 11, [(6, 0, 1)]),
            wl.Segment(1, 0, 4, 29, 9, [(4, 2, 4), (3, 0, 1), (8, 1, 2)], n_pad=53)]
    n, heads = wl.layout_tokens(segs), 3
    say(f"guard bands: ragged pack of {n} tokens, {heads} heads, {'fp32' if grad_f32 else 'bf16'} gradients")
    plan = nm.nomas_attn_plan(segs, segs, heads=heads, grad_f32=grad_f32)
    q, k, v, d_o = (dev(wl.randn((n, heads, 128), 9100 + i)) for i in range(4))
    ob, o = guarded(n, heads, torch.bfloat16)
    lb, lse = guarded_flat(heads * n)
    lse = lse.view(heads, n)
    nws = nm.nomas_attn_fwd_workspace_size(plan)
    wb, ws = guarded_flat((nws + 3) // 4)
    nm.nomas_attn_fwd(plan, None, q, k, v, o, lse, SCALE, workspace=ws.view(torch.uint8)[:max(nws, 16)])
    torch.cuda.synchronize()
    untouched(ob, n, heads, "O")
    flat_untouched(lb, heads * n, "LSE")
    flat_untouched(wb, (nws + 3) // 4, "forward workspace")
    assert torch.isfinite(o.float()).all()
    gd = torch.float32 if grad_f32 else torch.bfloat16
    # the backward takes q, o, dO and dQ (and k, v, dK, dV) with one token
    # stride: all of them in guarded buffers of the same padded stride
    bufs = [guarded(n, heads, gd) for _ in range(3)]
    qg, kg, vg, og, dog = (guarded(n, heads, torch.bfloat16) for _ in range(5))
    for (_, dst), src in zip((qg, kg, vg, og, dog), (q, k, v, o, d_o)):
        dst.copy_(src)
    nbw = nm.nomas_attn_bwd_workspace_size(plan)
    bwb, bws = guarded_flat((nbw + 3) // 4)
    dq, dk, dv = (b[1] for b in bufs)
    nm.nomas_attn_bwd(plan, qg[1], kg[1], vg[1], og[1], dog[1], lse, dq, dk, dv, SCALE,
                      workspace=bws.view(torch.uint8)[:max(nbw, 16)])
    torch.cuda.synchronize()
    for (b, _), name in zip(bufs, ("dQ", "dK", "dV")):
        untouched(b, n, heads, name)
    flat_untouched(bwb, (nbw + 3) // 4, "backward workspace")
    for b, name in zip((dq, dk, dv), ("dQ", "dK", "dV")):
        assert torch.isfinite(b.float()).all(), name


def test_append_writes_only_its_rows():
    """Each append fills exactly the next rows of every head; the capacity
    past the cache's length keeps its canary."""
    need_gpu()
    w = wl.cached_step_480p()
    kc, vc = w.cache_kv()
    cap = w.n_cached + w.n_new + 100
    kb = torch.full((16, cap, 128), CANARY16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    vb = kb.clone()
    cache = nm.nomas_kvcache_create(16, cap, kb, vb)
    kd, vd = dev(kc), dev(vc)
    off = 0
    for s in w.cached:
        nm.nomas_kvcache_append(cache, s, kd[off:off + s.n_tokens], vd[off:off + s.n_tokens])
        off += s.n_tokens
        torch.cuda.synchronize()
        n = nm.nomas_kvcache_len(cache)[0]
        for buf, name in ((kb, "K"), (vb, "V")):
            raw = buf.view(torch.int16)
            assert (raw[:, n:] == CANARY16).all(), f"{name} cache: rows past the length written"
            assert not (raw[:, :n] == CANARY16).all(dim=2).any(), f"{name} cache: a stored row not written"
