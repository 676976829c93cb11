"""GPU tests of the INT8 KV cache, through the C ABI: the codes and exponents
bit-exact against the oracle's quantizer, the expanded bf16 rows bit-exact
against its dequantized values, the forward over an expanded cache against
the fp64 attention oracle on those values, and the cache bookkeeping."""
import numpy as np
import pytest
import torch

import oracle
import segment_causal_masked_amd as nm
from oracle.int8cache import dequantize_rows, quantize_rows
from segment_causal_masked_amd import workloads as wl
from gpu_util import SCALE, check_lse, oracle_forward, check_o, dev, host, need_gpu, new_cache, run_fwd, say, stored_rows

pytestmark = pytest.mark.gpu


def fill_int8(cache, segments, k_tok, v_tok):
    off = 0
    for s in segments:
        nm.nomas_kvcache_int8_append(cache, s, k_tok[off:off + s.n_tokens], v_tok[off:off + s.n_tokens])
        off += s.n_tokens


def oracle_cache(segments, k, v):
    """Stored rows of K and V, head-major, quantized by the oracle."""
    rows = stored_rows(segments)
    out = []
    for x in (k, v):
        xs = np.transpose(x[rows], (1, 0, 2))  # [H][n][128]
        out.append(quantize_rows(xs))
    return out, rows


def test_int8_codes_and_expansion_bit_exact():
    need_gpu()
    w = wl.cached_step_480p()
    say("int8 cache: 4 cached 480p segments, 16 heads")
    kc, vc = w.cache_kv()
    cap = w.n_cached + 64
    c8 = nm.nomas_kvcache_int8_create(16, cap)
    fill_int8(c8, w.cached, dev(kc), dev(vc))
    torch.cuda.synchronize()
    (kq, ke), (vq, ve) = oracle_cache(w.cached, kc, vc)[0]
    n = kq.shape[1]
    assert nm.nomas_kvcache_int8_len(c8) == (n, 4)
    np.testing.assert_array_equal(c8.k_codes[:, :n].cpu().numpy(), kq)
    np.testing.assert_array_equal(c8.v_codes[:, :n].cpu().numpy(), vq)
    np.testing.assert_array_equal(c8.k_exp[:, :n].cpu().numpy(), ke)
    np.testing.assert_array_equal(c8.v_exp[:, :n].cpu().numpy(), ve)
    work = new_cache(16, cap)
    nm.nomas_kvcache_int8_expand(c8, work)
    torch.cuda.synchronize()
    assert nm.nomas_kvcache_len(work) == (n, 4)
    np.testing.assert_array_equal(host(work.k_buf[:, :n]), dequantize_rows(kq, ke).astype(np.float32))
    np.testing.assert_array_equal(host(work.v_buf[:, :n]), dequantize_rows(vq, ve).astype(np.float32))


def test_int8_forward_matches_oracle_on_dequantized_cache():
    need_gpu()
    w = wl.cached_step_480p()
    say("480p cached step over an expanded int8 cache, 16 heads, vs the oracle on the dequantized values")
    kc, vc = w.cache_kv()
    cap = w.n_cached + w.n_new
    c8 = nm.nomas_kvcache_int8_create(16, cap)
    fill_int8(c8, w.cached, dev(kc), dev(vc))
    work = new_cache(16, cap)
    nm.nomas_kvcache_int8_expand(c8, work)
    plan = nm.nomas_attn_plan(w.q_layout, w.new, work, heads=16)
    q, kn, vn = w.q(), w.k_new(), w.v_new()
    o, l = run_fwd(plan, work, dev(q), dev(kn), dev(vn), 16)
    (kq, ke), (vq, ve) = oracle_cache(w.cached, kc, vc)[0]
    k_all = np.concatenate([np.transpose(dequantize_rows(kq, ke), (1, 0, 2)), kn])
    v_all = np.concatenate([np.transpose(dequantize_rows(vq, ve), (1, 0, 2)), vn])
    # keys: the stored rows of the cached segments (video + head), then the new segment
    keys = [wl.Segment(s.video, s.index, s.n_frames, s.tokens_per_frame, s.n_head, []) for s in w.cached] + w.new
    tq, tk = oracle.expand(w.q_layout), oracle.expand(keys)
    o_ref, l_ref, l_bnd = oracle_forward(q, k_all, v_all, tq, tk, SCALE)
    check_o(host(o), o_ref, "int8 cache, 480p step")
    check_lse(host(l), l_ref, "int8 cache, 480p step", l_bnd)


def test_int8_plan_valid_across_layers_and_stale_on_other_segments():
    need_gpu()
    w = wl.cached_step_480p(n_cached=2)
    cap = w.n_cached + w.n_new
    layers = []
    for layer in range(2):
        kc, vc = w.cache_kv(layer)
        c8 = nm.nomas_kvcache_int8_create(16, cap)
        fill_int8(c8, w.cached, dev(kc), dev(vc))
        layers.append((c8, kc, vc))
    work = new_cache(16, cap)
    nm.nomas_kvcache_int8_expand(layers[0][0], work)
    plan = nm.nomas_attn_plan(w.q_layout, w.new, work, heads=16)
    q, kn, vn = dev(w.q()), dev(w.k_new()), dev(w.v_new())
    o0, _ = run_fwd(plan, work, q, kn, vn, 16)
    nm.nomas_kvcache_int8_expand(layers[1][0], work)   # same segments, other values
    o1, _ = run_fwd(plan, work, q, kn, vn, 16)
    assert not torch.equal(o0, o1)
    # layer 1 through a freshly built plan and a second working cache: identical
    work2 = new_cache(16, cap)
    nm.nomas_kvcache_int8_expand(layers[1][0], work2)
    plan2 = nm.nomas_attn_plan(w.q_layout, w.new, work2, heads=16)
    o1b, _ = run_fwd(plan2, work2, q, kn, vn, 16)
    assert torch.equal(o1, o1b)
    # a cache with other segments makes the plan stale
    nm.nomas_kvcache_int8_truncate(layers[1][0], 1)
    assert nm.nomas_kvcache_int8_len(layers[1][0])[1] == 1
    nm.nomas_kvcache_int8_expand(layers[1][0], work)
    with pytest.raises(nm.NomasError) as e:
        run_fwd(plan, work, q, kn, vn, 16)
    assert e.value.status == 5


def test_int8_expand_capacity_and_head_checks():
    need_gpu()
    w = wl.cached_step_480p(n_cached=2)
    kc, vc = w.cache_kv()
    c8 = nm.nomas_kvcache_int8_create(16, w.n_cached)
    fill_int8(c8, w.cached, dev(kc), dev(vc))
    small = new_cache(16, 100)
    before = small.k_buf.clone()
    with pytest.raises(nm.NomasError) as e:
        nm.nomas_kvcache_int8_expand(c8, small)
    assert e.value.status == 4 and nm.nomas_kvcache_len(small) == (0, 0)
    other = new_cache(8, w.n_cached)
    with pytest.raises(nm.NomasError) as e:
        nm.nomas_kvcache_int8_expand(c8, other)
    assert e.value.status == 1
    # over capacity: nothing written, nothing recorded
    full = nm.nomas_kvcache_int8_create(16, 100)
    with pytest.raises(nm.NomasError) as e:
        nm.nomas_kvcache_int8_append(full, w.cached[0], dev(kc[:w.cached[0].n_tokens]), dev(vc[:w.cached[0].n_tokens]))
    assert e.value.status == 4 and nm.nomas_kvcache_int8_len(full) == (0, 0)
    torch.cuda.synchronize()
    assert torch.equal(before, small.k_buf) and not full.k_codes.any()


def test_int8_codes_of_scaled_rows():
    """Rows far from unit scale (1e-20 .. 1e20) and rows with exact ties."""
    need_gpu()
    seg = wl.Segment(0, 0, 2, 24, 16, [])
    n = seg.n_tokens
    g = np.random.default_rng(9)
    k = wl.randn((n, 2, 128), 950) * (10.0 ** g.integers(-20, 21, size=(n, 2, 1)))
    k = wl.round_to_bf16(k.astype(np.float32))
    v = np.zeros((n, 2, 128), np.float32)
    v[:, :, 0] = 1.0
    v[:, :, 1:13] = np.arange(-6, 6) / 64.0 + 1 / 128.0   # halfway between codes at e = -6
    c8 = nm.nomas_kvcache_int8_create(2, 64)
    nm.nomas_kvcache_int8_append(c8, seg, dev(k), dev(v))
    torch.cuda.synchronize()
    (kq, ke), (vq, ve) = oracle_cache([seg], k, v)[0]
    np.testing.assert_array_equal(c8.k_codes[:, :n].cpu().numpy(), kq)
    np.testing.assert_array_equal(c8.k_exp[:, :n].cpu().numpy(), ke)
    np.testing.assert_array_equal(c8.v_codes[:, :n].cpu().numpy(), vq)
    np.testing.assert_array_equal(c8.v_exp[:, :n].cpu().numpy(), ve)
