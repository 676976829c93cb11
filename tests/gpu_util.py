"""Helpers shared by the GPU parity tests (inputs on the device, tolerances)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import segment_causal_masked_amd as nm
import tolerance as tol

SCALE = 128 ** -0.5

# Parity gate of the attention output: max-abs 1e-2 and mean-abs 1e-3 on
# unit-scale outputs (inputs ~ N(0,1)).  LSE: a per-row bound derived from the
# device's roundings (tolerance.lse_bound): the forward rounds Q * scale *
# log2(e) to bf16 before its products.
O_MAX_ABS, O_MEAN_ABS = 1e-2, 1e-3


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nm.load()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x, dtype=torch.bfloat16):
    """numpy fp32 (bf16-representable) -> device tensor (exact)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dtype)


def host(t):
    return t.float().cpu().numpy()


def check_o(o_gpu, o_ref, what=""):
    err = np.abs(o_gpu.astype(np.float64) - o_ref)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    say(f"  {what}: O max-abs {mx:.3e} mean-abs {mean:.3e}")
    assert mx <= O_MAX_ABS and mean <= O_MEAN_ABS, (what, mx, mean)
    assert np.isfinite(o_gpu).all()


def oracle_forward(q, k, v, tq, tk, scale=SCALE, u_inputs=0.0, **kw):
    """The oracle's (O, LSE) and the device LSE bound for the same rows and
    heads (kw as oracle.forward)."""
    o_ref, l_ref = oracle.forward(q, k, v, tq, tk, scale, **kw)
    bkw = {n: kw[n] for n in ("mode", "rows", "heads", "window", "tile_keep", "unit_rows",
                              "tile_keys") if n in kw}
    return o_ref, l_ref, tol.lse_bound(q, k, tq, tk, scale, u_inputs=u_inputs, **bkw)


def check_lse(lse_gpu, lse_ref, what, bound):
    """Rows that see no key: -inf exactly; others within their derived bound."""
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_gpu), fin), what
    assert np.all(lse_gpu[~fin] == -np.inf)
    if fin.any():
        d = np.abs(lse_gpu[fin] - lse_ref[fin])
        b = bound[fin]
        r = float((d / b).max())
        say(f"  {what}: LSE max-abs {float(d.max()):.3e}, max err/bound {r:.3f} "
            f"(bound median {float(np.median(b)):.2e})")
        assert r <= 1.0, (what, r)


def new_cache(heads, capacity):
    kb = torch.zeros((heads, capacity, 128), dtype=torch.bfloat16, device="cuda")
    vb = torch.zeros_like(kb)
    return nm.nomas_kvcache_create(heads, capacity, kb, vb)


def stored_rows(segments):
    """Row indices (into the segments' concatenated tokens) that a KV cache
    keeps: each segment's video and head tokens, which come first."""
    rows, off = [], 0
    for s in segments:
        rows.append(np.arange(off, off + s.n_frames * s.tokens_per_frame + s.n_head))
        off += s.n_tokens
    return np.concatenate(rows) if rows else np.zeros(0, np.int64)


def fill_cache(cache, segments, k_tok, v_tok):
    """Append segments one by one from token-major [T,H,D] device tensors."""
    off = 0
    for s in segments:
        n = s.n_tokens
        nm.nomas_kvcache_append(cache, s, k_tok[off:off + n], v_tok[off:off + n])
        off += n
    return off


def fwd_workspace(plan):
    n = nm.nomas_attn_fwd_workspace_size(plan)
    return torch.empty(max(n, 16), dtype=torch.uint8, device="cuda") if n else None


def run_fwd(plan, cache, q, k_new, v_new, heads, lse=True):
    o = torch.empty((q.shape[0], heads, 128), dtype=torch.bfloat16, device="cuda")
    l = torch.empty((heads, q.shape[0]), dtype=torch.float32, device="cuda") if lse else None
    nm.nomas_attn_fwd(plan, cache, q, k_new, v_new, o, l, SCALE, workspace=fwd_workspace(plan))
    torch.cuda.synchronize()
    return o, l
