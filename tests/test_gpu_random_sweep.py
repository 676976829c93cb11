"""Seeded random sweep of the forward and the backward over small
self-attention packs: one to
three videos of one to four segments each (in shuffled order), 1-6 latent
frames of 0-40 tokens, 0-20 head tokens, 0-5 actions with random frame
windows, 0-10 padding tokens, 1-4 heads, each text-query mode and segment
windows of 0 (none), 1 or 2 -- every case through the C ABI against the fp64
oracle on the same inputs.  The cases are the same on every run."""
import numpy as np
import pytest

import oracle
import segment_causal_masked_amd as nm
from segment_causal_masked_amd import workloads as wl
from gpu_util import SCALE, check_lse, oracle_forward, check_o, dev, host, need_gpu, run_fwd, say
from test_gpu_bwd import full_case

pytestmark = pytest.mark.gpu

MODES = ("R", "K", "H")


def random_pack(g):
    segs = []
    for video in range(int(g.integers(1, 4))):
        for index in range(int(g.integers(1, 5))):
            nf, tpf = int(g.integers(1, 7)), int(g.integers(0, 41))
            acts = []
            for _ in range(int(g.integers(0, 6))):
                lo = int(g.integers(0, nf))
                acts.append((int(g.integers(1, 9)), lo, int(g.integers(lo + 1, nf + 1))))
            n_head = int(g.integers(0, 21))
            if tpf == 0 and n_head == 0 and not acts:
                n_head = 1  # a segment holds at least one token
            segs.append(wl.Segment(video, index, nf, tpf, n_head, acts, n_pad=int(g.integers(0, 11))))
    return [segs[i] for i in g.permutation(len(segs))]


@pytest.mark.parametrize("case", range(16))
def test_random_pack_forward(case):
    need_gpu()
    g = np.random.default_rng(7000 + case)
    segs = random_pack(g)
    heads = int(g.integers(1, 5))
    mode = MODES[case % 3]
    window = int(g.integers(0, 3))
    n = sum(s.n_tokens for s in segs)
    say(f"random pack {case}: {len(segs)} segments, {n} tokens, {heads} heads, "
        f"text-query mode {mode}, window {window}")
    q, k, v = (wl.round_to_bf16(g.standard_normal((n, heads, 128), np.float32)) for _ in range(3))
    plan = nm.nomas_attn_plan(segs, segs, heads=heads, mode=mode, window=window)
    o, l = run_fwd(plan, None, dev(q), dev(k), dev(v), heads)
    t = oracle.expand(segs)
    o_ref, l_ref, l_bnd = oracle_forward(q, k, v, t, t, SCALE, mode=mode, window=window)
    check_o(host(o), o_ref, f"random pack {case}")
    check_lse(host(l), l_ref, f"random pack {case}", l_bnd)


@pytest.mark.parametrize("case", range(8))
def test_random_pack_backward(case):
    need_gpu()
    g = np.random.default_rng(7100 + case)
    segs = random_pack(g)
    heads = int(g.integers(1, 4))
    mode = MODES[case % 3]
    window = int(g.integers(0, 3))
    say(f"random pack backward {case}: {len(segs)} segments, {sum(s.n_tokens for s in segs)} tokens, "
        f"{heads} heads, text-query mode {mode}, window {window}")
    full_case(segs, heads, 7200 + case, mode=mode, window=window)
