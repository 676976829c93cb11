"""Seeded synthetic workloads for the action-aware causal attention.

This module only *describes* inputs: segment records (frames, tokens per frame,
head length, action tails with their latent-frame windows) and seeded bf16 /
fp32 tensors.  It holds none of the method's arithmetic -- no token expansion,
no mask, no attention -- so that the GPU path and the fp64 oracle can both be
fed from it without sharing any of the computation they are compared on.

Shapes follow the Hy-Nomas pages:
  * latent grid from the DCAE-V compression rule (Eq. 1, "Theoretical
    Foundation"): 32x spatial, so 480x848 -> 15x26 = 390 tokens per latent
    frame and 704x1280 (720p) -> 22x40 = 880;
  * 16 heads of 128 dims (dual-stream MMDiT, "Theoretical Foundation");
  * each segment = video tokens + a descriptive head + action tails a_0..a_n
    with temporal windows ("Action-Aware Causal Attention", "Model
    Architecture").

Token order inside a segment (the pages leave it open):
    [video, frame-major | head | a_0 | a_1 | ... | trailing pad]

Random numbers come from numpy's PCG64 with seed = the workload's seed base
(1000, 2000, 3000, 4000, 5000 for the five workloads below, in order) + tensor
id (Q=1, K=2, V=3, dO=4, windows=5, cache=6, camera K=7, camera V=8; the
n-th of several denoising calls adds 10*n).  Values are N(0,1) rounded to bf16 (round-to-nearest-even) except
the tiny fp32 case.
"""
from __future__ import annotations

import dataclasses
from typing import List, Sequence, Tuple

import numpy as np

HEADS = 16
HEAD_DIM = 128
TPF_480P = 15 * 26   # 480x848 / 32
TPF_720P = 22 * 40   # 704x1280 / 32

TID_Q, TID_K, TID_V, TID_DO, TID_WIN, TID_CACHE = 1, 2, 3, 4, 5, 6
TID_CAM_K, TID_CAM_V = 7, 8


@dataclasses.dataclass
class Segment:
    """One segment record.

    video / index: which video the segment belongs to and its position in that
    video's generation order (segment-causal attention compares these).
    actions: list of (n_tokens, frame_lo, frame_hi) with the window in latent
    frames, half-open [lo, hi).
    n_pad: padding tokens appended after the segment (never visible).
    """
    video: int
    index: int
    n_frames: int
    tokens_per_frame: int
    n_head: int
    actions: List[Tuple[int, int, int]]
    n_pad: int = 0

    @property
    def n_tokens(self) -> int:
        return (self.n_frames * self.tokens_per_frame + self.n_head
                + sum(a[0] for a in self.actions) + self.n_pad)


def layout_tokens(segs: Sequence[Segment]) -> int:
    return int(sum(s.n_tokens for s in segs))


# ----------------------------------------------------------------------------
# random numbers
# ----------------------------------------------------------------------------

def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as fp32 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16-representable fp32 values -> their 16-bit patterns (uint16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def randn(shape, seed: int, bf16: bool = True) -> np.ndarray:
    a = rng(seed).standard_normal(size=shape, dtype=np.float32)
    return round_to_bf16(a) if bf16 else a


def random_windows(g: np.random.Generator, n_actions: int, n_frames: int,
                   sorted_disjoint: bool = False) -> List[Tuple[int, int]]:
    """Random contiguous latent-frame windows [lo, hi).

    Default: independent per action, lo ~ U{0..F-1}, hi ~ U{lo+1..F}
    (overlap allowed).  sorted_disjoint: chronological, non-overlapping
    windows (cut points drawn without replacement), when F >= n_actions.
    """
    if sorted_disjoint and n_frames >= n_actions:
        cuts = np.sort(g.choice(np.arange(1, n_frames), size=n_actions - 1,
                                replace=False)) if n_actions > 1 else np.array([], int)
        edges = [0] + [int(c) for c in cuts] + [n_frames]
        return [(edges[i], edges[i + 1]) for i in range(n_actions)]
    out = []
    for _ in range(n_actions):
        lo = int(g.integers(0, n_frames))
        hi = int(g.integers(lo + 1, n_frames + 1))
        out.append((lo, hi))
    return out


def make_segment(g, video, index, n_frames, tpf, n_head, n_actions, tail_len,
                 n_pad=0, sorted_disjoint=False) -> Segment:
    wins = random_windows(g, n_actions, n_frames, sorted_disjoint)
    return Segment(video, index, n_frames, tpf, n_head,
                   [(tail_len, lo, hi) for lo, hi in wins], n_pad)


# ----------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    name: str
    heads: int
    head_dim: int
    q_layout: List[Segment]          # query tokens
    cached: List[Segment]            # segments already in the KV cache
    new: List[Segment]               # key/value tokens supplied with the call
    fp32_inputs: bool = False
    seed_base: int = 0

    @property
    def n_q(self):
        return layout_tokens(self.q_layout)

    @property
    def n_cached(self):
        return layout_tokens(self.cached)

    @property
    def n_new(self):
        return layout_tokens(self.new)

    @property
    def n_keys(self):
        return self.n_cached + self.n_new

    def tensor(self, tid: int, n_tokens: int, nfe: int = 0) -> np.ndarray:
        """[n_tokens, H, D] fp32 array of bf16 (or fp32) values."""
        return randn((n_tokens, self.heads, self.head_dim),
                     self.seed_base + tid + 10 * nfe, bf16=not self.fp32_inputs)

    def q(self, nfe=0):
        return self.tensor(TID_Q, self.n_q, nfe)

    def k_new(self, nfe=0):
        return self.tensor(TID_K, self.n_new, nfe)

    def v_new(self, nfe=0):
        return self.tensor(TID_V, self.n_new, nfe)

    def d_o(self, nfe=0):
        return self.tensor(TID_DO, self.n_q, nfe)

    @property
    def n_camera(self):
        """Camera tokens of the query layout: one per latent frame."""
        return int(sum(s.n_frames for s in self.q_layout))

    def camera_kv(self, nfe=0):
        """Camera-token K and V (already projected per head), [n_camera, H, D]."""
        return (self.tensor(TID_CAM_K, self.n_camera, nfe),
                self.tensor(TID_CAM_V, self.n_camera, nfe))

    def cache_kv(self, layer: int = 0):
        """Cached K and V as [n_cached, H, D] each (token-major)."""
        s = self.seed_base + TID_CACHE + 100 * layer
        k = randn((self.n_cached, self.heads, self.head_dim), s)
        v = randn((self.n_cached, self.heads, self.head_dim), s + 50)
        return k, v


def tiny_two_segments() -> Workload:
    """Tiny case: 1 head, fp32; 2 segments of 2 frames x 4x4 + 8 head + 2 tails
    of 4 tokens with windows [0,1) and [1,2)."""
    segs = [Segment(0, j, 2, 16, 8, [(4, 0, 1), (4, 1, 2)]) for j in range(2)]
    return Workload("tiny-2seg-1head-fp32", 1, HEAD_DIM, segs, [], segs,
                    fp32_inputs=True, seed_base=1000)


def single_segment_480p(seed_set: int = 0) -> Workload:
    """One 480p segment, no cache: 8 x 390 video + 64 head + 3 x 32 tails."""
    g = rng(2000 + TID_WIN + 7919 * seed_set)
    seg = make_segment(g, 0, 0, 8, TPF_480P, 64, 3, 32,
                       sorted_disjoint=(seed_set == 1))
    return Workload("480p-single-segment", HEADS, HEAD_DIM, [seg], [], [seg],
                    seed_base=2000)


def cached_step_480p(seed_set: int = 0, n_cached: int = 4) -> Workload:
    """480p cached step: 4 cached segments + 1 new one (queries)."""
    g = rng(3000 + TID_WIN + 7919 * seed_set)
    segs = [make_segment(g, 0, j, 8, TPF_480P, 64, 3, 32,
                         sorted_disjoint=(seed_set == 1))
            for j in range(n_cached + 1)]
    return Workload("480p-cached-step-4+1seg", HEADS, HEAD_DIM, [segs[-1]],
                    segs[:-1], [segs[-1]], seed_base=3000)


def long_session_720p(seed_set: int = 0, n_cached: int = 16) -> Workload:
    """720p long session: 16 cached segments + 1 new; 4 denoising calls."""
    g = rng(4000 + TID_WIN + 7919 * seed_set)
    segs = [make_segment(g, 0, j, 8, TPF_720P, 64, 4, 32,
                         sorted_disjoint=(seed_set == 1))
            for j in range(n_cached + 1)]
    return Workload("720p-long-session-16+1seg", HEADS, HEAD_DIM, [segs[-1]],
                    segs[:-1], [segs[-1]], seed_base=4000)


def pack_layout(g, n_videos, tokens_per_video, seg_range=(4, 8), tpf=TPF_480P,
                n_head=64, n_actions=3, tail_len=32) -> List[Segment]:
    """Training pack: n_videos independent videos of tokens_per_video tokens.

    Each video draws its segment count from seg_range, gives the frames it can
    hold to its segments as evenly as possible and pads the remainder at its
    end.
    """
    out = []
    text = n_head + n_actions * tail_len
    for v in range(n_videos):
        n_seg = int(g.integers(seg_range[0], seg_range[1] + 1))
        frames = (tokens_per_video - text * n_seg) // tpf
        assert frames >= n_seg, "video too short for its segments"
        base, extra = divmod(frames, n_seg)
        used = 0
        segs = []
        for j in range(n_seg):
            f = base + (1 if j < extra else 0)
            segs.append(make_segment(g, v, j, f, tpf, n_head, n_actions, tail_len))
            used += f * tpf + text
        segs[-1].n_pad = tokens_per_video - used
        out.extend(segs)
    return out


def training_pack_131k(seed_set: int = 0) -> Workload:
    """Training pack of 131072 tokens: 4 videos x 32768, 4-8 segments each."""
    g = rng(5000 + TID_WIN + 7919 * seed_set)
    segs = pack_layout(g, 4, 32768)
    return Workload("train-pack-131072tok-4videos", HEADS, HEAD_DIM, segs, [], segs,
                    seed_base=5000)


def small_pack(seed: int = 0, n_videos: int = 2, tokens_per_video: int = 2048,
               heads: int = HEADS) -> Workload:
    """Self-contained 4096-token pack (2 videos x 2-3 small segments)."""
    g = rng(5500 + 7919 * seed)
    segs = pack_layout(g, n_videos, tokens_per_video, seg_range=(2, 3), tpf=64,
                       n_head=32, n_actions=3, tail_len=16)
    return Workload("train-pack-4096tok-2videos", heads, HEAD_DIM, segs, [], segs,
                    seed_base=5500 + 100 * seed)


WORKLOADS = {"tiny_two_segments": tiny_two_segments, "single_segment_480p": single_segment_480p,
             "cached_step_480p": cached_step_480p, "long_session_720p": long_session_720p,
             "training_pack_131k": training_pack_131k}
