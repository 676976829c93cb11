"""fp64 CPU oracle for the Hy-Nomas action-aware causal attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The GPU library never calls it and
shares no code, table or helper with it.

What it computes is the plain definition: the visibility mask is materialised
pair by pair from the rules the pages state, then exact softmax attention (and
its gradient) is evaluated in float64 with numpy.  Block skipping and online
softmax, which the GPU path uses, are exact reformulations of this result, so
the oracle needs neither.

Sources (cited by page title and section throughout):
  [Summary]  "Summary (Overview)" page on Hy-Nomas (picx.dev/p/8H5X8y):
             Theoretical Foundation (Eq. 1, head geometry); Model Architecture
             (Segment-wise Causal Attention; Action-Aware Causal Attention,
             Figure 6b); Training Infrastructure (FLOPs-based packing, Eq. 6).
  [News]     "Tencent's Hy-Nomas Steers a 60-Second Video World With Text and
             Camera on One RTX 4090" (gpts24.com): "One World, Generated Segment
             by Segment" (K/V of each segment appended to a growing cache).
  [Review]   "Hy-Nomas가 8B 모델 하나로 다중 턴 세계 생성과 카메라 제어를 묶는다"
             (onedev.kr/papers/1434): section "무엇과 다른가" (the most explicit
             statement of which tokens a query in an action window reaches).
  [Guide]    "Hy-Nomas: Serbest Biçimli Etkileşimli Dünya Üretimine Doğru"
             (xyznot.com/tr/paper/2610.36729): "Eyleme Duyarlı Nedensel Dikkat"
             and "Dağıtık Paketleme FLOP Tahmini" (A_i = unmasked pairs, M = -inf
             on hidden pairs).

Readings taken where the pages are silent (each is a parameter or a documented
choice, never hidden):
  * text queries (mode "R", default): a head query sees no action tails; a
    query of tail a_k sees the tokens of a_k only.  Mode "K": no text query
    sees any tail.  Mode "H": head queries also see their own segment's tails.
  * overlapping windows: a video query sees every tail whose window holds its
    latent frame; a frame in no window sees no tail.
  * heads: every head of segments <= the query's segment (same video) is
    visible.
  * token order in a segment: [video frame-major | head | a_0 | ... | pad].
  * rows with no visible key (padding) give O = 0 and LSE = -inf.
  * sliding window (optional, mask.py rule 8): whole segments.
  * video-block sparsity (optional, sparse.py): which blocks are kept is
    stated there (the exact dot product of a query unit's sum and a key
    tile's sum, ties to the lower tile; geometry given as parameters).
  * camera cross-attention (camera.py, [Summary] Camera-Trajectory
    Conditioning, Eq. 3): one camera token per latent frame, a video query
    sees its own segment's camera tokens within a frame radius (all of them
    by default); text rows get 0.
  * INT8 KV cache (int8cache.py, [Summary] Inference): per (head, token) row,
    int8 codes and one power-of-two scale (the smallest keeping the codes
    within +-127, round half to even); dequantized values are exact in bf16.

Parity status: every function here is pinned by CPU tests (hand-built masks,
closed forms, library special cases, finite differences, brute force) except
the choice among text-query modes R / K / H, which the pages leave open
("parity unpinned" for that choice: it is pinned only to the reading above).
"""
from .tokens import TokenAttrs, expand, V, H, A, PAD  # noqa: F401
from .mask import visible_mask, visible_pair, brute_force_mask  # noqa: F401
from .attention import forward, backward  # noqa: F401
from .tiles import unmasked_pairs, tile_classes, EMPTY, FULL, PARTIAL  # noqa: F401
from . import sparse, camera, int8cache  # noqa: F401
