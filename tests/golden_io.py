"""Reader for the hand-written mask fixtures under tests/golden/."""
import os

import numpy as np

from segment_causal_masked_amd.workloads import Segment

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(tok):
    a, b = tok.split("-")
    return int(a), int(b)


def load_mask_fixture(name):
    segs, rows, A, tiles, tile_rows = [], [], {}, None, []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        f = line.split()
        if f[0] == "seg":
            video, index, nf, tpf, nh, npad = map(int, f[1:7])
            acts = [tuple(int(x) for x in a.split(":")) for a in f[7:]]
            segs.append(Segment(video, index, nf, tpf, nh, acts, npad))
        elif f[0] == "rows":
            left, right = line[len("rows"):].split(":", 1)
            r0, r1 = _rng(left.strip())
            keys_part, count = right.split(";")
            ranges = [_rng(t) for t in keys_part.split()]
            rows.append(((r0, r1), ranges, int(count)))
        elif f[0] == "A":
            A[f[1]] = int(f[2])
        elif f[0] == "tiles":
            tiles = (int(f[1]), int(f[2]))
        elif f[0] == "tilerow":
            tile_rows.append(f[1:])
    n = sum(s.n_tokens for s in segs)
    mask = np.zeros((n, n), bool)
    for (r0, r1), ranges, count in rows:
        for a, b in ranges:
            mask[r0:r1 + 1, a:b + 1] = True
        assert all(mask[r].sum() == count for r in range(r0, r1 + 1)), (r0, r1)
    code = {"E": 0, "F": 1, "P": 2}
    tmap = np.array([[code[c] for c in r] for r in tile_rows], np.uint8)
    return segs, mask, A, tiles, tmap
