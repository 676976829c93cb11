"""The plan core under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

csrc/plan.cpp is plain C++ (no HIP); it is built here with g++ together with
a small driver (tests/native/plan_driver.cpp) and sanitizers that abort on
the first error, then run on the five workloads' layouts, windows, sparse
options, random layouts and malformed records.  Every plan's invariants are
checked (validate_host_plan), and its unmasked-pair count is compared with
the oracle's."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from segment_causal_masked_amd import workloads as wl
from test_oracle_mask import random_tiny_layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "segment_causal_masked_amd", "csrc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not shutil.which("g++"):
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("asan") / "plan_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "plan.cpp"), os.path.join(ROOT, "tests", "native", "plan_driver.cpp"),
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def seg_line(tag, s):
    acts = " ".join(f"{n} {lo} {hi}" for n, lo, hi in s.actions)
    return f"{tag} {s.video} {s.index} {s.n_frames} {s.tokens_per_frame} {s.n_head} {s.n_pad} " \
           f"{len(s.actions)} {acts}"


def case(q, cached, kv, heads=16, mode=0, window=0, keep=0):
    lines = [f"P {heads} {mode} {window} {keep}"]
    lines += [seg_line("Q", s) for s in q] + [seg_line("C", s) for s in cached]
    lines += [seg_line("N", s) for s in kv] + ["E"]
    return "\n".join(lines)


def run(driver, cases):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([driver], input="\n".join(cases) + "\n", capture_output=True, text=True,
                       env=env, timeout=600)
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, (r.returncode, r.stderr[-4000:], r.stdout[-2000:])
    return r.stdout.strip().splitlines()


def test_workload_plans_clean_and_consistent(driver):
    cases, want = [], []
    for name, fn in wl.WORKLOADS.items():
        w = fn()
        for window, keep in ((0, 0), (2, 0), (0, 25)):
            cases.append(case(w.q_layout, w.cached, w.new, w.heads, 0, window, keep))
            want.append((name, window))
    out = run(driver, cases)
    assert len(out) == len(cases)
    for line, (name, window) in zip(out, want):
        assert line.startswith("ok "), (name, line)
    # A of the dense plans against the oracle (the two smallest workloads)
    for i, (name, window) in enumerate(want):
        if name in ("tiny_two_segments", "single_segment_480p") and window in (0, 2):
            w = wl.WORKLOADS[name]()
            tq, tk = oracle.expand(w.q_layout), oracle.expand(w.cached + w.new)
            assert int(out[i].split()[1]) == oracle.unmasked_pairs(tq, tk, window=window)


def test_random_layouts_clean_and_consistent(driver):
    g = np.random.default_rng(77)
    cases, layouts = [], []
    for i in range(60):
        segs = random_tiny_layout(g, n_videos=int(g.integers(1, 4)))
        mode, window, keep = i % 3, int(g.integers(0, 3)), int(g.choice([0, 0, 30, 100]))
        cases.append(case(segs, [], segs, int(g.integers(1, 5)), mode, window, keep))
        layouts.append((segs, "RKH"[mode], window))
    out = run(driver, cases)
    for line, (segs, mode, window) in zip(out, layouts):
        assert line.startswith("ok "), line
        t = oracle.expand(segs)
        assert int(line.split()[1]) == oracle.unmasked_pairs(t, t, mode, window=window)


def test_malformed_records_rejected_cleanly(driver):
    good = wl.Segment(0, 0, 2, 16, 8, [(4, 0, 1)])
    bad = [wl.Segment(0, 0, 2, 16, 8, [(4, 1, 1)]),        # lo >= hi
           wl.Segment(0, 0, 2, 16, 8, [(4, 0, 3)]),        # hi > n_frames
           wl.Segment(0, 0, 2, 16, 8, [(0, 0, 1)]),        # empty action
           wl.Segment(0, 0, 0, 16, 0, []),                 # no token
           wl.Segment(-1, 0, 2, 16, 8, [])]                # negative video
    cases = [case([s], [], [s], 1) for s in bad]
    cases.append(case([good], [], [good, good], 1))         # duplicate segment
    cases.append(case([good], [], [good], 1, mode=5))       # unknown mode
    out = run(driver, cases)
    assert all(line.startswith("status ") for line in out), out


def test_invariant_check_catches_planted_mistakes(driver):
    """Copies of the 480p step's plan with one mistake each (an uncovered
    iteration, a list out of order, a list entry on an EMPTY tile, a piece
    past its list, split units never merged, a rotation out of range, a mask
    bit cleared on a tile where a row that sees keys misses one): the
    invariant check flags every one."""
    w = wl.cached_step_480p()
    c = case(w.q_layout, w.cached, w.new).replace("\nE", "\nX")
    out = run(driver, [c])
    assert out == ["caught 7 7"], out
