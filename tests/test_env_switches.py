"""NOMAS_TRACE and NOMAS_DEBUG_CHECKS (CPU: host-only plans in a child
process, since the library reads the switches once per process)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PLAN_ALL = """
import segment_causal_masked_amd as nm
from segment_causal_masked_amd import workloads as wl
for fn in wl.WORKLOADS.values():
    w = fn()
    for keep in (0, 25):
        p = nm.nomas_attn_plan(w.q_layout, w.cached + w.new, heads=w.heads, host_only=True,
                               video_keep_percent=keep)
print("planned")
"""


def child(code, **env):
    e = dict(os.environ, PYTHONPATH=ROOT, **env)
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=e,
                          timeout=300)


def test_trace_prints_plan_statistics():
    r = child(PLAN_ALL, NOMAS_TRACE="1")
    assert r.returncode == 0 and "planned" in r.stdout, r.stderr
    lines = [l for l in r.stderr.splitlines() if l.startswith("nomas_attn_plan:")]
    assert len(lines) == 10
    # the 480p cached step: 3,280 queries, 16,400 keys, A = 52,370,432
    assert any("queries 3280 keys 16400" in l and "A 52370432" in l for l in lines), lines
    r = child(PLAN_ALL)
    assert "nomas_attn_plan:" not in r.stderr


def test_debug_checks_validate_every_plan():
    r = child(PLAN_ALL, NOMAS_DEBUG_CHECKS="1")
    assert r.returncode == 0 and "planned" in r.stdout, r.stderr
