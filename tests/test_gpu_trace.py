"""PAGEDATTN_TRACE: the launch trace of one grouped decode step (a shared-prefix
batch, bench.py's launch) in a child process, since the level is read once per
process. Level 2 also waits for the plan and prints its list; unset, the library
prints nothing."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
import torch
import bench, workloads
import paged_kv_cache_52_amd as pa
b = workloads.make_batch("shared_prefix_bf16", 5, "cuda", groups=2, suffix_max=300)
st = bench.Step(pa, b, 0, 0)
st()
torch.cuda.synchronize()
print("step done", flush=True)
"""


def _run(level):
    env = dict(os.environ)
    env.pop("PAGEDATTN_TRACE", None)
    if level is not None:
        env["PAGEDATTN_TRACE"] = level
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT], env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "step done" in r.stdout
    return [l for l in r.stderr.splitlines() if l.startswith("[pagedattn] ")]


@pytest.mark.gpu
def test_trace_level_2_prints_launches_and_plan():
    print("[case] PAGEDATTN_TRACE=2", flush=True)
    lines = _run("2")
    text = "\n".join(lines)
    for what in ("paged_decode_prepare:", "plan:", "paged_attn_decode_partial:",
                 "split kernel: MFMA engine", "paged_attn_reduce:"):
        assert f"[pagedattn] {what}" in text, (what, text)
    plan = [l for l in lines if l.startswith("[pagedattn] plan:")][0]
    entries = int(plan.split("plan: ")[1].split(" entries")[0])
    groups = int(plan.split("(")[1].split(" group entries")[0])
    assert entries > 0 and 0 < groups <= entries, plan


@pytest.mark.gpu
def test_trace_unset_is_silent():
    print("[case] PAGEDATTN_TRACE unset", flush=True)
    assert _run(None) == []
