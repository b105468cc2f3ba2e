"""CPU check of the planner's closed-form per-request arithmetic.

The device planner and the host sizing share `request_counts`,
`rw_row_of_item`, `chunk_item_of` and `chunk_merge_of` (pa_internal.h), which
compute item counts, record positions and partial-slot offsets without
looping over rows or q-tiles.  `plan_closed_forms_check.cpp` compares them,
on exhaustive small ranges and random large requests, with the same
quantities written as plain loops over every row and q-tile.  The program is
built here with hipcc (host code only runs) and must print "ok"."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def test_plan_closed_forms_match_their_loop_definitions(tmp_path):
    if not (os.path.exists(HIPCC) or shutil.which("hipcc")):
        pytest.skip("hipcc not available")
    exe = tmp_path / "plan_check"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17",
           "-I" + os.path.join(ROOT, "paged_kv_attention_reshape_amd", "csrc"),
           "-I" + os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "plan_closed_forms_check.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok"), out.stdout
