"""The debug build (libcsa_debug.so, CSA_DEBUG): its device-side index checks
count nothing on valid inputs (a fused decode step and csa_sparse_attn, the
fused top-k against the oracle), and an out-of-range CSA index given to
csa_sparse_attn is counted and treated as padding.  The debug library runs in
a process of its own (the binding picks it with CSA_LIBRARY=debug)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_debug_build_checks_indices():
    lib = os.path.join(ROOT, "long_context_compressed_05_amd", "libcsa_debug.so")
    assert os.path.exists(lib), "libcsa_debug.so is built by __graft_entry__.build()"
    env = dict(os.environ, CSA_LIBRARY="debug")
    r = subprocess.run([sys.executable, "-u", "-m", "tests._debug_checks_run"], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, f"{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
    res = json.loads(r.stdout.strip().splitlines()[-1])
    assert res["lib"] == "libcsa_debug.so"
    assert res["fused_violations"] == 0
    assert res["valid_violations"] == 0
    assert res["bad_violations"] > 0
    assert res["pad_violations"] == 0
    assert res["bad_equals_pad"]
    assert res["other_rows_unchanged"]
