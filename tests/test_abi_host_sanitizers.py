"""libcsa's host code (argument validation, workspace planning, launch
sizing) under AddressSanitizer and UndefinedBehaviorSanitizer: every source
compiled with the sanitizers on the host side only (device code is built as
usual and never runs here), linked with tests/abi_host_sanitize.cpp, which
calls every entry point with invalid and valid arguments on a machine without
a GPU and queries workspaces over extreme shapes.  A sanitizer report or an
unexpected status fails it."""
import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="no hipcc")
def test_abi_host_code_under_sanitizers(tmp_path):
    import torch
    if torch.cuda.is_available():
        pytest.skip("runs where no GPU is present (every valid call then stops at the device check)")
    from long_context_compressed_05_amd import build as B
    flags = [f"--offload-arch={B.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-Wno-unused-result",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN]

    def comp(src):
        obj = str(tmp_path / (os.path.splitext(os.path.basename(src))[0] + ".o"))
        r = subprocess.run([HIPCC, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    srcs = [os.path.join(B.CSRC, s) for s in B.SOURCES] + [os.path.join(ROOT, "tests", "abi_host_sanitize.cpp")]
    with cf.ThreadPoolExecutor(8) as ex:
        objs = list(ex.map(comp, srcs))
    exe = str(tmp_path / "abi_san")
    subprocess.run([HIPCC, f"--offload-arch={B.ARCH}", *HOST_SAN, *objs, "-o", exe], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"{r.stdout}\n{r.stderr[-4000:]}"
    assert "0 failures" in r.stdout
