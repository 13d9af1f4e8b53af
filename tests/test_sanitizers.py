"""The CPU code under sanitizers: the oracle (oracle/oracle.cpp) and the input
generator (synth/synth.c) built with AddressSanitizer and
UndefinedBehaviorSanitizer (and the multithreaded generator also with
ThreadSanitizer), each driven through every exported function on small and
degenerate inputs by its sanitize_check driver.  A sanitizer report makes the
driver exit non-zero.  Host compilers only; no GPU code is built here."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]


def _have(compiler, flag, tmp_path):
    src = tmp_path / "probe.c"
    src.write_text("int main(void) { return 0; }\n")
    r = subprocess.run([compiler, flag, str(src), "-o", str(tmp_path / "probe")], capture_output=True)
    return r.returncode == 0


def _build_and_run(cmd, exe):
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, f"{exe} failed:\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "0 failures" in r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="no g++")
def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    if not _have("g++", "-fsanitize=address,undefined", tmp_path):
        pytest.skip("the host compiler has no sanitizer runtime")
    exe = str(tmp_path / "oracle_san")
    _build_and_run(["g++", "-std=c++17", "-fsanitize=address,undefined", *SAN,
                    os.path.join(ROOT, "oracle", "oracle.cpp"), os.path.join(ROOT, "oracle", "sanitize_check.cpp"),
                    "-o", exe], exe)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
@pytest.mark.parametrize("sanitizer", ["address,undefined", "thread"])
def test_generator_under_sanitizers(tmp_path, sanitizer):
    if not _have("gcc", f"-fsanitize={sanitizer}", tmp_path):
        pytest.skip("the host compiler has no sanitizer runtime")
    exe = str(tmp_path / "synth_san")
    _build_and_run(["gcc", "-std=c11", f"-fsanitize={sanitizer}", *SAN, "-pthread",
                    os.path.join(ROOT, "synth", "synth.c"), os.path.join(ROOT, "synth", "sanitize_check.c"),
                    "-o", exe, "-lm"], exe)
