"""Host logic of bench.py that needs no GPU: the kernel-source digest that
ties a committed counter summary to the kernel it was taken on, and the
refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_release_lines_drop_comments_blanks_and_debug_blocks():
    src = [
        "int a;\n",
        "  // a comment\n",
        "\n",
        "#ifdef CSA_DEBUG\n",
        "#if 1\n",
        "int hidden;\n",
        "#endif\n",
        "int also_hidden;\n",
        "#endif\n",
        "#ifdef OTHER\n",
        "int kept;\n",
        "#endif\n",
        "int b;  // trailing comment stays\n",
    ]
    assert list(bench.release_lines(src)) == ["int a;", "#ifdef OTHER", "int kept;", "#endif",
                                              "int b;  // trailing comment stays"]


@pytest.mark.parametrize("bad", [["#ifdef CSA_DEBUG\n", "int x;\n"],
                                 ["#ifdef CSA_DEBUG\n", "#else\n", "int y;\n", "#endif\n"]])
def test_release_lines_reject_what_they_cannot_classify(bad):
    with pytest.raises(ValueError):
        list(bench.release_lines(bad))


def test_code_changes_outside_debug_blocks_change_the_digest():
    base = ["int a;\n", "#ifdef CSA_DEBUG\n", "int dbg;\n", "#endif\n"]
    assert list(bench.release_lines(base)) == list(bench.release_lines(base[:1]))
    assert list(bench.release_lines(base)) != list(bench.release_lines(["int a2;\n"] + base[1:]))


def test_committed_counter_summaries_parse():
    """Every traffic record under profiles/ names a kernel the digest knows;
    the ones whose sources are unchanged give a positive byte count."""
    import json
    prof = os.path.join(ROOT, "profiles")
    seen = 0
    for name in sorted(os.listdir(prof)):
        with open(os.path.join(prof, name)) as fh:
            for line in fh:
                if line.startswith("traffic-json: "):
                    rec = json.loads(line[len("traffic-json: "):])
                    assert rec["kernel"] in bench.KERNEL_SOURCES
                    t = bench.counted_traffic(rec["kernel"], rec["workload"])
                    if rec["source_sha256"] == bench.kernel_source_digest(rec["kernel"]):
                        assert t == rec["traffic_bytes_per_launch"] > 0
                    else:
                        assert t is None
                    seen += 1
    assert seen >= 1


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "--gpus 1" in (r.stdout + r.stderr)
