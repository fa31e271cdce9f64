"""CPU tests of bench.py's contract pieces that need no GPU: the refusal of
more than one GPU, and the source digest that ties committed profiler
counters to the kernel code they were taken on."""
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_digest_ignores_comments_and_whitespace_only(tmp_path):
    for f in {f for fs in bench.KERNEL_SOURCES.values() for f in fs}:
        shutil.copy(os.path.join(bench.CSRC, f), tmp_path / f)
    base = bench.source_digest("prefill", str(tmp_path))
    assert base == bench.source_digest("prefill")
    src = (tmp_path / "prefill.hip").read_text()
    # a comment (line and block) and re-indentation: same digest
    (tmp_path / "prefill.hip").write_text("// note\n/* block\n note */\n" +
                                          src.replace("\n", "\n  "))
    assert bench.source_digest("prefill", str(tmp_path)) == base
    # one character of code: another digest; the other family is unaffected
    (tmp_path / "prefill.hip").write_text(src.replace("BN = 64", "BN = 32", 1))
    assert bench.source_digest("prefill", str(tmp_path)) != base
    assert bench.source_digest("decode", str(tmp_path)) == bench.source_digest("decode")
    # elem.h belongs to both families
    (tmp_path / "prefill.hip").write_text(src)
    e = (tmp_path / "elem.h").read_text()
    (tmp_path / "elem.h").write_text(e.replace("max_parts = 3", "max_parts = 2", 1))
    assert bench.source_digest("prefill", str(tmp_path)) != base
    assert bench.source_digest("decode", str(tmp_path)) != bench.source_digest("decode")
