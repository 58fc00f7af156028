"""The bench's host-side contract (no GPU): one GPU only, and the argument
parser's defaults."""
import os
import subprocess
import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_help_lists_the_contract_flags():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--help"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup", "--no-cpu-baseline", "--sweep"):
        assert flag in r.stdout


def test_kernel_digest_ignores_comments_but_not_code(tmp_path, monkeypatch):
    """The digest that ties profiles/traffic.json to the sources changes with
    the code and stays put for comment and blank-line edits."""
    import shutil

    import bench

    pkg = tmp_path / "pkg"
    shutil.copytree(os.path.join(bench.PKG, "csrc"), pkg / "csrc")
    monkeypatch.setattr(bench, "PKG", str(pkg))
    base = bench.kernel_source_digest()
    src = pkg / "csrc" / "int4_gemv.hip"
    text = src.read_text()
    src.write_text("// a new comment\n\n" + text.replace("namespace qg {", "namespace qg {  // here", 1)
                   + "\n/* a block\n   comment */\n")
    assert bench.kernel_source_digest() == base
    src.write_text(text.replace("constexpr int kSpanRounds = 2;", "constexpr int kSpanRounds = 3;", 1))
    assert bench.kernel_source_digest() != base
