"""Host logic of bench.py that needs no GPU: the kernel-source hash that ties a
committed profile to the code it measured, and the one-GPU rule."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_code_only_drops_comments_and_keeps_literals():
    src = ('int a = 1;  // trailing\n/* block\n   comment */ const char* s = "x // y /* z */";\n'
           "char q = '\"';\tint b =\n  2; // \"quoted\" in a comment\n")
    assert bench._code_only(src) == 'int a = 1; const char* s = "x // y /* z */"; char q = \'"\'; int b = 2;'


def test_escaped_quote_inside_a_literal():
    assert bench._code_only('f("a\\"b // c"); // d') == 'f("a\\"b // c");'


@pytest.fixture
def source_copy(tmp_path, monkeypatch):
    for rel in bench.KERNEL_SOURCES:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def test_hash_ignores_comment_edits_but_not_code_edits(source_copy):
    before = bench.kernel_source_hash()
    rel = bench.KERNEL_SOURCES[0]
    path = source_copy / rel
    text = path.read_text(encoding="utf-8")
    path.write_text("// an added comment line\n" + text.replace("\n", "\n\n", 3), encoding="utf-8")
    assert bench.kernel_source_hash() == before
    path.write_text(text + "\nstatic int added_symbol = 1;\n", encoding="utf-8")
    assert bench.kernel_source_hash() != before


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
