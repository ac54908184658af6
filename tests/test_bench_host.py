"""Host-side helpers of bench.py (no GPU): the kernel-source digest that ties
a committed counter summary to the code it was measured on."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_code_only_drops_comments_and_layout():
    src = 'int a = 1; // it\'s a note\n/* block\n   comment */ const char* s = "x // y";\nchar q = \'/\';\n\n  int   c;'
    assert bench._code_only(src) == 'int a = 1; const char* s = "x // y"; char q = \'/\'; int c;'


def test_digest_ignores_comments_but_not_code(tmp_path, monkeypatch):
    files = {}
    for rel in bench.KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            files[rel] = f.read()
    for rel, text in files.items():
        os.makedirs(tmp_path / os.path.dirname(rel), exist_ok=True)
        (tmp_path / rel).write_text(text)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.kernel_source_digest()
    assert base == bench.kernel_source_digest()
    first = bench.KERNEL_SOURCES[0]
    (tmp_path / first).write_text(files[first] + "\n// a new comment\n/* and another */\n")
    assert bench.kernel_source_digest() == base
    (tmp_path / first).write_text(files[first] + "\nstatic int extra_symbol = 0;\n")
    assert bench.kernel_source_digest() != base

