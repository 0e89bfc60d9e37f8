"""Host-side pieces of bench.py: the source hash that ties the committed
counter summaries to the kernels' code, and the one-GPU guard."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_code_text_drops_comments_and_keeps_literals():
    src = ('int a = 1; // line comment with "quotes"\n'
           '/* block\n comment */ const char *s = "not // a comment";\n'
           "char c = '/'; char d = '\\''; float x = 2.0f; /* tail */")
    out = bench.code_text(src)
    assert "comment" not in out.replace("not // a comment", "")
    assert '"not // a comment"' in out
    assert "'/'" in out and "'\\''" in out
    assert out == ('int a = 1; const char *s = "not // a comment"; '
                   "char c = '/'; char d = '\\''; float x = 2.0f;")


def test_code_text_ignores_comment_and_whitespace_edits():
    a = "x = y + 1; // old note\nreturn x;"
    b = "x = y + 1;   /* new, longer\n note */\n\n  return x;"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text("x = y + 2; return x;")


def test_source_hash_is_stable():
    assert bench.source_hash() == bench.source_hash()
    assert len(bench.source_hash()) == 16


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
