"""bench.py's kernel-code hash, which keeps or voids the committed HBM-traffic
counters: comments and whitespace do not count, code does."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_comments_and_whitespace_do_not_count():
    code = "int f(int x) {\n  return x + 1;  // one more\n}\n"
    same = "/* a note\n   over lines */ int f(int x) {\n\n    return x + 1;\n}  // end\n"
    assert bench._code_only(code) == bench._code_only(same)


def test_code_changes_count():
    a = "int f(int x) { return x + 1; }"
    b = "int f(int x) { return x + 2; }"
    assert bench._code_only(a) != bench._code_only(b)
    # a token split by whitespace is a different program
    assert bench._code_only("a = b+c;") != bench._code_only("a = b + +c;")


def test_hash_is_stable():
    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()
