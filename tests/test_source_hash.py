"""The kernel-source hash that ties a measured HBM traffic record to the code
it was measured on: comments and whitespace do not count, code does."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402


def test_comments_and_whitespace_do_not_count():
    a = 'int f(int x) {\n  return x + 1;  // one more\n}\n'
    b = '/* doc */ int f(int x)\n{ return x + 1; }'
    assert bench.strip_comments(a) == bench.strip_comments(b)


def test_code_counts():
    a = 'int f(int x) { return x + 1; }'
    b = 'int f(int x) { return x + 2; }'
    assert bench.strip_comments(a) != bench.strip_comments(b)


def test_comment_markers_inside_literals_are_code():
    s = 'asm volatile("s_nop 0 // not a comment"); char c = \'/\'; int d = 1 /* gone */;'
    out = bench.strip_comments(s)
    assert '"s_nop 0 // not a comment"' in out
    assert "'/'" in out
    assert "gone" not in out

