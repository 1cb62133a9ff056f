"""The kernel-source hash that gates the measured HBM traffic in the bench line:
blind to comments and layout, sensitive to any change of code."""
import bench

SRC = '''// leading comment
#include "x.h"
/* block
   comment */ int f(int a) {  // trailing
  const char *s = "not // a comment";
  const char c = '/';
  return a + 1;
}
'''


def test_comments_and_layout_ignored():
    edited = SRC.replace("// leading comment", "// another wording\n// over two lines")
    edited = edited.replace("return a + 1;", "return   a +\n      1;   /* note */")
    assert bench.code_text(edited) == bench.code_text(SRC)


def test_code_changes_detected():
    assert bench.code_text(SRC.replace("a + 1", "a + 2")) != bench.code_text(SRC)
    assert bench.code_text(SRC.replace("'/'", "'*'")) != bench.code_text(SRC)


def test_literals_kept():
    t = bench.code_text(SRC)
    assert '"not // a comment"' in t and "'/'" in t
    assert "leading" not in t and "trailing" not in t and "block" not in t


def test_hash_is_stable():
    assert bench.kernel_source_hash() == bench.kernel_source_hash()
    assert len(bench.kernel_source_hash()) == 16
