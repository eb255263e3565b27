"""Host logic of bench.py's recorded evidence: the traffic records are keyed
to a hash of each kernel source's code, so that a comment edit keeps them and
a code edit drops them."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_code_text_ignores_comments_and_whitespace():
    a = 'int x = 1;   // one\n/* block\n comment */ float y = 2.f;\n'
    b = 'int x = 1;\n\n  float   y = 2.f;  // another\n'
    assert bench._code_text(a) == bench._code_text(b)
    assert bench._code_text('int x = 2;') != bench._code_text('int x = 1;')


def test_code_text_keeps_literals():
    # comment markers inside string and character literals are code
    s = 'const char *p = "a // not a comment"; char c = \'/\'; /* gone */ int z;'
    t = bench._code_text(s)
    assert '"a // not a comment"' in t and "'/'" in t and "gone" not in t
    assert bench._code_text('puts("a\\" // b");') == 'puts("a\\" // b");'


def test_traffic_record_used_only_while_the_code_matches(tmp_path, monkeypatch):
    """A record is reported while the kernel's code is unchanged (comments
    aside) and dropped once the code changes."""
    src = tmp_path / "k.hip"
    src.write_text("__global__ void k() { int x = 1; }  // v1\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setitem(bench.KERNEL_SOURCES, "k", "k.hip")
    rec = {"kernels": {"k": {"bytes_per_launch": 1234, "source_sha256": bench._sha("k.hip")}}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    assert bench._traffic("k") == 1234
    src.write_text("__global__ void k() {\n  int x = 1;   // v2: reworded\n}\n")
    assert bench._traffic("k") == 1234
    src.write_text("__global__ void k() { int x = 2; }\n")
    assert bench._traffic("k") is None
