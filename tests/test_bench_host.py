"""Host logic of bench.py that needs no GPU: the code hash that keys the
stored HBM traffic records."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402


def test_code_only_drops_comments_keeps_literals():
    src = ('#include "a.h"  // trailing\n'
           '/* block\n   comment */ int x = 1; /* inline */ int y = 2;\n'
           '\n'
           '    const char *s = "not // a comment /* either */";\n'
           "char c = '/'; char d = '\\''; // after a quote\n"
           'const char *e = "esc \\" // still a string";\n')
    got = bench.code_only(src)
    assert got.split("\n") == [
        '#include "a.h"',
        'int x = 1;   int y = 2;',
        'const char *s = "not // a comment /* either */";',
        "char c = '/'; char d = '\\'';",
        'const char *e = "esc \\" // still a string";',
    ]


def test_code_only_sees_code_changes():
    a = "int f() { return 1; }  // one\n"
    assert bench.code_only(a) == bench.code_only("// header\nint f() { return 1; }\n\n")
    assert bench.code_only(a) != bench.code_only("int f() { return 2; }\n")
    # tokens are not joined across a removed block comment
    assert bench.code_only("int/**/x;") == "int x;"


def test_kernel_source_hash_ignores_comment_edits(tmp_path, monkeypatch):
    p = tmp_path / "k.hip"
    p.write_text("__global__ void k(float *x) { x[0] = 1.f; }\n")
    monkeypatch.setitem(bench.KERNEL_SRCS, "probe", [str(p)])
    h0 = bench.kernel_source_hash("probe")
    p.write_text("// a kernel\n\n  __global__ void k(float *x) { x[0] = 1.f; }  /* one */\n")
    assert bench.kernel_source_hash("probe") == h0
    p.write_text("__global__ void k(float *x) { x[0] = 2.f; }\n")
    assert bench.kernel_source_hash("probe") != h0


def test_every_pass_hashes_existing_sources():
    for which, paths in bench.KERNEL_SRCS.items():
        assert paths and all(os.path.isfile(p) for p in paths), which
        assert len(bench.kernel_source_hash(which)) == 16
