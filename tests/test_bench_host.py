"""Host logic of bench.py that needs no GPU: the kernel-source digest that
ties the committed traffic records to the code they were measured on."""
import os
import shutil

import bench


def test_code_only_drops_comments_and_keeps_code():
    src = ('int a = 1; // a comment\n'
           '/* a block\n   comment */ int b = 2;\n'
           '\n'
           'const char* s = "http://x /* not a comment */";   \n'
           "char c = '/'; char d = '\\''; // done\n")
    out = bench._code_only(src)
    assert out == ('int a = 1;\n'
                   ' int b = 2;\n'
                   'const char* s = "http://x /* not a comment */";\n'
                   "char c = '/'; char d = '\\'';")


def test_digest_ignores_comments_but_not_code(tmp_path):
    csrc = tmp_path / "rejection_sampling_verify_12_amd" / "csrc"
    shutil.copytree(os.path.join(bench.ROOT, "rejection_sampling_verify_12_amd", "csrc"), csrc)
    root = bench.ROOT
    try:
        bench.ROOT = str(tmp_path)
        d0 = bench.source_digest()
        f = csrc / "verify_topp.h"
        text = f.read_text()
        f.write_text("// an added comment line\n" + text.replace("\n", "   \n", 3))
        assert bench.source_digest() == d0
        f.write_text(text.replace("kListCap = 1792", "kListCap = 1791"))
        assert bench.source_digest() != d0
    finally:
        bench.ROOT = root
