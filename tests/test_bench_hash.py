"""bench.kernel_source_hash: a traffic figure measured on some kernel sources is
reported only while the sources' code is unchanged; comments and layout do not
count as a change."""
import os

import bench


def _hash_of(tmp_path, text):
    d = tmp_path / "csrc"
    d.mkdir(exist_ok=True)
    (d / "k.hip").write_text(text)
    old = bench.CSRC
    bench.CSRC = str(d)
    try:
        return bench.kernel_source_hash()
    finally:
        bench.CSRC = old


def test_comments_and_layout_do_not_change_the_hash(tmp_path):
    base = "// a kernel\n__global__ void k(int* p) {\n  p[0] = 1;  // store\n}\n"
    edited = "/* another\n   comment */\n__global__   void k(int* p)\n{\n    p[0] = 1;\n}\n"
    assert _hash_of(tmp_path, base) == _hash_of(tmp_path, edited)


def test_code_changes_change_the_hash(tmp_path):
    base = "__global__ void k(int* p) { p[0] = 1; }\n"
    assert _hash_of(tmp_path, base) != _hash_of(tmp_path, base.replace("= 1", "= 2"))


def test_hash_of_the_tree_is_stable():
    assert bench.kernel_source_hash() == bench.kernel_source_hash()
    assert os.path.isdir(bench.CSRC)
