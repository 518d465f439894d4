"""Host logic of bench.py that decides whether committed profile figures still apply.

A counter summary under profiles/ carries the digest of the kernel code it was taken
on; the bench reports its traffic only while the tree's digest matches.  The digest
covers code only, so that editing a comment keeps the figures, while any change of
code drops them.
"""
import os

import bench


def test_code_only_drops_comments_and_keeps_literals():
    src = 'int a = 1; // note\n/* block\n  comment */ const char *s = "x // y /* z */";\nchar q = \'"\';'
    assert bench.code_only(src) == 'int a = 1; const char *s = "x // y /* z */"; char q = \'"\';'
    assert bench.code_only("a  =\n\n b ;") == "a = b ;"


def _fake_tree(tmp_path, text):
    csrc = tmp_path / "memory_hierarchy_optimisation_amd" / "csrc"
    csrc.mkdir(parents=True, exist_ok=True)
    (csrc / "k.hip").write_text(text)
    return tmp_path


def test_digest_ignores_comments_but_not_code(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(_fake_tree(tmp_path, "int f() { return 1; } // one\n")))
    d0 = bench.kernel_source_digest()
    _fake_tree(tmp_path, "/* a comment\n */ int f() {\n  return 1;\n}\n")
    assert bench.kernel_source_digest() == d0
    _fake_tree(tmp_path, "int f() { return 2; }\n")
    assert bench.kernel_source_digest() != d0


def test_traffic_only_for_the_matching_digest(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(_fake_tree(tmp_path, "int f();\n")))
    prof = tmp_path / "profiles"
    prof.mkdir()
    d = bench.kernel_source_digest()
    (prof / "counters_w.txt").write_text(f"# header\nkernel_source_digest: {d}\ntraffic_bytes_per_launch: 1234\n")
    assert bench.traffic_for("w") == 1234.0
    (prof / "counters_w.txt").write_text("kernel_source_digest: 0000000000000000\ntraffic_bytes_per_launch: 1234\n")
    assert bench.traffic_for("w") is None
    assert bench.traffic_for("absent") is None
    assert not os.path.exists(prof / "counters_absent.txt")
