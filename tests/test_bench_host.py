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


def test_trace_summary_takes_the_first_gemm_kernel_as_the_headline(tmp_path):
    # A later, shorter kernel with more dispatches (a per-shape line that settles for a
    # fixed time) must not be taken for the headline.
    rows = ["Kernel_Name,Start_Timestamp,End_Timestamp"]
    t = 1000
    for i in range(6):                         # headline: 2 untimed + 3 timed + 1 more
        rows.append(f'"void mhg::w8::w8_gemm<Big>(x)",{t},{t + 100 + i}')
        t += 200
    for i in range(20):
        rows.append(f'"void mhg::w8::w8_gemm<Small>(x)",{t},{t + 8}')
        t += 20
    rows.insert(1, f'"elementwise_copy",{10},{20}')
    csv_path, out = tmp_path / "kt.csv", tmp_path / "out.txt"
    csv_path.write_text("\n".join(rows) + "\n")
    bench.summarize_trace(str(csv_path), "d" * 16, str(out), 1, 1, 3, "w")
    text = out.read_text()
    assert "# Headline kernel (w): void mhg::w8::w8_gemm<Big>(x)" in text
    assert "headline_timed_mean_ns: 103  (dispatches 3 .. 5 of it)" in text


def test_tidy_keeps_times_to_the_nanosecond():
    # A mean printed to 0.1 us would fall outside percentiles printed in full.
    r = bench.tidy({"kernel_ms_event": 0.00849951, "ms_per_step": 0.0041234567, "tflops": 255.123456,
                    "kernel_ms_p10_p50_p90": [0.0084, 0.0085, 0.0086], "grid": 256})
    assert r == {"kernel_ms_event": 0.0085, "ms_per_step": 0.004123, "tflops": 255.1235,
                 "kernel_ms_p10_p50_p90": [0.0084, 0.0085, 0.0086], "grid": 256}
    assert bench.tidy({"kernel_ms_event": 0.0084996})["kernel_ms_event"] == 0.0085
    assert bench.tidy({"kernel_ms_event": 0.0085004})["kernel_ms_event"] == 0.0085
    assert bench.tidy({"kernel_ms_event": 0.0084994})["kernel_ms_event"] == 0.008499


def test_group_bounds_cover_the_calls_in_order():
    for steps, groups in [(300, 30), (3540, 30), (7, 7), (301, 30), (1, 1)]:
        b = bench.group_bounds(steps, groups)
        assert b[0] == 0 and b[-1] == steps and len(b) == groups + 1
        sizes = [b[g + 1] - b[g] for g in range(groups)]
        assert min(sizes) >= 1 and max(sizes) - min(sizes) <= 1
    assert bench.group_bounds(300, 30) == list(range(0, 301, 10))


def test_short_calls_get_groups_of_at_least_the_minimum_span():
    # 8.5 us calls: 118 a group of 1 ms, 30 groups.
    assert bench.steps_for_groups(300, 0.0085, 1.0) == 30 * 118
    # 100 us calls already span 1 ms in groups of 10: the 300 steps stay.
    assert bench.steps_for_groups(300, 0.1, 1.0) == 300
    # never fewer calls than asked for
    assert bench.steps_for_groups(900, 0.5, 1.0) == 900
