"""Host-side checks of the autotuning table (gemm_tune_load / gemm_tune_save /
gemm_tune_clear, and gemm_plan consulting the table) and of gemm_autotune's
argument checks.  The sweep itself times kernels and is covered by the GPU tests;
nothing here launches one."""

import pytest

import memory_hierarchy_optimisation_amd as mh

HEADER = "# mhgemm tuned configurations v1\n"
# 1024^3 fp16 -> fp16, row-major: the heuristic takes the 64x64 eight-wave tile.
P1024 = (1024, 1024, 1024, 1024, 1024, 1024, mh.GEMM_F16_F16, 0)
REG128 = (2, 128, 128, 64, 2, 2, 2, 1)      # register-staged 128x128 MFMA variant
W8_64 = (2, 64, 64, 128, 2, 4, 5, 1)


def _line(problem, cfg, us=1.0):
    return " ".join(map(str, problem)) + " | " + " ".join(map(str, cfg)) + f" | {us}\n"


def _describe(problem):
    p = mh.gemm_plan(*problem)
    try:
        return mh.gemm_plan_describe(p)
    finally:
        mh.gemm_destroy(p)


def _cfg_of(d):
    return tuple(d[k] for k in ("kind", "bm", "bn", "bk", "waves_m", "waves_n", "stages", "split_k"))


@pytest.fixture(autouse=True)
def _empty_table():
    mh.gemm_tune_clear()
    yield
    mh.gemm_tune_clear()


def test_catalogue_lists_every_compiled_variant_once():
    cat = mh.gemm_catalogue()
    assert len(cat) == len(set(cat)) > 10
    assert REG128 in cat and W8_64 in cat
    for c in cat:
        assert c[0] in (mh.GEMM_KIND_FMA, mh.GEMM_KIND_MFMA, mh.GEMM_KIND_SKINNY)
        # every listed configuration is accepted by gemm_plan_config for some problem
        M = 16 if c[0] == mh.GEMM_KIND_SKINNY else 512
        taken = 0
        for dt in (mh.GEMM_F32_F32, mh.GEMM_BF16_F32):
            try:
                p = mh.gemm_plan_config(M, 4096, 4096, 4096, 4096, 4096, dt, 0, c)
            except mh.GemmError as e:
                assert "input type" in str(e)
                continue
            assert _cfg_of(mh.gemm_plan_describe(p)) == c
            mh.gemm_destroy(p)
            taken += 1
        assert taken == 1        # every variant serves exactly one family of input types


def test_loaded_choice_overrides_the_heuristic_until_cleared(tmp_path):
    assert _cfg_of(_describe(P1024)) == W8_64
    f = tmp_path / "t.txt"
    f.write_text(HEADER + _line(P1024, REG128, 12.5))
    assert mh.gemm_tune_load(str(f)) == 1
    assert _cfg_of(_describe(P1024)) == REG128
    # another problem (different ldc) is not affected
    other = P1024[:5] + (2048,) + P1024[6:]
    assert _cfg_of(_describe(other)) == W8_64
    # a forced configuration still wins over the table
    p = mh.gemm_plan_config(*P1024, W8_64)
    assert _cfg_of(mh.gemm_plan_describe(p)) == W8_64
    mh.gemm_destroy(p)
    mh.gemm_tune_clear()
    assert _cfg_of(_describe(P1024)) == W8_64


def test_save_then_load_round_trip(tmp_path):
    probs = [P1024, (16, 8192, 8192, 8192, 8192, 8192, mh.GEMM_BF16_F32, 0),
             (2048, 2048, 2048, 2048, 2048, 2048, mh.GEMM_F16_F32, 2)]
    cfgs = [REG128, (3, 16, 128, 32, 1, 4, 2, 8), (2, 128, 128, 64, 2, 4, 5, 1)]
    f = tmp_path / "in.txt"
    f.write_text(HEADER + "".join(_line(p, c, 3.25 + i) for i, (p, c) in enumerate(zip(probs, cfgs))))
    assert mh.gemm_tune_load(str(f)) == 3
    g = tmp_path / "out.txt"
    assert mh.gemm_tune_save(str(g)) == 3
    mh.gemm_tune_clear()
    assert mh.gemm_tune_load(str(g)) == 3
    for p, c in zip(probs, cfgs):
        assert _cfg_of(_describe(p)) == c
    rows = [l for l in g.read_text().splitlines() if l and not l.startswith("#")]
    assert len(rows) == 3 and all(l.count("|") == 2 for l in rows)


def test_a_later_entry_replaces_an_earlier_one(tmp_path):
    f = tmp_path / "t.txt"
    f.write_text(HEADER + _line(P1024, REG128) + _line(P1024, W8_64))
    assert mh.gemm_tune_load(str(f)) == 1
    assert _cfg_of(_describe(P1024)) == W8_64


@pytest.mark.parametrize("bad,what", [
    ("1024 1024 1024 1024 1024 1024 1 0 | 2 128 128 64 2 2 2 | 1.0\n", "configuration fields"),
    ("1024 1024 1024 1024 1024 1024 1 0 | 2 128 128 64 2 2 2 1\n", "time"),
    ("1024 1024 1024 1000 1024 1024 1 0 | 2 128 128 64 2 2 2 1 | 1.0\n", "lda"),
    ("1024 1024 1024 1024 1024 1024 7 0 | 2 128 128 64 2 2 2 1 | 1.0\n", "dtype"),
    ("0 1024 1024 1024 1024 1024 1 0 | 2 128 128 64 2 2 2 1 | 1.0\n", "empty"),
    ("1024 1024 1024 1024 1024 1024 1 0 | 2 96 96 64 2 2 2 1 | 1.0\n", "not a compiled variant"),
    ("1024 1024 1024 1024 1024 1024 1 0 | 2 128 128 64 2 2 2 1 | 1.0 extra\n", "time"),
])
def test_a_bad_line_loads_nothing(tmp_path, bad, what):
    f = tmp_path / "t.txt"
    f.write_text(HEADER + _line(P1024, REG128) + "\n# comment\n" + bad)
    with pytest.raises(mh.GemmError, match="line 5") as e:
        mh.gemm_tune_load(str(f))
    assert e.value.code == mh.GEMM_ERR_INVALID_ARG
    assert what in str(e.value)
    assert _cfg_of(_describe(P1024)) == W8_64     # the good first line was not loaded either


def test_missing_file_and_unwritable_path(tmp_path):
    with pytest.raises(mh.GemmError, match="cannot open"):
        mh.gemm_tune_load(str(tmp_path / "absent.txt"))
    with pytest.raises(mh.GemmError, match="cannot open"):
        mh.gemm_tune_save(str(tmp_path / "no_such_dir" / "t.txt"))


def test_an_entry_that_no_longer_fits_falls_back_to_the_heuristic(tmp_path):
    # The eight-wave kernels need extents that are multiples of 8; a table entry naming
    # one for a ragged problem is accepted by the loader (both parts are valid) but the
    # planner then keeps its own choice.
    prob = (1001, 1001, 1001, 1001, 1001, 1001, mh.GEMM_F16_F16, 0)
    heuristic = _cfg_of(_describe(prob))
    assert heuristic != W8_64
    f = tmp_path / "t.txt"
    f.write_text(HEADER + _line(prob, W8_64))
    assert mh.gemm_tune_load(str(f)) == 1
    assert _cfg_of(_describe(prob)) == heuristic


def test_autotune_rejects_bad_arguments_before_touching_a_device():
    def tune(*a, **k):
        return mh.gemm_autotune(*a, **k)
    with pytest.raises(mh.GemmError, match="lda"):
        tune(64, 64, 64, 10, 64, 64, 0, 0, 1, 1, 1, stream=0)
    with pytest.raises(mh.GemmError, match="empty product"):
        tune(0, 64, 64, 64, 64, 64, 0, 0, 1, 1, 1, stream=0)
    with pytest.raises(mh.GemmError, match="NULL operand"):
        tune(64, 64, 64, 64, 64, 64, 0, 0, 0, 1, 1, stream=0)
    with pytest.raises(mh.GemmError, match="reps"):
        tune(64, 64, 64, 64, 64, 64, 0, 0, 1, 1, 1, stream=0, reps=0)
