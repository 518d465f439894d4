"""The autotuning sweep on the GPU: gemm_autotune times every variant that fits, the
fastest is what gemm_plan then picks for that exact problem, and every product the
sweep and the tuned plan compute matches the oracle.  The table is process-wide, so
each test empties it before and after."""
import pytest
import torch

import memory_hierarchy_optimisation_amd as mh
import synth
from gemm_cases import check_tolerance, dtype_code, oracle_ref, run_gpu

pytestmark = pytest.mark.gpu

CFG_KEYS = ("kind", "bm", "bn", "bk", "waves_m", "waves_n", "stages", "split_k")


@pytest.fixture(autouse=True)
def _empty_table():
    mh.gemm_tune_clear()
    yield
    mh.gemm_tune_clear()


@pytest.mark.parametrize("name,reps", [("f16_1024", 5), ("f16_2048_nt", 3), ("bf16_skinny", 3)])
def test_autotune_then_plan(name, reps):
    w = synth.WORKLOADS[name]
    As, lda, Bs, ldb, _, _ = synth.workload_operands(w)
    layout = (mh.GEMM_A_COL if w.a_col else 0) | (mh.GEMM_B_COL if w.b_col else 0)
    code = dtype_code(w.dtype, w.out)
    print(f"[autotune {name}] M={w.M} N={w.N} K={w.K} reps={reps}", flush=True)
    A, B = As.cuda(), Bs.cuda()
    C = torch.empty((w.M, w.N), dtype=synth.TORCH_DTYPES[w.out], device="cuda")
    p = mh.gemm_plan(w.M, w.N, w.K, lda, ldb, w.N, code, layout)
    heuristic = tuple(mh.gemm_plan_describe(p)[k] for k in CFG_KEYS)
    mh.gemm_destroy(p)

    best, best_us, times = mh.gemm_autotune(w.M, w.N, w.K, lda, ldb, w.N, code, layout, A, B, C, reps=reps)
    torch.cuda.synchronize()
    cat = mh.gemm_catalogue()
    timed = {cat[i]: t for i, t in enumerate(times) if t >= 0}
    print(f"[autotune {name}] heuristic {heuristic}; best {best} {best_us:.2f} us; "
          + ", ".join(f"{c[1]}x{c[2]}x{c[3]}/s{c[7]}: {t:.1f}" for c, t in timed.items()), flush=True)
    assert len(timed) >= 2
    assert heuristic in timed                     # the planner's own choice is a candidate
    assert best in timed and timed[best] == best_us == min(timed.values())
    assert all(0.0 < t < 1e6 for t in timed.values())

    # The sweep leaves the product of its last candidate in C.
    Cref = oracle_ref(As, lda, Bs, ldb, w.M, w.N, w.K, w.dtype, w.a_col, w.b_col)
    check_tolerance(C.double().cpu().numpy(), Cref, w.out, f"{name} after the sweep")

    # A new plan for the same problem takes the measured configuration, and is correct.
    vals, _, desc = run_gpu(As, lda, Bs, ldb, w.M, w.N, w.K, w.dtype, w.out, w.a_col, w.b_col)
    assert tuple(desc[k] for k in CFG_KEYS) == best
    check_tolerance(vals, Cref, w.out, f"{name} with the tuned plan")


def test_tuned_table_survives_a_save_and_load(tmp_path):
    w = synth.WORKLOADS["f16_1000"]
    As, lda, Bs, ldb, _, _ = synth.workload_operands(w)
    code = dtype_code(w.dtype, w.out)
    A, B = As.cuda(), Bs.cuda()
    C = torch.empty((w.M, w.N), dtype=synth.TORCH_DTYPES[w.out], device="cuda")
    print("[autotune f16_1000] save / load", flush=True)
    best, _, _ = mh.gemm_autotune(w.M, w.N, w.K, lda, ldb, w.N, code, 0, A, B, C, reps=3)
    path = str(tmp_path / "tuned.txt")
    assert mh.gemm_tune_save(path) == 1
    mh.gemm_tune_clear()
    assert mh.gemm_tune_load(path) == 1
    vals, _, desc = run_gpu(As, lda, Bs, ldb, w.M, w.N, w.K, w.dtype, w.out)
    assert tuple(desc[k] for k in CFG_KEYS) == best
    check_tolerance(vals, oracle_ref(As, lda, Bs, ldb, w.M, w.N, w.K, w.dtype), w.out, "tuned 1000^3")
