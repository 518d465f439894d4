"""Plans run concurrently on two streams, on the GPU.

Distinct plans own distinct workspaces, and a plan without a workspace may run on
several streams at once with distinct C.  This test enqueues, on two streams at
default priority, a skinny split-K plan and an eight-wave split-K plan (each with its
own workspace and, for the skinny kernel, its own arrival counters) alternating with
one plan that has no workspace writing two different C buffers, five rounds
without host synchronisation in between, and checks every output bit for bit
against the same calls run one after another.
"""
import pytest
import torch

import memory_hierarchy_optimisation_amd as mh
import synth

pytestmark = pytest.mark.gpu


def _operands(M, N, K, in_t, seed):
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, in_t, dist="int", r=3, seed=seed)
    return As.cuda(), lda, Bs.cuda(), ldb


def _bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).cpu()


def test_distinct_plans_on_two_streams_match_serial_runs():
    cases = [(16, 2048, 4096, "bf16", "f32"), (512, 512, 8192, "bf16", "bf16"), (512, 512, 512, "f16", "f16")]
    ops, plans = [], []
    try:
        for i, (M, N, K, in_t, out_t) in enumerate(cases):
            A, lda, B, ldb = _operands(M, N, K, in_t, seed=50 + i)
            ops.append((A, B, M, N, out_t))
            plans.append(mh.gemm_plan(M, N, K, lda, ldb, N, mh.DTYPE_OF[(in_t, out_t)], 0))
        descs = [mh.gemm_plan_describe(p) for p in plans]
        print(f"[streams] workspaces {[d['workspace_bytes'] for d in descs]}", flush=True)
        assert descs[0]["workspace_bytes"] > 0 and descs[1]["workspace_bytes"] > 0
        assert descs[2]["workspace_bytes"] == 0

        def out(i):
            _, _, M, N, out_t = ops[i]
            return torch.zeros((M, N), dtype=synth.TORCH_DTYPES[out_t], device="cuda")

        # Serial reference: each plan once on the current stream.
        want = []
        for i, p in enumerate(plans):
            C = out(i)
            mh.gemm_run(p, ops[i][0], ops[i][1], C)
            want.append(C)
        torch.cuda.synchronize()
        want = [_bits(c) for c in want]

        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        for rnd in range(5):
            C0, C1, C2a, C2b = out(0), out(1), out(2), out(2)
            torch.cuda.synchronize()
            print(f"[streams] round {rnd}", flush=True)
            mh.gemm_run(plans[0], ops[0][0], ops[0][1], C0, stream=s1)
            mh.gemm_run(plans[1], ops[1][0], ops[1][1], C1, stream=s2)
            mh.gemm_run(plans[2], ops[2][0], ops[2][1], C2a, stream=s1)
            mh.gemm_run(plans[2], ops[2][0], ops[2][1], C2b, stream=s2)
            torch.cuda.synchronize()
            for got, w, what in ((C0, want[0], "skinny split-K"), (C1, want[1], "eight-wave split-K"),
                                 (C2a, want[2], "no workspace, stream 1"), (C2b, want[2], "no workspace, stream 2")):
                assert torch.equal(_bits(got), w), f"round {rnd}: {what} differs from the serial run"
    finally:
        for p in plans:
            mh.gemm_destroy(p)
