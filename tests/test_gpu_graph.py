"""The product path under HIP graph capture, on the GPU.

gemm_run and gemm_run_epilogue allocate nothing and clear nothing with memset nodes:
plans own their workspaces, and the skinny kernel re-arms its arrival counters itself.
So a caller can capture calls into a graph once and replay it.  This test captures
one call of each kind that leaves state behind or launches more than one kernel (the
skinny split-K kernel with its counters, the eight-wave split-K kernel with its
reduction, the 256 x 256 tile with the prior C through LDS, a plain eight-wave call),
replays the graph three times with eager work between the replays (resetting C,
unrelated products), and checks every replay against the eager result bit for bit.
"""
import pytest
import torch

import memory_hierarchy_optimisation_amd as mh
import synth

pytestmark = pytest.mark.gpu

CFG256 = (2, 256, 256, 32, 2, 4, 5, 1)

# name, M, N, K, in, out, cfg, epilogue
CASES = [
    ("eight-wave", 512, 512, 512, "bf16", "bf16", None, None),
    ("skinny split-K", 16, 2048, 4096, "bf16", "f32", None, None),
    ("eight-wave split-K", 512, 512, 8192, "bf16", "bf16", None, None),
    ("256 tile, prior C through LDS", 300, 264, 136, "f16", "f16", CFG256, dict(alpha=0.5, beta=1.5)),
]


class _Call:
    def __init__(self, name, M, N, K, in_t, out_t, cfg, epi, seed):
        self.name = name
        As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, in_t, dist="int", r=3, seed=seed)
        Cs, bias = synth.epilogue_inputs(M, N, out_t, dist="int", r=4, seed=seed + 1)
        self.A, self.B = As.cuda(), Bs.cuda()
        self.C0 = Cs.cuda()
        self.C = self.C0.clone()
        self.bias = bias.to(torch.float32).cuda()
        code = mh.DTYPE_OF[(in_t, out_t)]
        self.plan = (mh.gemm_plan(M, N, K, lda, ldb, N, code, 0) if cfg is None
                     else mh.gemm_plan_config(M, N, K, lda, ldb, N, code, 0, cfg))
        self.epi = epi

    def run(self):
        if self.epi is None:
            mh.gemm_run(self.plan, self.A, self.B, self.C)
        else:
            mh.gemm_run_epilogue(self.plan, self.A, self.B, self.C, bias=self.bias, **self.epi)


def _bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).cpu()


def test_captured_calls_replay_like_eager_calls():
    calls = [_Call(*c, seed=31 + 7 * i) for i, c in enumerate(CASES)]
    try:
        for c in calls:
            print(f"[graph] eager {c.name}: {mh.gemm_plan_describe(c.plan)}", flush=True)
            c.run()
        torch.cuda.synchronize()
        want = [_bits(c.C) for c in calls]
        for c in calls:
            c.C.copy_(c.C0)
        torch.cuda.synchronize()

        print("[graph] capture", flush=True)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in calls:
                c.run()
        x = torch.randn(256, 256, device="cuda")
        for replay in range(3):
            for c in calls:
                c.C.copy_(c.C0)
            y = x @ x                      # eager work between the replays
            torch.cuda.synchronize()
            print(f"[graph] replay {replay}", flush=True)
            g.replay()
            torch.cuda.synchronize()
            assert torch.isfinite(y).all()
            for c, w in zip(calls, want):
                got = _bits(c.C)
                assert torch.equal(got, w), f"replay {replay}: {c.name} differs from the eager call"
    finally:
        for c in calls:
            mh.gemm_destroy(c.plan)
