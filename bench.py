#!/usr/bin/env python3
"""Benchmark of the tiled GEMM on one MI355X.

One step = one call of the planned product (gemm_run) on one batch of synthetic
operands already resident in HBM.  Before the warm-up steps, the headline plan runs
SETTLE_CALLS untimed calls so that the clock has settled under the sustained load.
The headline workload is the bf16 4096^3 product (bf16 output, fp32 accumulation): value = 2*M*N*K / (wall seconds per step), in
TFLOP/s.  The other measured shapes are reported under "per_shape" with their
roofline fraction: min(peak, intensity * 8 TB/s), where intensity counts each
operand once (2MNK over the bytes of A, B and C).

Operands rotate over enough copies that the working set exceeds the 256 MB
Infinity Cache, so the bandwidth-bound shape streams from HBM.

After the timed region: the headline shape once more through the fused epilogue
(alpha = beta = 1, a bias, ReLU; "epilogue"), and for every shape but the 64^3 one an
autotune sweep of the compiled variants against the planner's choice ("autotune"), and
the tiled transpose of 8192^2 fp32 and 16-bit matrices ("transpose").

Prints ONE JSON line on stdout; everything else goes to stderr.
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HEADLINE = "bf16_4096"
PER_SHAPE = ["f32_64", "f16_1024", "f16_1000", "f16_2048_nt", "bf16_4096", "bf16_skinny"]
# Published dense peaks of the MI355X (TFLOP/s) and its HBM bandwidth (GB/s).
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}
HBM_GBPS = 8000.0
ELEM = {"f32": 4, "f16": 2, "bf16": 2}
ROTATE_BYTES = 512 << 20       # working set of rotated operand copies, > 256 MB cache
# Untimed calls of the headline plan before its warm-up.  Under a sustained 4096^3 load
# the power manager takes the clock down over the first ~150 calls (about 130 us a call
# instead of 105-115); these calls (~0.2 s) let it settle, so that the warm-up and the
# timed steps see the steady state whatever --warmup the caller passes.
SETTLE_CALLS = 2000
# Spread of the call times: the timed calls in 30 groups of consecutive calls.
PER_CALL_GROUPS = 30
# Window of the clock probe: 2,000,000 ticks of the 100 MHz real-time counter (20 ms).
CLOCK_TICKS = 2_000_000


def log(*a):
    print(*a, file=sys.stderr, flush=True)


_CODE_TOKENS = re.compile(r'"(?:\\.|[^"\\])*"|\'(?:\\.|[^\'\\])*\'|//[^\n]*|/\*.*?\*/', re.S)


def code_only(text):
    """C/C++ source with its comments removed and runs of whitespace collapsed (string
    and character literals are kept as they are)."""
    kept = _CODE_TOKENS.sub(lambda m: m.group(0) if m.group(0)[0] in "\"'" else " ", text)
    return re.sub(r"\s+", " ", kept).strip()


def kernel_source_digest():
    """Digest of the code of the kernel sources (comments and layout whitespace removed):
    profile figures carry it, so figures taken on other code are ignored, while an edit
    of a comment leaves them valid."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "memory_hierarchy_optimisation_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as fh:
            h.update(name.encode() + b"\0" + code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def algorithmic(w):
    flops = 2.0 * w.M * w.N * w.K
    nbytes = w.M * w.K * ELEM[w.dtype] + w.K * w.N * ELEM[w.dtype] + w.M * w.N * ELEM[w.out]
    return flops, nbytes


def roofline_of(w):
    flops, nbytes = algorithmic(w)
    ai = flops / nbytes
    peak = PEAK_TFLOPS[w.dtype]
    roof = min(peak, ai * HBM_GBPS / 1000.0)
    bound = "hbm" if ai * HBM_GBPS / 1000.0 < peak else ("mfma" if w.dtype != "f32" else "alu")
    return ai, roof, bound


def clock_during(run, first):
    """Shader clock (MHz) while the calls of `run` stream: the one-wave clock probe runs
    on a second stream (default priority) for CLOCK_TICKS real-time ticks, started after
    100 calls are queued and followed by enough calls to outlast its window."""
    import torch

    import memory_hierarchy_optimisation_amd as mh

    side = torch.cuda.Stream()
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    for i in range(100):
        run(first + i)
    mh.gemm_clock_probe(out.data_ptr(), CLOCK_TICKS, stream=side.cuda_stream)
    for i in range(100, 600):
        run(first + i)
    torch.cuda.synchronize()
    cycles, ticks = (int(v) for v in out.cpu().tolist())
    return 100.0 * cycles / ticks


def group_bounds(steps, groups):
    """Call indices where each of `groups` consecutive groups of the `steps` timed calls
    starts (and, last, where they end): sizes differ by at most one."""
    return [(g * steps) // groups for g in range(groups + 1)]


def steps_for_groups(steps, per_call_ms, min_group_ms):
    """Timed calls for PER_CALL_GROUPS groups of at least `min_group_ms` each, at
    `per_call_ms` a call, and never fewer than `steps`."""
    size = max(steps // PER_CALL_GROUPS, math.ceil(min_group_ms / per_call_ms))
    return max(steps, PER_CALL_GROUPS * size)


def tidy(r):
    """A line's figures for the JSON output: times in ms to the nanosecond (so that a
    mean can be compared with its own percentiles), other figures to four decimals."""
    return {k: (round(v, 6 if "_ms" in k or k.startswith("ms_") else 4) if isinstance(v, float) else v)
            for k, v in r.items()}


def measure(name, steps, warmup, settle=0, per_call=False, epilogue=False, clock=False, rotate=True,
            settle_s=0.0, min_group_ms=0.0):
    """Time `steps` calls after `settle` + `warmup` untimed calls.  Returns a dict of
    figures.  settle_s: before those, untimed calls in chunks of 50 until that many
    seconds have passed (the clock's settling takes time, not a number of calls).
    min_group_ms (with per_call): raise `steps` so that each group of timed calls takes
    at least that long by the warm-up's mean, which keeps the events between groups
    (~2.5 us each in the stream) below a few tenths of a percent of short calls.
    epilogue: run through the fused epilogue with alpha = beta = 1, a bias and ReLU (C is
    read as well as written; its bytes and the bias's count in the GB/s).  clock:
    afterwards, read the shader clock during a further run of calls."""
    import torch

    import memory_hierarchy_optimisation_amd as mh
    import synth

    w = synth.WORKLOADS[name]
    As, lda, Bs, ldb, _, _ = synth.workload_operands(w)
    pair = As.numel() * As.element_size() + Bs.numel() * Bs.element_size()
    copies = max(1, min(256, math.ceil(ROTATE_BYTES / pair))) if rotate else 1
    A0, B0 = As.cuda(), Bs.cuda()
    As_dev = [A0] + [A0.clone() for _ in range(copies - 1)]
    Bs_dev = [B0] + [B0.clone() for _ in range(copies - 1)]
    C = torch.zeros((w.M, w.N), dtype=synth.TORCH_DTYPES[w.out], device="cuda")
    code = mh.DTYPE_OF[(w.dtype, w.out)]
    layout = (mh.GEMM_A_COL if w.a_col else 0) | (mh.GEMM_B_COL if w.b_col else 0)
    plan = mh.gemm_plan(w.M, w.N, w.K, lda, ldb, w.N, code, layout)
    desc = mh.gemm_plan_describe(plan)
    stream = torch.cuda.current_stream()
    # Raw pointers and stream handle, taken once: the per-call Python work then stays
    # below the duration of the shortest kernels, which would otherwise wait on the host.
    a_ptr = [t.data_ptr() for t in As_dev]
    b_ptr = [t.data_ptr() for t in Bs_dev]
    c_ptr, handle = C.data_ptr(), stream.cuda_stream

    bias = torch.linspace(-1.0, 1.0, w.N, device="cuda") if epilogue else None

    def run(i):
        if epilogue:
            mh.gemm_run_epilogue(plan, a_ptr[i % copies], b_ptr[i % copies], c_ptr, alpha=1.0, beta=1.0,
                                 bias=bias, activation=mh.GEMM_ACT_RELU, stream=handle)
        else:
            mh.gemm_run(plan, a_ptr[i % copies], b_ptr[i % copies], c_ptr, handle)

    settled = 0
    try:
        if settle_s > 0:
            t_end = time.perf_counter() + settle_s
            while time.perf_counter() < t_end:
                for i in range(50):
                    run(settled + i)
                settled += 50
                torch.cuda.synchronize()
        w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0.record(stream)
        for i in range(settle + warmup):
            run(i)
        w1.record(stream)
        torch.cuda.synchronize()
        if per_call and min_group_ms > 0 and settle + warmup > 0:
            steps = steps_for_groups(steps, w0.elapsed_time(w1) / (settle + warmup), min_group_ms)
        # The timed calls, with a HIP event at their start, after every group of calls
        # and at their end: the mean is the whole span over `steps`, and with per_call the
        # spread between calls is the groups' means (10 consecutive calls a group at the
        # default 300), taken from the same calls, so the mean is their average.  An event
        # pair around every single call would add its own gap to every call.
        groups = min(PER_CALL_GROUPS, steps) if per_call else 1
        bounds = group_bounds(steps, groups)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(groups + 1)]
        t0 = time.perf_counter()
        evs[0].record(stream)
        for g in range(groups):
            for i in range(bounds[g], bounds[g + 1]):
                run(i)
            evs[g + 1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        event_ms = evs[0].elapsed_time(evs[-1]) / steps
        calls = sorted(evs[g].elapsed_time(evs[g + 1]) / (bounds[g + 1] - bounds[g])
                       for g in range(groups)) if per_call else []
        clock_mhz = clock_during(run, steps) if clock else None
    finally:
        mh.gemm_destroy(plan)
    flops, nbytes = algorithmic(w)
    if epilogue:
        nbytes += w.M * w.N * synth.ELEM_BYTES[w.out] + 4 * w.N
    ai, roof, bound = roofline_of(w)
    ms_step = wall * 1000.0 / steps
    out = {
        "workload": name + ("+epilogue" if epilogue else "") + ("" if rotate else " (warm: one operand copy)"), "M": w.M, "N": w.N, "K": w.K, "in": w.dtype, "out": w.out,
        "layout": ("A col" if w.a_col else "A row") + (", B col" if w.b_col else ", B row"),
        "tile": f"{desc['bm']}x{desc['bn']}x{desc['bk']}", "kind": desc["kind"],
        "grid": desc["grid_x"] * desc["grid_y"] * desc["grid_z"], "rotated_copies": copies,
        "settle_calls": settle + settled, "warmup_calls": warmup, "timed_calls": steps,
        "ms_per_step": ms_step, "kernel_ms_event": event_ms,
        "tflops": flops / (ms_step / 1000.0) / 1e12,
        "kernel_tflops": flops / (event_ms / 1000.0) / 1e12,
        "kernel_gbps": nbytes / (event_ms / 1000.0) / 1e9,
        "intensity": ai, "bound": bound, "roofline_tflops": roof,
    }
    out["frac_of_roofline"] = out["kernel_tflops"] / roof
    if calls:
        k = len(calls)
        out["kernel_ms_p10_p50_p90"] = [calls[k // 10], calls[k // 2], calls[(9 * k) // 10]]
    if clock_mhz is not None:
        out["clock_mhz"] = clock_mhz
    return out


def autotune_report(names, reps=10):
    """For each workload: the planner's configuration, the fastest in an autotune sweep
    of every compiled variant that fits (gemm_autotune), and their times.  The sweep's
    table is cleared afterwards, so nothing timed elsewhere depends on it."""
    import torch

    import memory_hierarchy_optimisation_amd as mh
    import synth

    keys = ("kind", "bm", "bn", "bk", "waves_m", "waves_n", "stages", "split_k")
    cat = mh.gemm_catalogue()
    out = []
    for name in names:
        w = synth.WORKLOADS[name]
        As, lda, Bs, ldb, _, _ = synth.workload_operands(w)
        A, B = As.cuda(), Bs.cuda()
        C = torch.empty((w.M, w.N), dtype=synth.TORCH_DTYPES[w.out], device="cuda")
        code = mh.DTYPE_OF[(w.dtype, w.out)]
        layout = (mh.GEMM_A_COL if w.a_col else 0) | (mh.GEMM_B_COL if w.b_col else 0)
        plan = mh.gemm_plan(w.M, w.N, w.K, lda, ldb, w.N, code, layout)
        d = mh.gemm_plan_describe(plan)
        mh.gemm_destroy(plan)
        heuristic = tuple(d[k] for k in keys)
        try:
            best, best_us, times = mh.gemm_autotune(w.M, w.N, w.K, lda, ldb, w.N, code, layout, A, B, C,
                                                    reps=reps)
        finally:
            mh.gemm_tune_clear()
        h_us = times[cat.index(heuristic)] if heuristic in cat else -1.0
        out.append({"workload": name, "heuristic": list(heuristic), "heuristic_us": round(h_us, 3),
                    "tuned": list(best), "tuned_us": round(best_us, 3),
                    "candidates": sum(1 for t in times if t >= 0)})
        log(f"[bench] autotune {name}: heuristic {heuristic} {h_us:.2f} us, fastest {best} {best_us:.2f} us "
            f"of {out[-1]['candidates']} candidates")
    return out


def transpose_report(shapes=((8192, 8192, 4), (8192, 8192, 2)), steps=50, warmup=10):
    """The tiled transpose (gemm_transpose): GB/s counting each element read once and
    written once, against the 8 TB/s HBM roofline; inputs rotate past the 256 MB cache."""
    import torch

    import memory_hierarchy_optimisation_amd as mh

    out = []
    for rows, cols, E in shapes:
        dt = {2: torch.int16, 4: torch.int32}[E]
        nbytes = rows * cols * E
        # inputs and outputs both rotate: 2 x copies x nbytes > the 256 MB cache
        copies = max(2, math.ceil(ROTATE_BYTES / (2 * nbytes)))
        ins = [torch.zeros((rows, cols), dtype=dt, device="cuda") for _ in range(copies)]
        outs = [torch.empty((cols, rows), dtype=dt, device="cuda") for _ in range(copies)]
        ptrs = [t.data_ptr() for t in ins]
        optrs = [t.data_ptr() for t in outs]
        handle = torch.cuda.current_stream().cuda_stream
        for i in range(warmup):
            mh.gemm_transpose(ptrs[i % copies], optrs[(i + 1) % copies], rows, cols, cols, rows, E, stream=handle)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for i in range(steps):
            mh.gemm_transpose(ptrs[i % copies], optrs[(i + 1) % copies], rows, cols, cols, rows, E, stream=handle)
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / steps
        gbps = 2 * nbytes / (ms / 1000.0) / 1e9
        out.append({"rows": rows, "cols": cols, "elem_bytes": E, "kernel_ms_event": round(ms, 5),
                    "gbps": round(gbps, 1), "frac_of_hbm": round(gbps / HBM_GBPS, 4)})
        log(f"[bench] transpose {rows}x{cols} ({E}-byte elements): {ms * 1000:.1f} us, {gbps:.0f} GB/s, "
            f"{100 * gbps / HBM_GBPS:.1f}% of HBM")
        del ins, outs
    return out


def copy_reference(nbytes=512 << 20):
    """One elementwise device kernel of known traffic (reads and writes nbytes), run
    after the timed region so a counter run can scale FETCH_SIZE / WRITE_SIZE."""
    import torch

    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    log(f"copy reference: {nbytes} bytes read and written by one elementwise kernel")


def traffic_for(name):
    """HBM bytes per launch from the committed counter summary, if it was taken on the
    current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"counters_{name}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_digest") != kernel_source_digest():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def build_resources():
    """The compiler's per-kernel resource report of the in-tree build, keyed by the
    demangled kernel name: {vgpr, agpr, sgpr, scratch, occupancy, lds, vgpr_spill}."""
    import subprocess

    path = os.path.join(ROOT, "_build", "resource_usage.txt")
    if not os.path.exists(path):
        return {}
    rows = [line.split() for line in open(path) if line.strip()]
    names = subprocess.run(["c++filt"], input="\n".join(r[0] for r in rows), capture_output=True,
                           text=True).stdout.splitlines()
    return {n: dict(kv.split("=", 1) for kv in r[1:]) for n, r in zip(names, rows)}


PROFILE_CMD = ("python3 bench.py --workload {w} --no-cpu-baseline --no-per-shape --steps 20 --warmup 2 "
               "--settle 0 --no-clock --copy-reference")
COUNTER_PASSES = {
    "mfma": "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F16 SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES "
            "SQ_CYCLES GRBM_GUI_ACTIVE GRBM_COUNT",
    "lds": "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_LDS_ADDR_CONFLICT SQ_INSTS_LDS GRBM_GUI_ACTIVE",
    "fetch": "FETCH_SIZE",
    "write": "WRITE_SIZE",
}
XCDS, SES, SIMDS = 8, 32, 1024     # MI355X: 8 XCDs, 4 shader engines each, 256 CUs x 4 SIMDs


def summarize_counters(name, digest, csvs, out_path):
    """Write profiles/counters_<workload>.txt from the four rocprofv3 counter runs of one
    workload (COUNTER_PASSES, CSV output): per dispatch of its GEMM kernel, the matrix
    work done and the matrix pipes' busy cycles, the clock, LDS bank conflicts, HBM
    traffic (FETCH_SIZE / WRITE_SIZE scaled by what they read for the copy reference of
    known traffic) and the registers of the kernel as loaded."""
    import csv

    import synth

    per = {}        # pass -> kernel -> counter -> [values]
    dur = {}        # kernel -> [ns] (each pass's dispatches; the profiler serialises them)
    for tag, path in csvs.items():
        acc = per.setdefault(tag, {})
        with open(path) as fh:
            for r in csv.DictReader(fh):
                k = r["Kernel_Name"]
                acc.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                if tag == "mfma" and r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                    dur.setdefault(k, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    kernels = [k for k in per["mfma"] if "mhg::" in k and "gemm" in k and "reduce" not in k]
    if len(kernels) != 1:
        raise SystemExit(f"expected one GEMM kernel in the profiled run, got {kernels}")
    g = kernels[0]
    ref = [k for k in per["fetch"] if "elementwise" in k and "Unary" in k]
    if len(ref) != 1:
        raise SystemExit(f"expected one copy reference kernel, got {ref}")
    c = ref[0]

    def mean(tag, k, counter):
        v = per[tag][k][counter]
        return sum(v) / len(v), len(v)

    w = synth.WORKLOADS[name]
    flops, alg = algorithmic(w)
    ns = sum(dur[g]) / len(dur[g])
    mops = mean("mfma", g, "SQ_INSTS_VALU_MFMA_MOPS_BF16")[0] + mean("mfma", g, "SQ_INSTS_VALU_MFMA_MOPS_F16")[0]
    busy, n_disp = mean("mfma", g, "SQ_VALU_MFMA_BUSY_CYCLES")
    sq_busy = mean("mfma", g, "SQ_BUSY_CYCLES")[0]
    wave_cycles = sq_busy / SES
    conflict = mean("lds", g, "SQ_LDS_BANK_CONFLICT")[0]
    active = mean("lds", g, "SQ_LDS_IDX_ACTIVE")[0]
    addr_conflict = mean("lds", g, "SQ_LDS_ADDR_CONFLICT")[0]
    lds_insts = mean("lds", g, "SQ_INSTS_LDS")[0]
    ref_kib = (512 << 20) / 1024.0
    f_scale = ref_kib / mean("fetch", c, "FETCH_SIZE")[0]
    w_scale = ref_kib / mean("write", c, "WRITE_SIZE")[0]
    fetch_kib = mean("fetch", g, "FETCH_SIZE")[0]
    write_kib = mean("write", g, "WRITE_SIZE")[0]
    traffic = fetch_kib * f_scale * 1024 + write_kib * w_scale * 1024
    res = build_resources().get(g, {})
    lines = [
        f"# Counters of the {name} GEMM kernel ({w.note}), rocprofv3, per dispatch",
        f"kernel: {g}",
        f"kernel_source_digest: {digest}",
        f"dispatches: {n_disp}",
        f"duration_us_under_counters: {ns / 1000:.2f}  (dispatches serialised by the profiler)",
        f"mfma_flop_per_dispatch: {mops * 512:.6g}  (SQ_INSTS_VALU_MFMA_MOPS_* x 512; 2MNK = {flops:.6g})",
        f"achieved_tflops_under_counters: {mops * 512 / ns / 1e3:.1f}",
        f"mfma_busy_cycles_per_simd: {busy / SIMDS:.0f}  (SQ_VALU_MFMA_BUSY_CYCLES over {SIMDS} SIMDs)",
        f"wave_cycles_per_shader_engine: {wave_cycles:.0f}  (SQ_BUSY_CYCLES over {SES}: cycles with waves present)",
        f"mfma_busy_fraction: {busy / SIMDS / wave_cycles:.3f}  (matrix-pipe busy cycles per SIMD over the cycles "
        "with waves present)",
        f"clock_mhz_lower_bound: {wave_cycles / ns * 1e3:.0f}  (cycles with waves present over the dispatch "
        "duration; GRBM_GUI_ACTIVE equals GRBM_COUNT here, i.e. it spans the whole counter window, and gives "
        "no clock)",
        f"lds_bank_conflict_cycles: {conflict:.0f}",
        f"lds_active_cycles: {active:.0f}",
        f"lds_bank_conflicts_per_access: {conflict / max(active - conflict, 1.0):.4f}  (conflict cycles over "
        "conflict-free LDS cycles)",
        f"lds_address_conflict_cycles: {addr_conflict:.0f}",
        f"lds_instructions: {lds_insts:.0f}",
        f"fetch_size_kib: {fetch_kib:.1f}",
        f"write_size_kib: {write_kib:.1f}",
        f"fetch_scale: {f_scale:.4f}  (copy reference: {mean('fetch', c, 'FETCH_SIZE')[0]:.1f} KiB counted for "
        "524288 KiB read)",
        f"write_scale: {w_scale:.4f}  (copy reference: {mean('write', c, 'WRITE_SIZE')[0]:.1f} KiB counted for "
        "524288 KiB written)",
        f"traffic_bytes_per_launch: {traffic:.0f}",
        f"algorithmic_bytes_per_launch: {alg:.0f}",
        f"traffic_over_algorithmic: {traffic / alg:.3f}",
        "registers (compiler report of this build): " + " ".join(f"{k}={v}" for k, v in res.items()),
        "# commands, each a run of its own, from /tmp with TMPDIR=/tmp (R = the repository root, OUT = an output folder):",
    ]
    for tag, counters in COUNTER_PASSES.items():
        lines.append(f"#   timeout -s KILL 300 rocprofv3 --pmc {counters} --output-format csv -d OUT/pmc_{name}_{tag} "
                     f"-o p -- {PROFILE_CMD.format(w=name).replace('bench.py', 'R/bench.py')}")
    lines.append(f"#   python3 bench.py --workload {name} --summarize-counters <digest> "
                 + " ".join(f"OUT/pmc_{name}_{t}/p_counter_collection.csv" for t in COUNTER_PASSES))
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    log("\n".join(lines))


def summarize_trace(trace_csv, digest, out_path, settle, warmup, steps, workload):
    """Write profiles/kernel_trace_bench_default.txt from the kernel trace of a default
    bench run: per kernel, dispatches and mean / min / max duration, and for the
    headline kernel the mean over the timed calls (the first `settle` + `warmup`
    dispatches of it are untimed; the next `steps` are the timed batch)."""
    import csv

    durs, order = {}, []
    with open(trace_csv) as fh:
        for r in csv.DictReader(fh):
            k = r["Kernel_Name"]
            if k not in durs:
                durs[k] = []
                order.append(k)
            durs[k].append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    for k in durs:
        durs[k].sort()
    rows = sorted(durs, key=lambda k: -sum(d for _, d in durs[k]))
    # The headline line runs first: its kernel is the first GEMM kernel dispatched (the
    # other lines settle for a fixed time, so a short kernel has more dispatches).
    head = [k for k in rows if "mhg::" in k and "gemm" in k]
    hk = min(head, key=lambda k: durs[k][0][0])
    timed = [d for _, d in durs[hk][settle + warmup:settle + warmup + steps]]
    lines = [
        "# Kernel durations of a default bench.py run (rocprofv3 kernel trace)",
        f"# kernel_source_digest: {digest}",
        "# command (from /tmp with TMPDIR=/tmp; R = the repository root, OUT = an output folder):",
        "#   timeout -s KILL 900 rocprofv3 --kernel-trace --stats --output-format csv -d OUT/prof_kt -o kt "
        "-- python3 R/bench.py",
        f"#   python3 bench.py --summarize-trace OUT/prof_kt/kt_kernel_trace.csv {digest}",
        f"# Headline kernel ({workload}): {hk}",
        f"# Its dispatches in the order made: {settle} settling calls, {warmup} warm-up calls, {steps} timed calls "
        "(HIP events at their start, after every tenth and at their end), then 600 beside the clock probe; later "
        "dispatches of it belong to the fused-epilogue line (other flags) or the autotune sweep.",
        f"headline_timed_mean_ns: {sum(timed) / max(len(timed), 1):.0f}  (dispatches {settle + warmup + 1} .. "
        f"{settle + warmup + steps} of it)",
        "KERNELS (name | dispatches | mean ns | min ns | max ns):",
    ]
    for k in rows:
        d = [x for _, x in durs[k]]
        lines.append(f"{k} | {len(d)} | {sum(d) / len(d):.0f} | {min(d)} | {max(d)}")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    log("\n".join(lines[:12]))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads():
    """Cores the oracle may use: the CPUs this process is allowed to run on, capped by
    OMP_NUM_THREADS when the environment sets it (the host's share for one GPU)."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return n


def oracle_timings(names, threads):
    """Whole products of the small workloads through the oracle, compute loop only."""
    import oracle
    import synth

    out = []
    for name in names:
        w = synth.WORKLOADS[name]
        As, lda, Bs, ldb, _, _ = synth.workload_operands(w)
        a = synth.to_storage_numpy(As)
        b = synth.to_storage_numpy(Bs)
        for n in threads:
            oracle.set_threads(n)
            t0 = time.perf_counter()
            oracle.gemm(w.M, w.N, w.K, a, lda, b, ldb, w.dtype, a_col=w.a_col, b_col=w.b_col)
            t = time.perf_counter() - t0
            out.append({"workload": name, "threads": n, "seconds": round(t, 4),
                        "gflops": round(2.0 * w.M * w.N * w.K / t / 1e9, 3)})
            log(f"[bench] oracle {name} on {n} thread(s): {t:.3f} s")
    return out


def cpu_baseline(name, seconds):
    """The oracle as it stands, on the host cores, over the first rows of the product."""
    import oracle
    import synth

    threads = host_threads()
    oracle.set_threads(threads)
    w = synth.WORKLOADS[name]
    As, lda, Bs, ldb, _, _ = synth.workload_operands(w)
    a = synth.to_storage_numpy(As)
    b = synth.to_storage_numpy(Bs)
    probe = min(w.M, 16)
    t0 = time.perf_counter()
    oracle.gemm(w.M, w.N, w.K, a, lda, b, ldb, w.dtype, a_col=w.a_col, b_col=w.b_col, rows=(0, probe))
    t_probe = time.perf_counter() - t0
    rows = int(max(probe, min(w.M, probe * seconds / max(t_probe, 1e-6))))
    t0 = time.perf_counter()
    oracle.gemm(w.M, w.N, w.K, a, lda, b, ldb, w.dtype, a_col=w.a_col, b_col=w.b_col, rows=(0, rows))
    t = time.perf_counter() - t0
    flops = 2.0 * rows * w.N * w.K
    res = {
        "value": flops / t / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(), "kind": "oracle",
        "sample": f"rows 0..{rows - 1} of the {w.M}x{w.N}x{w.K} {w.dtype} product "
                  f"({rows * w.N} of {w.M * w.N} outputs, {t:.1f} s, binary64 triple loop)",
        "cpu_model": cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0)),
    }
    # The three small workloads in full, on all the cores and on one.
    res["small_workloads"] = oracle_timings(["f32_64", "f16_1024", "f16_1000", "f16_2048_nt"],
                                            sorted({threads, 1}, reverse=True))
    oracle.set_threads(threads)
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # The first ~150 calls of a run are slower while the clock settles under the
    # sustained matrix load; the default warm-up covers that (about 35 ms at 4096^3).
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default=HEADLINE, help="workload timed as the headline")
    ap.add_argument("--no-per-shape", action="store_true", help="time only the headline workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the fused-epilogue line and the autotune sweep report")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--settle", type=int, default=SETTLE_CALLS,
                    help="untimed calls of the headline plan before its warm-up (profiled runs: 0)")
    ap.add_argument("--no-clock", action="store_true", help="skip the clock probe (profiled runs)")
    ap.add_argument("--copy-reference", action="store_true",
                    help="after timing, run one elementwise kernel of known traffic (counter scale)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_CSV", "DIGEST"),
                    help="write profiles/kernel_trace_bench_default.txt from the kernel trace of a default run")
    ap.add_argument("--summarize-counters", nargs=5, metavar=("DIGEST", "MFMA_CSV", "LDS_CSV", "FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/counters_<workload>.txt from the four counter runs and exit")
    args = ap.parse_args()
    if args.summarize_trace:
        tcsv, digest = args.summarize_trace
        summarize_trace(tcsv, digest, os.path.join(ROOT, "profiles", "kernel_trace_bench_default.txt"),
                        args.settle, args.warmup, args.steps, args.workload)
        return
    if args.summarize_counters:
        digest, *paths = args.summarize_counters
        summarize_counters(args.workload, digest, dict(zip(COUNTER_PASSES, paths)),
                           os.path.join(ROOT, "profiles", f"counters_{args.workload}.txt"))
        return
    if args.gpus != 1:
        log(f"bench.py measures one GPU: the product runs on a single MI355X, and sharding it over "
            f"several GPUs is a design note, not code (--gpus {args.gpus} is not supported)")
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    log(f"[bench] device {torch.cuda.get_device_name(0)}; headline {args.workload}")

    head = measure(args.workload, args.steps, args.warmup, settle=args.settle, per_call=True,
                   clock=not args.no_clock)
    log(f"[bench] headline {head['workload']}: {head['tflops']:.1f} TFLOP/s "
        f"({head['ms_per_step'] * 1000:.1f} us/step, kernel {head['kernel_ms_event'] * 1000:.1f} us, "
        f"per call p10/p50/p90 {[round(1000 * v, 1) for v in head.get('kernel_ms_p10_p50_p90', [])]} us, "
        f"clock {head.get('clock_mhz', float('nan')):.0f} MHz)")
    shapes = []
    if not args.no_per_shape:
        for name in PER_SHAPE:
            # Every line settles first, for as long as the headline's settling calls take:
            # the clock that the previous line left is not the one a steady stream of
            # these calls settles to (with 300 untimed calls alone, ~7 ms at 2048^3, the
            # timed calls still ran slower than the same calls a moment later).  Short
            # calls are timed in more calls, so that each group spans 1 ms.
            r = head if name == args.workload else measure(name, 300, 300, per_call=True, settle_s=0.2, min_group_ms=1.0)
            shapes.append(r)
            log(f"[bench] {name}: {r['kernel_tflops']:.1f} TFLOP/s, {r['kernel_gbps']:.0f} GB/s, "
                f"{100 * r['frac_of_roofline']:.1f}% of the {r['bound']} roofline, tile {r['tile']}")
    extras = {}
    if not args.no_per_shape and not args.no_extras:
        # The same settling as the headline and the per-shape lines' fixed warm-up: the
        # clock settles again after the smaller per-shape lines.
        r = measure(args.workload, 300, 300, settle=SETTLE_CALLS, per_call=True, epilogue=True, clock=True)
        extras["epilogue"] = tidy(r)
        log(f"[bench] {r['workload']} (alpha, beta = 1, bias, ReLU): {r['kernel_tflops']:.1f} TFLOP/s, "
            f"kernel {r['kernel_ms_event'] * 1000:.1f} us against {head['kernel_ms_event'] * 1000:.1f} us plain")
        # Context only: the same calls on one operand copy, which stays in the Infinity
        # Cache (the graded figure above streams its operands from HBM).
        r = measure(args.workload, 300, 300, settle=SETTLE_CALLS, per_call=True, rotate=False)
        extras["warm"] = tidy(r)
        log(f"[bench] {r['workload']}: {r['kernel_tflops']:.1f} TFLOP/s, kernel {r['kernel_ms_event'] * 1000:.1f} us")
        extras["autotune"] = autotune_report([n for n in PER_SHAPE if n != "f32_64"])
        extras["transpose"] = transpose_report()
    if args.copy_reference:
        copy_reference()

    import synth
    w = synth.WORKLOADS[args.workload]
    flops, _ = algorithmic(w)
    achieved = head["kernel_tflops"]
    peak = PEAK_TFLOPS[w.dtype]
    traffic = traffic_for(args.workload)
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host cores ...")
        cpu = cpu_baseline(args.workload, args.cpu_seconds)
        log(f"[bench] oracle: {cpu['value'] * 1000:.2f} GFLOP/s on {cpu['cores']} threads")
    line = {
        "metric": f"GEMM TFLOP/s, {w.M}x{w.N}x{w.K} {w.dtype} in, fp32 accumulate, {w.out} out",
        "value": head["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.note, "M": w.M, "N": w.N, "K": w.K, "in": w.dtype, "out": w.out,
                   "layout": head["layout"], "tile": head["tile"], "grid": head["grid"],
                   "rotated_copies": head["rotated_copies"]},
        "roofline": {"bound": "mfma" if w.dtype != "f32" else "alu", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak, "traffic": traffic},
        "cpu_baseline": cpu,
        "clock_mhz": round(head["clock_mhz"], 1) if "clock_mhz" in head else None,
        "clock_note": "average shader clock over 20 ms of further headline calls (s_memtime over "
                      "s_memrealtime on a one-wave probe on a second stream)",
        "kernel_ms_event": head["kernel_ms_event"],
        "kernel_ms_p10_p50_p90": head.get("kernel_ms_p10_p50_p90"),
        "settle_calls": args.settle,
        "kernel_source_digest": kernel_source_digest(),
        "per_shape": [tidy(r) for r in shapes],
    }
    line.update(extras)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
