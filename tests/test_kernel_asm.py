"""The hot loops as the compiler emits them (device assembly of this repository's own
sources, built here for gfx950).  A buffer resource the compiler cannot prove
uniform makes it wrap every load in a loop over the lanes (readfirstlane, then
exec-mask steps); in the 256 x 256 kernel that once cost 15% of the whole call
without changing any result, so it is checked here, on the CPU, with the other
properties the kernels' speed depends on: no scratch and no spills."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "memory_hierarchy_optimisation_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")


SOURCES = ("kernels_w8.hip", "kernels_skinny.hip")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    """Device assembly of each source, compiled in parallel."""
    d = tmp_path_factory.mktemp("asm")
    procs = {}
    for src in SOURCES:
        cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", "-I" + os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
               os.path.join(CSRC, src), "-o", str(d / (src + ".s"))]
        procs[src] = subprocess.Popen(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.PIPE)
    for src, pr in procs.items():
        _, err = pr.communicate()
        assert pr.returncode == 0, err.decode()[-2000:]
    return {src: (d / (src + ".s")).read_text() for src in SOURCES}


def _functions(text, prefix):
    """name -> list of instruction lines, for the kernels whose symbol starts with prefix."""
    out = {}
    for m in re.finditer(r"^(" + re.escape(prefix) + r"[^\s:]*):", text, flags=re.M):
        body = text[m.end():]
        body = body[:body.index("s_endpgm")]
        out[m.group(1)] = [l.strip() for l in body.split("\n") if l.strip() and not l.strip().startswith(";")]
    return out


def _mfma_loops(lines):
    """Loops (a backward branch to a label) that contain matrix instructions and no
    other such loop: the kernels' main K loops, with any loop nested in them."""
    labels = {}
    for i, l in enumerate(lines):
        m = re.match(r"(\.LBB\S+):", l)
        if m:
            labels[m.group(1)] = i
    spans = []
    for i, l in enumerate(lines):
        m = re.search(r"s_cbranch_\w+ (\.LBB\S+)|s_branch (\.LBB\S+)", l)
        target = m and (m.group(1) or m.group(2))
        if target in labels and labels[target] < i:
            spans.append((labels[target], i))
    mfma = [a for a in spans if any(x.startswith("v_mfma") for x in lines[a[0]:a[1] + 1])]
    inner = [a for a in mfma if not any(b != a and a[0] <= b[0] and b[1] <= a[1] for b in mfma)]
    return [lines[a:b + 1] for a, b in inner]


@pytest.mark.parametrize("src,prefix,n_kernels", [
    ("kernels_w8.hip", "_ZN3mhg2w87w8_gemm", 48),
    ("kernels_skinny.hip", "_ZN3mhg6skinny11skinny_gemm", 2),
])
def test_hot_loops_have_no_lane_loops_and_no_scratch(src, prefix, n_kernels, asm):
    text = asm[src]
    funcs = _functions(text, prefix)
    assert len(funcs) == n_kernels
    for name, lines in funcs.items():
        loops = _mfma_loops(lines)
        assert loops, f"{name}: no MFMA loop found"
        for body in loops:
            waterfall = [b for b in body if "readfirstlane" in b or "saveexec" in b]
            assert not waterfall, f"{name}: loop over lanes inside the MFMA loop: {waterfall[:4]}"
        assert not any(l.startswith("scratch_") for l in lines), f"{name} touches scratch"
    # The kernel descriptors: no private segment (scratch) and no spills.
    for m in re.finditer(r"\.amdhsa_kernel (" + re.escape(prefix) + r"\S*)(.*?)\.end_amdhsa_kernel", text, flags=re.S):
        body = m.group(2)
        seg = re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", body)
        assert seg and int(seg.group(1)) == 0, f"{m.group(1)} uses scratch"


# Agent-scope atomics and fences as the compiler encodes them for gfx950.  The skinny
# kernel's split-K partials are published to other XCDs with hand-set cache-policy
# bits rather than a release fence; these two tests tie those bits to the compiler's
# own encoding of agent-scope relaxed atomic stores and loads, and check the ordering
# the kernel relies on in place of the fence's L2 write-back.
_MM_PROBE = r"""
#include <hip/hip_runtime.h>
extern "C" __global__ void st(float *p, float v) {
  __hip_atomic_store(p + threadIdx.x, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
extern "C" __global__ void ld(const float *p, float *o) {
  o[threadIdx.x] = __hip_atomic_load(p + threadIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
extern "C" __global__ void rel(float *p, unsigned *c) {
  p[threadIdx.x] = 1.0f;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  if (threadIdx.x == 0) __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
extern "C" __global__ void acq(unsigned *c, const float *p, float *o) {
  unsigned x = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  o[threadIdx.x] = p[threadIdx.x] + x;
}
"""


@pytest.fixture(scope="module")
def mm_probe(tmp_path_factory):
    d = tmp_path_factory.mktemp("mm")
    (d / "mm.hip").write_text(_MM_PROBE)
    r = subprocess.run([HIPCC, "-O3", "--offload-arch=gfx950", "--cuda-device-only", "-S", str(d / "mm.hip"),
                        "-o", str(d / "mm.s")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    text = (d / "mm.s").read_text()
    return {name: _functions(text, name)[name] for name in ("st", "ld", "rel", "acq")}


def _vm_ops(lines):
    return [l for l in lines if re.match(r"(global|buffer|flat)_|s_waitcnt", l)]


def test_compiler_encoding_of_agent_scope_atomics_and_fences(mm_probe):
    f = mm_probe
    # Relaxed agent-scope atomic store and load: plain accesses with the sc1 bit.
    assert any(re.match(r"global_store_dword .*\bsc1\b", l) for l in f["st"])
    assert any(re.match(r"global_load_dword .*\bsc1\b", l) for l in f["ld"])
    # Agent-scope release: write back L2 (what ordinary stores left dirty there), then
    # wait for every outstanding memory access, then the RMW.
    ops = _vm_ops(f["rel"])
    i = next(k for k, l in enumerate(ops) if l.startswith("buffer_wbl2"))
    assert re.search(r"\bsc1\b", ops[i])
    assert ops[i + 1].startswith("s_waitcnt vmcnt(0)") and ops[i + 2].startswith("global_atomic_add")
    # Agent-scope acquire: wait, then invalidate what ordinary loads may find stale.
    ops = _vm_ops(f["acq"])
    i = next(k for k, l in enumerate(ops) if l.startswith("buffer_inv"))
    assert re.search(r"\bsc1\b", ops[i]) and ops[i - 1].startswith("s_waitcnt vmcnt(0)")


def test_skinny_split_k_publishes_partials_as_agent_scope_atomics(asm):
    """Every partial store and load of the skinny kernel carries sc1 (the encoding of
    an agent-scope atomic store / load above), every lane's stores are complete
    (vmcnt 0) before the barrier that precedes the arrival RMW, the partial loads come
    after the RMW and the barrier that shares its result, and the kernel has no L2
    write-back or invalidate: the release fence's write-back and the acquire fence's
    invalidate serve ordinary accesses, and there are none to the workspace."""
    funcs = _functions(asm["kernels_skinny.hip"], "_ZN3mhg6skinny11skinny_gemm")
    assert len(funcs) == 2
    for name, lines in funcs.items():
        assert not any(l.startswith(("buffer_wbl2", "buffer_inv")) for l in lines), name
        rmw = [k for k, l in enumerate(lines) if l.startswith("global_atomic_add")]
        assert len(rmw) == 1, name
        r = rmw[0]
        before, after = lines[:r], lines[r:]
        stores = [k for k, l in enumerate(before) if l.startswith("buffer_store_dwordx4")]
        assert len(stores) == 2 and all(re.search(r"\bsc1\b", before[k]) for k in stores), name
        tail = before[stores[-1]:]
        # (The barrier alone does not wait for them: without the kernel's own wait the
        # compiler puts the barrier straight after the stores.)
        w = next((k for k, l in enumerate(tail) if l.startswith("s_waitcnt") and "vmcnt(0)" in l), None)
        b = next(k for k, l in enumerate(tail) if l.startswith("s_barrier"))
        assert w is not None and w < b, f"{name}: barrier before the partial stores are complete"
        loads = [l for l in after if l.startswith("buffer_load_dwordx4")]
        assert loads and all(re.search(r"\bsc1\b", l) for l in loads), name
        first_load = next(k for k, l in enumerate(after) if l.startswith("buffer_load_dwordx4"))
        assert any(l.startswith("s_barrier") for l in after[:first_load]), name
        assert any(l.startswith("s_waitcnt") and "vmcnt(0)" in l for l in after[:first_load]), name
