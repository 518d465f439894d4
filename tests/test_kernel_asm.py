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
