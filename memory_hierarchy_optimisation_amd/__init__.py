"""Python binding of libmhgemm (include/mhgemm.h): argument marshalling only.

Every step of the product runs in the HIP kernels of ``libmhgemm.so``; this module
loads that library (raising ImportError when it has not been built: there is no
fallback path), converts tensors to device pointers and streams to ``hipStream_t``
handles, and turns error codes into exceptions.  PyTorch is used only for device
memory and streams.
"""
import ctypes
import os

# torch is imported before the library is loaded: torch carries its own HIP and HSA
# runtimes, and the library's dependency on libamdhip64 then binds to the copy torch
# already mapped.  Loading the library first would bring a second HIP runtime into
# the process, whose streams, allocations and synchronisation the other cannot see.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmhgemm.so")

GEMM_F32_F32, GEMM_F16_F16, GEMM_F16_F32, GEMM_BF16_BF16, GEMM_BF16_F32 = range(5)
GEMM_A_ROW, GEMM_A_COL, GEMM_B_ROW, GEMM_B_COL = 0, 1, 0, 2
GEMM_OK, GEMM_ERR_INVALID_ARG, GEMM_ERR_UNSUPPORTED, GEMM_ERR_HIP, GEMM_ERR_ALLOC = 0, -1, -2, -3, -4
GEMM_KIND_NONE, GEMM_KIND_FMA, GEMM_KIND_MFMA, GEMM_KIND_SKINNY = range(4)
GEMM_ACT_NONE, GEMM_ACT_RELU = 0, 1

# (input element, output element) of each gemm_dtype, and back.
DTYPES = {
    GEMM_F32_F32: ("f32", "f32"),
    GEMM_F16_F16: ("f16", "f16"),
    GEMM_F16_F32: ("f16", "f32"),
    GEMM_BF16_BF16: ("bf16", "bf16"),
    GEMM_BF16_F32: ("bf16", "f32"),
}
DTYPE_OF = {v: k for k, v in DTYPES.items()}

DESCRIBE_FIELDS = ("kind", "bm", "bn", "bk", "waves_m", "waves_n", "stages", "split_k",
                   "grid_x", "grid_y", "grid_z", "threads", "lds_bytes", "cus", "variant",
                   "workspace_bytes")

EXPORTS = ("gemm_plan", "gemm_plan_config", "gemm_run", "gemm_run_epilogue", "gemm_destroy",
           "gemm_last_error", "gemm_plan_describe", "gemm_catalogue", "gemm_autotune", "gemm_tune_save",
           "gemm_tune_load", "gemm_tune_clear", "gemm_transpose", "gemm_clock_probe",
           "gemm_run_noalloc", "gemm_catalogue_registers")


class Epilogue(ctypes.Structure):
    """gemm_epilogue_t: C = act(alpha * product + beta * prior C + bias[column])."""
    _fields_ = [("alpha", ctypes.c_float), ("beta", ctypes.c_float), ("bias", ctypes.c_void_p),
                ("activation", ctypes.c_int32)]


class GemmError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"{message} (status {code})")
        self.code = code


def hip_runtimes_mapped():
    """Paths of the HIP runtime libraries mapped into this process."""
    paths = set()
    try:
        with open("/proc/self/maps") as fh:
            for line in fh:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return sorted(paths)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.gemm_plan.argtypes = [i64, i64, i64, i64, i64, i64, i32, i32]
    lib.gemm_plan.restype = vp
    lib.gemm_plan_config.argtypes = [i64, i64, i64, i64, i64, i64, i32, i32,
                                     ctypes.POINTER(ctypes.c_int32)]
    lib.gemm_plan_config.restype = vp
    lib.gemm_run.argtypes = [vp, vp, vp, vp, vp]
    lib.gemm_run.restype = i32
    lib.gemm_run_epilogue.argtypes = [vp, vp, vp, vp, ctypes.POINTER(Epilogue), vp]
    lib.gemm_run_epilogue.restype = i32
    lib.gemm_destroy.argtypes = [vp]
    lib.gemm_destroy.restype = None
    lib.gemm_last_error.argtypes = []
    lib.gemm_last_error.restype = ctypes.c_char_p
    lib.gemm_plan_describe.argtypes = [vp, ctypes.POINTER(ctypes.c_int32)]
    lib.gemm_plan_describe.restype = i32
    f32p, i32p = ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int32)
    lib.gemm_catalogue.argtypes = [i32p, i32]
    lib.gemm_catalogue.restype = i32
    lib.gemm_catalogue_registers.argtypes = [i32p, i32]
    lib.gemm_catalogue_registers.restype = i32
    lib.gemm_autotune.argtypes = [i64, i64, i64, i64, i64, i64, i32, i32, vp, vp, vp, vp, i32,
                                  i32p, f32p, f32p, i32]
    lib.gemm_autotune.restype = i32
    lib.gemm_tune_save.argtypes = [ctypes.c_char_p]
    lib.gemm_tune_save.restype = i32
    lib.gemm_tune_load.argtypes = [ctypes.c_char_p]
    lib.gemm_tune_load.restype = i32
    lib.gemm_tune_clear.argtypes = []
    lib.gemm_tune_clear.restype = None
    lib.gemm_transpose.argtypes = [vp, vp, i64, i64, i64, i64, i32, vp]
    lib.gemm_transpose.restype = i32
    lib.gemm_run_noalloc.argtypes = [i64, i64, i64, i64, i64, i64, i32, i32, vp, vp, vp,
                                     ctypes.POINTER(Epilogue), vp]
    lib.gemm_run_noalloc.restype = i32
    lib.gemm_clock_probe.argtypes = [vp, i64, vp]
    lib.gemm_clock_probe.restype = i32
    runtimes = hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError("more than one HIP runtime is mapped into this process "
                          f"({runtimes}); import torch before loading libmhgemm")
    return lib


_lib = _load()


def gemm_last_error():
    return _lib.gemm_last_error().decode()


def gemm_plan(M, N, K, lda, ldb, ldc, dtype, layout):
    """Plan handle (an int) for C[M,N] = A[M,K] x B[K,N]; raises GemmError on bad input."""
    h = _lib.gemm_plan(M, N, K, lda, ldb, ldc, dtype, layout)
    if not h:
        raise GemmError(GEMM_ERR_INVALID_ARG, gemm_last_error())
    return h


def gemm_plan_config(M, N, K, lda, ldb, ldc, dtype, layout, cfg):
    """Plan with a forced configuration cfg = (kind, BM, BN, BK, waves_m, waves_n, stages, split_k)."""
    arr = (ctypes.c_int32 * 8)(*[int(x) for x in cfg])
    h = _lib.gemm_plan_config(M, N, K, lda, ldb, ldc, dtype, layout, arr)
    if not h:
        raise GemmError(GEMM_ERR_INVALID_ARG, gemm_last_error())
    return h


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        if x.device.type != "cuda":
            raise ValueError("operands must be device tensors")
        return x.data_ptr()
    raise TypeError(f"cannot take a device pointer from {type(x).__name__}")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def gemm_run(plan, A, B, C, stream=None):
    """Enqueue the planned product on ``stream`` (default: torch's current stream)."""
    rc = _lib.gemm_run(plan, _ptr(A), _ptr(B), _ptr(C), _stream(stream))
    if rc != GEMM_OK:
        raise GemmError(rc, gemm_last_error())


def gemm_run_epilogue(plan, A, B, C, alpha=1.0, beta=0.0, bias=None, activation=GEMM_ACT_NONE,
                      stream=None):
    """Enqueue C = act(alpha * A x B + beta * C + bias[column]) (bias: N fp32 values on
    the device, or None) on ``stream``."""
    epi = Epilogue(float(alpha), float(beta), _ptr(bias), int(activation))
    rc = _lib.gemm_run_epilogue(plan, _ptr(A), _ptr(B), _ptr(C), ctypes.byref(epi), _stream(stream))
    if rc != GEMM_OK:
        raise GemmError(rc, gemm_last_error())


def gemm_destroy(plan):
    _lib.gemm_destroy(plan)


def gemm_plan_describe(plan):
    out = (ctypes.c_int32 * 16)()
    rc = _lib.gemm_plan_describe(plan, out)
    if rc != GEMM_OK:
        raise GemmError(rc, gemm_last_error())
    return dict(zip(DESCRIBE_FIELDS, list(out)))


def gemm_catalogue():
    """Compiled variants as (kind, BM, BN, BK, waves_m, waves_n, stages, split_k) tuples."""
    n = _lib.gemm_catalogue(None, 0)
    arr = (ctypes.c_int32 * (8 * n))()
    _lib.gemm_catalogue(arr, n)
    return [tuple(arr[8 * i:8 * i + 8]) for i in range(n)]


def gemm_catalogue_registers():
    """Registers per lane the planner's occupancy filter assumes, per catalogue entry."""
    n = _lib.gemm_catalogue_registers(None, 0)
    arr = (ctypes.c_int32 * n)()
    _lib.gemm_catalogue_registers(arr, n)
    return list(arr)


def gemm_autotune(M, N, K, lda, ldb, ldc, dtype, layout, A, B, C, stream=None, reps=20):
    """Time every variant that fits on these operands and record the fastest for gemm_plan.
    Returns (best configuration tuple, its microseconds per call, per-catalogue-entry
    times with -1 for variants that do not fit).  Synchronises the stream."""
    n = _lib.gemm_catalogue(None, 0)
    best = (ctypes.c_int32 * 8)()
    best_us = ctypes.c_float()
    times = (ctypes.c_float * n)()
    rc = _lib.gemm_autotune(M, N, K, lda, ldb, ldc, dtype, layout, _ptr(A), _ptr(B), _ptr(C),
                            _stream(stream), int(reps), best, ctypes.byref(best_us), times, n)
    if rc != GEMM_OK:
        raise GemmError(rc, gemm_last_error())
    return tuple(best), best_us.value, list(times)


def gemm_tune_save(path):
    """Write the table of tuned configurations; returns the number of entries."""
    rc = _lib.gemm_tune_save(os.fsencode(path))
    if rc < 0:
        raise GemmError(rc, gemm_last_error())
    return rc


def gemm_tune_load(path):
    """Merge a saved table of tuned configurations; returns the number of entries."""
    rc = _lib.gemm_tune_load(os.fsencode(path))
    if rc < 0:
        raise GemmError(rc, gemm_last_error())
    return rc


def gemm_tune_clear():
    _lib.gemm_tune_clear()


def gemm_transpose(inp, out, rows, cols, ld_in, ld_out, elem_bytes, stream=None):
    """out[c * ld_out + r] = inp[r * ld_in + c] for elem_bytes-byte elements (2 or 4)."""
    rc = _lib.gemm_transpose(_ptr(inp), _ptr(out), rows, cols, ld_in, ld_out, elem_bytes, _stream(stream))
    if rc != GEMM_OK:
        raise GemmError(rc, gemm_last_error())


def gemm_clock_probe(out, ticks, stream=None):
    """Enqueue the one-wave clock probe: out (device, two uint64) receives the shader
    cycles and the 100 MHz real-time ticks of a window of `ticks` ticks."""
    rc = _lib.gemm_clock_probe(_ptr(out), int(ticks), _stream(stream))
    if rc != GEMM_OK:
        raise GemmError(rc, gemm_last_error())


def gemm_run_noalloc(M, N, K, lda, ldb, ldc, dtype, layout, A, B, C, alpha=1.0, beta=0.0, bias=None,
                     activation=GEMM_ACT_NONE, stream=None, epilogue=False):
    """Plan and run in one call with no device allocation (split-K workspaces in the
    library's per-GPU scratch array).  epilogue=False passes no epilogue (gemm_run)."""
    epi = ctypes.byref(Epilogue(float(alpha), float(beta), _ptr(bias), int(activation))) if epilogue else None
    rc = _lib.gemm_run_noalloc(M, N, K, lda, ldb, ldc, dtype, layout, _ptr(A), _ptr(B), _ptr(C), epi,
                               _stream(stream))
    if rc != GEMM_OK:
        raise GemmError(rc, gemm_last_error())
