"""Pins of the oracle to things other than itself.

Each check is chosen so that a plausible mistake in the oracle fails it:
  * codecs: every fp16 / bf16 bit pattern against numpy / torch conversions, and the
    round-to-nearest-even encoders against numpy, torch and hand-made tie cases;
  * tiny shapes: brute force in exact rational arithmetic (fractions.Fraction),
    within Higham's bound for a recursively summed dot product;
  * closed forms: identity on either side gives the other operand exactly, a
    permutation matrix permutes rows exactly, all-ones gives C_ij = K;
  * integer inputs: exact int64 products from numpy;
  * a library routine: numpy's binary64 matmul within the same summation bound;
  * storage: every layout / leading-dimension combination of the same logical
    operands gives bit-identical results, and sampled elements equal whole rows.
The last tests plant mistakes in a copy of the oracle's call (on the CPU) and show
that the pins above catch them.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

U53 = 2.0 ** -53


def gamma(k):
    return k * U53 / (1 - k * U53)


def _store(X, col, ld=None):
    S, ld = synth.lay_out(X, col, ld)
    return synth.to_storage_numpy(S), ld


def _exact(A, B):
    """Exact rational product of two small logical tensors."""
    Af = [[Fraction(float(v)) for v in row] for row in A.to(torch.float64).tolist()]
    Bf = [[Fraction(float(v)) for v in row] for row in B.to(torch.float64).tolist()]
    M, K = len(Af), len(Af[0]) if Af else 0
    N = len(Bf[0]) if Bf else 0
    return [[sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0)) for j in range(N)] for i in range(M)]


def _ref(A, B, dtype, a_col=False, b_col=False, lda=None, ldb=None):
    M, K = A.shape
    N = B.shape[1]
    As, lda = _store(A, a_col, lda)
    Bs, ldb = _store(B, b_col, ldb)
    return oracle.gemm(M, N, K, As, lda, Bs, ldb, dtype, a_col=a_col, b_col=b_col)


# ---- codecs ----------------------------------------------------------------------------

def test_decode_f16_every_pattern_matches_numpy():
    bits = np.arange(1 << 16, dtype=np.uint16)
    got = oracle.decode(bits, "f16")
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # sign of zero survives
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_decode_bf16_every_pattern_matches_torch():
    bits = np.arange(1 << 16, dtype=np.uint16)
    got = oracle.decode(bits, "bf16")
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_decode_f32_is_identity():
    x = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    assert np.array_equal(oracle.decode(x, "f32"), x.astype(np.float64))


def test_encode_f16_matches_numpy_on_random_doubles():
    rng = np.random.default_rng(1)
    mag = np.exp2(rng.uniform(-30, 17, 200000))  # subnormals through overflow
    x = mag * rng.choice([-1.0, 1.0], mag.size)
    got = oracle.encode(x, "f16")
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_encode_f16_ties_go_to_even():
    # every finite positive half value h and the midpoint to its successor
    h = np.arange(0, 0x7bff, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2  # exact in binary64
    got = oracle.encode(mid, "f16")
    even = np.where(h % 2 == 0, h, h + 1).astype(np.uint16)
    assert np.array_equal(got, even)
    # a hair above the midpoint rounds up, a hair below rounds down
    assert np.array_equal(oracle.encode(np.nextafter(mid, np.inf), "f16"), (h + 1).astype(np.uint16))
    assert np.array_equal(oracle.encode(np.nextafter(mid, -np.inf), "f16")[1:], h[1:])
    assert oracle.encode(np.array([65520.0]), "f16")[0] == 0x7C00   # halfway to 2^16 -> inf
    assert oracle.encode(np.array([65519.99]), "f16")[0] == 0x7BFF
    assert oracle.encode(np.array([-0.0]), "f16")[0] == 0x8000
    assert oracle.encode(np.array([2.0 ** -25]), "f16")[0] == 0x0000  # tie between 0 and 2^-24
    assert oracle.encode(np.array([3 * 2.0 ** -25]), "f16")[0] == 0x0002


def test_encode_bf16_matches_torch_on_fp32_values():
    rng = np.random.default_rng(2)
    mag = np.exp2(rng.uniform(-140, 127, 200000)).astype(np.float32)
    x = (mag * rng.choice([-1.0, 1.0], mag.size).astype(np.float32)).astype(np.float32)
    got = oracle.encode(x.astype(np.float64), "bf16")
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_encode_bf16_ties_and_no_double_rounding():
    h = np.arange(0, 0x7f7f, 7, dtype=np.uint16)
    lo = oracle.decode(h, "bf16")
    hi = oracle.decode((h + 1).astype(np.uint16), "bf16")
    mid = (lo + hi) / 2
    even = np.where(h % 2 == 0, h, h + 1).astype(np.uint16)
    assert np.array_equal(oracle.encode(mid, "bf16"), even)
    # just above a midpoint by far less than an fp32 ulp: a direct binary64 -> bf16
    # rounding must go up; rounding through fp32 first would land on the tie.
    above = mid[1:] * (1 + 2.0 ** -40)
    assert np.array_equal(oracle.encode(above, "bf16"), (h[1:] + 1).astype(np.uint16))
    assert oracle.encode(np.array([1.0 + 2.0 ** -8]), "bf16")[0] == 0x3F80       # tie, 1.0 is even
    assert oracle.encode(np.array([1.0 + 3 * 2.0 ** -8]), "bf16")[0] == 0x3F82   # tie, round up to even
    assert oracle.encode(np.array([3.5e38]), "bf16")[0] == 0x7F80                 # overflow


# ---- tiny shapes against exact rational arithmetic ----------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_brute_force_all_tiny_shapes(dtype):
    seed = 0
    for M, N, K in itertools.product(range(1, 5), repeat=3):
        for a_col, b_col in itertools.product((False, True), repeat=2):
            seed += 1
            A, B = synth.logical(M, N, K, dtype, dist="normal_half", seed=seed)
            got = _ref(A, B, dtype, a_col, b_col)
            exact = _exact(A, B)
            Ad = A.to(torch.float64).numpy()
            Bd = B.to(torch.float64).numpy()
            bound = gamma(K) * (np.abs(Ad) @ np.abs(Bd))
            for i in range(M):
                for j in range(N):
                    err = abs(Fraction(float(got[i, j])) - exact[i][j])
                    assert err <= Fraction(float(bound[i, j])), (M, N, K, a_col, b_col, i, j)


def test_tiny_hand_example():
    # [[1, 2], [3, 4]] x [[5, 6], [7, 8]] = [[19, 22], [43, 50]]
    A = torch.tensor([[1.0, 2.0], [3.0, 4.0]])
    B = torch.tensor([[5.0, 6.0], [7.0, 8.0]])
    for dtype in ("f32", "f16", "bf16"):
        got = _ref(A.to(synth.TORCH_DTYPES[dtype]), B.to(synth.TORCH_DTYPES[dtype]), dtype)
        assert got.tolist() == [[19.0, 22.0], [43.0, 50.0]]
    # layouts: A column-major means storage [[1, 3], [2, 4]]
    As = np.array([[1, 3], [2, 4]], dtype=np.float32)
    Bs = np.array([[5, 7], [6, 8]], dtype=np.float32)
    got = oracle.gemm(2, 2, 2, As, 2, Bs, 2, "f32", a_col=True, b_col=True)
    assert got.tolist() == [[19.0, 22.0], [43.0, 50.0]]


# ---- closed forms -------------------------------------------------------------------------

SHAPES = [(64, 64, 64), (33, 17, 65), (128, 96, 80)]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("a_col,b_col", list(itertools.product((False, True), repeat=2)))
def test_identity_on_either_side(dtype, a_col, b_col):
    n = 96
    X, Y = synth.logical(n, n, n, dtype, dist="uniform", seed=7)
    I = torch.eye(n).to(synth.TORCH_DTYPES[dtype])
    assert np.array_equal(_ref(I, Y, dtype, a_col, b_col), Y.to(torch.float64).numpy())
    assert np.array_equal(_ref(X, I, dtype, a_col, b_col), X.to(torch.float64).numpy())


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_permutation_permutes_rows(dtype):
    n = 80
    P, Y = synth.logical(n, n, n, dtype, dist="perm", dist_b="uniform", seed=3)
    got = _ref(P, Y, dtype)
    p = P.to(torch.float64).numpy().argmax(axis=1)
    assert np.array_equal(got, Y.to(torch.float64).numpy()[p])


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_all_ones_gives_k(dtype, M, N, K):
    A, B = synth.logical(M, N, K, dtype, dist="ones")
    assert np.all(_ref(A, B, dtype) == K)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_all_ones_encodes_exactly_at_workload_depths(dtype):
    # C_ij = K is exact in every output type used: 64 ... 8192 are powers of two or
    # small integers.
    for K in (64, 1000, 1024, 2048, 4096, 8192):
        bits = oracle.encode(np.array([float(K)]), dtype)
        assert oracle.decode(bits, dtype)[0] == K


# ---- integer inputs: exact -----------------------------------------------------------------

@pytest.mark.parametrize("dtype,r", [("f32", 64), ("f16", 16), ("bf16", 8)])
@pytest.mark.parametrize("a_col,b_col", [(False, False), (False, True), (True, False)])
def test_integer_inputs_match_int64_product(dtype, r, a_col, b_col):
    M, N, K = 70, 45, 300
    A, B = synth.logical(M, N, K, dtype, dist="int", r=r, seed=11)
    got = _ref(A, B, dtype, a_col, b_col)
    want = A.to(torch.int64).numpy() @ B.to(torch.int64).numpy()
    assert np.array_equal(got, want.astype(np.float64))


def test_sparse_pm1_outputs_are_bounded_sums():
    M, N, K, period = 40, 50, 1000, 4
    A, B = synth.logical(M, N, K, "bf16", dist="sparse_pm1", seed=5, period=period)
    got = _ref(A, B, "bf16")
    want = A.to(torch.int64).numpy() @ B.to(torch.int64).numpy()
    assert np.array_equal(got, want.astype(np.float64))
    assert np.abs(got).max() <= -(-K // period)


# ---- a library routine -----------------------------------------------------------------------

@pytest.mark.parametrize("dtype,M,N,K", [("f32", 64, 64, 64), ("f16", 300, 200, 1000),
                                         ("bf16", 257, 129, 777)])
def test_against_numpy_binary64_matmul(dtype, M, N, K):
    A, B = synth.logical(M, N, K, dtype, dist="uniform", seed=21)
    got = _ref(A, B, dtype)
    Ad, Bd = A.to(torch.float64).numpy(), B.to(torch.float64).numpy()
    want = Ad @ Bd
    bound = 2 * gamma(K) * (np.abs(Ad) @ np.abs(Bd))  # both sides carry the summation error
    assert np.all(np.abs(got - want) <= bound)


# ---- storage ---------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_layouts_and_leading_dimensions_agree_bitwise(dtype):
    M, N, K = 37, 29, 53
    A, B = synth.logical(M, N, K, dtype, seed=9)
    base = _ref(A, B, dtype)
    for a_col, b_col in itertools.product((False, True), repeat=2):
        for pad_a, pad_b in ((0, 0), (3, 8), (11, 1)):
            lda = (M if a_col else K) + pad_a
            ldb = (K if b_col else N) + pad_b
            assert np.array_equal(_ref(A, B, dtype, a_col, b_col, lda, ldb), base)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sampled_elements_equal_rows(dtype):
    M, N, K = 50, 70, 129
    A, B = synth.logical(M, N, K, dtype, seed=4)
    As, lda = _store(A, False)
    Bs, ldb = _store(B, True)
    full = oracle.gemm(M, N, K, As, lda, Bs, ldb, dtype, b_col=True)
    rows = oracle.gemm(M, N, K, As, lda, Bs, ldb, dtype, b_col=True, rows=(10, 20))
    assert np.array_equal(rows, full[10:20])
    rng = np.random.default_rng(0)
    ii, jj = rng.integers(0, M, 300), rng.integers(0, N, 300)
    el = oracle.elements(M, N, K, As, lda, Bs, ldb, dtype, ii, jj, b_col=True)
    assert np.array_equal(el, full[ii, jj])


def test_degenerate_extents():
    A = np.zeros(0, dtype=np.float32)
    assert oracle.gemm(0, 5, 3, A, 3, np.ones(15, np.float32), 5, "f32").shape == (0, 5)
    # K = 0: the empty sum is zero
    C = oracle.gemm(4, 5, 0, A, 1, A, 5, "f32")
    assert C.shape == (4, 5) and np.all(C == 0)


def test_extent_checks_refuse_short_storage():
    with pytest.raises(ValueError):
        oracle.gemm(4, 4, 4, np.zeros(15, np.float32), 4, np.zeros(16, np.float32), 4, "f32")
    with pytest.raises(ValueError):
        oracle.gemm(4, 4, 4, np.zeros(16, np.float32), 3, np.zeros(16, np.float32), 4, "f32")
    with pytest.raises(TypeError):
        oracle.gemm(4, 4, 4, np.zeros(16, np.float64), 4, np.zeros(16, np.float32), 4, "f32")


# ---- planted mistakes are caught ---------------------------------------------------------------

def _pins_pass(gemm_fn):
    """Run the cheap closed-form and integer pins against a candidate gemm; a candidate
    that raises is caught as well."""
    n = 48
    try:
        X, Y = synth.logical(n, n, n, "f32", dist="uniform", seed=1)
        I = torch.eye(n)
        ok = np.array_equal(gemm_fn(I, Y), Y.double().numpy())
        ok = ok and np.array_equal(gemm_fn(X, I), X.double().numpy())
        A, B = synth.logical(20, 30, 40, "f32", dist="int", r=5, seed=2)
        ok = ok and np.array_equal(gemm_fn(A, B), (A.long().numpy() @ B.long().numpy()).astype(np.float64))
        P, Z = synth.logical(n, n, n, "f32", dist="perm", dist_b="uniform", seed=3)
        p = P.double().numpy().argmax(axis=1)
        ok = ok and np.array_equal(gemm_fn(P, Z), Z.double().numpy()[p])
    except (ValueError, IndexError):
        return False
    return ok


def test_pins_accept_the_oracle():
    assert _pins_pass(lambda A, B: _ref(A, B, "f32"))


@pytest.mark.parametrize("mistake", ["transpose_a", "transpose_b", "drop_last_k", "shift_column",
                                     "negate", "swap_operands"])
def test_pins_catch_planted_mistakes(mistake):
    def bad(A, B):
        M, K = A.shape
        N = B.shape[1]
        As, lda = _store(A, False)
        Bs, ldb = _store(B, False)
        if mistake == "transpose_a":      # reads A as if stored column-major
            return oracle.gemm(M, N, K, As, lda, Bs, ldb, "f32", a_col=True)
        if mistake == "transpose_b":      # reads B as if stored column-major
            return oracle.gemm(M, N, K, As, lda, Bs, ldb, "f32", b_col=True)
        if mistake == "drop_last_k":      # loop bound off by one
            return oracle.gemm(M, N, K - 1, As, lda, Bs, ldb, "f32")
        C = oracle.gemm(M, N, K, As, lda, Bs, ldb, "f32")
        if mistake == "shift_column":     # output column index off by one
            return np.roll(C, 1, axis=1)
        if mistake == "negate":           # sign error
            return -C
        return oracle.gemm(M, N, K, Bs, ldb, As, lda, "f32") if M == N == K else C.T  # swapped operands
    assert not _pins_pass(bad)
