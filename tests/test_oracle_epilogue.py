"""Pins of the oracle's fused epilogue (oracle.epilogue), on the CPU.

The epilogue is element-wise: T = act(alpha * S + beta * C_prior + bias[j]).  It is
pinned by a product worked out by hand (2 x 2 times 2 x 3, so that a bias indexed by
row instead of column, a sign error in beta, a missing alpha or ReLU applied in the
wrong place each change some printed value), by identities that reduce it to the
plain product or to a copy of C_prior, and by the ReLU's treatment of -0 and NaN.
Planted mistakes in an epilogue written the same way must fail these pins.
"""
import numpy as np
import pytest

import oracle

# A = [[1, 2], [3, 4]], B = [[5, 6, 7], [8, 9, 10]]: S = A B by hand.
A_HAND = np.array([[1, 2], [3, 4]], np.float32)
B_HAND = np.array([[5, 6, 7], [8, 9, 10]], np.float32)
S_HAND = np.array([[21, 24, 27], [47, 54, 61]], np.float64)
C_PRIOR = np.array([[1, 50, 0], [100, 0, -3]], np.float64)
BIAS = np.array([-40, 0.5, -60], np.float32)
# 2 S - C_PRIOR + BIAS, element by element:
#   2*21 - 1 - 40 = 1      2*24 - 50 + 0.5 = -1.5   2*27 - 0 - 60 = -6
#   2*47 - 100 - 40 = -46  2*54 - 0 + 0.5 = 108.5   2*61 + 3 - 60 = 65
T_HAND = np.array([[1, -1.5, -6], [-46, 108.5, 65]], np.float64)
T_HAND_RELU = np.array([[1, 0, 0], [0, 108.5, 65]], np.float64)


def _hand_product():
    S = oracle.gemm(2, 3, 2, A_HAND.reshape(-1), 2, B_HAND.reshape(-1), 3, "f32")
    assert np.array_equal(S, S_HAND)
    return S


def _pins_pass(epi):
    S = _hand_product()
    try:
        ok = np.array_equal(epi(S, 2.0, -1.0, C_PRIOR, BIAS, "none"), T_HAND)
        relu = epi(S, 2.0, -1.0, C_PRIOR, BIAS, "relu")
        ok = ok and np.array_equal(relu, T_HAND_RELU) and not np.signbit(relu).any()
        ok = ok and np.array_equal(epi(S, 1.0, 0.0, None, None, "none"), S)
        ok = ok and np.array_equal(epi(S, 0.0, 1.0, C_PRIOR, None, "none"), C_PRIOR)
        ok = ok and np.array_equal(epi(S, 0.0, 0.0, C_PRIOR, BIAS, "none"),
                                   np.broadcast_to(BIAS.astype(np.float64), (2, 3)))
    except (ValueError, IndexError, TypeError):
        return False
    return bool(ok)


def test_hand_example_and_identities():
    assert _pins_pass(oracle.epilogue)


def test_beta_zero_ignores_the_prior_c():
    S = _hand_product()
    nan = np.full((2, 3), np.nan)
    assert np.array_equal(oracle.epilogue(S, 2.0, 0.0, nan, BIAS), 2 * S + BIAS.astype(np.float64))


def test_relu_of_negative_zero_and_nan_is_positive_zero():
    T = oracle.epilogue(np.array([[-0.0, np.nan, -1e-30, 1e-30]]), activation="relu")
    assert np.array_equal(T, [[0.0, 0.0, 0.0, 1e-30]])
    assert not np.signbit(T).any()


def test_alpha_and_beta_are_the_fp32_values_passed():
    # 0.1 is not an fp32 value: the epilogue scales by the fp32 number nearest to it.
    T = oracle.epilogue(np.array([[1.0]]), alpha=0.1)
    assert T[0, 0] == float(np.float32(0.1)) != 0.1


def test_unknown_activation_is_refused():
    with pytest.raises(ValueError):
        oracle.epilogue(np.zeros((1, 1)), activation="gelu")


@pytest.mark.parametrize("mistake", ["bias_by_row", "beta_sign", "relu_first", "alpha_on_prior",
                                     "no_alpha", "relu_keeps_sign"])
def test_pins_catch_planted_mistakes(mistake):
    def bad(S, alpha, beta, C, bias, act):
        S = np.asarray(S, np.float64)
        b = None if bias is None else np.asarray(bias, np.float64)
        if mistake == "bias_by_row":
            T = alpha * S + (beta * C if beta else 0) + (b[:S.shape[0], None] if b is not None else 0)
        elif mistake == "beta_sign":
            T = alpha * S - (beta * C if beta else 0) + (b if b is not None else 0)
        elif mistake == "relu_first":
            T = alpha * S + (beta * C if beta else 0)
            T = (np.where(T > 0, T, 0.0) if act == "relu" else T) + (b if b is not None else 0)
            return T
        elif mistake == "alpha_on_prior":
            T = alpha * (S + (beta * C if beta else 0)) + (b if b is not None else 0)
        elif mistake == "no_alpha":
            T = S + (beta * C if beta else 0) + (b if b is not None else 0)
        else:
            T = alpha * S + (beta * C if beta else 0) + (b if b is not None else 0)
            return np.where(T > 0, T, -0.0) if act == "relu" and mistake == "relu_keeps_sign" else T
        return np.where(T > 0, T, 0.0) if act == "relu" else T
    assert not _pins_pass(bad)
