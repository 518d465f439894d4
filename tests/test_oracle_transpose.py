"""Pins of the oracle's transpose (oracle.transpose), on the CPU: a case worked by hand,
involution, agreement with numpy's own transposition on random shapes and padded
leading dimensions, and planted mistakes that these pins must catch."""
import numpy as np
import pytest

import oracle


def test_hand_example():
    # in (2 x 3) = [[1, 2, 3], [4, 5, 6]]  ->  out (3 x 2) = [[1, 4], [2, 5], [3, 6]]
    out = oracle.transpose(np.array([1, 2, 3, 4, 5, 6], np.int32), 2, 3, 3)
    assert out.tolist() == [1, 4, 2, 5, 3, 6]


@pytest.mark.parametrize("rows,cols,ld_in,ld_out", [(5, 7, 7, 5), (64, 64, 64, 64), (33, 17, 20, 40), (1, 9, 9, 1),
                                                    (9, 1, 3, 9)])
def test_agrees_with_numpy_transposition(rows, cols, ld_in, ld_out):
    rng = np.random.default_rng(rows * 100 + cols)
    x = rng.integers(0, 1 << 16, (rows, ld_in)).astype(np.uint16)
    out = oracle.transpose(x, rows, cols, ld_in, ld_out).reshape(cols, ld_out)
    assert np.array_equal(out[:, :rows], x[:, :cols].T)
    assert not out[:, rows:].any()                # padding columns of out stay zero


def test_twice_is_the_identity():
    x = np.random.default_rng(1).integers(-1 << 31, 1 << 31, 37 * 23).astype(np.int32)
    assert np.array_equal(oracle.transpose(oracle.transpose(x, 37, 23, 23), 23, 37, 37), x)


def test_refuses_short_storage_and_small_ld():
    with pytest.raises(ValueError):
        oracle.transpose(np.zeros(10, np.int32), 3, 4, 4)
    with pytest.raises(ValueError):
        oracle.transpose(np.zeros(12, np.int32), 3, 4, 3)


def _pins_pass(fn):
    try:
        ok = fn(np.array([1, 2, 3, 4, 5, 6], np.int32), 2, 3, 3).tolist() == [1, 4, 2, 5, 3, 6]
        rng = np.random.default_rng(2)
        x = rng.integers(0, 1000, (33, 20)).astype(np.int32)
        ok = ok and np.array_equal(fn(x, 33, 17, 20, 40).reshape(17, 40)[:, :33], x[:, :17].T)
    except (ValueError, IndexError):
        return False
    return bool(ok)


def test_pins_accept_the_oracle():
    assert _pins_pass(oracle.transpose)


@pytest.mark.parametrize("mistake", ["copy", "ld_in_as_cols", "ld_out_as_rows", "reverse_rows"])
def test_pins_catch_planted_mistakes(mistake):
    def bad(x, rows, cols, ld_in, ld_out=None):
        ld_out = rows if ld_out is None else ld_out
        x = np.asarray(x).reshape(-1)
        out = np.zeros(cols * ld_out, dtype=x.dtype)
        for r in range(rows):
            for c in range(cols):
                src = r * (cols if mistake == "ld_in_as_cols" else ld_in) + c
                dst = c * (rows if mistake == "ld_out_as_rows" else ld_out) + r
                if mistake == "copy":
                    dst = r * cols + c
                if mistake == "reverse_rows":
                    dst = c * ld_out + (rows - 1 - r)
                out[dst] = x[src]
        return out
    assert not _pins_pass(bad)
