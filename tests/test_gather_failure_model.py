"""The row-block failure class that ragged-tail tests must rule out.

ml-explore/mlx issue #3856 traces corrupt rows of the sorted affine
``gather_qmm`` to the remaining-row count ``M - (y_row + tm)`` being narrowed to
a 16-bit short before it is clamped: with 64-row tiles made of 32-row
subtiles, any subtile whose distance to the end is at least 32768 gets a
negative count and is never stored, unless M is a multiple of 64 (the aligned
path skips the count).  This pure-Python model of that arithmetic reproduces
every bad-row count the issue prints, which fixes the seam list used by the
GPU tail tests (our kernels keep every row count in int32 and must show zero
bad rows at all of these n).
"""

import numpy as np
import pytest

from tests.conftest import golden_rows

BM, SM = 64, 32


def _short(v: int) -> int:
    v &= 0xFFFF
    return v - 0x10000 if v >= 0x8000 else v


def bad_rows_16bit_model(n: int) -> np.ndarray:
    bad = np.zeros(n, bool)
    if n % BM == 0:
        return bad
    for y_row in range(0, n, BM):
        for tm in (0, SM):
            start = y_row + tm
            if start >= n:
                continue
            rows_left = _short(max(0, n - start))
            if min(SM, rows_left) <= 0:
                bad[start:start + SM] = True
    return bad


def bad_rows_int32(n: int) -> np.ndarray:
    """The fix: clamp in int, then narrow -- no subtile is ever skipped."""
    bad = np.zeros(n, bool)
    for y_row in range(0, n, BM):
        for tm in (0, SM):
            start = y_row + tm
            if start < n and min(SM, max(0, n - start)) <= 0:
                bad[start:start + SM] = True
    return bad


@pytest.mark.parametrize("row", golden_rows("gather_bad_rows.txt"))
def test_16bit_narrowing_reproduces_the_printed_bad_rows(row):
    n, count, first, last = (int(v) for v in row)
    bad = bad_rows_16bit_model(n)
    assert int(bad.sum()) == count
    if count:
        nz = np.nonzero(bad)[0]
        assert (nz[0], nz[-1]) == (first, last)
        assert np.all(np.diff(nz) == 1)          # one leading block of rows


@pytest.mark.parametrize("row", golden_rows("gather_bad_rows.txt"))
def test_int32_tile_arithmetic_has_no_bad_rows(row):
    assert not bad_rows_int32(int(row[0])).any()


def test_seams_below_32768_are_clean_even_with_narrowing():
    for n in (16068, 16065, 32767, 2048 * 8 + 4):
        assert not bad_rows_16bit_model(n).any()
