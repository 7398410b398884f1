"""Pins of the parity comparator (oracle/check.py) itself.

The GPU parity tests trust check_selection and compare_outputs to reject a
wrong result. These CPU tests hand them small, hand-written selections and
outputs (no oracle and no GPU involved) and show that each kind of mistake is
rejected and each allowed difference accepted:
  * a difference on a row the oracle did not flag as a near tie;
  * on a flagged row, a swapped block whose score lies outside the tie band;
  * a row without its own block, with a duplicated block, unsorted, with a
    block after the own block, or with the wrong number of blocks;
  * outputs or lse outside the tolerances, and non-finite outputs.
The near-tie band is the 1e-3 relative band between the (k-1)-th and k-th
ranked earlier-block scores (summary page, section 3.4 "Top-k Gating": the
own block counts toward k).
"""
import numpy as np
import pytest

from oracle import check

NAN = float("nan")


def one_row(gpu, ora, tie, scores, topk):
    g = np.asarray(gpu, np.int32).reshape(1, 1, topk)
    o = np.asarray(ora, np.int32).reshape(1, 1, topk)
    t = np.asarray([[tie]], bool)
    s = np.asarray(scores, np.float64).reshape(1, 1, -1)
    return check.check_selection(g, o, t, s, topk)


# topk 3: own block 5 plus the 2 best of blocks 0..4.
CLEAR = [5.0, 4.0, 3.0, 2.0, 1.0, NAN]        # unambiguous: {0, 1} + 5
TIED = [5.0, 3.001, 3.0, 1.0, 0.5, NAN]       # 2nd and 3rd within 1e-3 relative


def test_identical_selection_is_accepted():
    differs, ties = one_row([0, 1, 5], [0, 1, 5], False, CLEAR, 3)
    assert not differs.any() and ties == 0


def test_difference_on_an_unflagged_row_is_rejected():
    with pytest.raises(AssertionError, match="outside a near tie"):
        one_row([0, 2, 5], [0, 1, 5], False, CLEAR, 3)


def test_swap_inside_the_tie_band_is_accepted():
    differs, ties = one_row([0, 2, 5], [0, 1, 5], True, TIED, 3)
    assert differs.sum() == 1 and ties == 1


def test_swap_outside_the_tie_band_is_rejected():
    # block 3 (score 1.0) is far below the band [3.0 - tol, 3.001 + tol]
    with pytest.raises(AssertionError, match="tie band"):
        one_row([0, 3, 5], [0, 1, 5], True, TIED, 3)
    # dropping the clear winner (block 0, score 5.0) for a tied block
    with pytest.raises(AssertionError, match="tie band"):
        one_row([1, 2, 5], [0, 1, 5], True, TIED, 3)


@pytest.mark.parametrize("gpu", [
    [0, 1, -1],    # own block missing
    [0, 2, 2],     # duplicate (and own block missing)
    [2, 0, 5],     # not ascending
    [0, 5, 2],     # a block after the own block
    [0, 5, -1],    # one block too few
    [-1, 2, 5],    # hole before the own block
    [0, 2, 6],     # a later block in place of the own block
])
def test_invalid_selection_on_a_flagged_row_is_rejected(gpu):
    with pytest.raises(AssertionError):
        one_row(gpu, [0, 1, 5], True, TIED, 3)


def test_short_rows_keep_their_padding():
    # row in block 1 with topk 3: selection {0, 1}, one -1
    s = [2.0, NAN, NAN]
    one_row([0, 1, -1], [0, 1, -1], False, s, 3)
    with pytest.raises(AssertionError):
        one_row([0, 1, 1], [0, 1, -1], True, s, 3)


def test_every_row_mode_counts_and_rejects(monkeypatch):
    """check_selection_all on a tiny stand-in oracle: counts ties and
    differences, and rejects an unflagged difference in any chunk."""
    T, H, k = 5, 2, 3
    ora = np.tile(np.array([0, 1, 5], np.int32), (T, H, 1))
    tie = np.zeros((T, H), bool)
    tie[3, 1] = True
    scores = np.tile(np.asarray(TIED), (T, H, 1))

    def fake_select(q, kbar, cu, B, topk, rows=None, want_scores=False):
        r = np.asarray(rows)
        return ora[r], tie[r], (scores[r] if want_scores else None)

    monkeypatch.setattr(check, "select", fake_select)
    gpu = ora.copy()
    gpu[3, 1] = [0, 2, 5]
    res = check.check_selection_all(gpu, None, None, None, 4, k, chunk_rows=2)
    assert res == dict(rows_checked=T, near_ties=1, differing=1)
    gpu[4, 0] = [0, 2, 5]   # last chunk, unflagged
    with pytest.raises(AssertionError, match="outside a near tie"):
        check.check_selection_all(gpu, None, None, None, 4, k, chunk_rows=2)


def outputs(n=4, h=2, d=8, seed=0):
    rng = np.random.default_rng(seed)
    ref = rng.standard_normal((n, h, d))
    lse = rng.standard_normal((n, h))
    return ref, lse


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_outputs_within_tolerance_are_accepted(dtype):
    ref, lse = outputs()
    tol = check.TOL[dtype]
    # fp32: a uniform offset of half the bound; bf16: one bf16 rounding (2^-9
    # relative) on every element
    got = ref + 0.5 * tol["out_abs"] if dtype == "fp32" else ref * (1 + 2.0 ** -9)
    stats = check.compare_outputs(got, lse + 0.5 * tol["lse_abs"], ref, lse, dtype)
    assert stats["out_max_abs"] <= tol["out_abs"]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_output_beyond_max_abs_is_rejected(dtype):
    ref, lse = outputs()
    bad = ref.copy()
    bad[1, 0, 3] += 2.0 * check.TOL[dtype]["out_abs"]
    with pytest.raises(AssertionError):
        check.compare_outputs(bad, lse, ref, lse, dtype)


def test_bf16_mean_relative_error_is_rejected():
    ref, lse = outputs()
    # every element off by just under the max-abs bound: the mean relative
    # error (sum |diff| / sum |ref|) then exceeds 1e-2
    bad = ref + 0.9 * check.TOL["bf16"]["out_abs"] * np.sign(ref)
    assert np.abs(bad - ref).sum() / np.abs(ref).sum() > check.TOL["bf16"]["out_rel"]
    with pytest.raises(AssertionError):
        check.compare_outputs(bad, lse, ref, lse, "bf16")


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_lse_beyond_tolerance_is_rejected(dtype):
    ref, lse = outputs()
    bad = lse.copy()
    bad[2, 1] += 2.0 * check.TOL[dtype]["lse_abs"]
    with pytest.raises(AssertionError):
        check.compare_outputs(ref, bad, ref, lse, dtype)


@pytest.mark.parametrize("where", ["out", "lse"])
def test_non_finite_output_is_rejected(where):
    ref, lse = outputs()
    o, l = ref.copy(), lse.copy()
    if where == "out":
        o[0, 0, 0] = np.nan
    else:
        l[0, 0] = np.inf
    with pytest.raises(AssertionError):
        check.compare_outputs(o, l, ref, lse, "bf16")
