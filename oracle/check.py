"""Comparison of GPU results with the fp64 oracle.

TEST INFRASTRUCTURE (used by the test suite, the package smoke check and the
benchmark's CPU-baseline leg only).

Acceptance rules:
  * block selections must equal the oracle's bit for bit, except rows the
    oracle flags as near ties (k-th and (k+1)-th gate scores within 1e-3
    relative); on those rows the GPU's set may swap blocks whose oracle scores
    lie in the tie band, and the row's output is then checked against the
    oracle's attention over the GPU's selection, so every row is still checked;
  * outputs: fp32 max-abs 1e-4; bf16 max-abs 2e-2 and mean-relative
    (sum|diff| / sum|ref|) 1e-2; lse max-abs 1e-4 (fp32) and 1e-3 (bf16).
"""
from __future__ import annotations

import numpy as np

from . import attend, select

TOL = {
    "fp32": dict(out_abs=1e-4, out_rel=None, lse_abs=1e-4),
    "bf16": dict(out_abs=2e-2, out_rel=1e-2, lse_abs=1e-3),
}
TIE_REL = 1e-3


def sample_rows(cu_seqlens, block_size, per_block, seed, every_row_of_short_blocks=True):
    """Rows to check at full size: the first and last row of every block plus
    random rows, and every row of blocks shorter than block_size."""
    rng = np.random.default_rng(seed + 1000)
    rows = []
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for s in range(len(cu) - 1):
        a, L = int(cu[s]), int(cu[s + 1] - cu[s])
        for j in range(-(-L // block_size)):
            r0, r1 = a + j * block_size, a + min(L, (j + 1) * block_size)
            if every_row_of_short_blocks and r1 - r0 < block_size:
                rows.extend(range(r0, r1))
                continue
            rows.extend([r0, r1 - 1])
            if per_block > 2:
                rows.extend(rng.integers(r0, r1, per_block - 2).tolist())
    return np.unique(np.asarray(rows, dtype=np.int64))


def _row_structure_ok(g, o):
    """A selection row is valid when its chosen blocks form a strictly
    ascending prefix, padded with -1, that ends at the row's own block, with
    as many entries as the oracle's row (the own block is the oracle's last
    valid entry)."""
    n = int((o >= 0).sum())
    if int((g >= 0).sum()) != n or np.any(g[:n] < 0) or np.any(g[n:] != -1):
        return False
    if n and g[n - 1] != o[n - 1]:
        return False
    return bool(np.all(np.diff(g[:n]) > 0))


def check_selection(gpu_sel, ora_sel, ora_tie, ora_scores, topk):
    """Returns (differs[n][H] bool, n_near_ties). Raises on an unexplained
    difference.

    A row may differ from the oracle's only if the oracle flags it as a near
    tie; it must then still be a valid selection (see _row_structure_ok) and
    every block in which the two sets differ must score, in the oracle's fp64
    scores, inside the tie band [b - tol, a + tol], where a and b are the
    (k-1)-th and k-th ranked earlier-block scores and tol = TIE_REL * max(|a|, |b|).
    """
    gpu_sel = np.asarray(gpu_sel)
    differs = np.any(gpu_sel != ora_sel, axis=2)
    bad = differs & ~np.asarray(ora_tie, dtype=bool)
    if bad.any():
        r, h = map(int, np.argwhere(bad)[0])
        raise AssertionError("selection differs outside a near tie at sample row %d head %d: "
                             "gpu %s oracle %s" % (r, h, gpu_sel[r, h], ora_sel[r, h]))
    n = topk - 1
    for r, h in np.argwhere(differs):
        g, o = gpu_sel[r, h], ora_sel[r, h]
        if not _row_structure_ok(g, o):
            raise AssertionError("invalid selection at sample row %d head %d: gpu %s oracle %s"
                                 % (r, h, g, o))
        sc = ora_scores[r, h]
        cand = np.sort(sc[~np.isnan(sc)])[::-1]
        a, b = cand[n - 1], cand[n]
        tol = TIE_REL * max(abs(a), abs(b))
        for j in set(g[g >= 0].tolist()) ^ set(o[o >= 0].tolist()):
            if not (b - tol <= sc[j] <= a + tol):
                raise AssertionError("block %d swapped outside the tie band at sample row %d "
                                     "head %d: score %r, band [%r, %r]"
                                     % (j, r, h, sc[j], b - tol, a + tol))
    return differs, int(np.asarray(ora_tie).sum())


def check_selection_all(gpu_sel, q, kbar, cu_seqlens, block_size, topk, chunk_rows=1 << 15,
                        progress=None):
    """Every row of a full selection gpu_sel[T][Hq][topk] against the oracle's
    (select, in chunks of rows); oracle scores are computed only for rows
    that differ. Returns counts: rows, near ties, differing (row, head)."""
    gpu_sel = np.asarray(gpu_sel)
    T = gpu_sel.shape[0]
    ties = diff = 0
    for r0 in range(0, T, chunk_rows):
        rows = np.arange(r0, min(T, r0 + chunk_rows), dtype=np.int64)
        sel, tie, _ = select(q, kbar, cu_seqlens, block_size, topk, rows=rows)
        g = gpu_sel[r0:r0 + len(rows)]
        differs = np.any(g != sel, axis=2)
        if differs.any():
            rr = np.unique(np.nonzero(differs)[0])
            s2, t2, sc2 = select(q, kbar, cu_seqlens, block_size, topk, rows=rows[rr],
                                 want_scores=True)
            check_selection(g[rr], s2, t2, sc2, topk)
        ties += int(tie.sum())
        diff += int(differs.sum())
        if progress is not None and (r0 // chunk_rows) % 8 == 7:
            progress("selection checked on %d of %d rows" % (r0 + len(rows), T))
    return dict(rows_checked=int(T), near_ties=ties, differing=diff)


def compare_outputs(gpu_out, gpu_lse, ref_out, ref_lse, dtype):
    """gpu_out/ref_out [n][H][d], gpu_lse/ref_lse [n][H]; returns error stats."""
    tol = TOL[dtype]
    d_out = np.abs(np.asarray(gpu_out, np.float64) - ref_out)
    d_lse = np.abs(np.asarray(gpu_lse, np.float64) - ref_lse)
    stats = dict(out_max_abs=float(d_out.max(initial=0.0)),
                 out_mean_rel=float(d_out.sum() / max(np.abs(ref_out).sum(), 1e-300)),
                 lse_max_abs=float(d_lse.max(initial=0.0)))
    assert np.all(np.isfinite(gpu_out)) and np.all(np.isfinite(gpu_lse)), "non-finite GPU output"
    assert stats["out_max_abs"] <= tol["out_abs"], stats
    if tol["out_rel"] is not None:
        assert stats["out_mean_rel"] <= tol["out_rel"], stats
    assert stats["lse_max_abs"] <= tol["lse_abs"], stats
    return stats


def reference_for_rows(q, k, v, cu, kbar, block_size, topk, rows, gpu_sel_rows=None, scale=None,
                       out_rows=None):
    """Oracle selection (with near-tie flags and scores) for `rows`, and oracle
    outputs for `out_rows` (a subset of `rows`; default all of them). If the
    GPU's selection for `rows` is given it is checked, and near-tie rows where
    it differs get their reference output over the GPU's selection.
    Returns (sel, out, lse, info, out_index) with out_index the positions of
    the output rows inside `rows`."""
    rows = np.asarray(rows, dtype=np.int64)
    sel, tie, scores = select(q, kbar, cu, block_size, topk, rows=rows, want_scores=True)
    info = dict(rows_checked=int(len(rows)), near_ties=int(tie.sum()), differing=0)
    use = sel
    if gpu_sel_rows is not None:
        differs, _ = check_selection(gpu_sel_rows, sel, tie, scores, topk)
        info["differing"] = int(differs.sum())
        use = np.where(differs[..., None], gpu_sel_rows, sel)
    if out_rows is None:
        out_index = np.arange(len(rows))
    else:
        out_index = np.searchsorted(rows, np.asarray(out_rows, dtype=np.int64))
        assert np.all(rows[out_index] == out_rows), "out_rows must be a subset of rows"
    out, lse = attend(q, k, v, cu, block_size, topk, np.ascontiguousarray(use[out_index]),
                      scale=scale, rows=rows[out_index])
    info["output_rows"] = int(len(out_index))
    return sel, out, lse, info, out_index
