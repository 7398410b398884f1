"""Pins of the oracle's gate variants: the fixed gates (sliding window,
attention sink) and the gate with extra blocks from max- and min-pooled keys.

As for the mean gate, every expected value comes from an independent
computation: numpy reductions, masks written from the definition of the
window, reductions to the mean gate or to dense attention, planted blocks.
"""
import numpy as np
import pytest

import oracle
from test_oracle_pins import causal_mask, masked_attention, rand_inputs, seq_info


def window_mask(cu, hq, B, w, n_sink):
    """Key u is visible to row t iff same sequence, u <= t and u's block is one
    of the w most recent blocks up to t's, or one of the n_sink first."""
    start, local = seq_info(cu)
    T = int(cu[-1])
    blk = local // B
    idx = np.arange(T)
    same = start[:, None] == start[None, :]
    recent = blk[None, :] > blk[:, None] - w
    sink = blk[None, :] < n_sink
    m = same & (idx[None, :] <= idx[:, None]) & (recent | sink)
    return np.broadcast_to(m, (hq, T, T))


@pytest.mark.parametrize("lengths,B,topk,n_sink", [
    ([96], 8, 3, 0), ([96], 8, 4, 1), ([40, 57, 0, 70], 8, 5, 2), ([33], 16, 2, 1)])
def test_window_gate_attention_matches_distance_mask(lengths, B, topk, n_sink):
    hq, hkv, d = 4, 2, 8
    q, k, v, cu = rand_inputs(lengths, hq, hkv, d, 31 + topk)
    sel = oracle.select_window(cu, B, topk, n_sink, hq)
    out, lse = oracle.attend(q, k, v, cu, B, topk, sel)
    ref_out, ref_lse = masked_attention(q, k, v, window_mask(cu, hq, B, topk - n_sink, n_sink),
                                        1.0 / np.sqrt(d))
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


def test_window_gate_special_cases():
    lengths = [70, 130]
    B, hq, hkv, d = 16, 2, 1, 4
    q, k, v, cu = rand_inputs(lengths, hq, hkv, d, 40)
    # one slot: the own block only, which the mean gate with topk = 1 also gives
    kbar = oracle.meanpool(k, cu, B)
    mean1, _, _ = oracle.select(q, kbar, cu, B, 1)
    np.testing.assert_array_equal(oracle.select_window(cu, B, 1, 0, hq), mean1)
    # enough slots for every block: dense causal attention
    sel = oracle.select_window(cu, B, 9, 1, hq)
    out, lse = oracle.attend(q, k, v, cu, B, 9, sel)
    ref_out, ref_lse = masked_attention(q, k, v, causal_mask(cu, hq), 1.0 / np.sqrt(d))
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


def test_minmaxpool_matches_numpy_reductions():
    lengths = [37, 64, 5, 0]
    B, hkv, d = 16, 3, 6
    _, k, _, cu = rand_inputs(lengths, 3, hkv, d, 41)
    kmax, kmin = oracle.minmaxpool(k, cu, B)
    b = 0
    for s in range(len(lengths)):
        for j in range(-(-lengths[s] // B)):
            rows = k[cu[s] + j * B:cu[s] + min(lengths[s], (j + 1) * B)]
            np.testing.assert_array_equal(kmax[b], rows.max(axis=0))
            np.testing.assert_array_equal(kmin[b], rows.min(axis=0))
            b += 1
    assert b == kmax.shape[0]


def test_pooled_gate_without_extras_is_the_mean_gate():
    lengths = [100, 64]
    B, hq, hkv, d, topk = 8, 4, 2, 8, 4
    q, k, v, cu = rand_inputs(lengths, hq, hkv, d, 42)
    kbar = oracle.meanpool(k, cu, B)
    kmax, kmin = oracle.minmaxpool(k, cu, B)
    sel, tie = oracle.select_pooled(q, kbar, kmax, kmin, cu, B, topk, 0, 0)
    ref, ref_tie, _ = oracle.select(q, kbar, cu, B, topk)
    np.testing.assert_array_equal(sel, ref)
    np.testing.assert_array_equal(tie, ref_tie)


def test_pooled_gate_with_constant_blocks_adds_nothing():
    """Blocks whose key rows are all equal have max = min = mean: the three
    rankings coincide and the extra picks repeat the mean gate's."""
    lengths = [96]
    B, hq, hkv, d = 8, 2, 1, 8
    q, k, v, cu = rand_inputs(lengths, hq, hkv, d, 43)
    for j in range(96 // B):
        k[j * B:(j + 1) * B] = k[j * B]
    kbar = oracle.meanpool(k, cu, B)
    kmax, kmin = oracle.minmaxpool(k, cu, B)
    sel, _ = oracle.select_pooled(q, kbar, kmax, kmin, cu, B, 6, 1, 1)
    ref, _, _ = oracle.select(q, kbar, cu, B, 4)  # 3 earlier blocks by mean, own block
    _, local = seq_info(cu)
    c = local // B
    for t in range(96):
        nsel = min(6, c[t] + 1)
        for h in range(hq):
            got = sel[t, h]
            assert got[nsel - 1] == c[t] and np.all(got[nsel:] == -1)
            np.testing.assert_array_equal(got[got >= 0], ref[t, h][ref[t, h] >= 0])


@pytest.mark.parametrize("pool", ["max", "min"])
def test_pooled_gate_picks_a_block_planted_for_one_pooling(pool):
    """A block with two opposite key rows has a zero mean. With +-50 on the
    coordinates where q > 0 its max-pooled key is +50 there and its
    min-pooled key -50 (best max-pooled score, worst min-pooled one); with
    +-50 where q < 0 it is the other way round. It is selected only when the
    favoured ranking gets an extra slot."""
    lengths = [256]
    B, hq, hkv, d = 32, 2, 1, 16
    q, k, v, cu = rand_inputs(lengths, hq, hkv, d, 44, scale_k=0.05)
    t, h, jstar = 250, 1, 3
    on = q[t, h] > 0 if pool == "max" else q[t, h] < 0
    blk = np.zeros((B, d), np.float32)
    blk[0] = np.where(on, 50.0, 0.0)
    blk[1] = -blk[0]                    # block mean stays zero
    k[jstar * B:(jstar + 1) * B, 0, :] = blk
    kbar = oracle.meanpool(k, cu, B)
    kmax, kmin = oracle.minmaxpool(k, cu, B)
    ex = (1, 0) if pool == "max" else (0, 1)
    base, _ = oracle.select_pooled(q, kbar, kmax, kmin, cu, B, 3, 0, 0, rows=[t])
    with_extra, _ = oracle.select_pooled(q, kbar, kmax, kmin, cu, B, 4, *ex, rows=[t])
    assert jstar not in base[0, h]
    assert jstar in with_extra[0, h]
    # the other pooling's extra slot does not pick it
    other = (0, 1) if pool == "max" else (1, 0)
    without, _ = oracle.select_pooled(q, kbar, kmax, kmin, cu, B, 4, *other, rows=[t])
    assert jstar not in without[0, h]


def test_pooled_gate_union_on_tiny_integer_inputs():
    """Brute force: each ranking's best set by exhaustive comparison of every
    pair of candidates (a block is picked iff fewer than `pick` candidates beat
    it under (score desc, index asc)), then their union."""
    rng = np.random.default_rng(45)
    lengths = [60]
    B, hq, hkv, d, topk, ex_max, ex_min = 6, 2, 1, 3, 6, 1, 2
    T = sum(lengths)
    q = rng.integers(-2, 3, (T, hq, d)).astype(np.float32)
    k = rng.integers(-2, 3, (T, hkv, d)).astype(np.float32)
    cu = np.array([0, T], np.int32)
    kbar = oracle.meanpool(k, cu, B)
    kmax, kmin = oracle.minmaxpool(k, cu, B)
    sel, _ = oracle.select_pooled(q, kbar, kmax, kmin, cu, B, topk, ex_max, ex_min)
    picks = {"mean": topk - ex_max - ex_min - 1, "max": ex_max, "min": ex_min}
    tables = {"mean": kbar, "max": kmax, "min": kmin}
    for t in range(T):
        c = t // B
        for h in range(hq):
            chosen = set()
            for name, pick in picks.items():
                s = [float(q[t, h].astype(np.float64) @ tables[name][j, 0]) for j in range(c)]
                for j in range(c):
                    better = sum(1 for i in range(c) if s[i] > s[j] or (s[i] == s[j] and i < j))
                    if better < pick:
                        chosen.add(j)
            got = sel[t, h]
            assert sorted(chosen) == [int(x) for x in got if 0 <= x < c]
            nsel = min(topk, c + 1)
            assert got[nsel - 1] == c and np.all(got[nsel:] == -1)
