"""GPU parity of the gate variants (sliding window / attention sink, and the
gate with extra blocks from max- and min-pooled keys) through the C ABI,
against the fp64 oracle: every row of small shapes, sampled rows of the 128K
workload, and the stage entry points against the one-call path."""
import sys

import numpy as np
import pytest

import oracle
from oracle import check
from block_sparse_long_moba_amd import moba, synth
from block_sparse_long_moba_amd.tensors import to_device, to_host_f64, workspace_view

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moba.lib()
    yield
    torch.cuda.synchronize()


def setup(inp, B, topk, kv_heads_per_pass=0):
    """Inputs on the device, the plan for the pass size and a workspace of
    exactly that size (moba_fwd_gated then runs with that pass size)."""
    import torch
    q, kk, v, cu = (to_device(x) for x in (inp.q, inp.k, inp.v, inp.cu_seqlens))
    sh = moba.shape_of(q, kk, cu)
    lay = moba.moba_plan(sh, B, topk, kv_heads_per_pass)
    ws = torch.empty(lay.total_bytes, dtype=torch.uint8, device="cuda")
    return q, kk, v, cu, sh, lay, ws


def gpu_idx(ws, lay, T, Hp, topk):
    import torch
    return workspace_view(ws, lay.idx_offset, T * Hp * topk, torch.int32).view(
        T, Hp, topk).cpu().numpy()


def structure_ok(sel, c, topk):
    """Own block at min(topk, c+1)-1, earlier blocks ascending and distinct
    before it, -1 elsewhere."""
    nsel = min(topk, c + 1)
    if sel[nsel - 1] != c or np.any(sel[nsel:] != -1):
        return False
    e = sel[:nsel - 1]
    e = e[e >= 0]
    return bool(np.all((e >= 0) & (e < c)) and np.all(np.diff(e) > 0)
                and np.all(sel[:nsel - 1][len(e):] == -1))


WINDOW = [
    # lengths,            Hq, Hkv, dtype,  B,  k, n_sink, seed
    ([1000],               4,  2, "bf16", 128, 3, 0, 51),
    ([0, 300, 64, 1, 700], 8,  2, "bf16",  64, 4, 1, 52),
    ([513, 2048],          8,  8, "fp32", 256, 4, 2, 53),
    ([3000, 1000],        16,  2, "bf16", 192, 5, 1, 54),
]


@pytest.mark.parametrize("case", WINDOW, ids=lambda c: "L%s_%s_B%d_k%d_sink%d" % (
    "-".join(map(str, c[0])), c[3], c[4], c[5], c[6]))
def test_window_gate_every_row(case):
    import torch
    lengths, hq, hkv, dtype, B, k, n_sink, seed = case
    note("window case %s" % (case,))
    inp = synth.custom(lengths, hq, hkv, 128, dtype, B, k, seed)
    q, kk, v, cu, sh, lay, ws = setup(inp, B, k)
    out, lse = moba.moba_fwd_gated(q, kk, v, cu, B, k, moba.gate_window(n_sink), ws)
    torch.cuda.synchronize()
    T = inp.q.shape[0]
    sel = oracle.select_window(inp.cu_seqlens, B, k, n_sink, hq)
    np.testing.assert_array_equal(gpu_idx(ws, lay, T, hq, k), sel)  # one pass: all heads
    ref_out, ref_lse = oracle.attend(inp.q, inp.k, inp.v, inp.cu_seqlens, B, k, sel)
    stats = check.compare_outputs(to_host_f64(out), to_host_f64(lse).T, ref_out, ref_lse, dtype)
    note("stats %s" % stats)
    # stage entry points, passes of one kv head: the same bits
    q2, kk2, v2, cu2, sh2, lay2, ws2 = setup(inp, B, k, kv_heads_per_pass=1)
    out2 = torch.empty_like(q2)
    lse2 = torch.empty((hq, T), dtype=torch.float32, device="cuda")
    moba.moba_seqtable(cu2, sh2, B, lay2, ws2)
    for g0 in range(hkv):
        moba.moba_gate_window(sh2, B, k, n_sink, lay2, ws2, g0)
        moba.moba_dispatch(sh2, B, k, lay2, ws2, g0)
        moba.moba_attn_fwd(q2, kk2, v2, sh2, B, k, lay2, ws2, g0)
        moba.moba_merge(sh2, B, k, lay2, ws2, out2, lse2, g0)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def pooled_reference(inp, B, topk, ex_max, ex_min, gsel, rows):
    """Oracle selection for `rows`, the GPU selection checked against it, and
    the selection to compute reference outputs with (the GPU's on near-tie
    rows where it differs, after checking it is a valid choice)."""
    kbar = oracle.meanpool(inp.k, inp.cu_seqlens, B)
    kmax, kmin = oracle.minmaxpool(inp.k, inp.cu_seqlens, B)
    sel, tie = oracle.select_pooled(inp.q, kbar, kmax, kmin, inp.cu_seqlens, B, topk, ex_max,
                                    ex_min, rows=rows)
    start = np.repeat(inp.cu_seqlens[:-1], np.diff(inp.cu_seqlens))
    first = oracle.block_first(inp.cu_seqlens, B)
    seq = np.searchsorted(inp.cu_seqlens, rows, side="right") - 1
    G = inp.q.shape[1] // inp.k.shape[1]
    picks = [(kbar, topk - ex_max - ex_min - 1), (kmax, ex_max), (kmin, ex_min)]
    use = sel.copy()
    n_diff = 0
    for i, t in enumerate(rows):
        c = int((t - start[t]) // B)
        for h in range(sel.shape[1]):
            g = gsel[i, h]
            assert structure_ok(g, c, topk), (t, h, g)
            if np.array_equal(g, sel[i, h]):
                continue
            assert tie[i, h], ("selection differs outside a near tie", t, h, g, sel[i, h])
            n_diff += 1
            chosen = set(int(x) for x in g if 0 <= x < c)
            may, must = set(), set()
            qv = inp.q[t, h].astype(np.float64)
            if inp.q.dtype == np.uint16:
                qv = synth.bf16_bits_to_f32(inp.q[t, h]).astype(np.float64)
            for pool, pick in picks:
                if pick == 0 or c == 0:
                    continue
                s = pool[first[seq[i]]:first[seq[i]] + c, h // G] @ qv
                order = np.lexsort((np.arange(c), -s))
                if pick >= c:
                    must |= set(range(c))
                    continue
                a, b = s[order[pick - 1]], s[order[pick]]
                tol = 1e-3 * max(abs(a), abs(b))
                must |= set(int(j) for j in range(c) if s[j] > b + tol)
                may |= set(int(j) for j in range(c) if s[j] >= a - tol)
            assert must <= chosen <= (may | must), (t, h, sorted(chosen), sorted(must), sorted(may))
            use[i, h] = g
    return use, int(tie.sum()), n_diff


POOLED = [
    # lengths,          Hq, Hkv, dtype,  B,   k, ex_max, ex_min, seed
    ([2000],             8,  2, "bf16", 128,  5, 1, 1, 61),   # matrix-core gate (G = 4)
    ([0, 700, 1500],     4,  2, "bf16",  64,  6, 2, 1, 62),   # vector gate (G = 2)
    ([1500, 513],        8,  8, "fp32", 128,  4, 1, 1, 63),   # fp32
    ([4096],            32,  8, "bf16", 256,  8, 2, 2, 64),   # 8B head shape
    ([8192],             8,  2, "bf16",  64, 22, 2, 1, 65),   # mean ranking keeps 18 (list of 24)
]


@pytest.mark.parametrize("case", POOLED, ids=lambda c: "L%s_%s_B%d_k%d_x%d_n%d" % (
    "-".join(map(str, c[0])), c[3], c[4], c[5], c[6], c[7]))
def test_pooled_gate_every_row(case):
    import torch
    lengths, hq, hkv, dtype, B, k, ex_max, ex_min, seed = case
    note("pooled case %s" % (case,))
    inp = synth.custom(lengths, hq, hkv, 128, dtype, B, k, seed)
    q, kk, v, cu, sh, lay, ws = setup(inp, B, k)
    out, lse = moba.moba_fwd_gated(q, kk, v, cu, B, k, moba.gate_pooled(ex_max, ex_min), ws)
    torch.cuda.synchronize()
    T = inp.q.shape[0]
    # pooled keys: max and min are exact. The kbar region holds, per pooling,
    # an fp32 table and its bf16 hi/lo split: 8 bytes per element each.
    kmax_ref, kmin_ref = oracle.minmaxpool(inp.k, inp.cu_seqlens, B)
    nb = kmax_ref.shape[0]
    nkb = lay.num_blocks_bound * hkv * 128
    kmax = workspace_view(ws, lay.kbar_offset + 8 * nkb, nb * hkv * 128, torch.float32)
    kmin = workspace_view(ws, lay.kbar_offset + 16 * nkb, nb * hkv * 128, torch.float32)
    np.testing.assert_array_equal(kmax.view(nb, hkv, 128).cpu().numpy(), kmax_ref)
    np.testing.assert_array_equal(kmin.view(nb, hkv, 128).cpu().numpy(), kmin_ref)
    rows = np.arange(T)
    use, n_tie, n_diff = pooled_reference(inp, B, k, ex_max, ex_min, gpu_idx(ws, lay, T, hq, k),
                                          rows)
    ref_out, ref_lse = oracle.attend(inp.q, inp.k, inp.v, inp.cu_seqlens, B, k, use)
    stats = check.compare_outputs(to_host_f64(out), to_host_f64(lse).T, ref_out, ref_lse, dtype)
    note("stats %s near_ties %d differing %d" % (stats, n_tie, n_diff))
    # stage entry points, passes of one kv head: the same bits
    q2, kk2, v2, cu2, sh2, lay2, ws2 = setup(inp, B, k, kv_heads_per_pass=1)
    out2 = torch.empty_like(q2)
    lse2 = torch.empty((hq, T), dtype=torch.float32, device="cuda")
    moba.moba_seqtable(cu2, sh2, B, lay2, ws2)
    moba.moba_meanpool(kk2, sh2, B, lay2, ws2)
    moba.moba_minmaxpool(kk2, sh2, B, lay2, ws2)
    for g0 in range(hkv):
        moba.moba_gate_pooled(q2, sh2, B, k, ex_max, ex_min, lay2, ws2, g0)
        moba.moba_dispatch(sh2, B, k, lay2, ws2, g0)
        moba.moba_attn_fwd(q2, kk2, v2, sh2, B, k, lay2, ws2, g0)
        moba.moba_merge(sh2, B, k, lay2, ws2, out2, lse2, g0)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("name", ["gqa32x8_t128k_b4096_k12_bf16", "gqa32x8_t1m_b4096_k12_bf16"])
@pytest.mark.parametrize("kind", ["window", "pooled"])
def test_gates_on_full_workloads_sampled_rows(kind, name):
    """128K and 1M tokens, in the benchmark's launch configuration (its pass
    size; the pooled gate with one extra block per pooling on top of k = 12)."""
    import torch
    w = synth.WORKLOADS[name]
    inp = synth.generate(w)
    B = w.block_size
    topk = 12 if kind == "window" else 14
    gate = moba.gate_window(1) if kind == "window" else moba.gate_pooled(1, 1)
    P = w.num_kv_heads
    full = moba.make_shape(w.total_tokens, len(w.lengths), w.num_q_heads, w.num_kv_heads, 128,
                           w.dtype)
    while P > 1 and moba.moba_fwd_workspace_size(full, B, topk, P) > (48 << 30):
        P //= 2
    note("%s %s gate: GPU run, pass of %d kv heads" % (name, kind, P))
    q, kk, v, cu, sh, lay, ws = setup(inp, B, topk, kv_heads_per_pass=P)
    out, lse = moba.moba_fwd_gated(q, kk, v, cu, B, topk, gate, ws)
    torch.cuda.synchronize()
    rows = check.sample_rows(inp.cu_seqlens, B, 4, w.seed)
    rng = np.random.default_rng(w.seed + 3000)
    out_rows = np.unique(np.concatenate([rng.choice(rows, 96, replace=False), [0, len(inp.q) - 1]]))
    note("%s %s gate: oracle on %d rows" % (name, kind, len(out_rows)))
    if kind == "window":
        use = oracle.select_window(inp.cu_seqlens, B, topk, 1, w.num_q_heads, rows=out_rows)
    else:
        # the last pass's selection is in the workspace: check those heads' rows
        Hp = lay.q_heads_per_pass
        T = inp.q.shape[0]
        gsel = workspace_view(ws, lay.idx_offset, T * Hp * topk, torch.int32).view(
            T, Hp, topk).cpu().numpy()
        h0 = w.num_q_heads - Hp
        kbar = oracle.meanpool(inp.k, inp.cu_seqlens, B)
        kmax, kmin = oracle.minmaxpool(inp.k, inp.cu_seqlens, B)
        use, tie = oracle.select_pooled(inp.q, kbar, kmax, kmin, inp.cu_seqlens, B, topk, 1, 1,
                                        rows=out_rows)
        differs = np.any(gsel[out_rows] != use[:, h0:], axis=2)
        assert not np.any(differs & ~tie[:, h0:]), "selection differs outside a near tie"
        use[:, h0:] = np.where(differs[..., None], gsel[out_rows], use[:, h0:])
    ref_out, ref_lse = oracle.attend(inp.q, inp.k, inp.v, inp.cu_seqlens, B, topk, use,
                                     rows=out_rows)
    stats = check.compare_outputs(to_host_f64(out)[out_rows], to_host_f64(lse).T[out_rows],
                                  ref_out, ref_lse, "bf16")
    note("stats %s" % stats)
