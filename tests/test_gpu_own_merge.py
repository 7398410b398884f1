"""The own block merged with the earlier blocks in one kernel (bf16).

moba_fwd runs, per pass, the earlier-block attention first and then the
own-block attention combined with its partial results (moba_attn_prep,
moba_attn_fwd_hist, moba_attn_fwd_own_merge as stages). That combination has
the arithmetic of moba_merge in the same order, so all three of these give
the same bits: the stages with a separate merge (moba_attn_fwd then
moba_merge), the stages with the merged own block, and one moba_fwd_gated
call. Cases cover more than 16 slots per row (the merge's slot groups wrap),
top-k covering every block, top-k 1 (the own block alone), the pooled gate's
empty slots (lse -inf), fp32 (where the merged stage runs the two kernels),
and a NULL lse.
"""
import pytest

from block_sparse_long_moba_amd import moba, synth
from block_sparse_long_moba_amd.tensors import to_device

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moba.lib()  # the HIP library must be present; no fallback
    yield
    torch.cuda.synchronize()


CASES = [
    # lengths,              Hq, Hkv, dtype,  B,   k, gate,     seed
    ([8192],                 4,  1, "bf16",  64, 33, "mean",    91),  # up to 33 slots per row
    ([1500],                 4,  4, "bf16", 256, 16, "mean",    92),  # top-k covers every block
    ([2000],                 8,  1, "bf16", 128,  1, "mean",    93),  # own block only
    ([3000, 1000],          16,  2, "bf16", 192,  5, "pooled",  94),  # empty slots
    ([0, 300, 64, 1, 700],   8,  2, "bf16",  64,  4, "window",  95),  # empty and one-row sequences
    ([4096, 513],           32,  8, "bf16", 512,  3, "mean",    96),  # 8B head shape, ragged tail
    ([777, 1234],            2,  1, "fp32",  64,  6, "mean",    97),  # fp32: two kernels
]


def gate_of(name):
    return {"mean": moba.gate_mean(), "window": moba.gate_window(1),
            "pooled": moba.gate_pooled(1, 1)}[name]


def run_stages(q, kk, v, cu, B, k, gate, merged, with_lse=True):
    """The forward pass through the stage entry points, one kv head per pass."""
    import torch
    sh = moba.shape_of(q, kk, cu)
    lay = moba.moba_plan(sh, B, k, 1)
    ws = torch.empty(lay.total_bytes, dtype=torch.uint8, device="cuda")
    T, hq = q.shape[0], q.shape[1]
    out = torch.empty_like(q)
    lse = torch.empty((hq, T), dtype=torch.float32, device="cuda") if with_lse else None
    moba.moba_seqtable(cu, sh, B, lay, ws)
    if gate.kind != moba.GATE_WINDOW:
        moba.moba_meanpool(kk, sh, B, lay, ws)
    if gate.kind == moba.GATE_POOLED:
        moba.moba_minmaxpool(kk, sh, B, lay, ws)
    for g0 in range(kk.shape[1]):
        if gate.kind == moba.GATE_WINDOW:
            moba.moba_gate_window(sh, B, k, gate.n_sink, lay, ws, g0)
        elif gate.kind == moba.GATE_POOLED:
            moba.moba_gate_pooled(q, sh, B, k, gate.extra_max, gate.extra_min, lay, ws, g0)
        else:
            moba.moba_gate(q, sh, B, k, lay, ws, g0)
        moba.moba_dispatch(sh, B, k, lay, ws, g0)
        if merged:
            moba.moba_attn_prep(kk, v, sh, B, k, lay, ws, g0)
            moba.moba_attn_fwd_hist(q, kk, sh, B, k, lay, ws, g0)
            moba.moba_attn_fwd_own_merge(q, kk, sh, B, k, lay, ws, out, lse, g0)
        else:
            moba.moba_attn_fwd(q, kk, v, sh, B, k, lay, ws, g0)
            moba.moba_merge(sh, B, k, lay, ws, out, lse, g0)
    return out, lse


@pytest.mark.parametrize("case", CASES, ids=lambda c: "L%s_h%d_%d_%s_B%d_k%d_%s" % (
    "-".join(map(str, c[0])), c[1], c[2], c[3], c[4], c[5], c[6]))
def test_merged_own_block_has_the_bits_of_the_separate_merge(case):
    import torch
    lengths, hq, hkv, dtype, B, k, gname, seed = case
    note("own-merge case %s" % (case,))
    inp = synth.custom(lengths, hq, hkv, 128, dtype, B, k, seed)
    q, kk, v, cu = (to_device(x) for x in (inp.q, inp.k, inp.v, inp.cu_seqlens))
    gate = gate_of(gname)
    sep = run_stages(q, kk, v, cu, B, k, gate, merged=False)
    mer = run_stages(q, kk, v, cu, B, k, gate, merged=True)
    mer_nolse = run_stages(q, kk, v, cu, B, k, gate, merged=True, with_lse=False)
    sh = moba.shape_of(q, kk, cu)
    ws = torch.empty(moba.moba_fwd_workspace_size(sh, B, k, 0), dtype=torch.uint8, device="cuda")
    one = moba.moba_fwd_gated(q, kk, v, cu, B, k, gate, ws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(sep[0].float()).all()) and bool(torch.isfinite(sep[1]).all())
    assert torch.equal(sep[0], mer[0]) and torch.equal(sep[1], mer[1]), "merged stage differs"
    assert torch.equal(sep[0], mer_nolse[0]), "merged stage without lse differs"
    assert torch.equal(sep[0], one[0]) and torch.equal(sep[1], one[1]), "one call differs"
