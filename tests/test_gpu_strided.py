"""Strided tensors on the GPU: moba_fwd_strided over views (one fused qkv
tensor, head-major tensors, an output inside a wider buffer) gives the same
bits as moba_fwd_gated over contiguous copies, and writes nothing outside its
output rows. Also: a row's result does not depend on which rows share its
attention tile (pass sizes change the tiles; outputs stay bit-equal), on
inputs where some rows of a tile need the running tile maximum and others do
not."""
import numpy as np
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


def workspace(q, k, cu, B, topk, kv_heads_per_pass=0):
    import torch
    sh = moba.shape_of(q, k, cu)
    n = moba.moba_fwd_workspace_size(sh, B, topk, kv_heads_per_pass)
    return torch.empty(n, dtype=torch.uint8, device="cuda")


def fused_views(q, k, v):
    """q, k, v copied into one [T][Hq + 2 Hkv + 1][d] tensor (one spare head
    at the end), returned as views of it."""
    import torch
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    qkv = torch.empty((T, Hq + 2 * Hkv + 1, d), dtype=q.dtype, device=q.device)
    qkv[:, :Hq] = q
    qkv[:, Hq:Hq + Hkv] = k
    qkv[:, Hq + Hkv:Hq + 2 * Hkv] = v
    return qkv[:, :Hq], qkv[:, Hq:Hq + Hkv], qkv[:, Hq + Hkv:Hq + 2 * Hkv]


def head_major(x):
    """A [T][H][d] view of a [H][T][d] copy of x."""
    return x.transpose(0, 1).contiguous().transpose(0, 1)


GATES = {"mean": None, "window": moba.gate_window(1), "pooled": moba.gate_pooled(1, 1)}

CASES = [
    # lengths,       Hq, Hkv, dtype,  B,   k, gate,    layout,       seed
    ([3000, 1000],   16,  4, "bf16", 256,  4, "mean",   "fused",      81),  # resident gate
    ([20000],         8,  2, "bf16",  64,  5, "mean",   "fused",      82),  # 313 blocks
    ([1500, 700],     4,  2, "bf16", 128,  3, "pooled", "head_major", 83),  # vector gate
    ([2500],          8,  4, "bf16", 192,  4, "window", "head_major", 84),
    ([513, 2048],     8,  8, "fp32", 256,  4, "mean",   "fused",      85),  # fp32 path
    ([777, 1234],     2,  1, "fp32",  64,  6, "pooled", "head_major", 86),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "L%s_%s_B%d_k%d_%s_%s" % (
    "-".join(map(str, c[0])), c[3], c[4], c[5], c[6], c[7]))
def test_strided_equals_contiguous_bit_for_bit(case):
    import torch
    lengths, hq, hkv, dtype, B, k, gate_name, layout, seed = case
    note("strided case %s" % (case,))
    inp = synth.custom(lengths, hq, hkv, 128, dtype, B, k, seed)
    q, kk, v, cu = (to_device(x) for x in (inp.q, inp.k, inp.v, inp.cu_seqlens))
    gate = GATES[gate_name]
    ref_out, ref_lse = moba.moba_fwd_gated(q, kk, v, cu, B, k,
                                           gate if gate is not None else moba.gate_mean(),
                                           workspace(q, kk, cu, B, k))
    if layout == "fused":
        qs, ks, vs = fused_views(q, kk, v)
    else:
        qs, ks, vs = head_major(q), head_major(kk), head_major(v)
    # (a view with one head is contiguous whatever its head stride)
    assert not qs.is_contiguous()
    assert hkv == 1 or not (ks.is_contiguous() or vs.is_contiguous())
    # the output inside a wider buffer: one sentinel head on each side
    T = q.shape[0]
    buf = torch.full((T, hq + 2, 128), 7.0, dtype=q.dtype, device="cuda")
    out = buf[:, 1:hq + 1]
    lse = torch.empty((hq, T), dtype=torch.float32, device="cuda")
    moba.moba_fwd_strided(qs, ks, vs, cu, B, k, workspace(q, kk, cu, B, k), gate=gate, out=out,
                          lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), "strided output differs"
    assert torch.equal(lse, ref_lse), "strided lse differs"
    assert bool((buf[:, 0] == 7.0).all()) and bool((buf[:, hq + 1] == 7.0).all()), \
        "wrote outside the output rows"
    # a head-major output
    out_hm = torch.empty((hq, T, 128), dtype=q.dtype, device="cuda").transpose(0, 1)
    moba.moba_fwd_strided(qs, ks, vs, cu, B, k, workspace(q, kk, cu, B, k), gate=gate,
                          out=out_hm)
    torch.cuda.synchronize()
    assert torch.equal(out_hm, ref_out), "head-major output differs"


def test_contiguous_entry_points_refuse_strided_tensors():
    import torch
    inp = synth.custom([512], 4, 2, 128, "bf16", 64, 2, 87)
    q, kk, v, cu = (to_device(x) for x in (inp.q, inp.k, inp.v, inp.cu_seqlens))
    with pytest.raises(ValueError):
        moba.moba_fwd(head_major(q), kk, v, cu, 64, 2)
    torch.cuda.synchronize()


def test_rows_are_independent_of_their_tile_neighbours():
    """Queries scaled by 8 or by 1/2, row by row at random: in most tiles
    some rows need the running tile maximum (their score bound exceeds the
    first tile's maximum by a wide margin) and others keep the first tile's.
    Pass sizes regroup the rows into other tiles; every bit must agree."""
    import torch
    inp = synth.custom([6000, 2000], 16, 4, 128, "bf16", 256, 5, 88)
    rng = np.random.default_rng(88)
    fac = np.where(rng.random(inp.q.shape[0]) < 0.5, 8.0, 0.5).astype(np.float32)
    qf = synth.bf16_bits_to_f32(inp.q) * fac[:, None, None]
    q = to_device(synth.f32_to_bf16_bits(qf))
    kk, v, cu = (to_device(x) for x in (inp.k, inp.v, inp.cu_seqlens))
    runs = []
    for p in (0, 1, 2):
        runs.append(moba.moba_fwd_ex(q, kk, v, cu, 256, 5, workspace(q, kk, cu, 256, 5, p)))
    torch.cuda.synchronize()
    for out, lse in runs[1:]:
        assert torch.equal(runs[0][0], out) and torch.equal(runs[0][1], lse)
    assert bool(torch.isfinite(runs[0][0].float()).all())
