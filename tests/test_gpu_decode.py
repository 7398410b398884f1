"""GPU parity of decode (one new query per sequence over its KV cache)
through the C ABI. The decode query of sequence s is the token at its last
cache row, so the oracle's answer is the prefill result at that row: its
selection and its attention over the selected blocks (own block up to the
row)."""
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


def run_decode(inp, B, topk):
    """GPU decode of every sequence's last row; returns (rows, out, lse, idx)."""
    import torch
    cu = inp.cu_seqlens
    S = len(cu) - 1
    last = np.array([cu[s + 1] - 1 for s in range(S)])
    qd = np.zeros((S,) + inp.q.shape[1:], dtype=inp.q.dtype)
    for s in range(S):
        if cu[s + 1] > cu[s]:
            qd[s] = inp.q[last[s]]
    q, kc, vc, cud = (to_device(x) for x in (qd, inp.k, inp.v, cu))
    # the shape describes the cache: T rows in S sequences
    sh = moba.make_shape(inp.k.shape[0], S, inp.q.shape[1], inp.k.shape[1], 128,
                         inp.workload.dtype)
    nbytes = moba.moba_decode_workspace_size(sh, B, topk)
    assert nbytes > 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    moba.moba_decode_prepare(kc, cud, sh, B, topk, ws)
    out, lse = moba.moba_decode(q, kc, vc, sh, B, topk, ws)
    torch.cuda.synchronize()
    return last, to_host_f64(out), to_host_f64(lse).T, ws, sh


def decode_idx(ws, sh, B, topk):
    """The decode selection sits after the block table and the pooled keys."""
    import torch
    S, Hq = sh.num_seqs, sh.num_q_heads
    # offsets of the decode workspace: table, pooled keys (fp32 + bf16 split), idx
    align = lambda x: (x + 255) // 256 * 256
    NBb = -(-sh.total_tokens // B) + S
    table = (2 * 4 * (S + 1) + 15) // 16 * 16 + 16 * NBb
    off = align(table)
    off = align(off + 8 * NBb * sh.num_kv_heads * 128)
    return workspace_view(ws, off, S * Hq * topk, torch.int32).view(S, Hq, topk).cpu().numpy()


def check_decode(inp, B, topk, last, out, lse, idx, dtype):
    cu = inp.cu_seqlens
    nonempty = np.array([cu[s + 1] > cu[s] for s in range(len(cu) - 1)])
    rows = last[nonempty]
    if nonempty.any():
        kbar = oracle.meanpool(inp.k, cu, B)
        sel, ref_out, ref_lse, info, _ = check.reference_for_rows(
            inp.q, inp.k, inp.v, cu, kbar, B, topk, rows, gpu_sel_rows=idx[nonempty])
        stats = check.compare_outputs(out[nonempty], lse[nonempty], ref_out, ref_lse, dtype)
        note("stats %s %s" % (stats, info))
    # empty caches: zero output, lse -inf, no selection
    assert np.all(out[~nonempty] == 0) and np.all(np.isneginf(lse[~nonempty]))
    assert np.all(idx[~nonempty] == -1)


SMALL = [
    # lengths,                    Hq, Hkv, dtype,  B,   k, seed
    ([1000, 0, 1, 256, 4097],      8,  2, "bf16", 128,  3, 71),  # empty, one row, block ends
    ([513, 2048],                  8,  8, "fp32", 256,  4, 72),  # fp32 MHA
    ([8197],                      32,  8, "bf16", 512,  3, 73),  # 8B head shape
    ([1500, 700],                  4,  4, "bf16", 256, 16, 74),  # topk covers all: dense
    ([3000, 1000, 5000],          16,  2, "bf16", 192,  5, 75),  # G = 8, block 3*64
    ([40000, 17000],               4,  2, "bf16",  64,  6, 76),  # 624 and 265 earlier blocks
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "L%s_h%d_%d_%s_B%d_k%d" % (
    "-".join(map(str, c[0])), c[1], c[2], c[3], c[4], c[5]))
def test_decode_matches_prefill_last_rows(case):
    lengths, hq, hkv, dtype, B, k, seed = case
    note("decode case %s" % (case,))
    inp = synth.custom(lengths, hq, hkv, 128, dtype, B, k, seed)
    last, out, lse, ws, sh = run_decode(inp, B, k)
    check_decode(inp, B, k, last, out, lse, decode_idx(ws, sh, B, k), dtype)


@pytest.mark.parametrize("lengths,seed", [([1 << 20], 81), ([32768] * 32, 82)],
                         ids=["one_1M_sequence", "batch_32x32K"])
def test_decode_at_full_size(lengths, seed):
    B, k = 4096, 12
    note("decode %d sequence(s) of %d: generating" % (len(lengths), lengths[0]))
    inp = synth.custom(lengths, 32, 8, 128, "bf16", B, k, seed)
    last, out, lse, ws, sh = run_decode(inp, B, k)
    note("oracle on %d rows" % len(last))
    check_decode(inp, B, k, last, out, lse, decode_idx(ws, sh, B, k), "bf16")
