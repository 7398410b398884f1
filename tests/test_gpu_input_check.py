"""The device-side input check through the C ABI: a max_seqlen hint below the
longest sequence, and cu_seqlens that do not describe the tensors, must never
give numbers. Outputs become NaN, moba_workspace_status reports the failed
check, and with MOBA_CHECK=1 the whole-pass entry points return
MOBA_ERROR_INVALID_VALUE. A correct call on the same workspace afterwards
gives the same bits as on a fresh one.

The sequence table ("Context Partitioning" of the MoBA summary page, section
3.4: blocks restart in every sequence) is built from cu_seqlens on the device;
every later kernel reads rows only through it, and a failed check marks every
block invalid, so none of these calls reads outside its tensors.
"""
import os
import sys

import numpy as np
import pytest

from block_sparse_long_moba_amd import moba, synth
from block_sparse_long_moba_amd.tensors import to_device

pytestmark = pytest.mark.gpu

B, K = 256, 4


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


@pytest.fixture
def check_env():
    """Sets MOBA_CHECK=1 for the test and restores the environment."""
    old = os.environ.get("MOBA_CHECK")
    os.environ["MOBA_CHECK"] = "1"
    yield
    if old is None:
        del os.environ["MOBA_CHECK"]
    else:
        os.environ["MOBA_CHECK"] = old


def inputs(lengths=(3000, 1100), hq=8, hkv=2, seed=91):
    inp = synth.custom(list(lengths), hq, hkv, 128, "bf16", B, K, seed)
    q, k, v, cu = (to_device(x) for x in (inp.q, inp.k, inp.v, inp.cu_seqlens))
    return inp, q, k, v, cu


def all_nan(*ts):
    import torch
    return all(bool(torch.isnan(t.float()).all()) for t in ts)


def workspace(sh):
    import torch
    return torch.empty(moba.moba_fwd_workspace_size(sh, B, K, 0), dtype=torch.uint8,
                       device="cuda")


def test_understated_max_seqlen_gives_nan_and_a_status():
    import torch
    inp, q, k, v, cu = inputs()
    hint = 1100  # the longest sequence has 3000 rows: 12 blocks, the hint allows 5
    sh = moba.shape_of(q, k, cu, max_seqlen=hint)
    ws = workspace(sh)
    out = torch.zeros_like(q)
    lse = torch.zeros((q.shape[1], q.shape[0]), dtype=torch.float32, device="cuda")
    moba.moba_fwd_ex(q, k, v, cu, B, K, ws, out=out, lse=lse, max_seqlen=hint)
    torch.cuda.synchronize()
    assert all_nan(out, lse)
    with pytest.raises(moba.MobaError, match="max_seqlen"):
        moba.moba_workspace_status(sh.num_seqs, ws)
    # a correct call on the same workspace: the status clears and the result
    # equals a fresh run's bits
    sh2 = moba.shape_of(q, k, cu, max_seqlen=3000)
    ws2 = workspace(sh2)
    a = moba.moba_fwd_ex(q, k, v, cu, B, K, ws2, max_seqlen=3000)
    b = moba.moba_fwd_ex(q, k, v, cu, B, K, torch.empty_like(ws2), max_seqlen=3000)
    torch.cuda.synchronize()
    moba.moba_workspace_status(sh2.num_seqs, ws2)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert not torch.isnan(a[0].float()).any()


def test_understated_max_seqlen_with_moba_check(check_env):
    import torch
    inp, q, k, v, cu = inputs()
    sh = moba.shape_of(q, k, cu, max_seqlen=1100)
    ws = workspace(sh)
    out = torch.zeros_like(q)
    with pytest.raises(moba.MobaError) as e:
        moba.moba_fwd_ex(q, k, v, cu, B, K, ws, out=out, max_seqlen=1100)
    assert e.value.status == 1 and "max_seqlen" in str(e.value)
    torch.cuda.synchronize()
    assert not out.any()  # nothing after the check ran
    # moba_fwd (stream-ordered workspace) reports it the same way
    with pytest.raises(moba.MobaError):
        moba.moba_fwd(q, k, v, cu, B, K, max_seqlen=1100)
    # a correct hint passes the check
    moba.moba_fwd_ex(q, k, v, cu, B, K, workspace(moba.shape_of(q, k, cu, max_seqlen=3000)),
                     max_seqlen=3000)
    torch.cuda.synchronize()


@pytest.mark.parametrize("bad", ["short_total", "decreasing", "nonzero_start"])
def test_malformed_cu_seqlens(bad, check_env):
    import torch
    inp, q, k, v, cu = inputs()
    T = q.shape[0]
    cu_bad = {"short_total": [0, 3000, T - 100],
              "decreasing": [0, 3000, 2500, T],
              "nonzero_start": [64, 3000, T]}[bad]
    cud = torch.tensor(cu_bad, dtype=torch.int32, device="cuda")
    sh = moba.shape_of(q, k, cud)
    # without the check: NaN outputs and a reported status
    os.environ["MOBA_CHECK"] = "0"
    ws = workspace(sh)
    out, lse = moba.moba_fwd_ex(q, k, v, cud, B, K, ws)
    d_out, d_lse = moba.moba_dense_causal_fwd(q, k, v, cud)
    torch.cuda.synchronize()
    assert all_nan(out, lse, d_out, d_lse)
    with pytest.raises(moba.MobaError, match="cu_seqlens"):
        moba.moba_workspace_status(sh.num_seqs, ws)
    # with the check: an error before any further launch
    os.environ["MOBA_CHECK"] = "1"
    with pytest.raises(moba.MobaError, match="cu_seqlens"):
        moba.moba_fwd_ex(q, k, v, cud, B, K, ws)
    with pytest.raises(moba.MobaError, match="cu_seqlens"):
        moba.moba_dense_causal_fwd(q, k, v, cud)


def test_malformed_cu_seqlens_strided_output(check_env):
    """The NaN written for rejected cu_seqlens reaches every pass's output
    rows through the output strides (an output inside a wider buffer, one kv
    head per pass), and nothing outside them."""
    import torch
    inp, q, k, v, cu = inputs()
    T, hq = q.shape[0], q.shape[1]
    cud = torch.tensor([0, 3000, 2500, T], dtype=torch.int32, device="cuda")
    sh = moba.shape_of(q, k, cud)
    ws = torch.empty(moba.moba_fwd_workspace_size(sh, B, K, 1), dtype=torch.uint8,
                     device="cuda")
    buf = torch.full((T, hq + 2, 128), 7.0, dtype=q.dtype, device="cuda")
    out = buf[:, 1:hq + 1]
    lse = torch.zeros((hq, T), dtype=torch.float32, device="cuda")
    os.environ["MOBA_CHECK"] = "0"
    moba.moba_fwd_strided(q, k, v, cud, B, K, ws, out=out, lse=lse)
    torch.cuda.synchronize()
    assert all_nan(out, lse)
    assert bool((buf[:, 0] == 7.0).all()) and bool((buf[:, hq + 1] == 7.0).all())


def test_backward_and_decode_with_an_understated_hint():
    import torch
    inp, q, k, v, cu = inputs()
    hint = 1100
    # backward: gradients of a correct forward pass, with the bad hint
    out, lse = moba.moba_fwd(q, k, v, cu, B, K)
    dout = torch.randn_like(q)
    sh = moba.shape_of(q, k, cu, max_seqlen=hint)
    wsb = torch.empty(moba.moba_bwd_workspace_size(sh, B, K, 0), dtype=torch.uint8,
                      device="cuda")
    dq, dk, dv = moba.moba_bwd(q, k, v, out, lse, dout, cu, B, K, wsb, max_seqlen=hint)
    torch.cuda.synchronize()
    assert all_nan(dq, dk, dv)
    with pytest.raises(moba.MobaError, match="max_seqlen"):
        moba.moba_workspace_status(sh.num_seqs, wsb)
    # decode over the caches, with a hint below the longest cache
    S = len(inp.cu_seqlens) - 1
    qd = q[torch.tensor(inp.cu_seqlens[1:] - 1, dtype=torch.long, device="cuda")].contiguous()
    csh = moba.make_shape(q.shape[0], S, q.shape[1], k.shape[1], 128, "bf16", max_seqlen=hint)
    wsd = torch.empty(moba.moba_decode_workspace_size(csh, B, K), dtype=torch.uint8,
                      device="cuda")
    moba.moba_decode_prepare(k, cu, csh, B, K, wsd)
    o, l = moba.moba_decode(qd, k, v, csh, B, K, wsd)
    torch.cuda.synchronize()
    assert all_nan(o, l)
    with pytest.raises(moba.MobaError, match="max_seqlen"):
        moba.moba_workspace_status(S, wsd)
