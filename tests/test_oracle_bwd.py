"""Pins of the oracle's attention gradients: torch autograd in float64
through an explicit-mask softmax attention, central finite differences of the
oracle's own forward, and the dense case against torch's fused attention."""
import numpy as np
import pytest
import torch

import oracle
from test_oracle_pins import rand_inputs, selection_mask


def torch_masked_attention(q, k, v, mask, scale):
    """Explicit-mask attention in torch (float64), differentiable."""
    T, hq, d = q.shape
    G = hq // k.shape[1]
    kk = k.repeat_interleave(G, dim=1)
    vv = v.repeat_interleave(G, dim=1)
    z = scale * torch.einsum("thd,uhd->htu", q, kk)
    z = z.masked_fill(~mask, float("-inf"))
    p = torch.softmax(z, dim=-1)
    return torch.einsum("htu,uhd->thd", p, vv)


@pytest.mark.parametrize("lengths,B,hq,hkv,d,topk,seed", [
    ([96], 8, 2, 2, 8, 3, 1), ([40, 56], 4, 4, 2, 4, 4, 2), ([17, 0, 63], 16, 2, 1, 8, 2, 3)])
def test_gradients_match_autograd_through_explicit_mask(lengths, B, hq, hkv, d, topk, seed):
    q, k, v, cu = rand_inputs(lengths, hq, hkv, d, seed)
    _, _, sel, _ = oracle.moba(q, k, v, cu, B, topk)
    rng = np.random.default_rng(seed + 100)
    dout = rng.standard_normal(q.shape)
    scale = 1.0 / np.sqrt(d)
    dq, dk, dv = oracle.attend_bwd(q, k, v, dout, cu, B, topk, sel)
    tq, tk, tv = (torch.tensor(x.astype(np.float64), requires_grad=True) for x in (q, k, v))
    mask = torch.from_numpy(selection_mask(sel, cu, B))
    out = torch_masked_attention(tq, tk, tv, mask, scale)
    out.backward(torch.from_numpy(dout))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-11)


def test_gradients_match_finite_differences():
    lengths, B, hq, hkv, d, topk = [48], 8, 2, 1, 4, 3
    q, k, v, cu = rand_inputs(lengths, hq, hkv, d, 7)
    q, k, v = (x.astype(np.float64) for x in (q, k, v))
    _, _, sel, tie = oracle.moba(q.astype(np.float32), k.astype(np.float32),
                                 v.astype(np.float32), cu, B, topk)
    rng = np.random.default_rng(8)
    dout = rng.standard_normal(q.shape)

    def loss(qq, kk, vv):
        # the selection is held fixed (the gate is not differentiated)
        out, _ = oracle.attend(qq.astype(np.float32), kk.astype(np.float32),
                               vv.astype(np.float32), cu, B, topk, sel)
        return float((out * dout).sum())

    dq, dk, dv = oracle.attend_bwd(q.astype(np.float32), k.astype(np.float32),
                                   v.astype(np.float32), dout, cu, B, topk, sel)
    # perturbations of exactly representable size on float32 inputs: use values
    # that stay exact in float32 (the oracle widens its inputs exactly)
    h = 2.0 ** -10
    for arr, grad, name in ((q, dq, "q"), (k, dk, "k"), (v, dv, "v")):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in arr.shape)
            a = arr.astype(np.float32)
            plus, minus = a.copy(), a.copy()
            plus[idx] += np.float32(h)
            minus[idx] -= np.float32(h)
            args_p = [x.astype(np.float32) for x in (q, k, v)]
            args_m = [x.astype(np.float32) for x in (q, k, v)]
            which = "qkv".index(name)
            args_p[which], args_m[which] = plus, minus
            step = float(plus[idx]) - float(minus[idx])
            fd = (loss(*args_p) - loss(*args_m)) / step
            assert abs(fd - grad[idx]) <= 1e-5 * max(1.0, abs(grad[idx])), (name, idx, fd, grad[idx])


def test_dense_gradients_match_torch_sdpa():
    lengths, B, hq, hkv, d = [64, 40], 16, 4, 2, 8
    q, k, v, cu = rand_inputs(lengths, hq, hkv, d, 9)
    _, _, sel, _ = oracle.moba(q, k, v, cu, B, 4)  # 4 blocks cover both sequences
    rng = np.random.default_rng(10)
    dout = rng.standard_normal(q.shape)
    dq, dk, dv = oracle.attend_bwd(q, k, v, dout, cu, B, 4, sel)
    G = hq // hkv
    for s in range(len(lengths)):
        a, b = cu[s], cu[s + 1]
        Q = torch.tensor(q[a:b].astype(np.float64)).permute(1, 0, 2).requires_grad_()
        K = torch.tensor(k[a:b].astype(np.float64)).permute(1, 0, 2).requires_grad_()
        V = torch.tensor(v[a:b].astype(np.float64)).permute(1, 0, 2).requires_grad_()
        out = torch.nn.functional.scaled_dot_product_attention(
            Q, K.repeat_interleave(G, dim=0), V.repeat_interleave(G, dim=0), is_causal=True)
        out.backward(torch.tensor(dout[a:b]).permute(1, 0, 2))
        np.testing.assert_allclose(dq[a:b], Q.grad.permute(1, 0, 2).numpy(), rtol=0, atol=1e-11)
        np.testing.assert_allclose(dk[a:b], K.grad.permute(1, 0, 2).numpy(), rtol=0, atol=1e-11)
        np.testing.assert_allclose(dv[a:b], V.grad.permute(1, 0, 2).numpy(), rtol=0, atol=1e-11)


def test_dq_rows_equals_full_gradient_rows():
    """The row-subset dq follows the full gradient's arithmetic: equal on any
    subset of rows."""
    lengths, B, hq, hkv, d, topk = [70, 90], 16, 4, 2, 8, 3
    q, k, v, cu = rand_inputs(lengths, hq, hkv, d, 11)
    _, _, sel, _ = oracle.moba(q, k, v, cu, B, topk)
    dout = np.random.default_rng(12).standard_normal(q.shape)
    dq, _, _ = oracle.attend_bwd(q, k, v, dout, cu, B, topk, sel)
    rows = np.array([0, 5, 69, 70, 71, 100, 159])
    dq_r = oracle.attend_bwd_dq_rows(q, k, v, dout[rows], cu, B, topk, sel[rows], rows)
    assert np.array_equal(dq_r, dq[rows])


def test_gradient_identities():
    """Identities of softmax attention that hold at any size (sum_u dS_u = 0
    and sum_u P_u = 1 per row and head): sum over keys of dk is 0 per kv head;
    sum over keys of dv is the sum of dO over the group's rows; sum <dq, q> =
    sum <dk, k>; sum <dv, v> = sum over rows and heads of <dO, O>."""
    lengths, B, hq, hkv, d, topk = [150, 77], 32, 4, 2, 8, 3
    q, k, v, cu = rand_inputs(lengths, hq, hkv, d, 13)
    out, _, sel, _ = oracle.moba(q, k, v, cu, B, topk)
    dout = np.random.default_rng(14).standard_normal(q.shape)
    dq, dk, dv = oracle.attend_bwd(q, k, v, dout, cu, B, topk, sel)
    G = hq // hkv
    q64, k64, v64 = (x.astype(np.float64) for x in (q, k, v))
    scale_sum = np.abs(dk).sum()
    assert np.abs(dk.sum(axis=0)).max() <= 1e-12 * scale_sum
    dsum = dout.reshape(len(dout), hkv, G, d).sum(axis=(0, 2))
    np.testing.assert_allclose(dv.sum(axis=0), dsum, rtol=0, atol=1e-10)
    np.testing.assert_allclose((dq * q64).sum(), (dk * k64).sum(), rtol=1e-12, atol=1e-10)
    np.testing.assert_allclose((dv * v64).sum(), (dout * out).sum(), rtol=1e-12, atol=1e-10)
