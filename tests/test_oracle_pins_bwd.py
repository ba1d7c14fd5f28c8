"""Pins for the oracle's backward pass: every gradient (input, router weight
and bias, expert weights and biases, shared experts) against torch autograd
in fp64 on an independent dense formulation of the layer (every expert on
every token, masked by the kept top-k pairs, gates per mode, L_aux and z as
the pages print them). The routing decision is held fixed on both sides and
the fp32 rounding of the logits passes gradients straight through. CPU only."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import gen
import oracle
from test_oracle_pins import _dense_expert, _dispatch_by_stable_sort, _lexsort_topk, _t64, _tiny, _weights64, \
    _with_random_biases


def _autograd_layer(inp, dy, c_aux, c_z):
    wl = inp.wl
    T, N, k = wl.T, wl.n_experts, wl.top_k
    X = _t64(inp.x, wl.act_dtype).requires_grad_()
    Wr = _t64(inp.w_router, wl.act_dtype).requires_grad_()
    br = torch.from_numpy(inp.b_router).double().requires_grad_() if inp.b_router is not None else None
    W1, W3, W2 = (t.requires_grad_() if t is not None else None for t in _weights64(inp))
    b1 = torch.from_numpy(inp.b1).double().requires_grad_() if inp.b1 is not None else None
    b2 = torch.from_numpy(inp.b2).double().requires_grad_() if inp.b2 is not None else None
    l = F.linear(X, Wr, br)
    l = l + (l.detach().float().double() - l.detach())  # the fp32 router output, gradient straight through
    p = torch.softmax(l, dim=1)
    idx = _lexsort_topk(l.detach().numpy(), k).astype(np.int64)
    it = torch.from_numpy(idx)
    if wl.gating == gen.SOFTMAX_TOPK:
        g = p.gather(1, it)
    elif wl.gating == gen.SOFTMAX_TOPK_RENORM:
        g = p.gather(1, it)
        g = g / g.sum(1, keepdim=True)
    else:
        g = torch.softmax(l.gather(1, it), dim=1)
    _, _, _, inv, _ = _dispatch_by_stable_sort(idx.astype(np.int32), N, wl.capacity())
    kept = torch.from_numpy(inv >= 0).double()
    dense = torch.stack([_dense_expert(wl, W1, W3, W2, b1, b2, e, X) for e in range(N)], 1)  # [T, N, d]
    picked = dense.gather(1, it[:, :, None].expand(T, k, wl.d))                              # [T, k, d]
    y = ((g * kept)[:, :, None] * picked).sum(1)
    shared = []
    if wl.n_shared:
        S1, S3, S2 = (t.requires_grad_() if t is not None else None for t in _weights64(inp, shared=True))
        shared = [S1, S3, S2]
        for s in range(wl.n_shared):
            y = y + _dense_expert(wl, S1, S3, S2, None, None, s, X)
    counts = np.bincount(idx.reshape(-1), minlength=N)
    f = torch.from_numpy(counts / (T * k))
    l_aux = wl.aux_alpha * N * (f * p.mean(0)).sum()
    z = torch.logsumexp(l, dim=1).mean() ** 2
    loss = (y * torch.from_numpy(dy)).sum() + c_aux * l_aux + c_z * z
    loss.backward()
    out = {"dx": X.grad, "dWr": Wr.grad, "dbr": br.grad if br is not None else None, "dW1": W1.grad,
           "dW3": W3.grad if W3 is not None else None, "dW2": W2.grad, "db1": b1.grad if b1 is not None else None,
           "db2": b2.grad if b2 is not None else None}
    if shared:
        out.update(dsW1=shared[0].grad, dsW3=shared[1].grad if shared[1] is not None else None, dsW2=shared[2].grad)
    return {k2: (v.numpy() if v is not None else None) for k2, v in out.items()}


CASES = [
    dict(act=gen.GELU, gating=gen.SOFTMAX_TOPK_RENORM, cf=1.0, N=8, k=2),
    dict(act=gen.SWIGLU, gating=gen.TOPK_SOFTMAX, cf=None, N=6, k=2, n_shared=1, act_dtype=gen.BF16,
         w_dtype=gen.BF16),
    dict(act=gen.SWIGLU, gating=gen.SOFTMAX_TOPK, cf=0.75, N=8, k=3, zipf=1.0, act_dtype=gen.BF16,
         w_dtype=gen.BF16),
    dict(act=gen.GELU, gating=gen.SOFTMAX_TOPK, cf=None, N=4, k=1, zipf=1.2),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("c_aux,c_z", [(0.0, 0.0), (1.0, 0.1)])
def test_backward_against_torch_autograd(case, c_aux, c_z):
    case = dict(case)
    cf = case.pop("cf")
    wl = _tiny(T=40, d=32, d_ff=48, cf=cf, **case)
    inp = _with_random_biases(gen.make_inputs(wl, seed=21))
    dy = gen.normal(97, (wl.T, wl.d), 1.0, gen.F32, seed=3).astype(np.float64)
    if wl.act_dtype == gen.BF16:
        dy_in = gen.normal(97, (wl.T, wl.d), 1.0, gen.BF16, seed=3)
        dy = gen.bf16_to_f32(dy_in).astype(np.float64)
    else:
        dy_in = dy.astype(np.float32)
    got = oracle.backward(inp, dy_in, c_aux, c_z)
    ref = _autograd_layer(inp, dy, c_aux, c_z)
    for name, r in ref.items():
        g = getattr(got, name)
        if r is None:
            continue
        assert g is not None, name
        scale = max(np.abs(r).max(), 1e-30)
        assert np.allclose(g, r, rtol=0, atol=1e-11 * scale), (name, np.abs(g - r).max(), scale)
    if cf is not None and cf < 1:
        # drops happened: dropped pairs carry no gradient into their expert
        assert (_dispatch_by_stable_sort(_lexsort_topk(oracle.router_logits(oracle.shape_of(wl), inp.x, inp)[1],
                                                       wl.top_k), wl.n_experts, wl.capacity())[4]) > 0


def test_backward_linear_in_dy():
    """The gradient is linear in dy when the loss coefficients are zero."""
    wl = _tiny(gen.SWIGLU, gen.TOPK_SOFTMAX, T=24, d=32, d_ff=48, N=4, k=2)
    inp = gen.make_inputs(wl, seed=5)
    # on a 1/16 grid, so that a + 2 b is exact in fp32
    a = (np.round(gen.normal(90, (wl.T, wl.d), 1.0, gen.F32, seed=1) * 16) / 16).astype(np.float32)
    b = (np.round(gen.normal(91, (wl.T, wl.d), 1.0, gen.F32, seed=1) * 16) / 16).astype(np.float32)
    ga, gb = oracle.backward(inp, a), oracle.backward(inp, b)
    ab = (a.astype(np.float64) + 2 * b.astype(np.float64)).astype(np.float32)
    assert np.array_equal(ab.astype(np.float64), a.astype(np.float64) + 2 * b.astype(np.float64))
    gab = oracle.backward(inp, ab)
    for name in ("dx", "dWr", "dW1", "dW3", "dW2"):
        lhs = getattr(gab, name)
        rhs = getattr(ga, name) + 2 * getattr(gb, name)
        assert np.allclose(lhs, rhs, rtol=0, atol=1e-9 * np.abs(rhs).max()), name


@pytest.mark.parametrize("case", CASES)
def test_sampled_backward_equals_the_full_one(case):
    """backward_sampled's dx rows and dW1 / dW3 rows and dW2 columns are the
    matching entries of the full backward (itself pinned to autograd above)."""
    case = dict(case)
    cf = case.pop("cf")
    wl = _tiny(T=40, d=32, d_ff=48, cf=cf, **case)
    inp = _with_random_biases(gen.make_inputs(wl, seed=21))
    if wl.act_dtype == gen.BF16:
        dy = gen.normal(97, (wl.T, wl.d), 1.0, gen.BF16, seed=3)
    else:
        dy = gen.normal(97, (wl.T, wl.d), 1.0, gen.F32, seed=3)
    full = oracle.backward(inp, dy, 1.0, 0.1)
    tokens = [0, 7, 19, wl.T - 1]
    units = [(0, 0), (1, 5), (wl.n_experts - 1, wl.d_ff - 1), (wl.n_experts // 2, 17)]
    dx, d1, d3, d2 = oracle.backward_sampled(inp, dy, tokens, units, 1.0, 0.1)
    scale = np.abs(full.dx).max()
    assert np.allclose(dx, full.dx[tokens], rtol=0, atol=1e-12 * scale)
    for b, (e, i) in enumerate(units):
        assert np.allclose(d1[b], full.dW1[e, i], rtol=0, atol=1e-12 * np.abs(full.dW1).max()), (e, i)
        assert np.allclose(d2[b], full.dW2[e, :, i], rtol=0, atol=1e-12 * np.abs(full.dW2).max()), (e, i)
        if full.dW3 is not None:
            assert np.allclose(d3[b], full.dW3[e, i], rtol=0, atol=1e-12 * np.abs(full.dW3).max()), (e, i)
