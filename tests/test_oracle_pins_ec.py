"""Pins for the oracle's expert-choice routing (each expert takes the C tokens
of largest column-softmax probability). Every check ties the oracle to
something other than itself: brute force over token subsets, library softmax,
closed forms of additive logits, invariants of the row layout, and a dense
evaluation of every expert masked afterwards. A slip such as a softmax over
the wrong axis, ties broken toward the higher token, an off-by-one in C, a
gate taken from the wrong column or rows laid out out of order fails one of
them. CPU only."""
import itertools

import numpy as np
import pytest
import scipy.special as sps
import torch
import torch.nn.functional as F

import gen
import oracle
from test_oracle_pins import _dense_expert, _t64, _weights64, _with_random_biases


def _ec(act=gen.GELU, T=24, d=32, d_ff=48, N=4, cf=1.5, act_dtype=gen.F32, w_dtype=gen.F32, n_shared=0,
        zipf=None):
    return gen.Workload("tiny-ec", T, d, d_ff, N, 1, act, gen.EXPERT_CHOICE, act_dtype, w_dtype, cf,
                        n_shared=n_shared, zipf_s=zipf)


def _shape(T, N, C):
    return oracle.shape_of(_ec(T=T, N=N, cf=1.0), capacity=C)


def _subset_topc(col, C):
    """Brute force: over all C-subsets of tokens (generated in lexicographic
    order), the first with the largest sum of logits. Any strictly increasing
    map of the logits (the column softmax is one) has the same maximisers, and
    the lexicographically first of them keeps the lower token on a tie."""
    best, best_sum = None, None
    for sub in itertools.combinations(range(len(col)), C):
        s = sum(float(col[t]) for t in sub)  # exact: the logits sit on a coarse binary grid
        if best_sum is None or s > best_sum:
            best, best_sum = sub, s
    return np.array(best if best is not None else (), np.int32)


@pytest.mark.parametrize("seed", [1, 2, 3])
@pytest.mark.parametrize("C", [0, 1, 3, 5, 8])
def test_ec_selection_is_brute_force_best_subset(seed, C):
    T, N = 8, 3
    l32 = gen.given_logits(T, N, seed=seed, step=0.5)  # many exact ties inside a column
    r = oracle.route_ec(_shape(T, N, C), l32)
    assert r.ec_token.shape == (N, C)
    for e in range(N):
        assert np.array_equal(r.ec_token[e], _subset_topc(l32[:, e], C)), (e, l32[:, e])


def test_ec_ties_prefer_lower_tokens():
    T, N, C = 10, 2, 4
    l32 = np.zeros((T, N), np.float32)  # expert 0: all equal; expert 1: two groups of ties
    l32[:, 1] = [1, 0, 1, 0, 1, 0, 1, 1, 0, 1]
    r = oracle.route_ec(_shape(T, N, C), l32)
    assert r.ec_token[0].tolist() == [0, 1, 2, 3]
    assert r.ec_token[1].tolist() == [0, 2, 4, 6]
    assert np.allclose(r.ec_gate[0], 1.0 / T, rtol=1e-15, atol=0)


def test_ec_gates_are_the_column_softmax():
    T, N, C = 96, 8, 20
    l32 = gen.given_logits(T, N, seed=7, step=None)
    r = oracle.route_ec(_shape(T, N, C), l32)
    p_lib = sps.softmax(l32.astype(np.float64), axis=0)
    assert np.allclose(r.probs, p_lib, rtol=1e-14, atol=0)
    assert np.allclose(r.probs.sum(0), 1.0, rtol=0, atol=1e-14)
    for e in range(N):
        assert np.allclose(r.ec_gate[e], p_lib[r.ec_token[e], e], rtol=1e-14, atol=0)
        assert np.all(np.diff(r.ec_token[e]) > 0)
        # the taken tokens hold the C largest probabilities of the column
        assert r.ec_gate[e].min() >= np.sort(p_lib[:, e])[::-1][C - 1]
    # z statistics use the per-token logsumexp over the experts, as in token choice
    lse = sps.logsumexp(l32.astype(np.float64), axis=1)
    assert np.allclose(r.lse, lse, rtol=1e-14, atol=0)
    assert np.isclose(r.z, lse.mean() ** 2, rtol=1e-13) and np.isclose(r.lse_sq_mean, (lse ** 2).mean(), rtol=1e-13)


def test_ec_additive_logits_closed_form():
    """l[t][e] = a_t + b_e: every column ranks the tokens by a_t, so all experts
    take the same C tokens, and p[t][e] = exp(a_t) / sum exp(a) whatever b is.
    A softmax over experts instead of tokens gives p = softmax(b) and fails."""
    T, N, C = 40, 5, 7
    a = np.round(gen.normal(gen.T_LOGITS, (T,), 1.0, gen.F32, seed=21).astype(np.float64) * 8) / 8
    b = np.array([0.0, 3.0, -2.5, 1.25, 7.0])
    l32 = (a[:, None] + b[None, :]).astype(np.float32)
    assert np.array_equal(l32.astype(np.float64), a[:, None] + b[None, :])  # exact in fp32
    r = oracle.route_ec(_shape(T, N, C), l32)
    want = np.sort(sorted(range(T), key=lambda t: (-a[t], t))[:C]).astype(np.int32)
    pa = np.exp(a - a.max()) / np.exp(a - a.max()).sum()
    for e in range(N):
        assert np.array_equal(r.ec_token[e], want)
        assert np.allclose(r.ec_gate[e], pa[want], rtol=1e-13, atol=0)


def test_ec_dispatch_layout_invariants():
    T, N, C = 60, 6, 13
    l32 = gen.given_logits(T, N, seed=9, step=0.25)
    s = _shape(T, N, C)
    r = oracle.route_ec(s, l32)
    dsp = oracle.dispatch_ec(s, r.ec_token)
    assert dsp.offsets.tolist() == [e * C for e in range(N + 1)]
    assert np.array_equal(dsp.perm_token, r.ec_token.reshape(-1))
    taken = np.zeros(T, bool)
    for t in range(T):
        for e in range(N):
            row = dsp.inv_map[t, e]
            if row >= 0:
                assert e * C <= row < (e + 1) * C and dsp.perm_token[row] == t
                taken[t] = True
            else:
                assert t not in r.ec_token[e]
    assert (dsp.inv_map >= 0).sum() == N * C
    assert dsp.n_dropped == int((~taken).sum())
    bad = r.ec_token.copy()
    bad[0, :2] = bad[0, 1], bad[0, 0]  # not ascending: outside the contract
    with pytest.raises(ValueError):
        oracle.dispatch_ec(s, bad)


def _brute_force_ec(inp, C):
    """torch fp64 evaluation: logits, softmax over tokens, each expert on EVERY
    token, then the mask of the brute-force top-C sets times the gates."""
    wl = inp.wl
    T, N = wl.T, wl.n_experts
    X = _t64(inp.x, wl.act_dtype)
    l = F.linear(X, _t64(inp.w_router, wl.act_dtype))
    if inp.b_router is not None:
        l = l + torch.from_numpy(inp.b_router).double()
    l32 = l.numpy().astype(np.float32).astype(np.float64)
    p = sps.softmax(l32, axis=0)
    mask = np.zeros((T, N))
    for e in range(N):
        top = sorted(range(T), key=lambda t: (-l32[t, e], t))[:C]
        mask[top, e] = p[top, e]
    W1, W3, W2 = _weights64(inp)
    b1 = None if inp.b1 is None else torch.from_numpy(inp.b1).double()
    b2 = None if inp.b2 is None else torch.from_numpy(inp.b2).double()
    dense = torch.stack([_dense_expert(wl, W1, W3, W2, b1, b2, e, X) for e in range(N)], 1).numpy()
    y = np.einsum("tn,tnd->td", mask, dense)
    if wl.n_shared:
        S1, S3, S2 = _weights64(inp, shared=True)
        for s in range(wl.n_shared):
            y = y + _dense_expert(wl, S1, S3, S2, None, None, s, X).numpy()
    return y, mask


@pytest.mark.parametrize("case", [
    dict(act=gen.GELU, cf=1.5),
    dict(act=gen.GELU, cf=0.5, zipf=1.0),
    dict(act=gen.SWIGLU, cf=2.0, N=6, n_shared=1, act_dtype=gen.BF16, w_dtype=gen.BF16),
    dict(act=gen.SWIGLU, cf=1.0, N=8, act_dtype=gen.BF16, w_dtype=gen.E4M3),
])
def test_ec_layer_output_brute_force_dense_then_mask(case):
    wl = _ec(**case)
    inp = _with_random_biases(gen.make_inputs(wl, seed=17))
    fw = oracle.forward(inp)
    y_ref, mask = _brute_force_ec(inp, wl.capacity())
    assert wl.capacity() == int(wl.T * case["cf"] / wl.n_experts)
    got_mask = np.zeros_like(mask)
    for e in range(wl.n_experts):
        got_mask[fw.routing.ec_token[e], e] = fw.routing.ec_gate[e]
    assert np.allclose(got_mask, mask, rtol=1e-13, atol=0)
    assert np.allclose(fw.y, y_ref, rtol=0, atol=1e-12 * np.abs(y_ref).max())


def test_ec_bias_per_expert_does_not_change_routing():
    """A per-expert logit bias shifts a whole column, which the softmax over
    tokens cancels: same tokens, same gates."""
    T, N, C = 32, 4, 8
    l32 = gen.given_logits(T, N, seed=3, step=1.0 / 64)
    bias = np.array([0.0, 1.0, -2.0, 4.0])
    shifted = (l32.astype(np.float64) + bias).astype(np.float32)
    assert np.array_equal(shifted.astype(np.float64) - l32, np.tile(bias, (T, 1)))  # exact on the grid
    r0 = oracle.route_ec(_shape(T, N, C), l32)
    r1 = oracle.route_ec(_shape(T, N, C), shifted)
    assert np.array_equal(r0.ec_token, r1.ec_token)
    assert np.allclose(r0.ec_gate, r1.ec_gate, rtol=1e-13, atol=0)


def test_ec_degenerate_capacity_zero_and_all_tokens():
    wl = _ec(act=gen.SWIGLU, T=20, N=4, cf=1.0, n_shared=1, act_dtype=gen.BF16, w_dtype=gen.BF16)
    inp = gen.make_inputs(wl, seed=4)
    tok = np.arange(wl.T)
    _, l32 = oracle.router_logits(oracle.shape_of(wl), inp.x, inp)
    s0 = oracle.shape_of(wl, capacity=0)
    r0 = oracle.route_ec(s0, l32)
    assert oracle.dispatch_ec(s0, r0.ec_token).n_dropped == wl.T
    shared_only = oracle.expert_rows(s0, inp, 0, inp.x, shared=True)
    assert np.allclose(oracle.moe_output_ec(s0, inp.x, inp, r0, tok), shared_only, rtol=0,
                       atol=1e-13 * np.abs(shared_only).max())
    # C = T: every expert takes every token -> the dense mixture weighted by the column softmax
    sT = oracle.shape_of(wl, capacity=wl.T)
    rT = oracle.route_ec(sT, l32)
    assert np.array_equal(rT.ec_token, np.tile(np.arange(wl.T, dtype=np.int32), (wl.n_experts, 1)))
    X = _t64(inp.x, wl.act_dtype)
    W1, W3, W2 = _weights64(inp)
    p = sps.softmax(l32.astype(np.float64), axis=0)
    ref = sum(p[:, e:e + 1] * _dense_expert(wl, W1, W3, W2, None, None, e, X).numpy() for e in range(4))
    ref = ref + shared_only
    assert np.allclose(oracle.moe_output_ec(sT, inp.x, inp, rT, tok), ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_ec_identical_experts_scale_one_ffn():
    """All experts equal: y_t = (sum of t's gates) * E(x_t)."""
    wl = _ec(act=gen.GELU, T=30, N=5, cf=2.0)
    inp = _with_random_biases(gen.make_inputs(wl, seed=6))
    for a in (inp.w1, inp.w2, inp.b1, inp.b2):
        a[:] = a[0]
    fw = oracle.forward(inp)
    W1, _, W2 = _weights64(inp)
    X = _t64(inp.x, wl.act_dtype)
    one = F.linear(F.gelu(F.linear(X, W1[0], torch.from_numpy(inp.b1[0]).double())),
                   W2[0], torch.from_numpy(inp.b2[0]).double()).numpy()
    gsum = np.zeros(wl.T)
    for e in range(wl.n_experts):
        np.add.at(gsum, fw.routing.ec_token[e], fw.routing.ec_gate[e])
    ref = gsum[:, None] * one
    assert np.allclose(fw.y, ref, rtol=0, atol=1e-12 * np.abs(ref).max())
    assert (gsum == 0).any()  # some token was taken by no expert and gets zero


def test_ec_combine_against_numpy_gather():
    T, N, C, d, S = 40, 6, 9, 24, 2
    wl = _ec(act=gen.SWIGLU, T=T, N=N, d=d, cf=1.0, n_shared=S, act_dtype=gen.BF16, w_dtype=gen.BF16)
    shape = oracle.shape_of(wl, capacity=C)
    l32 = gen.given_logits(T, N, seed=8, step=None)
    r = oracle.route_ec(shape, l32)
    dsp = oracle.dispatch_ec(shape, r.ec_token)
    yp = gen.normal(99, (N * C, d), 1.0, gen.BF16, seed=2)
    ysh = gen.normal(98, (S, T, d), 1.0, gen.BF16, seed=2)
    g32 = r.ec_gate.reshape(-1).astype(np.float32)
    got = oracle.combine_ec(shape, yp, dsp.inv_map, g32, ysh)
    ypf = gen.bf16_to_f32(yp).astype(np.float64)
    ref = gen.bf16_to_f32(ysh).astype(np.float64).sum(0)
    for e in range(N):
        for j in range(C):
            ref[r.ec_token[e, j]] += float(g32[e * C + j]) * ypf[e * C + j]
    assert np.allclose(got, ref, rtol=0, atol=1e-13 * np.abs(ref).max())
