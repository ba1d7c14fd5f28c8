"""Pins for the CPU oracle: each check ties it to something other than itself
(library routines, brute force, closed forms, invariants, the pages' printed
numbers). A plausible slip in the oracle -- a dropped bias, a wrong gate mode,
a transposed weight, an off-by-one in the capacity cut, a tie broken the wrong
way -- fails at least one of these. CPU only."""
import math

import numpy as np
import pytest
import scipy.special as sps
import torch
import torch.nn.functional as F

import gen
import oracle


def _t64(a, dtype):
    """Decode a host buffer to torch float64 with torch's own conversions."""
    if dtype == gen.F32:
        return torch.from_numpy(np.asarray(a, np.float32)).double()
    if dtype == gen.BF16:
        return torch.from_numpy(np.asarray(a, np.uint16).view(np.int16)).view(torch.bfloat16).double()
    return torch.from_numpy(np.asarray(a, np.uint8)).view(torch.float8_e4m3fn).double()


def _weights64(inp, shared=False):
    wl = inp.wl
    if shared:
        w1, w3, w2, sc = inp.sw1, inp.sw3, inp.sw2, inp.sw_scale
    else:
        w1, w3, w2, sc = inp.w1, inp.w3, inp.w2, inp.w_scale
    if wl.w_dtype == gen.INT_W:
        # codes times one fp32 scale per weight row: W1 rows, W3 rows, W2 rows
        f = wl.d_ff
        s = torch.from_numpy(sc.astype(np.float64))
        W1 = torch.from_numpy(w1.astype(np.float64)) * s[:, :f, None]
        W3 = torch.from_numpy(w3.astype(np.float64)) * s[:, f:2 * f, None] if w3 is not None else None
        W2 = torch.from_numpy(w2.astype(np.float64)) * s[:, 2 * f:, None]
        return W1, W3, W2
    W1, W2 = _t64(w1, wl.w_dtype), _t64(w2, wl.w_dtype)
    W3 = _t64(w3, wl.w_dtype) if w3 is not None else None
    if wl.w_dtype == gen.E4M3:
        s = torch.from_numpy(sc.astype(np.float64))
        W1 = W1 * s[:, 0, None, None]
        W2 = W2 * s[:, 2, None, None]
        if W3 is not None:
            W3 = W3 * s[:, 1, None, None]
    return W1, W3, W2


def _dense_expert(wl, W1, W3, W2, b1, b2, e, X):
    """torch fp64 library evaluation of one expert on rows X."""
    if wl.act == gen.GELU:
        h = F.gelu(F.linear(X, W1[e], None if b1 is None else b1[e]), approximate="none")
        return F.linear(h, W2[e], None if b2 is None else b2[e])
    return F.linear(F.silu(F.linear(X, W1[e])) * F.linear(X, W3[e]), W2[e])


def _tiny(act, gating, w_dtype=gen.F32, act_dtype=gen.F32, T=48, d=32, d_ff=64, N=8, k=2, cf=None,
          n_shared=0, zipf=None, n_int8=None):
    return gen.Workload("tiny", T, d, d_ff, N, k, act, gating, act_dtype, w_dtype, cf, n_shared=n_shared,
                        zipf_s=zipf, n_int8=N // 3 if n_int8 is None else n_int8)


def _with_random_biases(inp, seed=5):
    rng = np.random.default_rng(seed)
    if inp.b1 is not None:
        inp.b1 = rng.standard_normal(inp.b1.shape).astype(np.float32)
        inp.b2 = rng.standard_normal(inp.b2.shape).astype(np.float32)
    return inp


# ---------------------------------------------------------------- decoders / activations

def test_bf16_decode_matches_torch():
    codes = np.arange(0, 1 << 16, 97, dtype=np.uint16)
    codes = codes[(codes & 0x7F80) != 0x7F80]  # finite only
    ref = _t64(codes, gen.BF16).numpy()
    got = np.array([oracle.bf16_value(int(c)) for c in codes])
    assert np.array_equal(ref, got)


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)  # drop the two NaNs
    ref = _t64(codes, gen.E4M3).numpy()
    got = np.array([oracle.e4m3_value(int(c)) for c in codes])
    assert np.array_equal(ref, got)
    assert oracle.e4m3_value(0x7E) == 448.0 and oracle.e4m3_value(0x01) == 2.0 ** -9


def test_gelu_silu_against_library():
    us = np.linspace(-12, 12, 241)
    g = np.array([oracle.gelu(u) for u in us])
    s = np.array([oracle.silu(u) for u in us])
    tu = torch.from_numpy(us)
    assert np.allclose(g, F.gelu(tu, approximate="none").numpy(), rtol=1e-14, atol=1e-15)
    assert np.allclose(s, F.silu(tu).numpy(), rtol=1e-14, atol=1e-15)
    assert oracle.gelu(0.0) == 0.0 and abs(oracle.gelu(40.0) - 40.0) < 1e-12


# ---------------------------------------------------------------- routing

def _lexsort_topk(l, k):
    """Brute force: sort by (-logit, expert) and take k."""
    T, N = l.shape
    out = np.empty((T, k), np.int32)
    for t in range(T):
        order = sorted(range(N), key=lambda e: (-float(l[t, e]), e))
        out[t] = order[:k]
    return out


@pytest.mark.parametrize("N,k", [(8, 2), (64, 1), (160, 6), (8, 8), (5, 3)])
def test_selection_is_brute_force_topk_with_lower_index_ties(N, k):
    T = 200
    l32 = gen.given_logits(T, N, seed=11, step=0.5)  # coarse grid: many exact ties
    wl = _tiny(gen.GELU, gen.SOFTMAX_TOPK, T=T, N=N, k=k)
    r = oracle.route(oracle.shape_of(wl), l32)
    assert np.array_equal(r.topk_idx, _lexsort_topk(l32, k))
    assert any(len(set(row)) < N for row in l32)  # ties were present


def test_gates_softmax_modes_and_library_softmax():
    T, N, k = 64, 8, 2
    l32 = gen.given_logits(T, N, seed=3, step=None)
    p_lib = sps.softmax(l32.astype(np.float64), axis=1)
    wl = _tiny(gen.GELU, gen.SOFTMAX_TOPK, T=T, N=N, k=k)
    r0 = oracle.route(oracle.shape_of(wl), l32)
    r1 = oracle.route(oracle.shape_of(wl.with_(gating=gen.SOFTMAX_TOPK_RENORM)), l32)
    r2 = oracle.route(oracle.shape_of(wl.with_(gating=gen.TOPK_SOFTMAX)), l32)
    sel = np.take_along_axis(p_lib, r0.topk_idx.astype(np.int64), 1)
    assert np.allclose(r0.topk_w, sel, rtol=1e-14)
    assert np.allclose(r0.probs, p_lib, rtol=1e-13)
    assert np.allclose(r1.topk_w.sum(1), 1.0, atol=1e-15)
    assert np.allclose(r1.topk_w, r2.topk_w, atol=1e-15)  # the two renormalised orders agree
    sub = np.take_along_axis(l32.astype(np.float64), r0.topk_idx.astype(np.int64), 1)
    assert np.allclose(r2.topk_w, sps.softmax(sub, axis=1), rtol=1e-14)
    assert np.allclose(r0.lse, sps.logsumexp(l32.astype(np.float64), axis=1), rtol=1e-14)
    assert np.all(np.diff(sub, axis=1) <= 0)  # slots in descending logit order


def test_k_equals_n_renorm_gates_are_the_full_softmax():
    T, N = 40, 6
    l32 = gen.given_logits(T, N, seed=4, step=None)
    wl = _tiny(gen.GELU, gen.SOFTMAX_TOPK_RENORM, T=T, N=N, k=N)
    r = oracle.route(oracle.shape_of(wl), l32)
    p = sps.softmax(l32.astype(np.float64), axis=1)
    assert np.allclose(r.topk_w, np.take_along_axis(p, r.topk_idx.astype(np.int64), 1), rtol=1e-14)
    assert np.all(np.isinf(r.margin_set))


def test_top1_renorm_gate_is_one():
    T, N = 40, 16
    l32 = gen.given_logits(T, N, seed=6, step=None)
    for mode in (gen.SOFTMAX_TOPK_RENORM, gen.TOPK_SOFTMAX):
        r = oracle.route(oracle.shape_of(_tiny(gen.GELU, mode, T=T, N=N, k=1)), l32)
        assert np.array_equal(r.topk_w, np.ones((T, 1)))


@pytest.mark.parametrize("N,k,m", [(8, 2, 5), (64, 1, 3), (160, 6, 2), (7, 3, 4)])
def test_aux_loss_closed_form_alpha_under_uniform_routing(N, k, m):
    """T = m*N tokens; token t puts logit b on experts t..t+k-1 (mod N) and 0
    elsewhere: every expert is chosen m*k times and P_e = 1/N exactly, so
    f_e = P_e = 1/N and L_aux = alpha*N*N*(1/N^2) = alpha."""
    T, b, alpha = m * N, 1.7, 0.01
    l = np.zeros((T, N), np.float32)
    for t in range(T):
        for j in range(k):
            l[t, (t + j) % N] = b
    wl = _tiny(gen.GELU, gen.SOFTMAX_TOPK, T=T, N=N, k=k)
    r = oracle.route(oracle.shape_of(wl), l)
    assert np.allclose(r.f, 1.0 / N, rtol=1e-15)
    assert np.allclose(r.P, 1.0 / N, rtol=1e-13)
    assert abs(r.l_aux - alpha) < 1e-15 * 100
    assert abs(r.f.sum() - 1) < 1e-14 and abs(r.P.sum() - 1) < 1e-13


def test_aux_loss_against_pages_module_form():
    """The aigrafen module computes f as a share of tokens (counts/T, summing to k)
    and omits alpha; ours is alpha * N * sum (f/k) P with f = counts/(T k)."""
    T, N, k = 300, 8, 2
    l32 = gen.given_logits(T, N, seed=8, step=None, bias=gen.zipf_bias(N, 1.0))
    wl = _tiny(gen.GELU, gen.SOFTMAX_TOPK_RENORM, T=T, N=N, k=k)
    r = oracle.route(oracle.shape_of(wl), l32)
    onehot = np.zeros((T, N))
    for t in range(T):
        onehot[t, r.topk_idx[t]] = 1.0
    f_page = onehot.mean(0)                       # share of tokens per expert
    P_page = sps.softmax(l32.astype(np.float64), axis=1).mean(0)
    aux_page = N * (f_page * P_page).sum()
    assert abs(r.l_aux - 0.01 * aux_page / k) < 1e-15
    assert np.array_equal(r.counts, onehot.sum(0).astype(np.int64))


def test_z_loss_closed_forms():
    T, N = 30, 8
    wl = _tiny(gen.GELU, gen.SOFTMAX_TOPK, T=T, N=N, k=2)
    r = oracle.route(oracle.shape_of(wl), np.zeros((T, N), np.float32))
    assert abs(r.z - math.log(N) ** 2) < 1e-14
    c = 2.5
    r = oracle.route(oracle.shape_of(wl), np.full((T, N), c, np.float32))
    assert abs(r.z - (c + math.log(N)) ** 2) < 1e-13
    assert abs(r.lse_sq_mean - (c + math.log(N)) ** 2) < 1e-13
    l32 = gen.given_logits(T, N, seed=1, step=None)
    r = oracle.route(oracle.shape_of(wl), l32)
    lse = sps.logsumexp(l32.astype(np.float64), axis=1)
    assert abs(r.z - lse.mean() ** 2) < 1e-13 and abs(r.lse_sq_mean - (lse ** 2).mean()) < 1e-13


# ---------------------------------------------------------------- dispatch

def _dispatch_by_stable_sort(topk_idx, N, C):
    """Second formulation: a stable sort of the (token, slot) pairs by expert."""
    T, k = topk_idx.shape
    flat = topk_idx.reshape(-1).astype(np.int64)
    order = np.argsort(flat, kind="stable")           # expert-major, token order kept
    counts = np.bincount(flat, minlength=N)
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
    rank = np.empty(T * k, np.int64)
    rank[order] = np.arange(T * k) - starts[flat[order]]
    keep = rank < (C if C >= 0 else T * k + 1)
    kept = np.bincount(flat[keep], minlength=N)
    offsets = np.concatenate([[0], np.cumsum(kept)])
    inv = np.where(keep, offsets[flat] + rank, -1)
    perm = np.full(T * k, -1, np.int64)
    perm[inv[keep]] = np.nonzero(keep)[0] // k
    return kept, offsets, perm, inv.reshape(T, k), int((~keep).sum())


@pytest.mark.parametrize("N,k,C,skew", [(8, 2, 80, None), (8, 2, 7, 1.0), (64, 1, 20, 1.2),
                                         (160, 6, 3, 1.0), (8, 2, -1, 1.0), (8, 2, 0, None),
                                         (6, 6, 4, None)])
def test_dispatch_matches_stable_sort_and_invariants(N, k, C, skew):
    T = 256
    bias = None if skew is None else gen.zipf_bias(N, skew)
    l32 = gen.given_logits(T, N, seed=21, step=0.25, bias=bias)
    wl = _tiny(gen.GELU, gen.SOFTMAX_TOPK, T=T, N=N, k=k)
    shape = oracle.shape_of(wl, capacity=C)
    r = oracle.route(shape, l32)
    d = oracle.dispatch(shape, r.topk_idx)
    kept, offsets, perm, inv, nd = _dispatch_by_stable_sort(r.topk_idx, N, C)
    assert np.array_equal(d.kept, kept) and np.array_equal(d.offsets, offsets)
    assert np.array_equal(d.perm_token, perm) and np.array_equal(d.inv_map, inv) and d.n_dropped == nd
    if C >= 0:
        assert (d.kept <= C).all()
    assert d.kept.sum() == T * k - d.n_dropped
    for e in range(N):  # each expert's kept set is the token-order prefix of its list
        toks = [t for t in range(T) if e in r.topk_idx[t]]
        rows = d.perm_token[d.offsets[e]:d.offsets[e + 1]]
        assert list(rows) == toks[:len(rows)]
    if C == 0:
        assert d.offsets[-1] == 0 and (d.inv_map == -1).all()


def test_capacity_formula_matches_pages_examples():
    assert gen.TINY_GELU.capacity() == 80       # int(1.25 * 256 * 2 / 8)
    assert gen.SWITCH_TOP1.capacity() == 320    # int(1.25 * 16384 * 1 / 64)
    assert gen.MIXTRAL_PREFILL.capacity() == -1


# ---------------------------------------------------------------- experts and the layer output

@pytest.mark.parametrize("act,w_dtype,act_dtype", [(gen.GELU, gen.F32, gen.F32), (gen.SWIGLU, gen.BF16, gen.BF16),
                                                   (gen.GELU, gen.E4M3, gen.BF16), (gen.SWIGLU, gen.E4M3, gen.BF16),
                                                   (gen.SWIGLU, gen.F32, gen.F32), (gen.SWIGLU, gen.INT_W, gen.BF16),
                                                   (gen.GELU, gen.INT_W, gen.BF16)])
def test_expert_rows_against_torch_fp64(act, w_dtype, act_dtype):
    wl = _tiny(act, gen.SOFTMAX_TOPK, w_dtype=w_dtype, act_dtype=act_dtype, T=24, d=48, d_ff=80, N=3, k=1)
    inp = _with_random_biases(gen.make_inputs(wl, seed=9))
    shape = oracle.shape_of(wl)
    W1, W3, W2 = _weights64(inp)
    b1 = None if inp.b1 is None else torch.from_numpy(inp.b1).double()
    b2 = None if inp.b2 is None else torch.from_numpy(inp.b2).double()
    X = _t64(inp.x, act_dtype)
    for e in range(wl.n_experts):
        got = oracle.expert_rows(shape, inp, e, inp.x)
        ref = _dense_expert(wl, W1, W3, W2, b1, b2, e, X).numpy()
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def _brute_force_layer(inp, C, gating):
    """Evaluate every expert on every token (torch fp64), then mask to the kept
    top-k with the gates, plus shared experts. Routing/drops are recomputed here
    with numpy/scipy from the fp32 router output."""
    wl = inp.wl
    T, N, k = wl.T, wl.n_experts, wl.top_k
    X = _t64(inp.x, wl.act_dtype)
    Wr = _t64(inp.w_router, wl.act_dtype)
    l = F.linear(X, Wr)
    if inp.b_router is not None:
        l = l + torch.from_numpy(inp.b_router).double()
    l32 = l.numpy().astype(np.float32).astype(np.float64)
    p = sps.softmax(l32, axis=1)
    idx = _lexsort_topk(l32, k)
    g = np.take_along_axis(p, idx.astype(np.int64), 1)
    if gating != gen.SOFTMAX_TOPK:
        g = g / g.sum(1, keepdims=True)
    _, _, _, inv, _ = _dispatch_by_stable_sort(idx, N, C)
    W1, W3, W2 = _weights64(inp)
    b1 = None if inp.b1 is None else torch.from_numpy(inp.b1).double()
    b2 = None if inp.b2 is None else torch.from_numpy(inp.b2).double()
    dense = torch.stack([_dense_expert(wl, W1, W3, W2, b1, b2, e, X) for e in range(N)], 1).numpy()  # [T,N,d]
    mask = np.zeros((T, N))
    for t in range(T):
        for j in range(k):
            if inv[t, j] >= 0:
                mask[t, idx[t, j]] = g[t, j]
    y = np.einsum("tn,tnd->td", mask, dense)
    if wl.n_shared:
        S1, S3, S2 = _weights64(inp, shared=True)
        for s in range(wl.n_shared):
            y = y + _dense_expert(wl, S1, S3, S2, None, None, s, X).numpy()
    return y, idx, inv


@pytest.mark.parametrize("case", [
    dict(act=gen.GELU, gating=gen.SOFTMAX_TOPK_RENORM, cf=1.25, N=8, k=2),
    dict(act=gen.GELU, gating=gen.SOFTMAX_TOPK_RENORM, cf=0.5, N=8, k=2, zipf=1.0),
    dict(act=gen.SWIGLU, gating=gen.TOPK_SOFTMAX, cf=None, N=8, k=2),
    dict(act=gen.SWIGLU, gating=gen.SOFTMAX_TOPK, cf=None, N=16, k=6, n_shared=2, zipf=1.0,
         act_dtype=gen.BF16, w_dtype=gen.BF16),
    dict(act=gen.GELU, gating=gen.SOFTMAX_TOPK, cf=1.25, N=8, k=1, zipf=1.2, act_dtype=gen.BF16,
         w_dtype=gen.E4M3),
    dict(act=gen.SWIGLU, gating=gen.TOPK_SOFTMAX, cf=None, N=8, k=2, n_shared=1, act_dtype=gen.BF16,
         w_dtype=gen.INT_W),
])
def test_layer_output_brute_force_dense_then_mask(case):
    case = dict(case)
    cf = case.pop("cf")
    wl = _tiny(T=64, d=32, d_ff=64, cf=cf, **case)
    inp = _with_random_biases(gen.make_inputs(wl, seed=13))
    fw = oracle.forward(inp)
    y_ref, idx, inv = _brute_force_layer(inp, wl.capacity(), wl.gating)
    assert np.array_equal(fw.routing.topk_idx, idx)
    assert np.array_equal(fw.disp.inv_map, inv)
    assert np.allclose(fw.y, y_ref, rtol=0, atol=1e-12 * np.abs(y_ref).max())
    if cf == 0.5:
        assert fw.disp.n_dropped > 0


def test_degenerate_identical_experts_reduce_to_one_ffn():
    """All experts equal, renormalised gates, no drops: y = E(x) (a plain FFN)."""
    wl = _tiny(gen.GELU, gen.SOFTMAX_TOPK_RENORM, T=40, d=32, d_ff=48, N=6, k=3, cf=None)
    inp = _with_random_biases(gen.make_inputs(wl, seed=2))
    for a in (inp.w1, inp.w2, inp.b1, inp.b2):
        a[:] = a[0]
    fw = oracle.forward(inp)
    W1, _, W2 = _weights64(inp)
    X = _t64(inp.x, wl.act_dtype)
    ref = F.linear(F.gelu(F.linear(X, W1[0], torch.from_numpy(inp.b1[0]).double())),
                   W2[0], torch.from_numpy(inp.b2[0]).double()).numpy()
    assert np.allclose(fw.y, ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_degenerate_k_equals_n_is_dense_soft_mixture():
    wl = _tiny(gen.SWIGLU, gen.SOFTMAX_TOPK_RENORM, T=32, d=32, d_ff=48, N=4, k=4, cf=None)
    inp = gen.make_inputs(wl, seed=3)
    fw = oracle.forward(inp)
    X = _t64(inp.x, wl.act_dtype)
    W1, W3, W2 = _weights64(inp)
    p = sps.softmax(fw.logits32.astype(np.float64), axis=1)
    ref = sum(p[:, e:e + 1] * _dense_expert(wl, W1, W3, W2, None, None, e, X).numpy() for e in range(4))
    assert np.allclose(fw.y, ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_degenerate_capacity_zero_and_capacity_at_least_T():
    wl = _tiny(gen.SWIGLU, gen.SOFTMAX_TOPK, T=48, d=32, d_ff=48, N=8, k=2, n_shared=1,
               act_dtype=gen.BF16, w_dtype=gen.BF16, cf=None)
    inp = gen.make_inputs(wl, seed=4)
    shape0 = oracle.shape_of(wl, capacity=0)
    l64, l32 = oracle.router_logits(shape0, inp.x, inp)
    r = oracle.route(shape0, l32)
    d0 = oracle.dispatch(shape0, r.topk_idx)
    tok = np.arange(wl.T)
    y0 = oracle.moe_output(shape0, inp.x, inp, r, d0, tok)
    shared_only = oracle.expert_rows(shape0, inp, 0, inp.x, shared=True)
    assert d0.n_dropped == wl.T * wl.top_k
    assert np.allclose(y0, shared_only, rtol=0, atol=1e-13 * np.abs(shared_only).max())
    shapeT = oracle.shape_of(wl, capacity=wl.T)
    dT = oracle.dispatch(shapeT, r.topk_idx)
    shapeInf = oracle.shape_of(wl, capacity=-1)
    dI = oracle.dispatch(shapeInf, r.topk_idx)
    assert np.array_equal(dT.inv_map, dI.inv_map) and dT.n_dropped == 0
    assert np.array_equal(oracle.moe_output(shapeT, inp.x, inp, r, dT, tok),
                          oracle.moe_output(shapeInf, inp.x, inp, r, dI, tok))


def test_combine_against_numpy_gather():
    wl = _tiny(gen.SWIGLU, gen.SOFTMAX_TOPK, T=50, d=40, N=8, k=3, n_shared=2, act_dtype=gen.BF16,
               w_dtype=gen.BF16, cf=0.6)
    shape = oracle.shape_of(wl)
    l32 = gen.given_logits(wl.T, wl.n_experts, seed=5, step=None)
    r = oracle.route(shape, l32)
    d = oracle.dispatch(shape, r.topk_idx)
    M = int(d.offsets[-1])
    yp = gen.normal(99, (M, wl.d), 1.0, gen.BF16, seed=1)
    ysh = gen.normal(98, (wl.n_shared, wl.T, wl.d), 1.0, gen.BF16, seed=1)
    g32 = r.topk_w.astype(np.float32)
    got = oracle.combine(shape, yp, d.inv_map, g32, ysh)
    ypf = gen.bf16_to_f32(yp).astype(np.float64)
    ref = gen.bf16_to_f32(ysh).astype(np.float64).sum(0)
    for j in range(wl.top_k):
        rows = d.inv_map[:, j]
        ok = rows >= 0
        ref[ok] += g32[ok, j, None].astype(np.float64) * ypf[rows[ok]]
    assert d.n_dropped > 0
    assert np.allclose(got, ref, rtol=0, atol=1e-13 * np.abs(ref).max())


# ---------------------------------------------------------------- the generator

@pytest.mark.parametrize("bits", [8, 4])
def test_int_rows_quantiser(bits):
    """Integer rows against the fp32 draws of the same tensor: symmetric codes
    within +-qmax, each row's largest weight on +-qmax, every weight within half
    a step of its code times the row scale, ties rounded to even."""
    rows, cols, qmax = 40, 96, (1 << (bits - 1)) - 1
    q, s = gen.int_rows(gen.T_W1, (rows, cols), 0.3, bits, seed=4, offset=1000)
    w = gen.normal(gen.T_W1, (rows, cols), 0.3, gen.F32, seed=4, offset=1000).astype(np.float64)
    assert q.dtype == np.int8 and np.abs(q).max() <= qmax
    amax = np.abs(w).max(1)
    assert np.allclose(s, (amax / qmax).astype(np.float32), rtol=0, atol=0)
    assert (np.abs(q).max(1) == qmax).all()
    err = np.abs(w - q.astype(np.float64) * s[:, None].astype(np.float64))
    assert (err <= s[:, None].astype(np.float64) * (0.5 + 1e-9)).all()
    assert np.array_equal(q, np.clip(np.round(w / s[:, None].astype(np.float64)), -qmax, qmax).astype(np.int8))


def test_int_workload_bits_and_scales_layout():
    wl = _tiny(gen.SWIGLU, gen.SOFTMAX_TOPK, w_dtype=gen.INT_W, act_dtype=gen.BF16, d=64, d_ff=96, N=6,
               n_shared=1, n_int8=2)
    inp = gen.make_inputs(wl, seed=3)
    assert inp.w_bits.tolist() == [8, 8, 4, 4, 4, 4] and inp.sw_bits.tolist() == [8]
    assert inp.w_scale.shape == (6, 2 * 96 + 64) and inp.w1.dtype == np.int8
    for e in range(6):
        qmax = 127 if e < 2 else 7
        for m in (inp.w1[e], inp.w3[e], inp.w2[e]):
            assert np.abs(m).max() == qmax
    # W3's scales are those of W3's own rows (tensor id 4), not W1's
    q3, s3 = gen.int_rows(gen.T_W3, (96, 64), 1.0 / 8.0, 8, seed=3, offset=0)
    assert np.array_equal(inp.w3[0], q3) and np.array_equal(inp.w_scale[0, 96:192], s3)


def test_generator_is_counter_based_and_prefix_stable():
    a = gen.normal(gen.T_X, (64, 32), 1.0, gen.BF16)
    b = gen.normal(gen.T_X, (16, 32), 1.0, gen.BF16)
    assert np.array_equal(a[:16], b)
    v = gen.normal(gen.T_X, (200000,), 1.0, gen.F32)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1) < 0.01


def test_generator_roundings_match_torch():
    v = gen.normal(7, (5000,), 3.0, gen.F32, seed=2)
    bf = np.array([gen.lib().gen_bf16_of(float(x)) for x in v], np.uint16)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf, ref)
    w = np.concatenate([np.linspace(-440, 440, 3001), np.linspace(-0.02, 0.02, 2001)])
    q = np.array([gen.lib().gen_e4m3_of(float(x)) for x in w], np.uint8)
    refq = torch.from_numpy(w).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, refq)


def test_router_grid_recipe_keeps_logits_exact():
    """With router_grid inputs every product is exact in fp32 and the sum of
    |products| stays below 2^24 grid units, so any summation order gives the
    same fp32 logits; the fp64 oracle logits are then exact fp32 numbers."""
    wl = gen.SWITCH_TOP1.with_(T=512)
    inp = gen.make_inputs(wl, router_grid=True)
    X = gen.bf16_to_f32(inp.x).astype(np.float64)
    W = gen.bf16_to_f32(inp.w_router).astype(np.float64)
    p = int(math.ceil(math.log2(32.0 * math.sqrt(wl.d))))
    unit = 2.0 ** -(4 + p)
    assert np.all(np.abs(X * 16 - np.round(X * 16)) == 0) and np.abs(X * 16).max() <= 255
    assert np.all(np.abs(W * 2 ** p - np.round(W * 2 ** p)) == 0)
    worst = (np.abs(X) @ np.abs(W).T).max() / unit
    assert worst < 2 ** 24
    l64, l32 = oracle.router_logits(oracle.shape_of(wl), inp.x, inp)
    assert np.array_equal(l64, l32.astype(np.float64))
