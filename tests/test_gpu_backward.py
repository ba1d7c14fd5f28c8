"""Layer backward on the GPU (moe_backward) against the oracle's fp64
backward on the same seeded inputs: dx, the router weight and bias, every
expert's and shared expert's weights, the GELU biases, with and without the
L_aux and z terms, in all three token-choice gate modes, with capacity drops,
skewed routing, empty experts and an all-dropped layer, on both forward-
recompute paths (the backward GEMM below 2048 rows, the forward's grouped FFN
from 2048 rows). Every size spans several tiles with ragged tails.

The gradients are only comparable when both sides route identically, so each
case first checks that the library's selection equals the oracle's (the seeds
give no near ties)."""
import numpy as np
import pytest

import gen
import oracle
import sparse_mixture_experts_36_amd as moe
from helpers import as_f64, dev, device_weights, host, rel_err, say, shape_of

pytestmark = pytest.mark.gpu

# bf16 rounding of H, g dy, dU, dV and dx (2^-9 relative each) in sums of
# hundreds of terms: about 1e-2 of the largest gradient at worst
TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()
    yield
    torch.cuda.synchronize()


def _wl(name, T, d, d_ff, N, k, act, gating, cf=None, n_shared=0, zipf=None):
    return gen.Workload(name, T, d, d_ff, N, k, act, gating, gen.BF16, gen.BF16, cf, n_shared=n_shared,
                        zipf_s=zipf)


CASES = {
    "swiglu-topk-softmax-shared1": _wl("b1", 640, 256, 384, 8, 2, gen.SWIGLU, gen.TOPK_SOFTMAX, n_shared=1),
    "gelu-renorm-cf0.75-biases": _wl("b2", 520, 128, 256, 6, 2, gen.GELU, gen.SOFTMAX_TOPK_RENORM, cf=0.75,
                                     zipf=1.0),
    "swiglu-softmax-topk-k3-cf1.25-shared2": _wl("b3", 300, 384, 256, 8, 3, gen.SWIGLU, gen.SOFTMAX_TOPK, cf=1.25,
                                                 n_shared=2, zipf=1.2),
    "gelu-top1-T1": _wl("b4", 1, 128, 128, 4, 1, gen.GELU, gen.SOFTMAX_TOPK),
    "swiglu-capacity0-shared1": _wl("b5", 64, 128, 128, 8, 1, gen.SWIGLU, gen.TOPK_SOFTMAX, cf=0.01, n_shared=1),
    "mixtral-like-T512": _wl("b6", 512, 1024, 1536, 8, 2, gen.SWIGLU, gen.TOPK_SOFTMAX),
    # 64 experts and two shared ones: 1536 routed + 512 shared rows, 128-row DMA tiles for the recompute
    "fine-grained-like-64x6-shared2": _wl("b7", 256, 256, 256, 64, 6, gen.SWIGLU, gen.SOFTMAX_TOPK, n_shared=2,
                                          zipf=1.0),
    # 2048 rows or more: the forward recompute runs on the forward's grouped
    # FFN: 256-row DMA tiles (SwiGLU with a shared expert; GELU with biases,
    # where three of the four experts end in a short tail on 128-row tiles)
    # and 128-row DMA tiles (GELU, biases and capacity drops)
    "swiglu-ffn-dma256-T2048-shared1": _wl("b8", 2048, 256, 512, 4, 2, gen.SWIGLU, gen.TOPK_SOFTMAX, n_shared=1),
    "gelu-ffn-dma128-renorm-cf1-biases": _wl("b9", 1024, 256, 512, 8, 2, gen.GELU, gen.SOFTMAX_TOPK_RENORM, cf=1.0,
                                             zipf=1.0),
    "gelu-ffn-dma256-tails-biases": _wl("b11", 2048, 256, 512, 4, 2, gen.GELU, gen.SOFTMAX_TOPK, zipf=0.5),
    # skewed groups on 256-row tiles: nine small groups whole on 128-row tiles
    "swiglu-ffn-dma256-small-groups-shared1": _wl("b12", 2048, 512, 512, 12, 2, gen.SWIGLU, gen.SOFTMAX_TOPK,
                                                  n_shared=1, zipf=1.0),
    # widths the 256-wide tiles do not divide: clamped columns in every
    # product, and the recompute on the backward GEMM although rows >= 2048
    "swiglu-d384-dff384-T1024-shared1": _wl("b10", 1024, 384, 384, 4, 2, gen.SWIGLU, gen.TOPK_SOFTMAX, n_shared=1),
}


# the kernel family of each case's forward recompute (moe_ffn_path)
RECOMPUTE_PATH = {
    "fine-grained-like-64x6-shared2": moe.PATH_DMA128,  # 2048 rows with the shared experts' T each
    "swiglu-ffn-dma256-T2048-shared1": moe.PATH_DMA256,
    "gelu-ffn-dma128-renorm-cf1-biases": moe.PATH_DMA128,
    "gelu-ffn-dma256-tails-biases": moe.PATH_DMA256,
    "swiglu-ffn-dma256-small-groups-shared1": moe.PATH_DMA256,
}


def test_backward_cases_reach_their_recompute_paths():
    for name, wl in CASES.items():
        got = moe.ffn_path(shape_of(wl), moe.ENTRY_BACKWARD)
        assert got == RECOMPUTE_PATH.get(name, moe.PATH_BGEMM), (name, got)


def _inputs(wl, seed):
    inp = gen.make_inputs(wl, seed=seed)
    if inp.b1 is not None:  # nonzero GELU biases, so that their paths carry weight
        rng = np.random.default_rng(seed)
        inp.b1 = (0.5 * rng.standard_normal(inp.b1.shape)).astype(np.float32)
        inp.b2 = (0.5 * rng.standard_normal(inp.b2.shape)).astype(np.float32)
    dy = gen.normal(97, (wl.T, wl.d), 1.0, gen.BF16, seed=seed)
    return inp, dy


def _same_routing(inp, t):
    """The library's top-k selection equals the oracle's for every token."""
    import torch
    wl = inp.wl
    s = shape_of(wl)
    logits = torch.empty(wl.T, wl.n_experts, dtype=torch.float32, device="cuda")
    idx = torch.empty(wl.T, wl.top_k, dtype=torch.int32, device="cuda")
    gw = torch.empty(wl.T, wl.top_k, dtype=torch.float32, device="cuda")
    moe.route(s, dev(inp.x), t["w_router"], t["b_router"], logits, idx, gw)
    torch.cuda.synchronize()
    so = oracle.shape_of(wl)
    _, l32 = oracle.router_logits(so, inp.x, inp)
    r = oracle.route(so, l32)
    return np.array_equal(host(idx), r.topk_idx)


def _check(inp, dy, c_aux, c_z, label, pad=0):
    import torch
    wl = inp.wl
    say(f"backward {label}: T={wl.T} d={wl.d} d_ff={wl.d_ff} N={wl.n_experts} k={wl.top_k} C={wl.capacity()} "
        f"shared={wl.n_shared} c_aux={c_aux} c_z={c_z} weight row pad={pad}")
    t = device_weights(inp, pad)
    assert _same_routing(inp, t), "routing differs from the oracle's: pick a seed without near ties"
    s = shape_of(wl)
    g = moe.alloc_grads(s)
    for v in g.values():  # poison: every output must be written
        if v is not None:
            v.fill_(float("nan"))
    moe.backward(s, dev(inp.x), moe.weights_struct(t), dev(dy), g, c_aux, c_z)
    torch.cuda.synchronize()
    ref = oracle.backward(inp, dy, c_aux, c_z)
    names = {"dx": "dx", "dw_router": "dWr", "db_router": "dbr", "dw1": "dW1", "dw3": "dW3", "dw2": "dW2",
             "db1": "db1", "db2": "db2", "dsw1": "dsW1", "dsw3": "dsW3", "dsw2": "dsW2"}
    for key, rn in names.items():
        r = getattr(ref, rn)
        got = g.get(key)
        if r is None:
            assert got is None, key
            continue
        a = as_f64(host(got))
        assert np.isfinite(a).all(), f"{key}: not every element written"
        if not np.abs(r).max() > 0:
            assert np.array_equal(a, np.zeros_like(a)), key
            say(f"  {key}: zero, as the oracle's")
            continue
        e = rel_err(a, r)
        say(f"  {key}: max|d|/max|ref| = {e:.3e}")
        assert e <= TOL, (key, e)
    return g


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("c_aux,c_z", [(0.0, 0.0), (1.0, 0.1)])
def test_backward_matches_oracle(name, c_aux, c_z):
    inp, dy = _inputs(CASES[name], seed=11)
    _check(inp, dy, c_aux, c_z, name)


@pytest.mark.parametrize("name", ["gelu-renorm-cf0.75-biases", "swiglu-ffn-dma256-T2048-shared1",
                                  "swiglu-d384-dff384-T1024-shared1"])
def test_backward_padded_weight_rows(name):
    """Expert matrices with rows 64 elements longer than their width (the
    layout the benchmark uses), on both recompute paths."""
    inp, dy = _inputs(CASES[name], seed=11)
    _check(inp, dy, 1.0, 0.1, name, pad=64)


def test_backward_is_deterministic():
    import torch
    wl = CASES["swiglu-topk-softmax-shared1"]
    inp, dy = _inputs(wl, seed=11)
    t = device_weights(inp)
    s = shape_of(wl)
    x, dyd, w = dev(inp.x), dev(dy), moe.weights_struct(t)
    outs = []
    for _ in range(2):
        g = moe.alloc_grads(s)
        moe.backward(s, x, w, dyd, g, 1.0, 0.1)
        torch.cuda.synchronize()
        outs.append({k: host(v) for k, v in g.items() if v is not None})
    for k in outs[0]:
        assert np.array_equal(outs[0][k].view(np.uint8), outs[1][k].view(np.uint8)), k


def test_backward_router_only_when_all_dropped():
    """Capacity 0 drops every pair: the routed experts get zero gradients, and
    with dy = 0 only the L_aux and z terms reach the router."""
    import torch
    wl = CASES["swiglu-capacity0-shared1"]
    inp, _ = _inputs(wl, seed=11)
    dy = np.zeros((wl.T, wl.d), np.uint16)
    g = _check(inp, dy, 1.0, 0.1, "capacity 0, dy = 0")
    for k in ("dw1", "dw3", "dw2", "dsw1", "dsw3", "dsw2"):
        assert not torch.any(g[k]).item(), k
    assert torch.any(g["dw_router"]).item()


def test_backward_mixtral_prefill_full_size_sampled():
    """The Mixtral-shape prefill layer at full size (T=4096, d=4096,
    d_ff=14336, 8 experts, top-2), weights with the padded rows the benchmark
    uses, same dy and loss coefficients: dx rows of sampled tokens and, for
    sampled (expert, hidden unit) pairs, the dW1 / dW3 rows and dW2 columns,
    against the oracle's sampled backward. Tokens routed differently from the
    oracle (near ties), and experts they touch, are left out of the sample."""
    import torch
    wl = gen.MIXTRAL_PREFILL
    say(f"backward full size {wl.name}: generating inputs")
    inp = gen.make_inputs(wl)
    dy = gen.normal(97, (wl.T, wl.d), 1.0, gen.BF16)
    t = device_weights(inp, pad=64)
    s = shape_of(wl)
    x = dev(inp.x)
    logits = torch.empty(wl.T, wl.n_experts, dtype=torch.float32, device="cuda")
    idx = torch.empty(wl.T, wl.top_k, dtype=torch.int32, device="cuda")
    gw = torch.empty(wl.T, wl.top_k, dtype=torch.float32, device="cuda")
    moe.route(s, x, t["w_router"], t["b_router"], logits, idx, gw)
    g = moe.alloc_grads(s)
    moe.backward(s, x, moe.weights_struct(t), dev(dy), g, 1.0, 1e-3)
    torch.cuda.synchronize()
    so = oracle.shape_of(wl)
    _, l32 = oracle.router_logits(so, inp.x, inp)
    r = oracle.route(so, l32)
    gi = host(idx)
    diff = (gi != r.topk_idx).any(1)
    moved = set(gi[diff].ravel().tolist()) | set(r.topk_idx[diff].ravel().tolist())
    tokens = [tk for tk in (0, 1, 2047, 3001, 4095) if not diff[tk]]
    units = [(e, i) for e, i in ((0, 0), (1, 4097), (3, 7777), (5, 12000), (7, 14335)) if e not in moved]
    say(f"  routed differently: {int(diff.sum())} tokens; sampled {len(tokens)} tokens, {len(units)} units")
    assert tokens and units
    dx, d1, d3, d2 = oracle.backward_sampled(inp, dy, tokens, units, 1.0, 1e-3)
    got = as_f64(host(g["dx"][torch.tensor(tokens, device="cuda")]))
    e = rel_err(got, dx)
    say(f"  dx rows: max|d|/max|ref| = {e:.3e}")
    assert e <= TOL
    for name, ref, pick in (("dw1", d1, lambda m, e_, i: m[e_, i]), ("dw3", d3, lambda m, e_, i: m[e_, i]),
                            ("dw2", d2, lambda m, e_, i: m[e_, :, i])):
        got = np.stack([host(pick(g[name], e_, i)).astype(np.float64) for e_, i in units])
        e = rel_err(got, ref)
        say(f"  {name} sampled: max|d|/max|ref| = {e:.3e}")
        assert e <= TOL, name
