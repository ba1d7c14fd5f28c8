"""End-to-end moe_forward against the CPU oracle, for every workload: reduced
sizes (every token compared) and the full sizes in the launch configuration the
benchmark times (sampled tokens, which the oracle computes one by one).

Routing: the GPU's fp32 logits are compared with the oracle's fp64 logits;
tokens whose top-k margin exceeds the logit error must route identically
(bit-exact). Tokens closer to a tie are reported, must still pick a valid top-k
set, and are left out of the output comparison together with every token whose
capacity slot they could have moved. The router_grid inputs make every logit an
exact fp32 number, so there the whole routing, permutation and drop set must
match bit for bit."""
import numpy as np
import pytest

import gen
import oracle
import sparse_mixture_experts_36_amd as moe
from helpers import as_f64, dev, device_weights, host, rel_err, say, shape_of, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()
    yield
    torch.cuda.synchronize()


MARGIN = 1e-3  # the checking protocol's near-tie threshold on the fp32 logits


def margin_report(r, diff, inv_gpu, inv_ref, capped):
    """Tokens whose top-k set margin l_(k) - l_(k+1) or slot-order margin
    min_j l_(j) - l_(j+1) (j < k) is below 1e-3, counted apart from the rest,
    with the routing differences among them and the tokens whose kept / dropped
    pattern differs. Returns the near-tie mask."""
    near_set = r.margin_set < MARGIN
    near_order = r.margin_order < MARGIN
    near = near_set | near_order
    drop_diff = ((inv_gpu < 0) != (inv_ref < 0)).any(1) if capped else np.zeros(len(diff), bool)
    say(f"  margin < {MARGIN:g}: set {int(near_set.sum())}, slot order {int(near_order.sum())}; "
        f"routed differently among them {int((diff & near).sum())}, elsewhere {int((diff & ~near).sum())}; "
        f"tokens with a different drop pattern {int(drop_diff.sum())}")
    return near


def run_and_check(inp, sample=None, exact_routing=False, label="", pad=0):
    import torch
    wl = inp.wl
    say(f"forward {label or wl.name}: T={wl.T} d={wl.d} d_ff={wl.d_ff} N={wl.n_experts} k={wl.top_k} "
        f"C={wl.capacity()} shared={wl.n_shared} w_dtype={wl.w_dtype} weight row pad={pad}")
    layer = moe.MoELayer(shape_of(wl), device_weights(inp, pad))
    out = layer(dev(inp.x))
    torch.cuda.synchronize()
    so = oracle.shape_of(wl)
    l64, l32 = oracle.router_logits(so, inp.x, inp)
    r = oracle.route(so, l32)
    dsp = oracle.dispatch(so, r.topk_idx)
    lg = host(out.logits)
    gi = host(out.topk_idx)
    err = float(np.abs(lg.astype(np.float64) - l64).max())
    lmax = float(np.abs(l64).max())
    assert err <= 1e-5 * lmax, f"logit error {err} vs max {lmax}"
    if exact_routing:
        assert np.array_equal(lg, l32)
        diff = np.zeros(wl.T, bool)
    else:
        thr = 4 * err + 1e-6 * lmax
        amb = ~((r.margin_set > thr) & (r.margin_order > thr))
        assert np.array_equal(gi[~amb], r.topk_idx[~amb])
        for t in np.nonzero(amb)[0]:
            kth = np.sort(l64[t])[::-1][wl.top_k - 1]
            assert (l64[t, gi[t]] >= kth - thr).all()
        diff = (gi != r.topk_idx).any(1)
        say(f"  logit err {err:.2e}; near-tie tokens {int(amb.sum())}; routed differently {int(diff.sum())}")
    near = margin_report(r, diff, host(out.inv_map), dsp.inv_map, wl.capacity() >= 0)
    # every token clear of a tie by the protocol's 1e-3 routes bit-identically
    assert not (diff & ~near).any()
    assert np.allclose(host(out.topk_w)[~diff], r.topk_w[~diff], rtol=1e-4, atol=1e-6)

    # tokens whose result the comparison can trust
    ok = ~diff
    if diff.any() and wl.capacity() >= 0:
        t0 = int(np.nonzero(diff)[0].min())
        moved = set(gi[diff].ravel()) | set(r.topk_idx[diff].ravel())
        for t in range(t0, wl.T):
            if set(r.topk_idx[t]) & moved:
                ok[t] = False
    if not diff.any():
        assert np.array_equal(host(out.inv_map), dsp.inv_map)
        assert np.array_equal(host(out.expert_offsets), dsp.offsets)
        M = int(dsp.offsets[-1])
        assert np.array_equal(host(out.perm_token)[:M], dsp.perm_token[:M])
        st = {k: host(v) for k, v in out.stats.items()}
        assert np.array_equal(st["counts"].astype(np.int64), r.counts)
        assert np.array_equal(st["kept"], dsp.kept) and int(st["n_dropped"][0]) == dsp.n_dropped
        assert np.allclose(st["P"], r.P, rtol=1e-4, atol=1e-7)
        assert abs(float(st["l_aux"][0]) - r.l_aux) <= 1e-4 * abs(r.l_aux)
        assert abs(float(st["z_loss"][0]) - r.z) <= 1e-4 * abs(r.z) + 1e-6
        say(f"  rows {M}, dropped {dsp.n_dropped}, L_aux {float(st['l_aux'][0]):.6f}, z {float(st['z_loss'][0]):.4f}")

    tokens = np.arange(wl.T) if sample is None else np.asarray(sample)
    tokens = tokens[ok[tokens]]
    assert len(tokens) > 0
    y_ref = oracle.moe_output(so, inp.x, inp, r, dsp, tokens)
    y_gpu = as_f64(host(out.y))[tokens]
    e = rel_err(y_gpu, y_ref)
    tol = tol_for(wl)
    say(f"  compared {len(tokens)} tokens: max|d|/max|ref| = {e:.3e} (tol {tol})")
    assert e <= tol
    return out


def _sample(T, n, seed=0):
    rng = np.random.default_rng(seed)
    s = set([0, T - 1]) | set(rng.choice(T, size=min(n, T), replace=False).tolist())
    return np.array(sorted(s)[:max(n, 2)], np.int64)


# ---------------------------------------------------------------- reduced sizes, every token

REDUCED = {
    "tiny-gelu-fp32": gen.TINY_GELU,
    "tiny-gelu-fp32-tight-capacity": gen.TINY_GELU.with_(capacity_factor=0.5),
    "mixtral-like": gen.MIXTRAL_PREFILL.with_(T=512, d=1024, d_ff=1536),
    "mixtral-like-renorm": gen.MIXTRAL_PREFILL.with_(T=300, d=512, d_ff=768, gating=gen.SOFTMAX_TOPK_RENORM),
    "fine-grained-like": gen.FINE_GRAINED.with_(T=512, d=512, d_ff=256),
    "switch-like": gen.SWITCH_TOP1.with_(T=2048, d=512, d_ff=1024),
    "switch-like-fp8": gen.SWITCH_TOP1_FP8.with_(T=2048, d=512, d_ff=1024),
    "switch-like-renorm": gen.SWITCH_TOP1.with_(T=1024, d=256, d_ff=512, gating=gen.SOFTMAX_TOPK_RENORM),
    # 2048 rows or more with widths the 256-column tiles do not fit (GELU
    # d_ff = 384; d = 384): the 128 x 128 tiles take them
    "switch-like-d_ff-384": gen.SWITCH_TOP1.with_(T=4096, d=512, d_ff=384),
    "mixtral-like-d-384": gen.MIXTRAL_PREFILL.with_(T=1024, d=384, d_ff=512),
    # 256-row tiles with skewed groups: nine of at most 384 rows run whole on
    # the 128-row tiles, two larger ones end in short tails, one shared expert
    "fine-grained-like-dma256-small-groups": gen.FINE_GRAINED.with_(T=2048, d=512, d_ff=512, n_experts=12, top_k=2,
                                                                    n_shared=1, zipf_s=1.0),
    # decode-sized: the weight-streaming path
    "mixtral-like-decode-T1": gen.MIXTRAL_PREFILL.with_(T=1, d=1024, d_ff=1536),
    # one token: the combine folded into the down GEMV (k + shared <= 4 slots,
    # bf16 or e4m3), dropped slots skipped; more slots take the separate combine
    "decode-T1-fused-fp8-gelu-shared": gen.SWITCH_TOP1_FP8.with_(T=1, d=1024, d_ff=2048, n_shared=1),
    "decode-T1-fused-k2-shared2": gen.FINE_GRAINED.with_(T=1, d=512, d_ff=1024, top_k=2),
    "decode-T1-fused-all-dropped-shared2": gen.FINE_GRAINED.with_(T=1, d=512, d_ff=1024, top_k=2, capacity_factor=0.0),
    "decode-T1-k6-shared2-separate-combine": gen.FINE_GRAINED.with_(T=1, d=512, d_ff=1024),
    "mixtral-like-decode-T64": gen.MIXTRAL_PREFILL.with_(T=64, d=1024, d_ff=1536),
    "fine-grained-like-decode": gen.FINE_GRAINED.with_(T=24, d=512, d_ff=256),
    "fine-grained-like-decode-T2": gen.FINE_GRAINED.with_(T=2, d=512, d_ff=1024),  # GEMV: two rows, shared experts
    "switch-like-decode-fp8": gen.SWITCH_TOP1_FP8.with_(T=128, d=512, d_ff=1024),
    # at most 16 tokens and 64 experts: router GEMM, routing and permutation in
    # one workgroup (capacity drops, router bias, a shared expert, 3 column blocks)
    "front-end-T16-N48-k4-cf2-shared": gen.FINE_GRAINED.with_(T=16, d=512, d_ff=256, n_experts=48, top_k=4,
                                                              capacity_factor=2.0, n_shared=1),
    "front-end-T5-N64-renorm": gen.MIXTRAL_PREFILL.with_(T=5, d=1024, d_ff=512, n_experts=64, top_k=3,
                                                         gating=gen.SOFTMAX_TOPK_RENORM),
    # one token through the front end: one wave routes it and builds its
    # statistics and permutation (all three gating modes, 3 and 4 column
    # blocks, k up to 8, a shared expert, every slot dropped at capacity 0)
    "front-end-T1-N48-k4-shared": gen.FINE_GRAINED.with_(T=1, d=512, d_ff=256, n_experts=48, top_k=4, n_shared=1),
    "front-end-T1-N64-k3-renorm": gen.MIXTRAL_PREFILL.with_(T=1, d=1024, d_ff=512, n_experts=64, top_k=3,
                                                            gating=gen.SOFTMAX_TOPK_RENORM),
    "front-end-T1-N64-k8": gen.MIXTRAL_PREFILL.with_(T=1, d=512, d_ff=512, n_experts=64, top_k=8),
    "front-end-T1-N48-k4-all-dropped": gen.FINE_GRAINED.with_(T=1, d=512, d_ff=256, n_experts=48, top_k=4,
                                                              capacity_factor=2.0),
    # one token, at most 16 experts: the router logits by dot products
    # (1024 / NP threads an expert), then the same one-token routing
    "front1-T1-N8-k2": gen.MIXTRAL_PREFILL.with_(T=1, d=1024, d_ff=512),
    "front1-T1-N16-k4-zipf-renorm-shared": gen.FINE_GRAINED.with_(T=1, d=1024, d_ff=256, n_experts=16, top_k=4,
                                                                  gating=gen.SOFTMAX_TOPK_RENORM, n_shared=1),
    "front1-T1-N5-k2-cf3": gen.MIXTRAL_PREFILL.with_(T=1, d=2048, d_ff=512, n_experts=5, top_k=2,
                                                     capacity_factor=3.0),
    "front1-T1-N2-k1-softmax-topk": gen.MIXTRAL_PREFILL.with_(T=1, d=4096, d_ff=256, n_experts=2, top_k=1,
                                                              gating=gen.SOFTMAX_TOPK),
}


@pytest.mark.parametrize("name", list(REDUCED))
def test_forward_reduced(name):
    run_and_check(gen.make_inputs(REDUCED[name]), label=name)


def test_forward_capacity_zero_gives_shared_only():
    wl = gen.FINE_GRAINED.with_(T=128, d=256, d_ff=256, capacity_factor=0.0)
    run_and_check(gen.make_inputs(wl), label="capacity 0")


def test_forward_is_deterministic():
    import torch
    wl = gen.SWITCH_TOP1.with_(T=4096, d=512, d_ff=1024)
    inp = gen.make_inputs(wl)
    layer = moe.MoELayer(shape_of(wl), device_weights(inp))
    x = dev(inp.x)
    a = layer(x)
    ya, la = a.y.clone(), a.logits.clone()
    sa = {k: v.clone() for k, v in a.stats.items()}
    b = layer(x)
    torch.cuda.synchronize()
    assert torch.equal(ya.view(torch.int16), b.y.view(torch.int16))
    assert torch.equal(la, b.logits)
    for k in sa:
        assert torch.equal(sa[k], b.stats[k]), k


def test_forward_shared_experts_from_two_streams():
    """Two layers with shared experts called back to back on two different
    streams, with no synchronisation between the calls, must each give the
    result of a call made alone (the library keeps no state between calls)."""
    import torch
    wa = gen.FINE_GRAINED.with_(T=512, d=512, d_ff=256)
    wb = gen.FINE_GRAINED.with_(T=96, d=512, d_ff=256, n_shared=1)
    ia, ib = gen.make_inputs(wa, seed=3), gen.make_inputs(wb, seed=4)
    la = moe.MoELayer(shape_of(wa), device_weights(ia))
    lb = moe.MoELayer(shape_of(wb), device_weights(ib))
    xa, xb = dev(ia.x), dev(ib.x)
    ya, yb = la(xa).y.clone(), lb(xb).y.clone()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        la.out.y.zero_()
        lb.out.y.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            la(xa, stream=s1)
        with torch.cuda.stream(s2):
            lb(xb, stream=s2)
        torch.cuda.synchronize()
        assert torch.equal(la.out.y.view(torch.int16), ya.view(torch.int16))
        assert torch.equal(lb.out.y.view(torch.int16), yb.view(torch.int16))


# ---------------------------------------------------------------- full sizes, sampled tokens

def test_full_tiny_gelu_fp32():
    run_and_check(gen.make_inputs(gen.TINY_GELU), label="tiny-gelu-fp32 (full)")


@pytest.mark.parametrize("pad", [0, 64])
def test_full_mixtral_prefill(pad):
    """pad=64 is the weight layout the benchmark times."""
    inp = gen.make_inputs(gen.MIXTRAL_PREFILL)
    run_and_check(inp, sample=_sample(4096, 64), label="mixtral-prefill (full)", pad=pad)


@pytest.mark.parametrize("T", [1, 16, 64])
def test_full_mixtral_decode(T):
    inp = gen.make_inputs(gen.MIXTRAL_DECODE[T])
    run_and_check(inp, sample=None, label=f"mixtral-decode T={T}", pad=64)


def test_full_fine_grained():
    inp = gen.make_inputs(gen.FINE_GRAINED)
    run_and_check(inp, sample=_sample(8192, 64), label="fine-grained (full)", pad=64)


@pytest.mark.parametrize("fp8", [False, True])
def test_full_switch(fp8):
    wl = gen.SWITCH_TOP1_FP8 if fp8 else gen.SWITCH_TOP1
    run_and_check(gen.make_inputs(wl), sample=_sample(16384, 64), label=wl.name + " (full)")


def test_full_switch_exact_routing_grid():
    """Every logit exact in fp32: routing, the 16384-token permutation, the drop
    set and the counts must match the oracle bit for bit."""
    inp = gen.make_inputs(gen.SWITCH_TOP1, router_grid=True)
    run_and_check(inp, sample=_sample(16384, 32), exact_routing=True, label="switch exact-grid (full)")


WS_CASES = {
    "decode-T1-gemv": gen.MIXTRAL_PREFILL.with_(T=1, d=1024, d_ff=1536),
    "decode-T2-gemv-shared": gen.FINE_GRAINED.with_(T=2, d=512, d_ff=1024),
    "decode-T16-stream": gen.MIXTRAL_PREFILL.with_(T=16, d=1024, d_ff=1536),
    "decode-T24-shared": gen.FINE_GRAINED.with_(T=24, d=512, d_ff=256),
    "prefill-dma128-drops": gen.SWITCH_TOP1.with_(T=2048, d=512, d_ff=1024),
    "prefill-dma256-split-tails": gen.MIXTRAL_PREFILL.with_(T=4096, d=1024, d_ff=1536),
    "prefill-reg128": gen.MIXTRAL_PREFILL.with_(T=512, d=1024, d_ff=1536),
    "prefill-fp8-dma128": gen.SWITCH_TOP1_FP8.with_(T=4096, d=512, d_ff=1024),
    "tiny-fp32": gen.TINY_GELU,
    "expert-choice": gen.WORKLOADS["tiny-gelu-fp32-ec"],
}


@pytest.mark.parametrize("name", list(WS_CASES))
def test_forward_ignores_workspace_contents(name):
    """The workspace's contents on entry do not matter: one filled with 0xFF
    bytes (NaN as floats) and one filled with zeros give the same bits."""
    import torch
    wl = WS_CASES[name]
    inp = gen.make_inputs(wl)
    s = shape_of(wl)
    t = device_weights(inp, 64 if wl.act_dtype == gen.BF16 else 0)  # kept alive: the struct holds raw pointers
    w = moe.weights_struct(t)
    x = dev(inp.x)
    res = []
    for fill in (0x00, 0xFF):
        ws = moe.workspace(s, moe.ENTRY_FORWARD)
        ws.view(torch.uint8).fill_(fill)
        o = moe.MoELayer(s, t).out  # its output tensors; the call below takes the workspace filled above
        moe.forward(s, x, w, o.y, o.logits, o.topk_idx, o.topk_w, o.expert_offsets, o.perm_token, o.inv_map,
                    o.stats, ws=ws)
        torch.cuda.synchronize()
        res.append({k: host(getattr(o, k)).copy() for k in ("y", "logits", "topk_idx", "topk_w", "inv_map")})
        res[-1].update({"stats." + k: host(v).copy() for k, v in o.stats.items()})
    for k in res[0]:
        assert np.array_equal(res[0][k].view(np.uint8), res[1][k].view(np.uint8)), k
    assert np.isfinite(as_f64(res[0]["y"])).all()
    say(f"workspace contents {name}: identical outputs")
