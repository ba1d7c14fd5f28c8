"""Stage-by-stage parity of the HIP path against the CPU oracle, at sizes the
oracle finishes in seconds that still span several tiles and ragged tails.
Every input comes from the seeded generator (or from the oracle's own routing);
nothing the GPU computes is fed to the oracle."""
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


def _wl(T, N, k, gating=gen.SOFTMAX_TOPK, act=gen.SWIGLU, d=256, d_ff=384, dt=gen.BF16, wdt=None, cf=None,
        n_shared=0, zipf=None, n_int8=0):
    return gen.Workload("t", T, d, d_ff, N, k, act, gating, dt, dt if wdt is None else wdt, cf, n_shared=n_shared,
                        zipf_s=zipf, n_int8=n_int8)


# ---------------------------------------------------------------- routing on given logits: bit-exact

ROUTE_CASES = [
    (1000, 8, 2, gen.SOFTMAX_TOPK_RENORM, 0.25),
    (1000, 8, 2, gen.TOPK_SOFTMAX, 0.25),
    (777, 160, 6, gen.SOFTMAX_TOPK, 0.5),
    (4096, 64, 1, gen.SOFTMAX_TOPK, None),
    (100, 256, 8, gen.SOFTMAX_TOPK_RENORM, 0.25),
    (1, 8, 2, gen.TOPK_SOFTMAX, None),
    (300, 5, 5, gen.SOFTMAX_TOPK_RENORM, 0.5),
    (65, 17, 3, gen.TOPK_SOFTMAX, 1.0),
]


@pytest.mark.parametrize("T,N,k,gating,step", ROUTE_CASES)
def test_route_given_logits_bit_exact(T, N, k, gating, step):
    import torch
    say(f"route given logits T={T} N={N} k={k} gating={gating} step={step}")
    wl = _wl(T, N, k, gating=gating)
    l32 = gen.given_logits(T, N, seed=T + N, step=step, bias=gen.zipf_bias(N, 1.0))
    ref = oracle.route(oracle.shape_of(wl), l32)
    shape = shape_of(wl)
    logits = dev(l32)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    st = moe.alloc_stats(N)
    moe.route(shape, None, None, None, logits, idx, w, st, flags=moe.ROUTE_LOGITS_GIVEN)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx), ref.topk_idx)
    assert np.allclose(host(w), ref.topk_w, rtol=1e-5, atol=1e-7)
    assert np.array_equal(host(st["counts"]).astype(np.int64), ref.counts)
    assert np.allclose(host(st["f"]), ref.f, rtol=1e-6, atol=0)
    assert np.allclose(host(st["P"]), ref.P, rtol=1e-5, atol=1e-8)
    assert abs(float(host(st["l_aux"])[0]) - ref.l_aux) <= 1e-5 * abs(ref.l_aux)
    assert abs(float(host(st["z_loss"])[0]) - ref.z) <= 1e-5 * abs(ref.z) + 1e-7
    assert abs(float(host(st["lse_sq_mean"])[0]) - ref.lse_sq_mean) <= 1e-5 * abs(ref.lse_sq_mean) + 1e-7
    assert np.array_equal(host(logits), l32)  # given logits are not modified


@pytest.mark.parametrize("T,N,k,dt,zipf", [(300, 8, 2, gen.BF16, None), (1000, 160, 6, gen.BF16, 1.0),
                                           (256, 8, 2, gen.F32, None), (513, 64, 1, gen.BF16, 1.2),
                                           (70, 256, 8, gen.BF16, None),
                                           # 1024 tokens or more: the router GEMM on the LDS-DMA ring
                                           # (6 stages; 4 above 160 experts; 3 column blocks padded)
                                           (1024, 256, 8, gen.BF16, None), (1536, 48, 4, gen.BF16, 1.0),
                                           (2048, 160, 6, gen.BF16, 1.0), (1100, 8, 2, gen.BF16, None)])
def test_router_gemm_and_routing(T, N, k, dt, zipf):
    """GPU logits against the fp64 oracle logits; tokens whose top-k margin is
    well above the logit error must route identically."""
    import torch
    say(f"router gemm T={T} N={N} k={k} dtype={dt}")
    wl = _wl(T, N, k, d=512, dt=dt, zipf=zipf)
    inp = gen.make_inputs(wl, seed=7)
    shape = shape_of(wl)
    l64, l32 = oracle.router_logits(oracle.shape_of(wl), inp.x, inp)
    ref = oracle.route(oracle.shape_of(wl), l32)
    logits = torch.empty((T, N), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.route(shape, dev(inp.x), dev(inp.w_router), dev(inp.b_router), logits, idx, w)
    torch.cuda.synchronize()
    lg = host(logits).astype(np.float64)
    err = float(np.abs(lg - l64).max())
    assert err <= 1e-5 * float(np.abs(l64).max())
    thr = 4 * err + 1e-6 * float(np.abs(l64).max())
    safe = (ref.margin_set > thr) & (ref.margin_order > thr)
    say(f"  logit err {err:.3e}; ambiguous tokens {int((~safe).sum())}")
    gi = host(idx)
    assert np.array_equal(gi[safe], ref.topk_idx[safe])
    # ambiguous tokens must still pick a valid top-k set under the exact logits
    for t in np.nonzero(~safe)[0]:
        kth = np.sort(l64[t])[::-1][k - 1]
        assert (l64[t, gi[t]] >= kth - thr).all()


# ---------------------------------------------------------------- permutation: bit-exact

PERM_CASES = [
    (1000, 8, 2, -1, None),
    (1000, 8, 2, 150, 1.0),
    (777, 160, 6, 20, 1.0),
    (16384, 64, 1, 320, 1.2),
    (256, 8, 2, 0, None),
    (1, 8, 2, -1, None),
    (513, 256, 8, 9, None),
    (4096, 8, 2, -1, None),
]


@pytest.mark.parametrize("copy_rows", [True, False], ids=["rows", "slots-only"])
@pytest.mark.parametrize("T,N,k,C,zipf", PERM_CASES)
def test_permute_bit_exact(T, N, k, C, zipf, copy_rows):
    """Slots, offsets, counts and drops match the oracle exactly; with x_perm
    given the rows are the tokens' rows. Without x_perm (no rows to copy), up
    to 256 tokens take the one-launch path that ranks, scans and writes the
    slots in one workgroup."""
    import torch
    say(f"permute T={T} N={N} k={k} C={C} copy_rows={copy_rows}")
    wl = _wl(T, N, k, d=256)
    shape_o = oracle.shape_of(wl, capacity=C)
    l32 = gen.given_logits(T, N, seed=3 * T + N, step=0.25, bias=None if zipf is None else gen.zipf_bias(N, zipf))
    r = oracle.route(shape_o, l32)
    ref = oracle.dispatch(shape_o, r.topk_idx)
    x = gen.normal(gen.T_X, (T, wl.d), 1.0, gen.BF16, seed=5)
    shape = shape_of(wl, capacity=C)
    offs = torch.full((N + 1,), -7, dtype=torch.int32, device="cuda")
    perm = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
    inv = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    xp = torch.zeros((T * k, wl.d), dtype=torch.bfloat16, device="cuda") if copy_rows else None
    st = moe.alloc_stats(N)
    moe.permute(shape, dev(r.topk_idx), dev(x), offs, perm, inv, xp, st)
    torch.cuda.synchronize()
    M = int(ref.offsets[-1])
    assert np.array_equal(host(offs), ref.offsets)
    assert np.array_equal(host(perm)[:M], ref.perm_token[:M])
    assert np.array_equal(host(inv), ref.inv_map)
    assert np.array_equal(host(st["kept"]), ref.kept)
    assert int(host(st["n_dropped"])[0]) == ref.n_dropped
    if copy_rows:
        assert np.array_equal(host(xp)[:M], x[ref.perm_token[:M]])
    say(f"  rows {M}, dropped {ref.n_dropped}")


# ---------------------------------------------------------------- grouped FFN against the oracle's experts

FFN_CASES = [
    dict(T=300, N=8, k=2, act=gen.SWIGLU, d=256, d_ff=384),
    dict(T=1000, N=8, k=2, act=gen.SWIGLU, d=512, d_ff=1024),
    dict(T=400, N=16, k=1, act=gen.GELU, d=256, d_ff=512, biases=True),
    dict(T=400, N=16, k=1, act=gen.GELU, d=256, d_ff=512, wdt=gen.E4M3, biases=True),
    dict(T=300, N=8, k=2, act=gen.SWIGLU, d=256, d_ff=384, wdt=gen.E4M3),
    dict(T=200, N=32, k=6, act=gen.SWIGLU, d=256, d_ff=256, n_shared=2, zipf=1.0),
    dict(T=256, N=8, k=2, act=gen.GELU, d=512, d_ff=2048, dt=gen.F32, biases=True),
    dict(T=130, N=8, k=2, act=gen.SWIGLU, d=128, d_ff=256, dt=gen.F32, n_shared=1),
    # decode-sized calls (<= 256 expert rows): the weight-streaming path
    dict(T=1, N=8, k=2, act=gen.SWIGLU, d=512, d_ff=1024),
    dict(T=100, N=8, k=2, act=gen.SWIGLU, d=256, d_ff=512),
    dict(T=128, N=8, k=2, act=gen.SWIGLU, d=512, d_ff=384),
    dict(T=64, N=16, k=1, act=gen.GELU, d=256, d_ff=512, wdt=gen.E4M3, biases=True),
    dict(T=64, N=16, k=1, act=gen.GELU, d=256, d_ff=512, biases=True),
    dict(T=40, N=32, k=4, act=gen.SWIGLU, d=256, d_ff=256, n_shared=2, zipf=1.0),
    dict(T=16, N=8, k=2, act=gen.SWIGLU, d=256, d_ff=1536, wdt=gen.E4M3),
    dict(T=16, N=8, k=2, act=gen.SWIGLU, d=256, d_ff=512, n_shared=1, pad=64),       # decode path, padded
    # 32- or 64-row passes whose k range holds whole pairs of two-step bursts:
    # token rows shared through LDS by the four waves of a workgroup
    dict(T=64, N=8, k=2, act=gen.SWIGLU, d=1024, d_ff=2048, zipf=1.5),             # 32 rows; skewed: two-pass groups
    dict(T=100, N=8, k=2, act=gen.SWIGLU, d=1024, d_ff=2048, pad=64),              # 64 rows, padded, split down
    dict(T=64, N=16, k=1, act=gen.GELU, d=1024, d_ff=1024, wdt=gen.E4M3, biases=True),  # e4m3, split in two
    dict(T=40, N=32, k=4, act=gen.SWIGLU, d=512, d_ff=512, n_shared=2, zipf=1.0),  # shared experts
    # one or two tokens with whole 1 KB weight segments: the vector-ALU GEMV
    dict(T=2, N=8, k=2, act=gen.SWIGLU, d=1024, d_ff=2048, n_shared=1, pad=64),      # two rows, shared, padded; up 8 rows a wave
    dict(T=1, N=8, k=2, act=gen.SWIGLU, d=1024, d_ff=4096, wdt=gen.E4M3),            # e4m3; up 8 rows a wave, down 4
    dict(T=2, N=4, k=1, act=gen.GELU, d=1024, d_ff=1024, wdt=gen.E4M3, biases=True, n_shared=1),
    dict(T=2, N=16, k=2, act=gen.GELU, d=512, d_ff=4096, biases=True),              # up 8 rows a wave, down 4
    dict(T=1, N=8, k=2, act=gen.SWIGLU, d=640, d_ff=1024),                           # d not whole segments: MFMA streaming
    dict(T=400, N=16, k=1, act=gen.GELU, d=256, d_ff=512, wdt=gen.E4M3, biases=True, pad=32),  # fp8, padded
    dict(T=130, N=8, k=2, act=gen.SWIGLU, d=128, d_ff=256, dt=gen.F32, n_shared=1, pad=16),    # fp32, padded
    # prefill-sized calls (>= 2048 expert rows): the LDS-DMA tiles, 128 x 256
    # when the groups average fewer than 384 rows, else 256 x 256. With 256
    # CUs, a launch whose last round holds r <= 128 tiles cuts those tiles
    # along k and sums the chunks in a fix-up pass; the comments give (tiles,
    # split) of the up and down GEMM.
    dict(T=2048, N=4, k=2, act=gen.SWIGLU, d=256, d_ff=512),                  # 256 rows: (~68, 2), (~17, 4)
    dict(T=2048, N=4, k=2, act=gen.SWIGLU, d=256, d_ff=512, pad=64),          # the same, padded weight rows
    dict(T=4096, N=4, k=2, act=gen.SWIGLU, d=512, d_ff=512),                  # 256 rows: (~144, none), (~72, 3)
    dict(T=3000, N=4, k=2, act=gen.SWIGLU, d=1024, d_ff=512),                 # 256 rows: (~100, 2), (~100, 2)
    dict(T=3072, N=4, k=1, act=gen.GELU, d=512, d_ff=1024, biases=True),      # 256 rows: (~52, 4), (~26, 8)
    dict(T=1200, N=8, k=2, act=gen.SWIGLU, d=512, d_ff=512),                  # 128 rows: (~80, 4), (~40, 4)
    dict(T=1200, N=8, k=2, act=gen.SWIGLU, d=512, d_ff=512, n_shared=1, pad=16),  # padded weights + shared; 256 rows
    dict(T=1100, N=8, k=2, act=gen.SWIGLU, d=256, d_ff=4096),                 # 128 rows: (~768, none), (~24, 8)
    dict(T=2048, N=16, k=1, act=gen.GELU, d=256, d_ff=1024, n_shared=1, biases=True),  # 128 rows: (~128, 2), (~32, 8)
    dict(T=1024, N=32, k=6, act=gen.SWIGLU, d=256, d_ff=256, n_shared=2, zipf=1.0),    # 128 rows: (~150, none), (~75, 2)
    # e4m3 weights on the LDS-DMA tiles (bytes DMA'd, fragments converted on read)
    dict(T=2048, N=16, k=1, act=gen.GELU, d=256, d_ff=1024, n_shared=1, biases=True, wdt=gen.E4M3),  # 128 rows
    dict(T=2048, N=4, k=2, act=gen.SWIGLU, d=256, d_ff=512, wdt=gen.E4M3),             # 256 rows, split, tails
    dict(T=3000, N=4, k=2, act=gen.SWIGLU, d=1024, d_ff=512, n_shared=1, pad=64, wdt=gen.E4M3),  # 256 rows, shared
    dict(T=2048, N=12, k=2, act=gen.SWIGLU, d=512, d_ff=512, n_shared=1, zipf=1.0, wdt=gen.E4M3),  # small groups
    # integer codes on the LDS-DMA tiles (INT8: byte rows as e4m3; INT4: 32-byte
    # stage rows), one launch per width present, row scales in the epilogue;
    # experts below n_int8 and the shared ones take 8 bits, the others 4
    dict(T=2048, N=16, k=1, act=gen.GELU, d=256, d_ff=1024, n_shared=1, biases=True, wdt=gen.INT_W, n_int8=6),  # 128
    dict(T=2048, N=4, k=2, act=gen.SWIGLU, d=256, d_ff=512, wdt=gen.INT_W, n_int8=2),  # 256 rows, split, tails
    dict(T=2048, N=4, k=2, act=gen.SWIGLU, d=256, d_ff=512, wdt=gen.INT_W, n_int8=0),  # all INT4
    dict(T=2048, N=4, k=2, act=gen.SWIGLU, d=256, d_ff=512, wdt=gen.INT_W, n_int8=4),  # all INT8
    dict(T=3000, N=4, k=2, act=gen.SWIGLU, d=1024, d_ff=512, n_shared=1, pad=64, wdt=gen.INT_W, n_int8=1),  # padded
    dict(T=2048, N=12, k=2, act=gen.SWIGLU, d=512, d_ff=512, n_shared=1, zipf=1.0, wdt=gen.INT_W, n_int8=4),  # small
]


@pytest.mark.parametrize("case", FFN_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_grouped_ffn_against_oracle(case):
    import torch
    case = dict(case)
    biases = case.pop("biases", False)
    pad = case.pop("pad", 0)
    say(f"grouped ffn {case}")
    wl = _wl(**case)
    inp = gen.make_inputs(wl, seed=11)
    if biases:
        rng = np.random.default_rng(3)
        inp.b1 = rng.standard_normal(inp.b1.shape).astype(np.float32)
        inp.b2 = rng.standard_normal(inp.b2.shape).astype(np.float32)
    so = oracle.shape_of(wl)
    _, l32 = oracle.router_logits(so, inp.x, inp)
    r = oracle.route(so, l32)
    dsp = oracle.dispatch(so, r.topk_idx)
    M = int(dsp.offsets[-1])
    x_perm = np.ascontiguousarray(inp.x[dsp.perm_token[:M]])
    shape = shape_of(wl)
    tdt = torch.float32 if wl.act_dtype == gen.F32 else torch.bfloat16
    yp = torch.zeros((max(M, 1), wl.d), dtype=tdt, device="cuda")
    ysh = torch.zeros((wl.n_shared, wl.T, wl.d), dtype=tdt, device="cuda") if wl.n_shared else None
    keep = device_weights(inp, pad)
    W = moe.weights_struct(keep)
    moe.grouped_ffn(shape, dev(x_perm) if M else yp, dev(dsp.offsets), dev(inp.x), W, yp, ysh)
    torch.cuda.synchronize()
    got = as_f64(host(yp))
    tol = tol_for(wl)
    worst = 0.0
    for e in range(wl.n_experts):
        a, b = int(dsp.offsets[e]), int(dsp.offsets[e + 1])
        if a == b:
            continue
        ref = oracle.expert_rows(so, inp, e, x_perm[a:b])
        worst = max(worst, rel_err(got[a:b], ref))
    for s in range(wl.n_shared):
        ref = oracle.expert_rows(so, inp, s, inp.x, shared=True)
        worst = max(worst, rel_err(as_f64(host(ysh[s])), ref))
    say(f"  rows {M}, worst rel err {worst:.3e} (tol {tol})")
    assert worst <= tol


# ---------------------------------------------------------------- combine

@pytest.mark.parametrize("T,N,k,n_shared,dt,C", [(300, 8, 2, 0, gen.BF16, 60), (200, 32, 6, 2, gen.BF16, -1),
                                                 (256, 8, 2, 0, gen.F32, 80), (1, 8, 2, 1, gen.BF16, -1)])
def test_combine_against_oracle(T, N, k, n_shared, dt, C):
    import torch
    say(f"combine T={T} N={N} k={k} shared={n_shared}")
    wl = _wl(T, N, k, d=256, dt=dt, n_shared=n_shared)
    so = oracle.shape_of(wl, capacity=C)
    l32 = gen.given_logits(T, N, seed=9, step=None)
    r = oracle.route(so, l32)
    dsp = oracle.dispatch(so, r.topk_idx)
    M = max(int(dsp.offsets[-1]), 1)
    yp = gen.normal(50, (M, wl.d), 1.0, dt, seed=2)
    ysh = gen.normal(51, (n_shared, T, wl.d), 1.0, dt, seed=2) if n_shared else None
    g32 = r.topk_w.astype(np.float32)
    ref = oracle.combine(so, yp, dsp.inv_map, g32, ysh)
    shape = shape_of(wl, capacity=C)
    y = torch.empty((T, wl.d), dtype=torch.float32 if dt == gen.F32 else torch.bfloat16, device="cuda")
    moe.combine(shape, dev(yp), dev(dsp.inv_map), dev(g32), dev(ysh), y)
    torch.cuda.synchronize()
    err = rel_err(as_f64(host(y)), ref)
    say(f"  rel err {err:.3e}")
    assert err <= (1e-6 if dt == gen.F32 else 8e-3)


def test_fp8_decode_is_exact():
    """The in-register e4m3 -> bf16 decode, code by code: two fp8 SwiGLU experts
    with x = e_0, W3 column 0 = 1.0, W1 column 0 = one finite code per hidden
    unit and W2 = identity give y_o = silu(value of code o) for each code."""
    import torch
    say("fp8 decode through the grouped GEMM")
    d, d_ff = 128, 128
    wl = _wl(2, 2, 1, act=gen.SWIGLU, d=d, d_ff=d_ff, wdt=gen.E4M3)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)  # 254 finite codes
    q1 = np.zeros((2, d_ff, d), np.uint8)
    q1[0, :128, 0] = codes[:128]
    q1[1, :126, 0] = codes[128:]
    q3 = np.zeros((2, d_ff, d), np.uint8)
    q3[:, :, 0] = 0x38                      # 1.0
    q2 = np.zeros((2, d, d_ff), np.uint8)
    q2[:, np.arange(d), np.arange(d)] = 0x38
    x = np.zeros((2, d), np.uint16)
    x[:, 0] = 0x3F80                        # 1.0 in bf16
    inp = gen.make_inputs(wl, seed=1)
    inp.w1, inp.w3, inp.w2, inp.x = q1, q3, q2, x
    inp.w_scale = np.ones((2, 3), np.float32)
    so = oracle.shape_of(wl)
    ref = np.concatenate([oracle.expert_rows(so, inp, e, x[e:e + 1]) for e in range(2)])
    shape = shape_of(wl)
    yp = torch.zeros((2, d), dtype=torch.bfloat16, device="cuda")
    keep = device_weights(inp)
    moe.grouped_ffn(shape, dev(x), dev(np.array([0, 1, 2], np.int32)), dev(x), moe.weights_struct(keep), yp)
    torch.cuda.synchronize()
    got = as_f64(host(yp))
    assert np.all(np.abs(got - ref) <= 1e-2 * np.abs(ref) + 1e-30)
