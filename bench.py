"""Benchmark of the MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one moe_forward (router GEMM + softmax/top-k/gates + statistics,
permutation with capacity, grouped up GEMM with the fused activation, grouped
down GEMM, combine) over one batch of seeded synthetic input that is already
resident in HBM when the timed region starts. Prints ONE JSON line.

Default workload: the Mixtral-shape prefill layer (T=4096, d=4096,
d_ff=14336, 8 experts, top-2, top-k-then-softmax, dropless, bf16 with fp32
accumulation). `value` is layer tokens/s. `roofline` describes the dominant
kernel (the grouped up GEMM with the fused SwiGLU): algorithmic flops per
launch = 4 * d * d_ff per kept (token, expert) pair, divided by that kernel's
mean launch time, measured with hipEvents on the stream it runs on over the
timed region. `decode` reports the Mixtral-shape decode layer (T = 1, 16, 64)
in HBM GB/s of algorithmic bytes (every touched expert's three matrices once,
the router weight, x and y): whole steps, timed both as eager launches
(`us_per_step_eager`) and replayed from captured HIP graphs
(`us_per_step_graph`); `us_per_step` is the faster of the two (`launch` names
it). The expert FFN alone is `ffn_us` (hipEvents on a separate pass). `cpu_baseline` times the
fp64 CPU oracle on a bounded sample of the same workload. `backward` times
moe_backward (forward recompute plus every gradient) on the prefill layer.
Other workloads (--workload): the expert-choice and INT8/INT4 variants of the
Mixtral-shape layer, the fine-grained and top-1 layers.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
GEMM_SOURCE = os.path.join(ROOT, "sparse_mixture_experts_36_amd", "csrc", "gemm.hip")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm-dma-up-swiglu_mixtral-prefill_hbm-traffic.txt")
COPY_BYTES = 1 << 30        # the calibration kernel reads and writes this many bytes


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(a):
    import numpy as np
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


WEIGHT_NAMES = ("w_router", "b_router", "w1", "w3", "w2", "b1", "b2", "w_scale", "sw1", "sw3", "sw2", "sw_scale")
ROW_PAD = 64  # elements added to the expert matrices' row pitch (moe_weights ld_up / ld_down)


def layer_weights(inp) -> dict:
    """Device weights in the layout the library reads fastest: expert matrices
    with rows ROW_PAD elements longer than d (W1, W3) or d_ff (W2). Integer
    weights: byte rows ROW_PAD bytes longer, 4-bit experts packed two codes a
    byte, bit widths as host arrays."""
    import gen
    import sparse_mixture_experts_36_amd as moe
    mats = ("w1", "w3", "w2", "sw1", "sw3", "sw2")
    if inp.wl.w_dtype == gen.INT_W:
        t = {n: to_dev(getattr(inp, n)) for n in WEIGHT_NAMES if n not in mats}
        for n in mats:
            codes = getattr(inp, n)
            bits = inp.sw_bits if n.startswith("s") else inp.w_bits
            t[n] = None if codes is None else to_dev(moe.pack_int_weights(codes, bits, ROW_PAD))[:, :, :codes.shape[2]]
        t["w_bits"], t["sw_bits"] = inp.w_bits, inp.sw_bits
        return t
    t = {n: to_dev(getattr(inp, n)) for n in WEIGHT_NAMES}
    for n in mats:
        t[n] = moe.padded(t[n], ROW_PAD)
    return t


def shape_for(wl):
    import sparse_mixture_experts_36_amd as moe
    return moe.make_shape(wl.T, wl.d, wl.d_ff, wl.n_experts, wl.top_k, wl.act, wl.gating, wl.act_dtype,
                          wl.w_dtype, wl.capacity(), wl.n_shared, wl.aux_alpha)


def weight_bytes_per_expert(wl, e: int = 0) -> int:
    """Bytes a kernel must read for routed expert e's weights: its matrices at
    the storage width, plus the fp32 row scales of integer weights."""
    import gen
    import sparse_mixture_experts_36_amd as moe
    params = moe.expert_params(wl.d, wl.d_ff, wl.act)
    if wl.w_dtype == gen.INT_W:
        rows = (2 if wl.act == gen.SWIGLU else 1) * wl.d_ff + wl.d
        return params * int(wl.expert_bits()[e]) // 8 + 4 * rows
    wb = {gen.F32: 4, gen.BF16: 2, gen.E4M3: 1}[wl.w_dtype]
    return params * wb


def layer_bytes(wl, kept) -> tuple[int, int, int]:
    """Algorithmic HBM bytes of one layer call: every touched expert's weights
    once (plus the shared experts'), the router weight, x read once and y
    written once. Returns (layer bytes, expert-weight bytes, touched experts)."""
    import gen
    import sparse_mixture_experts_36_amd as moe
    touched = [e for e in range(wl.n_experts) if kept[e] > 0]
    wbytes = sum(weight_bytes_per_expert(wl, e) for e in touched)
    if wl.n_shared:
        params = moe.expert_params(wl.d, wl.d_ff, wl.act)
        if wl.w_dtype == gen.INT_W:
            rows = (2 if wl.act == gen.SWIGLU else 1) * wl.d_ff + wl.d
            per = params * 8 // 8 + 4 * rows  # shared experts keep 8-bit codes
        else:
            per = params * {gen.F32: 4, gen.BF16: 2, gen.E4M3: 1}[wl.w_dtype]
        wbytes += wl.n_shared * per
    act_b = 4 if wl.act_dtype == gen.F32 else 2
    io = 2 * wl.T * wl.d * act_b + wl.n_experts * wl.d * act_b
    return wbytes + io, wbytes, len(touched)


def up_flops_per_pair(wl) -> float:
    """Up GEMM: d x d_ff per matrix, two matrices (W1, W3) for SwiGLU."""
    return 2.0 * wl.d * wl.d_ff * (2 if wl.act == 1 else 1)


def ffn_flops_per_pair(wl) -> float:
    return up_flops_per_pair(wl) + 2.0 * wl.d * wl.d_ff


def measured_traffic():
    """HBM bytes per launch of the up GEMM kernel from the committed PMC summary
    (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel calibration), or None
    when the summary is missing or was taken on another version of the GEMM
    source than the one built here."""
    import hashlib
    try:
        text = open(TRAFFIC_SUMMARY).read()
        src = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("gemm.hip sha256") != src or "hbm bytes per launch" not in fields:
        return None
    return int(float(fields["hbm bytes per launch"]))


def vendor_gemm_context(steps=20):
    """Context for the grouped GEMM: torch.matmul (the ROCm BLAS library) on
    one expert's GEMMs of the Mixtral prefill layer, at the rows one expert gets
    (1024 = 4096 tokens x top-2 / 8 experts) and at 8192 rows, bf16. Prints
    TFLOP/s per shape; nothing here is part of the layer."""
    import torch
    d, d_ff = 4096, 14336
    out = {}
    for M in (1024, 8192):
        for name, (K, Nn) in {"up (W1|W3)": (d, 2 * d_ff), "down (W2)": (d_ff, d)}.items():
            a = torch.randn(M, K, device="cuda", dtype=torch.bfloat16)
            b = torch.randn(Nn, K, device="cuda", dtype=torch.bfloat16)
            bt = b.t()  # [K][N] view: the NT product of the layer
            for _ in range(3):
                torch.matmul(a, bt)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(steps):
                torch.matmul(a, bt)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            out[f"M={M} {name}"] = {"ms": round(ms, 4), "TFLOP/s": round(2.0 * M * K * Nn / ms / 1e9, 1)}
    print(json.dumps({"vendor_gemm_bf16": out}), flush=True)


def copy_calibration():
    """A plain streaming kernel of known traffic (x * 1 over 1 GiB of fp32:
    1 GiB read, 1 GiB written), run under rocprofv3 --pmc to scale FETCH_SIZE
    and WRITE_SIZE to bytes."""
    import torch
    n = COPY_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_kernel": "elementwise mul by 1.0, fp32", "bytes_read": COPY_BYTES,
                      "bytes_written": COPY_BYTES, "launches": 3}), flush=True)


def run_gpu(wl, inp, steps, warmup):
    import numpy as np
    import torch

    import gen
    import sparse_mixture_experts_36_amd as moe

    tensors = layer_weights(inp)
    layer = moe.MoELayer(shape_for(wl), tensors)
    x = to_dev(inp.x)
    for _ in range(warmup):
        layer(x)
    torch.cuda.synchronize()
    moe.timing_start(8 * steps + 8)
    t0 = time.perf_counter()
    for _ in range(steps):
        layer(x)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stages = moe.timing_stop()
    latest = layer.latest()
    near = near_ties(layer.out.logits.cpu().numpy(), wl.top_k) if wl.gating != gen.EXPERT_CHOICE else None
    kept = int(sum(latest["kept"]))
    shared_rows = wl.n_shared * wl.T
    return {"ms_per_step": (t1 - t0) * 1e3 / steps, "stages": stages, "latest": latest, "kept": kept, "near": near,
            "rows": kept + shared_rows, "layer": layer, "tensors": tensors}


DECODE_WEIGHT_COPIES = 4  # consecutive decode steps read different copies of the weights


def run_decode(wl_prefill, inp, steps, warmup, Ts=(1, 16, 64)):
    """Decode shapes on the prefill weights. Each timed step takes a different
    slice of the prefill tokens and one of DECODE_WEIGHT_COPIES device copies of
    the layer's weights, in turn, so no step can find the weights it streams in
    the 256 MB last-level cache from the step before (each step reads at least
    two experts, 704 MB); the bytes of each step are counted from its own
    routing (read once before the timed loop)."""
    import numpy as np
    import torch

    import sparse_mixture_experts_36_amd as moe

    out = {}
    per_expert = [weight_bytes_per_expert(wl_prefill, e) for e in range(wl_prefill.n_experts)]
    x_all = to_dev(inp.x)
    copies = [layer_weights(inp) for _ in range(DECODE_WEIGHT_COPIES)]
    for T in Ts:
        wl = wl_prefill.with_(T=T)
        layers = [moe.MoELayer(shape_for(wl), tensors) for tensors in copies]
        nslices = min(steps, wl_prefill.T // T)
        xs = [x_all[i * T:(i + 1) * T].contiguous() for i in range(nslices)]
        lay = [layers[i % len(layers)] for i in range(nslices)]  # the copy step i reads
        layer = layers[0]
        touched, wbytes = [], []
        for li, xi in zip(lay, xs):
            o = li(xi)
            ex = set(o.topk_idx.cpu().numpy().ravel().tolist())
            touched.append(len(ex))
            wbytes.append(sum(per_expert[e] for e in ex))
        act_b = 2
        fixed = wl.n_experts * wl.d * act_b + 2 * T * wl.d * act_b  # router weight, x, y
        for _ in range(warmup):
            layer(xs[0])
        torch.cuda.synchronize()

        def timed(run):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            run()
            torch.cuda.synchronize()
            return (time.perf_counter() - t0) * 1e6 / nslices

        # eager launches, stage timing off
        us_eager = timed(lambda: [li(xi) for li, xi in zip(lay, xs)])
        # each step replayed from a captured HIP graph: no host launch gaps
        graphs = [li.capture(xi) for li, xi in zip(lay, xs)]
        for g in graphs[:warmup]:
            g.replay()
        us = timed(lambda: [g.replay() for g in graphs])
        del graphs
        # stage timing (hipEvents around the FFN launches) on a separate eager pass
        moe.timing_start(8 * nslices + 8)
        for li, xi in zip(lay, xs):
            li(xi)
        torch.cuda.synchronize()
        st = moe.timing_stop()
        nbytes = sum(b + fixed for b in wbytes) / nslices
        ffn_us = (st["ffn_up"][0] + st["ffn_down"][0]) * 1e3 / max(st["ffn_up"][1], 1)
        us_graph = us
        us = min(us_graph, us_eager)
        out[f"T{T}"] = {"us_per_step": round(us, 2), "launch": "graph" if us_graph <= us_eager else "eager",
                        "us_per_step_graph": round(us_graph, 2), "us_per_step_eager": round(us_eager, 2),
                        "touched_experts": round(sum(touched) / nslices, 2),
                        "GB": round(nbytes / 1e9, 4), "GB_per_s": round(nbytes / us / 1e3, 1),
                        "hbm_frac": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4),
                        "ffn_us": round(ffn_us, 2),
                        "ffn_GB_per_s": round((nbytes - fixed) / ffn_us / 1e3, 1),
                        "ffn_hbm_frac": round((nbytes - fixed) / ffn_us / 1e3 / PEAK_HBM_GBS, 4),
                        "steps": nslices, "weight_copies": len(layers)}
        log(f"decode T={T}: {out[f'T{T}']}")
    return out


def run_backward(wl, inp, steps, warmup):
    """moe_backward on the same layer and input with a seeded bf16 dy: dx and
    every weight gradient, L_aux and z terms on. One step recomputes the up
    GEMM (U = W1 x, V = W3 x) and runs the gradient GEMMs (dH = dy W2, dX =
    dU W1 + dV W3, dW2, dW1, dW3): per kept pair 3 x the up GEMM's flops plus
    2 x the down GEMM's (16 d d_ff for SwiGLU), plus the router's 5 x 2 d N per
    token. flops and MFMA fraction count all of them. Time from hipEvents
    around the whole step."""
    import torch

    import gen
    import sparse_mixture_experts_36_amd as moe

    shape = shape_for(wl)
    tensors = layer_weights(inp)
    w = moe.weights_struct(tensors)
    x = to_dev(inp.x)
    dy = to_dev(gen.normal(97, (wl.T, wl.d), 1.0, gen.BF16))
    g = moe.alloc_grads(shape)
    ws = moe.workspace(shape, moe.ENTRY_BACKWARD)
    for _ in range(warmup):
        moe.backward(shape, x, w, dy, g, 1.0, 1e-3, ws=ws)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(steps):
        moe.backward(shape, x, w, dy, g, 1.0, 1e-3, ws=ws)
    e1.record(s)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # rows: every kept pair (dropless here) plus T per shared expert
    rows = wl.T * wl.top_k + wl.n_shared * wl.T if wl.capacity() < 0 else None
    out = {"ms_per_step": round(ms, 4), "tokens_per_s": round(wl.T / (ms * 1e-3), 1),
           "workspace_GB": round(moe.workspace_size(shape, moe.ENTRY_BACKWARD) / 1e9, 3)}
    if rows is not None:
        flops = rows * (3 * up_flops_per_pair(wl) + 2 * 2.0 * wl.d * wl.d_ff) + 2.0 * wl.T * wl.d * wl.n_experts * 5
        out.update(flops_per_step=flops, TFLOP_per_s=round(flops / (ms * 1e-3) / 1e12, 1),
                   mfma_frac=round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4))
    log(f"backward: {out}")
    return out


def cpu_baseline(wl, inp, target_s=15.0):
    """The fp64 oracle, as it stands, on a bounded sample: the first S tokens as
    their own batch (S grown from 8 until one run takes a few seconds, then the
    sample is fixed so the timed run lasts about target_s)."""
    import numpy as np

    import gen
    import oracle

    def run(S):
        sub = gen.Inputs(wl.with_(T=S), inp.x[:S], inp.w_router, inp.b_router, inp.w1, inp.w3, inp.w2, inp.b1,
                         inp.b2, inp.w_scale, inp.sw1, inp.sw3, inp.sw2, inp.sw_scale)
        t = time.perf_counter()
        oracle.forward(sub)
        return time.perf_counter() - t

    run(4)  # first touch of the weight pages and the oracle library load
    S, dt = 8, run(8)
    while dt < 2.0 and S < wl.T:
        S = min(wl.T, S * 4)
        dt = run(S)
    S2 = int(min(wl.T, max(S, S * target_s / max(dt, 1e-3))))
    if S2 != S:
        S, dt = S2, run(S2)
    return {"value": round(S / dt, 3), "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"first {S} tokens of the {wl.name} input as one batch (all {wl.n_experts} experts' "
                      f"weights), fp64, {dt:.1f} s"}


NEAR_TIE = 1e-3  # the checking protocol's top-k margin threshold on the fp32 logits


def near_ties(logits, k: int) -> dict:
    """Tokens of the timed step whose top-k set margin l_(k) - l_(k+1) or
    slot-order margin min_j l_(j) - l_(j+1), j < k, is below 1e-3 on the
    layer's own fp32 logits: the tokens whose routing a last-bit change of a
    logit could move. (The tests compare these tokens' routing with the
    oracle's.)"""
    import numpy as np
    s = -np.sort(-logits.astype(np.float64), axis=1)
    n = s.shape[1]
    set_m = s[:, k - 1] - s[:, k] if k < n else np.full(s.shape[0], np.inf)
    order_m = (s[:, :k - 1] - s[:, 1:k]).min(1) if k > 1 else np.full(s.shape[0], np.inf)
    return {"threshold": NEAR_TIE, "set_margin_below": int((set_m < NEAR_TIE).sum()),
            "order_margin_below": int((order_m < NEAR_TIE).sum()),
            "either_below": int(((set_m < NEAR_TIE) | (order_m < NEAR_TIE)).sum()), "tokens": int(s.shape[0])}


def dropped_of(wl, latest) -> int:
    """Dropped (token, expert) pairs under token choice; under expert choice
    the tokens that no expert took."""
    import gen
    per = wl.T if wl.gating == gen.EXPERT_CHOICE else wl.T * wl.top_k
    return int(latest["dropped_share"] * per + 0.5)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mixtral-prefill-bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode shapes (T = 1, 16, 64) on the prefill weights; prints their JSON")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--backward-only", action="store_true",
                    help="only the layer backward (moe_backward) on the workload; prints its JSON")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only the copy kernel that scales the PMC byte counters")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="time only torch.matmul on one expert's GEMM shapes (context for the grouped GEMM)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch

    import gen
    import sparse_mixture_experts_36_amd as moe

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        copy_calibration()
        return
    if args.vendor_gemm:
        vendor_gemm_context()
        return
    moe.lib()  # raises when the HIP library is missing: there is no fallback
    wl = gen.WORKLOADS[args.workload]
    log(f"workload {wl}")
    t = time.perf_counter()
    inp = gen.make_inputs(wl)
    log(f"inputs generated in {time.perf_counter() - t:.1f} s")
    if args.decode_only:
        print(json.dumps({"decode": run_decode(wl, inp, max(args.steps, 16), args.warmup)}), flush=True)
        return
    if args.backward_only:
        print(json.dumps({"backward": run_backward(wl, inp, args.steps, args.warmup)}), flush=True)
        return

    r = run_gpu(wl, inp, args.steps, args.warmup)
    ms = r["ms_per_step"]
    st = r["stages"]
    log(f"ms/step {ms:.3f}; stages " + ", ".join(f"{k} {v[0] / max(v[1], 1):.3f} ms" for k, v in st.items()))
    up_ms = st["ffn_up"][0] / max(st["ffn_up"][1], 1)
    down_ms = st["ffn_down"][0] / max(st["ffn_down"][1], 1)
    up_flops = r["rows"] * up_flops_per_pair(wl)
    ffn_flops = r["rows"] * ffn_flops_per_pair(wl)
    router_flops = 2.0 * wl.T * wl.d * wl.n_experts
    bf16 = wl.act_dtype == gen.BF16
    achieved = up_flops / (up_ms * 1e-3) / 1e12
    lbytes, wbytes, touched = layer_bytes(wl, r["latest"]["kept"])
    result = {
        "metric": "MoE-layer tokens/s (Mixtral-shape prefill) + % bf16 MFMA peak; decode HBM GB/s",
        "value": round(wl.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/fan_in) weights)",
        "config": {"workload": wl.name, "T": wl.T, "d": wl.d, "d_ff": wl.d_ff, "n_experts": wl.n_experts,
                   "top_k": wl.top_k, "act": "swiglu" if wl.act == gen.SWIGLU else "gelu",
                   "gating": ["softmax_topk", "softmax_topk_renorm", "topk_softmax", "expert_choice"][wl.gating],
                   "capacity": wl.capacity(), "n_shared": wl.n_shared,
                   "w_dtype": {0: "f32", 1: "bf16", 2: "e4m3", 3: f"int8 x{wl.n_int8} + int4 x{wl.n_experts - wl.n_int8}"}[wl.w_dtype],
                   "parallelism": "single-gpu"},
        "roofline": {"kernel": "grouped up GEMM + fused activation", "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic() if wl.name == "mixtral-prefill-bf16" else None,
                     "algorithmic_flops_per_launch": up_flops, "mean_launch_ms": round(up_ms, 4)},
        "layer": {"mfma_frac": round((ffn_flops + router_flops) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                  "ffn_mfma_frac": round(ffn_flops / ((up_ms + down_ms) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                  "hbm_frac": round(lbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                  "ffn_hbm_frac": round(wbytes / ((up_ms + down_ms) * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                  "alg_bytes": lbytes, "expert_weight_bytes": wbytes, "touched_experts": touched,
                  "stage_ms": {k: round(v[0] / max(v[1], 1), 4) for k, v in st.items()},
                  "rows": r["rows"], "dropped": dropped_of(wl, r["latest"]), "near_tie_tokens": r["near"],
                  "l_aux": None if r["latest"]["aux_loss"] is None else round(r["latest"]["aux_loss"], 6),
                  "z_loss": round(r["latest"]["z_loss"], 5)},
    }
    if not args.no_decode and wl.name == "mixtral-prefill-bf16":
        del r
        result["decode"] = run_decode(wl, inp, max(args.steps, 16), args.warmup)
    if not args.no_backward and wl.name == "mixtral-prefill-bf16":
        result["backward"] = run_backward(wl, inp, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, inp)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
