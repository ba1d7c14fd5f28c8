"""The C ABI without a GPU: the library loads, exports every function that
include/moe.h declares, and rejects bad arguments on the host (before any
launch) with the documented status codes."""
import ctypes
import os
import re

import numpy as np
import pytest

import gen
import sparse_mixture_experts_36_amd as moe
from helpers import shape_of

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = _declared()
    assert {"moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_forward"} <= set(names)
    L = moe.lib()
    for n in names:
        assert hasattr(L, n), f"{n} declared in moe.h but not exported"
    assert L.moe_abi_version() == 1


def test_status_strings_and_capacity():
    L = moe.lib()
    for code in (0, -1, -2, -3, -4, 7):
        assert isinstance(L.moe_status_string(code), bytes)
    assert moe.capacity(256, 2, 8, 1.25) == 80
    assert moe.capacity(16384, 1, 64, 1.25) == 320
    assert moe.capacity(10, 1, 3, 1.0) == 3       # floor(3.33)
    assert moe.capacity(4096, 2, 8, None) == -1
    assert L.moe_capacity(10, 2, 0, 1.0) == -1


def _shape(**kw):
    base = dict(T=64, d=256, d_ff=512, n_experts=8, top_k=2, act=moe.SWIGLU, gating=moe.TOPK_SOFTMAX,
                act_dtype=moe.BF16, w_dtype=moe.BF16, capacity=-1)
    base.update(kw)
    return moe.make_shape(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(top_k=9, n_experts=16), moe.MOE_ERR_UNSUPPORTED),
    (dict(top_k=3, n_experts=2), moe.MOE_ERR_INVALID_ARG),
    (dict(top_k=0), moe.MOE_ERR_INVALID_ARG),
    (dict(n_experts=0), moe.MOE_ERR_INVALID_ARG),
    (dict(n_experts=300, top_k=2), moe.MOE_ERR_UNSUPPORTED),
    (dict(d=200), moe.MOE_ERR_UNSUPPORTED),
    (dict(d_ff=192), moe.MOE_ERR_UNSUPPORTED),
    (dict(act=5), moe.MOE_ERR_INVALID_ARG),
    (dict(gating=4), moe.MOE_ERR_INVALID_ARG),
    # expert choice: top_k 1 and 0 <= C <= T; at most 32768 tokens
    (dict(gating=moe.EXPERT_CHOICE, top_k=2, capacity=8), moe.MOE_ERR_INVALID_ARG),
    (dict(gating=moe.EXPERT_CHOICE, top_k=1, capacity=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(gating=moe.EXPERT_CHOICE, top_k=1, capacity=65), moe.MOE_ERR_INVALID_ARG),
    (dict(gating=moe.EXPERT_CHOICE, top_k=1, T=32769, capacity=8), moe.MOE_ERR_UNSUPPORTED),
    (dict(gating=moe.EXPERT_CHOICE, top_k=1, T=32768, d=65536, n_experts=256, capacity=32768),
     moe.MOE_ERR_UNSUPPORTED),
    (dict(act_dtype=moe.FP8_E4M3), moe.MOE_ERR_INVALID_ARG),
    (dict(act_dtype=moe.F32, w_dtype=moe.BF16), moe.MOE_ERR_UNSUPPORTED),
    (dict(act_dtype=moe.F32, w_dtype=moe.FP8_E4M3), moe.MOE_ERR_UNSUPPORTED),
    (dict(T=-1), moe.MOE_ERR_INVALID_ARG),
    (dict(capacity=-2), moe.MOE_ERR_INVALID_ARG),
    (dict(n_shared=5), moe.MOE_ERR_UNSUPPORTED),
    (dict(T=1, d=(1 << 20) + 128), moe.MOE_ERR_UNSUPPORTED),
    (dict(T=1, d_ff=(1 << 20) + 128), moe.MOE_ERR_UNSUPPORTED),
])
def test_invalid_shapes_rejected(kw, status):
    n = ctypes.c_size_t()
    assert moe.lib().moe_workspace_size(ctypes.byref(_shape(**kw)), moe.ENTRY_FORWARD, ctypes.byref(n)) == status


@pytest.mark.parametrize("T,C", [(64, 0), (64, 16), (64, 64), (32768, 8192)])
def test_expert_choice_shapes_accepted(T, C):
    s = _shape(T=T, top_k=1, gating=moe.EXPERT_CHOICE, capacity=C)
    sizes = [moe.workspace_size(s, e) for e in range(4)]
    # forward holds h and y_perm for the N*C routed rows
    assert sizes[3] >= 8 * C * (512 + 256) * 2
    rs = moe.routing_shapes(s)
    assert rs == {"topk": (8, C), "inv_map": (T, 8), "perm_token": (8 * C,)}


def test_expert_choice_capacity_is_the_pages_int():
    # int(num_tokens * capacity_factor / num_experts)
    for T, N, cf in [(4096, 8, 2.0), (8192, 160, 6.0), (256, 8, 2.0), (10, 3, 1.0), (100, 7, 1.25)]:
        assert moe.capacity(T, 1, N, cf) == int(T * cf / N)


def test_int_weights_shapes_and_packing():
    n = ctypes.c_size_t()
    ok = _shape(w_dtype=moe.INT_W)
    assert moe.lib().moe_workspace_size(ctypes.byref(ok), moe.ENTRY_FORWARD, ctypes.byref(n)) == moe.MOE_OK
    bad = _shape(w_dtype=moe.INT_W, act_dtype=moe.F32)
    assert moe.lib().moe_workspace_size(ctypes.byref(bad), moe.ENTRY_FORWARD, ctypes.byref(n)) == moe.MOE_ERR_UNSUPPORTED
    # byte rows: 8-bit experts verbatim, 4-bit experts two codes a byte (low nibble first)
    rng = np.random.default_rng(0)
    codes = np.concatenate([rng.integers(-127, 128, (1, 3, 8)), rng.integers(-7, 8, (2, 3, 8))]).astype(np.int8)
    packed = moe.pack_int_weights(codes, [8, 4, 4], pad=4)
    assert packed.shape == (3, 3, 12) and packed.dtype == np.uint8
    assert np.array_equal(packed[0, :, :8].view(np.int8), codes[0])
    for e in (1, 2):
        # one little-endian word per 8 codes: code 2j in bits 4j.., code 2j + 1 in bits 16 + 4j..
        word = packed[e, :, :4].copy().view("<u4")[:, 0]
        for j in range(4):
            for c, shift in ((2 * j, 4 * j), (2 * j + 1, 16 + 4 * j)):
                v = ((word >> shift) & 0xF).astype(np.int8)
                v[v > 7] -= 16
                assert np.array_equal(v, codes[e, :, c])
        assert (packed[e, :, 4:] == 0).all()


def test_workspace_sizes_grow_with_entry():
    s = _shape(T=4096, d=4096, d_ff=14336)
    sizes = [moe.workspace_size(s, e) for e in range(4)]
    assert all(v > 0 for v in sizes)
    # forward holds h, x_perm and y_perm: at least T*k*(d_ff + 2d) bf16 values
    assert sizes[3] >= 4096 * 2 * (14336 + 2 * 4096) * 2
    assert sizes[2] >= 4096 * 2 * 14336 * 2
    n = ctypes.c_size_t()
    assert moe.lib().moe_workspace_size(ctypes.byref(s), 9, ctypes.byref(n)) == moe.MOE_ERR_INVALID_ARG


def test_null_and_workspace_errors_return_before_launch():
    """These calls must fail on the host: no GPU exists here, so reaching a
    launch would report MOE_ERR_HIP instead of the expected code."""
    L = moe.lib()
    s = _shape()
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    # missing outputs
    assert L.moe_route(ctypes.byref(s), fake, fake, None, None, 0, fake, fake, None, fake, 1 << 20,
                       None) == moe.MOE_ERR_INVALID_ARG
    # unknown flag
    assert L.moe_route(ctypes.byref(s), fake, fake, None, fake, 6, fake, fake, None, fake, 1 << 20,
                       None) == moe.MOE_ERR_INVALID_ARG
    # workspace too small / misaligned / missing
    assert L.moe_route(ctypes.byref(s), fake, fake, None, fake, 0, fake, fake, None, fake, 16,
                       None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_route(ctypes.byref(s), fake, fake, None, fake, 0, fake, fake, None, ctypes.c_void_p((1 << 20) + 8),
                       1 << 30, None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_permute(ctypes.byref(s), fake, fake, fake, fake, fake, fake, None, None, 0,
                         None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_permute(ctypes.byref(s), None, fake, fake, fake, fake, fake, None, fake, 1 << 30,
                         None) == moe.MOE_ERR_INVALID_ARG
    # SwiGLU without W3
    w = moe.Weights(w_router=1 << 20, w1=1 << 20, w2=1 << 20)
    assert L.moe_grouped_ffn(ctypes.byref(s), fake, fake, None, ctypes.byref(w), fake, None, fake, 1 << 30,
                             None) == moe.MOE_ERR_INVALID_ARG
    # fp8 without scales
    s8 = _shape(w_dtype=moe.FP8_E4M3)
    w = moe.Weights(w_router=1 << 20, w1=1 << 20, w3=1 << 20, w2=1 << 20)
    assert L.moe_forward(ctypes.byref(s8), fake, ctypes.byref(w), fake, None, None, None, None, None, None, None,
                         fake, 1 << 34, None) == moe.MOE_ERR_INVALID_ARG
    # shared experts without their weights
    ss = _shape(n_shared=2)
    w = moe.Weights(w_router=1 << 20, w1=1 << 20, w3=1 << 20, w2=1 << 20)
    assert L.moe_forward(ctypes.byref(ss), fake, ctypes.byref(w), fake, None, None, None, None, None, None, None,
                         fake, 1 << 34, None) == moe.MOE_ERR_INVALID_ARG
    # misaligned activation pointer
    w = moe.Weights(w_router=1 << 20, w1=1 << 20, w3=1 << 20, w2=1 << 20)
    assert L.moe_forward(ctypes.byref(s), ctypes.c_void_p((1 << 20) + 2), ctypes.byref(w), fake, None, None, None,
                         None, None, None, None, fake, 1 << 34, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_combine(ctypes.byref(s), None, fake, fake, None, fake, None) == moe.MOE_ERR_INVALID_ARG
    # weight row pitches: shorter than a row, or not a multiple of 16
    for ld_up, ld_down in ((s.d - 16, 0), (s.d + 8, 0), (0, s.d_ff - 16), (0, s.d_ff + 4)):
        w = moe.Weights(w_router=1 << 20, w1=1 << 20, w3=1 << 20, w2=1 << 20, ld_up=ld_up, ld_down=ld_down)
        assert L.moe_forward(ctypes.byref(s), fake, ctypes.byref(w), fake, None, None, None, None, None, None,
                             None, fake, 1 << 34, None) == moe.MOE_ERR_INVALID_ARG, (ld_up, ld_down)
    # pitches past 2^21 elements: valid, but beyond the 32-bit row offsets of the kernels
    for ld_up, ld_down in (((1 << 21) + 16, 0), (0, (1 << 21) + 16)):
        w = moe.Weights(w_router=1 << 20, w1=1 << 20, w3=1 << 20, w2=1 << 20, ld_up=ld_up, ld_down=ld_down)
        assert L.moe_forward(ctypes.byref(s), fake, ctypes.byref(w), fake, None, None, None, None, None, None,
                             None, fake, 1 << 34, None) == moe.MOE_ERR_UNSUPPORTED, (ld_up, ld_down)


def test_weight_row_pitches_come_from_tensor_strides():
    import torch
    w1 = moe.padded(torch.zeros(3, 8, 32), 16)
    w3 = moe.padded(torch.ones(3, 8, 32), 16)
    w2 = moe.padded(torch.zeros(3, 32, 8), 24)
    assert w1.shape == (3, 8, 32) and w1.stride() == (8 * 48, 48, 1) and float(w3.sum()) == 3 * 8 * 32
    w = moe.weights_struct({"w1": w1, "w3": w3, "w2": w2})
    assert (w.ld_up, w.ld_down) == (48, 32)
    w = moe.weights_struct({"w1": torch.zeros(3, 8, 32), "w2": torch.zeros(3, 32, 8)})
    assert (w.ld_up, w.ld_down) == (32, 8)
    with pytest.raises(ValueError):  # W1 and W3 with different pitches
        moe.weights_struct({"w1": w1, "w3": torch.zeros(3, 8, 32), "w2": w2})
    with pytest.raises(ValueError):  # a gap between experts
        moe.weights_struct({"w1": torch.zeros(3, 16, 32)[:, :8], "w2": w2})


def test_host_helpers_reproduce_pages_worked_examples():
    """aigrafen.se 'Mixture of Experts': the parameter-count example prints
    45.1 / 11.3 / 4.0 and the entropy example 0.783 / 2.079 of max 2.079."""
    import json
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "aigrafen_worked_examples.json")))
    a = g["parameters"]["args"]
    per = moe.expert_params(a["d"], a["hidden"], moe.SWIGLU)
    total, active = a["layers"] * a["n_experts"] * per, a["layers"] * a["k"] * per
    pr = g["parameters"]["printed"]
    assert round(total / 1e9, 1) == pr["total_bn"] and round(active / 1e9, 1) == pr["active_bn"]
    assert round(total / active, 1) == pr["ratio"]
    ent = g["entropy"]
    for name in ("collapsed", "balanced"):
        assert round(moe.routing_entropy(ent[name]["f"]), ent["digits"]) == ent[name]["printed"]
    assert round(__import__("math").log(8), 3) == ent["max_printed"]


def test_backward_host_checks_return_before_launch():
    """moe_backward's validation, all on the host (a launch would report
    MOE_ERR_HIP here, where no GPU exists)."""
    L = moe.lib()
    fake = ctypes.c_void_p(1 << 20)
    s = _shape(act_dtype=moe.BF16, w_dtype=moe.BF16)
    w = moe.Weights(w_router=1 << 20, w1=1 << 20, w3=1 << 20, w2=1 << 20)
    g = moe.Grads(dx=1 << 20)
    n = ctypes.c_size_t()
    assert L.moe_workspace_size(ctypes.byref(s), moe.ENTRY_BACKWARD, ctypes.byref(n)) == moe.MOE_OK
    # the backward keeps U, V, H, dH, dU, dV and dX over every row
    rows = s.T * s.top_k
    assert n.value >= rows * s.d_ff * (4 + 4 + 2 + 4 + 2 + 2) + rows * s.d * 4
    assert L.moe_backward(ctypes.byref(s), fake, ctypes.byref(w), fake, 0.0, 0.0, ctypes.byref(g), fake, 16,
                          None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_backward(ctypes.byref(s), fake, ctypes.byref(w), None, 0.0, 0.0, ctypes.byref(g), fake, 1 << 40,
                          None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_backward(ctypes.byref(s), fake, ctypes.byref(w), fake, 0.0, 0.0, ctypes.byref(moe.Grads()), fake,
                          1 << 40, None) == moe.MOE_ERR_INVALID_ARG
    # router weight required
    w0 = moe.Weights(w1=1 << 20, w3=1 << 20, w2=1 << 20)
    assert L.moe_backward(ctypes.byref(s), fake, ctypes.byref(w0), fake, 0.0, 0.0, ctypes.byref(g), fake, 1 << 40,
                          None) == moe.MOE_ERR_INVALID_ARG
    # bf16 token choice only
    for kw in (dict(), dict(act_dtype=moe.BF16, w_dtype=moe.FP8_E4M3), dict(act_dtype=moe.F32, w_dtype=moe.F32),
               dict(act_dtype=moe.BF16, w_dtype=moe.BF16, gating=moe.EXPERT_CHOICE, top_k=1, capacity=8)):
        su = _shape(**kw) if kw else _shape(act_dtype=moe.BF16, w_dtype=moe.INT_W)
        assert L.moe_backward(ctypes.byref(su), fake, ctypes.byref(w), fake, 0.0, 0.0, ctypes.byref(g), fake,
                              1 << 40, None) == moe.MOE_ERR_UNSUPPORTED, kw


def test_ffn_path_of_each_workload():
    """moe_ffn_path (host only): the kernel family each workload's expert FFN
    takes, and the backward recompute's."""
    expect = {
        "tiny-gelu-fp32": moe.PATH_F32,
        "mixtral-prefill-bf16": moe.PATH_DMA256,
        "fine-grained-160x6-shared2-bf16": moe.PATH_DMA256,
        "switch-top1-bf16": moe.PATH_DMA128,
        "switch-top1-fp8w": moe.PATH_DMA128,
        "mixtral-prefill-int8x2-int4x6": moe.PATH_DMA256,
    }
    for name, path in expect.items():
        wl = gen.WORKLOADS[name]
        assert moe.ffn_path(shape_of(wl)) == path, name
    for T in (1, 16, 64):
        assert moe.ffn_path(shape_of(gen.MIXTRAL_DECODE[T])) == moe.PATH_STREAM
    assert moe.ffn_path(shape_of(gen.MIXTRAL_PREFILL), moe.ENTRY_BACKWARD) == moe.PATH_DMA256
    assert moe.ffn_path(shape_of(gen.MIXTRAL_PREFILL.with_(T=512)), moe.ENTRY_BACKWARD) == moe.PATH_BGEMM
    with pytest.raises(moe.MoEError):
        moe.ffn_path(shape_of(gen.MIXTRAL_PREFILL), moe.ENTRY_ROUTE)
