"""Seeded synthetic inputs for the MoE layer forward (shared by tests, bench and smoke).

This package only draws numbers and names workload shapes. It holds none of
the layer's arithmetic (no routing, no expert math), so that the GPU library
and the CPU oracle can both be fed from it without sharing any of the method.

Recipe (counter-based, see ``gen.c``): element i of tensor ``tau`` is
``scale * N(0,1)`` drawn from SplitMix64(seed ^ (tau << 40) ^ i) and Box-Muller,
rounded to the storage dtype. Seed 36 unless a test says otherwise.
Tensor ids: 1 x, 2 router weight, 3 W1, 4 W3, 5 W2, 6 b1, 7 b2, 8-10 shared
W1/W3/W2, 11 given logits (routing-only tests).
Weights are N(0, 1/fan_in) (fan_in = d for router, W1, W3; d_ff for W2), the
``nn.Linear`` layout [out][in], stacked per expert. GELU biases are zero.
Router skew: a fp32 per-expert logit bias b_e = -s*ln(e+1), whose softmax is
exactly the Zipf(s) law over experts 0..N-1 (expert 0 the most popular).
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgen.so")
SEED = 36

T_X, T_WR, T_W1, T_W3, T_W2, T_B1, T_B2, T_SW1, T_SW3, T_SW2, T_LOGITS = range(1, 12)

# dtype codes shared by convention with every consumer (plain integers)
F32, BF16, E4M3 = 0, 1, 2
INT_W = 3  # weight-only integers: 8 or 4 bits per expert, one fp32 scale per weight row
# activation / gating codes
GELU, SWIGLU = 0, 1
SOFTMAX_TOPK, SOFTMAX_TOPK_RENORM, TOPK_SOFTMAX = 0, 1, 2
EXPERT_CHOICE = 3  # each expert takes its C tokens (top_k is 1, C = floor(cf*T/N))


def build(verbose: bool = False) -> str:
    """Compile libgen.so with gcc (OpenMP)."""
    import subprocess

    src = os.path.join(_HERE, "gen.c")
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", LIB_PATH, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        u64, u32, dbl, i32, vp = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_double,
                                  ctypes.c_int32, ctypes.c_void_p)
        L.gen_normal_f32.argtypes = [u64, u32, u64, u64, dbl, vp]
        L.gen_normal_bf16.argtypes = [u64, u32, u64, u64, dbl, vp]
        L.gen_grid_f32.argtypes = [u64, u32, u64, u64, dbl, i32, i32, vp]
        L.gen_grid_bf16.argtypes = [u64, u32, u64, u64, dbl, i32, i32, vp]
        L.gen_e4m3_groups.argtypes = [u64, u32, u64, u64, u64, dbl, vp, vp, u64]
        L.gen_int_rows.argtypes = [u64, u32, u64, u64, u64, dbl, i32, vp, vp, u64]
        L.gen_bf16_of.argtypes = [ctypes.c_float]
        L.gen_bf16_of.restype = ctypes.c_uint16
        L.gen_e4m3_of.argtypes = [dbl]
        L.gen_e4m3_of.restype = ctypes.c_uint8
        L.gen_normal_at.argtypes = [u64, u32, u64]
        L.gen_normal_at.restype = dbl
        for f in (L.gen_normal_f32, L.gen_normal_bf16, L.gen_grid_f32, L.gen_grid_bf16,
                  L.gen_e4m3_groups, L.gen_int_rows):
            f.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def normal(tensor: int, shape, scale: float, dtype: int, seed: int = SEED, offset: int = 0) -> np.ndarray:
    """scale*N(0,1) draws of `tensor`; fp32 (float32 array) or bf16 (uint16 bit patterns)."""
    n = int(np.prod(shape))
    if dtype == F32:
        out = np.empty(shape, np.float32)
        lib().gen_normal_f32(seed, tensor, offset, n, scale, _ptr(out))
    elif dtype == BF16:
        out = np.empty(shape, np.uint16)
        lib().gen_normal_bf16(seed, tensor, offset, n, scale, _ptr(out))
    else:
        raise ValueError("normal(): dtype must be F32 or BF16")
    return out


def grid(tensor: int, shape, scale_int: float, limit: int, frac_bits: int, dtype: int,
         seed: int = SEED, offset: int = 0) -> np.ndarray:
    """round(scale_int*N(0,1)) clamped to +-limit, divided by 2^frac_bits."""
    n = int(np.prod(shape))
    if dtype == F32:
        out = np.empty(shape, np.float32)
        lib().gen_grid_f32(seed, tensor, offset, n, scale_int, limit, frac_bits, _ptr(out))
    elif dtype == BF16:
        out = np.empty(shape, np.uint16)
        lib().gen_grid_bf16(seed, tensor, offset, n, scale_int, limit, frac_bits, _ptr(out))
    else:
        raise ValueError("grid(): dtype must be F32 or BF16")
    return out


def e4m3_groups(tensor: int, n_groups: int, group_shape, scale: float, seed: int = SEED,
                scales_out: np.ndarray | None = None, scale_col: int = 0):
    """e4m3fn codes [n_groups, *group_shape] (uint8) and one fp32 scale per group."""
    ge = int(np.prod(group_shape))
    q = np.empty((n_groups,) + tuple(group_shape), np.uint8)
    if scales_out is None:
        s = np.empty((n_groups,), np.float32)
        lib().gen_e4m3_groups(seed, tensor, 0, n_groups, ge, scale, _ptr(q), _ptr(s), 1)
        return q, s
    assert scales_out.dtype == np.float32 and scales_out.flags["C_CONTIGUOUS"]
    stride = scales_out.shape[1]
    base = scales_out.ctypes.data + 4 * scale_col
    lib().gen_e4m3_groups(seed, tensor, 0, n_groups, ge, scale, _ptr(q), base, stride)
    return q, scales_out[:, scale_col]


def int_rows(tensor: int, shape, scale: float, bits: int, seed: int = SEED, offset: int = 0,
             scales_out: np.ndarray | None = None):
    """Integer weight rows [rows, cols] (int8 codes within +-(2^(bits-1) - 1),
    one per byte) and their fp32 row scales: round-half-even(w / s_r) with
    s_r = amax_r / qmax, w the fp32-rounded draws scale*N(0,1)."""
    rows, cols = shape
    q = np.empty((rows, cols), np.int8)
    s = np.empty(rows, np.float32) if scales_out is None else scales_out
    assert s.dtype == np.float32 and s.flags["C_CONTIGUOUS"] and s.shape == (rows,)
    lib().gen_int_rows(seed, tensor, offset, rows, cols, scale, (1 << (bits - 1)) - 1, _ptr(q), _ptr(s), 1)
    return q, s


def zipf_bias(n_experts: int, s: float) -> np.ndarray:
    """b_e = -s*ln(e+1): softmax(b) is the Zipf(s) law over experts."""
    return np.array([-s * math.log(e + 1) for e in range(n_experts)], np.float32)


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    d_ff: int
    n_experts: int
    top_k: int
    act: int
    gating: int
    act_dtype: int
    w_dtype: int
    capacity_factor: float | None  # None = dropless
    n_shared: int = 0
    zipf_s: float | None = None
    aux_alpha: float = 0.01
    n_int8: int = 0  # INT_W weights: experts 0 .. n_int8-1 take 8 bits, the others 4; shared experts 8

    def expert_bits(self) -> np.ndarray:
        """Bits per routed expert under INT_W weights (8 for the high-traffic ones)."""
        return np.array([8 if e < self.n_int8 else 4 for e in range(self.n_experts)], np.uint8)

    def capacity(self) -> int:
        """floor(cf*T*k/N) in fp64, or -1 for dropless."""
        if self.capacity_factor is None:
            return -1
        return int(math.floor(self.capacity_factor * self.T * self.top_k / self.n_experts))

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads: tiny GELU fp32; Mixtral-shape prefill; Mixtral-shape decode
# (T in {1,16,64}); fine-grained 160/6 + 2 shared; Switch top-1 with dropping.
TINY_GELU = Workload("tiny-gelu-fp32", 256, 512, 2048, 8, 2, GELU, SOFTMAX_TOPK_RENORM, F32, F32, 1.25)
MIXTRAL_PREFILL = Workload("mixtral-prefill-bf16", 4096, 4096, 14336, 8, 2, SWIGLU, TOPK_SOFTMAX, BF16, BF16, None)
MIXTRAL_DECODE = {T: MIXTRAL_PREFILL.with_(name=f"mixtral-decode-bf16-T{T}", T=T) for T in (1, 16, 64)}
FINE_GRAINED = Workload("fine-grained-160x6-shared2-bf16", 8192, 5120, 1536, 160, 6, SWIGLU, SOFTMAX_TOPK,
                        BF16, BF16, None, n_shared=2, zipf_s=1.0)
SWITCH_TOP1 = Workload("switch-top1-bf16", 16384, 1024, 4096, 64, 1, GELU, SOFTMAX_TOPK, BF16, BF16, 1.25,
                       zipf_s=1.2)
SWITCH_TOP1_FP8 = SWITCH_TOP1.with_(name="switch-top1-fp8w", w_dtype=E4M3)

# Expert-choice routing on the same layers: cf = 2 gives the Mixtral layer the
# rows of its top-2 token-choice form (C = 1024 tokens per expert at T = 4096).
TINY_GELU_EC = TINY_GELU.with_(name="tiny-gelu-fp32-ec", top_k=1, gating=EXPERT_CHOICE, capacity_factor=2.0)
MIXTRAL_PREFILL_EC = MIXTRAL_PREFILL.with_(name="mixtral-prefill-ec-bf16", top_k=1, gating=EXPERT_CHOICE,
                                           capacity_factor=2.0)
FINE_GRAINED_EC = FINE_GRAINED.with_(name="fine-grained-160-ec-shared2-bf16", top_k=1, gating=EXPERT_CHOICE,
                                     capacity_factor=6.0)

# Per-expert integer weights on the Mixtral layer: the two high-traffic experts
# (0 and 1) in INT8, the other six in INT4, one fp32 scale per weight row.
MIXTRAL_PREFILL_INT = MIXTRAL_PREFILL.with_(name="mixtral-prefill-int8x2-int4x6", w_dtype=INT_W, n_int8=2)
MIXTRAL_DECODE_INT = {T: MIXTRAL_PREFILL_INT.with_(name=f"mixtral-decode-int8x2-int4x6-T{T}", T=T)
                      for T in (1, 16, 64)}

WORKLOADS = {w.name: w for w in [TINY_GELU, MIXTRAL_PREFILL, *MIXTRAL_DECODE.values(), FINE_GRAINED,
                                  SWITCH_TOP1, SWITCH_TOP1_FP8, TINY_GELU_EC, MIXTRAL_PREFILL_EC,
                                  FINE_GRAINED_EC, MIXTRAL_PREFILL_INT, *MIXTRAL_DECODE_INT.values()]}


@dataclass
class Inputs:
    """Host-side input buffers (numpy). bf16 tensors are uint16 bit patterns."""
    wl: Workload
    x: np.ndarray
    w_router: np.ndarray
    b_router: np.ndarray | None
    w1: np.ndarray
    w3: np.ndarray | None
    w2: np.ndarray
    b1: np.ndarray | None
    b2: np.ndarray | None
    w_scale: np.ndarray | None       # [N][3] fp32 (W1, W3, W2) for e4m3 weights; [N][2 d_ff + d] row scales for INT_W
    sw1: np.ndarray | None = None
    sw3: np.ndarray | None = None
    sw2: np.ndarray | None = None
    sw_scale: np.ndarray | None = None
    w_bits: np.ndarray | None = None   # INT_W: [N] uint8, 8 or 4
    sw_bits: np.ndarray | None = None  # INT_W: [n_shared] uint8 (8)


def _weights(wl: Workload, ids, n: int, seed: int, bits=None):
    """Stacked expert weights for n experts: (w1, w3, w2, scales)."""
    t1, t3, t2 = ids
    s_in, s_hid = 1.0 / math.sqrt(wl.d), 1.0 / math.sqrt(wl.d_ff)
    shp1, shp2 = (wl.d_ff, wl.d), (wl.d, wl.d_ff)
    swiglu = wl.act == SWIGLU
    if wl.w_dtype == INT_W:
        # codes [n][rows][cols] (int8, one per weight) and row scales
        # [n][2 d_ff + d]: W1 rows, W3 rows (ones for GELU), W2 rows
        f, d = wl.d_ff, wl.d
        sc = np.ones((n, 2 * f + d), np.float32)
        w1 = np.empty((n,) + shp1, np.int8)
        w3 = np.empty((n,) + shp1, np.int8) if swiglu else None
        w2 = np.empty((n,) + shp2, np.int8)
        for e in range(n):
            b = int(bits[e])
            w1[e] = int_rows(t1, shp1, s_in, b, seed, e * f * d, sc[e, :f])[0]
            if swiglu:
                w3[e] = int_rows(t3, shp1, s_in, b, seed, e * f * d, sc[e, f:2 * f])[0]
            w2[e] = int_rows(t2, shp2, s_hid, b, seed, e * d * f, sc[e, 2 * f:])[0]
        return w1, w3, w2, sc
    if wl.w_dtype == E4M3:
        sc = np.ones((n, 3), np.float32)
        w1, _ = e4m3_groups(t1, n, shp1, s_in, seed, sc, 0)
        w3 = e4m3_groups(t3, n, shp1, s_in, seed, sc, 1)[0] if swiglu else None
        w2, _ = e4m3_groups(t2, n, shp2, s_hid, seed, sc, 2)
        return w1, w3, w2, sc
    w1 = normal(t1, (n,) + shp1, s_in, wl.w_dtype, seed)
    w3 = normal(t3, (n,) + shp1, s_in, wl.w_dtype, seed) if swiglu else None
    w2 = normal(t2, (n,) + shp2, s_hid, wl.w_dtype, seed)
    return w1, w3, w2, None


def make_inputs(wl: Workload, seed: int = SEED, router_grid: bool = False) -> Inputs:
    """All inputs of one workload.

    router_grid=True draws x and the router weight on fixed-point grids
    (x = i/16, |i| <= 255; W_r = j/2^p, |j| <= 255) and puts the Zipf bias on the
    2^-(4+p) grid, so that every router logit is an exact fp32 number under any
    summation order (the dot products' magnitude stays far below 2^24 grid units;
    tests check that bound on the host).
    """
    N, d = wl.n_experts, wl.d
    if router_grid:
        p = int(math.ceil(math.log2(32.0 * math.sqrt(d))))
        x = grid(T_X, (wl.T, d), 16.0, 255, 4, wl.act_dtype, seed)
        wr = grid(T_WR, (N, d), 2.0 ** p / math.sqrt(d), 255, p, wl.act_dtype, seed)
    else:
        x = normal(T_X, (wl.T, d), 1.0, wl.act_dtype, seed)
        wr = normal(T_WR, (N, d), 1.0 / math.sqrt(d), wl.act_dtype, seed)
    b_router = None
    if wl.zipf_s is not None:
        b_router = zipf_bias(N, wl.zipf_s)
        if router_grid:
            q = float(2 ** (4 + p))
            b_router = (np.round(b_router.astype(np.float64) * q) / q).astype(np.float32)
    bits = wl.expert_bits() if wl.w_dtype == INT_W else None
    w1, w3, w2, sc = _weights(wl, (T_W1, T_W3, T_W2), N, seed, bits)
    b1 = b2 = None
    if wl.act == GELU:
        b1 = np.zeros((N, wl.d_ff), np.float32)
        b2 = np.zeros((N, d), np.float32)
    inp = Inputs(wl, x, wr, b_router, w1, w3, w2, b1, b2, sc, w_bits=bits)
    if wl.n_shared:
        sbits = np.full(wl.n_shared, 8, np.uint8) if wl.w_dtype == INT_W else None
        inp.sw1, inp.sw3, inp.sw2, inp.sw_scale = _weights(wl, (T_SW1, T_SW3, T_SW2), wl.n_shared, seed, sbits)
        inp.sw_bits = sbits
    return inp


def given_logits(T: int, N: int, seed: int = SEED, step: float | None = 0.25,
                 bias: np.ndarray | None = None) -> np.ndarray:
    """fp32 logits [T, N] for routing-only tests: N(0,1) draws, optionally put on a
    coarse grid of `step` so that exact ties between experts occur often."""
    l = normal(T_LOGITS, (T, N), 1.0, F32, seed).astype(np.float64)
    if step is not None:
        l = np.round(l / step) * step
    if bias is not None:
        l = l + bias.astype(np.float64)[None, :]
    return l.astype(np.float32)


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    return (a.astype(np.uint32) << 16).view(np.float32)
