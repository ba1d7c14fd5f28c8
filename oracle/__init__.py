"""CPU oracle for the MoE layer forward -- TEST INFRASTRUCTURE ONLY.

ctypes wrapper around ``moe_oracle.cpp`` (plain C++17, fp64, per-expert masked
loop). Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package; the GPU library never calls it and it
never calls the GPU library.

Inputs come from the ``gen`` package (host numpy buffers); no input and no
expected value here is ever produced by the GPU path.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC = os.path.join(_HERE, "moe_oracle.cpp")


class OrcShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int64), ("d_ff", ctypes.c_int64),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("act", ctypes.c_int32), ("gating", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("w_dtype", ctypes.c_int32), ("capacity", ctypes.c_int64), ("aux_alpha", ctypes.c_double)]


class OrcWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_router", "b_router", "w1", "w3", "w2", "b1", "b2", "w_scale", "sw1", "sw3", "sw2",
                 "sw_scale")]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile liboracle.so with g++ (OpenMP). sanitize=True adds ASan/UBSan."""
    cmd = ["g++", "-std=c++17", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", LIB_PATH, SRC]
    if sanitize:
        cmd[3:3] = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer"]
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
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        sp, wp = ctypes.POINTER(OrcShape), ctypes.POINTER(OrcWeights)
        L.orc_router_logits.argtypes = [sp, vp, wp, vp, vp]
        L.orc_route.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.orc_dispatch.argtypes = [sp, vp, vp, vp, vp, vp, vp]
        L.orc_expert_rows.argtypes = [sp, wp, i32, i32, vp, i64, vp]
        L.orc_moe_output.argtypes = [sp, vp, wp, vp, vp, vp, vp, i64, vp]
        L.orc_combine.argtypes = [sp, vp, vp, vp, vp, vp]
        L.orc_route_ec.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp]
        L.orc_dispatch_ec.argtypes = [sp, vp, vp, vp, vp, vp]
        L.orc_moe_output_ec.argtypes = [sp, vp, wp, vp, vp, vp, i64, vp]
        L.orc_combine_ec.argtypes = [sp, vp, vp, vp, vp, vp]
        L.orc_backward.argtypes = [sp, vp, wp, vp, ctypes.c_double, ctypes.c_double] + [vp] * 11
        L.orc_backward_sampled.argtypes = [sp, vp, wp, vp, ctypes.c_double, ctypes.c_double, vp, ctypes.c_int64, vp,
                                           vp, ctypes.c_int64, vp, vp, vp]
        for name in ("orc_router_logits", "orc_route", "orc_dispatch", "orc_expert_rows",
                     "orc_moe_output", "orc_combine", "orc_route_ec", "orc_dispatch_ec", "orc_moe_output_ec",
                     "orc_combine_ec", "orc_backward", "orc_backward_sampled", "orc_abi_version", "orc_threads"):
            getattr(L, name).restype = ctypes.c_int
        for name in ("orc_bf16_value", "orc_gelu", "orc_silu"):
            getattr(L, name).restype = ctypes.c_double
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_gelu.argtypes = [ctypes.c_double]
        L.orc_silu.argtypes = [ctypes.c_double]
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def shape_of(wl, T: int | None = None, capacity: int | None = None) -> OrcShape:
    """OrcShape for a gen.Workload (T and capacity may be overridden)."""
    return OrcShape(T=wl.T if T is None else T, d=wl.d, d_ff=wl.d_ff, n_experts=wl.n_experts,
                    top_k=wl.top_k, n_shared=wl.n_shared, act=wl.act, gating=wl.gating,
                    act_dtype=wl.act_dtype, w_dtype=wl.w_dtype,
                    capacity=wl.capacity() if capacity is None else capacity, aux_alpha=wl.aux_alpha)


def weights_of(inp) -> tuple[OrcWeights, list]:
    keep = [inp.w_router, inp.b_router, inp.w1, inp.w3, inp.w2, inp.b1, inp.b2, inp.w_scale,
            inp.sw1, inp.sw3, inp.sw2, inp.sw_scale]
    w = OrcWeights(*[_p(a) for a in keep])
    return w, keep


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: arguments outside the contract")


def router_logits(shape: OrcShape, x, inp):
    w, _keep = weights_of(inp)
    l64 = np.empty((shape.T, shape.n_experts), np.float64)
    l32 = np.empty((shape.T, shape.n_experts), np.float32)
    _check(lib().orc_router_logits(ctypes.byref(shape), _p(x), ctypes.byref(w), _p(l64), _p(l32)),
           "router_logits")
    return l64, l32


@dataclass
class Routing:
    topk_idx: np.ndarray   # [T,k] int32
    topk_w: np.ndarray     # [T,k] fp64
    probs: np.ndarray      # [T,N] fp64
    lse: np.ndarray        # [T]
    margin_set: np.ndarray
    margin_order: np.ndarray
    counts: np.ndarray     # [N] int64, before drops
    f: np.ndarray
    P: np.ndarray
    l_aux: float
    z: float
    lse_sq_mean: float


def route(shape: OrcShape, logits32: np.ndarray) -> Routing:
    T, N, k = shape.T, shape.n_experts, shape.top_k
    logits32 = np.ascontiguousarray(logits32, np.float32)
    assert logits32.shape == (T, N)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    probs = np.empty((T, N), np.float64)
    lse = np.empty(T, np.float64)
    ms, mo = np.empty(T, np.float64), np.empty(T, np.float64)
    counts = np.empty(N, np.int64)
    f, P = np.empty(N, np.float64), np.empty(N, np.float64)
    la, z, lsq = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _check(lib().orc_route(ctypes.byref(shape), _p(logits32), _p(idx), _p(w), _p(probs), _p(lse), _p(ms),
                           _p(mo), _p(counts), _p(f), _p(P), ctypes.addressof(la), ctypes.addressof(z),
                           ctypes.addressof(lsq)), "route")
    return Routing(idx, w, probs, lse, ms, mo, counts, f, P, la.value, z.value, lsq.value)


@dataclass
class Dispatch:
    kept: np.ndarray        # [N] int32
    offsets: np.ndarray     # [N+1] int32
    perm_token: np.ndarray  # [T*k] int32 (rows >= M are -1)
    inv_map: np.ndarray     # [T,k] int32 (-1 = dropped)
    n_dropped: int


def dispatch(shape: OrcShape, topk_idx: np.ndarray) -> Dispatch:
    T, N, k = shape.T, shape.n_experts, shape.top_k
    topk_idx = np.ascontiguousarray(topk_idx, np.int32)
    kept = np.empty(N, np.int32)
    off = np.empty(N + 1, np.int32)
    perm = np.empty(T * k, np.int32)
    inv = np.empty((T, k), np.int32)
    nd = ctypes.c_int64()
    _check(lib().orc_dispatch(ctypes.byref(shape), _p(topk_idx), _p(kept), _p(off), _p(perm), _p(inv),
                              ctypes.addressof(nd)), "dispatch")
    return Dispatch(kept, off, perm, inv, nd.value)


def expert_rows(shape: OrcShape, inp, e: int, X: np.ndarray, shared: bool = False) -> np.ndarray:
    w, _keep = weights_of(inp)
    X = np.ascontiguousarray(X)
    n = X.shape[0]
    Y = np.empty((n, shape.d), np.float64)
    _check(lib().orc_expert_rows(ctypes.byref(shape), ctypes.byref(w), int(shared), e, _p(X), n, _p(Y)),
           "expert_rows")
    return Y


def moe_output(shape: OrcShape, x, inp, routing: Routing, disp: Dispatch | None,
               tokens: np.ndarray) -> np.ndarray:
    w, _keep = weights_of(inp)
    tokens = np.ascontiguousarray(tokens, np.int64)
    y = np.empty((len(tokens), shape.d), np.float64)
    inv = None if disp is None else disp.inv_map
    _check(lib().orc_moe_output(ctypes.byref(shape), _p(x), ctypes.byref(w), _p(routing.topk_idx),
                                _p(np.ascontiguousarray(routing.topk_w)), _p(inv), _p(tokens), len(tokens),
                                _p(y)), "moe_output")
    return y


def combine(shape: OrcShape, y_perm, inv_map, topk_w32, y_shared=None) -> np.ndarray:
    y = np.empty((shape.T, shape.d), np.float64)
    _check(lib().orc_combine(ctypes.byref(shape), _p(y_perm), _p(np.ascontiguousarray(inv_map, np.int32)),
                             _p(np.ascontiguousarray(topk_w32, np.float32)), _p(y_shared), _p(y)), "combine")
    return y


EXPERT_CHOICE = 3  # OrcShape.gating of expert-choice routing


@dataclass
class RoutingEC:
    ec_token: np.ndarray   # [N,C] int32, ascending per expert
    ec_gate: np.ndarray    # [N,C] fp64 column-softmax probabilities
    probs: np.ndarray      # [T,N] fp64 softmax over tokens, per expert
    lse: np.ndarray        # [T] per-token logsumexp over experts
    z: float
    lse_sq_mean: float


def route_ec(shape: OrcShape, logits32: np.ndarray) -> RoutingEC:
    """Expert-choice selection and gates from fp32 logits [T,N] (shape.gating 3)."""
    T, N, C = shape.T, shape.n_experts, shape.capacity
    logits32 = np.ascontiguousarray(logits32, np.float32)
    assert logits32.shape == (T, N)
    tok = np.empty((N, C), np.int32)
    gate = np.empty((N, C), np.float64)
    probs = np.empty((T, N), np.float64)
    lse = np.empty(T, np.float64)
    z, lsq = ctypes.c_double(), ctypes.c_double()
    _check(lib().orc_route_ec(ctypes.byref(shape), _p(logits32), _p(tok), _p(gate), _p(probs), _p(lse),
                              ctypes.addressof(z), ctypes.addressof(lsq)), "route_ec")
    return RoutingEC(tok, gate, probs, lse, z.value, lsq.value)


def dispatch_ec(shape: OrcShape, ec_token: np.ndarray) -> Dispatch:
    """Row layout of expert-choice assignments: rows e*C + j; inv_map [T,N];
    n_dropped = tokens that no expert took."""
    T, N, C = shape.T, shape.n_experts, shape.capacity
    ec_token = np.ascontiguousarray(ec_token, np.int32)
    off = np.empty(N + 1, np.int32)
    perm = np.empty(N * C, np.int32)
    inv = np.empty((T, N), np.int32)
    nd = ctypes.c_int64()
    _check(lib().orc_dispatch_ec(ctypes.byref(shape), _p(ec_token), _p(off), _p(perm), _p(inv),
                                 ctypes.addressof(nd)), "dispatch_ec")
    return Dispatch(np.full(N, C, np.int32), off, perm, inv, nd.value)


def moe_output_ec(shape: OrcShape, x, inp, r: RoutingEC, tokens: np.ndarray) -> np.ndarray:
    w, _keep = weights_of(inp)
    tokens = np.ascontiguousarray(tokens, np.int64)
    y = np.empty((len(tokens), shape.d), np.float64)
    _check(lib().orc_moe_output_ec(ctypes.byref(shape), _p(x), ctypes.byref(w), _p(r.ec_token),
                                   _p(np.ascontiguousarray(r.ec_gate)), _p(tokens), len(tokens), _p(y)),
           "moe_output_ec")
    return y


def combine_ec(shape: OrcShape, y_perm, inv_map, gate_row32, y_shared=None) -> np.ndarray:
    y = np.empty((shape.T, shape.d), np.float64)
    _check(lib().orc_combine_ec(ctypes.byref(shape), _p(y_perm), _p(np.ascontiguousarray(inv_map, np.int32)),
                                _p(np.ascontiguousarray(gate_row32, np.float32)), _p(y_shared), _p(y)),
           "combine_ec")
    return y


@dataclass
class Forward:
    logits64: np.ndarray
    logits32: np.ndarray
    routing: Routing | RoutingEC
    disp: Dispatch
    tokens: np.ndarray
    y: np.ndarray            # [len(tokens), d] fp64


def forward(inp, tokens: np.ndarray | None = None, logits32: np.ndarray | None = None) -> Forward:
    """Whole layer: logits -> routing/stats -> dispatch -> outputs of `tokens`
    (all tokens when None). `logits32` replaces the router GEMM when given."""
    wl = inp.wl
    shape = shape_of(wl)
    if logits32 is None:
        l64, l32 = router_logits(shape, inp.x, inp)
    else:
        l64, l32 = logits32.astype(np.float64), np.ascontiguousarray(logits32, np.float32)
    if tokens is None:
        tokens = np.arange(wl.T, dtype=np.int64)
    if shape.gating == EXPERT_CHOICE:
        r = route_ec(shape, l32)
        dsp = dispatch_ec(shape, r.ec_token)
        y = moe_output_ec(shape, inp.x, inp, r, tokens)
    else:
        r = route(shape, l32)
        dsp = dispatch(shape, r.topk_idx)
        y = moe_output(shape, inp.x, inp, r, dsp, tokens)
    return Forward(l64, l32, r, dsp, np.asarray(tokens, np.int64), y)


@dataclass
class Grads:
    dx: np.ndarray            # [T, d]
    dWr: np.ndarray           # [N, d]
    dbr: np.ndarray           # [N]
    dW1: np.ndarray           # [N, d_ff, d]
    dW3: np.ndarray | None
    dW2: np.ndarray           # [N, d, d_ff]
    db1: np.ndarray | None    # GELU
    db2: np.ndarray | None
    dsW1: np.ndarray | None   # shared experts
    dsW3: np.ndarray | None
    dsW2: np.ndarray | None


def backward(inp, dy: np.ndarray, c_aux: float = 0.0, c_z: float = 0.0) -> Grads:
    """Gradients of sum <dy, y> + c_aux L_aux + c_z z with respect to x and
    every parameter (fp64), routing decisions held fixed."""
    wl = inp.wl
    shape = shape_of(wl)
    w, _keep = weights_of(inp)
    T, d, f, N, S = wl.T, wl.d, wl.d_ff, wl.n_experts, wl.n_shared
    swi = wl.act == 1
    g = Grads(np.empty((T, d)), np.empty((N, d)), np.empty(N), np.empty((N, f, d)),
              np.empty((N, f, d)) if swi else None, np.empty((N, d, f)),
              None if swi else np.empty((N, f)), None if swi else np.empty((N, d)),
              np.empty((S, f, d)) if S else None, np.empty((S, f, d)) if (S and swi) else None,
              np.empty((S, d, f)) if S else None)
    dy = np.ascontiguousarray(dy)
    _check(lib().orc_backward(ctypes.byref(shape), _p(inp.x), ctypes.byref(w), _p(dy), c_aux, c_z, _p(g.dx),
                              _p(g.dWr), _p(g.dbr), _p(g.dW1), _p(g.dW3), _p(g.dW2), _p(g.db1), _p(g.db2),
                              _p(g.dsW1), _p(g.dsW3), _p(g.dsW2)), "backward")
    return g


def backward_sampled(inp, dy: np.ndarray, tokens, units, c_aux: float = 0.0, c_z: float = 0.0):
    """Parts of backward() at sizes where the whole pass is too slow: dx rows
    of `tokens`, and for each (expert e, hidden unit i) in `units`, row i of
    dW1[e] / dW3[e] and column i of dW2[e]. Returns (dx_rows [n][d],
    dW1_rows [m][d], dW3_rows [m][d] or None, dW2_cols [m][d]), fp64."""
    wl = inp.wl
    shape = shape_of(wl)
    w, _keep = weights_of(inp)
    tok = np.ascontiguousarray(tokens, np.int32)
    un = np.ascontiguousarray(units, np.int32).reshape(-1, 2)
    d = wl.d
    dx = np.empty((len(tok), d))
    d1, d2 = np.empty((len(un), d)), np.empty((len(un), d))
    d3 = np.empty((len(un), d)) if wl.act == 1 else None
    dy = np.ascontiguousarray(dy)
    _check(lib().orc_backward_sampled(ctypes.byref(shape), _p(inp.x), ctypes.byref(w), _p(dy), c_aux, c_z, _p(tok),
                                      len(tok), _p(dx), _p(un), len(un), _p(d1), _p(d3), _p(d2)),
           "backward_sampled")
    return dx, d1, d3, d2


def threads() -> int:
    """OpenMP threads the oracle runs on."""
    return lib().orc_threads()


def bf16_value(b: int) -> float:
    return lib().orc_bf16_value(b)


def e4m3_value(q: int) -> float:
    return lib().orc_e4m3_value(q)


def gelu(u: float) -> float:
    return lib().orc_gelu(u)


def silu(u: float) -> float:
    return lib().orc_silu(u)
