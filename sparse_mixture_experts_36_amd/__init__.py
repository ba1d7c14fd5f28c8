"""MI355X (gfx950) top-k token-choice Mixture-of-Experts layer forward, with
expert-choice routing as a second routing mode.

Thin Python binding over the C ABI in ``include/moe.h`` (``libmoe.so``, built
in-tree by ``sparse_mixture_experts_36_amd.build``). The functions here only
marshal torch tensors (device memory) and the current HIP stream into the C
entry points of the same names; every step of the layer runs in the library's
HIP kernels. There is no fallback: without the built library every call
raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP, MOE_ERR_WORKSPACE = 0, -1, -2, -3, -4
F32, BF16, FP8_E4M3, INT_W = 0, 1, 2, 3
GELU, SWIGLU = 0, 1
SOFTMAX_TOPK, SOFTMAX_TOPK_RENORM, TOPK_SOFTMAX, EXPERT_CHOICE = 0, 1, 2, 3
ENTRY_ROUTE, ENTRY_PERMUTE, ENTRY_GROUPED_FFN, ENTRY_FORWARD, ENTRY_BACKWARD = 0, 1, 2, 3, 4
ROUTE_LOGITS_GIVEN = 1


class Shape(ctypes.Structure):
    """moe_shape"""
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int64), ("d_ff", ctypes.c_int64),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("act", ctypes.c_int32), ("gating", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("w_dtype", ctypes.c_int32), ("capacity", ctypes.c_int64), ("aux_alpha", ctypes.c_float)]


class Weights(ctypes.Structure):
    """moe_weights (device pointers, the row pitches of the expert matrices,
    then the host arrays of integer bit widths)"""
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_router", "b_router", "w1", "w3", "w2", "b1", "b2", "w_scale", "sw1", "sw3", "sw2",
                 "sw_scale")] + [("ld_up", ctypes.c_int64), ("ld_down", ctypes.c_int64),
                                 ("w_bits", ctypes.c_void_p), ("sw_bits", ctypes.c_void_p)]


class Stats(ctypes.Structure):
    """moe_stats (device pointers)"""
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("counts", "kept", "f", "P", "l_aux", "z_loss", "lse_mean", "lse_sq_mean", "n_dropped")]


class Grads(ctypes.Structure):
    """moe_grads (device pointers)"""
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("dx", "dw_router", "db_router", "dw1", "dw3", "dw2", "db1", "db2", "dsw1", "dsw3", "dsw2")]


class MoEError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = lib().moe_status_string(status).decode()
        if status == MOE_ERR_HIP:
            msg += f" (hipError {lib().moe_last_hip_error()})"
        super().__init__(f"{what}: {msg}")
        self.status = status


_lib = None


def lib():
    """The loaded libmoe.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_mixture_experts_36_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        sp, wp, stp = ctypes.POINTER(Shape), ctypes.POINTER(Weights), ctypes.POINTER(Stats)
        L.moe_abi_version.restype = ctypes.c_int
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_hip_error.restype = ctypes.c_int
        L.moe_capacity.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_double]
        L.moe_capacity.restype = ctypes.c_int64
        L.moe_workspace_size.argtypes = [sp, ctypes.c_int32, ctypes.POINTER(sz)]
        L.moe_ffn_path.argtypes = [sp, ctypes.c_int32]
        L.moe_ffn_path.restype = ctypes.c_int32
        L.moe_route.argtypes = [sp, vp, vp, vp, vp, ctypes.c_uint32, vp, vp, stp, vp, sz, vp]
        L.moe_permute.argtypes = [sp, vp, vp, vp, vp, vp, vp, stp, vp, sz, vp]
        L.moe_grouped_ffn.argtypes = [sp, vp, vp, vp, wp, vp, vp, vp, sz, vp]
        L.moe_combine.argtypes = [sp, vp, vp, vp, vp, vp, vp]
        L.moe_forward.argtypes = [sp, vp, wp, vp, vp, vp, vp, vp, vp, vp, stp, vp, sz, vp]
        L.moe_forward_noalloc.argtypes = [sp, vp, wp, vp, vp, vp, vp, vp, vp, vp, stp, vp]
        L.moe_backward.argtypes = [sp, vp, wp, vp, ctypes.c_float, ctypes.c_float, ctypes.POINTER(Grads), vp, sz,
                                   vp]
        L.moe_timing_start.argtypes = [ctypes.c_int32]
        L.moe_timing_stop.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32)]
        for f in ("moe_workspace_size", "moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine",
                  "moe_forward", "moe_forward_noalloc", "moe_backward", "moe_timing_start", "moe_timing_stop"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(rc: int, what: str):
    if rc != MOE_OK:
        raise MoEError(rc, what)


def make_shape(T, d, d_ff, n_experts, top_k, act, gating, act_dtype, w_dtype, capacity=-1, n_shared=0,
               aux_alpha=0.01) -> Shape:
    return Shape(T=T, d=d, d_ff=d_ff, n_experts=n_experts, top_k=top_k, n_shared=n_shared, act=act,
                 gating=gating, act_dtype=act_dtype, w_dtype=w_dtype, capacity=capacity, aux_alpha=aux_alpha)


def capacity(T: int, k: int, N: int, cf: float | None) -> int:
    """floor(cf*T*k/N) (moe_capacity); -1 when cf is None (dropless). With k = 1
    it is the expert-choice capacity int(T*cf/N)."""
    return -1 if cf is None else lib().moe_capacity(T, k, N, cf)


def routing_shapes(shape: Shape) -> dict:
    """Shapes of the routing arrays for this layer: topk_idx / topk_w are
    [T, k] under token choice and [N, C] (expert-major) under expert choice;
    inv_map is [T, k] or [T, N]; perm_token has T*k or N*C entries."""
    T, N, k = shape.T, shape.n_experts, shape.top_k
    if shape.gating == EXPERT_CHOICE:
        C = shape.capacity
        return {"topk": (N, C), "inv_map": (T, N), "perm_token": (N * C,)}
    return {"topk": (T, k), "inv_map": (T, k), "perm_token": (T * k,)}


def workspace_size(shape: Shape, entry: int = ENTRY_FORWARD) -> int:
    n = ctypes.c_size_t()
    _check(lib().moe_workspace_size(ctypes.byref(shape), entry, ctypes.byref(n)), "moe_workspace_size")
    return n.value


PATH_F32, PATH_STREAM, PATH_REG128, PATH_DMA256, PATH_DMA128, PATH_BGEMM = range(6)


def ffn_path(shape: Shape, entry: int = ENTRY_FORWARD) -> int:
    """moe_ffn_path: the kernel family of the expert FFN (or of moe_backward's
    forward recompute) for this shape."""
    rc = lib().moe_ffn_path(ctypes.byref(shape), entry)
    _check(rc if rc < 0 else MOE_OK, "moe_ffn_path")
    return rc


def workspace(shape: Shape, entry: int = ENTRY_FORWARD, device="cuda"):
    """A device byte tensor big enough for `entry` (torch's allocator aligns to 256 B or more)."""
    import torch
    return torch.empty(workspace_size(shape, entry), dtype=torch.uint8, device=device)


def stats_struct(st: dict | None) -> Stats | None:
    if st is None:
        return None
    return Stats(**{k: _ptr(v) for k, v in st.items() if v is not None})


def alloc_stats(N: int, device="cuda") -> dict:
    import torch
    i32 = dict(dtype=torch.int32, device=device)
    f32 = dict(dtype=torch.float32, device=device)
    return {"counts": torch.zeros(N, **i32), "kept": torch.zeros(N, **i32), "f": torch.zeros(N, **f32),
            "P": torch.zeros(N, **f32), "l_aux": torch.zeros(1, **f32), "z_loss": torch.zeros(1, **f32),
            "lse_mean": torch.zeros(1, **f32), "lse_sq_mean": torch.zeros(1, **f32),
            "n_dropped": torch.zeros(1, **i32)}


def route(shape, x, w_router, b_router, logits, topk_idx, topk_w, stats=None, ws=None, flags=0, stream=None):
    st = stats_struct(stats)
    ws_ = ws if ws is not None else workspace(shape, ENTRY_ROUTE)
    rc = lib().moe_route(ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(b_router), _ptr(logits), flags,
                         _ptr(topk_idx), _ptr(topk_w), ctypes.byref(st) if st else None, _ptr(ws_),
                         ws_.numel(), _stream(stream))
    _check(rc, "moe_route")


def permute(shape, topk_idx, x, expert_offsets, perm_token, inv_map, x_perm, stats=None, ws=None, stream=None):
    st = stats_struct(stats)
    ws_ = ws if ws is not None else workspace(shape, ENTRY_PERMUTE)
    rc = lib().moe_permute(ctypes.byref(shape), _ptr(topk_idx), _ptr(x), _ptr(expert_offsets), _ptr(perm_token),
                           _ptr(inv_map), _ptr(x_perm), ctypes.byref(st) if st else None, _ptr(ws_), ws_.numel(),
                           _stream(stream))
    _check(rc, "moe_permute")


def grouped_ffn(shape, x_perm, expert_offsets, x, weights: Weights, y_perm, y_shared=None, ws=None, stream=None):
    ws_ = ws if ws is not None else workspace(shape, ENTRY_GROUPED_FFN)
    rc = lib().moe_grouped_ffn(ctypes.byref(shape), _ptr(x_perm), _ptr(expert_offsets), _ptr(x),
                               ctypes.byref(weights), _ptr(y_perm), _ptr(y_shared), _ptr(ws_), ws_.numel(),
                               _stream(stream))
    _check(rc, "moe_grouped_ffn")


def combine(shape, y_perm, inv_map, topk_w, y_shared, y, stream=None):
    rc = lib().moe_combine(ctypes.byref(shape), _ptr(y_perm), _ptr(inv_map), _ptr(topk_w), _ptr(y_shared),
                           _ptr(y), _stream(stream))
    _check(rc, "moe_combine")


def forward(shape, x, weights: Weights, y, logits=None, topk_idx=None, topk_w=None, expert_offsets=None,
            perm_token=None, inv_map=None, stats=None, ws=None, stream=None):
    st = stats_struct(stats)
    ws_ = ws if ws is not None else workspace(shape, ENTRY_FORWARD)
    rc = lib().moe_forward(ctypes.byref(shape), _ptr(x), ctypes.byref(weights), _ptr(y), _ptr(logits),
                           _ptr(topk_idx), _ptr(topk_w), _ptr(expert_offsets), _ptr(perm_token), _ptr(inv_map),
                           ctypes.byref(st) if st else None, _ptr(ws_), ws_.numel(), _stream(stream))
    _check(rc, "moe_forward")


NOALLOC_SCRATCH_BYTES = 32 << 20  # MOE_NOALLOC_SCRATCH_BYTES


def forward_noalloc(shape, x, weights: Weights, y, logits=None, topk_idx=None, topk_w=None, expert_offsets=None,
                    perm_token=None, inv_map=None, stats=None, stream=None):
    """moe_forward_noalloc: moe_forward with the library's own device scratch
    (no workspace argument, nothing allocated; shapes whose forward workspace
    exceeds NOALLOC_SCRATCH_BYTES raise MoEError with MOE_ERR_WORKSPACE)."""
    st = stats_struct(stats)
    rc = lib().moe_forward_noalloc(ctypes.byref(shape), _ptr(x), ctypes.byref(weights), _ptr(y), _ptr(logits),
                                   _ptr(topk_idx), _ptr(topk_w), _ptr(expert_offsets), _ptr(perm_token),
                                   _ptr(inv_map), ctypes.byref(st) if st else None, _stream(stream))
    _check(rc, "moe_forward_noalloc")


def alloc_grads(shape: Shape, device="cuda") -> dict:
    """Output tensors for moe_backward: dx bf16 [T][d], fp32 weight gradients
    for every weight the layer has (the router bias and GELU biases included)."""
    import torch
    T, d, f, N, S = shape.T, shape.d, shape.d_ff, shape.n_experts, shape.n_shared
    f32 = dict(dtype=torch.float32, device=device)
    swi = shape.act == SWIGLU
    g = {"dx": torch.empty(T, d, dtype=torch.bfloat16, device=device), "dw_router": torch.empty(N, d, **f32),
         "db_router": torch.empty(N, **f32), "dw1": torch.empty(N, f, d, **f32),
         "dw3": torch.empty(N, f, d, **f32) if swi else None, "dw2": torch.empty(N, d, f, **f32),
         "db1": None if swi else torch.empty(N, f, **f32), "db2": None if swi else torch.empty(N, d, **f32)}
    if S:
        g.update(dsw1=torch.empty(S, f, d, **f32), dsw3=torch.empty(S, f, d, **f32) if swi else None,
                 dsw2=torch.empty(S, d, f, **f32))
    return g


def backward(shape, x, weights: Weights, dy, grads: dict, c_aux: float = 0.0, c_z: float = 0.0, ws=None,
             stream=None):
    """moe_backward: gradients of sum <dy, y> + c_aux L_aux + c_z z into the
    tensors of `grads` (keys of moe_grads; missing or None: not computed)."""
    gs = Grads(**{k: _ptr(v) for k, v in grads.items() if v is not None})
    ws_ = ws if ws is not None else workspace(shape, ENTRY_BACKWARD)
    rc = lib().moe_backward(ctypes.byref(shape), _ptr(x), ctypes.byref(weights), _ptr(dy), c_aux, c_z,
                            ctypes.byref(gs), _ptr(ws_), ws_.numel(), _stream(stream))
    _check(rc, "moe_backward")


STAGES = ("route", "permute", "ffn_plan", "ffn_up", "ffn_down", "combine")


def timing_start(max_launches: int = 4096):
    """Start per-stage hipEvent timing (moe_timing_start)."""
    _check(lib().moe_timing_start(max_launches), "moe_timing_start")


def timing_stop() -> dict:
    """Stop stage timing; {stage: (total_ms, launches)} (waits for the events)."""
    ms = (ctypes.c_double * len(STAGES))()
    n = (ctypes.c_int32 * len(STAGES))()
    _check(lib().moe_timing_stop(ms, n), "moe_timing_stop")
    return {s: (ms[i], n[i]) for i, s in enumerate(STAGES)}


def _row_pitch(ts, what):
    """Row pitch (elements) shared by 3-D expert matrices [E][rows][cols] whose
    rows may be padded (a view [..., :cols] of a wider allocation); 0 if none."""
    ld = 0
    for t in ts:
        if t is None:
            continue
        if t.dim() != 3 or t.stride(2) != 1 or t.stride(0) != t.shape[1] * t.stride(1):
            raise ValueError(f"{what}: expert matrices must be [E][rows][cols] with unit column stride and "
                             f"no gap between experts")
        if ld and t.stride(1) != ld:
            raise ValueError(f"{what}: all matrices must share one row pitch")
        ld = t.stride(1)
    return ld


def weights_struct(t: dict) -> Weights:
    """moe_weights from a dict of device tensors (missing keys are NULL). The
    row pitches come from the strides of w1/w3/sw1/sw3 and of w2/sw2. Integer
    weights: "w_bits" / "sw_bits" are host numpy uint8 arrays, kept alive by
    the returned struct."""
    import numpy as np
    dev_keys = {k: v for k, v in t.items() if v is not None and k not in ("w_bits", "sw_bits")}
    w = Weights(**{k: _ptr(v) for k, v in dev_keys.items()})
    w.ld_up = _row_pitch([t.get(k) for k in ("w1", "w3", "sw1", "sw3")], "w1/w3/sw1/sw3")
    w.ld_down = _row_pitch([t.get(k) for k in ("w2", "sw2")], "w2/sw2")
    keep = []
    for k in ("w_bits", "sw_bits"):
        if t.get(k) is not None:
            a = np.ascontiguousarray(t[k], np.uint8)
            keep.append(a)
            setattr(w, k, a.ctypes.data)
    w._host_arrays = keep
    return w


def pack_int_weights(codes, bits, pad: int = 0):
    """Integer expert matrices in the library's layout: codes [E][rows][cols]
    (int8, one code per element) and bits [E] (8 or 4) -> uint8 [E][rows][cols
    + pad] byte rows. An 8-bit expert's row holds its codes. A 4-bit expert's
    row holds cols/2 bytes: each 8 consecutive codes form one little-endian
    32-bit word with code 8m + 2j in bits [4j, 4j + 4) and code 8m + 2j + 1 in
    bits [16 + 4j, 20 + 4j) (two's complement nibbles); the rest of the row is
    zero. Host numpy in, host numpy out."""
    import numpy as np
    codes = np.asarray(codes, np.int8)
    E, R, C = codes.shape
    out = np.zeros((E, R, C + pad), np.uint8)
    for e in range(E):
        if int(bits[e]) == 8:
            out[e, :, :C] = codes[e].view(np.uint8)
        else:
            u = (codes[e].view(np.uint8) & 0x0F).astype(np.uint32).reshape(R, C // 8, 8)
            word = np.zeros((R, C // 8), np.uint32)
            for j in range(4):
                word |= u[:, :, 2 * j] << (4 * j)
                word |= u[:, :, 2 * j + 1] << (16 + 4 * j)
            out[e, :, :C // 2] = word.astype("<u4").view(np.uint8).reshape(R, C // 2)
    return out


def padded(t, pad: int = 64):
    """A copy of expert matrices [E][rows][cols] whose rows are `pad` elements
    longer than cols (a view of the wider allocation): the layout the prefill
    GEMM reads fastest when cols is a multiple of 4096."""
    import torch
    if t is None:
        return None
    E, R, C = t.shape
    buf = torch.empty((E, R, C + pad), dtype=t.dtype, device=t.device)
    v = buf[:, :, :C]
    v.copy_(t)
    return v


@dataclass
class LayerOutputs:
    y: object
    logits: object
    topk_idx: object
    topk_w: object
    expert_offsets: object
    perm_token: object
    inv_map: object
    stats: dict


class MoELayer:
    """Device-resident weights + workspace for repeated moe_forward calls.

    `tensors` maps moe_weights member names to device tensors (bf16 data may be
    given as torch.bfloat16 or int16/uint16 bit patterns; e4m3 as uint8)."""

    def __init__(self, shape: Shape, tensors: dict, device="cuda"):
        import torch
        self.shape = shape
        self.tensors = tensors
        self.weights = weights_struct(tensors)
        self.ws = workspace(shape, ENTRY_FORWARD, device)
        T, N = shape.T, shape.n_experts
        rs = routing_shapes(shape)
        i32 = dict(dtype=torch.int32, device=device)
        self.out = LayerOutputs(
            y=torch.empty((T, shape.d), dtype=torch.float32 if shape.act_dtype == F32 else torch.bfloat16,
                          device=device),
            logits=torch.empty((T, N), dtype=torch.float32, device=device),
            topk_idx=torch.empty(rs["topk"], **i32), topk_w=torch.empty(rs["topk"], dtype=torch.float32, device=device),
            expert_offsets=torch.empty(N + 1, **i32), perm_token=torch.empty(rs["perm_token"], **i32),
            inv_map=torch.empty(rs["inv_map"], **i32), stats=alloc_stats(N, device))

    def __call__(self, x, stream=None) -> LayerOutputs:
        o = self.out
        forward(self.shape, x, self.weights, o.y, o.logits, o.topk_idx, o.topk_w, o.expert_offsets, o.perm_token,
                o.inv_map, o.stats, self.ws, stream)
        return o

    def capture(self, x):
        """Capture one forward on the device tensor x into a HIP graph
        (torch.cuda.CUDAGraph) and return it: each replay recomputes self.out
        from x's contents at replay time, with no host launch work. The
        library's kernels record no memset or copy nodes; stage timing must be
        off while capturing."""
        import torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self(x)  # one eager call outside the capture (library and device setup)
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self(x)
        return g

    def latest(self) -> dict:
        """Host copy of the router statistics (synchronises): aux loss, z-loss,
        dropped share and the per-expert token shares."""
        st = {k: v.cpu() for k, v in self.out.stats.items()}
        if self.shape.gating == EXPERT_CHOICE:
            # balanced by construction: every expert takes C tokens; the share
            # dropped is that of the tokens no expert took
            counts = [int(v) for v in st["counts"]]
            tot = max(sum(counts), 1)
            dist = [c / tot for c in counts]
            return {"aux_loss": None, "z_loss": float(st["z_loss"][0]),
                    "dropped_share": int(st["n_dropped"][0]) / max(self.shape.T, 1),
                    "distribution": dist, "counts": counts, "kept": [int(v) for v in st["kept"]],
                    "entropy": routing_entropy(dist)}
        tk = self.shape.T * self.shape.top_k
        return {"aux_loss": float(st["l_aux"][0]), "z_loss": float(st["z_loss"][0]),
                "dropped_share": int(st["n_dropped"][0]) / max(tk, 1),
                "distribution": [float(v) for v in st["f"]], "counts": [int(v) for v in st["counts"]],
                "kept": [int(v) for v in st["kept"]],
                "entropy": routing_entropy([float(v) for v in st["f"]])}


# ---------------------------------------------------------------- host-side helpers

def routing_entropy(f) -> float:
    """Entropy of the per-expert token shares f (natural log). A collapse
    detector: far below ln(N) means only a few experts are used (aigrafen.se
    "Mixture of Experts", the collapsed/balanced routing example)."""
    return -sum(p * math.log(p) for p in f if p > 0)


def expert_params(d: int, d_ff: int, act: int) -> int:
    """Weights of one expert: SwiGLU has three d x d_ff matrices, GELU two
    (aigrafen.se "Mixture of Experts", the total/active parameter example)."""
    return (3 if act == SWIGLU else 2) * d * d_ff
