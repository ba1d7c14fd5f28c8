"""Per-expert integer weights (INT8 for the high-traffic experts, INT4 for the
rest, one fp32 scale per weight row) through every expert path: the GEMV and
streaming decode kernels, which decode the codes in registers while the bytes
stream, the register-staged tiles (fewer than 2048 rows) and the LDS-DMA
tiles, which convert each fragment's codes after its LDS read. The library reads packed byte
rows (two INT4 codes a byte); the oracle reads the unpacked codes. End-to-end
against the CPU oracle, reduced sizes (every token) and full Mixtral sizes
(sampled tokens)."""
import numpy as np
import pytest

import gen
import sparse_mixture_experts_36_amd as moe
from test_gpu_forward import _sample, run_and_check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()
    yield
    torch.cuda.synchronize()


MIX = gen.MIXTRAL_PREFILL.with_(w_dtype=gen.INT_W, n_int8=2)
FG = gen.FINE_GRAINED.with_(w_dtype=gen.INT_W, n_int8=40)
SW = gen.SWITCH_TOP1.with_(w_dtype=gen.INT_W, n_int8=16)

REDUCED = {
    # GEMV (one or two rows per expert; k a multiple of 2048)
    "mixtral-like-int-T1-gemv": MIX.with_(T=1, d=2048, d_ff=4096),
    "mixtral-like-int-T2-gemv": MIX.with_(T=2, d=2048, d_ff=4096),
    "mixtral-like-int-T1-gemv-all-int4": MIX.with_(T=1, d=2048, d_ff=4096, n_int8=0),
    # streaming: 16-, 32- and 64-row passes, shared token rows through LDS
    "mixtral-like-int-T1-stream": MIX.with_(T=1, d=1024, d_ff=1536),
    "mixtral-like-int-T16": MIX.with_(T=16, d=1024, d_ff=1536),
    "mixtral-like-int-T64": MIX.with_(T=64, d=1024, d_ff=1536),
    "mixtral-like-int-T100": MIX.with_(T=100, d=1024, d_ff=1536),
    "mixtral-like-int-T64-all-int8": MIX.with_(T=64, d=1024, d_ff=1536, n_int8=8),
    "fine-grained-like-int-decode": FG.with_(T=24, d=512, d_ff=256),
    # prefill tiles: register-staged 128 x 128 below 2048 rows, else LDS-DMA
    # 128-row tiles (groups averaging under 384 rows) or 256-row tiles
    "mixtral-like-int-prefill-reg128": MIX.with_(T=300, d=1024, d_ff=1536),
    "mixtral-like-int-prefill-dma128": MIX.with_(T=1024, d=1024, d_ff=1536),
    "mixtral-like-int-prefill-dma256": MIX.with_(T=2048, d=1024, d_ff=1536),
    "mixtral-like-int-prefill-dma256-skewed": MIX.with_(T=2048, d=1024, d_ff=1536, zipf_s=1.2),
    "mixtral-like-int-prefill-all-int4": MIX.with_(T=1024, d=512, d_ff=768, n_int8=0),
    "fine-grained-like-int": FG.with_(T=512, d=512, d_ff=256),
    "switch-like-int-gelu": SW.with_(T=2048, d=512, d_ff=1024),
    "switch-like-int-gelu-decode": SW.with_(T=128, d=512, d_ff=1024),
    # 2048 rows or more, but a GELU d_ff the 256-column tiles do not fit: the
    # codes are decoded in registers on 128 x 128 tiles
    "switch-like-int-gelu-d_ff-384": SW.with_(T=4096, d=512, d_ff=384),
}


@pytest.mark.parametrize("name", list(REDUCED))
def test_int_forward_reduced(name):
    run_and_check(gen.make_inputs(REDUCED[name]), label=name)


@pytest.mark.parametrize("T", [64, 2048])
@pytest.mark.parametrize("pad", [0, 64])
def test_int_forward_reduced_padded_rows(pad, T):
    """Byte rows longer than the codes (ld_up / ld_down = d + pad, d_ff + pad),
    on the streaming kernels (T = 64) and the 256-row DMA tiles (T = 2048)."""
    run_and_check(gen.make_inputs(MIX.with_(T=T, d=1024, d_ff=1536)), label=f"int rows pad {pad} T={T}", pad=pad)


@pytest.mark.parametrize("T", [1, 16, 64])
def test_int_full_mixtral_decode(T):
    inp = gen.make_inputs(gen.MIXTRAL_DECODE_INT[T])
    run_and_check(inp, sample=None if T <= 16 else _sample(T, 12), label=f"mixtral-decode-int T={T}", pad=64)


def test_int_full_mixtral_prefill():
    inp = gen.make_inputs(gen.MIXTRAL_PREFILL_INT)
    run_and_check(inp, sample=_sample(4096, 64), label="mixtral-prefill-int (full)", pad=64)


def test_int_bits_validated_on_host():
    import ctypes
    wl = MIX.with_(T=4, d=256, d_ff=256)
    inp = gen.make_inputs(wl)
    from helpers import dev, device_weights, shape_of
    t = device_weights(inp)
    t["w_bits"] = np.array([8, 8, 4, 4, 4, 4, 4, 6], np.uint8)  # 6 bits: not a width the library runs
    w = moe.weights_struct(t)
    shape = shape_of(wl)
    ws = moe.workspace(shape)
    y = dev(np.zeros((wl.T, wl.d), np.uint16))
    rc = moe.lib().moe_forward(ctypes.byref(shape), moe._ptr(dev(inp.x)), ctypes.byref(w), moe._ptr(y), None, None,
                               None, None, None, None, None, moe._ptr(ws), ws.numel(), None)
    assert rc == moe.MOE_ERR_INVALID_ARG
