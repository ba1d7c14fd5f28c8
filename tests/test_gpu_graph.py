"""moe_forward captured in a HIP graph (torch.cuda.CUDAGraph) and replayed:
every replay, with eager work and synchronisations between replays, must give
the eager call's result bit for bit (the path is deterministic), for a decode
call, a prefill call and a capacity-limited call, and a replay must follow a
change of the captured input's contents."""
import numpy as np
import pytest

import gen
import sparse_mixture_experts_36_amd as moe
from helpers import dev, device_weights, say, shape_of

pytestmark = pytest.mark.gpu

CASES = {
    "decode-T1": gen.MIXTRAL_PREFILL.with_(T=1, d=1024, d_ff=1536),
    "decode-T16-shared": gen.FINE_GRAINED.with_(T=16, d=512, d_ff=256),
    "prefill-T512": gen.MIXTRAL_PREFILL.with_(T=512, d=1024, d_ff=1536),
    "switch-capacity": gen.SWITCH_TOP1.with_(T=2048, d=512, d_ff=1024),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager(name):
    import torch
    wl = CASES[name]
    say(f"graph {name}: T={wl.T} d={wl.d} d_ff={wl.d_ff} N={wl.n_experts} k={wl.top_k}")
    inp = gen.make_inputs(wl)
    layer = moe.MoELayer(shape_of(wl), device_weights(inp, pad=64))
    x = dev(inp.x)
    o = layer(x)
    torch.cuda.synchronize()
    ref = {k: getattr(o, k).clone() for k in ("y", "logits", "topk_idx", "topk_w", "inv_map")}
    ref_stats = {k: v.clone() for k, v in o.stats.items()}
    g = layer.capture(x)
    torch.cuda.synchronize()
    for rep in range(4):
        layer.out.y.zero_()
        layer.out.logits.zero_()
        junk = torch.randn(1 << 16, device="cuda").sum()  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        for k, v in ref.items():
            got = getattr(layer.out, k)
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                               v.view(torch.int16) if v.dtype == torch.bfloat16 else v), (rep, k)
        for k, v in ref_stats.items():
            assert torch.equal(layer.out.stats[k], v), (rep, k)
    # new contents of the captured input: the replay must follow them
    x2 = dev(gen.make_inputs(wl, seed=7).x)
    eager2 = layer(x2).y.clone()
    x.copy_(x2)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(layer.out.y.view(torch.int16), eager2.view(torch.int16))
    say(f"  4 replays + 1 on new input match eager")
