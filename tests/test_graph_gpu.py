"""The entry points that allocate nothing and never synchronise can be captured
in a HIP graph: kda_chunk_fwd (here with its segments along T, the varlen
chunk map and the gated form) and kda_layer_fwd. Each graph is replayed
several times with eager work on the same buffers in between (the outputs are
overwritten with NaN), and every replay must reproduce the eager call bitwise.
"""
import sys

import pytest

from helpers import dev_inputs, to_dev
from kimi_delta_attention_03_amd.synthetic import core_inputs, layer_inputs

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def capture(torch, fn):
    """Warm up on a side stream (default priority), then capture fn."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def check_replays(torch, g, outs, refs):
    for i in range(REPLAYS):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(o, r), f"replay {i} differs from the eager call"


@pytest.mark.parametrize("case", ["segmented", "varlen", "gated"])
def test_forward_graph_replays_match_eager(case):
    import torch
    import kimi_delta_attention_03_amd as kda
    _say(f"graph forward {case}")
    if case == "varlen":
        x = core_inputs(1, None, 4, 128, 128, dtype="bf16", seed=91, init_std=0.1, lengths=[700, 1, 0, 2048, 333])
    else:
        # T = 8192 at H = 32: the records of the whole problem exceed one
        # segment, so the forward runs several segments along T
        x = core_inputs(1, 8192, 32, 128, 128, dtype="bf16", seed=92, init_std=0.1)
    d = dev_inputs(x)
    gate = {}
    if case == "gated":
        H, K = 32, 128
        gen = torch.Generator(device="cuda:0").manual_seed(5)
        gate = dict(gate_mode="lower_bound_sigmoid", gate_lower_bound=-5.0,
                    A_log=torch.randn(H, device="cuda:0", generator=gen) * 0.3,
                    dt_bias=torch.randn(H * K, device="cuda:0", generator=gen) * 0.1)
    f = kda.KdaForward(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=x.scale, initial_state=d["initial_state"],
                       cu_seqlens=d["cu_seqlens"], **gate)
    if case != "varlen":
        assert kda.workspace_layout(f.params).segments > 1
    o, fs = f()
    torch.cuda.synchronize()
    refs = (o.clone(), fs.clone())
    g = capture(torch, f)
    check_replays(torch, g, (f.o, f.final_state), refs)


def test_layer_graph_replays_match_eager():
    import torch
    import kimi_delta_attention_03_amd as kda
    from test_layer_gpu import dev_weights
    B, T, M, H, D, r = 2, 256, 256, 2, 128, 32
    _say(f"graph layer B={B} T={T} M={M} H={H} D={D}")
    x, w = layer_inputs(B=B, T=T, M=M, H=H, D=D, rank=r, seed=93)
    xd = to_dev(x, torch.bfloat16)
    layer = kda.KdaLayer(dev_weights(w), B, T, H, D, keep_core_output=True)
    y = layer(xd)
    torch.cuda.synchronize()
    refs = (y.clone(), layer.core_out.clone())
    g = capture(torch, lambda: layer(xd))
    check_replays(torch, g, (layer.x_new, layer.core_out), refs)
