"""The library's launches captured in a HIP graph (torch.cuda.CUDAGraph over the calls of the
tiny MLP at tp 2: both ranks' colwise GEMM with bias and GELU, rowwise partials, and the SUM
with the bias) and replayed.  Each replay reads the buffers the graph was captured with, so
new input values written in place must give the same output as the eager calls on them.
Replays are interleaved with eager work and synchronisations, and every replay is checked
bit for bit against the eager result."""
import numpy as np
import pytest
import torch

import synth_inputs as si
import tensor_sharded_linear_amd as tsl

pytestmark = pytest.mark.gpu


def _up(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def test_tiny_mlp_graph_replays_equal_eager():
    wl = si.workload("tiny_mlp")
    a = {k: _up(v) for k, v in wl.arrays.items()}
    P = 2
    w1s = [tsl.tp_plan_shard_slice(a["w1"], a["b1"], "colwise", P, r) for r in range(P)]
    w2s = [tsl.tp_plan_shard_slice(a["w2"], None, "rowwise", P, r)[0] for r in range(P)]
    x = a["x"].clone()
    hs = [tsl.tp_linear_colwise(x, w, b, act="gelu_tanh") for w, b in w1s]
    parts = [tsl.tp_linear_rowwise(h, w) for h, w in zip(hs, w2s)]
    y = torch.empty(parts[0].shape, dtype=torch.float32, device="cuda")

    def forward():
        for r in range(P):
            tsl.tp_linear_colwise(x, w1s[r][0], w1s[r][1], act="gelu_tanh", out=hs[r])
            tsl.tp_linear_rowwise(hs[r], w2s[r], out=parts[r])
        tsl.tp_partial_combine(parts, "sum", bias=a["b2"], out=y)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        forward()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        forward()
    torch.cuda.synchronize()

    rng = np.random.default_rng(7)
    for i in range(4):
        xi = _up(si.normal_bf16(rng, tuple(x.shape)))
        x.copy_(xi)
        forward()                       # eager on the new input
        torch.cuda.synchronize()
        expect = y.clone()
        y.fill_(float("nan"))           # the replay must rewrite every element
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), expect.view(torch.int32)), f"replay {i}"
        tsl.tp_linear_colwise(xi, w1s[0][0], w1s[0][1])   # unrelated eager work between replays
