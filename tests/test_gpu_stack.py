"""A decode step through a stack of MoE layers, eager and as one HIP graph.

Three layers of the A3B-style shape with different weights (seeds 0, 1, 2),
each taking the previous layer's output as input and residual
(h_(l+1) = h_l + MoE_l(h_l)).  Every layer is checked against the oracle on
the input the GPU gave it (routing bit-exact, FFN rows by the tolerance,
combine bit-exact given the same rows); then the stack is captured in one
graph ("Luce Spark" page, sec. 3: the routed FFN of every layer in one graph
per token) and replayed with new inputs, eager work and synchronisations in
between, and every layer's output of every replay equals an eager run bit for
bit, with the sync counters back at zero.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import quantized_expert_ffn_gemv_amd as moe
from gpu_util import (check_combine_exact, check_ffn, check_logits, check_lookup, check_permute, check_topk,
                      host_outputs, say, to_dev, to_host, upload_layer)

pytestmark = pytest.mark.gpu

N_LAYERS, T = 3, 4


@pytest.fixture(scope="module")
def stack():
    shape = mi.CONFIGS["a3b"]
    Ls = []
    for seed in range(N_LAYERS):
        say(f"[upload] a3b layer seed {seed}")
        Ls.append(upload_layer(shape, 4, seed=seed))
    yield shape, Ls
    Ls.clear()
    torch.cuda.empty_cache()


def _stack_layers(Ls, shape):
    return [moe.StackLayer(L.Wr_d, L.bias_d, L.weights_d, L.table_d, shape.E) for L in Ls]


def _buffers(shape, n):
    d = moe.dims(T, shape.H, shape.I, shape.E, shape.k)
    bufs = [moe.LayerBuffers.allocate(d, 4) for _ in range(n)]
    outs = [torch.empty((T, shape.H), dtype=torch.int16, device="cuda") for _ in range(n)]
    return bufs, outs


def test_stack_eager_matches_the_oracle_layer_by_layer(stack):
    shape, Ls = stack
    bufs, outs = _buffers(shape, N_LAYERS)
    xb, _ = mi.make_activations(shape.H, T, 40)
    x = to_dev(xb)
    moe.stack_forward(bufs, x, _stack_layers(Ls, shape), outs)
    torch.cuda.synchronize()
    h = xb
    for l, (L, buf, out) in enumerate(zip(Ls, bufs, outs)):
        say(f"[layer {l}]")
        g = host_outputs(buf, out, T * shape.k)
        check_logits(g, L, h)
        check_topk(g, L)
        check_lookup(g, L)
        check_permute(g, L)
        check_ffn(g, L, h)
        check_combine_exact(g, L, h)              # the residual of layer l is its input
        h = g["out"]


def test_stack_graph_replays_match_eager(stack):
    shape, Ls = stack
    layers = _stack_layers(Ls, shape)
    gbufs, gouts = _buffers(shape, N_LAYERS)
    x_g = torch.zeros((T, shape.H), dtype=torch.int16, device="cuda")
    xb, _ = mi.make_activations(shape.H, T, 41)
    x_g.copy_(to_dev(xb))
    moe.stack_forward(gbufs, x_g, layers, gouts)          # eager once before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        moe.stack_forward(gbufs, x_g, layers, gouts)
    torch.cuda.synchronize()
    for seed in (42, 43, 44):
        xb, _ = mi.make_activations(shape.H, T, seed)
        x_g.copy_(to_dev(xb))
        torch.cuda.synchronize()
        say(f"[graph] replay seed {seed}")
        graph.replay()
        torch.cuda.synchronize()
        ebufs, eouts = _buffers(shape, N_LAYERS)
        moe.stack_forward(ebufs, to_dev(xb), layers, eouts)   # eager work between the replays
        torch.cuda.synchronize()
        for l in range(N_LAYERS):
            assert np.array_equal(to_host(gouts[l], np.uint16), to_host(eouts[l], np.uint16)), f"layer {l}"
            assert torch.equal(gbufs[l].topk_ids, ebufs[l].topk_ids)
            assert int(gbufs[l].sync.abs().sum().item()) == 0 and int(gbufs[l].ffn_sync.abs().sum().item()) == 0
