"""GPU parity at groups of 64 and 32 weights per scale and bias.

Groups of 64 ("Strata" page, section 4.4) and 32 (the laptop page, section
4.2) at the A3B-style decode shape (T = 8 and 32) and the 512-expert
single-token shape, 4-bit and 2-bit codes: every routed row of the FFN
against the oracle (which takes the group size from the scales), the routing
stages bit-exact, the combine bit-exact given the same rows.  The one-launch
FFN and the separate gate/up and down calls both run; the vector-ALU
algorithm runs where one scale covers a 16-byte chunk of codes.  Shapes whose
tiles do not fit LDS take the vector-ALU path under MOE_ALGO_AUTO.
"""
import dataclasses

import numpy as np
import pytest
import torch

import moe_inputs as mi
import quantized_expert_ffn_gemv_amd as moe
from gpu_util import (check_combine_exact, check_ffn, check_logits, check_lookup, check_permute, check_topk,
                      run_layer, say, upload_layer)

pytestmark = pytest.mark.gpu

_LAYERS = {}


def layer(shape, bits):
    key = (shape.name, shape.group, bits)
    if key not in _LAYERS:
        _LAYERS.clear()
        torch.cuda.empty_cache()
        say(f"[upload] {shape.name} g{shape.group} q{bits}")
        _LAYERS[key] = upload_layer(shape, bits, seed=0)
    return _LAYERS[key]


def stages(L, T, seed, algo=moe.ALGO_AUTO, fused=True):
    xb, res = mi.make_activations(L.shape.H, T, seed)
    say(f"[run] {L.shape.name} g{L.shape.group} q{L.bits} T={T} algo={algo} fused={fused}")
    g = run_layer(L, xb, res, algo=algo, fused=fused)
    check_logits(g, L, xb)
    check_topk(g, L)
    check_lookup(g, L)
    check_permute(g, L)
    mr, mae = check_ffn(g, L, xb)
    check_combine_exact(g, L, res)
    say(f"[ok] FFN max_rel {mr:.2e} mae_norm {mae:.2e}")


def grouped(name, group, bits):
    return dataclasses.replace(mi.CONFIGS[name], group=group, bits=(bits,))


DECODE = [("a3b", 64, 4, 8), ("a3b", 64, 4, 32), ("a3b", 32, 4, 8), ("a3b", 32, 4, 32),
          ("a3b", 64, 2, 32), ("a3b", 32, 2, 8), ("e512", 64, 4, 1), ("e512", 32, 2, 1)]


@pytest.mark.parametrize("name,group,bits,T", DECODE, ids=[f"{n}-g{g}-q{b}-T{t}" for n, g, b, t in DECODE])
def test_decode_kernels_at_finer_groups(name, group, bits, T):
    L = layer(grouped(name, group, bits), bits)
    stages(L, T, seed=21, fused=True)
    stages(L, T, seed=22, fused=False)


GEMV = [("a3b", 64, 2, 8), ("a3b", 32, 4, 32), ("a3b", 64, 4, 1)]


@pytest.mark.parametrize("name,group,bits,T", GEMV, ids=[f"{n}-g{g}-q{b}-T{t}" for n, g, b, t in GEMV])
def test_vector_alu_path_at_finer_groups(name, group, bits, T):
    L = layer(grouped(name, group, bits), bits)
    stages(L, T, seed=23, algo=moe.ALGO_GEMV, fused=False)


def test_large_tiles_take_the_vector_alu_path():
    """H 3072, I 2048, 16 tokens: neither decode tile fits LDS; with groups of
    64 the matrix-core algorithm refuses and AUTO runs the vector-ALU kernels."""
    shape = mi.LayerShape("big_g64", H=3072, E=4, k=2, I=2048, tokens=(16,), bits=(4,), zipf_s=None,
                          n_resident=2, group=64)
    L = layer(shape, 4)
    stages(L, 16, seed=24, algo=moe.ALGO_AUTO, fused=False)
    xb, res = mi.make_activations(shape.H, 16, 25)
    with pytest.raises(moe.MoeError) as ex:
        run_layer(L, xb, res, algo=moe.ALGO_MFMA, fused=False)
    assert ex.value.status == moe.ERR_UNSUPPORTED


# Grouped GEMM at groups of 64 and 32: token counts that make AUTO take it
# (at least 64 pairs per expert), items with fewer than 8 (gate/up) or 4 (down)
# tiles, row blocks past I and H (I = 384, H = 640), every FFN row checked.
GEMM_GROUPS = [
    (mi.LayerShape("gemm_g64a", H=256, E=4, k=2, I=256, tokens=(200,), bits=(4,), zipf_s=None, n_resident=2, group=64),
     200),
    (mi.LayerShape("gemm_g32a", H=256, E=4, k=2, I=256, tokens=(200,), bits=(4,), zipf_s=None, n_resident=2, group=32),
     200),
    (mi.LayerShape("gemm_g64b", H=1024, E=6, k=3, I=384, tokens=(130,), bits=(4,), zipf_s=0.8, n_resident=3, group=64),
     130),
    (mi.LayerShape("gemm_g32c", H=640, E=3, k=1, I=512, tokens=(197,), bits=(4,), zipf_s=None, n_resident=1,
                   group=32), 197),
]


@pytest.mark.parametrize("shape,T", GEMM_GROUPS, ids=[s.name for s, _ in GEMM_GROUPS])
def test_grouped_gemm_at_finer_groups(shape, T):
    L = layer(shape, 4)
    stages(L, T, seed=26, algo=moe.ALGO_GEMM, fused=False)
    stages(L, T, seed=27, algo=moe.ALGO_AUTO, fused=True)
