"""Groups whose fp16 scale is zero, on every FFN path, against the oracle.

A zero scale makes a group's weights equal to its bias (w = q s + b).  The
decode and vector kernels fold each group with its own scale, so they need
nothing special; the grouped GEMM's ratio chain divides by the next group's
scale and replaces a zero one by 2^-40 (its group then adds 2^-43 of its code
sum instead of 0, far below the tolerance).  About one group in nine of every
matrix gets a zero scale, in a fixed pattern, on the device and in the oracle's
copy of the weights alike.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
import quantized_expert_ffn_gemv_amd as moe

from gpu_util import run_layer, say, tolerance_metrics, upload_layer

pytestmark = pytest.mark.gpu

GEMM_SHAPE = mi.LayerShape("zs_gemm", H=256, E=4, k=2, I=256, tokens=(200,), bits=(4,), zipf_s=None, n_resident=2)
GEMM_G32 = mi.LayerShape("zs_gemm_g32", H=256, E=4, k=2, I=256, tokens=(200,), bits=(4,), zipf_s=None, n_resident=2,
                         group=32)
# the x tile does not fit 80 KB at T = 16: the x-tile gate/up and the streaming down
BIG_SHAPE = mi.LayerShape("zs_big", H=3072, E=4, k=2, I=2048, tokens=(16,), bits=(4, 2), zipf_s=None, n_resident=2)
# 8 token rows of H = 5120 do not fit the decode tile: the int8-plane x-tile gate/up
XT8_SHAPE = mi.LayerShape("zs_xt8", H=5120, E=4, k=2, I=1024, tokens=(8,), bits=(4, 2), zipf_s=None, n_resident=2)

CASES = [
    ("gemm_q4", GEMM_SHAPE, 4, moe.ALGO_GEMM),
    ("gemm_q4_g32", GEMM_G32, 4, moe.ALGO_GEMM),
    ("big_q4_mfma", BIG_SHAPE, 4, moe.ALGO_MFMA),
    ("big_q2_mfma", BIG_SHAPE, 2, moe.ALGO_MFMA),
    ("xt8_q4_mfma", XT8_SHAPE, 4, moe.ALGO_MFMA),
    ("xt8_q2_mfma", XT8_SHAPE, 2, moe.ALGO_MFMA),
    ("tiny_q4_mfma", mi.CONFIGS["tiny"], 4, moe.ALGO_MFMA),
    ("tiny_q2_gemv", mi.CONFIGS["tiny"], 2, moe.ALGO_GEMV),
]


def zero_mask(N: int, NG: int, e: int, mi_: int) -> np.ndarray:
    n = np.arange(N)[:, None]
    g = np.arange(NG)[None, :]
    return (n * 7 + g * 3 + e * 5 + mi_) % 9 == 0


@pytest.mark.parametrize("name,shape,bits,algo", CASES, ids=[c[0] for c in CASES])
def test_zero_scales_against_oracle(name, shape, bits, algo):
    L = upload_layer(shape, bits, seed=0)
    for i, m in enumerate(mi.MATRICES):
        s = L.weights_d.scale[i]
        for e in range(shape.E):
            mask = torch.from_numpy(zero_mask(s.shape[1], s.shape[2], e, i)).to(s.device)
            s[e][mask] = 0
    torch.cuda.synchronize()
    T = shape.tokens[0]
    xb, res = mi.make_activations(shape.H, T, 11)
    say(f"[run] zero scales {name} T={T} algo={algo}")
    g = run_layer(L, xb, res, algo=algo)
    ids = g["ids"].ravel()
    P = T * shape.k
    rows = list(range(P)) if P <= 64 else [int(r) for r in np.random.default_rng(2).choice(P, 64, replace=False)]
    W = mi.make_expert_weights(shape, bits, 0, experts=sorted({int(ids[int(g["sorted_pairs"][r])]) for r in rows}))
    for i, m in enumerate(mi.MATRICES):
        for j, e in enumerate(W.experts):
            sc = W.scale[m][j]
            sc[zero_mask(sc.shape[0], sc.shape[1], int(e), i)] = 0
    _, ys = oracle.expert_ffn(xb, ids, g["sorted_pairs"], W, shape.k, rows=rows)
    max_rel, mae = tolerance_metrics(np.stack([g["y_rows"][r] for r in rows]), np.stack([ys[r] for r in rows]))
    say(f"[ok] zero scales {name}: max_rel {max_rel:.2e} mae_norm {mae:.2e}")
    assert max_rel <= 1e-2 and mae <= 1e-3, (max_rel, mae)
    del L
    torch.cuda.empty_cache()
