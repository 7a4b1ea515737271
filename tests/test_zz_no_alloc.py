"""moe_expert_ffn_fused_noalloc, the FFN entry point that allocates nothing:
through the C ABI, on two calls in a row (the second with fewer tokens, so it
must not see the first call's counters or workspace), its expert rows equal
moe_expert_ffn_fused's bit for bit on the same routing; its fault word stays
zero; dims whose workspace exceeds the fixed array are refused before
anything is enqueued.  Shapes: the one-launch decode kernels (A3B-style
q4 and q2), the persistent kernels (a shape whose decode tile does not fit
LDS) and the vector path (two launches)."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import quantized_expert_ffn_gemv_amd as moe

from gpu_util import say, to_dev, to_host, upload_layer

pytestmark = pytest.mark.gpu

BIG_TILE = mi.LayerShape("big_tile", H=3072, E=4, k=2, I=2048, tokens=(16,), bits=(4, 2), zipf_s=None,
                         n_resident=2)
CASES = [("a3b", 4, (32, 8), moe.ALGO_AUTO), ("a3b", 2, (8, 1), moe.ALGO_AUTO),
         ("big_tile", 4, (16, 5), moe.ALGO_AUTO), ("big_tile", 2, (16, 3), moe.ALGO_AUTO),
         ("a3b", 4, (32, 8), moe.ALGO_GEMV)]


def _route(L, d, x_d):
    buf = moe.LayerBuffers.allocate(d, L.bits)
    sh = L.shape
    moe.route_dispatch(d, x_d, L.Wr_d, L.bias_d, True, buf.logits, buf.topk_ids, buf.topk_w, L.table_d, sh.E,
                       buf.pair_slot, buf.miss, buf.n_miss, buf.counts, buf.offsets, buf.sorted_pairs,
                       buf.pair_to_row, buf.active, buf.n_active, buf.work_list, buf.n_work, sync=buf.sync)
    return buf


_UPLOADED = {}


def _layer(name, bits):
    if (name, bits) not in _UPLOADED:
        _UPLOADED.clear()
        torch.cuda.empty_cache()
        shape = BIG_TILE if name == "big_tile" else mi.CONFIGS[name]
        say(f"[upload] {name} q{bits}")
        _UPLOADED[(name, bits)] = upload_layer(shape, bits, seed=0)
    return _UPLOADED[(name, bits)]


@pytest.mark.parametrize("name,bits,Ts,algo", CASES,
                         ids=[f"{c[0]}_q{c[1]}_T{c[2][0]}-{c[2][1]}_algo{c[3]}" for c in CASES])
def test_noalloc_matches_fused(name, bits, Ts, algo):
    L = _layer(name, bits)
    sh = L.shape
    fault = torch.zeros(1, dtype=torch.int32, device="cuda")
    for T, seed in zip(Ts, (41, 42)):
        d = moe.dims(T, sh.H, sh.I, sh.E, sh.k)
        xb, _ = mi.make_activations(sh.H, T, seed)
        x_d = to_dev(xb)
        buf = _route(L, d, x_d)
        ref = torch.full_like(buf.y_rows, -1)
        got = torch.full_like(buf.y_rows, -2)
        say(f"[run] noalloc {name} q{bits} T={T} algo={algo}")
        moe.expert_ffn_fused(d, bits, x_d, buf.work_list, buf.n_work, L.weights_d, buf.workspace, ref, buf.ffn_sync,
                             algo)
        moe.expert_ffn_fused_noalloc(d, bits, x_d, buf.work_list, buf.n_work, L.weights_d, got, fault, algo)
        torch.cuda.synchronize()
        P = T * sh.k
        a, b = to_host(got, np.uint16)[:P], to_host(ref, np.uint16)[:P]
        assert np.array_equal(a, b), f"{int((a != b).any(axis=1).sum())} of {P} rows differ"
        assert int(fault.item()) == 0
        assert int(buf.ffn_sync.abs().sum().item()) == 0


def test_noalloc_refuses_dims_beyond_the_fixed_array():
    """4096 tokens x 8 picks at intermediate 768 need ~150 MB of workspace on the
    per-tile path: refused on the host, nothing enqueued."""
    d = moe.dims(4096, 2048, 768, 128, 8)
    need = moe.workspace_bytes(d, moe.OP_FFN, 4, moe.ALGO_MFMA)
    assert need > moe.NOALLOC_WORKSPACE_BYTES
    L = moe.lib()
    w = moe.QWeightsC()
    fake = 0x10000000
    for m in range(3):
        w.q[m] = w.scale[m] = w.bias[m] = fake
    import ctypes
    st = L.moe_expert_ffn_fused_noalloc(ctypes.byref(d), 4, fake, fake, fake, ctypes.byref(w), moe.ALGO_MFMA, fake,
                                        None, None)
    assert st == moe.ERR_WORKSPACE and "fixed scratch" in moe.last_error()
