"""GPU parity: every stage of the layer through the C ABI against the oracle.

Shapes: the five workload shapes of the pages' models (tiny, A3B-style,
64-expert, 512-expert in 4 and 2 bits, 4096-token prefill) plus ragged shapes
(H, I not multiples of 256, odd token counts) and the degenerate T = 0.
Rules are listed in gpu_util.  The oracle never sees anything the GPU
computed except, where stated, the GPU's routing decisions (so that a
float32 near-tie cannot change which expert a row is compared against).
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
import quantized_expert_ffn_gemv_amd as moe

from work_tiles import expected_work_list
from gpu_util import (check_combine_exact, check_ffn, check_logits, check_lookup, check_permute,
                      check_topk, run_layer, say, to_dev, to_host, tolerance_metrics, upload_layer)

pytestmark = pytest.mark.gpu

_LAYERS = {}


def layer(name, bits=4, shape=None):
    key = (name, bits)
    if key not in _LAYERS:
        _LAYERS.clear()                     # keep at most one big layer resident
        torch.cuda.empty_cache()
        say(f"[upload] {name} q{bits}")
        _LAYERS[key] = upload_layer(shape or mi.CONFIGS[name], bits, seed=0)
    return _LAYERS[key]


def _stages(L, T, seed=0, ffn_rows=None, n_idx=None, algo=moe.ALGO_AUTO):
    xb, res = mi.make_activations(L.shape.H, T, seed)
    say(f"[run] {L.shape.name} q{L.bits} T={T} algo={algo}")
    g = run_layer(L, xb, res, algo=algo)
    check_logits(g, L, xb)
    check_topk(g, L)
    check_lookup(g, L)
    check_permute(g, L)
    mr, mae = check_ffn(g, L, xb, rows=ffn_rows, n_idx=n_idx)
    check_combine_exact(g, L, res)
    say(f"[ok] {L.shape.name} T={T}: FFN max_rel {mr:.2e} mae_norm {mae:.2e}")
    return g, xb, res


ALGOS = [moe.ALGO_MFMA, moe.ALGO_GEMV]
ALGO_IDS = ["mfma", "gemv"]


@pytest.mark.parametrize("algo", ALGOS, ids=ALGO_IDS)
def test_tiny_layer_all_stages_and_end_to_end(algo):
    L = layer("tiny")
    g, xb, res = _stages(L, 4, algo=algo)
    # end to end from raw inputs (oracle routes on its own logits)
    W = mi.make_expert_weights(L.shape, 4, 0)
    ref = oracle.layer(xb, L.Wr, L.bias, W, L.shape.k, L.table, L.shape.E, res)
    assert np.array_equal(ref["ids"], g["ids"])
    mr, mae = tolerance_metrics(g["out"], ref["out"])
    assert mr <= 1e-2 and mae <= 1e-3


@pytest.mark.parametrize("algo", ALGOS, ids=ALGO_IDS)
@pytest.mark.parametrize("T", [1, 8, 32])
def test_a3b_layer(T, algo):
    L = layer("a3b")
    P = T * L.shape.k
    rows = None if T <= 8 else list(range(0, P, 3))
    _stages(L, T, ffn_rows=rows, algo=algo)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_e64_layer_with_miss_list(seed):
    L = layer("e64")
    rng = np.random.default_rng(seed)
    n_idx = np.sort(rng.choice(L.shape.H, 96, replace=False)).astype(np.int32)
    g, _, _ = _stages(L, 8, seed=seed, n_idx=n_idx)
    assert (L.table >= 0).sum() == 24
    say(f"[e64 seed {seed}] n_miss={g['n_miss']} miss={g['miss'][:g['n_miss']].tolist()}")


@pytest.mark.parametrize("algo", ALGOS, ids=ALGO_IDS)
@pytest.mark.parametrize("bits", [4, 2])
def test_e512_layer(bits, algo):
    L = layer("e512", bits)
    _stages(L, 1, algo=algo)


@pytest.mark.parametrize("algo", [moe.ALGO_AUTO, moe.ALGO_MFMA], ids=["auto_gemm", "mfma"])
def test_prefill_layer_sampled_rows(algo):
    L = layer("prefill")
    T = 4096
    xb, res = mi.make_activations(L.shape.H, T, 0)
    say(f"[run] prefill T=4096 algo={algo}")
    g = run_layer(L, xb, res, algo=algo)
    check_logits(g, L, xb)
    check_topk(g, L)
    check_lookup(g, L)
    check_permute(g, L)
    # rows: first and last row of every 8th active expert plus the largest expert
    counts, offsets = g["counts"], g["offsets"]
    act = np.nonzero(counts)[0]
    big = int(np.argmax(counts))
    rows = set()
    for e in list(act[::8]) + [big]:
        rows.add(int(offsets[e]))
        rows.add(int(offsets[e] + counts[e] - 1))
    rows = sorted(rows)
    say(f"[prefill] checking {len(rows)} rows; largest expert {big} has {counts[big]} pairs")
    check_ffn(g, L, xb, rows=rows)
    check_combine_exact(g, L, res)


RAGGED = [
    mi.LayerShape("ragged_a", H=384, E=5, k=3, I=640, tokens=(7,), bits=(4,), zipf_s=None, n_resident=2),
    mi.LayerShape("ragged_b", H=640, E=12, k=4, I=384, tokens=(3,), bits=(4,), zipf_s=0.8, n_resident=5),
    mi.LayerShape("ragged_c", H=128, E=3, k=3, I=128, tokens=(5,), bits=(4,), zipf_s=None, n_resident=0),
]


@pytest.mark.parametrize("algo", ALGOS, ids=ALGO_IDS)
@pytest.mark.parametrize("shape", RAGGED, ids=[s.name for s in RAGGED])
@pytest.mark.parametrize("bits", [4, 2])
def test_ragged_shapes(shape, bits, algo):
    L = layer(shape.name, bits, shape)
    _stages(L, shape.tokens[0], seed=3, algo=algo)


# A shape whose decode tiles do not fit LDS at T = 16 (the x tile alone is 96 KB),
# so the matrix-core path takes the persistent kernels (the 64-expert layer's
# kernels) at a small E and I: every element checked, both algorithms, both
# code widths, several entries per expert and ragged rows.
BIG_TILE = mi.LayerShape("big_tile", H=3072, E=4, k=2, I=2048, tokens=(16,), bits=(4, 2), zipf_s=None,
                         n_resident=2)


@pytest.mark.parametrize("algo", ALGOS, ids=ALGO_IDS)
@pytest.mark.parametrize("bits", [4, 2])
def test_persistent_kernel_shape_every_element(bits, algo):
    L = layer(BIG_TILE.name, bits, BIG_TILE)
    g, _, _ = _stages(L, 16, seed=8, algo=algo)
    assert g["counts"].max() > 1


# Shapes whose down tile does not fit LDS, so the down projection streams h
# (as int8 planes) through LDS in chunks of K: tiles of 2, 7 and 12 token rows
# (one, two and three blocks of 4 tokens), every element checked.  The first
# three have fewer row blocks than CUs, so K is split over the workgroups; the
# last has enough for whole row blocks of 80 rows per workgroup.
STREAM_SHAPES = [
    mi.LayerShape("stream_1blk", H=512, E=3, k=1, I=16384, tokens=(2,), bits=(4, 2), zipf_s=None, n_resident=1),
    mi.LayerShape("stream_2blk", H=3072, E=2, k=2, I=2048, tokens=(7,), bits=(4, 2), zipf_s=None, n_resident=1),
    mi.LayerShape("stream_3blk", H=3072, E=2, k=2, I=2048, tokens=(12,), bits=(4, 2), zipf_s=None, n_resident=1),
    mi.LayerShape("rows_80", H=2560, E=8, k=2, I=2048, tokens=(16,), bits=(4, 2), zipf_s=None, n_resident=2),
]


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("shape", STREAM_SHAPES, ids=[s.name for s in STREAM_SHAPES])
def test_streaming_down_shapes(shape, bits):
    L = layer(shape.name, bits, shape)
    _stages(L, shape.tokens[0], seed=9, algo=moe.ALGO_MFMA)


@pytest.mark.parametrize("bits", [4, 2])
def test_row_block_down_second_round(bits):
    """More row blocks than the row-block down's grid (3 workgroups per CU, 80
    rows per block at H = 2560): some workgroups take a second block."""
    shape = mi.LayerShape("rows_multi", H=2560, E=32, k=2, I=2048, tokens=(32,), bits=(4, 2), zipf_s=None,
                          n_resident=2)
    L = layer(shape.name, bits, shape)
    g, _, _ = _stages(L, 32, seed=10, algo=moe.ALGO_MFMA)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert g["n_work"] * (shape.H // 80) > 3 * cus, g["n_work"]


@pytest.mark.parametrize("bits", [4, 2])
def test_many_tokens_per_expert_mfma(bits):
    """Experts serving more than one 16-token tile (several MFMA passes)."""
    shape = mi.LayerShape("crowd", H=512, E=4, k=2, I=256, tokens=(40,), bits=(bits,), zipf_s=None, n_resident=2)
    L = layer(shape.name, bits, shape)
    g, _, _ = _stages(L, 40, seed=4, algo=moe.ALGO_MFMA)
    assert g["counts"].max() > 16


# Grouped-GEMM shapes: ring depths 1, 2 and 4 on both kernels, items with fewer
# than 4 tiles, ragged last tiles, k = 1.
GEMM_SHAPES = [
    mi.LayerShape("gemm_a", H=256, E=4, k=2, I=256, tokens=(200,), bits=(4,), zipf_s=None, n_resident=2),
    mi.LayerShape("gemm_b", H=1024, E=6, k=3, I=384, tokens=(130,), bits=(4,), zipf_s=0.8, n_resident=3),
    mi.LayerShape("gemm_c", H=640, E=3, k=1, I=512, tokens=(97,), bits=(4,), zipf_s=None, n_resident=1),
]


@pytest.mark.parametrize("shape", GEMM_SHAPES, ids=[s.name for s in GEMM_SHAPES])
def test_grouped_gemm_shapes(shape):
    L = layer(shape.name, 4, shape)
    T = shape.tokens[0]
    rows = None if shape.name != "gemm_b" else list(range(0, T * shape.k, 4))
    g, _, _ = _stages(L, T, seed=5, ffn_rows=rows, algo=moe.ALGO_GEMM)
    assert g["counts"].max() > 16       # several work tiles per expert


def test_grouped_gemm_auto_choice():
    """AUTO takes the grouped GEMM when experts average >= 64 tokens, and its
    outputs agree with the per-tile path to the same tolerance."""
    shape = GEMM_SHAPES[0]
    L = layer(shape.name, 4, shape)
    xb, res = mi.make_activations(shape.H, 200, 6)
    a = run_layer(L, xb, res, algo=moe.ALGO_AUTO)
    b = run_layer(L, xb, res, algo=moe.ALGO_GEMM)
    c = run_layer(L, xb, res, algo=moe.ALGO_MFMA)
    assert np.array_equal(a["y_rows"], b["y_rows"])
    mr, mae = tolerance_metrics(b["y_rows"], c["y_rows"])
    assert mr <= 1e-2 and mae <= 1e-3


def test_split_calls_gateup_h_matches_oracle():
    """moe_expert_gateup alone (vector path): float32 h rows against the oracle."""
    L = layer("a3b")
    sh = L.shape
    T = 8
    xb, res = mi.make_activations(sh.H, T, 9)
    g = run_layer(L, xb, res, algo=moe.ALGO_GEMV)
    d = moe.dims(T, sh.H, sh.I, sh.E, sh.k)
    buf = moe.LayerBuffers.allocate(d, 4, moe.ALGO_GEMV)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    moe.expert_gateup(d, 4, dev(xb.view(np.int16)), dev(g["work_list"]), dev(np.array([g["n_work"]], np.int32)),
                      L.weights_d, buf.workspace, moe.ALGO_GEMV)
    torch.cuda.synchronize()
    P = T * sh.k
    h = buf.workspace[: P * sh.I * 4].view(torch.float32).reshape(P, sh.I).cpu().numpy()
    ids = g["ids"].ravel()
    W = mi.make_expert_weights(sh, 4, 0, experts=np.unique(ids))
    hs, _ = oracle.expert_ffn(xb, ids, g["sorted_pairs"], W, sh.k, rows=list(range(0, P, 5)), n_idx=np.array([0], np.int32))
    for r, href in hs.items():
        # float32 accumulation: error relative to the row's scale, not to h_i itself
        # (h_i = silu(a_i) * u_i has zero crossings)
        href = href.astype(np.float64)
        err = np.abs(h[r].astype(np.float64) - href) / (np.abs(href) + np.sqrt(np.mean(href ** 2)))
        assert err.max() < 1e-5, (r, err.max())


def test_zero_tokens_is_a_no_op():
    L = layer("tiny")
    sh = L.shape
    d = moe.dims(0, sh.H, sh.I, sh.E, sh.k)
    buf = moe.LayerBuffers.allocate(d, 4)
    x = torch.zeros((0, sh.H), dtype=torch.int16, device="cuda")
    out = torch.zeros((0, sh.H), dtype=torch.int16, device="cuda")
    moe.layer_forward(buf, x, L.Wr_d, L.bias_d, L.weights_d, L.table_d, sh.E, x, out)
    torch.cuda.synchronize()
    assert int(buf.n_miss.item()) == 0 and int(buf.n_active.item()) == 0 and int(buf.n_work.item()) == 0
    assert int(buf.counts.sum().item()) == 0


def test_deterministic_reruns():
    L = layer("a3b")
    xb, res = mi.make_activations(L.shape.H, 32, 5)
    a = run_layer(L, xb, res)
    b = run_layer(L, xb, res)
    for key in ("logits", "ids", "gates", "sorted_pairs", "y_rows", "out"):
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), key


def test_residency_never_changes_results():
    L = layer("a3b")
    xb, res = mi.make_activations(L.shape.H, 8, 6)
    part = run_layer(L, xb, res)
    full = run_layer(L, xb, res, table=np.arange(L.shape.E, dtype=np.int32))
    none = run_layer(L, xb, res, table=np.full(L.shape.E, -1, np.int32))
    for key in ("ids", "y_rows", "out"):
        assert np.array_equal(part[key], full[key]) and np.array_equal(part[key], none[key]), key
    assert full["n_miss"] == 0
    assert none["n_miss"] == len(np.unique(none["ids"]))
    assert part["n_miss"] > 0


def test_doorbell_and_last_use():
    L = layer("e64")
    sh = L.shape
    xb, res = mi.make_activations(sh.H, 8, 0)
    d = moe.dims(8, sh.H, sh.I, sh.E, sh.k)
    buf = moe.LayerBuffers.allocate(d, 4)
    x_d = torch.from_numpy(xb.view(np.int16)).cuda()
    moe.route_topk(d, x_d, L.Wr_d, L.bias_d, True, buf.logits, buf.topk_ids, buf.topk_w)
    bell = torch.zeros(1, dtype=torch.int32, pin_memory=True)
    last_use = torch.zeros(sh.E, dtype=torch.int32, device="cuda")
    # only the 4 most popular experts resident, so this batch is sure to miss
    table = mi.make_slot_table(sh, 0, n_resident=4)
    moe.slot_lookup(d, buf.topk_ids, torch.from_numpy(table).cuda(), sh.E, buf.pair_slot, buf.miss,
                    buf.n_miss, host_doorbell=bell, last_use=last_use, step=77)
    torch.cuda.synchronize()
    ids = buf.topk_ids.cpu().numpy()
    ref = oracle.slot_lookup(ids, table, sh.E, last_use=np.zeros(sh.E, np.uint32), step=77, doorbell=0)
    assert np.array_equal(buf.miss.cpu().numpy()[: ref["n_miss"]], ref["miss"])
    assert int(bell.item()) == ref["doorbell"] == ref["n_miss"] > 0
    assert np.array_equal(last_use.cpu().numpy().view(np.uint32), ref["last_use"])
    # all resident: the doorbell is not rung
    bell.zero_()
    moe.slot_lookup(d, buf.topk_ids, torch.arange(sh.E, dtype=torch.int32, device="cuda"), sh.E,
                    buf.pair_slot, buf.miss, buf.n_miss, host_doorbell=bell)
    torch.cuda.synchronize()
    assert int(bell.item()) == 0 and int(buf.n_miss.item()) == 0


@pytest.mark.parametrize("name,T", [("tiny", 4), ("a3b", 1), ("a3b", 32), ("e512", 1), ("e64", 8)])
def test_route_dispatch_matches_separate_calls(name, T):
    """moe_route_dispatch (one launch for top-k, lookup and grouping) gives the
    separate calls' outputs bit for bit; every layer test above also checks it
    against the oracle, since layer_forward uses it."""
    L = layer(name)
    xb, res = mi.make_activations(L.shape.H, T, 11)
    a = run_layer(L, xb, res, fused=True)
    b = run_layer(L, xb, res, fused=False)
    for key in ("logits", "ids", "gates", "pair_slot", "miss", "n_miss", "counts", "offsets", "sorted_pairs",
                "pair_to_row", "active", "n_active", "work_list", "n_work", "y_rows", "out"):
        if np.ndim(a[key]) == 0:
            assert a[key] == b[key], key
            continue
        va, vb = np.asarray(a[key]), np.asarray(b[key])
        if key in ("miss", "active"):
            n = a["n_miss"] if key == "miss" else a["n_active"]
            va, vb = va[:n], vb[:n]
        if key == "work_list":
            va, vb = va[: a["n_work"]], vb[: a["n_work"]]
        assert np.array_equal(va.view(np.uint8), vb.view(np.uint8)), key


@pytest.mark.parametrize("name,T,n_res", [("e64", 8, 4), ("a3b", 32, 20)])
def test_route_dispatch_doorbell_and_last_use(name, T, n_res):
    """The one-launch routing's slot lookup (one-wave path at T*k <= 64, workgroup
    path above) with a doorbell and last_use, against the oracle."""
    L = layer(name)
    sh = L.shape
    xb, _ = mi.make_activations(sh.H, T, 0)
    d = moe.dims(T, sh.H, sh.I, sh.E, sh.k)
    buf = moe.LayerBuffers.allocate(d, 4)
    x_d = torch.from_numpy(xb.view(np.int16)).cuda()
    bell = torch.zeros(1, dtype=torch.int32, pin_memory=True)
    last_use = torch.zeros(sh.E, dtype=torch.int32, device="cuda")
    table = mi.make_slot_table(sh, 0, n_resident=n_res)
    moe.route_dispatch(d, x_d, L.Wr_d, L.bias_d, True, buf.logits, buf.topk_ids, buf.topk_w,
                       torch.from_numpy(table).cuda(), sh.E, buf.pair_slot, buf.miss, buf.n_miss, buf.counts,
                       buf.offsets, buf.sorted_pairs, buf.pair_to_row, buf.active, buf.n_active, buf.work_list,
                       buf.n_work, host_doorbell=bell, last_use=last_use, step=91, sync=buf.sync)
    torch.cuda.synchronize()
    ids = buf.topk_ids.cpu().numpy()
    check_topk(dict(logits=buf.logits.cpu().numpy(), ids=ids, gates=buf.topk_w.cpu().numpy()), L)
    ref = oracle.slot_lookup(ids, table, sh.E, last_use=np.zeros(sh.E, np.uint32), step=91, doorbell=0)
    assert np.array_equal(buf.miss.cpu().numpy()[: ref["n_miss"]], ref["miss"])
    assert int(bell.item()) == ref["doorbell"] == ref["n_miss"] > 0
    assert np.array_equal(last_use.cpu().numpy().view(np.uint32), ref["last_use"])


@pytest.mark.parametrize("name,T", [("tiny", 4), ("a3b", 32), ("e512", 1)])
def test_route_dispatch_paths_agree(name, T):
    """The one-launch routing (with the sync counters), the two-launch routing
    (sync = NULL) and the separate calls give the same outputs bit for bit, and
    the counters are left zero for the next call (which is checked too), on
    two different batches in a row."""
    L = layer(name)
    sh = L.shape
    # two different batches through the same buffers: a stage that read the
    # previous call's logits or ids would show up in the second call
    xs = [torch.from_numpy(mi.make_activations(sh.H, T, seed)[0].view(np.int16)).cuda() for seed in (12, 13)]
    d = moe.dims(T, sh.H, sh.I, sh.E, sh.k)
    keys = ("logits", "topk_ids", "topk_w", "pair_slot", "n_miss", "counts", "offsets", "sorted_pairs",
            "pair_to_row", "n_active", "n_work")

    def dispatch(buf, sync, x_d):
        moe.route_dispatch(d, x_d, L.Wr_d, L.bias_d, True, buf.logits, buf.topk_ids, buf.topk_w, L.table_d, sh.E,
                           buf.pair_slot, buf.miss, buf.n_miss, buf.counts, buf.offsets, buf.sorted_pairs,
                           buf.pair_to_row, buf.active, buf.n_active, buf.work_list, buf.n_work, sync=sync)

    one = moe.LayerBuffers.allocate(d, 4)
    two = moe.LayerBuffers.allocate(d, 4)
    sep = moe.LayerBuffers.allocate(d, 4)
    for x_d in xs:                                       # the second call relies on the counters' reset
        dispatch(one, one.sync, x_d)
        dispatch(two, None, x_d)
        moe.route_topk(d, x_d, L.Wr_d, L.bias_d, True, sep.logits, sep.topk_ids, sep.topk_w)
        moe.slot_lookup(d, sep.topk_ids, L.table_d, sh.E, sep.pair_slot, sep.miss, sep.n_miss)
        moe.permute(d, sep.topk_ids, sep.counts, sep.offsets, sep.sorted_pairs, sep.pair_to_row, sep.active,
                    sep.n_active, sep.work_list, sep.n_work)
        torch.cuda.synchronize()
        assert int(one.sync.abs().sum().item()) == 0
        for key in keys:
            a = getattr(one, key).cpu().numpy().view(np.uint8)
            assert np.array_equal(a, getattr(two, key).cpu().numpy().view(np.uint8)), key
            assert np.array_equal(a, getattr(sep, key).cpu().numpy().view(np.uint8)), key
        nw = int(one.n_work.item())
        assert np.array_equal(one.work_list[:nw].cpu().numpy(), sep.work_list[:nw].cpu().numpy())
        na = int(one.n_active.item())
        assert np.array_equal(one.active[:na].cpu().numpy(), sep.active[:na].cpu().numpy())
        g = dict(logits=one.logits.cpu().numpy(), ids=one.topk_ids.cpu().numpy(), gates=one.topk_w.cpu().numpy())
        check_topk(g, L)


# (E, H, T, k, pool): the router is the identity on the first E features,
# so each token's logits are its crafted activations; experts come from a pool
# of `pool` ids, so they repeat across tokens and some get several tiles
CRAFTED = [(1000, 1024, 8, 8, 24), (300, 384, 16, 4, 40), (1000, 1024, 32, 8, 12), (520, 640, 2, 32, 520),
           (256, 256, 1, 8, 256), (64, 128, 64, 1, 5)]


@pytest.mark.parametrize("E,H,T,k,pool", CRAFTED, ids=[f"E{c[0]}_T{c[2]}_k{c[3]}" for c in CRAFTED])
def test_dispatch_crafted_ids(E, H, T, k, pool):
    """Lookup and grouping on chosen expert ids (wide expert counts, repeated
    experts, multi-tile experts, misses): the one-launch routing and the
    two-launch routing against the oracle's lookup, permutation and work list."""
    rng = np.random.default_rng(E + 7 * T + k)
    choices = rng.permutation(E)[:pool]
    ids_want = np.stack([rng.choice(choices, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    x = np.zeros((T, H), np.float32)
    for t in range(T):
        x[t, ids_want[t]] = 100.0 + np.arange(k)[::-1]          # exact in bf16, distinct, descending
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    w = np.zeros((E, H), np.float32)
    w[np.arange(E), np.arange(E)] = 1.0
    table = np.full(E, -1, np.int32)
    res = rng.permutation(E)[: E // 3]
    table[res] = np.arange(res.size, dtype=np.int32)
    d = moe.dims(T, H, 256, E, k)
    for sync in (True, False):
        buf = moe.LayerBuffers.allocate(d, 4)
        say(f"[run] crafted dispatch E={E} T={T} k={k} sync={sync}")
        moe.route_dispatch(d, to_dev(xb), to_dev(w), None, True, buf.logits, buf.topk_ids, buf.topk_w, to_dev(table),
                           res.size, buf.pair_slot, buf.miss, buf.n_miss, buf.counts, buf.offsets, buf.sorted_pairs,
                           buf.pair_to_row, buf.active, buf.n_active, buf.work_list, buf.n_work,
                           sync=buf.sync if sync else None)
        torch.cuda.synchronize()
        ids = to_host(buf.topk_ids)
        assert np.array_equal(ids, ids_want)
        P = T * k
        lk = oracle.slot_lookup(ids, table, res.size)
        assert np.array_equal(to_host(buf.pair_slot)[:P], lk["pair_slot"])
        n_miss = int(to_host(buf.n_miss)[0])
        assert n_miss == lk["n_miss"] and np.array_equal(to_host(buf.miss)[:n_miss], lk["miss"][:n_miss])
        ref = oracle.permute(ids, E)
        for key, n in (("counts", E), ("offsets", E + 1), ("sorted_pairs", P), ("pair_to_row", P)):
            assert np.array_equal(to_host(getattr(buf, key))[:n], ref[key]), key
        na = int(to_host(buf.n_active)[0])
        assert na == ref["n_active"] and np.array_equal(to_host(buf.active)[:na], ref["active"])
        wl = expected_work_list(ids, E, k, moe.WORK_TILE_ROWS)
        assert int(to_host(buf.n_work)[0]) == wl.shape[0]
        assert np.array_equal(to_host(buf.work_list)[: wl.shape[0]], wl)
        assert int(buf.sync.abs().sum().item()) == 0

FUSED_FFN_CASES = [("tiny", 4, 4, None), ("a3b", 4, 1, None), ("a3b", 2, 2, None), ("a3b", 4, 32, None), ("a3b", 2, 8, None),
                   ("a3b", 4, 64, None), ("a3b", 2, 32, None),
                   ("e512", 4, 1, None), ("e512", 2, 4, None), ("e64", 4, 8, None),
                   ("ragged_a", 4, 7, RAGGED[0]), ("ragged_b", 2, 3, RAGGED[1])]


@pytest.mark.parametrize("name,bits,T,shape", FUSED_FFN_CASES, ids=[f"{c[0]}_q{c[1]}_T{c[2]}" for c in FUSED_FFN_CASES])
def test_ffn_one_launch_matches_two_launches(name, bits, T, shape):
    """expert_ffn_fused (gate/up and down in one launch where a kernel exists,
    two launches elsewhere) gives the results of expert_gateup + expert_down
    bit for bit and leaves its counters zero, on two different batches in a
    row through the same buffers (the second relies on the reset)."""
    L = layer(name, bits, shape)
    sh = L.shape
    d = moe.dims(T, sh.H, sh.I, sh.E, sh.k)
    one = moe.LayerBuffers.allocate(d, bits)
    two = moe.LayerBuffers.allocate(d, bits)
    P = T * sh.k
    for seed in (21, 22):
        xb, _ = mi.make_activations(sh.H, T, seed)
        x_d = to_dev(xb)
        say(f"[run] fused FFN {name} q{bits} T={T} seed={seed}")
        moe.route_dispatch(d, x_d, L.Wr_d, L.bias_d, True, one.logits, one.topk_ids, one.topk_w, L.table_d, sh.E,
                           one.pair_slot, one.miss, one.n_miss, one.counts, one.offsets, one.sorted_pairs,
                           one.pair_to_row, one.active, one.n_active, one.work_list, one.n_work, sync=one.sync)
        one.y_rows.fill_(-1)
        two.y_rows.fill_(-2)
        moe.expert_ffn_fused(d, bits, x_d, one.work_list, one.n_work, L.weights_d, one.workspace, one.y_rows,
                             one.ffn_sync)
        moe.expert_gateup(d, bits, x_d, one.work_list, one.n_work, L.weights_d, two.workspace)
        moe.expert_down(d, bits, one.work_list, one.n_work, L.weights_d, two.workspace, two.y_rows)
        torch.cuda.synchronize()
        assert int(one.ffn_sync.abs().sum().item()) == 0        # counters back to zero, no wait timed out
        a, b = to_host(one.y_rows, np.uint16)[:P], to_host(two.y_rows, np.uint16)[:P]
        assert np.array_equal(a, b), f"{int((a != b).any(axis=1).sum())} of {P} rows differ"


@pytest.mark.parametrize("name,T", [("a3b", 8), ("a3b", 32), ("tiny", 4), ("e512", 1), ("e64", 8)])
def test_layer_step_graph_replay(name, T):
    """A layer step (one-launch routing, the FFN (one launch, or the x-tile
    gate/up and the streaming down at the 64-expert shape), combine) captured in a
    HIP graph and replayed three times, with eager work and synchronisations
    between the replays and new activations copied into the captured input
    buffer each time: every replay matches an eager run on the same input bit
    for bit, and the sync counters are zero after each."""
    L = layer(name)
    sh = L.shape
    d = moe.dims(T, sh.H, sh.I, sh.E, sh.k)
    gbuf = moe.LayerBuffers.allocate(d, 4)
    x_g = torch.zeros((T, sh.H), dtype=torch.int16, device="cuda")
    r_g = torch.zeros((T, sh.H), dtype=torch.int16, device="cuda")
    out_g = torch.zeros((T, sh.H), dtype=torch.int16, device="cuda")

    def step(buf, x_d, r_d, out_d):
        moe.layer_forward(buf, x_d, L.Wr_d, L.bias_d, L.weights_d, L.table_d, sh.E, r_d, out_d)

    xb, res = mi.make_activations(sh.H, T, 30)
    x_g.copy_(to_dev(xb))
    r_g.copy_(to_dev(res))
    step(gbuf, x_g, r_g, out_g)                       # eager once before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(gbuf, x_g, r_g, out_g)
    torch.cuda.synchronize()
    for seed in (31, 32, 33):
        xb, res = mi.make_activations(sh.H, T, seed)
        x_g.copy_(to_dev(xb))
        r_g.copy_(to_dev(res))
        torch.cuda.synchronize()
        say(f"[graph] {name} T={T} seed={seed}")
        g.replay()
        torch.cuda.synchronize()
        ebuf = moe.LayerBuffers.allocate(d, 4)
        x_e, r_e = to_dev(xb), to_dev(res)
        out_e = torch.empty_like(r_e)
        step(ebuf, x_e, r_e, out_e)                   # eager work between the replays
        torch.cuda.synchronize()
        for key in ("topk_ids", "topk_w", "sorted_pairs", "work_list", "y_rows"):
            a, b = getattr(gbuf, key), getattr(ebuf, key)
            if key == "work_list":
                nw = int(ebuf.n_work.item())
                a, b = a[:nw], b[:nw]
            assert torch.equal(a, b), key
        assert torch.equal(out_g, out_e)
        assert int(gbuf.sync.abs().sum().item()) == 0 and int(gbuf.ffn_sync.abs().sum().item()) == 0


def _edge_logits(T, E, seed):
    """Logits built to exercise every ranking rule: ties (to the lower id), -0 == +0,
    NaN below -inf, +-inf, and many exact duplicates."""
    rng = np.random.default_rng(seed)
    L = np.round(rng.standard_normal((T, E)), 1).astype(np.float32)   # ~60 distinct values: many ties
    L[0, :] = 0.5                                                        # all equal
    if T > 1:
        L[1, :] = -1.0
        L[1, rng.choice(E, size=min(E, 6), replace=False)] = -0.0
        L[1, rng.choice(E, size=min(E, 6), replace=False)] = 0.0
    if T > 2:
        L[2, rng.choice(E, size=E // 3, replace=False)] = np.nan
        L[2, rng.choice(E, size=min(E, 4), replace=False)] = -np.inf
        L[2, rng.choice(E, size=min(E, 2), replace=False)] = np.inf
    if T > 3:
        L[3, :] = np.nan
        L[3, rng.choice(E, size=min(E, 3), replace=False)] = rng.standard_normal(min(E, 3))
    if T > 4:
        L[4, E - 1] = 9.0
        L[4, E // 2] = 9.0                                               # equal maxima, far apart
    return L


@pytest.mark.parametrize("E,k", [(8, 2), (8, 8), (64, 8), (200, 8), (256, 32), (300, 5), (1000, 16), (1000, 1)])
@pytest.mark.parametrize("renorm", [1, 0])
def test_topk_edge_cases(E, k, renorm):
    """Top-k on constructed logits through moe_topk_from_logits: ids bit-exact against
    the oracle, gates within 2e-6 (NaN where the oracle gives NaN)."""
    T = 9
    L = _edge_logits(T, E, seed=E * 100 + k)
    d = moe.dims(T, 256, 256, E, k)
    ids_d = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    g_d = torch.full((T, k), -7.0, dtype=torch.float32, device="cuda")
    say(f"[topk] E={E} k={k} renorm={renorm}")
    moe.topk_from_logits(d, to_dev(L), bool(renorm), ids_d, g_d)
    torch.cuda.synchronize()
    ids_ref, g_ref = oracle.topk(L, k, bool(renorm))
    ids, g = to_host(ids_d), to_host(g_d)
    assert np.array_equal(ids, ids_ref), f"ids differ in rows {np.nonzero((ids != ids_ref).any(1))[0].tolist()}"
    nan_ref = np.isnan(g_ref)
    assert np.array_equal(np.isnan(g), nan_ref)
    assert np.max(np.abs(g[~nan_ref] - g_ref[~nan_ref]), initial=0.0) <= 2e-6


# ------------------------------------------------------ zero-point weights

@pytest.mark.parametrize("n", [1, 7, 100003])
def test_zero_point_bias_bit_exact(n):
    """moe_zero_point_bias equals the oracle bit for bit over scales of every
    finite fp16 class (subnormal, normal, negative, near the top of the range,
    where z s overflows to an infinity) and zero points 0..255; entries past n
    stay untouched; NaN in gives NaN out."""
    rng = np.random.default_rng(n)
    pats = rng.integers(0, 65536, size=n).astype(np.uint16)
    pats[(pats & 0x7C00) == 0x7C00] &= 0xBFFF                  # no inf / NaN scales here
    pats[: n // 2] = mi.f32_to_f16_bits(rng.uniform(0.005, 0.02, size=n // 2))
    z = rng.integers(0, 256, size=n).astype(np.uint8)
    ref = oracle.zero_point_bias(pats, z)
    out = torch.full((n + 64,), 0x1234, dtype=torch.int16, device="cuda")
    say(f"[run] zero_point_bias n={n}")
    moe.zero_point_bias(to_dev(pats), to_dev(z), out[:n])
    torch.cuda.synchronize()
    got = to_host(out, np.uint16)
    assert np.array_equal(got[:n], ref), f"{int((got[:n] != ref).sum())} of {n} differ"
    assert np.all(got[n:] == 0x1234)
    s_nan = to_dev(np.array([0x7E00, 0x7C00, 0xFC00], np.uint16))
    z_nan = to_dev(np.array([3, 0, 0], np.uint8))
    b_nan = torch.zeros(3, dtype=torch.int16, device="cuda")
    moe.zero_point_bias(s_nan, z_nan, b_nan)
    torch.cuda.synchronize()
    assert np.all(np.isnan(to_host(b_nan, np.uint16).view(np.float16)))


@pytest.mark.parametrize("name,bits,T", [("tiny", 4, 4), ("a3b", 2, 8), ("a3b", 4, 32)])
def test_zero_point_weights_through_the_layer(name, bits, T):
    """Zero-point weights (q - z) s: the biases moe_zero_point_bias makes on
    the GPU equal the oracle's bit for bit, and the layer run on them matches
    the oracle fed the oracle's biases (every FFN row, FFN tolerance; combine
    bit-exact).  The biases here reach 15 s, several times those of the
    scale-and-bias inputs, which loads the offset part of the exact-operand fold."""
    L = layer(name, bits)
    sh = L.shape
    saved = [b.clone() for b in L.weights_d.bias]
    try:
        zs = {}
        for i, m in enumerate(mi.MATRICES):
            zs[m] = np.stack([mi.make_zero_points(sh, m, e, bits, seed=5) for e in range(sh.E)])
            say(f"[run] zero-point biases {name} q{bits} {m}")
            moe.zero_point_bias(L.weights_d.scale[i], to_dev(zs[m]), L.weights_d.bias[i])
        torch.cuda.synchronize()
        for i, m in enumerate(mi.MATRICES):
            ref = oracle.zero_point_bias(to_host(L.weights_d.scale[i], np.uint16), zs[m])
            assert np.array_equal(to_host(L.weights_d.bias[i], np.uint16), ref), m
        xb, res = mi.make_activations(sh.H, T, 9)
        say(f"[run] zero-point layer {name} q{bits} T={T}")
        g = run_layer(L, xb, res)
        check_topk(g, L)
        check_permute(g, L)
        ids = g["ids"].ravel()
        used = sorted({int(e) for e in ids})
        W = mi.make_expert_weights(sh, bits, L.seed, experts=used)
        for m in mi.MATRICES:
            for i, e in enumerate(W.experts):
                W.bias[m][i] = oracle.zero_point_bias(W.scale[m][i], zs[m][int(e)])
        P = T * sh.k
        _, ys = oracle.expert_ffn(xb, ids, g["sorted_pairs"], W, sh.k)
        max_rel, mae = tolerance_metrics(g["y_rows"], np.stack([ys[r] for r in range(P)]))
        say(f"[ok] zero-point {name} q{bits} T={T}: FFN max_rel {max_rel:.2e} mae_norm {mae:.2e}")
        assert max_rel <= 1e-2 and mae <= 1e-3, (max_rel, mae)
        check_combine_exact(g, L, res)
    finally:
        for b, s in zip(L.weights_d.bias, saved):
            b.copy_(s)
        torch.cuda.synchronize()


# ------------------------------------------------------------ shared expert

def _upload_shared(mats, bits, gate_w, I):
    q, s, b = [], [], []
    for m in mi.MATRICES:
        qq, ss, bb = mats[m]
        q.append(torch.from_numpy(moe.group_major(qq, bits)[None].copy()).cuda())
        s.append(torch.from_numpy(ss.view(np.int16)[None].copy()).cuda())
        b.append(torch.from_numpy(bb.view(np.int16)[None].copy()).cuda())
    return moe.SharedExpert(moe.QWeights(bits, q, s, b), to_dev(gate_w), I)


@pytest.mark.parametrize("name,bits,T,i_mul", [("tiny", 4, 4, 2), ("a3b", 4, 32, 1), ("a3b", 2, 8, 1),
                                               ("e64", 4, 8, 1)])
def test_shared_expert_layer(name, bits, T, i_mul):
    """A layer step with an always-on shared expert (its FFN a launch of its
    own): the shared rows match the oracle's FFN (FFN tolerance), the gate
    values the oracle's sigmoid (logit bound as for the router), and the output
    is the oracle's combine_shared of the GPU's own rows and gates bit for bit;
    two steps in a row through the same buffers."""
    L = layer(name, bits)
    sh = L.shape
    one, mats, gw = mi.make_shared_expert(sh, bits, seed=4, I=sh.I * i_mul)
    shared = _upload_shared(mats, bits, gw, one.I)
    d = moe.dims(T, sh.H, sh.I, sh.E, sh.k)
    buf = moe.LayerBuffers.allocate(d, bits)
    sbuf = moe.SharedBuffers.allocate(T, sh.H, one.I, bits)
    for seed in (13, 14):
        xb, res = mi.make_activations(sh.H, T, seed)
        x_d, r_d = to_dev(xb), to_dev(res)
        out_d = torch.empty_like(r_d)
        say(f"[run] shared expert {name} q{bits} T={T} I_shared={one.I} seed={seed}")
        moe.layer_forward(buf, x_d, L.Wr_d, L.bias_d, L.weights_d, L.table_d, sh.E, r_d, out_d,
                          shared=shared, shared_buf=sbuf)
        torch.cuda.synchronize()
        P = T * sh.k
        g = dict(logits=to_host(buf.logits), ids=to_host(buf.topk_ids), gates=to_host(buf.topk_w))
        check_topk(g, L)
        ys = to_host(sbuf.buf.y_rows, np.uint16)[:T]
        ref_ys = np.stack([oracle.expert_ffn_row(xb[t], mats, bits)[1] for t in range(T)])
        max_rel, mae = tolerance_metrics(ys, ref_ys)
        assert max_rel <= 1e-2 and mae <= 1e-3, (max_rel, mae)
        sg = to_host(sbuf.gate_out)[:T].astype(np.float64)
        ref_sg = oracle.shared_gate(xb, gw).astype(np.float64)
        xabs = np.abs((xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
        bound = 0.25 * 1e-5 * (xabs @ np.abs(gw.astype(np.float64))) + 4e-7
        assert np.all(np.abs(sg - ref_sg) <= bound), np.max(np.abs(sg - ref_sg) / bound)
        ref_out = oracle.combine_shared(to_host(buf.y_rows, np.uint16)[:P], to_host(buf.pair_to_row)[:P],
                                        g["gates"], ys, to_host(sbuf.gate_out)[:T], res)
        assert np.array_equal(to_host(out_d, np.uint16), ref_out)
        say(f"[ok] shared expert {name} T={T}: FFN max_rel {max_rel:.2e} mae_norm {mae:.2e}")


@pytest.mark.parametrize("name,bits,T", [("tiny", 4, 4), ("a3b", 4, 1), ("a3b", 2, 8), ("a3b", 4, 32)])
def test_shared_expert_one_launch(name, bits, T):
    """The shared expert inside the routed FFN launch (expert_ffn_fused_shared,
    its weights the last of E + 1 experts): routed rows and shared rows match the
    oracle (FFN tolerance), the output is the oracle's combine_shared of the
    GPU's rows and gates bit for bit, the counters are left zero; two steps in a
    row.  Other algorithms are refused before anything is enqueued."""
    L = layer(name, bits)
    sh = L.shape
    one, mats, gw = mi.make_shared_expert(sh, bits, seed=4)
    sep = _upload_shared(mats, bits, gw, one.I)
    cat = lambda a, b: [torch.cat([u, v]) for u, v in zip(a, b)]
    fw = moe.QWeights(bits, cat(L.weights_d.q, sep.weights.q), cat(L.weights_d.scale, sep.weights.scale),
                      cat(L.weights_d.bias, sep.weights.bias))
    shared = moe.SharedExpert(sep.weights, sep.gate_w, one.I, fused_weights=fw)
    d = moe.dims(T, sh.H, sh.I, sh.E, sh.k)
    buf = moe.LayerBuffers.allocate(d, bits, shared_rows=True)
    sbuf = moe.SharedBuffers.allocate(T, sh.H, one.I, bits)
    P = T * sh.k
    for seed in (15, 16):
        xb, res = mi.make_activations(sh.H, T, seed)
        x_d, r_d = to_dev(xb), to_dev(res)
        out_d = torch.empty_like(r_d)
        say(f"[run] one-launch shared expert {name} q{bits} T={T} seed={seed}")
        moe.layer_forward(buf, x_d, L.Wr_d, L.bias_d, L.weights_d, L.table_d, sh.E, r_d, out_d,
                          shared=shared, shared_buf=sbuf)
        torch.cuda.synchronize()
        assert int(buf.ffn_sync.abs().sum().item()) == 0
        g = dict(logits=to_host(buf.logits), ids=to_host(buf.topk_ids), gates=to_host(buf.topk_w),
                 sorted_pairs=to_host(buf.sorted_pairs)[:P])
        check_topk(g, L)
        rows = to_host(buf.y_rows, np.uint16)
        ids = g["ids"].ravel()
        W = mi.make_expert_weights(sh, bits, L.seed, experts=sorted({int(e) for e in ids}))
        _, ys = oracle.expert_ffn(xb, ids, g["sorted_pairs"], W, sh.k)
        mr_r, mae_r = tolerance_metrics(rows[:P], np.stack([ys[r] for r in range(P)]))
        ref_s = np.stack([oracle.expert_ffn_row(xb[t], mats, bits)[1] for t in range(T)])
        mr_s, mae_s = tolerance_metrics(rows[P:P + T], ref_s)
        say(f"[ok] one-launch shared {name} T={T}: routed max_rel {mr_r:.2e} mae {mae_r:.2e}; "
            f"shared max_rel {mr_s:.2e} mae {mae_s:.2e}")
        assert mr_r <= 1e-2 and mae_r <= 1e-3 and mr_s <= 1e-2 and mae_s <= 1e-3
        ref_out = oracle.combine_shared(rows[:P], to_host(buf.pair_to_row)[:P], g["gates"], rows[P:P + T],
                                        to_host(sbuf.gate_out)[:T], res)
        assert np.array_equal(to_host(out_d, np.uint16), ref_out)
    with pytest.raises(moe.MoeError) as ex:
        moe.expert_ffn_fused_shared(d, bits, x_d, buf.work_list, buf.n_work, fw, buf.workspace, buf.y_rows,
                                    buf.ffn_sync, moe.ALGO_GEMV)
    assert ex.value.status == moe.ERR_UNSUPPORTED


@pytest.mark.parametrize("n_seq,n_draft", [(8, 4), (2, 8)])
def test_spec_verify_batch(n_seq, n_draft):
    """A speculative-verify batch (drafts of one sequence share most experts,
    so the FFN tiles hold several rows each) through every stage against the
    oracle: A3B-style shape, T = n_seq * n_draft."""
    L = layer("a3b")
    xb, res = mi.make_spec_verify_activations(L.shape.H, n_seq, n_draft, seed=7)
    say(f"[run] spec-verify a3b {n_seq} x {n_draft}")
    g = run_layer(L, xb, res)
    check_logits(g, L, xb)
    check_topk(g, L)
    check_lookup(g, L)
    check_permute(g, L)
    mr, mae = check_ffn(g, L, xb)
    check_combine_exact(g, L, res)
    say(f"[ok] spec-verify {n_seq} x {n_draft}: {g['n_active']} experts, FFN max_rel {mr:.2e} mae_norm {mae:.2e}")


@pytest.mark.parametrize("algo", [moe.ALGO_AUTO, moe.ALGO_MFMA], ids=["auto_gemm", "decode"])
def test_zero_point_weights_prefill(algo):
    """Zero-point weights at the prefill shape (T = 4096), on the grouped GEMM
    and on the decode kernels: 96 sampled rows against the oracle fed the
    oracle's biases.  (Large dequantised weights are where a down kernel that
    drops h's third bf16 plane leaves the tolerance.)"""
    L = layer("prefill")
    sh = L.shape
    saved = [b.clone() for b in L.weights_d.bias]
    try:
        zs = {}
        for i, m in enumerate(mi.MATRICES):
            zs[m] = np.stack([mi.make_zero_points(sh, m, e, 4, seed=5) for e in range(sh.E)])
            moe.zero_point_bias(L.weights_d.scale[i], to_dev(zs[m]), L.weights_d.bias[i])
        T = sh.tokens[0]
        xb, res = mi.make_activations(sh.H, T, 9)
        say(f"[run] zero-point prefill algo={algo}")
        g = run_layer(L, xb, res, algo=algo)
        ids = g["ids"].ravel()
        rows = [int(r) for r in np.random.default_rng(1).choice(T * sh.k, 96, replace=False)]
        W = mi.make_expert_weights(sh, 4, L.seed, experts=sorted({int(ids[int(g["sorted_pairs"][r])]) for r in rows}))
        for m in mi.MATRICES:
            for i, e in enumerate(W.experts):
                W.bias[m][i] = oracle.zero_point_bias(W.scale[m][i], zs[m][int(e)])
        _, ys = oracle.expert_ffn(xb, ids, g["sorted_pairs"], W, sh.k, rows=rows)
        max_rel, mae = tolerance_metrics(np.stack([g["y_rows"][r] for r in rows]), np.stack([ys[r] for r in rows]))
        say(f"[ok] zero-point prefill algo={algo}: max_rel {max_rel:.2e} mae_norm {mae:.2e}")
        assert max_rel <= 1e-2 and mae <= 1e-3, (max_rel, mae)
    finally:
        for b, s in zip(L.weights_d.bias, saved):
            b.copy_(s)
        torch.cuda.synchronize()
