"""GPU parity of the residency tiers ("Luce Spark" page, sec. 1: calibrated
hot set from routing counts; sec. 2: a bounded warm ring filled from pinned
host memory, least recently used slot evicted) through the C ABI:

  * routing counters and the hot set over 1024 calibration tokens, bit for
    bit against the oracle fed the GPU's own picks, and the hot set against
    the committed fixture the oracle wrote (tests/golden/resident_sets.json);
  * the plan over a run of steps: tables, stamps, copy list and the split
    work lists bit for bit against the oracle's warm ring and the work-list
    checker;
  * the copy kernel: pool slots equal the host experts byte for byte;
  * the whole layer behind the tiers: expert rows and outputs bit for bit
    equal to the layer with every expert resident, step after step (with a
    copy stream and without), a miss at one step served from its new slot at
    the next, and a ring too small for a step's misses (experts read straight
    from host memory).
"""
import json
import os

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
import quantized_expert_ffn_gemv_amd as moe
from gpu_util import say, to_dev, to_host, upload_layer
from work_tiles import expected_work_list

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "resident_sets.json")


def _route(d, x_d, Wr_d, bias_d, table_d, n_slots, buf, last_use=None, step=0):
    moe.route_dispatch(d, x_d, Wr_d, bias_d, True, buf.logits, buf.topk_ids, buf.topk_w, table_d, n_slots,
                       buf.pair_slot, buf.miss, buf.n_miss, buf.counts, buf.offsets, buf.sorted_pairs,
                       buf.pair_to_row, buf.active, buf.n_active, buf.work_list, buf.n_work, None, last_use, step,
                       buf.sync)


@pytest.mark.parametrize("name", mi.CONFIG_ORDER)
def test_calibrated_hot_set(name):
    """1024 calibration tokens (seed 1) through the one-launch routing in
    batches of 64, the counters summed on the device, the hot set ranked on the
    device: counters equal the oracle's over the GPU's picks, the hot set the
    oracle's of those counters, and the committed fixture's."""
    shape = mi.CONFIGS[name]
    Wr, bias = mi.make_router(shape, 0)
    x, _ = mi.make_activations(shape.H, 1024, 1)
    T = 64
    d = moe.dims(T, shape.H, shape.I, shape.E, shape.k)
    buf = moe.LayerBuffers.allocate(d, 4)
    table = torch.full((shape.E,), -1, dtype=torch.int32, device="cuda")
    freq = torch.zeros(shape.E, dtype=torch.int32, device="cuda")
    Wr_d, bias_d = to_dev(Wr), None if bias is None else to_dev(bias)
    ids = []
    say(f"[calibrate] {name}")
    for b in range(0, 1024, T):
        _route(d, to_dev(x[b:b + T]), Wr_d, bias_d, table, shape.E, buf)
        moe.route_counts(d, buf.counts, freq)
        ids.append(to_host(buf.topk_ids).copy())
    hot = torch.full((shape.n_resident,), -7, dtype=torch.int32, device="cuda")
    moe.hot_set(d, freq, shape.n_resident, hot)
    torch.cuda.synchronize()
    ids = np.concatenate(ids)
    ref_freq = oracle.freq_update(oracle.permute(ids, shape.E)["counts"], np.zeros(shape.E, np.uint32))
    got_freq = to_host(freq, np.uint32)
    assert np.array_equal(got_freq, ref_freq)
    assert np.array_equal(to_host(hot), oracle.hot_set(ref_freq, shape.n_resident))
    fixture = json.load(open(GOLDEN))["shapes"][name]
    assert to_host(hot).tolist() == fixture["hot"], "hot set differs from the oracle's on its own logits"


def _plan_case(E, n_hot, n_slots, T, k, steps, seed):
    """Random picks each step (ids set directly), lookup and grouping on the
    GPU, then the plan; every output against the oracle and the checker."""
    rng = np.random.default_rng(seed)
    d = moe.dims(T, 256, 256, E, k)
    buf = moe.LayerBuffers.allocate(d, 4)
    cap = moe.work_list_capacity(d)
    soe = torch.full((E,), -1, dtype=torch.int32, device="cuda")
    eos = torch.full((n_slots,), -1, dtype=torch.int32, device="cuda")
    lu = torch.zeros(n_slots, dtype=torch.int32, device="cuda")
    hot = rng.permutation(E)[:n_hot].astype(np.int32)
    soe[torch.from_numpy(hot).long().cuda()] = torch.arange(n_hot, dtype=torch.int32, device="cuda")
    eos[:n_hot] = to_dev(hot)
    lists = torch.full((3, max(cap, 1), moe.WORK_ENTRY_INTS), -9, dtype=torch.int32, device="cuda")
    counts = torch.zeros(3, dtype=torch.int32, device="cuda")
    copies = torch.full((n_slots, 2), -9, dtype=torch.int32, device="cuda")
    n_copy = torch.zeros(1, dtype=torch.int32, device="cuda")
    pool = rng.permutation(E)[: max(k, E * 2 // 3)]          # skewed: some experts never picked
    for step in range(1, steps + 1):
        ids = np.stack([rng.choice(pool, k, replace=False) for _ in range(T)]).astype(np.int32)
        ids_d = to_dev(ids)
        st_soe, st_eos, st_lu = to_host(soe), to_host(eos), to_host(lu, np.uint32)
        moe.slot_lookup(d, ids_d, soe, n_slots, buf.pair_slot, buf.miss, buf.n_miss, None, lu, step)
        moe.permute(d, ids_d, buf.counts, buf.offsets, buf.sorted_pairs, buf.pair_to_row, buf.active, buf.n_active,
                    buf.work_list, buf.n_work)
        moe.residency_plan(d, n_hot, n_slots, soe, eos, lu, buf.miss, buf.n_miss, step, buf.work_list, buf.n_work,
                           lists, counts, copies, n_copy)
        torch.cuda.synchronize()
        look = oracle.slot_lookup(ids, st_soe, n_slots, last_use=st_lu, step=step)
        ring = oracle.warm_ring_step(n_hot, look["miss"], step, st_soe, st_eos, look["last_use"])
        assert np.array_equal(to_host(soe), ring["slot_of_expert"]), step
        assert np.array_equal(to_host(eos), ring["expert_of_slot"]), step
        assert np.array_equal(to_host(lu, np.uint32), ring["last_use"]), step
        nc = int(n_copy.item())
        assert [tuple(r) for r in to_host(copies)[:nc].tolist()] == ring["copies"], step
        # the split lists: every entry of the work list, in order, by where its expert is read
        wl = expected_work_list(ids, E, k)
        new = dict(ring["copies"])
        want = [[], [], []]
        for ent in wl.tolist():
            e = ent[0]
            if e not in set(look["miss"].tolist()):
                want[0].append([int(st_soe[e])] + ent[1:])
            elif e in new:
                want[1].append([new[e]] + ent[1:])
            else:
                want[2].append(ent)
        got_counts = to_host(counts).tolist()
        assert got_counts == [len(w) for w in want], step
        for L in range(3):
            got = to_host(lists[L])[: got_counts[L]].tolist()
            assert got == want[L], (step, L)
    return True


@pytest.mark.parametrize("E,n_hot,n_slots,T,k,seed", [(16, 4, 8, 4, 2, 1), (64, 24, 32, 8, 2, 2), (256, 0, 40, 32, 8, 3),
                                                     (40, 10, 12, 16, 4, 4), (1000, 300, 400, 64, 8, 5)],
                         ids=["E16", "E64", "E256_nohot", "E40_overflow", "E1000"])
def test_residency_plan_over_steps(E, n_hot, n_slots, T, k, seed):
    say(f"[plan] E={E} hot={n_hot} slots={n_slots} T={T} k={k}")
    assert _plan_case(E, n_hot, n_slots, T, k, steps=8, seed=seed)


def _pinned_host_weights(L):
    """The layer's experts copied into pinned host tensors (device-visible)."""
    def pin(t):
        h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
        h.copy_(t.cpu())
        return h
    w = L.weights_d
    return moe.QWeights(w.bits, [pin(t) for t in w.q], [pin(t) for t in w.scale], [pin(t) for t in w.bias])


@pytest.mark.parametrize("bits", [4, 2])
def test_expert_copy_from_host(bits):
    shape = mi.CONFIGS["tiny"]
    L = upload_layer(shape, bits, seed=0)
    host = _pinned_host_weights(L)
    d = moe.dims(4, shape.H, shape.I, shape.E, shape.k)
    res = moe.ResidentExperts.allocate(d, bits, host, n_hot=2, n_slots=5)
    order = torch.tensor([6, 3, 0, 7, 2], dtype=torch.int32, device="cuda")
    res.install(order)
    torch.cuda.synchronize()
    for m in range(3):
        for i, e in enumerate(order.tolist()):
            assert torch.equal(res.pool.q[m][i], L.weights_d.q[m][e])
            assert torch.equal(res.pool.scale[m][i], L.weights_d.scale[m][e])
            assert torch.equal(res.pool.bias[m][i], L.weights_d.bias[m][e])
    assert to_host(res.slot_of_expert).tolist() == [2, -1, 4, 1, -1, -1, 0, 3]


# (shape, bits, T, hot slots, all slots, copy stream, a step must overflow the ring)
RES_CASES = [("a3b", 4, 8, 32, 48, True, False), ("a3b", 2, 8, 32, 48, False, False),
             ("a3b", 4, 32, 100, 104, True, True), ("e512", 4, 1, 200, 204, True, False),
             ("tiny", 4, 4, 2, 4, False, False)]


@pytest.mark.parametrize("name,bits,T,n_hot,n_slots,copy_stream,overflow", RES_CASES,
                         ids=[f"{c[0]}_q{c[1]}_T{c[2]}_hot{c[3]}_slots{c[4]}_{'2streams' if c[5] else '1stream'}"
                              for c in RES_CASES])
def test_resident_layer_matches_all_resident(name, bits, T, n_hot, n_slots, copy_stream, overflow):
    """Steps of the layer behind the tiers against the layer with every expert
    resident: expert rows and outputs bit for bit.  Batches: 6 distinct ones,
    then the first again (its misses were copied in at step 1: the lookup now
    finds them unless the ring evicted them since).  With 4 ring slots at
    A3B-style T = 32 a step has more misses than free slots, so list 2 (read
    from host memory) is used."""
    shape = mi.CONFIGS[name]
    L = upload_layer(shape, bits, seed=0)
    host = _pinned_host_weights(L)
    d = moe.dims(T, shape.H, shape.I, shape.E, shape.k)
    hot = torch.from_numpy(np.array(json.load(open(GOLDEN))["shapes"][name]["hot"][:n_hot], np.int32)).cuda()
    res = moe.ResidentExperts.allocate(d, bits, host, n_hot=n_hot, n_slots=n_slots)
    res.install(hot)
    buf = moe.LayerBuffers.allocate(d, bits)
    ref = moe.LayerBuffers.allocate(d, bits)
    side = torch.cuda.Stream() if copy_stream else None
    all_res = torch.arange(shape.E, dtype=torch.int32, device="cuda")
    seeds = [50, 51, 52, 53, 54, 55, 50]
    used_cold = 0
    for step, seed in enumerate(seeds, start=1):
        xb, rb = mi.make_activations(shape.H, T, seed)
        x_d, r_d = to_dev(xb), to_dev(rb)
        out = torch.empty_like(r_d)
        out_ref = torch.empty_like(r_d)
        soe_before = to_host(res.slot_of_expert).copy()
        say(f"[resident] {name} q{bits} T={T} step {step}")
        moe.resident_layer_forward(buf, res, x_d, L.Wr_d, L.bias_d, r_d, out, step, copy_stream=side)
        moe.layer_forward(ref, x_d, L.Wr_d, L.bias_d, L.weights_d, all_res, shape.E, r_d, out_ref)
        torch.cuda.synchronize()
        P = T * shape.k
        assert np.array_equal(to_host(buf.topk_ids), to_host(ref.topk_ids))
        assert np.array_equal(to_host(buf.y_rows, np.uint16)[:P], to_host(ref.y_rows, np.uint16)[:P]), step
        assert torch.equal(out, out_ref), step
        assert buf.counters_clean()
        ids = to_host(buf.topk_ids)
        look = oracle.slot_lookup(ids, soe_before, n_slots)
        assert int(buf.n_miss.item()) == look["n_miss"]
        used_cold += to_host(res.list_counts).tolist()[2]
    if overflow:
        assert used_cold > 0, "the overflow case never read an expert from host memory"


def test_miss_then_hit_next_step():
    """A miss at step i is served from its new warm slot at step i + 1: the
    same batch twice, a ring big enough for one step's misses; the second step
    has no misses, its pairs' slots are the ones the first step's plan gave."""
    shape = mi.CONFIGS["a3b"]
    L = upload_layer(shape, 4, seed=0)
    host = _pinned_host_weights(L)
    T = 8
    d = moe.dims(T, shape.H, shape.I, shape.E, shape.k)
    res = moe.ResidentExperts.allocate(d, 4, host, n_hot=16, n_slots=16 + T * shape.k)
    res.install(torch.arange(16, dtype=torch.int32, device="cuda"))
    buf = moe.LayerBuffers.allocate(d, 4)
    xb, rb = mi.make_activations(shape.H, T, 60)
    x_d, r_d = to_dev(xb), to_dev(rb)
    out1, out2 = torch.empty_like(r_d), torch.empty_like(r_d)
    moe.resident_layer_forward(buf, res, x_d, L.Wr_d, L.bias_d, r_d, out1, 1)
    torch.cuda.synchronize()
    n_miss1 = int(buf.n_miss.item())
    copies = to_host(res.copies)[: int(res.n_copy.item())]
    assert n_miss1 > 0 and len(copies) == n_miss1
    moe.resident_layer_forward(buf, res, x_d, L.Wr_d, L.bias_d, r_d, out2, 2)
    torch.cuda.synchronize()
    assert int(buf.n_miss.item()) == 0 and int(res.n_copy.item()) == 0
    ids = to_host(buf.topk_ids).ravel()
    pair_slot = to_host(buf.pair_slot)[: T * shape.k]
    new = {int(e): int(s) for e, s in copies}
    for p, e in enumerate(ids):
        if int(e) in new:
            assert pair_slot[p] == new[int(e)]
    assert to_host(res.list_counts).tolist()[1:] == [0, 0]
    assert torch.equal(out1, out2)
