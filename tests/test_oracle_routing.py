"""Pins for the oracle's routing stages: logits, top-k, gates, slot lookup and
the grouping of tokens by expert.

Router scoring and top-k selection follow the MoE primer on the page "12GB card
runs a 68GB model (Betelgeuse)"; the resident-slot lookup follows the same
page's in-stream doorbell and the hot/warm/cold tiers of the "Luce Spark" page;
grouping by expert follows the "Strata" page, section 2.3.  Every check below
uses an independent computation: numpy's float64 matmul, brute-force search
over orders and subsets, closed forms, set arithmetic, numpy's stable sort.
"""
import itertools
import math

import numpy as np
import pytest

import moe_inputs as mi


def _x_bits(rng, T, H):
    return mi.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))


@pytest.mark.parametrize("with_bias", [False, True])
def test_router_logits_vs_float64_matmul(orc, with_bias):
    rng = np.random.default_rng(1)
    T, H, E = 5, 384, 12
    xb = _x_bits(rng, T, H)
    Wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    bias = rng.standard_normal(E).astype(np.float32) if with_bias else None
    got = orc.router_logits(xb, Wr, bias)
    x = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = x @ Wr.astype(np.float64).T
    if with_bias:
        ref = ref + bias.astype(np.float64)
    # both sides are (near-)exact double sums rounded once to float32
    assert np.max(np.abs(got.astype(np.float64) - ref)) <= 1e-6 * np.max(np.abs(ref))
    assert np.array_equal(got, ref.astype(np.float32))


def _rank_key(v, e):
    return (1 if math.isnan(v) else 0, 0.0 if math.isnan(v) else -v, e)


def _brute_topk(L, k):
    order = sorted(range(len(L)), key=lambda e: _rank_key(float(L[e]), e))
    return order[:k]


def test_topk_bruteforce_random(orc):
    rng = np.random.default_rng(2)
    T, E, k = 40, 24, 5
    L = rng.standard_normal((T, E)).astype(np.float32)
    ids, _ = orc.topk(L, k)
    for t in range(T):
        assert ids[t].tolist() == _brute_topk(L[t], k)


def test_topk_ties_signed_zero_nan(orc):
    inf = np.float32(np.inf)
    nan = np.float32(np.nan)
    rows = [
        ([1, 3, 3, 2, 3, 0, 0, 0], 3, [1, 2, 4]),          # equal maxima: lower ids first
        ([0.0, -0.0, 0.0, -1, -1, -1, -1, -1], 2, [0, 1]),  # -0 == +0 is a tie
        ([-0.0, 0.0, -5, -5, -5, -5, -5, -5], 2, [0, 1]),
        ([nan, -inf, 1, nan, -2, -3, -4, -5], 6, [2, 4, 5, 6, 7, 1]),  # NaN below -inf
        ([nan, nan, nan, nan, nan, nan, 7, nan], 3, [6, 0, 1]),        # NaNs by id when needed
    ]
    for vals, k, expect in rows:
        L = np.array([vals], dtype=np.float32)
        ids, _ = orc.topk(L, k)
        assert ids[0].tolist() == expect, (vals, ids)
        assert _brute_topk(L[0], k) == expect


def test_topk_exhaustive_subsets_tiny(orc):
    """Tiny shape (8 experts, top-2): the picked pair is the unique subset whose
    members all rank before every non-member."""
    rng = np.random.default_rng(3)
    L = rng.standard_normal((64, 8)).astype(np.float32)
    L[::7, 3] = L[::7, 5]                      # plant exact ties
    ids, _ = orc.topk(L, 2)
    for t in range(L.shape[0]):
        winners = []
        for sub in itertools.combinations(range(8), 2):
            rest = [e for e in range(8) if e not in sub]
            if all(_rank_key(float(L[t, a]), a) < _rank_key(float(L[t, b]), b) for a in sub for b in rest):
                winners.append(sub)
        assert len(winners) == 1
        assert sorted(ids[t].tolist()) == list(winners[0])
        a, b = ids[t]
        assert _rank_key(float(L[t, a]), a) < _rank_key(float(L[t, b]), b)


def test_gates_renormalised(orc):
    rng = np.random.default_rng(4)
    T, E, k = 30, 16, 4
    L = (rng.standard_normal((T, E)) * 3).astype(np.float32)
    ids, g = orc.topk(L, k, renormalize=True)
    assert np.all(np.abs(g.astype(np.float64).sum(1) - 1.0) <= 4e-7)
    assert np.all(np.diff(g, axis=1) <= 0)                     # rank order -> non-increasing
    # closed form for two picks: g0 = 1 / (1 + e^(L1 - L0))
    ids2, g2 = orc.topk(L, 2, renormalize=True)
    for t in range(T):
        l0, l1 = float(L[t, ids2[t, 0]]), float(L[t, ids2[t, 1]])
        assert g2[t, 0] == np.float32(1.0 / (1.0 + math.exp(l1 - l0)))
        assert g2[t, 1] == np.float32(math.exp(l1 - l0) / (1.0 + math.exp(l1 - l0)))


def test_gates_full_softmax(orc):
    from scipy.special import softmax
    rng = np.random.default_rng(5)
    L = (rng.standard_normal((10, 20)) * 2).astype(np.float32)
    ids, g = orc.topk(L, 3, renormalize=False)
    ref = softmax(L.astype(np.float64), axis=1)
    for t in range(10):
        assert np.allclose(g[t], ref[t, ids[t]], rtol=1e-6, atol=0)
        assert g[t].sum() < 1.0


def _brute_lookup(ids, table, n_slots):
    ids = ids.ravel().tolist()
    pair_slot = [int(table[e]) if 0 <= table[e] < n_slots else -1 for e in ids]
    miss = sorted({e for e, s in zip(ids, pair_slot) if s == -1})
    return pair_slot, miss


def test_slot_lookup_bruteforce(orc):
    rng = np.random.default_rng(6)
    E, T, k = 32, 9, 4
    n_slots = 20
    for trial in range(20):
        table = np.full(E, -1, np.int32)
        res = rng.choice(E, size=rng.integers(0, E + 1), replace=False)
        table[res] = rng.choice(n_slots + 4, size=len(res), replace=True)   # some >= n_slots: invalid
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        out = orc.slot_lookup(ids, table, n_slots)
        ps, miss = _brute_lookup(ids, table, n_slots)
        assert out["pair_slot"].tolist() == ps
        assert out["miss"].tolist() == miss
        assert out["n_miss"] == len(miss)


def test_slot_lookup_special_cases(orc):
    E, T, k = 16, 6, 3
    rng = np.random.default_rng(7)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    all_res = np.arange(E, dtype=np.int32)
    out = orc.slot_lookup(ids, all_res, E, last_use=np.zeros(E, np.uint32), step=9, doorbell=0)
    assert out["n_miss"] == 0 and out["miss"].size == 0
    assert out["doorbell"] == 0                              # not rung without a miss
    used = np.zeros(E, np.uint32)
    used[np.unique(ids)] = 9
    assert np.array_equal(out["last_use"], used)
    none_res = np.full(E, -1, np.int32)
    out = orc.slot_lookup(ids, none_res, E, doorbell=0)
    assert out["miss"].tolist() == sorted(set(ids.ravel().tolist()))
    assert out["doorbell"] == out["n_miss"] > 0
    assert np.all(out["pair_slot"] == -1)


def test_permute_invariants_and_stable_sort(orc):
    rng = np.random.default_rng(8)
    for E, T, k in [(8, 4, 2), (64, 37, 6), (128, 200, 8)]:
        p = rng.random(E) ** 3
        p /= p.sum()
        ids = np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
        out = orc.permute(ids, E)
        flat = ids.ravel()
        assert out["counts"].sum() == T * k
        assert np.array_equal(out["counts"], np.bincount(flat, minlength=E))
        assert out["offsets"][0] == 0 and out["offsets"][-1] == T * k
        assert np.all(np.diff(out["offsets"]) == out["counts"])
        assert np.array_equal(out["sorted_pairs"], np.argsort(flat, kind="stable"))
        assert np.array_equal(out["pair_to_row"][out["sorted_pairs"]], np.arange(T * k))
        assert np.array_equal(out["active"], np.nonzero(np.bincount(flat, minlength=E))[0])
        assert out["n_active"] == len(np.unique(flat))


def test_permute_empty(orc):
    out = orc.permute(np.zeros((0, 4), np.int32), 8)
    assert out["counts"].sum() == 0 and out["n_active"] == 0
    assert np.all(out["offsets"] == 0)


def test_spec_verify_drafts_share_experts(orc):
    """The speculative-verify inputs ("Strata" page, sec. 3.4: several draft
    tokens of one sequence verified in one pass share expert fetches): drafts of
    one sequence correlate at rho, tokens of different sequences do not, and
    through the oracle's router and top-k the drafts of a sequence pick more
    common experts than tokens of different sequences."""
    sh = mi.CONFIGS["a3b"]
    n_seq, n_draft = 8, 4
    xb, _ = mi.make_spec_verify_activations(sh.H, n_seq, n_draft, seed=3)
    x = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    c = np.corrcoef(x)
    same = np.array([c[i, j] for i in range(len(x)) for j in range(len(x)) if i != j and i // n_draft == j // n_draft])
    diff = np.array([c[i, j] for i in range(len(x)) for j in range(len(x)) if i // n_draft != j // n_draft])
    assert abs(same.mean() - 0.64) < 0.05 and abs(diff.mean()) < 0.05      # rho^2 with unit-variance parts
    Wr, bias = mi.make_router(sh, 0)
    ids, _ = orc.topk(orc.router_logits(xb, Wr, bias), sh.k, True)
    sets = [set(r) for r in ids.tolist()]
    share = lambda i, j: len(sets[i] & sets[j])
    within = np.mean([share(i, j) for i in range(len(sets)) for j in range(len(sets)) if i != j and i // n_draft == j // n_draft])
    across = np.mean([share(i, j) for i in range(len(sets)) for j in range(len(sets)) if i // n_draft != j // n_draft])
    assert within > across + 1.0
    xi, _ = mi.make_activations(sh.H, n_seq * n_draft, 3)
    ids_i, _ = orc.topk(orc.router_logits(xi, Wr, bias), sh.k, True)
    assert len(set(ids.ravel().tolist())) < len(set(ids_i.ravel().tolist()))  # fewer distinct experts per batch
