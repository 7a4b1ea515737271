"""Pins for the oracle's residency tiers ("Luce Spark" page, sec. 1: routing
frequencies counted from traffic pick the hot set kept resident; sec. 2: a
bounded ring of spare slots, filled from pinned host memory on a miss, the
least recently used slot giving way).

  * counters: numpy's uint32 addition (wrapping like the device's);
  * hot set: numpy's lexsort of (-count, id) -- a library sort, not the
    oracle's selection loop -- on random counts with many ties;
  * warm ring: a separate pure-Python model written from the page's rule
    (the slot with the oldest last use, ties to the lowest slot, among those
    not used in this step; hot slots never), run over random step sequences,
    plus invariants (the two tables stay inverse, hot slots untouched, no slot
    taken twice in a step, a miss with no free slot stays cold) and a hand
    worked case.
"""
import numpy as np
import pytest


def test_freq_update_is_uint32_addition(orc):
    rng = np.random.default_rng(70)
    for E in (1, 8, 1000):
        freq = rng.integers(0, 2 ** 32, E, dtype=np.uint64).astype(np.uint32)
        freq[0] = 2 ** 32 - 3                                  # wraps like the device counter
        counts = rng.integers(0, 200, E).astype(np.int32)
        counts[0] = 5
        assert np.array_equal(orc.freq_update(counts, freq), ((freq.astype(np.uint64) + counts.astype(np.uint64)) % 2 ** 32).astype(np.uint32))


def test_hot_set_matches_a_library_sort(orc):
    rng = np.random.default_rng(71)
    for E, n in ((8, 5), (64, 24), (256, 154), (512, 307), (1000, 1), (7, 7)):
        freq = rng.integers(0, 12, E).astype(np.uint32)      # few distinct values: many ties
        want = np.lexsort((np.arange(E), -freq.astype(np.int64)))[:n]
        assert np.array_equal(orc.hot_set(freq, n), want)
    # hand case: ties go to the lower id, most used first
    assert orc.hot_set(np.array([3, 9, 9, 1, 0, 9], np.uint32), 4).tolist() == [1, 2, 5, 0]


def _py_ring(n_hot, miss, step, soe, eos, lu):
    """The page's rule, written out again in plain Python."""
    soe, eos, lu = list(soe), list(eos), list(lu)
    copies = []
    for e in miss:
        cands = [(lu[s], s) for s in range(n_hot, len(eos)) if lu[s] != step]
        if not cands:
            continue
        _, s = min(cands)
        if eos[s] >= 0:
            soe[eos[s]] = -1
        eos[s], soe[e], lu[s] = e, s, step
        copies.append((e, s))
    return soe, eos, lu, copies


def test_warm_ring_against_a_python_model(orc):
    rng = np.random.default_rng(72)
    for trial in range(40):
        E = int(rng.integers(4, 40))
        n_slots = int(rng.integers(1, E + 1))
        n_hot = int(rng.integers(0, n_slots + 1))
        soe = np.full(E, -1, np.int32)
        eos = np.full(n_slots, -1, np.int32)
        hot = rng.permutation(E)[:n_hot]
        soe[hot] = np.arange(n_hot)
        eos[:n_hot] = hot
        lu = np.zeros(n_slots, np.uint32)
        for step in range(1, 12):
            picked = np.unique(rng.choice(E, int(rng.integers(1, E + 1))))
            # this step's hits are stamped first (as the slot lookup does)
            for e in picked:
                if soe[e] >= 0:
                    lu[soe[e]] = step
            miss = np.array([e for e in picked if soe[e] < 0], np.int32)
            got = orc.warm_ring_step(n_hot, miss, step, soe, eos, lu)
            want = _py_ring(n_hot, miss.tolist(), step, soe.tolist(), eos.tolist(), lu.tolist())
            assert got["slot_of_expert"].tolist() == want[0]
            assert got["expert_of_slot"].tolist() == want[1]
            assert got["last_use"].tolist() == want[2]
            assert got["copies"] == want[3]
            # invariants
            s2, e2 = got["slot_of_expert"], got["expert_of_slot"]
            assert np.array_equal(e2[:n_hot], eos[:n_hot]) and np.all(got["last_use"][:n_hot] == lu[:n_hot])
            for s in range(n_slots):
                if e2[s] >= 0:
                    assert s2[e2[s]] == s
            for e in range(E):
                if s2[e] >= 0:
                    assert e2[s2[e]] == e
            slots = [s for _, s in got["copies"]]
            assert len(slots) == len(set(slots)) and all(s >= n_hot for s in slots)
            n_free = int(np.sum(lu[n_hot:] != step))
            assert len(got["copies"]) == min(len(miss), n_free)
            soe, eos, lu = s2, e2, got["last_use"]


def test_warm_ring_hand_case(orc):
    """Two hot slots, two ring slots.  Step 3 misses experts 1, 4, 6: slot 2
    (never used) takes 1, slot 3 (last used at step 1) takes 4, and 6 finds no
    free slot (both were used this step) and stays cold.  Step 4 misses 6
    again and 5: slot 2 and slot 3 were both used at step 3, so the lower slot
    (2) goes first and its expert 1 stops being resident."""
    soe = np.array([0, -1, 1, -1, -1, -1, -1], np.int32)
    eos = np.array([0, 2, -1, 5], np.int32)
    soe[5] = 3
    lu = np.array([3, 3, 0, 1], np.uint32)
    r = orc.warm_ring_step(2, np.array([1, 4, 6], np.int32), 3, soe, eos, lu)
    assert r["copies"] == [(1, 2), (4, 3)]
    assert r["slot_of_expert"].tolist() == [0, 2, 1, -1, 3, -1, -1]
    assert r["expert_of_slot"].tolist() == [0, 2, 1, 4] and r["last_use"].tolist() == [3, 3, 3, 3]
    r2 = orc.warm_ring_step(2, np.array([5, 6], np.int32), 4, r["slot_of_expert"], r["expert_of_slot"],
                            r["last_use"])
    assert r2["copies"] == [(5, 2), (6, 3)]
    assert r2["slot_of_expert"][1] == -1 and r2["slot_of_expert"][4] == -1
