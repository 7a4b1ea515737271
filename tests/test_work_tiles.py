"""The work-list checker (tests/work_tiles.py) against properties any correct
tiling of the grouped pairs has: every (token, expert) pair exactly once, in a
tile of its expert, tiles of at most 16 consecutive rows, expert-major, tile
indices counting up from 0 within each expert."""
import numpy as np

from work_tiles import expected_work_list


def test_work_list_covers_every_pair_once():
    rng = np.random.default_rng(9)
    for E, T, k in [(8, 4, 2), (4, 40, 2), (64, 37, 6), (16, 300, 4)]:
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        wl = expected_work_list(ids, E, k, 16)
        counts = np.bincount(ids.ravel(), minlength=E)
        assert wl.shape == (int(np.sum((counts + 15) // 16)), 20)
        assert np.all(np.diff(wl[:, 0]) >= 0)
        # tile index within the expert: 0 at each expert's first tile, then +1
        first = np.r_[True, wl[1:, 0] != wl[:-1, 0]]
        assert np.all(wl[first, 3] == 0) and np.all(wl[~first, 3] == wl[np.r_[~first[1:], False], 3] + 1)
        assert np.all((wl[:, 2] >= 1) & (wl[:, 2] <= 16))
        # rows tile [0, T*k) contiguously in order
        assert wl[0, 1] == 0 and np.array_equal(wl[1:, 1], (wl[:, 1] + wl[:, 2])[:-1])
        assert wl[-1, 1] + wl[-1, 2] == T * k
        seen = []
        for e, r0, n, _, *toks in wl.tolist():
            for j in range(16):
                t = toks[j] if j < n else toks[0]
                assert toks[j] == t
                if j < n:
                    assert e in ids[t]
                    seen.append((t, e))
        assert sorted(seen) == sorted((t, int(e)) for t in range(T) for e in ids[t])
    assert expected_work_list(np.zeros((0, 2), np.int32), 8, 2).shape == (0, 20)


