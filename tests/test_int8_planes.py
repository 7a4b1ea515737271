"""The int8-plane split of activations that the integer-MFMA kernels use, checked
as arithmetic on the CPU (no GPU, no oracle).

Per row and group of 128 the kernels take hs = 2^e with
e = max(exponent(max |v|) - 5, -100) and planes q_p = rint(rem_p / 2^(e - 7p)),
rem_{p+1} = rem_p - q_p 2^(e - 7p).  These tests restate that split in float32
numpy and check what the design relies on: every remainder is exact, every
plane fits [-64, 64] (int8, and 15 * 64 * 128 per plane sum fits int32 with
room), the tail after P planes is at most 2^(e - 7P + 6) <= 2^-(7P - 1) of the
group's largest magnitude, and three planes represent every bf16 value within
2^12 of the group's largest exactly (its last bit is 2^-19 of the largest's
leading power of two or coarser).  A dropped remainder update, a wrong
exponent offset or a plane base other than 2^7 fails one of them.
"""
import numpy as np
import pytest


def split_planes(v, planes):
    """float32 values of one group -> (e, int planes [planes][n], tail)."""
    v = np.asarray(v, dtype=np.float32)
    mx = np.float32(np.max(np.abs(v)))
    ex = int((mx.view(np.uint32) >> 23) & 0xFF) - 127
    e = max(ex - 5, -100)
    rem = v.copy()
    qs = []
    for p in range(planes):
        up = np.float32(2.0 ** (7 * p - e))
        dn = np.float32(2.0 ** (e - 7 * p))
        q = np.rint(rem * up).astype(np.float32)          # rem * up is exact (a power of two)
        new = (rem - q * dn).astype(np.float32)           # float32 subtraction, as fmaf(-q, dn, rem)
        # exactness of the step: the float32 result equals the exact difference
        assert np.array_equal(new.astype(np.float64), rem.astype(np.float64) - q.astype(np.float64) * float(dn))
        qs.append(q.astype(np.int64))
        rem = new
    return e, np.stack(qs), rem


def rebuild(e, qs):
    return sum(q.astype(np.float64) * 2.0 ** (e - 7 * p) for p, q in enumerate(qs))


GROUPS = {
    "gauss": lambda r: r.standard_normal(128).astype(np.float32),
    "wide": lambda r: (r.standard_normal(128) * np.exp2(r.integers(-30, 10, 128))).astype(np.float32),
    "one_big": lambda r: np.concatenate([[np.float32(3e4)], r.standard_normal(127).astype(np.float32) * 1e-3]),
    "tiny": lambda r: (r.standard_normal(128) * 1e-35).astype(np.float32),
    "zeros": lambda r: np.zeros(128, np.float32),
    "max_pow2": lambda r: np.full(128, 64.0, np.float32) * np.where(r.random(128) < 0.5, -1, 1).astype(np.float32),
    "near_next_pow2": lambda r: np.full(128, np.float32(np.nextafter(np.float32(2.0), np.float32(0)))),
}


@pytest.mark.parametrize("kind", sorted(GROUPS))
@pytest.mark.parametrize("planes", [3, 4])
def test_planes_fit_int8_and_tail_is_bounded(kind, planes):
    r = np.random.default_rng(7)
    for _ in range(20):
        v = GROUPS[kind](r)
        e, qs, tail = split_planes(v, planes)
        assert np.all(np.abs(qs) <= 64), "a plane left [-64, 64]"
        mx = float(np.max(np.abs(v)))
        # what the planes represent plus the tail is the input, exactly
        assert np.array_equal(rebuild(e, qs) + tail.astype(np.float64), v.astype(np.float64))
        bound = 2.0 ** (e - 7 * planes + 6)
        assert np.all(np.abs(tail.astype(np.float64)) <= bound)
        if mx >= 2.0 ** -94:                              # e not clamped: the bound relative to the largest
            assert bound <= mx * 2.0 ** -(7 * planes - 1)


def test_int32_plane_sums_have_room():
    """Worst case per plane and group: 15 * 64 * 128 (4-bit codes against |q| <= 64)."""
    assert 15 * 64 * 128 < 2 ** 31 // 1000


def test_three_planes_hold_bf16_near_the_max_exactly():
    """bf16 values (8 significant bits) within 2^12 of the group's largest are exact with 3 planes,
    and one a power of two smaller need not be."""
    r = np.random.default_rng(3)
    for _ in range(50):
        v = (r.standard_normal(128) * np.exp2(r.integers(-12, 1, 128))).astype(np.float32)
        v = (v.view(np.uint32) & 0xFFFF0000).view(np.float32)          # round toward zero to bf16
        mx = float(np.max(np.abs(v)))
        e, qs, tail = split_planes(v, 3)
        near = np.abs(v) >= mx * 2.0 ** -12
        assert np.all(tail[near] == 0)
    # the limit is tight: the largest 1.0, an element 2^-13 with all 8 significant bits set
    v = np.zeros(128, np.float32)
    v[0] = 1.0
    v[1] = np.float32(2.0 ** -13 * (1 + 127 / 128))
    e, qs, tail = split_planes(v, 3)
    assert tail[1] != 0


def test_a_wrong_plane_base_breaks_the_bound():
    """Planes 2^-8 apart (a plausible slip) overflow int8 on the second plane."""
    v = np.random.default_rng(5).standard_normal(128).astype(np.float32)
    mx = np.float32(np.max(np.abs(v)))
    e = max(int((mx.view(np.uint32) >> 23) & 0xFF) - 127 - 5, -100)
    q0 = np.rint(v * np.float32(2.0 ** -e))
    rem = v - q0 * np.float32(2.0 ** e)
    q1 = np.rint(rem * np.float32(2.0 ** (8 - e)))
    assert np.max(np.abs(q1)) > 64
