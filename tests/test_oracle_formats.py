"""Pins for the oracle's number formats and weight decoding.

Each check compares the oracle with something other than itself: numpy's own
binary16 conversion, brute-force nearest-value search, hand-encoded bytes,
and the closed form weight = code * scale + bias (page "Flash-MoE ...
(translation)", section 2; groups of 128 from the "Strata" page, section 2.2).
"""
import json
import math
import os
import struct

import numpy as np
import pytest

import moe_inputs as mi


def _f32(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits) & 0xFFFFFFFF))[0]


def test_f16_decode_all_patterns(orc):
    """Every binary16 pattern decodes like numpy's float16 (subnormals included)."""
    pats = np.arange(65536, dtype=np.uint16)
    ref = pats.view(np.float16).astype(np.float32)
    got = orc.f16_to_f32(pats)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_decode_known_values(orc):
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x0000: 0.0, 0x4300: 128.0, 0x4301: 129.0,
             0x7F80: math.inf, 0xFF80: -math.inf, 0x0001: 2.0 ** -133}
    for b, v in cases.items():
        assert orc.bf16_to_f32(np.array([b], np.uint16))[0] == np.float32(v)
    assert math.isnan(orc.bf16_to_f32(np.array([0x7FC0], np.uint16))[0])


def _nearest_bf16_bruteforce(v: float) -> int:
    """Nearest bf16 to v by searching the two neighbours (ties to even mantissa)."""
    if math.isnan(v):
        return 0x7FC0
    f = np.float32(v) if abs(v) < 3.5e38 else None
    # candidates: truncation of the float32 pattern and the next pattern up
    if f is None or math.isinf(f):
        return 0x7F80 if v > 0 else 0xFF80
    u = int(np.array([v], np.float64).astype(np.float32).view(np.uint32)[0])
    lo = u >> 16
    cands = [lo, lo + 1, max(lo - 1, 0)]
    best, bestd = None, None
    for c in cands:
        cv = _f32((c & 0xFFFF) << 16)
        if math.isnan(cv):
            continue
        d = abs(cv - v)
        if best is None or d < bestd or (d == bestd and (c & 1) == 0 and (best & 1) == 1):
            best, bestd = c & 0xFFFF, d
    return best


def test_f32_to_bf16_rounding(orc):
    rng = np.random.default_rng(11)
    vals = np.concatenate([rng.standard_normal(3000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 3000),
                           np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0, -0.0], np.float32)])
    vals = vals.astype(np.float32)
    got = orc.f32_to_bf16(vals)
    for v, g in zip(vals, got):
        assert int(g) == _nearest_bf16_bruteforce(float(v)), (v, hex(int(g)))
    # explicit ties: 1 + half-ulp goes to even (down), 1 + 3 half-ulps goes up
    assert int(orc.f32_to_bf16(np.array([_f32(0x3F808000)], np.float32))[0]) == 0x3F80
    assert int(orc.f32_to_bf16(np.array([_f32(0x3F818000)], np.float32))[0]) == 0x3F82
    assert int(orc.f32_to_bf16(np.array([np.nan], np.float32))[0]) == 0x7FC0


def test_f64_to_bf16_single_rounding(orc):
    rng = np.random.default_rng(12)
    vals = rng.standard_normal(3000) * 10.0 ** rng.integers(-20, 20, 3000)
    got = orc.f64_to_bf16(vals)
    for v, g in zip(vals, got):
        cands = []
        u = int(np.array([v]).astype(np.float32).view(np.uint32)[0]) >> 16
        for c in (u - 1, u, u + 1):
            cands.append((abs(_f32((c & 0xFFFF) << 16) - v), c & 1, c & 0xFFFF))
        cands.sort()
        assert int(g) == cands[0][2], (v, hex(int(g)), cands)
    # a value just above a bf16 midpoint that a double->float->bf16 path would
    # round down: 1 + 2^-8 + 2^-40 must round up to 1 + 2^-7
    assert int(orc.f64_to_bf16(np.array([1.0 + 2 ** -8 + 2 ** -40]))[0]) == 0x3F81
    assert int(orc.f64_to_bf16(np.array([1e39]))[0]) == 0x7F80
    assert int(orc.f64_to_bf16(np.array([2.0 ** -133]))[0]) == 0x0001


def test_code_unpack_hand_encoded(orc):
    # 4-bit: low nibble = even k
    assert orc.code(np.array([0xA3], np.uint8), 0, 4) == 0x3
    assert orc.code(np.array([0xA3], np.uint8), 1, 4) == 0xA
    # 2-bit: bits 2j..2j+1 hold k % 4 == j
    row = np.array([0b11100100], np.uint8)
    assert [orc.code(row, k, 2) for k in range(4)] == [0, 1, 2, 3]


@pytest.mark.parametrize("bits", [4, 2])
def test_code_unpack_roundtrip(orc, bits):
    rng = np.random.default_rng(bits)
    K = 256
    q = rng.integers(0, 2 ** bits, size=(3, K)).astype(np.uint8)
    packed = mi.pack_codes(q, bits)
    for n in range(3):
        assert [orc.code(packed[n], k, bits) for k in range(K)] == q[n].tolist()


@pytest.mark.parametrize("bits", [4, 2])
def test_dequant_closed_form(orc, bits):
    """w[n,k] = q * scale[n, k//128] + bias[n, k//128], decoded independently."""
    rng = np.random.default_rng(20 + bits)
    N, K = 5, 384
    q = rng.integers(0, 2 ** bits, size=(N, K)).astype(np.uint8)
    s = mi.f32_to_f16_bits(rng.uniform(0.005, 0.02, (N, K // 128)))
    b = mi.f32_to_f16_bits(rng.normal(0, 0.01, (N, K // 128)))
    # edge cases: a subnormal bias, q at both ends
    b[0, 0] = 0x0003                      # 3 * 2^-24
    q[1, :] = 2 ** bits - 1
    q[2, :] = 0
    w = orc.dequant_matrix(mi.pack_codes(q, bits), s, b, bits)
    sf = s.view(np.float16).astype(np.float64)
    bf = b.view(np.float16).astype(np.float64)
    g = np.arange(K) // 128
    ref = q.astype(np.float64) * sf[:, g] + bf[:, g]
    assert np.array_equal(w, ref)
    assert np.array_equal(w[2], bf[2, g])                             # q = 0 -> bias
    assert np.array_equal(w[1], (2 ** bits - 1) * sf[1, g] + bf[1, g])
    assert w[0, 0] == q[0, 0] * sf[0, 0] + 3 * 2.0 ** -24


def test_fma_form_identity(orc):
    """(code*scale + bias)*x == fma(code, scale*x, bias*x): the page's FMA
    rewrite (Flash-MoE page sec. 2) agrees with the oracle's dequantised dot
    product to float32 rounding."""
    rng = np.random.default_rng(5)
    K = 512
    q = rng.integers(0, 16, size=(1, K)).astype(np.uint8)
    s = mi.f32_to_f16_bits(rng.uniform(0.005, 0.02, (1, K // 128)))
    b = mi.f32_to_f16_bits(rng.normal(0, 0.01, (1, K // 128)))
    x = rng.standard_normal(K).astype(np.float32)
    w = orc.dequant_matrix(mi.pack_codes(q, 4), s, b, 4)[0]
    exact = float(np.dot(w, x.astype(np.float64)))
    sf = s.view(np.float16).astype(np.float32)[0][np.arange(K) // 128]
    bf = b.view(np.float16).astype(np.float32)[0][np.arange(K) // 128]
    fma_form = np.float32(0)
    for kk in range(K):
        sx = np.float32(sf[kk] * x[kk])
        bx = np.float32(bf[kk] * x[kk])
        fma_form = np.float32(fma_form + np.float32(np.float64(q[0, kk]) * sx + bx))
    assert abs(float(fma_form) - exact) <= 1e-5 * float(np.sum(np.abs(w * x)))


def test_expert_bytes_match_page_figure():
    """Page 5 (Flash-MoE, 'SSD expert streaming') quotes about 6.75 MB per
    expert for its 512-expert top-4 model; the 4-bit g128 layout of the
    512-expert shape (hidden 4096, intermediate 1024) gives 6,684,672 bytes."""
    here = os.path.dirname(__file__)
    with open(os.path.join(here, "golden", "expert_bytes.json")) as f:
        gold = json.load(f)
    shape = mi.CONFIGS["e512"]
    got = shape.bytes_per_expert(4)
    assert got == gold["layout_bytes_q4_g128"]
    assert abs(got / 1e6 - gold["page_value_MB"]) / gold["page_value_MB"] < gold["rel_tolerance"]


def _f16_neighbours(n, rng):
    """Doubles across the binary16 range: random, exact ties between neighbours,
    the subnormal range and the edge of overflow."""
    pats = rng.integers(0, 0x7C00, size=n).astype(np.uint16)          # finite, non-negative
    lo = pats.view(np.float16).astype(np.float64)
    hi = (pats + 1).view(np.float16).astype(np.float64)               # next value up (0x7C00: inf)
    hi = np.where(np.isinf(hi), 65536.0, hi)
    mid = 0.5 * (lo + hi)                                             # exact ties
    frac = lo + (hi - lo) * rng.random(n)
    edge = np.array([0.0, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -24, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25,
                     65504.0, 65519.99, 65520.0, 1e6, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11])
    v = np.concatenate([lo, mid, frac, edge])
    return np.concatenate([v, -v])


def test_f64_to_f16_matches_numpy(orc):
    """Rounding to binary16 (nearest, ties to even, overflow to inf) agrees with
    numpy's own float64 -> float16 conversion bit for bit."""
    v = _f16_neighbours(4000, np.random.default_rng(7))
    got = orc.f64_to_f16(v)
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref), v[got != ref][:5]
    assert orc.f64_to_f16(np.array([np.nan]))[0] == 0x7E00


def test_zero_point_bias_reproduces_zero_point_weights(orc):
    """(q - z) s written as q s + b with b = -(z s): every weight agrees with
    the zero-point form within b's one rounding (half an fp16 spacing of z s),
    and exactly where z s is an fp16 value (power-of-two scales)."""
    rng = np.random.default_rng(11)
    for bits in (4, 2):
        N, K = 6, 512
        codes = rng.integers(0, 1 << bits, size=(N, K))
        q = mi.pack_codes(codes, bits)
        s = mi.f32_to_f16_bits(rng.uniform(0.005, 0.02, size=(N, K // 128)))
        z = rng.integers(0, 1 << bits, size=(N, K // 128)).astype(np.uint8)
        b = orc.zero_point_bias(s, z)
        sv = s.view(np.float16).astype(np.float64)
        zs = z.astype(np.float64) * sv
        exact = (codes - np.repeat(z.astype(np.float64), 128, axis=1)) * np.repeat(sv, 128, axis=1)
        got = orc.dequant_matrix(q, s, b, bits)
        bound = np.repeat(np.abs(zs) * 2.0 ** -11, 128, axis=1)
        assert np.all(np.abs(got - exact) <= bound)
        # b is -(z s) rounded once: the nearest fp16 value
        bv = b.view(np.float16).astype(np.float64)
        assert np.all(np.abs(bv + zs) <= np.abs(zs) * 2.0 ** -11)
        # power-of-two scales: z s is exact in fp16, so are the weights
        s2 = mi.f32_to_f16_bits(2.0 ** rng.integers(-10, -4, size=(N, K // 128)).astype(np.float32))
        b2 = orc.zero_point_bias(s2, z)
        exact2 = (codes - np.repeat(z.astype(np.float64), 128, axis=1)) * \
            np.repeat(s2.view(np.float16).astype(np.float64), 128, axis=1)
        assert np.array_equal(orc.dequant_matrix(q, s2, b2, bits), exact2)


def test_zero_point_bias_special_cases(orc):
    """z = 0 gives -0 (weights q s); a negative scale flips the sign; z s past
    the fp16 range gives an infinite bias."""
    s = mi.f32_to_f16_bits(np.array([0.5, -0.25, 60000.0, 2.0 ** -24], np.float32))
    z = np.array([0, 3, 2, 255], np.uint8)
    b = orc.zero_point_bias(s, z)
    assert b[0] == 0x8000
    assert b[1] == np.float16(0.75).view(np.uint16)
    assert b[2] == 0xFC00
    assert b[3] == np.float16(-255 * 2.0 ** -24).view(np.uint16)
    with pytest.raises(ValueError):
        orc.zero_point_bias(s, z[:3])
