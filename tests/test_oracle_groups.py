"""Pins for the oracle's group size (32, 64 or 128 weights per scale and bias).

Groups of 128 are the default format ("Strata" page, section 2.2); 64 is the
finer group for quality ("Strata" page, section 4.4) and 32 the laptop page's
(section 4.2: 32 weights share a scale and a zero point).  A weight is
code * scale + bias of its group (page "Flash-MoE ... (translation)",
section 2).  The pins:
  * locality: changing the scale of group j of row n changes exactly the
    weights of that row with k in [j g, (j + 1) g), each by code * (change);
  * coarsening: finer groups whose scales and biases repeat a coarser
    matrix's give the same weights and the same FFN outputs, bit for bit;
  * a closed form for the FFN with unit activations and per-group scales
    (powers of two, exact) that differ from group to group;
  * the format's byte count at the 512-expert shape with groups of 64, against
    the "Flash-MoE" page's "about 6.75 MB per expert".
A wrong divisor (k / 128 for every size), a scale row stride of K / 128, or
a matrix left at the default group fails one of them.
"""
import math

import numpy as np
import pytest

import moe_inputs as mi
import oracle

GROUPS = (32, 64, 128)


def _codes(rng, N, K, bits):
    return rng.integers(0, 1 << bits, size=(N, K), dtype=np.uint8)


def _f16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("group", [32, 64])
def test_scale_change_touches_only_its_group(bits, group):
    rng = np.random.default_rng(11)
    N, K = 3, 256
    codes = _codes(rng, N, K, bits)
    q = mi.pack_codes(codes, bits)
    s = mi.f32_to_f16_bits(rng.uniform(0.5, 1.0, size=(N, K // group)))
    b = mi.f32_to_f16_bits(rng.normal(0.0, 0.1, size=(N, K // group)))
    w0 = oracle.dequant_matrix(q, s, b, bits)
    for n0, j in [(0, 0), (1, K // group - 1), (2, 1)]:
        s1 = s.copy()
        s1[n0, j] = np.float16(2.0).view(np.uint16)
        w1 = oracle.dequant_matrix(q, s1, b, bits)
        diff = w1 - w0
        inside = np.zeros_like(diff, dtype=bool)
        inside[n0, j * group:(j + 1) * group] = True
        assert np.all(diff[~inside] == 0.0)
        expect = codes[n0, j * group:(j + 1) * group] * (2.0 - _f16(s[n0, j]))
        np.testing.assert_array_equal(diff[n0, j * group:(j + 1) * group], expect)


def _coarse_expert(rng, H, I, bits):
    mats = {}
    for m, (N, K) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        q = mi.pack_codes(_codes(rng, N, K, bits), bits)
        s = mi.f32_to_f16_bits(rng.uniform(0.005, 0.02, size=(N, K // 128)))
        b = mi.f32_to_f16_bits(rng.normal(0.0, 0.01, size=(N, K // 128)))
        mats[m] = (q, s, b)
    return mats


def _refine(mats, group):
    """The same weights written with groups of `group`: every scale and bias repeated."""
    r = 128 // group
    return {m: (q, np.repeat(s, r, axis=1), np.repeat(b, r, axis=1)) for m, (q, s, b) in mats.items()}


@pytest.mark.parametrize("bits", [4, 2])
def test_finer_groups_with_repeated_scales_match(bits):
    rng = np.random.default_rng(5)
    H, I = 256, 384
    mats = _coarse_expert(rng, H, I, bits)
    x = mi.f32_to_bf16_bits(rng.normal(0.0, 1.0, size=H).astype(np.float32))
    h0, y0 = oracle.expert_ffn_row(x, mats, bits)
    for group in (64, 32):
        fine = _refine(mats, group)
        for m in mats:
            np.testing.assert_array_equal(oracle.dequant_matrix(*fine[m], bits), oracle.dequant_matrix(*mats[m], bits))
        h1, y1 = oracle.expert_ffn_row(x, fine, bits)
        np.testing.assert_array_equal(h1, h0)
        np.testing.assert_array_equal(y1, y0)


@pytest.mark.parametrize("group", [32, 64])
def test_ffn_closed_form_with_per_group_scales(group):
    """Unit activations, constant codes, scale 2^-(j mod 3) for group j, no bias:
    a_i = c_g g sum_j 2^-(j mod 3), u_i the same with c_u, and the down output
    y_n = c_d sum_j 2^-(j mod 3) (sum of h over group j) with h constant."""
    bits = 4
    H, I = 256, 128
    cg, cu, cd = 3, 5, 2
    x = mi.f32_to_bf16_bits(np.ones(H, np.float32))

    def mat(N, K, c):
        q = mi.pack_codes(np.full((N, K), c, np.uint8), bits)
        sc = np.array([2.0 ** -(j % 3) for j in range(K // group)])
        s = mi.f32_to_f16_bits(np.tile(sc, (N, 1)))
        return q, s, mi.f32_to_f16_bits(np.zeros((N, K // group)))

    mats = {"gate": mat(I, H, cg), "up": mat(I, H, cu), "down": mat(H, I, cd)}
    h, y = oracle.expert_ffn_row(x, mats, bits)
    ssum_h = sum(2.0 ** -(j % 3) for j in range(H // group))
    a = cg * group * ssum_h
    u = cu * group * ssum_h
    hv = float(np.float32(a / (1.0 + math.exp(-a)) * u))
    np.testing.assert_allclose(h, np.full(I, hv, np.float32), rtol=1e-6)
    ssum_i = sum(2.0 ** -(j % 3) for j in range(I // group))
    yv = cd * group * ssum_i * float(h[0])
    yb = (np.asarray(y, np.uint32) << 16).view(np.float32)
    np.testing.assert_allclose(yb, np.full(H, yv, np.float32), rtol=2 ** -8)


def test_expert_bytes_at_group_64_match_the_flash_moe_figure():
    """512-expert shape (H 4096, I 1024), 4-bit codes, fp16 scale and bias:
    groups of 64 give 7,077,888 B per expert, the page's "about 6.75 MB"
    read as MiB (6.75 * 2^20); groups of 128 give 6,684,672 B."""
    e512 = mi.CONFIGS["e512"]
    assert mi.dataclasses.replace(e512, group=64).bytes_per_expert(4) == 7_077_888
    assert 7_077_888 == 6.75 * 2 ** 20
    assert e512.bytes_per_expert(4) == 6_684_672


def test_group_size_is_read_from_the_scales():
    rng = np.random.default_rng(2)
    q = mi.pack_codes(_codes(rng, 2, 128, 4), 4)
    with pytest.raises(ValueError):
        oracle.dequant_matrix(q, np.zeros((2, 3), np.uint16), np.zeros((2, 3), np.uint16), 4)
    for group in GROUPS:
        w = oracle.dequant_matrix(q, np.zeros((2, 128 // group), np.uint16), np.zeros((2, 128 // group), np.uint16), 4)
        assert w.shape == (2, 128) and np.all(w == 0.0)
