"""Pins for the oracle's expert FFN and combine.

The FFN is gate/up matvec -> SwiGLU -> down matvec over group-wise dequantised
weights (fused SwiGLU and combine + residual: page "Flash-MoE ...
(translation)", section 3; weight = code * scale + bias: same page, section 2).
Structured experts give closed forms that a dropped term, a wrong group or row
index, a swapped gate/up or a transposed matrix would all break:
  * permutation experts (each row picks one input) -> Y_n = silu(x_a) * c x_b;
  * zero expert -> Y = 0;
  * per-group constant experts -> sums of group sums of x;
  * per-(row, group) scales with unit codes;
  * a dense float64 reference built from numpy-decoded weights on the tiny shape.
"""
import math

import numpy as np
import pytest

import moe_inputs as mi


def _bf16_f64(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def _f16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def _pack_matrix(codes, scale_f, bias_f, bits=4):
    return (mi.pack_codes(codes, bits), mi.f32_to_f16_bits(scale_f), mi.f32_to_f16_bits(bias_f))


def _selection_expert(N, K, cols, value_code=1, scale=1.0, bits=4):
    """Row n has a single nonzero code at column cols[n] (bias 0)."""
    q = np.zeros((N, K), np.uint8)
    q[np.arange(N), cols] = value_code
    return _pack_matrix(q, np.full((N, K // 128), scale), np.zeros((N, K // 128)), bits)


@pytest.mark.parametrize("bits", [4, 2])
def test_ffn_permutation_expert_closed_form(orc, bits):
    H, I = 256, 512
    rng = np.random.default_rng(30 + bits)
    x = mi.f32_to_bf16_bits(rng.standard_normal(H).astype(np.float32))
    pg = rng.integers(0, H, I)                    # gate row i reads x[pg[i]]
    pu = rng.integers(0, H, I)                    # up row i reads x[pu[i]]
    pd = rng.permutation(I)[:H]                   # down row n reads h[pd[n]]
    w = {"gate": _selection_expert(I, H, pg, 1, 1.0, bits),
         "up": _selection_expert(I, H, pu, 2, 0.25, bits),       # weight 0.5
         "down": _selection_expert(H, I, pd, 3, 0.5, bits)}      # weight 1.5
    h, y = orc.expert_ffn_row(x, w, bits)
    xf = _bf16_f64(x)
    a = xf[pg]
    u = 0.5 * xf[pu]
    h_ref = (a / (1.0 + np.exp(-a)) * u).astype(np.float32)
    assert np.array_equal(h, h_ref)
    y_ref = mi.f32_to_bf16_bits((1.5 * h_ref[pd].astype(np.float64)).astype(np.float32))
    assert np.array_equal(y, y_ref)


def test_ffn_identity_expert_is_swiglu_of_input(orc):
    """Identity gate/up/down (code 1, scale 1, bias 0): Y_n = silu(x_n) * x_n for
    n < min(H, I) and 0 beyond."""
    H, I = 256, 512
    rng = np.random.default_rng(40)
    x = mi.f32_to_bf16_bits(rng.standard_normal(H).astype(np.float32))
    eye_gu = np.arange(I) % H                     # rows >= H repeat (still one pick per row)
    w = {"gate": _selection_expert(I, H, eye_gu), "up": _selection_expert(I, H, eye_gu),
         "down": _selection_expert(H, I, np.arange(H))}
    _, y = orc.expert_ffn_row(x, w, 4)
    xf = _bf16_f64(x)
    ref = mi.f32_to_bf16_bits((xf / (1 + np.exp(-xf)) * xf).astype(np.float32))
    assert np.array_equal(y, ref)


def test_ffn_zero_expert(orc):
    H, I = 256, 256
    z = _pack_matrix(np.zeros((I, H), np.uint8), np.full((I, 2), 0.01), np.zeros((I, 2)))
    w = {"gate": z, "up": z, "down": z}
    x = mi.f32_to_bf16_bits(np.random.default_rng(1).standard_normal(H).astype(np.float32))
    h, y = orc.expert_ffn_row(x, w, 4)
    assert np.all(h == 0) and np.all(y == 0)


def test_ffn_group_constants_closed_form(orc):
    """Codes 0, bias beta[n, g]: a_i = sum_g beta_g(i) * X_g with X_g the sum of x
    over group g; codes 1 with scale s[n, g] and bias 0 give the same form."""
    H, I = 512, 256
    rng = np.random.default_rng(50)
    x = mi.f32_to_bf16_bits(rng.standard_normal(H).astype(np.float32))
    xf = _bf16_f64(x)
    Xg = xf.reshape(4, 128).sum(1)
    beta = mi.f32_to_f16_bits(rng.normal(0, 0.01, (I, 4)))
    sc = mi.f32_to_f16_bits(rng.uniform(0.005, 0.02, (I, 4)))
    gate = (mi.pack_codes(np.zeros((I, H), np.uint8), 4), sc, beta)          # a = sum beta X
    up = (mi.pack_codes(np.ones((I, H), np.uint8), 4), sc, np.zeros((I, 4), np.uint16))  # u = sum s X
    down = _selection_expert(H, I, np.arange(H) % I)
    h, y = orc.expert_ffn_row(x, {"gate": gate, "up": up, "down": down}, 4)
    a = (_f16(beta) * Xg).sum(1).astype(np.float32).astype(np.float64)
    u = (_f16(sc) * Xg).sum(1).astype(np.float32).astype(np.float64)
    h_ref = (a / (1 + np.exp(-a)) * u).astype(np.float32)
    assert np.allclose(h, h_ref, rtol=1e-6, atol=0)
    # down: per-group constant again, now over h
    dn_beta = mi.f32_to_f16_bits(rng.normal(0, 0.01, (H, 2)))
    down2 = (mi.pack_codes(np.zeros((H, I), np.uint8), 4), np.zeros((H, 2), np.uint16), dn_beta)
    h2, y2 = orc.expert_ffn_row(x, {"gate": gate, "up": up, "down": down2}, 4)
    Hg = h2.astype(np.float64).reshape(2, 128).sum(1)
    y_ref = (_f16(dn_beta) * Hg).sum(1)
    assert np.allclose(_bf16_f64(y2), y_ref, rtol=2 ** -8, atol=0)


def test_ffn_dense_float64_reference_tiny(orc):
    """Random tiny-shape expert against a dense float64 evaluation whose weights
    are decoded by numpy bit operations (not by the oracle)."""
    shape = mi.CONFIGS["tiny"]
    W = mi.make_expert_weights(shape, 4, seed=0, experts=[3])
    xb, _ = mi.make_activations(shape.H, 2, seed=0)
    dense = {}
    for m in mi.MATRICES:
        q = W.q[m][0]
        codes = np.stack([q & 0xF, q >> 4], axis=-1).reshape(q.shape[0], -1).astype(np.float64)
        g = np.arange(codes.shape[1]) // 128
        dense[m] = codes * _f16(W.scale[m][0])[:, g] + _f16(W.bias[m][0])[:, g]
    ow = {m: (W.q[m][0], W.scale[m][0], W.bias[m][0]) for m in mi.MATRICES}
    for t in range(2):
        h, y = orc.expert_ffn_row(xb[t], ow, 4)
        xf = _bf16_f64(xb[t])
        a = (dense["gate"] @ xf).astype(np.float32).astype(np.float64)
        u = (dense["up"] @ xf).astype(np.float32).astype(np.float64)
        h_ref = (a / (1 + np.exp(-a)) * u).astype(np.float32)
        assert np.allclose(h, h_ref, rtol=1e-6, atol=1e-6)
        yd = dense["down"] @ h.astype(np.float64)
        assert np.max(np.abs(_bf16_f64(y) - yd) / np.maximum(np.abs(yd), 1e-3)) <= 2 ** -8


def test_ffn_sampled_outputs_match_full(orc):
    shape = mi.CONFIGS["tiny"]
    W = mi.make_expert_weights(shape, 4, seed=0, experts=[1])
    xb, _ = mi.make_activations(shape.H, 1, seed=0)
    ow = {m: (W.q[m][0], W.scale[m][0], W.bias[m][0]) for m in mi.MATRICES}
    h, y = orc.expert_ffn_row(xb[0], ow, 4)
    idx = np.array([0, 17, 255, 128], np.int32)
    h2, ys = orc.expert_ffn_row(xb[0], ow, 4, n_idx=idx)
    assert np.array_equal(h, h2) and np.array_equal(ys, y[idx])


def test_combine_closed_forms(orc):
    rng = np.random.default_rng(60)
    T, H, k = 3, 256, 2
    res = mi.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    Y = mi.f32_to_bf16_bits(rng.standard_normal((T * k, H)).astype(np.float32) * 100)
    # every pair of token t uses the same Y row; gates 0.5 + 0.5 (exact halves)
    Yr = np.repeat(Y[::k], k, axis=0)
    p2r = np.arange(T * k, dtype=np.int32)
    g = np.full((T, k), 0.5, np.float32)
    out = orc.combine(Yr, p2r, g, res)
    r32 = _bf16_f64(res).astype(np.float32)
    y32 = _bf16_f64(Y[::k]).astype(np.float32)
    # fma(0.5, y, r) = round(r + y/2) since y/2 is exact; applied twice in order
    acc = (r32 + np.float32(0.5) * y32).astype(np.float32)
    acc = (acc + np.float32(0.5) * y32).astype(np.float32)
    assert np.array_equal(out, mi.f32_to_bf16_bits(acc))
    # one pick with gate 1: out = bf16(residual + Y)
    out1 = orc.combine(Y[:T], np.arange(T, dtype=np.int32), np.ones((T, 1), np.float32), res)
    assert np.array_equal(out1, mi.f32_to_bf16_bits((r32 + _bf16_f64(Y[:T]).astype(np.float32)).astype(np.float32)))
    # rows are gathered through pair_to_row: reversing the storage order of Y
    # together with the map leaves the result unchanged
    rev = np.arange(T * k)[::-1].astype(np.int32)
    g2 = rng.random((T, k)).astype(np.float32)
    a = orc.combine(Y, p2r, g2, res)
    b = orc.combine(Y[::-1].copy(), rev, g2, res)
    assert np.array_equal(a, b)


def test_layer_identity_experts_end_to_end(orc):
    """All experts identity, gates sum to 1: out ~= residual + silu(x) * x."""
    shape = mi.CONFIGS["tiny"]
    H, I, E, k, T = shape.H, shape.I, shape.E, shape.k, 4
    eye_gu = np.arange(I) % H
    one = {"gate": _selection_expert(I, H, eye_gu), "up": _selection_expert(I, H, eye_gu),
           "down": _selection_expert(H, I, np.arange(H))}
    W = mi.ExpertWeights(bits=4, experts=np.arange(E),
                         q={m: np.stack([one[m][0]] * E) for m in mi.MATRICES},
                         scale={m: np.stack([one[m][1]] * E) for m in mi.MATRICES},
                         bias={m: np.stack([one[m][2]] * E) for m in mi.MATRICES})
    xb, res = mi.make_activations(H, T, seed=3)
    Wr, _ = mi.make_router(shape, seed=3)
    out = orc.layer(xb, Wr, None, W, k, np.arange(E, dtype=np.int32), E, res)
    assert out["perm"]["counts"].sum() == T * k
    assert np.allclose(out["gates"].sum(1), 1.0, atol=4e-7)
    xf = _bf16_f64(xb)
    y = _bf16_f64(mi.f32_to_bf16_bits((xf / (1 + np.exp(-xf)) * xf).astype(np.float32)))
    ref = _bf16_f64(res) + y
    got = _bf16_f64(out["out"])
    # one bf16 rounding of the sum plus float32 gate rounding (gates sum to 1 +- 4e-7)
    assert np.all(np.abs(got - ref) <= 2 ** -8 * np.abs(ref) + 1e-6 * np.abs(y))


def test_shared_gate_against_scipy_and_closed_forms(orc):
    """Sigmoid gate of the shared expert: scipy's expit of numpy's float64 dot
    product (to one float32 rounding), and closed forms: w = 0 gives 1/2 for
    every token; L = ln 3 gives 3/4; a large |L| saturates to 0 or 1."""
    from scipy.special import expit
    rng = np.random.default_rng(61)
    T, H = 5, 512
    x = mi.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    w = (rng.standard_normal(H) * 0.05).astype(np.float32)
    got = orc.shared_gate(x, w)
    L = _bf16_f64(x) @ w.astype(np.float64)
    assert np.max(np.abs(got.astype(np.float64) - expit(L))) <= 2.0 ** -24
    assert np.all(orc.shared_gate(x, np.zeros(H, np.float32)) == np.float32(0.5))
    x1 = np.zeros((3, H), np.uint16)
    x1[:, 0] = mi.f32_to_bf16_bits(np.array([1.0, 1.0, -1.0], np.float32))
    for wv, want, tol in ((math.log(3.0), 0.75, 1e-7), (1000.0, 1.0, 0.0)):
        w1 = np.zeros(H, np.float32)
        w1[0] = wv
        g = orc.shared_gate(x1, w1)
        assert abs(float(g[0]) - want) <= tol and abs(float(g[1]) - want) <= tol
        assert abs(float(g[2]) - (1.0 - want)) <= tol


def test_combine_shared_closed_forms(orc):
    """The shared row enters as one more float32 FMA after the routed picks:
    a zero shared gate gives combine() bit for bit; with exact halves the result
    is the float32 chain residual + Y/2 + Y/2 + Ys/2."""
    rng = np.random.default_rng(62)
    T, H, k = 3, 256, 2
    res = mi.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    Y = mi.f32_to_bf16_bits(rng.standard_normal((T * k, H)).astype(np.float32) * 100)
    Ys = mi.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32) * 10)
    p2r = np.arange(T * k, dtype=np.int32)
    g = rng.random((T, k)).astype(np.float32)
    base = orc.combine(Y, p2r, g, res)
    assert np.array_equal(orc.combine_shared(Y, p2r, g, Ys, np.zeros(T, np.float32), res), base)
    Yr = np.repeat(Y[::k], k, axis=0)
    half = np.full((T, k), 0.5, np.float32)
    out = orc.combine_shared(Yr, p2r, half, Ys, np.full(T, 0.5, np.float32), res)
    r32 = _bf16_f64(res).astype(np.float32)
    y32 = _bf16_f64(Y[::k]).astype(np.float32)
    s32 = _bf16_f64(Ys).astype(np.float32)
    acc = (r32 + np.float32(0.5) * y32).astype(np.float32)
    acc = (acc + np.float32(0.5) * y32).astype(np.float32)
    acc = (acc + np.float32(0.5) * s32).astype(np.float32)
    assert np.array_equal(out, mi.f32_to_bf16_bits(acc))
    # the shared gate is per token: gate 1 on token 0 only adds Ys[0] to row 0
    sg = np.array([1.0, 0.0, 0.0], np.float32)
    one = orc.combine_shared(Y, p2r, g, Ys, sg, res)
    assert np.array_equal(one[1:], base[1:])
    assert not np.array_equal(one[0], base[0])


# ------------------------------------------- combine: an independent float32 chain
#
# The combine accumulates in float32 in pick order, one fused multiply-add per
# pick, and rounds once to bf16 (the "Flash-MoE" page, sec. 3: combine +
# residual in one kernel; the pick order and the rounding points are this
# library's reading).  The reference below does not call fmaf: it takes every
# step exactly in float64 -- the inputs have few significant bits (bf16 rows,
# gates m/64), so g*y is exact and so is acc + g*y, which TwoSum verifies -- and
# rounds that exact value once to float32, which is what a fused multiply-add
# returns.  Crafted columns make the chain's order visible in the bf16 output.

def _two_sum_exact(a, b):
    s = a + b
    bb = s - a
    err = (a - (s - bb)) + (b - bb)
    assert np.all(err == 0.0), "an exact float64 step was expected"
    return s


def _chain(res_bits, terms):
    """acc = float32(residual); for (g, y) in order: acc = float32(exact(acc + g*y)).
    terms: list of (g float64 [T, 1 or H], y float64 [T, H]).  Returns bf16 bits."""
    acc = _bf16_f64(res_bits).astype(np.float32)
    for g, y in terms:
        prod = np.asarray(g, np.float64) * np.asarray(y, np.float64)
        acc = _two_sum_exact(acc.astype(np.float64), prod).astype(np.float32)
    u = acc.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)     # bf16, nearest even


def _few_bit_bf16(rng, shape, emin, emax):
    """bf16 values m * 2^(e-7), m in [128, 255] with a random sign: 8 significant bits."""
    m = rng.integers(128, 256, shape).astype(np.float64) * rng.choice([-1.0, 1.0], shape)
    e = rng.integers(emin, emax + 1, shape)
    return mi.f32_to_bf16_bits(np.ldexp(m, e - 7).astype(np.float32))


def _combine_case(seed=63):
    """Six tokens, four picks each over seven experts; rows stored in expert order
    through a permutation that is not its own inverse.  Token 0 has power-of-two
    gates and crafted columns 0-1 (see below); the others random gates m/64."""
    rng = np.random.default_rng(seed)
    T, H, k, E = 6, 64, 4, 7
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    sorted_pairs = np.argsort(ids.ravel(), kind="stable").astype(np.int32)
    pair_to_row = np.empty_like(sorted_pairs)
    pair_to_row[sorted_pairs] = np.arange(T * k, dtype=np.int32)
    assert not np.array_equal(sorted_pairs, pair_to_row)
    g = np.stack([rng.choice(np.arange(1, 64), k, replace=False) / 64.0 for _ in range(T)]).astype(np.float32)
    g[0] = [0.5, 0.25, 0.125, 0.0625]
    Y = _few_bit_bf16(rng, (T * k, H), -12, 6)          # row r serves pair sorted_pairs[r]
    res = _few_bit_bf16(rng, (T, H), -2, 6)
    f = lambda v: int(mi.f32_to_bf16_bits(np.array([v], np.float32))[0])
    row = lambda j: pair_to_row[0 * k + j]
    # column 0: residual 1, pick 0 adds 0.75 float32 ulp of 1 (rounds up to one
    # ulp), pick 1 adds -1: forward order leaves 2^-23, reversed 1.5 * 2^-24
    res[0, 0] = f(1.0)
    Y[row(0), 0], Y[row(1), 0], Y[row(2), 0], Y[row(3), 0] = f(1.5 * 2.0 ** -23), f(-4.0), f(0.0), f(0.0)
    # column 1: the same with the -1 from the last pick (any single reordering shows)
    res[0, 1] = f(1.0)
    Y[row(0), 1], Y[row(1), 1], Y[row(2), 1], Y[row(3), 1] = f(1.5 * 2.0 ** -23), f(0.0), f(0.0), f(-16.0)
    return dict(T=T, H=H, k=k, ids=ids, sorted_pairs=sorted_pairs, pair_to_row=pair_to_row, g=g, Y=Y, res=res)


def _routed_terms(c, gate_of=None, row_map=None, order=None):
    T, k = c["T"], c["k"]
    gate_of = gate_of or (lambda t, j: c["g"][t, j])
    row_map = c["pair_to_row"] if row_map is None else row_map
    order = list(range(k)) if order is None else order
    Yf = _bf16_f64(c["Y"])
    terms = []
    for j in order:
        gj = np.array([[float(gate_of(t, j))] for t in range(T)])
        yj = np.stack([Yf[row_map[t * k + j]] for t in range(T)])
        terms.append((gj, yj))
    return terms


def test_combine_matches_an_exact_float32_chain(orc):
    """orc_combine, bit for bit, against the chain computed exactly step by step,
    with distinct rows per pick and unequal gates; and each plausible slip --
    picks in reverse order, a gate of the wrong pick or token, rows gathered
    through sorted_pairs instead of pair_to_row -- changes the bf16 output."""
    c = _combine_case()
    T, k = c["T"], c["k"]
    ref = _chain(c["res"], _routed_terms(c))
    got = orc.combine(c["Y"], c["pair_to_row"], c["g"], c["res"])
    assert np.array_equal(got, ref)
    assert got[0, 0] == mi.f32_to_bf16_bits(np.array([2.0 ** -23], np.float32))[0]
    slips = {
        "reversed picks": _routed_terms(c, order=list(range(k))[::-1]),
        "gate of the mirrored pick": _routed_terms(c, gate_of=lambda t, j: c["g"][t, k - 1 - j]),
        "gate of the next token": _routed_terms(c, gate_of=lambda t, j: c["g"][(t + 1) % T, j]),
        "rows through sorted_pairs": _routed_terms(c, row_map=c["sorted_pairs"]),
    }
    for name, terms in slips.items():
        assert not np.array_equal(_chain(c["res"], terms), ref), name
    # the reversal shows in the crafted columns of token 0 even where rows agree
    rev = _chain(c["res"], slips["reversed picks"])
    assert rev[0, 0] != ref[0, 0] and rev[0, 1] != ref[0, 1]


def test_combine_shared_matches_an_exact_float32_chain(orc):
    """orc_combine_shared: the routed chain, then the shared row's term last, bit
    for bit against the exact step-by-step chain; the shared term taken first,
    or with another token's gate, changes the output."""
    c = _combine_case(64)
    T, H = c["T"], c["H"]
    rng = np.random.default_rng(65)
    Ys = _few_bit_bf16(rng, (T, H), -12, 6)
    sg = (rng.choice(np.arange(1, 64), T, replace=False) / 64.0).astype(np.float32)
    # token 0, column 2: residual 1, pick 0 adds 0.75 ulp, the shared term -1
    f = lambda v: int(mi.f32_to_bf16_bits(np.array([v], np.float32))[0])
    k = c["k"]
    c["res"][0, 2] = f(1.0)
    for j in range(k):
        c["Y"][c["pair_to_row"][j], 2] = f(1.5 * 2.0 ** -23 if j == 0 else 0.0)
    sg[0] = 0.5
    Ys[0, 2] = f(-2.0)
    Ys[0, 0] = Ys[0, 1] = f(0.0)        # the routed crafted columns stay visible
    shared = (sg.astype(np.float64)[:, None], _bf16_f64(Ys))
    routed = _routed_terms(c)
    ref = _chain(c["res"], routed + [shared])
    got = orc.combine_shared(c["Y"], c["pair_to_row"], c["g"], Ys, sg, c["res"])
    assert np.array_equal(got, ref)
    first = _chain(c["res"], [shared] + routed)
    assert first[0, 2] != ref[0, 2]
    other = (np.roll(sg, -1).astype(np.float64)[:, None], _bf16_f64(Ys))
    assert not np.array_equal(_chain(c["res"], routed + [other]), ref)
    # the routed slips show through the shared chain as well
    T = c["T"]
    for name, terms in {
        "reversed picks": _routed_terms(c, order=list(range(k))[::-1]),
        "gate of the mirrored pick": _routed_terms(c, gate_of=lambda t, j: c["g"][t, k - 1 - j]),
        "gate of the next token": _routed_terms(c, gate_of=lambda t, j: c["g"][(t + 1) % T, j]),
        "rows through sorted_pairs": _routed_terms(c, row_map=c["sorted_pairs"]),
    }.items():
        assert not np.array_equal(_chain(c["res"], terms + [shared]), ref), name
