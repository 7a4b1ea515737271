"""Seeded synthetic inputs for the routed MoE decode layer.

This module is shared by the oracle tests, the GPU parity tests and the bench.
It only draws random numbers and lays them out in the storage formats the
layer consumes (bf16 / fp16 bit patterns, packed low-bit codes).  It contains
none of the layer's arithmetic: no routing, no dequantisation, no matvec.

Workload shapes follow the pages' models (see the shape table in ``CONFIGS``):
an A3B-style layer (256 experts, ~8 routed, page 3 "Background"), a 64-expert
top-2 layer (page 2 section 1.1), a 512-expert top-4 layer with ~6.75 MB
experts (page 5 "SSD expert streaming"), plus a tiny correctness shape and a
4096-token prefill shape.

Storage formats (fixed for the whole library):
  * activations / residual: bf16 bit patterns, uint16 [T, H], row-major;
  * router weight: float32 [E, H]; router bias: float32 [E] (or None);
  * expert weights: for matrix m in (gate, up, down) an array
      q[m]     uint8  [E, N, K*bits/8]  codes packed along K; for 4-bit the low
               nibble holds the even k, for 2-bit bits 2j..2j+1 of a byte hold
               k % 4 == j;
      scale[m] uint16 [E, N, K/group]   fp16 bit patterns;
      bias[m]  uint16 [E, N, K/group]   fp16 bit patterns;
    with (N, K) = (I, H) for gate and up and (H, I) for down.  The dequantised
    weight is code * scale + bias of the element's group along K, 128 wide
    by default (page 2 section 2.2 for the group of 128; 64 and 32 from the
    finer-group passages: page 2 section 4.4, the laptop page section 4.2;
    page 5 section 2 for the nibble*scale+bias form).

Random draws: every tensor has its own ``numpy.random.Generator`` (PCG64)
seeded from ``SeedSequence([seed, tag, ...])`` so that any expert can be
regenerated on its own, e.g. by the oracle for the experts it needs.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

GROUP = 128
MATRICES = ("gate", "up", "down")

# tags of the independent random streams
_TAG_X, _TAG_RES, _TAG_WR, _TAG_PERM, _TAG_Q, _TAG_S, _TAG_B, _TAG_Z, _TAG_SG, _TAG_SV = 1, 2, 3, 4, 5, 6, 7, 8, 9, 10


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """Shape of one routed-MoE layer and its workload."""
    name: str
    H: int            # hidden size
    E: int            # routed experts
    k: int            # experts per token
    I: int            # expert intermediate size
    tokens: Tuple[int, ...]   # token counts the workload is run at
    bits: Tuple[int, ...]     # weight code widths exercised
    zipf_s: Optional[float]   # Zipf exponent of expert popularity; None = uniform
    n_resident: int           # experts marked resident in the slot table
    description: str = ""
    group: int = GROUP        # quantisation group along K: 128, 64 or 32

    def bytes_per_expert(self, bits: int) -> int:
        """Bytes of one expert's three matrices: codes plus fp16 scale and bias."""
        per_matrix = self.H * self.I * bits // 8 + (self.H * self.I // self.group) * 4
        return 3 * per_matrix


def _resident_60(E: int) -> int:
    return int(math.floor(0.6 * E + 0.5))


CONFIGS: Dict[str, LayerShape] = {
    "tiny": LayerShape("tiny", H=256, E=8, k=2, I=512, tokens=(4,), bits=(4,),
                       zipf_s=None, n_resident=_resident_60(8),
                       description="tiny MoE layer, 4 tokens"),
    "a3b": LayerShape("a3b", H=2048, E=256, k=8, I=512, tokens=(1, 8, 32), bits=(4,),
                      zipf_s=1.1, n_resident=_resident_60(256),
                      description="A3B-style decode layer, 256 experts top-8"),
    "e64": LayerShape("e64", H=5120, E=64, k=2, I=8192, tokens=(8,), bits=(4,),
                      zipf_s=1.2, n_resident=24,
                      description="64-expert top-2 layer, hidden 5120, continuous-batch decode"),
    "e512": LayerShape("e512", H=4096, E=512, k=4, I=1024, tokens=(1,), bits=(4, 2),
                       zipf_s=None, n_resident=_resident_60(512),
                       description="512-expert top-4 layer, single-token decode"),
    "prefill": LayerShape("prefill", H=2048, E=128, k=8, I=768, tokens=(4096,), bits=(4,),
                          zipf_s=1.0, n_resident=_resident_60(128),
                          description="prefill / large-batch layer, 4096 tokens"),
}
CONFIG_ORDER = ("tiny", "a3b", "e64", "e512", "prefill")


def _rng(seed: int, *keys: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed)] + [int(v) for v in keys]))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even) and return the bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        rounded = rounded.copy()
        rounded[nan] = 0x7FC0
    return rounded


def f32_to_f16_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32).astype(np.float16)).view(np.uint16)


def make_activations(H: int, T: int, seed: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """x and residual, both N(0,1) rounded to bf16; uint16 [T, H]."""
    x = _rng(seed, _TAG_X, T, H).standard_normal((T, H), dtype=np.float32)
    r = _rng(seed, _TAG_RES, T, H).standard_normal((T, H), dtype=np.float32)
    return f32_to_bf16_bits(x), f32_to_bf16_bits(r)


def make_spec_verify_activations(H: int, n_seq: int, n_draft: int = 4, seed: int = 0,
                                 rho: float = 0.8) -> Tuple[np.ndarray, np.ndarray]:
    """A speculative-verify batch: n_seq sequences of n_draft draft tokens each,
    token (b, d) at row b * n_draft + d, x = rho * base_b + sqrt(1 - rho^2) * noise
    (unit variance, correlation rho between the drafts of one sequence, none
    across sequences), so the drafts of a sequence tend to pick the same experts.
    Returns (x, residual) as bf16 bits [n_seq * n_draft, H]."""
    T = n_seq * n_draft
    base = _rng(seed, _TAG_SV, 0, n_seq, H).standard_normal((n_seq, H), dtype=np.float32)
    noise = _rng(seed, _TAG_SV, 1, T, H).standard_normal((T, H), dtype=np.float32)
    x = rho * np.repeat(base, n_draft, axis=0) + np.float32(math.sqrt(1.0 - rho * rho)) * noise
    r = _rng(seed, _TAG_RES, T, H).standard_normal((T, H), dtype=np.float32)
    return f32_to_bf16_bits(x.astype(np.float32)), f32_to_bf16_bits(r)


def expert_popularity(shape: LayerShape, seed: int = 0) -> np.ndarray:
    """Intended share of routing picks per expert (sums to 1).

    Zipf(s): the expert of popularity rank r (1-based) gets weight r^-s; ranks are
    assigned to expert ids by a seeded permutation.  Uniform when zipf_s is None.
    """
    E = shape.E
    if shape.zipf_s is None:
        return np.full(E, 1.0 / E)
    perm = _rng(seed, _TAG_PERM, E).permutation(E)       # perm[rank-1] = expert id
    w = np.arange(1, E + 1, dtype=np.float64) ** (-shape.zipf_s)
    p = np.empty(E)
    p[perm] = w / w.sum()
    return p


def popularity_order(shape: LayerShape, seed: int = 0) -> np.ndarray:
    """Expert ids from most to least popular (ties: lower id first)."""
    p = expert_popularity(shape, seed)
    if shape.zipf_s is None:
        return _rng(seed, _TAG_PERM, shape.E).permutation(shape.E)
    return np.lexsort((np.arange(shape.E), -p))


def make_router(shape: LayerShape, seed: int = 0) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """Router weight N(0, 0.02) float32 [E, H] and the popularity bias (None if uniform).

    The bias b_e = beta * ln p_e with beta = sigma * sqrt(6) / pi, where
    sigma = 0.02 * sqrt(H) is the spread of an unbiased logit.  This scales the
    logit noise to a unit-scale Gumbel so that picks follow p_e approximately.
    """
    Wr = (_rng(seed, _TAG_WR, shape.E, shape.H).standard_normal((shape.E, shape.H), dtype=np.float32)
          * np.float32(0.02)).astype(np.float32)
    if shape.zipf_s is None:
        return Wr, None
    p = expert_popularity(shape, seed)
    beta = 0.02 * math.sqrt(shape.H) * math.sqrt(6.0) / math.pi
    return Wr, (beta * np.log(p)).astype(np.float32)


def make_slot_table(shape: LayerShape, seed: int = 0, n_resident: Optional[int] = None) -> np.ndarray:
    """slot_of_expert int32 [E]: the n most popular experts get slots 0..n-1 in
    popularity order, the rest -1 (not resident)."""
    n = shape.n_resident if n_resident is None else n_resident
    order = popularity_order(shape, seed)
    table = np.full(shape.E, -1, dtype=np.int32)
    table[order[:n]] = np.arange(n, dtype=np.int32)
    return table


def matrix_dims(shape: LayerShape, m: str) -> Tuple[int, int]:
    """(N, K) of matrix m: output rows and reduction length."""
    return (shape.I, shape.H) if m in ("gate", "up") else (shape.H, shape.I)


def _draw_expert_matrix(shape: LayerShape, m: str, e: int, bits: int, seed: int):
    N, K = matrix_dims(shape, m)
    mi = MATRICES.index(m)
    nbytes = N * K * bits // 8
    raw = _rng(seed, _TAG_Q, bits, mi, e).bit_generator.random_raw((nbytes + 7) // 8)
    # every byte is 8/bits independent uniform codes in 0..2^bits-1
    q = raw.view(np.uint8)[:nbytes].reshape(N, K * bits // 8)
    ng = K // shape.group
    s = _rng(seed, _TAG_S, bits, mi, e).uniform(0.005, 0.02, size=(N, ng))
    b = _rng(seed, _TAG_B, bits, mi, e).normal(0.0, 0.01, size=(N, ng))
    return q, f32_to_f16_bits(s), f32_to_f16_bits(b)


@dataclasses.dataclass
class ExpertWeights:
    """Packed weights of some experts of one layer (host numpy arrays)."""
    bits: int
    experts: np.ndarray                     # expert ids held, in storage order
    q: Dict[str, np.ndarray]                # m -> uint8 [n, N, K*bits/8]
    scale: Dict[str, np.ndarray]            # m -> uint16 [n, N, K/group]
    bias: Dict[str, np.ndarray]             # m -> uint16 [n, N, K/group]

    def index_of(self, e: int) -> int:
        hit = np.nonzero(self.experts == e)[0]
        if hit.size == 0:
            raise KeyError(f"expert {e} not generated")
        return int(hit[0])


def make_expert_weights(shape: LayerShape, bits: int = 4, seed: int = 0,
                        experts: Optional[Iterable[int]] = None) -> ExpertWeights:
    """Packed weights for the listed experts (all experts when None)."""
    if bits not in (2, 4):
        raise ValueError("bits must be 2 or 4")
    ids = np.arange(shape.E) if experts is None else np.asarray(sorted(set(int(e) for e in experts)), dtype=np.int64)
    q, s, b = {}, {}, {}
    for m in MATRICES:
        N, K = matrix_dims(shape, m)
        q[m] = np.empty((len(ids), N, K * bits // 8), dtype=np.uint8)
        s[m] = np.empty((len(ids), N, K // shape.group), dtype=np.uint16)
        b[m] = np.empty((len(ids), N, K // shape.group), dtype=np.uint16)
        for i, e in enumerate(ids):
            q[m][i], s[m][i], b[m][i] = _draw_expert_matrix(shape, m, int(e), bits, seed)
    return ExpertWeights(bits=bits, experts=np.asarray(ids), q=q, scale=s, bias=b)


def iter_expert_weights(shape: LayerShape, bits: int = 4, seed: int = 0):
    """Yield (e, {m: (q, scale, bias)}) one expert at a time (bounded host memory)."""
    for e in range(shape.E):
        yield e, {m: _draw_expert_matrix(shape, m, e, bits, seed) for m in MATRICES}


def make_zero_points(shape: LayerShape, m: str, e: int, bits: int = 4, seed: int = 0) -> np.ndarray:
    """Zero points of matrix m of expert e for zero-point weights (q - z) s:
    uint8 [N][K/group], uniform over the codes 0 .. 2^bits - 1."""
    N, K = matrix_dims(shape, m)
    return _rng(seed, _TAG_Z, bits, MATRICES.index(m), e).integers(0, 1 << bits, size=(N, K // shape.group),
                                                                    dtype=np.uint8)


def make_shared_expert(shape: LayerShape, bits: int = 4, seed: int = 0, I: Optional[int] = None):
    """An always-on shared expert for `shape`: (its one-expert LayerShape of
    intermediate size I, {m: (q, scale, bias)} drawn like a routed expert's but
    from streams keyed past the routed experts, its gate's weight row fp32 [H]
    ~ N(0, 0.02^2), the router's scale, so that x . w spreads the sigmoid over
    (0, 1))."""
    one = dataclasses.replace(shape, name=shape.name + "_shared", E=1, k=1, I=shape.I if I is None else int(I),
                              n_resident=1)
    mats = {m: _draw_expert_matrix(one, m, shape.E, bits, seed) for m in MATRICES}
    w = (_rng(seed, _TAG_SG, shape.H).standard_normal(shape.H) * 0.02).astype(np.float32)
    return one, mats, w


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack integer codes [..., K] into bytes along the last axis (format above)."""
    codes = np.asarray(codes, dtype=np.uint8)
    per = 8 // bits
    if codes.shape[-1] % per:
        raise ValueError("K must be a multiple of codes per byte")
    c = codes.reshape(codes.shape[:-1] + (codes.shape[-1] // per, per)).astype(np.uint16)
    out = np.zeros(c.shape[:-1], dtype=np.uint16)
    for j in range(per):
        out |= c[..., j] << (bits * j)
    return out.astype(np.uint8)


__all__ = [
    "GROUP", "MATRICES", "LayerShape", "CONFIGS", "CONFIG_ORDER", "ExpertWeights",
    "make_activations", "make_router", "make_slot_table", "make_expert_weights",
    "iter_expert_weights", "make_zero_points", "make_shared_expert", "make_spec_verify_activations", "expert_popularity", "popularity_order", "matrix_dims",
    "pack_codes", "f32_to_bf16_bits", "f32_to_f16_bits",
]
