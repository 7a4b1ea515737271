"""CPU oracle for the routed MoE decode layer -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does.

The arithmetic lives in ``oracle.c`` (plain single-threaded C, double
accumulation); this module builds it with gcc and exposes each stage on numpy
arrays.  ``layer`` composes the stages end to end from raw inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

CFLAGS = ["-O2", "-std=c99", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, u32, f64 = ctypes.c_int32, ctypes.c_uint32, ctypes.c_double
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]; L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]; L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_f64_to_bf16.argtypes = [f64]; L.orc_f64_to_bf16.restype = ctypes.c_uint16
        L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]; L.orc_f16_to_f32.restype = ctypes.c_float
        L.orc_f64_to_f16.argtypes = [f64]; L.orc_f64_to_f16.restype = ctypes.c_uint16
        L.orc_zero_point_bias.argtypes = [ctypes.c_int64, P, P, P]; L.orc_zero_point_bias.restype = None
        L.orc_code.argtypes = [P, i32, i32]; L.orc_code.restype = i32
        L.orc_weight.argtypes = [P, P, P, i32, i32, i32]; L.orc_weight.restype = f64
        L.orc_dequant_matrix.argtypes = [i32, i32, i32, i32, P, P, P, P]; L.orc_dequant_matrix.restype = None
        L.orc_router_logits.argtypes = [i32, i32, i32, P, P, P, P]; L.orc_router_logits.restype = None
        L.orc_topk.argtypes = [i32, i32, i32, P, i32, P, P]; L.orc_topk.restype = None
        L.orc_slot_lookup.argtypes = [i32, i32, i32, P, P, P, P, P, P, u32, P]; L.orc_slot_lookup.restype = i32
        L.orc_permute.argtypes = [i32, i32, P, P, P, P, P, P, P]; L.orc_permute.restype = None
        L.orc_expert_ffn_row.argtypes = [i32, i32, i32, i32, P] + [P] * 9 + [i32, P, P, P]
        L.orc_expert_ffn_row.restype = None
        L.orc_combine.argtypes = [i32, i32, i32, P, P, P, P, P]; L.orc_combine.restype = None
        L.orc_shared_gate.argtypes = [i32, i32, P, P, P]; L.orc_shared_gate.restype = None
        L.orc_combine_shared.argtypes = [i32, i32, i32] + [P] * 7; L.orc_combine_shared.restype = None
        L.orc_freq_update.argtypes = [i32, P, P]; L.orc_freq_update.restype = None
        L.orc_hot_set.argtypes = [i32, P, i32, P]; L.orc_hot_set.restype = None
        L.orc_warm_ring_step.argtypes = [i32, i32, P, i32, u32, P, P, P, P, P]; L.orc_warm_ring_step.restype = i32
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------ formats

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    L = lib()
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([L.orc_bf16_to_f32(int(v)) for v in flat], dtype=np.float32).reshape(np.shape(bits))


def f16_to_f32(bits: np.ndarray) -> np.ndarray:
    L = lib()
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([L.orc_f16_to_f32(int(v)) for v in flat], dtype=np.float32).reshape(np.shape(bits))


def f32_to_bf16(vals) -> np.ndarray:
    L = lib()
    flat = np.asarray(vals, dtype=np.float32).ravel()
    return np.array([L.orc_f32_to_bf16(float(v)) for v in flat], dtype=np.uint16).reshape(np.shape(vals))


def f64_to_bf16(vals) -> np.ndarray:
    L = lib()
    flat = np.asarray(vals, dtype=np.float64).ravel()
    return np.array([L.orc_f64_to_bf16(float(v)) for v in flat], dtype=np.uint16).reshape(np.shape(vals))


def f64_to_f16(vals) -> np.ndarray:
    """IEEE binary16 bit patterns of float64 values, one rounding (nearest, ties to even)."""
    L = lib()
    flat = np.asarray(vals, dtype=np.float64).ravel()
    return np.array([L.orc_f64_to_f16(float(v)) for v in flat], dtype=np.uint16).reshape(np.shape(vals))


def zero_point_bias(scale: np.ndarray, zeros: np.ndarray) -> np.ndarray:
    """fp16 bias bits b = -(z s) per group for zero-point weights w = (q - z) s,
    so that q s + b is the same weight up to b's one rounding."""
    scale, zeros = _c(scale, np.uint16), _c(zeros, np.uint8)
    if scale.shape != zeros.shape:
        raise ValueError("scale and zeros must have one entry per group each")
    out = np.empty(scale.shape, dtype=np.uint16)
    lib().orc_zero_point_bias(int(scale.size), _p(scale), _p(zeros), _p(out))
    return out


def code(row: np.ndarray, k: int, bits: int) -> int:
    row = _c(row, np.uint8)
    return int(lib().orc_code(_p(row), k, bits))


def group_of(K: int, scale: np.ndarray) -> int:
    """Group size of a matrix with reduction length K and scales [..., K/group]."""
    ng = int(np.asarray(scale).shape[-1])
    if ng <= 0 or K % ng or K // ng not in (32, 64, 128):
        raise ValueError(f"{ng} scales per row of {K} do not make groups of 32, 64 or 128")
    return K // ng


def dequant_matrix(q: np.ndarray, scale: np.ndarray, bias: np.ndarray, bits: int) -> np.ndarray:
    """Dense float64 [N, K] weights of one packed matrix (group size from the
    scales' shape)."""
    q, scale, bias = _c(q, np.uint8), _c(scale, np.uint16), _c(bias, np.uint16)
    N = q.shape[0]
    K = q.shape[1] * 8 // bits
    out = np.empty((N, K), dtype=np.float64)
    lib().orc_dequant_matrix(N, K, bits, group_of(K, scale), _p(q), _p(scale), _p(bias), _p(out))
    return out


# ------------------------------------------------------------------- stages

def router_logits(x_bits: np.ndarray, Wr: np.ndarray, bias: Optional[np.ndarray]) -> np.ndarray:
    x_bits, Wr = _c(x_bits, np.uint16), _c(Wr, np.float32)
    bias = None if bias is None else _c(bias, np.float32)
    T, H = x_bits.shape
    E = Wr.shape[0]
    out = np.empty((T, E), dtype=np.float32)
    lib().orc_router_logits(T, H, E, _p(x_bits), _p(Wr), _p(bias), _p(out))
    return out


def topk(logits: np.ndarray, k: int, renormalize: bool = True):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    gates = np.empty((T, k), dtype=np.float32)
    lib().orc_topk(T, E, k, _p(logits), int(bool(renormalize)), _p(ids), _p(gates))
    return ids, gates


def slot_lookup(ids: np.ndarray, slot_of_expert: np.ndarray, n_slots: int,
                last_use: Optional[np.ndarray] = None, step: int = 0, doorbell: Optional[int] = None):
    """Returns dict(pair_slot, miss, n_miss, last_use, doorbell)."""
    ids = _c(ids, np.int32).ravel()
    table = _c(slot_of_expert, np.int32)
    E = table.shape[0]
    P = ids.shape[0]
    pair_slot = np.empty(P, dtype=np.int32)
    miss = np.zeros(E, dtype=np.int32)
    n_miss = np.zeros(1, dtype=np.int32)
    lu = None if last_use is None else np.array(last_use, dtype=np.uint32, copy=True)
    bell = None if doorbell is None else np.array([doorbell], dtype=np.int32)
    lib().orc_slot_lookup(P, E, int(n_slots), _p(ids), _p(table), _p(pair_slot), _p(miss),
                          _p(n_miss), _p(lu), int(step), _p(bell))
    nm = int(n_miss[0])
    return dict(pair_slot=pair_slot, miss=miss[:nm].copy(), n_miss=nm, last_use=lu,
                doorbell=None if bell is None else int(bell[0]))


def permute(ids: np.ndarray, E: int):
    """Returns dict(counts, offsets, sorted_pairs, pair_to_row, active, n_active)."""
    ids = _c(ids, np.int32).ravel()
    P = ids.shape[0]
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    sp = np.empty(P, dtype=np.int32)
    p2r = np.empty(P, dtype=np.int32)
    active = np.zeros(E, dtype=np.int32)
    n_active = np.zeros(1, dtype=np.int32)
    lib().orc_permute(P, E, _p(ids), _p(counts), _p(offsets), _p(sp), _p(p2r), _p(active), _p(n_active))
    na = int(n_active[0])
    return dict(counts=counts, offsets=offsets, sorted_pairs=sp, pair_to_row=p2r,
                active=active[:na].copy(), n_active=na)


def expert_ffn_row(x_row: np.ndarray, w: Dict[str, Sequence[np.ndarray]], bits: int,
                   n_idx: Optional[np.ndarray] = None):
    """FFN of one expert on one token.  w[m] = (q [N, K*bits/8], scale, bias);
    the group size follows from the scales' shape.

    Returns (h float32 [I], y bf16 bits [H] or [len(n_idx)])."""
    x_row = _c(x_row, np.uint16)
    qg, sg, bg = (_c(a, t) for a, t in zip(w["gate"], (np.uint8, np.uint16, np.uint16)))
    qu, su, bu = (_c(a, t) for a, t in zip(w["up"], (np.uint8, np.uint16, np.uint16)))
    qd, sd, bd = (_c(a, t) for a, t in zip(w["down"], (np.uint8, np.uint16, np.uint16)))
    H = x_row.shape[0]
    I = qg.shape[0]
    group = group_of(H, sg)
    if group_of(I, sd) != group:
        raise ValueError("gate/up and down weights have different group sizes")
    h = np.empty(I, dtype=np.float32)
    if n_idx is None:
        y = np.empty(H, dtype=np.uint16)
        lib().orc_expert_ffn_row(H, I, bits, group, _p(x_row), _p(qg), _p(sg), _p(bg), _p(qu), _p(su), _p(bu),
                                 _p(qd), _p(sd), _p(bd), 0, None, _p(h), _p(y))
    else:
        n_idx = _c(n_idx, np.int32)
        y = np.empty(n_idx.shape[0], dtype=np.uint16)
        lib().orc_expert_ffn_row(H, I, bits, group, _p(x_row), _p(qg), _p(sg), _p(bg), _p(qu), _p(su), _p(bu),
                                 _p(qd), _p(sd), _p(bd), int(n_idx.shape[0]), _p(n_idx), _p(h), _p(y))
    return h, y


def expert_weights_of(weights, e: int) -> Dict[str, tuple]:
    """Slice one expert out of an ExpertWeights-like object."""
    i = weights.index_of(e)
    return {m: (weights.q[m][i], weights.scale[m][i], weights.bias[m][i]) for m in ("gate", "up", "down")}


def expert_ffn(x_bits: np.ndarray, ids: np.ndarray, sorted_pairs: np.ndarray, weights, k: int,
               rows: Optional[Sequence[int]] = None, n_idx: Optional[np.ndarray] = None):
    """FFN for routed rows in sorted order.  Row r serves pair sorted_pairs[r]
    (token sorted_pairs[r] // k, expert ids.flat[sorted_pairs[r]]).

    rows=None computes every row; otherwise only the listed ones.
    Returns (h dict r -> float32 [I], y dict r -> bf16 bits)."""
    ids = np.asarray(ids).ravel()
    x_bits = np.asarray(x_bits)
    todo = range(len(sorted_pairs)) if rows is None else rows
    hs, ys = {}, {}
    for r in todo:
        p = int(sorted_pairs[r])
        e = int(ids[p])
        hs[r], ys[r] = expert_ffn_row(x_bits[p // k], expert_weights_of(weights, e), weights.bits, n_idx)
    return hs, ys


def combine(y_rows: np.ndarray, pair_to_row: np.ndarray, gates: np.ndarray, residual: np.ndarray) -> np.ndarray:
    y_rows, residual = _c(y_rows, np.uint16), _c(residual, np.uint16)
    p2r, gates = _c(pair_to_row, np.int32), _c(gates, np.float32)
    T, H = residual.shape
    k = gates.shape[1]
    out = np.empty((T, H), dtype=np.uint16)
    lib().orc_combine(T, H, k, _p(y_rows), _p(p2r), _p(gates), _p(residual), _p(out))
    return out


def shared_gate(x_bits: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Sigmoid gate of the shared expert per token: float32 [T]."""
    x_bits, w = _c(x_bits, np.uint16), _c(w, np.float32)
    T, H = x_bits.shape
    if w.shape != (H,):
        raise ValueError("the gate weight has one entry per hidden unit")
    out = np.empty(T, dtype=np.float32)
    lib().orc_shared_gate(T, H, _p(x_bits), _p(w), _p(out))
    return out


def combine_shared(y_rows: np.ndarray, pair_to_row: np.ndarray, gates: np.ndarray, y_shared: np.ndarray,
                   sgate: np.ndarray, residual: np.ndarray) -> np.ndarray:
    """combine(), then + sgate[t] * y_shared[t] as one more float32 FMA, rounded once to bf16."""
    y_rows, residual, y_shared = _c(y_rows, np.uint16), _c(residual, np.uint16), _c(y_shared, np.uint16)
    p2r, gates, sgate = _c(pair_to_row, np.int32), _c(gates, np.float32), _c(sgate, np.float32)
    T, H = residual.shape
    k = gates.shape[1]
    if y_shared.shape != (T, H) or sgate.shape != (T,):
        raise ValueError("y_shared must be [T, H] and sgate [T]")
    out = np.empty((T, H), dtype=np.uint16)
    lib().orc_combine_shared(T, H, k, _p(y_rows), _p(p2r), _p(gates), _p(y_shared), _p(sgate), _p(residual),
                             _p(out))
    return out


# --------------------------------------------------------- residency tiers

def freq_update(counts: np.ndarray, freq: np.ndarray) -> np.ndarray:
    """Routing-frequency counters after one call: freq + counts (uint32)."""
    counts = _c(counts, np.int32)
    out = np.array(freq, dtype=np.uint32, copy=True)
    lib().orc_freq_update(int(counts.shape[0]), _p(counts), _p(out))
    return out


def hot_set(freq: np.ndarray, n: int) -> np.ndarray:
    """The n most routed experts, most used first, ties to the lower id."""
    freq = _c(freq, np.uint32)
    out = np.empty(n, dtype=np.int32)
    lib().orc_hot_set(int(freq.shape[0]), _p(freq), int(n), _p(out))
    return out


def warm_ring_step(n_hot: int, miss: np.ndarray, step: int, slot_of_expert: np.ndarray,
                   expert_of_slot: np.ndarray, last_use: np.ndarray):
    """One step of the LRU warm ring for this step's missing experts (ascending).
    Returns dict(slot_of_expert, expert_of_slot, last_use, copies [(expert, slot)])
    with new arrays (the inputs are not modified)."""
    miss = _c(miss, np.int32)
    soe = np.array(slot_of_expert, dtype=np.int32, copy=True)
    eos = np.array(expert_of_slot, dtype=np.int32, copy=True)
    lu = np.array(last_use, dtype=np.uint32, copy=True)
    n_slots = int(eos.shape[0])
    ce = np.zeros(max(n_slots, 1), np.int32)
    cs = np.zeros(max(n_slots, 1), np.int32)
    n = lib().orc_warm_ring_step(int(n_hot), n_slots, _p(miss), int(miss.shape[0]), int(step) & 0xFFFFFFFF,
                                 _p(soe), _p(eos), _p(lu), _p(ce), _p(cs))
    return dict(slot_of_expert=soe, expert_of_slot=eos, last_use=lu,
                copies=[(int(ce[i]), int(cs[i])) for i in range(n)])


def layer(x_bits, Wr, router_bias, weights, k: int, slot_of_expert, n_slots: int, residual,
          renormalize: bool = True):
    """End-to-end layer from raw inputs; returns every intermediate."""
    T, H = np.asarray(x_bits).shape
    E = np.asarray(Wr).shape[0]
    logits = router_logits(x_bits, Wr, router_bias)
    ids, gates = topk(logits, k, renormalize)
    look = slot_lookup(ids, slot_of_expert, n_slots)
    perm = permute(ids, E)
    hs, ys = expert_ffn(x_bits, ids, perm["sorted_pairs"], weights, k)
    y_rows = np.stack([ys[r] for r in range(T * k)]) if T * k else np.zeros((0, H), np.uint16)
    out = combine(y_rows, perm["pair_to_row"], gates, residual)
    return dict(logits=logits, ids=ids, gates=gates, lookup=look, perm=perm,
                h=hs, y_rows=y_rows, out=out)
