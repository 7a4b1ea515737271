"""Helpers for the GPU parity tests: upload seeded inputs, run each stage of the
layer through the C ABI, and compare with the oracle by the agreement rules.

Agreement rules (fixed before any kernel was written):
  * integer outputs (ids, slots, miss list, counts, offsets, permutation,
    active list) are bit-exact; ids are checked against the oracle's top-k of
    the GPU's own float32 logits, later integer stages against the oracle fed
    the GPU's ids;
  * logits: |d| <= 1e-5 * sum_h |x_h * Wr_eh| per element;
  * gates: |d| <= 2e-6 and |sum_j g_j - 1| <= 2e-6;
  * FFN rows Y and the layer output: max_rel <= 1e-2 and mae_norm <= 1e-3 with
    max_rel = max |a - b| / max(|b|, 1e-3 * rms(b)) and
    mae_norm = mean |a - b| / rms(b);
  * combine given identical Y and gates: bit-exact (same float32 FMA order).
"""
from __future__ import annotations

import dataclasses
import sys
from typing import Dict, List, Optional

import numpy as np
import torch

import moe_inputs as mi
import oracle
from work_tiles import expected_work_list
import quantized_expert_ffn_gemv_amd as moe

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to(DEV)


def to_host(t: torch.Tensor, dtype=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclasses.dataclass
class Layer:
    shape: mi.LayerShape
    bits: int
    seed: int
    Wr: np.ndarray
    bias: Optional[np.ndarray]
    table: np.ndarray
    Wr_d: torch.Tensor
    bias_d: Optional[torch.Tensor]
    table_d: torch.Tensor
    weights_d: moe.QWeights


def upload_layer(shape: mi.LayerShape, bits: int = 4, seed: int = 0) -> Layer:
    """Generate the full layer on the host one expert at a time and copy it to the GPU."""
    Wr, bias = mi.make_router(shape, seed)
    table = mi.make_slot_table(shape, seed)
    q, s, b = [], [], []
    for m in mi.MATRICES:
        N, K = mi.matrix_dims(shape, m)
        q.append(torch.empty((shape.E, K // 128, N, 16 * bits), dtype=torch.uint8, device=DEV))
        s.append(torch.empty((shape.E, N, K // shape.group), dtype=torch.int16, device=DEV))
        b.append(torch.empty((shape.E, N, K // shape.group), dtype=torch.int16, device=DEV))
    for e, mats in mi.iter_expert_weights(shape, bits, seed):
        for i, m in enumerate(mi.MATRICES):
            qq, ss, bb = mats[m]
            q[i][e].copy_(torch.from_numpy(moe.group_major(qq, bits)))
            s[i][e].copy_(torch.from_numpy(ss.view(np.int16)))
            b[i][e].copy_(torch.from_numpy(bb.view(np.int16)))
    return Layer(shape, bits, seed, Wr, bias, table, to_dev(Wr), None if bias is None else to_dev(bias),
                 to_dev(table), moe.QWeights(bits, q, s, b))


def poison_(t: torch.Tensor):
    """Fill an output buffer with a NaN/garbage pattern so unwritten entries show."""
    if t.dtype == torch.float32:
        t.fill_(float("nan"))
    elif t.dtype == torch.int16:
        t.fill_(0x7FC1)                  # a NaN bf16 pattern
    else:
        t.fill_(-7777)


def run_layer(L: Layer, xb: np.ndarray, res: np.ndarray, algo=moe.ALGO_AUTO, table: Optional[np.ndarray] = None,
              fused: bool = True):
    """All stages on the GPU; returns host copies of every output."""
    sh = L.shape
    T = xb.shape[0]
    d = moe.dims(T, sh.H, sh.I, sh.E, sh.k, sh.group)
    buf = moe.LayerBuffers.allocate(d, L.bits, algo)
    for name in ("logits", "topk_ids", "topk_w", "pair_slot", "miss", "counts", "offsets",
                 "sorted_pairs", "pair_to_row", "active", "work_list", "y_rows"):
        poison_(getattr(buf, name))
    x_d, r_d = to_dev(xb), to_dev(res)
    out_d = torch.empty_like(r_d)
    poison_(out_d)
    tab = L.table_d if table is None else to_dev(table)
    moe.layer_forward(buf, x_d, L.Wr_d, L.bias_d, L.weights_d, tab, sh.E, r_d, out_d, algo=algo, fused=fused)
    torch.cuda.synchronize()
    return host_outputs(buf, out_d, T * sh.k)


def host_outputs(buf, out_d: torch.Tensor, P: int) -> Dict:
    """Host copies of every output of a layer step (buffers `buf`, output out_d)."""
    return dict(
        logits=to_host(buf.logits), ids=to_host(buf.topk_ids), gates=to_host(buf.topk_w),
        pair_slot=to_host(buf.pair_slot)[:P], miss=to_host(buf.miss), n_miss=int(to_host(buf.n_miss)[0]),
        counts=to_host(buf.counts), offsets=to_host(buf.offsets), sorted_pairs=to_host(buf.sorted_pairs)[:P],
        pair_to_row=to_host(buf.pair_to_row)[:P], active=to_host(buf.active), n_active=int(to_host(buf.n_active)[0]),
        work_list=to_host(buf.work_list), n_work=int(to_host(buf.n_work)[0]),
        y_rows=to_host(buf.y_rows, np.uint16)[:P], out=to_host(out_d, np.uint16),
    )


# ------------------------------------------------------------ comparisons

def check_logits(g: Dict, L: Layer, xb: np.ndarray):
    x = bf16_to_f64(xb)
    ref = oracle.router_logits(xb, L.Wr, L.bias).astype(np.float64)
    bound = 1e-5 * (np.abs(x) @ np.abs(L.Wr.astype(np.float64)).T)
    err = np.abs(g["logits"].astype(np.float64) - ref)
    assert np.all(err <= bound + 1e-30), f"logits: worst ratio {np.max(err / (bound + 1e-30)):.3g}"
    return float(np.max(err / (bound + 1e-30)))


def check_topk(g: Dict, L: Layer):
    ids, gates = oracle.topk(g["logits"], L.shape.k, True)
    assert np.array_equal(g["ids"], ids), "top-k ids differ from the oracle on the GPU logits"
    assert np.max(np.abs(g["gates"] - gates)) <= 2e-6
    assert np.max(np.abs(g["gates"].astype(np.float64).sum(1) - 1.0)) <= 2e-6


def check_lookup(g: Dict, L: Layer, table=None):
    tab = L.table if table is None else table
    ref = oracle.slot_lookup(g["ids"], tab, L.shape.E)
    assert np.array_equal(g["pair_slot"], ref["pair_slot"])
    assert g["n_miss"] == ref["n_miss"]
    assert np.array_equal(g["miss"][: ref["n_miss"]], ref["miss"])


def check_permute(g: Dict, L: Layer):
    ref = oracle.permute(g["ids"], L.shape.E)
    for key in ("counts", "offsets", "sorted_pairs", "pair_to_row"):
        assert np.array_equal(g[key], ref[key]), key
    assert g["n_active"] == ref["n_active"]
    assert np.array_equal(g["active"][: ref["n_active"]], ref["active"])
    wl = expected_work_list(g["ids"], L.shape.E, L.shape.k, moe.WORK_TILE_ROWS)
    assert g["n_work"] == wl.shape[0]
    assert np.array_equal(g["work_list"][: wl.shape[0]], wl), "work list"


def tolerance_metrics(a_bits: np.ndarray, b_bits: np.ndarray):
    a, b = bf16_to_f64(a_bits), bf16_to_f64(b_bits)
    rms = float(np.sqrt(np.mean(b * b))) if b.size else 0.0
    if rms == 0.0:
        return (0.0 if np.array_equal(a, b) else np.inf), 0.0
    denom = np.maximum(np.abs(b), 1e-3 * rms)
    max_rel = float(np.max(np.abs(a - b) / denom))
    mae_norm = float(np.mean(np.abs(a - b)) / rms)
    return max_rel, mae_norm


def oracle_rows(g: Dict, L: Layer, xb: np.ndarray, rows: List[int], n_idx=None):
    """Oracle FFN for the listed sorted rows, fed the GPU's ids and permutation."""
    sh = L.shape
    ids = g["ids"].ravel()
    experts = sorted({int(ids[int(g['sorted_pairs'][r])]) for r in rows})
    W = mi.make_expert_weights(sh, L.bits, L.seed, experts=experts)
    _, ys = oracle.expert_ffn(xb, ids, g["sorted_pairs"], W, sh.k, rows=rows, n_idx=n_idx)
    return ys


def check_ffn(g: Dict, L: Layer, xb: np.ndarray, rows: Optional[List[int]] = None, n_idx=None):
    P = xb.shape[0] * L.shape.k
    rows = list(range(P)) if rows is None else rows
    ys = oracle_rows(g, L, xb, rows, n_idx)
    got = np.stack([g["y_rows"][r] if n_idx is None else g["y_rows"][r][n_idx] for r in rows])
    ref = np.stack([ys[r] for r in rows])
    max_rel, mae = tolerance_metrics(got, ref)
    assert max_rel <= 1e-2 and mae <= 1e-3, f"FFN rows: max_rel {max_rel:.3g}, mae_norm {mae:.3g}"
    return max_rel, mae


def check_combine_exact(g: Dict, L: Layer, res: np.ndarray):
    ref = oracle.combine(g["y_rows"], g["pair_to_row"], g["gates"], res)
    assert np.array_equal(g["out"], ref), "combine differs from the oracle given identical Y and gates"
