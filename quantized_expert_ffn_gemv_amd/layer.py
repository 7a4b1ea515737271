"""One routed-MoE layer step as a fixed sequence of library calls.

``LayerBuffers`` preallocates every intermediate once (logits, picks, slot
lookup results, permutation, workspace, expert outputs) so that a step is three
C calls on one stream with no allocation and no host synchronisation:

    route_dispatch (route_topk + slot_lookup + permute) -> expert_ffn_fused -> combine

``fused=False`` makes the same step from the separate routing calls and the
two-launch FFN (expert_ffn_q{4,2}).

With a shared expert (``SharedExpert``: one more quantised FFN that every token
uses, scaled by a per-token sigmoid gate) ``combine_shared`` replaces
``combine``, and its FFN runs either
  * inside the routed FFN launch (``expert_ffn_fused_shared``), when its weights
    are given as the last of E + 1 experts (``fused_weights``) and the buffers
    were allocated with ``shared_rows``; or
  * as a launch of its own before the routing, a one-expert layer whose work
    list (every token on expert 0) depends only on T and is built once, when
    ``SharedBuffers`` are allocated.  (A second stream measured slower here:
    the cross-stream event wait held the host for the whole step.)

This module only orders the calls; the arithmetic is in the HIP kernels.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import (ALGO_AUTO, DISPATCH_SYNC_INTS, FFN_SYNC_INTS, OP_FFN, WORK_ENTRY_INTS, Dims, QWeights, combine,
               combine_shared, dims, expert_ffn_fused, expert_ffn_fused_shared, expert_ffn_q2, expert_ffn_q4, permute, route_dispatch,
               route_topk, slot_lookup, work_list_capacity, workspace_bytes)


@dataclass
class LayerBuffers:
    d: Dims
    bits: int
    logits: torch.Tensor          # float32 [T, E]
    topk_ids: torch.Tensor        # int32 [T, k]
    topk_w: torch.Tensor          # float32 [T, k]
    pair_slot: torch.Tensor       # int32 [T*k]
    miss: torch.Tensor            # int32 [E]
    n_miss: torch.Tensor          # int32 [1]
    counts: torch.Tensor          # int32 [E]
    offsets: torch.Tensor         # int32 [E+1]
    sorted_pairs: torch.Tensor    # int32 [T*k]
    pair_to_row: torch.Tensor     # int32 [T*k]
    active: torch.Tensor          # int32 [E]
    n_active: torch.Tensor        # int32 [1]
    work_list: torch.Tensor       # int32 [capacity, WORK_ENTRY_INTS]
    n_work: torch.Tensor          # int32 [1]
    workspace: torch.Tensor       # uint8, 256-byte aligned by the allocator
    y_rows: torch.Tensor          # bf16 bits as int16 [T*k, H]
    sync: torch.Tensor            # int32 [DISPATCH_SYNC_INTS], zeros (route_dispatch's counters)
    ffn_sync: torch.Tensor        # int32 [FFN_SYNC_INTS], zeros (expert_ffn_fused's counters)
    shared_rows: bool = False     # y_rows and workspace also hold a shared expert's T rows

    @staticmethod
    def allocate(d: Dims, bits: int = 4, algo: int = ALGO_AUTO, device="cuda",
                 shared_rows: bool = False) -> "LayerBuffers":
        T, H, E, k = d.T, d.H, d.E, d.k
        i32 = dict(dtype=torch.int32, device=device)
        ws = workspace_bytes(dims(T, H, d.I, E + 1, k + 1) if shared_rows else d, OP_FFN, bits, algo)
        rows = T * (k + 1) if shared_rows else T * k
        cap = work_list_capacity(d)
        return LayerBuffers(
            d=d, bits=bits,
            logits=torch.empty((T, E), dtype=torch.float32, device=device),
            topk_ids=torch.empty((T, k), **i32),
            topk_w=torch.empty((T, k), dtype=torch.float32, device=device),
            pair_slot=torch.empty((T * k,), **i32),
            miss=torch.empty((E,), **i32),
            n_miss=torch.zeros((1,), **i32),
            counts=torch.empty((E,), **i32),
            offsets=torch.empty((E + 1,), **i32),
            sorted_pairs=torch.empty((max(T * k, 1),), **i32),
            pair_to_row=torch.empty((max(T * k, 1),), **i32),
            active=torch.empty((E,), **i32),
            n_active=torch.zeros((1,), **i32),
            work_list=torch.empty((max(cap, 1), WORK_ENTRY_INTS), **i32),
            n_work=torch.zeros((1,), **i32),
            workspace=torch.empty((max(ws, 256),), dtype=torch.uint8, device=device),
            y_rows=torch.empty((max(rows, 1), H), dtype=torch.int16, device=device),
            sync=torch.zeros((DISPATCH_SYNC_INTS,), **i32),
            ffn_sync=torch.zeros((FFN_SYNC_INTS,), **i32),
            shared_rows=shared_rows,
        )


@dataclass
class SharedExpert:
    """An always-on shared expert: a quantised FFN of intermediate size I (one
    expert, the library's weight format) and its sigmoid gate's weight row."""
    weights: QWeights             # one expert: q[m] [1][K/128][N][16*bits], scale / bias [1][N][K/128]
    gate_w: torch.Tensor          # float32 [H]
    I: int
    fused_weights: Optional[QWeights] = None   # the routed experts, then this one (E + 1): one FFN launch


@dataclass
class SharedBuffers:
    d: Dims                       # (T, H, I_shared, E = 1, k = 1)
    buf: LayerBuffers             # the one-expert layer's work list, workspace, rows and counters
    zeros: torch.Tensor           # int32 [T]: every token picks expert 0
    gate_out: torch.Tensor        # float32 [T]: the gate values the last combine used

    @staticmethod
    def allocate(T: int, H: int, I: int, bits: int = 4, algo: int = ALGO_AUTO, device="cuda") -> "SharedBuffers":
        d = dims(T, H, I, 1, 1)
        buf = LayerBuffers.allocate(d, bits, algo, device)
        zeros = torch.zeros((max(T, 1),), dtype=torch.int32, device=device)
        permute(d, zeros, buf.counts, buf.offsets, buf.sorted_pairs, buf.pair_to_row, buf.active, buf.n_active,
                buf.work_list, buf.n_work)
        return SharedBuffers(d=d, buf=buf, zeros=zeros,
                             gate_out=torch.empty((max(T, 1),), dtype=torch.float32, device=device))


def layer_forward(buf: LayerBuffers, x: torch.Tensor, w_router: torch.Tensor,
                  router_bias: Optional[torch.Tensor], weights: QWeights,
                  slot_of_expert: torch.Tensor, n_slots: int, residual: torch.Tensor,
                  out: torch.Tensor, algo: int = ALGO_AUTO, renormalize: bool = True,
                  host_doorbell=None, last_use=None, step: int = 0, stream=None, fused: bool = True,
                  shared: Optional[SharedExpert] = None, shared_buf: Optional[SharedBuffers] = None) -> None:
    """Enqueue one layer step; `out` may be `residual`.  With `shared`, the
    combine adds the shared expert's gated rows; its FFN runs inside the routed
    FFN launch when shared.fused_weights is set (buffers with shared_rows;
    `shared_buf`, if given, only receives the gate values), else first, as its
    own launch on `shared_buf`."""
    d = buf.d
    one_launch = shared is not None and shared.fused_weights is not None
    if one_launch and not buf.shared_rows:
        raise ValueError("the one-launch shared expert needs LayerBuffers allocated with shared_rows")
    if shared is not None and not one_launch:
        sb = shared_buf
        if sb is None or sb.d.T != d.T or sb.d.H != d.H or sb.d.I != shared.I:
            raise ValueError("shared expert needs SharedBuffers allocated for this T, H and its I")
        expert_ffn_fused(sb.d, shared.weights.bits, x, sb.buf.work_list, sb.buf.n_work, shared.weights,
                         sb.buf.workspace, sb.buf.y_rows, sb.buf.ffn_sync, algo, stream)
    if fused:
        route_dispatch(d, x, w_router, router_bias, renormalize, buf.logits, buf.topk_ids, buf.topk_w,
                       slot_of_expert, n_slots, buf.pair_slot, buf.miss, buf.n_miss, buf.counts, buf.offsets,
                       buf.sorted_pairs, buf.pair_to_row, buf.active, buf.n_active, buf.work_list, buf.n_work,
                       host_doorbell, last_use, step, buf.sync, stream)
    else:
        route_topk(d, x, w_router, router_bias, renormalize, buf.logits, buf.topk_ids, buf.topk_w, stream)
        slot_lookup(d, buf.topk_ids, slot_of_expert, n_slots, buf.pair_slot, buf.miss, buf.n_miss,
                    host_doorbell, last_use, step, stream)
        permute(d, buf.topk_ids, buf.counts, buf.offsets, buf.sorted_pairs, buf.pair_to_row, buf.active,
                buf.n_active, buf.work_list, buf.n_work, stream)
    if one_launch:
        expert_ffn_fused_shared(d, weights.bits, x, buf.work_list, buf.n_work, shared.fused_weights, buf.workspace,
                                buf.y_rows, buf.ffn_sync, algo, stream)
    elif fused:
        expert_ffn_fused(d, weights.bits, x, buf.work_list, buf.n_work, weights, buf.workspace, buf.y_rows,
                         buf.ffn_sync, algo, stream)
    else:
        ffn = expert_ffn_q4 if weights.bits == 4 else expert_ffn_q2
        ffn(d, x, buf.work_list, buf.n_work, weights, buf.y_rows, algo, buf.workspace, None, stream)
    if shared is None:
        combine(d, buf.y_rows, buf.pair_to_row, buf.topk_w, residual, out, stream)
        return
    if one_launch:
        ys = buf.y_rows[d.T * d.k: d.T * d.k + d.T]
        gate_out = shared_buf.gate_out if shared_buf is not None else None
    else:
        ys, gate_out = sb.buf.y_rows, sb.gate_out
    combine_shared(d, buf.y_rows, buf.pair_to_row, buf.topk_w, ys, x, shared.gate_w, residual, out, gate_out,
                   stream)
