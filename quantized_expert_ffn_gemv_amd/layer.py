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

``ResidentExperts`` and ``resident_layer_forward`` run the step with the
experts behind residency tiers (pinned host memory, an HBM pool of hot and
warm slots): the plan kernel after the routing picks warm slots for the
misses, the copies run on a second stream while the FFN of the experts
already resident runs, then the FFN of the rest and the combine.

``StackLayer`` and ``stack_forward`` run a decode step through several
layers back to back (each layer's output is the next one's input), the unit
that is captured once in a HIP graph and replayed per token.

This module only orders the calls; the arithmetic is in the HIP kernels.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import torch

from . import (ALGO_AUTO, DISPATCH_SYNC_INTS, FFN_SYNC_INTS, OP_FFN, RESIDENCY_LISTS, WORK_ENTRY_INTS, Dims,
               QWeights, combine, combine_shared, dims, expert_copy, expert_ffn_fused, expert_ffn_fused_shared,
               expert_ffn_q2, expert_ffn_q4, permute, residency_plan, route_counts, route_dispatch, route_topk,
               slot_lookup, work_list_capacity, workspace_bytes)


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

    def ffn_timed_out(self) -> bool:
        """True if an expert_ffn_fused call on these buffers had a down item give
        up waiting for its h (that call's rows are not valid).  Reads the flag at
        the end of ffn_sync, so it waits for the stream's work so far."""
        return bool(int(self.ffn_sync[FFN_SYNC_INTS - 32:].abs().sum().item()))

    def counters_clean(self) -> bool:
        """True if both counter buffers are back to all zeros, as every call that
        completed normally leaves them (waits for the stream's work so far)."""
        return int(self.sync.abs().sum().item()) == 0 and int(self.ffn_sync.abs().sum().item()) == 0

    def reset_counters(self) -> None:
        """After a time-out: zero both counter buffers (a fill kernel on the
        current stream) before the next call uses them."""
        self.sync.zero_()
        self.ffn_sync.zero_()

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


@dataclass
class StackLayer:
    """One layer of a stack: its router and expert weights."""
    w_router: torch.Tensor
    router_bias: Optional[torch.Tensor]
    weights: QWeights
    slot_of_expert: torch.Tensor
    n_slots: int


def stack_forward(bufs: Sequence[LayerBuffers], x: torch.Tensor, layers: Sequence[StackLayer],
                  outs: Sequence[torch.Tensor], algo: int = ALGO_AUTO, stream=None) -> torch.Tensor:
    """A decode step through a stack of MoE layers, back to back on one batch:
    layer l takes h_l (h_0 = x) as its input and its residual and writes
    h_(l+1) = h_l + MoE_l(h_l) to outs[l] ("Luce Spark" page, sec. 3: the
    routed FFN of every layer in one graph per token).  Nothing here waits on
    the host, so the whole stack can be captured in one HIP graph and replayed
    once per token step.  Returns outs[-1]."""
    if not (len(bufs) == len(layers) == len(outs)):
        raise ValueError("one buffer set and one output per layer")
    h = x
    for buf, L, out in zip(bufs, layers, outs):
        layer_forward(buf, h, L.w_router, L.router_bias, L.weights, L.slot_of_expert, L.n_slots, h, out,
                      algo=algo, stream=stream)
        h = out
    return h


@dataclass
class ResidentExperts:
    """The residency tiers of one layer's experts ("Luce Spark" page, sec. 1-2):
    every expert in pinned host memory (cold, `host`), an HBM pool of n_slots
    slots (`pool`): slots [0, n_hot) the calibrated hot set, the rest the warm
    ring.  The tables, the routing-frequency counters and the plan's outputs
    are device tensors; the library's kernels update them at every step."""
    d: Dims
    bits: int
    n_hot: int
    n_slots: int
    host: QWeights                # E experts, pinned host tensors (device-visible)
    pool: QWeights                # n_slots experts, device tensors
    slot_of_expert: torch.Tensor  # int32 [E], -1 = cold
    expert_of_slot: torch.Tensor  # int32 [n_slots], -1 = empty
    last_use: torch.Tensor        # int32 [n_slots] (uint32 step stamps, 0 = never)
    freq: torch.Tensor            # int32 [E] (uint32 routing-frequency counters)
    lists: torch.Tensor           # int32 [RESIDENCY_LISTS, capacity, WORK_ENTRY_INTS]
    list_counts: torch.Tensor     # int32 [RESIDENCY_LISTS]
    copies: torch.Tensor          # int32 [n_slots, 2]
    n_copy: torch.Tensor          # int32 [1]

    @staticmethod
    def allocate(d: Dims, bits: int, host: QWeights, n_hot: int, n_slots: int, device="cuda") -> "ResidentExperts":
        if not 0 <= n_hot <= n_slots <= d.E:
            raise ValueError("need 0 <= n_hot <= n_slots <= E")
        i32 = dict(dtype=torch.int32, device=device)
        pool = QWeights(bits, [torch.empty((n_slots,) + tuple(t.shape[1:]), dtype=t.dtype, device=device) for t in host.q],
                        [torch.empty((n_slots,) + tuple(t.shape[1:]), dtype=t.dtype, device=device) for t in host.scale],
                        [torch.empty((n_slots,) + tuple(t.shape[1:]), dtype=t.dtype, device=device) for t in host.bias])
        cap = max(work_list_capacity(d), 1)
        return ResidentExperts(
            d=d, bits=bits, n_hot=n_hot, n_slots=n_slots, host=host, pool=pool,
            slot_of_expert=torch.full((d.E,), -1, **i32), expert_of_slot=torch.full((n_slots,), -1, **i32),
            last_use=torch.zeros((n_slots,), **i32), freq=torch.zeros((d.E,), **i32),
            lists=torch.empty((RESIDENCY_LISTS, cap, WORK_ENTRY_INTS), **i32),
            list_counts=torch.zeros((RESIDENCY_LISTS,), **i32),
            copies=torch.zeros((n_slots, 2), **i32), n_copy=torch.zeros((1,), **i32))

    def install(self, experts: torch.Tensor, stream=None) -> None:
        """Make slots 0 .. len(experts)-1 hold these experts (e.g. the hot set
        from hot_set()), every other slot empty and every stamp 0: the tables
        are set here and the weights copied from host memory by the library."""
        n = int(experts.numel())
        if n > self.n_slots:
            raise ValueError("more experts than slots")
        e = experts.to(torch.int32)
        slots = torch.arange(n, dtype=torch.int32, device=e.device)
        self.slot_of_expert.fill_(-1)
        self.slot_of_expert[e.long()] = slots
        self.expert_of_slot.fill_(-1)
        self.expert_of_slot[:n] = e
        self.last_use.zero_()
        self.copies[:n, 0] = e
        self.copies[:n, 1] = slots
        self.n_copy.fill_(n)
        expert_copy(self.d, self.bits, self.host, self.pool, self.n_slots, self.copies, self.n_copy, max(n, 1), stream)


def resident_layer_forward(buf: LayerBuffers, res: ResidentExperts, x: torch.Tensor, w_router: torch.Tensor,
                           router_bias: Optional[torch.Tensor], residual: torch.Tensor, out: torch.Tensor,
                           step: int, algo: int = ALGO_AUTO, copy_stream=None, count: bool = True,
                           host_doorbell=None) -> None:
    """Enqueue one layer step with the experts behind the residency tiers
    (steps count from 1).  Routing and the slot lookup run against res's
    tables (stamping the slots they hit); the routing counters are updated
    (count); the plan picks warm slots for the misses and splits the work
    list; the copies from host memory run on copy_stream (or the current
    stream) while the FFN of the experts already resident runs; then the FFN
    of the experts copied in this step and of those still cold (read from host
    memory), then the combine.  The expert rows are bit for bit those of
    layer_forward with every expert resident."""
    import torch as _t
    d = buf.d
    main = _t.cuda.current_stream() if copy_stream is not None else None
    route_dispatch(d, x, w_router, router_bias, True, buf.logits, buf.topk_ids, buf.topk_w, res.slot_of_expert,
                   res.n_slots, buf.pair_slot, buf.miss, buf.n_miss, buf.counts, buf.offsets, buf.sorted_pairs,
                   buf.pair_to_row, buf.active, buf.n_active, buf.work_list, buf.n_work, host_doorbell,
                   res.last_use, step, buf.sync)
    if count:
        route_counts(d, buf.counts, res.freq)
    residency_plan(d, res.n_hot, res.n_slots, res.slot_of_expert, res.expert_of_slot, res.last_use, buf.miss,
                   buf.n_miss, step, buf.work_list, buf.n_work, res.lists, res.list_counts, res.copies, res.n_copy)
    n_warm = max(res.n_slots - res.n_hot, 1)
    if copy_stream is not None:
        planned = _t.cuda.Event()
        planned.record(main)
        copy_stream.wait_event(planned)
        expert_copy(d, res.bits, res.host, res.pool, res.n_slots, res.copies, res.n_copy, n_warm,
                    copy_stream.cuda_stream)
        copied = _t.cuda.Event()
        copied.record(copy_stream)
    else:
        expert_copy(d, res.bits, res.host, res.pool, res.n_slots, res.copies, res.n_copy, n_warm)
    lists = [res.lists[i] for i in range(RESIDENCY_LISTS)]
    counts = [res.list_counts[i:i + 1] for i in range(RESIDENCY_LISTS)]
    expert_ffn_fused(d, res.bits, x, lists[0], counts[0], res.pool, buf.workspace, buf.y_rows, buf.ffn_sync, algo)
    if copy_stream is not None:
        main.wait_event(copied)
    expert_ffn_fused(d, res.bits, x, lists[1], counts[1], res.pool, buf.workspace, buf.y_rows, buf.ffn_sync, algo)
    expert_ffn_fused(d, res.bits, x, lists[2], counts[2], res.host, buf.workspace, buf.y_rows, buf.ffn_sync, algo)
    combine(d, buf.y_rows, buf.pair_to_row, buf.topk_w, residual, out)
