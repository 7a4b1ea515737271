"""Routed MoE decode layer for AMD Instinct MI355X (gfx950).

Python binding of libmoe.so, the C ABI declared in include/moe.h.  Each
function here has the name of a C entry point without the ``moe_`` prefix and
only marshals arguments: tensors become device pointers, the current torch
stream becomes the HIP stream, and a non-zero status becomes a ``MoeError``.
Every step of the layer runs in the library's HIP kernels; there is no
Python or CPU fallback, and a missing library raises at first use.

PyTorch supplies device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, 1, 2, 3, 4
ALGO_AUTO, ALGO_GEMV, ALGO_MFMA, ALGO_GEMM = 0, 1, 2, 3
OP_ROUTE, OP_LOOKUP, OP_PERMUTE, OP_FFN, OP_COMBINE = 0, 1, 2, 3, 4

# entry points declared in include/moe.h
EXPORTS = (
    "moe_abi_version", "moe_status_string", "moe_last_error", "moe_workspace_bytes",
    "moe_route_topk", "moe_topk_from_logits", "moe_slot_lookup", "moe_permute", "moe_work_list_capacity",
    "moe_route_dispatch",
    "moe_expert_ffn_q4", "moe_expert_ffn_q2", "moe_expert_gateup", "moe_expert_down", "moe_expert_ffn_fused",
    "moe_expert_ffn_fused_shared", "moe_expert_ffn_fused_noalloc",
    "moe_combine", "moe_combine_shared",
    "moe_zero_point_bias", "moe_stream_read",
    "moe_route_counts", "moe_hot_set", "moe_residency_plan", "moe_expert_copy",
)


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[status {status}] {message}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("group_size", ctypes.c_int32)]


class DispatchC(ctypes.Structure):
    """struct moe_dispatch (include/moe.h)."""
    _fields_ = [("topk_ids", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
                ("slot_of_expert", ctypes.c_void_p), ("n_slots", ctypes.c_int32),
                ("pair_slot", ctypes.c_void_p), ("miss_experts", ctypes.c_void_p), ("n_miss", ctypes.c_void_p),
                ("host_doorbell", ctypes.c_void_p), ("last_use", ctypes.c_void_p), ("step", ctypes.c_uint32),
                ("expert_counts", ctypes.c_void_p), ("expert_offsets", ctypes.c_void_p),
                ("sorted_pairs", ctypes.c_void_p), ("pair_to_row", ctypes.c_void_p),
                ("active_experts", ctypes.c_void_p), ("n_active", ctypes.c_void_p),
                ("work_list", ctypes.c_void_p), ("n_work", ctypes.c_void_p), ("sync", ctypes.c_void_p)]


class QWeightsC(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p * 3), ("scale", ctypes.c_void_p * 3), ("bias", ctypes.c_void_p * 3)]


class ResidencyC(ctypes.Structure):
    """struct moe_residency (include/moe.h)."""
    _fields_ = [("n_hot", ctypes.c_int32), ("n_slots", ctypes.c_int32), ("slot_of_expert", ctypes.c_void_p),
                ("expert_of_slot", ctypes.c_void_p), ("last_use", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m quantized_expert_ffn_gemv_amd._build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
    Dp, Wp = ctypes.POINTER(Dims), ctypes.POINTER(QWeightsC)
    L.moe_abi_version.argtypes = []; L.moe_abi_version.restype = ctypes.c_int
    L.moe_status_string.argtypes = [ctypes.c_int]; L.moe_status_string.restype = ctypes.c_char_p
    L.moe_last_error.argtypes = []; L.moe_last_error.restype = ctypes.c_char_p
    L.moe_workspace_bytes.argtypes = [Dp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(sz)]
    L.moe_route_topk.argtypes = [Dp, P, P, P, ctypes.c_int, P, P, P, P]
    L.moe_topk_from_logits.argtypes = [Dp, P, ctypes.c_int, P, P, P]
    L.moe_slot_lookup.argtypes = [Dp, P, P, i32, P, P, P, P, P, u32, P]
    L.moe_permute.argtypes = [Dp, P, P, P, P, P, P, P, P, P, P]
    L.moe_work_list_capacity.argtypes = [Dp, ctypes.POINTER(i32)]
    L.moe_route_dispatch.argtypes = [Dp, P, P, P, ctypes.c_int, P, ctypes.POINTER(DispatchC), P]
    for name in ("moe_expert_ffn_q4", "moe_expert_ffn_q2"):
        getattr(L, name).argtypes = [Dp, P, P, P, Wp, P, ctypes.c_int, P, sz, P]
    L.moe_expert_gateup.argtypes = [Dp, ctypes.c_int, P, P, P, Wp, ctypes.c_int, P, sz, P]
    L.moe_expert_down.argtypes = [Dp, ctypes.c_int, P, P, Wp, ctypes.c_int, P, sz, P, P]
    L.moe_expert_ffn_fused.argtypes = [Dp, ctypes.c_int, P, P, P, Wp, ctypes.c_int, P, sz, P, P, P]
    L.moe_expert_ffn_fused_shared.argtypes = [Dp, ctypes.c_int, P, P, P, Wp, ctypes.c_int, P, sz, P, P, P]
    L.moe_expert_ffn_fused_noalloc.argtypes = [Dp, ctypes.c_int, P, P, P, Wp, ctypes.c_int, P, P, P]
    L.moe_combine.argtypes = [Dp, P, P, P, P, P, P]
    L.moe_combine_shared.argtypes = [Dp, P, P, P, P, P, P, P, P, P, P]
    L.moe_zero_point_bias.argtypes = [ctypes.c_int64, P, P, P, P]
    L.moe_stream_read.argtypes = [P, sz, P, P]
    L.moe_route_counts.argtypes = [Dp, P, P, P]
    L.moe_hot_set.argtypes = [Dp, P, i32, P, P]
    L.moe_residency_plan.argtypes = [Dp, ctypes.POINTER(ResidencyC), P, P, u32, P, P, P, P, P, P, P]
    L.moe_expert_copy.argtypes = [Dp, ctypes.c_int, Wp, Wp, i32, P, P, i32, P]
    for name in EXPORTS[3:]:
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def abi_version() -> int:
    return int(lib().moe_abi_version())


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def last_error() -> str:
    return lib().moe_last_error().decode()


def _check(status: int):
    if status != OK:
        raise MoeError(status, last_error() or status_string(status))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def dims(T: int, H: int, I: int, E: int, k: int, group_size: int = 128) -> Dims:
    return Dims(T, H, I, E, k, group_size)


def group_major(q, bits: int):
    """Codes laid out [..., N, K*bits/8] (each row along K) -> the library's
    layout [..., K/128, N, 16*bits] (for each group of 128 along K, all rows'
    pieces of it in a row).  A view change and a copy; numpy in, numpy out."""
    import numpy as np
    gb = 16 * bits
    *lead, n, kb = q.shape
    if kb % gb:
        raise ValueError(f"rows of {kb} bytes are not whole groups of {gb}")
    return np.ascontiguousarray(np.asarray(q).reshape(*lead, n, kb // gb, gb).swapaxes(-3, -2))


@dataclass
class QWeights:
    """Device tensors of the quantised expert weights (layout in include/moe.h)."""
    bits: int
    q: Sequence          # [gate, up, down] uint8 tensors [E, K/128, N, 16*bits] (group-major)
    scale: Sequence      # fp16 bit patterns (int16/uint16 tensors) [E, N, K/128]
    bias: Sequence

    def c_struct(self) -> QWeightsC:
        w = QWeightsC()
        for m in range(3):
            w.q[m] = _ptr(self.q[m])
            w.scale[m] = _ptr(self.scale[m])
            w.bias[m] = _ptr(self.bias[m])
        return w


def workspace_bytes(d: Dims, op: int, bits: int = 4, algo: int = ALGO_AUTO) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().moe_workspace_bytes(ctypes.byref(d), op, bits, algo, ctypes.byref(out)))
    return int(out.value)


def route_topk(d: Dims, x, w_router, router_bias, renormalize: bool, logits, topk_ids, topk_w, stream=None):
    _check(lib().moe_route_topk(ctypes.byref(d), _ptr(x), _ptr(w_router), _ptr(router_bias),
                                int(bool(renormalize)), _ptr(logits), _ptr(topk_ids), _ptr(topk_w),
                                _stream(stream)))


def topk_from_logits(d: Dims, logits, renormalize: bool, topk_ids, topk_w, stream=None):
    _check(lib().moe_topk_from_logits(ctypes.byref(d), _ptr(logits), int(bool(renormalize)),
                                      _ptr(topk_ids), _ptr(topk_w), _stream(stream)))


def slot_lookup(d: Dims, topk_ids, slot_of_expert, n_slots: int, pair_slot, miss_experts, n_miss,
                host_doorbell=None, last_use=None, step: int = 0, stream=None):
    _check(lib().moe_slot_lookup(ctypes.byref(d), _ptr(topk_ids), _ptr(slot_of_expert), int(n_slots),
                                 _ptr(pair_slot), _ptr(miss_experts), _ptr(n_miss), _ptr(host_doorbell),
                                 _ptr(last_use), int(step) & 0xFFFFFFFF, _stream(stream)))


WORK_TILE_ROWS, WORK_ENTRY_INTS = 16, 20     # MOE_WORK_TILE_ROWS, MOE_WORK_ENTRY_INTS
DISPATCH_SYNC_INTS = 576                     # MOE_DISPATCH_SYNC_INTS
FFN_SYNC_INTS = 32800                        # MOE_FFN_SYNC_INTS (the last 32: the fault flag)
NOALLOC_WORKSPACE_BYTES = 16 << 20           # MOE_NOALLOC_WORKSPACE_BYTES
STREAM_SINK_INTS = 4096                      # MOE_STREAM_SINK_INTS
RESIDENCY_LISTS = 3                          # MOE_RESIDENCY_LISTS


def work_list_capacity(d: Dims) -> int:
    out = ctypes.c_int32(0)
    _check(lib().moe_work_list_capacity(ctypes.byref(d), ctypes.byref(out)))
    return int(out.value)


def permute(d: Dims, topk_ids, expert_counts, expert_offsets, sorted_pairs, pair_to_row,
            active_experts, n_active, work_list, n_work, stream=None):
    _check(lib().moe_permute(ctypes.byref(d), _ptr(topk_ids), _ptr(expert_counts), _ptr(expert_offsets),
                             _ptr(sorted_pairs), _ptr(pair_to_row), _ptr(active_experts), _ptr(n_active),
                             _ptr(work_list), _ptr(n_work), _stream(stream)))


def route_dispatch(d: Dims, x, w_router, router_bias, renormalize: bool, logits, topk_ids, topk_w,
                   slot_of_expert, n_slots: int, pair_slot, miss_experts, n_miss, expert_counts, expert_offsets,
                   sorted_pairs, pair_to_row, active_experts, n_active, work_list, n_work,
                   host_doorbell=None, last_use=None, step: int = 0, sync=None, stream=None):
    """moe_route_dispatch: route_topk + slot_lookup + permute in one call.  `sync`:
    None, or an int32 device tensor of DISPATCH_SYNC_INTS zeros (left zero)."""
    o = DispatchC(_ptr(topk_ids), _ptr(topk_w), _ptr(slot_of_expert), int(n_slots), _ptr(pair_slot),
                  _ptr(miss_experts), _ptr(n_miss), _ptr(host_doorbell), _ptr(last_use), int(step) & 0xFFFFFFFF,
                  _ptr(expert_counts), _ptr(expert_offsets), _ptr(sorted_pairs), _ptr(pair_to_row),
                  _ptr(active_experts), _ptr(n_active), _ptr(work_list), _ptr(n_work), _ptr(sync))
    _check(lib().moe_route_dispatch(ctypes.byref(d), _ptr(x), _ptr(w_router), _ptr(router_bias),
                                    int(bool(renormalize)), _ptr(logits), ctypes.byref(o), _stream(stream)))


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _ffn(fn, d, x, work_list, n_work, weights: QWeights, y_rows, algo, workspace, workspace_bytes_, stream):
    w = weights.c_struct()
    nbytes = workspace_bytes_ if workspace_bytes_ is not None else _nbytes(workspace)
    _check(fn(ctypes.byref(d), _ptr(x), _ptr(work_list), _ptr(n_work), ctypes.byref(w), _ptr(y_rows),
              int(algo), _ptr(workspace), nbytes, _stream(stream)))


def expert_ffn_q4(d: Dims, x, work_list, n_work, weights: QWeights, y_rows, algo: int = ALGO_AUTO,
                  workspace=None, workspace_bytes_: Optional[int] = None, stream=None):
    _ffn(lib().moe_expert_ffn_q4, d, x, work_list, n_work, weights, y_rows, algo, workspace,
         workspace_bytes_, stream)


def expert_ffn_q2(d: Dims, x, work_list, n_work, weights: QWeights, y_rows, algo: int = ALGO_AUTO,
                  workspace=None, workspace_bytes_: Optional[int] = None, stream=None):
    _ffn(lib().moe_expert_ffn_q2, d, x, work_list, n_work, weights, y_rows, algo, workspace,
         workspace_bytes_, stream)


def expert_gateup(d: Dims, bits: int, x, work_list, n_work, weights: QWeights, workspace,
                  algo: int = ALGO_AUTO, stream=None):
    w = weights.c_struct()
    _check(lib().moe_expert_gateup(ctypes.byref(d), int(bits), _ptr(x), _ptr(work_list), _ptr(n_work),
                                   ctypes.byref(w), int(algo), _ptr(workspace), _nbytes(workspace),
                                   _stream(stream)))


def expert_down(d: Dims, bits: int, work_list, n_work, weights: QWeights, workspace, y_rows,
                algo: int = ALGO_AUTO, stream=None):
    w = weights.c_struct()
    _check(lib().moe_expert_down(ctypes.byref(d), int(bits), _ptr(work_list), _ptr(n_work), ctypes.byref(w),
                                 int(algo), _ptr(workspace), _nbytes(workspace), _ptr(y_rows),
                                 _stream(stream)))


def expert_ffn_fused(d: Dims, bits: int, x, work_list, n_work, weights: QWeights, workspace, y_rows, sync,
                     algo: int = ALGO_AUTO, stream=None):
    """moe_expert_ffn_fused: gate/up and down in one launch where a kernel exists
    (else two); `sync` is an int32 device tensor of FFN_SYNC_INTS zeros (left zero)."""
    w = weights.c_struct()
    _check(lib().moe_expert_ffn_fused(ctypes.byref(d), int(bits), _ptr(x), _ptr(work_list), _ptr(n_work),
                                      ctypes.byref(w), int(algo), _ptr(workspace), _nbytes(workspace),
                                      _ptr(y_rows), _ptr(sync), _stream(stream)))


def expert_ffn_fused_noalloc(d: Dims, bits: int, x, work_list, n_work, weights: QWeights, y_rows, fault=None,
                             algo: int = ALGO_AUTO, stream=None):
    """moe_expert_ffn_fused_noalloc: expert_ffn_fused with the workspace and
    counters in the library's fixed device array (nothing allocated); `fault`:
    None or an int32 device tensor set to 1 if a wait timed out."""
    w = weights.c_struct()
    _check(lib().moe_expert_ffn_fused_noalloc(ctypes.byref(d), int(bits), _ptr(x), _ptr(work_list), _ptr(n_work),
                                              ctypes.byref(w), int(algo), _ptr(y_rows), _ptr(fault), _stream(stream)))


def expert_ffn_fused_shared(d: Dims, bits: int, x, work_list, n_work, weights: QWeights, workspace, y_rows, sync,
                            algo: int = ALGO_AUTO, stream=None):
    """moe_expert_ffn_fused_shared: the routed FFN and an always-on shared expert
    (the last of E + 1 experts in `weights`) in one launch; y_rows has T*(k+1)
    rows, the shared expert's T last."""
    w = weights.c_struct()
    _check(lib().moe_expert_ffn_fused_shared(ctypes.byref(d), int(bits), _ptr(x), _ptr(work_list), _ptr(n_work),
                                             ctypes.byref(w), int(algo), _ptr(workspace), _nbytes(workspace),
                                             _ptr(y_rows), _ptr(sync), _stream(stream)))


def combine(d: Dims, y_rows, pair_to_row, topk_w, residual, out, stream=None):
    _check(lib().moe_combine(ctypes.byref(d), _ptr(y_rows), _ptr(pair_to_row), _ptr(topk_w),
                             _ptr(residual), _ptr(out), _stream(stream)))


def combine_shared(d: Dims, y_rows, pair_to_row, topk_w, y_shared, x, shared_gate_w, residual, out,
                   shared_gate_out=None, stream=None):
    """moe_combine_shared: combine() plus sigmoid(x . shared_gate_w) * y_shared."""
    _check(lib().moe_combine_shared(ctypes.byref(d), _ptr(y_rows), _ptr(pair_to_row), _ptr(topk_w), _ptr(y_shared),
                                    _ptr(x), _ptr(shared_gate_w), _ptr(residual), _ptr(out), _ptr(shared_gate_out),
                                    _stream(stream)))


def zero_point_bias(scale, zeros, bias, stream=None):
    """moe_zero_point_bias: bias = fp16(-(zeros * scale)) per group, turning
    zero-point weights (q - z) s into this library's q s + b.  scale and bias
    are int16 device tensors (fp16 bits), zeros uint8, all of one size."""
    n = int(scale.numel())
    if int(zeros.numel()) != n or int(bias.numel()) != n:
        raise ValueError("scale, zeros and bias must have one entry per group each")
    _check(lib().moe_zero_point_bias(n, _ptr(scale), _ptr(zeros), _ptr(bias), _stream(stream)))


def stream_read(src, sink, nbytes: Optional[int] = None, stream=None):
    """moe_stream_read: one streaming read of `src` (nbytes, default all of it);
    sink is a uint32/int32 device tensor of STREAM_SINK_INTS entries."""
    n = _nbytes(src) if nbytes is None else int(nbytes)
    _check(lib().moe_stream_read(_ptr(src), n, _ptr(sink), _stream(stream)))


def route_counts(d: Dims, expert_counts, freq, stream=None):
    """moe_route_counts: freq[e] += expert_counts[e] (uint32 counters as int32 tensors)."""
    _check(lib().moe_route_counts(ctypes.byref(d), _ptr(expert_counts), _ptr(freq), _stream(stream)))


def hot_set(d: Dims, freq, n: int, hot, stream=None):
    """moe_hot_set: hot[0..n) = the n most routed experts (ties to the lower id)."""
    _check(lib().moe_hot_set(ctypes.byref(d), _ptr(freq), int(n), _ptr(hot), _stream(stream)))


def residency_plan(d: Dims, n_hot: int, n_slots: int, slot_of_expert, expert_of_slot, last_use, miss, n_miss,
                   step: int, work_list, n_work, lists, list_counts, copies, n_copy, stream=None):
    """moe_residency_plan: one step of the warm ring (victims, tables, copy list,
    and the work list split into resident / copied / cold lists)."""
    r = ResidencyC(int(n_hot), int(n_slots), _ptr(slot_of_expert), _ptr(expert_of_slot), _ptr(last_use))
    _check(lib().moe_residency_plan(ctypes.byref(d), ctypes.byref(r), _ptr(miss), _ptr(n_miss),
                                    int(step) & 0xFFFFFFFF, _ptr(work_list), _ptr(n_work), _ptr(lists),
                                    _ptr(list_counts), _ptr(copies), _ptr(n_copy), _stream(stream)))


def expert_copy(d: Dims, bits: int, src: "QWeights", dst: "QWeights", n_dst: int, copies, n_copy, max_copies: int,
                stream=None):
    """moe_expert_copy: experts copies[2i] of src into slots copies[2i+1] of dst."""
    ws, wd = src.c_struct(), dst.c_struct()
    _check(lib().moe_expert_copy(ctypes.byref(d), int(bits), ctypes.byref(ws), ctypes.byref(wd), int(n_dst),
                                 _ptr(copies), _ptr(n_copy), int(max_copies), _stream(stream)))


from .layer import (LayerBuffers, ResidentExperts, SharedBuffers, SharedExpert, StackLayer, layer_forward,  # noqa: E402
                    resident_layer_forward, stack_forward)  # (orchestration of the calls above)

__all__ = [
    "lib", "abi_version", "status_string", "last_error", "MoeError", "Dims", "dims", "QWeights",
    "workspace_bytes", "work_list_capacity", "WORK_TILE_ROWS", "WORK_ENTRY_INTS", "route_topk", "route_dispatch", "DISPATCH_SYNC_INTS", "FFN_SYNC_INTS",
    "topk_from_logits", "slot_lookup", "permute", "expert_ffn_q4",
    "expert_ffn_q2", "expert_gateup", "expert_down", "expert_ffn_fused", "expert_ffn_fused_shared", "expert_ffn_fused_noalloc", "NOALLOC_WORKSPACE_BYTES", "combine", "combine_shared", "zero_point_bias", "stream_read", "STREAM_SINK_INTS", "route_counts", "hot_set", "residency_plan",
    "expert_copy", "RESIDENCY_LISTS", "ResidencyC", "LayerBuffers", "ResidentExperts", "resident_layer_forward", "SharedBuffers", "SharedExpert", "layer_forward", "StackLayer", "stack_forward", "EXPORTS",
    "group_major", "ALGO_AUTO", "ALGO_GEMV", "ALGO_MFMA", "ALGO_GEMM", "OP_ROUTE", "OP_LOOKUP", "OP_PERMUTE", "OP_FFN", "OP_COMBINE",
]
