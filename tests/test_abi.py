"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

* libmoe.so loads and exports every entry point that include/moe.h declares;
* argument validation rejects bad calls before anything is enqueued, with the
  documented status code and a readable moe_last_error().
Pointers used here are fake addresses: every call below fails validation on
the host, which is exactly what is being tested.
"""
import ctypes
import os
import re

import pytest

import quantized_expert_ffn_gemv_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000000          # 256-byte aligned, never dereferenced
MISALIGNED = FAKE + 2


def header_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_what_the_binding_lists():
    assert header_functions() == sorted(moe.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    for name in header_functions():
        assert hasattr(L, name), name
    assert moe.abi_version() == 1
    assert moe.status_string(moe.ERR_WORKSPACE).startswith("workspace")


def test_library_exports_nothing_else_with_the_prefix():
    out = os.popen(f"nm -D --defined-only {moe.LIB_PATH}").read()
    exported = sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\b", out)))
    assert exported == header_functions()


@pytest.mark.parametrize("T,H,I,E,k,g,status", [
    (-1, 256, 256, 8, 2, 128, moe.ERR_INVALID_ARG),
    (4, 250, 256, 8, 2, 128, moe.ERR_UNSUPPORTED),      # H not a multiple of 128
    (4, 256, 200, 8, 2, 128, moe.ERR_UNSUPPORTED),      # I not a multiple of 128
    (4, 256, 256, 8, 9, 128, moe.ERR_UNSUPPORTED),      # k > E
    (4, 256, 256, 2000, 2, 128, moe.ERR_UNSUPPORTED),   # E too large
    (4, 256, 256, 8, 2, 96, moe.ERR_UNSUPPORTED),       # group size (32, 64 or 128)
    (4, 256, 256, 8, 2, 16, moe.ERR_UNSUPPORTED),
    (40000, 256, 256, 8, 2, 128, moe.ERR_UNSUPPORTED),  # T*k too large
    (4, 16384, 256, 8, 2, 128, moe.ERR_UNSUPPORTED),    # H too large
])
def test_dims_validation(T, H, I, E, k, g, status):
    d = moe.Dims(T, H, I, E, k, g)
    with pytest.raises(moe.MoeError) as ex:
        moe.workspace_bytes(d, moe.OP_FFN, 4)
    assert ex.value.status == status
    assert moe.last_error()


def test_workspace_size():
    # the grouped GEMM adds its heads list after the matrix-core workspace
    dp = moe.dims(4096, 2048, 768, 128, 8)
    assert moe.workspace_bytes(dp, moe.OP_FFN, 4, moe.ALGO_GEMM) > moe.workspace_bytes(dp, moe.OP_FFN, 4, moe.ALGO_MFMA)
    assert moe.workspace_bytes(dp, moe.OP_FFN, 4) == moe.workspace_bytes(dp, moe.OP_FFN, 4, moe.ALGO_GEMM)
    d = moe.dims(32, 2048, 512, 256, 8)
    assert moe.workspace_bytes(d, moe.OP_FFN, 4) >= 32 * 8 * 512 * 4
    assert moe.workspace_bytes(d, moe.OP_ROUTE, 4) == 0
    with pytest.raises(moe.MoeError):
        moe.workspace_bytes(d, moe.OP_FFN, 3)


def test_group_sizes_by_path():
    """Groups of 64 and 32: the decode kernels (tiles that fit LDS), the
    grouped GEMM (4-bit codes), and the vector-ALU path where one scale covers
    a 16-byte chunk of codes; the persistent and streaming kernels of larger
    shapes take groups of 128 only."""
    L = moe.lib()
    w = _qw()
    small = moe.dims(8, 2048, 512, 256, 8, 64)               # decode tiles fit
    for algo in (moe.ALGO_AUTO, moe.ALGO_MFMA, moe.ALGO_GEMV, moe.ALGO_GEMM):
        moe.workspace_bytes(small, moe.OP_FFN, 4, algo)
    # the grouped GEMM takes the finer group; the check stops at the workspace
    assert _ffn(small, algo=moe.ALGO_GEMM, ws_bytes=1) == moe.ERR_WORKSPACE
    # its per-group activation sums grow with the group count
    g128 = moe.dims(8, 2048, 512, 256, 8)
    assert moe.workspace_bytes(small, moe.OP_FFN, 4, moe.ALGO_GEMM) > moe.workspace_bytes(g128, moe.OP_FFN, 4, moe.ALGO_GEMM)
    prefill64 = moe.dims(4096, 2048, 768, 128, 8, 64)        # 256 pairs per expert: AUTO takes the GEMM
    assert moe.workspace_bytes(prefill64, moe.OP_FFN, 4) == moe.workspace_bytes(prefill64, moe.OP_FFN, 4, moe.ALGO_GEMM)
    g32 = moe.dims(8, 2048, 512, 256, 8, 32)
    # 2-bit codes: 64 per 16-byte chunk, more than a group of 32
    assert L.moe_expert_ffn_q2(ctypes.byref(g32), FAKE, FAKE, FAKE, ctypes.byref(w), FAKE, moe.ALGO_GEMV, FAKE,
                               1 << 30, None) == moe.ERR_UNSUPPORTED
    assert "groups of 32" in moe.last_error()
    big = moe.dims(8, 5120, 8192, 64, 2, 64)                 # the down tile does not fit LDS
    assert _ffn(big, algo=moe.ALGO_MFMA) == moe.ERR_UNSUPPORTED
    assert _ffn(big, algo=moe.ALGO_AUTO, ws_bytes=1) == moe.ERR_WORKSPACE   # AUTO takes the vector-ALU path
    assert moe.workspace_bytes(big, moe.OP_FFN, 4) == moe.workspace_bytes(big, moe.OP_FFN, 4, moe.ALGO_GEMV)


def _qw(ptr=FAKE):
    w = moe.QWeightsC()
    for m in range(3):
        w.q[m] = ptr
        w.scale[m] = FAKE
        w.bias[m] = FAKE
    return w


def _ffn(d, x=FAKE, y=FAKE, w=None, algo=0, ws=FAKE, ws_bytes=1 << 30, wl=FAKE, nw=FAKE):
    L = moe.lib()
    w = w or _qw()
    return L.moe_expert_ffn_q4(ctypes.byref(d), x, wl, nw, ctypes.byref(w), y, algo, ws, ws_bytes, None)


def test_work_list_capacity():
    # min(E, T*k) + T*k / 16: enough for every expert's partial tile plus the full ones
    assert moe.work_list_capacity(moe.dims(32, 2048, 512, 256, 8)) == 256 + 16
    assert moe.work_list_capacity(moe.dims(1, 4096, 1024, 512, 4)) == 4
    assert moe.work_list_capacity(moe.dims(0, 256, 512, 8, 2)) == 0
    assert moe.lib().moe_work_list_capacity(ctypes.byref(moe.dims(1, 256, 512, 8, 2)), None) == moe.ERR_INVALID_ARG


def test_ffn_validation_paths():
    d = moe.dims(4, 256, 512, 8, 2)
    assert _ffn(d, x=None) == moe.ERR_INVALID_ARG
    assert "x is NULL" in moe.last_error()
    assert _ffn(d, x=MISALIGNED) == moe.ERR_INVALID_ARG
    assert "aligned" in moe.last_error()
    assert _ffn(d, wl=None) == moe.ERR_INVALID_ARG
    assert _ffn(d, wl=FAKE + 4) == moe.ERR_INVALID_ARG
    assert _ffn(d, nw=None) == moe.ERR_INVALID_ARG
    assert _ffn(d, w=_qw(MISALIGNED)) == moe.ERR_INVALID_ARG
    assert _ffn(d, algo=7) == moe.ERR_UNSUPPORTED
    # the grouped GEMM takes 4-bit codes only
    L = moe.lib()
    w = _qw()
    assert L.moe_expert_ffn_q2(ctypes.byref(d), FAKE, FAKE, FAKE, ctypes.byref(w), FAKE, moe.ALGO_GEMM, FAKE,
                               1 << 30, None) == moe.ERR_UNSUPPORTED
    assert "grouped GEMM" in moe.last_error()
    assert _ffn(d, ws=None) == moe.ERR_WORKSPACE
    assert _ffn(d, ws_bytes=100) == moe.ERR_WORKSPACE
    assert "workspace" in moe.last_error()
    assert _ffn(d, ws=FAKE + 16) == moe.ERR_INVALID_ARG


def test_fused_ffn_validation():
    L = moe.lib()
    d = moe.dims(4, 256, 512, 8, 2)
    w = _qw()
    call = lambda x=FAKE, y=FAKE, sync=FAKE, ws=FAKE, bits=4: L.moe_expert_ffn_fused(
        ctypes.byref(d), bits, x, FAKE, FAKE, ctypes.byref(w), moe.ALGO_AUTO, ws, 1 << 30, y, sync, None)
    assert call(sync=None) == moe.ERR_INVALID_ARG
    assert "sync is NULL" in moe.last_error()
    assert call(sync=FAKE + 128) == moe.ERR_INVALID_ARG          # counters need 256-byte alignment
    assert "sync" in moe.last_error()
    assert call(x=None) == moe.ERR_INVALID_ARG
    assert call(y=MISALIGNED) == moe.ERR_INVALID_ARG
    assert call(ws=FAKE + 16) == moe.ERR_INVALID_ARG
    assert call(bits=3) == moe.ERR_UNSUPPORTED
    z = moe.dims(0, 256, 512, 8, 2)
    assert L.moe_expert_ffn_fused(ctypes.byref(z), 4, None, None, None, ctypes.byref(w), 0, None, 0, None, None,
                                  None) == moe.OK


def test_route_and_combine_validation():
    L = moe.lib()
    d = moe.dims(4, 256, 512, 8, 2)
    assert L.moe_route_topk(ctypes.byref(d), FAKE, None, None, 1, FAKE, FAKE, FAKE, None) == moe.ERR_INVALID_ARG
    assert L.moe_route_topk(ctypes.byref(d), MISALIGNED, FAKE, None, 1, FAKE, FAKE, FAKE, None) == moe.ERR_INVALID_ARG
    assert L.moe_topk_from_logits(ctypes.byref(d), None, 1, FAKE, FAKE, None) == moe.ERR_INVALID_ARG
    assert L.moe_combine(ctypes.byref(d), FAKE, FAKE, FAKE, MISALIGNED, FAKE, None) == moe.ERR_INVALID_ARG
    assert L.moe_slot_lookup(ctypes.byref(d), FAKE, FAKE, -1, FAKE, FAKE, FAKE, None, None, 0, None) == moe.ERR_INVALID_ARG
    assert L.moe_permute(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == moe.ERR_INVALID_ARG
    assert L.moe_permute(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == moe.ERR_INVALID_ARG
    assert L.moe_permute(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == moe.ERR_INVALID_ARG
    assert L.moe_workspace_bytes(None, 3, 4, 0, None) == moe.ERR_INVALID_ARG


def test_zero_tokens_need_no_buffers():
    """T = 0: route, FFN and combine return OK without touching any pointer."""
    L = moe.lib()
    d = moe.dims(0, 256, 512, 8, 2)
    assert L.moe_route_topk(ctypes.byref(d), None, None, None, 1, None, None, None, None) == moe.OK
    assert L.moe_combine(ctypes.byref(d), None, None, None, None, None, None) == moe.OK
    w = _qw()
    assert L.moe_expert_ffn_q4(ctypes.byref(d), None, None, None, ctypes.byref(w), None, 0, None, 0,
                               None) == moe.OK


def _dispatch(**over):
    f = {name: FAKE for name, _ in moe.DispatchC._fields_}
    f.update(n_slots=8, step=0, host_doorbell=None, last_use=None)
    f.update(over)
    return moe.DispatchC(**f)


def test_route_dispatch_validation():
    L = moe.lib()
    d = moe.dims(4, 256, 512, 8, 2)
    call = lambda o, x=FAKE, bias=None: L.moe_route_dispatch(ctypes.byref(d), x, FAKE, bias, 1, FAKE,
                                                              None if o is None else ctypes.byref(o), None)
    assert call(None) == moe.ERR_INVALID_ARG
    assert "out is NULL" in moe.last_error()
    assert call(_dispatch(), x=MISALIGNED) == moe.ERR_INVALID_ARG
    assert call(_dispatch(), bias=MISALIGNED) == moe.ERR_INVALID_ARG
    assert call(_dispatch(n_slots=-1)) == moe.ERR_INVALID_ARG
    for name in ("topk_ids", "slot_of_expert", "pair_slot", "miss_experts", "n_miss", "expert_counts",
                 "expert_offsets", "sorted_pairs", "pair_to_row", "active_experts", "n_active", "work_list",
                 "n_work"):
        assert call(_dispatch(**{name: None})) == moe.ERR_INVALID_ARG, name
        assert name in moe.last_error()
    assert call(_dispatch(work_list=FAKE + 4)) == moe.ERR_INVALID_ARG
    assert call(_dispatch(host_doorbell=MISALIGNED)) == moe.ERR_INVALID_ARG
    assert call(_dispatch(sync=MISALIGNED)) == moe.ERR_INVALID_ARG
    assert call(_dispatch(sync=FAKE + 128)) == moe.ERR_INVALID_ARG          # counters need 256-byte alignment
    assert "sync" in moe.last_error()
    bad = moe.Dims(4, 256, 512, 8, 9, 128)
    assert L.moe_route_dispatch(ctypes.byref(bad), FAKE, FAKE, None, 1, FAKE, ctypes.byref(_dispatch()),
                                None) == moe.ERR_UNSUPPORTED


def test_zero_point_bias_validation():
    L = moe.lib()
    assert L.moe_zero_point_bias(-1, FAKE, FAKE, FAKE, None) == moe.ERR_INVALID_ARG
    assert L.moe_zero_point_bias(0, None, None, None, None) == moe.OK
    assert L.moe_zero_point_bias(8, None, FAKE, FAKE + 4096, None) == moe.ERR_INVALID_ARG
    assert L.moe_zero_point_bias(8, FAKE + 1, FAKE, FAKE + 4096, None) == moe.ERR_INVALID_ARG
    assert L.moe_zero_point_bias(8, FAKE, FAKE + 4096, FAKE + 8, None) == moe.ERR_INVALID_ARG   # bias overlaps scale
    assert "overlaps" in moe.last_error()
    assert L.moe_zero_point_bias(8, FAKE + 4096, FAKE, FAKE + 4, None) == moe.ERR_INVALID_ARG   # bias overlaps zeros


def test_combine_shared_validation():
    L = moe.lib()
    d = moe.dims(4, 256, 512, 8, 2)
    args = [FAKE] * 8
    for i in range(8):
        bad = list(args)
        bad[i] = None
        assert L.moe_combine_shared(ctypes.byref(d), *bad, None, None) == moe.ERR_INVALID_ARG
    bad = list(args)
    bad[4] = MISALIGNED                                                  # x
    assert L.moe_combine_shared(ctypes.byref(d), *bad, None, None) == moe.ERR_INVALID_ARG
    assert L.moe_combine_shared(ctypes.byref(d), *args, FAKE + 1, None) == moe.ERR_INVALID_ARG
    d0 = moe.dims(0, 256, 512, 8, 2)
    assert L.moe_combine_shared(ctypes.byref(d0), *([None] * 9), None) == moe.OK


def test_fused_shared_ffn_validation():
    L = moe.lib()
    d = moe.dims(4, 256, 512, 8, 2)
    w = moe.QWeightsC()
    for m in range(3):
        w.q[m], w.scale[m], w.bias[m] = FAKE, FAKE, FAKE
    args = (ctypes.byref(d), 4, FAKE, FAKE, FAKE, ctypes.byref(w), moe.ALGO_AUTO)
    assert L.moe_expert_ffn_fused_shared(*args, FAKE, 1 << 30, FAKE, None, None) == moe.ERR_INVALID_ARG  # no sync
    assert L.moe_expert_ffn_fused_shared(*args, FAKE, 16, FAKE, FAKE, None) == moe.ERR_WORKSPACE        # too small
    d32 = moe.dims(4, 256, 512, 8, 32)
    assert L.moe_expert_ffn_fused_shared(ctypes.byref(d32), *args[1:], FAKE, 1 << 30, FAKE, FAKE,
                                         None) == moe.ERR_UNSUPPORTED                                   # k + 1 > 32


def test_stream_read_validation():
    L = moe.lib()
    assert L.moe_stream_read(None, 0, None, None) == moe.OK                       # nothing to read
    assert L.moe_stream_read(None, 4096, FAKE, None) == moe.ERR_INVALID_ARG
    assert L.moe_stream_read(MISALIGNED, 4096, FAKE, None) == moe.ERR_INVALID_ARG
    assert L.moe_stream_read(FAKE, 4100, FAKE, None) == moe.ERR_INVALID_ARG         # not whole 16-byte words
    assert "multiple of 16" in moe.last_error()
    assert L.moe_stream_read(FAKE, 4096, None, None) == moe.ERR_INVALID_ARG


def _res(**over):
    f = dict(n_hot=2, n_slots=4, slot_of_expert=FAKE, expert_of_slot=FAKE, last_use=FAKE)
    f.update(over)
    return moe.ResidencyC(**f)


def test_residency_validation():
    L = moe.lib()
    d = moe.dims(4, 256, 512, 8, 2)
    plan = lambda r, step=1, lists=FAKE: L.moe_residency_plan(ctypes.byref(d), None if r is None else ctypes.byref(r),
                                                               FAKE, FAKE, step, FAKE, FAKE, lists, FAKE, FAKE, FAKE,
                                                               None)
    assert plan(None) == moe.ERR_INVALID_ARG
    assert plan(_res(n_slots=9)) == moe.ERR_INVALID_ARG                            # more slots than experts
    assert plan(_res(n_hot=5)) == moe.ERR_INVALID_ARG                              # hot set beyond the pool
    assert plan(_res(n_slots=0, n_hot=0)) == moe.ERR_INVALID_ARG
    assert plan(_res(), step=0) == moe.ERR_INVALID_ARG                             # 0 marks never-used slots
    assert "steps count from 1" in moe.last_error()
    assert plan(_res(last_use=None)) == moe.ERR_INVALID_ARG
    assert plan(_res(), lists=FAKE + 4) == moe.ERR_INVALID_ARG
    assert L.moe_hot_set(ctypes.byref(d), FAKE, 9, FAKE, None) == moe.ERR_INVALID_ARG   # n > E
    assert L.moe_hot_set(ctypes.byref(d), None, 0, None, None) == moe.OK
    assert L.moe_hot_set(ctypes.byref(d), None, 3, FAKE, None) == moe.ERR_INVALID_ARG
    assert L.moe_route_counts(ctypes.byref(d), FAKE, None, None) == moe.ERR_INVALID_ARG
    w = _qw()
    copy = lambda bits=4, n_dst=4, maxc=4, src=w: L.moe_expert_copy(ctypes.byref(d), bits, ctypes.byref(src),
                                                                    ctypes.byref(w), n_dst, FAKE, FAKE, maxc, None)
    assert copy(bits=3) == moe.ERR_UNSUPPORTED
    assert copy(n_dst=0) == moe.ERR_INVALID_ARG
    assert copy(maxc=-1) == moe.ERR_INVALID_ARG
    assert copy(maxc=0) == moe.OK
    bad = _qw()
    bad.q[1] = MISALIGNED
    assert copy(src=bad) == moe.ERR_INVALID_ARG


def test_noalloc_validation():
    L = moe.lib()
    d = moe.dims(4, 256, 512, 8, 2)
    w = _qw()
    call = lambda x=FAKE, y=FAKE, fault=None, bits=4: L.moe_expert_ffn_fused_noalloc(
        ctypes.byref(d), bits, x, FAKE, FAKE, ctypes.byref(w), moe.ALGO_AUTO, y, fault, None)
    assert call(x=None) == moe.ERR_INVALID_ARG
    assert call(y=MISALIGNED) == moe.ERR_INVALID_ARG
    assert call(fault=MISALIGNED) == moe.ERR_INVALID_ARG
    assert call(bits=3) == moe.ERR_UNSUPPORTED
    big = moe.dims(4096, 2048, 768, 128, 8)
    assert L.moe_expert_ffn_fused_noalloc(ctypes.byref(big), 4, FAKE, FAKE, FAKE, ctypes.byref(w), moe.ALGO_MFMA,
                                          FAKE, None, None) == moe.ERR_WORKSPACE
    z = moe.dims(0, 256, 512, 8, 2)
    assert L.moe_expert_ffn_fused_noalloc(ctypes.byref(z), 4, None, None, None, ctypes.byref(w), 0, None, None,
                                          None) == moe.OK
