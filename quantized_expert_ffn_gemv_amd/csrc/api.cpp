// C ABI of libmoe.so: argument validation, status codes and dispatch to the
// kernel launchers.  Every check runs on the host before anything is
// enqueued, so a call that fails leaves the stream untouched.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "common.h"
#include "moe.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_last_error[0] = '\0';
    return MOE_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define REQUIRE_PTR(p, align)                                                            \
    do {                                                                                 \
        if ((p) == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s: %s is NULL", fn, #p);  \
        if (!aligned((p), (align)))                                                      \
            return fail(MOE_ERR_INVALID_ARG, "%s: %s is not %d-byte aligned", fn, #p,    \
                        (int)(align));                                                   \
    } while (0)

// Checks shared by every call; `need_hi` also checks H/I (FFN, route, combine).
int check_dims(const char* fn, const moe_dims* d, bool need_h, bool need_i) {
    if (d == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s: dims is NULL", fn);
    if (d->T < 0) return fail(MOE_ERR_INVALID_ARG, "%s: T = %d is negative", fn, d->T);
    if (d->E < 1 || d->E > 1024)
        return fail(MOE_ERR_UNSUPPORTED, "%s: E = %d outside [1, 1024]", fn, d->E);
    if (d->k < 1 || d->k > d->E || d->k > 32)
        return fail(MOE_ERR_UNSUPPORTED, "%s: k = %d outside [1, min(E, 32)]", fn, d->k);
    if ((long long)d->T * d->k > 65536)
        return fail(MOE_ERR_UNSUPPORTED, "%s: T*k = %lld exceeds 65536", fn, (long long)d->T * d->k);
    if (d->group_size != 128 && d->group_size != 64 && d->group_size != 32)
        return fail(MOE_ERR_UNSUPPORTED, "%s: group_size = %d (32, 64 or 128)", fn, d->group_size);
    if (need_h && (d->H < 128 || d->H > 8192 || d->H % 128 != 0))
        return fail(MOE_ERR_UNSUPPORTED, "%s: H = %d must be a multiple of 128 in [128, 8192]", fn, d->H);
    if (need_i && (d->I < 128 || d->I > 16384 || d->I % 128 != 0))
        return fail(MOE_ERR_UNSUPPORTED, "%s: I = %d must be a multiple of 128 in [128, 16384]", fn, d->I);
    return MOE_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Checks shared by the FFN calls.  Matrices [m_begin, m_end) of `w` are used.
int check_ffn_args(const char* fn, const moe_dims* d, int bits, const int32_t* work_list,
                   const int32_t* n_work, const moe_qweights* w, int algo, int m_begin, int m_end) {
    int st = check_dims(fn, d, true, true);
    if (st) return st;
    if (bits != 2 && bits != 4) return fail(MOE_ERR_UNSUPPORTED, "%s: bits = %d (2 or 4)", fn, bits);
    if (w == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s: weights is NULL", fn);
    if (algo != MOE_ALGO_AUTO && algo != MOE_ALGO_GEMV && algo != MOE_ALGO_MFMA && algo != MOE_ALGO_GEMM)
        return fail(MOE_ERR_UNSUPPORTED, "%s: unknown algo %d", fn, algo);
    if (algo == MOE_ALGO_GEMM && !moe::gemm_supported(*d, bits))
        return fail(MOE_ERR_UNSUPPORTED,
                    "%s: the grouped GEMM needs 4-bit codes, groups of 32, 64 or 128 and H, I multiples of 128, at "
                    "least 256", fn);
    if (!moe::ffn_group_supported(*d, bits, algo))
        return fail(MOE_ERR_UNSUPPORTED,
                    "%s: groups of %d need the decode kernels (tiles that fit LDS) or, for groups of at least one "
                    "16-byte chunk of codes (%d), the vector-ALU path",
                    fn, d->group_size, 128 / bits);
    if (d->T == 0) return MOE_OK;
    REQUIRE_PTR(work_list, 16);
    REQUIRE_PTR(n_work, 4);
    for (int m = m_begin; m < m_end; ++m) {
        if (!w->q[m] || !w->scale[m] || !w->bias[m])
            return fail(MOE_ERR_INVALID_ARG, "%s: weights matrix %d has a NULL pointer", fn, m);
        if (!aligned(w->q[m], 16))
            return fail(MOE_ERR_INVALID_ARG, "%s: weights.q[%d] is not 16-byte aligned", fn, m);
        if (!aligned(w->scale[m], 16) || !aligned(w->bias[m], 16))
            return fail(MOE_ERR_INVALID_ARG, "%s: weights.scale/bias[%d] is not 16-byte aligned", fn, m);
    }
    return MOE_OK;
}

moe::FfnArgs ffn_args(const moe_dims* d, int bits, const uint16_t* x, const int32_t* work_list,
                      const int32_t* n_work, const moe_qweights* w, float* h, uint16_t* y) {
    moe::FfnArgs a{};
    a.d = *d;
    a.bits = bits;
    a.x = x;
    a.work = work_list;
    a.n_work = n_work;
    a.w = *w;
    a.y = y;
    a.h = h;
    return a;
}

int check_workspace(const char* fn, const moe_dims* d, int bits, int algo, const void* ws, size_t ws_bytes) {
    const size_t need = moe::ffn_workspace_bytes(*d, bits, algo);
    if (ws == nullptr || ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                    ws == nullptr ? (size_t)0 : ws_bytes);
    if (!aligned(ws, 256)) return fail(MOE_ERR_INVALID_ARG, "%s: workspace is not 256-byte aligned", fn);
    return MOE_OK;
}

int launch_gateup(int alg, const moe::FfnArgs& a, hipStream_t s) {
    switch (alg) {
        case MOE_ALGO_GEMV: return moe::launch_gateup_gemv(a, s);
        case MOE_ALGO_GEMM: return moe::launch_gateup_gemm(a, s);
        default: return moe::launch_gateup_mfma(a, s);
    }
}

int launch_down(int alg, const moe::FfnArgs& a, hipStream_t s) {
    switch (alg) {
        case MOE_ALGO_GEMV: return moe::launch_down_gemv(a, s);
        case MOE_ALGO_GEMM: return moe::launch_down_gemm(a, s);
        default: return moe::launch_down_mfma(a, s);
    }
}

int ffn_common(const char* fn, int bits, const moe_dims* d, const uint16_t* x,
               const int32_t* work_list, const int32_t* n_work, const moe_qweights* w, uint16_t* y,
               int algo, void* ws, size_t ws_bytes, void* stream) {
    int st = check_ffn_args(fn, d, bits, work_list, n_work, w, algo, 0, 3);
    if (st) return st;
    if (d->T == 0) return ok();
    REQUIRE_PTR(x, 16);
    REQUIRE_PTR(y, 16);
    st = check_workspace(fn, d, bits, algo, ws, ws_bytes);
    if (st) return st;
    moe::FfnArgs a = ffn_args(d, bits, x, work_list, n_work, w, static_cast<float*>(ws), y);
    const int alg = moe::resolve_algo(*d, bits, algo);
    st = launch_gateup(alg, a, as_stream(stream));
    if (!st) st = launch_down(alg, a, as_stream(stream));
    if (st) return fail(st, "%s: kernel launch failed: %s", fn, hipGetErrorString(hipGetLastError()));
    return ok();
}


}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape or option";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* moe_last_error(void) { return g_last_error; }

int moe_workspace_bytes(const moe_dims* d, int op, int bits, int algo, size_t* bytes) {
    const char* fn = "moe_workspace_bytes";
    if (bytes == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s: bytes is NULL", fn);
    if (bits != 2 && bits != 4) return fail(MOE_ERR_UNSUPPORTED, "%s: bits = %d", fn, bits);
    if (op < MOE_OP_ROUTE || op > MOE_OP_COMBINE) return fail(MOE_ERR_INVALID_ARG, "%s: op = %d", fn, op);
    int st = check_dims(fn, d, op == MOE_OP_FFN, op == MOE_OP_FFN);
    if (st) return st;
    *bytes = (op == MOE_OP_FFN) ? moe::ffn_workspace_bytes(*d, bits, algo) : 0;
    return ok();
}

int moe_route_topk(const moe_dims* d, const uint16_t* x, const float* w_router,
                   const float* router_bias, int renormalize, float* logits, int32_t* topk_ids,
                   float* topk_w, void* stream) {
    const char* fn = "moe_route_topk";
    int st = check_dims(fn, d, true, false);
    if (st) return st;
    if (d->T == 0) return ok();
    REQUIRE_PTR(x, 16);
    REQUIRE_PTR(w_router, 16);
    if (router_bias && !aligned(router_bias, 4))
        return fail(MOE_ERR_INVALID_ARG, "%s: router_bias misaligned", fn);
    REQUIRE_PTR(logits, 4);
    REQUIRE_PTR(topk_ids, 4);
    REQUIRE_PTR(topk_w, 4);
    st = moe::launch_router_logits(*d, x, w_router, router_bias, logits, as_stream(stream));
    if (!st) st = moe::launch_topk(*d, logits, renormalize, topk_ids, topk_w, as_stream(stream));
    if (st) return fail(st, "%s: kernel launch failed: %s", fn, hipGetErrorString(hipGetLastError()));
    return ok();
}

int moe_topk_from_logits(const moe_dims* d, const float* logits, int renormalize, int32_t* topk_ids,
                         float* topk_w, void* stream) {
    const char* fn = "moe_topk_from_logits";
    int st = check_dims(fn, d, false, false);
    if (st) return st;
    if (d->T == 0) return ok();
    REQUIRE_PTR(logits, 4);
    REQUIRE_PTR(topk_ids, 4);
    REQUIRE_PTR(topk_w, 4);
    st = moe::launch_topk(*d, logits, renormalize, topk_ids, topk_w, as_stream(stream));
    if (st) return fail(st, "%s: kernel launch failed: %s", fn, hipGetErrorString(hipGetLastError()));
    return ok();
}

int moe_slot_lookup(const moe_dims* d, const int32_t* topk_ids, const int32_t* slot_of_expert,
                    int32_t n_slots, int32_t* pair_slot, int32_t* miss_experts, int32_t* n_miss,
                    int32_t* host_doorbell, uint32_t* last_use, uint32_t step, void* stream) {
    const char* fn = "moe_slot_lookup";
    int st = check_dims(fn, d, false, false);
    if (st) return st;
    if (n_slots < 0) return fail(MOE_ERR_INVALID_ARG, "%s: n_slots = %d is negative", fn, n_slots);
    REQUIRE_PTR(slot_of_expert, 4);
    REQUIRE_PTR(miss_experts, 4);
    REQUIRE_PTR(n_miss, 4);
    if (d->T > 0) {
        REQUIRE_PTR(topk_ids, 4);
        REQUIRE_PTR(pair_slot, 4);
    }
    if (host_doorbell && !aligned(host_doorbell, 4))
        return fail(MOE_ERR_INVALID_ARG, "%s: host_doorbell misaligned", fn);
    if (last_use && !aligned(last_use, 4)) return fail(MOE_ERR_INVALID_ARG, "%s: last_use misaligned", fn);
    st = moe::launch_slot_lookup(*d, topk_ids, slot_of_expert, n_slots, pair_slot, miss_experts,
                                 n_miss, host_doorbell, last_use, step, as_stream(stream));
    if (st) return fail(st, "%s: kernel launch failed: %s", fn, hipGetErrorString(hipGetLastError()));
    return ok();
}

int moe_work_list_capacity(const moe_dims* d, int32_t* entries) {
    const char* fn = "moe_work_list_capacity";
    int st = check_dims(fn, d, false, false);
    if (st) return st;
    if (entries == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s: entries is NULL", fn);
    *entries = (int32_t)moe::work_capacity(*d);
    return ok();
}

int moe_permute(const moe_dims* d, const int32_t* topk_ids, int32_t* counts, int32_t* offsets,
                int32_t* sorted_pairs, int32_t* pair_to_row, int32_t* active, int32_t* n_active,
                int32_t* work_list, int32_t* n_work, void* stream) {
    const char* fn = "moe_permute";
    int st = check_dims(fn, d, false, false);
    if (st) return st;
    REQUIRE_PTR(counts, 4);
    REQUIRE_PTR(offsets, 4);
    REQUIRE_PTR(active, 4);
    REQUIRE_PTR(n_active, 4);
    REQUIRE_PTR(n_work, 4);
    if (d->T > 0) {
        REQUIRE_PTR(topk_ids, 4);
        REQUIRE_PTR(sorted_pairs, 4);
        REQUIRE_PTR(pair_to_row, 4);
        REQUIRE_PTR(work_list, 16);
    }
    st = moe::launch_permute(*d, topk_ids, counts, offsets, sorted_pairs, pair_to_row, active,
                             n_active, work_list, n_work, as_stream(stream));
    if (st) return fail(st, "%s: kernel launch failed: %s", fn, hipGetErrorString(hipGetLastError()));
    return ok();
}

int moe_route_dispatch(const moe_dims* d, const uint16_t* x, const float* w_router, const float* router_bias,
                       int renormalize, float* logits, const moe_dispatch* o, void* stream) {
    const char* fn = "moe_route_dispatch";
    int st = check_dims(fn, d, true, false);
    if (st) return st;
    if (o == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s: out is NULL", fn);
    if (o->n_slots < 0) return fail(MOE_ERR_INVALID_ARG, "%s: n_slots = %d is negative", fn, o->n_slots);
    REQUIRE_PTR(o->slot_of_expert, 4);
    REQUIRE_PTR(o->miss_experts, 4);
    REQUIRE_PTR(o->n_miss, 4);
    REQUIRE_PTR(o->expert_counts, 4);
    REQUIRE_PTR(o->expert_offsets, 4);
    REQUIRE_PTR(o->active_experts, 4);
    REQUIRE_PTR(o->n_active, 4);
    REQUIRE_PTR(o->n_work, 4);
    if (d->T > 0) {
        REQUIRE_PTR(x, 16);
        REQUIRE_PTR(w_router, 16);
        REQUIRE_PTR(logits, 4);
        REQUIRE_PTR(o->topk_ids, 4);
        REQUIRE_PTR(o->topk_w, 4);
        REQUIRE_PTR(o->pair_slot, 4);
        REQUIRE_PTR(o->sorted_pairs, 4);
        REQUIRE_PTR(o->pair_to_row, 4);
        REQUIRE_PTR(o->work_list, 16);
    }
    if (router_bias && !aligned(router_bias, 4))
        return fail(MOE_ERR_INVALID_ARG, "%s: router_bias misaligned", fn);
    if (o->host_doorbell && !aligned(o->host_doorbell, 4))
        return fail(MOE_ERR_INVALID_ARG, "%s: host_doorbell misaligned", fn);
    if (o->last_use && !aligned(o->last_use, 4)) return fail(MOE_ERR_INVALID_ARG, "%s: last_use misaligned", fn);
    if (o->sync && !aligned(o->sync, 256)) return fail(MOE_ERR_INVALID_ARG, "%s: sync not 256-byte aligned", fn);
    const hipStream_t s = as_stream(stream);
    moe::DispatchArgs a{};
    a.renorm = renormalize;
    a.ids = o->topk_ids; a.gates = o->topk_w;
    a.table = o->slot_of_expert; a.n_slots = o->n_slots;
    a.pair_slot = o->pair_slot; a.miss = o->miss_experts; a.n_miss = o->n_miss;
    a.doorbell = o->host_doorbell; a.last_use = o->last_use; a.step = o->step;
    a.counts = o->expert_counts; a.offsets = o->expert_offsets; a.sorted_pairs = o->sorted_pairs;
    a.pair_to_row = o->pair_to_row; a.active = o->active_experts; a.n_active = o->n_active;
    a.work = o->work_list; a.n_work = o->n_work;
    if (o->sync && moe::route_dispatch_fused(*d)) {
        // the whole routing in one launch
        st = moe::launch_route_dispatch(*d, x, w_router, router_bias, logits, a, o->sync, s);
        if (st) return fail(st, "%s: kernel launch failed: %s", fn, hipGetErrorString(hipGetLastError()));
        return ok();
    }
    st = moe::launch_router_logits(*d, x, w_router, router_bias, logits, s);
    if (!st && moe::dispatch_fused(*d)) {
        st = moe::launch_dispatch(*d, logits, a, s);
    } else if (!st) {
        // too many pairs for one workgroup's LDS: the three kernels of the separate calls
        if (d->T > 0) st = moe::launch_topk(*d, logits, renormalize, o->topk_ids, o->topk_w, s);
        if (!st)
            st = moe::launch_slot_lookup(*d, o->topk_ids, o->slot_of_expert, o->n_slots, o->pair_slot,
                                         o->miss_experts, o->n_miss, o->host_doorbell, o->last_use, o->step, s);
        if (!st)
            st = moe::launch_permute(*d, o->topk_ids, o->expert_counts, o->expert_offsets, o->sorted_pairs,
                                     o->pair_to_row, o->active_experts, o->n_active, o->work_list, o->n_work, s);
    }
    if (st) return fail(st, "%s: kernel launch failed: %s", fn, hipGetErrorString(hipGetLastError()));
    return ok();
}

int moe_expert_ffn_q4(const moe_dims* d, const uint16_t* x, const int32_t* work_list,
                      const int32_t* n_work, const moe_qweights* w, uint16_t* y, int algo, void* ws,
                      size_t ws_bytes, void* stream) {
    return ffn_common("moe_expert_ffn_q4", 4, d, x, work_list, n_work, w, y, algo, ws, ws_bytes, stream);
}

int moe_expert_ffn_q2(const moe_dims* d, const uint16_t* x, const int32_t* work_list,
                      const int32_t* n_work, const moe_qweights* w, uint16_t* y, int algo, void* ws,
                      size_t ws_bytes, void* stream) {
    return ffn_common("moe_expert_ffn_q2", 2, d, x, work_list, n_work, w, y, algo, ws, ws_bytes, stream);
}

int moe_expert_gateup(const moe_dims* d, int bits, const uint16_t* x, const int32_t* work_list,
                      const int32_t* n_work, const moe_qweights* w, int algo, void* ws, size_t ws_bytes,
                      void* stream) {
    const char* fn = "moe_expert_gateup";
    int st = check_ffn_args(fn, d, bits, work_list, n_work, w, algo, 0, 2);
    if (st) return st;
    if (d->T == 0) return ok();
    REQUIRE_PTR(x, 16);
    st = check_workspace(fn, d, bits, algo, ws, ws_bytes);
    if (st) return st;
    moe::FfnArgs a = ffn_args(d, bits, x, work_list, n_work, w, static_cast<float*>(ws), nullptr);
    st = launch_gateup(moe::resolve_algo(*d, bits, algo), a, as_stream(stream));
    if (st) return fail(st, "%s: kernel launch failed: %s", fn, hipGetErrorString(hipGetLastError()));
    return ok();
}

int moe_expert_down(const moe_dims* d, int bits, const int32_t* work_list, const int32_t* n_work,
                    const moe_qweights* w, int algo, void* ws, size_t ws_bytes, uint16_t* y,
                    void* stream) {
    const char* fn = "moe_expert_down";
    int st = check_ffn_args(fn, d, bits, work_list, n_work, w, algo, 2, 3);
    if (st) return st;
    if (d->T == 0) return ok();
    REQUIRE_PTR(y, 16);
    st = check_workspace(fn, d, bits, algo, ws, ws_bytes);
    if (st) return st;
    moe::FfnArgs a = ffn_args(d, bits, nullptr, work_list, n_work, w, static_cast<float*>(ws), y);
    st = launch_down(moe::resolve_algo(*d, bits, algo), a, as_stream(stream));
    if (st) return fail(st, "%s: kernel launch failed: %s", fn, hipGetErrorString(hipGetLastError()));
    return ok();
}

int moe_expert_ffn_fused(const moe_dims* d, int bits, const uint16_t* x, const int32_t* work_list,
                         const int32_t* n_work, const moe_qweights* w, int algo, void* ws, size_t ws_bytes,
                         uint16_t* y, int32_t* sync, void* stream) {
    const char* fn = "moe_expert_ffn_fused";
    int st = check_ffn_args(fn, d, bits, work_list, n_work, w, algo, 0, 3);
    if (st) return st;
    if (d->T == 0) return ok();
    REQUIRE_PTR(x, 16);
    REQUIRE_PTR(y, 16);
    REQUIRE_PTR(sync, 256);
    st = check_workspace(fn, d, bits, algo, ws, ws_bytes);
    if (st) return st;
    moe::FfnArgs a = ffn_args(d, bits, x, work_list, n_work, w, static_cast<float*>(ws), y);
    const int alg = moe::resolve_algo(*d, bits, algo);
    const hipStream_t s = as_stream(stream);
    st = alg == MOE_ALGO_MFMA ? moe::launch_ffn_fused_dec(a, sync, s) : MOE_ERR_UNSUPPORTED;
    if (st == MOE_ERR_UNSUPPORTED) {
        st = launch_gateup(alg, a, s);
        if (!st) st = launch_down(alg, a, s);
    }
    if (st) return fail(st, "%s: kernel launch failed: %s", fn, hipGetErrorString(hipGetLastError()));
    return ok();
}

int moe_expert_ffn_fused_noalloc(const moe_dims* d, int bits, const uint16_t* x, const int32_t* work_list,
                                 const int32_t* n_work, const moe_qweights* w, int algo, uint16_t* y, int32_t* fault,
                                 void* stream) {
    const char* fn = "moe_expert_ffn_fused_noalloc";
    int st = check_ffn_args(fn, d, bits, work_list, n_work, w, algo, 0, 3);
    if (st) return st;
    if (d->T == 0) return ok();
    REQUIRE_PTR(x, 16);
    REQUIRE_PTR(y, 16);
    if (fault && !aligned(fault, 4)) return fail(MOE_ERR_INVALID_ARG, "%s: fault misaligned", fn);
    const size_t need = moe::ffn_workspace_bytes(*d, bits, algo);
    if (need > (size_t)MOE_NOALLOC_WORKSPACE_BYTES)
        return fail(MOE_ERR_WORKSPACE, "%s: these dims need %zu bytes of workspace; the fixed scratch holds %zu",
                    fn, need, (size_t)MOE_NOALLOC_WORKSPACE_BYTES);
    int32_t* sync = nullptr;
    void* ws = nullptr;
    size_t ws_bytes = 0;
    if (moe::noalloc_scratch(&sync, &ws, &ws_bytes) != MOE_OK)
        return fail(MOE_ERR_HIP, "%s: looking up the scratch array failed: %s", fn,
                    hipGetErrorString(hipGetLastError()));
    moe::FfnArgs a = ffn_args(d, bits, x, work_list, n_work, w, static_cast<float*>(ws), y);
    const int alg = moe::resolve_algo(*d, bits, algo);
    const hipStream_t s = as_stream(stream);
    st = MOE_ERR_UNSUPPORTED;
    if (alg == MOE_ALGO_MFMA) {
        st = moe::launch_clear_sync(sync, s);
        if (!st) st = moe::launch_ffn_fused_dec(a, sync, s, fault);
    }
    if (st == MOE_ERR_UNSUPPORTED) {
        st = launch_gateup(alg, a, s);
        if (!st) st = launch_down(alg, a, s);
    }
    if (st) return fail(st, "%s: kernel launch failed: %s", fn, hipGetErrorString(hipGetLastError()));
    return ok();
}

int moe_expert_ffn_fused_shared(const moe_dims* d, int bits, const uint16_t* x, const int32_t* work_list,
                                const int32_t* n_work, const moe_qweights* w, int algo, void* ws, size_t ws_bytes,
                                uint16_t* y, int32_t* sync, void* stream) {
    const char* fn = "moe_expert_ffn_fused_shared";
    int st = check_ffn_args(fn, d, bits, work_list, n_work, w, algo, 0, 3);
    if (st) return st;
    if (d->T == 0) return ok();
    if (d->E + 1 > 1024 || d->k + 1 > 32)
        return fail(MOE_ERR_UNSUPPORTED, "%s: E + 1 or k + 1 beyond the library's limits", fn);
    REQUIRE_PTR(x, 16);
    REQUIRE_PTR(y, 16);
    REQUIRE_PTR(sync, 256);
    moe_dims d1 = *d;
    d1.E = d->E + 1;
    d1.k = d->k + 1;
    st = check_workspace(fn, &d1, bits, algo, ws, ws_bytes);
    if (st) return st;
    if (moe::resolve_algo(d1, bits, algo) != MOE_ALGO_MFMA)
        return fail(MOE_ERR_UNSUPPORTED, "%s: only the matrix-core decode path takes a shared expert", fn);
    moe::FfnArgs a = ffn_args(d, bits, x, work_list, n_work, w, static_cast<float*>(ws), y);
    st = moe::launch_ffn_fused_dec_shared(a, sync, as_stream(stream));
    if (st == MOE_ERR_UNSUPPORTED)
        return fail(st, "%s: the decode kernels do not take this shape; run the shared expert as its own call", fn);
    if (st) return fail(st, "%s: kernel launch failed: %s", fn, hipGetErrorString(hipGetLastError()));
    return ok();
}

int moe_combine(const moe_dims* d, const uint16_t* y_rows, const int32_t* pair_to_row,
                const float* topk_w, const uint16_t* residual, uint16_t* out, void* stream) {
    const char* fn = "moe_combine";
    int st = check_dims(fn, d, true, false);
    if (st) return st;
    if (d->T == 0) return ok();
    REQUIRE_PTR(y_rows, 16);
    REQUIRE_PTR(pair_to_row, 4);
    REQUIRE_PTR(topk_w, 4);
    REQUIRE_PTR(residual, 16);
    REQUIRE_PTR(out, 16);
    st = moe::launch_combine(*d, y_rows, pair_to_row, topk_w, residual, out, as_stream(stream));
    if (st) return fail(st, "%s: kernel launch failed: %s", fn, hipGetErrorString(hipGetLastError()));
    return ok();
}

int moe_combine_shared(const moe_dims* d, const uint16_t* y_rows, const int32_t* pair_to_row, const float* topk_w,
                       const uint16_t* y_shared, const uint16_t* x, const float* shared_gate_w,
                       const uint16_t* residual, uint16_t* out, float* shared_gate_out, void* stream) {
    const char* fn = "moe_combine_shared";
    int st = check_dims(fn, d, true, false);
    if (st) return st;
    if (d->T == 0) return ok();
    REQUIRE_PTR(y_rows, 16);
    REQUIRE_PTR(pair_to_row, 4);
    REQUIRE_PTR(topk_w, 4);
    REQUIRE_PTR(y_shared, 16);
    REQUIRE_PTR(x, 16);
    REQUIRE_PTR(shared_gate_w, 16);
    REQUIRE_PTR(residual, 16);
    REQUIRE_PTR(out, 16);
    if (shared_gate_out && !aligned(shared_gate_out, 4))
        return fail(MOE_ERR_INVALID_ARG, "%s: shared_gate_out misaligned", fn);
    st = moe::launch_combine_shared(*d, y_rows, pair_to_row, topk_w, y_shared, x, shared_gate_w, residual, out,
                                    shared_gate_out, as_stream(stream));
    if (st) return fail(st, "%s: kernel launch failed: %s", fn, hipGetErrorString(hipGetLastError()));
    return ok();
}

int moe_zero_point_bias(int64_t n, const uint16_t* scale, const uint8_t* zeros, uint16_t* bias, void* stream) {
    const char* fn = "moe_zero_point_bias";
    if (n < 0) return fail(MOE_ERR_INVALID_ARG, "%s: n = %lld is negative", fn, (long long)n);
    if (n == 0) return ok();
    REQUIRE_PTR(scale, 2);
    REQUIRE_PTR(zeros, 1);
    REQUIRE_PTR(bias, 2);
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(bias), b1 = b0 + 2 * (uintptr_t)n;
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(scale), s1 = s0 + 2 * (uintptr_t)n;
    const uintptr_t z0 = reinterpret_cast<uintptr_t>(zeros), z1 = z0 + (uintptr_t)n;
    if ((b0 < s1 && s0 < b1) || (b0 < z1 && z0 < b1))
        return fail(MOE_ERR_INVALID_ARG, "%s: bias overlaps scale or zeros", fn);
    const int st = moe::launch_zero_point_bias((long)n, scale, zeros, bias, as_stream(stream));
    if (st) return fail(st, "%s: kernel launch failed: %s", fn, hipGetErrorString(hipGetLastError()));
    return ok();
}

int moe_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
    const char* fn = "moe_stream_read";
    if (bytes == 0) return ok();
    REQUIRE_PTR(src, 16);
    REQUIRE_PTR(sink, 4);
    if (bytes % 16 != 0) return fail(MOE_ERR_INVALID_ARG, "%s: bytes = %zu is not a multiple of 16", fn, bytes);
    const int st = moe::launch_stream_read(src, bytes, sink, as_stream(stream));
    if (st) return fail(st, "%s: kernel launch failed: %s", fn, hipGetErrorString(hipGetLastError()));
    return ok();
}

int moe_route_counts(const moe_dims* d, const int32_t* counts, uint32_t* freq, void* stream) {
    const char* fn = "moe_route_counts";
    int st = check_dims(fn, d, false, false);
    if (st) return st;
    REQUIRE_PTR(counts, 4);
    REQUIRE_PTR(freq, 4);
    st = moe::launch_route_counts(counts, freq, d->E, as_stream(stream));
    if (st) return fail(st, "%s: kernel launch failed: %s", fn, hipGetErrorString(hipGetLastError()));
    return ok();
}

int moe_hot_set(const moe_dims* d, const uint32_t* freq, int32_t n, int32_t* hot, void* stream) {
    const char* fn = "moe_hot_set";
    int st = check_dims(fn, d, false, false);
    if (st) return st;
    if (n < 0 || n > d->E) return fail(MOE_ERR_INVALID_ARG, "%s: n = %d outside [0, E = %d]", fn, n, d->E);
    if (n == 0) return ok();
    REQUIRE_PTR(freq, 4);
    REQUIRE_PTR(hot, 4);
    st = moe::launch_hot_set(freq, d->E, n, hot, as_stream(stream));
    if (st) return fail(st, "%s: kernel launch failed: %s", fn, hipGetErrorString(hipGetLastError()));
    return ok();
}

int moe_residency_plan(const moe_dims* d, const moe_residency* r, const int32_t* miss, const int32_t* n_miss,
                       uint32_t step, const int32_t* work_list, const int32_t* n_work, int32_t* lists,
                       int32_t* list_counts, int32_t* copies, int32_t* n_copy, void* stream) {
    const char* fn = "moe_residency_plan";
    int st = check_dims(fn, d, false, false);
    if (st) return st;
    if (r == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s: residency is NULL", fn);
    if (r->n_slots < 1 || r->n_slots > d->E || r->n_hot < 0 || r->n_hot > r->n_slots)
        return fail(MOE_ERR_INVALID_ARG, "%s: need 0 <= n_hot (%d) <= n_slots (%d) <= E (%d), n_slots >= 1", fn,
                    r->n_hot, r->n_slots, d->E);
    if (step == 0) return fail(MOE_ERR_INVALID_ARG, "%s: step 0 marks never-used slots; steps count from 1", fn);
    REQUIRE_PTR(r->slot_of_expert, 4);
    REQUIRE_PTR(r->expert_of_slot, 4);
    REQUIRE_PTR(r->last_use, 4);
    REQUIRE_PTR(miss, 4);
    REQUIRE_PTR(n_miss, 4);
    REQUIRE_PTR(n_work, 4);
    REQUIRE_PTR(list_counts, 4);
    REQUIRE_PTR(copies, 4);
    REQUIRE_PTR(n_copy, 4);
    const long cap = moe::work_capacity(*d);
    if (cap > 0) {
        REQUIRE_PTR(work_list, 16);
        REQUIRE_PTR(lists, 16);
    }
    moe::PlanArgs a{};
    a.E = d->E; a.n_hot = r->n_hot; a.n_slots = r->n_slots; a.cap = (int)cap; a.step = step;
    a.slot_of_expert = r->slot_of_expert; a.expert_of_slot = r->expert_of_slot; a.last_use = r->last_use;
    a.miss = miss; a.n_miss = n_miss; a.work = work_list; a.n_work = n_work;
    a.lists = lists; a.list_counts = list_counts; a.copies = copies; a.n_copy = n_copy;
    st = moe::launch_residency_plan(a, as_stream(stream));
    if (st) return fail(st, "%s: kernel launch failed: %s", fn, hipGetErrorString(hipGetLastError()));
    return ok();
}

int moe_expert_copy(const moe_dims* d, int bits, const moe_qweights* src, const moe_qweights* dst, int32_t n_dst,
                    const int32_t* copies, const int32_t* n_copy, int32_t max_copies, void* stream) {
    const char* fn = "moe_expert_copy";
    int st = check_dims(fn, d, true, true);
    if (st) return st;
    if (bits != 2 && bits != 4) return fail(MOE_ERR_UNSUPPORTED, "%s: bits = %d (2 or 4)", fn, bits);
    if (src == nullptr || dst == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s: weights is NULL", fn);
    if (n_dst < 1) return fail(MOE_ERR_INVALID_ARG, "%s: n_dst = %d", fn, n_dst);
    if (max_copies < 0 || max_copies > 65535) return fail(MOE_ERR_INVALID_ARG, "%s: max_copies = %d", fn, max_copies);
    if (max_copies == 0) return ok();
    REQUIRE_PTR(copies, 4);
    REQUIRE_PTR(n_copy, 4);
    for (int m = 0; m < 3; ++m) {
        if (!src->q[m] || !src->scale[m] || !src->bias[m] || !dst->q[m] || !dst->scale[m] || !dst->bias[m])
            return fail(MOE_ERR_INVALID_ARG, "%s: matrix %d has a NULL pointer", fn, m);
        if (!aligned(src->q[m], 16) || !aligned(dst->q[m], 16) || !aligned(src->scale[m], 16) ||
            !aligned(dst->scale[m], 16) || !aligned(src->bias[m], 16) || !aligned(dst->bias[m], 16))
            return fail(MOE_ERR_INVALID_ARG, "%s: matrix %d is not 16-byte aligned", fn, m);
    }
    st = moe::launch_expert_copy(*d, bits, *src, *dst, n_dst, copies, n_copy, max_copies, as_stream(stream));
    if (st) return fail(st, "%s: kernel launch failed: %s", fn, hipGetErrorString(hipGetLastError()));
    return ok();
}

}  // extern "C"
