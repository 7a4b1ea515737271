// Top-k selection of one token's experts by one wave (Betelgeuse page, MoE
// primer: the router scores every expert and only the k best run; the gates
// are a softmax renormalised over the k picked).
//
// Each candidate gets a 64-bit key whose unsigned order is the ranking:
// class (removed < NaN < number), then the value (with -0 folded onto +0, so
// equal values tie), then the lower expert id.  k rounds of a wave-wide
// maximum pick the experts in rank order.  The maximum runs on DPP row
// shifts and row broadcasts (about a dozen VALU steps, no LDS traffic).
#pragma once

#include "common.h"

namespace moe {

__device__ __forceinline__ uint64_t rank_key(float v, int id) {
    const uint64_t idpart = (uint64_t)(0xFFFFFu - (uint32_t)id);
    if (v != v) return (1ull << 62) | idpart;
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7FFFFFFFu) == 0u) u = 0u;   // -0 -> +0: equal values tie
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (2ull << 62) | ((uint64_t)ord << 20) | idpart;
}

__device__ __forceinline__ int rank_key_id(uint64_t key) { return (int)(0xFFFFFu - (uint32_t)(key & 0xFFFFFu)); }

// max(v, v of the lane that the DPP pattern CTRL names); lanes whose source
// is outside the row, or whose row is not in ROWS, see 0 (every key > 0 except
// a removed candidate, which is 0).
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t max_dpp_step(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)v, CTRL, ROWS, 0xF, true);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(v >> 32), CTRL, ROWS, 0xF, true);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    return o > v ? o : v;
}

// Maximum over the 64 lanes, returned to every lane: row_shr 1, 2, 4, 8 leave
// each row's maximum in its lane 15; row_bcast 15 and 31 carry it into lane 63.
__device__ __forceinline__ uint64_t wave_max_u64_dpp(uint64_t v) {
    v = max_dpp_step<0x111, 0xF>(v);   // row_shr:1
    v = max_dpp_step<0x112, 0xF>(v);   // row_shr:2
    v = max_dpp_step<0x114, 0xF>(v);   // row_shr:4
    v = max_dpp_step<0x118, 0xF>(v);   // row_shr:8
    v = max_dpp_step<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
    v = max_dpp_step<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, 63);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

// One token: the wave reads its E logits L[0..E) (PER per lane), picks k
// (k <= 64) and returns, in lane j < k, the j-th pick and its gate.
// renorm = 1: gates are a softmax over the k picked; 0: over all E.
// COHERENT: read the logits with device-scope atomic loads (written by other
// CUs in the same kernel).
template <int PER, bool COHERENT = false>
__device__ __forceinline__ void topk_one_token(const float* __restrict__ L, int E, int k, int renorm,
                                               int& my_id, float& my_gate) {
    const int lane = threadIdx.x & 63;
    float v[PER];
    uint64_t key[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        if constexpr (COHERENT) v[i] = (e < E) ? __hip_atomic_load(L + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.f;
        else v[i] = (e < E) ? L[e] : 0.f;
        key[i] = (e < E) ? rank_key(v[i], e) : 0ull;
    }
    my_id = -1;
    float my_v = 0.f;
    for (int j = 0; j < k; ++j) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_u64_dpp(best);
        const int id = rank_key_id(best);
        // the owner removes the pick and hands its logit to lane j
        float picked = 0.f;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if (lane + 64 * i == id) {
                key[i] = 0ull;
                picked = v[i];
            }
        }
        const float pv = __shfl(picked, id & 63, kWave);
        if (lane == j && id < E) {
            my_id = id;
            my_v = pv;
        }
    }
    const float top = __shfl(my_v, 0, kWave);
    const float num = (lane < k) ? expf(my_v - top) : 0.f;
    float den;
    if (renorm) {
        den = wave_sum_xor(num, kWave);
    } else {
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if (lane + 64 * i < E) part += expf(v[i] - top);
        den = wave_sum_xor(part, kWave);
    }
    my_gate = num / den;
}

}  // namespace moe
