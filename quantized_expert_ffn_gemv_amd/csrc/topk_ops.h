// Top-k selection of one token's experts by one wave (Betelgeuse page, MoE
// primer: the router scores every expert and only the k best run; the gates
// are a softmax renormalised over the k picked).
//
// Ranking: larger logit first, equal logits (-0 == +0) to the lower expert id,
// NaN below every number (-inf included).  Each logit becomes a 32-bit key
// whose unsigned order is the logit order (numbers in [0x007FFFFF,
// 0xFF800000], NaN = 1, 0 = taken or absent).  Each lane sorts its own
// candidates; then k rounds each take the wave-wide maximum of the lanes'
// heads (DPP row shifts and row broadcasts, no LDS traffic), resolve the owner
// (one ballot; on a tie, the lowest id wins through a second DPP reduction) and
// drop that lane's head.  The picked logit comes back from its key, so no
// lane-to-lane copy is needed.
#pragma once

#include "common.h"

namespace moe {

__device__ __forceinline__ uint32_t order_key(float v) {
    if (v != v) return 1u;
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7FFFFFFFu) == 0u) u = 0u;            // -0 -> +0: equal values tie
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The logit a key came from (-0 comes back as +0; NaN as the default NaN).
__device__ __forceinline__ float key_value(uint32_t key) {
    if (key == 1u) return __builtin_nanf("");
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// op(v, v of the lane the DPP pattern CTRL names); lanes whose source is
// outside the row, or whose row is not in ROWS, combine with `fill`.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, uint32_t fill) {
    return __builtin_amdgcn_update_dpp(fill, v, CTRL, ROWS, 0xF, false);
}

// Maximum / minimum / float sum over the 64 lanes, returned in every lane:
// row_shr 1, 2, 4, 8 leave each 16-lane row's result in its lane 15;
// row_bcast 15 and 31 carry it into lane 63, which is read back.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp_u32<0x111, 0xF>(v, 0u));   // row_shr:1
    v = max(v, dpp_u32<0x112, 0xF>(v, 0u));   // row_shr:2
    v = max(v, dpp_u32<0x114, 0xF>(v, 0u));   // row_shr:4
    v = max(v, dpp_u32<0x118, 0xF>(v, 0u));   // row_shr:8
    v = max(v, dpp_u32<0x142, 0xA>(v, 0u));   // row_bcast:15 into rows 1 and 3
    v = max(v, dpp_u32<0x143, 0xC>(v, 0u));   // row_bcast:31 into rows 2 and 3
    return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    constexpr uint32_t F = 0xFFFFFFFFu;
    v = min(v, dpp_u32<0x111, 0xF>(v, F));
    v = min(v, dpp_u32<0x112, 0xF>(v, F));
    v = min(v, dpp_u32<0x114, 0xF>(v, F));
    v = min(v, dpp_u32<0x118, 0xF>(v, F));
    v = min(v, dpp_u32<0x142, 0xA>(v, F));
    v = min(v, dpp_u32<0x143, 0xC>(v, F));
    return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ float wave_sum_dpp(float x) {
    uint32_t v = __float_as_uint(x);
    v = __float_as_uint(__uint_as_float(v) + __uint_as_float(dpp_u32<0x111, 0xF>(v, 0u)));
    v = __float_as_uint(__uint_as_float(v) + __uint_as_float(dpp_u32<0x112, 0xF>(v, 0u)));
    v = __float_as_uint(__uint_as_float(v) + __uint_as_float(dpp_u32<0x114, 0xF>(v, 0u)));
    v = __float_as_uint(__uint_as_float(v) + __uint_as_float(dpp_u32<0x118, 0xF>(v, 0u)));
    v = __float_as_uint(__uint_as_float(v) + __uint_as_float(dpp_u32<0x142, 0xA>(v, 0u)));
    v = __float_as_uint(__uint_as_float(v) + __uint_as_float(dpp_u32<0x143, 0xC>(v, 0u)));
    return __uint_as_float(__builtin_amdgcn_readlane(v, 63));
}

// The wave's view of one token's E logits: expert lane + 64 i in slot i.
// COHERENT: device-scope atomic loads (logits written by other CUs in the
// same kernel).  Absent experts read 0 (their keys are 0 in topk_select).
template <int PER, bool COHERENT = false>
__device__ __forceinline__ void topk_load(const float* __restrict__ L, int E, float (&v)[PER]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        if constexpr (COHERENT) v[i] = (e < E) ? __hip_atomic_load(L + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.f;
        else v[i] = (e < E) ? L[e] : 0.f;
    }
}

// Picks k (1 <= k <= min(E, 64)) of the token whose logits topk_load read and
// returns, in lane j < k, the j-th pick and its gate.
// renorm = 1: gates are a softmax over the k picked; 0: over all E.
// With at most 4 candidates per lane (E <= 256), each lane first sorts its
// candidates (key descending, then id ascending: a total order), so that a
// round only reduces each lane's head: the wave maximum of the heads is the
// next pick's key, the lowest id among the lanes whose head has that key is the
// pick, and that lane drops its head.
template <int PER>
__device__ __forceinline__ void topk_select(const float (&v)[PER], int E, int k, int renorm, int& my_id,
                                            float& my_gate) {
    const int lane = threadIdx.x & 63;
    uint32_t key[PER], kid[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        key[i] = (lane + 64 * i < E) ? order_key(v[i]) : 0u;
        kid[i] = (uint32_t)(lane + 64 * i);
    }
    my_id = -1;
    uint32_t my_key = 0u;
    if constexpr (PER > 4) {
        // many candidates per lane: sorting them costs more than it saves, so
        // each round takes the lane's best by a scan and clears the pick
        for (int j = 0; j < k; ++j) {
            uint32_t best = key[0];
#pragma unroll
            for (int i = 1; i < PER; ++i) best = max(best, key[i]);
            const uint32_t M = wave_max_u32(best);
            // this lane's lowest id holding M (slots ascend in id), or 0xFFFFFFFF
            uint32_t mine = 0xFFFFFFFFu;
#pragma unroll
            for (int i = PER - 1; i >= 0; --i) mine = (key[i] == M) ? kid[i] : mine;
            const uint64_t holders = __ballot(mine != 0xFFFFFFFFu);
            uint32_t id;
            if (__popcll(holders) == 1) id = __builtin_amdgcn_readlane(mine, __builtin_ctzll(holders));
            else id = wave_min_u32(mine);
            const int owner = (int)(id & 63u), slot = (int)(id >> 6);
#pragma unroll
            for (int i = 0; i < PER; ++i)
                if (i == slot && lane == owner) key[i] = 0u;
            if (lane == j) {
                my_id = (int)id;
                my_key = M;
            }
        }
    } else {
        // sorted by compare-exchange of neighbours (PER - 1 passes)
#pragma unroll
        for (int pass = 0; pass < PER - 1; ++pass)
#pragma unroll
            for (int i = 0; i + 1 < PER - pass; ++i) {
                const bool sw = key[i + 1] > key[i] || (key[i + 1] == key[i] && kid[i + 1] < kid[i]);
                const uint32_t ka = key[i], kb = key[i + 1], ia = kid[i], ib = kid[i + 1];
                key[i] = sw ? kb : ka;
                key[i + 1] = sw ? ka : kb;
                kid[i] = sw ? ib : ia;
                kid[i + 1] = sw ? ia : ib;
            }
        for (int j = 0; j < k; ++j) {
            const uint32_t M = wave_max_u32(key[0]);
            const uint64_t holders = __ballot(key[0] == M);
            uint32_t id;
            if (__popcll(holders) == 1) id = __builtin_amdgcn_readlane(kid[0], __builtin_ctzll(holders));
            else id = wave_min_u32(key[0] == M ? kid[0] : 0xFFFFFFFFu);   // equal logits: the lowest id
            if (lane == (int)(id & 63u)) {
#pragma unroll
                for (int i = 0; i + 1 < PER; ++i) {
                    key[i] = key[i + 1];
                    kid[i] = kid[i + 1];
                }
                key[PER - 1] = 0u;
            }
            if (lane == j) {
                my_id = (int)id;
                my_key = M;
            }
        }
    }
    const float top = key_value(__builtin_amdgcn_readfirstlane(my_key));
    const float num = (lane < k) ? expf(key_value(my_key) - top) : 0.f;
    float den;
    if (renorm) {
        den = wave_sum_dpp(num);
    } else {
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if (lane + 64 * i < E) part += expf(v[i] - top);
        den = wave_sum_dpp(part);
    }
    my_gate = num / den;
}

// One token, loaded and picked.
template <int PER, bool COHERENT = false>
__device__ __forceinline__ void topk_one_token(const float* __restrict__ L, int E, int k, int renorm,
                                               int& my_id, float& my_gate) {
    float v[PER];
    topk_load<PER, COHERENT>(L, E, v);
    topk_select<PER>(v, E, k, renorm, my_id, my_gate);
}

}  // namespace moe
