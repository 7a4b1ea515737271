// Router logits for decode batches (Betelgeuse page, MoE primer: the router
// scores every expert from the token's hidden state):
//   logits[t][e] = sum_h x[t][h] * w[e][h] + bias[e]      (float32)
#pragma once

#include "common.h"

namespace moe {

// One 256-thread group (stid = 0..255) computes experts [e0, e0 + EB) for
// tokens [tb, te).  Its 4 waves split K into quarters and each lane covers 4
// consecutive k per 256-wide step (NJ steps).  All router-weight loads are
// issued up front (EB * NJ float4 per lane), then tokens are processed TT at a
// time with their activation loads independent of each other, so the group
// is a couple of memory latencies long instead of a chain of dependent loads.
// Partial sums are reduced across the wave with xor shuffles and across the 4
// waves through `part` (LDS, this group's own).  Contains __syncthreads():
// every group of the workgroup must call it with the same token range.
// COHERENT: store the logits with device-scope atomic stores, which reach the
// device's point of coherence without a cache write-back (for readers on
// other CUs in the same kernel).
template <int EB, int TT, int NJ, bool COHERENT = false>
__device__ __forceinline__ void router_block(const uint16_t* __restrict__ x, const float* __restrict__ w,
                                             const float* __restrict__ bias, float* __restrict__ logits, int H,
                                             int E, int e0, int tb, int te, float (*part)[EB][TT], int stid) {
    const int lane = stid & 63, wv = stid >> 6;
    const int kq = H / 4;                        // this wave's quarter of K
    const int kbase = wv * kq + lane * 4;
    float4 wr[EB][NJ];
#pragma unroll
    for (int a = 0; a < EB; ++a)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int k = kbase + 256 * j;
            const bool ok = (e0 + a < E) && (lane * 4 + 256 * j < kq);
            wr[a][j] = ok ? *reinterpret_cast<const float4*>(w + (size_t)(e0 + a) * H + k)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    for (int t0 = tb; t0 < te; t0 += TT) {
        uint2 xv[TT][NJ];
#pragma unroll
        for (int b = 0; b < TT; ++b)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const bool ok = (t0 + b < te) && (lane * 4 + 256 * j < kq);
                xv[b][j] = ok ? *reinterpret_cast<const uint2*>(x + (size_t)(t0 + b) * H + kbase + 256 * j)
                              : make_uint2(0, 0);
            }
        float acc[EB][TT];
#pragma unroll
        for (int b = 0; b < TT; ++b) {
#pragma unroll
            for (int a = 0; a < EB; ++a) acc[a][b] = 0.f;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const float x0 = bf16_bits_to_f32(xv[b][j].x & 0xFFFFu), x1 = bf16_bits_to_f32(xv[b][j].x >> 16);
                const float x2 = bf16_bits_to_f32(xv[b][j].y & 0xFFFFu), x3 = bf16_bits_to_f32(xv[b][j].y >> 16);
#pragma unroll
                for (int a = 0; a < EB; ++a) {
                    float s = acc[a][b];
                    s = fmaf(x0, wr[a][j].x, s);
                    s = fmaf(x1, wr[a][j].y, s);
                    s = fmaf(x2, wr[a][j].z, s);
                    s = fmaf(x3, wr[a][j].w, s);
                    acc[a][b] = s;
                }
            }
        }
        float flat[EB * TT];
#pragma unroll
        for (int a = 0; a < EB; ++a)
#pragma unroll
            for (int b = 0; b < TT; ++b) flat[a * TT + b] = acc[a][b];
        const float tot = wave_transpose_sum<EB * TT>(flat);
        const int idx = wave_transpose_index<EB * TT>(lane);
        if ((lane & ((64 / (EB * TT)) - 1)) == 0) part[wv][idx / TT][idx % TT] = tot;
        __syncthreads();
        if (stid < EB * TT) {
            const int a = stid / TT, b = stid % TT;
            if (e0 + a < E && t0 + b < te) {
                const float v = (part[0][a][b] + part[1][a][b]) + (part[2][a][b] + part[3][a][b]);
                const float out = v + (bias ? bias[e0 + a] : 0.f);
                float* dst = logits + (size_t)(t0 + b) * E + e0 + a;
                if constexpr (COHERENT) __hip_atomic_store(dst, out, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                else *dst = out;
            }
        }
        __syncthreads();
    }
}

// The whole 1024-thread workgroup on one expert e0 (layers with few experts,
// where one expert per 256-thread group would leave most of the chip idle):
// its 16 waves split K into 16 parts, each lane covering 4 consecutive k per
// 256-wide step (NJ steps); partial sums are reduced across the wave with
// xor shuffles and across the 16 waves through `part` in a fixed order.  The
// same loads-first structure as router_block; contains __syncthreads().
template <int TT, int NJ, bool COHERENT = false>
__device__ __forceinline__ void router_block_wide(const uint16_t* __restrict__ x, const float* __restrict__ w,
                                                  const float* __restrict__ bias, float* __restrict__ logits,
                                                  int H, int E, int e0, int tb, int te, float (*part)[TT]) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int kp = H / 16;                       // this wave's part of K
    const int kbase = wv * kp + lane * 4;
    float4 wr[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const bool ok = (e0 < E) && (lane * 4 + 256 * j < kp);
        wr[j] = ok ? *reinterpret_cast<const float4*>(w + (size_t)e0 * H + kbase + 256 * j)
                   : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    for (int t0 = tb; t0 < te; t0 += TT) {
        uint2 xv[TT][NJ];
#pragma unroll
        for (int b = 0; b < TT; ++b)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const bool ok = (t0 + b < te) && (lane * 4 + 256 * j < kp);
                xv[b][j] = ok ? *reinterpret_cast<const uint2*>(x + (size_t)(t0 + b) * H + kbase + 256 * j)
                              : make_uint2(0, 0);
            }
        float acc[TT];
#pragma unroll
        for (int b = 0; b < TT; ++b) {
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                s = fmaf(bf16_bits_to_f32(xv[b][j].x & 0xFFFFu), wr[j].x, s);
                s = fmaf(bf16_bits_to_f32(xv[b][j].x >> 16), wr[j].y, s);
                s = fmaf(bf16_bits_to_f32(xv[b][j].y & 0xFFFFu), wr[j].z, s);
                s = fmaf(bf16_bits_to_f32(xv[b][j].y >> 16), wr[j].w, s);
            }
            acc[b] = s;
        }
        const float tot = wave_transpose_sum<TT>(acc);
        const int idx = wave_transpose_index<TT>(lane);
        if ((lane & ((64 / TT) - 1)) == 0) part[wv][idx] = tot;
        __syncthreads();
        if (tid < TT && e0 < E && t0 + tid < te) {
            float v = 0.f;
#pragma unroll
            for (int q = 0; q < 16; ++q) v += part[q][tid];
            const float out = v + (bias ? bias[e0] : 0.f);
            float* dst = logits + (size_t)(t0 + tid) * E + e0;
            if constexpr (COHERENT) __hip_atomic_store(dst, out, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else *dst = out;
        }
        __syncthreads();
    }
}

}  // namespace moe
