// Router logits and top-k gating (Betelgeuse page, MoE primer: the router
// scores every expert from the token's hidden state and only the k best run;
// gates are a softmax renormalised over the k picked).
#include "mfma_ops.h"
#include "router_ops.h"
#include "topk_ops.h"

namespace moe {

// ------------------------------------------------------------ router, small T
// Decode shapes: T <= 64, router_ops.h; one 256-thread workgroup per EB
// experts, all tokens.
template <int EB, int TT, int NJ>
__global__ __launch_bounds__(256) void router_gemv_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ w,
                                                          const float* __restrict__ bias,
                                                          float* __restrict__ logits, int T, int H,
                                                          int E) {
    __shared__ float part[4][EB][TT];
    router_block<EB, TT, NJ>(x, w, bias, logits, H, E, (int)blockIdx.x * EB, 0, T, part, threadIdx.x);
}

// Layers with at most 64 experts: one 1024-thread workgroup per expert, its 16
// waves splitting K (the same sums, in the same order, as the one-launch
// routing's router phase at these sizes).
template <int NJ>
__global__ __launch_bounds__(1024) void router_gemv_wide_kernel(const uint16_t* __restrict__ x,
                                                                const float* __restrict__ w,
                                                                const float* __restrict__ bias,
                                                                float* __restrict__ logits, int T, int H, int E) {
    __shared__ float part[16][8];
    router_block_wide<8, NJ>(x, w, bias, logits, H, E, (int)blockIdx.x, 0, T, part);
}

// ------------------------------------------------------------ router, large T
// Prefill shapes: a 64x64 (tokens x experts) tile per 256-thread workgroup,
// K staged through LDS 32 at a time, 4x4 outputs per thread, float32 FMA.
constexpr int RT_BM = 64, RT_BN = 64, RT_BK = 32;

__global__ __launch_bounds__(256) void router_tiled_kernel(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ w,
                                                            const float* __restrict__ bias,
                                                            float* __restrict__ logits, int T, int H,
                                                            int E) {
    __shared__ float xs[RT_BK][RT_BM + 4];
    __shared__ float ws[RT_BK][RT_BN + 4];
    const int tid = threadIdx.x;
    const int m0 = blockIdx.x * RT_BM;   // tokens
    const int n0 = blockIdx.y * RT_BN;   // experts
    const int ty = tid / 16, tx = tid % 16;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < H; k0 += RT_BK) {
        // x tile: 64 tokens x 32 k bf16 = 256 x 8 values
        {
            int row = tid / 4, col = (tid % 4) * 8;
            int t = m0 + row;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (t < T) v = *reinterpret_cast<const uint4*>(x + (size_t)t * H + k0 + col);
            uint32_t wds[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                xs[col + 2 * i][row] = bf16_bits_to_f32(wds[i] & 0xFFFFu);
                xs[col + 2 * i + 1][row] = bf16_bits_to_f32(wds[i] >> 16);
            }
        }
        // w tile: 64 experts x 32 k float = 256 x 8 values
        {
            int row = tid / 4, col = (tid % 4) * 8;
            int e = n0 + row;
            float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
            if (e < E) {
                a = *reinterpret_cast<const float4*>(w + (size_t)e * H + k0 + col);
                b = *reinterpret_cast<const float4*>(w + (size_t)e * H + k0 + col + 4);
            }
            ws[col + 0][row] = a.x; ws[col + 1][row] = a.y; ws[col + 2][row] = a.z; ws[col + 3][row] = a.w;
            ws[col + 4][row] = b.x; ws[col + 5][row] = b.y; ws[col + 6][row] = b.z; ws[col + 7][row] = b.w;
        }
        __syncthreads();
#pragma unroll 8
        for (int kk = 0; kk < RT_BK; ++kk) {
            float4 av = *reinterpret_cast<const float4*>(&xs[kk][ty * 4]);
            float4 bv = *reinterpret_cast<const float4*>(&ws[kk][tx * 4]);
            float ar[4] = {av.x, av.y, av.z, av.w}, br[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(ar[i], br[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int t = m0 + ty * 4 + i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int e = n0 + tx * 4 + j;
            if (e < E) logits[(size_t)t * E + e] = acc[i][j] + (bias ? bias[e] : 0.f);
        }
    }
}

// Prefill shapes on the matrix cores (v_mfma_f32_16x16x4f32, float32
// operands: x converted exactly from bf16, Wr as given): a workgroup of 4
// waves owns 32 tokens x 32 experts, each wave a 16 x 16 tile; K runs in
// chunks of 64 staged through LDS k-major (so that the 16 lanes of an operand
// read 16 consecutive words), with the global loads of the next RM_P chunks in
// flight in registers (one chunk's arithmetic is far shorter than a round
// trip).  Four accumulators (k steps taken in turn) keep four independent
// MFMA chains in flight; they are added in a fixed order at the end.  Lane
// layout: A lane l row l % 16, k = l / 16; B column l % 16, the
// same k; D rows 4 (l / 16) + i of column l % 16.
constexpr int RM_T = 32, RM_E = 32, RM_K = 64, RM_P = 6;
// Words per LDS row: 49, so that the 8 lanes of a staging write (one column,
// k rows 8 apart) fall in 8 different banks; an operand read (16 columns of 4
// k rows) then meets at most one doubled bank.
constexpr int RM_ROW = 49;

__global__ __launch_bounds__(256) void router_mfma_kernel(const uint16_t* __restrict__ x,
                                                           const float* __restrict__ w,
                                                           const float* __restrict__ bias,
                                                           float* __restrict__ logits, int T, int H, int E) {
    __shared__ float xs[2][RM_K][RM_ROW];                     // two buffers: one barrier per chunk
    __shared__ float ws[2][RM_K][RM_ROW];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int t0 = blockIdx.x * RM_T, e0 = blockIdx.y * RM_E;
    // staging: thread tid loads 8 k of one token row (16 bytes of bf16) and of
    // one expert row (32 bytes of float)
    const int sr = tid >> 3, sk = (tid & 7) * 8;               // row 0..31, k 0..56
    const int st = min(t0 + sr, T - 1), se = min(e0 + sr, E - 1);
    const uint16_t* xsrc = x + (size_t)st * H + sk;
    const float* wsrc = w + (size_t)se * H + sk;
    const int NC = H / RM_K;
    uint4 xr[RM_P];
    float4 wr[RM_P][2];
    auto load = [&](int slot, int c) {
        xr[slot] = *reinterpret_cast<const uint4*>(xsrc + c * RM_K);
        wr[slot][0] = *reinterpret_cast<const float4*>(wsrc + c * RM_K);
        wr[slot][1] = *reinterpret_cast<const float4*>(wsrc + c * RM_K + 4);
    };
    auto put = [&](int slot, int buf) {
        const uint32_t xw[4] = {xr[slot].x, xr[slot].y, xr[slot].z, xr[slot].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            xs[buf][sk + 2 * i][sr] = bf16_bits_to_f32(xw[i] & 0xFFFFu);
            xs[buf][sk + 2 * i + 1][sr] = bf16_bits_to_f32(xw[i] >> 16);
        }
        ws[buf][sk + 0][sr] = wr[slot][0].x; ws[buf][sk + 1][sr] = wr[slot][0].y;
        ws[buf][sk + 2][sr] = wr[slot][0].z; ws[buf][sk + 3][sr] = wr[slot][0].w;
        ws[buf][sk + 4][sr] = wr[slot][1].x; ws[buf][sk + 5][sr] = wr[slot][1].y;
        ws[buf][sk + 6][sr] = wr[slot][1].z; ws[buf][sk + 7][sr] = wr[slot][1].w;
    };
#pragma unroll
    for (int j = 0; j < RM_P; ++j)
        if (j < NC) load(j, j);
    const int m = lane & 15, kq = lane >> 4;
    const int wt = (wv >> 1) * 16, we = (wv & 1) * 16;        // this wave's tile in the workgroup's
    floatx4_t acc[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) acc[a] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    put(0, 0);
    __syncthreads();
    if (RM_P < NC) load(0, RM_P);
    for (int c0 = 0; c0 < NC; c0 += RM_P) {
#pragma unroll
        for (int j = 0; j < RM_P; ++j) {
            // chunk c is in buffer c & 1; chunk c + 1 waits in slot (j + 1) % RM_P
            const int c = c0 + j;
            if (c >= NC) break;
            const int buf = c & 1;
#pragma unroll
            for (int kk = 0; kk < RM_K; kk += 4)
                acc[(kk >> 2) & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(xs[buf][kk + kq][wt + m],
                                                                         ws[buf][kk + kq][we + m],
                                                                         acc[(kk >> 2) & 3], 0, 0, 0);
            if (c + 1 < NC) {
                const int nj = (j + 1) % RM_P;
                put(nj, buf ^ 1);                    // the other buffer: last read before the previous barrier
                if (c + 1 + RM_P < NC) load(nj, c + 1 + RM_P);
            }
            __syncthreads();
        }
    }
    const int e = e0 + we + m;
    if (e < E) {
        const float b = bias ? bias[e] : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + wt + 4 * kq + i;
            if (t < T) logits[(size_t)t * E + e] = ((acc[0][i] + acc[1][i]) + (acc[2][i] + acc[3][i])) + b;
        }
    }
}

int launch_router_logits(const moe_dims& d, const uint16_t* x, const float* w, const float* bias,
                         float* logits, hipStream_t s) {
    if (d.T == 0) return MOE_OK;
    if (d.T <= 64 && d.E <= 64) {
        if ((d.H / 16 + 255) / 256 <= 1)
            hipLaunchKernelGGL(router_gemv_wide_kernel<1>, dim3(d.E), dim3(1024), 0, s, x, w, bias, logits, d.T, d.H, d.E);
        else
            hipLaunchKernelGGL(router_gemv_wide_kernel<2>, dim3(d.E), dim3(1024), 0, s, x, w, bias, logits, d.T, d.H, d.E);
    } else if (d.T <= 64) {
        // each lane covers NJ steps of 4 k within its wave's quarter of H
        const int nj = (d.H / 4 + 255) / 256;
        constexpr int EB = 4, TT = 8;
        dim3 grid((d.E + EB - 1) / EB);
        switch (nj) {
            case 1: hipLaunchKernelGGL((router_gemv_kernel<EB, TT, 1>), grid, dim3(256), 0, s, x, w, bias, logits, d.T, d.H, d.E); break;
            case 2: hipLaunchKernelGGL((router_gemv_kernel<EB, TT, 2>), grid, dim3(256), 0, s, x, w, bias, logits, d.T, d.H, d.E); break;
            case 3: hipLaunchKernelGGL((router_gemv_kernel<EB, TT, 3>), grid, dim3(256), 0, s, x, w, bias, logits, d.T, d.H, d.E); break;
            case 4: hipLaunchKernelGGL((router_gemv_kernel<EB, TT, 4>), grid, dim3(256), 0, s, x, w, bias, logits, d.T, d.H, d.E); break;
            case 5: case 6: hipLaunchKernelGGL((router_gemv_kernel<2, TT, 6>), dim3((d.E + 1) / 2), dim3(256), 0, s, x, w, bias, logits, d.T, d.H, d.E); break;
            default: hipLaunchKernelGGL((router_gemv_kernel<2, TT, 8>), dim3((d.E + 1) / 2), dim3(256), 0, s, x, w, bias, logits, d.T, d.H, d.E); break;
        }
    } else if (d.H % RM_K == 0) {
        dim3 grid((d.T + RM_T - 1) / RM_T, (d.E + RM_E - 1) / RM_E);
        hipLaunchKernelGGL(router_mfma_kernel, grid, dim3(256), 0, s, x, w, bias, logits, d.T, d.H, d.E);
    } else {
        dim3 grid((d.T + RT_BM - 1) / RT_BM, (d.E + RT_BN - 1) / RT_BN);
        hipLaunchKernelGGL(router_tiled_kernel, grid, dim3(256), 0, s, x, w, bias, logits, d.T, d.H,
                           d.E);
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// ------------------------------------------------------------------- top-k
// One wave per token (topk_ops.h); lane j writes the j-th pick.
template <int PER>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                    int k, int renorm, int32_t* __restrict__ ids,
                                                    float* __restrict__ gates) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    int my_id;
    float my_gate;
    topk_one_token<PER>(logits + (size_t)t * E, E, k, renorm, my_id, my_gate);
    if (lane < k) {
        ids[(size_t)t * k + lane] = my_id;
        gates[(size_t)t * k + lane] = my_gate;
    }
}

int launch_topk(const moe_dims& d, const float* logits, int renorm, int32_t* ids, float* gates,
                hipStream_t s) {
    if (d.T == 0) return MOE_OK;
    dim3 grid((d.T + 3) / 4), block(256);
    if (d.E <= 64)
        hipLaunchKernelGGL(topk_kernel<1>, grid, block, 0, s, logits, d.T, d.E, d.k, renorm, ids, gates);
    else if (d.E <= 256)
        hipLaunchKernelGGL(topk_kernel<4>, grid, block, 0, s, logits, d.T, d.E, d.k, renorm, ids, gates);
    else if (d.E <= 512)
        hipLaunchKernelGGL(topk_kernel<8>, grid, block, 0, s, logits, d.T, d.E, d.k, renorm, ids, gates);
    else
        hipLaunchKernelGGL(topk_kernel<16>, grid, block, 0, s, logits, d.T, d.E, d.k, renorm, ids, gates);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
