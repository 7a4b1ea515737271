// Combine + residual (Flash-MoE page, sec. 3: MoE combine fused with the
// residual add).  out[t][n] = bf16(residual[t][n] + sum_j g[t][j] * Y[row][n])
// as a float32 chain of fused multiply-adds in pick order, so the result is a
// deterministic gather (no atomics) and reproducible bit for bit.
// With a shared expert (the same page's sigmoid gate, read as the gate of an
// always-on shared expert) the chain takes one more step after the picks,
// acc = fmaf(sigmoid(x[t] . w), Ys[t][n], acc), the gate's dot product summed
// in a fixed order inside each workgroup.
#include "common.h"

namespace moe {

// One workgroup per (token, 256 x 8 outputs of its row): the token's k rows
// and gates are workgroup-uniform and arrive through scalar loads; then the
// residual and all k Y pieces are requested together, so the whole kernel is
// two memory round trips.
constexpr int kCombineChunk = 256 * 8;   // outputs per workgroup

// Shared-expert inputs of the combine (unused without one).
struct SharedArgs {
    const uint16_t* ys;     // bf16 [T][H]: the shared expert's output rows
    const uint16_t* x;      // bf16 [T][H]: the layer input
    const float* w;         // fp32 [H]: the gate's weight
    float* gate_out;        // fp32 [T] or null: the gate values used
};

template <bool SHARED>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y,
                                                      const int32_t* __restrict__ p2r,
                                                      const float* __restrict__ gates,
                                                      const uint16_t* residual, uint16_t* out, int T,
                                                      int H, int k, SharedArgs sh) {
    const int chunks = (H + kCombineChunk - 1) / kCombineChunk;
    const int t = (int)blockIdx.x / chunks;
    const int n0 = ((int)blockIdx.x % chunks) * kCombineChunk + 8 * (int)threadIdx.x;
    if (t >= T) return;
    const bool live = n0 < H;
    const int P = T * k;
    typedef int int4v __attribute__((ext_vector_type(4)));
    typedef float float4v __attribute__((ext_vector_type(4)));
    const uint4 rv = live ? *reinterpret_cast<const uint4*>(residual + (size_t)t * H + n0) : make_uint4(0, 0, 0, 0);
    uint4 sv = make_uint4(0, 0, 0, 0);
    float dot = 0.f;                                      // this thread's part of x[t] . w
    if constexpr (SHARED) {
        if (live) sv = *reinterpret_cast<const uint4*>(sh.ys + (size_t)t * H + n0);
        for (int h0 = 8 * (int)threadIdx.x; h0 < H; h0 += kCombineChunk) {
            const uint4 xv = *reinterpret_cast<const uint4*>(sh.x + (size_t)t * H + h0);
            const float4v w0 = *reinterpret_cast<const float4v*>(sh.w + h0);
            const float4v w1 = *reinterpret_cast<const float4v*>(sh.w + h0 + 4);
            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                dot = fmaf(bf16_bits_to_f32(xw[i] & 0xFFFFu), w0[2 * i], dot);
                dot = fmaf(bf16_bits_to_f32(xw[i] >> 16), w0[2 * i + 1], dot);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                dot = fmaf(bf16_bits_to_f32(xw[2 + i] & 0xFFFFu), w1[2 * i], dot);
                dot = fmaf(bf16_bits_to_f32(xw[2 + i] >> 16), w1[2 * i + 1], dot);
            }
        }
    }
    float acc[8];
    // picks in order, 8 at a time: all loads of a batch are in flight together
    for (int j0 = 0; j0 < k; j0 += 8) {
        int row[8];
        float g[8];
        if ((k & 3) == 0) {                               // 16-byte scalar loads of the pick lists
#pragma unroll
            for (int jb = 0; jb < 8; jb += 4) {
                int4v r4 = {-1, -1, -1, -1};
                float4v g4 = {0.f, 0.f, 0.f, 0.f};
                if (j0 + jb < k) {
                    r4 = ld_scalar(reinterpret_cast<const int4v*>(p2r + (size_t)t * k + j0 + jb), 0);
                    g4 = ld_scalar(reinterpret_cast<const float4v*>(gates + (size_t)t * k + j0 + jb), 0);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) { row[jb + i] = r4[i]; g[jb + i] = g4[i]; }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const bool in = j0 + j < k;
                row[j] = in ? ld_scalar(p2r, (size_t)t * k + j0 + j) : -1;
                g[j] = in ? ld_scalar(gates, (size_t)t * k + j0 + j) : 0.f;
            }
        }
        uint4 yv[8];
        uint32_t used = 0;                                // picks with a valid row
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bool ok = row[j] >= 0 && row[j] < P;
            used |= ok ? (1u << j) : 0u;
            yv[j] = (ok && live) ? *reinterpret_cast<const uint4*>(y + (size_t)row[j] * H + n0) : make_uint4(0, 0, 0, 0);
        }
        if (j0 == 0) {                                    // the residual, once its load has had time
            const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] = bf16_bits_to_f32(rw[i] & 0xFFFFu);
                acc[2 * i + 1] = bf16_bits_to_f32(rw[i] >> 16);
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (!((used >> j) & 1u)) continue;
            const uint32_t yw[4] = {yv[j].x, yv[j].y, yv[j].z, yv[j].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] = fmaf(g[j], bf16_bits_to_f32(yw[i] & 0xFFFFu), acc[2 * i]);
                acc[2 * i + 1] = fmaf(g[j], bf16_bits_to_f32(yw[i] >> 16), acc[2 * i + 1]);
            }
        }
    }
    if constexpr (SHARED) {
        // gate: the 256 parts summed by a fixed tree (lanes, then waves in order)
        __shared__ float wave_sum[4];
        __shared__ float gate_s;
        const float part = wave_sum_xor(dot, kWave);
        if ((threadIdx.x & 63) == 0) wave_sum[threadIdx.x >> 6] = part;
        __syncthreads();
        if (threadIdx.x == 0) {
            const float L = ((wave_sum[0] + wave_sum[1]) + wave_sum[2]) + wave_sum[3];
            const float g = 1.f / (1.f + expf(-L));
            gate_s = g;
            if (sh.gate_out && (int)blockIdx.x % chunks == 0) sh.gate_out[t] = g;
        }
        __syncthreads();
        const float g = gate_s;
        const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] = fmaf(g, bf16_bits_to_f32(sw[i] & 0xFFFFu), acc[2 * i]);
            acc[2 * i + 1] = fmaf(g, bf16_bits_to_f32(sw[i] >> 16), acc[2 * i + 1]);
        }
    }
    if (!live) return;
    uint4 o;
    o.x = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
    o.y = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
    o.z = f32_to_bf16_bits(acc[4]) | (f32_to_bf16_bits(acc[5]) << 16);
    o.w = f32_to_bf16_bits(acc[6]) | (f32_to_bf16_bits(acc[7]) << 16);
    *reinterpret_cast<uint4*>(out + (size_t)t * H + n0) = o;
}

int launch_combine(const moe_dims& d, const uint16_t* y, const int32_t* p2r, const float* gates,
                   const uint16_t* residual, uint16_t* out, hipStream_t s) {
    if (d.T == 0) return MOE_OK;
    const long blocks = (long)d.T * ((d.H + kCombineChunk - 1) / kCombineChunk);
    hipLaunchKernelGGL(combine_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, y, p2r, gates,
                       residual, out, d.T, d.H, d.k, SharedArgs{});
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_combine_shared(const moe_dims& d, const uint16_t* y, const int32_t* p2r, const float* gates,
                          const uint16_t* ys, const uint16_t* x, const float* w, const uint16_t* residual,
                          uint16_t* out, float* gate_out, hipStream_t s) {
    if (d.T == 0) return MOE_OK;
    const long blocks = (long)d.T * ((d.H + kCombineChunk - 1) / kCombineChunk);
    hipLaunchKernelGGL(combine_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, y, p2r, gates,
                       residual, out, d.T, d.H, d.k, SharedArgs{ys, x, w, gate_out});
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
