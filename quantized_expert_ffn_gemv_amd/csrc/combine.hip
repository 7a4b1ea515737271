// Combine + residual (Flash-MoE page, sec. 3: MoE combine fused with the
// residual add).  out[t][n] = bf16(residual[t][n] + sum_j g[t][j] * Y[row][n])
// as a float32 chain of fused multiply-adds in pick order, so the result is a
// deterministic gather (no atomics) and reproducible bit for bit.
#include "common.h"

namespace moe {

// One workgroup per (token, 256 x 8 outputs of its row): the token's k rows
// and gates are workgroup-uniform and arrive through scalar loads; then the
// residual and all k Y pieces are requested together, so the whole kernel is
// two memory round trips.
constexpr int kCombineChunk = 256 * 8;   // outputs per workgroup

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y,
                                                      const int32_t* __restrict__ p2r,
                                                      const float* __restrict__ gates,
                                                      const uint16_t* residual, uint16_t* out, int T,
                                                      int H, int k) {
    const int chunks = (H + kCombineChunk - 1) / kCombineChunk;
    const int t = (int)blockIdx.x / chunks;
    const int n0 = ((int)blockIdx.x % chunks) * kCombineChunk + 8 * (int)threadIdx.x;
    if (t >= T) return;
    const bool live = n0 < H;
    const int P = T * k;
    typedef int int4v __attribute__((ext_vector_type(4)));
    typedef float float4v __attribute__((ext_vector_type(4)));
    const uint4 rv = live ? *reinterpret_cast<const uint4*>(residual + (size_t)t * H + n0) : make_uint4(0, 0, 0, 0);
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
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, s, y, p2r, gates,
                       residual, out, d.T, d.H, d.k);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
