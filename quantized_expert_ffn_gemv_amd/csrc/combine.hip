// Combine + residual (Flash-MoE page, sec. 3: MoE combine fused with the
// residual add).  out[t][n] = bf16(residual[t][n] + sum_j g[t][j] * Y[row][n])
// as a float32 chain of fused multiply-adds in pick order, so the result is a
// deterministic gather (no atomics) and reproducible bit for bit.
#include "common.h"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y,
                                                      const int32_t* __restrict__ p2r,
                                                      const float* __restrict__ gates,
                                                      const uint16_t* residual, uint16_t* out, int T,
                                                      int H, int k) {
    const int per_tok = H / 8;   // 16-byte pieces per token row
    const long total = (long)T * per_tok;
    for (long idx = (long)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (long)gridDim.x * blockDim.x) {
        const int t = (int)(idx / per_tok), c = (int)(idx % per_tok);
        const uint4 rv = *reinterpret_cast<const uint4*>(residual + (size_t)t * H + c * 8);
        uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
        float acc[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] = bf16_bits_to_f32(rw[i] & 0xFFFFu);
            acc[2 * i + 1] = bf16_bits_to_f32(rw[i] >> 16);
        }
        const int P = T * k;
        for (int j = 0; j < k; ++j) {
            const int row = p2r[t * k + j];
            if (row < 0 || row >= P) continue;
            const float g = gates[t * k + j];
            const uint4 yv = *reinterpret_cast<const uint4*>(y + (size_t)row * H + c * 8);
            uint32_t yw[4] = {yv.x, yv.y, yv.z, yv.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] = fmaf(g, bf16_bits_to_f32(yw[i] & 0xFFFFu), acc[2 * i]);
                acc[2 * i + 1] = fmaf(g, bf16_bits_to_f32(yw[i] >> 16), acc[2 * i + 1]);
            }
        }
        uint4 o;
        o.x = f32_to_bf16_bits(acc[0]) | (f32_to_bf16_bits(acc[1]) << 16);
        o.y = f32_to_bf16_bits(acc[2]) | (f32_to_bf16_bits(acc[3]) << 16);
        o.z = f32_to_bf16_bits(acc[4]) | (f32_to_bf16_bits(acc[5]) << 16);
        o.w = f32_to_bf16_bits(acc[6]) | (f32_to_bf16_bits(acc[7]) << 16);
        *reinterpret_cast<uint4*>(out + (size_t)t * H + c * 8) = o;
    }
}

int launch_combine(const moe_dims& d, const uint16_t* y, const int32_t* p2r, const float* gates,
                   const uint16_t* residual, uint16_t* out, hipStream_t s) {
    if (d.T == 0) return MOE_OK;
    const long total = (long)d.T * (d.H / 8);
    long blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, s, y, p2r, gates,
                       residual, out, d.T, d.H, d.k);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
