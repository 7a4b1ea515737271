// Weight-format adapter: zero-point groups into this library's scale + bias.
//
// Zero-point quantisation stores w = (q - z) s per group (the "Strata" page,
// sec. 2.2: each group of 128 weights shares a scale and a zero point; the
// laptop page, sec. 4.2, the same form over groups of 32).  The kernels here
// take w = q s + b, so b = -(z s).  z is an integer below 256 and s an fp16
// value (11 significant bits), so z s is exact in float32 and the only
// rounding is the final one to fp16 (nearest, ties to even).
//
// One pass over memory, 5 bytes per entry: each thread converts kPer
// consecutive entries; the grid is capped and strides over the rest.
#include "common.h"

namespace moe {

namespace {

constexpr int kPer = 4;
constexpr int kZpThreads = 256;
constexpr long kZpMaxBlocks = 4096;

__global__ __launch_bounds__(kZpThreads) void zero_point_bias_kernel(long n, const uint16_t* __restrict__ scale,
                                                                      const uint8_t* __restrict__ zeros,
                                                                      uint16_t* __restrict__ bias) {
    const long stride = (long)gridDim.x * kZpThreads * kPer;
    for (long i0 = ((long)blockIdx.x * kZpThreads + threadIdx.x) * kPer; i0 < n; i0 += stride) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const long i = i0 + j;
            if (i < n) {
                // z s rounded to fp16, then the sign flipped as bits (rounding to
                // nearest even is symmetric).  A zero product takes its sign from
                // the float32 product: the compiler folds product and conversion
                // into one mixed-precision FMA with a +0 addend, which would turn
                // the -0 of z = 0 into +0.
                const float p = (float)zeros[i] * f16_bits_to_f32(scale[i]);
                uint32_t h = __builtin_bit_cast(uint16_t, (_Float16)p);
                if (p == 0.0f) h = (__float_as_uint(p) >> 16) & 0x8000u;
                bias[i] = (uint16_t)(h ^ 0x8000u);
            }
        }
    }
}

}  // namespace

int launch_zero_point_bias(long n, const uint16_t* scale, const uint8_t* zeros, uint16_t* bias, hipStream_t s) {
    if (n == 0) return MOE_OK;
    long blocks = (n + (long)kZpThreads * kPer - 1) / ((long)kZpThreads * kPer);
    if (blocks > kZpMaxBlocks) blocks = kZpMaxBlocks;
    hipLaunchKernelGGL(zero_point_bias_kernel, dim3((unsigned)blocks), dim3(kZpThreads), 0, s, n, scale, zeros, bias);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
