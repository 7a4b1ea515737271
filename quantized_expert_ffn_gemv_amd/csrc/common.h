// Internal helpers shared by the HIP kernels of libmoe.so (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;
constexpr int kGroup = 128;

// ---------------------------------------------------------------- formats

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}

// float -> bf16 bits, round to nearest even; NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// --------------------------------------------------------- wave reductions

__device__ __forceinline__ float wave_sum_xor(float v, int width) {
    for (int off = width >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// ---------------------------------------------------------- launch helpers

struct LaunchCtx {
    hipStream_t stream;
};

}  // namespace moe

// Host-side launchers, one per kernel family.  Each returns a moe status and
// assumes the caller validated the arguments.
namespace moe {

int launch_router_logits(const moe_dims& d, const uint16_t* x, const float* w, const float* bias,
                         float* logits, hipStream_t s);
int launch_topk(const moe_dims& d, const float* logits, int renorm, int32_t* ids, float* gates,
                hipStream_t s);
int launch_slot_lookup(const moe_dims& d, const int32_t* ids, const int32_t* table, int32_t n_slots,
                       int32_t* pair_slot, int32_t* miss, int32_t* n_miss, int32_t* doorbell,
                       uint32_t* last_use, uint32_t step, hipStream_t s);
int launch_permute(const moe_dims& d, const int32_t* ids, int32_t* counts, int32_t* offsets,
                   int32_t* sorted_pairs, int32_t* pair_to_row, int32_t* active, int32_t* n_active,
                   hipStream_t s);

struct FfnArgs {
    moe_dims d;
    int bits;
    const uint16_t* x;
    const int32_t* sorted_pairs;
    const int32_t* counts;
    const int32_t* offsets;
    const int32_t* active;
    const int32_t* n_active;
    moe_qweights w;
    uint16_t* y;
    float* h;          // workspace: float32 [T*k][I]
};

size_t ffn_workspace_bytes(const moe_dims& d, int bits, int algo);
int launch_gateup_gemv(const FfnArgs& a, hipStream_t s);
int launch_down_gemv(const FfnArgs& a, hipStream_t s);
int launch_combine(const moe_dims& d, const uint16_t* y, const int32_t* p2r, const float* gates,
                   const uint16_t* residual, uint16_t* out, hipStream_t s);

}  // namespace moe
