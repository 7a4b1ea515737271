// Internal helpers shared by the HIP kernels of libmoe.so (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;
constexpr int kGroup = 128;
constexpr int kWorkRows = MOE_WORK_TILE_ROWS;      // rows per FFN work-list tile
constexpr int kWorkInts = MOE_WORK_ENTRY_INTS;     // int32 per work-list entry

// Entries a work list needs: sum over experts of ceil(count / kWorkRows), at
// most min(E, T*k) + T*k / kWorkRows.
inline long work_capacity(const moe_dims& d) {
    const long P = (long)d.T * d.k;
    return (d.E < P ? d.E : P) + P / kWorkRows;
}

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

// ------------------------------------------------------ exact code operands
// A code q of BITS bits is OR-ed into the mantissa of the bf16 value 128
// (pattern 0x4300): the result 128 + kLever * q is exact (all values lie in
// [128, 256) where the bf16 spacing is 1).  A dot product with such operands
// is C = 128 * sum(x) + kLever * sum(q x), hence
//   sum((q s + b) x) = (s / kLever) * C + (b - kOffset * s) * sum(x),
// with kOffset = 128 / kLever.  The lever keeps the 128 sum(x) part of C
// within a few times the code part, so the float32 rounding of C stays small
// next to the result: 4-bit codes take the top four mantissa bits (L = 8);
// 2-bit codes take bits 4-5 (L = 16), where the codes at bit 4 of a packed
// word need no shift.  (L = 1 would free a shift for 4-bit codes too, but the
// offset part then outweighs the code part ~17 times and the 2-bit case ~43
// times, which measurably degrades the results.)
template <int BITS> constexpr int kLever = (BITS == 4) ? 8 : 16;
template <int BITS> constexpr float kInvLever = 1.0f / (float)kLever<BITS>;
template <int BITS> constexpr float kOffset = 128.0f / (float)kLever<BITS>;

// Read a value that no kernel writes while this one runs through the scalar
// path: uniform addresses in the constant address space become s_load, which
// waits on its own counter instead of queueing behind vector loads.  Used for
// the routing lists written by earlier kernels.
template <typename T>
__device__ __forceinline__ T ld_scalar(const T* p, size_t i) {
    typedef const __attribute__((address_space(4))) T* cptr;
    return ((cptr)(p))[i];
}

// v >> sh for sh >= 0, v << -sh otherwise (sh is a compile-time constant)
__device__ __forceinline__ uint32_t shift_to(uint32_t v, int sh) { return sh >= 0 ? (v >> sh) : (v << (-sh)); }


// --------------------------------------------------------- wave reductions

__device__ __forceinline__ float wave_sum_xor(float v, int width) {
    for (int off = width >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// Sum N values per lane over all 64 lanes of the wave (N a power of two <= 64)
// by a butterfly transpose: at each of log2(N) stages lanes exchange half of
// their values with the partner lane and add, so the cost is ~N shuffles in
// total instead of N * 6.  Afterwards lane l holds the sum of value index
// (l >> (6 - log2 N)) & (N - 1) ... see wave_transpose_index.
template <int N>
constexpr int log2_of() { return (N <= 1) ? 0 : 1 + log2_of<N / 2>(); }

// One butterfly stage: n values in play, exchanged with the lane at xor `off`.
template <int N, int STAGE>
__device__ __forceinline__ void transpose_stage(float (&v)[N], int lane) {
    constexpr int n = N >> STAGE, off = 32 >> STAGE, h = n / 2;
    const bool upper = (lane & off) != 0;
#pragma unroll
    for (int i = 0; i < h; ++i) {
        const float keep = upper ? v[i + h] : v[i];
        const float send = upper ? v[i] : v[i + h];
        v[i] = keep + __shfl_xor(send, off, kWave);
    }
}

template <int N, int STAGE>
__device__ __forceinline__ void transpose_stages(float (&v)[N], int lane) {
    if constexpr ((N >> STAGE) > 1) {
        transpose_stage<N, STAGE>(v, lane);
        transpose_stages<N, STAGE + 1>(v, lane);
    }
}

template <int N>
__device__ __forceinline__ float wave_transpose_sum(float (&v)[N]) {
    const int lane = threadIdx.x & 63;
    transpose_stages<N, 0>(v, lane);
    // remaining lane bits: plain butterfly over the lanes that share an index
    float r = v[0];
#pragma unroll
    for (int off = 32 >> log2_of<N>(); off > 0; off >>= 1) r += __shfl_xor(r, off, kWave);
    return r;
}

// Value index whose total lane `lane` holds after wave_transpose_sum<N>.
template <int N>
__device__ __forceinline__ int wave_transpose_index(int lane) {
    return (lane >> (6 - log2_of<N>())) & (N - 1);
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
                   int32_t* work, int32_t* n_work, hipStream_t s);

// Outputs of top-k, slot lookup and grouping, for the one-launch dispatch.
struct DispatchArgs {
    int T, H, E, k, P, renorm;
    int32_t* ids;
    float* gates;
    const int32_t* table;
    int n_slots;
    int32_t* pair_slot;
    int32_t* miss;
    int32_t* n_miss;
    int32_t* doorbell;
    uint32_t* last_use;
    uint32_t step;
    int32_t* counts;
    int32_t* offsets;
    int32_t* sorted_pairs;
    int32_t* pair_to_row;
    int32_t* active;
    int32_t* n_active;
    int32_t* work;
    int32_t* n_work;
};
bool dispatch_fused(const moe_dims& d);
int launch_dispatch(const moe_dims& d, const float* logits, const DispatchArgs& a, hipStream_t s);
bool route_dispatch_fused(const moe_dims& d);
int launch_route_dispatch(const moe_dims& d, const uint16_t* x, const float* w, const float* bias, float* logits,
                          const DispatchArgs& a, int32_t* sync, hipStream_t s);

struct FfnArgs {
    moe_dims d;
    int bits;
    const uint16_t* x;
    const int32_t* work;       // work list (entries of kWorkInts int32)
    const int32_t* n_work;     // number of entries (device)
    moe_qweights w;
    uint16_t* y;
    float* h;          // FFN workspace (layout depends on the algorithm)
};

size_t gemv_workspace_bytes(const moe_dims& d);
size_t mfma_workspace_bytes(const moe_dims& d);
size_t ffn_workspace_bytes(const moe_dims& d, int bits, int algo);
bool gemm_supported(const moe_dims& d, int bits);
size_t gemm_workspace_bytes(const moe_dims& d);
int launch_gateup_gemm(const FfnArgs& a, hipStream_t s);
int launch_down_gemm(const FfnArgs& a, hipStream_t s);
int resolve_algo(const moe_dims& d, int bits, int algo);
bool ffn_group_supported(const moe_dims& d, int bits, int algo);
int launch_gateup_gemv(const FfnArgs& a, hipStream_t s);
int launch_down_gemv(const FfnArgs& a, hipStream_t s);
int launch_gateup_mfma(const FfnArgs& a, hipStream_t s);
int launch_down_mfma(const FfnArgs& a, hipStream_t s);
bool dec_gateup_fits(const moe_dims& d);
bool dec_down_fits(const moe_dims& d);
int launch_gateup_dec(const FfnArgs& a, hipStream_t s);
int launch_down_dec(const FfnArgs& a, hipStream_t s);
int launch_down_stream(const FfnArgs& a, hipStream_t s);

// The streaming down (shapes whose h tile does not fit LDS): output rows per
// row block, and workgroups per launch (two per CU of a 256-CU device).  Its
// arrival counters, partial sums and int8 planes of h follow the bf16 planes
// in the workspace; the gate/up kernels clear the counters.
constexpr int kStreamRows = 128;
constexpr int kStreamWaves = 4;     // waves per workgroup, 32 rows each
constexpr int kStreamGrid = 512;
struct SplitSpace {
    int32_t* ctr;       // [cap][H / kStreamRows]
    float* part;        // [2 kStreamGrid][rows_cap][kStreamRows]
    int8_t* hq;         // int8 planes of h [P][I / 128][4][128]
    float* tab;         // their scale and group sum [P][I / 128][2]
    int n_ctr;          // 0: the down projection does not stream at these dims
};
size_t down_split_bytes(const moe_dims& d);
SplitSpace down_split_space(const moe_dims& d, void* ws);
// err: where a down item that gives up waiting writes 1 (NULL: the flag at the
// end of sync).
int launch_ffn_fused_dec(const FfnArgs& a, int32_t* sync, hipStream_t s, int32_t* err = nullptr);
// The fixed scratch of the entry point that allocates nothing (noalloc.hip):
// the current device's counters and workspace, and a fill that zeroes the counters.
int noalloc_scratch(int32_t** sync, void** workspace, size_t* workspace_bytes);
int launch_clear_sync(int32_t* sync, hipStream_t s);
int launch_ffn_fused_dec_shared(const FfnArgs& a, int32_t* sync, hipStream_t s);
int launch_combine(const moe_dims& d, const uint16_t* y, const int32_t* p2r, const float* gates,
                   const uint16_t* residual, uint16_t* out, hipStream_t s);
int launch_combine_shared(const moe_dims& d, const uint16_t* y, const int32_t* p2r, const float* gates,
                          const uint16_t* ys, const uint16_t* x, const float* w, const uint16_t* residual,
                          uint16_t* out, float* gate_out, hipStream_t s);
int launch_zero_point_bias(long n, const uint16_t* scale, const uint8_t* zeros, uint16_t* bias, hipStream_t s);
int launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s);

// Residency tiers (residency.hip).
struct PlanArgs {
    int E, n_hot, n_slots, cap;
    uint32_t step;
    int32_t* slot_of_expert;
    int32_t* expert_of_slot;
    uint32_t* last_use;
    const int32_t* miss;
    const int32_t* n_miss;
    const int32_t* work;
    const int32_t* n_work;
    int32_t* lists;            // [3][cap][kWorkInts]
    int32_t* list_counts;      // [3]
    int32_t* copies;           // [n_slots][2]: (expert, slot)
    int32_t* n_copy;
};
int launch_residency_plan(const PlanArgs& a, hipStream_t s);
int launch_route_counts(const int32_t* counts, uint32_t* freq, int E, hipStream_t s);
int launch_hot_set(const uint32_t* freq, int E, int n, int32_t* hot, hipStream_t s);
int launch_expert_copy(const moe_dims& d, int bits, const moe_qweights& src, const moe_qweights& dst, int n_dst,
                       const int32_t* copies, const int32_t* n_copy, int max_copies, hipStream_t s);

}  // namespace moe
