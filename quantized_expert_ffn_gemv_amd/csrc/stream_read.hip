// Measurement aid: a plain streaming read of device memory, the practical
// ceiling the expert FFN's weight stream is compared against.  Every lane
// reads 16-byte words in a grid-stride loop with U loads in flight
// (non-temporal, since nothing is read twice); consecutive lanes read
// consecutive words, so each wave instruction covers 1 KB contiguous.  The XOR
// of everything a workgroup read goes to sink[workgroup], so no load can be
// dropped as dead.
#include "common.h"
#include "launch_util.h"

namespace moe {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;

template <int U>
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4* __restrict__ src, long n16,
                                                                    uint32_t* __restrict__ sink) {
    const long stride = (long)gridDim.x * kStreamThreads;
    long i = (long)blockIdx.x * kStreamThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, kWave);
    __shared__ uint32_t part[kStreamThreads / kWave];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

int launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s) {
    const long n16 = (long)(bytes / 16);
    if (n16 == 0) return MOE_OK;
    // one workgroup per compute unit (8 MB in flight over the chip): a sweep of
    // 1 to 16 workgroups per CU and 1 to 16 loads in flight per lane read
    // fastest here, 7.1 TB/s at 1.5 GB; more requests in flight read slower
    long blocks = (long)device_cus();
    const long need = (n16 + (long)kStreamThreads * kStreamUnroll - 1) / ((long)kStreamThreads * kStreamUnroll);
    if (blocks > need) blocks = need;
    if (blocks > MOE_STREAM_SINK_INTS) blocks = MOE_STREAM_SINK_INTS;
    hipLaunchKernelGGL(stream_read_kernel<kStreamUnroll>, dim3((unsigned)blocks), dim3(kStreamThreads), 0, s,
                       static_cast<const u32x4*>(src), n16, sink);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
