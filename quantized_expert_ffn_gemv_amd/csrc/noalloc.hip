// Fixed device scratch for moe_expert_ffn_fused_noalloc, the FFN entry point
// that allocates nothing (for callers that cannot allocate: code under HIP
// graph capture, tight serving loops).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy, at its own address, for the life of the process.  In host
// code the name `scratch` is only a host-side stand-in for that symbol, so the
// device address is taken once per device with hipGetSymbolAddress (with that
// device current) and kept; kernels and fills get that pointer, never the name.
// Layout: the one-launch FFN's counters (MOE_FFN_SYNC_INTS int32, rounded to
// 256 bytes), then MOE_NOALLOC_WORKSPACE_BYTES of FFN workspace.
#include <mutex>

#include "common.h"

namespace moe {

namespace {

constexpr size_t kSyncBytes = ((size_t)MOE_FFN_SYNC_INTS * 4 + 255) / 256 * 256;
constexpr size_t kScratchBytes = kSyncBytes + (size_t)MOE_NOALLOC_WORKSPACE_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Zero n int32 words (n a multiple of 4, p 16-byte aligned) with vector stores.
__global__ __launch_bounds__(256) void zero_words_kernel(int4* p, int n4) {
    const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i < n4) p[i] = make_int4(0, 0, 0, 0);
}

static_assert(MOE_FFN_SYNC_INTS % 4 == 0, "the fill writes 16-byte words");

}  // namespace

int noalloc_scratch(int32_t** sync, void** workspace, size_t* workspace_bytes) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
    void* p = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        p = g_scratch[dev];
        if (p == nullptr) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ERR_HIP;
            g_scratch[dev] = p;
        }
    }
    *sync = static_cast<int32_t*>(p);
    *workspace = static_cast<uint8_t*>(p) + kSyncBytes;
    *workspace_bytes = (size_t)MOE_NOALLOC_WORKSPACE_BYTES;
    return MOE_OK;
}

// The counters must start at zero: a call whose wait timed out can leave some
// set, so every call clears them first (a kernel, not hipMemsetAsync, so the
// call can be captured into a graph).
int launch_clear_sync(int32_t* sync, hipStream_t s) {
    const int n4 = MOE_FFN_SYNC_INTS / 4;
    hipLaunchKernelGGL(zero_words_kernel, dim3((n4 + 255) / 256), dim3(256), 0, s, reinterpret_cast<int4*>(sync), n4);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
