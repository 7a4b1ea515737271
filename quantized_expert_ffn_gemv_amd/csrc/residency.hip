// Residency tiers of the experts ("Luce Spark" page, sec. 1 and 2; "Strata"
// page, sec. 2.4 and 4.5).
//
// All E experts of a layer sit in pinned host memory (cold); an HBM pool of
// n_slots expert slots holds the resident ones.  Slots [0, n_hot) hold the
// calibrated hot set -- the experts that traffic routes to most, counted by
// route_counts_kernel and ranked by hot_set_kernel -- and are never evicted.
// Slots [n_hot, n_slots) are the warm ring: an expert that a step routes to
// and finds cold takes the least recently used ring slot that this step does
// not use, and is copied into it from host memory by expert_copy_kernel.
//
// Everything runs on the device, so a step never waits for the host: the
// plan kernel reads the step's miss list (written by the slot lookup, which
// also stamped last_use of every slot hit in the step), chooses the victims,
// updates the two slot tables, lists the copies, and splits the FFN work list
// into entries served from slots already resident (list 0), from slots filled
// in this step (list 1) and, when the ring has fewer free slots than the step
// has misses, straight from host memory (list 2).  The caller runs the list-0
// FFN while the copies stream in on a second stream, then lists 1 and 2.
//
// Victims in parallel: taking, for each miss in turn, the eligible ring slot
// with the smallest (last_use, slot) and stamping it with the step (which
// makes it ineligible) picks the eligible slots in ascending (last_use, slot)
// order, since the other slots' keys do not change.  So the i-th miss gets
// the slot of rank i, and each slot's rank is a count over the ring.
#include "common.h"

namespace moe {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / kWave;
constexpr int kMaxE = 1024;
constexpr int kCopyThreads = 256;

__device__ __forceinline__ uint64_t lanes_below() {
    const int lane = threadIdx.x & 63;
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace

__global__ __launch_bounds__(kPlanThreads) void residency_plan_kernel(PlanArgs a) {
    __shared__ uint32_t missed[kMaxE / 32];
    __shared__ int new_slot[kMaxE];
    __shared__ int victim[kMaxE];
    __shared__ int wave_tot[3][kPlanWaves];
    __shared__ int list_base[3];
    __shared__ int n_eligible;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int E = a.E;
    int n_miss = *a.n_miss;
    n_miss = n_miss < 0 ? 0 : (n_miss > E ? E : n_miss);
    for (int i = tid; i < kMaxE / 32; i += kPlanThreads) missed[i] = 0;
    for (int e = tid; e < kMaxE; e += kPlanThreads) new_slot[e] = -1;
    if (tid < 3) list_base[tid] = 0;
    if (tid == 0) n_eligible = 0;
    __syncthreads();
    for (int i = tid; i < n_miss; i += kPlanThreads) {
        const int e = a.miss[i];
        if (e >= 0 && e < E) atomicOr(&missed[e >> 5], 1u << (e & 31));
    }

    // ---- victims: eligible ring slots ranked by (last_use, slot)
    const uint32_t step = a.step;
    for (int s = a.n_hot + tid; s < a.n_slots; s += kPlanThreads) {
        const uint32_t lu = a.last_use[s];
        if (lu == step) continue;
        int rank = 0;
        for (int s2 = a.n_hot; s2 < a.n_slots; ++s2) {
            const uint32_t l2 = a.last_use[s2];
            rank += (l2 != step) && (l2 < lu || (l2 == lu && s2 < s));
        }
        atomicAdd(&n_eligible, 1);
        if (rank < n_miss) victim[rank] = s;
    }
    __syncthreads();
    const int n_copy = n_miss < n_eligible ? n_miss : n_eligible;

    // ---- the i-th missing expert (ascending id) takes the slot of rank i
    // (decided in LDS here; the tables are written last, after every read).
    for (int i = tid; i < n_copy; i += kPlanThreads) {
        const int e = a.miss[i];
        if (e >= 0 && e < E) new_slot[e] = victim[i];
    }
    __syncthreads();

    // ---- split the work list: 0 = resident before this step (expert field
    // -> its slot), 1 = copied in this step (-> its new slot), 2 = still cold
    // (expert id kept).  Order within each list is the work list's.
    const int n_work = *a.n_work;
    const int nw = n_work < 0 ? 0 : (n_work > a.cap ? a.cap : n_work);
    for (int b0 = 0; b0 < nw; b0 += kPlanThreads) {
        const int j = b0 + tid;
        int l = -1, tgt = 0;
        if (j < nw) {
            const int e = a.work[(size_t)j * kWorkInts];
            const bool in_range = e >= 0 && e < E;
            const bool is_miss = in_range && ((missed[e >> 5] >> (e & 31)) & 1u);
            if (!is_miss) {
                l = 0;
                tgt = in_range ? a.slot_of_expert[e] : -1;
            } else if (new_slot[e] >= 0) {
                l = 1;
                tgt = new_slot[e];
            } else {
                l = 2;
                tgt = e;
            }
        }
        int pre[3];
#pragma unroll
        for (int L = 0; L < 3; ++L) {
            const uint64_t m = __ballot(l == L);
            pre[L] = __popcll(m & lanes_below());
            if (lane == 0) wave_tot[L][wid] = __popcll(m);
        }
        __syncthreads();
        if (l >= 0) {
            int off = list_base[l] + pre[l];
            for (int w = 0; w < wid; ++w) off += wave_tot[l][w];
            const int32_t* src = a.work + (size_t)j * kWorkInts;
            int32_t* dst = a.lists + ((size_t)l * a.cap + off) * kWorkInts;
            dst[0] = tgt;
#pragma unroll
            for (int f = 1; f < kWorkInts; ++f) dst[f] = src[f];
        }
        __syncthreads();
        if (tid < 3) {
            int add = 0;
            for (int w = 0; w < kPlanWaves; ++w) add += wave_tot[tid][w];
            list_base[tid] += add;
        }
        __syncthreads();
    }
    if (tid < 3) a.list_counts[tid] = list_base[tid];

    // ---- tables and copy list.  The evicted expert is resident, so it is not
    // missing, and this step does not use its slot (the lookup stamped every
    // slot the step hit), so no two threads touch the same entry.
    for (int i = tid; i < n_copy; i += kPlanThreads) {
        const int e = a.miss[i], s = victim[i];
        if (e < 0 || e >= E) {              // not an id the lookup writes: no copy
            a.copies[2 * i] = -1;
            a.copies[2 * i + 1] = -1;
            continue;
        }
        const int old = a.expert_of_slot[s];
        if (old >= 0 && old < E) a.slot_of_expert[old] = -1;
        a.slot_of_expert[e] = s;
        a.expert_of_slot[s] = e;
        a.last_use[s] = step;
        a.copies[2 * i] = e;
        a.copies[2 * i + 1] = s;
    }
    if (tid == 0) *a.n_copy = n_copy;
}

// freq[e] += counts[e]
__global__ __launch_bounds__(256) void route_counts_kernel(const int32_t* __restrict__ counts, uint32_t* freq,
                                                           int E) {
    const int e = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (e < E) freq[e] += (uint32_t)counts[e];
}

// hot[rank] = e for the n experts of highest count (ties to the lower id)
__global__ __launch_bounds__(kPlanThreads) void hot_set_kernel(const uint32_t* __restrict__ freq, int E, int n,
                                                               int32_t* hot) {
    __shared__ uint32_t f[kMaxE];
    for (int e = threadIdx.x; e < E; e += kPlanThreads) f[e] = freq[e];
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kPlanThreads) {
        const uint32_t v = f[e];
        int rank = 0;
        for (int e2 = 0; e2 < E; ++e2) rank += (f[e2] > v) || (f[e2] == v && e2 < e);
        if (rank < n) hot[rank] = e;
    }
}

struct CopyArgs {
    const uint8_t* src[9];           // per matrix: codes, scales, biases of expert 0
    uint8_t* dst[9];                 // the same runs of slot 0
    size_t bytes[9];                 // one expert's (or slot's) bytes of each run
    const int32_t* copies;
    const int32_t* n_copy;
    int E, n_dst;
};

// Copy i = blockIdx.y: expert copies[2i] of src into slot copies[2i+1] of dst,
// the nine per-expert runs (codes, scales, biases of three matrices) in 16-byte
// words, blockIdx.x striding over them.
__global__ __launch_bounds__(kCopyThreads) void expert_copy_kernel(CopyArgs a) {
    const int i = (int)blockIdx.y;
    if (i >= *a.n_copy) return;
    const int e = a.copies[2 * i], s = a.copies[2 * i + 1];
    if (e < 0 || e >= a.E || s < 0 || s >= a.n_dst) return;
    const long stride = (long)gridDim.x * kCopyThreads;
    for (int r = 0; r < 9; ++r) {
        const uint4* sp = reinterpret_cast<const uint4*>(a.src[r] + (size_t)e * a.bytes[r]);
        uint4* dp = reinterpret_cast<uint4*>(a.dst[r] + (size_t)s * a.bytes[r]);
        const long n16 = (long)(a.bytes[r] / 16);
        long w = (long)blockIdx.x * kCopyThreads + threadIdx.x;
        for (; w + 3 * stride < n16; w += 4 * stride) {
            const uint4 v0 = sp[w], v1 = sp[w + stride], v2 = sp[w + 2 * stride], v3 = sp[w + 3 * stride];
            dp[w] = v0; dp[w + stride] = v1; dp[w + 2 * stride] = v2; dp[w + 3 * stride] = v3;
        }
        for (; w < n16; w += stride) dp[w] = sp[w];
    }
}

int launch_residency_plan(const PlanArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(residency_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_route_counts(const int32_t* counts, uint32_t* freq, int E, hipStream_t s) {
    hipLaunchKernelGGL(route_counts_kernel, dim3((E + 255) / 256), dim3(256), 0, s, counts, freq, E);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_hot_set(const uint32_t* freq, int E, int n, int32_t* hot, hipStream_t s) {
    hipLaunchKernelGGL(hot_set_kernel, dim3(1), dim3(kPlanThreads), 0, s, freq, E, n, hot);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_expert_copy(const moe_dims& d, int bits, const moe_qweights& src, const moe_qweights& dst, int n_dst,
                       const int32_t* copies, const int32_t* n_copy, int max_copies, hipStream_t s) {
    if (max_copies <= 0) return MOE_OK;
    CopyArgs a{};
    for (int m = 0; m < 3; ++m) {
        const size_t N = m < 2 ? d.I : d.H, K = m < 2 ? d.H : d.I;
        a.bytes[3 * m] = N * K * bits / 8;
        a.bytes[3 * m + 1] = a.bytes[3 * m + 2] = N * (K / d.group_size) * 2;
        a.src[3 * m] = src.q[m];
        a.src[3 * m + 1] = reinterpret_cast<const uint8_t*>(src.scale[m]);
        a.src[3 * m + 2] = reinterpret_cast<const uint8_t*>(src.bias[m]);
        // the destination pool is written: its pointers are const only in the struct's type
        a.dst[3 * m] = const_cast<uint8_t*>(dst.q[m]);
        a.dst[3 * m + 1] = reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(dst.scale[m]));
        a.dst[3 * m + 2] = reinterpret_cast<uint8_t*>(const_cast<uint16_t*>(dst.bias[m]));
    }
    a.copies = copies;
    a.n_copy = n_copy;
    a.E = d.E;
    a.n_dst = n_dst;
    // a few workgroups per copy: the host link, not the CUs, sets the rate
    const dim3 grid(32, (unsigned)max_copies);
    hipLaunchKernelGGL(expert_copy_kernel, grid, dim3(kCopyThreads), 0, s, a);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
