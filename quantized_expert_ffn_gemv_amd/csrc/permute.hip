// Resident-slot lookup and grouping of (token, expert) pairs by expert.
//
// Slot lookup follows the Betelgeuse page ("in-stream GPU doorbell"): the
// device resolves hits against the resident table and signals the host only
// on a miss.  Grouping follows the "Strata" page, sec. 2.3: tokens that picked
// the same expert are served by one pass over its weights.
//
// Both run as a single workgroup: at decode sizes they touch a few KB, so one
// CU finishes them in a few microseconds without any grid-wide sync, and the
// integer results are deterministic by construction.  dispatch_kernel runs
// top-k, the lookup and the grouping back to back in one workgroup, so a
// decode step pays one launch for all three.
#include "router_ops.h"
#include "topk_ops.h"

namespace moe {

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for
// every global store of the wave to complete, a memory round trip each time;
// the bodies below write global outputs that no other thread of the
// workgroup reads, so their barriers need only LDS order.
__device__ __forceinline__ void lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Threads (and waves) of every workgroup that runs the bodies below.  A
// constant rather than blockDim: reading blockDim is a scalar load from the
// dispatch packet, a memory round trip each time.
constexpr int kBodyThreads = 1024;
constexpr int kBodyWaves = kBodyThreads / 64;

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int lane = threadIdx.x & 63;
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Inclusive prefix sum over the 64 lanes of a wave on DPP (Hillis-Steele
// within each 16-lane row by row_shr 1, 2, 4, 8, then the row totals carried
// by row_bcast 15 and 31); no LDS round trips.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    v += (int)__builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += (int)__builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += (int)__builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += (int)__builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
    v += (int)__builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15 into rows 1, 3
    v += (int)__builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31 into rows 2, 3
    return v;
}

// Exclusive scans of N counts per thread over the workgroup (at most 16
// waves), with one pair of barriers for all N.  Returns the thread's
// exclusive prefixes in v; total[n] gets the sums.  `wsum` is LDS scratch of
// 16 N ints.
template <int N>
__device__ void block_exclusive_scan(int (&v)[N], int* wsum, int (&total)[N]) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    constexpr int nw = kBodyWaves;
    int incl[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        incl[n] = wave_inclusive_scan(v[n]);
        if (lane == 63) wsum[16 * n + wid] = incl[n];
    }
    lds_sync();
    // the wave totals: lane w reads wave w's, one more wave scan gives every
    // wave its base (all reads in parallel, no chain of LDS round trips)
#pragma unroll
    for (int n = 0; n < N; ++n) {
        const int s = (lane < nw) ? wsum[16 * n + lane] : 0;
        const int ws = wave_inclusive_scan(s);
        const int base = __builtin_amdgcn_readlane(ws - s, wid);
        total[n] = __builtin_amdgcn_readlane(ws, nw - 1);
        v[n] = base + incl[n] - v[n];
    }
    lds_sync();
}

constexpr int kMaxE = 1024;

// ---------------------------------------------------------------- lookup
// Workgroup-wide body (blockDim = 1024): `ids` may live in global memory or
// LDS; `table` is the caller's LDS copy of slot_of_expert (staged early, so
// the lookup waits on no global load); `flag` is LDS scratch of E ints,
// `wsum` of 32.
__device__ void slot_lookup_body(const int32_t* ids, int P, int E, const int* table,
                                 int n_slots, int32_t* __restrict__ pair_slot, int32_t* __restrict__ miss,
                                 int32_t* __restrict__ n_miss, int32_t* doorbell,
                                 uint32_t* __restrict__ last_use, uint32_t step, int* flag, int* wsum) {
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kBodyThreads) flag[e] = 0;
    lds_sync();
    for (int p = tid; p < P; p += kBodyThreads) {
        const int e = ids[p];
        if (e < 0 || e >= E) {
            pair_slot[p] = -1;
            continue;
        }
        const int s = table[e];
        const bool hit = (s >= 0 && s < n_slots);
        pair_slot[p] = hit ? s : -1;
        if (!hit) flag[e] = 1;
        else if (last_use) last_use[s] = step;
    }
    lds_sync();
    int count = 0;
    for (int e0 = 0; e0 < E; e0 += kBodyThreads) {
        const int e = e0 + tid;
        const int f = (e < E) ? flag[e] : 0;
        int pos[1] = {f}, total[1];
        block_exclusive_scan<1>(pos, wsum, total);
        if (f) miss[count + pos[0]] = e;
        count += total[0];
    }
    // the doorbell is a release to the host: every wave's miss-list stores
    // must be complete before it, hence the full barrier (it waits for them)
    if (doorbell) __syncthreads();
    if (tid == 0) {
        *n_miss = count;
        if (doorbell && count > 0) {
            __hip_atomic_store(doorbell, count, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
        }
    }
}

__global__ __launch_bounds__(1024) void slot_lookup_kernel(const int32_t* __restrict__ ids, int P,
                                                           int E, const int32_t* __restrict__ table,
                                                           int n_slots, int32_t* __restrict__ pair_slot,
                                                           int32_t* __restrict__ miss,
                                                           int32_t* __restrict__ n_miss,
                                                           int32_t* doorbell,
                                                           uint32_t* __restrict__ last_use,
                                                           uint32_t step) {
    __shared__ int flag[kMaxE];
    __shared__ int tab[kMaxE];
    __shared__ int wsum[32];
    for (int e = (int)threadIdx.x; e < E; e += kBodyThreads) tab[e] = table[e];
    lds_sync();
    slot_lookup_body(ids, P, E, tab, n_slots, pair_slot, miss, n_miss, doorbell, last_use, step, flag, wsum);
}

int launch_slot_lookup(const moe_dims& d, const int32_t* ids, const int32_t* table, int32_t n_slots,
                       int32_t* pair_slot, int32_t* miss, int32_t* n_miss, int32_t* doorbell,
                       uint32_t* last_use, uint32_t step, hipStream_t s) {
    hipLaunchKernelGGL(slot_lookup_kernel, dim3(1), dim3(1024), 0, s, ids, d.T * d.k, d.E, table,
                       n_slots, pair_slot, miss, n_miss, doorbell, last_use, step);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// --------------------------------------------------------------- permute
// Stable counting sort of the P pairs by expert with 8 waves:
//   1. wave w counts the experts of its contiguous pair range into cnt[w][e];
//   2. one pass over experts: totals, a single exclusive scan (offsets), and
//      per-(wave, expert) starting rows base[w][e] = offsets[e] + earlier waves;
//   3. each wave walks its range in order, 64 pairs at a time; lanes holding
//      the same expert find each other with ballots over the id bits, take
//      rank = earlier equal lanes, and the last of them advances base[w][e].
// Pairs of one expert therefore keep ascending p order.
// The same pass writes the FFN work list: one entry per tile of up to
// kWorkRows consecutive rows of an expert (expert-major), holding the expert,
// the tile's first row, its row count, its index among the expert's tiles and
// the tokens of its rows, so that an FFN workgroup learns everything about its
// tile from one 80-byte read.
constexpr int kPermWaves = 8;

// Workgroup-wide body (blockDim = 1024).  LDS scratch: `cnt` kPermWaves x E
// ints (row stride E), `offs`, `cnts`, `wpos` E ints each, `wsum` 32.
// Slot lookup folded into the grouping (the routing kernels): the same
// outputs as slot_lookup_body, with the miss flags set in the counting pass
// (held in `offs` until the scan) and the miss list placed by the scan.
struct LookupArgs {
    const int* table;                 // LDS copy of slot_of_expert [E]
    int n_slots;
    int32_t* pair_slot;
    int32_t* miss;
    int32_t* n_miss;
    int32_t* doorbell;
    uint32_t* last_use;
    uint32_t step;
};

// R > 0: each wave first loads its whole range of ids into registers (R per
// lane, all loads in flight at once) and walks them from there, so the two
// passes do not wait on a load per 64 pairs; requires P <= kPermWaves * 64 * R.
template <bool LOOKUP, int R = 0>
__device__ void permute_body(const int32_t* ids, int P, int E, int k, int32_t* __restrict__ counts,
                             int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
                             int32_t* __restrict__ pair_to_row, int32_t* __restrict__ active,
                             int32_t* __restrict__ n_active, int32_t* __restrict__ work,
                             int32_t* __restrict__ n_work, int* cnt_flat, int* offs, int* cnts, int* wpos,
                             int* wsum, const LookupArgs& lk = LookupArgs{}) {
    auto cnt = [&](int w, int e) -> int& { return cnt_flat[w * E + e]; };
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int chunk = (P + kPermWaves - 1) / kPermWaves;

    for (int i = tid; i < kPermWaves * E; i += kBodyThreads) cnt_flat[i] = 0;
    if constexpr (LOOKUP)
        for (int e = tid; e < E; e += kBodyThreads) offs[e] = 0;
    lds_sync();
    constexpr int RU = R > 0 ? R : 1;                   // unroll count of the two passes
    int idr[RU];
    if constexpr (R > 0) {
        const int p0 = wid * chunk, p1 = min(P, p0 + chunk);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int p = p0 + lane + 64 * r;
            idr[r] = (wid < kPermWaves && p < p1) ? ids[p] : -1;
        }
    }
    auto id_at = [&](int r, int p) -> int {
        if constexpr (R > 0) return idr[r];
        else return ids[p];
    };
    if (wid < kPermWaves) {
        const int p0 = wid * chunk, p1 = min(P, p0 + chunk);
#pragma unroll RU
        for (int r = 0; r < (R > 0 ? R : (p1 - p0 + 63) / 64); ++r) {
            const int p = p0 + lane + 64 * r;
            if (p >= p1) continue;
            const int e = id_at(r, p);
            const bool ok = e >= 0 && e < E;
            if (ok) atomicAdd(&cnt(wid, e), 1);
            if constexpr (LOOKUP) {
                int sl = -1;
                if (ok) {
                    const int t = lk.table[e];
                    if (t >= 0 && t < lk.n_slots) sl = t;
                }
                lk.pair_slot[p] = sl;
                if (ok && sl < 0) offs[e] = 1;
                if (sl >= 0 && lk.last_use) lk.last_use[sl] = lk.step;
            }
        }
    }
    lds_sync();

    int running = 0, nact = 0, ntile_run = 0, nmiss = 0;
    for (int e0 = 0; e0 < E; e0 += kBodyThreads) {
        const int e = e0 + tid;
        int tot = 0;
        if (e < E)
#pragma unroll
            for (int w = 0; w < kPermWaves; ++w) tot += cnt(w, e);
        const int f = (LOOKUP && e < E) ? offs[e] : 0;     // miss flag
        // one scan of (count | active flag << 16) and (tiles | miss flag << 16):
        // counts sum to at most 4096, tiles to at most 4096 / 16 + 1024, and the
        // flags to at most 1024, so the halves never mix
        const int tiles = (tot + kWorkRows - 1) / kWorkRows;
        int sc[2] = {tot | ((tot > 0 ? 1 : 0) << 16), tiles | (f << 16)}, st[2];
        block_exclusive_scan<2>(sc, wsum, st);
        const int excl = sc[0] & 0xFFFF, apos = sc[0] >> 16, tpos = sc[1] & 0xFFFF, mpos = sc[1] >> 16;
        const int sum = st[0] & 0xFFFF, nsum = st[0] >> 16, tsum = st[1] & 0xFFFF, msum = st[1] >> 16;
        if constexpr (LOOKUP)
            if (f) lk.miss[nmiss + mpos] = e;
        if (e < E) {
            counts[e] = tot;
            offsets[e] = running + excl;
            offs[e] = running + excl;
            cnts[e] = tot;
            wpos[e] = ntile_run + tpos;
            if (tot > 0) active[nact + apos] = e;
            int b = running + excl;
#pragma unroll
            for (int w = 0; w < kPermWaves; ++w) {
                const int c = cnt(w, e);
                cnt(w, e) = b;
                b += c;
            }
        }
        running += sum;
        nact += nsum;
        ntile_run += tsum;
        nmiss += msum;
    }
    if constexpr (LOOKUP) {
        // the doorbell is a release to the host: every wave's miss-list stores
        // must be complete before it, hence the full barrier (it waits for them)
        if (lk.doorbell) __syncthreads();
        if (tid == 0) {
            *lk.n_miss = nmiss;
            if (lk.doorbell && nmiss > 0)
                __hip_atomic_store(lk.doorbell, nmiss, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
        }
    }
    if (tid == 0) {
        offsets[E] = running;
        *n_active = nact;
        *n_work = ntile_run;
    }
    lds_sync();

    if (wid < kPermWaves) {
        const int p0 = wid * chunk, p1 = min(P, p0 + chunk);
#pragma unroll RU
        for (int r = 0; r < (R > 0 ? R : (p1 - p0 + 63) / 64); ++r) {
            const int pb = p0 + 64 * r;
            if (pb >= p1) break;
            const int p = pb + lane;
            const bool live = p < p1;
            int e = live ? id_at(r, p) : -1;
            const bool ok = live && e >= 0 && e < E;
            if (!ok) e = -1;
            // lanes with the same expert id: AND over the id's bits of the
            // ballot (bit set) or its complement (bit clear)
            uint64_t same = __ballot(ok);
#pragma unroll
            for (int b = 0; b < 10; ++b) {
                const uint64_t bal = __ballot(ok && ((e >> b) & 1));
                same &= ((e >> b) & 1) ? bal : ~bal;
            }
            const int rank = __popcll(same & lanemask_lt());
            const int n_same = __popcll(same);
            int row = 0;
            if (ok) row = cnt(wid, e) + rank;
            // all reads of this step happen before the last lane's update
            __builtin_amdgcn_wave_barrier();
            if (ok) {
                sorted_pairs[row] = p;
                pair_to_row[p] = row;
                if (rank == n_same - 1) cnt(wid, e) = row + 1;
                // work list: the row's slot in its expert's tile of kWorkRows rows
                const int off = row - offs[e];
                int32_t* ent = work + (size_t)(wpos[e] + off / kWorkRows) * kWorkInts;
                const int slot = off % kWorkRows;
                const int tok = p / k;
                ent[4 + slot] = tok;
                if (slot == 0) {
                    // header, and the token of slot 0 in the unused slots of a short tile
                    const int rows = min(kWorkRows, cnts[e] - off);
                    ent[0] = e;
                    ent[1] = row;
                    ent[2] = rows;
                    ent[3] = off / kWorkRows;   // the tile's index within its expert
                    for (int j = rows; j < kWorkRows; ++j) ent[4 + j] = tok;
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
}

// ------------------------------------------------- lookup + grouping, one wave
// The same outputs as slot_lookup_body followed by permute_body, computed by
// one wave 64 pairs (or experts) at a time: no workgroup barriers, and LDS
// accesses of one wave complete in program order.  Used for decode batches
// (P <= kWaveMaxP), where the barriers of the workgroup version cost more than
// the work.  LDS: `tab` the resident table, `cnt`, `offs`, `wpos` E ints each,
// `rank` P ints.
constexpr int kWaveMaxP = 64;

__device__ void lookup_permute_wave(const int* ids, int P, int E, int k, const int* tab, int n_slots,
                                    int32_t* __restrict__ pair_slot, int32_t* __restrict__ miss,
                                    int32_t* __restrict__ n_miss, int32_t* doorbell,
                                    uint32_t* __restrict__ last_use, uint32_t step, int32_t* __restrict__ counts,
                                    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
                                    int32_t* __restrict__ pair_to_row, int32_t* __restrict__ active,
                                    int32_t* __restrict__ n_active, int32_t* __restrict__ work,
                                    int32_t* __restrict__ n_work, int* cnt, int* offs, int* wpos, int* rank) {
    const int lane = threadIdx.x & 63;
    // 1. per-expert counters, and miss flags (held in offs until step 3)
    for (int e = lane; e < E; e += 64) {
        cnt[e] = 0;
        offs[e] = 0;
    }
    // 2. lookup, and each pair's stable rank within its expert
    for (int p0 = 0; p0 < P; p0 += 64) {
        const int p = p0 + lane;
        const bool live = p < P;
        int e = live ? ids[p] : -1;
        const bool ok = live && e >= 0 && e < E;
        if (live) {
            int sl = -1;
            if (ok) {
                const int t = tab[e];
                if (t >= 0 && t < n_slots) sl = t;
            }
            pair_slot[p] = sl;
            if (ok && sl < 0) offs[e] = 1;
            if (sl >= 0 && last_use) last_use[sl] = step;
        }
        if (!ok) e = -1;
        uint64_t same = __ballot(ok);
#pragma unroll
        for (int b = 0; b < 10; ++b) {
            const uint64_t bal = __ballot(ok && ((e >> b) & 1));
            same &= ((e >> b) & 1) ? bal : ~bal;
        }
        const int r = __popcll(same & lanemask_lt()), n_same = __popcll(same);
        const int base = ok ? cnt[e] : 0;
        __builtin_amdgcn_wave_barrier();             // every read of cnt before the update
        if (ok) {
            rank[p] = base + r;
            if (r == n_same - 1) cnt[e] = base + n_same;
        }
        __builtin_amdgcn_wave_barrier();
    }
    // 3. per chunk of 64 experts: counts, offsets, active list, miss list and
    // each expert's first work-list entry, from two packed scans (within a
    // chunk, rows sum to at most P < 2^16, tiles to at most P + 64, and the
    // active and missed experts to at most 64 each)
    int running = 0, nact = 0, ntiles = 0, nmiss = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
        const int e = e0 + lane;
        const bool in = e < E;
        const int c = in ? cnt[e] : 0;
        const int f = in ? offs[e] : 0;
        const int tiles = (c + kWorkRows - 1) / kWorkRows;
        const int v1 = c | ((c > 0 ? 1 : 0) << 16), v2 = tiles | (f << 16);
        const int i1 = wave_inclusive_scan(v1), i2 = wave_inclusive_scan(v2);
        const int x1 = i1 - v1, x2 = i2 - v2;
        if (in) {
            const int off = running + (x1 & 0xFFFF);
            counts[e] = c;
            offsets[e] = off;
            offs[e] = off;
            wpos[e] = ntiles + (x2 & 0xFFFF);
            if (c > 0) active[nact + (x1 >> 16)] = e;
            if (f) miss[nmiss + (x2 >> 16)] = e;
        }
        const int t1 = __builtin_amdgcn_readlane(i1, 63), t2 = __builtin_amdgcn_readlane(i2, 63);
        running += t1 & 0xFFFF;
        nact += t1 >> 16;
        ntiles += t2 & 0xFFFF;
        nmiss += t2 >> 16;
    }
    if (lane == 0) {
        offsets[E] = running;
        *n_active = nact;
        *n_work = ntiles;
        *n_miss = nmiss;
        // a release to the host: the miss-list stores above are this wave's
        if (doorbell && nmiss > 0) __hip_atomic_store(doorbell, nmiss, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    // 4. scatter, inverse map and work list
    for (int p = lane; p < P; p += 64) {
        const int e = ids[p];
        if (e < 0 || e >= E) continue;
        const int off = rank[p], row = offs[e] + off;
        sorted_pairs[row] = p;
        pair_to_row[p] = row;
        int32_t* ent = work + (size_t)(wpos[e] + off / kWorkRows) * kWorkInts;
        const int slot = off % kWorkRows, tok = p / k;
        ent[4 + slot] = tok;
        if (slot == 0) {
            // header, and the token of slot 0 in the unused slots of a short tile
            const int rows = min(kWorkRows, cnt[e] - off);
            ent[0] = e;
            ent[1] = row;
            ent[2] = rows;
            ent[3] = off / kWorkRows;
            for (int j = rows; j < kWorkRows; ++j) ent[4 + j] = tok;
        }
    }
}

template <int R>
__global__ __launch_bounds__(1024) void permute_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                       int k, int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ sorted_pairs,
                                                       int32_t* __restrict__ pair_to_row,
                                                       int32_t* __restrict__ active,
                                                       int32_t* __restrict__ n_active,
                                                       int32_t* __restrict__ work,
                                                       int32_t* __restrict__ n_work) {
    __shared__ int cnt[kPermWaves * kMaxE];
    __shared__ int offs[kMaxE];
    __shared__ int cnts[kMaxE];
    __shared__ int wpos[kMaxE];
    __shared__ int wsum[32];
    permute_body<false, R>(ids, P, E, k, counts, offsets, sorted_pairs, pair_to_row, active, n_active, work, n_work,
                           cnt, offs, cnts, wpos, wsum);
}

// ids per lane held in registers by the separate-call permutation (prefill
// sizes: T k <= 32768 pairs)
constexpr int kPermRegIds = 64;

int launch_permute(const moe_dims& d, const int32_t* ids, int32_t* counts, int32_t* offsets,
                   int32_t* sorted_pairs, int32_t* pair_to_row, int32_t* active, int32_t* n_active,
                   int32_t* work, int32_t* n_work, hipStream_t s) {
    const int P = d.T * d.k;
    if (P <= kPermWaves * 64 * kPermRegIds)
        hipLaunchKernelGGL(permute_kernel<kPermRegIds>, dim3(1), dim3(1024), 0, s, ids, P, d.E, d.k, counts,
                           offsets, sorted_pairs, pair_to_row, active, n_active, work, n_work);
    else
        hipLaunchKernelGGL(permute_kernel<0>, dim3(1), dim3(1024), 0, s, ids, P, d.E, d.k, counts,
                           offsets, sorted_pairs, pair_to_row, active, n_active, work, n_work);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// -------------------------------------------------------------- dispatch
// Top-k, slot lookup and grouping in one workgroup of 16 waves: wave w picks
// the experts of tokens w, w + 16, ...; the ids also go to LDS, from where the
// lookup and the counting sort read them.  P = T k <= kDispatchMaxP.
constexpr int kDispatchMaxP = 4096;

template <int PER>
__global__ __launch_bounds__(1024) void dispatch_kernel(const float* __restrict__ logits, DispatchArgs a) {
    __shared__ int ids_s[kDispatchMaxP];
    __shared__ int scratch[kPermWaves * kMaxE];          // counting-sort counts
    __shared__ int offs[kMaxE];
    __shared__ int cnts[kMaxE];
    __shared__ int wpos[kMaxE];
    __shared__ int wsum[32];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    // the resident table is requested first and parked in `cnts` (free until
    // the grouping) once the top-k is done: the lookup then reads only LDS
    const int tab_v = tid < a.E ? a.table[tid] : -1;
    for (int t = wid; t < a.T; t += 16) {
        int my_id;
        float my_gate;
        topk_one_token<PER>(logits + (size_t)t * a.E, a.E, a.k, a.renorm, my_id, my_gate);
        if (lane < a.k) {
            a.ids[(size_t)t * a.k + lane] = my_id;
            a.gates[(size_t)t * a.k + lane] = my_gate;
            ids_s[t * a.k + lane] = my_id;
        }
    }
    if (tid < a.E) cnts[tid] = tab_v;
    lds_sync();
    if (a.P <= kWaveMaxP) {
        if (wid == 0)
            lookup_permute_wave(ids_s, a.P, a.E, a.k, cnts, a.n_slots, a.pair_slot, a.miss, a.n_miss, a.doorbell,
                                a.last_use, a.step, a.counts, a.offsets, a.sorted_pairs, a.pair_to_row, a.active,
                                a.n_active, a.work, a.n_work, scratch, offs, wpos, scratch + kMaxE);
        return;
    }
    const LookupArgs lk{cnts, a.n_slots, a.pair_slot, a.miss, a.n_miss, a.doorbell, a.last_use, a.step};
    permute_body<true>(ids_s, a.P, a.E, a.k, a.counts, a.offsets, a.sorted_pairs, a.pair_to_row, a.active,
                       a.n_active, a.work, a.n_work, scratch, offs, cnts, wpos, wsum, lk);
}

bool dispatch_fused(const moe_dims& d) { return (long)d.T * d.k <= kDispatchMaxP && d.E <= kMaxE; }

// T = 0 still launches: the lookup and grouping outputs (zero counts) are written.
int launch_dispatch(const moe_dims& d, const float* logits, const DispatchArgs& args, hipStream_t s) {
    if (!dispatch_fused(d)) return MOE_ERR_UNSUPPORTED;
    DispatchArgs a = args;
    a.T = d.T; a.E = d.E; a.k = d.k; a.P = d.T * d.k;
    if (d.E <= 64)
        hipLaunchKernelGGL(dispatch_kernel<1>, dim3(1), dim3(1024), 0, s, logits, a);
    else if (d.E <= 256)
        hipLaunchKernelGGL(dispatch_kernel<4>, dim3(1), dim3(1024), 0, s, logits, a);
    else if (d.E <= 512)
        hipLaunchKernelGGL(dispatch_kernel<8>, dim3(1), dim3(1024), 0, s, logits, a);
    else
        hipLaunchKernelGGL(dispatch_kernel<16>, dim3(1), dim3(1024), 0, s, logits, a);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// --------------------------------------------------------- route + dispatch
// The whole routing of a decode batch in one launch.  Grid = (expert blocks)
// x (token groups of kRouteTG tokens); workgroups of 1024 threads:
//   1. every workgroup computes the logits of its 4 EB experts for its token
//      group (router_ops.h, four 256-thread groups side by side);
//   2. the last workgroup to finish a token group (a ticket counter per
//      group) picks the top-k of that group's tokens, one wave per token;
//   3. the last token group to finish (a second ticket; none with one token
//      group) copies all ids to LDS and runs the slot lookup and the
//      counting sort.
// Nothing waits on another workgroup: the late arrivals do the next stage.
// Logits and ids cross workgroups as device-scope atomic stores and loads
// (see ticket()), so they are seen on other CUs and L2 slices.  Counters sit
// kSyncStride ints (256 bytes) apart: arrivals at counters in one cache line
// queue behind each other at the atomic unit, which cost ~2 us per call with
// 256 arrivals.  sync[0] counts token groups done, sync[kSyncStride (1 + g)]
// the expert blocks done for group g; each winner puts its counter back to 0,
// so the buffer is all zero between calls.
constexpr int kRouteTG = 8;
constexpr int kRouteMaxT = 64;
constexpr int kSyncStride = 64;
static_assert(kSyncStride * (1 + kRouteMaxT / kRouteTG) == MOE_DISPATCH_SYNC_INTS, "sync buffer layout");

// Arrive at `counter` (out of `n` arrivals); true in every thread of the last
// workgroup to arrive.  Data handed between workgroups through a ticket is
// written with device-scope atomic stores and read with device-scope atomic
// loads: those bypass the non-coherent per-CU caches, so the only ordering
// needed is that this workgroup's stores have completed before its arrival is
// counted, which the full s_waitcnt gives (no cache flush).
__device__ bool ticket(int32_t* counter, int n, int* winner) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
        *winner = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n - 1;
    __syncthreads();
    return *winner;
}

template <int EB, int NJ, int PER, bool WIDE = false>
__global__ __launch_bounds__(1024) void route_dispatch_kernel(const uint16_t* __restrict__ x,
                                                              const float* __restrict__ w,
                                                              const float* __restrict__ bias,
                                                              float* __restrict__ logits, DispatchArgs a,
                                                              int32_t* __restrict__ sync) {
    // tokens per pass of the router: fewer for wide H, whose weight and
    // activation registers would not fit the 1024-thread budget
    constexpr int TT = NJ >= 6 ? kRouteTG / 2 : kRouteTG;
    __shared__ float part[4][4][EB][TT];
    __shared__ float partw[16][kRouteTG];
    __shared__ int ids_s[kDispatchMaxP];
    __shared__ int scratch[kPermWaves * kMaxE];
    __shared__ int offs[kMaxE];
    __shared__ int cnts[kMaxE];
    __shared__ int wpos[kMaxE];
    __shared__ int wsum[32];
    __shared__ int winner;
    const int tid = threadIdx.x, sub = tid >> 8, lane = tid & 63, wid = tid >> 6;
    const int tg = blockIdx.y;
    const int tb = tg * kRouteTG, te = min(a.T, tb + kRouteTG);
    int32_t* group_counter = sync + kSyncStride * (1 + tg);

    // 1. logits of this (expert block, token group)
    if constexpr (WIDE)
        router_block_wide<kRouteTG, NJ, true>(x, w, bias, logits, a.H, a.E, (int)blockIdx.x, tb, te, partw);
    else
        router_block<EB, TT, NJ, true>(x, w, bias, logits, a.H, a.E, ((int)blockIdx.x * 4 + sub) * EB, tb, te,
                                       part[sub], tid & 255);
    if (!ticket(group_counter, (int)gridDim.x, &winner)) return;
    // the resident table, requested now, parked in `cnts` for the lookup
    const int tab_v = tid < a.E ? a.table[tid] : -1;

    // 2. top-k of the group's tokens.  With one token group this workgroup is
    // also the last group: its ids go straight to LDS and the second ticket
    // is skipped.
    const bool single = gridDim.y == 1;
    if (wid < te - tb) {
        const int t = tb + wid;
        int my_id;
        float my_gate;
        topk_one_token<PER, true>(logits + (size_t)t * a.E, a.E, a.k, a.renorm, my_id, my_gate);
        if (lane < a.k) {
            if (single) {
                a.ids[(size_t)t * a.k + lane] = my_id;
                ids_s[t * a.k + lane] = my_id;
            } else {
                __hip_atomic_store(a.ids + (size_t)t * a.k + lane, my_id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            a.gates[(size_t)t * a.k + lane] = my_gate;
        }
    }
    if (tid == 0) __hip_atomic_store(group_counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!single) {
        if (!ticket(&sync[0], (int)gridDim.y, &winner)) return;
        // 3. lookup and grouping over all pairs
        for (int p = tid; p < a.P; p += kBodyThreads)
            ids_s[p] = __hip_atomic_load(a.ids + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid < a.E) cnts[tid] = tab_v;
    lds_sync();
    if (a.P <= kWaveMaxP) {
        if (wid == 0) {
            lookup_permute_wave(ids_s, a.P, a.E, a.k, cnts, a.n_slots, a.pair_slot, a.miss, a.n_miss, a.doorbell,
                                a.last_use, a.step, a.counts, a.offsets, a.sorted_pairs, a.pair_to_row, a.active,
                                a.n_active, a.work, a.n_work, scratch, offs, wpos, scratch + kMaxE);
            if (lane == 0 && !single) __hip_atomic_store(&sync[0], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        return;
    }
    const LookupArgs lk{cnts, a.n_slots, a.pair_slot, a.miss, a.n_miss, a.doorbell, a.last_use, a.step};
    permute_body<true>(ids_s, a.P, a.E, a.k, a.counts, a.offsets, a.sorted_pairs, a.pair_to_row, a.active,
                       a.n_active, a.work, a.n_work, scratch, offs, cnts, wpos, wsum, lk);
    if (tid == 0 && !single) __hip_atomic_store(&sync[0], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

bool route_dispatch_fused(const moe_dims& d) {
    return d.T >= 1 && d.T <= kRouteMaxT && dispatch_fused(d) && (d.H / 4 + 255) / 256 <= 8;
}

template <int EB, int NJ>
static void rd_go(const moe_dims& d, const uint16_t* x, const float* w, const float* bias, float* logits,
                  const DispatchArgs& a, int32_t* sync, hipStream_t s) {
    const dim3 grid((unsigned)((d.E + 4 * EB - 1) / (4 * EB)), (unsigned)((d.T + kRouteTG - 1) / kRouteTG));
    if (d.E <= 64)
        hipLaunchKernelGGL((route_dispatch_kernel<EB, NJ, 1>), grid, dim3(1024), 0, s, x, w, bias, logits, a, sync);
    else if (d.E <= 256)
        hipLaunchKernelGGL((route_dispatch_kernel<EB, NJ, 4>), grid, dim3(1024), 0, s, x, w, bias, logits, a, sync);
    else if (d.E <= 512)
        hipLaunchKernelGGL((route_dispatch_kernel<EB, NJ, 8>), grid, dim3(1024), 0, s, x, w, bias, logits, a, sync);
    else
        hipLaunchKernelGGL((route_dispatch_kernel<EB, NJ, 16>), grid, dim3(1024), 0, s, x, w, bias, logits, a, sync);
}

int launch_route_dispatch(const moe_dims& d, const uint16_t* x, const float* w, const float* bias, float* logits,
                          const DispatchArgs& args, int32_t* sync, hipStream_t s) {
    if (!route_dispatch_fused(d)) return MOE_ERR_UNSUPPORTED;
    DispatchArgs a = args;
    a.T = d.T; a.H = d.H; a.E = d.E; a.k = d.k; a.P = d.T * d.k;
    // layers with at most 64 experts: one expert per workgroup (16 waves split K),
    // else one expert per 256-thread group (NJ 256-wide steps cover a quarter of H)
    if (d.E <= 64) {
        const dim3 grid((unsigned)d.E, (unsigned)((d.T + kRouteTG - 1) / kRouteTG));
        const int njw = (d.H / 16 + 255) / 256;
        if (njw <= 1)
            hipLaunchKernelGGL((route_dispatch_kernel<1, 1, 1, true>), grid, dim3(1024), 0, s, x, w, bias, logits, a, sync);
        else
            hipLaunchKernelGGL((route_dispatch_kernel<1, 2, 1, true>), grid, dim3(1024), 0, s, x, w, bias, logits, a, sync);
        return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
    }
    const int nj = (d.H / 4 + 255) / 256;
    switch (nj) {
        case 1: rd_go<1, 1>(d, x, w, bias, logits, a, sync, s); break;
        case 2: rd_go<1, 2>(d, x, w, bias, logits, a, sync, s); break;
        case 3: rd_go<1, 3>(d, x, w, bias, logits, a, sync, s); break;
        case 4: rd_go<1, 4>(d, x, w, bias, logits, a, sync, s); break;
        case 5: case 6: rd_go<1, 6>(d, x, w, bias, logits, a, sync, s); break;
        default: rd_go<1, 8>(d, x, w, bias, logits, a, sync, s); break;
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
