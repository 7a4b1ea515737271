// Decode-sized expert FFN on the matrix cores: one work-list tile (up to 16
// tokens of one expert) per workgroup, its activations staged once in LDS.
//
// The exact code operands and the per-group fold are those of mfma_ops.h.
// What differs from the kernels in ffn_mfma.hip:
//   * the tile's activations (gate/up: x rows; down: the three bf16 planes of
//     h) and the item's scales and biases go from HBM/L2 straight into LDS
//     with direct-to-LDS loads (global_load_lds_dwordx4), issued before the
//     code ring and holding no registers; gate/up then rewrites its x tile
//     once into the pair order of the code operands;
//   * activations are the A operand (rows = tokens) and the codes the B
//     operand (columns = weight rows): a lane's accumulators belong to one
//     weight row, so each lane folds with a single scale pair per group;
//   * the per-group activation sums come from an MFMA with an all-ones B
//     operand on the same LDS data;
//   * one item per workgroup (no persistent loop): the grid covers every
//     possible tile, and workgroups past the device-side tile count exit.
// Gate/up: RW waves split the item's rows (16 gate + 16 up rows each) and
// KS = 4 / RW waves split K; partial sums over K are added in LDS in a fixed
// order.  Down: each wave owns RT tiles of 16 output rows over all of K.
// h leaves gate/up in the layout of the other matrix-core kernels (three bf16
// planes in code pair order plus 16-row partial sums), so either down kernel
// can follow either gate/up kernel.
#include <algorithm>

#include "launch_util.h"
#include "mfma_ops.h"

namespace moe {

namespace {

// Largest LDS a decode item may take (two workgroups per CU at 160 KB, with
// room for the rest); bigger shapes use the kernels of ffn_mfma.hip.
constexpr size_t kDecLdsLimit = 80 * 1024;

// One-launch FFN (ffn_fused_dec_kernel): work-list entries per chunk of the
// grid, the per-entry counters in `sync` (one 128-byte line each), the
// time-out flag after them, and the bound on a down item's wait (polls of
// about 0.5 us: some 10 ms in all, against waits of a few us).
constexpr int kFfnChunk = 64;
constexpr int kFfnStride = 32;
constexpr int kFfnMaxEntries = MOE_FFN_SYNC_INTS / kFfnStride - 1;
constexpr int kFfnErr = kFfnMaxEntries * kFfnStride;
constexpr int kFfnSpinMax = 20000;

struct DecParams {
    const uint16_t* x;
    const int32_t* work;
    const int32_t* n_work;
    const uint8_t* qa; const uint16_t* sa; const uint16_t* ba;   // gate, or down
    const uint8_t* qb; const uint16_t* sb; const uint16_t* bb;   // up
    uint16_t* hp;       // bf16 planes [3][P][I]
    float* hpart;       // [P][I/16]
    uint16_t* y;        // [P][H]
    int T, H, I, E, P;
    int ipe;            // items per work-list entry
    int cap;            // work-list capacity (entries); the grid covers cap + n_shared
    int rows_cap;       // token rows of the LDS tile: min(16, T)
    int n_shared;       // shared-expert tiles after the routed entries (0: none)
    int shared_row0;    // first row of the shared expert's rows (the routed pair count)
    int32_t* split_ctr; // streaming down: arrival counters [cap][ipe] (gate/up clears them)
    float* split_part;  // streaming down: partial sums [2 G][rows_cap][RI]
    const int8_t* hq;   // streaming down: int8 planes of h [P][I / 128][4][128]
    const float* htab;  // streaming down: (hs, X) per row and group [P][I / 128][2]
    int n_split_ctr;    // gate/up: counters to clear (0: none)
    int split_plan_off; // streaming down: LDS offset of the work split's tables
};

__host__ __device__ constexpr size_t round_dma(size_t b) { return (b + kDma - 1) / kDma * kDma; }

// Item of a decode launch: work-list entry and row block of blockIdx.x; the
// entry's expert, first sorted row, row count (n = 0: nothing to do) and the
// tokens of its rows, spread over lanes (lane l holds the token of row
// l % 16, clamped into [0, T)).  The whole entry is read with the count,
// before any branch, so all of it arrives in one scalar round trip (every
// entry below the grid's capacity is allocated, whatever the count).
// With a shared expert, entries n_work .. n_work + n_shared - 1 are its tiles,
// made here rather than read: expert E - 1 (the last of the weight arrays),
// tokens 16 j .. 16 j + 15 of tile j, rows shared_row0 + token.
struct DecItem {
    int entry, rb, e, row0, n;
    int tokv;
};

template <bool SHARED = false>
__device__ __forceinline__ DecItem dec_item_at(const DecParams& p, int entry, int rb) {
    typedef int int4v __attribute__((ext_vector_type(4)));
    DecItem it;
    it.entry = entry;
    it.rb = rb;
    const int re = it.entry < p.cap ? it.entry : p.cap - 1;      // grids round entries up
    const int4v* ent = reinterpret_cast<const int4v*>(p.work + (size_t)re * kWorkInts);
    const int n_work = ld_scalar(p.n_work, 0);
    int4v v[kWorkInts / 4];
#pragma unroll
    for (int i = 0; i < kWorkInts / 4; ++i) v[i] = ld_scalar(ent, i);
    if constexpr (SHARED) {
        // The values are taken here, so the loads stay unconditional and fly
        // with the count's (else the compiler sinks them under the shared-tile
        // test below, one more scalar round trip per item).
#pragma unroll
        for (int i = 0; i < kWorkInts / 4; ++i) asm volatile("" : "+s"(v[i]));
    }
    const int l16 = threadIdx.x & 15;
    int tok = v[1][0];
#pragma unroll
    for (int j = 1; j < kWorkRows; ++j) tok = (l16 == j) ? v[1 + j / 4][j % 4] : tok;
    int e = v[0][0], row0 = v[0][1], n = v[0][2];
    bool shared = false;
    if constexpr (SHARED) {
        const int sj = it.entry - n_work;             // shared tile index, if in [0, n_shared)
        shared = sj >= 0 && sj < p.n_shared;
        if (shared) {
            e = p.E - 1;
            row0 = p.shared_row0 + 16 * sj;
            n = min(16, p.T - 16 * sj);
            tok = 16 * sj + l16;
        }
    }
    it.tokv = (tok >= 0 && tok < p.T) ? tok : 0;
    const bool ok = (it.entry < n_work || shared) && e >= 0 && e < p.E && row0 >= 0 && n >= 1 &&
                    n <= p.rows_cap && row0 + n <= p.P;
    it.e = ok ? e : 0;
    it.row0 = ok ? row0 : 0;
    it.n = ok ? n : 0;
    return it;
}

// Workgroups are dispatched to the 8 XCDs in turn (workgroup b to XCD b % 8).
// Slot r of a range of 8 ipe m workgroups takes entry (r / 8 / ipe) 8 + r % 8
// and row block (r / 8) % ipe: the items of entry e all run on one XCD, so its
// activation or h tile is fetched into that XCD's L2 once and hit by the other
// items.
template <bool SHARED = false>
__device__ __forceinline__ DecItem dec_item_xcd(const DecParams& p, int entry0, int r) {
    const int xcd = r & 7, s = r >> 3;
    return dec_item_at<SHARED>(p, entry0 + (s / p.ipe) * 8 + xcd, s % p.ipe);
}

// The activation tile in LDS: rows of `rowb` bytes, each group of 128 along K
// a run of 16 chunks of 16 bytes (8 values in natural order), the chunks
// XOR-swizzled by the row's low 4 bits so that the 16 rows a quarter-wave
// reads at once hit 16 bank groups.  Chunk c of group g of row j:
__device__ __forceinline__ int tile_off(int j, int g, int c, int rowb) {
    return j * rowb + g * 256 + 16 * (c ^ (j & 15));
}

// Direct-to-LDS staging of `n` rows of such a tile (`rows_cap` rows of room):
// piece i of the tile (1 KB) is loaded by one wave, lane l filling slot
// 64 i + l.  src(j, g, c) is the global address of chunk c of group g of row
// j; slots of rows past n reload a chunk of row 0 into unused room.
template <bool COH = false, typename Src>
__device__ __forceinline__ void dma_tile(uint8_t* tile, int n, int rowb, int wid, int lane, Src src) {
    const int chunks_row = rowb / 16;
    const int pieces = (n * rowb + kDma - 1) / kDma;
    for (int i = wid; i < pieces; i += 4) {
        const int slot = i * (kDma / 16) + lane;
        int j = slot / chunks_row;
        const int r = slot - j * chunks_row, g = r >> 4, cs = r & 15;
        j = j < n ? j : 0;
        dma16<COH>(src(j, g, cs ^ (j & 15)), tile + i * kDma);
    }
}

// acc += (s / L) C + (b - (128 / L) s) X for one fp16 scale and bias.
template <int BITS>
__device__ __forceinline__ void fold(floatx4_t& acc, const floatx4_t& C, uint32_t s16, uint32_t b16,
                                     const floatx4_t& X) {
    const float sv = f16_bits_to_f32(s16), bv = f16_bits_to_f32(b16);
    const float s1 = sv * kInvLever<BITS>, b1 = fmaf(-kOffset<BITS>, sv, bv);
    acc[0] = fmaf(s1, C[0], fmaf(b1, X[0], acc[0]));
    acc[1] = fmaf(s1, C[1], fmaf(b1, X[1], acc[1]));
    acc[2] = fmaf(s1, C[2], fmaf(b1, X[2], acc[2]));
    acc[3] = fmaf(s1, C[3], fmaf(b1, X[3], acc[3]));
}

constexpr uint32_t kOnesBf16 = 0x3F803F80u;   // two bf16 ones

}  // namespace

// --------------------------------------------------------------- gate / up
// Item = (work-list tile, block of 16 RW rows of gate and of up).  Wave
// (wr, wk) = (wid / KS, wid % KS) computes rows 16 wr .. +16 of the block
// (pair order) over its share of the K groups, with a D-deep register ring of
// code loads.  LDS: the x tile [rows_cap][H] bf16, then the raw fp16 scales
// and biases of the block's gate and up rows, [RI][NG] each; after the loop
// the first 8 KB holds the partial sums over K.
// COH: h leaves through device-scope stores (read by down items of the same
// launch) and without the 16-row partial sums (only the non-staged down
// kernel reads those).
template <int BITS, int RW, int D, bool COH, int SPG = 1>
__device__ __forceinline__ void gateup_item(const DecParams& p, const DecItem& it, uint8_t* smem) {
    constexpr int KS = 4 / RW;
    constexpr int LB = 128 * BITS / 8 / 4;     // code bytes per lane per group
    constexpr bool TR = SPG > 1;               // steps swapped: one quarter of the 128 codes per step
    constexpr int LW = TR ? 4 : LB / 4;        // code words per lane per group
    constexpr int SST = 4 / SPG;               // MFMA steps per scale group
    constexpr int RI = 16 * RW;                // gate (and up) rows per item
    if (it.n == 0) return;
    const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, q = lane >> 4;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wid / KS, wk = wid % KS;
    const int H = p.H, I = p.I, NG = H / kGroup, NS = NG * SPG, rowb = H * 2;
    const int sc_bytes = RI * NS * 2;
    const int sc_stride = (int)round_dma(sc_bytes);
    uint8_t* xs = smem;
    uint8_t* scl = smem + round_dma((size_t)p.rows_cap * rowb);          // gate s, gate b, up s, up b

    // ---- x tile and scales straight to LDS.  Loads complete in issue order,
    // so these go first: waiting for them leaves the code ring in flight.
    const int tokv = it.tokv;
    dma_tile(xs, it.n, rowb, wid, lane, [&](int j, int g, int c) {
        return p.x + (size_t)__shfl(tokv, j, kWave) * H + g * kGroup + 8 * c;
    });
    {
        const size_t first = ((size_t)it.e * I + (size_t)it.rb * RI) * NS;
        dma_copy(reinterpret_cast<const uint8_t*>(p.sa + first), scl, sc_bytes, wid, lane);
        dma_copy(reinterpret_cast<const uint8_t*>(p.ba + first), scl + sc_stride, sc_bytes, wid, lane);
        dma_copy(reinterpret_cast<const uint8_t*>(p.sb + first), scl + 2 * sc_stride, sc_bytes, wid, lane);
        dma_copy(reinterpret_cast<const uint8_t*>(p.bb + first), scl + 3 * sc_stride, sc_bytes, wid, lane);
    }

    // ---- code ring: rows of this lane (pair order), groups [gb, gb + ng)
    const int gb = (wk * NG) / KS, ng = ((wk + 1) * NG) / KS - gb;
    const int rloc = 16 * wr + pair_order_row<BITS>(m);
    // codes are group-major: row r of expert e, group g at ((e NG + g) I + r) 4 LB
    const size_t gstride = (size_t)I * (4 * LB);
    const size_t cbase = (size_t)it.e * NG * gstride + ((size_t)it.rb * RI + rloc) * (4 * LB) + (TR ? 0 : q * LB);
    const uint8_t* cg = p.qa + cbase;
    const uint8_t* cu = p.qb + cbase;
    uint32_t rg[D][LW], ru[D][LW];
    auto issue = [&](int slot, int gl) {
        const size_t off = (size_t)(gb + (gl < ng ? gl : ng - 1)) * gstride;
        if constexpr (TR) {
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                rg[slot][st] = *reinterpret_cast<const uint32_t*>(cg + off + tr_word_offset<BITS>(st, q));
                ru[slot][st] = *reinterpret_cast<const uint32_t*>(cu + off + tr_word_offset<BITS>(st, q));
            }
        } else if constexpr (BITS == 4) {
            const uint4 A = *reinterpret_cast<const uint4*>(cg + off);
            const uint4 B = *reinterpret_cast<const uint4*>(cu + off);
            rg[slot][0] = A.x; rg[slot][1] = A.y; rg[slot][2] = A.z; rg[slot][3] = A.w;
            ru[slot][0] = B.x; ru[slot][1] = B.y; ru[slot][2] = B.z; ru[slot][3] = B.w;
        } else {
            const uint2 A = *reinterpret_cast<const uint2*>(cg + off);
            const uint2 B = *reinterpret_cast<const uint2*>(cu + off);
            rg[slot][0] = A.x; rg[slot][1] = A.y;
            ru[slot][0] = B.x; ru[slot][1] = B.y;
        }
    };
#pragma unroll
    for (int d = 0; d < D; ++d) issue(d, d);
    wait_vmem<2 * D * (TR ? 4 : 1)>();         // the staging loads, older than the ring loads
    lds_barrier();

    // ---- the x tile into code pair order, once per workgroup.  Unit (j, g,
    // qq) is the 32 activations that a lane of quarter qq uses for group g of
    // row j; afterwards chunk 4 qq + st of the unit holds that lane's A operand
    // of MFMA step st.  Each unit is read and rewritten by one thread.
    {
        const int units = it.n * NG * 4;
        for (int u = tid; u < units; u += 256) {
            const int j = u / (NG * 4), r = u - j * (NG * 4), g = r >> 2, qq = r & 3;
            uint8_t* base = xs + j * rowb + g * 256;
            uint32_t X[16];
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                const uint4 v = *reinterpret_cast<const uint4*>(base + 16 * ((4 * qq + st) ^ (j & 15)));
                X[4 * st] = v.x; X[4 * st + 1] = v.y; X[4 * st + 2] = v.z; X[4 * st + 3] = v.w;
            }
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                uint32_t A[4];
                act_operand<BITS>(X, st, A);
                *reinterpret_cast<uint4*>(base + 16 * ((4 * qq + st) ^ (j & 15))) = make_uint4(A[0], A[1], A[2], A[3]);
            }
        }
        lds_barrier();
    }

    const int mrow = m < it.n ? m : 0;         // rows past the tile read row 0 (never stored)
    const uint8_t* xrow = xs + mrow * rowb;
    int coff[4];                               // swizzled chunk offsets of this lane's quarter
#pragma unroll
    for (int st = 0; st < 4; ++st) coff[st] = 16 * ((TR ? 4 * st + q : 4 * q + st) ^ (mrow & 15));
    const uint16_t* gsc = reinterpret_cast<const uint16_t*>(scl) + rloc * NS;
    const uint16_t* gbi = reinterpret_cast<const uint16_t*>(scl + sc_stride) + rloc * NS;
    const uint16_t* usc = reinterpret_cast<const uint16_t*>(scl + 2 * sc_stride) + rloc * NS;
    const uint16_t* ubi = reinterpret_cast<const uint16_t*>(scl + 3 * sc_stride) + rloc * NS;
    const uint32_t ONES[4] = {kOnesBf16, kOnesBf16, kOnesBf16, kOnesBf16};

    floatx4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = accg;
    // One group: `valid` false for the padding steps of the last block, which
    // repeat the last group (codes and activations) with zero scale and bias.
    auto step = [&](int d, int gl, bool valid) {
        const int g = gb + gl;
        const uint32_t keep = valid ? 0xFFFFu : 0u;    // loads stay unconditional (no branch)
        floatx4_t Cg = {0.f, 0.f, 0.f, 0.f}, Cu = Cg, Cx = Cg;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const uint4 v = *reinterpret_cast<const uint4*>(xrow + g * 256 + coff[st]);
            const uint32_t A[4] = {v.x, v.y, v.z, v.w};
            uint32_t Bg[4], Bu[4];
            if constexpr (TR) {
                code_operand_tr<BITS>(rg[d], st, q, Bg);
                code_operand_tr<BITS>(ru[d], st, q, Bu);
            } else {
                code_operand<BITS>(rg[d], st, Bg);
                code_operand<BITS>(ru[d], st, Bu);
            }
            Cg = mfma16(A, Bg, Cg);
            Cu = mfma16(A, Bu, Cu);
            Cx = mfma16(A, ONES, Cx);           // group sum of x per token (any order)
            if (st % SST == SST - 1) {          // the scale group's last step
                const int sg = g * SPG + st / SST;
                fold<BITS>(accg, Cg, gsc[sg] & keep, gbi[sg] & keep, Cx);
                fold<BITS>(accu, Cu, usc[sg] & keep, ubi[sg] & keep, Cx);
                Cg = floatx4_t{0.f, 0.f, 0.f, 0.f};
                Cu = Cg;
                Cx = Cg;
            }
        }
    };
    // Full blocks refill every slot unconditionally (the compiler then keeps
    // exact load counts across the loop and waits only for the slot it
    // consumes); the last block, peeled, issues nothing.
    const int NGP = (ng + D - 1) / D * D;
    int g0 = 0;
    for (; g0 + D < NGP; g0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            step(d, g0 + d, true);
            __builtin_amdgcn_sched_barrier(0);
            issue(d, g0 + d + D);
        }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
        step(d, g0 + d < ng ? g0 + d : ng - 1, g0 + d < ng);
        __builtin_amdgcn_sched_barrier(0);     // keep the steps' operands from all going live at once
    }

    // ---- partial sums over K (fixed order), then SwiGLU in the wk = 0 waves
    if constexpr (KS > 1) {
        __syncthreads();                                  // the x tile is no longer read
        float* red = reinterpret_cast<float*>(smem);      // [4 waves][64][8]
        float* mine = red + (wid * 64 + lane) * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) { mine[i] = accg[i]; mine[4 + i] = accu[i]; }
        __syncthreads();
        if (wk != 0) return;
#pragma unroll
        for (int k2 = 1; k2 < KS; ++k2) {
            const float* o = red + ((wid + k2) * 64 + lane) * 8;
#pragma unroll
            for (int i = 0; i < 4; ++i) { accg[i] += o[i]; accu[i] += o[4 + i]; }
        }
    }
    // lane (m, q) holds rows 4q + i (tokens) of column m (weight row)
    float hv[4], part[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float gt = accg[i];
        hv[i] = gt / (1.f + expf(-gt)) * accu[i];
        part[i] = hv[i];
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1)
#pragma unroll
        for (int i = 0; i < 4; ++i) part[i] += __shfl_xor(part[i], off, kWave);
    const size_t plane = (size_t)p.P * I;
    const int ibase = it.rb * RI + 16 * wr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = 4 * q + i;
        if (t < it.n) {
            const size_t r = (size_t)(it.row0 + t);
            uint32_t hi, mid, lo;
            split3_bf16(hv[i], hi, mid, lo);
            uint16_t* dst = p.hp + r * I + ibase + m;
            if constexpr (COH) {
                __hip_atomic_store(dst, (uint16_t)hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(dst + plane, (uint16_t)mid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(dst + 2 * plane, (uint16_t)lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
                dst[0] = (uint16_t)hi;
                dst[plane] = (uint16_t)mid;
                dst[2 * plane] = (uint16_t)lo;
                if (m == 0) p.hpart[r * (I / 16) + ibase / 16] = part[i];
            }
        }
    }
}

template <int BITS, int RW, int D, bool SHARED = false, int SPG = 1>
__global__ __launch_bounds__(256, 2) void ffn_gateup_dec_kernel(DecParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    if (blockIdx.x == 0)                                  // the streaming down's counters start at zero
        for (int i = threadIdx.x; i < p.n_split_ctr; i += 256) p.split_ctr[i] = 0;
    gateup_item<BITS, RW, D, false, SPG>(p, dec_item_xcd<SHARED>(p, 0, (int)blockIdx.x), smem);
}

// ------------------------------------------------------------------- down
// Item = (work-list tile, block of 64 RT output rows).  Wave wid computes rows
// 16 RT wid .. +16 RT (RT tiles of 16, natural order) over all K = I groups.
// LDS: the three h planes [3][rows_cap][I] bf16 (already in pair order), then
// the raw fp16 scales and biases [64 RT][NG].  The group sums of h come from
// all-ones MFMAs on the three planes.
// WAIT (one-launch FFN): h comes from gate/up items of the same launch.  The
// scales and the first code-ring slots are requested first; then thread 0
// waits until *ready reaches `need` (bounded; on time-out *err is set), and
// only then are the h planes loaded (device-scope loads).
template <int BITS, int RT, int D, bool WAIT, int SPG = 1>
__device__ __forceinline__ void down_item(const DecParams& p, const DecItem& it, uint8_t* smem,
                                          int32_t* ready = nullptr, int need = 0, int32_t* err = nullptr) {
    constexpr int LB = 128 * BITS / 8 / 4;
    constexpr bool TR = SPG > 1;               // steps swapped (groups of 64 or 32)
    constexpr int LW = TR ? 4 : LB / 4;
    constexpr int SST = 4 / SPG;
    constexpr int RI = 64 * RT;
    if (it.n == 0) return;
    const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, q = lane >> 4;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = p.H, I = p.I, NG = I / kGroup, NS = NG * SPG, rowb = I * 2;
    const int plane_b = (int)round_dma((size_t)p.rows_cap * rowb);
    const int sc_bytes = RI * NS * 2;
    const int sc_stride = (int)round_dma(sc_bytes);
    uint8_t* hs = smem;
    uint8_t* scl = smem + 3 * (size_t)plane_b;                          // s, then b

    // ---- h planes and scales straight to LDS, ahead of the code ring
    auto stage_h = [&]() {
        const size_t plane = (size_t)p.P * I;
#pragma unroll
        for (int pl = 0; pl < 3; ++pl) {
            const uint16_t* hrows = p.hp + pl * plane + (size_t)it.row0 * I;
            dma_tile<WAIT>(hs + (size_t)pl * plane_b, it.n, rowb, wid, lane,
                           [&](int j, int g, int c) { return hrows + (size_t)j * I + g * kGroup + 8 * c; });
        }
    };
    if constexpr (!WAIT) stage_h();
    {
        const size_t first = ((size_t)it.e * H + (size_t)it.rb * RI) * NS;
        dma_copy(reinterpret_cast<const uint8_t*>(p.sa + first), scl, sc_bytes, wid, lane);
        dma_copy(reinterpret_cast<const uint8_t*>(p.ba + first), scl + sc_stride, sc_bytes, wid, lane);
    }

    // ---- code ring: RT rows of this lane, all groups
    const int rloc = 16 * RT * wid + m;               // + 16 rt
    // codes are group-major: row r of expert e, group g at ((e NG + g) H + r) 4 LB
    const size_t gstride = (size_t)H * (4 * LB);
    const uint8_t* cp = p.qa + (size_t)it.e * NG * gstride + ((size_t)it.rb * RI + rloc) * (4 * LB) + (TR ? 0 : q * LB);
    uint32_t rc[D][RT][LW];
    auto issue = [&](int slot, int g) {
        const size_t off = (size_t)(g < NG ? g : NG - 1) * gstride;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const uint8_t* src = cp + (size_t)(16 * rt) * (4 * LB) + off;
            if constexpr (TR) {
#pragma unroll
                for (int st = 0; st < 4; ++st)
                    rc[slot][rt][st] = *reinterpret_cast<const uint32_t*>(src + tr_word_offset<BITS>(st, q));
            } else if constexpr (BITS == 4) {
                const uint4 A = *reinterpret_cast<const uint4*>(src);
                rc[slot][rt][0] = A.x; rc[slot][rt][1] = A.y; rc[slot][rt][2] = A.z; rc[slot][rt][3] = A.w;
            } else {
                const uint2 A = *reinterpret_cast<const uint2*>(src);
                rc[slot][rt][0] = A.x; rc[slot][rt][1] = A.y;
            }
        }
    };
    constexpr int LPI = TR ? 4 : 1;            // loads per ring slot and row tile
#pragma unroll
    for (int d = 0; d < D; ++d) issue(d, d);
    if constexpr (WAIT) {
        if (tid == 0) {
            int v = __hip_atomic_load(ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int spin = 0; v < need && spin < kFfnSpinMax; ++spin) {
                __builtin_amdgcn_s_sleep(8);
                v = __hip_atomic_load(ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            if (v < need) __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();                       // (also waits for the ring slots above)
        stage_h();
        wait_vmem<0>();
    } else {
        wait_vmem<RT * D * LPI>();
    }
    lds_barrier();

    const int mrow = m < it.n ? m : 0;
    const uint8_t* hrow = hs + mrow * rowb;
    int coff[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) coff[st] = 16 * ((TR ? 4 * st + q : 4 * q + st) ^ (mrow & 15));
    const uint16_t* dsc = reinterpret_cast<const uint16_t*>(scl) + rloc * NS;
    const uint16_t* dbi = reinterpret_cast<const uint16_t*>(scl + sc_stride) + rloc * NS;
    const uint32_t ONES[4] = {kOnesBf16, kOnesBf16, kOnesBf16, kOnesBf16};
    floatx4_t acc[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[rt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    // `valid` false: padding step of the last block (last group again, zero
    // scale and bias)
    auto step = [&](int d, int g, bool valid) {
        const uint32_t keep = valid ? 0xFFFFu : 0u;    // loads stay unconditional (no branch)
        floatx4_t C[RT], Cx = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) C[rt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            uint32_t A[3][4];
#pragma unroll
            for (int pl = 0; pl < 3; ++pl) {
                const uint4 a4 = *reinterpret_cast<const uint4*>(hrow + (size_t)pl * plane_b + g * 256 + coff[st]);
                A[pl][0] = a4.x; A[pl][1] = a4.y; A[pl][2] = a4.z; A[pl][3] = a4.w;
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                uint32_t B[4];
                if constexpr (TR) code_operand_tr<BITS>(rc[d][rt], st, q, B);
                else code_operand<BITS>(rc[d][rt], st, B);
                C[rt] = mfma16(A[0], B, C[rt]);
                C[rt] = mfma16(A[1], B, C[rt]);
                C[rt] = mfma16(A[2], B, C[rt]);
            }
            Cx = mfma16(A[0], ONES, Cx);        // group sum of h per token, all three planes
            Cx = mfma16(A[1], ONES, Cx);
            Cx = mfma16(A[2], ONES, Cx);
            if (st % SST == SST - 1) {          // the scale group's last step
                const int sg = g * SPG + st / SST;
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    fold<BITS>(acc[rt], C[rt], dsc[16 * rt * NS + sg] & keep, dbi[16 * rt * NS + sg] & keep, Cx);
                    C[rt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
                }
                Cx = floatx4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
    };
    // full blocks refill unconditionally, the peeled last block issues nothing
    const int NGP = (NG + D - 1) / D * D;
    int g0 = 0;
    for (; g0 + D < NGP; g0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            step(d, g0 + d, true);
            __builtin_amdgcn_sched_barrier(0);
            issue(d, g0 + d + D);
        }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
        step(d, g0 + d < NG ? g0 + d : NG - 1, g0 + d < NG);
        __builtin_amdgcn_sched_barrier(0);
    }

    // ---- Y rows in bf16: token 4q + i, output row rloc + 16 rt
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = 4 * q + i;
        if (t < it.n) {
            uint16_t* yrow = p.y + (size_t)(it.row0 + t) * H + (size_t)it.rb * RI + rloc;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) yrow[16 * rt] = (uint16_t)f32_to_bf16_bits(acc[rt][i]);
        }
    }
}

template <int BITS, int RT, int D, bool SHARED = false, int SPG = 1>
__global__ __launch_bounds__(256, 2) void ffn_down_dec_kernel(DecParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    down_item<BITS, RT, D, false, SPG>(p, dec_item_xcd<SHARED>(p, 0, (int)blockIdx.x), smem);
}

// ------------------------------------------------------------ streaming down
// The down projection for shapes whose h tile does not fit LDS (a large
// intermediate size I) when the call has fewer row blocks than CUs (few
// entries, or few rows: e.g. two entries of a 3072-row output); calls with
// more take the row-block kernel below.  Work: every (work-list entry, block
// of RI = 128 output rows, group of K) unit, cut into G ranges of equal
// estimated cost, one per workgroup (G: two workgroups per CU), so every
// workgroup stays busy to the end even with few row blocks.  A range covers the tail
// of one row block, whole row blocks, and the head of another: the row blocks
// it covers whole are written straight to y; a part of a row block leaves its
// float partial sums in the workspace, and the last of the row block's
// workgroups to arrive (a counter per row block) adds the parts in the order
// of K and writes y.  Workgroup b takes range (b % 8) (G / 8) + b / 8, so the
// ranges of one XCD are adjacent and an entry's h rows are fetched into few
// L2s.
// In a part of a row block, the item's h rows pass through LDS one chunk of
// CG groups of K at a time, double-buffered: chunk c + 1 goes straight from
// L2 into the other buffer (direct-to-LDS loads, no registers) while chunk c
// is consumed, and the code ring runs on across chunk boundaries.  The waves
// share each staged chunk, so a part reads its h rows once, not once per wave.
// A lane's fp16 scales and biases come straight to registers, 8 groups (16
// bytes) per row at a time, a block of 8 groups ahead; the loop runs over
// whole such blocks and skips the groups outside the part.
// Integer planes: the products run on v_mfma_i32_16x16x64_i8 (codes as bytes
// 0..15 or 0..3, h as four int8 planes with a power-of-two scale per row and
// group, made by ffn_hquant_kernel), so the sum over a group is exact in
// int32 and costs 2 MFMAs per 16-row tile for up to 4 tokens.  The A
// operand's 16 rows are 4 tokens x 4 planes (row 4 t + p of block b is plane p
// of token 4 b + t), so a lane's four accumulators (D rows 4 q .. 4 q + 3) are
// the four planes of one token and fold into one float in the lane:
// F = C0 + 2^-7 C1 + 2^-14 C2 + 2^-21 C3, y += s hs F + b X, with hs the
// row's scale and X its float sum of h over the group.
// Wave wid computes rows 16 RT wid .. +16 RT of the row block.  LDS: two h
// buffers [4 n][CG][128 B] (row r's groups swizzled by r & 1 and its 16-byte
// pieces by (r / 2) & 7: the 16 rows one read phase touches fall on distinct
// banks), then the (hs, X) table [groups][rows_cap rounded up to 4]; the work
// split's tables follow.
// Waits: a wave's loads complete in issue order.  The first chunk is waited
// for past the scale and ring loads issued after it; every later chunk's
// loads are issued at the start of the chunk before it, and exactly CG RT
// ring loads follow them before the wait at that chunk's end (a block's scale
// loads are issued before its first chunk load).
// The work split.  Units (entry e, row block rb, group g) are numbered entry
// by entry, U = e per + rb NG + g (per = ipe NG), and a unit of entry e
// weighs w_e = kSplitW0 + kSplitW1 n_e: its codes cost the same in every
// entry, and its h planes are staged per token (the products take one MFMA
// per 4 tokens).  Measured at the 64-expert shape: token weight 1 43.5 us, 2
// and 4 44.0, 0 45.8.  The weight axis [0, Wt) is cut into
// G equal ranges (G <= the number of units); range v owns the units whose
// weight start lies in [v Wt / G, (v + 1) Wt / G), a run of consecutive
// units [F(v), F(v + 1)) that may be empty when a unit outweighs a range.
constexpr int kSplitW0 = 16, kSplitW1 = 1;

struct SplitPlan {
    const int* base;    // LDS: weight before entry e, e = 0 .. nw
    const int* wt;      // LDS: weight of one unit of entry e
    const int* first;   // LDS: F(v), v = 0 .. G
    int nw, per, G;
    long long Wt;
};

__device__ __forceinline__ long long split_start(const SplitPlan& s, int v) { return (long long)v * s.Wt / s.G; }

// The first unit whose weight start is at least x (the tables' set-up).
__device__ __forceinline__ int split_first_unit(const SplitPlan& s, long long x) {
    if (x >= s.Wt) return s.nw * s.per;
    int lo = 0, hi = s.nw - 1;                  // the entry e with base[e] <= x < base[e + 1]
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s.base[mid] <= x) lo = mid;
        else hi = mid - 1;
    }
    const long long off = x - s.base[lo];
    return lo * s.per + (int)((off + s.wt[lo] - 1) / s.wt[lo]);   // per: the next entry's first unit
}

__device__ __forceinline__ int split_first(const SplitPlan& s, int v) { return s.first[v]; }

// The range owning unit u: the largest v with F(v) <= u (its range is not
// empty: F(v + 1) > u).
__device__ __forceinline__ int split_owner(const SplitPlan& s, int u) {
    int lo = 0, hi = s.G - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s.first[mid] <= u) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Partial-sum slot of range v's part of the row block starting at unit u0:
// 2 v for the range's first part, 2 v + 1 for its last.
__device__ __forceinline__ int split_slot(const SplitPlan& s, int v, int u0) {
    return 2 * v + (split_first(s, v) < u0 ? 1 : 0);
}

// ---------------------------------------------- int8 planes of h (down input)
// For row r and group g of 128 along I: e = max(exponent(max |h|) - 5, -100),
// hs = 2^e (so max |h| / hs lies in [32, 64)), and planes q_p in [-64, 64]:
// q_p = rint(rem_p / 2^(e - 7 p)), rem_{p+1} = rem_p - q_p 2^(e - 7 p) (every
// remainder exact), so h = hs (q_0 + 2^-7 q_1 + 2^-14 q_2 + 2^-21 q_3) + a
// tail of at most 2^-22 hs.  h itself is hi + mid + lo of the bf16 planes,
// exactly.  Layout: hq [P][NG][4][128 B], the bytes of a plane's 16-code runs
// ordered as i8_code_operand delivers codes; tab [P][NG] of (hs, X), X the
// float sum of h over the group (a fixed butterfly order).
template <int BITS>
__device__ __forceinline__ int i8_operand_byte(int kl) {
    if constexpr (BITS == 4) return 4 * (2 * (kl >> 3) + (kl & 1)) + ((kl & 7) >> 1);
    else return 4 * (kl & 3) + (kl >> 2);
}

// One wave per (row, group); lane l takes stored positions 2 l and 2 l + 1.
template <int BITS>
__global__ __launch_bounds__(256) void ffn_hquant_kernel(const uint16_t* hp, int8_t* hq, float* tab, int P, int I) {
    const int NG = I / kGroup, lane = threadIdx.x & 63;
    const int wv = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wv >= P * NG) return;
    const int r = wv / NG, g = wv - r * NG;
    const size_t plane = (size_t)P * I, at = (size_t)r * I + (size_t)g * kGroup + 2 * lane;
    const uint32_t a = *reinterpret_cast<const uint32_t*>(hp + at);
    const uint32_t b = *reinterpret_cast<const uint32_t*>(hp + at + plane);
    const uint32_t c = *reinterpret_cast<const uint32_t*>(hp + at + 2 * plane);
    float h[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int sh = 16 * e;
        h[e] = (bf16_bits_to_f32((a >> sh) & 0xFFFFu) + bf16_bits_to_f32((b >> sh) & 0xFFFFu)) +
               bf16_bits_to_f32((c >> sh) & 0xFFFFu);
    }
    float mx = fmaxf(fabsf(h[0]), fabsf(h[1])), sum = h[0] + h[1];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
        sum += __shfl_xor(sum, o, kWave);
    }
    const int ex = (int)((__float_as_uint(mx) >> 23) & 0xFFu) - 127;
    const int e0 = max(ex - 5, -100);
    // stored position j of a 16-row tile holds weight row pair_order_row(j)
    const int j0 = (2 * lane) & 15, tile = (2 * lane) >> 4;
    int8_t* dst = hq + ((size_t)r * NG + g) * 4 * 128 + 16 * tile;
    float rem[2] = {h[0], h[1]};
#pragma unroll
    for (int pl = 0; pl < 4; ++pl) {
        const float up = ldexpf(1.f, 7 * pl - e0), dn = ldexpf(1.f, e0 - 7 * pl);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float qv = __builtin_rintf(rem[e] * up);
            rem[e] = fmaf(-qv, dn, rem[e]);
            dst[pl * 128 + i8_operand_byte<BITS>(pair_order_row<BITS>(j0 + e))] = (int8_t)(int)qv;
        }
    }
    if (lane == 0) {
        tab[2 * ((size_t)r * NG + g)] = ldexpf(1.f, e0);
        tab[2 * ((size_t)r * NG + g) + 1] = sum;
    }
}

template <int BITS, int NW, int RT, int D, int CG, int NBM>
__device__ __forceinline__ void down_stream_part(const DecParams& p, const DecItem& it, int ga, int gb,
                                                 uint8_t* smem, const SplitPlan& sp, int v, int u0) {
    constexpr int LB = 128 * BITS / 8 / 4;
    constexpr int LW = LB / 4;
    constexpr int RI = 16 * RT * NW;           // output rows of a row block
    constexpr int NT = 64 * NW;                // threads
    constexpr int U = 8;                       // groups per unrolled block: one 16-byte run of fp16 scales
    constexpr int rowb = CG * 128;             // one packed row of a chunk in LDS
    static_assert(U % CG == 0 && U % D == 0 && CG >= 2, "chunks and ring turns must tile the block");
    const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, q = lane >> 4;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = p.H, I = p.I, NG = I / kGroup;
    const int n = it.n, rows4 = 4 * n;         // packed rows
    const int NB = (n + 3) / 4;                // row blocks of 4 tokens (NB <= NBM)
    const int buf_b = (int)round_dma((size_t)4 * p.rows_cap * rowb);
    const int g8a = ga & ~(U - 1);             // the part runs over whole blocks of U groups from here,
    const int nch = (gb - g8a + CG - 1) / CG;  // skipping groups outside [ga, gb); chunks from g8a

    // ---- chunk c (groups g8a + CG c ..) of the packed rows into buffer c & 1;
    // slots past the 4 n rows (the last 1 KB load's tail) reload row 0 into
    // slack, and groups outside the part load its nearest group
    auto stage = [&](int c) {
        uint8_t* dst = smem + (size_t)(c & 1) * buf_b;
        const int pieces = (rows4 * rowb + kDma - 1) / kDma;
        for (int i = wid; i < pieces; i += NW) {
            const int slot = i * (kDma / 16) + lane;
            int r = slot / (CG * 8);
            const int rem = slot - r * (CG * 8);
            r = r < rows4 ? r : 0;
            const int gl = (rem >> 3) ^ (r & 1), pc = (rem & 7) ^ ((r >> 1) & 7);
            const int g = min(max(g8a + c * CG + gl, ga), gb - 1);
            const int8_t* src = p.hq + (((size_t)(it.row0 + (r >> 2)) * NG + g) * 4 + (r & 3)) * 128 + 16 * pc;
            dma16(src, dst + i * kDma);
        }
    };

    // ---- fp16 scales and biases of this lane's RT rows, one block of U groups
    // (16 bytes per row) at a time, a block ahead
    const int rloc = 16 * RT * wid + m;
    const size_t srow = ((size_t)it.e * H + (size_t)it.rb * RI + rloc) * NG;
    uint4 sc[RT], bc[RT], sn[RT], bn[RT];
    auto load_scales = [&](int g8, uint4 (&s_)[RT], uint4 (&b_)[RT]) {
        const int gg = g8 < gb ? g8 : g8a;                     // past the part: an in-range block, unused
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            s_[rt] = *reinterpret_cast<const uint4*>(p.sa + srow + (size_t)(16 * rt) * NG + gg);
            b_[rt] = *reinterpret_cast<const uint4*>(p.ba + srow + (size_t)(16 * rt) * NG + gg);
        }
    };

    // ---- code ring: RT rows of this lane, groups clamped to [ga, gb); a
    // group's codes of the wave's rows start at a uniform base (scalar-base
    // loads, the lane's offset in one VGPR)
    const size_t gstride = (size_t)H * (4 * LB);
    const uint8_t* cbase = p.qa + (size_t)it.e * NG * gstride + ((size_t)it.rb * RI + 16 * RT * wid) * (4 * LB);
    const uint32_t clane = (uint32_t)(m * (4 * LB) + q * LB);
    uint32_t rc[D][RT][LW];
    auto issue = [&](int slot, int g) {
        const gbytes_t src0 = uniform_gptr(cbase + (size_t)min(max(g, ga), gb - 1) * gstride);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const gbytes_t src = src0 + clane + (16 * rt) * (4 * LB);
            if constexpr (BITS == 4) {
                const u32x4_t A = __builtin_nontemporal_load(reinterpret_cast<gu32x4_t>(src));
                rc[slot][rt][0] = A.x; rc[slot][rt][1] = A.y; rc[slot][rt][2] = A.z; rc[slot][rt][3] = A.w;
            } else {
                const u32x2_t A = *reinterpret_cast<gu32x2_t>(src);
                rc[slot][rt][0] = A.x; rc[slot][rt][1] = A.y;
            }
        }
    };
    // ---- the (hs, X) table of the part's tokens and groups; rows t in
    // [n, rowsX) are zero
    const int rowsX = (p.rows_cap + 3) & ~3;
    const int W = ((gb + U - 1) & ~(U - 1)) - g8a;              // groups of the table (whole blocks)
    float2* xg = reinterpret_cast<float2*>(smem + 2 * (size_t)buf_b);   // [W][rowsX]
    const float2* htab = reinterpret_cast<const float2*>(p.htab) + (size_t)it.row0 * NG + g8a;
    constexpr int XPT = 4;                                     // table entries per thread per pass
    float2 xa[XPT];
    auto x_load = [&](int base) {
#pragma unroll
        for (int k = 0; k < XPT; ++k) {
            const int o = base + tid + NT * k, gg = o / rowsX, t = o - gg * rowsX;
            const bool ok = gg < W && t < n;
            xa[k] = htab[(size_t)(ok ? t : 0) * NG + (ok ? gg : 0)];
        }
    };
    auto x_store = [&](int base) {
#pragma unroll
        for (int k = 0; k < XPT; ++k) {
            const int o = base + tid + NT * k, gg = o / rowsX, t = o - gg * rowsX;
            if (gg < W) xg[o] = t < n ? xa[k] : make_float2(0.f, 0.f);
        }
    };
    x_load(0);                                  // first, so that the waits for it do not cover the ring
    stage(0);
    load_scales(g8a, sc, bc);
#pragma unroll
    for (int d = 0; d < D; ++d) issue(d, g8a + d);
    x_store(0);
    for (int base = NT * XPT; base < W * rowsX; base += NT * XPT) {   // parts longer than 64 groups
        x_load(base);
        x_store(base);
    }
    wait_vmem<RT * D + 2 * RT>();              // chunk 0 (older than the scales and the ring loads)
    lds_barrier();

    // packed row of this lane in block b (rows past 4 n read row m & 3, a
    // plane of token 0; never stored): its offsets for even and odd groups
    // and for the two steps' 16-byte pieces
    int off0[NBM], off1[NBM], pco[NBM][2];
#pragma unroll
    for (int b = 0; b < NBM; ++b) {
        const int r = 16 * b + m < rows4 ? 16 * b + m : (m & 3);
        off0[b] = r * rowb + 128 * (r & 1);
        off1[b] = r * rowb + 128 * ((r & 1) ^ 1);
#pragma unroll
        for (int st = 0; st < 2; ++st) pco[b][st] = 16 * ((2 * q + st) ^ ((r >> 1) & 7));
    }
    float acc[NBM][RT];
#pragma unroll
    for (int b = 0; b < NBM; ++b)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[b][rt] = 0.f;

    for (int g0 = g8a; g0 < gb; g0 += U) {
        load_scales(g0 + U, sn, bn);                     // before this block's chunk loads (the waits count after them)
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int g = g0 + u, gl = u % CG, c = (g0 - g8a) / CG + u / CG, d = u % D;
            if (gl == 0 && c + 1 < nch) stage(c + 1);           // the other buffer: its chunk was read before the last barrier
            if (g >= ga && g < gb) {                            // uniform per workgroup
                const uint8_t* hb = smem + (size_t)(c & 1) * buf_b + 128 * (gl & ~1);
                uint32_t B[RT][2][4];
                float sv[RT], bv[RT];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    i8_code_operand<BITS>(rc[d][rt], 0, B[rt][0]);
                    i8_code_operand<BITS>(rc[d][rt], 1, B[rt][1]);
                    const uint32_t sw = (&sc[rt].x)[u >> 1], bw = (&bc[rt].x)[u >> 1];
                    sv[rt] = f16_bits_to_f32((u & 1) ? sw >> 16 : sw & 0xFFFFu);
                    bv[rt] = f16_bits_to_f32((u & 1) ? bw >> 16 : bw & 0xFFFFu);
                }
#pragma unroll
                for (int b = 0; b < NBM; ++b) {
                    if (b < NB) {
                        int32x4_t C[RT];
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt) C[rt] = int32x4_t{0, 0, 0, 0};
#pragma unroll
                        for (int st = 0; st < 2; ++st) {
                            const uint4 a4 = *reinterpret_cast<const uint4*>(hb + ((gl & 1) ? off1[b] : off0[b]) + pco[b][st]);
                            const uint32_t A[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
                            for (int rt = 0; rt < RT; ++rt) C[rt] = mfma_i8(A, B[rt][st], C[rt]);
                        }
                        const float2 hx = xg[(g - g8a) * rowsX + 4 * b + q];   // token 4 b + q
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt) {
                            const float F = fmaf(0x1p-7f, fmaf(0x1p-7f, fmaf(0x1p-7f, (float)C[rt][3], (float)C[rt][2]),
                                                               (float)C[rt][1]), (float)C[rt][0]);
                            acc[b][rt] = fmaf(sv[rt] * hx.x, F, fmaf(bv[rt], hx.y, acc[b][rt]));
                        }
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            issue(d, g + D);                            // past the part: reloads its last group, unused
            if (gl == CG - 1 && c + 1 < nch) {
                wait_vmem<CG * RT>();                   // chunk c + 1: issued before this chunk's CG RT ring loads
                lds_barrier();                          // every wave's pieces landed; chunk c no longer read
            }
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) { sc[rt] = sn[rt]; bc[rt] = bn[rt]; }
    }
    // ---- lane (q, m) holds token 4 b + q of output rows rloc + 16 rt
    if (ga == 0 && gb == NG) {                          // the whole row block: y in bf16
        uint16_t* yb = p.y + (size_t)it.row0 * H + (size_t)it.rb * RI + rloc;
#pragma unroll
        for (int b = 0; b < NBM; ++b)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
                if (b < NB && 4 * b + q < n) yb[(size_t)(4 * b + q) * H + 16 * rt] = (uint16_t)f32_to_bf16_bits(acc[b][rt]);
        return;
    }
    // a part: its sums to slot split_slot(v, u0), then the caller arrives at
    // the row block's counter
    float* mine = p.split_part + (size_t)split_slot(sp, v, u0) * (p.rows_cap * RI) + rloc;
#pragma unroll
    for (int b = 0; b < NBM; ++b)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            if (b < NB && 4 * b + q < n)
                __hip_atomic_store(mine + (4 * b + q) * RI + 16 * rt, acc[b][rt], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The parts of the row block starting at unit u0: the non-empty ranges from
// its first unit's owner to its last unit's.  Returns their number; with
// lst, thread 0 also lists their slots there.
__device__ __forceinline__ int split_parts(const SplitPlan& sp, int u0, int NG, int* lst) {
    const int vf = split_owner(sp, u0), vl = split_owner(sp, u0 + NG - 1);
    int parts = 0;
    for (int w = vf, f0 = split_first(sp, vf); w <= vl; ++w) {
        const int f1 = split_first(sp, w + 1);
        if (f0 < f1) {
            if (lst && threadIdx.x == 0) lst[parts] = 2 * w + (f0 < u0 ? 1 : 0);
            ++parts;
        }
        f0 = f1;
    }
    return parts;
}

// The last workgroup to arrive at a row block adds its parts in the order of
// their ranges (of K), writes y and clears the counter for the next call.
template <int NT, int RI>
__device__ __forceinline__ void split_reduce(const DecParams& p, const SplitPlan& sp, int u0, int* lst) {
    const int NG = p.I / kGroup, blk = u0 / NG;
    const DecItem it = dec_item_at<false>(p, blk / p.ipe, blk % p.ipe);
    const int parts = split_parts(sp, u0, NG, lst);
    __syncthreads();
    const int rsz = p.rows_cap * RI;
    uint16_t* yb = p.y + (size_t)it.row0 * p.H + (size_t)it.rb * RI;
    for (int o = threadIdx.x; o < it.n * RI; o += NT) {
        const int t = o / RI, col = o - t * RI;
        float y = 0.f;
        for (int j = 0; j < parts; ++j)
            y += __hip_atomic_load(p.split_part + (size_t)lst[j] * rsz + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        yb[(size_t)t * p.H + col] = (uint16_t)f32_to_bf16_bits(y);
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(p.split_ctr + blk, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // ready for the next call
    __syncthreads();                                    // lst is reused
}

template <int BITS, int NW, int RT, int D, int CG, int NBM>
__global__ __launch_bounds__(64 * NW, NW / 2) void ffn_down_stream_kernel(DecParams p) {   // two workgroups per CU
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int NG = p.I / kGroup;
    SplitPlan sp;
    sp.nw = max(0, min(ld_scalar(p.n_work, 0), p.cap));
    sp.per = p.ipe * NG;
    if (sp.nw == 0) return;
    // ---- unit weights and their prefix sums over the entries (LDS, after the part's space)
    int* pbase = reinterpret_cast<int*>(smem + p.split_plan_off);
    int* pwt = pbase + p.cap + 1;
    for (int e = tid; e < sp.nw; e += 64 * NW) {
        const int32_t* ent = p.work + (size_t)e * kWorkInts;
        const int ee = ent[0], r0 = ent[1], nn = ent[2];
        const bool ok = ee >= 0 && ee < p.E && r0 >= 0 && nn >= 1 && nn <= p.rows_cap && r0 + nn <= p.P;
        pwt[e] = kSplitW0 + kSplitW1 * (ok ? nn : 0);
    }
    __syncthreads();
    if (tid < 64) {
        int carry = 0;
        for (int c0 = 0; c0 < sp.nw; c0 += 64) {
            const int e = c0 + lane;
            int x = e < sp.nw ? pwt[e] * sp.per : 0;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_up(x, off, kWave);
                if (lane >= off) x += y;
            }
            if (e < sp.nw) pbase[e + 1] = carry + x;
            carry += __shfl(x, 63, kWave);
        }
        if (lane == 0) pbase[0] = 0;
    }
    __syncthreads();
    sp.base = pbase;
    sp.wt = pwt;
    sp.Wt = pbase[sp.nw];
    sp.G = (int)min((long long)gridDim.x, (long long)sp.nw * sp.per);
    int* pfirst = pwt + p.cap;
    for (int w = tid; w <= sp.G; w += 64 * NW) pfirst[w] = split_first_unit(sp, split_start(sp, w));
    sp.first = pfirst;
    __syncthreads();
    const int b = (int)blockIdx.x, v = (b & 7) * ((int)gridDim.x >> 3) + (b >> 3);
    if (v >= sp.G) return;
    const int first = split_first(sp, v), end = split_first(sp, v + 1);
    int* lst = reinterpret_cast<int*>(smem);            // after a part: its LDS is no longer read
    for (int u = first; u < end;) {
        const int blk = u / NG, u0 = blk * NG;
        const int ga = u - u0, gb = min(NG, end - u0);
        const DecItem it = dec_item_at<false>(p, blk / p.ipe, blk % p.ipe);
        if (u > first) lds_barrier();                   // the last part's LDS is no longer read
        if (it.n > 0) {
            down_stream_part<BITS, NW, RT, D, CG, NBM>(p, it, ga, gb, smem, sp, v, u0);
            if (ga > 0 || gb < NG) {
                // arrival: this workgroup's part stores have completed (the
                // full wait), then one count; partial sums pass between
                // workgroups as device-scope atomic stores and loads, which
                // bypass the non-coherent per-CU caches
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                if (tid == 0)
                    lst[64] = __hip_atomic_fetch_add(p.split_ctr + blk, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                              split_parts(sp, u0, NG, nullptr) - 1;
                __syncthreads();
                if (lst[64]) split_reduce<64 * NW, 16 * RT * NW>(p, sp, u0, lst + 128);
            }
        }
        u = u0 + gb;
    }
}

// ---------------------------------------------------------- down by row block
// The streaming down's parts with no split of K: workgroup b takes the items
// (entry, block of 16 NW rows) b, b + G, ... over all of K, each a whole row
// block written straight to y, so there are no partial sums, arrivals or range
// tables.  NW waves of one 16-row tile each, the code ring D groups deep.
// Taken when the work list's capacity gives at least one item per CU: at the
// 64-expert shape (about 7 entries of 64 blocks of 80 rows) the items fill the
// chip once, and the fixed costs of the split (range tables, part prologues,
// partial sums and their reduction: about a third of its time) are gone.
template <int BITS, int NW, int D, int CG, int NBM>
__global__ __launch_bounds__(64 * NW) void ffn_down_rows_kernel(DecParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int NG = p.I / kGroup;
    const int nw = max(0, min(ld_scalar(p.n_work, 0), p.cap));
    const int items = nw * p.ipe;
    SplitPlan sp{};                                     // unused: every part is a whole row block
    for (int item = (int)blockIdx.x; item < items; item += (int)gridDim.x) {
        const DecItem it = dec_item_at<false>(p, item / p.ipe, item % p.ipe);
        if (item != (int)blockIdx.x) lds_barrier();     // the last item's LDS is no longer read
        if (it.n > 0) down_stream_part<BITS, NW, 1, D, CG, NBM>(p, it, 0, NG, smem, sp, 0, 0);
    }
}

// ------------------------------------------------------------ one-launch FFN
// Gate/up and down in one launch.  The grid is cut into chunks of kFfnChunk
// work-list entries; a chunk is its gate/up items, then its down items, each
// numbered as in the two-launch kernels (an entry's items on one XCD).  A down
// item requests its scales and first code slots, then waits until the gate/up
// items of its entry have published h (a per-entry counter), then loads h.  So
// the down items start streaming weights while the last gate/up items finish,
// and the two halves share one ramp-up and one tail.
// Why the wait ends: workgroups are dispatched in index order, and every
// gate/up item a down item waits for has a lower index, so it is already
// running (on the same XCD, since an entry's items share one), and gate/up
// items wait for nothing.  The wait is bounded anyway: on time-out the item
// goes on (its results are then wrong) and the flag sync[kFfnErr] is set.
// h crosses workgroups as device-scope stores and loads (no cache flush).
// Counters of entry e at sync[kFfnStride e]: [0] gate/up items done, [1] down
// items done; the last down item puts both back to zero.
struct FusedParams {
    DecParams p;                                                 // gate/up: weights qa..bb, ipe
    const uint8_t* qd; const uint16_t* sd; const uint16_t* bd;   // down weights
    int ipe_d;                                                   // down items per entry
    int32_t* err;                                                // set to 1 when a wait times out
};

template <int BITS, int RW, int DG, int RT, int DD, bool SHARED = false, int SPG = 1>
__global__ __launch_bounds__(256, 2) void ffn_fused_dec_kernel(FusedParams f, int32_t* sync) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int ng = kFfnChunk * f.p.ipe, span = ng + kFfnChunk * f.ipe_d;
    const int b = (int)blockIdx.x, chunk = b / span, r = b - chunk * span;
    const int entry0 = chunk * kFfnChunk;
    if (r < ng) {
        const DecItem it = dec_item_xcd<SHARED>(f.p, entry0, r);
        gateup_item<BITS, RW, DG, true, SPG>(f.p, it, smem);
        if (it.n == 0) return;
        __builtin_amdgcn_s_waitcnt(0);          // this wave's h stores have completed
        __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_fetch_add(&sync[kFfnStride * it.entry], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        DecParams pd = f.p;
        pd.qa = f.qd; pd.sa = f.sd; pd.ba = f.bd; pd.ipe = f.ipe_d;
        const DecItem it = dec_item_xcd<SHARED>(pd, entry0, r - ng);
        if (it.n == 0) return;
        int32_t* ctr = &sync[kFfnStride * it.entry];
        down_item<BITS, RT, DD, true, SPG>(pd, it, smem, ctr, f.p.ipe, f.err);
        if (threadIdx.x == 0 &&
            __hip_atomic_fetch_add(ctr + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == f.ipe_d - 1) {
            __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(ctr + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ------------------------------------------------------------------ launch

static DecParams dec_params(const FfnArgs& a) {
    const moe_dims& d = a.d;
    DecParams p{};
    p.x = a.x; p.work = a.work; p.n_work = a.n_work; p.y = a.y;
    p.T = d.T; p.H = d.H; p.I = d.I; p.E = d.E; p.P = d.T * d.k;
    p.rows_cap = d.T < kWorkRows ? d.T : kWorkRows;
    p.cap = (int)work_capacity(d);
    char* ws = reinterpret_cast<char*>(a.h);
    const size_t P = (size_t)p.P;
    p.hp = reinterpret_cast<uint16_t*>(ws);
    p.hpart = reinterpret_cast<float*>(ws + ((3 * P * d.I * sizeof(uint16_t) + 255) & ~(size_t)255));
    const SplitSpace sp = down_split_space(d, a.h);
    p.split_ctr = sp.ctr;
    p.split_part = sp.part;
    p.hq = sp.hq;
    p.htab = sp.tab;
    p.n_split_ctr = sp.n_ctr;
    return p;
}

// Waves along rows in gate/up: more rows per item once there are enough tiles
// to fill the chip; at least one group of K per wave.
static int dec_gateup_rw(const moe_dims& d) {
    const long P = (long)d.T * d.k;
    int rw = P >= 32 ? 4 : 1;
    const int NG = d.H / kGroup;
    while (rw < 4 && 4 / rw > NG) rw *= 2;
    return rw;
}

// Down rows per wave (RT tiles of 16): bigger items once there are enough
// tiles, so that every item of the launch is resident at once.
static int dec_down_rt(const moe_dims& d) {
    const long P = (long)d.T * d.k;
    if (P >= 128 && d.H % 256 == 0) return 4;
    return (P >= 32) ? 2 : 1;
}

static size_t dec_gateup_lds(const moe_dims& d, int rw) {
    const int rows_cap = d.T < kWorkRows ? d.T : kWorkRows;
    const int NS = d.H / d.group_size;                  // scale groups per row
    const size_t stage = round_dma((size_t)rows_cap * d.H * 2) + 4 * round_dma((size_t)16 * rw * NS * 2);
    const size_t red = (rw < 4) ? (size_t)4 * 64 * 8 * 4 : 0;
    return stage > red ? stage : red;
}

static size_t dec_down_lds(const moe_dims& d, int rt) {
    const int rows_cap = d.T < kWorkRows ? d.T : kWorkRows;
    const int NS = d.I / d.group_size;
    return 3 * round_dma((size_t)rows_cap * d.I * 2) + 2 * round_dma((size_t)64 * rt * NS * 2);
}

// Ring depth: the deepest of `cap`, cap / 2, ..., 2 that pads a wave's groups
// by at most a quarter.  Shallow rings measure faster than requesting a wave's
// whole stream at once: a wave that issues many loads stalls at issue (the
// memory pipeline is full) and only starts its arithmetic once the last load
// is out, so its compute no longer overlaps the stream.
static int dec_depth(int ng, int cap) {
    for (int dd = cap; dd > 1; dd >>= 1) {
        if (dd > ng) continue;
        const int ngp = (ng + dd - 1) / dd * dd;
        if (4 * ngp <= 5 * ng) return dd;
    }
    return 1;
}

bool dec_gateup_fits(const moe_dims& d) { return dec_gateup_lds(d, dec_gateup_rw(d)) <= kDecLdsLimit; }
bool dec_down_fits(const moe_dims& d) { return dec_down_lds(d, dec_down_rt(d)) <= kDecLdsLimit; }

template <int BITS, int RW, int D, bool SHARED, int SPG>
static void gu_go(const moe_dims& d, size_t lds, hipStream_t s, const DecParams& p) {
    const dim3 grid((unsigned)((p.cap + p.n_shared + 7) / 8 * 8 * p.ipe));   // entries rounded up to 8 (one per XCD)
    hipLaunchKernelGGL((ffn_gateup_dec_kernel<BITS, RW, D, SHARED, SPG>), grid, dim3(256), lds, s, p);
}

template <int BITS, int RW, bool SHARED, int SPG>
static void gu_depth(int D, const moe_dims& d, size_t lds, hipStream_t s, const DecParams& p) {
    if (D >= 4) gu_go<BITS, RW, 4, SHARED, SPG>(d, lds, s, p);
    else if (D >= 2) gu_go<BITS, RW, 2, SHARED, SPG>(d, lds, s, p);
    else gu_go<BITS, RW, 1, SHARED, SPG>(d, lds, s, p);
}

template <int BITS, bool SHARED, int SPG>
static void gu_rw(int rw, int D, const moe_dims& d, size_t lds, hipStream_t s, const DecParams& p) {
    if (rw == 4) gu_depth<BITS, 4, SHARED, SPG>(D, d, lds, s, p);
    else if (rw == 2) gu_depth<BITS, 2, SHARED, SPG>(D, d, lds, s, p);
    else gu_depth<BITS, 1, SHARED, SPG>(D, d, lds, s, p);
}

// Scale groups per run of 128 codes: 1, 2 or 4 (groups of 128, 64 or 32).
inline int scale_groups(const moe_dims& d) { return kGroup / d.group_size; }

template <int BITS, bool SHARED>
static void gu_spg(int rw, int D, const moe_dims& d, size_t lds, hipStream_t s, const DecParams& p) {
    switch (scale_groups(d)) {
        case 4: gu_rw<BITS, SHARED, 4>(rw, D, d, lds, s, p); break;
        case 2: gu_rw<BITS, SHARED, 2>(rw, D, d, lds, s, p); break;
        default: gu_rw<BITS, SHARED, 1>(rw, D, d, lds, s, p); break;
    }
}

// d sizes the items; p carries the entries (and any shared tiles).
template <bool SHARED>
static int gateup_dec_run(const FfnArgs& a, const moe_dims& d, DecParams p, hipStream_t s) {
    p.qa = a.w.q[0]; p.sa = a.w.scale[0]; p.ba = a.w.bias[0];
    p.qb = a.w.q[1]; p.sb = a.w.scale[1]; p.bb = a.w.bias[1];
    const int rw = dec_gateup_rw(d);
    p.ipe = d.I / (16 * rw);
    const size_t lds = dec_gateup_lds(d, rw);
    if (lds > kDecLdsLimit) return MOE_ERR_UNSUPPORTED;
    const int D = dec_depth((d.H / kGroup) / (4 / rw), 4);
    if (a.bits == 4) gu_spg<4, SHARED>(rw, D, d, lds, s, p);
    else gu_spg<2, SHARED>(rw, D, d, lds, s, p);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_gateup_dec(const FfnArgs& a, hipStream_t s) {
    if (a.d.T * a.d.k == 0) return MOE_OK;
    return gateup_dec_run<false>(a, a.d, dec_params(a), s);
}

template <int BITS, int RT, int D, bool SHARED, int SPG>
static void dn_go(const moe_dims& d, size_t lds, hipStream_t s, const DecParams& p) {
    const dim3 grid((unsigned)((p.cap + p.n_shared + 7) / 8 * 8 * p.ipe));   // entries rounded up to 8 (one per XCD)
    hipLaunchKernelGGL((ffn_down_dec_kernel<BITS, RT, D, SHARED, SPG>), grid, dim3(256), lds, s, p);
}

template <int BITS, int RT, bool SHARED, int SPG>
static void dn_depth(int D, const moe_dims& d, size_t lds, hipStream_t s, const DecParams& p) {
    if (D >= 2) dn_go<BITS, RT, 2, SHARED, SPG>(d, lds, s, p);
    else dn_go<BITS, RT, 1, SHARED, SPG>(d, lds, s, p);
}

template <int BITS, bool SHARED, int SPG>
static void dn_rt(int rt, int D, const moe_dims& d, size_t lds, hipStream_t s, const DecParams& p) {
    if (rt == 4) dn_depth<BITS, 4, SHARED, SPG>(D, d, lds, s, p);
    else if (rt == 2) dn_depth<BITS, 2, SHARED, SPG>(D, d, lds, s, p);
    else dn_depth<BITS, 1, SHARED, SPG>(D, d, lds, s, p);
}

template <int BITS, bool SHARED>
static void dn_spg(int rt, int D, const moe_dims& d, size_t lds, hipStream_t s, const DecParams& p) {
    switch (scale_groups(d)) {
        case 4: dn_rt<BITS, SHARED, 4>(rt, D, d, lds, s, p); break;
        case 2: dn_rt<BITS, SHARED, 2>(rt, D, d, lds, s, p); break;
        default: dn_rt<BITS, SHARED, 1>(rt, D, d, lds, s, p); break;
    }
}

template <bool SHARED>
static int down_dec_run(const FfnArgs& a, const moe_dims& d, DecParams p, hipStream_t s) {
    p.qa = a.w.q[2]; p.sa = a.w.scale[2]; p.ba = a.w.bias[2];
    const int rt = dec_down_rt(d);
    p.ipe = d.H / (64 * rt);
    const size_t lds = dec_down_lds(d, rt);
    if (lds > kDecLdsLimit) return MOE_ERR_UNSUPPORTED;
    const int D = dec_depth(d.I / kGroup, 2);
    if (a.bits == 4) dn_spg<4, SHARED>(rt, D, d, lds, s, p);
    else dn_spg<2, SHARED>(rt, D, d, lds, s, p);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_down_dec(const FfnArgs& a, hipStream_t s) {
    if (a.d.T * a.d.k == 0) return MOE_OK;
    return down_dec_run<false>(a, a.d, dec_params(a), s);
}

// ------------------------------------------------------------ streaming down

// Chunk of K groups staged at a time: 4, or 2 for tiles of more rows than fit
// two buffers of 4 groups in the decode LDS limit.  Then the (hs, X) table
// [NG][rows_cap rounded up to 4] of float pairs.
static size_t down_stream_lds(const moe_dims& d, int cg) {
    const int rows_cap = d.T < kWorkRows ? d.T : kWorkRows;
    const size_t bufs = 2 * round_dma((size_t)4 * rows_cap * cg * 128);
    const size_t xtab = (size_t)(d.I / kGroup) * ((rows_cap + 3) & ~3) * 2 * sizeof(float);
    return bufs + ((xtab + 255) & ~(size_t)255);
}

// The work split's tables (entry weights, their prefix sums, the ranges'
// first units) after the part's LDS.
static size_t down_stream_plan_lds(const moe_dims& d) {
    return (size_t)(2 * work_capacity(d) + 1 + kStreamGrid + 1) * sizeof(int);
}

// The chunk size of the streaming down at these dims, or 0 where it does not
// run: where the decode down kernel fits, or K is not whole blocks of 8 groups,
// or H is not whole row blocks, or no chunk size fits LDS.
static int down_stream_cg(const moe_dims& d) {
    if (d.T * d.k == 0 || dec_down_fits(d) || d.group_size != kGroup) return 0;
    if ((d.I / kGroup) % 8 != 0 || d.H % kStreamRows != 0) return 0;
    if (work_capacity(d) > 1024) return 0;     // the work split's tables
    for (int c = 4; c >= 2; c >>= 1)
        if (down_stream_lds(d, c) + down_stream_plan_lds(d) <= kDecLdsLimit) return c;
    return 0;
}

// Counters [cap][H / RI], partial sums [2 G][rows_cap][RI], the int8 planes
// of h [P][NG][4][128] and their (hs, X) table [P][NG][2] of the streaming
// down, after the bf16 planes and their partial sums in the workspace.
static size_t r256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t down_split_bytes(const moe_dims& d) {
    if (down_stream_cg(d) == 0) return 0;
    const int rows_cap = d.T < kWorkRows ? d.T : kWorkRows;
    const size_t P = (size_t)d.T * d.k;
    const size_t ctr = work_capacity(d) * (size_t)(d.H / kStreamRows) * sizeof(int32_t);
    const size_t part = (size_t)2 * kStreamGrid * rows_cap * kStreamRows * sizeof(float);
    const size_t hq = P * (size_t)d.I * 4;
    const size_t tab = P * (size_t)(d.I / kGroup) * 2 * sizeof(float);
    return r256(ctr) + r256(part) + r256(hq) + tab;
}

SplitSpace down_split_space(const moe_dims& d, void* ws) {
    SplitSpace sp{nullptr, nullptr, nullptr, nullptr, 0};
    if (down_split_bytes(d) == 0) return sp;
    const int rows_cap = d.T < kWorkRows ? d.T : kWorkRows;
    const size_t P = (size_t)d.T * d.k;
    const size_t planes = r256(3 * P * d.I * sizeof(uint16_t));
    const size_t hpart = r256(P * (d.I / 16) * sizeof(float));
    char* base = reinterpret_cast<char*>(ws) + planes + hpart;
    sp.n_ctr = (int)(work_capacity(d) * (size_t)(d.H / kStreamRows));
    sp.ctr = reinterpret_cast<int32_t*>(base);
    base += r256(sp.n_ctr * sizeof(int32_t));
    sp.part = reinterpret_cast<float*>(base);
    base += r256((size_t)2 * kStreamGrid * rows_cap * kStreamRows * sizeof(float));
    sp.hq = reinterpret_cast<int8_t*>(base);
    base += r256(P * (size_t)d.I * 4);
    sp.tab = reinterpret_cast<float*>(base);
    return sp;
}

template <int BITS, int D, int CG, int NBM>
static void ds_go(size_t lds, hipStream_t s, const DecParams& p) {
    hipLaunchKernelGGL((ffn_down_stream_kernel<BITS, kStreamWaves, kStreamRows / (16 * kStreamWaves), D, CG, NBM>),
                       dim3(kStreamGrid), dim3(64 * kStreamWaves),
                       lds, s, p);
}

// NBM: row blocks of 4 tokens the tile can need, ceil(rows_cap / 4)
template <int BITS>
static void ds_cg(int cg, size_t lds, hipStream_t s, const DecParams& p) {
    const int nbm = (p.rows_cap + 3) / 4;
    if (cg == 4) {
        if (nbm == 1) ds_go<BITS, 4, 4, 1>(lds, s, p);
        else if (nbm == 2) ds_go<BITS, 4, 4, 2>(lds, s, p);
        else if (nbm == 3) ds_go<BITS, 4, 4, 3>(lds, s, p);
        else ds_go<BITS, 4, 4, 4>(lds, s, p);
    } else {
        ds_go<BITS, 4, 2, 4>(lds, s, p);
    }
}

// The row-block down: waves per workgroup (one 16-row tile each): 5 where H
// is a multiple of 80, else 4 (H is a multiple of 128 here); its code ring
// depth and workgroups per CU.  Measured at the 64-expert shape (down call
// with the conversion, us): 5 waves ring 4 32.4-33.2, ring 8 33.4-34.1; 4
// waves 33.9-34.4; 8 waves 37.4-38.1; against 43.5-44.1 for the split of K.
constexpr int kRowsDepth = 4, kRowsPerCu = 3;

static int down_rows_waves(const moe_dims& d) { return d.H % 80 == 0 ? 5 : (d.H % 64 == 0 ? 4 : 0); }

template <int BITS, int NW, int NBM>
static void dr_go(int cg, size_t lds, hipStream_t s, const DecParams& p, int grid) {
    if (cg == 4) hipLaunchKernelGGL((ffn_down_rows_kernel<BITS, NW, kRowsDepth, 4, NBM>), dim3(grid), dim3(64 * NW), lds, s, p);
    else hipLaunchKernelGGL((ffn_down_rows_kernel<BITS, NW, kRowsDepth, 2, NBM>), dim3(grid), dim3(64 * NW), lds, s, p);
}

template <int BITS, int NW>
static void dr_nbm(int nbm, int cg, size_t lds, hipStream_t s, const DecParams& p, int grid) {
    if (nbm == 1) dr_go<BITS, NW, 1>(cg, lds, s, p, grid);
    else if (nbm == 2) dr_go<BITS, NW, 2>(cg, lds, s, p, grid);
    else dr_go<BITS, NW, 4>(cg, lds, s, p, grid);
}

// The row-block down (ffn_down_rows_kernel): the conversion of h, then whole
// row blocks of 16 rw rows per workgroup.
static int launch_down_rows(const FfnArgs& a, hipStream_t s, int cg, int rw) {
    const moe_dims& d = a.d;
    DecParams p = dec_params(a);
    p.qa = a.w.q[2]; p.sa = a.w.scale[2]; p.ba = a.w.bias[2];
    p.ipe = d.H / (16 * rw);
    p.n_split_ctr = 0;
    const size_t lds = down_stream_lds(d, cg);
    const int P = d.T * d.k, nq = P * (d.I / kGroup);
    const int grid = (int)std::min<long>((long)p.cap * p.ipe, (long)kRowsPerCu * device_cus());
    int8_t* hq = const_cast<int8_t*>(p.hq);
    float* tab = const_cast<float*>(p.htab);
    const int nbm = (p.rows_cap + 3) / 4;
    if (a.bits == 4) {
        hipLaunchKernelGGL(ffn_hquant_kernel<4>, dim3((nq + 3) / 4), dim3(256), 0, s, p.hp, hq, tab, P, d.I);
        if (rw == 5) dr_nbm<4, 5>(nbm, cg, lds, s, p, grid);
        else dr_nbm<4, 4>(nbm, cg, lds, s, p, grid);
    } else {
        hipLaunchKernelGGL(ffn_hquant_kernel<2>, dim3((nq + 3) / 4), dim3(256), 0, s, p.hp, hq, tab, P, d.I);
        if (rw == 5) dr_nbm<2, 5>(nbm, cg, lds, s, p, grid);
        else dr_nbm<2, 4>(nbm, cg, lds, s, p, grid);
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_down_stream(const FfnArgs& a, hipStream_t s) {
    const moe_dims& d = a.d;
    if (d.T * d.k == 0) return MOE_OK;
    const int cg = down_stream_cg(d);
    if (cg == 0) return MOE_ERR_UNSUPPORTED;
    // whole row blocks per workgroup when the call can have at least one per
    // CU (the work-list capacity's worth); else K split over the workgroups
    const int rw = down_rows_waves(d);
    if (rw > 0 && (long)work_capacity(d) * (d.H / (16 * rw)) >= device_cus()) return launch_down_rows(a, s, cg, rw);
    DecParams p = dec_params(a);
    p.qa = a.w.q[2]; p.sa = a.w.scale[2]; p.ba = a.w.bias[2];
    p.ipe = d.H / kStreamRows;
    p.n_split_ctr = 0;                                    // the counters are the gate/up call's to clear
    p.split_plan_off = (int)down_stream_lds(d, cg);
    const size_t lds = down_stream_lds(d, cg) + down_stream_plan_lds(d);
    const int P = d.T * d.k, nq = P * (d.I / kGroup);
    int8_t* hq = const_cast<int8_t*>(p.hq);
    float* tab = const_cast<float*>(p.htab);
    if (a.bits == 4) {
        hipLaunchKernelGGL(ffn_hquant_kernel<4>, dim3((nq + 3) / 4), dim3(256), 0, s, p.hp, hq, tab, P, d.I);
        ds_cg<4>(cg, lds, s, p);
    } else {
        hipLaunchKernelGGL(ffn_hquant_kernel<2>, dim3((nq + 3) / 4), dim3(256), 0, s, p.hp, hq, tab, P, d.I);
        ds_cg<2>(cg, lds, s, p);
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// ------------------------------------------------------------ one-launch FFN

template <int BITS, int RW, int DG, int RT, int DD, bool SHARED, int SPG>
static int fused_go(size_t lds, hipStream_t s, const FusedParams& f, int32_t* sync) {
    const int chunks = (f.p.cap + f.p.n_shared + kFfnChunk - 1) / kFfnChunk;
    const dim3 grid((unsigned)(chunks * kFfnChunk * (f.p.ipe + f.ipe_d)));
    hipLaunchKernelGGL((ffn_fused_dec_kernel<BITS, RW, DG, RT, DD, SHARED, SPG>), grid, dim3(256), lds, s, f, sync);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// The decode configurations with a one-launch kernel; others take two launches.
template <int BITS, bool SHARED, int SPG>
static int fused_cfg(int rw, int dg, int rt, int dd, size_t lds, hipStream_t s, const FusedParams& f,
                     int32_t* sync) {
    if (rw == 4 && dg == 4 && rt == 4 && dd == 2) return fused_go<BITS, 4, 4, 4, 2, SHARED, SPG>(lds, s, f, sync);
    if (rw == 4 && dg == 4 && rt == 2 && dd == 2) return fused_go<BITS, 4, 4, 2, 2, SHARED, SPG>(lds, s, f, sync);
    if (rw == 1 && dg == 4 && rt == 1 && dd == 4) return fused_go<BITS, 1, 4, 1, 4, SHARED, SPG>(lds, s, f, sync);
    if (rw == 1 && dg == 4 && rt == 1 && dd == 2) return fused_go<BITS, 1, 4, 1, 2, SHARED, SPG>(lds, s, f, sync);
    return MOE_ERR_UNSUPPORTED;
}

template <int BITS, bool SHARED>
static int fused_pick(int spg, int rw, int dg, int rt, int dd, size_t lds, hipStream_t s, const FusedParams& f,
                      int32_t* sync) {
    // groups of 32 take the two decode launches: their one-launch variants
    // spill registers (a fold per MFMA step on top of both items' state)
    switch (spg) {
        case 2: return fused_cfg<BITS, SHARED, 2>(rw, dg, rt, dd, lds, s, f, sync);
        case 1: return fused_cfg<BITS, SHARED, 1>(rw, dg, rt, dd, lds, s, f, sync);
        default: return MOE_ERR_UNSUPPORTED;
    }
}

// The one-launch FFN with decode parameters p; d sizes the items.
template <bool SHARED>
static int fused_run(const FfnArgs& a, const moe_dims& d, const DecParams& p, int32_t* sync, hipStream_t s,
                     int32_t* err = nullptr) {
    FusedParams f{};
    f.p = p;
    f.err = err != nullptr ? err : sync + kFfnErr;
    f.p.qa = a.w.q[0]; f.p.sa = a.w.scale[0]; f.p.ba = a.w.bias[0];
    f.p.qb = a.w.q[1]; f.p.sb = a.w.scale[1]; f.p.bb = a.w.bias[1];
    f.qd = a.w.q[2]; f.sd = a.w.scale[2]; f.bd = a.w.bias[2];
    const int rw = dec_gateup_rw(d), rt = dec_down_rt(d);
    f.p.ipe = d.I / (16 * rw);
    f.ipe_d = d.H / (64 * rt);
    // One-tile down items (the smallest batches, where a few entries make the
    // critical path) request up to four code groups before their wait, so that
    // no HBM round trip is left once h arrives; with more entries the deeper
    // ring measured no faster.
    const int dg = dec_depth((d.H / kGroup) / (4 / rw), 4), dd = dec_depth(d.I / kGroup, rt == 1 ? 4 : 2);
    const size_t lg = dec_gateup_lds(d, rw), ld = dec_down_lds(d, rt);
    const size_t lds = lg > ld ? lg : ld;
    const int spg = scale_groups(d);
    return a.bits == 4 ? fused_pick<4, SHARED>(spg, rw, dg, rt, dd, lds, s, f, sync)
                       : fused_pick<2, SHARED>(spg, rw, dg, rt, dd, lds, s, f, sync);
}

int launch_ffn_fused_dec(const FfnArgs& a, int32_t* sync, hipStream_t s, int32_t* err) {
    const moe_dims& d = a.d;
    if (d.T * d.k == 0) return MOE_OK;
    if (!dec_gateup_fits(d) || !dec_down_fits(d) || work_capacity(d) > kFfnMaxEntries) return MOE_ERR_UNSUPPORTED;
    return fused_run<false>(a, d, dec_params(a), sync, s, err);
}

// With a shared expert: a.d are the routed dims; the weights hold E + 1
// experts (the shared one last) and y / the workspace have T (k + 1) rows.  The
// shared tiles are ceil(T / 16) entries after the routed ones (dec_item_at),
// so one launch streams the shared expert with the routed ones; shapes without
// a one-launch kernel take the two decode launches, with the same entries.
int launch_ffn_fused_dec_shared(const FfnArgs& a, int32_t* sync, hipStream_t s) {
    const moe_dims& d = a.d;
    if (d.T == 0) return MOE_OK;
    moe_dims d1 = d;
    d1.E = d.E + 1;
    d1.k = d.k + 1;
    const int n_sh = (d.T + kWorkRows - 1) / kWorkRows;
    if (!dec_gateup_fits(d1) || !dec_down_fits(d1) || work_capacity(d) + n_sh > kFfnMaxEntries)
        return MOE_ERR_UNSUPPORTED;
    FfnArgs a1 = a;
    a1.d = d1;
    DecParams p = dec_params(a1);          // E + 1 experts, T (k + 1) rows
    p.cap = (int)work_capacity(d);         // the routed work list's size
    p.n_shared = n_sh;
    p.shared_row0 = d.T * d.k;
    int st = fused_run<true>(a1, d1, p, sync, s);
    if (st != MOE_ERR_UNSUPPORTED) return st;
    st = gateup_dec_run<true>(a1, d1, p, s);
    return st ? st : down_dec_run<true>(a1, d1, p, s);
}

}  // namespace moe

