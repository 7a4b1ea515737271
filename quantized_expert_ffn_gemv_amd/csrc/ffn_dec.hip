// Decode-sized expert FFN on the matrix cores: one work-list tile (up to 16
// tokens of one expert) per workgroup, its activations staged once in LDS.
//
// The exact code operands and the per-group fold are those of mfma_ops.h.
// What differs from the kernels in ffn_mfma.hip:
//   * the tile's activations (gate/up: x rows; down: the three bf16 planes of
//     h) are loaded once per workgroup into LDS, already in the pair order of
//     the code operands, together with each row's sum over every group of
//     128, so the waves read their MFMA operand with one LDS load per step and
//     need neither a permute nor an all-ones MFMA for the group sums;
//   * activations are the A operand (rows = tokens) and the codes the B
//     operand (columns = weight rows): a lane's accumulators belong to one
//     weight row, so each lane folds with a single scale pair per group, read
//     from an LDS copy of the item's scales;
//   * one item per workgroup (no persistent loop): the grid covers every
//     possible tile, and workgroups past the device-side tile count exit.
// Gate/up: RW waves split the item's rows (16 gate + 16 up rows each) and
// KS = 4 / RW waves split K; partial sums over K are added in LDS in a fixed
// order.  Down: each wave owns RT tiles of 16 output rows over all of K.
// h leaves gate/up in the layout of the other matrix-core kernels (three bf16
// planes in code pair order plus 16-row partial sums), so either down kernel
// can follow either gate/up kernel.
#include <algorithm>

#include "mfma_ops.h"

namespace moe {

namespace {

// Largest LDS a decode item may take (two workgroups per CU at 160 KB, with
// room for the rest); bigger shapes use the kernels of ffn_mfma.hip.
constexpr size_t kDecLdsLimit = 80 * 1024;

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
    int rows_cap;       // token rows of the LDS tile: min(16, T)
};

// LDS byte offset of 16-byte chunk c (0..15) of group g of token row j, rows
// of `rowb` bytes (a multiple of 256).  Chunks are XOR-swizzled by the row's
// low 4 bits: the 16 rows a quarter-wave reads at once hit 16 bank groups.
__device__ __forceinline__ int tile_off(int j, int g, int c, int rowb) {
    return j * rowb + g * 256 + 16 * (c ^ (j & 15));
}

// Item of a decode launch: work-list entry and row block of blockIdx.x; the
// entry's expert, first sorted row, row count (n = 0: nothing to do) and the
// tokens of its rows, spread over lanes (lane l holds the token of row
// l % 16, clamped into [0, T)).  The whole entry is read with the count,
// before any branch, so all of it arrives in one scalar round trip (every
// entry below the grid's capacity is allocated, whatever the count).
struct DecItem {
    int entry, rb, e, row0, n;
    int tokv;
};

__device__ __forceinline__ DecItem dec_item(const DecParams& p) {
    typedef int int4v __attribute__((ext_vector_type(4)));
    DecItem it;
    it.entry = (int)blockIdx.x / p.ipe;
    it.rb = (int)blockIdx.x % p.ipe;
    const int4v* ent = reinterpret_cast<const int4v*>(p.work + (size_t)it.entry * kWorkInts);
    const int n_work = ld_scalar(p.n_work, 0);
    int4v v[kWorkInts / 4];
#pragma unroll
    for (int i = 0; i < kWorkInts / 4; ++i) v[i] = ld_scalar(ent, i);
    const int l16 = threadIdx.x & 15;
    int tok = v[1][0];
#pragma unroll
    for (int j = 1; j < kWorkRows; ++j) tok = (l16 == j) ? v[1 + j / 4][j % 4] : tok;
    it.tokv = (tok >= 0 && tok < p.T) ? tok : 0;
    const int e = v[0][0], row0 = v[0][1], n = v[0][2];
    const bool ok = it.entry < n_work && e >= 0 && e < p.E && row0 >= 0 && n >= 1 && n <= p.rows_cap &&
                    row0 + n <= p.P;
    it.e = ok ? e : 0;
    it.row0 = ok ? row0 : 0;
    it.n = ok ? n : 0;
    return it;
}

// Scale staging, split in an issue half and a store half so that its loads
// join the other staging loads in one memory round trip.  Chunk c (of
// rows * NG / 8) holds 8 consecutive fp16 scales and the matching biases of
// the contiguous block starting at row `first`; the store half writes them to
// LDS as packed (scale | bias << 16) words, row stride NGp.
struct ScaleChunk {
    uint4 s, b;
};

__device__ __forceinline__ ScaleChunk scale_chunk(const uint16_t* __restrict__ s, const uint16_t* __restrict__ b,
                                                  size_t first, int NG, int c) {
    ScaleChunk r;
    r.s = *reinterpret_cast<const uint4*>(s + first * NG + (size_t)c * 8);
    r.b = *reinterpret_cast<const uint4*>(b + first * NG + (size_t)c * 8);
    return r;
}

__device__ __forceinline__ void store_scale_chunk(const ScaleChunk& k, int c, int NG, int NGp, uint32_t* dst) {
    const uint32_t sw[4] = {k.s.x, k.s.y, k.s.z, k.s.w}, bw[4] = {k.b.x, k.b.y, k.b.z, k.b.w};
#pragma unroll
    for (int v = 0; v < 8; ++v) {
        const int f = c * 8 + v, r = f / NG, g = f - r * NG;
        const uint32_t sv = (sw[v >> 1] >> (16 * (v & 1))) & 0xFFFFu;
        const uint32_t bv = (bw[v >> 1] >> (16 * (v & 1))) & 0xFFFFu;
        dst[r * NGp + g] = sv | (bv << 16);
    }
}

// Staging tasks per thread per round (16 rows x 16 groups x 4 quarters fill
// one round of 256 threads).
constexpr int kStageX = 4;

// acc += (s / L) C + (b - (128 / L) s) X for one packed (scale, bias) word.
template <int BITS>
__device__ __forceinline__ void fold(floatx4_t& acc, const floatx4_t& C, uint32_t sb, const float4& X) {
    const float sv = f16_bits_to_f32(sb & 0xFFFFu), bv = f16_bits_to_f32(sb >> 16);
    const float s1 = sv * kInvLever<BITS>, b1 = fmaf(-kOffset<BITS>, sv, bv);
    acc[0] = fmaf(s1, C[0], fmaf(b1, X.x, acc[0]));
    acc[1] = fmaf(s1, C[1], fmaf(b1, X.y, acc[1]));
    acc[2] = fmaf(s1, C[2], fmaf(b1, X.z, acc[2]));
    acc[3] = fmaf(s1, C[3], fmaf(b1, X.w, acc[3]));
}

}  // namespace

// --------------------------------------------------------------- gate / up
// Item = (work-list tile, block of 16 RW rows of gate and of up).  Wave
// (wr, wk) = (wid / KS, wid % KS) computes rows 16 wr .. +16 of the block
// (pair order) over its share of the K groups, with a D-deep register ring of
// code loads.  LDS: x tile [rows_cap][H] bf16 (pair order, swizzled), group
// sums [NG][16] float, scales [2][16 RW][NGp] packed; after the loop the
// first 8 KB is reused for the partial sums over K.
template <int BITS, int RW, int D>
__global__ __launch_bounds__(256) void ffn_gateup_dec_kernel(DecParams p) {
    constexpr int KS = 4 / RW;
    constexpr int LB = 128 * BITS / 8 / 4;     // code bytes per lane per group
    constexpr int LW = LB / 4;
    constexpr int RI = 16 * RW;                // gate (and up) rows per item
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const DecItem it = dec_item(p);
    if (it.n == 0) return;
    const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, q = lane >> 4;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wid / KS, wk = wid % KS;
    const int H = p.H, I = p.I, NG = H / kGroup, NGp = NG | 1, rowb = H * 2;
    uint8_t* xs = smem;
    float* xsum = reinterpret_cast<float*>(smem + (size_t)p.rows_cap * rowb);
    uint32_t* sc = reinterpret_cast<uint32_t*>(xsum + NG * 16);

    // ---- code ring: rows of this lane (pair order), groups [gb, gb + ng)
    const int gb = (wk * NG) / KS, ng = ((wk + 1) * NG) / KS - gb;
    const int rloc = 16 * wr + pair_order_row<BITS>(m);
    const size_t grow = (size_t)it.e * I + (size_t)it.rb * RI + rloc;
    const size_t rowbytes = (size_t)H * BITS / 8;
    const uint8_t* cg = p.qa + grow * rowbytes + q * LB;
    const uint8_t* cu = p.qb + grow * rowbytes + q * LB;
    uint32_t rg[D][LW], ru[D][LW];
    auto issue = [&](int slot, int gl) {
        const size_t off = (size_t)(gb + (gl < ng ? gl : ng - 1)) * (4 * LB);
        if constexpr (BITS == 4) {
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
    // ---- staging of the x tile (pair order) with its group sums, and the
    // scales, in rounds of kStageX tasks per thread.  A round issues all its
    // loads, then stores; tasks past the end repeat the last task and write
    // the same values to the same place, so the stores need no guard (a guard
    // lets the compiler sink each load into its branch: one round trip per
    // task).
    const int tokv = it.tokv;
    const int nq = it.n * NG * 4, nsc = 2 * (RI * NG / 8);
    const size_t first = (size_t)it.e * I + (size_t)it.rb * RI;
    struct Stage {
        uint32_t X[kStageX][16];
        int tj[kStageX], tg[kStageX], tqq[kStageX];
        ScaleChunk sk;
        int cc, cmat;
    };
    auto stage_issue = [&](int rd, Stage& S) {
#pragma unroll
        for (int u = 0; u < kStageX; ++u) {
            int t = (rd * kStageX + u) * 256 + tid;
            t = t < nq ? t : nq - 1;
            const int j = t / (NG * 4), r = t - j * (NG * 4);
            S.tj[u] = j; S.tg[u] = r >> 2; S.tqq[u] = r & 3;
            const int tok = __shfl(tokv, j, kWave);
            const uint4* src = reinterpret_cast<const uint4*>(p.x + (size_t)tok * H + S.tg[u] * kGroup + 32 * S.tqq[u]);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const uint4 w = src[v];
                S.X[u][4 * v] = w.x; S.X[u][4 * v + 1] = w.y; S.X[u][4 * v + 2] = w.z; S.X[u][4 * v + 3] = w.w;
            }
        }
        int c = rd * 256 + tid;
        c = c < nsc ? c : nsc - 1;
        S.cmat = c >= nsc / 2;
        S.cc = c - S.cmat * (nsc / 2);
        S.sk = scale_chunk(S.cmat ? p.sb : p.sa, S.cmat ? p.bb : p.ba, first, NG, S.cc);
    };
    auto stage_store = [&](const Stage& S) {
#pragma unroll
        for (int u = 0; u < kStageX; ++u) {
#pragma unroll
            for (int st = 0; st < 4; ++st) {
                uint32_t o[4];
                act_operand<BITS>(S.X[u], st, o);
                *reinterpret_cast<uint4*>(xs + tile_off(S.tj[u], S.tg[u], 4 * S.tqq[u] + st, rowb)) =
                    make_uint4(o[0], o[1], o[2], o[3]);
            }
            float sum = 0.f;
#pragma unroll
            for (int v = 0; v < 16; ++v) sum += bf16_bits_to_f32(S.X[u][v] & 0xFFFFu) + bf16_bits_to_f32(S.X[u][v] >> 16);
            sum += __shfl_xor(sum, 1, kWave);
            sum += __shfl_xor(sum, 2, kWave);
            if (S.tqq[u] == 0) xsum[S.tg[u] * 16 + S.tj[u]] = sum;
        }
        store_scale_chunk(S.sk, S.cc, NG, NGp, sc + S.cmat * RI * NGp);
    };
    {
        // Loads complete in issue order, so round 0 is issued before the code
        // ring: waiting for it then leaves the ring in flight.  Scheduling
        // barriers keep the compiler from moving either across the other.
        Stage S;
        stage_issue(0, S);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int d = 0; d < D; ++d) issue(d, d);
        __builtin_amdgcn_sched_barrier(0);
        stage_store(S);
        const int rounds = max((nq + 256 * kStageX - 1) / (256 * kStageX), (nsc + 255) / 256);
        for (int rd = 1; rd < rounds; ++rd) {
            stage_issue(rd, S);
            stage_store(S);
        }
    }
    __syncthreads();

    // ---- main loop: consume a ring slot, refill it D groups on
    const int mrow = m < it.n ? m : 0;         // rows past the tile read row 0 (never stored)
    const uint32_t* scg = sc + rloc * NGp;
    const uint32_t* scu = sc + (RI + rloc) * NGp;
    floatx4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = accg;
    auto step = [&](int d, int gl) {
        const int g = gb + gl;
        floatx4_t Cg = {0.f, 0.f, 0.f, 0.f}, Cu = Cg;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const uint4 a4 = *reinterpret_cast<const uint4*>(xs + tile_off(mrow, g, 4 * q + st, rowb));
            const uint32_t A[4] = {a4.x, a4.y, a4.z, a4.w};
            uint32_t Bg[4], Bu[4];
            code_operand<BITS>(rg[d], st, Bg);
            code_operand<BITS>(ru[d], st, Bu);
            Cg = mfma16(A, Bg, Cg);
            Cu = mfma16(A, Bu, Cu);
        }
        const float4 X = *reinterpret_cast<const float4*>(xsum + g * 16 + 4 * q);
        fold<BITS>(accg, Cg, scg[g], X);
        fold<BITS>(accu, Cu, scu[g], X);
    };
    // Full blocks refill every slot unconditionally (the compiler then keeps
    // exact load counts across the loop and waits only for the slot it
    // consumes); the last block, peeled, issues nothing.
    const int NGP = (ng + D - 1) / D * D;
    int g0 = 0;
    for (; g0 + D < NGP; g0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            step(d, g0 + d);
            __builtin_amdgcn_sched_barrier(0);
            issue(d, g0 + d + D);
        }
    }
#pragma unroll
    for (int d = 0; d < D; ++d)
        if (g0 + d < ng) step(d, g0 + d);

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
            dst[0] = (uint16_t)hi;
            dst[plane] = (uint16_t)mid;
            dst[2 * plane] = (uint16_t)lo;
            if (m == 0) p.hpart[r * (I / 16) + ibase / 16] = part[i];
        }
    }
}

// ------------------------------------------------------------------- down
// Item = (work-list tile, block of 64 RT output rows).  Wave wid computes rows
// 16 RT wid .. +16 RT (RT tiles of 16, natural order) over all K = I groups.
// LDS: the three h planes [3][rows_cap][I] bf16 (pair order, swizzled), the
// group sums [NG][16] float (from the 16-row partial sums of h), scales
// [64 RT][NGp] packed.
template <int BITS, int RT, int D>
__global__ __launch_bounds__(256) void ffn_down_dec_kernel(DecParams p) {
    constexpr int LB = 128 * BITS / 8 / 4;
    constexpr int LW = LB / 4;
    constexpr int RI = 64 * RT;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const DecItem it = dec_item(p);
    if (it.n == 0) return;
    const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, q = lane >> 4;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = p.H, I = p.I, NG = I / kGroup, NGp = NG | 1, rowb = I * 2;
    const size_t plane_b = (size_t)p.rows_cap * rowb;
    uint8_t* hs = smem;
    float* hsum = reinterpret_cast<float*>(smem + 3 * plane_b);
    uint32_t* sc = reinterpret_cast<uint32_t*>(hsum + NG * 16);

    // ---- code ring: RT rows of this lane, all groups
    const int rloc = 16 * RT * wid + m;               // + 16 rt
    const size_t grow = (size_t)it.e * H + (size_t)it.rb * RI + rloc;
    const size_t rowbytes = (size_t)I * BITS / 8;
    const uint8_t* cp = p.qa + grow * rowbytes + q * LB;
    uint32_t rc[D][RT][LW];
    auto issue = [&](int slot, int g) {
        const size_t off = (size_t)(g < NG ? g : NG - 1) * (4 * LB);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const uint8_t* src = cp + (size_t)(16 * rt) * rowbytes + off;
            if constexpr (BITS == 4) {
                const uint4 A = *reinterpret_cast<const uint4*>(src);
                rc[slot][rt][0] = A.x; rc[slot][rt][1] = A.y; rc[slot][rt][2] = A.z; rc[slot][rt][3] = A.w;
            } else {
                const uint2 A = *reinterpret_cast<const uint2*>(src);
                rc[slot][rt][0] = A.x; rc[slot][rt][1] = A.y;
            }
        }
    };
    // ---- staging of the h planes (already in pair order), group sums and
    // scales, in rounds as in the gate/up kernel (round 0 with the ring)
    const size_t plane = (size_t)p.P * I;
    const int per_plane = it.n * NG * 4;
    const int nq = 3 * per_plane, nhs = it.n * NG, nsc = RI * NG / 8;
    const size_t first = (size_t)it.e * H + (size_t)it.rb * RI;
    struct Stage {
        uint32_t V[kStageX][16];
        int tpl[kStageX], tj[kStageX], tg[kStageX], tqq[kStageX];
        float4 ha, hb;
        int hj, hg;
        ScaleChunk sk;
        int c;
    };
    auto stage_issue = [&](int rd, Stage& S) {
#pragma unroll
        for (int u = 0; u < kStageX; ++u) {
            int t = (rd * kStageX + u) * 256 + tid;
            t = t < nq ? t : nq - 1;
            const int pl = t / per_plane, r = t - pl * per_plane;
            const int j = r / (NG * 4), r2 = r - j * (NG * 4);
            S.tpl[u] = pl; S.tj[u] = j; S.tg[u] = r2 >> 2; S.tqq[u] = r2 & 3;
            const uint4* src = reinterpret_cast<const uint4*>(p.hp + pl * plane + (size_t)(it.row0 + j) * I +
                                                              S.tg[u] * kGroup + 32 * S.tqq[u]);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const uint4 w = src[v];
                S.V[u][4 * v] = w.x; S.V[u][4 * v + 1] = w.y; S.V[u][4 * v + 2] = w.z; S.V[u][4 * v + 3] = w.w;
            }
        }
        int th = rd * 256 + tid;
        th = th < nhs ? th : nhs - 1;
        S.hj = th / NG;
        S.hg = th - S.hj * NG;
        const float4* hsrc = reinterpret_cast<const float4*>(p.hpart + (size_t)(it.row0 + S.hj) * (I / 16) + 8 * S.hg);
        S.ha = hsrc[0];
        S.hb = hsrc[1];
        int c = rd * 256 + tid;
        S.c = c < nsc ? c : nsc - 1;
        S.sk = scale_chunk(p.sa, p.ba, first, NG, S.c);
    };
    auto stage_store = [&](const Stage& S) {
#pragma unroll
        for (int u = 0; u < kStageX; ++u) {
            uint8_t* dst = hs + S.tpl[u] * plane_b;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                *reinterpret_cast<uint4*>(dst + tile_off(S.tj[u], S.tg[u], 4 * S.tqq[u] + v, rowb)) =
                    make_uint4(S.V[u][4 * v], S.V[u][4 * v + 1], S.V[u][4 * v + 2], S.V[u][4 * v + 3]);
        }
        hsum[S.hg * 16 + S.hj] = ((S.ha.x + S.ha.y) + (S.ha.z + S.ha.w)) + ((S.hb.x + S.hb.y) + (S.hb.z + S.hb.w));
        store_scale_chunk(S.sk, S.c, NG, NGp, sc);
    };
    {
        // round 0 ahead of the ring (see the gate/up kernel)
        Stage S;
        stage_issue(0, S);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int d = 0; d < D; ++d) issue(d, d);
        __builtin_amdgcn_sched_barrier(0);
        stage_store(S);
        int rounds = (nq + 256 * kStageX - 1) / (256 * kStageX);
        rounds = max(rounds, max((nhs + 255) / 256, (nsc + 255) / 256));
        for (int rd = 1; rd < rounds; ++rd) {
            stage_issue(rd, S);
            stage_store(S);
        }
    }
    __syncthreads();

    const int mrow = m < it.n ? m : 0;
    floatx4_t acc[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[rt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    auto step = [&](int d, int g) {
        floatx4_t C[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) C[rt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            uint32_t A[3][4];
#pragma unroll
            for (int pl = 0; pl < 3; ++pl) {
                const uint4 a4 = *reinterpret_cast<const uint4*>(hs + pl * plane_b + tile_off(mrow, g, 4 * q + st, rowb));
                A[pl][0] = a4.x; A[pl][1] = a4.y; A[pl][2] = a4.z; A[pl][3] = a4.w;
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                uint32_t B[4];
                code_operand<BITS>(rc[d][rt], st, B);
                C[rt] = mfma16(A[0], B, C[rt]);
                C[rt] = mfma16(A[1], B, C[rt]);
                C[rt] = mfma16(A[2], B, C[rt]);
            }
        }
        const float4 X = *reinterpret_cast<const float4*>(hsum + g * 16 + 4 * q);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) fold<BITS>(acc[rt], C[rt], sc[(rloc + 16 * rt) * NGp + g], X);
    };
    // full blocks refill unconditionally, the peeled last block issues nothing
    const int NGP = (NG + D - 1) / D * D;
    int g0 = 0;
    for (; g0 + D < NGP; g0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            step(d, g0 + d);
            __builtin_amdgcn_sched_barrier(0);
            issue(d, g0 + d + D);
        }
    }
#pragma unroll
    for (int d = 0; d < D; ++d)
        if (g0 + d < NG) step(d, g0 + d);

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

// ------------------------------------------------------------------ launch

static DecParams dec_params(const FfnArgs& a) {
    const moe_dims& d = a.d;
    DecParams p{};
    p.x = a.x; p.work = a.work; p.n_work = a.n_work; p.y = a.y;
    p.T = d.T; p.H = d.H; p.I = d.I; p.E = d.E; p.P = d.T * d.k;
    p.rows_cap = d.T < kWorkRows ? d.T : kWorkRows;
    char* ws = reinterpret_cast<char*>(a.h);
    const size_t P = (size_t)p.P;
    p.hp = reinterpret_cast<uint16_t*>(ws);
    p.hpart = reinterpret_cast<float*>(ws + ((3 * P * d.I * sizeof(uint16_t) + 255) & ~(size_t)255));
    return p;
}

// Waves along rows in gate/up: more rows per item once there are enough tiles
// to fill the chip; at least one group of K per wave.
static int dec_gateup_rw(const moe_dims& d) {
    const long P = (long)d.T * d.k;
    int rw = P >= 128 ? 4 : (P >= 32 ? 2 : 1);
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
    const int NG = d.H / kGroup, NGp = NG | 1;
    const size_t stage = (size_t)rows_cap * d.H * 2 + (size_t)NG * 16 * 4 + (size_t)2 * 16 * rw * NGp * 4;
    const size_t red = (rw < 4) ? (size_t)4 * 64 * 8 * 4 : 0;
    return stage > red ? stage : red;
}

static size_t dec_down_lds(const moe_dims& d, int rt) {
    const int rows_cap = d.T < kWorkRows ? d.T : kWorkRows;
    const int NG = d.I / kGroup, NGp = NG | 1;
    return (size_t)3 * rows_cap * d.I * 2 + (size_t)NG * 16 * 4 + (size_t)64 * rt * NGp * 4;
}

// Ring depth: the deepest of 16, 8, 4, 2 that pads the wave's groups by at
// most a quarter.  At decode sizes a wave's whole stream (16 groups or fewer)
// is then requested at once, before the first use.
static int dec_depth(int ng) {
    for (int dd = 16; dd > 1; dd >>= 1) {
        if (dd > ng) continue;
        const int ngp = (ng + dd - 1) / dd * dd;
        if (4 * ngp <= 5 * ng) return dd;
    }
    return 1;
}

bool dec_gateup_fits(const moe_dims& d) { return dec_gateup_lds(d, dec_gateup_rw(d)) <= kDecLdsLimit; }
bool dec_down_fits(const moe_dims& d) { return dec_down_lds(d, dec_down_rt(d)) <= kDecLdsLimit; }

template <int BITS, int RW, int D>
static void gu_go(const moe_dims& d, size_t lds, hipStream_t s, const DecParams& p) {
    const dim3 grid((unsigned)(work_capacity(d) * p.ipe));
    hipLaunchKernelGGL((ffn_gateup_dec_kernel<BITS, RW, D>), grid, dim3(256), lds, s, p);
}

template <int BITS, int RW>
static void gu_depth(int D, const moe_dims& d, size_t lds, hipStream_t s, const DecParams& p) {
    if (D >= 8) gu_go<BITS, RW, 8>(d, lds, s, p);
    else if (D >= 4) gu_go<BITS, RW, 4>(d, lds, s, p);
    else if (D >= 2) gu_go<BITS, RW, 2>(d, lds, s, p);
    else gu_go<BITS, RW, 1>(d, lds, s, p);
}

template <int BITS>
static void gu_rw(int rw, int D, const moe_dims& d, size_t lds, hipStream_t s, const DecParams& p) {
    if (rw == 4) gu_depth<BITS, 4>(D, d, lds, s, p);
    else if (rw == 2) gu_depth<BITS, 2>(D, d, lds, s, p);
    else gu_depth<BITS, 1>(D, d, lds, s, p);
}

int launch_gateup_dec(const FfnArgs& a, hipStream_t s) {
    const moe_dims& d = a.d;
    if (d.T * d.k == 0) return MOE_OK;
    DecParams p = dec_params(a);
    p.qa = a.w.q[0]; p.sa = a.w.scale[0]; p.ba = a.w.bias[0];
    p.qb = a.w.q[1]; p.sb = a.w.scale[1]; p.bb = a.w.bias[1];
    const int rw = dec_gateup_rw(d);
    p.ipe = d.I / (16 * rw);
    const size_t lds = dec_gateup_lds(d, rw);
    if (lds > kDecLdsLimit) return MOE_ERR_UNSUPPORTED;
    // the ring shares the registers with the staging round: at most 8 deep
    const int D = std::min(8, dec_depth((d.H / kGroup) / (4 / rw)));
    if (a.bits == 4) gu_rw<4>(rw, D, d, lds, s, p);
    else gu_rw<2>(rw, D, d, lds, s, p);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

template <int BITS, int RT, int D>
static void dn_go(const moe_dims& d, size_t lds, hipStream_t s, const DecParams& p) {
    const dim3 grid((unsigned)(work_capacity(d) * p.ipe));
    hipLaunchKernelGGL((ffn_down_dec_kernel<BITS, RT, D>), grid, dim3(256), lds, s, p);
}

template <int BITS, int RT>
static void dn_depth(int D, const moe_dims& d, size_t lds, hipStream_t s, const DecParams& p) {
    if (D >= 8) dn_go<BITS, RT, 8>(d, lds, s, p);
    else if (D >= 4) dn_go<BITS, RT, 4>(d, lds, s, p);
    else if (D >= 2) dn_go<BITS, RT, 2>(d, lds, s, p);
    else dn_go<BITS, RT, 1>(d, lds, s, p);
}

int launch_down_dec(const FfnArgs& a, hipStream_t s) {
    const moe_dims& d = a.d;
    if (d.T * d.k == 0) return MOE_OK;
    DecParams p = dec_params(a);
    p.qa = a.w.q[2]; p.sa = a.w.scale[2]; p.ba = a.w.bias[2];
    const int rt = dec_down_rt(d);
    p.ipe = d.H / (64 * rt);
    const size_t lds = dec_down_lds(d, rt);
    if (lds > kDecLdsLimit) return MOE_ERR_UNSUPPORTED;
    const int D = std::min(8, dec_depth(d.I / kGroup));
    if (a.bits == 4) {
        if (rt == 4) dn_depth<4, 4>(D, d, lds, s, p);
        else if (rt == 2) dn_depth<4, 2>(D, d, lds, s, p);
        else dn_depth<4, 1>(D, d, lds, s, p);
    } else {
        if (rt == 4) dn_depth<2, 4>(D, d, lds, s, p);
        else if (rt == 2) dn_depth<2, 2>(D, d, lds, s, p);
        else dn_depth<2, 1>(D, d, lds, s, p);
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
