// Quantised expert FFN on the matrix cores (v_mfma_f32_16x16x32_bf16).
//
// Why MFMA at decode: a vector-ALU matvec spends about one dot2 instruction per
// two weights per token; with the HBM stream at 8 TB/s the CU array can afford
// about 2.5 lane-instructions per 4-bit weight in total, so once an expert
// serves three or more tokens (sec. 2.3 of the "Strata" page: tokens of one
// batch share an expert) the vector path becomes compute-bound.  A 16-token
// MFMA tile costs the same few vector instructions per weight (unpacking) at
// any token count up to 16.
//
// Exactness: a code q becomes the bf16 value 128 + L q (q OR-ed into the
// mantissa of 0x4300; L = kLever: 8 for 4-bit, 16 for 2-bit codes), exact, and
// activations are bf16, so every product is exact and the matrix core
// accumulates in float32.  Per group of 128 along K the tile accumulator
// C = sum (128 + L q) x is folded into the output as
//     (s / L) * C + (b - (128 / L) s) * X,    X = sum of x over the group,
// which is sum (q s + b) x (the FMA form of the Flash-MoE page, sec. 2).  X
// comes from a third MFMA with an all-ones A operand.  The lever keeps the
// 128 X part of C within a few times the code part, so float32 rounding in C
// stays at float32 level relative to the result.
//
// Layout of one wave's MFMA work: rows m = lane % 16 of a 16-row tile (A operand),
// tokens n = lane % 16 of a 16-token tile (B operand), quad q = lane / 16 owns
// k = 128 g + 32 q .. +32 of group g, one 16-byte (4-bit) or 8-byte (2-bit)
// load per row per group.  The four MFMA steps of a group take 8 of the quad's
// 32 k each; inside the 8 (or 16) codes of a 32-bit word the pair layout of the
// unpacked codes (q_i, q_{i+W/2}) is mirrored on the activations.
//
// Gate/up writes h = silu(a) * u as three bf16 planes hi + mid + lo (about 24
// significant bits, i.e. float32 h) in the pair order the down kernel's B
// operand needs, plus per-16-row partial sums of h for the down bias fold.
#include <algorithm>
#include <atomic>

#include "launch_util.h"
#include "mfma_ops.h"

namespace moe {

// Work split: a 256-thread workgroup owns an output block (16 gate + 16 up
// rows, or 32 down rows) of one expert; its 4 waves take disjoint quarters of
// the K groups, so each wave streams only a few groups and can have all of them
// in flight at once (decode batches are small: the whole FFN of one token at
// the A3B-style shape is ~1.6 MB, a few KB per wave).  Partial accumulators
// are summed in LDS in a fixed wave order, then wave 0 runs the epilogue.
constexpr int kWaves = 4;

struct MfmaParams {
    const uint16_t* x;
    const int32_t* work;        // work list entries (kWorkInts int32 each)
    const int32_t* n_work;
    const uint8_t* qa;  const uint16_t* sa;  const uint16_t* ba;   // gate, or down
    const uint8_t* qb;  const uint16_t* sb;  const uint16_t* bb;   // up
    uint16_t* hp;       // bf16 planes [3][P][I]
    float* hpart;       // [P][I/16] partial sums of h over 16-row tiles
    uint16_t* y;        // [P][H]
    int T, H, I, k, E, P;
    int items_per_entry;        // output blocks per work-list entry
    int32_t* split_ctr;         // gate/up: counters of the streaming down to clear
    int n_split_ctr;
};

// Groups [gb, ge) of K handled by wave w (an even split; a wave may get none).
__device__ __forceinline__ void wave_groups(int NG, int w, int& gb, int& ng) {
    gb = (w * NG) / kWaves;
    ng = ((w + 1) * NG) / kWaves - gb;
}

// --------------------------------------------------------------- gate / up
// Persistent: workgroup b handles items b, b + G, b + 2G, ... (G = grid size)
// of the n_work * (I / 16) items; an item is one work-list tile (<= 16 tokens
// of one expert) times 16 output rows of gate and up.  Wave w streams its
// quarter of the K groups; its D-deep prefetch ring runs across item
// boundaries: during the last D groups of item j it already loads item j+1,
// whose metadata, token ids and scales were fetched while item j computed.
// LDS: [kWaves][2][NGW][4][16] float scales (double-buffered by item parity;
// per wave: s/L and b - (128/L) s of gate, then up, for the 16 output rows),
// then [kWaves][64][8] partial sums.  SJ = scale entries per lane per matrix.
// D must divide the groups of every wave (the launcher guarantees it).
template <int BITS, int D, int SJ>
__global__ __launch_bounds__(256) void ffn_gateup_mfma_kernel(MfmaParams p) {
    constexpr int LB = 128 * BITS / 8 / 4;     // bytes per lane per group (16 or 8)
    constexpr int LW = LB / 4;                 // code words per lane per group
    extern __shared__ float lds[];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, m = lane & 15, q = lane >> 4;
    const int ipe = p.items_per_entry;
    if (blockIdx.x == 0)                                  // the streaming down's counters start at zero
        for (int i = tid; i < p.n_split_ctr; i += 256) p.split_ctr[i] = 0;
    const int n_items = ld_scalar(p.n_work, 0) * ipe;
    if ((int)blockIdx.x >= n_items) return;
    const int n_my = (n_items - 1 - (int)blockIdx.x) / (int)gridDim.x + 1;
    const int H = p.H, I = p.I, NG = H / kGroup, NGW = (NG + kWaves - 1) / kWaves;
    int gb, ng;
    wave_groups(NG, w, gb, ng);
    constexpr int GB = kGroup * BITS / 8;      // code bytes of one row in one group
    const size_t gstride = (size_t)I * GB;     // from one group of all I rows to the next
    float* sc_base = lds + w * 2 * NGW * 64;
    float* red = lds + kWaves * 2 * NGW * 64;
    uint32_t ONE[4] = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};

    // ---- per-item state: uniform metadata + this lane's pointers and scales
    struct Item {
        int e, it, row0, n;
        const uint8_t* g;
        const uint8_t* u;
        const uint16_t* x;
        uint32_t sv[4][SJ];
    };
    auto fetch = [&](int j, Item& I_) {
        const int idx = (int)blockIdx.x + j * (int)gridDim.x;
        const int32_t* ent = p.work + (size_t)(idx / ipe) * kWorkInts;
        I_.it = idx % ipe;
        I_.e = ld_scalar(ent, 0);
        I_.row0 = ld_scalar(ent, 1);
        I_.n = ld_scalar(ent, 2);
        int tok = ld_scalar(ent, 4);
#pragma unroll
        for (int jj = 1; jj < kWorkRows; ++jj) {
            const int v = ld_scalar(ent, 4 + jj);
            tok = (m == jj) ? v : tok;
        }
        const int e = (I_.e >= 0 && I_.e < p.E) ? I_.e : 0;
        tok = (tok >= 0 && tok < p.T) ? tok : 0;
        const size_t wcode = (size_t)e * NG * gstride + (size_t)(I_.it * 16 + pair_order_row<BITS>(m)) * GB + q * LB;
        I_.g = p.qa + wcode;
        I_.u = p.qb + wcode;
        I_.x = p.x + (size_t)tok * H + q * 32;
        if (ng > 0) {
#pragma unroll
            for (int jj = 0; jj < SJ; ++jj) {
                const int id2 = lane + 64 * jj;
                const int gl = min(id2 >> 4, ng - 1), r = id2 & 15;
                const size_t src = ((size_t)e * I + I_.it * 16 + pair_order_row<BITS>(r)) * NG + gb + gl;
                I_.sv[0][jj] = p.sa[src]; I_.sv[1][jj] = p.ba[src];
                I_.sv[2][jj] = p.sb[src]; I_.sv[3][jj] = p.bb[src];
            }
        }
    };
    auto stage = [&](const Item& I_, float* dst_base) {
#pragma unroll
        for (int jj = 0; jj < SJ; ++jj) {
            const int id2 = lane + 64 * jj;
            const int gl = id2 >> 4, r = id2 & 15;
            if (gl < ng) {
                const float s1 = f16_bits_to_f32(I_.sv[0][jj]), b1 = f16_bits_to_f32(I_.sv[1][jj]);
                const float s2 = f16_bits_to_f32(I_.sv[2][jj]), b2 = f16_bits_to_f32(I_.sv[3][jj]);
                float* dst = dst_base + gl * 64 + r;
                dst[0] = s1 * kInvLever<BITS>;
                dst[16] = fmaf(-kOffset<BITS>, s1, b1);
                dst[32] = s2 * kInvLever<BITS>;
                dst[48] = fmaf(-kOffset<BITS>, s2, b2);
            }
        }
    };

    uint32_t wg[D][LW], wu[D][LW], xv[D][16];
    // codes: non-temporal loads, since each byte is read once (72 -> 67 us for
    // the 64-expert shape's gate/up with the grid and depth below)
    auto issue = [&](int slot, const uint8_t* gp, const uint8_t* up, const uint16_t* xp, int g) {
        if constexpr (BITS == 4) {
            const u32x4_t A = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(gp + (size_t)g * gstride));
            const u32x4_t B = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(up + (size_t)g * gstride));
            wg[slot][0] = A.x; wg[slot][1] = A.y; wg[slot][2] = A.z; wg[slot][3] = A.w;
            wu[slot][0] = B.x; wu[slot][1] = B.y; wu[slot][2] = B.z; wu[slot][3] = B.w;
        } else {
            const uint2 A = *reinterpret_cast<const uint2*>(gp + (size_t)g * gstride);
            const uint2 B = *reinterpret_cast<const uint2*>(up + (size_t)g * gstride);
            wg[slot][0] = A.x; wg[slot][1] = A.y;
            wu[slot][0] = B.x; wu[slot][1] = B.y;
        }
        const uint4* xs = reinterpret_cast<const uint4*>(xp + (size_t)g * kGroup);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const uint4 X = xs[v];
            xv[slot][4 * v] = X.x; xv[slot][4 * v + 1] = X.y;
            xv[slot][4 * v + 2] = X.z; xv[slot][4 * v + 3] = X.w;
        }
    };

    Item cur, nxt;
    fetch(0, cur);
    // every wave walks NGP = NGW rounded up to D ring steps; steps past its own
    // ng groups reload its last group (or group gb) and skip the math
    const int NGP = (NGW + D - 1) / D * D;
    auto gaddr = [&](int gl) { return gb + max(0, min(gl, ng - 1)); };
#pragma unroll
    for (int d = 0; d < D; ++d) issue(d, cur.g, cur.u, cur.x, gaddr(d));
    stage(cur, sc_base);

    for (int j = 0; j < n_my; ++j) {
        const bool has_next = j + 1 < n_my;
        if (has_next) fetch(j + 1, nxt);
        else nxt = cur;
        const float* my_sc = sc_base + (j & 1) * NGW * 64;
        floatx4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};

        // do-while: the body runs at least once (NGP >= D), so the loads of the next
        // item's scales are always followed by ring refills and the wait before
        // staging them leaves the refills in flight
        int g0 = 0;
        do {
            const bool last = g0 + D >= NGP;
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int gl = g0 + d;
                // consume slot d, then refill the same registers: the old and new
                // contents are never live together, so the ring needs no register
                // copies (which would wait for the refill) at the block's end
                if (gl < ng) {
                    floatx4_t Cg = {0.f, 0.f, 0.f, 0.f}, Cu = Cg, Cx = Cg;
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        uint32_t Ag[4], Au[4], Bx[4];
                        code_operand<BITS>(wg[d], s, Ag);
                        code_operand<BITS>(wu[d], s, Au);
                        act_operand<BITS>(xv[d], s, Bx);
                        Cg = mfma16(Ag, Bx, Cg);
                        Cu = mfma16(Au, Bx, Cu);
                        Cx = mfma16(ONE, Bx, Cx);
                    }
                    const float* scg = my_sc + gl * 64 + 4 * q;
                    const float4 sg = *reinterpret_cast<const float4*>(scg);
                    const float4 bg = *reinterpret_cast<const float4*>(scg + 16);
                    const float4 su = *reinterpret_cast<const float4*>(scg + 32);
                    const float4 bu = *reinterpret_cast<const float4*>(scg + 48);
                    accg[0] = fmaf(sg.x, Cg[0], fmaf(bg.x, Cx[0], accg[0]));
                    accg[1] = fmaf(sg.y, Cg[1], fmaf(bg.y, Cx[1], accg[1]));
                    accg[2] = fmaf(sg.z, Cg[2], fmaf(bg.z, Cx[2], accg[2]));
                    accg[3] = fmaf(sg.w, Cg[3], fmaf(bg.w, Cx[3], accg[3]));
                    accu[0] = fmaf(su.x, Cu[0], fmaf(bu.x, Cx[0], accu[0]));
                    accu[1] = fmaf(su.y, Cu[1], fmaf(bu.y, Cx[1], accu[1]));
                    accu[2] = fmaf(su.z, Cu[2], fmaf(bu.z, Cx[2], accu[2]));
                    accu[3] = fmaf(su.w, Cu[3], fmaf(bu.w, Cx[3], accu[3]));
                }
                __builtin_amdgcn_sched_barrier(0);
                // refill: same item D groups on, else the next item's group at
                // the same ring position (the last item reloads its own last
                // group: harmless, keeps every step's loads alike)
                const bool go_next = last && has_next;
                issue(d, go_next ? nxt.g : cur.g, go_next ? nxt.u : cur.u, go_next ? nxt.x : cur.x,
                      gaddr(!last ? gl + D : (has_next ? d : ng - 1)));
            }
            g0 += D;
        } while (g0 < NGP);

        // ---- sum the 4 waves' partials (fixed order), epilogue in wave 0
        float* mine = red + (w * 64 + lane) * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) { mine[i] = accg[i]; mine[4 + i] = accu[i]; }
        __syncthreads();
        if (w == 0) {
            float hv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float gt = ((red[(0 * 64 + lane) * 8 + i] + red[(1 * 64 + lane) * 8 + i]) +
                                  red[(2 * 64 + lane) * 8 + i]) + red[(3 * 64 + lane) * 8 + i];
                const float upv = ((red[(0 * 64 + lane) * 8 + 4 + i] + red[(1 * 64 + lane) * 8 + 4 + i]) +
                                   red[(2 * 64 + lane) * 8 + 4 + i]) + red[(3 * 64 + lane) * 8 + 4 + i];
                hv[i] = gt / (1.f + expf(-gt)) * upv;
            }
            // sum of h over the tile's 16 rows for this token (fixed order)
            float part = (hv[0] + hv[1]) + (hv[2] + hv[3]);
            part += __shfl_xor(part, 16, kWave);
            part += __shfl_xor(part, 32, kWave);
            if (m < cur.n && cur.row0 >= 0 && cur.row0 + cur.n <= p.P) {
                const int r = cur.row0 + m;
                const int i0 = cur.it * 16;
                if (q == 0) p.hpart[(size_t)r * (I / 16) + cur.it] = part;
                // positions 4q..4q+3 of the tile in all three planes
                uint32_t hi[4], mid[4], lo[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) split3_bf16(hv[i], hi[i], mid[i], lo[i]);
                const size_t plane = (size_t)p.P * I;
                uint16_t* base = p.hp + (size_t)r * I + i0 + 4 * q;
                *reinterpret_cast<uint2*>(base) = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
                *reinterpret_cast<uint2*>(base + plane) = make_uint2(mid[0] | (mid[1] << 16), mid[2] | (mid[3] << 16));
                *reinterpret_cast<uint2*>(base + 2 * plane) = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
            }
        }
        __syncthreads();   // red is reused by the next item
        if (has_next) stage(nxt, sc_base + ((j + 1) & 1) * NGW * 64);
        cur = nxt;
    }
}

// ------------------------------------ gate / up with the activation tile in LDS
// For shapes whose tile of x rows (min(T, 16) rows of H bf16) fits in LDS at
// one workgroup per CU.  Workgroup b owns a contiguous range of items, so its
// consecutive items mostly belong to one work-list entry: it stages that
// entry's x rows in LDS once, already in the pair order of the code operands
// (each 8-element run as 0,4,1,5,2,6,3,7 for 4-bit codes, each 16-element run
// as 0,8,1,9,...,7,15 for 2-bit codes), so a step's B operand is one 16-byte
// LDS read and needs no permutes, together with the rows' float32 sums over
// each group of 128 (the X of the per-group fold, so no all-ones MFMA).  Only the codes stream, through a
// D-deep register ring per wave that runs across item boundaries.  The NW
// waves split K as in the kernel above; the partial sums meet in LDS, and
// four waves share the epilogue (each takes four token columns), adding the
// partials in wave order; the groups of four waves take turns by item, so
// that none falls behind the others.  The partial sums are double-buffered by item
// parity, so an item costs one barrier.  Token columns past the tile's rows
// read one row of zeros.  Rows of the x tile are padded by 16 bytes, so the 16
// rows one step reads fall in 16 different bank groups.
// LDS: x tile [rows_cap + 1][H + 8] bf16 (the last row zero); group sums
// [rows_cap + 1][NG] float (the last row zero); scales [NW][NGW][64] float (a
// wave reads only its own, and stages the next item's once its K loop is
// done); partial sums [2][NW][64][8] float.
template <int BITS, int D, int SJ, int NW>
__global__ __launch_bounds__(64 * NW, 1) void ffn_gateup_xt_kernel(MfmaParams p) {
    static_assert(NW >= 4 && NW % 4 == 0, "groups of four waves share the epilogue");
    constexpr int LB = 128 * BITS / 8 / 4;     // bytes per lane per group (16 or 8)
    constexpr int LW = LB / 4;                 // code words per lane per group
    constexpr int NT = 64 * NW;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, q = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ipe = p.items_per_entry;
    if (blockIdx.x == 0)                                  // the streaming down's counters start at zero
        for (int i = tid; i < p.n_split_ctr; i += NT) p.split_ctr[i] = 0;
    const int n_items = ld_scalar(p.n_work, 0) * ipe;
    const int per = (n_items + (int)gridDim.x - 1) / (int)gridDim.x;
    const int i0 = (int)blockIdx.x * per;
    const int n_my = min(n_items - i0, per);
    if (n_my <= 0) return;
    const int H = p.H, I = p.I, NG = H / kGroup, NGW = (NG + NW - 1) / NW;
    const int rows_cap = p.T < kWorkRows ? p.T : kWorkRows;
    const int xrow = H + 8;                               // bf16 per LDS row of the x tile
    const int gb = (w * NG) / NW, ng = ((w + 1) * NG) / NW - gb;
    constexpr int GB = kGroup * BITS / 8;      // code bytes of one row in one group
    const size_t gstride = (size_t)I * GB;     // from one group of all I rows to the next
    uint16_t* xt = reinterpret_cast<uint16_t*>(smem);
    float* xs = reinterpret_cast<float*>(smem + (((size_t)(rows_cap + 1) * xrow * 2 + 15) & ~(size_t)15));
    float* sc_all = xs + (((rows_cap + 1) * NG + 3) & ~3);
    float* sc_base = sc_all + w * NGW * 64;
    float* red = sc_all + NW * NGW * 64;

    // a lane's codes of group g: base + g * gstride + loff (base uniform)
    const uint32_t loff = (uint32_t)(pair_order_row<BITS>(m) * GB + q * LB);
    struct Item {
        int entry, e, it, row0, n;
        const uint8_t* g;
        const uint8_t* u;
        uint32_t sv[4][SJ];
    };
    auto fetch = [&](int j, Item& I_) {
        const int idx = i0 + j;
        I_.entry = idx / ipe;
        I_.it = idx - I_.entry * ipe;
        const int32_t* ent = p.work + (size_t)I_.entry * kWorkInts;
        I_.e = ld_scalar(ent, 0);
        I_.row0 = ld_scalar(ent, 1);
        I_.n = ld_scalar(ent, 2);
        const int e = (I_.e >= 0 && I_.e < p.E) ? I_.e : 0;
        const size_t wcode = (size_t)e * NG * gstride + (size_t)I_.it * 16 * GB;
        I_.g = p.qa + wcode;
        I_.u = p.qb + wcode;
        if (ng > 0) {
#pragma unroll
            for (int jj = 0; jj < SJ; ++jj) {
                const int id2 = lane + 64 * jj;
                const int gl = min(id2 >> 4, ng - 1), r = id2 & 15;
                const size_t src = ((size_t)e * I + I_.it * 16 + pair_order_row<BITS>(r)) * NG + gb + gl;
                I_.sv[0][jj] = p.sa[src]; I_.sv[1][jj] = p.ba[src];
                I_.sv[2][jj] = p.sb[src]; I_.sv[3][jj] = p.bb[src];
            }
        }
    };
    auto stage = [&](const Item& I_, float* dst_base) {
#pragma unroll
        for (int jj = 0; jj < SJ; ++jj) {
            const int id2 = lane + 64 * jj;
            const int gl = id2 >> 4, r = id2 & 15;
            if (gl < ng) {
                const float s1 = f16_bits_to_f32(I_.sv[0][jj]), b1 = f16_bits_to_f32(I_.sv[1][jj]);
                const float s2 = f16_bits_to_f32(I_.sv[2][jj]), b2 = f16_bits_to_f32(I_.sv[3][jj]);
                float* dst = dst_base + gl * 64 + r;
                dst[0] = s1 * kInvLever<BITS>;
                dst[16] = fmaf(-kOffset<BITS>, s1, b1);
                dst[32] = s2 * kInvLever<BITS>;
                dst[48] = fmaf(-kOffset<BITS>, s2, b2);
            }
        }
    };
    // the entry's x rows into the tile, in pair order (all threads)
    auto stage_x = [&](int entry) {
        const int32_t* ent = p.work + (size_t)entry * kWorkInts;
        const int n = max(0, min(ld_scalar(ent, 2), rows_cap));
        constexpr uint32_t LO = 0x05040100u, HI = 0x07060302u;
        constexpr int RUN = BITS == 4 ? 8 : 16;           // elements per permuted run
        const int runs = H / RUN;
        for (int idx = tid; idx < n * runs; idx += NT) {
            const int t = idx / runs, c = idx - t * runs;
            int tok = ent[4 + t];
            tok = (tok >= 0 && tok < p.T) ? tok : 0;
            const uint4* src = reinterpret_cast<const uint4*>(p.x + (size_t)tok * H + c * RUN);
            uint4* dst = reinterpret_cast<uint4*>(xt + t * xrow + c * RUN);
            if constexpr (BITS == 4) {
                const uint4 v = src[0];                   // (x0,x1) (x2,x3) (x4,x5) (x6,x7)
                dst[0] = make_uint4(__builtin_amdgcn_perm(v.z, v.x, LO), __builtin_amdgcn_perm(v.z, v.x, HI),
                                    __builtin_amdgcn_perm(v.w, v.y, LO), __builtin_amdgcn_perm(v.w, v.y, HI));
            } else {
                const uint4 a = src[0], b = src[1];       // (x0,x1) .. (x6,x7), (x8,x9) .. (x14,x15)
                dst[0] = make_uint4(__builtin_amdgcn_perm(b.x, a.x, LO), __builtin_amdgcn_perm(b.x, a.x, HI),
                                    __builtin_amdgcn_perm(b.y, a.y, LO), __builtin_amdgcn_perm(b.y, a.y, HI));
                dst[1] = make_uint4(__builtin_amdgcn_perm(b.z, a.z, LO), __builtin_amdgcn_perm(b.z, a.z, HI),
                                    __builtin_amdgcn_perm(b.w, a.w, LO), __builtin_amdgcn_perm(b.w, a.w, HI));
            }
        }
        // X of row t, group g: the float32 sum of its 128 elements in order
        for (int idx = tid; idx < n * NG; idx += NT) {
            const int t = idx / NG, g = idx - t * NG;
            int tok = ent[4 + t];
            tok = (tok >= 0 && tok < p.T) ? tok : 0;
            const uint4* src = reinterpret_cast<const uint4*>(p.x + (size_t)tok * H + g * kGroup);
            float sum = 0.f;
            for (int c = 0; c < kGroup / 8; ++c) {
                const uint4 v = src[c];
                const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    sum += __uint_as_float(wv[e2] << 16);
                    sum += __uint_as_float(wv[e2] & 0xFFFF0000u);
                }
            }
            xs[t * NG + g] = sum;
        }
    };

    uint32_t wg[D][LW], wu[D][LW];
    auto issue = [&](int slot, const uint8_t* gp, const uint8_t* up, int g) {
        const gbytes_t gq = uniform_gptr(gp + (size_t)g * gstride);
        const gbytes_t uq = uniform_gptr(up + (size_t)g * gstride);
        if constexpr (BITS == 4) {
            const u32x4_t A = __builtin_nontemporal_load(reinterpret_cast<gu32x4_t>(gq + loff));
            const u32x4_t B = __builtin_nontemporal_load(reinterpret_cast<gu32x4_t>(uq + loff));
            wg[slot][0] = A.x; wg[slot][1] = A.y; wg[slot][2] = A.z; wg[slot][3] = A.w;
            wu[slot][0] = B.x; wu[slot][1] = B.y; wu[slot][2] = B.z; wu[slot][3] = B.w;
        } else {
            const u32x2_t A = *reinterpret_cast<gu32x2_t>(gq + loff);
            const u32x2_t B = *reinterpret_cast<gu32x2_t>(uq + loff);
            wg[slot][0] = A.x; wg[slot][1] = A.y;
            wu[slot][0] = B.x; wu[slot][1] = B.y;
        }
    };

    Item cur, nxt;
    fetch(0, cur);
    const int NGP = (NGW + D - 1) / D * D;
    auto gaddr = [&](int gl) { return gb + max(0, min(gl, ng - 1)); };
#pragma unroll
    for (int d = 0; d < D; ++d) issue(d, cur.g, cur.u, gaddr(d));
    stage(cur, sc_base);
    for (int i = tid; i < xrow / 8; i += NT)
        reinterpret_cast<uint4*>(xt + rows_cap * xrow)[i] = make_uint4(0u, 0u, 0u, 0u);
    for (int i = tid; i < NG; i += NT) xs[rows_cap * NG + i] = 0.f;
    stage_x(cur.entry);
    lds_barrier();

    for (int j = 0; j < n_my; ++j) {
        const bool has_next = j + 1 < n_my;
        if (has_next) fetch(j + 1, nxt);
        else nxt = cur;
        const float* my_sc = sc_base;
        const int xr = m < cur.n ? m : rows_cap;
        const uint16_t* xcol = xt + xr * xrow + 32 * q;
        const float* xsum = xs + xr * NG + gb;
        floatx4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
        int g0 = 0;
        do {
            const bool last = g0 + D >= NGP;
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int gl = g0 + d;
                if (gl < ng) {
                    floatx4_t Cg = {0.f, 0.f, 0.f, 0.f}, Cu = Cg;
                    const uint16_t* xg = xcol + (gb + gl) * kGroup;
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        uint32_t Ag[4], Au[4];
                        code_operand<BITS>(wg[d], s, Ag);
                        code_operand<BITS>(wu[d], s, Au);
                        const uint4 X = *reinterpret_cast<const uint4*>(xg + 8 * s);
                        const uint32_t Bx[4] = {X.x, X.y, X.z, X.w};
                        Cg = mfma16(Ag, Bx, Cg);
                        Cu = mfma16(Au, Bx, Cu);
                    }
                    const float Xg = xsum[gl];
                    const float* scg = my_sc + gl * 64 + 4 * q;
                    const float4 sg = *reinterpret_cast<const float4*>(scg);
                    const float4 bg = *reinterpret_cast<const float4*>(scg + 16);
                    const float4 su = *reinterpret_cast<const float4*>(scg + 32);
                    const float4 bu = *reinterpret_cast<const float4*>(scg + 48);
                    accg[0] = fmaf(sg.x, Cg[0], fmaf(bg.x, Xg, accg[0]));
                    accg[1] = fmaf(sg.y, Cg[1], fmaf(bg.y, Xg, accg[1]));
                    accg[2] = fmaf(sg.z, Cg[2], fmaf(bg.z, Xg, accg[2]));
                    accg[3] = fmaf(sg.w, Cg[3], fmaf(bg.w, Xg, accg[3]));
                    accu[0] = fmaf(su.x, Cu[0], fmaf(bu.x, Xg, accu[0]));
                    accu[1] = fmaf(su.y, Cu[1], fmaf(bu.y, Xg, accu[1]));
                    accu[2] = fmaf(su.z, Cu[2], fmaf(bu.z, Xg, accu[2]));
                    accu[3] = fmaf(su.w, Cu[3], fmaf(bu.w, Xg, accu[3]));
                }
                // consume slot d, then refill the same registers (a scheduling
                // barrier keeps the refill after the use and in ring order)
                __builtin_amdgcn_sched_barrier(0);
                const bool go_next = last && has_next;
                issue(d, go_next ? nxt.g : cur.g, go_next ? nxt.u : cur.u,
                      gaddr(!last ? gl + D : (has_next ? d : ng - 1)));
            }
            g0 += D;
        } while (g0 < NGP);

        // ---- the NW waves' partials meet in LDS; waves ew..ew+3 finish the
        // item: wave ew + w takes token columns 4w..4w+3, lane v = 64 w + lane
        // holds column v / 16, rows 4 ((v / 4) % 4) + v % 4 of the 16-row tile
        float* redb = red + (j & 1) * (NW * 64 * 8);
        float* mine = redb + (w * 64 + lane) * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) { mine[i] = accg[i]; mine[4 + i] = accu[i]; }
        lds_barrier();
        const int ew = 4 * (j % (NW / 4));
        if (w >= ew && w < ew + 4) {
            const int v = (w - ew) * 64 + lane, mc = v >> 4, qc = (v >> 2) & 3, ic = v & 3;
            const int src = (qc * 16 + mc) * 8 + ic;      // the MFMA lane (qc, mc), value ic
            float gt = redb[src], upv = redb[src + 4];
            for (int w2 = 1; w2 < NW; ++w2) {
                gt += redb[w2 * 64 * 8 + src];
                upv += redb[w2 * 64 * 8 + src + 4];
            }
            const float hv = gt / (1.f + expf(-gt)) * upv;
            // sum of h over the tile's 16 rows for this token (fixed order)
            float part = hv + __shfl_xor(hv, 1, kWave);
            part += __shfl_xor(part, 2, kWave);
            part += __shfl_xor(part, 4, kWave);
            part += __shfl_xor(part, 8, kWave);
            if (mc < cur.n && cur.row0 >= 0 && cur.row0 + cur.n <= p.P) {
                const int r = cur.row0 + mc;
                if ((v & 15) == 0) p.hpart[(size_t)r * (I / 16) + cur.it] = part;
                uint32_t hi, mid, lo;
                split3_bf16(hv, hi, mid, lo);
                const size_t plane = (size_t)p.P * I;
                uint16_t* base = p.hp + (size_t)r * I + cur.it * 16 + 4 * qc + ic;
                base[0] = (uint16_t)hi;
                base[plane] = (uint16_t)mid;
                base[2 * plane] = (uint16_t)lo;
            }
        }
        if (has_next) {
            stage(nxt, sc_base);
            // past the barrier above every wave is done with the old x rows
            if (nxt.entry != cur.entry) {
                stage_x(nxt.entry);
                lds_barrier();
            }
        }
        cur = nxt;
    }
}

// ------------------------------ gate / up with int8 activation planes in LDS
// The x-tile kernel above with the products on v_mfma_i32_16x16x64_i8.  Each
// entry's x rows are staged once as three int8 planes per group of 128 with a
// power-of-two scale: hs = 2^e, e = max(exponent(max |x|) - 5, -100), so that
// max |x| / hs lies in [32, 64), and q_p = rint(rem_p / 2^(e - 7 p)) with
// rem_{p+1} = rem_p - q_p 2^(e - 7 p) (each remainder exact), i.e.
// x = hs (q_0 + 2^-7 q_1 + 2^-14 q_2) + a tail of at most 2^-15 hs.  The codes
// are bytes (i8_code_operand) and the B operand (columns = weight rows in
// pair order, as the A rows of the kernel above); the A operand's 16 rows are
// 4 tokens x (planes 0-2 and a zero row), so a lane's D rows are the planes of
// one token and the group sum over K is exact in int32: the lane folds
// F = C_0 + 2^-7 C_1 + 2^-14 C_2 as s hs F + b X per group (s, b: the weight
// row's fp16 scale and bias; X: the token's float sum of x over the group).
// Two MFMAs per 16-row tile, matrix and group for up to 4 tokens, against 8
// in the kernel above.  NW is 10 or 12 (the launcher picks the count that
// splits K most evenly); with 10, waves 0-3 and 4-7 take the epilogue in turns.
// LDS: planes [rows_cap][NG][3][128] int8 (the 16-byte pieces of plane row
// (t, p) swizzled by (t % 4) | 4 (p / 2): the 12 rows one read phase touches
// fall on distinct banks), a 128-byte zero row, (hs, X) [rows_cap][NG] float
// pairs, scales [NW][NGW][16][4] float (gate s, b, up s, b of weight row m),
// partial sums [2][NW][64][2 NBM] float.
constexpr int kXt8Row = 3 * 128;                  // bytes of one (token, group) of the plane tile

__device__ __forceinline__ int xt8_swz(int t, int pl) { return (t & 3) | ((pl >> 1) << 2); }

template <int BITS, int D, int SJ, int NW, int NBM>
__global__ __launch_bounds__(64 * NW, 1) void ffn_gateup_xt8_kernel(MfmaParams p) {
    static_assert(NW >= 4, "groups of four waves share the epilogue");
    constexpr int LB = 128 * BITS / 8 / 4;     // bytes per lane per group (16 or 8)
    constexpr int LW = LB / 4;                 // code words per lane per group
    constexpr int NT = 64 * NW;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, q = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ipe = p.items_per_entry;
    if (blockIdx.x == 0)                                  // the streaming down's counters start at zero
        for (int i = tid; i < p.n_split_ctr; i += NT) p.split_ctr[i] = 0;
    const int n_items = ld_scalar(p.n_work, 0) * ipe;
    const int per = (n_items + (int)gridDim.x - 1) / (int)gridDim.x;
    const int i0 = (int)blockIdx.x * per;
    const int n_my = min(n_items - i0, per);
    if (n_my <= 0) return;
    const int H = p.H, I = p.I, NG = H / kGroup, NGW = (NG + NW - 1) / NW;
    const int rows_cap = p.T < kWorkRows ? p.T : kWorkRows;
    const int gb = (w * NG) / NW, ng = ((w + 1) * NG) / NW - gb;
    constexpr int GB = kGroup * BITS / 8;      // code bytes of one row in one group
    const size_t gstride = (size_t)I * GB;     // from one group of all I rows to the next
    uint8_t* xq = smem;
    const int zoff = rows_cap * NG * kXt8Row;             // the zero row
    float2* xs = reinterpret_cast<float2*>(smem + zoff + 128);
    float* sc_all = reinterpret_cast<float*>(smem + ((zoff + 128 + rows_cap * NG * 8 + 15) & ~15));
    float* sc_base = sc_all + w * NGW * 64;
    float* red = sc_all + NW * NGW * 64;

    // a lane's codes of group g: base + g * gstride + loff (base uniform)
    const uint32_t loff = (uint32_t)(pair_order_row<BITS>(m) * GB + q * LB);
    struct Item {
        int entry, e, it, row0, n;
        const uint8_t* g;
        const uint8_t* u;
        uint32_t sv[4][SJ];
    };
    auto fetch = [&](int j, Item& I_) {
        const int idx = i0 + j;
        I_.entry = idx / ipe;
        I_.it = idx - I_.entry * ipe;
        const int32_t* ent = p.work + (size_t)I_.entry * kWorkInts;
        I_.e = ld_scalar(ent, 0);
        I_.row0 = ld_scalar(ent, 1);
        I_.n = ld_scalar(ent, 2);
        const int e = (I_.e >= 0 && I_.e < p.E) ? I_.e : 0;
        const size_t wcode = (size_t)e * NG * gstride + (size_t)I_.it * 16 * GB;
        I_.g = p.qa + wcode;
        I_.u = p.qb + wcode;
        if (ng > 0) {
#pragma unroll
            for (int jj = 0; jj < SJ; ++jj) {
                const int id2 = lane + 64 * jj;
                const int gl = min(id2 >> 4, ng - 1), r = id2 & 15;
                const size_t src = ((size_t)e * I + I_.it * 16 + pair_order_row<BITS>(r)) * NG + gb + gl;
                I_.sv[0][jj] = p.sa[src]; I_.sv[1][jj] = p.ba[src];
                I_.sv[2][jj] = p.sb[src]; I_.sv[3][jj] = p.bb[src];
            }
        }
    };
    auto stage = [&](const Item& I_, float* dst_base) {
#pragma unroll
        for (int jj = 0; jj < SJ; ++jj) {
            const int id2 = lane + 64 * jj;
            const int gl = id2 >> 4, r = id2 & 15;
            if (gl < ng)
                *reinterpret_cast<float4*>(dst_base + gl * 64 + 4 * r) =
                    make_float4(f16_bits_to_f32(I_.sv[0][jj]), f16_bits_to_f32(I_.sv[1][jj]),
                                f16_bits_to_f32(I_.sv[2][jj]), f16_bits_to_f32(I_.sv[3][jj]));
        }
    };
    // the entry's x rows as int8 planes (all threads): a thread takes runs of
    // RUN consecutive elements of one row, whose bytes are contiguous in the
    // operand order (8 for 4-bit codes: half a 16-byte piece; 16 for 2-bit: a
    // whole piece); the RPG threads of a group are adjacent lanes and reduce
    // max |x| and the sum of x among themselves in a fixed butterfly order.
    auto stage_x = [&](int entry) {
        const int32_t* ent = p.work + (size_t)entry * kWorkInts;
        const int n = max(0, min(ld_scalar(ent, 2), rows_cap));
        constexpr int RUN = BITS == 4 ? 8 : 16, RPG = kGroup / RUN, V = RUN / 8;
        constexpr int U = 4;                                    // runs per thread per pass, loads in flight together
        const int runs = H / RUN, total = n * runs;
        constexpr float kMagic = 12582912.f;                    // 1.5 * 2^23: adding it rounds to an integer
        for (int base = 0; base < total; base += U * NT) {
            uint4 v[U][V];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int idx = base + u * NT + tid, ii = idx < total ? idx : 0;
                const int t = ii / runs, c = ii - t * runs;
                int tok = ent[4 + t];
                tok = (tok >= 0 && tok < p.T) ? tok : 0;
                const uint4* src = reinterpret_cast<const uint4*>(p.x + (size_t)tok * H + c * RUN);
#pragma unroll
                for (int r8 = 0; r8 < V; ++r8) v[u][r8] = src[r8];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int idx = base + u * NT + tid;          // a group's RPG lanes agree on idx < total
                const int ii = idx < total ? idx : 0;
                const int t = ii / runs, c = ii - t * runs, g = c / RPG, cr = c - g * RPG;
                float xf[RUN];
#pragma unroll
                for (int r8 = 0; r8 < V; ++r8) {
                    const uint32_t wv[4] = {v[u][r8].x, v[u][r8].y, v[u][r8].z, v[u][r8].w};
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) {
                        xf[8 * r8 + 2 * e2] = __uint_as_float(wv[e2] << 16);
                        xf[8 * r8 + 2 * e2 + 1] = __uint_as_float(wv[e2] & 0xFFFF0000u);
                    }
                }
                float mx = 0.f, sm = 0.f;
#pragma unroll
                for (int e2 = 0; e2 < RUN; ++e2) {
                    mx = fmaxf(mx, fabsf(xf[e2]));
                    sm += xf[e2];
                }
#pragma unroll
                for (int o = 1; o < RPG; o <<= 1) {
                    mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
                    sm += __shfl_xor(sm, o, kWave);
                }
                const int e0 = max((int)((__float_as_uint(mx) >> 23) & 0xFFu) - 127 - 5, -100);
                uint32_t tb[3][RUN];
#pragma unroll
                for (int e2 = 0; e2 < RUN; ++e2) {
                    float rem = xf[e2];
#pragma unroll
                    for (int pl = 0; pl < 3; ++pl) {
                        const float tv = fmaf(rem, ldexpf(1.f, 7 * pl - e0), kMagic);
                        tb[pl][e2] = __float_as_uint(tv);              // low byte: the plane's int8 value
                        rem = fmaf(-(tv - kMagic), ldexpf(1.f, e0 - 7 * pl), rem);
                    }
                }
                if (idx < total) {
                    uint8_t* row = xq + ((size_t)t * NG + g) * kXt8Row;
#pragma unroll
                    for (int pl = 0; pl < 3; ++pl) {
                        // dword d of a piece holds elements kl with byte order 4 d + b (i8_code_operand)
                        if constexpr (BITS == 4) {
                            // elements 0..7 of the run -> dword 0: 0, 2, 4, 6; dword 1: 1, 3, 5, 7
                            const uint32_t d0 = __builtin_amdgcn_perm(__builtin_amdgcn_perm(tb[pl][6], tb[pl][4], 0x0C0C0400u),
                                                                      __builtin_amdgcn_perm(tb[pl][2], tb[pl][0], 0x0C0C0400u), 0x05040100u);
                            const uint32_t d1 = __builtin_amdgcn_perm(__builtin_amdgcn_perm(tb[pl][7], tb[pl][5], 0x0C0C0400u),
                                                                      __builtin_amdgcn_perm(tb[pl][3], tb[pl][1], 0x0C0C0400u), 0x05040100u);
                            const int piece = (cr >> 1) ^ xt8_swz(t, pl);
                            *reinterpret_cast<uint2*>(row + pl * 128 + 16 * piece + 8 * (cr & 1)) = make_uint2(d0, d1);
                        } else {
                            // dword d holds elements d, d + 4, d + 8, d + 12
                            uint32_t dd[4];
#pragma unroll
                            for (int d = 0; d < 4; ++d)
                                dd[d] = __builtin_amdgcn_perm(__builtin_amdgcn_perm(tb[pl][d + 12], tb[pl][d + 8], 0x0C0C0400u),
                                                              __builtin_amdgcn_perm(tb[pl][d + 4], tb[pl][d], 0x0C0C0400u), 0x05040100u);
                            const int piece = cr ^ xt8_swz(t, pl);
                            *reinterpret_cast<uint4*>(row + pl * 128 + 16 * piece) = make_uint4(dd[0], dd[1], dd[2], dd[3]);
                        }
                    }
                    if (cr == 0) xs[t * NG + g] = make_float2(ldexpf(1.f, e0), sm);
                }
            }
        }
    };

    uint32_t wg[D][LW], wu[D][LW];
    auto issue = [&](int slot, const uint8_t* gp, const uint8_t* up, int g) {
        const gbytes_t gq = uniform_gptr(gp + (size_t)g * gstride);
        const gbytes_t uq = uniform_gptr(up + (size_t)g * gstride);
        if constexpr (BITS == 4) {
            const u32x4_t A = __builtin_nontemporal_load(reinterpret_cast<gu32x4_t>(gq + loff));
            const u32x4_t B = __builtin_nontemporal_load(reinterpret_cast<gu32x4_t>(uq + loff));
            wg[slot][0] = A.x; wg[slot][1] = A.y; wg[slot][2] = A.z; wg[slot][3] = A.w;
            wu[slot][0] = B.x; wu[slot][1] = B.y; wu[slot][2] = B.z; wu[slot][3] = B.w;
        } else {
            const u32x2_t A = *reinterpret_cast<gu32x2_t>(gq + loff);
            const u32x2_t B = *reinterpret_cast<gu32x2_t>(uq + loff);
            wg[slot][0] = A.x; wg[slot][1] = A.y;
            wu[slot][0] = B.x; wu[slot][1] = B.y;
        }
    };

    Item cur, nxt;
    fetch(0, cur);
    const int NGP = (NGW + D - 1) / D * D;
    auto gaddr = [&](int gl) { return gb + max(0, min(gl, ng - 1)); };
#pragma unroll
    for (int d = 0; d < D; ++d) issue(d, cur.g, cur.u, gaddr(d));
    stage(cur, sc_base);
    if (tid < 8) reinterpret_cast<uint4*>(smem + zoff)[tid] = make_uint4(0u, 0u, 0u, 0u);
    stage_x(cur.entry);
    lds_barrier();

    // A operand rows: lane row m = 4 t + pl of token 4 b + t (tokens past the
    // tile's rows read token 0; pl = 3 reads the zero row)
    const int at = m >> 2, apl = m & 3;
    const int gsz = apl == 3 ? 0 : kXt8Row;            // a group's step in the plane tile
    for (int j = 0; j < n_my; ++j) {
        const bool has_next = j + 1 < n_my;
        if (has_next) fetch(j + 1, nxt);
        else nxt = cur;
        const float* my_sc = sc_base;
        const int ncl = max(1, min(cur.n, rows_cap));
        const int NB = (ncl + 3) >> 2;
        int aoff[NBM][2];
#pragma unroll
        for (int b = 0; b < NBM; ++b) {
            const int t = 4 * b + at < ncl ? 4 * b + at : 0;
#pragma unroll
            for (int st = 0; st < 2; ++st)
                aoff[b][st] = apl == 3 ? zoff + 16 * (2 * q + st)
                                       : t * NG * kXt8Row + apl * 128 + 16 * ((2 * q + st) ^ xt8_swz(t, apl));
        }
        float accg[NBM], accu[NBM];
#pragma unroll
        for (int b = 0; b < NBM; ++b) { accg[b] = 0.f; accu[b] = 0.f; }
        int g0 = 0;
        do {
            const bool last = g0 + D >= NGP;
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int gl = g0 + d;
                if (gl < ng) {
                    uint32_t Bg[2][4], Bu[2][4];
                    i8_code_operand<BITS>(wg[d], 0, Bg[0]);
                    i8_code_operand<BITS>(wg[d], 1, Bg[1]);
                    i8_code_operand<BITS>(wu[d], 0, Bu[0]);
                    i8_code_operand<BITS>(wu[d], 1, Bu[1]);
                    const float4 sv = *reinterpret_cast<const float4*>(my_sc + gl * 64 + 4 * m);
                    const int goff = (gb + gl) * gsz;
#pragma unroll
                    for (int b = 0; b < NBM; ++b) {
                        if (b < NB) {
                            int32x4_t Cg = {0, 0, 0, 0}, Cu = Cg;
#pragma unroll
                            for (int st = 0; st < 2; ++st) {
                                const uint4 a4 = *reinterpret_cast<const uint4*>(smem + aoff[b][st] + goff);
                                const uint32_t A[4] = {a4.x, a4.y, a4.z, a4.w};
                                Cg = mfma_i8(A, Bg[st], Cg);
                                Cu = mfma_i8(A, Bu[st], Cu);
                            }
                            const float2 hx = xs[min(4 * b + q, rows_cap - 1) * NG + gb + gl];
                            const float Fg = fmaf(0x1p-7f, fmaf(0x1p-7f, (float)Cg[2], (float)Cg[1]), (float)Cg[0]);
                            const float Fu = fmaf(0x1p-7f, fmaf(0x1p-7f, (float)Cu[2], (float)Cu[1]), (float)Cu[0]);
                            accg[b] = fmaf(sv.x * hx.x, Fg, fmaf(sv.y, hx.y, accg[b]));
                            accu[b] = fmaf(sv.z * hx.x, Fu, fmaf(sv.w, hx.y, accu[b]));
                        }
                    }
                }
                // consume slot d, then refill the same registers (a scheduling
                // barrier keeps the refill after the use and in ring order)
                __builtin_amdgcn_sched_barrier(0);
                const bool go_next = last && has_next;
                issue(d, go_next ? nxt.g : cur.g, go_next ? nxt.u : cur.u,
                      gaddr(!last ? gl + D : (has_next ? d : ng - 1)));
            }
            g0 += D;
        } while (g0 < NGP);

        // ---- the NW waves' partials meet in LDS; waves ew..ew+3 finish the
        // item: lane v = 64 (w - ew) + lane takes token v / 16, row v % 16 (the
        // MFMA lane (token % 4) * 16 + row, block token / 4)
        float* redb = red + (j & 1) * (NW * 64 * 2 * NBM);
        float* mine = redb + (w * 64 + lane) * (2 * NBM);
#pragma unroll
        for (int b = 0; b < NBM; ++b) { mine[2 * b] = accg[b]; mine[2 * b + 1] = accu[b]; }
        lds_barrier();
        const int ew = 4 * (j % (NW / 4));
        if (w >= ew && w < ew + 4) {
            const int v = (w - ew) * 64 + lane, t = v >> 4, mm = v & 15;
            if (t < 4 * NBM) {                                // uniform over the 16 lanes of a token
                const int src = ((t & 3) * 16 + mm) * (2 * NBM) + 2 * (t >> 2);
                float gt = redb[src], upv = redb[src + 1];
                for (int w2 = 1; w2 < NW; ++w2) {
                    gt += redb[w2 * 64 * 2 * NBM + src];
                    upv += redb[w2 * 64 * 2 * NBM + src + 1];
                }
                const float hv = gt / (1.f + expf(-gt)) * upv;
                // sum of h over the tile's 16 rows for this token (fixed order)
                float part = hv + __shfl_xor(hv, 1, kWave);
                part += __shfl_xor(part, 2, kWave);
                part += __shfl_xor(part, 4, kWave);
                part += __shfl_xor(part, 8, kWave);
                if (t < ncl && cur.row0 >= 0 && cur.row0 + cur.n <= p.P) {
                    const int r = cur.row0 + t;
                    if (mm == 0) p.hpart[(size_t)r * (I / 16) + cur.it] = part;
                    uint32_t hi, mid, lo;
                    split3_bf16(hv, hi, mid, lo);
                    const size_t plane = (size_t)p.P * I;
                    uint16_t* hb = p.hp + (size_t)r * I + cur.it * 16 + mm;
                    hb[0] = (uint16_t)hi;
                    hb[plane] = (uint16_t)mid;
                    hb[2 * plane] = (uint16_t)lo;
                }
            }
        }
        if (has_next) {
            stage(nxt, sc_base);
            // past the barrier above every wave is done with the old x planes
            if (nxt.entry != cur.entry) {
                stage_x(nxt.entry);
                lds_barrier();
            }
        }
        cur = nxt;
    }
}

// ------------------------------------------------------------------- down
// Persistent like gate/up.  The 4 waves form 4/KS row tiles of 32 output rows
// times KS parts of K: with a short K (I / 128 small) each wave keeps several
// groups to stream, so its ring has something to prefetch.  An item is one
// work-list tile times 32 * 4/KS output rows.  B operand = the three bf16
// planes of h (already in pair order), three MFMAs per step; the bias term
// uses the per-16-row partial sums of h.
// LDS: [kWaves][2][NGW][2][32] float scales (s/L, b - (128/L) s) by item
// parity, then [kWaves][64][8] partial sums.
template <int BITS, int D, int SJ, int KS>
__global__ __launch_bounds__(256) void ffn_down_mfma_kernel(MfmaParams p) {
    constexpr int LB = 128 * BITS / 8 / 4;
    constexpr int LW = LB / 4;
    extern __shared__ float lds[];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, m = lane & 15, q = lane >> 4;
    const int ipe = p.items_per_entry;
    const int n_items = ld_scalar(p.n_work, 0) * ipe;
    if ((int)blockIdx.x >= n_items) return;
    const int n_my = (n_items - 1 - (int)blockIdx.x) / (int)gridDim.x + 1;
    constexpr int RT = kWaves / KS;            // row tiles per item
    const int tw = w / KS, kp = w % KS;        // this wave's row tile and K part
    const int H = p.H, I = p.I, NG = I / kGroup, NGW = (NG + KS - 1) / KS;
    const int gb = (kp * NG) / KS, ng = ((kp + 1) * NG) / KS - gb;
    constexpr int GB = kGroup * BITS / 8;      // code bytes of one row in one group
    const size_t gstride = (size_t)H * GB;     // from one group of all H rows to the next
    float* sc_base = lds + w * 2 * NGW * 64;
    float* red = lds + kWaves * 2 * NGW * 64;
    const size_t plane = (size_t)p.P * I;

    struct Item {
        int e, it, row0, n;
        const uint8_t* c0;
        const uint16_t* h;
        const float* part;
        uint32_t sv[2][SJ];
    };
    auto fetch = [&](int j, Item& I_) {
        const int idx = (int)blockIdx.x + j * (int)gridDim.x;
        const int32_t* ent = p.work + (size_t)(idx / ipe) * kWorkInts;
        I_.it = idx % ipe;
        I_.e = ld_scalar(ent, 0);
        I_.row0 = ld_scalar(ent, 1);
        I_.n = ld_scalar(ent, 2);
        const int e = (I_.e >= 0 && I_.e < p.E) ? I_.e : 0;
        const bool ok_rows = I_.row0 >= 0 && I_.n >= 1 && I_.n <= kWorkRows && I_.row0 + I_.n <= p.P;
        const int r = ok_rows ? I_.row0 + (m < I_.n ? m : 0) : 0;   // empty columns reuse row 0
        const int n0 = (I_.it * RT + tw) * 32;
        I_.c0 = p.qa + (size_t)e * NG * gstride + (size_t)(n0 + m) * GB + q * LB;
        I_.h = p.hp + (size_t)r * I + q * 32;
        I_.part = p.hpart + (size_t)r * (I / 16);
        if (ng > 0) {
#pragma unroll
            for (int jj = 0; jj < SJ; ++jj) {
                const int id2 = lane + 64 * jj;
                const int gl = min(id2 >> 5, ng - 1), rr = id2 & 31;
                const size_t src = ((size_t)e * H + n0 + rr) * NG + gb + gl;
                I_.sv[0][jj] = p.sa[src]; I_.sv[1][jj] = p.ba[src];
            }
        }
    };
    auto stage = [&](const Item& I_, float* dst_base) {
#pragma unroll
        for (int jj = 0; jj < SJ; ++jj) {
            const int id2 = lane + 64 * jj;
            const int gl = id2 >> 5, rr = id2 & 31;
            if (gl < ng) {
                const float sv = f16_bits_to_f32(I_.sv[0][jj]), bv = f16_bits_to_f32(I_.sv[1][jj]);
                dst_base[gl * 64 + rr] = sv * kInvLever<BITS>;
                dst_base[gl * 64 + 32 + rr] = fmaf(-kOffset<BITS>, sv, bv);
            }
        }
    };

    uint32_t w0[D][LW], w1[D][LW], hv[D][3][16];
    float4 hp0[D], hp1[D];
    auto issue = [&](int slot, const uint8_t* cp, const uint16_t* hpp, const float* pp, int g) {
        if constexpr (BITS == 4) {
            const uint4 A = *reinterpret_cast<const uint4*>(cp + (size_t)g * gstride);
            const uint4 B = *reinterpret_cast<const uint4*>(cp + 16 * GB + (size_t)g * gstride);
            w0[slot][0] = A.x; w0[slot][1] = A.y; w0[slot][2] = A.z; w0[slot][3] = A.w;
            w1[slot][0] = B.x; w1[slot][1] = B.y; w1[slot][2] = B.z; w1[slot][3] = B.w;
        } else {
            const uint2 A = *reinterpret_cast<const uint2*>(cp + (size_t)g * gstride);
            const uint2 B = *reinterpret_cast<const uint2*>(cp + 16 * GB + (size_t)g * gstride);
            w0[slot][0] = A.x; w0[slot][1] = A.y;
            w1[slot][0] = B.x; w1[slot][1] = B.y;
        }
#pragma unroll
        for (int pl = 0; pl < 3; ++pl) {
            const uint4* src = reinterpret_cast<const uint4*>(hpp + pl * plane + (size_t)g * kGroup);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const uint4 X = src[v];
                hv[slot][pl][4 * v] = X.x; hv[slot][pl][4 * v + 1] = X.y;
                hv[slot][pl][4 * v + 2] = X.z; hv[slot][pl][4 * v + 3] = X.w;
            }
        }
        hp0[slot] = *reinterpret_cast<const float4*>(pp + 8 * g);
        hp1[slot] = *reinterpret_cast<const float4*>(pp + 8 * g + 4);
    };

    Item cur, nxt;
    fetch(0, cur);
    const int NGP = (NGW + D - 1) / D * D;
    auto gaddr = [&](int gl) { return gb + max(0, min(gl, ng - 1)); };
#pragma unroll
    for (int d = 0; d < D; ++d) issue(d, cur.c0, cur.h, cur.part, gaddr(d));
    stage(cur, sc_base);

    for (int j = 0; j < n_my; ++j) {
        const bool has_next = j + 1 < n_my;
        if (has_next) fetch(j + 1, nxt);
        else nxt = cur;
        const float* my_sc = sc_base + (j & 1) * NGW * 64;
        floatx4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;

        // do-while: the body runs at least once (NGP >= D), so the loads of the next
        // item's scales are always followed by ring refills and the wait before
        // staging them leaves the refills in flight
        int g0 = 0;
        do {
            const bool last = g0 + D >= NGP;
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int gl = g0 + d;
                // consume slot d, then refill it (see the gate/up kernel)
                if (gl < ng) {
                    // sum of this lane's token's h over group g (8 partial sums)
                    const float Hs = ((hp0[d].x + hp0[d].y) + (hp0[d].z + hp0[d].w)) +
                                     ((hp1[d].x + hp1[d].y) + (hp1[d].z + hp1[d].w));
                    floatx4_t C0 = {0.f, 0.f, 0.f, 0.f}, C1 = C0;
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        uint32_t A0[4], A1[4];
                        code_operand<BITS>(w0[d], s, A0);
                        code_operand<BITS>(w1[d], s, A1);
#pragma unroll
                        for (int pl = 0; pl < 3; ++pl) {
                            // planes are stored in pair order: step s = words 4s..4s+3
                            const uint32_t Bh[4] = {hv[d][pl][4 * s], hv[d][pl][4 * s + 1], hv[d][pl][4 * s + 2],
                                                    hv[d][pl][4 * s + 3]};
                            C0 = mfma16(A0, Bh, C0);
                            C1 = mfma16(A1, Bh, C1);
                        }
                    }
                    const float* scg = my_sc + gl * 64 + 4 * q;
                    const float4 s0 = *reinterpret_cast<const float4*>(scg);
                    const float4 s1 = *reinterpret_cast<const float4*>(scg + 16);
                    const float4 b0 = *reinterpret_cast<const float4*>(scg + 32);
                    const float4 b1 = *reinterpret_cast<const float4*>(scg + 48);
                    // C = sum (128 + L q) h  ->  (s/L) C + (b - (128/L) s) Hsum
                    acc0[0] = fmaf(s0.x, C0[0], fmaf(b0.x, Hs, acc0[0]));
                    acc0[1] = fmaf(s0.y, C0[1], fmaf(b0.y, Hs, acc0[1]));
                    acc0[2] = fmaf(s0.z, C0[2], fmaf(b0.z, Hs, acc0[2]));
                    acc0[3] = fmaf(s0.w, C0[3], fmaf(b0.w, Hs, acc0[3]));
                    acc1[0] = fmaf(s1.x, C1[0], fmaf(b1.x, Hs, acc1[0]));
                    acc1[1] = fmaf(s1.y, C1[1], fmaf(b1.y, Hs, acc1[1]));
                    acc1[2] = fmaf(s1.z, C1[2], fmaf(b1.z, Hs, acc1[2]));
                    acc1[3] = fmaf(s1.w, C1[3], fmaf(b1.w, Hs, acc1[3]));
                }
                __builtin_amdgcn_sched_barrier(0);
                const bool go_next = last && has_next;
                issue(d, go_next ? nxt.c0 : cur.c0, go_next ? nxt.h : cur.h, go_next ? nxt.part : cur.part,
                      gaddr(!last ? gl + D : (has_next ? d : ng - 1)));
            }
            g0 += D;
        } while (g0 < NGP);
        float* mine = red + (w * 64 + lane) * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) { mine[i] = acc0[i]; mine[4 + i] = acc1[i]; }
        __syncthreads();
        if (kp == 0 && m < cur.n && cur.row0 >= 0 && cur.row0 + cur.n <= p.P) {
            // the tile's KS partial sums in fixed order
            float o[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float v = red[(w * 64 + lane) * 8 + i];
#pragma unroll
                for (int k2 = 1; k2 < KS; ++k2) v += red[((w + k2) * 64 + lane) * 8 + i];
                o[i] = v;
            }
            uint16_t* yrow = p.y + (size_t)(cur.row0 + m) * H + (cur.it * RT + tw) * 32 + 4 * q;
            uint2 o0, o1;
            o0.x = f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16);
            o0.y = f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16);
            o1.x = f32_to_bf16_bits(o[4]) | (f32_to_bf16_bits(o[5]) << 16);
            o1.y = f32_to_bf16_bits(o[6]) | (f32_to_bf16_bits(o[7]) << 16);
            *reinterpret_cast<uint2*>(yrow) = o0;
            *reinterpret_cast<uint2*>(yrow + 16) = o1;
        }
        __syncthreads();
        if (has_next) stage(nxt, sc_base + ((j + 1) & 1) * NGW * 64);
        cur = nxt;
    }
}

// ------------------------------------------------------------------ launch

size_t mfma_workspace_bytes(const moe_dims& d) {
    const size_t P = (size_t)d.T * d.k;
    const size_t planes = 3 * P * d.I * sizeof(uint16_t);
    const size_t part = P * (d.I / 16) * sizeof(float);
    return ((planes + 255) & ~(size_t)255) + ((part + 255) & ~(size_t)255) + down_split_bytes(d);
}

static MfmaParams mfma_params(const FfnArgs& a) {
    const moe_dims& d = a.d;
    MfmaParams p{};
    p.x = a.x; p.work = a.work; p.n_work = a.n_work; p.y = a.y;
    p.T = d.T; p.H = d.H; p.I = d.I; p.k = d.k; p.E = d.E; p.P = d.T * d.k;
    const size_t P = (size_t)p.P;
    char* ws = reinterpret_cast<char*>(a.h);
    p.hp = reinterpret_cast<uint16_t*>(ws);
    p.hpart = reinterpret_cast<float*>(ws + ((3 * P * d.I * sizeof(uint16_t) + 255) & ~(size_t)255));
    return p;
}

static size_t mfma_lds_bytes(int NG) {
    const int NGW = (NG + kWaves - 1) / kWaves;
    return ((size_t)kWaves * 2 * NGW * 64 + (size_t)kWaves * 64 * 8) * sizeof(float);
}

// Workgroups of a persistent launch (launch_util.h): as many as fit on the
// chip at once, never more than there can be items.
template <typename K>
static dim3 persistent_grid(K kernel, std::atomic<uint64_t>& cache, size_t lds, const moe_dims& d,
                            int items_per_entry) {
    return dim3(persistent_blocks(kernel, cache, 256, lds, work_capacity(d) * items_per_entry));
}

// Prefetch depth: the deepest ring (up to cap) that pads a wave's NGW groups
// by at most a quarter; padded steps cost a reload of a cached group.
static int ring_depth_waves(int NG, int parts, int cap) {
    const int NGW = (NG + parts - 1) / parts;
    for (int d = cap < NGW ? cap : NGW; d > 1; --d) {
        const int ngp = (NGW + d - 1) / d * d;
        if (4 * ngp <= 5 * NGW) return d;
    }
    return 1;
}

static int ring_depth(int NG, int cap) { return ring_depth_waves(NG, kWaves, cap); }

// Gate/up: at most 3 workgroups per CU.  The HBM streams fastest with a
// moderate number of loads in flight (a plain read peaks at one to two
// workgroups per CU with 8 loads each and slows down past that); measured on
// the 64-expert shape: 1 / 2 / 3 / 4 per CU = 97 / 77 / 72 / 75 us.
constexpr int kGateupMaxPerCu = 3;

template <int BITS, int D, int SJ>
static void gateup_launch(const moe_dims& d, size_t lds, hipStream_t s, const MfmaParams& p) {
    static std::atomic<uint64_t> occ{0};
    dim3 grid = persistent_grid(ffn_gateup_mfma_kernel<BITS, D, SJ>, occ, lds, d, p.items_per_entry);
    grid.x = std::min<unsigned>(grid.x, (unsigned)(kGateupMaxPerCu * device_cus()));
    hipLaunchKernelGGL((ffn_gateup_mfma_kernel<BITS, D, SJ>), grid, dim3(256), lds, s, p);
}

template <int BITS, int D, int SJ, int KS>
static void down_launch(const moe_dims& d, size_t lds, hipStream_t s, const MfmaParams& p) {
    static std::atomic<uint64_t> occ{0};
    const dim3 grid = persistent_grid(ffn_down_mfma_kernel<BITS, D, SJ, KS>, occ, lds, d, p.items_per_entry);
    hipLaunchKernelGGL((ffn_down_mfma_kernel<BITS, D, SJ, KS>), grid, dim3(256), lds, s, p);
}

template <int BITS, int D>
static void gateup_sj(int SJ, const moe_dims& d, size_t lds, hipStream_t s, const MfmaParams& p) {
    // SJ >= ceil(16 * NGW / 64) scale entries per lane per matrix
    if (SJ <= 1) gateup_launch<BITS, D, 1>(d, lds, s, p);
    else if (SJ <= 2) gateup_launch<BITS, D, 2>(d, lds, s, p);
    else if (SJ <= 3) gateup_launch<BITS, D, 3>(d, lds, s, p);
    else gateup_launch<BITS, D, 4>(d, lds, s, p);
}

template <int BITS>
static void gateup_dispatch(int D, int SJ, const moe_dims& d, size_t lds, hipStream_t s, const MfmaParams& p) {
    if (D == 4) gateup_sj<BITS, 4>(SJ, d, lds, s, p);
    else if (D == 3) gateup_sj<BITS, 3>(SJ, d, lds, s, p);
    else if (D == 2) gateup_sj<BITS, 2>(SJ, d, lds, s, p);
    else gateup_sj<BITS, 1>(SJ, d, lds, s, p);
}

template <int BITS, int D, int KS>
static void down_sj(int SJ, const moe_dims& d, size_t lds, hipStream_t s, const MfmaParams& p) {
    // SJ >= ceil(32 * NGW / 64) scale entries per lane per matrix
    if (SJ <= 1) down_launch<BITS, D, 1, KS>(d, lds, s, p);
    else if (SJ <= 2) down_launch<BITS, D, 2, KS>(d, lds, s, p);
    else if (SJ <= 4) down_launch<BITS, D, 4, KS>(d, lds, s, p);
    else if (SJ <= 8) down_launch<BITS, D, 8, KS>(d, lds, s, p);
    else down_launch<BITS, D, 16, KS>(d, lds, s, p);
}

template <int BITS>
static void down_dispatch(int D, int SJ, int KS, const moe_dims& d, size_t lds, hipStream_t s,
                          const MfmaParams& p) {
    if (KS == 4) {
        if (D >= 2) down_sj<BITS, 2, 4>(SJ, d, lds, s, p);
        else down_sj<BITS, 1, 4>(SJ, d, lds, s, p);
    } else if (KS == 2) {
        if (D >= 2) down_sj<BITS, 2, 2>(SJ, d, lds, s, p);
        else down_sj<BITS, 1, 2>(SJ, d, lds, s, p);
    } else {
        if (D >= 2) down_sj<BITS, 2, 1>(SJ, d, lds, s, p);
        else down_sj<BITS, 1, 1>(SJ, d, lds, s, p);
    }
}

// The x-tile gate/up kernel: waves per workgroup (one workgroup per CU), the
// LDS it needs, and its launch.
constexpr int kXtWaves = 12;

// Waves of the int8 x-tile kernel: 10 or 12, whichever gives the waves fewer
// groups of K each (10 on a tie: 40 groups split 4 each over 10 waves took
// 55.0-55.6 us at the 64-expert shape, 3 or 4 over 12 waves 56.9-57.8, 5 over 8
// 57.5-58.7).
static int xt8_waves(int NG) {
    return (NG + 9) / 10 <= (NG + 11) / 12 ? 10 : 12;
}
constexpr size_t kXtLdsLimit = 160 * 1024;

static size_t xt_lds_bytes(const moe_dims& d, int nw) {
    const int rows_cap = d.T < kWorkRows ? d.T : kWorkRows;
    const int NG = d.H / kGroup, NGW = (NG + nw - 1) / nw;
    const size_t xb = ((size_t)(rows_cap + 1) * (d.H + 8) * 2 + 15) & ~(size_t)15;
    const size_t xsb = (size_t)(((rows_cap + 1) * NG + 3) & ~3) * sizeof(float);
    return xb + xsb + ((size_t)nw * NGW * 64 + (size_t)2 * nw * 64 * 8) * sizeof(float);
}

template <int BITS, int D, int SJ, int NW>
static void xt_launch(size_t lds, hipStream_t s, const MfmaParams& p) {
    hipLaunchKernelGGL((ffn_gateup_xt_kernel<BITS, D, SJ, NW>), dim3((unsigned)device_cus()), dim3(64 * NW), lds, s, p);
}

// The int8-plane x-tile kernel: LDS for NBM blocks of 4 tokens, and launch.
static size_t xt8_lds_bytes(const moe_dims& d, int nw, int nbm) {
    const int rows_cap = d.T < kWorkRows ? d.T : kWorkRows;
    const int NG = d.H / kGroup, NGW = (NG + nw - 1) / nw;
    const size_t tiles = (((size_t)rows_cap * NG * kXt8Row + 128 + (size_t)rows_cap * NG * 8) + 15) & ~(size_t)15;
    return tiles + ((size_t)nw * NGW * 64 + (size_t)2 * nw * 64 * 2 * nbm) * sizeof(float);
}

template <int BITS, int D, int SJ, int NW, int NBM>
static void xt8_launch(size_t lds, hipStream_t s, const MfmaParams& p) {
    hipLaunchKernelGGL((ffn_gateup_xt8_kernel<BITS, D, SJ, NW, NBM>), dim3((unsigned)device_cus()), dim3(64 * NW), lds, s,
                       p);
}

template <int BITS, int SJ, int NW, int NBM>
static void xt8_depth(int D, size_t lds, hipStream_t s, const MfmaParams& p) {
    switch (D) {
        case 8: xt8_launch<BITS, 8, SJ, NW, NBM>(lds, s, p); break;
        case 6: xt8_launch<BITS, 6, SJ, NW, NBM>(lds, s, p); break;
        case 5: xt8_launch<BITS, 5, SJ, NW, NBM>(lds, s, p); break;
        case 4: xt8_launch<BITS, 4, SJ, NW, NBM>(lds, s, p); break;
        case 3: xt8_launch<BITS, 3, SJ, NW, NBM>(lds, s, p); break;
        case 2: xt8_launch<BITS, 2, SJ, NW, NBM>(lds, s, p); break;
        default: xt8_launch<BITS, 1, SJ, NW, NBM>(lds, s, p); break;
    }
}

// Tiles of 5 to 8 token rows (two blocks of 4); fewer rows fit the decode
// kernels' LDS tile at any H whose plane tile fits here.
template <int BITS, int NW>
static void xt8_dispatch(int D, int SJ, size_t lds, hipStream_t s, const MfmaParams& p) {
    if (SJ <= 1) xt8_depth<BITS, 1, NW, 2>(D, lds, s, p);
    else xt8_depth<BITS, 2, NW, 2>(D, lds, s, p);
}

template <int BITS, int SJ, int NW>
static void xt_depth(int D, size_t lds, hipStream_t s, const MfmaParams& p) {
    switch (D) {
        case 8: xt_launch<BITS, 8, SJ, NW>(lds, s, p); break;
        case 6: xt_launch<BITS, 6, SJ, NW>(lds, s, p); break;
        case 5: xt_launch<BITS, 5, SJ, NW>(lds, s, p); break;
        case 4: xt_launch<BITS, 4, SJ, NW>(lds, s, p); break;
        case 3: xt_launch<BITS, 3, SJ, NW>(lds, s, p); break;
        case 2: xt_launch<BITS, 2, SJ, NW>(lds, s, p); break;
        default: xt_launch<BITS, 1, SJ, NW>(lds, s, p); break;
    }
}

template <int BITS, int NW>
static void xt_dispatch(int D, int SJ, size_t lds, hipStream_t s, const MfmaParams& p) {
    if (SJ <= 1) xt_depth<BITS, 1, NW>(D, lds, s, p);
    else xt_depth<BITS, 2, NW>(D, lds, s, p);
}

// Ring depth of the x-tile kernel: the deepest of 8, 6, 5, 4, 3, 2 that pads a
// wave's groups by at most a quarter.  With a wave's whole share of K in its
// ring, each workgroup keeps the next item's codes in flight while it computes
// the current one, which is what keeps this HBM busy (about 2.5 us per round
// trip under load against about 2 us of arithmetic per item).
static int xt_depth_for(int NG, int nw) {
    const int NGW = (NG + nw - 1) / nw;
    for (int d : {8, 6, 5, 4, 3, 2}) {
        if (d > NGW) continue;
        const int ngp = (NGW + d - 1) / d * d;
        if (4 * ngp <= 5 * NGW) return d;
    }
    return 1;
}

int launch_gateup_mfma(const FfnArgs& a, hipStream_t s) {
    const moe_dims& d = a.d;
    if (d.T * d.k == 0) return MOE_OK;
    // shapes whose activation tile fits in LDS take the staged-tile kernel
    if (dec_gateup_fits(d)) return launch_gateup_dec(a, s);
    if (d.group_size != kGroup) return MOE_ERR_UNSUPPORTED;     // one scale per 128 codes here
    MfmaParams p = mfma_params(a);
    p.qa = a.w.q[0]; p.sa = a.w.scale[0]; p.ba = a.w.bias[0];
    p.qb = a.w.q[1]; p.sb = a.w.scale[1]; p.bb = a.w.bias[1];
    p.items_per_entry = d.I / 16;
    const SplitSpace sp = down_split_space(d, a.h);
    p.split_ctr = sp.ctr;
    p.n_split_ctr = sp.n_ctr;
    {
        const int NG = d.H / kGroup, NGW = (NG + kXtWaves - 1) / kXtWaves;
        const int SJ = (16 * NGW + 63) / 64;
        const int rows_cap = d.T < kWorkRows ? d.T : kWorkRows, nbm = (rows_cap + 3) / 4;
        const int nw8 = xt8_waves(NG), NGW8 = (NG + nw8 - 1) / nw8, SJ8 = (16 * NGW8 + 63) / 64;
        const size_t lds8 = xt8_lds_bytes(d, nw8, nbm);
        if (SJ8 <= 2 && nbm == 2 && lds8 <= kXtLdsLimit) {
            const int D = xt_depth_for(NG, nw8);
            if (nw8 == 10) {
                if (a.bits == 4) xt8_dispatch<4, 10>(D, SJ8, lds8, s, p);
                else xt8_dispatch<2, 10>(D, SJ8, lds8, s, p);
            } else {
                if (a.bits == 4) xt8_dispatch<4, 12>(D, SJ8, lds8, s, p);
                else xt8_dispatch<2, 12>(D, SJ8, lds8, s, p);
            }
            return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
        }
        const size_t lds = xt_lds_bytes(d, kXtWaves);
        if (SJ <= 2 && lds <= kXtLdsLimit) {
            const int D = xt_depth_for(NG, kXtWaves);
            if (a.bits == 4) xt_dispatch<4, kXtWaves>(D, SJ, lds, s, p);
            else xt_dispatch<2, kXtWaves>(D, SJ, lds, s, p);
            return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
        }
    }
    const int NG = d.H / kGroup, NGW = (NG + kWaves - 1) / kWaves;
    const int SJ = (16 * NGW + 63) / 64;
    if (SJ > 4) return MOE_ERR_UNSUPPORTED;
    const size_t lds = mfma_lds_bytes(NG);
    const int D = ring_depth(NG, 2);           // 2 deep: 72 us against 81 us at 4 (64-expert shape)
    if (a.bits == 4) gateup_dispatch<4>(D, SJ, d, lds, s, p);
    else gateup_dispatch<2>(D, SJ, d, lds, s, p);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// K parts of the down kernel: enough that each wave streams at least 4 groups
// when K allows, the rest of the waves spread over output rows.
static int down_k_split(int NG) { return NG >= 16 ? 4 : (NG >= 8 ? 2 : 1); }

int launch_down_mfma(const FfnArgs& a, hipStream_t s) {
    const moe_dims& d = a.d;
    if (d.T * d.k == 0) return MOE_OK;
    if (dec_down_fits(d)) return launch_down_dec(a, s);
    if (d.group_size != kGroup) return MOE_ERR_UNSUPPORTED;     // one scale per 128 codes here
    {
        const int st = launch_down_stream(a, s);        // h through LDS in chunks of K
        if (st != MOE_ERR_UNSUPPORTED) return st;
    }
    MfmaParams p = mfma_params(a);
    p.qa = a.w.q[2]; p.sa = a.w.scale[2]; p.ba = a.w.bias[2];
    const int NG = d.I / kGroup, KS = down_k_split(NG), NGW = (NG + KS - 1) / KS;
    p.items_per_entry = d.H / (32 * (kWaves / KS));
    const int SJ = (32 * NGW + 63) / 64;
    if (SJ > 16) return MOE_ERR_UNSUPPORTED;
    const size_t lds = ((size_t)kWaves * 2 * NGW * 64 + (size_t)kWaves * 64 * 8) * sizeof(float);
    const int D = ring_depth_waves(NG, KS, 2);
    if (a.bits == 4) down_dispatch<4>(D, SJ, KS, d, lds, s, p);
    else down_dispatch<2>(D, SJ, KS, d, lds, s, p);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
