// Grouped GEMM on the matrix cores for experts that serve many tokens (prefill
// and large batches): the same maths as the decode kernels in ffn_mfma.hip,
// tiled for reuse of each weight tile across 64 tokens.
//
// Why a separate path: the decode kernels give each 16-token work tile its own
// pass over the expert's weights and put K across the 4 waves of a workgroup,
// which is right when a weight byte meets a handful of tokens.  With hundreds
// of tokens per expert ("Strata" page, sec. 2.3: a batch's tokens share an
// expert) the contraction is dense and matrix-core bound, so here
//   * an item is 64 tokens (4 consecutive work-list tiles of one expert, one
//     per wave) times 128 rows of gate and 128 of up (or 128 down rows);
//   * the activation tile of a group of 128 along K (64 tokens) is staged once
//     in LDS and shared by the 4 waves; each wave streams its own 32 gate and
//     32 up rows (or 32 down rows) of codes straight into registers;
//   * activations are the A operand (rows = tokens) and codes the B operand
//     (columns = weight rows), so a lane's accumulators belong to one weight
//     row and the per-group fold (s / L) C + (b - (128 / L) s) X needs one
//     scale pair per tile; X = sum of the activations over the group is added
//     up while the tile is staged.
// The exact code operands and the fold are those of mfma_ops.h.  h leaves the
// gate/up kernel in the same three bf16 planes (plus 16-row partial sums) as
// the decode path, and the down kernel here reads all three (h to about 24
// significant bits: with two, h's 2^-18 relative error summed over I moved
// outputs far below the rms by a few bf16 ulps where the weights are large,
// as zero-point weights are).
#include <atomic>

#include "launch_util.h"
#include "mfma_ops.h"

namespace moe {

namespace {

constexpr int kTilesPerHead = 4;                     // work-list tiles per item = one per wave
constexpr int kTokRows = kTilesPerHead * kWorkRows;  // token rows per item (64)
constexpr int kGuRows = 128;                         // gate rows (and up rows) per gate/up item
constexpr int kDnRows = 128;                         // down rows per down item
constexpr int kCodeRowBytes = 64;                    // one 4-bit row of a 128-wide group (contiguous rows)
constexpr int kActRowBytes = kGroup * 2;             // one bf16 row of a 128-wide group

struct GemmParams {
    const uint16_t* x;
    const int32_t* work;
    const int32_t* n_work;
    const int32_t* heads;             // work-list index of each item's first tile
    const int32_t* n_heads;
    const uint8_t* qa; const uint16_t* sa; const uint16_t* ba;   // gate, or down
    const uint8_t* qb; const uint16_t* sb; const uint16_t* bb;   // up
    uint16_t* hp;                     // bf16 planes [3][P][I]
    float* hpart;                     // [P][I/16]
    uint16_t* y;                      // [P][H]
    int T, H, I, E, P;
    int blocks;                       // output row blocks per head
};

// Byte offset of 16-byte chunk c (0..15) of LDS activation row r: chunks are
// XOR-swizzled by the row's low 4 bits, so the 16 rows that a quarter-wave
// reads at once (same chunk, rows 16 tk + 0..15) hit 16 different bank groups.
__device__ __forceinline__ int act_lds_offset(int r, int c) {
    return r * kActRowBytes + 16 * (c ^ (r & 15));
}

// Sum N values per lane over the 16 lanes of each quarter-wave (lane bits 0-3)
// by a butterfly transpose: afterwards v[0], v[1] of lane m (= lane % 16) hold
// the totals of value indices 2m and 2m + 1 (N = 32).
template <int N, int STAGE>
__device__ __forceinline__ void row16_stage(float (&v)[N], int lane) {
    constexpr int n = N >> STAGE, off = 8 >> STAGE, h = n / 2;
    const bool upper = (lane & off) != 0;
#pragma unroll
    for (int i = 0; i < h; ++i) {
        const float keep = upper ? v[i + h] : v[i];
        const float send = upper ? v[i] : v[i + h];
        v[i] = keep + __shfl_xor(send, off, kWave);
    }
}

// Uniform description of one item, shared by both kernels: the expert, the
// output row block, and this wave's work-list tile (its first sorted row and
// row count; n = 0 when the item has fewer than 4 tiles and this wave's slot
// is empty) plus the token of the row this thread stages.
struct ItemMeta {
    int e, blk, row0, n, tok;
};

__device__ __forceinline__ void item_meta(const GemmParams& p, int idx, int wu, int lane, ItemMeta& it) {
    const int n_work = ld_scalar(p.n_work, 0);
    const int head = ld_scalar(p.heads, (size_t)(idx / p.blocks));
    it.blk = idx % p.blocks;
    const int32_t* h0 = p.work + (size_t)head * kWorkInts;
    const int e0 = ld_scalar(h0, 0), t0 = ld_scalar(h0, 3);
    it.e = (e0 >= 0 && e0 < p.E) ? e0 : 0;
    // this wave's tile: head + wu, if it is the same expert's next tile
    const int wi = head + wu;
    const int32_t* ent = p.work + (size_t)(wi < n_work ? wi : head) * kWorkInts;
    const bool mine = wi < n_work && ld_scalar(ent, 0) == e0 && ld_scalar(ent, 3) == t0 + wu;
    const int row0 = ld_scalar(ent, 1), n = ld_scalar(ent, 2);
    const bool rows_ok = row0 >= 0 && n >= 1 && n <= kWorkRows && row0 + n <= p.P;
    it.row0 = (mine && rows_ok) ? row0 : 0;
    it.n = (mine && rows_ok) ? n : 0;
    // token of slot lane / 4 of the tile (slots past the tile's rows repeat row 0)
    int tok = ld_scalar(ent, 4);
#pragma unroll
    for (int jj = 1; jj < kWorkRows; ++jj) {
        const int v = ld_scalar(ent, 4 + jj);
        tok = ((lane >> 2) == jj) ? v : tok;
    }
    it.tok = (tok >= 0 && tok < p.T) ? tok : 0;
}

}  // namespace

// ----------------------------------------------------------------- heads
// Work-list tiles whose index within their expert is a multiple of 4 start an
// item; their work-list indices, in order, and the count.  One workgroup.
__global__ __launch_bounds__(1024) void gemm_heads_kernel(const int32_t* __restrict__ work,
                                                         const int32_t* __restrict__ n_work, int cap,
                                                         int32_t* __restrict__ heads,
                                                         int32_t* __restrict__ n_heads) {
    __shared__ int wsum[16];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, nw_waves = blockDim.x >> 6;
    const int nw = min(*n_work, cap);
    int count = 0;
    for (int i0 = 0; i0 < nw; i0 += blockDim.x) {
        const int i = i0 + tid;
        const int f = (i < nw && work[(size_t)i * kWorkInts + 3] % kTilesPerHead == 0) ? 1 : 0;
        const uint64_t bal = __ballot(f);
        const int before = __popcll(bal & (lane == 0 ? 0ull : (~0ull >> (64 - lane))));
        if (lane == 0) wsum[wid] = __popcll(bal);
        __syncthreads();
        int base = 0, tot = 0;
        for (int w = 0; w < nw_waves; ++w) {
            base += (w < wid) ? wsum[w] : 0;
            tot += wsum[w];
        }
        if (f) heads[count + base + before] = i;
        count += tot;
        __syncthreads();
    }
    if (tid == 0) *n_heads = count;
}

// -------------------------------------------------------------- gate / up
// Item = (head, block): 64 token rows (tiles head .. head+3 of one expert; wave
// w stages the rows of tile head + w) times intermediate rows block*128 .. +128
// of gate and of up.  Wave w computes all 64 tokens against its own 32 gate
// and 32 up rows (4 weight tiles x 4 token tiles = 16 accumulator tiles), so
// each unpacked code operand feeds 4 MFMAs.  Per group of 128 along H:
//   LDS: the activation tile, 64 rows x 128 bf16 in code pair order (16 KB),
//        and each row's sum X over the group; double-buffered.
//   Rings of depth D (steps = groups, continuing into the next item): each
//   thread's share of the activation tile (64 bytes), staged into LDS one
//   step ahead; each lane's 4 weight pieces (16 bytes each) and their scales.
// D divides the group count and is smaller than it (the launcher checks).
template <int D>
__global__ __launch_bounds__(256) void ffn_gateup_gemm_kernel(GemmParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int kTileBytes = kTokRows * kActRowBytes;       // activation tile of one group
    constexpr int kBufBytes = kTileBytes + kTokRows * 4;      // + sums
    int* rows_lds = reinterpret_cast<int*>(smem + 2 * kBufBytes);   // [4][2] tile row0, n
    const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, q = lane >> 4;
    const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, known uniform
    const int n_items = ld_scalar(p.n_heads, 0) * p.blocks;
    if ((int)blockIdx.x >= n_items) return;
    const int n_my = (n_items - 1 - (int)blockIdx.x) / (int)gridDim.x + 1;
    const int H = p.H, I = p.I, NG = H / kGroup;
    const int tr = tid >> 2, tq = tid & 3;                     // staged token row, quarter

    // this lane's 4 weight rows relative to the item's first gate/up row:
    // tiles 0, 1 gate, 2, 3 up (pair order within 16)
    int lrow[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) lrow[hf] = 32 * wu + 16 * hf + pair_order_row<4>(m);
    struct Item {
        ItemMeta mt;
        int rbase;                           // e * I + first row of the block
        const uint16_t* x;                   // staged row's activations, quarter tq
    };
    auto fetch = [&](int j, Item& it) {
        item_meta(p, (int)blockIdx.x + j * (int)gridDim.x, wu, lane, it.mt);
        it.rbase = it.mt.e * I + it.mt.blk * kGuRows;
        it.x = p.x + (size_t)it.mt.tok * H + 32 * tq;
    };

    uint32_t xr[D][16];                       // staged activations: 32 bf16
    uint32_t cr[D][4][4];                     // 4 weight pieces of 16 bytes
    uint32_t ssr[D][4], sbr[D][4];            // their scales and biases (fp16 bits)
    auto issue_x = [&](int slot, const uint16_t* xp, int g) {
        const uint4* src = reinterpret_cast<const uint4*>(xp + (size_t)g * kGroup);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const uint4 X = src[v];
            xr[slot][4 * v] = X.x; xr[slot][4 * v + 1] = X.y; xr[slot][4 * v + 2] = X.z; xr[slot][4 * v + 3] = X.w;
        }
    };
    auto issue_c = [&](int slot, const Item& it, int g) {
#pragma unroll
        for (int wt = 0; wt < 4; ++wt) {
            const size_t row = (size_t)(it.rbase + lrow[wt & 1]);
            // codes are group-major: row r of expert e, group g at ((e NG + g) I + r) 64
            const size_t crow = row + (size_t)it.mt.e * (NG - 1) * I + (size_t)g * I;
            const uint8_t* cp = (wt < 2 ? p.qa : p.qb) + crow * kCodeRowBytes + 16 * q;
            const uint4 C = *reinterpret_cast<const uint4*>(cp);
            cr[slot][wt][0] = C.x; cr[slot][wt][1] = C.y; cr[slot][wt][2] = C.z; cr[slot][wt][3] = C.w;
            ssr[slot][wt] = (wt < 2 ? p.sa : p.sb)[row * NG + g];
            sbr[slot][wt] = (wt < 2 ? p.ba : p.bb)[row * NG + g];
        }
    };
    // activation piece -> LDS in code pair order, plus the row's sum
    auto stage = [&](int slot, int buf) {
        uint8_t* base = smem + buf * kBufBytes;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            uint32_t o[4];
            act_operand<4>(xr[slot], st, o);
            *reinterpret_cast<uint4*>(base + act_lds_offset(tr, 4 * tq + st)) = make_uint4(o[0], o[1], o[2], o[3]);
        }
        float sum = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) sum += bf16_bits_to_f32(xr[slot][v] & 0xFFFFu) + bf16_bits_to_f32(xr[slot][v] >> 16);
        sum += __shfl_xor(sum, 1, kWave);
        sum += __shfl_xor(sum, 2, kWave);
        if (tq == 0) reinterpret_cast<float*>(base + kTileBytes)[tr] = sum;
    };

    Item cur, nxt;
    fetch(0, cur);
#pragma unroll
    for (int d = 0; d < D; ++d) { issue_x(d, cur.x, d); issue_c(d, cur, d); }
    stage(0, 0);
    issue_x(0, cur.x, D);
    if (lane == 0) { rows_lds[2 * wu] = cur.mt.row0; rows_lds[2 * wu + 1] = cur.mt.n; }
    __syncthreads();

    int t = 0;
    for (int j = 0; j < n_my; ++j) {
        const bool has_next = j + 1 < n_my;
        if (has_next) fetch(j + 1, nxt);
        else nxt = cur;
        floatx4_t acc[4][4];
#pragma unroll
        for (int wt = 0; wt < 4; ++wt)
#pragma unroll
            for (int tk = 0; tk < 4; ++tk) acc[wt][tk] = floatx4_t{0.f, 0.f, 0.f, 0.f};

        int g0 = 0;
        do {
            const bool last = g0 + D >= NG;
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int g = g0 + d;
                const uint8_t* base = smem + (t & 1) * kBufBytes;
                floatx4_t C[4][4];
#pragma unroll
                for (int wt = 0; wt < 4; ++wt)
#pragma unroll
                    for (int tk = 0; tk < 4; ++tk) C[wt][tk] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    uint32_t A[4][4];
#pragma unroll
                    for (int tk = 0; tk < 4; ++tk) {
                        const uint4 a4 = *reinterpret_cast<const uint4*>(base + act_lds_offset(16 * tk + m, 4 * q + st));
                        A[tk][0] = a4.x; A[tk][1] = a4.y; A[tk][2] = a4.z; A[tk][3] = a4.w;
                    }
#pragma unroll
                    for (int wt = 0; wt < 4; ++wt) {
                        uint32_t B[4];
                        code_operand<4>(cr[d][wt], st, B);
#pragma unroll
                        for (int tk = 0; tk < 4; ++tk) C[wt][tk] = mfma16(A[tk], B, C[wt][tk]);
                    }
                }
                // fold: acc += (s/8) C + (b - 16 s) X, X of the 4 token rows of each tile
                const float* Xs = reinterpret_cast<const float*>(base + kTileBytes);
                float4 X[4];
#pragma unroll
                for (int tk = 0; tk < 4; ++tk) X[tk] = *reinterpret_cast<const float4*>(Xs + 16 * tk + 4 * q);
#pragma unroll
                for (int wt = 0; wt < 4; ++wt) {
                    const float sv = f16_bits_to_f32(ssr[d][wt]), bv = f16_bits_to_f32(sbr[d][wt]);
                    const float s1 = sv * kInvLever<4>, b1 = fmaf(-kOffset<4>, sv, bv);
#pragma unroll
                    for (int tk = 0; tk < 4; ++tk) {
                        acc[wt][tk][0] = fmaf(s1, C[wt][tk][0], fmaf(b1, X[tk].x, acc[wt][tk][0]));
                        acc[wt][tk][1] = fmaf(s1, C[wt][tk][1], fmaf(b1, X[tk].y, acc[wt][tk][1]));
                        acc[wt][tk][2] = fmaf(s1, C[wt][tk][2], fmaf(b1, X[tk].z, acc[wt][tk][2]));
                        acc[wt][tk][3] = fmaf(s1, C[wt][tk][3], fmaf(b1, X[tk].w, acc[wt][tk][3]));
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                // refill this code slot with the step D ahead (into the next item
                // during the item's last D steps)
                const bool go_next = last && has_next;
                issue_c(d, go_next ? nxt : cur, !last ? g + D : (has_next ? d : NG - 1));
                // stage the next step's activations into the other buffer, then
                // refill that slot with the step D after it
                {
                    const int dn = (d + 1) % D;
                    stage(dn, (t + 1) & 1);
                    const int gf = g + 1 + D;
                    const bool f_next = gf >= NG && has_next;
                    const int gg = gf < NG ? gf : (has_next ? gf - NG : NG - 1);
                    issue_x(dn, f_next ? nxt.x : cur.x, gg);
                }
                __syncthreads();
                ++t;
            }
            g0 += D;
        } while (g0 < NG);

        // ---- epilogue: h = silu(gate) * up, three planes, 16-row partial sums
        // value index v = 16 * hf + 4 * tk + i: hf 0 = rows 0..15 of the wave's
        // 32, hf 1 = rows 16..31; token row 16 tk + 4 q + i
        float hv[32];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int tk = 0; tk < 4; ++tk)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float gt = acc[hf][tk][i], upv = acc[2 + hf][tk][i];
                    hv[16 * hf + 4 * tk + i] = gt / (1.f + expf(-gt)) * upv;
                }
        const size_t plane = (size_t)p.P * I;
        const int i0 = cur.mt.blk * kGuRows + 32 * wu;
        // token tile tk holds the rows of wave tk's work-list tile
#pragma unroll
        for (int tk = 0; tk < 4; ++tk) {
            const int r0 = rows_lds[2 * tk], rn = rows_lds[2 * tk + 1];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 4 * q + i;
                    if (row < rn) {
                        uint32_t hi, mid, lo;
                        split3_bf16(hv[16 * hf + 4 * tk + i], hi, mid, lo);
                        uint16_t* dst = p.hp + (size_t)(r0 + row) * I + i0 + 16 * hf + m;
                        dst[0] = (uint16_t)hi;
                        dst[plane] = (uint16_t)mid;
                        dst[2 * plane] = (uint16_t)lo;
                    }
                }
        }
        // partial sums over each 16-row tile of h: lane m ends with values 2m, 2m+1
        row16_stage<32, 0>(hv, lane);
        row16_stage<32, 1>(hv, lane);
        row16_stage<32, 2>(hv, lane);
        row16_stage<32, 3>(hv, lane);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int vi = 2 * m + u, hf = vi >> 4, tk = (vi >> 2) & 3, row = 4 * q + (vi & 3);
            const int r0 = rows_lds[2 * tk], rn = rows_lds[2 * tk + 1];
            if (row < rn) p.hpart[(size_t)(r0 + row) * (I / 16) + (i0 + 16 * hf) / 16] = hv[u];
        }
        __syncthreads();                      // rows_lds is rewritten for the next item
        if (lane == 0) { rows_lds[2 * wu] = nxt.mt.row0; rows_lds[2 * wu + 1] = nxt.mt.n; }
        cur = nxt;
    }
}

// ------------------------------------------------------------------- down
// Item = (head, block): the same 64 token rows times output rows
// block*128 .. +128.  Wave w computes all 64 tokens against its own 32 down
// rows (2 weight tiles x 4 token tiles x 3 planes of h = 24 MFMAs per step).
// Per group of 128 along I:
//   LDS: the three planes of h for the 64 rows (3 x 16 KB; h is already
//        stored in code pair order) and each row's sum of h over the group,
//        taken from the 16-row partial sums; double-buffered.
//   Rings of depth D: each thread's share of the h tile (64 bytes per plane)
//   and two partial sums; each lane's 2 weight pieces and their scales.
constexpr int kGemmDnPlanes = 3;    // bf16 planes of h the down kernel multiplies

template <int D>
__global__ __launch_bounds__(256) void ffn_down_gemm_kernel(GemmParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int kTileBytes = kTokRows * kActRowBytes;       // one plane of one group
    constexpr int kBufBytes = kGemmDnPlanes * kTileBytes + kTokRows * 4;  // hi, mid, lo, sums
    int* rows_lds = reinterpret_cast<int*>(smem + 2 * kBufBytes);
    const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, q = lane >> 4;
    const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n_items = ld_scalar(p.n_heads, 0) * p.blocks;
    if ((int)blockIdx.x >= n_items) return;
    const int n_my = (n_items - 1 - (int)blockIdx.x) / (int)gridDim.x + 1;
    const int H = p.H, I = p.I, NG = I / kGroup;
    const size_t plane = (size_t)p.P * I;
    const int tr = tid >> 2, tq = tid & 3;

    struct Item {
        ItemMeta mt;
        int rbase;                           // e * H + first row of the block + this lane's row
        const uint16_t* h;                   // staged row's h (hi plane), quarter tq
        const float* part;                   // staged row's partial sums, pair tq
    };
    auto fetch = [&](int j, Item& it) {
        item_meta(p, (int)blockIdx.x + j * (int)gridDim.x, wu, lane, it.mt);
        // rows of an empty slot or past the tile's end stage a valid row (the
        // tile's first, or row 0): computed, never stored
        const int slot = lane >> 2;
        const int r = it.mt.n > 0 ? it.mt.row0 + (slot < it.mt.n ? slot : 0) : 0;
        it.h = p.hp + (size_t)r * I + 32 * tq;
        it.part = p.hpart + (size_t)r * (I / 16) + 2 * tq;
        it.rbase = it.mt.e * H + it.mt.blk * kDnRows + 32 * wu + m;
    };

    uint32_t hr[D][kGemmDnPlanes][16];        // staged h: 32 values of each plane
    float2 pr[D];                             // 2 partial sums of the staged row
    uint32_t cr[D][2][4];
    uint32_t ssr[D][2], sbr[D][2];
    auto issue_h = [&](int slot, const Item& it, int g) {
#pragma unroll
        for (int pl = 0; pl < kGemmDnPlanes; ++pl) {
            const uint4* src = reinterpret_cast<const uint4*>(it.h + pl * plane + (size_t)g * kGroup);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const uint4 X = src[v];
                hr[slot][pl][4 * v] = X.x; hr[slot][pl][4 * v + 1] = X.y;
                hr[slot][pl][4 * v + 2] = X.z; hr[slot][pl][4 * v + 3] = X.w;
            }
        }
        pr[slot] = *reinterpret_cast<const float2*>(it.part + 8 * g);
    };
    auto issue_c = [&](int slot, const Item& it, int g) {
#pragma unroll
        for (int wt = 0; wt < 2; ++wt) {
            const size_t row = (size_t)(it.rbase + 16 * wt);
            // codes are group-major: row r of expert e, group g at ((e NG + g) H + r) 64
            const size_t crow = row + (size_t)it.mt.e * (NG - 1) * H + (size_t)g * H;
            const uint4 C = *reinterpret_cast<const uint4*>(p.qa + crow * kCodeRowBytes + 16 * q);
            cr[slot][wt][0] = C.x; cr[slot][wt][1] = C.y; cr[slot][wt][2] = C.z; cr[slot][wt][3] = C.w;
            ssr[slot][wt] = p.sa[row * NG + g];
            sbr[slot][wt] = p.ba[row * NG + g];
        }
    };
    auto stage = [&](int slot, int buf) {
        uint8_t* base = smem + buf * kBufBytes;
#pragma unroll
        for (int pl = 0; pl < kGemmDnPlanes; ++pl)
#pragma unroll
            for (int st = 0; st < 4; ++st)
                *reinterpret_cast<uint4*>(base + pl * kTileBytes + act_lds_offset(tr, 4 * tq + st)) =
                    make_uint4(hr[slot][pl][4 * st], hr[slot][pl][4 * st + 1], hr[slot][pl][4 * st + 2],
                               hr[slot][pl][4 * st + 3]);
        float sum = pr[slot].x + pr[slot].y;
        sum += __shfl_xor(sum, 1, kWave);
        sum += __shfl_xor(sum, 2, kWave);
        if (tq == 0) reinterpret_cast<float*>(base + kGemmDnPlanes * kTileBytes)[tr] = sum;
    };

    Item cur, nxt;
    fetch(0, cur);
#pragma unroll
    for (int d = 0; d < D; ++d) { issue_h(d, cur, d); issue_c(d, cur, d); }
    stage(0, 0);
    issue_h(0, cur, D);
    if (lane == 0) { rows_lds[2 * wu] = cur.mt.row0; rows_lds[2 * wu + 1] = cur.mt.n; }
    __syncthreads();

    int t = 0;
    for (int j = 0; j < n_my; ++j) {
        const bool has_next = j + 1 < n_my;
        if (has_next) fetch(j + 1, nxt);
        else nxt = cur;
        floatx4_t acc[2][4];
#pragma unroll
        for (int wt = 0; wt < 2; ++wt)
#pragma unroll
            for (int tk = 0; tk < 4; ++tk) acc[wt][tk] = floatx4_t{0.f, 0.f, 0.f, 0.f};

        int g0 = 0;
        do {
            const bool last = g0 + D >= NG;
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int g = g0 + d;
                const uint8_t* base = smem + (t & 1) * kBufBytes;
                floatx4_t C[2][4];
#pragma unroll
                for (int wt = 0; wt < 2; ++wt)
#pragma unroll
                    for (int tk = 0; tk < 4; ++tk) C[wt][tk] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    uint32_t A[kGemmDnPlanes][4][4];
#pragma unroll
                    for (int pl = 0; pl < kGemmDnPlanes; ++pl)
#pragma unroll
                        for (int tk = 0; tk < 4; ++tk) {
                            const uint4 a4 = *reinterpret_cast<const uint4*>(
                                base + pl * kTileBytes + act_lds_offset(16 * tk + m, 4 * q + st));
                            A[pl][tk][0] = a4.x; A[pl][tk][1] = a4.y; A[pl][tk][2] = a4.z; A[pl][tk][3] = a4.w;
                        }
#pragma unroll
                    for (int wt = 0; wt < 2; ++wt) {
                        uint32_t B[4];
                        code_operand<4>(cr[d][wt], st, B);
#pragma unroll
                        for (int tk = 0; tk < 4; ++tk) {
                            C[wt][tk] = mfma16(A[0][tk], B, C[wt][tk]);
                            C[wt][tk] = mfma16(A[1][tk], B, C[wt][tk]);
                            C[wt][tk] = mfma16(A[2][tk], B, C[wt][tk]);
                        }
                    }
                }
                const float* Xs = reinterpret_cast<const float*>(base + kGemmDnPlanes * kTileBytes);
                float4 X[4];
#pragma unroll
                for (int tk = 0; tk < 4; ++tk) X[tk] = *reinterpret_cast<const float4*>(Xs + 16 * tk + 4 * q);
#pragma unroll
                for (int wt = 0; wt < 2; ++wt) {
                    const float sv = f16_bits_to_f32(ssr[d][wt]), bv = f16_bits_to_f32(sbr[d][wt]);
                    const float s1 = sv * kInvLever<4>, b1 = fmaf(-kOffset<4>, sv, bv);
#pragma unroll
                    for (int tk = 0; tk < 4; ++tk) {
                        acc[wt][tk][0] = fmaf(s1, C[wt][tk][0], fmaf(b1, X[tk].x, acc[wt][tk][0]));
                        acc[wt][tk][1] = fmaf(s1, C[wt][tk][1], fmaf(b1, X[tk].y, acc[wt][tk][1]));
                        acc[wt][tk][2] = fmaf(s1, C[wt][tk][2], fmaf(b1, X[tk].z, acc[wt][tk][2]));
                        acc[wt][tk][3] = fmaf(s1, C[wt][tk][3], fmaf(b1, X[tk].w, acc[wt][tk][3]));
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                const bool go_next = last && has_next;
                issue_c(d, go_next ? nxt : cur, !last ? g + D : (has_next ? d : NG - 1));
                {
                    const int dn = (d + 1) % D;
                    stage(dn, (t + 1) & 1);
                    const int gf = g + 1 + D;
                    const bool f_next = gf >= NG && has_next;
                    const int gg = gf < NG ? gf : (has_next ? gf - NG : NG - 1);
                    issue_h(dn, f_next ? nxt : cur, gg);
                }
                __syncthreads();
                ++t;
            }
            g0 += D;
        } while (g0 < NG);

        // ---- epilogue: Y rows in bf16 (token 16 tk + 4 q + i, column 16 wt + m)
        const int n0 = cur.mt.blk * kDnRows + 32 * wu;
#pragma unroll
        for (int tk = 0; tk < 4; ++tk) {
            const int r0 = rows_lds[2 * tk], rn = rows_lds[2 * tk + 1];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * q + i;
                if (row < rn) {
                    uint16_t* yrow = p.y + (size_t)(r0 + row) * H + n0 + m;
                    yrow[0] = (uint16_t)f32_to_bf16_bits(acc[0][tk][i]);
                    yrow[16] = (uint16_t)f32_to_bf16_bits(acc[1][tk][i]);
                }
            }
        }
        __syncthreads();
        if (lane == 0) { rows_lds[2 * wu] = nxt.mt.row0; rows_lds[2 * wu + 1] = nxt.mt.n; }
        cur = nxt;
    }
}

// ---------------------------------------------------------------- launch

constexpr size_t kGuLds = 2 * ((size_t)kTokRows * kActRowBytes + kTokRows * 4) + 8 * sizeof(int);
constexpr size_t kDnLds = 2 * ((size_t)kGemmDnPlanes * kTokRows * kActRowBytes + kTokRows * 4) + 8 * sizeof(int);

// LDS one workgroup may take on the current device (gfx950: 160 KB).
static size_t max_lds_per_block() {
    static size_t bytes = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || n <= 0)
            n = 0;
        return (size_t)n;
    }();
    return bytes;
}

// The rings read up to D + 1 groups ahead and at most into the next item,
// which needs at least two groups along each K.
bool gemm_supported(const moe_dims& d, int bits) {
    return bits == 4 && d.group_size == kGroup && d.I % kGuRows == 0 && d.H % kDnRows == 0 && d.H >= 2 * kGroup &&
           d.I >= 2 * kGroup;
}

// Ring depth: D must divide the group count and stay below it (the activation
// ring reads D + 1 steps ahead, at most into the next item).
static int gemm_depth(int NG) { return (NG % 2 == 0 && NG > 2) ? 2 : 1; }

static long max_heads(const moe_dims& d) {
    return work_capacity(d) / kTilesPerHead + (d.E < (long)d.T * d.k ? d.E : (long)d.T * d.k);
}

// Heads list and count live after the h planes and partial sums.
size_t gemm_workspace_bytes(const moe_dims& d) {
    return mfma_workspace_bytes(d) + (((size_t)max_heads(d) + 1 + 64) * sizeof(int32_t) + 255) / 256 * 256;
}

template <typename K>
static dim3 gemm_grid(K kernel, std::atomic<uint64_t>& cache, size_t lds, long max_items) {
    return dim3(persistent_blocks(kernel, cache, 256, lds, max_items));
}

static GemmParams gemm_params(const FfnArgs& a) {
    const moe_dims& d = a.d;
    GemmParams p{};
    p.x = a.x; p.work = a.work; p.n_work = a.n_work; p.y = a.y;
    p.T = d.T; p.H = d.H; p.I = d.I; p.E = d.E; p.P = d.T * d.k;
    char* ws = reinterpret_cast<char*>(a.h);
    const size_t P = (size_t)p.P;
    p.hp = reinterpret_cast<uint16_t*>(ws);
    p.hpart = reinterpret_cast<float*>(ws + ((3 * P * d.I * sizeof(uint16_t) + 255) & ~(size_t)255));
    int32_t* hl = reinterpret_cast<int32_t*>(ws + mfma_workspace_bytes(d));
    p.n_heads = hl;
    p.heads = hl + 64;
    return p;
}

int launch_gateup_gemm(const FfnArgs& a, hipStream_t s) {
    const moe_dims& d = a.d;
    if (d.T * d.k == 0) return MOE_OK;
    // the down kernel's double-buffered h tile takes more than 64 KB of LDS
    if (!gemm_supported(d, a.bits) || max_lds_per_block() < kDnLds) return MOE_ERR_UNSUPPORTED;
    GemmParams p = gemm_params(a);
    p.qa = a.w.q[0]; p.sa = a.w.scale[0]; p.ba = a.w.bias[0];
    p.qb = a.w.q[1]; p.sb = a.w.scale[1]; p.bb = a.w.bias[1];
    p.blocks = d.I / kGuRows;
    hipLaunchKernelGGL(gemm_heads_kernel, dim3(1), dim3(1024), 0, s, a.work, a.n_work, (int)work_capacity(d),
                       const_cast<int32_t*>(p.heads), const_cast<int32_t*>(p.n_heads));
    const long max_items = max_heads(d) * p.blocks;
    if (gemm_depth(d.H / kGroup) == 2) {
        static std::atomic<uint64_t> occ{0};
        const dim3 grid = gemm_grid(ffn_gateup_gemm_kernel<2>, occ, kGuLds, max_items);
        hipLaunchKernelGGL(ffn_gateup_gemm_kernel<2>, grid, dim3(256), kGuLds, s, p);
    } else {
        static std::atomic<uint64_t> occ{0};
        const dim3 grid = gemm_grid(ffn_gateup_gemm_kernel<1>, occ, kGuLds, max_items);
        hipLaunchKernelGGL(ffn_gateup_gemm_kernel<1>, grid, dim3(256), kGuLds, s, p);
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// The heads list is the one the gate/up launch of the same call (or of the
// split gate/up call that filled this workspace) wrote.
int launch_down_gemm(const FfnArgs& a, hipStream_t s) {
    const moe_dims& d = a.d;
    if (d.T * d.k == 0) return MOE_OK;
    if (!gemm_supported(d, a.bits) || max_lds_per_block() < kDnLds) return MOE_ERR_UNSUPPORTED;
    GemmParams p = gemm_params(a);
    p.qa = a.w.q[2]; p.sa = a.w.scale[2]; p.ba = a.w.bias[2];
    p.blocks = d.H / kDnRows;
    const long max_items = max_heads(d) * p.blocks;
    if (gemm_depth(d.I / kGroup) == 2) {
        static std::atomic<uint64_t> occ{0};
        const dim3 grid = gemm_grid(ffn_down_gemm_kernel<2>, occ, kDnLds, max_items);
        hipLaunchKernelGGL(ffn_down_gemm_kernel<2>, grid, dim3(256), kDnLds, s, p);
    } else {
        static std::atomic<uint64_t> occ{0};
        const dim3 grid = gemm_grid(ffn_down_gemm_kernel<1>, occ, kDnLds, max_items);
        hipLaunchKernelGGL(ffn_down_gemm_kernel<1>, grid, dim3(256), kDnLds, s, p);
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
