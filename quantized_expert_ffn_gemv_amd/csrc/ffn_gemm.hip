// Grouped GEMM on the matrix cores for experts that serve many tokens (prefill
// and large batches): the same products as the decode kernels (exact code
// operands, mfma_ops.h), tiled for reuse of each unpacked code across 128
// tokens and of each staged activation across 256 weight rows.
//
// Why a separate path: the decode kernels give each 16-token work tile its own
// pass over the expert's weights, which is right when a weight byte meets a
// handful of tokens.  With hundreds of tokens per expert ("Strata" page, sec.
// 2.3: a batch's tokens share an expert) the contraction is dense and the
// matrix cores should set the pace, so
//   * a gate/up item is 128 token rows (8 consecutive work-list tiles of one
//     expert) times 256 intermediate rows of gate and of up; each of the 8
//     waves owns 32 of them (two 16-row tiles of gate and the same two of up,
//     a 4 x 8 grid of 16 x 16 accumulator tiles), so one unpacked code
//     operand feeds 8 MFMAs and one activation operand 4;
//   * a down item is 64 token rows times 512 output rows, 64 per wave, with
//     the three bf16 planes of h (4 x 4 tiles x 3 planes);
//   * activations (x, pre-permuted into code pair order by gemm_xprep_kernel,
//     or the h planes) and the codes of the item's rows go from L2/HBM
//     straight into LDS ring slots with direct-to-LDS loads, one group of 128
//     along K per slot, one group ahead, shared by the 8 waves;
//   * workgroups take items in an order that keeps all row blocks of one token
//     chunk on one XCD, so the chunk's activations are fetched into that XCD's
//     L2 once.
// The per-group fold uses a ratio chain instead of a separate accumulator per
// group.  With t_j = s_j / L for scale group j of a weight row and
// C_j = sum (128 + L q) x over the group (the matrix cores' sum),
//     acc_j = acc_(j-1) * (t_(j-1) / t_j) + C_j,
// so after the last group J, acc_J * t_J = sum_j t_j C_j.  The group sums of
// the activations enter once per item: acc += (sum_j beta_j X_j) / t_J with
// beta_j = b_j - (128 / L) s_j and X_j = sum x over the group, which is four
// float32 MFMAs (16 x 16 x 4) per tile and 16 groups, and y = acc * t_J is
// sum_j (s_j sum q x + b_j X_j) = sum (q s + b) x: the FMA form of the
// Flash-MoE page, sec. 2, per group.  A zero scale is replaced by 2^-40 in the
// ratios (its group's code part then adds 2^-43 C instead of 0), so that no
// ratio divides by zero.
// h leaves the gate/up kernel in three bf16 planes in code pair order plus
// 16-row partial sums, as from every other gate/up kernel; the down kernel
// multiplies all three planes (with two, h's 2^-18 relative error summed over
// I moved outputs far below the rms by a few bf16 ulps where the weights are
// large, as zero-point weights are).
#include <atomic>
#include <type_traits>

#include "launch_util.h"
#include "mfma_ops.h"

namespace moe {

namespace {

constexpr int kWaves = 8;                              // waves per workgroup (both kernels)
constexpr int kThreads = kWaves * kWave;
constexpr int kGuTiles = 8;                            // work-list tiles per gate/up item
constexpr int kDnTiles = 4;                            // per down item
constexpr int kGuTok = kGuTiles * kWorkRows;           // token rows per gate/up item (128)
constexpr int kDnTok = kDnTiles * kWorkRows;           // per down item (64)
constexpr int kGuRows = 32 * kWaves;                   // intermediate rows per gate/up item (256)
constexpr int kDnRows = 64 * kWaves;                   // output rows per down item (512)
constexpr int kRowB = kGroup * 2;                      // one bf16 row of a 128-wide group in LDS
constexpr int kGuSlot = kGuTok * kRowB;                // LDS ring slot of gate/up (32 KB)
constexpr int kDnSlot = 3 * kDnTok * kRowB;            // of down: three planes (48 KB)
constexpr int kGuStage = kGuSlot / kDma / kWaves;      // direct-to-LDS loads per wave and group (4)
constexpr int kDnStage = kDnSlot / kDma / kWaves;      // (6)
constexpr float kTinyScale = 0x1p-40f;

struct GemmParams {
    const uint16_t* x;                // [T][H]
    const uint16_t* xp;               // x with each 8-element run in code pair order [T][H]
    float* xs;                        // sums of x over each scale group [T][NGS]
    const int32_t* work;
    const int32_t* n_work;
    int32_t* heads;                   // work-list index of each item's first tile
    int32_t* n_heads;
    const uint8_t* qa; const uint16_t* sa; const uint16_t* ba;   // gate, or down
    const uint8_t* qb; const uint16_t* sb; const uint16_t* bb;   // up
    uint16_t* hp;                     // bf16 planes [3][P][I]
    float* hpart;                     // [P][I/16]
    uint16_t* y;                      // [P][H]
    int T, H, I, E, P;
    int blocks;                       // row blocks per head
    int NGS;                          // scale groups along this kernel's K
};

__device__ __forceinline__ floatx4_t mfma16_f32(float a, float b, floatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Sum N values per lane over the 16 lanes of each quarter-wave (lane bits 0-3)
// by a butterfly transpose: afterwards v[0 .. N/16) of lane m (= lane % 16)
// hold the totals of value indices m N/16 + u.
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

// fp16 scale of the ring word(s) `w` for scale group j of a 128-run, as a
// float, zero replaced (see the file comment).
__device__ __forceinline__ float ring_scale(const uint32_t* w, int j) {
    const float s = f16_bits_to_f32((w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
    return s == 0.f ? kTinyScale : s;
}

// Items of a launch in XCD order: slot s (workgroup b takes slots b, b + G,
// ...; with G a multiple of 8 they all run on XCD b % 8) maps to item
// (s % 8) * per + s / 8, so consecutive items (the row blocks of one token
// chunk, then the next chunk of the same expert) share an XCD.
__device__ __forceinline__ int xcd_item(int slot, int per) { return (slot & 7) * per + (slot >> 3); }

// The item's head: expert, row block, and the (first sorted row, row count) of
// each of its TILES work-list tiles (count 0: past the expert's last tile), the
// number of tiles up to the last non-empty one, and the head's work-list index.
template <int TILES>
struct Meta {
    int e, blk, ntk, h0;
    int row0[TILES], n[TILES];
};

template <int TILES>
__device__ __forceinline__ void gemm_meta(const GemmParams& p, int item, Meta<TILES>& mt) {
    const int n_work = ld_scalar(p.n_work, 0);
    const int hd = item / p.blocks;
    mt.blk = item - hd * p.blocks;
    mt.h0 = ld_scalar(p.heads, (size_t)hd);
    const int32_t* h0 = p.work + (size_t)mt.h0 * kWorkInts;
    const int e0 = ld_scalar(h0, 0), t0 = ld_scalar(h0, 3);
    mt.e = (e0 >= 0 && e0 < p.E) ? e0 : 0;
    mt.ntk = 0;
#pragma unroll
    for (int jt = 0; jt < TILES; ++jt) {
        const int wi = mt.h0 + jt;
        const int32_t* ent = p.work + (size_t)(wi < n_work ? wi : mt.h0) * kWorkInts;
        const bool mine = wi < n_work && ld_scalar(ent, 0) == e0 && ld_scalar(ent, 3) == t0 + jt;
        const int row0 = ld_scalar(ent, 1), n = ld_scalar(ent, 2);
        const bool ok = mine && row0 >= 0 && n >= 1 && n <= kWorkRows && row0 + n <= p.P;
        mt.row0[jt] = ok ? row0 : 0;
        mt.n[jt] = ok ? n : 0;
        mt.ntk = ok ? jt + 1 : mt.ntk;
    }
}

// Token of slot `slot` of tile jt of an item (slots past the tile's rows, and
// empty tiles, give a valid token whose results are never stored).
template <int TILES>
__device__ __forceinline__ int meta_token(const GemmParams& p, const Meta<TILES>& mt, int jt, int slot) {
    if (mt.n[jt] == 0) return 0;
    const int s = slot < mt.n[jt] ? slot : 0;
    const int t = p.work[(size_t)(mt.h0 + jt) * kWorkInts + 4 + s];
    return (t >= 0 && t < p.T) ? t : 0;
}

template <int TILES>
__device__ __forceinline__ int meta_row(const Meta<TILES>& mt, int jt, int slot) {
    return mt.row0[jt] + (slot < mt.n[jt] ? slot : 0);
}

}  // namespace

// ----------------------------------------------------------------- heads
// Work-list tiles whose index within their expert is a multiple of 8 (gate/up
// items) and of 4 (down items); their work-list indices in order, and counts.
// One workgroup.
__global__ __launch_bounds__(1024) void gemm_heads_kernel(const int32_t* __restrict__ work,
                                                         const int32_t* __restrict__ n_work, int cap,
                                                         int32_t* __restrict__ heads8, int32_t* __restrict__ n8,
                                                         int32_t* __restrict__ heads4, int32_t* __restrict__ n4) {
    __shared__ int wsum[2][16];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, nw_waves = blockDim.x >> 6;
    const int nw = min(*n_work, cap);
    int c8 = 0, c4 = 0;
    for (int i0 = 0; i0 < nw; i0 += blockDim.x) {
        const int i = i0 + tid;
        const int t = i < nw ? work[(size_t)i * kWorkInts + 3] : 1;
        const int f8 = (t % kGuTiles == 0) ? 1 : 0, f4 = (t % kDnTiles == 0) ? 1 : 0;
        const uint64_t b8 = __ballot(f8), b4 = __ballot(f4);
        const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
        if (lane == 0) { wsum[0][wid] = __popcll(b8); wsum[1][wid] = __popcll(b4); }
        __syncthreads();
        int base8 = 0, tot8 = 0, base4 = 0, tot4 = 0;
        for (int w = 0; w < nw_waves; ++w) {
            base8 += (w < wid) ? wsum[0][w] : 0;
            tot8 += wsum[0][w];
            base4 += (w < wid) ? wsum[1][w] : 0;
            tot4 += wsum[1][w];
        }
        if (f8) heads8[c8 + base8 + __popcll(b8 & below)] = i;
        if (f4) heads4[c4 + base4 + __popcll(b4 & below)] = i;
        c8 += tot8;
        c4 += tot4;
        __syncthreads();
    }
    if (tid == 0) { *n8 = c8; *n4 = c4; }
}

// ---------------------------------------------------------- activations
// Per token: x with each run of 8 elements in the pair order of the 4-bit code
// operands (elements 0,4,1,5,2,6,3,7: code_operand<4> pairs codes i and i + 4
// of a word), and the float32 sum of x over each scale group of G elements.
// One workgroup of 256 per token; H a multiple of 128.
template <int G>
__global__ __launch_bounds__(256) void gemm_xprep_kernel(const uint16_t* __restrict__ x, int H,
                                                        uint16_t* __restrict__ xp, float* __restrict__ xs) {
    constexpr uint32_t LO = 0x05040100u, HI = 0x07060302u;
    constexpr int L = G / 8;                           // lanes per scale group
    const size_t t = blockIdx.x;
    const uint4* src = reinterpret_cast<const uint4*>(x + t * H);
    uint4* dst = reinterpret_cast<uint4*>(xp + t * H);
    const int NGS = H / G;
    for (int c = threadIdx.x; c < H / 8; c += blockDim.x) {
        const uint4 v = src[c];
        uint4 o;
        o.x = __builtin_amdgcn_perm(v.z, v.x, LO);     // elements 0, 4
        o.y = __builtin_amdgcn_perm(v.z, v.x, HI);     // 1, 5
        o.z = __builtin_amdgcn_perm(v.w, v.y, LO);     // 2, 6
        o.w = __builtin_amdgcn_perm(v.w, v.y, HI);     // 3, 7
        dst[c] = o;
        float s = 0.f;
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) s += bf16_bits_to_f32(w[i] & 0xFFFFu) + bf16_bits_to_f32(w[i] >> 16);
#pragma unroll
        for (int off = 1; off < L; off <<= 1) s += __shfl_xor(s, off, kWave);
        if ((c % L) == 0) xs[t * NGS + c / L] = s;
    }
}

// ---------------------------------------------------------------- rings
// LDS of one workgroup: activation ring slots, then code ring slots.  A code
// slot holds the group's codes of the item's rows (gate then up, or down),
// 64 bytes per row, the 16-byte pieces of row r at positions piece ^ ((r >> 2)
// & 3) so that 16 consecutive rows read at one piece hit 16 bank groups.
__device__ __forceinline__ int code_lds_offset(int r, int piece) { return r * 64 + 16 * (piece ^ ((r >> 2) & 3)); }

// Stage one ring slot of codes: `rows` contiguous rows of 64 bytes from `src`
// (rows at or past `valid` re-read row valid - 1), pieces of 1 KB (16 rows)
// ii = NPW w + j of wave w.
template <int NPW>
__device__ __forceinline__ void stage_codes(const uint8_t* src, int valid, uint8_t* dst, int wu, int lane) {
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
        const int ii = NPW * wu + j;
        const int rr = 16 * ii + (lane >> 2), pp = lane & 3;
        const int rc = rr < valid ? rr : valid - 1;
        dma16(src + (size_t)rc * 64 + 16 * (pp ^ ((rr >> 2) & 3)), dst + ii * kDma);
    }
}

// The code word of one weight tile for MFMA step st (natural order: word st of
// the lane's piece q; swapped order: word q of quarter st's piece).
template <bool TR>
__device__ __forceinline__ uint32_t read_code_word(const uint8_t* slot, int r, int q, int st) {
    return TR ? *reinterpret_cast<const uint32_t*>(slot + code_lds_offset(r, st) + 4 * q)
              : *reinterpret_cast<const uint32_t*>(slot + code_lds_offset(r, q) + 4 * st);
}

// Scales of one weight row for group g (SPG fp16 values) into NSW words.
template <int SPG, int NSW>
__device__ __forceinline__ void load_scales(const uint16_t* sp, uint32_t (&w)[NSW]) {
    if constexpr (SPG == 1) {
        w[0] = *sp;
    } else if constexpr (SPG == 2) {
        w[0] = *reinterpret_cast<const uint32_t*>(sp);
    } else {
        const uint2 S = *reinterpret_cast<const uint2*>(sp);
        w[0] = S.x;
        w[NSW - 1] = S.y;
    }
}

// Rows of tile jt of an item (0 when past the expert's tiles), for a tile
// index known only at run time (the staging wave's own tile).
__device__ __forceinline__ void tile_rows(const GemmParams& p, int h0, int jt, int& row0, int& n) {
    const int n_work = ld_scalar(p.n_work, 0);
    const int32_t* e0p = p.work + (size_t)h0 * kWorkInts;
    const int e0 = ld_scalar(e0p, 0), t0 = ld_scalar(e0p, 3);
    const int wi = h0 + jt;
    const int32_t* ent = p.work + (size_t)(wi < n_work ? wi : h0) * kWorkInts;
    const bool mine = wi < n_work && ld_scalar(ent, 0) == e0 && ld_scalar(ent, 3) == t0 + jt;
    const int r0 = ld_scalar(ent, 1), nn = ld_scalar(ent, 2);
    const bool ok = mine && r0 >= 0 && nn >= 1 && nn <= kWorkRows && r0 + nn <= p.P;
    row0 = ok ? r0 : 0;
    n = ok ? nn : 0;
}

// -------------------------------------------------------------- gate/up
// Item = (head of 8 tiles, block of 256 intermediate rows).  Wave w: gate and
// up rows blk*256 + 32 w + 16 hf + (pair order of m), hf = 0, 1; weight tiles
// wt = 0, 1 gate (hf), 2, 3 up (hf); token tiles tk = 0..7 (rows 16 tk ..).
// Per group g of 128 along H: activation slot g % 2 holds the 128 x rows of
// the group (wave w stages tile w), code slot g % 2 the codes of the 256 gate
// and 256 up rows, both staged one group ahead, and registers the wave's
// scales of the next group.
// SPG scale groups per 128 (1, 2 or 4): for SPG > 1 the steps carry one
// quarter of the run each (tr_word_offset), and the ratio chain advances at
// each scale group.
constexpr int kGuActRing = 2, kGuCodeRing = 2;
constexpr int kGuCodeSlot = 2 * kGuRows * 64;          // 32 KB
constexpr int kGuCodeStage = kGuCodeSlot / kDma / kWaves;   // 4
constexpr size_t kGuLds = (size_t)kGuActRing * kGuSlot + (size_t)kGuCodeRing * kGuCodeSlot;   // 128 KB

template <int SPG>
__global__ __launch_bounds__(kThreads, 1) void ffn_gateup_gemm_kernel(GemmParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr bool TR = SPG > 1;
    constexpr int SPS = 4 / SPG;                       // MFMA steps per scale group
    constexpr int NSW = SPG > 2 ? 2 : 1;               // 32-bit scale words per weight row and group
    uint8_t* const abuf = smem;
    uint8_t* const cbuf = smem + kGuActRing * kGuSlot;
    const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, q = lane >> 4;
    const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = p.H, I = p.I, NG = H / kGroup, NGS = p.NGS;
    const int n_items = ld_scalar(p.n_heads, 0) * p.blocks;
    const int per = (n_items + 7) >> 3;

    int lrow[4];                                       // row within the block, per weight tile
#pragma unroll
    for (int wt = 0; wt < 4; ++wt) lrow[wt] = 32 * wu + 16 * (wt & 1) + pair_order_row<4>(m);

    for (int slot_i = blockIdx.x; slot_i < 8 * per; slot_i += gridDim.x) {
        const int item = xcd_item(slot_i, per);
        if (item >= n_items) continue;
        Meta<kGuTiles> mt;
        gemm_meta<kGuTiles>(p, item, mt);
        const int row_base = mt.blk * kGuRows;
        const int valid = I - row_base < kGuRows ? I - row_base : kGuRows;   // rows of the block inside I
        const bool rows_ok = 32 * wu < valid;          // waves past I stage and wait, nothing more
        // activation staging: wave wu stages tile wu (rows 16 wu + 4 j + q)
        uint32_t soff[kGuStage];
        {
            int r0, rn;
            tile_rows(p, mt.h0, wu, r0, rn);
#pragma unroll
            for (int j = 0; j < kGuStage; ++j) {
                int tok = 0;
                if (rn > 0) {
                    const int sl = 4 * j + q;
                    tok = p.work[(size_t)(mt.h0 + wu) * kWorkInts + 4 + (sl < rn ? sl : 0)];
                    tok = (tok >= 0 && tok < p.T) ? tok : 0;
                }
                soff[j] = (uint32_t)tok * (uint32_t)(H * 2) + 16u * (uint32_t)(m ^ ((4 * j + q) & 15));
            }
        }
        const uint8_t* xbytes = reinterpret_cast<const uint8_t*>(p.xp);
        auto stage_act = [&](int g) {
            uint8_t* dst = abuf + (g % kGuActRing) * kGuSlot + (kGuStage * wu) * kDma;
#pragma unroll
            for (int j = 0; j < kGuStage; ++j) dma16(xbytes + soff[j] + (size_t)g * kRowB, dst + j * kDma);
        };
        // codes: waves 0-3 stage the gate rows, 4-7 the up rows
        const uint8_t* cmat = wu < 4 ? p.qa : p.qb;
        auto stage_cod = [&](int g) {
            const uint8_t* src = cmat + (((size_t)mt.e * NG + g) * I + row_base) * 64;
            stage_codes<kGuCodeStage>(src, valid, cbuf + (g % kGuCodeRing) * kGuCodeSlot + (wu >> 2) * (kGuCodeSlot / 2),
                                          wu & 3, lane);
        };
        const int rows_c = rows_ok ? row_base : 0;     // idle waves load valid scales
        uint32_t srn[4][NSW];                          // scales of the next group
        auto load_sc = [&](int g) {
#pragma unroll
            for (int wt = 0; wt < 4; ++wt)
                load_scales<SPG, NSW>((wt < 2 ? p.sa : p.sb) + ((size_t)mt.e * I + rows_c + lrow[wt]) * NGS + (size_t)g * SPG,
                                      srn[wt]);
        };

        // Every ring is one group deep: at the top of iteration g all loads are
        // waited for, the scales of g are taken out of the registers, and only
        // then are the next group's scales, activations and codes issued.  (The
        // direct-to-LDS loads are invisible to the compiler's load tracking, so
        // a tracked scale load with direct-to-LDS loads behind it would make
        // the compiler's own wait for it wait for those as well.)
        load_sc(0);
        stage_act(0);
        stage_cod(0);
        // the item's body for NT token tiles (8, or 4 when the item has at most
        // 4 non-empty tiles)
        auto run = [&](auto ntc) {
            constexpr int NT = decltype(ntc)::value;
            floatx4_t acc[4][NT];
#pragma unroll
            for (int wt = 0; wt < 4; ++wt)
#pragma unroll
                for (int tk = 0; tk < NT; ++tk) acc[wt][tk] = floatx4_t{0.f, 0.f, 0.f, 0.f};
            float sprev[4] = {1.f, 1.f, 1.f, 1.f};

            for (int g = 0; g < NG; ++g) {
                wait_vmem<0>();
                lds_barrier();
                float scg[SPG][4];
#pragma unroll
                for (int j = 0; j < SPG; ++j)
#pragma unroll
                    for (int wt = 0; wt < 4; ++wt) {
                        scg[j][wt] = ring_scale(srn[wt], j);
                        asm volatile("" : : "v"(scg[j][wt]));   // taken before the next loads are issued
                    }
                if (g + 1 < NG) {
                    load_sc(g + 1);
                    stage_act(g + 1);
                    stage_cod(g + 1);
                }
                const uint8_t* buf = abuf + (g % kGuActRing) * kGuSlot;
                const uint8_t* cslot = cbuf + (g % kGuCodeRing) * kGuCodeSlot;
                if (rows_ok) {
                    // Software pipeline: the activation operand of the next
                    // token tile (or of tile 0 of the next step) is read while
                    // the current tile's MFMAs run, and a step's code words
                    // during the step before.
                    auto lds_a = [&](int tk, int st) {
                        const int c = TR ? 4 * st + q : 4 * q + st;
                        return *reinterpret_cast<const uint4*>(buf + (16 * tk + m) * kRowB + 16 * (c ^ m));
                    };
                    auto code_w = [&](int wt, int st) {
                        return read_code_word<TR>(cslot + (wt >> 1) * (kGuCodeSlot / 2), lrow[wt], q, st);
                    };
                    uint32_t cw[4];
#pragma unroll
                    for (int wt = 0; wt < 4; ++wt) cw[wt] = code_w(wt, 0);
                    uint4 a_cur = lds_a(0, 0);
#pragma unroll
                    for (int st = 0; st < 4; ++st) {
                        if (st % SPS == 0) {
                            const int j = st / SPS;
                            if (g > 0 || j > 0) {
#pragma unroll
                                for (int wt = 0; wt < 4; ++wt) {
                                    const float r = sprev[wt] * __builtin_amdgcn_rcpf(scg[j][wt]);
#pragma unroll
                                    for (int tk = 0; tk < NT; ++tk) acc[wt][tk] *= r;
                                }
                            }
#pragma unroll
                            for (int wt = 0; wt < 4; ++wt) sprev[wt] = scg[j][wt];
                        }
                        uint32_t B[4][4];
#pragma unroll
                        for (int wt = 0; wt < 4; ++wt) code_operand<4>(&cw[wt], 0, B[wt]);
                        if (st + 1 < 4) {
#pragma unroll
                            for (int wt = 0; wt < 4; ++wt) cw[wt] = code_w(wt, st + 1);
                        }
#pragma unroll
                        for (int tk = 0; tk < NT; ++tk) {
                            uint4 a_nxt = a_cur;
                            if (tk + 1 < NT) a_nxt = lds_a(tk + 1, st);
                            else if (st + 1 < 4) a_nxt = lds_a(0, st + 1);
                            const uint32_t A[4] = {a_cur.x, a_cur.y, a_cur.z, a_cur.w};
#pragma unroll
                            for (int wt = 0; wt < 4; ++wt) acc[wt][tk] = mfma16(A, B[wt], acc[wt][tk]);
                            a_cur = a_nxt;
                            __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);   // one LDS read, then
                            __builtin_amdgcn_sched_group_barrier(0x0008, 4, 0);   // four MFMAs
                        }
                        __builtin_amdgcn_sched_barrier(0);   // one step's operands live at a time
                    }
                }
            }

            // ---- group sums of x: acc += (sum_j beta_j X_j) / t_J per tile, on
            // float32 MFMAs (A: token row 16 tk + m, group 4 jb + q; B: weight row
            // m of tile wt, the same group)
            wait_vmem<0>();
            if (rows_ok) {
                float invt[4];
#pragma unroll
                for (int wt = 0; wt < 4; ++wt) invt[wt] = kLever<4> * __builtin_amdgcn_rcpf(sprev[wt]);
                int tokx[NT];
#pragma unroll
                for (int tk = 0; tk < NT; ++tk) tokx[tk] = meta_token<kGuTiles>(p, mt, tk, m);
                // loads of step jb + 1 are issued before the MFMAs of step jb
                uint32_t sn[4], bn[4];
                float xn[NT];
                auto load_bias = [&](int jb) {
                    const int gs = 4 * jb + q < NGS ? 4 * jb + q : 0;
#pragma unroll
                    for (int wt = 0; wt < 4; ++wt) {
                        const size_t o = ((size_t)mt.e * I + row_base + lrow[wt]) * NGS + gs;
                        sn[wt] = (wt < 2 ? p.sa : p.sb)[o];
                        bn[wt] = (wt < 2 ? p.ba : p.bb)[o];
                    }
#pragma unroll
                    for (int tk = 0; tk < NT; ++tk) xn[tk] = p.xs[(size_t)tokx[tk] * NGS + gs];
                };
                const int NJ = (NGS + 3) / 4;
                load_bias(0);
                for (int jb = 0; jb < NJ; ++jb) {
                    const bool gv = 4 * jb + q < NGS;
                    float Bv[4], Xv[NT];
#pragma unroll
                    for (int wt = 0; wt < 4; ++wt)
                        Bv[wt] = gv ? fmaf(-kOffset<4>, f16_bits_to_f32(sn[wt]), f16_bits_to_f32(bn[wt])) * invt[wt] : 0.f;
#pragma unroll
                    for (int tk = 0; tk < NT; ++tk) Xv[tk] = gv ? xn[tk] : 0.f;
                    if (jb + 1 < NJ) load_bias(jb + 1);
#pragma unroll
                    for (int tk = 0; tk < NT; ++tk)
#pragma unroll
                        for (int wt = 0; wt < 4; ++wt) acc[wt][tk] = mfma16_f32(Xv[tk], Bv[wt], acc[wt][tk]);
                }

                // ---- epilogue: h = silu(gate) * up, three planes, 16-row partial
                // sums; value index v = 32 hf + 4 tk + i: token row 16 tk + 4 q + i,
                // column 32 w + 16 hf + m of the block
                float hv[8 * NT];
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const float tg = sprev[hf] * kInvLever<4>, tu = sprev[2 + hf] * kInvLever<4>;
#pragma unroll
                    for (int tk = 0; tk < NT; ++tk)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float gt = acc[hf][tk][i] * tg, upv = acc[2 + hf][tk][i] * tu;
                            hv[4 * NT * hf + 4 * tk + i] = gt / (1.f + expf(-gt)) * upv;
                        }
                }
                const size_t plane = (size_t)p.P * I;
                const int i0 = row_base + 32 * wu;
#pragma unroll
                for (int tk = 0; tk < NT; ++tk) {
                    const int r0 = mt.row0[tk], rn = mt.n[tk];
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int row = 4 * q + i;
                            if (row < rn) {
                                uint32_t hi, mid, lo;
                                split3_bf16(hv[4 * NT * hf + 4 * tk + i], hi, mid, lo);
                                uint16_t* dst = p.hp + (size_t)(r0 + row) * I + i0 + 16 * hf + m;
                                dst[0] = (uint16_t)hi;
                                dst[plane] = (uint16_t)mid;
                                dst[2 * plane] = (uint16_t)lo;
                            }
                        }
                }
                // partial sums over each 16 columns: lane m ends with value indices
                // NV m .. NV m + NV - 1 (NV = NT / 2), i.e. token rows of one tile
                // and one 16-column half of the wave
                row16_stage<8 * NT, 0>(hv, lane);
                row16_stage<8 * NT, 1>(hv, lane);
                row16_stage<8 * NT, 2>(hv, lane);
                row16_stage<8 * NT, 3>(hv, lane);
                constexpr int NV = NT / 2;                 // totals per lane
                const int tk = (NV * m / 4) % NT, hf = NV * m / (4 * NT);
                int r0 = 0, rn = 0;
#pragma unroll
                for (int t2 = 0; t2 < NT; ++t2) {
                    r0 = t2 == tk ? mt.row0[t2] : r0;
                    rn = t2 == tk ? mt.n[t2] : rn;
                }
#pragma unroll
                for (int u = 0; u < NV; ++u) {
                    const int row = 4 * q + (NV * m + u) % 4;
                    if (row < rn) p.hpart[(size_t)(r0 + row) * (I / 16) + (i0 + 16 * hf) / 16] = hv[u];
                }
            }
        };
        if (mt.ntk > 4) run(std::integral_constant<int, 8>{});
        else run(std::integral_constant<int, 4>{});
        lds_barrier();                       // every wave is done with the rings before the next item
    }
}

// ------------------------------------------------------------------- down
// Item = (head of 4 tiles, block of 512 output rows).  Wave w: output rows
// blk*512 + 64 w + 16 wt + m, wt = 0..3; token tiles tk = 0..3 (rows 16 tk ..).
// Per group g of 128 along I: activation slot g % 2 holds the three planes of
// h for the 64 rows (plane pl, row r at (pl * 64 + r) * 256, chunks swizzled
// by the row's low 4 bits), code slot g % 2 the codes of the 512 rows, both
// staged one group ahead, and registers the wave's scales of the next group.
constexpr int kDnActRing = 2, kDnCodeRing = 2;
constexpr int kDnCodeSlot = kDnRows * 64;              // 32 KB
constexpr int kDnCodeStage = kDnCodeSlot / kDma / kWaves;   // 4
constexpr size_t kDnLds = (size_t)kDnActRing * kDnSlot + (size_t)kDnCodeRing * kDnCodeSlot;   // 160 KB

template <int SPG>
__global__ __launch_bounds__(kThreads, 1) void ffn_down_gemm_kernel(GemmParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr bool TR = SPG > 1;
    constexpr int SPS = 4 / SPG;
    constexpr int NSW = SPG > 2 ? 2 : 1;
    constexpr int G = kGroup / SPG;
    uint8_t* const abuf = smem;
    uint8_t* const cbuf = smem + kDnActRing * kDnSlot;
    const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, q = lane >> 4;
    const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = p.H, I = p.I, NG = I / kGroup, NGS = p.NGS;
    const int n_items = ld_scalar(p.n_heads, 0) * p.blocks;
    const int per = (n_items + 7) >> 3;
    const size_t plane_b = (size_t)p.P * I * 2;

    for (int slot_i = blockIdx.x; slot_i < 8 * per; slot_i += gridDim.x) {
        const int item = xcd_item(slot_i, per);
        if (item >= n_items) continue;
        Meta<kDnTiles> mt;
        gemm_meta<kDnTiles>(p, item, mt);
        const int blk_base = mt.blk * kDnRows;
        const int valid = H - blk_base < kDnRows ? H - blk_base : kDnRows;
        const int n_base = blk_base + 64 * wu;
        const bool rows_ok = 64 * wu < valid;
        // activation staging: load j of wave wu is LDS piece ii = 6 wu + j:
        // plane ii / 16, rows 4 (ii % 16) + q
        uint64_t soff[kDnStage];
#pragma unroll
        for (int j = 0; j < kDnStage; ++j) {
            const int ii = kDnStage * wu + j, pl = ii >> 4, rr = 4 * (ii & 15) + q;
            int row = 0;
#pragma unroll
            for (int t2 = 0; t2 < kDnTiles; ++t2)
                row = (rr >> 4) == t2 ? meta_row<kDnTiles>(mt, t2, rr & 15) : row;
            soff[j] = pl * plane_b + (uint64_t)row * (I * 2) + 16u * (uint32_t)(m ^ (rr & 15));
        }
        const uint8_t* hbytes = reinterpret_cast<const uint8_t*>(p.hp);
        auto stage_act = [&](int g) {
            uint8_t* dst = abuf + (g % kDnActRing) * kDnSlot + (kDnStage * wu) * kDma;
#pragma unroll
            for (int j = 0; j < kDnStage; ++j) dma16(hbytes + soff[j] + (size_t)g * kRowB, dst + j * kDma);
        };
        auto stage_cod = [&](int g) {
            const uint8_t* src = p.qa + (((size_t)mt.e * NG + g) * H + blk_base) * 64;
            stage_codes<kDnCodeStage>(src, valid, cbuf + (g % kDnCodeRing) * kDnCodeSlot, wu, lane);
        };
        const int nb_c = rows_ok ? n_base : 0;
        uint32_t srn[4][NSW];
        auto load_sc = [&](int g) {
#pragma unroll
            for (int wt = 0; wt < 4; ++wt)
                load_scales<SPG, NSW>(p.sa + ((size_t)mt.e * H + nb_c + 16 * wt + m) * NGS + (size_t)g * SPG, srn[wt]);
        };

        // The same one-group rings as the gate/up kernel.
        load_sc(0);
        stage_act(0);
        stage_cod(0);
        // the item's body for NT token tiles (4, or 2 when the item has at most
        // 2 non-empty tiles)
        auto run = [&](auto ntc) {
            constexpr int NT = decltype(ntc)::value;
            floatx4_t acc[4][NT];
#pragma unroll
            for (int wt = 0; wt < 4; ++wt)
#pragma unroll
                for (int tk = 0; tk < NT; ++tk) acc[wt][tk] = floatx4_t{0.f, 0.f, 0.f, 0.f};
            float sprev[4] = {1.f, 1.f, 1.f, 1.f};

            for (int g = 0; g < NG; ++g) {
                wait_vmem<0>();
                lds_barrier();
                float scg[SPG][4];
#pragma unroll
                for (int j = 0; j < SPG; ++j)
#pragma unroll
                    for (int wt = 0; wt < 4; ++wt) {
                        scg[j][wt] = ring_scale(srn[wt], j);
                        asm volatile("" : : "v"(scg[j][wt]));
                    }
                if (g + 1 < NG) {
                    load_sc(g + 1);
                    stage_act(g + 1);
                    stage_cod(g + 1);
                }
                const uint8_t* buf = abuf + (g % kDnActRing) * kDnSlot;
                const uint8_t* cslot = cbuf + (g % kDnCodeRing) * kDnCodeSlot;
                if (rows_ok) {
#pragma unroll
                    for (int j = 0; j < SPG; ++j) {
                        float sc[4];
#pragma unroll
                        for (int wt = 0; wt < 4; ++wt) sc[wt] = scg[j][wt];
                        if (g > 0 || j > 0) {
#pragma unroll
                            for (int wt = 0; wt < 4; ++wt) {
                                const float r = sprev[wt] * __builtin_amdgcn_rcpf(sc[wt]);
#pragma unroll
                                for (int tk = 0; tk < NT; ++tk) acc[wt][tk] *= r;
                            }
                        }
#pragma unroll
                        for (int wt = 0; wt < 4; ++wt) sprev[wt] = sc[wt];
#pragma unroll
                        for (int s2 = 0; s2 < SPS; ++s2) {
                            const int st = j * SPS + s2;
                            const int c = TR ? 4 * st + q : 4 * q + st;
                            uint32_t B[4][4];
#pragma unroll
                            for (int wt = 0; wt < 4; ++wt) {
                                const uint32_t w = read_code_word<TR>(cslot, 64 * wu + 16 * wt + m, q, st);
                                code_operand<4>(&w, 0, B[wt]);
                            }
#pragma unroll
                            for (int tk = 0; tk < NT; ++tk) {
#pragma unroll
                                for (int pl = 0; pl < 3; ++pl) {
                                    const uint4 a4 = *reinterpret_cast<const uint4*>(
                                        buf + (pl * kDnTok + 16 * tk + m) * kRowB + 16 * (c ^ m));
                                    const uint32_t A[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
                                    for (int wt = 0; wt < 4; ++wt) acc[wt][tk] = mfma16(A, B[wt], acc[wt][tk]);
                                }
                            }
                            __builtin_amdgcn_sched_barrier(0);
                        }
                    }
                }
            }

            wait_vmem<0>();
            if (rows_ok) {
                // ---- group sums of h (from the 16-row partial sums), as in gate/up
                float invt[4];
#pragma unroll
                for (int wt = 0; wt < 4; ++wt) invt[wt] = kLever<4> * __builtin_amdgcn_rcpf(sprev[wt]);
                int rowx[NT];
#pragma unroll
                for (int tk = 0; tk < NT; ++tk) rowx[tk] = meta_row<kDnTiles>(mt, tk, m);
                // loads of step jb + 1 are issued before the MFMAs of step jb
                uint32_t sn[4], bn[4];
                float xn[NT][G / 16];
                auto load_bias = [&](int jb) {
                    const int gs = 4 * jb + q < NGS ? 4 * jb + q : 0;
#pragma unroll
                    for (int wt = 0; wt < 4; ++wt) {
                        const size_t o = ((size_t)mt.e * H + n_base + 16 * wt + m) * NGS + gs;
                        sn[wt] = p.sa[o];
                        bn[wt] = p.ba[o];
                    }
#pragma unroll
                    for (int tk = 0; tk < NT; ++tk) {
                        const float* hp = p.hpart + (size_t)rowx[tk] * (I / 16) + gs * (G / 16);
#pragma unroll
                        for (int u = 0; u < G / 16; ++u) xn[tk][u] = hp[u];
                    }
                };
                const int NJ = (NGS + 3) / 4;
                load_bias(0);
                for (int jb = 0; jb < NJ; ++jb) {
                    const bool gv = 4 * jb + q < NGS;
                    float Bv[4], Xv[NT];
#pragma unroll
                    for (int wt = 0; wt < 4; ++wt)
                        Bv[wt] = gv ? fmaf(-kOffset<4>, f16_bits_to_f32(sn[wt]), f16_bits_to_f32(bn[wt])) * invt[wt] : 0.f;
#pragma unroll
                    for (int tk = 0; tk < NT; ++tk) {
                        float xs = 0.f;
#pragma unroll
                        for (int u = 0; u < G / 16; ++u) xs += xn[tk][u];
                        Xv[tk] = gv ? xs : 0.f;
                    }
                    if (jb + 1 < NJ) load_bias(jb + 1);
#pragma unroll
                    for (int tk = 0; tk < NT; ++tk)
#pragma unroll
                        for (int wt = 0; wt < 4; ++wt) acc[wt][tk] = mfma16_f32(Xv[tk], Bv[wt], acc[wt][tk]);
                }
                // ---- Y rows in bf16 (token row 16 tk + 4 q + i, column 16 wt + m)
#pragma unroll
                for (int tk = 0; tk < NT; ++tk) {
                    const int r0 = mt.row0[tk], rn = mt.n[tk];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = 4 * q + i;
                        if (row < rn) {
                            uint16_t* yrow = p.y + (size_t)(r0 + row) * H + n_base + m;
#pragma unroll
                            for (int wt = 0; wt < 4; ++wt)
                                yrow[16 * wt] = (uint16_t)f32_to_bf16_bits(acc[wt][tk][i] * sprev[wt] * kInvLever<4>);
                        }
                    }
                }
            }
        };
        if (mt.ntk > 2) run(std::integral_constant<int, 4>{});
        else run(std::integral_constant<int, 2>{});
        lds_barrier();
    }
}

// ---------------------------------------------------------------- launch

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

// The rings stage two groups ahead within an item, so each K holds at least
// two groups of 128; 4-bit codes; groups of 128, 64 or 32.
bool gemm_supported(const moe_dims& d, int bits) {
    return bits == 4 && (d.group_size == 128 || d.group_size == 64 || d.group_size == 32) && d.I % kGroup == 0 &&
           d.H % kGroup == 0 && d.H >= 2 * kGroup && d.I >= 2 * kGroup;
}

static long max_heads(const moe_dims& d, int tiles) {
    return work_capacity(d) / tiles + (d.E < (long)d.T * d.k ? d.E : (long)d.T * d.k);
}

static size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// After the matrix-core workspace: the two heads lists (count, then indices),
// x in pair order, and the sums of x per scale group.
struct GemmSpace {
    size_t heads8, heads4, xp, xs, total;
};

static GemmSpace gemm_space(const moe_dims& d) {
    GemmSpace g{};
    size_t o = mfma_workspace_bytes(d);
    g.heads8 = o;
    o += round256((size_t)(max_heads(d, kGuTiles) + 64) * sizeof(int32_t));
    g.heads4 = o;
    o += round256((size_t)(max_heads(d, kDnTiles) + 64) * sizeof(int32_t));
    g.xp = o;
    o += round256((size_t)d.T * d.H * sizeof(uint16_t));
    g.xs = o;
    const int gs = d.group_size > 0 ? d.group_size : kGroup;
    o += round256((size_t)d.T * (d.H / gs) * sizeof(float));
    g.total = o;
    return g;
}

size_t gemm_workspace_bytes(const moe_dims& d) { return gemm_space(d).total; }

static GemmParams gemm_params(const FfnArgs& a, bool down) {
    const moe_dims& d = a.d;
    GemmParams p{};
    p.x = a.x; p.work = a.work; p.n_work = a.n_work; p.y = a.y;
    p.T = d.T; p.H = d.H; p.I = d.I; p.E = d.E; p.P = d.T * d.k;
    char* ws = reinterpret_cast<char*>(a.h);
    const size_t P = (size_t)p.P;
    p.hp = reinterpret_cast<uint16_t*>(ws);
    p.hpart = reinterpret_cast<float*>(ws + ((3 * P * d.I * sizeof(uint16_t) + 255) & ~(size_t)255));
    const GemmSpace g = gemm_space(d);
    int32_t* hl = reinterpret_cast<int32_t*>(ws + (down ? g.heads4 : g.heads8));
    p.n_heads = hl;
    p.heads = hl + 64;
    p.xp = reinterpret_cast<const uint16_t*>(ws + g.xp);
    p.xs = reinterpret_cast<float*>(ws + g.xs);
    p.NGS = (down ? d.I : d.H) / d.group_size;
    return p;
}

// Workgroups of a launch: one per CU, a multiple of 8 (the XCD order).
static unsigned gemm_grid() {
    const int cus = device_cus();
    return (unsigned)(cus >= 8 ? cus / 8 * 8 : 8);
}

template <int SPG>
static void launch_gu(const GemmParams& p, hipStream_t s) {
    hipLaunchKernelGGL(ffn_gateup_gemm_kernel<SPG>, dim3(gemm_grid()), dim3(kThreads), kGuLds, s, p);
}

template <int SPG>
static void launch_dn(const GemmParams& p, hipStream_t s) {
    hipLaunchKernelGGL(ffn_down_gemm_kernel<SPG>, dim3(gemm_grid()), dim3(kThreads), kDnLds, s, p);
}

int launch_gateup_gemm(const FfnArgs& a, hipStream_t s) {
    const moe_dims& d = a.d;
    if (d.T * d.k == 0) return MOE_OK;
    if (!gemm_supported(d, a.bits) || max_lds_per_block() < kDnLds) return MOE_ERR_UNSUPPORTED;
    GemmParams p = gemm_params(a, false);
    p.qa = a.w.q[0]; p.sa = a.w.scale[0]; p.ba = a.w.bias[0];
    p.qb = a.w.q[1]; p.sb = a.w.scale[1]; p.bb = a.w.bias[1];
    p.blocks = (d.I + kGuRows - 1) / kGuRows;
    const GemmParams p4 = gemm_params(a, true);
    hipLaunchKernelGGL(gemm_heads_kernel, dim3(1), dim3(1024), 0, s, a.work, a.n_work, (int)work_capacity(d),
                       p.heads, p.n_heads, p4.heads, p4.n_heads);
    uint16_t* xp = const_cast<uint16_t*>(p.xp);
    switch (d.group_size) {
        case 32: hipLaunchKernelGGL(gemm_xprep_kernel<32>, dim3(d.T), dim3(256), 0, s, a.x, d.H, xp, p.xs); break;
        case 64: hipLaunchKernelGGL(gemm_xprep_kernel<64>, dim3(d.T), dim3(256), 0, s, a.x, d.H, xp, p.xs); break;
        default: hipLaunchKernelGGL(gemm_xprep_kernel<128>, dim3(d.T), dim3(256), 0, s, a.x, d.H, xp, p.xs); break;
    }
    switch (d.group_size) {
        case 32: launch_gu<4>(p, s); break;
        case 64: launch_gu<2>(p, s); break;
        default: launch_gu<1>(p, s); break;
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// The down heads list is the one the gate/up launch of the same call (or of
// the split gate/up call that filled this workspace) wrote.
int launch_down_gemm(const FfnArgs& a, hipStream_t s) {
    const moe_dims& d = a.d;
    if (d.T * d.k == 0) return MOE_OK;
    if (!gemm_supported(d, a.bits) || max_lds_per_block() < kDnLds) return MOE_ERR_UNSUPPORTED;
    GemmParams p = gemm_params(a, true);
    p.qa = a.w.q[2]; p.sa = a.w.scale[2]; p.ba = a.w.bias[2];
    p.blocks = (d.H + kDnRows - 1) / kDnRows;
    switch (d.group_size) {
        case 32: launch_dn<4>(p, s); break;
        case 64: launch_dn<2>(p, s); break;
        default: launch_dn<1>(p, s); break;
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
