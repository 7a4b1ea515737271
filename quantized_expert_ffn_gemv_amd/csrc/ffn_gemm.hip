// Grouped GEMM on the matrix cores for experts that serve many tokens (prefill
// and large batches): the same products as the decode kernels (exact code
// operands, mfma_ops.h), on v_mfma_f32_32x32x16_bf16, which does twice the
// work per cycle of the 16 x 16 x 32 form on gfx950.
//
// Why a separate path: the decode kernels give each 16-token work tile its own
// pass over the expert's weights, which is right when a weight byte meets a
// handful of tokens.  With hundreds of tokens per expert ("Strata" page, sec.
// 2.3: a batch's tokens share an expert) the contraction is dense and the
// matrix cores should set the pace, so
//   * a gate/up item is 128 token rows (8 consecutive work-list tiles of one
//     expert) times 128 intermediate rows of gate and of up, on a workgroup of
//     4 waves (two workgroups per CU); each wave owns 32 rows (a gate tile and
//     an up tile of 32 x 32 accumulators for each 32 tokens);
//   * a down item is 64 token rows times 512 output rows, on 8 waves of 64
//     rows, with the three bf16 planes of h;
//   * activations (x, pre-permuted into code pair order by gemm_xprep_kernel,
//     or the h planes), the codes of the item's rows and their scales go from
//     L2/HBM straight into LDS ring slots with direct-to-LDS loads, half a
//     group (64 along K) per slot, two slots ahead, shared by the waves;
//   * workgroups take items in an order that keeps consecutive items (the
//     row blocks of one token chunk, then the next chunk of the same expert)
//     on one XCD, so their activations and codes meet in that XCD's L2.
// The per-group fold uses a ratio chain instead of a separate accumulator per
// group.  With t_j = s_j / L for scale group j of a weight row and
// C_j = sum (128 + L q) x over the group (the matrix cores' sum),
//     acc_j = acc_(j-1) * (t_(j-1) / t_j) + C_j,
// so after the last group J, acc_J * t_J = sum_j t_j C_j.  The group sums of
// the activations enter once per item: acc += (sum_j beta_j X_j) / t_J with
// beta_j = b_j - (128 / L) s_j and X_j = sum x over the group, on float32
// MFMAs (32 x 32 x 2), and y = acc * t_J is sum_j (s_j sum q x + b_j X_j) =
// sum (q s + b) x: the FMA form of the Flash-MoE page, sec. 2, per group.  A
// zero scale is replaced by 2^-40 in the ratios (its group's code part then
// adds 2^-43 C instead of 0), so that no ratio divides by zero.
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
constexpr int kDnRows = 64 * kWaves;                   // output rows per down item (512)
constexpr int kRowB = kGroup * 2;                      // one bf16 row of a 128-wide group in LDS
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

// h = hi + mid + lo exactly, each part the top 16 bits of what is left (a
// float32 significand has 24 bits: 8 per part).
__device__ __forceinline__ void split3_trunc(float h, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
#pragma clang fp contract(off)
    const uint32_t u = __float_as_uint(h);
    const float r1 = h - __uint_as_float(u & 0xFFFF0000u);
    const uint32_t v = __float_as_uint(r1);
    const float r2 = r1 - __uint_as_float(v & 0xFFFF0000u);
    hi = u >> 16;
    mid = v >> 16;
    lo = __float_as_uint(r2) >> 16;
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

// Codes of one ring slot: contiguous rows of 64 bytes from a block's first
// row, pieces of 1 KB (16 rows) ii = NPW w + j of wave w.  The lane offsets
// are fixed per item (rows at or past `valid` re-read row valid - 1); the
// block's base moves along K.
template <int NPW>
struct CodeStage {
    uint32_t off[NPW];
    __device__ __forceinline__ void init(int valid, int wu, int lane) {
#pragma unroll
        for (int j = 0; j < NPW; ++j) {
            const int ii = NPW * wu + j;
            const int rr = 16 * ii + (lane >> 2), pp = lane & 3;
            const int rc = rr < valid ? rr : valid - 1;
            off[j] = (uint32_t)rc * 64u + 16u * (uint32_t)(pp ^ ((rr >> 2) & 3));
        }
    }
    __device__ __forceinline__ void issue(const uint8_t* base, uint8_t* dst, int wu) const {
#pragma unroll
        for (int j = 0; j < NPW; ++j) dma16_sv(base, off[j], dst + (NPW * wu + j) * kDma);
    }
};

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
// On v_mfma_f32_32x32x16_bf16 (lane layout: A lane l holds row l % 32 and
// k = 8 (l / 32) + i; B column l % 32, the same k; accumulator element 4 j + i
// is row 8 j + 4 (l / 32) + i of column l % 32).  Activations are A (rows =
// tokens), codes B (columns = weight rows), so a lane's accumulators belong
// to one weight row and one scale.
// Item = (head of 8 tiles = 128 token rows, block of 256 intermediate rows).
// Wave w: gate and up rows blk*256 + 32 w + (pair order of n), n = lane % 32,
// weight tiles wt = 0 (gate) and 1 (up); token tiles tk = 0..NT-1 of 32 rows.
// The pipeline unit is half a group: unit u = (g, f) covers K 128 g + 64 f ..
// + 63, four MFMA steps of 16.  Step s (0..3) of a unit takes from lane half
// h = lane / 32 the 8 codes (and the 8 pair-ordered activations) of chunk
//     c(s, h) = (s / S) 2 S + h S + s % S   (S = 4 for groups of 128 and 64, 2 for 32)
// of the unit's 8 chunks, so a step stays inside one scale group and a lane's
// code words of a unit are contiguous in the row.
// Two workgroups of 4 waves per CU (80 KB of LDS each), so that one
// workgroup's barriers, prologue and epilogue overlap the other's MFMAs.
// LDS: three unit slots (the 128 x rows, 128 bytes each; 32 bytes of codes of
// each of the 128 gate and 128 up rows) and two scale slots (each row's
// 16-byte aligned run of scales holding group g's).  Units are staged two
// ahead, scales with the first half of their group; every load of the main
// loop goes straight to LDS and is waited for by count.
constexpr int kGuWarps = 4;                                      // waves per gate/up workgroup
constexpr int kGuThreads = kGuWarps * kWave;
constexpr int kGuWaveRows = 32;                                  // gate (and up) rows per wave
constexpr int kGuRows = kGuWaveRows * kGuWarps;                  // 128 per item
constexpr int kUnitRowB = 128;                                   // bytes of one x row per unit
constexpr int kGuActUnit = kGuTok * kUnitRowB;                   // 16 KB
constexpr int kGuCodeUnit = 2 * kGuRows * 32;                    // 8 KB
constexpr int kGuUnitB = kGuActUnit + kGuCodeUnit;               // 24 KB
constexpr int kGuUnits = 3;
constexpr int kGuScaleSlot = 2 * kGuRows * 16;                   // 4 KB
constexpr int kGuScaleSlots = 2;
constexpr size_t kGuLds = (size_t)kGuUnits * kGuUnitB + (size_t)kGuScaleSlots * kGuScaleSlot;   // 80 KB
constexpr int kGuActDma = kGuActUnit / kDma / kGuWarps;          // 4 per wave
constexpr int kGuCodeDma = kGuCodeUnit / kDma / kGuWarps;        // 2 per wave

typedef float floatx16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ floatx16_t mfma32(const uint32_t (&a)[4], const uint32_t (&b)[4], floatx16_t c) {
    const bf16x8_t A = __builtin_bit_cast(bf16x8_t, a);
    const bf16x8_t B = __builtin_bit_cast(bf16x8_t, b);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B, c, 0, 0, 0);
}

// Weight row held by column n (0..31) of a 32-row tile: pair order within each
// run of 8 (0,4,1,5,2,6,3,7), so that h stored at column n lands in the pair
// order of the down kernels' operands.
__device__ __forceinline__ int pair_order_row32(int n) { return 8 * (n >> 3) + ((n & 7) >> 1) + 4 * (n & 1); }

// LDS placement of the unit slots, for 64 banks served 16 lanes at a time: a
// unit's x (or h) row is 128 bytes, its 16-byte chunk c at position
// c ^ ((r >> 1) & 7), so that the 16 rows one read touches at one chunk (two
// rows per 256-byte bank line) hit 16 distinct bank groups; a row's codes are
// 32 bytes, piece p at position p ^ ((r >> 3) & 1), for the same reason.
__device__ __forceinline__ int unit_act_pos(int r, int c) { return c ^ ((r >> 1) & 7); }
__device__ __forceinline__ int unit_code_offset(int r, int piece) { return r * 32 + 16 * (piece ^ ((r >> 3) & 1)); }

template <int SPG>
__global__ __launch_bounds__(kGuThreads, 2) __attribute__((amdgpu_waves_per_eu(2, 2))) void ffn_gateup_gemm_kernel(GemmParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int S = SPG == 4 ? 2 : 4;                 // MFMA steps per scale group within a unit
    constexpr int GPU = 4 / S;                          // scale groups per unit
    const int tid = threadIdx.x, lane = tid & 63, n = lane & 31, hh = lane >> 5;
    const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = p.H, I = p.I, NG = H / kGroup, NGS = p.NGS, NU = 2 * NG;
    const int n_items = ld_scalar(p.n_heads, 0) * p.blocks;
    const int per = (n_items + 7) >> 3;
    const int lrow = kGuWaveRows * wu + pair_order_row32(n);        // row within the block
    uint8_t* const sbuf = smem + kGuUnits * kGuUnitB;

    for (int slot_i = blockIdx.x; slot_i < 8 * per; slot_i += gridDim.x) {
        const int item = xcd_item(slot_i, per);
        if (item >= n_items) continue;
        Meta<kGuTiles> mt;
        gemm_meta<kGuTiles>(p, item, mt);
        const int row_base = mt.blk * kGuRows;
        const int valid = I - row_base < kGuRows ? I - row_base : kGuRows;
        const bool rows_ok = kGuWaveRows * wu < valid;     // waves past I stage and wait, nothing more
        // activation staging: load j of wave w is 1 KB piece 4 w + j of the
        // unit slot: token rows 32 w + 8 j + lane / 8 (work tile 2 w + j / 2),
        // 16-byte position lane % 8, which holds the chunk unit_act_pos maps there
        uint32_t soff[kGuActDma];
#pragma unroll
        for (int j = 0; j < kGuActDma; ++j) {
            int r0, rn;
            tile_rows(p, mt.h0, 2 * wu + (j >> 1), r0, rn);
            const int sl = 8 * (j & 1) + (lane >> 3);
            int tok = 0;
            if (rn > 0) {
                tok = p.work[(size_t)(mt.h0 + 2 * wu + (j >> 1)) * kWorkInts + 4 + (sl < rn ? sl : 0)];
                tok = (tok >= 0 && tok < p.T) ? tok : 0;
            }
            const int row = 32 * wu + 8 * j + (lane >> 3);
            soff[j] = (uint32_t)tok * (uint32_t)(H * 2) + 16u * (uint32_t)unit_act_pos(row, lane & 7);
        }
        // code staging: load j of wave w is piece ii = 2 (w & 1) + j of the
        // gate (w < 2) or up rows: rows 32 ii + lane / 2, piece lane % 2
        uint32_t coff[kGuCodeDma];
#pragma unroll
        for (int j = 0; j < kGuCodeDma; ++j) {
            const int rr = 32 * (kGuCodeDma * (wu & 1) + j) + (lane >> 1);
            const int rc = rr < valid ? rr : valid - 1;
            coff[j] = (uint32_t)rc * 64u + 16u * (uint32_t)((lane & 1) ^ ((rr >> 3) & 1));
        }
        const uint8_t* xbytes = reinterpret_cast<const uint8_t*>(p.xp);
        const uint8_t* cmat = wu < 2 ? p.qa : p.qb;
        // scales: waves 0-1 gate rows 64 (w & 1) + lane, waves 2-3 up rows
        const int srow = 64 * (wu & 1) + lane;
        const uint16_t* smat = wu < 2 ? p.sa : p.sb;
        const size_t srow_g = (size_t)mt.e * I + row_base + (srow < valid ? srow : valid - 1);
        // stage unit u (and, for the first half of a group, its scales)
        auto stage = [&](int u) {
            const int g = u >> 1, f = u & 1;
            uint8_t* base = smem + (u % kGuUnits) * kGuUnitB;
#pragma unroll
            for (int j = 0; j < kGuActDma; ++j)
                dma16_sv(xbytes + (size_t)g * kRowB + f * kUnitRowB, soff[j], base + (kGuActDma * wu + j) * kDma);
            const uint8_t* cb = cmat + (((size_t)mt.e * NG + g) * I + row_base) * 64 + f * 32;
#pragma unroll
            for (int j = 0; j < kGuCodeDma; ++j)
                dma16_sv(cb, coff[j], base + kGuActUnit + (wu >> 1) * (kGuCodeUnit / 2) + (kGuCodeDma * (wu & 1) + j) * kDma);
            if (f == 0) {
                const size_t e_off = (srow_g * NGS + (size_t)g * SPG) * 2;
                dma16(reinterpret_cast<const uint8_t*>(smat) + (e_off & ~(size_t)15),
                      sbuf + (g % kGuScaleSlots) * kGuScaleSlot + wu * kDma);
            }
        };
        const size_t lrow_g = (size_t)mt.e * I + row_base + (rows_ok ? lrow : 0);
        auto scale_at = [&](int g, int j) {                // j: scale group within group g
            const uint32_t k = (uint32_t)(lrow_g * NGS + (size_t)g * SPG + j) & 7u;
            const uint8_t* sb = sbuf + (g % kGuScaleSlots) * kGuScaleSlot + lrow * 16 + 2 * k;
            const float f0 = f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(sb));
            const float f1 = f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(sb + kGuScaleSlot / 2));
            return float2{f0 == 0.f ? kTinyScale : f0, f1 == 0.f ? kTinyScale : f1};
        };

        stage(0);
        stage(1);
        auto run = [&](auto ntc) {
            constexpr int NT = decltype(ntc)::value;
            floatx16_t acc[2][NT];
#pragma unroll
            for (int wt = 0; wt < 2; ++wt)
#pragma unroll
                for (int tk = 0; tk < NT; ++tk)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[wt][tk][e] = 0.f;
            float sprev[2] = {1.f, 1.f};

            for (int u = 0; u < NU; ++u) {
                // unit u has landed: the loads after it are unit u + 1's (6 per
                // wave, plus 1 when it starts a group)
                if (u + 1 < NU) {
                    if ((u & 1) != 0) wait_vmem<kGuActDma + kGuCodeDma + 1>();
                    else wait_vmem<kGuActDma + kGuCodeDma>();
                } else {
                    wait_vmem<0>();
                }
                lds_barrier();
                if (u + 2 < NU) stage(u + 2);
                const int g = u >> 1, f = u & 1;
                const uint8_t* base = smem + (u % kGuUnits) * kGuUnitB;
                if (rows_ok) {
                    // this lane's 4 code words of the unit: words h S .. of each
                    // scale group's 2 S words (S = 4: piece h; S = 2: half of
                    // pieces 0 and 1)
                    uint32_t cw[2][4];
#pragma unroll
                    for (int wt = 0; wt < 2; ++wt) {
                        const uint8_t* cs = base + kGuActUnit + wt * (kGuCodeUnit / 2);
                        if constexpr (S == 4) {
                            const uint4 c = *reinterpret_cast<const uint4*>(cs + unit_code_offset(lrow, hh));
                            cw[wt][0] = c.x; cw[wt][1] = c.y; cw[wt][2] = c.z; cw[wt][3] = c.w;
                        } else {
#pragma unroll
                            for (int pc = 0; pc < 2; ++pc) {
                                const uint2 c = *reinterpret_cast<const uint2*>(cs + unit_code_offset(lrow, pc) + 8 * hh);
                                cw[wt][2 * pc] = c.x; cw[wt][2 * pc + 1] = c.y;
                            }
                        }
                    }
#pragma unroll
                    for (int j = 0; j < GPU; ++j) {
                        const int gj = f * GPU + j;               // scale group within group g
                        if (gj < SPG) {
                            const float2 sc = scale_at(g, gj);
                            if (g > 0 || gj > 0) {
                                const float r0 = sprev[0] * __builtin_amdgcn_rcpf(sc.x);
                                const float r1 = sprev[1] * __builtin_amdgcn_rcpf(sc.y);
#pragma unroll
                                for (int tk = 0; tk < NT; ++tk) {
                                    acc[0][tk] *= r0;
                                    acc[1][tk] *= r1;
                                }
                            }
                            sprev[0] = sc.x;
                            sprev[1] = sc.y;
                        }
#pragma unroll
                        for (int s2 = 0; s2 < S; ++s2) {
                            const int c = j * 2 * S + hh * S + s2;       // chunk of the unit
                            uint32_t B[2][4];
                            code_operand<4>(&cw[0][j * S + s2], 0, B[0]);
                            code_operand<4>(&cw[1][j * S + s2], 0, B[1]);
#pragma unroll
                            for (int tk = 0; tk < NT; ++tk) {
                                const int r = 32 * tk + n;
                                const uint4 a4 =
                                    *reinterpret_cast<const uint4*>(base + r * kUnitRowB + 16 * unit_act_pos(r, c));
                                const uint32_t A[4] = {a4.x, a4.y, a4.z, a4.w};
                                acc[0][tk] = mfma32(A, B[0], acc[0][tk]);
                                acc[1][tk] = mfma32(A, B[1], acc[1][tk]);
                            }
                        }
                    }
                }
            }

            // ---- group sums of x on float32 MFMAs (32 x 32 x 2: A lane l: token
            // row l % 32, group 2 jb + h; B: weight row n, the same group)
            wait_vmem<0>();
            if (rows_ok) {
                const float invt[2] = {kLever<4> * __builtin_amdgcn_rcpf(sprev[0]),
                                       kLever<4> * __builtin_amdgcn_rcpf(sprev[1])};
                int tokx[NT];
#pragma unroll
                for (int tk = 0; tk < NT; ++tk) tokx[tk] = meta_token<kGuTiles>(p, mt, 2 * tk + (n >> 4), n & 15);
                // inputs of 4 MFMA steps (8 groups) per batch, all loads of a
                // batch issued together
                constexpr int BJ = 4;
                const size_t orow = ((size_t)mt.e * I + row_base + lrow) * NGS;
                const int NJ = (NGS + 1) / 2;
                for (int jb0 = 0; jb0 < NJ; jb0 += BJ) {
                    uint32_t sn[BJ][2], bn[BJ][2];
                    float xn[BJ][NT];
#pragma unroll
                    for (int b = 0; b < BJ; ++b) {
                        const int gs0 = 2 * (jb0 + b) + hh;
                        const int gs = gs0 < NGS ? gs0 : 0;
                        sn[b][0] = p.sa[orow + gs]; bn[b][0] = p.ba[orow + gs];
                        sn[b][1] = p.sb[orow + gs]; bn[b][1] = p.bb[orow + gs];
#pragma unroll
                        for (int tk = 0; tk < NT; ++tk) xn[b][tk] = p.xs[(size_t)tokx[tk] * NGS + gs];
                    }
#pragma unroll
                    for (int b = 0; b < BJ; ++b) {
                        const bool gv = 2 * (jb0 + b) + hh < NGS;
                        float Bv[2];
#pragma unroll
                        for (int wt = 0; wt < 2; ++wt)
                            Bv[wt] = gv ? fmaf(-kOffset<4>, f16_bits_to_f32(sn[b][wt]), f16_bits_to_f32(bn[b][wt])) * invt[wt]
                                        : 0.f;
#pragma unroll
                        for (int tk = 0; tk < NT; ++tk) {
                            const float Xv = gv ? xn[b][tk] : 0.f;
                            acc[0][tk] = __builtin_amdgcn_mfma_f32_32x32x2f32(Xv, Bv[0], acc[0][tk], 0, 0, 0);
                            acc[1][tk] = __builtin_amdgcn_mfma_f32_32x32x2f32(Xv, Bv[1], acc[1][tk], 0, 0, 0);
                        }
                    }
                }

                // ---- epilogue: h = silu(gate) * up, three planes, partial sums
                // over each 16 columns.  Value index v = 16 tk + 4 j + i: token
                // row 32 tk + 8 j + 4 h + i, column 32 w + n of the block.
                float hv[16 * NT];
                const float tg = sprev[0] * kInvLever<4>, tu = sprev[1] * kInvLever<4>;
#pragma unroll
                for (int tk = 0; tk < NT; ++tk)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const float gt = acc[0][tk][e] * tg, upv = acc[1][tk][e] * tu;
                        hv[16 * tk + e] = gt * __builtin_amdgcn_rcpf(1.f + __expf(-gt)) * upv;
                    }
                const size_t plane = (size_t)p.P * I;
                const int col = row_base + kGuWaveRows * wu + n;
#pragma unroll
                for (int tk = 0; tk < NT; ++tk)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        // token rows 32 tk + 8 jj + 4 h + i lie in work tile 2 tk + jj / 2
                        const int wt_tile = 2 * tk + (jj >> 1);
                        const int r0 = mt.row0[wt_tile], rn = mt.n[wt_tile];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int slot = 8 * (jj & 1) + 4 * hh + i;
                            if (slot < rn) {
                                uint32_t hi, mid, lo;
                                split3_trunc(hv[16 * tk + 4 * jj + i], hi, mid, lo);
                                uint16_t* dst = p.hp + (size_t)(r0 + slot) * I + col;
                                dst[0] = (uint16_t)hi;
                                dst[plane] = (uint16_t)mid;
                                dst[2 * plane] = (uint16_t)lo;
                            }
                        }
                    }
                // partial sums over 16 columns (lanes of the same n / 16 and h):
                // lane n % 16 ends with value indices NT (n % 16) .. + NT - 1
                row16_stage<16 * NT, 0>(hv, lane);
                row16_stage<16 * NT, 1>(hv, lane);
                row16_stage<16 * NT, 2>(hv, lane);
                row16_stage<16 * NT, 3>(hv, lane);
#pragma unroll
                for (int uu = 0; uu < NT; ++uu) {
                    const int v = NT * (n & 15) + uu;           // value index: 16 tk + 4 jj + i
                    const int tk = v >> 4, jj = (v >> 2) & 3, i = v & 3;
                    const int wt_tile = 2 * tk + (jj >> 1);
                    int r0 = 0, rn = 0;
#pragma unroll
                    for (int t2 = 0; t2 < kGuTiles; ++t2) {
                        r0 = t2 == wt_tile ? mt.row0[t2] : r0;
                        rn = t2 == wt_tile ? mt.n[t2] : rn;
                    }
                    const int slot = 8 * (jj & 1) + 4 * hh + i;
                    if (slot < rn)
                        p.hpart[(size_t)(r0 + slot) * (I / 16) + (row_base + kGuWaveRows * wu + 16 * (n >> 4)) / 16] = hv[uu];
                }
            }
        };
        if (mt.ntk > 4) run(std::integral_constant<int, 4>{});
        else run(std::integral_constant<int, 2>{});
        lds_barrier();                       // every wave is done with the ring before the next item
    }
}

// ------------------------------------------------------------------- down
// On v_mfma_f32_32x32x16_bf16, as the gate/up kernel: A = the three bf16 planes
// of h (rows = tokens), B = codes (columns = output rows).
// Item = (head of 4 tiles = 64 token rows, block of 512 output rows).  Wave w:
// output rows blk*512 + 64 w + 32 wt + n, wt = 0, 1; token tiles tk = 0..NT-1
// of 32 rows.  Units of 64 along I with the chunk mapping of the gate/up
// kernel.  LDS: three unit slots (each: the three planes of h for the 64 token
// rows, 128 bytes per row and plane; 32 bytes of codes of each of the 512
// rows) and two scale slots; units staged two ahead.
constexpr int kDnActUnit = 3 * kDnTok * kUnitRowB;               // 24 KB
constexpr int kDnCodeUnit = kDnRows * 32;                        // 16 KB
constexpr int kDnUnitB = kDnActUnit + kDnCodeUnit;               // 40 KB
constexpr int kDnUnits = 3;
constexpr int kDnScaleSlot = kDnRows * 16;                       // 8 KB
constexpr int kDnScaleSlots = 2;
constexpr size_t kDnLds = (size_t)kDnUnits * kDnUnitB + (size_t)kDnScaleSlots * kDnScaleSlot;   // 136 KB
constexpr int kDnActDma = kDnActUnit / kDma / kWaves;            // 3 per wave
constexpr int kDnCodeDma = kDnCodeUnit / kDma / kWaves;          // 2 per wave

template <int SPG>
__global__ __launch_bounds__(kThreads, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void ffn_down_gemm_kernel(GemmParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int S = SPG == 4 ? 2 : 4;                 // MFMA steps per scale group within a unit
    constexpr int GPU = 4 / S;                          // scale groups per unit
    constexpr int G = kGroup / SPG;
    const int tid = threadIdx.x, lane = tid & 63, n = lane & 31, hh = lane >> 5;
    const int wu = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int H = p.H, I = p.I, NG = I / kGroup, NGS = p.NGS, NU = 2 * NG;
    const int n_items = ld_scalar(p.n_heads, 0) * p.blocks;
    const int per = (n_items + 7) >> 3;
    const size_t plane_b = (size_t)p.P * I * 2;
    uint8_t* const sbuf = smem + kDnUnits * kDnUnitB;

    for (int slot_i = blockIdx.x; slot_i < 8 * per; slot_i += gridDim.x) {
        const int item = xcd_item(slot_i, per);
        if (item >= n_items) continue;
        Meta<kDnTiles> mt;
        gemm_meta<kDnTiles>(p, item, mt);
        const int blk_base = mt.blk * kDnRows;
        const int valid = H - blk_base < kDnRows ? H - blk_base : kDnRows;
        const bool rows_ok = 64 * wu < valid;
        // activation staging: load j of wave w is 1 KB piece ii = 3 w + j of
        // the unit slot: plane ii / 8, token rows 8 (ii % 8) + lane / 8 (work
        // tile (ii % 8) / 2), position lane % 8 holding the chunk unit_act_pos maps there
        uint32_t soff[kDnActDma];
#pragma unroll
        for (int j = 0; j < kDnActDma; ++j) {
            const int ii = kDnActDma * wu + j, pl = ii >> 3, rr = 8 * (ii & 7) + (lane >> 3);
            int row = 0;
#pragma unroll
            for (int t2 = 0; t2 < kDnTiles; ++t2)
                row = (rr >> 4) == t2 ? meta_row<kDnTiles>(mt, t2, rr & 15) : row;
            soff[j] = (uint32_t)(pl * plane_b + (size_t)row * (I * 2)) + 16u * (uint32_t)unit_act_pos(rr, lane & 7);
        }
        // code staging: load j of wave w is piece ii = 2 w + j: rows 32 ii + lane / 2, piece lane % 2
        uint32_t coff[kDnCodeDma];
#pragma unroll
        for (int j = 0; j < kDnCodeDma; ++j) {
            const int rr = 32 * (kDnCodeDma * wu + j) + (lane >> 1);
            const int rc = rr < valid ? rr : valid - 1;
            coff[j] = (uint32_t)rc * 64u + 16u * (uint32_t)((lane & 1) ^ ((rr >> 3) & 1));
        }
        // scales: wave w stages rows 64 w + lane
        const int srow = 64 * wu + lane;
        const size_t srow_g = (size_t)mt.e * H + blk_base + (srow < valid ? srow : valid - 1);
        const uint8_t* hbytes = reinterpret_cast<const uint8_t*>(p.hp);
        auto stage = [&](int u) {
            const int g = u >> 1, f = u & 1;
            uint8_t* base = smem + (u % kDnUnits) * kDnUnitB;
#pragma unroll
            for (int j = 0; j < kDnActDma; ++j)
                dma16_sv(hbytes + (size_t)g * kRowB + f * kUnitRowB, soff[j], base + (kDnActDma * wu + j) * kDma);
            const uint8_t* cb = p.qa + (((size_t)mt.e * NG + g) * H + blk_base) * 64 + f * 32;
#pragma unroll
            for (int j = 0; j < kDnCodeDma; ++j) dma16_sv(cb, coff[j], base + kDnActUnit + (kDnCodeDma * wu + j) * kDma);
            if (f == 0) {
                const size_t e_off = (srow_g * NGS + (size_t)g * SPG) * 2;
                dma16(reinterpret_cast<const uint8_t*>(p.sa) + (e_off & ~(size_t)15),
                      sbuf + (g % kDnScaleSlots) * kDnScaleSlot + wu * kDma);
            }
        };
        int lrow[2];
#pragma unroll
        for (int wt = 0; wt < 2; ++wt) lrow[wt] = 64 * wu + 32 * wt + n;
        const size_t lrow_g0 = (size_t)mt.e * H + blk_base + (rows_ok ? lrow[0] : 0);
        auto scale_at = [&](int g, int j) {
            float2 r;
#pragma unroll
            for (int wt = 0; wt < 2; ++wt) {
                const uint32_t k = (uint32_t)((lrow_g0 + 32 * wt) * NGS + (size_t)g * SPG + j) & 7u;
                const float v = f16_bits_to_f32(
                    *reinterpret_cast<const uint16_t*>(sbuf + (g % kDnScaleSlots) * kDnScaleSlot + lrow[wt] * 16 + 2 * k));
                const float vv = v == 0.f ? kTinyScale : v;
                if (wt == 0) r.x = vv; else r.y = vv;
            }
            return r;
        };

        stage(0);
        stage(1);
        auto run = [&](auto ntc) {
            constexpr int NT = decltype(ntc)::value;
            floatx16_t acc[2][NT];
#pragma unroll
            for (int wt = 0; wt < 2; ++wt)
#pragma unroll
                for (int tk = 0; tk < NT; ++tk)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[wt][tk][e] = 0.f;
            float sprev[2] = {1.f, 1.f};

            for (int u = 0; u < NU; ++u) {
                // unit u has landed: the loads after it are unit u + 1's (5 per
                // wave, plus 1 when it starts a group)
                if (u + 1 < NU) {
                    if ((u & 1) != 0) wait_vmem<kDnActDma + kDnCodeDma + 1>();
                    else wait_vmem<kDnActDma + kDnCodeDma>();
                } else {
                    wait_vmem<0>();
                }
                lds_barrier();
                if (u + 2 < NU) stage(u + 2);
                const int g = u >> 1, f = u & 1;
                const uint8_t* base = smem + (u % kDnUnits) * kDnUnitB;
                if (rows_ok) {
                    uint32_t cw[2][4];
#pragma unroll
                    for (int wt = 0; wt < 2; ++wt) {
                        const uint8_t* cs = base + kDnActUnit;
                        if constexpr (S == 4) {
                            const uint4 c = *reinterpret_cast<const uint4*>(cs + unit_code_offset(lrow[wt], hh));
                            cw[wt][0] = c.x; cw[wt][1] = c.y; cw[wt][2] = c.z; cw[wt][3] = c.w;
                        } else {
#pragma unroll
                            for (int pc = 0; pc < 2; ++pc) {
                                const uint2 c = *reinterpret_cast<const uint2*>(cs + unit_code_offset(lrow[wt], pc) + 8 * hh);
                                cw[wt][2 * pc] = c.x; cw[wt][2 * pc + 1] = c.y;
                            }
                        }
                    }
#pragma unroll
                    for (int j = 0; j < GPU; ++j) {
                        const int gj = f * GPU + j;
                        if (gj < SPG) {
                            const float2 sc = scale_at(g, gj);
                            if (g > 0 || gj > 0) {
                                const float r0 = sprev[0] * __builtin_amdgcn_rcpf(sc.x);
                                const float r1 = sprev[1] * __builtin_amdgcn_rcpf(sc.y);
#pragma unroll
                                for (int tk = 0; tk < NT; ++tk) {
                                    acc[0][tk] *= r0;
                                    acc[1][tk] *= r1;
                                }
                            }
                            sprev[0] = sc.x;
                            sprev[1] = sc.y;
                        }
#pragma unroll
                        for (int s2 = 0; s2 < S; ++s2) {
                            const int c = j * 2 * S + hh * S + s2;
                            uint32_t B[2][4];
                            code_operand<4>(&cw[0][j * S + s2], 0, B[0]);
                            code_operand<4>(&cw[1][j * S + s2], 0, B[1]);
#pragma unroll
                            for (int tk = 0; tk < NT; ++tk) {
                                const int r = 32 * tk + n;
#pragma unroll
                                for (int pl = 0; pl < 3; ++pl) {
                                    const uint4 a4 = *reinterpret_cast<const uint4*>(
                                        base + (pl * kDnTok + r) * kUnitRowB + 16 * unit_act_pos(r, c));
                                    const uint32_t A[4] = {a4.x, a4.y, a4.z, a4.w};
                                    acc[0][tk] = mfma32(A, B[0], acc[0][tk]);
                                    acc[1][tk] = mfma32(A, B[1], acc[1][tk]);
                                }
                            }
                        }
                    }
                }
            }

            wait_vmem<0>();
            if (rows_ok) {
                // ---- group sums of h (from the 16-row partial sums) on float32
                // MFMAs (32 x 32 x 2: A token row l % 32, group 2 jb + h)
                const float invt[2] = {kLever<4> * __builtin_amdgcn_rcpf(sprev[0]),
                                       kLever<4> * __builtin_amdgcn_rcpf(sprev[1])};
                int rowx[NT];
#pragma unroll
                for (int tk = 0; tk < NT; ++tk) {
                    const int rr = 32 * tk + n;
                    int row = 0;
#pragma unroll
                    for (int t2 = 0; t2 < kDnTiles; ++t2)
                        row = (rr >> 4) == t2 ? meta_row<kDnTiles>(mt, t2, rr & 15) : row;
                    rowx[tk] = row;
                }
                constexpr int BJ = 4;
                const int NJ = (NGS + 1) / 2;
                for (int jb0 = 0; jb0 < NJ; jb0 += BJ) {
                    uint32_t sn[BJ][2], bn[BJ][2];
                    float xn[BJ][NT][G / 16];
#pragma unroll
                    for (int b = 0; b < BJ; ++b) {
                        const int gs0 = 2 * (jb0 + b) + hh;
                        const int gs = gs0 < NGS ? gs0 : 0;
#pragma unroll
                        for (int wt = 0; wt < 2; ++wt) {
                            const size_t o = ((size_t)mt.e * H + blk_base + lrow[wt]) * NGS + gs;
                            sn[b][wt] = p.sa[o];
                            bn[b][wt] = p.ba[o];
                        }
#pragma unroll
                        for (int tk = 0; tk < NT; ++tk) {
                            const float* hp = p.hpart + (size_t)rowx[tk] * (I / 16) + gs * (G / 16);
#pragma unroll
                            for (int uu = 0; uu < G / 16; ++uu) xn[b][tk][uu] = hp[uu];
                        }
                    }
#pragma unroll
                    for (int b = 0; b < BJ; ++b) {
                        const bool gv = 2 * (jb0 + b) + hh < NGS;
                        float Bv[2];
#pragma unroll
                        for (int wt = 0; wt < 2; ++wt)
                            Bv[wt] = gv ? fmaf(-kOffset<4>, f16_bits_to_f32(sn[b][wt]), f16_bits_to_f32(bn[b][wt])) * invt[wt]
                                        : 0.f;
#pragma unroll
                        for (int tk = 0; tk < NT; ++tk) {
                            float xs = 0.f;
#pragma unroll
                            for (int uu = 0; uu < G / 16; ++uu) xs += xn[b][tk][uu];
                            const float Xv = gv ? xs : 0.f;
                            acc[0][tk] = __builtin_amdgcn_mfma_f32_32x32x2f32(Xv, Bv[0], acc[0][tk], 0, 0, 0);
                            acc[1][tk] = __builtin_amdgcn_mfma_f32_32x32x2f32(Xv, Bv[1], acc[1][tk], 0, 0, 0);
                        }
                    }
                }
                // ---- Y rows in bf16: token row 32 tk + 8 jj + 4 h + i (work
                // tile 2 tk + jj / 2, slot 8 (jj % 2) + 4 h + i), column lrow[wt]
#pragma unroll
                for (int tk = 0; tk < NT; ++tk)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int wt_tile = 2 * tk + (jj >> 1);
                        const int r0 = mt.row0[wt_tile], rn = mt.n[wt_tile];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int slot = 8 * (jj & 1) + 4 * hh + i;
                            if (slot < rn) {
                                uint16_t* yrow = p.y + (size_t)(r0 + slot) * H + blk_base;
#pragma unroll
                                for (int wt = 0; wt < 2; ++wt)
                                    yrow[lrow[wt]] = (uint16_t)f32_to_bf16_bits(acc[wt][tk][4 * jj + i] * sprev[wt] * kInvLever<4>);
                            }
                        }
                    }
            }
        };
        if (mt.ntk > 2) run(std::integral_constant<int, 2>{});
        else run(std::integral_constant<int, 1>{});
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
// two groups of 128; 4-bit codes; groups of 128, 64 or 32; the staging
// offsets into x and into the h planes fit 32 bits.
bool gemm_supported(const moe_dims& d, int bits) {
    const uint64_t P = (uint64_t)d.T * d.k;
    return bits == 4 && (d.group_size == 128 || d.group_size == 64 || d.group_size == 32) && d.I % kGroup == 0 &&
           d.H % kGroup == 0 && d.H >= 2 * kGroup && d.I >= 2 * kGroup && (uint64_t)d.T * d.H * 2 < (1ull << 32) &&
           3 * P * d.I * 2 < (1ull << 32);
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
    // two workgroups per CU
    hipLaunchKernelGGL(ffn_gateup_gemm_kernel<SPG>, dim3(2 * gemm_grid()), dim3(kGuThreads), kGuLds, s, p);
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
