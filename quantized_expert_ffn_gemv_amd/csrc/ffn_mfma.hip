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
// Exactness: a code q becomes the bf16 value 128 + L q (q OR-ed into the top
// mantissa bits of 0x4300; L = 8 for 4-bit, 32 for 2-bit codes), exact, and
// activations are bf16, so every product is exact and the matrix core
// accumulates in float32.  Per group of 128 along K the tile accumulator
// C = sum (128 + L q) x is folded into the output as
//     (s / L) * C + (b - (128 / L) s) * X,    X = sum of x over the group,
// which is sum (q s + b) x (the FMA form of the Flash-MoE page, sec. 2).  X
// comes from a third MFMA with an all-ones A operand.  Putting q in the top
// mantissa bits keeps the 128 X part of C within a few times the code part,
// so float32 rounding in C stays at float32 level relative to the result.
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
#include "common.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

// Work split: a 256-thread workgroup owns an output block (16 gate + 16 up
// rows, or 32 down rows) of one expert; its 4 waves take disjoint quarters of
// the K groups, so each wave streams only a few groups and can have all of them
// in flight at once (decode batches are small: the whole FFN of one token at
// the A3B-style shape is ~1.6 MB, a few KB per wave).  Partial accumulators
// are summed in LDS in a fixed wave order, then wave 0 runs the epilogue.
constexpr int kWaves = 4;

struct MfmaParams {
    const uint16_t* x;
    const int32_t* sorted_pairs;
    const int32_t* counts;
    const int32_t* offsets;
    const int32_t* active;
    const int32_t* n_active;
    const uint8_t* qa;  const uint16_t* sa;  const uint16_t* ba;   // gate, or down
    const uint8_t* qb;  const uint16_t* sb;  const uint16_t* bb;   // up
    uint16_t* hp;       // bf16 planes [3][P][I]
    float* hpart;       // [P][I/16] partial sums of h over 16-row tiles
    uint16_t* y;        // [P][H]
    int T, H, I, k, E, P;
    int items_per_expert;
};

__device__ __forceinline__ floatx4_t mfma16(const uint32_t (&a)[4], const uint32_t (&b)[4], floatx4_t c) {
    const bf16x8_t A = __builtin_bit_cast(bf16x8_t, a);
    const bf16x8_t B = __builtin_bit_cast(bf16x8_t, b);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, c, 0, 0, 0);
}

// A operand of MFMA step s for one group: the lane's codes (4-bit: 4 words,
// 2-bit: 2 words) -> 4 packed pairs of bf16 128 + L*q (see kLever).  Pair i of
// a word holds codes (i, i + W/2) of that word (W codes per word).
template <int BITS>
__device__ __forceinline__ void code_operand(const uint32_t* w, int s, uint32_t (&out)[4]) {
    if constexpr (BITS == 4) {
        const uint32_t v = w[s];
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = (shift_to(v, 4 * i - 3) & 0x00780078u) | 0x43004300u;
    } else {
        const uint32_t v = w[s >> 1];
        const int base = 4 * (s & 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = (shift_to(v, 2 * (base + i) - 5) & 0x00600060u) | 0x43004300u;
    }
}

// B operand of MFMA step s from the lane's 32 natural-order bf16 activations
// X (16 packed words), in the pair order of code_operand: pair i = elements
// (a, a + W/2), built with one v_perm_b32.
template <int BITS>
__device__ __forceinline__ void act_operand(const uint32_t* X, int s, uint32_t (&out)[4]) {
    constexpr uint32_t LO = 0x05040100u, HI = 0x07060302u;   // low / high halves of two words
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int lo_word, hi_word;
        if constexpr (BITS == 4) {            // elements 8s + i and 8s + i + 4
            lo_word = 4 * s + (i >> 1);
            hi_word = lo_word + 2;
        } else {                              // elements 16(s/2) + 4(s%2) + i and that + 8
            lo_word = 8 * (s >> 1) + 2 * (s & 1) + (i >> 1);
            hi_word = lo_word + 4;
        }
        out[i] = __builtin_amdgcn_perm(X[hi_word], X[lo_word], (i & 1) ? HI : LO);
    }
}

__device__ __forceinline__ void split3_bf16(float h, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
    hi = f32_to_bf16_bits(h);
    const float r1 = h - bf16_bits_to_f32(hi);
    mid = f32_to_bf16_bits(r1);
    const float r2 = r1 - bf16_bits_to_f32(mid);
    lo = f32_to_bf16_bits(r2);
}

// Groups [gb, ge) of K handled by wave w (an even split; a wave may get none).
__device__ __forceinline__ void wave_groups(int NG, int w, int& gb, int& ng) {
    gb = (w * NG) / kWaves;
    ng = ((w + 1) * NG) / kWaves - gb;
}

// Read a value that no kernel writes while this one runs through the scalar
// path: uniform addresses in the constant address space become s_load, which
// waits on its own counter instead of queueing behind the vector loads of the
// code stream.  Used for the routing lists written by earlier kernels.
template <typename T>
__device__ __forceinline__ T ld_scalar(const T* p, size_t i) {
    typedef const __attribute__((address_space(4))) T* cptr;
    return ((cptr)(p))[i];
}

// Weight row held by output row m (0..15) of a 16-row tile.  The gate/up
// kernel stores h of its output rows 4q..4q+3 at consecutive positions, and
// the down kernel reads h in the pair order of its code operands; loading the
// gate/up rows in that order makes the two agree with no data exchange.
template <int BITS>
__device__ __forceinline__ int pair_order_row(int m) {
    if constexpr (BITS == 4) return 8 * (m >> 3) + ((m & 7) >> 1) + 4 * (m & 1);   // 0,4,1,5,2,6,3,7 per 8
    else return (m >> 1) + 8 * (m & 1);                                           // 0,8,1,9,...,7,15
}

// --------------------------------------------------------------- gate / up
// LDS: [kWaves][NGW][4][16] float scales (per wave: s/L and b - (128/L) s of
// gate, then of up, for the tile's 16 output rows), then [kWaves][64][8]
// partial sums.  SJ = scale entries per lane per matrix (>= NGW / 4).
template <int BITS, int D, int SJ>
__global__ __launch_bounds__(256) void ffn_gateup_mfma_kernel(MfmaParams p) {
    constexpr int LB = 128 * BITS / 8 / 4;     // bytes per lane per group (16 or 8)
    constexpr int LW = LB / 4;                 // code words per lane per group
    extern __shared__ float lds[];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, m = lane & 15, q = lane >> 4;
    const int a = blockIdx.x / p.items_per_expert, it = blockIdx.x % p.items_per_expert;
    if (a >= ld_scalar(p.n_active, 0)) return;
    const int e = ld_scalar(p.active, a);
    if (e < 0 || e >= p.E) return;
    const int H = p.H, I = p.I, NG = H / kGroup, NGW = (NG + kWaves - 1) / kWaves;
    int gb, ng;
    wave_groups(NG, w, gb, ng);
    const int i0 = it * 16;
    const size_t rowbytes = (size_t)H * BITS / 8;
    const size_t wrow = (size_t)e * I + i0 + pair_order_row<BITS>(m);   // this lane's weight row
    const uint8_t* grow = p.qa + wrow * rowbytes + q * LB;
    const uint8_t* urow = p.qb + wrow * rowbytes + q * LB;
    const int cnt = ld_scalar(p.counts, e), r0 = ld_scalar(p.offsets, e);
    float* my_sc = lds + w * NGW * 64;
    float* red = lds + kWaves * NGW * 64;
    uint32_t ONE[4] = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};

    for (int t0 = 0; t0 < cnt; t0 += 16) {
        const int n_tile = min(16, cnt - t0);
        const bool tok_ok = m < n_tile;
        floatx4_t accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};

        if (ng > 0) {
            // 1. scales of this wave's groups (oldest loads: waiting for them
            //    does not wait for the code stream issued after them)
            uint32_t sv[4][SJ];
            if (t0 == 0) {
#pragma unroll
                for (int j = 0; j < SJ; ++j) {
                    const int idx = lane + 64 * j;
                    const int gl = min(idx >> 4, ng - 1), r = idx & 15;
                    const size_t src = ((size_t)e * I + i0 + pair_order_row<BITS>(r)) * NG + gb + gl;
                    sv[0][j] = p.sa[src]; sv[1][j] = p.ba[src];
                    sv[2][j] = p.sb[src]; sv[3][j] = p.bb[src];
                }
            }
            // 2. the code stream
            uint32_t wg[D][LW], wu[D][LW], xv[D][16];
            auto issue_codes = [&](int slot, int g) {
                if constexpr (BITS == 4) {
                    const uint4 A = *reinterpret_cast<const uint4*>(grow + (size_t)g * 64);
                    const uint4 B = *reinterpret_cast<const uint4*>(urow + (size_t)g * 64);
                    wg[slot][0] = A.x; wg[slot][1] = A.y; wg[slot][2] = A.z; wg[slot][3] = A.w;
                    wu[slot][0] = B.x; wu[slot][1] = B.y; wu[slot][2] = B.z; wu[slot][3] = B.w;
                } else {
                    const uint2 A = *reinterpret_cast<const uint2*>(grow + (size_t)g * 32);
                    const uint2 B = *reinterpret_cast<const uint2*>(urow + (size_t)g * 32);
                    wg[slot][0] = A.x; wg[slot][1] = A.y;
                    wu[slot][0] = B.x; wu[slot][1] = B.y;
                }
            };
#pragma unroll
            for (int d = 0; d < D; ++d) issue_codes(d, gb + min(d, ng - 1));

            // 3. token of this lane's column from scalar loads (columns past the
            //    tile's end reuse the first token; their outputs are never written)
            int pr = ld_scalar(p.sorted_pairs, r0 + t0);
#pragma unroll
            for (int j = 1; j < 16; ++j) {
                const int v = ld_scalar(p.sorted_pairs, r0 + t0 + min(j, n_tile - 1));
                pr = (m == j && j < n_tile) ? v : pr;
            }
            const int tok = (pr >= 0 && pr < p.P) ? pr / p.k : 0;
            const uint16_t* xrow = p.x + (size_t)tok * H + q * 32;
            auto issue_act = [&](int slot, int g) {
                const uint4* xs = reinterpret_cast<const uint4*>(xrow + (size_t)g * kGroup);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const uint4 X = xs[v];
                    xv[slot][4 * v] = X.x; xv[slot][4 * v + 1] = X.y;
                    xv[slot][4 * v + 2] = X.z; xv[slot][4 * v + 3] = X.w;
                }
            };
#pragma unroll
            for (int d = 0; d < D; ++d) issue_act(d, gb + min(d, ng - 1));

            // 4. scales -> LDS, converted once: s/L and b - (128/L) s
            if (t0 == 0) {
#pragma unroll
                for (int j = 0; j < SJ; ++j) {
                    const int idx = lane + 64 * j;
                    const int gl = idx >> 4, r = idx & 15;
                    if (gl < ng) {
                        const float s1 = f16_bits_to_f32(sv[0][j]), b1 = f16_bits_to_f32(sv[1][j]);
                        const float s2 = f16_bits_to_f32(sv[2][j]), b2 = f16_bits_to_f32(sv[3][j]);
                        float* dst = my_sc + gl * 64 + r;
                        dst[0] = s1 * kInvLever<BITS>;
                        dst[16] = fmaf(-kOffset<BITS>, s1, b1);
                        dst[32] = s2 * kInvLever<BITS>;
                        dst[48] = fmaf(-kOffset<BITS>, s2, b2);
                    }
                }
            }

            for (int g0 = 0; g0 < ng; g0 += D) {
#pragma unroll
                for (int d = 0; d < D; ++d) {
                    const int gl = g0 + d;
                    uint32_t cw[LW], cu[LW], cx[16];
#pragma unroll
                    for (int v = 0; v < LW; ++v) { cw[v] = wg[d][v]; cu[v] = wu[d][v]; }
#pragma unroll
                    for (int v = 0; v < 16; ++v) cx[v] = xv[d][v];
                    const int gn = gb + min(gl + D, ng - 1);   // past the end: a harmless reload
                    issue_codes(d, gn);
                    issue_act(d, gn);
                    if (gl < ng) {
                        floatx4_t Cg = {0.f, 0.f, 0.f, 0.f}, Cu = Cg, Cx = Cg;
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            uint32_t Ag[4], Au[4], Bx[4];
                            code_operand<BITS>(cw, s, Ag);
                            code_operand<BITS>(cu, s, Au);
                            act_operand<BITS>(cx, s, Bx);
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
                }
            }
        }

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
                const float up = ((red[(0 * 64 + lane) * 8 + 4 + i] + red[(1 * 64 + lane) * 8 + 4 + i]) +
                                  red[(2 * 64 + lane) * 8 + 4 + i]) + red[(3 * 64 + lane) * 8 + 4 + i];
                hv[i] = gt / (1.f + expf(-gt)) * up;
            }
            // sum of h over the tile's 16 rows for this token (fixed order)
            float part = (hv[0] + hv[1]) + (hv[2] + hv[3]);
            part += __shfl_xor(part, 16, kWave);
            part += __shfl_xor(part, 32, kWave);
            if (tok_ok) {
                const int r = r0 + t0 + m;
                if (q == 0) p.hpart[(size_t)r * (I / 16) + it] = part;
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
        __syncthreads();   // red is reused by the next pass
    }
}

// ------------------------------------------------------------------- down
// Output block: 2 tiles of 16 rows of one expert.  B operand = the three bf16
// planes of h (already in pair order), three MFMAs per step; the bias term
// uses the per-16-row partial sums of h.  LDS: [kWaves][NGW][2][32] float
// scales (s/L, b - (128/L) s), then [kWaves][64][8] partial sums.
template <int BITS, int D>
__global__ __launch_bounds__(256) void ffn_down_mfma_kernel(MfmaParams p) {
    constexpr int LB = 128 * BITS / 8 / 4;
    constexpr int LW = LB / 4;
    extern __shared__ float lds[];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, m = lane & 15, q = lane >> 4;
    const int a = blockIdx.x / p.items_per_expert, nt = blockIdx.x % p.items_per_expert;
    if (a >= *p.n_active) return;
    const int e = p.active[a];
    if (e < 0 || e >= p.E) return;
    const int H = p.H, I = p.I, NG = I / kGroup, NGW = (NG + kWaves - 1) / kWaves;
    int gb, ng;
    wave_groups(NG, w, gb, ng);
    const int n0 = nt * 32;
    const size_t rowbytes = (size_t)I * BITS / 8;
    const uint8_t* row0 = p.qa + ((size_t)e * H + n0 + m) * rowbytes + q * LB;
    const uint8_t* row1 = row0 + 16 * rowbytes;
    const int cnt = p.counts[e], r0 = p.offsets[e];
    float* my_sc = lds + w * NGW * 64;
    float* red = lds + kWaves * NGW * 64;
    const size_t plane = (size_t)p.P * I;

    for (int t0 = 0; t0 < cnt; t0 += 16) {
        const bool tok_ok = t0 + m < cnt;
        floatx4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
        if (ng > 0) {
            const int r = r0 + t0 + (tok_ok ? m : 0);      // empty columns reuse a valid row
            const uint16_t* hrow = p.hp + (size_t)r * I + q * 32;
            const float* prow = p.hpart + (size_t)r * (I / 16);
            uint32_t w0[D][LW], w1[D][LW], hv[D][3][16];
            float4 hp0[D], hp1[D];
            auto issue_codes = [&](int slot, int g) {
                if constexpr (BITS == 4) {
                    const uint4 A = *reinterpret_cast<const uint4*>(row0 + (size_t)g * 64);
                    const uint4 B = *reinterpret_cast<const uint4*>(row1 + (size_t)g * 64);
                    w0[slot][0] = A.x; w0[slot][1] = A.y; w0[slot][2] = A.z; w0[slot][3] = A.w;
                    w1[slot][0] = B.x; w1[slot][1] = B.y; w1[slot][2] = B.z; w1[slot][3] = B.w;
                } else {
                    const uint2 A = *reinterpret_cast<const uint2*>(row0 + (size_t)g * 32);
                    const uint2 B = *reinterpret_cast<const uint2*>(row1 + (size_t)g * 32);
                    w0[slot][0] = A.x; w0[slot][1] = A.y;
                    w1[slot][0] = B.x; w1[slot][1] = B.y;
                }
            };
            auto issue_act = [&](int slot, int g) {
#pragma unroll
                for (int pl = 0; pl < 3; ++pl) {
                    const uint4* src = reinterpret_cast<const uint4*>(hrow + pl * plane + (size_t)g * kGroup);
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const uint4 X = src[v];
                        hv[slot][pl][4 * v] = X.x; hv[slot][pl][4 * v + 1] = X.y;
                        hv[slot][pl][4 * v + 2] = X.z; hv[slot][pl][4 * v + 3] = X.w;
                    }
                }
                hp0[slot] = *reinterpret_cast<const float4*>(prow + 8 * g);
                hp1[slot] = *reinterpret_cast<const float4*>(prow + 8 * g + 4);
            };
#pragma unroll
            for (int d = 0; d < D; ++d) issue_codes(d, gb + min(d, ng - 1));
            if (t0 == 0) {
                const size_t rb = ((size_t)e * H + n0) * NG + gb;
                for (int idx = lane; idx < ng * 32; idx += 64) {
                    const int gl = idx >> 5, rr = idx & 31;
                    const size_t src = rb + (size_t)rr * NG + gl;
                    const float sv = f16_bits_to_f32(p.sa[src]), bv = f16_bits_to_f32(p.ba[src]);
                    my_sc[gl * 64 + rr] = sv * kInvLever<BITS>;
                    my_sc[gl * 64 + 32 + rr] = fmaf(-kOffset<BITS>, sv, bv);
                }
            }
#pragma unroll
            for (int d = 0; d < D; ++d) issue_act(d, gb + min(d, ng - 1));

            for (int g0 = 0; g0 < ng; g0 += D) {
#pragma unroll
                for (int d = 0; d < D; ++d) {
                    const int gl = g0 + d;
                    uint32_t c0[LW], c1[LW], ch[3][16];
#pragma unroll
                    for (int v = 0; v < LW; ++v) { c0[v] = w0[d][v]; c1[v] = w1[d][v]; }
#pragma unroll
                    for (int pl = 0; pl < 3; ++pl)
#pragma unroll
                        for (int v = 0; v < 16; ++v) ch[pl][v] = hv[d][pl][v];
                    const float4 q0 = hp0[d], q1 = hp1[d];
                    const int gn = gb + min(gl + D, ng - 1);
                    issue_codes(d, gn);
                    issue_act(d, gn);
                    if (gl < ng) {
                        // sum of this lane's token's h over the group (8 partial sums)
                        const float Hs = ((q0.x + q0.y) + (q0.z + q0.w)) + ((q1.x + q1.y) + (q1.z + q1.w));
                        floatx4_t C0 = {0.f, 0.f, 0.f, 0.f}, C1 = C0;
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            uint32_t A0[4], A1[4];
                            code_operand<BITS>(c0, s, A0);
                            code_operand<BITS>(c1, s, A1);
#pragma unroll
                            for (int pl = 0; pl < 3; ++pl) {
                                // planes are stored in pair order: step s = words 4s..4s+3
                                const uint32_t Bh[4] = {ch[pl][4 * s], ch[pl][4 * s + 1], ch[pl][4 * s + 2],
                                                        ch[pl][4 * s + 3]};
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
                }
            }
        }
        float* mine = red + (w * 64 + lane) * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) { mine[i] = acc0[i]; mine[4 + i] = acc1[i]; }
        __syncthreads();
        if (w == 0 && tok_ok) {
            float o[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                o[i] = ((red[(0 * 64 + lane) * 8 + i] + red[(1 * 64 + lane) * 8 + i]) +
                        red[(2 * 64 + lane) * 8 + i]) + red[(3 * 64 + lane) * 8 + i];
            uint16_t* yrow = p.y + (size_t)(r0 + t0 + m) * H + n0 + 4 * q;
            uint2 o0, o1;
            o0.x = f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16);
            o0.y = f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16);
            o1.x = f32_to_bf16_bits(o[4]) | (f32_to_bf16_bits(o[5]) << 16);
            o1.y = f32_to_bf16_bits(o[6]) | (f32_to_bf16_bits(o[7]) << 16);
            *reinterpret_cast<uint2*>(yrow) = o0;
            *reinterpret_cast<uint2*>(yrow + 16) = o1;
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ launch

size_t mfma_workspace_bytes(const moe_dims& d) {
    const size_t P = (size_t)d.T * d.k;
    const size_t planes = 3 * P * d.I * sizeof(uint16_t);
    const size_t part = P * (d.I / 16) * sizeof(float);
    return ((planes + 255) & ~(size_t)255) + ((part + 255) & ~(size_t)255);
}

static MfmaParams mfma_params(const FfnArgs& a) {
    const moe_dims& d = a.d;
    MfmaParams p{};
    p.x = a.x; p.sorted_pairs = a.sorted_pairs; p.counts = a.counts; p.offsets = a.offsets;
    p.active = a.active; p.n_active = a.n_active; p.y = a.y;
    p.T = d.T; p.H = d.H; p.I = d.I; p.k = d.k; p.E = d.E; p.P = d.T * d.k;
    const size_t P = (size_t)p.P;
    char* ws = reinterpret_cast<char*>(a.h);
    p.hp = reinterpret_cast<uint16_t*>(ws);
    p.hpart = reinterpret_cast<float*>(ws + ((3 * P * d.I * sizeof(uint16_t) + 255) & ~(size_t)255));
    return p;
}

static long max_experts(const moe_dims& d) {
    const long P = (long)d.T * d.k;
    return d.E < P ? d.E : P;
}

static size_t mfma_lds_bytes(int NG) {
    const int NGW = (NG + kWaves - 1) / kWaves;
    return ((size_t)kWaves * NGW * 64 + (size_t)kWaves * 64 * 8) * sizeof(float);
}

// Prefetch depth per wave: each wave streams at most ceil(NG/4) groups; up to
// 4 (gate/up) or 2 (down, whose slots also hold three activation planes) are
// kept in flight.
template <int BITS, int D, int SJ>
static void gateup_launch(dim3 grid, size_t lds, hipStream_t s, const MfmaParams& p) {
    hipLaunchKernelGGL((ffn_gateup_mfma_kernel<BITS, D, SJ>), grid, dim3(256), lds, s, p);
}

// (depth, scale entries per lane) for a wave of NGW groups
template <int BITS>
static void gateup_dispatch(int NGW, dim3 grid, size_t lds, hipStream_t s, const MfmaParams& p) {
    if (NGW <= 1) gateup_launch<BITS, 1, 1>(grid, lds, s, p);
    else if (NGW <= 2) gateup_launch<BITS, 2, 1>(grid, lds, s, p);
    else if (NGW <= 4) gateup_launch<BITS, 4, 1>(grid, lds, s, p);
    else if (NGW <= 8) gateup_launch<BITS, 4, 2>(grid, lds, s, p);
    else if (NGW <= 12) gateup_launch<BITS, 4, 3>(grid, lds, s, p);
    else gateup_launch<BITS, 4, 4>(grid, lds, s, p);
}

template <int BITS, int D>
static void down_launch(dim3 grid, size_t lds, hipStream_t s, const MfmaParams& p) {
    hipLaunchKernelGGL((ffn_down_mfma_kernel<BITS, D>), grid, dim3(256), lds, s, p);
}

int launch_gateup_mfma(const FfnArgs& a, hipStream_t s) {
    const moe_dims& d = a.d;
    if (d.T * d.k == 0) return MOE_OK;
    MfmaParams p = mfma_params(a);
    p.qa = a.w.q[0]; p.sa = a.w.scale[0]; p.ba = a.w.bias[0];
    p.qb = a.w.q[1]; p.sb = a.w.scale[1]; p.bb = a.w.bias[1];
    p.items_per_expert = d.I / 16;
    const dim3 grid((unsigned)(max_experts(d) * p.items_per_expert));
    const int NG = d.H / kGroup, NGW = (NG + kWaves - 1) / kWaves;
    const size_t lds = mfma_lds_bytes(NG);
    if (a.bits == 4) gateup_dispatch<4>(NGW, grid, lds, s, p);
    else gateup_dispatch<2>(NGW, grid, lds, s, p);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int launch_down_mfma(const FfnArgs& a, hipStream_t s) {
    const moe_dims& d = a.d;
    if (d.T * d.k == 0) return MOE_OK;
    MfmaParams p = mfma_params(a);
    p.qa = a.w.q[2]; p.sa = a.w.scale[2]; p.ba = a.w.bias[2];
    p.items_per_expert = d.H / 32;
    const dim3 grid((unsigned)(max_experts(d) * p.items_per_expert));
    const int NG = d.I / kGroup, NGW = (NG + kWaves - 1) / kWaves;
    const size_t lds = mfma_lds_bytes(NG);
    // depth 2 costs two thirds of the waves per SIMD: only worth it for long K
    if (a.bits == 4) {
        if (NGW >= 4) down_launch<4, 2>(grid, lds, s, p);
        else down_launch<4, 1>(grid, lds, s, p);
    } else {
        if (NGW >= 4) down_launch<2, 2>(grid, lds, s, p);
        else down_launch<2, 1>(grid, lds, s, p);
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
