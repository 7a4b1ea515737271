// Quantised expert FFN, vector-ALU matvec path.
//
// Prior art on the pages: the hand-written INT4 decode GEMV of the "Strata"
// page (sec. 3.4: weights laid out group-contiguously, dequantise then
// multiply-add per group, experts merged in one buffer) and the 4/2-bit
// dequant matvec of the Flash-MoE page (sec. 3: tiled, SIMD reduction, shared
// input cache; sec. 2: weight = nibble*scale + bias with the FMA rewrite).
// This is a fresh design for wave64 CDNA4:
//
//  * Work item = (work-list tile of up to 16 rows of one expert, block of
//    output rows).  Items are pulled by a grid-stride loop over
//    n_work * items_per_expert, with n_work read on the device, so the launch
//    never depends on routing results.
//  * Each row of codes is read once per token tile with 16-byte loads; LG
//    consecutive lanes cover one row (LG * 16 contiguous bytes per load), each
//    lane group carries 4 rows so every activation fetch from LDS serves 4 rows.
//  * Gate/up: a code q is turned into the exact bf16 value 128 + L q by OR-ing
//    it into the mantissa of the bf16 pattern 0x4300 (L = kLever: 8 for 4-bit,
//    16 for 2-bit), two codes per 32-bit register, and multiplied against bf16
//    activation pairs with v_dot2_f32_bf16 (products exact, float32
//    accumulation).  Per 16-byte chunk (inside one group) the sum
//    D = sum (128 + L q) x folds into the row total as
//        (s / L) D + (b - (128 / L) s) X,      X = sum of x over the chunk,
//    i.e. sum (q s + b) x with the scale and bias applied once per chunk -- the
//    FMA form of the Flash-MoE page with the bias term carried by X.
//  * Down: the activations h are float32, so codes are converted with
//    v_cvt_f32_ubyte and accumulated with FMA; the same per-chunk fold applies.
//  * Row totals are reduced across the LG lanes with xor shuffles; SwiGLU is
//    applied in the gate/up epilogue, bf16 rounding in the down epilogue.
#include "common.h"

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct GemvParams {
    const uint16_t* x;
    const int32_t* work;        // work list entries (kWorkInts int32 each)
    const int32_t* n_work;
    const uint8_t* qa;  const uint16_t* sa;  const uint16_t* ba;   // gate, or down
    const uint8_t* qb;  const uint16_t* sb;  const uint16_t* bb;   // up (gate/up kernel only)
    float* h;
    uint16_t* y;
    int T, H, I, k, E;
    int LG;                 // lanes per row (power of two, divides the chunks per row)
    int items_per_expert;
    int gs;                 // scale group along K: 128, 64 or 32 (at least one 16-byte chunk)
};

// codes of one 32-bit word -> bf16 pairs (128 + L q_j, 128 + L q_{j+W/2})
template <int BITS>
__device__ __forceinline__ void codes_to_bf16_pairs(uint32_t w, uint32_t* out) {
    if constexpr (BITS == 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) out[j] = (shift_to(w, 4 * j - 3) & 0x00780078u) | 0x43004300u;
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) out[j] = (shift_to(w, 2 * j - 4) & 0x00300030u) | 0x43004300u;
    }
}

// codes of one 32-bit word -> floats in k order
template <int BITS>
__device__ __forceinline__ void codes_to_f32(uint32_t w, float* f) {
    if constexpr (BITS == 4) {
        const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            f[2 * b] = (float)((lo >> (8 * b)) & 0xFFu);
            f[2 * b + 1] = (float)((hi >> (8 * b)) & 0xFFu);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t m = (w >> (2 * j)) & 0x03030303u;
#pragma unroll
            for (int b = 0; b < 4; ++b) f[4 * b + j] = (float)((m >> (8 * b)) & 0xFFu);
        }
    }
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ int clamp_token(int t, int T) { return (t >= 0 && t < T) ? t : -1; }

// --------------------------------------------------------------- gate / up
// LDS: xs = bf16 activation pairs of the token tile, laid out
// [t][word][chunk][pair] so that consecutive lanes read consecutive 16 bytes,
// followed by xc = float32 chunk sums [t][chunk].
template <int BITS, int PT>
__global__ __launch_bounds__(256) void ffn_gateup_gemv_kernel(GemvParams p) {
    constexpr int CK = 128 / BITS;       // codes per 16-byte chunk (one lane load)
    constexpr int PPW = 16 / BITS;       // bf16 pairs per 32-bit code word
    extern __shared__ uint32_t smem[];
    const int H = p.H, I = p.I, NC = H / CK, NG = H / kGroup, NS = H / p.gs;
    const int P = p.T * p.k;
    uint32_t* xs = smem;
    float* xc = reinterpret_cast<float*>(smem + PT * (H / 2));

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int LG = p.LG, RPW = 64 / LG;
    const int rs = lane / LG, sub = lane % LG;
    const int IB = 8 * RPW;
    // codes are group-major: row r of expert e, group g at ((e NG + g) I + r) GB;
    // chunk c of a row (16 bytes) lies in group c / BITS
    constexpr int GB = kGroup * BITS / 8;
    const size_t gskip = (size_t)(I - 1) * GB;

    const int n_items = (*p.n_work) * p.items_per_expert;
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int wi = item / p.items_per_expert, ib = item % p.items_per_expert;
        const int32_t* ent = p.work + (size_t)wi * kWorkInts;
        const int e = ent[0], r0 = ent[1], cnt = ent[2];
        if (e < 0 || e >= p.E || cnt < 1 || cnt > kWorkRows || r0 < 0 || r0 + cnt > P) continue;
        const int i0 = ib * IB + (wv * RPW + rs) * 2;
        const bool v0 = i0 < I, v1 = i0 + 1 < I;
        const uint8_t* qrow[4];
        const uint16_t* srow[4];
        const uint16_t* brow[4];
        {
            const size_t ri0 = (size_t)e * I + (v0 ? i0 : 0), ri1 = (size_t)e * I + (v1 ? i0 + 1 : 0);
            const size_t ci0 = ((size_t)e * NG * I + (v0 ? i0 : 0)) * GB, ci1 = ((size_t)e * NG * I + (v1 ? i0 + 1 : 0)) * GB;
            qrow[0] = p.qa + ci0; srow[0] = p.sa + ri0 * NS; brow[0] = p.ba + ri0 * NS;
            qrow[1] = p.qa + ci1; srow[1] = p.sa + ri1 * NS; brow[1] = p.ba + ri1 * NS;
            qrow[2] = p.qb + ci0; srow[2] = p.sb + ri0 * NS; brow[2] = p.bb + ri0 * NS;
            qrow[3] = p.qb + ci1; srow[3] = p.sb + ri1 * NS; brow[3] = p.bb + ri1 * NS;
        }

        for (int tt = 0; tt < cnt; tt += PT) {
            const int np = min(PT, cnt - tt);
            __syncthreads();   // previous tile's readers are done with LDS
            // ---- stage the tile's activations as permuted bf16 pairs + chunk sums
            for (int idx = tid; idx < PT * NC; idx += blockDim.x) {
                const int t = idx / NC, c = idx % NC;
                uint32_t in[CK / 2];
                if (t < np) {
                    const int tk = clamp_token(ent[4 + tt + t], p.T);
                    const int tok = tk < 0 ? 0 : tk;
                    const uint4* src = reinterpret_cast<const uint4*>(p.x + (size_t)tok * H + c * CK);
#pragma unroll
                    for (int v = 0; v < CK / 8; ++v) {
                        uint4 q = tk < 0 ? make_uint4(0, 0, 0, 0) : src[v];
                        in[4 * v] = q.x; in[4 * v + 1] = q.y; in[4 * v + 2] = q.z; in[4 * v + 3] = q.w;
                    }
                } else {
#pragma unroll
                    for (int v = 0; v < CK / 2; ++v) in[v] = 0;
                }
                float sum = 0.f;
#pragma unroll
                for (int v = 0; v < CK / 2; ++v)
                    sum += bf16_bits_to_f32(in[v] & 0xFFFFu) + bf16_bits_to_f32(in[v] >> 16);
                // word w of the chunk holds codes [w*CK/4, (w+1)*CK/4); its pair j
                // pairs element j with element j + CK/8 of that range
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    uint32_t* dst = xs + ((size_t)(t * 4 + w) * NC + c) * PPW;
                    const uint32_t* src = in + w * (CK / 8);   // CK/4 elements = CK/8 words
#pragma unroll
                    for (int j = 0; j < PPW; ++j) {
                        // element j and j + PPW of this word's range
                        const uint32_t lo = (src[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
                        const uint32_t hi = (src[(j + PPW) >> 1] >> (16 * ((j + PPW) & 1))) & 0xFFFFu;
                        dst[j] = lo | (hi << 16);
                    }
                }
                xc[t * NC + c] = sum;
            }
            __syncthreads();

            float acc[4][PT];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int t = 0; t < PT; ++t) acc[r][t] = 0.f;

            for (int c = sub; c < NC; c += LG) {
                uint4 raw[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool ok = (r & 1) ? v1 : v0;
                    raw[r] = ok ? *reinterpret_cast<const uint4*>(qrow[r] + (size_t)c * 16 + (size_t)(c / BITS) * gskip)
                                : make_uint4(0, 0, 0, 0);
                }
                const int g = (c * CK) / p.gs;          // the chunk's scale group
                float sc[4], bc[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool ok = (r & 1) ? v1 : v0;
                    sc[r] = ok ? f16_bits_to_f32(srow[r][g]) : 0.f;
                    bc[r] = ok ? f16_bits_to_f32(brow[r][g]) : 0.f;
                    bc[r] = fmaf(-kOffset<BITS>, sc[r], bc[r]);
                    sc[r] *= kInvLever<BITS>;
                }
                float d[4][PT];
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int t = 0; t < PT; ++t) d[r][t] = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    uint32_t xp[PT][PPW];
#pragma unroll
                    for (int t = 0; t < PT; ++t) {
                        if (t < np) {
                            const uint32_t* src = xs + ((size_t)(t * 4 + w) * NC + c) * PPW;
#pragma unroll
                            for (int j = 0; j < PPW; j += 4) {
                                uint4 v = *reinterpret_cast<const uint4*>(src + j);
                                xp[t][j] = v.x; xp[t][j + 1] = v.y; xp[t][j + 2] = v.z; xp[t][j + 3] = v.w;
                            }
                        }
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const uint32_t word = (w == 0) ? raw[r].x : (w == 1) ? raw[r].y : (w == 2) ? raw[r].z : raw[r].w;
                        uint32_t qp[PPW];
                        codes_to_bf16_pairs<BITS>(word, qp);
#pragma unroll
                        for (int t = 0; t < PT; ++t) {
                            if (t < np) {
                                float s = d[r][t];
#pragma unroll
                                for (int j = 0; j < PPW; ++j) s = dot2_bf16(qp[j], xp[t][j], s);
                                d[r][t] = s;
                            }
                        }
                    }
                }
#pragma unroll
                for (int t = 0; t < PT; ++t) {
                    if (t < np) {
                        const float X = xc[t * NC + c];
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[r][t] = fmaf(sc[r], d[r][t], fmaf(bc[r], X, acc[r][t]));
                    }
                }
            }
            // ---- reduce across the LG lanes of the row group
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int t = 0; t < PT; ++t) acc[r][t] = wave_sum_xor(acc[r][t], LG);
            if (sub == 0) {
#pragma unroll
                for (int t = 0; t < PT; ++t) {
                    if (t < np) {
                        float* hrow = p.h + (size_t)(r0 + tt + t) * I;
#pragma unroll
                        for (int j = 0; j < 2; ++j) {
                            if (j == 0 ? v0 : v1) {
                                const float gt = acc[j][t], up = acc[2 + j][t];
                                hrow[i0 + j] = gt / (1.f + expf(-gt)) * up;
                            }
                        }
                    }
                }
            }
        }
    }
}

// ------------------------------------------------------------------- down
// LDS: hs = float32 activations of the token tile, [t][word][chunk][value],
// then hc = float32 chunk sums [t][chunk].
template <int BITS, int PT>
__global__ __launch_bounds__(256) void ffn_down_gemv_kernel(GemvParams p) {
    constexpr int CK = 128 / BITS;       // codes per 16-byte chunk
    constexpr int WC = 32 / BITS;        // codes per 32-bit word
    extern __shared__ uint32_t smem[];
    const int H = p.H, I = p.I, NC = I / CK, NG = I / kGroup, NS = I / p.gs;
    float* hs = reinterpret_cast<float*>(smem);
    float* hc = hs + PT * I;

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int LG = p.LG, RPW = 64 / LG;
    const int rs = lane / LG, sub = lane % LG;
    const int NB = 16 * RPW;                // rows per item
    // codes are group-major: row r of expert e, group g at ((e NG + g) H + r) GB;
    // chunk c of a row (16 bytes) lies in group c / BITS
    constexpr int GB = kGroup * BITS / 8;
    const size_t gskip = (size_t)(H - 1) * GB;

    const int P = p.T * p.k;
    const int n_items = (*p.n_work) * p.items_per_expert;
    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const int wi = item / p.items_per_expert, nb = item % p.items_per_expert;
        const int32_t* ent = p.work + (size_t)wi * kWorkInts;
        const int e = ent[0], r0 = ent[1], cnt = ent[2];
        if (e < 0 || e >= p.E || cnt < 1 || cnt > kWorkRows || r0 < 0 || r0 + cnt > P) continue;
        const int n0 = nb * NB + (wv * RPW + rs) * 4;
        const uint8_t* qrow[4];
        const uint16_t* srow[4];
        const uint16_t* brow[4];
        bool vr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            vr[r] = n0 + r < H;
            const size_t ri = (size_t)e * H + (vr[r] ? n0 + r : 0);
            qrow[r] = p.qa + ((size_t)e * NG * H + (vr[r] ? n0 + r : 0)) * GB;
            srow[r] = p.sa + ri * NS; brow[r] = p.ba + ri * NS;
        }

        for (int tt = 0; tt < cnt; tt += PT) {
            const int np = min(PT, cnt - tt);
            __syncthreads();
            for (int idx = tid; idx < PT * NC; idx += blockDim.x) {
                const int t = idx / NC, c = idx % NC;
                float v[CK];
                if (t < np) {
                    const float4* src = reinterpret_cast<const float4*>(p.h + (size_t)(r0 + tt + t) * I + c * CK);
#pragma unroll
                    for (int q = 0; q < CK / 4; ++q) {
                        float4 f = src[q];
                        v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < CK; ++q) v[q] = 0.f;
                }
                float sum = 0.f;
#pragma unroll
                for (int q = 0; q < CK; ++q) sum += v[q];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    float4* dst = reinterpret_cast<float4*>(hs + ((size_t)(t * 4 + w) * NC + c) * WC);
#pragma unroll
                    for (int q = 0; q < WC / 4; ++q)
                        dst[q] = make_float4(v[w * WC + 4 * q], v[w * WC + 4 * q + 1], v[w * WC + 4 * q + 2],
                                             v[w * WC + 4 * q + 3]);
                }
                hc[t * NC + c] = sum;
            }
            __syncthreads();

            float acc[4][PT];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int t = 0; t < PT; ++t) acc[r][t] = 0.f;

            for (int c = sub; c < NC; c += LG) {
                uint4 raw[4];
                float sc[4], bc[4];
                const int g = (c * CK) / p.gs;          // the chunk's scale group
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    raw[r] = vr[r] ? *reinterpret_cast<const uint4*>(qrow[r] + (size_t)c * 16 + (size_t)(c / BITS) * gskip)
                                   : make_uint4(0, 0, 0, 0);
                    sc[r] = vr[r] ? f16_bits_to_f32(srow[r][g]) : 0.f;
                    bc[r] = vr[r] ? f16_bits_to_f32(brow[r][g]) : 0.f;
                }
                float d[4][PT];
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int t = 0; t < PT; ++t) d[r][t] = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    float hv[PT][WC];
#pragma unroll
                    for (int t = 0; t < PT; ++t) {
                        if (t < np) {
                            const float4* src = reinterpret_cast<const float4*>(hs + ((size_t)(t * 4 + w) * NC + c) * WC);
#pragma unroll
                            for (int q = 0; q < WC / 4; ++q) {
                                float4 f = src[q];
                                hv[t][4 * q] = f.x; hv[t][4 * q + 1] = f.y; hv[t][4 * q + 2] = f.z; hv[t][4 * q + 3] = f.w;
                            }
                        }
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const uint32_t word = (w == 0) ? raw[r].x : (w == 1) ? raw[r].y : (w == 2) ? raw[r].z : raw[r].w;
                        float qf[WC];
                        codes_to_f32<BITS>(word, qf);
#pragma unroll
                        for (int t = 0; t < PT; ++t) {
                            if (t < np) {
                                float s = d[r][t];
#pragma unroll
                                for (int j = 0; j < WC; ++j) s = fmaf(qf[j], hv[t][j], s);
                                d[r][t] = s;
                            }
                        }
                    }
                }
#pragma unroll
                for (int t = 0; t < PT; ++t) {
                    if (t < np) {
                        const float X = hc[t * NC + c];
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[r][t] = fmaf(sc[r], d[r][t], fmaf(bc[r], X, acc[r][t]));
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int t = 0; t < PT; ++t) acc[r][t] = wave_sum_xor(acc[r][t], LG);
            if (sub == 0) {
#pragma unroll
                for (int t = 0; t < PT; ++t) {
                    if (t < np) {
                        uint16_t* yrow = p.y + (size_t)(r0 + tt + t) * H;
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (vr[r]) yrow[n0 + r] = (uint16_t)f32_to_bf16_bits(acc[r][t]);
                    }
                }
            }
        }
    }
}

// ------------------------------------------------------------------ launch

static int lanes_per_row(int chunks) {
    int lg = 64;
    while (lg > 1 && (chunks % lg) != 0) lg >>= 1;
    return lg;
}

template <int BITS>
static GemvParams base_params(const FfnArgs& a) {
    const moe_dims& d = a.d;
    GemvParams p{};
    p.x = a.x; p.work = a.work; p.n_work = a.n_work; p.h = a.h; p.y = a.y;
    p.T = d.T; p.H = d.H; p.I = d.I; p.k = d.k; p.E = d.E;
    p.gs = d.group_size;
    return p;
}

static int grid_for(const moe_dims& d, int items_per_expert) {
    const long max_items = work_capacity(d) * items_per_expert;
    return (int)(max_items < 4096 ? max_items : 4096);
}

template <int BITS>
static int launch_gateup_bits(const FfnArgs& a, hipStream_t s) {
    const moe_dims& d = a.d;
    if (d.T * d.k == 0) return MOE_OK;
    constexpr int CK = 128 / BITS;
    if (d.group_size < CK) return MOE_ERR_UNSUPPORTED;     // one scale per 16-byte chunk
    GemvParams p = base_params<BITS>(a);
    p.qa = a.w.q[0]; p.sa = a.w.scale[0]; p.ba = a.w.bias[0];
    p.qb = a.w.q[1]; p.sb = a.w.scale[1]; p.bb = a.w.bias[1];
    const int NC = d.H / CK;
    p.LG = lanes_per_row(NC);
    const int IB = 8 * (64 / p.LG);
    p.items_per_expert = (d.I + IB - 1) / IB;
    const int grid = grid_for(d, p.items_per_expert);
    const int PT = (d.H <= 6144) ? 4 : 2;
    const size_t lds = (size_t)PT * (d.H / 2) * 4 + (size_t)PT * NC * 4;
    if (PT == 4)
        hipLaunchKernelGGL((ffn_gateup_gemv_kernel<BITS, 4>), dim3(grid), dim3(256), lds, s, p);
    else
        hipLaunchKernelGGL((ffn_gateup_gemv_kernel<BITS, 2>), dim3(grid), dim3(256), lds, s, p);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

template <int BITS>
static int launch_down_bits(const FfnArgs& a, hipStream_t s) {
    const moe_dims& d = a.d;
    if (d.T * d.k == 0) return MOE_OK;
    constexpr int CK = 128 / BITS;
    if (d.group_size < CK) return MOE_ERR_UNSUPPORTED;     // one scale per 16-byte chunk
    GemvParams p = base_params<BITS>(a);
    p.qa = a.w.q[2]; p.sa = a.w.scale[2]; p.ba = a.w.bias[2];
    const int NC = d.I / CK;
    p.LG = lanes_per_row(NC);
    const int NB = 16 * (64 / p.LG);
    p.items_per_expert = (d.H + NB - 1) / NB;
    const int grid = grid_for(d, p.items_per_expert);
    const int PT = (d.I <= 3840) ? 4 : (d.I <= 7680 ? 2 : 1);
    const size_t lds = (size_t)PT * d.I * 4 + (size_t)PT * NC * 4;
    if (PT == 4)
        hipLaunchKernelGGL((ffn_down_gemv_kernel<BITS, 4>), dim3(grid), dim3(256), lds, s, p);
    else if (PT == 2)
        hipLaunchKernelGGL((ffn_down_gemv_kernel<BITS, 2>), dim3(grid), dim3(256), lds, s, p);
    else
        hipLaunchKernelGGL((ffn_down_gemv_kernel<BITS, 1>), dim3(grid), dim3(256), lds, s, p);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

size_t gemv_workspace_bytes(const moe_dims& d) {
    const size_t h = (size_t)d.T * d.k * d.I * sizeof(float);
    return (h + 255) & ~(size_t)255;
}

// MOE_ALGO_AUTO -> the matrix-core path (its cost per weight does not grow with
// the tokens an expert serves); explicit choices are kept.
// AUTO: the grouped GEMM once experts average at least 64 tokens (a weight
// tile then meets most of a 128-token item), else the per-tile matrix-core
// path; groups of 64 or 32 whose decode tiles do not fit LDS take the
// vector-ALU path.
int resolve_algo(const moe_dims& d, int bits, int algo) {
    if (algo != MOE_ALGO_AUTO) return algo;
    const long P = (long)d.T * d.k;
    if (gemm_supported(d, bits) && P >= 64L * d.E) return MOE_ALGO_GEMM;
    if (d.group_size < kGroup && !(dec_gateup_fits(d) && dec_down_fits(d)))
        return MOE_ALGO_GEMV;
    return MOE_ALGO_MFMA;
}

// Groups of 64 or 32: the decode kernels take them (matrix cores, tiles that
// fit LDS), the grouped GEMM, and the vector-ALU kernels where one scale covers
// a 16-byte chunk of codes (32 codes at 4 bits, 64 at 2 bits); the persistent
// and streaming kernels take groups of 128 only.
bool ffn_group_supported(const moe_dims& d, int bits, int algo) {
    if (d.group_size == kGroup) return true;
    switch (resolve_algo(d, bits, algo)) {
        case MOE_ALGO_GEMV: return d.group_size >= 128 / bits;
        case MOE_ALGO_GEMM: return gemm_supported(d, bits);
        default: return dec_gateup_fits(d) && dec_down_fits(d);
    }
}

size_t ffn_workspace_bytes(const moe_dims& d, int bits, int algo) {
    switch (resolve_algo(d, bits, algo)) {
        case MOE_ALGO_GEMV: return gemv_workspace_bytes(d);
        case MOE_ALGO_GEMM: return gemm_workspace_bytes(d);
        default: return mfma_workspace_bytes(d);
    }
}

int launch_gateup_gemv(const FfnArgs& a, hipStream_t s) {
    return a.bits == 4 ? launch_gateup_bits<4>(a, s) : launch_gateup_bits<2>(a, s);
}

int launch_down_gemv(const FfnArgs& a, hipStream_t s) {
    return a.bits == 4 ? launch_down_bits<4>(a, s) : launch_down_bits<2>(a, s);
}

}  // namespace moe
