// Matrix-core building blocks shared by the FFN kernels (v_mfma_f32_16x16x32_bf16).
//
// Lane layout of the instruction (checked on gfx950): A operand, lane l holds
// row l % 16 and k = 8 (l / 16) + i; B operand, column l % 16 and the same k;
// D, rows 4 (l / 16) + i of column l % 16.
//
// Exact code operands: a code q becomes the bf16 value 128 + L q (q OR-ed
// into the mantissa of 0x4300; L = kLever: 8 for 4-bit, 16 for 2-bit codes),
// so products with bf16 activations are exact and the matrix core accumulates
// in float32.  Per group of 128 along K the accumulator C = sum (128 + L q) x
// folds into the output as (s / L) C + (b - (128 / L) s) X with X = sum x,
// which is sum (q s + b) x: the FMA form of the Flash-MoE page, sec. 2, taken
// per group instead of per element.
#pragma once

#include "common.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4_t mfma16(const uint32_t (&a)[4], const uint32_t (&b)[4], floatx4_t c) {
    const bf16x8_t A = __builtin_bit_cast(bf16x8_t, a);
    const bf16x8_t B = __builtin_bit_cast(bf16x8_t, b);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, c, 0, 0, 0);
}

// A operand of MFMA step s for one group: the lane's codes (4-bit: 4 words,
// 2-bit: 2 words) -> 4 packed pairs of bf16 128 + L q (see kLever).  Pair i of
// a word holds codes (i, i + W/2) of that word (W codes per word).
// A constant the optimiser cannot see through, held in a VGPR (the empty
// statement emits no instruction).
__device__ __forceinline__ uint32_t vreg_const(uint32_t v) {
    asm("" : "+v"(v));
    return v;
}

// (x & m) | c in one v_and_or_b32.  gfx9 VOP3 takes no literal and reads at
// most one scalar operand, so with both constants visible the compiler emits
// a separate AND and OR; with m and c opaque VGPR values it selects the one
// instruction.  Written in plain C on purpose: the compiler then knows it is a
// VALU write and keeps the wait states the matrix core needs before reading
// the result (an instruction hidden in inline assembly gets none).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) { return (x & m) | c; }

template <int BITS>
__device__ __forceinline__ void code_operand(const uint32_t* w, int s, uint32_t (&out)[4]) {
    const uint32_t hi = vreg_const(0x43004300u);
    if constexpr (BITS == 4) {
        const uint32_t v = w[s], m = vreg_const(0x00780078u);            // L = 8: bits 3-6
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = and_or(shift_to(v, 4 * i - 3), m, hi);
    } else {
        const uint32_t v = w[s >> 1], m = vreg_const(0x00300030u);       // L = 16: bits 4-5
        const int base = 4 * (s & 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = and_or(shift_to(v, 2 * (base + i) - 4), m, hi);
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

// h = hi + mid + lo exactly (each difference below is exact in float32).
// Contraction is off: otherwise the compiler may fuse the multiply that made h
// into h - hi, splitting the unrounded product instead, and then two kernels
// that compute the same h would store different planes.
__device__ __forceinline__ void split3_bf16(float h, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
#pragma clang fp contract(off)
    hi = f32_to_bf16_bits(h);
    const float r1 = h - bf16_bits_to_f32(hi);
    mid = f32_to_bf16_bits(r1);
    const float r2 = r1 - bf16_bits_to_f32(mid);
    lo = f32_to_bf16_bits(r2);
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

// ---------------------------------------------- integer matrix cores
// Codes of MFMA step st (16 of the lane's 32 codes of a group) as bytes: 4-bit,
// dword d holds nibbles (d & 1) + 2 b of word 2 st + d / 2; 2-bit, dword t holds
// crumbs t + 4 b of word st (b: byte in the dword).
template <int BITS>
__device__ __forceinline__ void i8_code_operand(const uint32_t* w, int st, uint32_t (&out)[4]) {
    if constexpr (BITS == 4) {
        const uint32_t a = w[2 * st], b = w[2 * st + 1], M = 0x0F0F0F0Fu;
        out[0] = a & M; out[1] = (a >> 4) & M;
        out[2] = b & M; out[3] = (b >> 4) & M;
    } else {
        const uint32_t a = w[st], M = 0x03030303u;
        out[0] = a & M; out[1] = (a >> 2) & M; out[2] = (a >> 4) & M; out[3] = (a >> 6) & M;
    }
}

typedef int int32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int32x4_t mfma_i8(const uint32_t (&a)[4], const uint32_t (&b)[4], int32x4_t c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(int32x4_t, a), __builtin_bit_cast(int32x4_t, b),
                                                 c, 0, 0, 0);
}

// A wave-uniform global pointer, passed through readfirstlane so that the
// compiler keeps it whole: a load at uniform_gptr(base) + (32-bit lane offset)
// then takes the scalar-base form (base in SGPRs, offset in one VGPR) instead
// of 64-bit per-lane address arithmetic.
typedef const __attribute__((address_space(1))) uint8_t* gbytes_t;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) u32x4_t* gu32x4_t;
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(1))) u32x2_t* gu32x2_t;

__device__ __forceinline__ gbytes_t uniform_gptr(const uint8_t* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<gbytes_t>(((uint64_t)hi << 32) | lo);
}

// ------------------------------------------------- direct-to-LDS staging

constexpr int kDma = 1024;          // bytes one wave moves with one direct-to-LDS load

typedef const __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// One direct-to-LDS load of the wave: lane l copies 16 bytes from `src` to
// lds_base + 16 l (lds_base must be the same in every lane).  Written as
// inline assembly so that the compiler does not track it: its own tracking
// waits for every outstanding load (the code ring too) before the first LDS
// access after it; completion is waited for explicitly with wait_vmem.
// M0 holds the LDS address; one wait state between writing M0 and the load.
// COH: a device-scope load (sc1), for data that other workgroups of the same
// launch wrote with device-scope stores.
template <bool COH = false>
__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
    const uint32_t lds = (uint32_t)(uintptr_t)(lptr_t)lds_base;
    if constexpr (COH)
        asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off sc1" : : "v"(src), "{m0}"(lds) : "memory");
    else
        asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "{m0}"(lds) : "memory");
}

// The same load addressed as a wave-uniform 64-bit base (scalar registers)
// plus a 32-bit per-lane byte offset, so that moving the base along K costs
// scalar instructions only.  A vector-memory instruction that reads an SGPR a
// VALU instruction wrote (v_readlane, v_readfirstlane: the compiler restores
// spilled scalars that way) needs 5 wait states in between, and the
// compiler's hazard checks do not look inside inline assembly: s_nop 5
// provides 6 (and the one M0 needs).
__device__ __forceinline__ void dma16_sv(const void* sbase, uint32_t voff, void* lds_base) {
    const uint32_t lds = (uint32_t)(uintptr_t)(lptr_t)lds_base;
    asm volatile("s_nop 5\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}

// Copy `bytes` (a multiple of 16) of contiguous global memory to LDS, waves
// taking 1 KB pieces in turn; lanes past the end reload the last 16 bytes into
// the padding (the LDS region is rounded up to a whole piece).
__device__ __forceinline__ void dma_copy(const uint8_t* src, uint8_t* dst, int bytes, int wid, int lane) {
    const int pieces = (bytes + kDma - 1) / kDma;
    for (int i = wid; i < pieces; i += 4) {
        const int off = i * kDma + 16 * lane;
        dma16(src + (off < bytes ? off : bytes - 16), dst + i * kDma);
    }
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt bits 3:0 and 15:14; expcnt and lgkmcnt off).
template <int N>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier that orders LDS only: global loads stay in flight (a plain
// __syncthreads() waits for every outstanding load, the code ring included).
// Direct-to-LDS data must be waited for with wait_vmem first.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Groups of 64 or 32 (SPG = 2 or 4 scale groups per 128 codes).  In the
// natural operand order, lane quarter q holds the 32 codes k = 32 q .. +31
// of a 128-code run and MFMA step st takes 8 of them from every quarter, so a
// step mixes all four quarters.  For finer groups the roles of q and st are
// swapped: lane quarter q at step st supplies what quarter st supplies at step
// q in the natural order (codes: one 32-bit word per step, from quarter st's
// bytes; activations: chunk 4 st + q of the pair-ordered row instead of
// 4 q + st), so step st covers exactly quarter st, i.e. k = 32 st .. +31, and
// a group of 32 is one step, a group of 64 two.  The products and their pair
// order are unchanged; only which step carries them moves.
// Byte offset of the word lane quarter q loads for step st, within a row's
// run of 128 codes.
template <int BITS>
__device__ __forceinline__ int tr_word_offset(int st, int q) {
    return BITS == 4 ? 16 * st + 4 * q : 8 * st + 4 * (q >> 1);
}

// B operand of step st in the swapped order from the step's word w[st].
template <int BITS>
__device__ __forceinline__ void code_operand_tr(const uint32_t* w, int st, int q, uint32_t (&out)[4]) {
    if constexpr (BITS == 4) {
        code_operand<4>(w, st, out);
    } else {
        const uint32_t v[2] = {w[st] >> (8 * (q & 1)), 0u};   // 2-bit: quarter st's half word for step q
        code_operand<2>(v, 0, out);
    }
}

}  // namespace moe
