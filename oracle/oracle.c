/*
 * CPU oracle for the routed MoE decode layer -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the bench's CPU-baseline leg may load
 * this library.  The product path (the HIP library) never calls it.
 *
 * Plain, single-threaded C99.  Sums run in double in ascending index order and
 * are rounded once at the points the layer defines; no blocking, no fusion.
 * It shares no code, header or table with the HIP implementation.
 *
 * Steps and the passages they follow (pages are cited by title):
 *   decode of codes       "Flash-MoE ... (translation)" sec. 2, FMA-optimised
 *                         dequant: weight = nibble * scale + bias;
 *                         "Strata" page sec. 2.2: groups of 128 weights share
 *                         one scale/offset pair; finer groups: "Strata" page
 *                         sec. 4.4 (64 for quality), the laptop page sec. 4.2
 *                         (32 weights per scale and zero point).
 *   router logits         "12GB card runs a 68GB model (Betelgeuse)", MoE
 *                         primer: the router scores every expert from the
 *                         token's hidden state.
 *   top-k + gates         same primer: only the k best-scoring experts run;
 *                         softmax gates renormalised over the k picked.
 *   slot lookup           Betelgeuse page, "in-stream GPU doorbell": hits are
 *                         resolved on the device, the host is told only about
 *                         misses; "Luce Spark" page, hot/warm/cold tiers.
 *   permutation           "Strata" page sec. 2.3: tokens that picked the same
 *                         expert share one fetch of its weights.
 *   expert FFN            Flash-MoE page sec. 3: fused SwiGLU between the
 *                         gate/up and down matvecs.
 *   combine               Flash-MoE page sec. 3: MoE combine + residual.
 *   shared expert         Flash-MoE page sec. 3: combine + residual + sigmoid
 *                         gate in one kernel (the gate read as that of an
 *                         always-on shared expert).
 *   zero-point adapter    "Strata" page sec. 2.2 and the laptop page sec. 4.2:
 *                         (q - zero) scale groups, as bias = -zero scale.
 *
 * Parity status of every function is recorded in the test suite that pins
 * it; none is unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ---------------------------------------------------------------- formats */

float orc_bf16_to_f32(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* float -> bf16, round to nearest, ties to even; NaN -> 0x7FC0 */
uint16_t orc_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if (isnan(f)) return 0x7FC0;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* double -> bf16, one rounding (nearest, ties to even).  bf16 keeps 8
 * significant bits and the float exponent range. */
uint16_t orc_f64_to_bf16(double d) {
    if (isnan(d)) return 0x7FC0;
    double a = fabs(d);
    double r;
    if (a == 0.0 || isinf(d)) {
        r = d;
    } else if (a < ldexp(1.0, -126)) {
        /* subnormal range: spacing 2^-133 */
        r = nearbyint(d * ldexp(1.0, 133)) * ldexp(1.0, -133);
    } else {
        int e;
        double m = frexp(d, &e);          /* |m| in [0.5, 1) */
        r = ldexp(nearbyint(ldexp(m, 8)), e - 8);
    }
    /* r has at most 8 significant bits; beyond the float range it is inf */
    float f = (float)r;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

/* double -> IEEE binary16, one rounding (nearest, ties to even).  binary16
 * keeps 11 significant bits from 2^-14 up, a fixed spacing of 2^-24 below it,
 * and its largest finite value is 65504: anything that rounds past it is an
 * infinity.  NaN -> 0x7E00. */
uint16_t orc_f64_to_f16(double d) {
    const uint16_t sign = signbit(d) ? 0x8000u : 0u;
    if (isnan(d)) return 0x7E00u;
    const double a = fabs(d);
    if (isinf(a)) return (uint16_t)(sign | 0x7C00u);
    if (a < ldexp(1.0, -14)) {
        /* units of 2^-24; 1024 units is the smallest normal, whose bits are 0x0400 */
        return (uint16_t)(sign | (uint16_t)nearbyint(a * ldexp(1.0, 24)));
    }
    int e;
    const double m = frexp(a, &e);               /* a = m 2^e, m in [0.5, 1) */
    double r = nearbyint(ldexp(m, 11));          /* a ~ (r / 1024) 2^(e-1), r in [1024, 2048] */
    if (r == 2048.0) {
        r = 1024.0;
        e += 1;
    }
    const int ex = e - 1 + 15;                   /* biased exponent, >= 1 here */
    if (ex >= 31) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (uint16_t)(ex << 10) | (uint16_t)((int)r - 1024));
}

/* IEEE binary16 -> float, exact for normals, subnormals, inf and NaN */
float orc_f16_to_f32(uint16_t h) {
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1F;
    int man = h & 0x3FF;
    double v;
    if (ex == 0) {
        v = ldexp((double)man, -24);                  /* 0 or subnormal */
    } else if (ex == 31) {
        v = man ? NAN : INFINITY;
    } else {
        v = ldexp((double)(man | 0x400), ex - 25);
    }
    return (float)(sign ? -v : v);
}

/* Zero-point groups, w = (q - z) s (the "Strata" page, sec. 2.2: each group of
 * 128 weights shares one scale and one zero point; the laptop page, sec. 4.2,
 * the same form over groups of 32), written in this format's w = q s + b:
 * b = -(z s), rounded once to fp16.  One entry per (row, group). */
void orc_zero_point_bias(int64_t n, const uint16_t* scale, const uint8_t* zeros, uint16_t* bias) {
    for (int64_t i = 0; i < n; ++i)
        bias[i] = orc_f64_to_f16(-((double)zeros[i] * (double)orc_f16_to_f32(scale[i])));
}

/* Code of element k in a packed row: bits = 4 (low nibble = even k) or
 * 2 (bits 2j..2j+1 of a byte hold k % 4 == j). */
int orc_code(const uint8_t* row, int k, int bits) {
    if (bits == 4) return (row[k >> 1] >> (4 * (k & 1))) & 0xF;
    return (row[k >> 2] >> (2 * (k & 3))) & 0x3;
}

/* Dequantised weight (exact in double): code * scale + bias of k's group, the
 * group being `group` consecutive k (32, 64 or 128). */
double orc_weight(const uint8_t* qrow, const uint16_t* srow, const uint16_t* brow, int k, int bits, int group) {
    int g = k / group;
    return (double)orc_code(qrow, k, bits) * (double)orc_f16_to_f32(srow[g])
         + (double)orc_f16_to_f32(brow[g]);
}

/* Dequantise rows [N, K] into a dense double matrix (test helper). */
void orc_dequant_matrix(int N, int K, int bits, int group, const uint8_t* q, const uint16_t* s,
                        const uint16_t* b, double* out) {
    size_t rowb = (size_t)K * bits / 8, ng = (size_t)K / group;
    for (int n = 0; n < N; ++n)
        for (int k = 0; k < K; ++k)
            out[(size_t)n * K + k] =
                orc_weight(q + (size_t)n * rowb, s + (size_t)n * ng, b + (size_t)n * ng, k, bits, group);
}

/* ---------------------------------------------------------- router logits */

/* L[t,e] = sum_h x[t,h] * Wr[e,h] (+ bias[e]); double sum, one rounding. */
void orc_router_logits(int T, int H, int E, const uint16_t* x, const float* Wr,
                       const float* bias, float* logits) {
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h)
                acc += (double)orc_bf16_to_f32(x[(size_t)t * H + h]) * (double)Wr[(size_t)e * H + h];
            if (bias) acc += (double)bias[e];
            logits[(size_t)t * E + e] = (float)acc;
        }
}

/* -------------------------------------------------------- top-k and gates */

/* 1 if (va, ia) ranks before (vb, ib): larger value first, equal values
 * (including -0 == +0) by lower id, NaN below every number. */
static int orc_before(float va, int ia, float vb, int ib) {
    int na = isnan(va), nb = isnan(vb);
    if (na != nb) return nb;              /* the non-NaN one wins */
    if (!na && va != vb) return va > vb;
    return ia < ib;
}

void orc_topk(int T, int E, int k, const float* logits, int renormalize,
              int32_t* ids, float* gates) {
    for (int t = 0; t < T; ++t) {
        const float* L = logits + (size_t)t * E;
        int32_t* out = ids + (size_t)t * k;
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                int taken = 0;
                for (int jj = 0; jj < j; ++jj) taken |= (out[jj] == e);
                if (taken) continue;
                if (best < 0 || orc_before(L[e], e, L[best], best)) best = e;
            }
            out[j] = best;
        }
        double top = (double)L[out[0]];
        double den = 0.0;
        if (renormalize) {
            for (int j = 0; j < k; ++j) den += exp((double)L[out[j]] - top);
        } else {
            for (int e = 0; e < E; ++e) den += exp((double)L[e] - top);
        }
        for (int j = 0; j < k; ++j)
            gates[(size_t)t * k + j] = (float)(exp((double)L[out[j]] - top) / den);
    }
}

/* ------------------------------------------------------------ slot lookup */

/* pair_slot[p] = slot of the pair's expert, or -1 when the expert has no
 * valid slot (slot < 0 or >= n_slots).  miss = ascending distinct experts
 * with pair_slot == -1.  last_use[slot] = step for every hit (if given).
 * *doorbell = n_miss when n_miss > 0 (if given); untouched otherwise. */
int orc_slot_lookup(int P, int E, int n_slots, const int32_t* ids, const int32_t* slot_of_expert,
                    int32_t* pair_slot, int32_t* miss, int32_t* n_miss,
                    uint32_t* last_use, uint32_t step, int32_t* doorbell) {
    int nm = 0;
    for (int e = 0; e < E; ++e) {
        int missed = 0;
        for (int p = 0; p < P; ++p) {
            if (ids[p] != e) continue;
            int s = slot_of_expert[e];
            int valid = (s >= 0 && s < n_slots);
            pair_slot[p] = valid ? s : -1;
            if (!valid) missed = 1;
            else if (last_use) last_use[s] = step;
        }
        if (missed) miss[nm++] = e;
    }
    *n_miss = nm;
    if (doorbell && nm > 0) *doorbell = nm;
    return nm;
}

/* ------------------------------------------------------------ permutation */

/* Stable grouping of pairs p = t*k + j by expert. */
void orc_permute(int P, int E, const int32_t* ids, int32_t* counts, int32_t* offsets,
                 int32_t* sorted_pairs, int32_t* pair_to_row, int32_t* active, int32_t* n_active) {
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int p = 0; p < P; ++p) counts[ids[p]] += 1;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int r = 0, na = 0;
    for (int e = 0; e < E; ++e) {
        if (counts[e] > 0) active[na++] = e;
        for (int p = 0; p < P; ++p)
            if (ids[p] == e) {
                sorted_pairs[r] = p;
                pair_to_row[p] = r;
                ++r;
            }
    }
    *n_active = na;
}

/* ------------------------------------------------------------- expert FFN */

/* One routed row: the expert FFN applied to one token.
 *   a_i = sum_k Wg[i,k] x_k,  u_i = sum_k Wu[i,k] x_k      (double, -> float)
 *   h_i = silu(a_i) * u_i,  silu(z) = z / (1 + e^-z)        (double, -> float)
 *   y_n = sum_i Wd[n,i] h_i                                 (double, -> bf16)
 * Weights: gate/up rows [I][H*bits/8] with scale/bias [I][H/group]; down rows
 * [H][I*bits/8] with scale/bias [H][I/group].
 * n_idx == NULL: y_out[n] for every n < H.  Otherwise y_out[j] holds output
 * n_idx[j] for j < n_count (a sample of the row's outputs). */
void orc_expert_ffn_row(int H, int I, int bits, int group, const uint16_t* x,
                        const uint8_t* qg, const uint16_t* sg, const uint16_t* bg,
                        const uint8_t* qu, const uint16_t* su, const uint16_t* bu,
                        const uint8_t* qd, const uint16_t* sd, const uint16_t* bd,
                        int n_count, const int32_t* n_idx,
                        float* h_out, uint16_t* y_out) {
    size_t rowH = (size_t)H * bits / 8, ngH = (size_t)H / group;
    size_t rowI = (size_t)I * bits / 8, ngI = (size_t)I / group;
    for (int i = 0; i < I; ++i) {
        double a = 0.0, u = 0.0;
        for (int kk = 0; kk < H; ++kk) {
            double xv = (double)orc_bf16_to_f32(x[kk]);
            a += orc_weight(qg + (size_t)i * rowH, sg + (size_t)i * ngH, bg + (size_t)i * ngH, kk, bits, group) * xv;
            u += orc_weight(qu + (size_t)i * rowH, su + (size_t)i * ngH, bu + (size_t)i * ngH, kk, bits, group) * xv;
        }
        double af = (double)(float)a, uf = (double)(float)u;
        double silu = af / (1.0 + exp(-af));
        h_out[i] = (float)(silu * uf);
    }
    int count = n_idx ? n_count : H;
    for (int j = 0; j < count; ++j) {
        int n = n_idx ? n_idx[j] : j;
        double y = 0.0;
        for (int i = 0; i < I; ++i)
            y += orc_weight(qd + (size_t)n * rowI, sd + (size_t)n * ngI, bd + (size_t)n * ngI, i, bits, group)
               * (double)h_out[i];
        y_out[j] = orc_f64_to_bf16(y);
    }
}

/* ---------------------------------------------------------------- combine */

/* out[t,n] = residual[t,n] + sum_j g[t,j] * Y[row(t,j), n], accumulated in
 * float in j order with fused multiply-adds, then rounded to bf16. */
/* Shared-expert gate (Flash-MoE page, sec. 3: the combine kernel also applies
 * a sigmoid gate; read here as the gate of an always-on shared expert):
 * gate[t] = 1 / (1 + exp(-L)), L = sum_h x[t][h] w[h] in double, rounded once. */
void orc_shared_gate(int T, int H, const uint16_t* x, const float* w, float* gate) {
    for (int t = 0; t < T; ++t) {
        double L = 0.0;
        for (int h = 0; h < H; ++h) L += (double)orc_bf16_to_f32(x[(size_t)t * H + h]) * (double)w[h];
        gate[t] = (float)(1.0 / (1.0 + exp(-L)));
    }
}

/* Combine with a shared expert: the routed chain of orc_combine, then one more
 * float32 fused multiply-add of the shared row, rounded once to bf16:
 *   acc = fmaf(sgate[t], y_shared[t][n], acc). */
void orc_combine_shared(int T, int H, int k, const uint16_t* y_rows, const int32_t* pair_to_row,
                        const float* gates, const uint16_t* y_shared, const float* sgate,
                        const uint16_t* residual, uint16_t* out) {
    for (int t = 0; t < T; ++t)
        for (int n = 0; n < H; ++n) {
            float acc = orc_bf16_to_f32(residual[(size_t)t * H + n]);
            for (int j = 0; j < k; ++j) {
                int row = pair_to_row[(size_t)t * k + j];
                acc = fmaf(gates[(size_t)t * k + j], orc_bf16_to_f32(y_rows[(size_t)row * H + n]), acc);
            }
            acc = fmaf(sgate[t], orc_bf16_to_f32(y_shared[(size_t)t * H + n]), acc);
            out[(size_t)t * H + n] = orc_f32_to_bf16(acc);
        }
}

void orc_combine(int T, int H, int k, const uint16_t* y_rows, const int32_t* pair_to_row,
                 const float* gates, const uint16_t* residual, uint16_t* out) {
    for (int t = 0; t < T; ++t)
        for (int n = 0; n < H; ++n) {
            float acc = orc_bf16_to_f32(residual[(size_t)t * H + n]);
            for (int j = 0; j < k; ++j) {
                int row = pair_to_row[(size_t)t * k + j];
                acc = fmaf(gates[(size_t)t * k + j], orc_bf16_to_f32(y_rows[(size_t)row * H + n]), acc);
            }
            out[(size_t)t * H + n] = orc_f32_to_bf16(acc);
        }
}

/* ---------------------------------------------------------- residency tiers */
/* "Luce Spark" page, sec. 1 (calibrated placement: count how often traffic
 * routes to each expert, keep the most used set resident, "hot") and sec. 2
 * (a bounded ring of spare slots: a routed expert that is not resident is
 * copied from pinned host memory into a spare slot, the least recently used
 * entry making room when the ring is full; tiers hot / warm / cold). */

/* Routing-frequency counters: freq[e] += counts[e] (counts = pairs routed to
 * expert e in one call, as orc_permute gives them). */
void orc_freq_update(int E, const int32_t* counts, uint32_t* freq) {
    for (int e = 0; e < E; ++e) freq[e] += (uint32_t)counts[e];
}

/* Calibrated hot set: the n experts with the highest counts, most used first,
 * equal counts to the lower expert id. */
void orc_hot_set(int E, const uint32_t* freq, int n, int32_t* hot) {
    for (int j = 0; j < n; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            int taken = 0;
            for (int jj = 0; jj < j; ++jj) taken |= (hot[jj] == e);
            if (taken) continue;
            if (best < 0 || freq[e] > freq[best]) best = e;     /* ascending e: ties keep the lower id */
        }
        hot[j] = best;
    }
}

/* One step of the warm ring.  Slots [0, n_hot) hold the hot set and are never
 * evicted; slots [n_hot, n_slots) are the ring.  last_use[s] is the step a
 * slot was last used (0 = never; steps count from 1); slots already used in
 * this step carry last_use == step.  For each missing expert, in ascending
 * id order (miss[0..n_miss)), the ring slot with the oldest last_use, ties to
 * the lowest slot, among those not used in this step, takes it: the slot's
 * previous expert (if any) stops being resident, the new one becomes
 * resident there, the slot is stamped with this step, and (expert, slot) is
 * listed as a copy to make.  A missing expert that finds no such slot stays
 * cold for this step.  Returns the number of copies. */
int orc_warm_ring_step(int n_hot, int n_slots, const int32_t* miss, int n_miss, uint32_t step,
                       int32_t* slot_of_expert, int32_t* expert_of_slot, uint32_t* last_use,
                       int32_t* copy_expert, int32_t* copy_slot) {
    int n_copy = 0;
    for (int i = 0; i < n_miss; ++i) {
        const int e = miss[i];
        int victim = -1;
        for (int s = n_hot; s < n_slots; ++s) {
            if (last_use[s] == step) continue;
            if (victim < 0 || last_use[s] < last_use[victim]) victim = s;   /* ascending s: ties keep the lower slot */
        }
        if (victim < 0) continue;
        const int old = expert_of_slot[victim];
        if (old >= 0) slot_of_expert[old] = -1;
        expert_of_slot[victim] = e;
        slot_of_expert[e] = victim;
        last_use[victim] = step;
        copy_expert[n_copy] = e;
        copy_slot[n_copy] = victim;
        ++n_copy;
    }
    return n_copy;
}
