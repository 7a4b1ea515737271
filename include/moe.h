/*
 * moe.h -- C ABI of libmoe.so: the routed mixture-of-experts layer at decode
 * time on one AMD Instinct MI355X (gfx950).
 *
 * One call per step of the layer.  For T tokens of hidden size H the layer
 *   1. scores every expert with a linear router             (moe_route_topk)
 *   2. keeps the k best experts per token, softmax gates     (moe_route_topk /
 *      renormalised over the k picked                          moe_topk_from_logits)
 *   3. looks up each picked expert in a resident-slot table  (moe_slot_lookup)
 *      and lists the experts that miss it
 *   4. groups the T*k (token, expert) pairs by expert        (moe_permute)
 *      and writes the FFN's device work list
 *   5. runs each expert's quantised FFN on its tokens:       (moe_expert_ffn_q4 /
 *      gate/up matvec with fused group-wise dequant, SwiGLU,   moe_expert_ffn_q2)
 *      down matvec
 *   6. adds the gate-weighted expert outputs to the residual (moe_combine)
 *
 * Sources (pages cited by title and section):
 *   - "12GB card runs a 68GB model: Betelgeuse engine measured at 22 tok/s",
 *     MoE primer (router scores each expert from the hidden state, top-k run)
 *     and "in-stream GPU doorbell" (hits resolved on the device, the host is
 *     told only about misses);
 *   - "Luce Spark: running a 35B MoE in 16GB", hot / warm / cold expert tiers;
 *   - "Strata" (125B MoE at 100+ tok/s on one RTX 3090), sec. 2.2 (INT4,
 *     groups of 128 with a scale and offset), sec. 2.3 (tokens that picked the
 *     same expert share one fetch of its weights), sec. 3.4 (hand-written
 *     INT4 decode GEMV, group-contiguous weights, experts in one buffer);
 *   - "Flash-MoE: running a big model on a small laptop (translation)",
 *     sec. 2 (weight = nibble*scale + bias, FMA form) and sec. 3 (4/2-bit
 *     dequant matvec, fused SwiGLU, fused combine + residual).
 *
 * Conventions for every call
 *   - All array pointers are DEVICE pointers unless a parameter says
 *     otherwise.  The caller allocates and owns every buffer, including the
 *     workspace; the library keeps no device memory between calls, except the
 *     fixed per-GPU array of moe_expert_ffn_fused_noalloc.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *     Calls only enqueue work on `stream` and return; they never synchronise
 *     and never allocate.
 *   - Arguments are validated on the host before anything is enqueued: a
 *     call that returns an error has enqueued nothing.  moe_last_error()
 *     returns a thread-local description of the last failure.  Errors raised
 *     by the GPU while the work runs surface at the caller's next
 *     synchronisation.
 *   - Limits: 0 <= T, T*k <= 65536; 1 <= E <= 1024; 1 <= k <= min(E, 32);
 *     H and I multiples of 128 with 128 <= H <= 8192 and 128 <= I <= 16384;
 *     group_size 128, 64 or 32.  Device pointers to codes and activations must be
 *     16-byte aligned, and so must scale and bias arrays.
 *   - Ids passed back in must come from these calls (or satisfy the same
 *     invariants); kernels skip out-of-range ids rather than touch memory
 *     outside the buffers, and the results for such ids are unspecified.
 *
 * Data layout
 *   x, residual, out   bf16 bit patterns (uint16) [T][H], row-major
 *   w_router           float32 [E][H]; router_bias float32 [E] or NULL
 *   logits             float32 [T][E]
 *   topk_ids           int32 [T][k], in rank order (best first)
 *   topk_w             float32 [T][k], gates in the same order
 *   pairs              p = t*k + j is the j-th pick of token t
 *   expert weights     see moe_qweights; codes packed along K, groups of 128
 *                      along K, one fp16 scale and one fp16 bias per group:
 *                      w[n][k] = code[n][k] * scale[n][k/128] + bias[n][k/128]
 *   y_rows             bf16 [T*k][H]: row r is the FFN output for the pair
 *                      sorted_pairs[r] (rows in expert-grouped order)
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

/* Status codes returned by every call. */
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG 1   /* null pointer, bad size, misalignment */
#define MOE_ERR_UNSUPPORTED 2   /* outside the limits above, unknown algo */
#define MOE_ERR_WORKSPACE 3     /* workspace missing or too small */
#define MOE_ERR_HIP 4           /* the HIP runtime rejected a launch */

/* FFN algorithms (argument `algo` of the FFN calls). */
#define MOE_ALGO_AUTO 0   /* choose per call from the shape */
#define MOE_ALGO_GEMV 1   /* vector-ALU matvec, one pass over the weights per token tile */
#define MOE_ALGO_MFMA 2   /* matrix-core tiles (bf16 MFMA with exact code operands) */
#define MOE_ALGO_GEMM 3   /* grouped GEMM on the matrix cores for experts with many
                             tokens (prefill): 64-token items, 4-bit codes only,
                             I and H multiples of 128 and at least 256; AUTO
                             picks it when the experts average at least 64
                             tokens */

/* FFN work list (written by moe_permute, read by the FFN calls): one entry per
 * tile of up to MOE_WORK_TILE_ROWS consecutive sorted rows of one expert,
 * expert-major in ascending expert order.  Entry = int32[MOE_WORK_ENTRY_INTS]:
 *   [0] expert id   [1] first sorted row of the tile   [2] rows in the tile
 *   [3] index of the tile among its expert's tiles (0, 1, ...)
 *   [4 + j] token of row j (j < rows; slots past the tile's rows repeat the
 *           token of row 0) */
#define MOE_WORK_TILE_ROWS 16
#define MOE_WORK_ENTRY_INTS 20

/* Operations for moe_workspace_bytes. */
#define MOE_OP_ROUTE 0
#define MOE_OP_LOOKUP 1
#define MOE_OP_PERMUTE 2
#define MOE_OP_FFN 3
#define MOE_OP_COMBINE 4

typedef struct moe_dims {
    int32_t T;           /* tokens in this call */
    int32_t H;           /* hidden size */
    int32_t I;           /* expert intermediate size */
    int32_t E;           /* routed experts */
    int32_t k;           /* experts per token */
    int32_t group_size;  /* quantisation group along K: 128, 64 or 32 (see the
                            FFN calls for which paths take 64 and 32) */
} moe_dims;

/* Quantised expert weights, expert-major so that every expert's matrices sit
 * in one buffer per matrix ("Strata" sec. 3.4).  Index m: 0 = gate [I][H],
 * 1 = up [I][H], 2 = down [H][I], written [N][K] below; G = dims.group_size
 * (one scale and bias per G consecutive k: 128, the "Strata" page sec. 2.2;
 * 64, the same page sec. 4.4; 32, the laptop page sec. 4.2).
 *   q[m]      uint8 [E][K/128][N][16*bits], group-major: for each group of
 *             128 along K, the codes of that group of all N rows follow one
 *             another (row n's piece of group g at ((e K/128 + g) N + n)
 *             16 bits), so a tile of rows reads one contiguous run per group.
 *             Within a row's piece of a group, 4-bit: byte j holds k = 2j in
 *             its low nibble and k = 2j+1 in its high nibble; 2-bit: bits
 *             2i..2i+1 of byte j hold k = 4j + i (k counted from the group's
 *             start).  A row-major [N][K*bits/8] array becomes this layout by
 *             viewing it as [N][K/128][16*bits] and swapping the first two
 *             axes (group_major() in the Python binding).
 *   scale[m]  fp16 bit patterns [E][N][K/G]
 *   bias[m]   fp16 bit patterns [E][N][K/G]
 * The struct itself is a host object holding device pointers; it is read
 * during the call only. */
typedef struct moe_qweights {
    const uint8_t* q[3];
    const uint16_t* scale[3];
    const uint16_t* bias[3];
} moe_qweights;

/* Version of this ABI (MOE_ABI_VERSION). */
int moe_abi_version(void);

/* Static text for a status code. */
const char* moe_status_string(int status);

/* Thread-local description of this thread's last failed call ("" if none). */
const char* moe_last_error(void);

/* Device workspace that `op` needs for these dims (host-only, no GPU work).
 * Only MOE_OP_FFN needs any (the SwiGLU activations between the two halves of
 * the FFN: 4*T*k*I bytes for MOE_ALGO_GEMV, about 6.25*T*k*I for
 * MOE_ALGO_MFMA and AUTO); the others report 0.  bits in {2, 4}. */
int moe_workspace_bytes(const moe_dims* dims, int op, int bits, int algo, size_t* bytes);

/* Router logits and top-k (steps 1-2; Betelgeuse page, MoE primer).
 *   logits[t][e] = sum_h x[t][h] * w_router[e][h] (+ router_bias[e]),
 *                  float32 accumulation
 *   topk_ids[t][0..k)  the k experts with the largest logits, best first;
 *                  equal logits (also -0 vs +0) rank the lower expert id
 *                  first; NaN ranks below every number
 *   topk_w[t][j]   renormalize != 0: exp(L_j - L_0) / sum_{j'<k} exp(L_j' - L_0)
 *                  renormalize == 0: softmax over all E logits at the pick
 * logits is a required [T][E] output (it is also the input of the top-k). */
int moe_route_topk(const moe_dims* dims, const uint16_t* x, const float* w_router,
                   const float* router_bias, int renormalize, float* logits,
                   int32_t* topk_ids, float* topk_w, void* stream);

/* Step 2 alone, from caller-provided float32 logits [T][E]; same rules. */
int moe_topk_from_logits(const moe_dims* dims, const float* logits, int renormalize,
                         int32_t* topk_ids, float* topk_w, void* stream);

/* Resident-slot lookup (step 3; Betelgeuse page, "in-stream GPU doorbell";
 * Luce Spark page, hot/warm/cold tiers).
 *   slot_of_expert int32 [E]: slot holding the expert, or any value outside
 *                  [0, n_slots) when it is not resident
 *   pair_slot      int32 [T*k] out: the pair's slot, or -1 on a miss
 *   miss_experts   int32 [E] out: the distinct missing experts, ascending, in
 *                  entries [0, *n_miss); the rest is left untouched
 *   n_miss         int32 [1] out
 *   host_doorbell  NULL, or a device-visible pointer to pinned host memory
 *                  (hipHostMalloc): set to n_miss only when n_miss > 0,
 *                  never written otherwise -- the host clears it
 *   last_use       NULL, or uint32 [n_slots]: last_use[slot] = step for
 *                  every slot hit in this call */
int moe_slot_lookup(const moe_dims* dims, const int32_t* topk_ids, const int32_t* slot_of_expert,
                    int32_t n_slots, int32_t* pair_slot, int32_t* miss_experts, int32_t* n_miss,
                    int32_t* host_doorbell, uint32_t* last_use, uint32_t step, void* stream);

/* Group pairs by expert (step 4; "Strata" sec. 2.3).  A stable counting sort.
 *   expert_counts  int32 [E]     pairs per expert
 *   expert_offsets int32 [E+1]   exclusive prefix sum, offsets[E] = T*k
 *   sorted_pairs   int32 [T*k]   pairs grouped by expert, ascending p within
 *                                an expert
 *   pair_to_row    int32 [T*k]   inverse: sorted_pairs[pair_to_row[p]] == p
 *   active_experts int32 [E]     experts with count > 0, ascending, first
 *                                *n_active entries written
 *   n_active       int32 [1]
 *   work_list      int32 [capacity][MOE_WORK_ENTRY_INTS], capacity from
 *                  moe_work_list_capacity, 16-byte aligned; first *n_work
 *                  entries written
 *   n_work         int32 [1] */
int moe_permute(const moe_dims* dims, const int32_t* topk_ids, int32_t* expert_counts,
                int32_t* expert_offsets, int32_t* sorted_pairs, int32_t* pair_to_row,
                int32_t* active_experts, int32_t* n_active, int32_t* work_list, int32_t* n_work,
                void* stream);

/* Steps 1-4 with one argument block: moe_route_topk, then moe_slot_lookup and
 * moe_permute on the ids it picked, with the same outputs bit for bit.  Every
 * field has the meaning, layout and alignment it has in those calls;
 * host_doorbell and last_use may be NULL.  The struct itself is read on the
 * host during the call only.
 *   sync  NULL, or int32 [MOE_DISPATCH_SYNC_INTS] device memory, 256-byte
 *         aligned, that holds zeros before the first call (each call leaves
 *         it zero again).  Its counters sit 256 bytes apart: arrivals at
 *         counters that share a cache line queue behind each other.
 *         With sync and 1 <= T <= 64, T*k <= 4096, the whole routing is one
 *         launch: workgroups that finish a stage late run the next one,
 *         signalled through these counters.  Calls that share one sync
 *         buffer must be ordered (one stream).  Without sync, or for larger
 *         calls, the router runs first, then (T*k <= 4096) top-k, lookup and
 *         grouping in one workgroup, else the separate calls' kernels. */
#define MOE_DISPATCH_SYNC_INTS 576
typedef struct moe_dispatch {
    int32_t* topk_ids;              /* [T][k] */
    float* topk_w;                  /* [T][k] */
    const int32_t* slot_of_expert;  /* [E] */
    int32_t n_slots;
    int32_t* pair_slot;             /* [T*k] */
    int32_t* miss_experts;          /* [E] */
    int32_t* n_miss;                /* [1] */
    int32_t* host_doorbell;         /* pinned host, or NULL */
    uint32_t* last_use;             /* [n_slots], or NULL */
    uint32_t step;
    int32_t* expert_counts;         /* [E] */
    int32_t* expert_offsets;        /* [E+1] */
    int32_t* sorted_pairs;          /* [T*k] */
    int32_t* pair_to_row;           /* [T*k] */
    int32_t* active_experts;        /* [E] */
    int32_t* n_active;              /* [1] */
    int32_t* work_list;             /* [capacity][MOE_WORK_ENTRY_INTS] */
    int32_t* n_work;                /* [1] */
    int32_t* sync;                  /* [MOE_DISPATCH_SYNC_INTS], or NULL */
} moe_dispatch;

int moe_route_dispatch(const moe_dims* dims, const uint16_t* x, const float* w_router,
                       const float* router_bias, int renormalize, float* logits,
                       const moe_dispatch* out, void* stream);

/* Entries the work list of these dims can need (host-only):
 * min(E, T*k) + T*k / MOE_WORK_TILE_ROWS. */
int moe_work_list_capacity(const moe_dims* dims, int32_t* entries);

/* Quantised expert FFN (step 5), 4-bit codes.  For every sorted row r of
 * expert e and token t (from the work list of moe_permute):
 *   a_i = sum_k Wg[e][i][k] x[t][k],  u_i = sum_k Wu[e][i][k] x[t][k]
 *   h_i = silu(a_i) * u_i                            (float32)
 *   y_rows[r][n] = bf16( sum_i Wd[e][n][i] h_i )     (round to nearest even)
 * Each expert's weights are read once per call for all of its tokens (once per
 * work-list tile of up to 16 tokens).  n_work is read on the device, so the
 * call never waits for routing results on the host.
 * Groups of 64 and 32 (dims.group_size): the matrix-core algorithm takes them
 * where the decode kernels' tiles fit LDS (T up to 16 tokens per tile, the
 * activation row and h planes in 80 KB); the vector-ALU algorithm where one
 * scale group holds a whole 16-byte chunk of codes (groups of 64 and 32 at
 * 4 bits, 64 at 2 bits); MOE_ALGO_AUTO picks one of these.  Other cases
 * (the grouped GEMM, the persistent and streaming matrix-core kernels of
 * larger shapes) fail with MOE_ERR_UNSUPPORTED.
 * workspace: at least moe_workspace_bytes(dims, MOE_OP_FFN, 4, algo), 256-byte
 * aligned.  algo: MOE_ALGO_*. */
int moe_expert_ffn_q4(const moe_dims* dims, const uint16_t* x, const int32_t* work_list,
                      const int32_t* n_work, const moe_qweights* weights, uint16_t* y_rows, int algo,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Same as moe_expert_ffn_q4 with 2-bit codes (Flash-MoE page, sec. 3). */
int moe_expert_ffn_q2(const moe_dims* dims, const uint16_t* x, const int32_t* work_list,
                      const int32_t* n_work, const moe_qweights* weights, uint16_t* y_rows, int algo,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Step 5 in two halves (the scope rows "gate/up matvec + SwiGLU" and "down
 * matvec"), for callers that time or schedule them apart.  bits in {2, 4};
 * the other arguments are as for moe_expert_ffn_q4.  moe_expert_gateup writes
 * the SwiGLU activations h_i = silu(a_i) * u_i of every routed row into the
 * workspace and moe_expert_down reads them from there, so both calls must get
 * the same workspace, dims, bits and algo.  Workspace contents:
 *   MOE_ALGO_GEMV: float32 h [T*k][I] at offset 0;
 *   MOE_ALGO_MFMA (and AUTO): h as three bf16 planes hi, mid, lo [3][T*k][I]
 *     with hi + mid + lo == h to float32 precision, stored in the pair order
 *     of the matrix-core operands, followed by float32 partial sums of h over
 *     16 consecutive i [T*k][I/16]; at dims whose down projection streams h
 *     through LDS in chunks of K (a large I), then int32 arrival counters,
 *     float32 partial output sums and four int8 planes of h per group of 128
 *     with their scale and sum, all of which moe_expert_down uses as scratch:
 *     the gate/up call clears the counters and every down call leaves them
 *     clear.
 * moe_expert_ffn_q4/q2 == moe_expert_gateup followed by moe_expert_down. */
int moe_expert_gateup(const moe_dims* dims, int bits, const uint16_t* x, const int32_t* work_list,
                      const int32_t* n_work, const moe_qweights* weights, int algo, void* workspace,
                      size_t workspace_bytes, void* stream);

int moe_expert_down(const moe_dims* dims, int bits, const int32_t* work_list, const int32_t* n_work,
                    const moe_qweights* weights, int algo, void* workspace,
                    size_t workspace_bytes, uint16_t* y_rows, void* stream);

/* Step 5 in one launch: the same results as moe_expert_gateup followed by
 * moe_expert_down, bit for bit, for bits in {2, 4}.  At the decode shapes that
 * have a one-launch kernel (matrix-core algorithm; tiles that fit the decode
 * kernels; a work-list capacity of at most MOE_FFN_SYNC_INTS / 32 - 1
 * entries), the gate/up and down items of the work list run in one launch and
 * an entry's down items start streaming their weights while other entries are
 * still in gate/up; they read h once its gate/up items have signalled through
 * `sync`.  Other shapes, and algo GEMV or GEMM, run the two halves as two
 * launches.  Arguments as for moe_expert_gateup / moe_expert_down, plus:
 *   sync  int32 [MOE_FFN_SYNC_INTS] device memory, 256-byte aligned, holding
 *         zeros before the first call; each call leaves it zero.  Calls that
 *         share one sync buffer must be ordered (one stream).  The last 32
 *         ints are a fault flag: nonzero after a call means a down item gave
 *         up waiting for its h (about 10 ms), and that call's outputs are not
 *         valid.  After such a call the counters may not be back to zero
 *         either: the caller zeroes the whole buffer before the next call. */
#define MOE_FFN_SYNC_INTS 32800
int moe_expert_ffn_fused(const moe_dims* dims, int bits, const uint16_t* x, const int32_t* work_list,
                         const int32_t* n_work, const moe_qweights* weights, int algo, void* workspace,
                         size_t workspace_bytes, uint16_t* y_rows, int32_t* sync, void* stream);

/* Step 5 in one launch without allocating: moe_expert_ffn_fused with its
 * workspace and counters taken from a fixed device array of the library.  For
 * callers that cannot allocate (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  It runs the same kernels, so its
 * y_rows equal moe_expert_ffn_fused's bit for bit.
 *   The array holds MOE_NOALLOC_WORKSPACE_BYTES of workspace: a call whose
 *   moe_workspace_bytes(dims, MOE_OP_FFN, bits, algo) is larger fails with
 *   MOE_ERR_WORKSPACE before anything is enqueued.
 *   Every GPU the library runs on holds one such array until the process ends,
 *   and every call on a GPU (the current device) uses that GPU's array and
 *   leaves its last contents there: calls that overlap on one GPU (two
 *   streams, two threads) race, so order them.  Each call first clears the
 *   counters with a small kernel on `stream` (no memset node, so the call can
 *   be captured).  The first call on a device looks the array up (no
 *   allocation); make that call outside graph capture.
 *   fault  NULL, or device int32 set to 1 by a call whose down items gave up
 *          waiting for their h (that call's y_rows are then invalid); never
 *          cleared by the library.  4-byte aligned.
 * Other arguments, alignment and errors as for moe_expert_ffn_fused. */
#define MOE_NOALLOC_WORKSPACE_BYTES (16u << 20)
int moe_expert_ffn_fused_noalloc(const moe_dims* dims, int bits, const uint16_t* x, const int32_t* work_list,
                                 const int32_t* n_work, const moe_qweights* weights, int algo, uint16_t* y_rows,
                                 int32_t* fault, void* stream);

/* Step 5 with an always-on shared expert in the same launch: the results of
 * moe_expert_ffn_fused for the routed rows, and the shared expert's FFN for
 * every token, the shared expert's tiles being extra entries after the routed
 * ones (one launch streams both; the Flash-MoE page, sec. 3, gates the shared
 * expert's output into the combine, see moe_combine_shared).
 *   dims     the routed layer (E routed experts, k picks).
 *   weights  E + 1 experts: the routed ones, then the shared expert (same H
 *            and I), in the layout of moe_qweights.
 *   y_rows   bf16 [T*(k+1)][H]: rows 0 .. T*k-1 as moe_expert_ffn_fused's,
 *            then row T*k + t = the shared expert's output for token t.
 *   workspace  at least moe_workspace_bytes of dims with E+1 and k+1.
 *   work_list, n_work, x, sync, algo, stream as for moe_expert_ffn_fused.
 * Runs on the matrix-core decode kernels (one launch where a one-launch kernel
 * exists for the shape, else their two launches, with the same entries); for
 * shapes they do not take, other algorithms, or E + 1 or k + 1 beyond the
 * limits: MOE_ERR_UNSUPPORTED before anything is enqueued, and the caller runs
 * the shared expert as its own moe_expert_ffn_* call (E = 1, k = 1).  Routed
 * rows may differ from moe_expert_ffn_fused's in the last bits where the larger
 * row count changes the split of K among a workgroup's waves. */
int moe_expert_ffn_fused_shared(const moe_dims* dims, int bits, const uint16_t* x, const int32_t* work_list,
                                const int32_t* n_work, const moe_qweights* weights, int algo, void* workspace,
                                size_t workspace_bytes, uint16_t* y_rows, int32_t* sync, void* stream);

/* Combine + residual (step 6; Flash-MoE page, sec. 3):
 *   acc = residual[t][n];  for j = 0..k-1 in order:
 *       acc = fmaf(topk_w[t][j], y_rows[pair_to_row[t*k+j]][n], acc)
 *   out[t][n] = bf16(acc)   (float32 accumulation, round to nearest even)
 * out may be the same buffer as residual. */
int moe_combine(const moe_dims* dims, const uint16_t* y_rows, const int32_t* pair_to_row,
                const float* topk_w, const uint16_t* residual, uint16_t* out, void* stream);

/* Combine + residual with a shared expert (step 6 with the sigmoid gate of the
 * Flash-MoE page, sec. 3, which lists combine, residual and a sigmoid gate as
 * one fused kernel; the gate is read as that of an always-on shared expert):
 *   L_t = x[t] . shared_gate_w  (float32; a fixed summation order, the same on
 *         every call), s_t = 1 / (1 + expf(-L_t)),
 *   acc = residual[t][n];  for j = 0..k-1 in order:
 *       acc = fmaf(topk_w[t][j], y_rows[pair_to_row[t*k+j]][n], acc)
 *   acc = fmaf(s_t, y_shared[t][n], acc);   out[t][n] = bf16(acc) (RNE).
 *   y_shared        bf16 [T][H]: the shared expert's FFN output per token, e.g.
 *                   moe_expert_ffn_* run with E = 1, k = 1 on a work list of
 *                   every token (moe_permute of all-zero ids).
 *   x               bf16 [T][H]: the layer input the router saw.
 *   shared_gate_w   fp32 [H]: the gate's weight row.
 *   shared_gate_out fp32 [T] or NULL: receives s_t as used.
 * Other arguments, alignment and errors as for moe_combine; y_shared, x and
 * shared_gate_w 16-byte aligned, shared_gate_out 4-byte aligned.  out may be
 * the same buffer as residual. */
int moe_combine_shared(const moe_dims* dims, const uint16_t* y_rows, const int32_t* pair_to_row,
                       const float* topk_w, const uint16_t* y_shared, const uint16_t* x,
                       const float* shared_gate_w, const uint16_t* residual, uint16_t* out,
                       float* shared_gate_out, void* stream);

/* Weight-format adapter (run once when weights are loaded; not a step of the
 * layer).  Zero-point groups, w = (q - z) s ("Strata" page, sec. 2.2: each
 * group of 128 weights shares one scale and one zero point; the laptop page,
 * sec. 4.2, the same form), are this library's w = q s + b with b = -(z s):
 *   bias[i] = fp16(-(float)zeros[i] * scale[i]),  0 <= i < n.
 * z s is exact in float32, so the one rounding is to fp16 (nearest, ties to
 * even; past 65504 an infinity).  A NaN scale, or z = 0 with an infinite
 * scale, gives a NaN bias.  The codes q are used unchanged.
 *   n      number of (row, group) entries, e.g. E*N*(K/128) for one matrix;
 *          0 is a no-op and the pointers are not used.
 *   scale  fp16 bits [n], device memory, 2-byte aligned (moe_qweights.scale[m]).
 *   zeros  uint8 [n], device memory: one zero point per entry, not packed.
 *   bias   fp16 bits [n], device memory, 2-byte aligned (moe_qweights.bias[m]);
 *          must not overlap scale or zeros.
 * Errors: n < 0, a NULL or misaligned pointer, or overlapping buffers:
 * MOE_ERR_INVALID_ARG before anything is enqueued.  Asynchronous on `stream`. */
int moe_zero_point_bias(int64_t n, const uint16_t* scale, const uint8_t* zeros, uint16_t* bias, void* stream);

/* ------------------------------------------------------ residency tiers
 * "Luce Spark" page, sec. 1 (calibrated placement: count how often traffic
 * routes to each expert and keep the most used set resident, the hot tier)
 * and sec. 2 (a bounded ring of spare slots: an expert routed to while not
 * resident is copied from pinned host memory into a spare slot, the least
 * recently used slot giving way; hot / warm / cold tiers); "Strata" page,
 * sec. 2.4 (copies run on a stream of their own beside the compute) and
 * sec. 4.5 (pinned host memory).
 *
 * The layer's E experts live in pinned host memory in the moe_qweights
 * layout (the cold tier; device-visible pointers, e.g. hipHostMalloc); an
 * HBM pool of n_slots expert slots, in the same layout with n_slots experts,
 * holds the resident ones.  Slots [0, n_hot) hold the hot set and are never
 * evicted; slots [n_hot, n_slots) are the warm ring.  The tables are device
 * memory the caller owns and the calls below update:
 *   slot_of_expert  int32 [E]: slot holding expert e, -1 when cold; it is the
 *                   resident table of the slot lookup (moe_slot_lookup /
 *                   moe_route_dispatch with this n_slots);
 *   expert_of_slot  int32 [n_slots]: expert in slot s, -1 when empty;
 *   last_use        uint32 [n_slots]: step of the slot's last use, 0 = never.
 *                   Steps count up from 1; the slot lookup of each step stamps
 *                   the slots it hits (pass last_use and the same step).
 * A step: slot lookup (stamps hits, lists misses) -> moe_residency_plan ->
 * moe_expert_copy of its copy list (src = host experts, dst = pool), on a
 * second stream after an event -> the FFN on list 0 with the pool's weights,
 * overlapping the copy -> (after the copy's event) the FFN on list 1 with the
 * pool's weights and on list 2 with the host experts -> combine.  The FFN's
 * rows are the same bits as with every expert resident. */
typedef struct moe_residency {
    int32_t n_hot;            /* 0 <= n_hot <= n_slots */
    int32_t n_slots;          /* 1 <= n_slots <= E */
    int32_t* slot_of_expert;  /* [E] */
    int32_t* expert_of_slot;  /* [n_slots] */
    uint32_t* last_use;       /* [n_slots] */
} moe_residency;

/* Routing-frequency counters: freq[e] += expert_counts[e] for e < E (the
 * per-expert pair counts moe_permute / moe_route_dispatch wrote).  freq:
 * uint32 [E] device memory (wraps at 2^32). */
int moe_route_counts(const moe_dims* dims, const int32_t* expert_counts, uint32_t* freq, void* stream);

/* The calibrated hot set: hot[0..n) = the n experts of highest freq, most used
 * first, equal counts to the lower id.  0 <= n <= E; hot: int32 [n]. */
int moe_hot_set(const moe_dims* dims, const uint32_t* freq, int32_t n, int32_t* hot, void* stream);

/* One step of the warm ring, on the device.  Inputs: this step's miss list
 * (miss_experts / n_miss, ascending, from the slot lookup on r's tables) and
 * FFN work list (work_list / n_work, from moe_permute).  For each missing
 * expert in ascending id order, the ring slot with the oldest last_use (ties
 * to the lowest slot) that this step has not used takes it: the slot's old
 * expert goes cold, the tables point the new one at the slot, the slot is
 * stamped with `step`, and (expert, slot) is appended to copies.  A missing
 * expert that finds no such slot stays cold this step.  Outputs:
 *   copies       int32 [n_slots][2]: (expert, slot) pairs, *n_copy of them;
 *   lists        int32 [MOE_RESIDENCY_LISTS][capacity][MOE_WORK_ENTRY_INTS]
 *                (capacity from moe_work_list_capacity), 16-byte aligned: the
 *                work list's entries in order, split by where their expert is
 *                read: list 0 = resident before this step, list 1 = copied in
 *                this step (expert field replaced by the slot in both), list 2
 *                = still cold (expert field unchanged, read from host memory);
 *   list_counts  int32 [MOE_RESIDENCY_LISTS]: entries in each list.
 * Each list is a work list for the FFN calls with n_work = list_counts + i. */
#define MOE_RESIDENCY_LISTS 3
int moe_residency_plan(const moe_dims* dims, const moe_residency* r, const int32_t* miss_experts,
                       const int32_t* n_miss, uint32_t step, const int32_t* work_list, const int32_t* n_work,
                       int32_t* lists, int32_t* list_counts, int32_t* copies, int32_t* n_copy, void* stream);

/* Copy experts between two weight sets of one layer shape and code width:
 * for i < *n_copy, expert copies[2i] of src (E experts) into slot copies[2i+1]
 * of dst (n_dst experts), all three matrices' codes, scales and biases.  src
 * may be pinned host memory (device-visible pointers).  max_copies bounds
 * *n_copy (the grid is sized for it); pairs out of range are skipped. */
int moe_expert_copy(const moe_dims* dims, int bits, const moe_qweights* src, const moe_qweights* dst, int32_t n_dst,
                    const int32_t* copies, const int32_t* n_copy, int32_t max_copies, void* stream);

/* Measurement aid, not a step of the layer: reads `bytes` of device memory at
 * `src` once, with 16-byte loads spread over every compute unit, and writes
 * the XOR of what each workgroup read into sink[0 .. MOE_STREAM_SINK_INTS),
 * so that the HBM read rate of a plain stream can be timed beside the expert
 * FFN's weight stream ("Strata" page, sec. 1.2: decode is bound by how fast
 * weights move).  src 16-byte aligned and bytes a multiple of 16; sink
 * uint32 [MOE_STREAM_SINK_INTS] device memory, 4-byte aligned.  bytes == 0 is
 * a no-op.  Errors: MOE_ERR_INVALID_ARG before anything is enqueued. */
#define MOE_STREAM_SINK_INTS 4096
int moe_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
