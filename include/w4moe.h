/*
 * w4moe: the fused W4A16 SwiGLU Mixture-of-Experts FFN layer on one AMD Instinct MI355X (gfx950).
 *
 * What the layer computes (source pages: "The Pivot to Real Hardware: Diagnosing Throughput and
 * Building the INT4 MoE Benchmark for Kimi K2.6", Step 1: Understanding the Weight Format and
 * Input Knowledge Required item 1; "The Weight-Streaming Threshold", Input Knowledge Required,
 * Mixture-of-Experts architecture):
 *
 *   for each token m and slot j < topk, with e = topk_ids[m][j]:
 *     h      = x[m] . W1_e                      (W1_e: [K, 2N], gate columns [0,N), up [N,2N))
 *     a      = SiLU(h[0:N]) * h[N:2N]            SiLU(z) = z / (1 + exp(-z))
 *     y_mj   = a . W2_e                          (W2_e: [N, K])
 *   out[m]  = sum_j topk_weights[m][j] * y_mj    (slots summed in order j = 0..topk-1)
 *
 * W1_e and W2_e are signed INT4 values times one bf16 scale per group of g consecutive elements of
 * the reduction dimension (hidden K for W1, intermediate N for W2); g = group_size is 32 at K2.6
 * ("The Pivot to Real Hardware...", Input Knowledge Required, INT4 with group size 32), and 64 or
 * 128 are accepted as well. Activations and output are bf16;
 * every product is accumulated in fp32; the intermediate a is rounded to bf16; above 64 slots per
 * call (the aligned plans) each slot's weighted output is rounded to bf16 before the slots are
 * added in fp32; the output is rounded to bf16 with round-to-nearest-even.
 *
 * Logical weight format accepted by w4moe_prepack (the GPTQ-style layout the pages name as the
 * repack input, eight 4-bit codes to each 32-bit word, no activation-order permutation: "The Pivot to
 * Real Hardware...", Step 1: Understanding the Weight Format; the pages' repack also takes the bit
 * width, and 8-bit codes are accepted with num_bits = 8):
 *   w1_q      int32  [E][K/8][2N]   word (i, c) holds rows 8i..8i+7 of column c; row 8i+t sits in
 *                                   bits 4t..4t+3 as the code value+8 (offset binary, -8..7)
 *   w1_scales bf16   [E][K/g][2N]   scale of rows g*i..g*i+g-1 of column c
 *   w2_q      int32  [E][N/8][K]    same packing, reduction dimension N
 *   w2_scales bf16   [E][N/g][K]
 * With num_bits = 8: w1_q int32 [E][K/4][2N] and w2_q int32 [E][N/4][K], row 4i+t in bits 8t..8t+7
 * as the code value+128 (-128..127); scales as above. The layer is then W8A16, computed the same way.
 * bf16 values travel as uint16_t bit patterns.
 *
 * Conventions for every entry point:
 *   - Pointers named "device" point to GPU memory on the handle's device; the caller owns them and
 *     keeps them alive until the stream has passed the call. The handle owns its packed weights
 *     and workspace.
 *   - `stream` is a hipStream_t passed as void* (NULL = the device's null stream). Calls enqueue
 *     work and return without synchronising, except where stated.
 *   - Errors are returned as w4moe_status; nothing throws across this boundary. All argument
 *     checks run on the host before any HIP call. w4moe_last_error() gives a thread-local detail.
 *   - Supported shapes: 1 <= E <= 1024 (the alignment keeps per-expert state in one workgroup's LDS),
 *     group_size 32, 64 or 128, K and N multiples of group_size (so K % 32 == 0 and N % 32 == 0 at
 *     K2.6's group of 32), K and N at most 2^30, 1 <= topk <= E, 1 <= max_tokens and
 *     max_tokens * topk <= 1<<20. Anything else is W4MOE_ERR_UNSUPPORTED. Inside, the reduction
 *     dimensions are padded up to whole 128-row blocks and the output columns of W2 up to whole
 *     64-column blocks (see w4moe_prepack); K2.6 (K = 7168, N = 2048) needs no padding.
 */
#ifndef W4MOE_H
#define W4MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W4MOE_OK = 0,
    W4MOE_ERR_INVALID_ARG = 1,   /* null handle or pointer, negative size, M > max_tokens, bad range */
    W4MOE_ERR_UNSUPPORTED = 2,   /* a shape or option outside the supported set above */
    W4MOE_ERR_NOT_PREPACKED = 3, /* forward before every expert was prepacked */
    W4MOE_ERR_OUT_OF_MEMORY = 4, /* device allocation failed in w4moe_create */
    W4MOE_ERR_HIP = 5            /* a HIP call or kernel launch failed (detail in w4moe_last_error) */
} w4moe_status;

typedef struct w4moe_ctx *w4moe_handle;

typedef struct {
    int32_t num_experts; /* E */
    int32_t hidden;      /* K: model width, reduction dimension of W1, output width */
    int32_t inter;       /* N: per-expert intermediate width (W1 has 2N columns: gate | up) */
    int32_t topk;        /* experts per token */
    int32_t group_size;  /* scale group along the reduction dimension: 32, 64 or 128 */
    int32_t max_tokens;  /* largest M forward accepts; sizes the workspace */
    int32_t num_bits;    /* code width: 4 (also when 0) or 8 */
    int32_t act_order;   /* 0: consecutive scale groups (w4moe_prepack); 1: activation-ordered weights
                            (w4moe_prepack_act_order; hidden <= 65536) */
} w4moe_config;

/* Creates a layer of the configuration above (the pages' workload is E = 384, K = 7168, N = 2048,
 * top-8, INT4 with groups of 32: "The Commit That Captured a Plateau", the commit message it quotes,
 * and "The Pivot to Real Hardware...", Step 1: Understanding the Weight Format). Allocates the
 * packed-weight buffers (the logical codes' bytes plus one bf16 scale per 32 rows and column: the
 * logical byte count for group_size 32 when K and N are multiples of 128 and K of 64, slightly more
 * for larger groups and for padded shapes) and a workspace sized for max_tokens on the current HIP
 * device (with act_order, also 2*Kp bytes per expert for the kept permutations and 2*Kp bytes per
 * routed entry, max_tokens*topk of them, for the gathered hidden rows; with K % 128 != 0, 2*Kp bytes
 * per token for the zero-padded hidden rows; Kp = K rounded up to 128). The handle is bound to that
 * device. The first create on a device also looks up and clears that device's static scratch array
 * (w4moe_forward_noalloc). */
w4moe_status w4moe_create(const w4moe_config *cfg, w4moe_handle *out);

/* One-time transform of experts [first_expert, first_expert + num_experts) from the logical layout
 * above into the library's own layout (the counterpart of the pages' gptq_marlin_moe_repack with an
 * empty permutation, "The Pivot to Real Hardware...", Step 2: The Repack Pipeline). The four device
 * pointers point at the first of those experts (e.g. w1_q + first_expert*K/8*2N of a full array).
 * The packed layout: for each matrix, expert e, column superblock cs of 64 output columns and
 * group quad gq (4 groups = 128 rows), a block of B = 4608 bytes (num_bits 4) or 8704 (num_bits 8)
 * at ((e*ncs + cs)*GQ + gq)*B holds P = 1 (4-bit) or 2 (8-bit) nibble planes and then the scales:
 *   bytes [p*4096, p*4096 + 4096): plane p; for gsub 0..3, lane 0..63, slot j 0..3: one 32-bit word
 *                      with rows (4gq+gsub)*32 + (lane/16)*8 + t (t = 0..7) of column col(cs, j, lane%16);
 *                      row t's nibble sits at bit 0,16,4,20,8,24,12,28 for t = 0..7 (4-bit: the code;
 *                      8-bit: plane 0 the low and plane 1 the high nibble of the code)
 *   bytes [P*4096, B): bf16 scales, index (m*4 + gsub)*4 + j, of rows (4gq+gsub)*32 .. +31 (their
 *                      group's scale, repeated for each 32 rows of a larger group), column col(cs, j, m)
 * with col(cs, j, m) = 32cs + 16j + m (j < 2) or N + 32cs + 16(j-2) + m (j >= 2) for W1 (gate and
 * up column n of a superblock share a lane), and 64cs + 16j + m for W2. A matrix has GQ = ceil(R/128)
 * group quads (R = K for W1, N for W2) and ncs = 2N/64 (W1) or ceil(K/64) (W2) superblocks: rows from
 * R and W2 columns from K on are padding, holding the code of the value 0 (4-bit: 8; 8-bit: 128) and
 * the scale 0, and forward feeds them zeros. The inputs may be freed once the stream has passed the
 * call. Experts may be prepacked in any order and more than once. */
w4moe_status w4moe_prepack(w4moe_handle h, int32_t first_expert, int32_t num_experts, const int32_t *w1_q,
                           const uint16_t *w1_scales, const int32_t *w2_q, const uint16_t *w2_scales,
                           void *stream);

/* Prepack of activation-ordered (GPTQ act-order) experts: the counterpart of the pages' repack with
 * a non-empty `perm` ("The Pivot to Real Hardware...", Step 2: The Repack Pipeline; K2.6 itself uses
 * none). Such a checkpoint records a group for every row of the reduction dimension; w1_perm int32
 * [num_experts][K] and w2_perm int32 [num_experts][N] (device) list each expert's rows in group
 * order: the group of row perm[i] is i / group_size (a stable argsort of the checkpoint's g_idx), so
 * row r of w1 is dequantised with w1_scales[e][i / group_size][c] for the i with w1_perm[e][i] = r.
 * Codes and scales are otherwise as for w4moe_prepack. W1 and W2 rows are stored in group order, and
 * W1's gate and up columns in w2_perm's order (so GEMM1 produces the intermediate features in the
 * order of W2's rows); w1_perm is also kept (as uint16, 2*K bytes per expert) for forward, which
 * reads each routed entry's hidden row in its expert's order (pair mode while staging the row for
 * GEMM1, the aligned plans through one gather kernel before GEMM1). Each permutation must
 * list every row once (a precondition; a value outside [0, K) or [0, N) is read as 0 and raises bit
 * 2 of the device flags). Requires a layer created with act_order = 1 (and w4moe_prepack requires
 * one created without). The inputs may be freed once the stream has passed the call. */
w4moe_status w4moe_prepack_act_order(w4moe_handle h, int32_t first_expert, int32_t num_experts, const int32_t *w1_q,
                                     const uint16_t *w1_scales, const int32_t *w1_perm, const int32_t *w2_q,
                                     const uint16_t *w2_scales, const int32_t *w2_perm, void *stream);

/* The layer (see top) for M tokens: hidden bf16 [M][K] (device), topk_ids int32 [M][topk] (device),
 * topk_weights fp32 [M][topk] (device), out bf16 [M][K] (device, written entirely). 0 <= M <= max_tokens;
 * M == 0 does nothing. ids must lie in [0, E): an id outside that range is dropped (its slot adds
 * nothing) and raises the flag read by w4moe_device_error. Under w4moe_set_expert_range the ids
 * name experts of the whole layer: they must lie in [0, global_experts), and a slot whose expert
 * another shard holds adds nothing (no flag), so out is this shard's partial sum. Duplicate ids
 * within a token are two separate slots. Allocates nothing, never synchronises; calls that overlap on one handle race on
 * its workspace. */
w4moe_status w4moe_forward(w4moe_handle h, const uint16_t *hidden, int32_t M, const int32_t *topk_ids,
                           const float *topk_weights, uint16_t *out, void *stream);

/* For callers that cannot allocate device memory at call time (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): w4moe_forward computed by the same kernels, with
 * the call's workspace (SwiGLU rows, slot outputs, partial sums, hand-off counters and flags) taken
 * from a static array of 8 MiB that the library holds once per GPU, for the life of the process,
 * instead of the handle's workspace. It always runs the single-launch pair mode (plan 3), so it takes
 * at most 64 routed entries (M * topk <= 64, else UNSUPPORTED), and the call's buffers must fit the
 * array: 2.5 MiB of counters and flags (about 256 B per routed entry and 64-column block of K) and
 * 5.5 MiB of data (about (2N + 4K) B per routed entry; UNSUPPORTED with the sizes in
 * w4moe_last_error otherwise). Allocates nothing and never synchronises. Every handle on a GPU shares
 * that GPU's array, so calls of this entry point that overlap on one GPU race (serialise them on one
 * stream); they do not race with w4moe_forward, which uses the handle's own workspace. Arguments,
 * output and errors are as for w4moe_forward. */
w4moe_status w4moe_forward_noalloc(w4moe_handle h, const uint16_t *hidden, int32_t M, const int32_t *topk_ids,
                                   const float *topk_weights, uint16_t *out, void *stream);

/* Router step (pages: "The Pivot to Real Hardware...", Input Knowledge Required, item 1, and "The
 * Weight-Streaming Threshold...", Input Knowledge Required: each token picks its top-8 of the 384
 * experts through a gating network; the routing recipe of the workloads is a softmax over fp32
 * logits, top-k, renormalised). For each token m of logits fp32 [M][E] (device): topk_ids[m][j]
 * (int32 [M][topk], device, written) are the topk experts with the largest logits, largest first,
 * equal logits in ascending expert index; topk_weights[m][j] (fp32 [M][topk], device, written) =
 * exp(l_j - l_0) / sum_i exp(l_i - l_0) over the chosen ones (a softmax over all E renormalised
 * over the chosen topk). Under w4moe_set_expert_range the logits and ids cover all global_experts
 * experts (every shard routes alike). Logits are compared as fp32, so the ids are exact. NaN logits are never
 * chosen; a slot left without a candidate gets id -1, weight 0 and raises bit 0 of the device flags.
 * -inf marks an expert as masked (chosen only when nothing larger is left, weight 0); each token
 * needs a finite largest logit. Requires topk <= 64 (else UNSUPPORTED). Asynchronous on stream. */
w4moe_status w4moe_route(w4moe_handle h, const float *logits, int32_t M, int32_t *topk_ids, float *topk_weights,
                         void *stream);

/* Router and layer in one call: routes as w4moe_route (writing topk_ids and topk_weights, which
 * the caller owns; the router kernel runs first, on the same stream) and runs w4moe_forward with
 * that route. Same requirements and asynchrony as both calls. */
w4moe_status w4moe_forward_logits(w4moe_handle h, const uint16_t *hidden, int32_t M, const float *logits,
                                  int32_t *topk_ids, float *topk_weights, uint16_t *out, void *stream);

/* The token-to-expert alignment the aligned plans run first, exposed for checking. The pages do not
 * describe this step (it runs inside the fused kernel they time, "The Commit That Captured a
 * Plateau", the commit message it quotes); what it computes here is the plain stable counting sort
 * of the routing entries by expert, padded per expert to whole blocks of the GEMMs' token tile. For
 * the T = M*topk flat entries f = m*topk + j of topk_ids (device) and a block size B (1..1024), writes
 * (device):
 *   counts[E]; offsets[E+1] (offsets[e+1] = offsets[e] + B*ceil(counts[e]/B));
 *   sorted_ids[offsets[E]]: rows offsets[e] + r (r < counts[e]) hold the r-th smallest f routed to e,
 *                           the other rows of expert e hold the sentinel T;
 *   block_expert[offsets[E]/B]: the expert of each block of B rows;
 *   active[n]: experts with counts > 0, ascending; n_active[1] = n (both optional, may be NULL).
 * Capacities the caller provides: sorted_ids and block_expert at least T + min(E, T)*(B-1) entries,
 * active E entries. Ids outside [0, E) are dropped as in forward (under w4moe_set_expert_range, e
 * is local expert e = global id first_expert + e, and the other shards' ids are dropped). */
w4moe_status w4moe_moe_align(w4moe_handle h, const int32_t *topk_ids, int32_t M, int32_t block, int32_t *counts,
                             int32_t *offsets, int32_t *sorted_ids, int32_t *block_expert, int32_t *active,
                             int32_t *n_active, void *stream);

/* The block size B (rows per MFMA token tile) forward uses for its alignment on this handle (16),
 * or -1 for a NULL handle. */
int32_t w4moe_align_block(w4moe_handle h);

/* Device pointer and byte size of the packed W1 (which = 1) or W2 (which = 2) buffer. */
w4moe_status w4moe_packed_weights(w4moe_handle h, int32_t which, const void **ptr, int64_t *bytes);

/* Kernel plan for forward: 0 = chosen from M (default: 3 while M * topk <= 120, else 4);
 * 1 = 16-row work items from the alignment, the reduction of a 64-column superblock split over the
 * waves of a workgroup as the entry count needs; 2 = 32-row work items, each wave owning a superblock
 * over the whole reduction; 3 = pair mode, no alignment pass: up to 128 routed entries, from 48 entries
 * on the entries routed to the same expert taken two at a time as one work item (its rows staged in
 * LDS), GEMM1 and GEMM2 in one launch whose GEMM2 workgroups wait, per item, for that item's GEMM1
 * workgroups (above 128 entries plan 5 runs instead); 4 = the wide kernel: work items of 48 rows for
 * 4-bit codes and 32 for 8-bit (32, 48 or 64 when the environment variable W4MOE_WIDE_ROWS says so at
 * create), the workgroup staging the item's token rows in LDS for four superblocks that walk the
 * reduction together (a GEMM2 over one or two group quads walks several superblocks per wave). With
 * 4-bit codes both GEMMs run in one launch, each GEMM2 workgroup waiting, bounded as in plan 3, for
 * its work item's GEMM1 workgroups, where GEMM2 is that short one or GEMM1's workgroups are expected
 * to fit one round of the GPU (W4MOE_WIDE_FUSED=0 at create keeps two launches, =1 takes one launch
 * for every 4-bit shape with items of at most 48 rows);
 * 5 = pair mode in two launches (GEMM1, then
 * GEMM2). Pair mode needs hidden and inter of at most 24576 (one row in LDS); otherwise plan 1 runs in
 * its place. Calls that overlap on one handle race in every plan (they share the workspace). */
w4moe_status w4moe_set_plan(w4moe_handle h, int32_t plan);

/* Expert parallelism, one GPU's share (pages: "The Weight-Streaming Threshold...", Input Knowledge
 * Required, the tensor-parallelism item, and Assumption 1: each of 8 GPUs holds a subset of the
 * experts, computes its portion, and an AllReduce combines the outputs): this handle's num_experts experts are experts
 * [first_expert, first_expert + num_experts) of a layer of global_experts experts (prepacked at
 * local indices 0 .. num_experts - 1). forward, forward_logits and moe_align then read routing ids
 * as global ids: local ones run as usual, those of other shards add nothing and raise no flag, and
 * only ids outside [0, global_experts) raise it. The sum over shards of their outputs is the whole
 * layer's output (rounded per shard). Default: first_expert 0, global_experts num_experts.
 * INVALID_ARG unless 0 <= first_expert, first_expert + num_experts <= global_experts and
 * topk <= global_experts; UNSUPPORTED for global_experts > 1024. */
w4moe_status w4moe_set_expert_range(w4moe_handle h, int32_t first_expert, int32_t global_experts);

/* The plan (1 to 5, as above) that forward runs for M tokens under the plan set. Writes *plan;
 * errors as forward for M outside [0, max_tokens]. */
w4moe_status w4moe_resolved_plan(w4moe_handle h, int32_t M, int32_t *plan);

/* Per-kernel timing: while enabled, forward records HIP events around each kernel it launches on
 * its stream (timing-only events: no system-scope fence at record time; a stage with no kernel records
 * nothing and reads 0). w4moe_read_profile
 * synchronises the handle's device, writes the summed milliseconds of
 * align, GEMM1 (+SwiGLU), GEMM2 and combine into ms[0..3] and the number of forward calls timed
 * (the single-launch pair mode counts both GEMMs under GEMM1; its align and combine are empty),
 * and clears the record. At most 1024 calls are kept between reads (older ones are dropped). */
w4moe_status w4moe_set_profiling(w4moe_handle h, int32_t enable);
w4moe_status w4moe_read_profile(w4moe_handle h, double ms[4], int64_t *calls);

/* The same record read per call: writes each timed call's interval from before its first kernel to
 * after its last (milliseconds, oldest first) into call_ms[0 .. min(*calls, capacity)), sets *calls
 * to the number of calls recorded, and clears the record (as w4moe_read_profile, which it replaces
 * for that read). */
w4moe_status w4moe_read_profile_calls(w4moe_handle h, double *call_ms, int64_t capacity, int64_t *calls);

/* Synchronises the handle's device and returns the device-side error flags raised since the last
 * read, then clears them. Bit 0: an id outside [0, E) was dropped. Bit 1: in the single-launch pair
 * mode (plan 3), a GEMM2 workgroup's wait for its entry's GEMM1 workgroups reached the wait limit
 * (w4moe_set_wait_limit) and went on without them: the output columns that workgroup served (64
 * columns of the entry's token, or all of them) are NaN in that call's out; other values and later
 * calls are unaffected (the per-entry hand-off state returns to zero within the call either way).
 * The same holds for plan 4 where it runs in one launch: a GEMM2 workgroup that gave up waiting for
 * its work item leaves NaN in the output columns it served for the item's tokens.
 * A wait can expire without any fault when the GPU runs other work for longer than the limit.
 * Bit 2: w4moe_prepack_act_order read a permutation value out of range. */
w4moe_status w4moe_device_error(w4moe_handle h, int32_t *flags);

/* Bound of the single-launch hand-off wait (plan 3, and plan 4 in one launch): how long a GEMM2
 * workgroup waits for its entry's or work item's GEMM1 workgroups before it gives up as described
 * under w4moe_device_error, in
 * microseconds of the GPU's constant clock. Negative restores the default (100000, i.e. 100 ms);
 * 0 makes every wait that does not find its entry finished at the first look give up at once, so
 * that tests can reach the give-up path from the host while every kernel still ends normally.
 * Applies to the calls that follow on this handle. */
w4moe_status w4moe_set_wait_limit(w4moe_handle h, int64_t microseconds);

/* Frees the handle's device memory. NULL-safe. */
void w4moe_destroy(w4moe_handle h);

const char *w4moe_status_string(w4moe_status s);
const char *w4moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* W4MOE_H */
