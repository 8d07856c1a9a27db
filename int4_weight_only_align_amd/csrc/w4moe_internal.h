// Internal declarations shared by the host runtime and the kernel translation units of libw4moe.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace w4moe {

constexpr int kGroup = 32;          // rows of the reduction dimension per scale
// One packed block: 4 groups x 64 columns of codes (one 4 KiB nibble plane for 4-bit codes, two for
// 8-bit ones: low nibbles, then high nibbles) followed by 512 B of their scales.
__host__ __device__ constexpr int block_bytes(int bits) { return bits == 8 ? 8704 : 4608; }
__host__ __device__ constexpr int code_bytes(int bits) { return bits == 8 ? 8192 : 4096; }
constexpr int kAlignBlock = 16;     // rows per MFMA token tile (forward's alignment block)
constexpr int kFusedMaxEntries = 128;  // entries T up to which pair mode can run as one launch
constexpr int kReadyStride = 64;       // words between two ready flags (256 bytes)
constexpr int kWideReadyStride = 16;   // the single-launch wide plan's flags (64 bytes apart; rarely polled)
constexpr int kSplitSlots = 8192;      // partial-sum slots (superblock x split) per GEMM and call
constexpr int kMaxSplit = 16;          // workgroups one superblock's reduction may be split over
constexpr int kMaxExperts = 1024;   // the alignment kernel keeps per-expert state in LDS

// Expert parallelism: routing ids name experts of the whole layer (E_all of them); this layer holds
// [e_first, e_first + E). The local index of an id (unsigned arithmetic, so any id maps without
// overflow); an id in [0, E_all) outside the local range belongs to another shard and contributes
// nothing, an id outside [0, E_all) is an error (dropped, flag bit 0). Unsharded: e_first = 0, E_all = E.
__host__ __device__ inline int local_expert(int32_t id, int32_t e_first) {
    return (int)((uint32_t)id - (uint32_t)e_first);
}
__host__ __device__ inline bool bad_expert(int32_t id, int32_t E_all) { return (uint32_t)id >= (uint32_t)E_all; }

// Work item of the grouped GEMMs: rows [p0, p0 + nrows) of the sorted order, all routed to expert e.
// flags: kItemShared when the expert has more rows than one item holds, so that other items of the
// same launch stream the same weights (which the GEMMs then load with the caches' default policy).
struct WorkItem {
    int32_t e, p0, nrows, flags;
};
constexpr int32_t kItemShared = 1;

struct AlignArgs {
    const int32_t *ids;      // flat routing ids [T]
    int32_t T, E, B, CH;     // entries, experts, block rows, rows per work item (multiple of B)
    int32_t *counts;         // [E]
    int32_t *offsets;        // [E + 1]
    int32_t *sorted_ids;     // [T + min(E,T)(B-1)]
    int32_t *block_expert;   // [(T + min(E,T)(B-1)) / B]
    int32_t *active;         // [E]
    int32_t *n_active;       // [1]
    WorkItem *work;          // [T/CH + min(E,T)]
    int32_t *n_work;         // [1]
    int32_t *err;            // [1] bit 0: an id outside [0, E_all) was dropped
    int32_t e_first, E_all;  // expert range of this layer within the whole layer (local_expert)
    // above 1024 entries (two launches): per-chunk expert counts, then their per-chunk prefixes
    int32_t *hist;           // [ceil(T / 1024)][E]
    int32_t *arrive;         // [1], zero between calls
};

struct PrepackArgs {
    const int32_t *codes;    // logical words of experts [e0, e0+ne): [ne][R/8][C]
    const uint16_t *scales;  // [ne][R/group][C]
    uint8_t *packed;         // packed matrix base (expert 0)
    int32_t e0, ne, R, C, N; // R: reduction rows, C: output columns, N: intermediate width (W1 column map);
                             // packed rows and columns past R and C (up to whole blocks) are padding
    int32_t is_w1;
    int32_t group;           // rows per logical scale: 32, 64 or 128 (the packed layout keeps one per 32 rows)
    int32_t bits;            // code width: 4 (8 codes per word) or 8 (4 codes per word)
    // activation order: packed row i holds logical row row_perm[i] ([ne][R], or null for none); for
    // W1, packed gate / up column n holds logical column col_perm[n] / N + col_perm[n] ([ne][N], or
    // null). Values outside range raise bit 2 of err and read as 0.
    const int32_t *row_perm;
    const int32_t *col_perm;
    int32_t *err;
};

// Activation order at run time: xg[f][i] = x[f / topk][perm[ids[f]][i]] for every flat entry f
// whose id lies in [0, E) (the others are left as they are: no GEMM reads them).
struct GatherArgs {
    const uint16_t *x;       // bf16 [M][K]
    const int32_t *ids;      // [T]
    const uint16_t *perm;    // [E][K]: the group-sorted order of each expert's hidden features
    int32_t T, K, topk, E;   // K: the padded row length Kp (a multiple of 128)
    uint16_t *xg;            // bf16 [T][K]
    int32_t e_first;         // global id of local expert 0 (local_expert)
};

struct GemmArgs {
    // pair mode: work item i is flat routing entry i (expert ids[i], row i), no alignment pass
    int32_t pair_mode;
    int32_t dedup;               // pair mode, n_items <= 128: entries of one expert share a work item (two at a time)
    int32_t bits;                // code width of the packed weights: 4 or 8
    const int32_t *ids;          // flat routing ids [T] (pair mode)
    int32_t n_items;             // T (pair mode)
    int32_t E;
    uint32_t dq_mask, dq_exp;    // 0x000F000F and 0x43004300, passed at run time so that the decode
    uint32_t dq_zero;            // compiles to one v_and_or_b32 per bf16 pair; dq_zero is 0
    const uint8_t *wpk;          // packed matrix base (expert 0)
    int32_t ncs, gq_total;       // column superblocks (64 columns) and group quads (128 rows)
    const uint16_t *act;         // GEMM1: hidden [M][Kp] (gathered by token); GEMM2: a1 [P][Np] (sorted rows)
    int64_t act_ld;              // elements per activation row: gq_total * 128 (whole group quads)
    int32_t act_len;             // elements of a row that hold data; staging fills the rest with zeros
    int32_t act_div;             // GEMM1: flat entry f reads activation row f / act_div (topk: the token's
                                 // hidden row; 1: the entry's own row, gathered in activation order)
    const uint16_t *perm;        // pair-mode GEMM1 in activation order: [E][act_ld] feature order of each
                                 // expert; the staged row is act[f / act_div][perm[e][i]] (null: none)
    int32_t perm_lds;            // 1: the row is staged in LDS in its own order and permuted there (the
                                 // workgroup holds two rows of LDS); 0: gathered from global memory
    const int32_t *sorted_ids;   // [P]
    const WorkItem *work;
    const int32_t *n_work;
    int32_t topk, ncb;           // top-k; column blocks per work item (grid = max items * ncb)
    int32_t sbw;                 // wide GEMM2 over <= 2 group quads: superblocks per wave (1: one)
    uint16_t *a1;                // GEMM1 output, bf16 [P][Np] (columns [N, Np) are never written)
    int64_t a1_ld;
    float *y;                    // pair-mode GEMM2 output, fp32 [T][Kc], already multiplied by the routing weight
    uint16_t *yb;                // aligned-mode GEMM2 output, the same rounded to bf16 [T][Kc] (same buffer)
    int64_t y_ld;                // Kc = ncs * 64 (GEMM2)
    const float *topk_w;         // [T]
    // pair-mode GEMM2 fuses the top-k combine
    uint16_t *out;               // bf16 [M][out_ld]; columns from out_len on are not stored
    int64_t out_ld;
    int32_t out_len;
    int32_t *counters;           // [max_tokens][ncs], zero between calls
    int32_t *err;                // [1] bit 0: a dropped id was seen; bit 1: a bounded wait timed out
                                 // (bit 2: a permutation value out of range, raised by the prepack)
    // fused pair mode: GEMM1 superblocks count themselves per entry; the last raises the ready
    // flags of the entry's GEMM2 workgroups
    int32_t *done;               // [kFusedMaxEntries], zero between calls
    int32_t *ready;              // [kFusedMaxEntries * ready_n * kReadyStride], zero between calls (each flag
                                 // gets one +1 and one -1 per launch)
    int32_t phases;              // fused pair mode: entry groups, each dispatched as its GEMM1 then its GEMM2 workgroups
    int32_t done_target;         // GEMM1 superblocks per entry
    int32_t ready_n;             // GEMM2 workgroups per entry
    int64_t wait_ticks;          // bound of a GEMM2 workgroup's wait, in ticks of the 100 MHz constant clock
    // pair mode, reduction split across xsplit workgroups: each writes its partial sums of a
    // superblock to its own slot; the last of them (xcnt) adds the slots in order and finishes
    int32_t xsplit;              // 1 = no split
    float *part;                 // [T][ncs][xsplit][64]
    int32_t *xcnt;               // [T][ncs], zero between calls
    int32_t e_first, E_all;      // pair mode: expert range of this layer within the whole layer
};

struct RouteArgs {
    const float *logits;         // [M][E] fp32
    int32_t M, E, k;
    int32_t *ids;                // [M][k] out
    float *w;                    // [M][k] out
    int32_t *err;                // [1] bit 0 raised for a slot left without a candidate (NaN logits)
};

struct CombineArgs {
    const uint16_t *y;           // bf16 [T][y_ld]
    const int32_t *ids;          // [T]
    int32_t M, K, topk, E;       // K: output columns (a multiple of 8)
    int32_t y_ld;
    uint16_t *out;               // bf16 [M][K]
    int32_t *err;                // [1] bit 0 raised for a slot whose id lies outside [0, E_all)
    int32_t e_first, E_all;      // expert range of this layer (local_expert): remote slots add nothing
};

hipError_t launch_prepack(const PrepackArgs &a, int ncs, int gq_total, hipStream_t s);
// Keeps an activation-order permutation of hidden features for the run-time gather: dst[(e0+el)*Kp + i]
// = perm[el*K + i] for el < ne and i < K (values outside [0, K) raise bit 2 of err and are stored as
// 0), and K for K <= i < Kp (the padded hidden row holds 0 there).
hipError_t launch_store_perm(const int32_t *perm, int32_t e0, int32_t ne, int32_t K, int32_t Kp, uint16_t *dst,
                             int32_t *err, hipStream_t s);
hipError_t launch_gather(const GatherArgs &a, hipStream_t s);
// xp[m][i] = x[m][i] (i < K), 0 (K <= i < Kp) for m < M; K and Kp multiples of 8.
hipError_t launch_pad_rows(const uint16_t *x, int32_t M, int32_t K, int32_t Kp, uint16_t *xp, hipStream_t s);
hipError_t launch_align(const AlignArgs &a, hipStream_t s);
// pair: one (token, slot) entry per item, the token row staged in LDS; otherwise items come from the
// alignment. S (1, 2 or 4) waves of a workgroup split the reduction of one 64-column superblock; the
// workgroup covers 4 / S superblocks (a.ncb superblock groups per item). max_rows (16, 32 or 64)
// bounds the rows of an item; 64-row items run the wide kernel (S must be 1), whose workgroup stages
// the item's token rows in LDS for its four superblocks.
// kSorted: aligned work items of up to max_rows rows (16 or 32), A fragments from global memory;
// kWide: aligned items of up to max_rows rows (32 or 64) with the rows staged in LDS; kPair: pair mode.
enum class GemmKind { kSorted, kWide, kPair };
hipError_t launch_gemm(bool gemm1, GemmKind kind, int S, int max_rows, const GemmArgs &a, int64_t items,
                       hipStream_t s);
// Both pair-mode GEMMs in one launch (GEMM1 workgroups first; GEMM2 waits per entry). skip_dropped:
// the workgroups of dropped entries (another shard's experts, on an expert shard) skip the hand-off.
// The wide plan's two GEMMs in one launch (4-bit codes, items of at most 48 rows): g1.done [items] and
// g1.ready = g2.ready [items * g2.ncb * kWideReadyStride] zero between calls.
hipError_t launch_wide_fused(const GemmArgs &g1, const GemmArgs &g2, int64_t items, hipStream_t s);
hipError_t launch_pair_fused(int S1, int S2, const GemmArgs &g1, const GemmArgs &g2, bool skip_dropped,
                             hipStream_t s);
hipError_t launch_combine(const CombineArgs &a, hipStream_t s);
hipError_t launch_route(const RouteArgs &a, hipStream_t s);

}  // namespace w4moe
