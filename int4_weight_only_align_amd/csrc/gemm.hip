// Grouped W4A16 GEMMs of the MoE layer for gfx950: GEMM1 (gate|up, fused SiLU(gate)*up epilogue)
// and GEMM2 (down projection, routing-weight epilogue).
//
// What is computed (pages: "The Pivot to Real Hardware...", Step 1: Understanding the Weight
// Format; "The Commit That Captured a Plateau", Regime 1 and Regime 2): for every row p routed to
// expert e,
//   GEMM1: a1[p][n] = bf16( SiLU(sum_k x[tok(p)][k] W1_e[k][n]) * sum_k x[tok(p)][k] W1_e[k][N+n] )
//   GEMM2: y[f(p)][c] = w[f(p)] * sum_n a1[p][n] W2_e[n][c]
// with W[k][c] = q[k][c] * s[k/32][c], q a signed 4-bit code.
//
// How (gfx950, wave64):
//  * Tokens are the A operand of v_mfma_f32_16x16x32_bf16 (16 token rows per tile, padded) and the
//    weights the B operand, so one MFMA covers 16 output columns x one 32-row scale group.
//  * A lane's B operand is exactly one packed 32-bit word (8 codes of one column): it becomes four
//    bf16 pairs with three shifts and four v_and_or_b32 (mask the two codes of a pair, OR in the
//    exponent pattern of 128.0), giving the exact values 128 + code = 136 + q (the "magic number"
//    conversion of Kim et al. 2022, "Who Says Elephants Can't Run"). An MFMA against a constant -136 operand yields
//    -136 * sum_k x[k] per token row; it enters the four weight MFMAs as their C operand, so each
//    result is exactly sum_k x[k] q[k] (fp32 accumulation). One fp32 FMA per output then applies
//    the group scale; no scale rounding enters the weights.
//  * Each wave streams packed blocks (4 KiB of codes + 512 B of scales = 64 columns x 128 rows)
//    with 128-bit loads that are contiguous across the wave, through a register ring of kRing blocks
//    (kRing - 1 blocks in flight while one is consumed; no register copies, exact waitcnts). The
//    blocks load non-temporal, so the weight stream does not evict the activation rows the
//    workgroups re-read (an expert read again by other work items of the launch is the exception).
//  * Padding token rows read a valid row (their results are never stored), so their loads are
//    unconditional.
#include "w4moe_internal.h"

namespace w4moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRing = 3;   // blocks held per wave: two in flight while one is consumed

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 8 codes (row t at bit 0,16,4,20,8,24,12,28) -> bf16 values 128 + code for rows 0..7 in order.
// `mask` is uniform (SGPR) and `expo` is held per lane (VGPR), so each pair compiles to one
// v_and_or_b32 (a VALU op may read only one SGPR).
__device__ __forceinline__ bf16x8 decode_word(uint32_t w, uint32_t mask, uint32_t expo) {
    u32x4 v;
    v.x = (w & mask) | expo;
    v.y = ((w >> 4) & mask) | expo;
    v.z = ((w >> 8) & mask) | expo;
    v.w = ((w >> 12) & mask) | expo;
    return as_bf16x8(v);
}

// The exponent pattern as a per-lane value: OR-ing in lane bits masked by a run-time zero keeps
// the compiler from folding it back into a uniform constant.
__device__ __forceinline__ uint32_t lane_expo(const GemmArgs &a) { return a.dq_exp | (threadIdx.x & a.dq_zero); }

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld128(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
// 16 bytes as two agent-coherent 8-byte loads: data another workgroup of the same launch published,
// possibly from another XCD (whose L2 holds no copy of this one's lines)
__device__ __forceinline__ u32x4 ld128_agent(const void *p) {
    const uint64_t *q = reinterpret_cast<const uint64_t *>(p);
    const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return u32x4{(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
}

// The ring's last loads repeat the final block and their results are never read. The backend may
// hand their destination registers to later values while those loads are still in flight, so every
// ring loop ends by waiting for all of its loads.
__device__ __forceinline__ void drain_loads() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ float bf16_word_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_word_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// The four scales of group gsub (slots j = 0..3) from the lane's 16 scales (index gsub*4 + j).
__device__ __forceinline__ void scales_of(const u32x4 s[2], int gsub, float out[4]) {
    const u32x4 v = s[gsub >> 1];
    const uint32_t w0 = v[(gsub & 1) * 2], w1 = v[(gsub & 1) * 2 + 1];
    out[0] = bf16_word_lo(w0);
    out[1] = bf16_word_hi(w0);
    out[2] = bf16_word_lo(w1);
    out[3] = bf16_word_hi(w1);
}

// Block format per code width. 4-bit: one 4 KiB nibble plane (128 + code = 136 + q) and a bias of
// -136 per row. 8-bit: code u = q + 128 split into a low-nibble plane (128 + (u & 15)) and a
// high-nibble plane decoded with the exponent pattern of 2048 (2048 + 16 * (u >> 4), exact in bf16:
// 128 + h scaled by 16); the two chained MFMAs give sum x * (2176 + u), and the bias of -2304 per
// row leaves sum x * q. The 512 B of scales follow the planes.
template <int BITS>
struct Fmt;
template <>
struct Fmt<4> {
    static constexpr int kPlanes = 1, kCode = 4096, kBlock = 4608;
    static constexpr uint32_t kBias = 0xC308C308u;   // bf16 -136, twice
};
template <>
struct Fmt<8> {
    static constexpr int kPlanes = 2, kCode = 8192, kBlock = 8704;
    static constexpr uint32_t kBias = 0xC510C510u;   // bf16 -2304, twice
};
constexpr uint32_t kHiPlaneExpo = 0x02000200u;      // 0x4300 + 0x0200 = 0x4500: the pattern of 2048

template <int BITS>
struct WStage {
    u32x4 w[4 * Fmt<BITS>::kPlanes];   // plane p, group gsub: four words (slots j) per lane at [p * 4 + gsub]
    u32x4 s[2];                        // 16 bf16 scales: index gsub*4 + j
};

// STREAM: the block's codes and scales are loaded non-temporal (the caches give them a streaming
// policy, so they do not displace the staged activation rows and the other workgroups' data); an
// item whose expert other items of the same launch read again loads them with the default policy.
template <int BITS, bool STREAM = true>
__device__ __forceinline__ void load_w(WStage<BITS> &st, const uint8_t *wl, const uint8_t *sl, int i) {
    auto ld = [](const uint8_t *p) {
        if constexpr (STREAM) return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
        else return ld128(p);
    };
    const uint8_t *b = wl + (int64_t)i * Fmt<BITS>::kBlock;
#pragma unroll
    for (int p = 0; p < Fmt<BITS>::kPlanes; ++p)
#pragma unroll
        for (int g = 0; g < 4; ++g) st.w[p * 4 + g] = ld(b + p * 4096 + g * 1024);
    const uint8_t *s = sl + (int64_t)i * Fmt<BITS>::kBlock;
    st.s[0] = ld(s);
    st.s[1] = ld(s + 16);
}

// The decoded B operands of group gsub: slot j of plane p at [p * 4 + j].
template <int BITS>
struct BOps {
    bf16x8 b[4 * Fmt<BITS>::kPlanes];
};

template <int BITS>
__device__ __forceinline__ void decode_group(const WStage<BITS> &c, int g, uint32_t mask, uint32_t expo,
                                             BOps<BITS> &o) {
#pragma unroll
    for (int j = 0; j < 4; ++j) o.b[j] = decode_word(c.w[g][j], mask, expo);
    if constexpr (BITS == 8) {
        const uint32_t expo_hi = expo + kHiPlaneExpo;
#pragma unroll
        for (int j = 0; j < 4; ++j) o.b[4 + j] = decode_word(c.w[4 + g][j], mask, expo_hi);
    }
}

// d[j] = sum over the group's 32 rows of a * q for the four 16-column slots (exact products, fp32
// sums): a bias MFMA, then the code MFMAs chained through the C operand.
template <int BITS>
__device__ __forceinline__ void dot_group(bf16x8 a, const BOps<BITS> &o, f32x4 d[4]) {
    const uint32_t kb = Fmt<BITS>::kBias;
    const bf16x8 bias_b = as_bf16x8(u32x4{kb, kb, kb, kb});
    const f32x4 bias = mfma16(a, bias_b, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int j = 0; j < 4; ++j) d[j] = mfma16(a, o.b[j], bias);
    if constexpr (BITS == 8) {
#pragma unroll
        for (int j = 0; j < 4; ++j) d[j] = mfma16(a, o.b[4 + j], d[j]);
    }
}

// ---------------------------------------------------------------------------------------------
// Single token row (pair mode): the row lives in LDS, every MFMA row carries it, only element 0 of
// each lane's result is accumulated (lane l holds column l % 16 of each 16-column slot).
// ---------------------------------------------------------------------------------------------
// `between` runs after the first weight loads are issued and before the first block is consumed
// (the caller stages the token rows there, so HBM is busy during the workgroup prologue).
// NR token rows (1 or 2) sit in LDS xs_ld elements apart: MFMA row 0 carries row 0 and rows 1..15
// carry row NR - 1, so lane l < 16 finds row q of its column in element q of each result.
template <int NR>
__device__ __forceinline__ const uint16_t *row_of_lane(const uint16_t *xs, int xs_ld, int lane) {
    return NR > 1 ? xs + min(lane & 15, NR - 1) * xs_ld : xs;
}

template <int BITS, int NR>
__device__ __forceinline__ void consume_block(const WStage<BITS> &c, const uint16_t *xg, uint32_t mask, uint32_t expo,
                                              float acc[NR][4]) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4 *>(xg + g * kGroup));
        BOps<BITS> b;
        decode_group<BITS>(c, g, mask, expo, b);
        f32x4 d[4];
        dot_group<BITS>(a, b, d);
        float s[4];
        scales_of(c.s, g, s);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < NR; ++q) acc[q][j] += s[j] * d[j][q];
    }
}

template <int BITS, int R, int NR, bool kSkipTail, typename Between>
__device__ __forceinline__ void mainloop_row(const uint8_t *__restrict__ wl, const uint8_t *__restrict__ sl,
                                             int ngq, int gq0, const uint16_t *xs, int xs_ld, int lane, uint32_t mask,
                                             uint32_t expo, float acc[NR][4], Between between) {
    const uint16_t *xr = row_of_lane<NR>(xs, xs_ld, lane) + (lane >> 4) * 8;
    const int last = max(ngq - 1, 0);
    WStage<BITS> st[R];
    // kSkipTail: past the end no block is loaded (a repeat of the last one, streamed non-temporal,
    // would miss the caches and cost its bytes again). Elsewhere the last block is repeated: skipping
    // costs the 8-bit single-launch kernel a wave per SIMD (175 VGPRs instead of 150) and makes the
    // two-launch pair kernels, held to 128 VGPRs, spill.
    auto load = [&](int i) {
        if constexpr (kSkipTail) {
            if (i <= last) load_w<BITS>(st[i % R], wl, sl, i);
        } else {
            load_w<BITS>(st[i % R], wl, sl, min(i, last));
        }
    };
#pragma unroll
    for (int r = 0; r < R - 1; ++r) load(r);
    between();
    for (int i0 = 0; i0 < ngq; i0 += R) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = i0 + r;
            load(i + R - 1);
            if (i < ngq) consume_block<BITS, NR>(st[r], xr + (gq0 + i) * 128, mask, expo, acc);
        }
    }
    drain_loads();
}

// The whole share of a wave (ngq <= NB blocks) is loaded before `between` runs: a wave that waits
// inside `between` (GEMM2 of the single-launch pair mode) holds all of its weights when it is
// released, so only the token rows and the MFMAs remain after the hand-off.
template <int BITS, int NB, int NR, bool kSkipTail, typename Between>
__device__ __forceinline__ void mainloop_row_all(const uint8_t *__restrict__ wl, const uint8_t *__restrict__ sl,
                                                 int ngq, int gq0, const uint16_t *xs, int xs_ld, int lane,
                                                 uint32_t mask, uint32_t expo, float acc[NR][4], Between between) {
    const uint16_t *xr = row_of_lane<NR>(xs, xs_ld, lane) + (lane >> 4) * 8;
    const int last = max(ngq - 1, 0);
    WStage<BITS> st[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        if constexpr (kSkipTail) {
            if (i <= last) load_w<BITS>(st[i], wl, sl, i);
        } else {
            load_w<BITS>(st[i], wl, sl, min(i, last));
        }
    }
    between();
#pragma unroll
    for (int i = 0; i < NB; ++i)
        if (i < ngq) consume_block<BITS, NR>(st[i], xr + (gq0 + i) * 128, mask, expo, acc);
    drain_loads();
}

// ---------------------------------------------------------------------------------------------
// Up to NT tiles of 16 token rows, A fragments loaded from global memory with the block they go with.
// ---------------------------------------------------------------------------------------------
template <int NT>
struct AStage {
    u32x4 a[NT][4];
};

template <int NT>
__device__ __forceinline__ void load_a(AStage<NT> &st, const uint16_t *const arow[NT], int gq, int koff) {
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int g = 0; g < 4; ++g) st.a[tt][g] = ld128(arow[tt] + (gq * 4 + g) * kGroup + koff);
}

template <int BITS, int NT>
__device__ __forceinline__ void mainloop_tiles(const uint8_t *__restrict__ wl, const uint8_t *__restrict__ sl,
                                               int ngq, int gq0, const uint16_t *const arow[NT], int lane,
                                               uint32_t mask, uint32_t expo, f32x4 acc[NT][4]) {
    if (ngq <= 0) return;
    const int koff = (lane >> 4) * 8;
    const int last = ngq - 1;
    WStage<BITS> st[kRing];
    AStage<NT> as[kRing];
#pragma unroll
    for (int r = 0; r < kRing - 1; ++r) {
        load_w<BITS>(st[r], wl, sl, min(r, last));
        load_a<NT>(as[r], arow, gq0 + min(r, last), koff);
    }
    for (int i0 = 0; i0 < ngq; i0 += kRing) {
#pragma unroll
        for (int r = 0; r < kRing; ++r) {
            const int i = i0 + r;
            const int nxt = min(i + kRing - 1, last);
            load_w<BITS>(st[(r + kRing - 1) % kRing], wl, sl, nxt);
            load_a<NT>(as[(r + kRing - 1) % kRing], arow, gq0 + nxt, koff);
            if (i < ngq) {
                const WStage<BITS> &c = st[r];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    BOps<BITS> b;
                    decode_group<BITS>(c, g, mask, expo, b);
                    float s[4];
                    scales_of(c.s, g, s);
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt) {
                        const bf16x8 a = as_bf16x8(as[r].a[tt][g]);
                        f32x4 d[4];
                        dot_group<BITS>(a, b, d);
#pragma unroll
                        for (int j = 0; j < 4; ++j) acc[tt][j] += s[j] * d[j];
                    }
                }
            }
        }
    }
    drain_loads();
}

// Output row layout of the MFMA result: lane holds rows 4*(lane/16) + r (r = 0..3) of column lane%16.
// COH (GEMM1 of the single-launch wide plan): the SwiGLU rows are stored agent-coherent, for GEMM2
// workgroups of the same launch. late (its GEMM2): the hand-off wait gave up, the slot outputs are NaN.
template <bool G1, int NT, bool COH = false>
__device__ __forceinline__ void epilogue(const GemmArgs &a, const WorkItem &it, int cs, int lane, f32x4 acc[NT][4],
                                         bool late = false) {
    const int col = lane & 15;
    if constexpr (G1) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = tt * 16 + (lane >> 4) * 4 + r;
                if (row >= it.nrows) continue;
                uint16_t *dst = a.a1 + (it.p0 + row) * a.a1_ld + cs * 32 + col;
                const uint16_t v0 = f32_to_bf16_rne(silu(acc[tt][0][r]) * acc[tt][2][r]);
                const uint16_t v1 = f32_to_bf16_rne(silu(acc[tt][1][r]) * acc[tt][3][r]);
                if constexpr (COH) {
                    __hip_atomic_store(dst, v0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(dst + 16, v1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                } else {
                    dst[0] = v0;
                    dst[16] = v1;
                }
            }
        }
    } else {
        // each slot's weighted output, rounded to bf16 (the combine adds the slots in fp32). The rows'
        // slot ids are loaded together, then their routing weights together (rows past the item's
        // end load its last row's, unused), so the epilogue waits two round trips, not two per row.
        int32_t f[NT][4];
        float wt[NT][4];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                f[tt][r] = a.sorted_ids[it.p0 + min(tt * 16 + (lane >> 4) * 4 + r, it.nrows - 1)];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) wt[tt][r] = late ? __int_as_float(0x7FC00000) : a.topk_w[f[tt][r]];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (tt * 16 + (lane >> 4) * 4 + r >= it.nrows) continue;
                uint16_t *dst = a.yb + (int64_t)f[tt][r] * a.y_ld + cs * 64 + col;
#pragma unroll
                for (int j = 0; j < 4; ++j) dst[16 * j] = f32_to_bf16_rne(wt[tt][r] * acc[tt][j][r]);
            }
        }
    }
}

// Per-lane activation rows of the NT tiles; padding rows point at the item's first row.
template <bool G1, int NT>
__device__ __forceinline__ void setup_rows(const GemmArgs &a, const WorkItem &it, int lane, const uint16_t *arow[NT]) {
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
        int row = tt * 16 + (lane & 15);
        if (row >= it.nrows) row = 0;
        const int64_t p = it.p0 + row;
        const int64_t r = G1 ? (int64_t)(a.sorted_ids[p] / a.act_div) : p;
        arow[tt] = a.act + r * a.act_ld;
    }
}

// The 8 bf16 of `row` at the 8 feature indices packed in p (index t in the low or high half of word
// t / 2): one chunk of a row in activation order.
__device__ __forceinline__ u32x4 gather8(const uint16_t *row, u32x4 p) {
    u32x4 v;
#pragma unroll
    for (int w = 0; w < 4; ++w) v[w] = (uint32_t)row[p[w] & 0xFFFFu] | ((uint32_t)row[p[w] >> 16] << 16);
    return v;
}

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Workgroup geometry: the four waves cover SPW = 4 / S superblocks, S waves per superblock, each of
// those taking one contiguous slice of the group quads. The S partial sums of a superblock are
// added in LDS in slice order (deterministic) by its slice-0 wave, which runs the epilogue.
template <int S>
struct Geo {
    static constexpr int SPW = 4 / S;
    int cs, ks, gq0, gq1;
    bool active;
    // wave `wave` of the workgroup for superblock group cb and reduction part x of X
    __device__ Geo(const GemmArgs &a, int cb, int wave, int x = 0, int X = 1) {
        cs = cb * SPW + wave / S;
        ks = wave % S;
        active = cs < a.ncs;
        const int lo = x * a.gq_total / X, len = (x + 1) * a.gq_total / X - lo;
        gq0 = lo + ks * len / S;
        gq1 = lo + (ks + 1) * len / S;
    }
};

// Pair mode: workgroup = (flat entry f, superblock group cb, reduction part x of X). The activation
// row (x[f / topk], or the entry's gathered row f in activation order, for GEMM1; a1[f] for GEMM2)
// is staged in LDS once per workgroup. With X > 1 each
// workgroup writes its partial sums of a superblock to slot x, and the last of the X to arrive (a
// per-(f, cs) counter) adds the X slots in slot order -- the same order whichever arrives last -- and
// finishes the superblock as an unsplit workgroup would. GEMM2 also performs the top-k
// combine: the last of the topk workgroups of token m and superblock cs to finish (a per-(m, cs)
// counter) sums y[m*topk + j][cs's 64 columns] over j in slot order and writes out[m]; it then
// resets the counter for the next call.
//
// FUSED: both GEMMs run in one launch, GEMM1 workgroups first. A GEMM1 superblock publishes its a1
// slice with agent-coherent stores, waits for their completion and counts itself in done[f]; the
// last one of entry f re-zeroes done[f] and adds 1 to the ready flag of every GEMM2 workgroup of the
// entry. The flags sit kReadyStride words apart, so the waiting workgroups poll distinct cache lines
// (and memory channels) rather than one hot line. A GEMM2 workgroup issues its first weight loads,
// waits until its flag is positive, subtracts 1 from it and reads the row with agent-coherent loads.
// Each flag thus receives exactly one +1 and one -1 per launch, in either order, and is zero again
// when the launch ends -- also when a wait gives up: the wait is bounded by a.wait_ticks of the
// constant clock, after which the workgroup raises error bit 1, still subtracts its 1 (the late +1
// brings the flag back to zero within the same launch, so no later call can be released by it) and
// writes NaN in place of its results, so the affected output columns of the token read NaN.
// Workgroups are dispatched in index order, so every GEMM1 workgroup a GEMM2 workgroup waits for has
// already been dispatched; the bound only guarantees that every wave finishes.
constexpr int kG2Blocks = 4;                 // GEMM2 blocks a waiting wave may hold in registers

// kSkipDropped (single-launch mode on an expert shard, where most entries are other shards'): the
// workgroups of a dropped entry take no part in the ready-flag hand-off (see below); otherwise they
// count themselves and pass flags like any other.
//
// Deduplicated items (a.dedup, up to 64 entries): the entries routed to the same local expert are
// taken kItemRows at a time in flat order, and the workgroups of the first entry of each such item
// stream the expert's weights once for all of its entries (MFMA rows 0 and 1 carry their rows); the
// workgroups of the other entries end at once. Without it every entry is an item of its own.
constexpr int kItemRows = 2;
constexpr int kSplitBatch = 4;   // partial slots of a split reduction whose loads are in flight together
constexpr int kSlotBatch = 8;    // slots of a token whose loads the combining workgroup issues together
constexpr uint64_t kNaNx4 = 0x7FC07FC07FC07FC0ull;   // four bf16 quiet NaNs

// The item's entries f0 < f1 (f1 = f0 when it has one) and staged rows of NR (1 or 2) entries.
template <bool G1, int S, bool FUSED, int R, int BITS, bool kSkipDropped, int NR>
__device__ __forceinline__ void pair_item_body(const GemmArgs &a, int bid, int f0, int f1, uint16_t *xs) {
    constexpr int SPW = 4 / S;
    __shared__ float red[SPW][S][NR][4][16];
    const int per_entry = a.ncb * a.xsplit;
    const int r = bid % per_entry, cb = r % a.ncb, x = r / a.ncb;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const Geo<S> geo(a, cb, wave, x, a.xsplit);
    const int fr[2] = {f0, f1};
    const int e = local_expert(a.ids[f0], a.e_first);
    const bool valid = (unsigned)e < (unsigned)a.E;   // uniform over the workgroup; false for remote entries
    // GEMM2: the entries' routing weights, read now so that the epilogue's slot stores need not wait
    // for them after the MFMAs
    float wt[NR];
#pragma unroll
    for (int q = 0; q < NR; ++q) wt[q] = G1 ? 0.f : a.topk_w[fr[q]];
    const int xs_ld = (int)a.act_ld;                   // LDS row q of the item at xs + q * xs_ld
    const uint16_t *row = a.act + (int64_t)(G1 ? f0 / a.act_div : f0) * a.act_ld;
    const int nchunk = a.act_ld / 8;                    // 16-byte chunks of the row

    // GEMM2 of the fused launch: wait for the item's a1 rows, then stage them. Thread 0 reads the flag
    // once before the weight loads are issued (`early`): loads complete in order, so that read returns
    // ahead of the weights, and a workgroup that starts after its item's GEMM1 finished issues the
    // a1 row loads while its weights are still in flight. Otherwise it polls behind them.
    __shared__ int s_late;   // GEMM2 of the fused launch: the bounded wait gave up
    int32_t early = 0;
    if (FUSED && !G1 && valid && tid == 0)
        early = __hip_atomic_load(a.ready + ((int64_t)f0 * a.ready_n + r) * kReadyStride, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
    auto wait_and_stage = [&]() {
        if (tid == 0) {
            asm volatile("" : "+v"(early));   // read here, behind the weight loads, not where it was loaded
            int32_t *flag = a.ready + ((int64_t)f0 * a.ready_n + r) * kReadyStride;
            const long long t0 = wall_clock64();
            int late = 0;
            while (early <= 0 && __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <= 0) {
                if (wall_clock64() - t0 >= a.wait_ticks) {
                    atomicOr(a.err, 2);
                    late = 1;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
            __hip_atomic_fetch_add(flag, -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_late = late;
        }
        __syncthreads();
        // after an expired wait the rows read are not the item's: NaN is staged in their place, so this
        // workgroup's share of the output comes out NaN
        const bool late = s_late;
        if (valid) {   // four 8-byte loads in flight per thread; past the end they repeat the last word
            // (features past act_len are staged as zeros: the row's padding up to whole group quads)
            const int n64 = a.act_ld / 4, nval = a.act_len / 4;
#pragma unroll
            for (int q = 0; q < NR; ++q) {
                const uint64_t *row64 = reinterpret_cast<const uint64_t *>(a.act + (int64_t)fr[q] * a.act_ld);
                uint64_t *xs64 = reinterpret_cast<uint64_t *>(xs + q * xs_ld);
                for (int i0 = tid; i0 < n64; i0 += 4 * 256) {
                    uint64_t v[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        v[c] = __hip_atomic_load(row64 + min(i0 + c * 256, nval - 1), __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int j = min(i0 + c * 256, n64 - 1);
                        xs64[j] = late ? kNaNx4 : j < nval ? v[c] : 0ull;
                    }
                }
            }
        }
        __syncthreads();
    };

    float acc[NR][4];
#pragma unroll
    for (int q = 0; q < NR; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[q][j] = 0.f;
    if (valid) {
        const int cs = min(geo.cs, a.ncs - 1);           // inactive waves stream nothing but share the barrier
        const int ngq = geo.active ? geo.gq1 - geo.gq0 : 0;
        const uint8_t *blk = a.wpk + (((int64_t)e * a.ncs + cs) * a.gq_total + geo.gq0) * Fmt<BITS>::kBlock;
        const uint8_t *wl = blk + lane * 16, *sl = blk + Fmt<BITS>::kCode + (lane & 15) * 32;
        if (FUSED && !G1) {
            // a share of up to kG2Blocks 4-bit blocks is held whole across the wait (8-bit blocks are
            // twice the registers and keep the ring)
            if (BITS == 4 && ngq <= kG2Blocks)
                mainloop_row_all<BITS, kG2Blocks, NR, BITS == 4>(wl, sl, ngq, geo.gq0, xs, xs_ld, lane, a.dq_mask, lane_expo(a), acc,
                                                      wait_and_stage);
            else
                mainloop_row<BITS, R, NR, BITS == 4>(wl, sl, ngq, geo.gq0, xs, xs_ld, lane, a.dq_mask, lane_expo(a), acc,
                                          wait_and_stage);
        } else {
            // row chunks of the first entry -- in activation order, the chunks of the expert's feature
            // order -- are loaded before the weight prologue so that waiting for them leaves the weight
            // loads in flight; a second row is loaded while the prologue is in flight
            constexpr int kPre = 4;
            const uint16_t *prow = (G1 && a.perm) ? a.perm + (int64_t)e * a.act_ld : nullptr;   // uniform
            const uint16_t *src = prow ? prow : row;
            u32x4 pre[kPre];
#pragma unroll
            for (int c = 0; c < kPre; ++c) pre[c] = ld128(src + min(tid + c * 256, nchunk - 1) * 8);
            // activation order staged through LDS: the row's own chunks load beside the feature order,
            // and the gather runs on LDS (no dependent global round trip before GEMM1 starts)
            const bool lds_perm = prow && a.perm_lds;   // uniform
            u32x4 nat[kPre];
            if (lds_perm) {
#pragma unroll
                for (int c = 0; c < kPre; ++c) nat[c] = ld128(row + min(tid + c * 256, nchunk - 1) * 8);
            }
            mainloop_row<BITS, R, NR, FUSED && BITS == 4>(wl, sl, ngq, geo.gq0, xs, xs_ld, lane, a.dq_mask, lane_expo(a), acc, [&]() {
                // every prefetched chunk is used (past the end, the last chunk again, stored over
                // itself), so no load result is dead on some path
                u32x4 *xs4 = reinterpret_cast<u32x4 *>(xs);
                const uint16_t *xa = xs + NR * xs_ld;   // activation order in LDS: a row in its own order
                u32x4 *xa4 = reinterpret_cast<u32x4 *>(xs + NR * xs_ld);
                if (lds_perm) {
#pragma unroll
                    for (int c = 0; c < kPre; ++c) xa4[min(tid + c * 256, nchunk - 1)] = nat[c];
                    for (int i = tid + kPre * 256; i < nchunk; i += 256) xa4[i] = ld128(row + i * 8);
                    __syncthreads();
#pragma unroll
                    for (int c = 0; c < kPre; ++c) xs4[min(tid + c * 256, nchunk - 1)] = gather8(xa, pre[c]);
                    for (int i = tid + kPre * 256; i < nchunk; i += 256) xs4[i] = gather8(xa, ld128(prow + i * 8));
                } else if (prow) {
#pragma unroll
                    for (int c = 0; c < kPre; ++c) xs4[min(tid + c * 256, nchunk - 1)] = gather8(row, pre[c]);
                    for (int i = tid + kPre * 256; i < nchunk; i += 256) xs4[i] = gather8(row, ld128(prow + i * 8));
                } else {
#pragma unroll
                    for (int c = 0; c < kPre; ++c) xs4[min(tid + c * 256, nchunk - 1)] = pre[c];
                    for (int i = tid + kPre * 256; i < nchunk; i += 256) xs4[i] = ld128(row + i * 8);
                }
                if constexpr (NR > 1) {   // the item's second row (a token row, gathered in activation order)
                    const uint16_t *row1 = a.act + (int64_t)(G1 ? f1 / a.act_div : f1) * a.act_ld;
                    u32x4 *xs4b = reinterpret_cast<u32x4 *>(xs + xs_ld);
                    if (lds_perm) {
                        __syncthreads();   // every gather from the first row is done
                        for (int i = tid; i < nchunk; i += 256) xa4[i] = ld128(row1 + i * 8);
                        __syncthreads();
                        for (int i = tid; i < nchunk; i += 256) xs4b[i] = gather8(xa, ld128(prow + i * 8));
                    } else if (prow) {
                        for (int i = tid; i < nchunk; i += 256) xs4b[i] = gather8(row1, ld128(prow + i * 8));
                    } else {
                        for (int i = tid; i < nchunk; i += 256) xs4b[i] = ld128(row1 + i * 8);
                    }
                }
                __syncthreads();
            });
        }
        if constexpr (S > 1) {
            if (geo.ks > 0 && lane < 16) {
#pragma unroll
                for (int q = 0; q < NR; ++q)
#pragma unroll
                    for (int j = 0; j < 4; ++j) red[wave / S][geo.ks][q][j][lane] = acc[q][j];
            }
            __syncthreads();
        }
        if (!geo.active || geo.ks != 0) return;
        if (lane < 16) {
#pragma unroll
            for (int k = 1; k < S; ++k)
#pragma unroll
                for (int q = 0; q < NR; ++q)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[q][j] += red[wave / S][k][q][j][lane];
        }
        if (a.xsplit > 1) {   // uniform over the wave
            const int64_t sb0 = (int64_t)f0 * a.ncs + geo.cs;
            if (lane < 16) {
#pragma unroll
                for (int q = 0; q < NR; ++q) {
                    float *slot = a.part + (((int64_t)fr[q] * a.ncs + geo.cs) * a.xsplit + x) * 64 + lane;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        __hip_atomic_store(slot + j * 16, acc[q][j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            __builtin_amdgcn_s_waitcnt(0);
            int old = 0;
            if (lane == 0) old = __hip_atomic_fetch_add(a.xcnt + sb0, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            old = __shfl(old, 0);
            if (old != a.xsplit - 1) return;
            if (lane == 0) __hip_atomic_store(a.xcnt + sb0, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (lane < 16) {   // the slots added in slot order, kSplitBatch of them loaded at a time
#pragma unroll
                for (int q = 0; q < NR; ++q) {
                    const float *slot = a.part + (((int64_t)fr[q] * a.ncs + geo.cs) * a.xsplit) * 64 + lane;
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[q][j] = 0.f;
                    for (int x0 = 0; x0 < a.xsplit; x0 += kSplitBatch) {
                        float v[kSplitBatch][4];
#pragma unroll
                        for (int xb = 0; xb < kSplitBatch; ++xb)   // past the last slot, the last one again
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                v[xb][j] = __hip_atomic_load(slot + min(x0 + xb, a.xsplit - 1) * 64 + j * 16,
                                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
                        for (int xb = 0; xb < kSplitBatch; ++xb)
                            if (x0 + xb < a.xsplit)
#pragma unroll
                                for (int j = 0; j < 4; ++j) acc[q][j] += v[xb][j];
                    }
                }
            }
        }
        if (lane < 16) {
#pragma unroll
            for (int q = 0; q < NR; ++q) {
                if constexpr (G1) {
                    uint16_t *dst = a.a1 + (int64_t)fr[q] * a.a1_ld + geo.cs * 32 + lane;
                    const uint16_t v0 = f32_to_bf16_rne(silu(acc[q][0]) * acc[q][2]);
                    const uint16_t v1 = f32_to_bf16_rne(silu(acc[q][1]) * acc[q][3]);
                    if constexpr (FUSED) {   // read by GEMM2 workgroups of this launch, possibly on other XCDs
                        __hip_atomic_store(dst, v0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        __hip_atomic_store(dst + 16, v1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    } else {
                        dst[0] = v0;
                        dst[16] = v1;
                    }
                } else {
                    // agent-coherent stores: the combining workgroup may run on another XCD
                    float *dst = a.y + (int64_t)fr[q] * a.y_ld + geo.cs * 64 + lane;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        __hip_atomic_store(dst + 16 * j, wt[q] * acc[q][j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
    } else {
        // a dropped entry, or one of another shard's experts, streams nothing. With kSkipDropped its
        // GEMM1 workgroups neither count themselves nor raise ready flags and its GEMM2 workgroups
        // wait for none; otherwise they go through the hand-off with nothing to publish. Either way
        // one wave per GEMM2 superblock counts its arrival for the combine.
        if constexpr (kSkipDropped) {
            if (G1) return;
        } else {
            if (FUSED && !G1) wait_and_stage();   // consumes this workgroup's ready flag
        }
        if (!geo.active || geo.ks != 0 || x != 0) return;   // one wave per superblock goes on
        if (!G1 && wave == 0 && lane == 0 && bad_expert(a.ids[f0], a.E_all)) atomicOr(a.err, 1);
    }
    if constexpr (G1) {
        if constexpr (FUSED) {   // the slices (or nothing, for a dropped entry) are published
            __builtin_amdgcn_s_waitcnt(0);
            int old = 0;
            if (lane == 0) old = __hip_atomic_fetch_add(a.done + f0, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            old = __shfl(old, 0);
            if (old != a.done_target - 1) return;
            if (lane == 0) __hip_atomic_store(a.done + f0, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int cb2 = lane; cb2 < a.ready_n; cb2 += 64)
                __hip_atomic_fetch_add(a.ready + ((int64_t)f0 * a.ready_n + cb2) * kReadyStride, 1, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        }
    } else {
        // the slice-0 wave of every active superblock of every item, dropped entries included,
        // reaches here, and counts one arrival per entry of the item. The y slices were written with
        // agent-coherent stores; waiting for their completion before the counter increments publishes
        // them without a cache-wide release. The last of a token's topk arrivals sums its slots.
        __builtin_amdgcn_s_waitcnt(0);
        const int c = geo.cs * 64 + lane;
#pragma unroll
        for (int q = 0; q < NR; ++q) {
            const int m = fr[q] / a.topk;
            int32_t *cnt = a.counters + (int64_t)m * a.ncs + geo.cs;
            int old = 0;
            if (lane == 0) old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            old = __shfl(old, 0);
            if (old != a.topk - 1) continue;
            // the slots' ids and outputs are loaded together (a slot of another shard's expert, or a
            // dropped one, has a row in y that this call did not write: read, then left out) and added
            // in slot order
            float sum = 0.f;
            for (int j0 = 0; j0 < a.topk; j0 += kSlotBatch) {
                int idv[kSlotBatch];
                float yv[kSlotBatch];
#pragma unroll
                for (int jb = 0; jb < kSlotBatch; ++jb) {   // past the last slot, the last one again
                    const int64_t fj = (int64_t)m * a.topk + min(j0 + jb, a.topk - 1);
                    idv[jb] = a.ids[fj];
                    yv[jb] = __hip_atomic_load(a.y + fj * a.y_ld + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
#pragma unroll
                for (int jb = 0; jb < kSlotBatch; ++jb)
                    if (j0 + jb < a.topk && (unsigned)local_expert(idv[jb], a.e_first) < (unsigned)a.E)
                        sum += yv[jb];
            }
            if (c < a.out_len) a.out[(int64_t)m * a.out_ld + c] = (uint16_t)bf16_rne_bits(sum);
            if (lane == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Workgroup `bid` of a pair-mode launch: finds its entry's item (a.dedup) and runs it, or ends when
// its entry belongs to an earlier entry's item.
__device__ __forceinline__ uint64_t low_bits(int n) { return n >= 64 ? ~0ull : ((1ull << n) - 1ull); }

template <bool G1, int S, bool FUSED, int R, int BITS, bool kSkipDropped = false>
__device__ __forceinline__ void pair_body(const GemmArgs &a, int bid, uint16_t *xs) {
    const int f = bid / (a.ncb * a.xsplit);
    if (a.dedup) {   // uniform; a.n_items <= 128: routing ids f and 64 + f in lane f of every wave
        const int lane = threadIdx.x & 63, n = a.n_items;
        const int my0 = lane < n ? a.ids[lane] : 0, my1 = 64 + lane < n ? a.ids[64 + lane] : 0;
        const int idf = f < 64 ? __shfl(my0, f) : __shfl(my1, f - 64);
        if ((unsigned)local_expert(idf, a.e_first) < (unsigned)a.E) {
            const uint64_t s0 = __ballot(lane < n && my0 == idf), s1 = __ballot(64 + lane < n && my1 == idf);
            // entries before f with the same expert, and the first one after it
            const int rank = __popcll(s0 & low_bits(f)) + (f >= 64 ? __popcll(s1 & low_bits(f - 64)) : 0);
            if (rank % kItemRows) return;   // the item of an earlier entry covers this one
            const uint64_t a0 = f < 64 ? s0 & ~low_bits(f + 1) : 0ull;
            const uint64_t a1 = s1 & ~low_bits(f < 64 ? 0 : f - 63);
            const int f1 = a0 ? __ffsll((long long)a0) - 1 : a1 ? 64 + __ffsll((long long)a1) - 1 : -1;
            if (f1 >= 0) {
                pair_item_body<G1, S, FUSED, R, BITS, kSkipDropped, 2>(a, bid, f, f1, xs);
                return;
            }
        }
    }
    pair_item_body<G1, S, FUSED, R, BITS, kSkipDropped, 1>(a, bid, f, f, xs);
}

template <bool G1, int S, int BITS>
// (held to the occupancy the ring alone allows: 4 waves per SIMD for 4-bit blocks, 2 for 8-bit)
__global__ __launch_bounds__(256, BITS == 4 ? 4 : 2) void gemm_pair_kernel(GemmArgs a) {
    extern __shared__ __align__(16) uint16_t xs[];
    pair_body<G1, S, false, kRing, BITS>(a, blockIdx.x, xs);
}

// Both GEMMs of pair mode in one launch. The entries are taken in g1.phases consecutive groups; for
// each group in turn, the GEMM1 workgroups of its entries come first and then their GEMM2 workgroups
// (with one group: workgroups [0, n1) run GEMM1, the rest GEMM2). A GEMM2 workgroup thus waits only
// for GEMM1 workgroups of lower index, which are dispatched before it.
template <int S1, int S2, int R, int BITS, bool SKIP>
__global__ __launch_bounds__(256) void gemm_pair_fused_kernel(GemmArgs g1, GemmArgs g2) {
    extern __shared__ __align__(16) uint16_t xs[];
    const int per1 = g1.ncb * g1.xsplit, per2 = g2.ncb * g2.xsplit, T = g1.n_items, P = g1.phases;
    int b = blockIdx.x;
    for (int p = 0; p < P; ++p) {   // uniform
        const int e0 = p * T / P, e1 = (p + 1) * T / P;
        const int n1 = (e1 - e0) * per1, n2 = (e1 - e0) * per2;
        if (b < n1) {
            pair_body<true, S1, true, R, BITS, SKIP>(g1, e0 * per1 + b, xs);
            return;
        }
        b -= n1;
        if (b < n2) {
            pair_body<false, S2, true, R, BITS, SKIP>(g2, e0 * per2 + b, xs);
            return;
        }
        b -= n2;
    }
}

// Sorted mode: workgroup = (work item, superblock group cb); items of up to 16 * NT rows.
template <bool G1, int S, int NT, int BITS>
__device__ __forceinline__ void sorted_body(const GemmArgs &a, const WorkItem &it, const Geo<S> &geo, int wave,
                                            int lane) {
    constexpr int SPW = 4 / S;
    const uint16_t *arow[NT];
    setup_rows<G1, NT>(a, it, lane, arow);
    f32x4 acc[NT][4];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[tt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (geo.active) {
        const uint8_t *blk = a.wpk + (((int64_t)it.e * a.ncs + geo.cs) * a.gq_total + geo.gq0) * Fmt<BITS>::kBlock;
        mainloop_tiles<BITS, NT>(blk + lane * 16, blk + Fmt<BITS>::kCode + (lane & 15) * 32, geo.gq1 - geo.gq0, geo.gq0, arow,
                           lane, a.dq_mask, lane_expo(a), acc);
    }
    if constexpr (S > 1) {
        __shared__ float red[SPW][S - 1][NT * 16][64];
        if (geo.active && geo.ks > 0) {
#pragma unroll
            for (int v = 0; v < NT * 16; ++v) red[wave / S][geo.ks - 1][v][lane] = acc[v >> 4][(v >> 2) & 3][v & 3];
        }
        __syncthreads();
        if (!geo.active || geo.ks != 0) return;
#pragma unroll
        for (int k = 0; k < S - 1; ++k)
#pragma unroll
            for (int v = 0; v < NT * 16; ++v) acc[v >> 4][(v >> 2) & 3][v & 3] += red[wave / S][k][v][lane];
    } else {
        if (!geo.active) return;
    }
    epilogue<G1, NT>(a, it, geo.cs, lane, acc);
}

// MAXNT = 1: items of at most 16 rows; MAXNT = 2: up to 32 rows (16-row items take the 1-tile body).
template <bool G1, int S, int MAXNT, int BITS>
__global__ __launch_bounds__(256) void gemm_sorted_kernel(GemmArgs a) {
    const int wi = blockIdx.x / a.ncb, cb = blockIdx.x % a.ncb;
    if (wi >= *a.n_work) return;
    const WorkItem it = a.work[wi];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const Geo<S> geo(a, cb, wave);
    if (MAXNT == 1 || it.nrows <= 16) sorted_body<G1, S, 1, BITS>(a, it, geo, wave, lane);
    else sorted_body<G1, S, MAXNT, BITS>(a, it, geo, wave, lane);
}

// ---------------------------------------------------------------------------------------------
// Wide items (large M): workgroup = (work item of up to 64 rows, group of 4 superblocks). Each wave
// owns one superblock; the four walk the reduction together, block by block. The item's token rows
// for the current block (rows x 128 k) are staged in LDS once per workgroup, double-buffered, with
// rows padded to 272 bytes so the 16 rows of a 128-bit fragment read fall in distinct banks.
// ---------------------------------------------------------------------------------------------
constexpr int kWideRows = 64;
constexpr int kRowStride = 136;   // bf16 per staged row: 128 + 8 padding

struct NoWait {
    __device__ bool operator()() const { return false; }
};

// COH && !G1 (GEMM2 of the single-launch wide plan): `wait` returns once the item's rows are
// published (true: the wait gave up); it is called with the first weight blocks in flight, and the
// rows are loaded after it.
template <bool G1, int NT, int kWideRing, int BITS, bool STREAM, bool COH = false, typename Wait = NoWait>
__device__ __forceinline__ void wide_body(const GemmArgs &a, const WorkItem &it, int cs, bool active, int tid,
                                          int lane, uint16_t (*as)[kWideRows * kRowStride], Wait wait = Wait{}) {
    const f32x4 kZero = {0.f, 0.f, 0.f, 0.f};
    const uint32_t mask = a.dq_mask, expo = lane_expo(a);
    const int ngq = a.gq_total, last = ngq - 1;
    // staging: NT*16 rows x 16 chunks of 16 B per block; thread tid moves chunks tid + 256c, c < NT
    const uint16_t *srow[NT];
    int soff[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) {
        const int q = tid + 256 * c, r = q >> 4, kc = q & 15;
        const int rr = r < it.nrows ? r : 0;               // padding rows copy the item's first row
        const int64_t p = it.p0 + rr;
        const int64_t arow = G1 ? (int64_t)(a.sorted_ids[p] / a.act_div) : p;
        srow[c] = a.act + arow * a.act_ld + kc * 8;
        soff[c] = r * kRowStride + kc * 8;
    }
    auto load_a = [&](u32x4 (&v)[NT], int gq) {
#pragma unroll
        for (int c = 0; c < NT; ++c) v[c] = (COH && !G1) ? ld128_agent(srow[c] + gq * 128) : ld128(srow[c] + gq * 128);
    };
    auto store_a = [&](const u32x4 (&v)[NT], int buf) {
#pragma unroll
        for (int c = 0; c < NT; ++c) *reinterpret_cast<u32x4 *>(&as[buf][soff[c]]) = v[c];
    };

    const int cs_ld = min(cs, a.ncs - 1);   // inactive waves load a valid block and discard it
    const int64_t blk0 = ((int64_t)it.e * a.ncs + cs_ld) * a.gq_total;   // the wave's first block
    const uint8_t *blk = a.wpk + blk0 * (int64_t)Fmt<BITS>::kBlock;
    const uint8_t *wl = blk + lane * 16, *sl = blk + Fmt<BITS>::kCode + (lane & 15) * 32;
    // the ring's loads past the end read the buffer's first block, which every wave's tail reads and
    // the caches keep, rather than repeating the wave's last block (streamed, that would miss)
    const int tail = (int)-blk0;
    f32x4 acc[NT][4];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[tt][j] = kZero;

    WStage<BITS> st[kWideRing];
    u32x4 av[NT];
    bool late = false;
    if constexpr (COH && !G1) {
#pragma unroll
        for (int r = 0; r < kWideRing - 1; ++r) load_w<BITS, STREAM>(st[r], wl, sl, min(r, last));
        late = wait();
        load_a(av, 0);
    } else {
        load_a(av, 0);
#pragma unroll
        for (int r = 0; r < kWideRing - 1; ++r) load_w<BITS, STREAM>(st[r], wl, sl, min(r, last));
    }
    store_a(av, 0);
    __syncthreads();
    const int arow_lds = (lane & 15) * kRowStride + (lane >> 4) * 8;
    for (int i0 = 0; i0 < ngq; i0 += kWideRing) {
#pragma unroll
        for (int r = 0; r < kWideRing; ++r) {
            const int i = i0 + r;
            if (i < ngq) {   // uniform over the workgroup (every wave walks the same blocks)
                load_a(av, min(i + 1, last));   // next block's rows: issued before the next weights
                load_w<BITS, STREAM>(st[(r + kWideRing - 1) % kWideRing], wl, sl,
                                     i + kWideRing - 1 <= last ? i + kWideRing - 1 : tail);
                if constexpr (NT <= 2) __builtin_amdgcn_sched_barrier(0);   // the loads stay ahead of the block's work
                const WStage<BITS> &c = st[r];
                const uint16_t *ab = &as[i & 1][arow_lds];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    BOps<BITS> b;
                    decode_group<BITS>(c, g, mask, expo, b);
                    float s[4];
                    scales_of(c.s, g, s);
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt) {
                        const bf16x8 av8 =
                            as_bf16x8(*reinterpret_cast<const u32x4 *>(ab + tt * 16 * kRowStride + g * kGroup));
                        f32x4 d[4];
                        dot_group<BITS>(av8, b, d);
#pragma unroll
                        for (int j = 0; j < 4; ++j) acc[tt][j] += s[j] * d[j];
                    }
                }
                store_a(av, (i + 1) & 1);
                __syncthreads();
            }
        }
    }
    drain_loads();
    if (active) epilogue<G1, NT, COH>(a, it, cs, lane, acc, late);
}

// GEMM2 over a short reduction (one or two group quads: N <= 256, as on a tensor-parallel shard),
// several superblocks per wave. The item's rows are staged in LDS once, whole, so the waves run
// without barriers; each wave streams the blocks of its superblocks back to back through one ring
// (superblocks cs0, cs0 + 4, ..., the workgroup's four waves side by side) and writes a superblock's
// slot outputs as soon as its last block is in. The per-wave work of one superblock alone (one or
// two blocks) would leave the workgroup's prologue and epilogue as most of its lifetime.
template <int NT, int R, int BITS, bool STREAM, bool COH = false, typename Wait = NoWait>
__device__ __forceinline__ void wide_body_thin(const GemmArgs &a, const WorkItem &it, int cb, int wave, int tid,
                                               int lane, uint16_t (*as)[kWideRows * kRowStride], int32_t *s_f,
                                               float *s_w, Wait wait = Wait{}) {
    const f32x4 kZero = {0.f, 0.f, 0.f, 0.f};
    const uint32_t mask = a.dq_mask, expo = lane_expo(a);
    const int ngq = a.gq_total, sh = ngq - 1;   // one or two blocks per superblock
    const int cs0 = cb * a.sbw * 4 + wave;
    // superblocks of this wave below ncs (none: the wave streams a valid block, unused, for the barrier)
    const int nsb = cs0 < a.ncs ? min(a.sbw, (a.ncs - 1 - cs0) / 4 + 1) : 1;
    const bool any = cs0 < a.ncs;
    const int ns = nsb * ngq;
    const int cs_ld = min(cs0, a.ncs - 1);
    const uint8_t *blk = a.wpk + ((int64_t)it.e * a.ncs + cs_ld) * a.gq_total * (int64_t)Fmt<BITS>::kBlock;
    const uint8_t *wl = blk + lane * 16, *sl = blk + Fmt<BITS>::kCode + (lane & 15) * 32;
    // step j: block j & sh of superblock cs0 + 4 * (j >> sh)
    auto blk_of = [&](int j) { return (j >> sh) * 4 * ngq + (j & sh); };

    WStage<BITS> st[R];
#pragma unroll
    for (int r = 0; r < R - 1; ++r) load_w<BITS, STREAM>(st[r], wl, sl, blk_of(min(r, ns - 1)));
    const bool late = wait();   // the single launch: the item's rows are published (weights in flight)
    // rows: NT*16 rows x 16 chunks of 16 B per block, for every block of the reduction
#pragma unroll
    for (int c = 0; c < NT; ++c) {
        const int q = tid + 256 * c, r = q >> 4, kc = q & 15;
        const int rr = r < it.nrows ? r : 0;   // padding rows copy the item's first row
        const uint16_t *src = a.act + (int64_t)(it.p0 + rr) * a.act_ld + kc * 8;
        u32x4 v[2];
#pragma unroll
        for (int g = 0; g < 2; ++g) v[g] = COH ? ld128_agent(src + min(g, sh) * 128) : ld128(src + min(g, sh) * 128);
#pragma unroll
        for (int g = 0; g < 2; ++g) *reinterpret_cast<u32x4 *>(&as[g][r * kRowStride + kc * 8]) = v[g];
    }
    if (tid < it.nrows) {
        const int32_t f = a.sorted_ids[it.p0 + tid];
        s_f[tid] = f;
        s_w[tid] = late ? __int_as_float(0x7FC00000) : a.topk_w[f];
    }
    __syncthreads();

    f32x4 acc[NT][4];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[tt][j] = kZero;
    const int arow_lds = (lane & 15) * kRowStride + (lane >> 4) * 8;
    const int col = lane & 15;
    for (int i0 = 0; i0 < ns; i0 += R) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = i0 + r;
            if (i < ns) {   // uniform over the wave
                if constexpr (STREAM) {   // nothing past the end (a streamed repeat would miss the caches)
                    if (i + R - 1 <= ns - 1) load_w<BITS, STREAM>(st[(r + R - 1) % R], wl, sl, blk_of(i + R - 1));
                } else {
                    load_w<BITS, STREAM>(st[(r + R - 1) % R], wl, sl, blk_of(min(i + R - 1, ns - 1)));
                }
                if constexpr (NT <= 2) __builtin_amdgcn_sched_barrier(0);   // the loads stay ahead of the block's work
                const WStage<BITS> &c = st[r];
                const uint16_t *ab = &as[i & sh][arow_lds];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    BOps<BITS> b;
                    decode_group<BITS>(c, g, mask, expo, b);
                    float s[4];
                    scales_of(c.s, g, s);
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt) {
                        const bf16x8 av8 =
                            as_bf16x8(*reinterpret_cast<const u32x4 *>(ab + tt * 16 * kRowStride + g * kGroup));
                        f32x4 d[4];
                        dot_group<BITS>(av8, b, d);
#pragma unroll
                        for (int j = 0; j < 4; ++j) acc[tt][j] += s[j] * d[j];
                    }
                }
                if ((i & sh) == sh) {   // the superblock's last block: its slot outputs, in bf16
                    if (any) {
                        const int cs = cs0 + 4 * (i >> sh);
#pragma unroll
                        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                            for (int rr = 0; rr < 4; ++rr) {
                                const int row = tt * 16 + (lane >> 4) * 4 + rr;
                                if (row >= it.nrows) continue;
                                uint16_t *dst = a.yb + (int64_t)s_f[row] * a.y_ld + cs * 64 + col;
                                const float wt = s_w[row];
#pragma unroll
                                for (int j = 0; j < 4; ++j) dst[16 * j] = f32_to_bf16_rne(wt * acc[tt][j][rr]);
                            }
                    }
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                        for (int j = 0; j < 4; ++j) acc[tt][j] = kZero;
                }
            }
        }
    }
    drain_loads();
}

// An item's body for its tile count (MAXNT: the most the launch may hold)
template <bool G1, int MAXNT, int R, int BITS, bool STREAM, bool COH = false, typename Wait = NoWait>
__device__ __forceinline__ void wide_item(const GemmArgs &a, const WorkItem &it, int cs, bool active, int tid,
                                          int lane, uint16_t (*as)[kWideRows * kRowStride], Wait wait = Wait{}) {
    const int nt = (it.nrows + 15) >> 4;
    if (nt <= 1) wide_body<G1, 1, R, BITS, STREAM, COH>(a, it, cs, active, tid, lane, as, wait);
    else if (MAXNT <= 2 || nt == 2) wide_body<G1, 2, R, BITS, STREAM, COH>(a, it, cs, active, tid, lane, as, wait);
    else if (MAXNT <= 3 || nt == 3)
        wide_body<G1, (MAXNT > 2 ? 3 : 2), R, BITS, STREAM, COH>(a, it, cs, active, tid, lane, as, wait);
    else wide_body<G1, (MAXNT > 3 ? 4 : 2), R, BITS, STREAM, COH>(a, it, cs, active, tid, lane, as, wait);
}

template <int MAXNT, int R, int BITS, bool STREAM, bool COH = false, typename Wait = NoWait>
__device__ __forceinline__ void thin_item(const GemmArgs &a, const WorkItem &it, int cb, int wave, int tid, int lane,
                                          uint16_t (*as)[kWideRows * kRowStride], int32_t *s_f, float *s_w,
                                          Wait wait = Wait{}) {
    const int nt = (it.nrows + 15) >> 4;
    if (nt <= 1) wide_body_thin<1, R, BITS, STREAM, COH>(a, it, cb, wave, tid, lane, as, s_f, s_w, wait);
    else if (MAXNT <= 2 || nt == 2) wide_body_thin<2, R, BITS, STREAM, COH>(a, it, cb, wave, tid, lane, as, s_f, s_w, wait);
    else if (MAXNT <= 3 || nt == 3)
        wide_body_thin<(MAXNT > 2 ? 3 : 2), R, BITS, STREAM, COH>(a, it, cb, wave, tid, lane, as, s_f, s_w, wait);
    else wide_body_thin<(MAXNT > 3 ? 4 : 2), R, BITS, STREAM, COH>(a, it, cb, wave, tid, lane, as, s_f, s_w, wait);
}

// MAXNT: the largest item (16-row tiles) the launch may hold; R: blocks held per wave in the ring
template <bool G1, int MAXNT, int R, int BITS>
__device__ __forceinline__ void wide_kernel_body(const GemmArgs &a) {
    __shared__ __align__(16) uint16_t as[2][kWideRows * kRowStride];
    const int wi = blockIdx.x / a.ncb, cb = blockIdx.x % a.ncb;
    if (wi >= *a.n_work) return;
    const WorkItem it = a.work[wi];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int cs = cb * 4 + wave;
    const bool active = cs < a.ncs;
    if (it.flags & kItemShared) wide_item<G1, MAXNT, R, BITS, false>(a, it, cs, active, tid, lane, as);
    else wide_item<G1, MAXNT, R, BITS, true>(a, it, cs, active, tid, lane, as);
}


template <bool G1, int MAXNT, int R, int BITS>
__global__ __launch_bounds__(256) void gemm_wide_kernel(GemmArgs a) {
    wide_kernel_body<G1, MAXNT, R, BITS>(a);
}

// GEMM2 with several superblocks per wave (a.sbw > 1; reductions of one or two blocks)
// (8-bit blocks are twice the registers: 2 waves per SIMD, unspilled)
template <int MAXNT, int R, int BITS>
__global__ __launch_bounds__(256, BITS == 4 ? 3 : 2) void gemm_thin_kernel(GemmArgs a) {
    __shared__ __align__(16) uint16_t as[2][kWideRows * kRowStride];
    __shared__ int32_t s_f[kWideRows];
    __shared__ float s_w[kWideRows];
    const int wi = blockIdx.x / a.ncb, cb = blockIdx.x % a.ncb;
    if (wi >= *a.n_work) return;
    const WorkItem it = a.work[wi];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if (it.flags & kItemShared) thin_item<MAXNT, R, BITS, false>(a, it, cb, wave, tid, lane, as, s_f, s_w);
    else thin_item<MAXNT, R, BITS, true>(a, it, cb, wave, tid, lane, as, s_f, s_w);
}

// Items of up to three 16-row tiles, held to 3 waves per SIMD (at most 168 VGPRs; unconstrained the
// compiler takes 188 and 2 waves per SIMD, constrained it spills 4 registers, 16 bytes per lane).
template <bool G1, int R, int BITS>
__global__ __launch_bounds__(256, 3) void gemm_wide48_kernel(GemmArgs a) {
    wide_kernel_body<G1, 3, R, BITS>(a);
}

// The wide plan in one launch (4-bit codes, items of up to three tiles): the first grid1 workgroups
// are GEMM1's (work item x column block), the rest GEMM2's. Workgroups are dispatched in index order,
// so GEMM2 workgroups take the compute units that GEMM1's last workgroups leave idle, rather than
// waiting for a second launch. The hand-off is per work item: a GEMM1 workgroup stores its SwiGLU
// slice agent-coherent, waits for the stores, and counts itself in done[item]; the last of the item's
// g1.ncb workgroups re-zeroes the count and adds 1 to the ready flag of each of the item's g2.ncb
// GEMM2 workgroups. A GEMM2 workgroup waits until its flag is positive (bounded by wait_ticks of the
// constant clock, as in the pair mode: on expiry it raises error bit 1 and its outputs are NaN),
// subtracts 1, and reads the item's rows with agent-coherent loads. Every flag gets one +1 and one -1
// per launch, so it is zero again when the launch ends. THIN: GEMM2 over one or two group quads
// (several superblocks per wave).
template <int R, int BITS, bool THIN>
__global__ __launch_bounds__(256, 3) void gemm_wide_fused_kernel(GemmArgs g1, GemmArgs g2, int32_t grid1) {
    __shared__ __align__(16) uint16_t as[2][kWideRows * kRowStride];
    __shared__ int32_t s_f[kWideRows];
    __shared__ float s_w[kWideRows];
    __shared__ int s_late;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if ((int)blockIdx.x < grid1) {
        const GemmArgs &a = g1;
        const int wi = blockIdx.x / a.ncb, cb = blockIdx.x % a.ncb;
        if (wi >= *a.n_work) return;
        const WorkItem it = a.work[wi];
        const int cs = cb * 4 + wave;
        const bool active = cs < a.ncs;
        if (it.flags & kItemShared) wide_item<true, 3, R, BITS, false, true>(a, it, cs, active, tid, lane, as);
        else wide_item<true, 3, R, BITS, true, true>(a, it, cs, active, tid, lane, as);
        __builtin_amdgcn_s_waitcnt(0);   // this wave's rows are stored
        __syncthreads();                 // and every other wave's
        if (wave == 0) {
            int old = 0;
            if (lane == 0) old = __hip_atomic_fetch_add(a.done + wi, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            old = __shfl(old, 0);
            if (old == a.ncb - 1) {
                if (lane == 0) __hip_atomic_store(a.done + wi, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                for (int c2 = lane; c2 < g2.ncb; c2 += 64)
                    __hip_atomic_fetch_add(a.ready + ((int64_t)wi * g2.ncb + c2) * kWideReadyStride, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        return;
    }
    const GemmArgs &a = g2;
    const int bid = (int)blockIdx.x - grid1;
    const int wi = bid / a.ncb, cb = bid % a.ncb;
    if (wi >= *a.n_work) return;
    // called by every thread once the first weight blocks are requested
    auto wait = [&]() -> bool {
        if (tid == 0) {
            int32_t *flag = a.ready + ((int64_t)wi * a.ncb + cb) * kWideReadyStride;
            const long long t0 = wall_clock64();
            int late = 0;
            while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <= 0) {
                if (wall_clock64() - t0 >= a.wait_ticks) {
                    atomicOr(a.err, 2);
                    late = 1;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
            __hip_atomic_fetch_add(flag, -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_late = late;
        }
        __syncthreads();
        return s_late != 0;
    };
    const WorkItem it = a.work[wi];
    const bool shared = it.flags & kItemShared;
    if constexpr (THIN) {
        if (shared) thin_item<3, R, BITS, false, true>(a, it, cb, wave, tid, lane, as, s_f, s_w, wait);
        else thin_item<3, R, BITS, true, true>(a, it, cb, wave, tid, lane, as, s_f, s_w, wait);
    } else {
        const int cs = cb * 4 + wave;
        const bool active = cs < a.ncs;
        if (shared) wide_item<false, 3, R, BITS, false, true>(a, it, cs, active, tid, lane, as, wait);
        else wide_item<false, 3, R, BITS, true, true>(a, it, cs, active, tid, lane, as, wait);
    }
}

}  // namespace

template <bool G1, int BITS>
hipError_t launch_one(GemmKind kind, int S, int maxnt, const GemmArgs &a, dim3 g, hipStream_t s) {
    const bool pair = kind == GemmKind::kPair;
    const size_t rows = (a.dedup ? kItemRows : 1) + (G1 && a.perm && a.perm_lds ? 1 : 0);
    const size_t lds = pair ? (size_t)a.act_ld * rows * sizeof(uint16_t) : 0;
    const int wide = !G1 && a.sbw > 1 ? 2000 : 1000;   // several superblocks per wave: the thin GEMM2
    const int key = pair ? 100 + S : kind == GemmKind::kWide ? wide + maxnt : S * 10 + maxnt;
    switch (key) {
        case 2001:
        case 2002: hipLaunchKernelGGL((gemm_thin_kernel<2, 2, BITS>), g, dim3(256), 0, s, a); break;
        case 2003: hipLaunchKernelGGL((gemm_thin_kernel<3, 2, BITS>), g, dim3(256), 0, s, a); break;
        case 2004: hipLaunchKernelGGL((gemm_thin_kernel<4, 2, BITS>), g, dim3(256), 0, s, a); break;
        case 1001:
        case 1002: hipLaunchKernelGGL((gemm_wide_kernel<G1, 2, 2, BITS>), g, dim3(256), 0, s, a); break;
        case 1003: hipLaunchKernelGGL((gemm_wide48_kernel<G1, 2, BITS>), g, dim3(256), 0, s, a); break;
        case 1004: hipLaunchKernelGGL((gemm_wide_kernel<G1, 4, 2, BITS>), g, dim3(256), 0, s, a); break;
        case 11: hipLaunchKernelGGL((gemm_sorted_kernel<G1, 1, 1, BITS>), g, dim3(256), 0, s, a); break;
        case 21: hipLaunchKernelGGL((gemm_sorted_kernel<G1, 2, 1, BITS>), g, dim3(256), 0, s, a); break;
        case 41: hipLaunchKernelGGL((gemm_sorted_kernel<G1, 4, 1, BITS>), g, dim3(256), 0, s, a); break;
        case 12: hipLaunchKernelGGL((gemm_sorted_kernel<G1, 1, 2, BITS>), g, dim3(256), 0, s, a); break;
        case 22: hipLaunchKernelGGL((gemm_sorted_kernel<G1, 2, 2, BITS>), g, dim3(256), 0, s, a); break;
        case 42: hipLaunchKernelGGL((gemm_sorted_kernel<G1, 4, 2, BITS>), g, dim3(256), 0, s, a); break;
        case 101: hipLaunchKernelGGL((gemm_pair_kernel<G1, 1, BITS>), g, dim3(256), lds, s, a); break;
        case 102: hipLaunchKernelGGL((gemm_pair_kernel<G1, 2, BITS>), g, dim3(256), lds, s, a); break;
        case 104: hipLaunchKernelGGL((gemm_pair_kernel<G1, 4, BITS>), g, dim3(256), lds, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// 8-bit blocks are twice the registers: a ring of two keeps the single-launch kernel at 149 VGPRs
// (3 waves per SIMD) instead of 230 (2 waves), 1.5-3% faster at M = 1-4.
template <int BITS, bool SKIP>
hipError_t launch_fused(int S1, int S2, const GemmArgs &g1, const GemmArgs &g2, dim3 g, size_t lds, hipStream_t s) {
    switch (S1 * 10 + S2) {
#define W4MOE_FUSED_CASE(A, B) \
    case A * 10 + B: hipLaunchKernelGGL((gemm_pair_fused_kernel<A, B, (BITS == 8 ? 2 : kRing), BITS, SKIP>), g, dim3(256), lds, s, g1, g2); break;
        W4MOE_FUSED_CASE(1, 1) W4MOE_FUSED_CASE(1, 2) W4MOE_FUSED_CASE(1, 4)
        W4MOE_FUSED_CASE(2, 1) W4MOE_FUSED_CASE(2, 2) W4MOE_FUSED_CASE(2, 4)
        W4MOE_FUSED_CASE(4, 1) W4MOE_FUSED_CASE(4, 2) W4MOE_FUSED_CASE(4, 4)
#undef W4MOE_FUSED_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_pair_fused(int S1, int S2, const GemmArgs &g1, const GemmArgs &g2, bool skip_dropped, hipStream_t s) {
    const int64_t grid = (int64_t)g1.n_items * g1.ncb * g1.xsplit + (int64_t)g2.n_items * g2.ncb * g2.xsplit;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const int64_t rows = g1.dedup ? kItemRows : 1;
    const size_t lds = (size_t)std::max(g1.act_ld * (rows + (g1.perm && g1.perm_lds ? 1 : 0)), g2.act_ld * rows) *
                       sizeof(uint16_t);
    const dim3 g((unsigned)grid);
    if (g1.bits == 8)
        return skip_dropped ? launch_fused<8, true>(S1, S2, g1, g2, g, lds, s) : launch_fused<8, false>(S1, S2, g1, g2, g, lds, s);
    if (g1.bits == 4)
        return skip_dropped ? launch_fused<4, true>(S1, S2, g1, g2, g, lds, s) : launch_fused<4, false>(S1, S2, g1, g2, g, lds, s);
    return hipErrorInvalidValue;
}

hipError_t launch_wide_fused(const GemmArgs &g1, const GemmArgs &g2, int64_t items, hipStream_t s) {
    const int64_t grid1 = items * g1.ncb, grid = grid1 + items * g2.ncb;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    if (g1.bits != 4 || g2.bits != 4) return hipErrorInvalidValue;
    if (g2.sbw > 1)
        hipLaunchKernelGGL((gemm_wide_fused_kernel<2, 4, true>), dim3((unsigned)grid), dim3(256), 0, s, g1, g2, (int32_t)grid1);
    else
        hipLaunchKernelGGL((gemm_wide_fused_kernel<2, 4, false>), dim3((unsigned)grid), dim3(256), 0, s, g1, g2, (int32_t)grid1);
    return hipGetLastError();
}

hipError_t launch_gemm(bool gemm1, GemmKind kind, int S, int max_rows, const GemmArgs &a, int64_t items,
                       hipStream_t s) {
    const int64_t grid = items * a.ncb * (kind == GemmKind::kPair ? a.xsplit : 1);
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const int maxnt = (max_rows + 15) / 16;
    if (maxnt < 1 || maxnt > 4) return hipErrorInvalidValue;
    const dim3 g((unsigned)grid);
    if (a.bits == 8)
        return gemm1 ? launch_one<true, 8>(kind, S, maxnt, a, g, s) : launch_one<false, 8>(kind, S, maxnt, a, g, s);
    if (a.bits == 4)
        return gemm1 ? launch_one<true, 4>(kind, S, maxnt, a, g, s) : launch_one<false, 4>(kind, S, maxnt, a, g, s);
    return hipErrorInvalidValue;
}

}  // namespace w4moe
