// Grouped W4A16 GEMMs of the MoE layer for gfx950: GEMM1 (gate|up, fused SiLU(gate)*up epilogue)
// and GEMM2 (down projection, routing-weight epilogue).
//
// What is computed (pages: "The Pivot to Real Hardware...", Step 1: Understanding the Weight
// Format; "The Commit That Captured a Plateau", Regime 1 and Regime 2): for every row p of the
// sorted token order routed to expert e,
//   GEMM1: a1[p][n] = bf16( SiLU(sum_k x[tok(p)][k] W1_e[k][n]) * sum_k x[tok(p)][k] W1_e[k][N+n] )
//   GEMM2: y[f(p)][c] = w[f(p)] * sum_n a1[p][n] W2_e[n][c]
// with W[k][c] = q[k][c] * s[k/32][c], q a signed 4-bit code.
//
// How (gfx950, wave64):
//  * Tokens are the A operand of v_mfma_f32_16x16x32_bf16 (16 token rows per tile, zero-padded) and
//    the weights the B operand, so one MFMA covers 16 output columns x one 32-row scale group.
//  * A lane's B operand is exactly one packed 32-bit word (8 codes of one column): it is turned into
//    four bf16 pairs with a mask and an OR into the exponent pattern of 128.0, giving the exact
//    values 128 + code = 136 + q (the "magic number" conversion of Kim et al. 2022, "Who Says
//    Elephants Can't Run"). A fifth MFMA against a constant -136 operand yields -136 * sum_k x[k]
//    per token row, which enters the four weight MFMAs as their C operand, so each MFMA result is
//    exactly sum_k x[k] q[k] (fp32 accumulation); one fp32 FMA per output then applies the group
//    scale. No scale rounding enters the weights.
//  * Each wave streams its packed blocks (4 KiB of codes + 512 B of scales for 64 columns x 128
//    rows) with 128-bit loads that are contiguous across the wave, prefetching the next block.
#include "w4moe_internal.h"

namespace w4moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 8 codes (row t at bit 0,16,4,20,8,24,12,28) -> bf16 values 128 + code for rows 0..7 in order.
__device__ __forceinline__ bf16x8 decode_word(uint32_t w) {
    constexpr uint32_t kMask = 0x000F000Fu, kExp = 0x43004300u;
    u32x4 v;
    v.x = (w & kMask) | kExp;
    v.y = ((w >> 4) & kMask) | kExp;
    v.z = ((w >> 8) & kMask) | kExp;
    v.w = ((w >> 12) & kMask) | kExp;
    return as_bf16x8(v);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld128(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

__device__ __forceinline__ float bf16_word_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_word_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// Scale of slot j of group gsub from the lane's 16 scales (index gsub*4 + j, two per word).
__device__ __forceinline__ float scale_of(const u32x4 s[2], int gsub, int j) {
    const int idx = gsub * 4 + j;
    const u32x4 v = s[idx >> 3];
    const uint32_t w = v[(idx & 7) >> 1];
    return (idx & 1) ? bf16_word_hi(w) : bf16_word_lo(w);
}

// One wave: NT token tiles x 4 column tiles (one 64-column superblock) over ngq group quads.
// The next block's codes and scales are always in flight while the current one is consumed; token
// fragments are prefetched one block ahead for a single tile and loaded per block otherwise.
template <int NT>
__device__ __forceinline__ void wave_mainloop(const uint8_t *__restrict__ blk, int ngq, int gq0,
                                              const uint16_t *const arow[NT], int lane, f32x4 acc[NT][4]) {
    constexpr bool kPrefetchA = NT == 1;
    const int koff = (lane >> 4) * 8;
    const uint8_t *wl = blk + lane * 16;
    const uint8_t *sl = blk + kCodeBytes + (lane & 15) * 32;
    const bf16x8 kBias = as_bf16x8(u32x4{0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u});  // -136
    const f32x4 kZero = {0.f, 0.f, 0.f, 0.f};
    auto load_a = [&](u32x4 (&dst)[NT][4], int gq) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                dst[tt][g] = arow[tt] ? ld128(arow[tt] + (gq * 4 + g) * kGroup + koff) : u32x4{0, 0, 0, 0};
    };

    if (ngq <= 0) return;
    u32x4 wc[4], sc[2], ac[NT][4];
#pragma unroll
    for (int g = 0; g < 4; ++g) wc[g] = ld128(wl + g * 1024);
    sc[0] = ld128(sl);
    sc[1] = ld128(sl + 16);
    if (kPrefetchA) load_a(ac, gq0);

    for (int i = 0; i < ngq; ++i) {
        u32x4 wn[4], sn[2], an[NT][4];
        const bool more = (i + 1) < ngq;
        if (!kPrefetchA) load_a(ac, gq0 + i);
        if (more) {
            const uint8_t *b = wl + (int64_t)(i + 1) * kBlockBytes;
#pragma unroll
            for (int g = 0; g < 4; ++g) wn[g] = ld128(b + g * 1024);
            const uint8_t *s = sl + (int64_t)(i + 1) * kBlockBytes;
            sn[0] = ld128(s);
            sn[1] = ld128(s + 16);
            if (kPrefetchA) load_a(an, gq0 + i + 1);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            bf16x8 b[4];
            float s[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                b[j] = decode_word(wc[g][j]);
                s[j] = scale_of(sc, g, j);
            }
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                const bf16x8 a = as_bf16x8(ac[tt][g]);
                const f32x4 bias = mfma16(a, kBias, kZero);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4 d = mfma16(a, b[j], bias);
                    acc[tt][j] += s[j] * d;
                }
            }
        }
        if (more) {
#pragma unroll
            for (int g = 0; g < 4; ++g) wc[g] = wn[g];
            sc[0] = sn[0];
            sc[1] = sn[1];
            if (kPrefetchA) {
#pragma unroll
                for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                    for (int g = 0; g < 4; ++g) ac[tt][g] = an[tt][g];
            }
        }
    }
}

// Output row layout of the MFMA result: lane holds rows 4*(lane/16) + r (r = 0..3) of column lane%16.
template <bool G1, int NT>
__device__ __forceinline__ void epilogue(const GemmArgs &a, const WorkItem &it, int cs, int lane, f32x4 acc[NT][4]) {
    const int col = lane & 15;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = tt * 16 + (lane >> 4) * 4 + r;
            if (row >= it.nrows) continue;
            const int64_t p = it.p0 + row;
            if constexpr (G1) {
                uint16_t *dst = a.a1 + p * a.a1_ld + cs * 32 + col;
                dst[0] = f32_to_bf16_rne(silu(acc[tt][0][r]) * acc[tt][2][r]);
                dst[16] = f32_to_bf16_rne(silu(acc[tt][1][r]) * acc[tt][3][r]);
            } else {
                const int32_t f = a.sorted_ids[p];
                const float wt = a.topk_w[f];
                float *dst = a.y + (int64_t)f * a.y_ld + cs * 64 + col;
#pragma unroll
                for (int j = 0; j < 4; ++j) dst[16 * j] = wt * acc[tt][j][r];
            }
        }
    }
}

template <bool G1, int NT>
__device__ __forceinline__ void setup_rows(const GemmArgs &a, const WorkItem &it, int lane, const uint16_t *arow[NT]) {
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
        const int row = tt * 16 + (lane & 15);
        arow[tt] = nullptr;
        if (row < it.nrows) {
            const int64_t p = it.p0 + row;
            const int64_t r = G1 ? (int64_t)(a.sorted_ids[p] / a.topk) : p;
            arow[tt] = a.act + r * a.act_ld;
        }
    }
}

// Plan 1: the four waves of a workgroup split the group quads of one superblock; 16-row items.
template <bool G1>
__global__ __launch_bounds__(256) void gemm_ksplit_kernel(GemmArgs a) {
    const int wi = blockIdx.x / a.ncb, cs = blockIdx.x % a.ncb;
    if (wi >= *a.n_work) return;
    const WorkItem it = a.work[wi];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int gq0 = wave * a.gq_total / 4, gq1 = (wave + 1) * a.gq_total / 4;

    const uint16_t *arow[1];
    setup_rows<G1, 1>(a, it, lane, arow);
    f32x4 acc[1][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[0][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint8_t *blk = a.wpk + (((int64_t)it.e * a.ncs + cs) * a.gq_total + gq0) * kBlockBytes;
    wave_mainloop<1>(blk, gq1 - gq0, gq0, arow, lane, acc);

    __shared__ float red[3][16][64];
    if (wave > 0) {
#pragma unroll
        for (int v = 0; v < 16; ++v) red[wave - 1][v][lane] = acc[0][v >> 2][v & 3];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int w = 0; w < 3; ++w)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[0][v >> 2][v & 3] += red[w][v][lane];
        epilogue<G1, 1>(a, it, cs, lane, acc);
    }
}

template <bool G1, int NT>
__device__ __forceinline__ void colsplit_body(const GemmArgs &a, const WorkItem &it, int cs, int lane) {
    const uint16_t *arow[NT];
    setup_rows<G1, NT>(a, it, lane, arow);
    f32x4 acc[NT][4];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[tt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint8_t *blk = a.wpk + ((int64_t)it.e * a.ncs + cs) * a.gq_total * (int64_t)kBlockBytes;
    wave_mainloop<NT>(blk, a.gq_total, 0, arow, lane, acc);
    epilogue<G1, NT>(a, it, cs, lane, acc);
}

// Plan 2: each wave owns one superblock over the whole reduction; items of up to 32 rows.
template <bool G1>
__global__ __launch_bounds__(256) void gemm_colsplit_kernel(GemmArgs a) {
    const int wi = blockIdx.x / a.ncb, cb = blockIdx.x % a.ncb;
    if (wi >= *a.n_work) return;
    const WorkItem it = a.work[wi];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int cs = cb * 4 + wave;
    if (cs >= a.ncs) return;
    const int nt = (it.nrows + 15) >> 4;
    if (nt == 1) colsplit_body<G1, 1>(a, it, cs, lane);
    else colsplit_body<G1, 2>(a, it, cs, lane);
}

}  // namespace

hipError_t launch_gemm(bool gemm1, int plan, const GemmArgs &a, int64_t grid, hipStream_t s) {
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    const dim3 g((unsigned)grid), b(256);
    if (plan == 1) {
        if (gemm1) hipLaunchKernelGGL(gemm_ksplit_kernel<true>, g, b, 0, s, a);
        else hipLaunchKernelGGL(gemm_ksplit_kernel<false>, g, b, 0, s, a);
    } else {
        if (gemm1) hipLaunchKernelGGL(gemm_colsplit_kernel<true>, g, b, 0, s, a);
        else hipLaunchKernelGGL(gemm_colsplit_kernel<false>, g, b, 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace w4moe
