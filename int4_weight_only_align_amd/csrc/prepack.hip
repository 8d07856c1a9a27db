// One-time transform of expert weights from the logical GPTQ-style layout into the library's own
// layout (the role of the pages' repack step: "The Pivot to Real Hardware...", Step 2: The Repack
// Pipeline; here with a layout designed for gfx950 rather than the pages' tile format).
//
// Logical input: codes int32 [ne][R/8][C] (row 8i+t of column c in bits 4t..4t+3 of word (i, c));
// with 8-bit codes [ne][R/4][C] (row 4i+t in bits 8t..8t+7); scales bf16 [ne][R/group][C]. Output,
// per expert e, column superblock cs (64 columns) and group quad gq (128 rows), one block of 4608
// bytes (4-bit) or 8704 bytes (8-bit):
//   codes:  plane p (one plane of the 4-bit codes; the low, then the high nibbles of 8-bit codes),
//           word at p*4096 + gsub*1024 + lane*16 + j*4 holds rows (4gq+gsub)*32 + (lane/16)*8 + t of
//           column col(cs, j, lane%16), row t at bit 0,16,4,20,8,24,12,28 (so that masking pairs
//           (t, t+1) out of a shifted word yields bf16 pairs in row order);
//   scales: bf16 at planes*4096 + ((m*4 + gsub)*4 + j)*2 for rows (4gq+gsub)*32.. of column
//           col(cs, j, m) (the scale of the group they belong to).
// A wave that owns superblock cs thus reads 1 KiB of codes per 128-bit load instruction and one
// 32-byte scale record per lane per block; the transform is a bijection on bits (codes) and a
// permutation (scales).
//
// Shapes whose reduction rows are not a multiple of 128 or whose W2 columns are not a multiple of 64
// are padded up to whole blocks: a padded row or column holds the code of the value 0 (nibble 8 for
// 4-bit codes; 8-bit code 128, i.e. low nibble 0 and high nibble 8) and the scale 0, and the layer
// feeds zeros into the padded rows, so they add exactly nothing.
//
// Activation order (the repack's `perm` argument): packed row i takes logical row row_perm[i], so that
// each scale group becomes 32-row aligned and contiguous again; for W1 the gate and up columns also
// follow W2's row order (col_perm), so GEMM1 writes the intermediate features in the order W2's
// packed rows expect and nothing permutes them at run time.
#include "w4moe_internal.h"

namespace w4moe {
namespace {

__device__ __forceinline__ int column_of(const PrepackArgs &a, int cs, int j, int m) {
    if (a.is_w1) return (j < 2) ? (32 * cs + 16 * j + m) : (a.N + 32 * cs + 16 * (j - 2) + m);
    return 64 * cs + 16 * j + m;
}

// Logical source row of packed row `row` of expert el (identity without activation order).
__device__ __forceinline__ int src_row(const PrepackArgs &a, int64_t el, int row) {
    if (!a.row_perm) return row;
    const int v = a.row_perm[el * a.R + row];
    if ((unsigned)v < (unsigned)a.R) return v;
    atomicOr(a.err, 4);
    return 0;
}

// Logical source column of packed column `col` (W1 gate / up columns follow col_perm).
__device__ __forceinline__ int src_col(const PrepackArgs &a, int64_t el, int col) {
    if (!a.col_perm) return col;
    const bool up = col >= a.N;
    int v = a.col_perm[el * a.N + (up ? col - a.N : col)];
    if ((unsigned)v >= (unsigned)a.N) {
        atomicOr(a.err, 4);
        v = 0;
    }
    return up ? a.N + v : v;
}

__global__ __launch_bounds__(256) void prepack_codes_kernel(PrepackArgs a, int ncs, int gq_total, int64_t total) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const int j = (int)(idx & 3), lane = (int)((idx >> 2) & 63), gsub = (int)((idx >> 8) & 3);
    const int planes = a.bits / 4;
    int64_t rest = idx >> 10;
    const int plane = (int)(rest % planes);
    rest /= planes;
    const int gq = (int)(rest % gq_total);
    rest /= gq_total;
    const int cs = (int)(rest % ncs);
    const int64_t el = rest / ncs;
    const int pcol = column_of(a, cs, j, lane & 15);
    const int64_t row0 = (int64_t)(4 * gq + gsub) * 32 + (lane >> 4) * 8;   // first of the word's 8 rows
    uint32_t o = 0;
    // rows come in whole groups of 32 and columns in whole groups of 16, so a word is all padding or none
    if (row0 >= a.R || pcol >= a.C) {
        const uint32_t zero_nib = (a.bits == 4 || plane == 1) ? 8u : 0u;
        o = zero_nib * 0x11111111u;
    } else if (a.row_perm) {   // each of the 8 rows comes from its own logical word
        const int col = src_col(a, el, pcol);
        const int per = 32 / a.bits;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int sr = src_row(a, el, (int)row0 + t);
            const uint32_t w = (uint32_t)a.codes[(el * (a.R / per) + sr / per) * a.C + col];
            const uint32_t u = (w >> (a.bits * (sr % per))) & ((1u << a.bits) - 1u);
            const uint32_t nib = a.bits == 4 ? u : (plane == 0 ? (u & 0xFu) : (u >> 4));
            o |= nib << (4 * (t >> 1) + 16 * (t & 1));
        }
    } else if (a.bits == 4) {
        const int col = src_col(a, el, pcol);
        const uint32_t w = (uint32_t)a.codes[(el * (a.R / 8) + row0 / 8) * a.C + col];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int pos = 4 * (t >> 1) + 16 * (t & 1);
            o |= ((w >> (4 * t)) & 0xFu) << pos;
        }
    } else {   // 8-bit: the 8 rows span two logical words; this plane takes one nibble of each code
        const int col = src_col(a, el, pcol);
        const int64_t w0 = (el * (a.R / 4) + row0 / 4) * a.C + col;
        const uint32_t lo = (uint32_t)a.codes[w0], hi = (uint32_t)a.codes[w0 + a.C];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int pos = 4 * (t >> 1) + 16 * (t & 1);
            const uint32_t u = ((t < 4 ? lo : hi) >> (8 * (t & 3))) & 0xFFu;
            o |= (plane == 0 ? (u & 0xFu) : (u >> 4)) << pos;
        }
    }
    const int64_t blk = (((a.e0 + el) * ncs + cs) * gq_total + gq) * block_bytes(a.bits);
    *reinterpret_cast<uint32_t *>(a.packed + blk + plane * 4096 + gsub * 1024 + lane * 16 + j * 4) = o;
}

__global__ __launch_bounds__(256) void prepack_scales_kernel(PrepackArgs a, int ncs, int gq_total, int64_t total) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const int j = (int)(idx & 3), gsub = (int)((idx >> 2) & 3), m = (int)((idx >> 4) & 15);
    int64_t rest = idx >> 8;
    const int gq = (int)(rest % gq_total);
    rest /= gq_total;
    const int cs = (int)(rest % ncs);
    const int64_t el = rest / ncs;
    const int pcol = column_of(a, cs, j, m);
    const int64_t row = (int64_t)(4 * gq + gsub) * kGroup;
    uint16_t v = 0;   // padding rows and columns: scale 0
    if (row < a.R && pcol < a.C) {
        const int col = src_col(a, el, pcol);
        // the packed layout holds one scale per 32 rows; a larger logical group repeats its scale (with
        // activation order the packed rows are in group order, so the same holds)
        const int64_t g = row / a.group;
        v = a.scales[(el * (a.R / a.group) + g) * a.C + col];
    }
    const int64_t blk = (((a.e0 + el) * ncs + cs) * gq_total + gq) * block_bytes(a.bits);
    *reinterpret_cast<uint16_t *>(a.packed + blk + code_bytes(a.bits) + (idx & 255) * 2) = v;
}

// Row i < K of expert el: its feature index; rows [K, Kp) of the padded order name feature K, which
// the padded hidden row holds as zero.
__global__ __launch_bounds__(256) void store_perm_kernel(const int32_t *perm, int32_t e0, int32_t K, int32_t Kp,
                                                         uint16_t *dst, int32_t *err, int64_t total) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const int64_t el = idx / Kp;
    const int i = (int)(idx % Kp);
    int v = K;
    if (i < K) {
        v = perm[el * K + i];
        if ((unsigned)v >= (unsigned)K) {
            atomicOr(err, 4);
            v = 0;
        }
    }
    dst[(int64_t)e0 * Kp + idx] = (uint16_t)v;
}

}  // namespace

hipError_t launch_store_perm(const int32_t *perm, int32_t e0, int32_t ne, int32_t K, int32_t Kp, uint16_t *dst,
                             int32_t *err, hipStream_t s) {
    const int64_t total = (int64_t)ne * Kp;
    if (total <= 0) return hipSuccess;
    if ((total + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(store_perm_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, perm, e0, K, Kp, dst,
                       err, total);
    return hipGetLastError();
}

hipError_t launch_prepack(const PrepackArgs &a, int ncs, int gq_total, hipStream_t s) {
    const int64_t nblk = (int64_t)a.ne * ncs * gq_total;
    const int64_t words = nblk * 1024 * (a.bits / 4), scales = nblk * 256;
    if ((words + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    if (words > 0)
        hipLaunchKernelGGL(prepack_codes_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s, a, ncs,
                           gq_total, words);
    if (scales > 0)
        hipLaunchKernelGGL(prepack_scales_kernel, dim3((unsigned)((scales + 255) / 256)), dim3(256), 0, s, a, ncs,
                           gq_total, scales);
    return hipGetLastError();
}

}  // namespace w4moe
