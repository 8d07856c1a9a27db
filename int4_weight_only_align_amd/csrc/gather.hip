// Run-time half of activation order (GPTQ act-order weights; the repack's `perm` argument, "The
// Pivot to Real Hardware...", Step 2: The Repack Pipeline): each routed entry's hidden row is put
// in its expert's group-sorted feature order, the order the prepack gave that expert's W1 rows, so
// GEMM1 reads contiguous rows as without activation order.
//
// One thread per 8 consecutive features of one entry: a 16-byte load of the 8 permutation indices,
// 8 two-byte reads of the token's row (a 14 KiB row stays in cache across the entries and chunks
// that read it) and one 16-byte store.
#include "w4moe_internal.h"

namespace w4moe {
namespace {

typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a, int64_t total) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const int chunks = a.K / 8;
    const int64_t f = idx / chunks;
    const int c = (int)(idx % chunks);
    const int e = local_expert(a.ids[f], a.e_first);
    if ((unsigned)e >= (unsigned)a.E) return;   // a dropped or remote entry: no GEMM reads its row
    const uint16_t *xr = a.x + (f / a.topk) * (int64_t)a.K;
    const u16x8 p = *reinterpret_cast<const u16x8 *>(a.perm + (int64_t)e * a.K + c * 8);
    u16x8 v;
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = xr[p[t]];   // stored indices lie in [0, K)
    *reinterpret_cast<u16x8 *>(a.xg + f * (int64_t)a.K + c * 8) = v;
}

// Hidden rows widened to whole 128-feature group quads: xp[m][i] = x[m][i] for i < K, 0 for
// K <= i < Kp (the padded weight rows meet zeros). One thread per 8 features.
__global__ __launch_bounds__(256) void pad_rows_kernel(const uint16_t *x, int32_t K, int32_t Kp, uint16_t *xp,
                                                       int64_t total) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const int chunks = Kp / 8;
    const int64_t m = idx / chunks;
    const int c = (int)(idx % chunks) * 8;
    u16x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
    if (c < K) v = *reinterpret_cast<const u16x8 *>(x + m * K + c);   // K is a multiple of 8
    *reinterpret_cast<u16x8 *>(xp + m * Kp + c) = v;
}

}  // namespace

hipError_t launch_pad_rows(const uint16_t *x, int32_t M, int32_t K, int32_t Kp, uint16_t *xp, hipStream_t s) {
    const int64_t total = (int64_t)M * (Kp / 8);
    if (total <= 0) return hipSuccess;
    if ((total + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(pad_rows_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, x, K, Kp, xp, total);
    return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs &a, hipStream_t s) {
    const int64_t total = (int64_t)a.T * (a.K / 8);
    if (total <= 0) return hipSuccess;
    if ((total + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(gather_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a, total);
    return hipGetLastError();
}

}  // namespace w4moe
