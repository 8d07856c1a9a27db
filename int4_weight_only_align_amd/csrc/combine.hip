// Top-k combine: out[m][c] = bf16_rne( sum_{j = 0..topk-1} y[m*topk + j][c] ), slots summed in order
// in fp32. y (bf16) already carries the routing weight (applied in the GEMM2 epilogue); a slot whose id lies outside
// [0, E) was dropped by the alignment and is skipped here. The weighted sum over the selected
// experts is the MoE combine of the pages ("The Weight-Streaming Threshold", Input Knowledge
// Required, Mixture-of-Experts architecture: each token uses its top-8 experts).
#include "w4moe_internal.h"

namespace w4moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSlotsInFlight = 8;   // slot rows whose loads are issued before any is summed

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// One thread per 8 output columns of one token: the slot rows' 16-byte chunks are loaded together
// (up to kSlotsInFlight at a time), then added in slot order. kAllLocal (a layer holding every
// expert): the rows are loaded beside their ids rather than behind them, one memory latency instead
// of two, and a dropped slot's row (never written this call) is read but not added. On an expert
// shard most slots belong to other shards, and their rows are not read at all.
template <bool kAllLocal>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a, int64_t total) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const int cpr = a.K / 8;   // 8-column chunks per row
    const int m = (int)(idx / cpr);
    const int c = (int)(idx % cpr) * 8;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < a.topk; j0 += kSlotsInFlight) {
        u32x4 v[kSlotsInFlight];
        bool ok[kSlotsInFlight];
#pragma unroll
        for (int jj = 0; jj < kSlotsInFlight; ++jj) {
            const int j = j0 + jj;
            const int64_t f = (int64_t)m * a.topk + j;
            ok[jj] = j < a.topk && (unsigned)local_expert(a.ids[f], a.e_first) < (unsigned)a.E;
            const bool load = kAllLocal ? j < a.topk : ok[jj];
            v[jj] = load ? *reinterpret_cast<const u32x4 *>(a.y + f * a.y_ld + c) : u32x4{0u, 0u, 0u, 0u};
            if (j < a.topk && c == 0 && bad_expert(a.ids[f], a.E_all)) atomicOr(a.err, 1);
        }
#pragma unroll
        for (int jj = 0; jj < kSlotsInFlight; ++jj) {
            if (!ok[jj]) continue;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                s[2 * w] += __uint_as_float(v[jj][w] << 16);
                s[2 * w + 1] += __uint_as_float(v[jj][w] & 0xFFFF0000u);
            }
        }
    }
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) o[w] = bf16_rne_bits(s[2 * w]) | (bf16_rne_bits(s[2 * w + 1]) << 16);
    *reinterpret_cast<u32x4 *>(a.out + (int64_t)m * a.K + c) = o;
}

}  // namespace

hipError_t launch_combine(const CombineArgs &a, hipStream_t s) {
    if (a.M <= 0) return hipSuccess;
    const int64_t total = (int64_t)a.M * (a.K / 8);
    const int64_t grid = (total + 255) / 256;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    if (a.e_first == 0 && a.E == a.E_all)
        hipLaunchKernelGGL(combine_kernel<true>, dim3((unsigned)grid), dim3(256), 0, s, a, total);
    else
        hipLaunchKernelGGL(combine_kernel<false>, dim3((unsigned)grid), dim3(256), 0, s, a, total);
    return hipGetLastError();
}

}  // namespace w4moe
