// Top-k combine: out[m][c] = bf16_rne( sum_{j = 0..topk-1} y[m*topk + j][c] ), slots summed in order
// in fp32. y (bf16) already carries the routing weight (applied in the GEMM2 epilogue); a slot whose id lies outside
// [0, E) was dropped by the alignment and is skipped here. The weighted sum over the selected
// experts is the MoE combine of the pages ("The Weight-Streaming Threshold", Input Knowledge
// Required, Mixture-of-Experts architecture: each token uses its top-8 experts).
#include "w4moe_internal.h"

namespace w4moe {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a, int nchunks) {
    const int m = blockIdx.x / nchunks;
    const int c = ((blockIdx.x % nchunks) * 256 + threadIdx.x) * 4;
    if (c >= a.K) return;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < a.topk; ++j) {
        const int64_t f = (int64_t)m * a.topk + j;
        const int e = a.ids[f];
        if ((unsigned)e >= (unsigned)a.E) {
            if (c == 0) atomicOr(a.err, 1);
            continue;
        }
        const uint2 v = *reinterpret_cast<const uint2 *>(a.y + f * a.K + c);   // 4 bf16
        s += f32x4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u), __uint_as_float(v.y << 16),
                   __uint_as_float(v.y & 0xFFFF0000u)};
    }
    uint2 o;
    o.x = bf16_rne_bits(s.x) | (bf16_rne_bits(s.y) << 16);
    o.y = bf16_rne_bits(s.z) | (bf16_rne_bits(s.w) << 16);
    *reinterpret_cast<uint2 *>(a.out + (int64_t)m * a.K + c) = o;
}

}  // namespace

hipError_t launch_combine(const CombineArgs &a, hipStream_t s) {
    if (a.M <= 0) return hipSuccess;
    const int nchunks = (a.K / 4 + 255) / 256;
    const int64_t grid = (int64_t)a.M * nchunks;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)grid), dim3(256), 0, s, a, nchunks);
    return hipGetLastError();
}

}  // namespace w4moe
