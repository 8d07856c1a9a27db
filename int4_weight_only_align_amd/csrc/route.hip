// Router kernel: top-k of each token's fp32 logits and the renormalised softmax weights, one wave per
// token (the selection and weights are the wave routine in route_dev.h).
#include "w4moe_internal.h"
#include "route_dev.h"

namespace w4moe {
namespace {

__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= a.M) return;   // uniform over the wave
    int32_t id;
    float w;
    route_wave_any(a.logits + m * a.E, a.E, a.k, lane, &id, &w);
    if (lane < a.k) {
        a.ids[m * a.k + lane] = id;
        a.w[m * a.k + lane] = w;
        if (id < 0) atomicOr(a.err, 1);
    }
}

}  // namespace

hipError_t launch_route(const RouteArgs &a, hipStream_t s) {
    if (a.M <= 0) return hipSuccess;
    hipLaunchKernelGGL(route_kernel, dim3((unsigned)((a.M + 3) / 4)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace w4moe
