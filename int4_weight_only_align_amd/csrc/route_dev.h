// Top-k router over one token's logits, computed by one wave (device code shared by the router
// kernel and the single-launch pair-mode GEMM kernel).
//
// What is computed (pages: "The Pivot to Real Hardware...", Input Knowledge Required, item 1, and
// "The Weight-Streaming Threshold...", Input Knowledge Required: top-8 routing by a gating network;
// the workload routes by softmax over fp32 logits, top-k, renormalised): the k experts with the
// largest logits, largest first, equal logits taken in ascending expert index, and weights
// w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the chosen k (a softmax over all experts
// renormalised over the chosen ones). NaN logits are never chosen; a slot left without a candidate
// gets id -1 and weight 0. -inf logits are ordinary candidates (weight 0 when a finite one leads);
// each token needs a finite largest logit.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace w4moe {

// (value, index) a beats (value, index) b: larger value, or equal value and lower index. NaN never
// beats anything (its comparisons are false).
__device__ __forceinline__ bool route_beats(float av, int ai, float bv, int bi) {
    return av > bv || (av == bv && ai < bi);
}

// PER logits per lane (expert lane + 64 i), E <= 64 * PER, k <= 64. Every lane takes part; lane
// j < k returns slot j: *id (-1 if no candidate was left) and *w.
template <int PER>
__device__ __forceinline__ void route_wave(const float *row, int E, int k, int lane, int32_t *id, float *w) {
    const float kNaN = __builtin_nanf("");
    float v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? row[e] : kNaN;
    }
    float lead = 0.f, my_lg = 0.f;
    int my_id = -1;
    for (int j = 0; j < k; ++j) {
        float bv = -__builtin_inff();
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < PER; ++i)
            if (route_beats(v[i], lane + 64 * i, bv, bi)) {
                bv = v[i];
                bi = lane + 64 * i;
            }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {   // every lane ends with the wave's best
            const float ov = __shfl_xor(bv, off);
            const int oi = __shfl_xor(bi, off);
            if (route_beats(ov, oi, bv, bi)) {
                bv = ov;
                bi = oi;
            }
        }
        const bool found = bi != 0x7fffffff;
        if (found && (bi & 63) == lane) {
#pragma unroll
            for (int i = 0; i < PER; ++i)
                if (i == (bi >> 6)) v[i] = kNaN;   // taken
        }
        if (j == 0) lead = bv;
        if (lane == j) {
            my_id = found ? bi : -1;
            my_lg = bv;
        }
    }
    const float z = (lane < k && my_id >= 0) ? expf(my_lg - lead) : 0.f;
    float sum = z;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) sum += __shfl_xor(sum, off);
    *id = my_id;
    *w = my_id >= 0 ? z / sum : 0.f;
}

// Dispatch on the logits per lane needed for E experts (E <= 1024).
__device__ __forceinline__ void route_wave_any(const float *row, int E, int k, int lane, int32_t *id, float *w) {
    const int per = (E + 63) >> 6;
    if (per <= 1) route_wave<1>(row, E, k, lane, id, w);
    else if (per <= 2) route_wave<2>(row, E, k, lane, id, w);
    else if (per <= 4) route_wave<4>(row, E, k, lane, id, w);
    else if (per <= 8) route_wave<8>(row, E, k, lane, id, w);
    else route_wave<16>(row, E, k, lane, id, w);
}

}  // namespace w4moe
