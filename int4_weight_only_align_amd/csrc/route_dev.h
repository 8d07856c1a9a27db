// Top-k router over one token's logits, computed by one wave (the router kernel's device code).
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

// Largest value over the wave, in every lane, with VALU lane moves only: DPP quad permutations and
// row mirrors reduce each row of 16 lanes, then the four row results are read into scalars. NaN
// never wins (fmaxf returns the other operand); the result is NaN only if every lane holds NaN.
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));   // quad [1,0,3,2]
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));   // quad [2,3,0,1]
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));  // row half mirror
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)));  // row mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Sum over the wave, in every lane, with the same lane moves.
__device__ __forceinline__ float wave_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

// PER logits per lane (expert lane + 64 i), E <= 64 * PER, k <= 64. Every lane takes part; lane
// j < k returns slot j: *id (-1 if no candidate was left) and *w. Each slot: the wave's largest
// remaining logit, then the lowest expert index holding it (one ballot per register slot: indices
// grow with the register slot, then with the lane).
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
        float lm = v[0];
#pragma unroll
        for (int i = 1; i < PER; ++i) lm = fmaxf(lm, v[i]);
        const float best = wave_max(lm);
        int bi = -1;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const unsigned long long hit = __ballot(v[i] == best);
            if (bi < 0 && hit) bi = 64 * i + (__ffsll((long long)hit) - 1);
        }
        if (bi >= 0 && (bi & 63) == lane) {
#pragma unroll
            for (int i = 0; i < PER; ++i)
                if (i == (bi >> 6)) v[i] = kNaN;   // taken
        }
        if (j == 0) lead = best;
        if (lane == j) {
            my_id = bi;
            my_lg = best;
        }
    }
    const float z = (lane < k && my_id >= 0) ? expf(my_lg - lead) : 0.f;
    const float sum = wave_sum(z);
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
