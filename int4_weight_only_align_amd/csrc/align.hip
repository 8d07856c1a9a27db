// Token-to-expert alignment for the grouped GEMMs, one workgroup of 1024 threads (16 wave64s).
//
// For the T flat routing entries f = m*topk + j: per-expert counts, block-padded offsets (exclusive
// scan), the stable padded sort (rows offsets[e] + r hold the r-th smallest f routed to e; padding
// rows hold T), the expert of every B-row block, the ascending list of active experts, and the GEMM
// work items (chunks of at most CH rows of one expert). The pages do not describe this step (it sits
// inside the fused kernel they time, "The Commit That Captured a Plateau", the commit message); the
// definition above is the plain stable counting sort.
//
// Below 4096 entries one workgroup does everything. From there two launches share the work, one
// workgroup per chunk of 1024 entries each: the first counts its chunk's experts, and the last of them
// to finish turns the per-chunk counts into per-chunk prefixes and writes the per-expert outputs; the
// second scatters each chunk at its prefix. Either way the order is the stable one.
//
// Stability without a serial pass: entries are taken in chunks of 1024 in flat order. Inside a wave,
// the lanes holding the same expert id are found with ten ballots (one per bit of the id), so a lane's
// rank among equal ids is a popcount of the matching lanes below it. Per-wave counts go to LDS, an
// exclusive prefix over the 16 waves (in wave order) per expert turns them into wave offsets, and a
// running per-expert cursor carries the count across chunks.
#include "w4moe_internal.h"

namespace w4moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

// Inclusive prefix sum over the 64 lanes of a wave in six DPP adds (no LDS round trips): shifts by 1,
// 2, 4 and 8 lanes within each row of 16 give the row prefixes, then lane 15 of each row is added into
// the next row (rows 1 and 3) and lane 31 into rows 2 and 3. A lane whose source lies outside its row,
// or in a row the step does not write, adds the 0 it starts from.
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15, rows 1 and 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31, rows 2 and 3
    return v;
}

// Exclusive block scan of three values at once; returns the three block totals in tot[].
__device__ __forceinline__ void block_excl_scan3(int v[3], int tot[3], int (*wsum)[kWaves], int tid) {
    const int lane = tid & 63, wave = tid >> 6;
    int incl[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        incl[i] = wave_incl_scan(v[i]);
        if (lane == 63) wsum[i][wave] = incl[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        int before = 0, total = 0;
        for (int w = 0; w < kWaves; ++w) {
            const int s = wsum[i][w];
            before += (w < wave) ? s : 0;
            total += s;
        }
        v[i] = before + incl[i] - v[i];
        tot[i] = total;
    }
    __syncthreads();
}

// One chunk of 1024 flat entries, in flat order: rank each entry among the equal ids of its wave,
// turn per-wave counts into offsets and scatter at s_cur[e] (the row where the chunk's first entry of
// expert e goes); with `advance` the cursors then move past the chunk.
__device__ __forceinline__ void scatter_chunk(const AlignArgs &a, int base, int e, int tid, int lane, int wave,
                                              uint64_t below, int *s_cur, uint16_t (*s_wave)[kMaxExperts],
                                              bool advance) {
    const int E = a.E;
    if (tid < E) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s_wave[w][tid] = 0;
    }
    __syncthreads();
    const int f = base + tid;
    const bool valid = (unsigned)e < (unsigned)E;
    if (!valid) e = 0;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 10; ++bit) {
        const bool b = (e >> bit) & 1;
        const uint64_t m = __ballot(valid && b);
        peers &= b ? m : ~m;
    }
    const int rank = __popcll(peers & below);
    if (valid && rank == 0) s_wave[wave][e] = (uint16_t)__popcll(peers);
    __syncthreads();
    // exclusive prefix over the waves of this chunk (< 1024, fits 16 bits)
    int chunk_total = 0;
    if (tid < E) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int c = s_wave[w][tid];
            s_wave[w][tid] = (uint16_t)chunk_total;
            chunk_total += c;
        }
    }
    __syncthreads();
    if (valid) a.sorted_ids[s_cur[e] + s_wave[wave][e] + rank] = f;
    if (advance) {
        __syncthreads();
        if (tid < E) s_cur[tid] += chunk_total;
    }
}

// Sentinel T in rows [lo, hi) of sorted_ids, one coalesced pass of the workgroup. The rows later
// written by the scatter are overwritten after at least one barrier (the stores of this pass are
// complete by then); the others are the padding rows of each expert's last block (and unused rows
// past the last expert's).
__device__ __forceinline__ void fill_sentinel(const AlignArgs &a, int64_t lo, int64_t hi, int tid) {
    for (int64_t p = lo + tid; p < hi; p += kThreads) a.sorted_ids[p] = a.T;
}

// Rows of sorted_ids a call may use: T entries plus at most B - 1 padding rows for each of the at most
// min(E, T) experts that receive any.
__device__ __forceinline__ int64_t sorted_rows(const AlignArgs &a) {
    return (int64_t)a.T + (int64_t)min(a.E, a.T) * (a.B - 1);
}

// Per-expert outputs from the expert counts (thread tid < E holds expert tid's count; every thread
// of the workgroup calls this): counts, block-padded offsets, the expert of every block, the active
// list and the work items (the padding rows already hold the sentinel). The experts' first rows are
// left in s_o (E entries).
__device__ __forceinline__ void expert_outputs(const AlignArgs &a, int cnt, int tid, int (*s_wsum)[kWaves], int *s_o) {
    const int E = a.E, B = a.B, CH = a.CH;
    const int pad_rows = ((cnt + B - 1) / B) * B;
    const int nitems = (cnt + CH - 1) / CH;
    int v[3] = {pad_rows, nitems, cnt > 0 ? 1 : 0};
    int tot[3];
    block_excl_scan3(v, tot, s_wsum, tid);
    if (tid < E) {
        const int e = tid, off = v[0];
        s_o[e] = off;
        a.counts[e] = cnt;
        a.offsets[e] = off;
        if (e == E - 1) a.offsets[E] = tot[0];
        for (int b = off / B; b < (off + pad_rows) / B; ++b) a.block_expert[b] = e;
        if (cnt > 0 && a.active) a.active[v[2]] = e;
        for (int c = 0; a.work && c < nitems; ++c) {
            WorkItem w;
            w.e = e;
            w.p0 = off + c * CH;
            w.nrows = min(CH, cnt - c * CH);
            w.flags = nitems > 1 ? kItemShared : 0;
            a.work[v[1] + c] = w;
        }
    }
    if (tid == 0) {
        if (a.n_active) *a.n_active = tot[2];
        if (a.n_work) *a.n_work = tot[1];
    }
    __syncthreads();
}

__global__ __launch_bounds__(kThreads) void align_kernel(AlignArgs a) {
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int s_cur[kMaxExperts];
    __shared__ uint16_t s_wave[kWaves][kMaxExperts];
    __shared__ int s_wsum[3][kWaves];
    __shared__ int s_bad;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = a.E, T = a.T;

    // the ids of the first kRegChunks chunks are loaded once and kept in registers
    constexpr int kRegChunks = 8;
    int rid[kRegChunks];
#pragma unroll
    for (int c = 0; c < kRegChunks; ++c) {
        const int f = c * kThreads + tid;
        rid[c] = f < T ? local_expert(a.ids[f], a.e_first) : -1;
    }
    if (tid < E) s_cnt[tid] = 0;
    if (tid == 0) s_bad = 0;
    fill_sentinel(a, 0, sorted_rows(a), tid);
    __syncthreads();

    // 1. histogram (order-free)
    auto count = [&](int f, int e) {
        if (f >= T) return;
        if ((unsigned)e < (unsigned)E) atomicAdd(&s_cnt[e], 1);
        else if (bad_expert((int32_t)((uint32_t)e + (uint32_t)a.e_first), a.E_all)) s_bad = 1;
    };
#pragma unroll
    for (int c = 0; c < kRegChunks; ++c) count(c * kThreads + tid, rid[c]);
    for (int f = kRegChunks * kThreads + tid; f < T; f += kThreads) count(f, local_expert(a.ids[f], a.e_first));
    __syncthreads();

    // 2. scans and per-expert outputs
    const int cnt = tid < E ? s_cnt[tid] : 0;
    expert_outputs(a, cnt, tid, s_wsum, s_cur);   // s_cur[e] = the expert's first row

    // 3. stable scatter, chunk by chunk in flat order
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int c = 0; c < kRegChunks; ++c)
        if (c * kThreads < T) scatter_chunk(a, c * kThreads, rid[c], tid, lane, wave, below, s_cur, s_wave, true);
    for (int base = kRegChunks * kThreads; base < T; base += kThreads) {
        const int f = base + tid;
        scatter_chunk(a, base, f < T ? local_expert(a.ids[f], a.e_first) : -1, tid, lane, wave, below, s_cur, s_wave,
                      true);
    }
    if (tid == 0 && s_bad) atomicOr(a.err, 1);
}

// Two-launch alignment, first launch: workgroup c counts the local experts of entries
// [c * 1024, (c + 1) * 1024) and publishes the counts as hist[c][e] (agent-coherent stores, complete
// before the arrival is counted). The last workgroup to arrive replaces every hist[c][e] by the
// exclusive prefix over chunks c' < c, writes the per-expert outputs, and re-zeroes the counter.
__global__ __launch_bounds__(kThreads) void align_hist_kernel(AlignArgs a) {
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int s_off[kMaxExperts];
    __shared__ int s_wsum[3][kWaves];
    __shared__ int s_bad, s_last;
    const int tid = threadIdx.x, E = a.E, T = a.T, nchunks = gridDim.x, c = blockIdx.x;
    const int f = c * kThreads + tid;
    const int e = f < T ? local_expert(a.ids[f], a.e_first) : -1;
    if (tid < E) s_cnt[tid] = 0;
    if (tid == 0) s_bad = 0;
    {   // this chunk's share of the sentinel rows (the scatter launch overwrites the entries' rows)
        const int64_t P = sorted_rows(a), S = (P + nchunks - 1) / nchunks;
        fill_sentinel(a, c * S, min(P, (c + 1) * S), tid);
    }
    __syncthreads();
    if (f < T) {
        if ((unsigned)e < (unsigned)E) atomicAdd(&s_cnt[e], 1);
        else if (bad_expert((int32_t)((uint32_t)e + (uint32_t)a.e_first), a.E_all)) s_bad = 1;
    }
    __syncthreads();
    if (tid < E)
        __hip_atomic_store(a.hist + (int64_t)c * E + tid, s_cnt[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        if (s_bad) atomicOr(a.err, 1);
        s_last = __hip_atomic_fetch_add(a.arrive, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nchunks - 1;
    }
    __syncthreads();
    if (!s_last) return;
    int cnt = 0;
    if (tid < E) {   // eight chunks' counts in flight at a time, then their prefixes written back
        constexpr int kBatch = 8;
        for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
            int v[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                v[j] = c0 + j < nchunks ? __hip_atomic_load(a.hist + (int64_t)(c0 + j) * E + tid, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT)
                                        : 0;
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                if (c0 + j < nchunks) a.hist[(int64_t)(c0 + j) * E + tid] = cnt;
                cnt += v[j];
            }
        }
    }
    expert_outputs(a, cnt, tid, s_wsum, s_off);
    if (tid == 0) __hip_atomic_store(a.arrive, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Second launch: workgroup c scatters its chunk at offsets[e] + hist[c][e].
__global__ __launch_bounds__(kThreads) void align_scatter_kernel(AlignArgs a) {
    __shared__ int s_cur[kMaxExperts];
    __shared__ uint16_t s_wave[kWaves][kMaxExperts];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = blockIdx.x;
    const int f = c * kThreads + tid;
    const int e = f < a.T ? local_expert(a.ids[f], a.e_first) : -1;
    if (tid < a.E) s_cur[tid] = a.offsets[tid] + a.hist[(int64_t)c * a.E + tid];
    __syncthreads();
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    scatter_chunk(a, c * kThreads, e, tid, lane, wave, below, s_cur, s_wave, false);
}

}  // namespace

hipError_t launch_align(const AlignArgs &a, hipStream_t s) {
    // two launches from 4 chunks on: their second launch costs about as much as one workgroup's pass
    // over 2-3 chunks (K2.6, with events: 13.2-14.7 against 11.4-13.0 us at 2 chunks, 19.3-22.5
    // against 23.6-31.5 us at 8)
    const int64_t nchunks = ((int64_t)a.T + kThreads - 1) / kThreads;
    if (nchunks < 4 || !a.hist || !a.arrive) {
        hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kThreads), 0, s, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(align_hist_kernel, dim3((unsigned)nchunks), dim3(kThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(align_scatter_kernel, dim3((unsigned)nchunks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace w4moe
