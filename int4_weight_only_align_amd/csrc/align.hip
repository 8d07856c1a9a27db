// Token-to-expert alignment for the grouped GEMMs, one workgroup of 1024 threads (16 wave64s).
//
// For the T flat routing entries f = m*topk + j: per-expert counts, block-padded offsets (exclusive
// scan), the stable padded sort (rows offsets[e] + r hold the r-th smallest f routed to e; padding
// rows hold T), the expert of every B-row block, the ascending list of active experts, and the GEMM
// work items (chunks of at most CH rows of one expert). The pages do not describe this step (it sits
// inside the fused kernel they time, "The Commit That Captured a Plateau", the commit message); the
// definition above is the plain stable counting sort.
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

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(v, d, 64);
        if (lane >= d) v += t;
    }
    return v;
}

// Exclusive block scan of three values at once; returns the three block totals in tot[].
__device__ __forceinline__ void block_excl_scan3(int v[3], int tot[3], int (*wsum)[kWaves], int tid) {
    const int lane = tid & 63, wave = tid >> 6;
    int incl[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        incl[i] = wave_incl_scan(v[i], lane);
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
// turn per-wave counts into offsets and scatter.
__device__ __forceinline__ void scatter_chunk(const AlignArgs &a, int base, int e, int tid, int lane, int wave,
                                              uint64_t below, int *s_off, int *s_cursor,
                                              uint16_t (*s_wave)[kMaxExperts]) {
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
    // exclusive prefix over the waves of this chunk (< 1024, fits 16 bits); the cursor carries the
    // counts of earlier chunks
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
    if (valid) a.sorted_ids[s_off[e] + s_cursor[e] + s_wave[wave][e] + rank] = f;
    __syncthreads();
    if (tid < E) s_cursor[tid] += chunk_total;
}

__global__ __launch_bounds__(kThreads) void align_kernel(AlignArgs a) {
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int s_off[kMaxExperts];
    __shared__ int s_cursor[kMaxExperts];
    __shared__ uint16_t s_wave[kWaves][kMaxExperts];
    __shared__ int s_wsum[3][kWaves];
    __shared__ int s_bad;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = a.E, T = a.T, B = a.B, CH = a.CH;

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

    // 2. scans: padded rows, work items, active flags
    const int cnt = tid < E ? s_cnt[tid] : 0;
    const int pad_rows = ((cnt + B - 1) / B) * B;
    const int nitems = (cnt + CH - 1) / CH;
    int v[3] = {pad_rows, nitems, cnt > 0 ? 1 : 0};
    int tot[3];
    block_excl_scan3(v, tot, s_wsum, tid);

    // 3. per-expert outputs
    if (tid < E) {
        const int e = tid, off = v[0];
        s_off[e] = off;
        s_cursor[e] = 0;
        a.counts[e] = cnt;
        a.offsets[e] = off;
        if (e == E - 1) a.offsets[E] = tot[0];
        for (int b = off / B; b < (off + pad_rows) / B; ++b) a.block_expert[b] = e;
        for (int p = off + cnt; p < off + pad_rows; ++p) a.sorted_ids[p] = T;
        if (cnt > 0 && a.active) a.active[v[2]] = e;
        for (int c = 0; a.work && c < nitems; ++c) {
            WorkItem w;
            w.e = e;
            w.p0 = off + c * CH;
            w.nrows = min(CH, cnt - c * CH);
            w.pad = 0;
            a.work[v[1] + c] = w;
        }
    }
    if (tid == 0) {
        if (a.n_active) *a.n_active = tot[2];
        if (a.n_work) *a.n_work = tot[1];
    }
    __syncthreads();

    // 4. stable scatter, chunk by chunk in flat order
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int c = 0; c < kRegChunks; ++c)
        if (c * kThreads < T) scatter_chunk(a, c * kThreads, rid[c], tid, lane, wave, below, s_off, s_cursor, s_wave);
    for (int base = kRegChunks * kThreads; base < T; base += kThreads) {
        const int f = base + tid;
        scatter_chunk(a, base, f < T ? local_expert(a.ids[f], a.e_first) : -1, tid, lane, wave, below, s_off, s_cursor,
                      s_wave);
    }
    if (tid == 0 && s_bad) atomicOr(a.err, 1);
}

}  // namespace

hipError_t launch_align(const AlignArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace w4moe
