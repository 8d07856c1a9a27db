// Host runtime of libw4moe: argument checks (all before any HIP call), device buffers, the launch
// plan of forward, and per-kernel event timing. The C-ABI it implements is declared and documented
// in include/w4moe.h.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <atomic>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "w4moe.h"
#include "w4moe_internal.h"

using namespace w4moe;

namespace {

thread_local std::string g_last_error;

w4moe_status fail(w4moe_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

w4moe_status hip_fail(hipError_t e, const char *what) {
    return fail(W4MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kProfCap = 1024;          // forward calls kept between profile reads
constexpr int kStages = 4;              // align, gemm1, gemm2, combine
constexpr int64_t kMaxEntries = 1 << 20;
// T at or below which the single-launch pair mode (no alignment) is chosen. Side by side on one box
// (K2.6, two entry groups, deduplicated items) against the aligned wide kernel: M = 9 286.4 vs 305.1 us,
// M = 10 318.8 vs 323.6, M = 12 375.9 vs 388.7, M = 14 433.9 vs 441.0, M = 16 487.7 vs 481.5.
constexpr int kPairMaxEntries = 120;
constexpr int kNoallocMaxEntries = 64;  // routed entries the no-allocation forward takes
constexpr int kDedupMinEntries = 48;    // pair mode: entries of one expert share items from here on
constexpr int64_t kTargetWaves = 2048;       // waves a GEMM launch should offer before splitting reductions
constexpr size_t kPairMaxRowBytes = 48 * 1024;   // pair mode stages one activation row in LDS
constexpr size_t kPermLdsMaxBytes = 64 * 1024;   // activation order permutes the row in LDS up to two rows here
constexpr int64_t kTicksPerUs = 100;             // the constant clock the kernels' bounded waits read runs at 100 MHz
constexpr int64_t kDefaultWaitUs = 100000;       // bound of a GEMM2 workgroup's wait for its entry's GEMM1 (100 ms)

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace of w4moe_forward_noalloc: one static array per GPU the library runs on, held until the
// process ends. Its first kScratchFlagBytes hold only counters and flags, each of which the kernels
// return to zero before they end, so that zone is all zeros between calls whatever shape the last
// call had; the rest holds data (SwiGLU rows, slot outputs, partial sums). In host code the array's
// name is not a device address: the kernels get the address hipGetSymbolAddress returns for each
// device (looked up once per device, by w4moe_create).
constexpr size_t kScratchFlagBytes = (size_t)5 << 19;    // 2.5 MiB
constexpr size_t kScratchDataBytes = (size_t)11 << 19;   // 5.5 MiB
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchFlagBytes + kScratchDataBytes];
std::mutex g_scratch_mu;
std::atomic<uint8_t *> g_scratch[kMaxDevices];   // per device: the address of `scratch`, or null


bool misaligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) != 0; }

}  // namespace

struct w4moe_ctx {
    w4moe_config cfg{};
    int device = 0;
    uint8_t *w1pk = nullptr, *w2pk = nullptr;
    int64_t w1_bytes = 0, w2_bytes = 0;
    int ncs1 = 0, gq1 = 0, ncs2 = 0, gq2 = 0;
    // K and N rounded up to whole blocks: Kp = 128 * gq1 (W1 rows, staged hidden rows), Np = 128 * gq2
    // (W2 rows, a1 row stride), Kc = 64 * ncs2 (W2 columns, slot-output row stride)
    int32_t Kp = 0, Np = 0, Kc = 0;
    void *ws = nullptr;
    int32_t *counts = nullptr, *offsets = nullptr, *sorted_ids = nullptr, *block_expert = nullptr;
    int32_t *active = nullptr, *n_active = nullptr, *n_work = nullptr, *err = nullptr, *counters = nullptr;
    int32_t *hist = nullptr, *arrive = nullptr;   // alignment above 1024 entries: chunk counts, arrivals
    int32_t *done = nullptr, *ready = nullptr;   // fused pair mode: per-entry GEMM1 count, GEMM2 ready flags
    size_t ready_bytes = 0;
    int64_t ready_cap = 0;                        // ready flags available
    int32_t *wdone = nullptr, *wready = nullptr;  // single-launch wide plan: per-item GEMM1 count, GEMM2 flags
    int64_t wready_cap = 0;                       // its flags available
    float *part1 = nullptr, *part2 = nullptr;     // pair mode split across workgroups: partial sums
    int32_t *xcnt1 = nullptr, *xcnt2 = nullptr;   // and per-superblock arrival counters
    WorkItem *work = nullptr;
    uint16_t *perm1 = nullptr;   // activation order: [E][Kp] group-sorted hidden-feature order per expert
    uint16_t *xg = nullptr;      // activation order: [T_max][Kp] hidden rows gathered per entry
    uint16_t *xpad = nullptr;    // K % 128 != 0: [max_tokens][Kp] hidden rows padded with zeros
    uint16_t *a1 = nullptr;
    float *y = nullptr;
    int64_t T_max = 0, P_cap = 0, W_cap = 0;
    std::vector<uint8_t> packed;
    int64_t n_packed = 0;
    int plan = 0;
    int32_t e_first = 0, E_all = 0;   // expert range held within the whole layer (unsharded: 0, E)
    int force_s1 = 0, force_s2 = 0;   // tuning overrides of the reduction split (W4MOE_S1 / W4MOE_S2)
    // rows per work item of the wide kernel (W4MOE_WIDE_ROWS: 32, 48 or 64; 0: by code width). 4-bit
    // codes take 48 (up to three 16-row tiles): at K2.6 M=1024 the 384 experts average 21 rows, so each
    // takes one item and GEMM1 of the TP8 shard fills exactly one round of resident workgroups (side by
    // side: TP8 M=1024 381.7 -> 355.4 us, TP8 Zipf M=512 313.9 -> 294.0, K2.6 Zipf M=1024 2238 ->
    // 2172, the rest within +-0.5%). 8-bit codes take 32: three tiles of their blocks spill at 3
    // waves per SIMD (W8A16 M=1024: 3.81 ms against 3.53 with 32-row items)
    int wide_rows = 0;
    // the wide plan's GEMMs in one launch: -1 where GEMM2 is the thin kernel (the default), 1 also for the
    // wide GEMM2, 0 never (W4MOE_WIDE_FUSED = 1 / 0 at create)
    int wide_fused = -1;
    int n_cu = 256;   // compute units of the device (hipDeviceAttributeMultiprocessorCount)
    int pair_max = 0;                 // tuning override of kPairMaxEntries (W4MOE_PAIR_MAX, up to 128)
    int dedup_mode = -1;              // tuning switch of the pair-mode item rule (W4MOE_DEDUP: 0 off, 1 on, unset: by T)
    int force_phases = 0;             // tuning override: entry groups of the single-launch mode (W4MOE_PHASES)
    int force_x1 = 0, force_x2 = 0;   // tuning override of the pair-mode split across workgroups (W4MOE_X1 / W4MOE_X2)
    int force_sbw = 0;                // tuning override: superblocks per wave of the thin wide GEMM2 (W4MOE_SBW)
    int64_t wait_ticks = kDefaultWaitUs * kTicksPerUs;   // w4moe_set_wait_limit
    bool prof = false;
    std::vector<hipEvent_t> events;     // kProfCap * (kStages + 1)
    std::vector<uint8_t> recorded;      // per event: recorded in its call (only around launched kernels)
    int64_t prof_calls = 0;
};

namespace {

void free_ctx(w4moe_ctx *h) {
    if (!h) return;
    for (hipEvent_t e : h->events)
        if (e) (void)hipEventDestroy(e);
    if (h->w1pk) (void)hipFree(h->w1pk);
    if (h->w2pk) (void)hipFree(h->w2pk);
    if (h->ws) (void)hipFree(h->ws);
    delete h;
}

w4moe_status check_config(const w4moe_config *c) {
    if (c->num_experts <= 0 || c->hidden <= 0 || c->inter <= 0 || c->topk <= 0 || c->group_size <= 0 ||
        c->max_tokens <= 0)
        return fail(W4MOE_ERR_INVALID_ARG, "config fields must be positive");
    if (c->num_experts > kMaxExperts) return fail(W4MOE_ERR_UNSUPPORTED, "num_experts %d > %d", c->num_experts, kMaxExperts);
    if (c->num_bits != 0 && c->num_bits != 4 && c->num_bits != 8)
        return fail(W4MOE_ERR_UNSUPPORTED, "num_bits must be 4 or 8 (0 means 4; got %d)", c->num_bits);
    if (c->act_order != 0 && c->act_order != 1)
        return fail(W4MOE_ERR_INVALID_ARG, "act_order must be 0 or 1 (got %d)", c->act_order);
    if (c->act_order && c->hidden > 65536)
        return fail(W4MOE_ERR_UNSUPPORTED, "act_order supports hidden <= 65536 (got %d)", c->hidden);
    if (c->hidden > (1 << 30) || c->inter > (1 << 30))
        return fail(W4MOE_ERR_UNSUPPORTED, "hidden and inter must not exceed 2^30");
    if (c->group_size != 32 && c->group_size != 64 && c->group_size != 128)
        return fail(W4MOE_ERR_UNSUPPORTED, "group_size must be 32, 64 or 128 (got %d)", c->group_size);
    // the logical scales cover whole groups of the reduction dimensions (group_size is a multiple of
    // 32, so the packed layout's 32-row scale rows and 16-column slots never straddle data and padding)
    if (c->hidden % c->group_size)
        return fail(W4MOE_ERR_UNSUPPORTED, "hidden %d is not a multiple of group_size %d", c->hidden, c->group_size);
    if (c->inter % c->group_size)
        return fail(W4MOE_ERR_UNSUPPORTED, "inter %d is not a multiple of group_size %d", c->inter, c->group_size);
    if (c->topk > c->num_experts) return fail(W4MOE_ERR_UNSUPPORTED, "topk %d > num_experts %d", c->topk, c->num_experts);
    if ((int64_t)c->max_tokens * c->topk > kMaxEntries)
        return fail(W4MOE_ERR_UNSUPPORTED, "max_tokens * topk exceeds %lld", (long long)kMaxEntries);
    return W4MOE_OK;
}

// Makes the handle's device current for one entry point's duration and gives the calling thread
// its previous device back on the way out (launches are asynchronous, so the switch back is safe).
class DeviceScope {
  public:
    explicit DeviceScope(const w4moe_ctx *h) {
        hipError_t e = hipGetDevice(&prev_);
        if (e != hipSuccess) {
            status_ = hip_fail(e, "hipGetDevice");
            prev_ = -1;
            return;
        }
        if (prev_ != h->device) {
            e = hipSetDevice(h->device);
            if (e != hipSuccess) status_ = hip_fail(e, "hipSetDevice");
            else switched_ = true;
        }
    }
    ~DeviceScope() {
        if (switched_) (void)hipSetDevice(prev_);
    }
    DeviceScope(const DeviceScope &) = delete;
    DeviceScope &operator=(const DeviceScope &) = delete;
    w4moe_status status() const { return status_; }

  private:
    int prev_ = -1;
    bool switched_ = false;
    w4moe_status status_ = W4MOE_OK;
};

AlignArgs align_args(w4moe_ctx *h, const int32_t *ids, int32_t T, int32_t B, int32_t CH) {
    AlignArgs a{};
    a.ids = ids;
    a.T = T;
    a.E = h->cfg.num_experts;
    a.B = B;
    a.CH = CH;
    a.counts = h->counts;
    a.offsets = h->offsets;
    a.sorted_ids = h->sorted_ids;
    a.block_expert = h->block_expert;
    a.active = h->active;
    a.n_active = h->n_active;
    a.work = h->work;
    a.n_work = h->n_work;
    a.err = h->err;
    a.e_first = h->e_first;
    a.E_all = h->E_all;
    a.hist = h->hist;
    a.arrive = h->arrive;
    return a;
}

// The plan forward runs for T = M * topk entries: the one set, 0 resolved from T, pair mode
// replaced by plan 1 when a token row does not fit the LDS budget.
int resolve_plan(const w4moe_ctx *h, int64_t T) {
    int plan = h->plan;
    if (plan == 0) plan = T <= (h->pair_max ? h->pair_max : kPairMaxEntries) ? 3 : 4;
    if (plan == 3 && T > kFusedMaxEntries) plan = 5;
    if ((plan == 3 || plan == 5) &&
        ((size_t)h->Kp * 2 > kPairMaxRowBytes || (size_t)h->Np * 2 > kPairMaxRowBytes))
        plan = 1;
    return plan;
}

// With `device` current: looks up and clears this device's scratch array the first time.
w4moe_status scratch_setup(int device) {
    if (device < 0 || device >= kMaxDevices) return W4MOE_OK;   // w4moe_forward_noalloc reports it
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[device].load()) return W4MOE_OK;
    void *p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(W4MOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned null");
    e = hipMemset(p, 0, kScratchFlagBytes);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "clearing the scratch array");
    g_scratch[device].store(static_cast<uint8_t *>(p));
    return W4MOE_OK;
}

}  // namespace

extern "C" {

const char *w4moe_status_string(w4moe_status s) {
    switch (s) {
        case W4MOE_OK: return "ok";
        case W4MOE_ERR_INVALID_ARG: return "invalid argument";
        case W4MOE_ERR_UNSUPPORTED: return "unsupported";
        case W4MOE_ERR_NOT_PREPACKED: return "weights not prepacked";
        case W4MOE_ERR_OUT_OF_MEMORY: return "out of device memory";
        case W4MOE_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char *w4moe_last_error(void) { return g_last_error.c_str(); }

int32_t w4moe_align_block(w4moe_handle h) { return h ? kAlignBlock : -1; }

w4moe_status w4moe_create(const w4moe_config *cfg, w4moe_handle *out) {
    if (!cfg || !out) return fail(W4MOE_ERR_INVALID_ARG, "null config or output pointer");
    *out = nullptr;
    w4moe_status st = check_config(cfg);
    if (st != W4MOE_OK) return st;

    w4moe_ctx *h = new (std::nothrow) w4moe_ctx();
    if (!h) return fail(W4MOE_ERR_OUT_OF_MEMORY, "host allocation failed");
    h->cfg = *cfg;
    if (h->cfg.num_bits == 0) h->cfg.num_bits = 4;
    h->E_all = cfg->num_experts;
    const int64_t E = cfg->num_experts, K = cfg->hidden, N = cfg->inter, k = cfg->topk;
    h->ncs1 = (int)(2 * N / 64);
    h->gq1 = (int)((K + 127) / 128);
    h->ncs2 = (int)((K + 63) / 64);
    h->gq2 = (int)((N + 127) / 128);
    h->Kp = h->gq1 * 128;
    h->Np = h->gq2 * 128;
    h->Kc = h->ncs2 * 64;
    h->w1_bytes = E * h->ncs1 * h->gq1 * (int64_t)block_bytes(h->cfg.num_bits);
    h->w2_bytes = E * h->ncs2 * h->gq2 * (int64_t)block_bytes(h->cfg.num_bits);
    h->T_max = (int64_t)cfg->max_tokens * k;
    h->P_cap = h->T_max + std::min<int64_t>(E, h->T_max) * (kAlignBlock - 1);
    h->W_cap = h->T_max / kAlignBlock + std::min<int64_t>(E, h->T_max);
    try {
        h->packed.assign((size_t)E, 0);
    } catch (const std::bad_alloc &) {
        delete h;
        return fail(W4MOE_ERR_OUT_OF_MEMORY, "host allocation failed");
    }
    auto env_s = [](const char *name) {
        const char *v = getenv(name);
        const int s = v ? atoi(v) : 0;
        return (s == 1 || s == 2 || s == 4) ? s : 0;
    };
    h->force_s1 = env_s("W4MOE_S1");
    h->force_s2 = env_s("W4MOE_S2");
    {
        const char *x1 = getenv("W4MOE_X1"), *x2 = getenv("W4MOE_X2");
        auto pow2 = [](const char *v) {
            const int x = v ? atoi(v) : 0;
            return (x >= 1 && x <= kMaxSplit && (x & (x - 1)) == 0) ? x : 0;
        };
        h->force_x1 = pow2(x1);
        h->force_x2 = pow2(x2);
        const char *wr = getenv("W4MOE_WIDE_ROWS");
        if (wr && (atoi(wr) == 32 || atoi(wr) == 48 || atoi(wr) == 64)) h->wide_rows = atoi(wr);
        const char *wf = getenv("W4MOE_WIDE_FUSED");
        if (wf) h->wide_fused = atoi(wf) != 0 ? 1 : 0;
        const char *dd = getenv("W4MOE_DEDUP");
        h->dedup_mode = dd ? (atoi(dd) != 0) : -1;
        const char *pm = getenv("W4MOE_PAIR_MAX");
        h->pair_max = pm ? std::max(0, std::min(kFusedMaxEntries, atoi(pm))) : 0;
        const char *ph = getenv("W4MOE_PHASES");
        h->force_phases = ph ? std::max(0, std::min(8, atoi(ph))) : 0;
        const char *sb = getenv("W4MOE_SBW");
        h->force_sbw = sb ? std::max(0, std::min(64, atoi(sb))) : 0;
    }

    hipError_t e = hipGetDevice(&h->device);
    if (e != hipSuccess) {
        free_ctx(h);
        return hip_fail(e, "hipGetDevice");
    }
    {
        int ncu = 0;
        if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, h->device) == hipSuccess && ncu > 0)
            h->n_cu = ncu;
    }
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
    const size_t o_counts = take(E * 4), o_offsets = take((E + 1) * 4), o_sorted = take(h->P_cap * 4);
    const size_t o_blocks = take((h->P_cap / kAlignBlock + 1) * 4), o_active = take(E * 4);
    const size_t o_nact = take(4), o_nwork = take(4), o_err = take(4), o_arrive = take(4);
    const size_t o_hist = take((size_t)((h->T_max + 1023) / 1024) * E * 4);
    const size_t o_work = take(h->W_cap * sizeof(WorkItem));
    const size_t o_cnt = take((size_t)cfg->max_tokens * h->ncs2 * 4);
    h->ready_cap = std::max<int64_t>(kSplitSlots, (int64_t)kFusedMaxEntries * h->ncs2);
    h->ready_bytes = (size_t)h->ready_cap * kReadyStride * 4;
    const size_t o_done = take((size_t)kFusedMaxEntries * 4), o_ready = take(h->ready_bytes);
    h->wready_cap = h->W_cap * ((h->ncs2 + 3) / 4);   // items x GEMM2 column blocks of one superblock per wave
    const size_t o_wdone = take((size_t)h->W_cap * 4), o_wready = take((size_t)h->wready_cap * kWideReadyStride * 4);
    const size_t o_part1 = take((size_t)kSplitSlots * 64 * 4), o_part2 = take((size_t)kSplitSlots * 64 * 4);
    const size_t o_xcnt1 = take((size_t)kSplitSlots * 4), o_xcnt2 = take((size_t)kSplitSlots * 4);
    const size_t o_a1 = take((size_t)h->P_cap * h->Np * 2), o_y = take((size_t)h->T_max * h->Kc * 4);
    const bool ao = cfg->act_order != 0;
    const size_t o_perm1 = ao ? take((size_t)E * h->Kp * 2) : 0, o_xg = ao ? take((size_t)h->T_max * h->Kp * 2) : 0;
    const size_t o_xpad = h->Kp != K ? take((size_t)cfg->max_tokens * h->Kp * 2) : 0;
    const size_t ws_bytes = off;

    if ((e = hipMalloc(&h->w1pk, h->w1_bytes)) != hipSuccess || (e = hipMalloc(&h->w2pk, h->w2_bytes)) != hipSuccess ||
        (e = hipMalloc(&h->ws, ws_bytes)) != hipSuccess) {
        free_ctx(h);
        return fail(W4MOE_ERR_OUT_OF_MEMORY, "device allocation failed: %s", hipGetErrorString(e));
    }
    uint8_t *b = static_cast<uint8_t *>(h->ws);
    h->counts = reinterpret_cast<int32_t *>(b + o_counts);
    h->offsets = reinterpret_cast<int32_t *>(b + o_offsets);
    h->sorted_ids = reinterpret_cast<int32_t *>(b + o_sorted);
    h->block_expert = reinterpret_cast<int32_t *>(b + o_blocks);
    h->active = reinterpret_cast<int32_t *>(b + o_active);
    h->n_active = reinterpret_cast<int32_t *>(b + o_nact);
    h->n_work = reinterpret_cast<int32_t *>(b + o_nwork);
    h->arrive = reinterpret_cast<int32_t *>(b + o_arrive);
    h->hist = reinterpret_cast<int32_t *>(b + o_hist);
    h->err = reinterpret_cast<int32_t *>(b + o_err);
    h->work = reinterpret_cast<WorkItem *>(b + o_work);
    h->counters = reinterpret_cast<int32_t *>(b + o_cnt);
    h->done = reinterpret_cast<int32_t *>(b + o_done);
    h->ready = reinterpret_cast<int32_t *>(b + o_ready);
    h->wdone = reinterpret_cast<int32_t *>(b + o_wdone);
    h->wready = reinterpret_cast<int32_t *>(b + o_wready);
    h->part1 = reinterpret_cast<float *>(b + o_part1);
    h->part2 = reinterpret_cast<float *>(b + o_part2);
    h->xcnt1 = reinterpret_cast<int32_t *>(b + o_xcnt1);
    h->xcnt2 = reinterpret_cast<int32_t *>(b + o_xcnt2);
    h->a1 = reinterpret_cast<uint16_t *>(b + o_a1);
    if (ao) {
        h->perm1 = reinterpret_cast<uint16_t *>(b + o_perm1);
        h->xg = reinterpret_cast<uint16_t *>(b + o_xg);
    }
    if (h->Kp != K) h->xpad = reinterpret_cast<uint16_t *>(b + o_xpad);
    h->y = reinterpret_cast<float *>(b + o_y);
    if ((e = hipMemset(h->ws, 0, ws_bytes)) != hipSuccess) {
        free_ctx(h);
        return hip_fail(e, "hipMemset(workspace)");
    }
    if ((st = scratch_setup(h->device)) != W4MOE_OK) {
        free_ctx(h);
        return st;
    }
    *out = h;
    return W4MOE_OK;
}

void w4moe_destroy(w4moe_handle h) {
    if (!h) return;
    const int dev = h->device;
    int cur = -1;
    if (hipGetDevice(&cur) == hipSuccess && cur != dev) (void)hipSetDevice(dev);
    free_ctx(h);
    if (cur >= 0 && cur != dev) (void)hipSetDevice(cur);
}

}  // extern "C"

namespace {

// Both prepack entry points; w1_perm / w2_perm are null without activation order.
w4moe_status prepack_impl(w4moe_handle h, int32_t first_expert, int32_t num_experts, const int32_t *w1_q,
                          const uint16_t *w1_scales, const int32_t *w1_perm, const int32_t *w2_q,
                          const uint16_t *w2_scales, const int32_t *w2_perm, void *stream) {
    const int32_t E = h->cfg.num_experts;
    if (first_expert < 0 || num_experts < 0 || (int64_t)first_expert + num_experts > E)
        return fail(W4MOE_ERR_INVALID_ARG, "expert range [%d, %d) outside [0, %d)", first_expert,
                    first_expert + num_experts, E);
    if (num_experts == 0) return W4MOE_OK;
    if (!w1_q || !w1_scales || !w2_q || !w2_scales) return fail(W4MOE_ERR_INVALID_ARG, "null weight pointer");
    if (misaligned(w1_q, 4) || misaligned(w2_q, 4) || misaligned(w1_scales, 2) || misaligned(w2_scales, 2) ||
        misaligned(w1_perm, 4) || misaligned(w2_perm, 4))
        return fail(W4MOE_ERR_INVALID_ARG, "misaligned weight or permutation pointer");
    DeviceScope scope(h);
    if (scope.status() != W4MOE_OK) return scope.status();
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int32_t K = h->cfg.hidden, N = h->cfg.inter;
    const int32_t g = h->cfg.group_size;
    const int32_t bits = h->cfg.num_bits;
    // W1: rows in w1_perm's order, gate / up columns in w2_perm's (the intermediate features in the
    // order of W2's packed rows); W2: rows in w2_perm's order
    PrepackArgs p1{w1_q, w1_scales, h->w1pk, first_expert, num_experts, K, 2 * N, N, 1, g, bits, w1_perm, w2_perm,
                   h->err};
    hipError_t e = launch_prepack(p1, h->ncs1, h->gq1, s);
    if (e != hipSuccess) return hip_fail(e, "prepack W1 launch");
    PrepackArgs p2{w2_q, w2_scales, h->w2pk, first_expert, num_experts, N, K, N, 0, g, bits, w2_perm, nullptr,
                   h->err};
    e = launch_prepack(p2, h->ncs2, h->gq2, s);
    if (e != hipSuccess) return hip_fail(e, "prepack W2 launch");
    if (w1_perm) {
        e = launch_store_perm(w1_perm, first_expert, num_experts, K, h->Kp, h->perm1, h->err, s);
        if (e != hipSuccess) return hip_fail(e, "permutation store launch");
    }
    for (int32_t i = first_expert; i < first_expert + num_experts; ++i) {
        if (!h->packed[i]) {
            h->packed[i] = 1;
            ++h->n_packed;
        }
    }
    return W4MOE_OK;
}

}  // namespace

extern "C" {

w4moe_status w4moe_prepack(w4moe_handle h, int32_t first_expert, int32_t num_experts, const int32_t *w1_q,
                           const uint16_t *w1_scales, const int32_t *w2_q, const uint16_t *w2_scales, void *stream) {
    if (!h) return fail(W4MOE_ERR_INVALID_ARG, "null handle");
    if (h->cfg.act_order)
        return fail(W4MOE_ERR_INVALID_ARG, "the layer was created with act_order: use w4moe_prepack_act_order");
    return prepack_impl(h, first_expert, num_experts, w1_q, w1_scales, nullptr, w2_q, w2_scales, nullptr, stream);
}

w4moe_status w4moe_prepack_act_order(w4moe_handle h, int32_t first_expert, int32_t num_experts, const int32_t *w1_q,
                                     const uint16_t *w1_scales, const int32_t *w1_perm, const int32_t *w2_q,
                                     const uint16_t *w2_scales, const int32_t *w2_perm, void *stream) {
    if (!h) return fail(W4MOE_ERR_INVALID_ARG, "null handle");
    if (!h->cfg.act_order)
        return fail(W4MOE_ERR_INVALID_ARG, "the layer was created without act_order: use w4moe_prepack");
    if (num_experts > 0 && (!w1_perm || !w2_perm)) return fail(W4MOE_ERR_INVALID_ARG, "null permutation pointer");
    return prepack_impl(h, first_expert, num_experts, w1_q, w1_scales, w1_perm, w2_q, w2_scales, w2_perm, stream);
}

namespace {

constexpr int kRouteMaxTopk = 64;   // the router gives each slot to one lane of a wave

// Whether GEMM1 of the wide plan is expected to fit one round of resident workgroups (three of the
// wide kernel per compute unit): the distinct experts a uniform routing of `entries` local entries
// reaches, each in ceil(rows / CH) work items, times the column blocks per item. Within one round
// the GEMM1 workgroups all start together and its last ones leave most units idle, which the
// single launch fills with GEMM2 work.
bool wide_one_round(const w4moe_ctx *h, int64_t entries, int CH, int ncb1) {
    const double E = h->cfg.num_experts;
    const double experts = E * (1.0 - std::exp(-(double)entries / E));
    const double rows = (double)entries / std::max(experts, 1.0);
    return experts * std::ceil(rows / CH) * ncb1 <= 3.0 * h->n_cu;
}

// The layer's forward. With logits, the route is computed here (into ids_out / w_out, which then
// serve as the layer's ids and weights); without, topk_ids / topk_weights are the inputs.
// scratch_base: null for the handle's workspace, else this device's scratch array (the no-allocation
// forward, single-launch pair mode only).
w4moe_status forward_impl(w4moe_handle h, const uint16_t *hidden, int32_t M, const int32_t *topk_ids,
                          const float *topk_weights, const float *logits, int32_t *ids_out, float *w_out,
                          uint16_t *out, void *stream, uint8_t *scratch_base = nullptr) {
    if (!h) return fail(W4MOE_ERR_INVALID_ARG, "null handle");
    if (M < 0 || M > h->cfg.max_tokens)
        return fail(W4MOE_ERR_INVALID_ARG, "M = %d outside [0, max_tokens = %d]", M, h->cfg.max_tokens);
    if (M == 0) return W4MOE_OK;
    if (logits) {
        if (!ids_out || !w_out) return fail(W4MOE_ERR_INVALID_ARG, "null route output pointer");
        if (misaligned(logits, 4) || misaligned(ids_out, 4) || misaligned(w_out, 4))
            return fail(W4MOE_ERR_INVALID_ARG, "misaligned logits or route output pointer");
        if (h->cfg.topk > kRouteMaxTopk)
            return fail(W4MOE_ERR_UNSUPPORTED, "routing supports topk <= %d (got %d)", kRouteMaxTopk, h->cfg.topk);
        topk_ids = ids_out;
        topk_weights = w_out;
    }
    if (!hidden || !topk_ids || !topk_weights || !out) return fail(W4MOE_ERR_INVALID_ARG, "null tensor pointer");
    if (misaligned(hidden, 16) || misaligned(out, 8) || misaligned(topk_ids, 4) || misaligned(topk_weights, 4))
        return fail(W4MOE_ERR_INVALID_ARG, "misaligned tensor pointer (hidden needs 16 B, out 8 B)");
    if (h->n_packed < h->cfg.num_experts)
        return fail(W4MOE_ERR_NOT_PREPACKED, "%lld of %d experts prepacked", (long long)h->n_packed,
                    h->cfg.num_experts);
    DeviceScope scope(h);
    if (scope.status() != W4MOE_OK) return scope.status();

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int32_t E = h->cfg.num_experts, K = h->cfg.hidden, N = h->cfg.inter, k = h->cfg.topk;
    const int32_t T = M * k;
    // plan: 3 = pair mode (no alignment; one item per (token, slot)), both GEMMs in one launch;
    // 5 = pair mode in two launches; 1 = 16-row items, reductions split over the four waves;
    // 2 = 32-row items, one superblock per wave; 4 = the wide kernel (32- or 64-row items); 0 = chosen here
    int plan = resolve_plan(h, T);
    if (scratch_base) {
        if (T > kNoallocMaxEntries)
            return fail(W4MOE_ERR_UNSUPPORTED, "the no-allocation forward runs up to %d routed entries (M * topk); "
                        "got %d", kNoallocMaxEntries, T);
        plan = 3;   // the single-launch pair mode, whatever plan is set
        if (resolve_plan(h, T) == 1)
            return fail(W4MOE_ERR_UNSUPPORTED, "the no-allocation forward needs hidden and inter rows of at most %zu "
                        "bytes (one row in LDS)", kPairMaxRowBytes);
    }
    const bool pair = plan == 3 || plan == 5, fused = plan == 3;
    int32_t CH = kAlignBlock;
    if (plan == 2) CH = 2 * kAlignBlock;
    if (plan == 4) CH = h->wide_rows ? h->wide_rows : h->cfg.num_bits == 8 ? 32 : 48;
    const int64_t max_work = T / CH + std::min<int32_t>(E, T);
    // reduction split per GEMM: the smallest S in {1, 2, 4} that offers `target` waves. The
    // single-launch mode asks for more: its GEMM2 waves wait for GEMM1 holding their first blocks,
    // so shorter shares (four blocks fit in registers whole) leave less to stream after the hand-off
    // entries expected to hold a local expert: all of them, or about T * E / E_all on an expert shard
    // (pair mode runs a workgroup per entry, but the other shards' entries stream nothing)
    const int64_t est_local = std::max<int64_t>(1, ((int64_t)T * E + h->E_all - 1) / h->E_all);
    const int64_t est_items = pair ? est_local : std::min<int64_t>(E, T);
    auto pick_s = [&](int ncs, int gq, int forced, int64_t target) {
        if (plan == 4) return 1;   // the wide kernel: one superblock per wave
        if (plan == 2) return 1;
        if (forced) return forced;
        for (int S = 1; S < 4; S *= 2)
            if (est_items * ncs * S >= target || 2 * S > gq) return S;
        return 4;
    };
    const int S1 = pick_s(h->ncs1, h->gq1, h->force_s1, fused ? 2 * kTargetWaves : kTargetWaves);
    const int S2 = pick_s(h->ncs2, h->gq2, h->force_s2, fused ? 4 * kTargetWaves : kTargetWaves);
    // pair mode with few entries: split each superblock's reduction over X workgroups as well, the
    // smallest power of two that offers `target` waves while every wave keeps a block and the
    // partial slots suffice. Each split adds a partial-sum hop to the decode chain, so the targets
    // are lower than the streaming ones: 1024 waves for GEMM1, 256 for GEMM2 (measured on the TP8
    // and EP8 shares at M = 1..8, where GEMM1 split 8 ways and GEMM2 2 ways cost up to 22%)
    auto pick_x = [&](int ncs, int gq, int S, int forced, int64_t target) {
        if (!pair || T > kFusedMaxEntries) return 1;
        int X = 1;
        if (forced) X = forced;
        else
            while (X < kMaxSplit && est_local * ncs * S * X < target && 2 * S * X <= gq) X *= 2;
        while (X > 1 && ((int64_t)T * ncs * X > kSplitSlots || S * X > gq)) X /= 2;
        return X;
    };
    const int X1 = pick_x(h->ncs1, h->gq1, S1, h->force_x1, kTargetWaves / 2);
    const int X2 = pick_x(h->ncs2, h->gq2, S2, h->force_x2, kTargetWaves / 8);
    auto ncb = [](int ncs, int S) { return (ncs + 4 / S - 1) / (4 / S); };

    // the buffers this call works in
    int32_t *counters = h->counters, *done = h->done, *ready = h->ready, *xcnt1 = h->xcnt1, *xcnt2 = h->xcnt2;
    float *part1 = h->part1, *part2 = h->part2, *ybuf = h->y;
    uint16_t *a1 = h->a1, *xpad = h->xpad;
    int64_t ready_cap = h->ready_cap;
    if (scratch_base) {   // carve this call's buffers out of the scratch array's two zones
        size_t fo = 0, dofs = 0;
        auto flag = [&](size_t bytes) { size_t o = fo; fo = align_up(fo + bytes, 256); return o; };
        auto data = [&](size_t bytes) { size_t o = dofs; dofs = align_up(dofs + bytes, 256); return o; };
        ready_cap = (int64_t)T * ncb(h->ncs2, S2) * X2;
        const size_t o_done = flag((size_t)kNoallocMaxEntries * 4), o_cnt = flag((size_t)M * h->ncs2 * 4);
        const size_t o_x1 = flag((size_t)T * h->ncs1 * 4), o_x2 = flag((size_t)T * h->ncs2 * 4);
        const size_t o_ready = flag((size_t)ready_cap * kReadyStride * 4);
        const size_t o_a1 = data((size_t)T * h->Np * 2), o_y = data((size_t)T * h->Kc * 4);
        const size_t o_xp = data(h->xpad ? (size_t)M * h->Kp * 2 : 0);
        const size_t o_p1 = data(X1 > 1 ? (size_t)T * h->ncs1 * X1 * 64 * 4 : 0);
        const size_t o_p2 = data(X2 > 1 ? (size_t)T * h->ncs2 * X2 * 64 * 4 : 0);
        if (fo > kScratchFlagBytes || dofs > kScratchDataBytes)
            return fail(W4MOE_ERR_UNSUPPORTED,
                        "the no-allocation forward needs %zu B of counters and %zu B of data for M = %d; its scratch "
                        "array holds %zu and %zu", fo, dofs, M, kScratchFlagBytes, kScratchDataBytes);
        uint8_t *fz = scratch_base, *dz = scratch_base + kScratchFlagBytes;
        done = reinterpret_cast<int32_t *>(fz + o_done);
        counters = reinterpret_cast<int32_t *>(fz + o_cnt);
        xcnt1 = reinterpret_cast<int32_t *>(fz + o_x1);
        xcnt2 = reinterpret_cast<int32_t *>(fz + o_x2);
        ready = reinterpret_cast<int32_t *>(fz + o_ready);
        a1 = reinterpret_cast<uint16_t *>(dz + o_a1);
        ybuf = reinterpret_cast<float *>(dz + o_y);
        part1 = reinterpret_cast<float *>(dz + o_p1);
        part2 = reinterpret_cast<float *>(dz + o_p2);
        xpad = h->xpad ? reinterpret_cast<uint16_t *>(dz + o_xp) : nullptr;
    }

    // profiling: event i closes stage i - 1; only boundaries next to a launched kernel are recorded
    // (an event record costs a few microseconds of stream time), a missing one reads as the last
    // recorded before it
    hipEvent_t *ev = nullptr;
    uint8_t *rec = nullptr;
    if (h->prof) {
        const size_t slot = (size_t)(h->prof_calls % kProfCap) * (kStages + 1);
        ev = &h->events[slot];
        rec = &h->recorded[slot];
        for (int i = 0; i <= kStages; ++i) rec[i] = 0;
    }
    auto mark = [&](int i) {
        if (ev) {
            (void)hipEventRecord(ev[i], s);
            rec[i] = 1;
        }
    };

    hipError_t e;
    mark(0);
    bool stage0 = false;   // routing, the activation-order gather and alignment
    // activation order: pair mode gathers each entry's row through its expert's feature order while
    // staging it; the aligned plans read rows gathered per entry by a kernel of their own
    const bool ao = h->cfg.act_order != 0, gather = ao && !pair;
    // hidden rows as the kernels read them: widened to whole group quads with zeros when K % 128 != 0
    const uint16_t *xin = hidden;
    if (xpad) {
        e = launch_pad_rows(hidden, M, K, h->Kp, xpad, s);
        if (e != hipSuccess) return hip_fail(e, "pad launch");
        xin = xpad;
        stage0 = true;
    }
    if (logits) {
        RouteArgs ra{logits, M, h->E_all, k, ids_out, w_out, h->err};
        e = launch_route(ra, s);
        if (e != hipSuccess) return hip_fail(e, "route launch");
        stage0 = true;
    }
    if (gather) {
        GatherArgs ga{xin, topk_ids, h->perm1, T, h->Kp, k, E, h->xg, h->e_first};
        e = launch_gather(ga, s);
        if (e != hipSuccess) return hip_fail(e, "gather launch");
        stage0 = true;
    }
    if (!pair) {
        e = launch_align(align_args(h, topk_ids, T, kAlignBlock, CH), s);
        if (e != hipSuccess) return hip_fail(e, "align launch");
        stage0 = true;
    }
    if (stage0) mark(1);

    GemmArgs g{};
    g.pair_mode = pair;
    // pair mode from 48 to 128 entries: entries of one expert share a work item, so its weights stream
    // once for two of them (rows of both entries staged in LDS: within the per-workgroup budget). Below
    // 48 entries two entries rarely share an expert, and finding an item's entries (every workgroup
    // reads all ids and ranks its own by ballot) costs more than it saves: K2.6 side by side, per-entry
    // items against shared ones, M=1 43.55 / 44.01 us, M=2 74.59 / 76.08, M=4 139.99 / 140.92, M=8
    // 269.46 / 261.86
    const size_t row1 = (size_t)h->Kp * 2, row2 = (size_t)h->Np * 2;
    const bool perm_lds_fits = (size_t)h->Kp * 4 <= kPermLdsMaxBytes;
    bool dedup = pair && h->dedup_mode != 0 && (h->dedup_mode == 1 || T >= kDedupMinEntries) &&
                 T <= kFusedMaxEntries && std::max(row1, row2) * 2 <= kPermLdsMaxBytes;
    bool perm_lds = perm_lds_fits && (!dedup || row1 * 3 <= kPermLdsMaxBytes);
    g.dedup = dedup;
    g.bits = h->cfg.num_bits;
    g.ids = topk_ids;
    g.n_items = T;
    g.E = E;
    g.dq_mask = 0x000F000Fu;
    g.dq_exp = 0x43004300u;
    g.dq_zero = 0u;
    g.sorted_ids = h->sorted_ids;
    g.work = h->work;
    g.n_work = h->n_work;
    g.topk = k;
    g.act_div = k;
    g.a1 = a1;
    g.a1_ld = h->Np;
    g.y = ybuf;
    g.yb = reinterpret_cast<uint16_t *>(ybuf);
    g.y_ld = h->Kc;
    g.topk_w = topk_weights;
    g.out = out;
    g.out_ld = K;
    g.out_len = K;
    g.counters = counters;
    g.err = h->err;
    g.done = done;
    g.ready = ready;
    g.xsplit = 1;
    g.sbw = 1;
    g.e_first = h->e_first;
    g.E_all = h->E_all;
    g.wait_ticks = h->wait_ticks;
    const int64_t items = pair ? T : max_work;

    GemmArgs g1 = g;
    g1.wpk = h->w1pk;
    g1.ncs = h->ncs1;
    g1.gq_total = h->gq1;
    g1.act = gather ? h->xg : xin;
    g1.act_ld = h->Kp;
    g1.act_len = h->Kp;   // padded with zeros already
    g1.act_div = gather ? 1 : k;
    g1.perm = ao && pair ? h->perm1 : nullptr;
    g1.perm_lds = perm_lds;   // a row of LDS per workgroup beside the staged rows
    g1.ncb = ncb(h->ncs1, S1);
    g1.xsplit = X1;
    g1.part = part1;
    g1.xcnt = xcnt1;
    GemmArgs g2 = g;
    g2.wpk = h->w2pk;
    g2.ncs = h->ncs2;
    g2.gq_total = h->gq2;
    g2.act = a1;
    g2.act_ld = h->Np;
    g2.act_len = N;
    g2.ncb = ncb(h->ncs2, S2);
    if (plan == 4 && h->gq2 <= 2) {
        // a reduction of one or two blocks (N <= 256): each wave takes two superblocks of two blocks (four
        // of one). TP8 shard, side by side, per call: M=1024 356.3 -> 331.2 us (GEMM2 142.7 -> 113.8),
        // M=330 267.0 -> 258.0, M=90 217.8 -> 212.6; 4, 7 and 14 superblocks per wave were slower (fewer
        // workgroups balance the items' 1-3 tiles worse). Over K2.6's 16 blocks the same walk, with the
        // rows restaged per block, was 1-2% slower at M = 256 and 1024 with two superblocks per wave.
        const int64_t per_item = (h->ncs2 + 3) / 4;
        int64_t sbw = h->force_sbw ? h->force_sbw : (h->gq2 == 1 ? 4 : 2);
        sbw = std::max<int64_t>(1, std::min(sbw, per_item));
        g2.sbw = (int32_t)sbw;
        g2.ncb = (int32_t)((h->ncs2 + 4 * sbw - 1) / (4 * sbw));
    }
    g2.xsplit = X2;
    g2.part = part2;
    g2.xcnt = xcnt2;
    if (fused) {   // one launch; the GEMM1 stage's time covers both GEMMs
        g1.done_target = h->ncs1;
        // two entry groups at 64 routed entries (K2.6 M=8: 261.7 against 271.7 us, side by side); at 8 to
        // 32 entries one group is faster (M=1: 44.0 against 48.3 us with two): the second group's GEMM1
        // then streams with too few workgroups beside the first group's waiting GEMM2 ones
        const int phases = h->force_phases ? h->force_phases : (T >= 64 ? 2 : 1);
        g1.phases = g2.phases = std::max(1, std::min<int>(T, phases));
        g1.ready_n = g2.ready_n = g2.ncb * X2;
        if ((int64_t)T * g2.ready_n > ready_cap)
            return fail(W4MOE_ERR_UNSUPPORTED, "internal: %lld ready flags needed, %lld available",
                        (long long)T * g2.ready_n, (long long)ready_cap);
        e = launch_pair_fused(S1, S2, g1, g2, h->E_all != E || h->e_first != 0, s);
        if (e != hipSuccess) return hip_fail(e, "fused GEMM launch");
        mark(2);
    } else if (plan == 4 && h->cfg.num_bits == 4 && CH <= 48 && !scratch_base &&
               (h->wide_fused == 1 || (h->wide_fused < 0 && (g2.sbw > 1 || wide_one_round(h, est_local, CH, g1.ncb))))) {
        // both GEMMs in one launch, GEMM2 workgroups taking the compute units GEMM1's last ones free. By
        // default where GEMM2 is the thin kernel (N <= 256) or GEMM1 fits one round. Side by side, one
        // against two launches: TP8 shard M = 90 / 330 / 1024 201 / 252 / 322 against 209 / 255 / 335 us,
        // Zipf routing M = 330 / 1024 219 / 345 against 252 / 382; EP8 share (48 experts) M = 90 / 330 /
        // 1024 193 / 237 / 282 against 203 / 242 / 299 us. Over K2.6's several rounds of GEMM1 each
        // workgroup's hand-off (the stores' completion and the count at GEMM1's end, the flag at GEMM2's
        // start) costs more than the overlap returns: 494 / 829 / 1240 against 488 / 799 / 1186 us at
        // M = 16 / 32 / 64, 1470 / 1731 / 2055 against 1367 / 1633 / 2039 at M = 90 / 256 / 1024.
        g1.done = h->wdone;
        g1.ready = g2.ready = h->wready;
        if (items * g2.ncb > h->wready_cap)
            return fail(W4MOE_ERR_UNSUPPORTED, "internal: %lld wide ready flags needed, %lld available",
                        (long long)(items * g2.ncb), (long long)h->wready_cap);
        e = launch_wide_fused(g1, g2, items, s);
        if (e != hipSuccess) return hip_fail(e, "fused wide GEMM launch");
        mark(2);
    } else {
        const GemmKind kind = pair ? GemmKind::kPair : plan == 4 ? GemmKind::kWide : GemmKind::kSorted;
        e = launch_gemm(true, kind, S1, CH, g1, items, s);
        if (e != hipSuccess) return hip_fail(e, "GEMM1 launch");
        mark(2);
        e = launch_gemm(false, kind, S2, CH, g2, items, s);
        if (e != hipSuccess) return hip_fail(e, "GEMM2 launch");
        mark(3);
    }

    if (!pair) {   // pair mode combines inside GEMM2
        CombineArgs c{reinterpret_cast<const uint16_t *>(ybuf), topk_ids, M, K, k, E, h->Kc, out, h->err, h->e_first,
                      h->E_all};
        e = launch_combine(c, s);
        if (e != hipSuccess) return hip_fail(e, "combine launch");
        mark(4);
    }
    if (ev) ++h->prof_calls;
    return W4MOE_OK;
}

}  // namespace

w4moe_status w4moe_forward(w4moe_handle h, const uint16_t *hidden, int32_t M, const int32_t *topk_ids,
                           const float *topk_weights, uint16_t *out, void *stream) {
    return forward_impl(h, hidden, M, topk_ids, topk_weights, nullptr, nullptr, nullptr, out, stream);
}

w4moe_status w4moe_forward_noalloc(w4moe_handle h, const uint16_t *hidden, int32_t M, const int32_t *topk_ids,
                                   const float *topk_weights, uint16_t *out, void *stream) {
    if (!h) return fail(W4MOE_ERR_INVALID_ARG, "null handle");
    uint8_t *base = (h->device >= 0 && h->device < kMaxDevices) ? g_scratch[h->device].load() : nullptr;
    if (!base) return fail(W4MOE_ERR_UNSUPPORTED, "no scratch array address for device %d", h->device);
    return forward_impl(h, hidden, M, topk_ids, topk_weights, nullptr, nullptr, nullptr, out, stream, base);
}

w4moe_status w4moe_forward_logits(w4moe_handle h, const uint16_t *hidden, int32_t M, const float *logits,
                                  int32_t *topk_ids, float *topk_weights, uint16_t *out, void *stream) {
    if (!logits && M > 0) return fail(W4MOE_ERR_INVALID_ARG, "null logits");
    return forward_impl(h, hidden, M, nullptr, nullptr, logits, topk_ids, topk_weights, out, stream);
}

w4moe_status w4moe_route(w4moe_handle h, const float *logits, int32_t M, int32_t *topk_ids, float *topk_weights,
                         void *stream) {
    if (!h) return fail(W4MOE_ERR_INVALID_ARG, "null handle");
    if (M < 0 || M > h->cfg.max_tokens)
        return fail(W4MOE_ERR_INVALID_ARG, "M = %d outside [0, max_tokens = %d]", M, h->cfg.max_tokens);
    if (M == 0) return W4MOE_OK;
    if (!logits || !topk_ids || !topk_weights) return fail(W4MOE_ERR_INVALID_ARG, "null pointer");
    if (misaligned(logits, 4) || misaligned(topk_ids, 4) || misaligned(topk_weights, 4))
        return fail(W4MOE_ERR_INVALID_ARG, "misaligned pointer");
    if (h->cfg.topk > kRouteMaxTopk)
        return fail(W4MOE_ERR_UNSUPPORTED, "routing supports topk <= %d (got %d)", kRouteMaxTopk, h->cfg.topk);
    DeviceScope scope(h);
    if (scope.status() != W4MOE_OK) return scope.status();
    RouteArgs ra{logits, M, h->E_all, h->cfg.topk, topk_ids, topk_weights, h->err};
    const hipError_t e = launch_route(ra, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "route launch");
    return W4MOE_OK;
}

w4moe_status w4moe_moe_align(w4moe_handle h, const int32_t *topk_ids, int32_t M, int32_t block, int32_t *counts,
                             int32_t *offsets, int32_t *sorted_ids, int32_t *block_expert, int32_t *active,
                             int32_t *n_active, void *stream) {
    if (!h) return fail(W4MOE_ERR_INVALID_ARG, "null handle");
    if (M < 0 || M > h->cfg.max_tokens)
        return fail(W4MOE_ERR_INVALID_ARG, "M = %d outside [0, max_tokens = %d]", M, h->cfg.max_tokens);
    if (block < 1 || block > 1024) return fail(W4MOE_ERR_INVALID_ARG, "block %d outside [1, 1024]", block);
    if ((M > 0 && !topk_ids) || !counts || !offsets || !sorted_ids || !block_expert)
        return fail(W4MOE_ERR_INVALID_ARG, "null pointer");
    if (misaligned(topk_ids, 4) || misaligned(counts, 4) || misaligned(offsets, 4) || misaligned(sorted_ids, 4) ||
        misaligned(block_expert, 4) || misaligned(active, 4) || misaligned(n_active, 4))
        return fail(W4MOE_ERR_INVALID_ARG, "misaligned pointer (int32 arrays need 4-byte alignment)");
    DeviceScope scope(h);
    if (scope.status() != W4MOE_OK) return scope.status();
    AlignArgs a = align_args(h, topk_ids, M * h->cfg.topk, block, block);
    a.counts = counts;
    a.offsets = offsets;
    a.sorted_ids = sorted_ids;
    a.block_expert = block_expert;
    a.active = active;
    a.n_active = n_active;
    a.work = nullptr;
    a.n_work = nullptr;
    hipError_t e = launch_align(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "align launch");
    return W4MOE_OK;
}

w4moe_status w4moe_packed_weights(w4moe_handle h, int32_t which, const void **ptr, int64_t *bytes) {
    if (!h || !ptr || !bytes) return fail(W4MOE_ERR_INVALID_ARG, "null argument");
    if (which == 1) {
        *ptr = h->w1pk;
        *bytes = h->w1_bytes;
    } else if (which == 2) {
        *ptr = h->w2pk;
        *bytes = h->w2_bytes;
    } else {
        return fail(W4MOE_ERR_INVALID_ARG, "which must be 1 or 2");
    }
    return W4MOE_OK;
}

w4moe_status w4moe_resolved_plan(w4moe_handle h, int32_t M, int32_t *plan) {
    if (!h || !plan) return fail(W4MOE_ERR_INVALID_ARG, "null argument");
    if (M < 0 || M > h->cfg.max_tokens)
        return fail(W4MOE_ERR_INVALID_ARG, "M = %d outside [0, max_tokens = %d]", M, h->cfg.max_tokens);
    *plan = resolve_plan(h, (int64_t)M * h->cfg.topk);
    return W4MOE_OK;
}

w4moe_status w4moe_set_expert_range(w4moe_handle h, int32_t first_expert, int32_t global_experts) {
    if (!h) return fail(W4MOE_ERR_INVALID_ARG, "null handle");
    if (global_experts > kMaxExperts)
        return fail(W4MOE_ERR_UNSUPPORTED, "global_experts %d > %d", global_experts, kMaxExperts);
    if (first_expert < 0 || global_experts < h->cfg.topk || (int64_t)first_expert + h->cfg.num_experts > global_experts)
        return fail(W4MOE_ERR_INVALID_ARG,
                    "expert range [%d, %d + %d) does not lie in [0, global_experts = %d), or topk %d > global_experts",
                    first_expert, first_expert, h->cfg.num_experts, global_experts, h->cfg.topk);
    h->e_first = first_expert;
    h->E_all = global_experts;
    return W4MOE_OK;
}

w4moe_status w4moe_set_plan(w4moe_handle h, int32_t plan) {
    if (!h) return fail(W4MOE_ERR_INVALID_ARG, "null handle");
    if (plan < 0 || plan > 5) return fail(W4MOE_ERR_INVALID_ARG, "plan must be 0, 1, 2, 3, 4 or 5");
    h->plan = plan;
    return W4MOE_OK;
}

w4moe_status w4moe_set_profiling(w4moe_handle h, int32_t enable) {
    if (!h) return fail(W4MOE_ERR_INVALID_ARG, "null handle");
    if (enable && h->events.empty()) {
        DeviceScope scope(h);
        if (scope.status() != W4MOE_OK) return scope.status();
        try {
            h->events.resize((size_t)kProfCap * (kStages + 1), nullptr);
            h->recorded.assign((size_t)kProfCap * (kStages + 1), 0);
        } catch (const std::bad_alloc &) {
            h->events.clear();
            return fail(W4MOE_ERR_OUT_OF_MEMORY, "host allocation failed");
        }
        for (auto &ev : h->events) {
            // timing-only events: no system-scope fence (cache writeback and invalidate) at record
            // time, which would otherwise stretch the interval of the kernel that follows
            hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableSystemFence);
            if (e != hipSuccess) {   // leave no half-made event set behind
                for (hipEvent_t made : h->events)
                    if (made) (void)hipEventDestroy(made);
                h->events.clear();
                return hip_fail(e, "hipEventCreateWithFlags");
            }
        }
    }
    h->prof = enable != 0;
    h->prof_calls = 0;
    return W4MOE_OK;
}

namespace {

// Sums the recorded stage intervals into ms (if given) and writes each call's align-to-combine
// interval into call_ms[0 .. min(calls, cap)) (if given); clears the record.
w4moe_status read_profile_impl(w4moe_handle h, double *ms, double *call_ms, int64_t cap, int64_t *calls) {
    if (ms)
        for (int i = 0; i < kStages; ++i) ms[i] = 0.0;
    const int64_t n = std::min<int64_t>(h->prof_calls, kProfCap);
    *calls = n;
    if (n == 0) return W4MOE_OK;
    DeviceScope scope(h);
    if (scope.status() != W4MOE_OK) return scope.status();
    hipError_t e0 = hipDeviceSynchronize();   // the events carry no fence of their own
    if (e0 != hipSuccess) return hip_fail(e0, "hipDeviceSynchronize");
    // oldest recorded call first
    const int64_t first = h->prof_calls > kProfCap ? h->prof_calls % kProfCap : 0;
    for (int64_t c = 0; c < n; ++c) {
        const size_t slot = (size_t)((first + c) % kProfCap) * (kStages + 1);
        hipEvent_t *ev = &h->events[slot];
        const uint8_t *rec = &h->recorded[slot];
        int at[kStages + 1];   // event standing for boundary i: the last recorded at or before it
        for (int i = 0; i <= kStages; ++i) at[i] = rec[i] ? i : (i ? at[i - 1] : 0);
        hipError_t e = hipEventSynchronize(ev[at[kStages]]);
        if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
        float t = 0.f;
        if (ms) {
            for (int i = 0; i < kStages; ++i) {
                if (at[i] == at[i + 1]) continue;   // nothing launched in this stage
                e = hipEventElapsedTime(&t, ev[at[i]], ev[at[i + 1]]);
                if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
                ms[i] += t;
            }
        }
        if (call_ms && c < cap) {
            e = hipEventElapsedTime(&t, ev[0], ev[at[kStages]]);
            if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
            call_ms[c] = t;
        }
    }
    h->prof_calls = 0;
    return W4MOE_OK;
}

}  // namespace

w4moe_status w4moe_read_profile(w4moe_handle h, double ms[4], int64_t *calls) {
    if (!h || !ms || !calls) return fail(W4MOE_ERR_INVALID_ARG, "null argument");
    return read_profile_impl(h, ms, nullptr, 0, calls);
}

w4moe_status w4moe_read_profile_calls(w4moe_handle h, double *call_ms, int64_t capacity, int64_t *calls) {
    if (!h || !call_ms || !calls) return fail(W4MOE_ERR_INVALID_ARG, "null argument");
    if (capacity < 0) return fail(W4MOE_ERR_INVALID_ARG, "negative capacity");
    return read_profile_impl(h, nullptr, call_ms, capacity, calls);
}

w4moe_status w4moe_device_error(w4moe_handle h, int32_t *flags) {
    if (!h || !flags) return fail(W4MOE_ERR_INVALID_ARG, "null argument");
    DeviceScope scope(h);
    if (scope.status() != W4MOE_OK) return scope.status();
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
    if ((e = hipMemcpy(flags, h->err, 4, hipMemcpyDeviceToHost)) != hipSuccess) return hip_fail(e, "hipMemcpy");
    if ((e = hipMemset(h->err, 0, 4)) != hipSuccess) return hip_fail(e, "hipMemset");
    return W4MOE_OK;
}

w4moe_status w4moe_set_wait_limit(w4moe_handle h, int64_t microseconds) {
    if (!h) return fail(W4MOE_ERR_INVALID_ARG, "null handle");
    if (microseconds > INT64_MAX / kTicksPerUs) return fail(W4MOE_ERR_INVALID_ARG, "wait limit too large");
    h->wait_ticks = (microseconds < 0 ? kDefaultWaitUs : microseconds) * kTicksPerUs;
    return W4MOE_OK;
}

}  // extern "C"
