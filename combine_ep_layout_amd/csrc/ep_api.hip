// C ABI of the dispatch/combine library: handle management, host-side
// argument checks and kernel launches.  Declarations and the meaning of every
// argument are in include/ep_layout.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <chrono>
#include <new>
#include <thread>

#include "ep_layout.h"
#include "ep_internal.h"

struct ep_handle {
    ep_config cfg;
    int64_t cap;              // pool capacity rows
    int32_t max_tiles;
    int32_t max_slots;        // max_tokens * top_k
    int32_t ws_blocks;        // workgroups the layout workspace holds
    int device;
    int wall_khz;             // device wall-clock rate (kHz)
    int num_cu;               // compute units of the device
    void* block;              // single device allocation holding every array
    int32_t* counts;
    int32_t* offsets;
    int32_t* num_tiles;
    int32_t* tile_expert;
    int32_t* tile_target;
    uint32_t* arrival;
    uint32_t* tile_ready;
    int32_t* slot_to_row;
    int32_t* recv_token;
    float* weights;
    uint32_t* error;
    int32_t* ws;
    uint32_t* y_done;         // per-token done counts of the combine gate
    uint64_t* tile_stamp;     // consumer acquire stamps (EP_CONSUME_STAMPS)
    // routing density (epk::Density) of a layout, tagged with its epoch
    // (epoch << 32 | density), written by the layout kernel into pinned host
    // memory and read by the combine calls for their launch shape;
    // density_dev is the device's address of the word
    uint64_t* density_host;
    uint64_t* density_dev;
    int32_t density_hint;     // EP_DENSITY_* set by ep_set_density_hint
    // host state of the current layout
    int32_t T;                // tokens of the current layout, -1 before the first
    uint32_t epoch;
    uint32_t seq;
    uint32_t round;           // TILE_READY dispatches since the layout
    // graph capture of the current layout: 0 when it was enqueued eagerly,
    // else the id of the capture it was recorded in
    unsigned long long layout_capture;
    // borrowed-view lease
    bool lease;               // a borrowing dispatch's view is out
    bool lease_wait;          // the next call waits for lease_event first
    hipEvent_t lease_event;   // recorded on the consumer stream at release
};

namespace {

constexpr int32_t kMaxTopK = 32;
constexpr int32_t kMaxExperts = 1024;
constexpr int32_t kMaxBlockM = 4096;
constexpr int32_t kMaxHidden = 1 << 16;
// Work items are (token, row segment) pairs, at most 64 segments per row
// (hidden 65536 in 1024-channel segments), each one wave of a 4-wave
// workgroup: 2^19 tokens keep every grid below 2^31 threads.
constexpr int32_t kMaxTokens = 1 << 19;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

constexpr uint32_t kScaleFlags = EP_SCALE_F32 | EP_SCALE_ROUND | EP_SCALE_MN_MAJOR;

// Scale flavour chosen by the EP_SCALE_* flags.
int32_t scale_kind(uint32_t flags) {
    if (!(flags & EP_SCALE_F32)) return epk::kScaleUe8m0;
    return (flags & EP_SCALE_ROUND) ? epk::kScalePow2F32 : epk::kScaleF32;
}

// Alignment the scale array needs: floats and packed words are 4 bytes.
bool scales_aligned(const void* p, uint32_t flags) {
    return (flags & (EP_SCALE_F32 | EP_SCALE_MN_MAJOR)) ? aligned4(p) : true;
}

int64_t scale_ld_of(int64_t cap) { return (cap + 3) / 4 * 4; }

ep_status check_config(const ep_config* c) {
    if (!c) return EP_ERR_INVALID_ARGUMENT;
    if (c->max_tokens < 0 || c->max_tokens > kMaxTokens || c->top_k < 1 || c->top_k > kMaxTopK || c->num_experts < 1 ||
        c->num_experts > kMaxExperts || c->block_m < 1 || c->block_m > kMaxBlockM)
        return EP_ERR_INVALID_ARGUMENT;
    const int64_t slots = (int64_t)c->max_tokens * c->top_k;
    const int64_t cap = slots + (int64_t)c->num_experts * (c->block_m - 1);
    if (cap > INT32_MAX / 2) return EP_ERR_INVALID_ARGUMENT;
    return EP_OK;
}

ep_status hip_status(hipError_t e) { return e == hipSuccess ? EP_OK : EP_ERR_HIP; }

// Longest a combine call waits on the host for its layout's density word.
constexpr auto kDensityWait = std::chrono::milliseconds(200);

// Routing density of the handle's current layout, for the launch shape of
// the bf16 dispatch, the plain combine and the dispatch backward.  The layout kernel stores it,
// tagged with its epoch, as soon as its total is known; when that store has
// not arrived yet the call waits for it on the host (for the layout kernel
// only, not for the rest of the stream), so the shape follows the routing
// and never the timing.  Under HIP graph capture nothing has run yet, and a
// captured call takes the dense shape.  A layout that has not run after
// kDensityWait (a stream held back by work the host has not enqueued yet)
// also gets the dense shape.  Sizes whose shape does not depend on the
// density do not wait.
// The density report of the current layout, waiting up to kDensityWait;
// kDensityUnknown when it does not arrive.
int32_t reported_density(const ep_handle* h) {
    const auto start = std::chrono::steady_clock::now();
    for (;;) {
        const uint64_t w = __atomic_load_n(h->density_host, __ATOMIC_ACQUIRE);
        if ((uint32_t)(w >> 32) == h->epoch) return (int32_t)(uint32_t)w;
        if (std::chrono::steady_clock::now() - start > kDensityWait) return epk::kDensityUnknown;
        std::this_thread::yield();
    }
}

int32_t current_density(const ep_handle* h, bool shape_depends, hipStream_t stream) {
    if (h->density_hint == EP_DENSITY_SPARSE) return epk::kDensitySparse;
    if (h->density_hint == EP_DENSITY_DENSE) return epk::kDensityDense;
    if (!shape_depends) return epk::kDensityDense;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) {
        (void)hipGetLastError();
        return epk::kDensityDense;
    }
    const int32_t d = reported_density(h);
    return d == epk::kDensityUnknown ? epk::kDensityDense : d;
}

// Id of the graph capture `stream` is in, 0 when it is not capturing.
unsigned long long capture_id(hipStream_t stream) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    unsigned long long id = 0;
    if (hipStreamGetCaptureInfo(stream, &cs, &id) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return cs == hipStreamCaptureStatusActive ? (id ? id : ~0ull) : 0;
}

// A streaming dispatch and a gated combine rely on counts that only the
// layout resets (tile arrivals, per-token done counts).  Captured into a
// graph without that layout, a replay would find the previous replay's
// counts and stamps and its consumers could pass early: refuse it.
bool capture_without_layout(const ep_handle* h, hipStream_t stream) {
    const unsigned long long id = capture_id(stream);
    return id != 0 && id != h->layout_capture;
}

// Calls that rewrite the row map wait for the consumers of a released view.
ep_status wait_lease(ep_handle* h, hipStream_t stream) {
    if (!h->lease_wait) return EP_OK;
    if (hipStreamWaitEvent(stream, h->lease_event, 0) != hipSuccess) return EP_ERR_HIP;
    h->lease_wait = false;
    return EP_OK;
}

}  // namespace

extern "C" {

const char* ep_status_string(ep_status s) {
    switch (s) {
        case EP_OK: return "ok";
        case EP_ERR_INVALID_ARGUMENT: return "invalid argument";
        case EP_ERR_UNSUPPORTED: return "unsupported";
        case EP_ERR_OUT_OF_MEMORY: return "out of device memory";
        case EP_ERR_HANDLE_STATE: return "handle has no layout or the epoch does not match";
        case EP_ERR_BAD_ROUTING: return "expert id outside [-1, num_experts)";
        case EP_ERR_TIMEOUT: return "consumer wait timed out";
        case EP_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

ep_status ep_handle_create(const ep_config* cfg, ep_handle** out) {
    if (!out) return EP_ERR_INVALID_ARGUMENT;
    *out = nullptr;
    ep_status st = check_config(cfg);
    if (st != EP_OK) return st;

    ep_handle* h = new (std::nothrow) ep_handle();
    if (!h) return EP_ERR_OUT_OF_MEMORY;
    h->cfg = *cfg;
    const int32_t K = cfg->top_k, E = cfg->num_experts, BM = cfg->block_m;
    h->max_slots = cfg->max_tokens * K;
    h->cap = (int64_t)h->max_slots + (int64_t)E * (BM - 1);
    h->max_tiles = (int32_t)(h->cap / BM);
    h->ws_blocks = epk::layout_blocks(h->max_slots);
    h->T = -1;
    h->layout_capture = 0;
    h->epoch = 0;
    h->seq = 0;
    h->round = 0;

    if (hipGetDevice(&h->device) != hipSuccess ||
        hipDeviceGetAttribute(&h->wall_khz, hipDeviceAttributeWallClockRate, h->device) != hipSuccess ||
        hipDeviceGetAttribute(&h->num_cu, hipDeviceAttributeMultiprocessorCount, h->device) != hipSuccess) {
        delete h;
        return EP_ERR_HIP;
    }
    if (h->wall_khz <= 0) h->wall_khz = 100000;
    if (h->num_cu <= 0) h->num_cu = 1;

    // one allocation, every array 256-byte aligned
    struct Part { void** dst; size_t bytes; };
    const size_t mt = (size_t)h->max_tiles, ms = (size_t)h->max_slots;
    Part parts[] = {
        {(void**)&h->counts, sizeof(int32_t) * E},
        {(void**)&h->offsets, sizeof(int32_t) * (E + 1)},
        {(void**)&h->num_tiles, sizeof(int32_t)},
        {(void**)&h->tile_expert, sizeof(int32_t) * mt},
        {(void**)&h->tile_target, sizeof(int32_t) * mt},
        {(void**)&h->arrival, sizeof(uint32_t) * mt},
        {(void**)&h->tile_ready, sizeof(uint32_t) * mt},
        {(void**)&h->slot_to_row, sizeof(int32_t) * ms},
        {(void**)&h->recv_token, sizeof(int32_t) * (size_t)h->cap},
        {(void**)&h->weights, sizeof(float) * ms},
        {(void**)&h->error, sizeof(uint32_t)},
        {(void**)&h->ws, sizeof(int32_t) * (size_t)h->ws_blocks * E},
        {(void**)&h->y_done, sizeof(uint32_t) * (size_t)cfg->max_tokens},
        {(void**)&h->tile_stamp, sizeof(uint64_t) * mt},
    };
    size_t total = 0;
    for (const Part& p : parts) total += round_up(p.bytes ? p.bytes : 1, 256);
    if (hipMalloc(&h->block, total) != hipSuccess) {
        (void)hipGetLastError();
        delete h;
        return EP_ERR_OUT_OF_MEMORY;
    }
    size_t off = 0;
    for (const Part& p : parts) {
        *p.dst = (char*)h->block + off;
        off += round_up(p.bytes ? p.bytes : 1, 256);
    }
    if (hipMemset(h->block, 0, total) != hipSuccess || hipDeviceSynchronize() != hipSuccess ||
        hipEventCreateWithFlags(&h->lease_event, hipEventDisableTiming) != hipSuccess) {
        (void)hipFree(h->block);
        delete h;
        return EP_ERR_HIP;
    }
    if (hipHostMalloc((void**)&h->density_host, 64, hipHostMallocDefault) != hipSuccess) {
        (void)hipGetLastError();
        (void)hipEventDestroy(h->lease_event);
        (void)hipFree(h->block);
        delete h;
        return EP_ERR_OUT_OF_MEMORY;
    }
    __atomic_store_n(h->density_host, (uint64_t)epk::kDensityUnknown, __ATOMIC_RELAXED);
    if (hipHostGetDevicePointer((void**)&h->density_dev, h->density_host, 0) != hipSuccess ||
        !h->density_dev) {
        (void)hipHostFree(h->density_host);
        (void)hipEventDestroy(h->lease_event);
        (void)hipFree(h->block);
        delete h;
        return EP_ERR_HIP;
    }
    h->lease = false;
    h->lease_wait = false;
    h->density_hint = EP_DENSITY_AUTO;
    *out = h;
    return EP_OK;
}

ep_status ep_handle_destroy(ep_handle* h) {
    if (!h) return EP_OK;
    if (h->lease) return EP_ERR_HANDLE_STATE;
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != h->device) e = hipSetDevice(h->device);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    hipError_t f = hipFree(h->block);
    if (f == hipSuccess) f = hipHostFree(h->density_host);
    else (void)hipHostFree(h->density_host);
    (void)hipEventDestroy(h->lease_event);
    if (cur != h->device) (void)hipSetDevice(cur);
    delete h;
    return (e == hipSuccess && f == hipSuccess) ? EP_OK : EP_ERR_HIP;
}

int64_t ep_pool_capacity_rows(const ep_handle* h) { return h ? h->cap : -1; }

int32_t ep_max_tiles(const ep_handle* h) { return h ? h->max_tiles : -1; }

int32_t ep_num_tokens(const ep_handle* h) { return h ? h->T : -1; }

int64_t ep_scale_ld(const ep_handle* h) { return h ? scale_ld_of(h->cap) : -1; }

namespace {

// Argument checks of a layout of num_tokens tokens (no state change).
ep_status check_layout(const ep_handle* h, const int32_t* topk_idx, const float* topk_weights,
                       int32_t num_tokens) {
    if (!h || num_tokens < 0 || num_tokens > h->cfg.max_tokens) return EP_ERR_INVALID_ARGUMENT;
    if (num_tokens > 0 && (!topk_idx || !topk_weights || !aligned4(topk_idx) ||
                           !aligned4(topk_weights)))
        return EP_ERR_INVALID_ARGUMENT;
    if (h->lease) return EP_ERR_HANDLE_STATE;
    return EP_OK;
}

epk::LayoutArgs layout_args(const ep_handle* h, const int32_t* topk_idx, const float* topk_weights,
                            int32_t num_tokens) {
    epk::LayoutArgs a{};
    a.topk_idx = topk_idx;
    a.topk_w = topk_weights;
    a.S = num_tokens * h->cfg.top_k;
    a.K = h->cfg.top_k;
    a.E = h->cfg.num_experts;
    a.BM = h->cfg.block_m;
    a.cap = (int32_t)h->cap;
    a.max_tiles = h->max_tiles;
    a.counts = h->counts;
    a.offsets = h->offsets;
    a.num_tiles = h->num_tiles;
    a.tile_expert = h->tile_expert;
    a.tile_target = h->tile_target;
    a.arrival = h->arrival;
    a.tile_ready = h->tile_ready;
    a.seq_base = h->seq;
    a.slot_to_row = h->slot_to_row;
    a.recv_token = h->recv_token;
    a.weights = h->weights;
    a.error = h->error;
    a.ws = h->ws;
    a.y_done = h->y_done;
    a.density = h->density_dev;
    a.epoch = h->epoch + 1;
    return a;
}

// Handle state once a layout of num_tokens tokens is enqueued.
void after_layout(ep_handle* h, int32_t num_tokens, hipStream_t stream, uint32_t* epoch_out) {
    h->layout_capture = capture_id(stream);
    h->T = num_tokens;
    h->epoch += 1;
    h->round = 0;
    if (epoch_out) *epoch_out = h->epoch;
}

// Argument checks of a copying dispatch (not BORROW) of T tokens.
ep_status check_dispatch(const ep_handle* h, int32_t T, const void* x, int32_t hidden, const void* pool,
                         const void* pool_scales, uint32_t flags) {
    if (flags & ~(EP_DISPATCH_FP8 | EP_DISPATCH_TILE_READY | kScaleFlags)) return EP_ERR_INVALID_ARGUMENT;
    const bool fp8 = (flags & EP_DISPATCH_FP8) != 0;
    if (!fp8 && (flags & kScaleFlags)) return EP_ERR_INVALID_ARGUMENT;
    if (hidden <= 0 || hidden % 8 != 0) return EP_ERR_INVALID_ARGUMENT;
    if (hidden > kMaxHidden) return EP_ERR_UNSUPPORTED;
    if (fp8 && (hidden % 128 != 0 || !pool_scales || !scales_aligned(pool_scales, flags)))
        return EP_ERR_INVALID_ARGUMENT;
    if (!fp8 && pool_scales) return EP_ERR_INVALID_ARGUMENT;
    if (T < 0 || h->lease) return EP_ERR_HANDLE_STATE;
    if (T > 0 && (!x || !pool || !aligned16(x) || !aligned16(pool))) return EP_ERR_INVALID_ARGUMENT;
    return EP_OK;
}

epk::DispatchArgs dispatch_args(const ep_handle* h, int32_t T, uint32_t round, const void* x, int32_t hidden,
                                void* pool, void* pool_scales, uint32_t flags) {
    const bool ready = (flags & EP_DISPATCH_TILE_READY) != 0;
    epk::DispatchArgs a{};
    a.x = x;
    a.T = T;
    a.K = h->cfg.top_k;
    a.H = hidden;
    a.BM = h->cfg.block_m;
    a.E = h->cfg.num_experts;
    a.slot_to_row = h->slot_to_row;
    a.tile_expert = h->tile_expert;
    a.tile_target = h->tile_target;
    a.pool = pool;
    a.scales = pool_scales;
    a.scale_kind = scale_kind(flags);
    a.scale_mn = (flags & EP_SCALE_MN_MAJOR) ? 1 : 0;
    a.scale_ld = scale_ld_of(h->cap);
    a.max_tiles = h->max_tiles;
    a.arrival = h->arrival;
    a.tile_ready = h->tile_ready;
    a.seq = h->seq + 1;
    a.round = round + (ready ? 1u : 0u);
    a.density = epk::kDensitySparse;
    return a;
}

void after_dispatch(ep_handle* h, const epk::DispatchArgs& a, uint32_t* seq_out) {
    h->seq = a.seq;
    h->round = a.round;
    if (seq_out) *seq_out = a.seq;
}

}  // namespace

ep_status ep_layout(ep_handle* h, const int32_t* topk_idx, const float* topk_weights,
                    int32_t num_tokens, hipStream_t stream, uint32_t* epoch_out) {
    ep_status cs = check_layout(h, topk_idx, topk_weights, num_tokens);
    if (cs != EP_OK) return cs;
    ep_status ws = wait_lease(h, stream);
    if (ws != EP_OK) return ws;
    ep_status st = hip_status(epk::launch_layout(layout_args(h, topk_idx, topk_weights, num_tokens), stream));
    if (st != EP_OK) return st;
    after_layout(h, num_tokens, stream, epoch_out);
    return EP_OK;
}

ep_status ep_dispatch(ep_handle* h, const void* x, int32_t hidden, void* pool,
                      void* pool_scales, uint32_t flags, hipStream_t stream,
                      uint32_t* seq_out) {
    if (!h) return EP_ERR_INVALID_ARGUMENT;
    if (flags & ~(EP_DISPATCH_FP8 | EP_DISPATCH_TILE_READY | EP_DISPATCH_BORROW | kScaleFlags))
        return EP_ERR_INVALID_ARGUMENT;
    const bool fp8 = (flags & EP_DISPATCH_FP8) != 0;
    if (!fp8 && (flags & kScaleFlags)) return EP_ERR_INVALID_ARGUMENT;
    const bool ready = (flags & EP_DISPATCH_TILE_READY) != 0;
    if (hidden <= 0 || hidden % 8 != 0) return EP_ERR_INVALID_ARGUMENT;
    if (hidden > kMaxHidden) return EP_ERR_UNSUPPORTED;
    if (flags & EP_DISPATCH_BORROW) {
        // lend x through the row map: bf16 only, nothing to copy into
        if (fp8 || ready) return EP_ERR_UNSUPPORTED;
        if (pool || pool_scales) return EP_ERR_INVALID_ARGUMENT;
        if (h->T < 0 || h->lease) return EP_ERR_HANDLE_STATE;
        if (h->T > 0 && (!x || !aligned16(x))) return EP_ERR_INVALID_ARGUMENT;
        h->lease = true;
        h->seq += 1;
        if (seq_out) *seq_out = h->seq;
        return EP_OK;
    }
    ep_status cs = check_dispatch(h, h->T, x, hidden, pool, pool_scales, flags);
    if (cs != EP_OK) return cs;
    if (ready && capture_without_layout(h, stream)) return EP_ERR_UNSUPPORTED;
    ep_status ws = wait_lease(h, stream);
    if (ws != EP_OK) return ws;
    epk::DispatchArgs a = dispatch_args(h, h->T, h->round, x, hidden, pool, pool_scales, flags);
    // launch shape of the bf16 dispatch (dense routing: one workgroup per
    // token segment), from the current layout's report as for ep_combine
    const bool shape_depends = !fp8 && !ready && epk::dispatch_shape_uses_density(a.T, a.H, a.K);
    if (shape_depends) a.density = current_density(h, true, stream);
    ep_status st = hip_status(epk::launch_dispatch(a, fp8, ready, stream));
    if (st != EP_OK) return st;
    after_dispatch(h, a, seq_out);
    return EP_OK;
}

ep_status ep_layout_dispatch(ep_handle* h, const int32_t* topk_idx, const float* topk_weights,
                             int32_t num_tokens, const void* x, int32_t hidden, void* pool,
                             void* pool_scales, uint32_t flags, hipStream_t stream,
                             uint32_t* epoch_out, uint32_t* seq_out) {
    ep_status cs = check_layout(h, topk_idx, topk_weights, num_tokens);
    if (cs != EP_OK) return cs;
    if (flags & EP_DISPATCH_BORROW) return EP_ERR_UNSUPPORTED;
    cs = check_dispatch(h, num_tokens, x, hidden, pool, pool_scales, flags);
    if (cs != EP_OK) return cs;
    const bool fp8 = (flags & EP_DISPATCH_FP8) != 0;
    const bool ready = (flags & EP_DISPATCH_TILE_READY) != 0;
    const int64_t slots = (int64_t)num_tokens * h->cfg.top_k;
    if (ready || num_tokens == 0 || slots > epk::kLayoutSlotsPerBlock) {
        // the two calls, one after the other (the arguments are already checked)
        ep_status st = ep_layout(h, topk_idx, topk_weights, num_tokens, stream, epoch_out);
        if (st != EP_OK) return st;
        return ep_dispatch(h, x, hidden, pool, pool_scales, flags, stream, seq_out);
    }
    ep_status ws = wait_lease(h, stream);
    if (ws != EP_OK) return ws;
    const epk::LayoutArgs la = layout_args(h, topk_idx, topk_weights, num_tokens);
    const epk::DispatchArgs a = dispatch_args(h, num_tokens, 0u, x, hidden, pool, pool_scales, flags);
    ep_status st = hip_status(epk::launch_layout_dispatch(la, a, fp8, stream));
    if (st != EP_OK) return st;
    after_layout(h, num_tokens, stream, epoch_out);
    after_dispatch(h, a, seq_out);
    return EP_OK;
}

ep_status ep_combine(const ep_handle* h, uint32_t epoch, const void* expert_out, int32_t hidden,
                     void* y, hipStream_t stream) {
    if (!h) return EP_ERR_INVALID_ARGUMENT;
    if (hidden <= 0 || hidden % 8 != 0) return EP_ERR_INVALID_ARGUMENT;
    if (hidden > kMaxHidden) return EP_ERR_UNSUPPORTED;
    if (h->T < 0 || epoch != h->epoch || h->lease) return EP_ERR_HANDLE_STATE;
    if (h->T > 0 && (!expert_out || !y || !aligned16(expert_out) || !aligned16(y)))
        return EP_ERR_INVALID_ARGUMENT;
    epk::CombineArgs a{};
    a.expert_out = expert_out;
    a.T = h->T;
    a.K = h->cfg.top_k;
    a.H = hidden;
    a.slot_to_row = h->slot_to_row;
    a.weights = h->weights;
    a.y = y;
    a.num_cu = h->num_cu;
    // launch shape only
    a.density = current_density(h, epk::combine_shape_uses_density(h->T, hidden, h->num_cu), stream);
    return hip_status(epk::launch_combine(a, stream));
}

ep_status ep_combine_gated(const ep_handle* h, uint32_t epoch, const void* expert_out,
                           int32_t hidden, void* y, uint32_t round, uint32_t spin_limit_us,
                           hipStream_t stream) {
    if (!h) return EP_ERR_INVALID_ARGUMENT;
    if (hidden <= 0 || hidden % 8 != 0 || round == 0) return EP_ERR_INVALID_ARGUMENT;
    if (hidden > kMaxHidden) return EP_ERR_UNSUPPORTED;
    if (h->T < 0 || epoch != h->epoch || h->lease) return EP_ERR_HANDLE_STATE;
    if (h->T > 0 && (!expert_out || !y || !aligned16(expert_out) || !aligned16(y)))
        return EP_ERR_INVALID_ARGUMENT;
    if (capture_without_layout(h, stream)) return EP_ERR_UNSUPPORTED;
    epk::CombineArgs a{};
    a.expert_out = expert_out;
    a.T = h->T;
    a.K = h->cfg.top_k;
    a.H = hidden;
    a.slot_to_row = h->slot_to_row;
    a.weights = h->weights;
    a.y = y;
    a.y_done = h->y_done;
    a.round = round;
    a.limit_ticks = (uint64_t)spin_limit_us * (uint64_t)h->wall_khz / 1000u;
    a.error = h->error;
    a.num_cu = h->num_cu;
    return hip_status(epk::launch_combine_gated(a, stream));
}

ep_status ep_fp8_cast_back(const void* q, const void* scales, uint32_t flags, int64_t rows,
                           int64_t scale_ld, int32_t hidden, void* out, hipStream_t stream) {
    if (flags & ~(kScaleFlags | EP_DISPATCH_FP8)) return EP_ERR_INVALID_ARGUMENT;
    if (rows < 0 || hidden <= 0 || hidden % 128 != 0) return EP_ERR_INVALID_ARGUMENT;
    if (hidden > kMaxHidden) return EP_ERR_UNSUPPORTED;
    if ((flags & EP_SCALE_MN_MAJOR) && scale_ld < rows) return EP_ERR_INVALID_ARGUMENT;
    if (rows == 0) return EP_OK;
    if (!q || !scales || !out || !aligned16(q) || !aligned16(out) || !scales_aligned(scales, flags))
        return EP_ERR_INVALID_ARGUMENT;
    epk::CastBackArgs a{};
    a.q = q;
    a.scales = scales;
    a.scale_kind = scale_kind(flags);
    a.scale_mn = (flags & EP_SCALE_MN_MAJOR) ? 1 : 0;
    a.scale_ld = scale_ld;
    a.rows = rows;
    a.H = hidden;
    a.out = out;
    return hip_status(epk::launch_cast_back(a, stream));
}

ep_status ep_combine_backward(const ep_handle* h, uint32_t epoch, const void* grad_y,
                              const void* expert_out, int32_t hidden, void* grad_expert_out,
                              float* grad_weights, hipStream_t stream) {
    if (!h) return EP_ERR_INVALID_ARGUMENT;
    if (hidden <= 0 || hidden % 8 != 0) return EP_ERR_INVALID_ARGUMENT;
    if (hidden > kMaxHidden) return EP_ERR_UNSUPPORTED;
    if (h->T < 0 || epoch != h->epoch || h->lease) return EP_ERR_HANDLE_STATE;
    if (h->T > 0 && (!grad_y || !expert_out || !grad_expert_out || !grad_weights ||
                     !aligned16(grad_y) || !aligned16(expert_out) ||
                     !aligned16(grad_expert_out) || !aligned4(grad_weights)))
        return EP_ERR_INVALID_ARGUMENT;
    epk::CombineBwdArgs a{};
    a.grad_y = grad_y;
    a.expert_out = expert_out;
    a.T = h->T;
    a.K = h->cfg.top_k;
    a.H = hidden;
    a.slot_to_row = h->slot_to_row;
    a.weights = h->weights;
    a.grad_eo = grad_expert_out;
    a.grad_w = grad_weights;
    a.num_cu = h->num_cu;
    // launch shape from the layout's routing density, as ep_combine
    a.density = current_density(h, epk::combine_bwd_shape_uses_density(h->T, a.K, h->num_cu), stream);
    return hip_status(epk::launch_combine_bwd(a, stream));
}

ep_status ep_dispatch_backward(const ep_handle* h, uint32_t epoch, const void* grad_pool,
                               int32_t hidden, void* grad_x, hipStream_t stream) {
    if (!h) return EP_ERR_INVALID_ARGUMENT;
    if (hidden <= 0 || hidden % 8 != 0) return EP_ERR_INVALID_ARGUMENT;
    if (hidden > kMaxHidden) return EP_ERR_UNSUPPORTED;
    if (h->T < 0 || epoch != h->epoch || h->lease) return EP_ERR_HANDLE_STATE;
    if (h->T > 0 && (!grad_pool || !grad_x || !aligned16(grad_pool) || !aligned16(grad_x)))
        return EP_ERR_INVALID_ARGUMENT;
    epk::CombineArgs a{};
    a.expert_out = grad_pool;
    a.T = h->T;
    a.K = h->cfg.top_k;
    a.H = hidden;
    a.slot_to_row = h->slot_to_row;
    a.weights = nullptr;
    a.y = grad_x;
    a.num_cu = h->num_cu;
    // launch shape, as ep_combine
    a.density = current_density(h, epk::combine_shape_uses_density(h->T, hidden, h->num_cu), stream);
    return hip_status(epk::launch_combine_unit(a, stream));
}

ep_status ep_set_density_hint(ep_handle* h, int32_t hint) {
    if (!h || hint < EP_DENSITY_AUTO || hint > EP_DENSITY_DENSE) return EP_ERR_INVALID_ARGUMENT;
    h->density_hint = hint;
    return EP_OK;
}

int32_t ep_layout_density(ep_handle* h, hipStream_t stream) {
    (void)stream;
    if (!h || h->T < 0) return EP_DENSITY_AUTO;
    const int32_t d = reported_density(h);
    return d == epk::kDensitySparse ? EP_DENSITY_SPARSE
         : d == epk::kDensityDense ? EP_DENSITY_DENSE : EP_DENSITY_AUTO;
}

ep_status ep_borrow_release(ep_handle* h, hipStream_t consumer_stream) {
    if (!h) return EP_ERR_INVALID_ARGUMENT;
    if (!h->lease) return EP_ERR_HANDLE_STATE;
    if (hipEventRecord(h->lease_event, consumer_stream) != hipSuccess) return EP_ERR_HIP;
    h->lease = false;
    h->lease_wait = true;
    return EP_OK;
}

ep_status ep_handle_get_view(const ep_handle* h, ep_handle_view* out) {
    if (!h || !out) return EP_ERR_INVALID_ARGUMENT;
    out->expert_counts = h->counts;
    out->expert_pool_block_offset = h->offsets;
    out->num_tiles = h->num_tiles;
    out->tile_expert = h->tile_expert;
    out->pool_arrival_target = h->tile_target;
    out->pool_arrival_count = h->arrival;
    out->tile_ready = h->tile_ready;
    out->slot_to_pool_row = h->slot_to_row;
    out->pool_recv_token = h->recv_token;
    out->topk_weights = h->weights;
    out->y_done_per_token = h->y_done;
    return EP_OK;
}

int64_t ep_array_bytes(const ep_handle* h, ep_array which) {
    if (!h) return -1;
    const int64_t E = h->cfg.num_experts, mt = h->max_tiles;
    const int64_t slots = (int64_t)(h->T < 0 ? 0 : h->T) * h->cfg.top_k;
    switch (which) {
        case EP_ARRAY_EXPERT_COUNTS: return 4 * E;
        case EP_ARRAY_BLOCK_OFFSET: return 4 * (E + 1);
        case EP_ARRAY_NUM_TILES: return 4;
        case EP_ARRAY_TILE_EXPERT:
        case EP_ARRAY_ARRIVAL_TARGET:
        case EP_ARRAY_ARRIVAL_COUNT:
        case EP_ARRAY_TILE_READY: return 4 * mt;
        case EP_ARRAY_SLOT_TO_POOL_ROW:
        case EP_ARRAY_TOPK_WEIGHTS: return 4 * slots;
        case EP_ARRAY_POOL_RECV_TOKEN: return 4 * h->cap;
        case EP_ARRAY_Y_DONE: return 4 * (int64_t)(h->T < 0 ? 0 : h->T);
        case EP_ARRAY_TILE_STAMP: return 8 * mt;
    }
    return -1;
}

ep_status ep_copy_array(const ep_handle* h, ep_array which, void* dst, int64_t dst_bytes,
                        hipStream_t stream) {
    const int64_t n = ep_array_bytes(h, which);
    if (n < 0 || dst_bytes < n) return EP_ERR_INVALID_ARGUMENT;
    if (n == 0) return EP_OK;
    if (!dst) return EP_ERR_INVALID_ARGUMENT;
    const void* src = nullptr;
    switch (which) {
        case EP_ARRAY_EXPERT_COUNTS: src = h->counts; break;
        case EP_ARRAY_BLOCK_OFFSET: src = h->offsets; break;
        case EP_ARRAY_NUM_TILES: src = h->num_tiles; break;
        case EP_ARRAY_TILE_EXPERT: src = h->tile_expert; break;
        case EP_ARRAY_ARRIVAL_TARGET: src = h->tile_target; break;
        case EP_ARRAY_ARRIVAL_COUNT: src = h->arrival; break;
        case EP_ARRAY_TILE_READY: src = h->tile_ready; break;
        case EP_ARRAY_SLOT_TO_POOL_ROW: src = h->slot_to_row; break;
        case EP_ARRAY_POOL_RECV_TOKEN: src = h->recv_token; break;
        case EP_ARRAY_TOPK_WEIGHTS: src = h->weights; break;
        case EP_ARRAY_Y_DONE: src = h->y_done; break;
        case EP_ARRAY_TILE_STAMP: src = h->tile_stamp; break;
    }
    return hip_status(hipMemcpyAsync(dst, src, (size_t)n, hipMemcpyDeviceToDevice, stream));
}

ep_status ep_counts_to_host(ep_handle* h, int32_t* counts_host, int32_t* num_tiles_host,
                            hipStream_t stream) {
    if (!h || !counts_host || !num_tiles_host) return EP_ERR_INVALID_ARGUMENT;
    if (h->T < 0) return EP_ERR_HANDLE_STATE;
    if (hipStreamSynchronize(stream) != hipSuccess) return EP_ERR_HIP;
    if (hipMemcpy(counts_host, h->counts, sizeof(int32_t) * h->cfg.num_experts,
                  hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(num_tiles_host, h->num_tiles, sizeof(int32_t), hipMemcpyDeviceToHost) !=
            hipSuccess)
        return EP_ERR_HIP;
    return EP_OK;
}

ep_status ep_handle_sync_status(ep_handle* h, hipStream_t stream) {
    if (!h) return EP_ERR_INVALID_ARGUMENT;
    if (hipStreamSynchronize(stream) != hipSuccess) return EP_ERR_HIP;
    uint32_t word = 0;
    if (hipMemcpy(&word, h->error, sizeof word, hipMemcpyDeviceToHost) != hipSuccess)
        return EP_ERR_HIP;
    if (word) {
        const uint32_t zero = 0;
        if (hipMemcpy(h->error, &zero, sizeof zero, hipMemcpyHostToDevice) != hipSuccess)
            return EP_ERR_HIP;
    }
    if (word & 1u) return EP_ERR_BAD_ROUTING;
    if (word & 2u) return EP_ERR_TIMEOUT;
    return EP_OK;
}

ep_status ep_tile_consume(const ep_handle* h, uint32_t seq, const void* pool,
                          const void* pool_scales, int32_t hidden, uint32_t flags, void* out,
                          int32_t workgroups, uint32_t spin_limit_us, hipStream_t stream) {
    if (!h) return EP_ERR_INVALID_ARGUMENT;
    if (flags & ~(EP_DISPATCH_FP8 | EP_DISPATCH_TILE_READY | EP_CONSUME_GATHER |
                  EP_CONSUME_SIGNAL_DONE | EP_CONSUME_STAMPS | kScaleFlags))
        return EP_ERR_INVALID_ARGUMENT;
    const bool fp8 = (flags & EP_DISPATCH_FP8) != 0;
    const bool gather = (flags & EP_CONSUME_GATHER) != 0;
    if (!fp8 && (flags & kScaleFlags)) return EP_ERR_INVALID_ARGUMENT;
    if (fp8 && gather) return EP_ERR_UNSUPPORTED;
    if (hidden <= 0 || hidden % 8 != 0 ||
        (fp8 && (hidden % 128 != 0 || !pool_scales || !scales_aligned(pool_scales, flags))))
        return EP_ERR_INVALID_ARGUMENT;
    if (hidden > kMaxHidden) return EP_ERR_UNSUPPORTED;
    if (workgroups < 1 || workgroups > 65536) return EP_ERR_INVALID_ARGUMENT;
    if (h->T < 0) return EP_ERR_HANDLE_STATE;
    if (!pool || !out || !aligned16(pool) || !aligned16(out)) return EP_ERR_INVALID_ARGUMENT;
    epk::ConsumeArgs a{};
    a.pool = pool;
    a.scales = pool_scales;
    a.H = hidden;
    a.BM = h->cfg.block_m;
    a.fp8 = fp8 ? 1 : 0;
    a.gather = gather ? 1 : 0;
    a.num_tiles = h->num_tiles;
    a.recv_token = h->recv_token;
    a.tile_ready = h->tile_ready;
    a.seq = seq;
    a.limit_ticks = (uint64_t)spin_limit_us * (uint64_t)h->wall_khz / 1000u;
    a.out = out;
    a.error = h->error;
    a.y_done = (flags & EP_CONSUME_SIGNAL_DONE) ? h->y_done : nullptr;
    a.stamps = (flags & EP_CONSUME_STAMPS) ? h->tile_stamp : nullptr;
    a.scale_kind = scale_kind(flags);
    a.scale_mn = (flags & EP_SCALE_MN_MAJOR) ? 1 : 0;
    a.scale_ld = scale_ld_of(h->cap);
    return hip_status(epk::launch_consume(a, workgroups, stream));
}

}  // extern "C"
