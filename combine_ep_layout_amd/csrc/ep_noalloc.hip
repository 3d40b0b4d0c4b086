// ep_layout_noalloc: the layout of one routing into arrays the caller owns,
// for callers that cannot allocate device memory (code under HIP graph
// capture, serving loops that forbid it).  It runs the same kernels as
// ep_layout; the per-workgroup expert histograms that ep_layout keeps in its
// handle live here in `scratch`, a fixed device array of this library.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <mutex>

#include "ep_layout.h"
#include "ep_internal.h"

namespace {

// Workspace of the multi-workgroup layout: one int32 count per (workgroup,
// expert), ceil(num_tokens * top_k / 2048) workgroups.  1 MiB per GPU, held
// until the process ends.  Every workgroup writes its whole row before any
// workgroup reads it, so nothing needs clearing between calls.
constexpr int64_t kScratchInts = int64_t(1) << 18;
static __device__ __align__(256) int32_t scratch[kScratchInts];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
int32_t* g_scratch[kMaxDevices] = {};   // device address of `scratch`, per device

// The device address of this GPU's copy of `scratch`, looked up once per
// device with that device current.  In host code the array's name is only a
// stand-in, never a device address.
ep_status scratch_of_current_device(int32_t** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return EP_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return EP_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return EP_ERR_HIP;
        }
        g_scratch[dev] = (int32_t*)p;
    }
    *out = g_scratch[dev];
    return EP_OK;
}

bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

}  // namespace

extern "C" ep_status ep_layout_noalloc(const int32_t* topk_idx, int32_t num_tokens, int32_t top_k,
                                       int32_t num_experts, int32_t block_m, int64_t capacity_rows,
                                       int32_t* expert_counts, int32_t* expert_pool_block_offset,
                                       int32_t* num_tiles, int32_t* tile_expert,
                                       int32_t* pool_arrival_target, int32_t* slot_to_pool_row,
                                       int32_t* pool_recv_token, uint32_t* error_word,
                                       hipStream_t stream) {
    if (num_tokens < 0 || num_tokens > (1 << 19) || top_k < 1 || top_k > 32 || num_experts < 1 ||
        num_experts > 1024 || block_m < 1 || block_m > 4096)
        return EP_ERR_INVALID_ARGUMENT;
    const int64_t slots = (int64_t)num_tokens * top_k;
    if (capacity_rows < slots + (int64_t)num_experts * (block_m - 1) || capacity_rows > INT32_MAX / 2)
        return EP_ERR_INVALID_ARGUMENT;
    const int64_t nb = slots > epk::kLayoutSlotsPerBlock ? epk::layout_blocks(slots) : 0;
    if (nb * num_experts > kScratchInts) return EP_ERR_UNSUPPORTED;
    const void* out[] = {expert_counts, expert_pool_block_offset, num_tiles, tile_expert,
                         pool_arrival_target, pool_recv_token};
    for (const void* p : out)
        if (!p || !aligned4(p)) return EP_ERR_INVALID_ARGUMENT;
    if (slots > 0 && (!topk_idx || !slot_to_pool_row || !aligned4(topk_idx) ||
                      !aligned4(slot_to_pool_row)))
        return EP_ERR_INVALID_ARGUMENT;
    if (error_word && !aligned4(error_word)) return EP_ERR_INVALID_ARGUMENT;
    int32_t* ws = nullptr;
    ep_status st = scratch_of_current_device(&ws);
    if (st != EP_OK) return st;
    epk::LayoutArgs a{};
    a.topk_idx = topk_idx;
    a.S = (int32_t)slots;
    a.K = top_k;
    a.E = num_experts;
    a.BM = block_m;
    a.cap = (int32_t)capacity_rows;
    a.max_tiles = (int32_t)(capacity_rows / block_m);
    a.counts = expert_counts;
    a.offsets = expert_pool_block_offset;
    a.num_tiles = num_tiles;
    a.tile_expert = tile_expert;
    a.tile_target = pool_arrival_target;
    a.slot_to_row = slot_to_pool_row;
    a.recv_token = pool_recv_token;
    a.error = error_word;
    a.ws = ws;
    // no weights copy, arrival counts, tile stamps, done counts or density
    // report: those belong to a handle
    return epk::launch_layout(a, stream) == hipSuccess ? EP_OK : EP_ERR_HIP;
}
