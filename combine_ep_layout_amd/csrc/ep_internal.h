// Internal interface between the C ABI (ep_api.hip) and the gfx950 kernels
// (ep_kernels.hip).  Not installed; callers use include/ep_layout.h.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

namespace epk {

// Slots ranked by one layout workgroup (1024 threads x 2 slots per lane).
// Up to this many slots the whole layout runs in a single workgroup and launch.
constexpr int kLayoutSlotsPerBlock = 1024 * 2;

// Layout arguments.  topk_w / weights, arrival / tile_ready, y_done, error
// and density may be null (a layout into caller-owned arrays has none of
// them); the other arrays are required.
struct LayoutArgs {
    const int32_t* topk_idx;    // [S]
    const float* topk_w;        // [S]
    int32_t S;                  // num_tokens * top_k
    int32_t K;
    int32_t E;
    int32_t BM;
    int32_t cap;                // pool capacity rows
    int32_t max_tiles;
    int32_t* counts;            // [E]
    int32_t* offsets;           // [E+1]
    int32_t* num_tiles;         // [1]
    int32_t* tile_expert;       // [max_tiles]
    int32_t* tile_target;       // [max_tiles]
    uint32_t* arrival;          // [max_tiles]
    uint32_t* tile_ready;       // [max_tiles], used tiles set to seq_base
    uint32_t seq_base;          // sequence number of the handle's last dispatch
    int32_t* slot_to_row;       // [S]
    int32_t* recv_token;        // [cap]
    float* weights;             // [S]
    uint32_t* error;            // [1]
    int32_t* ws;                // [blocks * E] per-workgroup expert counts
    uint32_t* y_done;           // [T] per-token done counts, zeroed here
    uint64_t* density;          // host-mapped word: epoch << 32 | Density (may be null)
    uint32_t epoch;             // the epoch this layout starts
};

// Routing density of a layout, as the layout reports it for the launch shapes
// of the bf16 dispatch and the combine that follow it (results never depend
// on it).
enum Density : int32_t {
    kDensityUnknown = 0,        // no layout reported yet
    kDensitySparse = 1,         // fewer than 4 real rows per token on average
    kDensityDense = 2,          // 4 or more
};

// Scale flavours of the FP8 dispatch and the cast back.
enum ScaleKind : int32_t {
    kScaleUe8m0 = 0,            // UE8M0 exponent byte
    kScaleF32 = 1,              // float32 amax / 448
    kScalePow2F32 = 2,          // float32 2^e (the UE8M0 exponent as a float)
};

struct DispatchArgs {
    const void* x;
    int32_t T;
    int32_t K;
    int32_t H;
    int32_t BM;
    int32_t E;
    const int32_t* slot_to_row;
    const int32_t* tile_expert;
    const int32_t* tile_target;
    void* pool;
    void* scales;
    int32_t scale_kind;         // ScaleKind
    int32_t scale_mn;           // 1: MN-major [G, scale_ld] (UE8M0 packed 4 per word)
    int64_t scale_ld;
    // streaming release
    int32_t max_tiles;
    uint32_t* arrival;
    uint32_t* tile_ready;
    uint32_t seq;
    uint32_t round;             // TILE_READY dispatches since the layout (1, 2, ...)
    int32_t density;            // Density of the current layout (launch shape of the bf16 dispatch)
};

struct CombineArgs {
    const void* expert_out;
    int32_t T;
    int32_t K;
    int32_t H;
    const int32_t* slot_to_row;
    const float* weights;
    void* y;
    // per-token gate (ep_combine_gated): wait for y_done[t] >= round * slots(t)
    const uint32_t* y_done;
    uint32_t round;
    uint64_t limit_ticks;
    uint32_t* error;
    int32_t num_cu;             // compute units of the device (launch shapes)
    int32_t density;            // Density of the current layout (launch shape of the plain combine)
};

struct CombineBwdArgs {
    const void* grad_y;         // bf16 [T, H]
    const void* expert_out;     // bf16 [cap, H]
    int32_t T;
    int32_t K;
    int32_t H;
    const int32_t* slot_to_row;
    const float* weights;
    void* grad_eo;              // bf16 [cap, H], real rows written
    float* grad_w;              // fp32 [T, K]
    int32_t density;            // Density of the layout: the launch shape
    int32_t num_cu;
};

struct ConsumeArgs {
    const void* pool;
    const void* scales;
    int32_t H;
    int32_t BM;
    int32_t fp8;
    int32_t gather;             // rows come from slab row recv_token[r]
    const int32_t* num_tiles;
    const int32_t* recv_token;
    const uint32_t* tile_ready;
    uint32_t seq;
    uint64_t limit_ticks;
    void* out;
    uint32_t* error;
    uint32_t* y_done;           // non-null: count each written row for its token
    uint64_t* stamps;           // non-null: per tile, acquire clock | waited << 63
    int32_t scale_kind;         // FP8 scales: ScaleKind, layout and leading dimension
    int32_t scale_mn;
    int64_t scale_ld;
};

struct CastBackArgs {
    const void* q;              // e4m3fn [rows, H]
    const void* scales;
    int32_t scale_kind;
    int32_t scale_mn;
    int64_t scale_ld;
    int64_t rows;
    int32_t H;
    void* out;                  // bf16 [rows, H]
};

hipError_t launch_layout(const LayoutArgs& a, hipStream_t stream);
// The one-workgroup layout and the dispatch of its tokens in one launch
// (la.S <= kLayoutSlotsPerBlock, T > 0, no streaming release): the same
// results as launch_layout followed by launch_dispatch.
hipError_t launch_layout_dispatch(const LayoutArgs& la, const DispatchArgs& a, bool fp8, hipStream_t stream);
hipError_t launch_dispatch(const DispatchArgs& a, bool fp8, bool tile_ready, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);
hipError_t launch_combine_gated(const CombineArgs& a, hipStream_t stream);
hipError_t launch_cast_back(const CastBackArgs& a, hipStream_t stream);
// unit_weights: every unmasked slot weighs 1 (the backward of dispatch)
hipError_t launch_combine_unit(const CombineArgs& a, hipStream_t stream);
hipError_t launch_combine_bwd(const CombineBwdArgs& a, hipStream_t stream);
hipError_t launch_consume(const ConsumeArgs& a, int workgroups, hipStream_t stream);
// Whether the plain combine's (and the dispatch backward's) launch shape for
// these sizes depends on the routing density (it does not for grids that are
// resident at once, nor when there are no tokens).
bool combine_shape_uses_density(int T, int H, int num_cu);
// Whether the launch shape of the bf16 dispatch without the streaming release
// depends on the routing density for these sizes (top_k up to 8 and at least
// 64 MiB of x).
bool dispatch_shape_uses_density(int T, int H, int K);
// Whether the combine backward's launch shape depends on the routing density
// (top_k from 5 to 8, on grids that are not resident at once).
bool combine_bwd_shape_uses_density(int T, int K, int num_cu);

// Workgroups the multi-workgroup layout path needs for S slots.
inline int layout_blocks(int64_t S) {
    int64_t nb = (S + kLayoutSlotsPerBlock - 1) / kLayoutSlotsPerBlock;
    return nb < 1 ? 1 : (int)nb;
}

}  // namespace epk
