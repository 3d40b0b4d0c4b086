/*
 * ep_layout.h -- C ABI of an MI355X (gfx950) library for one GPU's share of
 * Mixture-of-Experts expert-parallel dispatch and combine.
 *
 * The operations follow the pages this library is built from:
 *   [SEP]  StreamEP README, "Streaming dispatch in one paragraph": the
 *          expert-major, BLOCK_M-padded pool, expert_pool_block_offset (in
 *          tiles), pool_recv_token (-1 on padding rows), pool_arrival_count /
 *          pool_arrival_target per tile, and tile_ready[tile] release-stamped
 *          with the dispatch sequence number for a consumer on another stream.
 *   [ROUND] blog "DeepEP MoE dispatch/combine", section on one DeepEP round:
 *          dispatch takes x[num_tokens, hidden], topk_idx and topk_weights,
 *          counts assignments per expert, lays them out, returns tokens grouped
 *          per local expert plus a handle; combine takes the same handle and
 *          returns the weighted reduction in original token order.
 *   [HANDLE] same blog, EPHandle section: the handle carries the layout, the
 *          source mapping, per-expert counts and the top-k index/weight
 *          association; it is valid only for the routing that produced it.
 *   [CONTRACT] same blog, integration data-contract section: a per-execution
 *          epoch guards against reusing a stale handle.
 *   [WEIGHTS] same blog, router-weight section: y_t = sum_j p_{t,j} o_{t,j}.
 *   [FP8]  instagit DeepEP low-latency page, "FP8 and Quantization Support"
 *          and "API Signature and Return Values": float8_e4m3fn payload with
 *          UE8M0 scales (use_ue8m0), float32 scales otherwise, optionally
 *          rounded to a power of two (round_scale); per_token_cast_back turns
 *          the payload back into bf16 (the page's example usage).
 *   [GATE] StreamEP README, opening paragraph: a per-receive-token gate on
 *          combine (y_done_per_token) lets combine start on a token as soon
 *          as that token's expert compute has drained.
 *   [BORROW] DeepEP PR #769, "Add opt-in borrowed receive storage for compact
 *          BF16 dispatch", Description: instead of copying activations,
 *          dispatch may give an indexed consumer a view made of a slab and row
 *          indices; the view is held exclusively until the consumer streams
 *          hand it back, calls that would change it fail meanwhile, and a mode
 *          the borrow cannot serve fails before any work is queued.
 *
 * Conventions for every call:
 *   - Pointers marked "device" are device memory on the handle's GPU, 16-byte
 *     aligned; pointers marked "host" are ordinary host memory.
 *   - Calls are stream-ordered and return once work is enqueued on `stream`,
 *     except those marked BLOCKING.  A NULL stream is the device's null stream.
 *   - Argument errors are detected on the host before anything is enqueued and
 *     return EP_ERR_INVALID_ARGUMENT / EP_ERR_UNSUPPORTED / EP_ERR_HANDLE_STATE
 *     with no side effect.  Data-dependent errors seen on the device (expert ids
 *     outside [-1, num_experts), a consumer wait that timed out) set a sticky
 *     error word that ep_handle_sync_status() reports and clears.
 *   - A handle is used from one host thread and one stream at a time.  The
 *     caller keeps every buffer it passes alive until the stream work that uses
 *     it has completed.
 *   - Arrays: x, pool, expert_out and y are row-major; bf16 values are passed
 *     as their 16-bit patterns.
 *   - HIP graph capture: ep_layout, ep_dispatch, ep_combine, ep_combine_gated,
 *     the backward calls and ep_fp8_cast_back only launch kernels (nothing is
 *     allocated and no memory is set through the runtime), so they can be
 *     captured and replayed.  The host-side counters advance when a call is
 *     captured, not when it is replayed: a replay repeats the captured epoch,
 *     sequence number and streaming round.  A replayed ep_layout re-zeroes the
 *     arrival counts and the per-token done counts and re-stamps its tiles'
 *     tile_ready with the captured base (the sequence number before the
 *     captured dispatches), so a streaming dispatch and its consumer captured
 *     after the layout wait for that replay's stamps, not the last replay's.
 *     A streaming dispatch or a gated combine captured without its layout
 *     would find the last replay's stamps and counts, and its consumers could
 *     pass early: such calls return EP_ERR_UNSUPPORTED when the stream is
 *     capturing and the handle's current layout was not recorded in the same
 *     capture.  The BLOCKING calls and ep_borrow_release (which records an
 *     event) are not for capture.
 */
#ifndef EP_LAYOUT_H
#define EP_LAYOUT_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ep_status {
    EP_OK = 0,
    EP_ERR_INVALID_ARGUMENT = 1, /* bad pointer, size or flag                      */
    EP_ERR_UNSUPPORTED = 2,      /* valid request outside what the library supports */
    EP_ERR_OUT_OF_MEMORY = 3,    /* device allocation failed in ep_handle_create   */
    EP_ERR_HANDLE_STATE = 4,     /* no layout yet, or epoch does not match         */
    EP_ERR_BAD_ROUTING = 5,      /* device saw expert ids outside [-1, E)          */
    EP_ERR_TIMEOUT = 6,          /* a bounded consumer wait expired                */
    EP_ERR_HIP = 7               /* a HIP runtime call failed                      */
} ep_status;

/* Opaque; owns every metadata array of one layout ([HANDLE]). */
typedef struct ep_handle ep_handle;

/* Capacities fixed at creation ([ROUND]; the blog's buffer section: the
 * buffer is sized once from max tokens, hidden size and top-k).
 *   max_tokens  0..2^19 largest num_tokens ep_layout will accept
 *   top_k       1..32  slots per token
 *   num_experts 1..1024 experts handled by this GPU (local experts)
 *   block_m     1..4096 rows per pool tile (BLOCK_M) */
typedef struct ep_config {
    int32_t max_tokens;
    int32_t top_k;
    int32_t num_experts;
    int32_t block_m;
} ep_config;

/* ep_dispatch flags. */
#define EP_DISPATCH_FP8        (1u << 0) /* e4m3fn payload + per-128-channel scales ([FP8]) */
#define EP_DISPATCH_TILE_READY (1u << 1) /* per-tile arrival counts release tile_ready ([SEP]) */
#define EP_DISPATCH_BORROW     (1u << 2) /* no copy: lend x through the row map ([BORROW]) */

/* Scale flavour and layout of an FP8 dispatch (and of ep_fp8_cast_back).
 * Without EP_SCALE_F32 a scale is a UE8M0 byte 2^(byte-127) (use_ue8m0).
 *   EP_SCALE_F32          float32 scales s = a/448 with a = max(amax,
 *                         448*2^-126); codes are float(x * (448/a)) rounded
 *                         to nearest-even e4m3fn, saturating at 448.
 *   EP_SCALE_F32 | EP_SCALE_ROUND
 *                         float32 scales rounded to a power of two: the UE8M0
 *                         exponent e as the float 2^e, codes as for UE8M0.
 *                         (EP_SCALE_ROUND alone changes nothing: UE8M0 scales
 *                         are powers of two already.)
 *   EP_SCALE_MN_MAJOR     group g of pool row r at [g, r] with leading
 *                         dimension ep_scale_ld(); UE8M0 bytes are then packed
 *                         four groups to a uint32 word, group 4w+j in byte j of
 *                         word w (bytes past the last group are 0), an array
 *                         uint32 [ceil(G/4), ld].  Without it scales are
 *                         row-major [capacity_rows, G], G = hidden/128.
 * The flavour names and the per-128-channel grouping follow [FP8]; the page
 * gives no formulas, the ones above are this library's reading. */
#define EP_SCALE_F32           (1u << 4)
#define EP_SCALE_ROUND         (1u << 5)
#define EP_SCALE_MN_MAJOR      (1u << 6)

/* ep_tile_consume flags: EP_CONSUME_GATHER reads rows from a borrowed slab
 * through pool_recv_token instead of from a pool ([BORROW]);
 * EP_CONSUME_SIGNAL_DONE makes the consumer act as the expert-output
 * producer of the per-token gate ([GATE]): after writing a tile it publishes
 * the rows at device scope and adds 1 to y_done_per_token[pool_recv_token[r]]
 * for each real row r of the tile. */
#define EP_CONSUME_GATHER      (1u << 3)
#define EP_CONSUME_SIGNAL_DONE (1u << 7)
/* EP_CONSUME_STAMPS: the consumer records, for each tile it takes, the
 * device's constant-rate wall clock (hipDeviceAttributeWallClockRate) at the
 * moment it saw tile_ready reach seq, with bit 63 set when its first look
 * found the tile not yet ready (the dispatch was still landing rows), in the
 * handle's array EP_ARRAY_TILE_STAMP (uint64 [max_tiles]; a tile that timed
 * out keeps its old stamp).  Evidence that, and in which order, tiles were
 * released while the dispatch ran. */
#define EP_CONSUME_STAMPS      (1u << 8)

/* Allocate a handle and all its device metadata on the current device.
 * Returns EP_ERR_INVALID_ARGUMENT for out-of-range fields or when the pool
 * capacity does not fit int32 rows; EP_ERR_OUT_OF_MEMORY when allocation
 * fails.  *out receives the handle (host pointer, owned by the library). */
ep_status ep_handle_create(const ep_config* cfg, ep_handle** out);

/* Free the handle (synchronises the device first).  NULL is a no-op. */
ep_status ep_handle_destroy(ep_handle* h);

/* Worst-case pool rows: max_tokens * top_k + num_experts * (block_m - 1).
 * Every pool / expert_out buffer must have at least this many rows. */
int64_t ep_pool_capacity_rows(const ep_handle* h);

/* Tile slots: ep_pool_capacity_rows(h) / block_m (never fewer than needed). */
int32_t ep_max_tiles(const ep_handle* h);

/* Tokens of the current layout, or -1 when there is none. */
int32_t ep_num_tokens(const ep_handle* h);

/* Leading dimension of MN-major scales: capacity_rows rounded up to a
 * multiple of 4 (16-byte aligned columns). */
int64_t ep_scale_ld(const ep_handle* h);

/* Build the expert-major layout of one routing ([SEP], [ROUND]).
 *   topk_idx      device int32 [num_tokens, top_k]; -1 marks a masked slot.
 *   topk_weights  device fp32  [num_tokens, top_k]; copied into the handle.
 *   num_tokens    0..max_tokens.
 *   epoch_out     host; receives the new epoch that ep_combine must quote.
 * Device results (read them with ep_handle_get_view / ep_copy_array):
 *   expert_counts[e]             rows of expert e
 *   expert_pool_block_offset[e]  first tile of expert e (E+1 entries, last = num_tiles)
 *   tile_expert[j], pool_arrival_target[j]  expert and real rows of tile j
 *                                           (-1 and 0 for j >= num_tiles)
 *   slot_to_pool_row[t*K+k]      pool row of slot (t,k), -1 if masked
 *   pool_recv_token[r]           source token of pool row r, -1 for padding
 * Rows of one expert are in ascending slot order t*K+k.  pool_arrival_count is
 * zeroed for the layout's tiles and y_done_per_token for its tokens, and the
 * layout's tiles get tile_ready = the sequence number of the handle's last
 * dispatch (0 before the first), so no tile reads as ready for a dispatch
 * that comes after the layout.  Ids outside [-1, E) are treated as masked and
 * set EP_ERR_BAD_ROUTING in the error word.  Invalidates earlier epochs. */
ep_status ep_layout(ep_handle* h, const int32_t* topk_idx, const float* topk_weights,
                    int32_t num_tokens, hipStream_t stream, uint32_t* epoch_out);

/* Copy activations into the pool of the current layout ([SEP], [ROUND]).
 *   x            device bf16 [num_tokens, hidden], hidden % 8 == 0.
 *   pool         device; bf16 [capacity_rows, hidden], or with EP_DISPATCH_FP8
 *                e4m3fn bytes [capacity_rows, hidden] (hidden % 128 == 0).
 *   pool_scales  device, with EP_DISPATCH_FP8 only (else must be NULL): the
 *                scales in the flavour and layout the EP_SCALE_* flags choose
 *                (default u8 [capacity_rows, hidden/128] UE8M0 bytes, scale =
 *                2^(byte-127)); 4-byte aligned for float32 or MN-major scales.
 *   flags        EP_DISPATCH_FP8 | EP_DISPATCH_TILE_READY | EP_SCALE_*
 *                (EP_SCALE_* only with EP_DISPATCH_FP8).
 *   seq_out      host, may be NULL; receives this dispatch's sequence number
 *                (1, 2, ... per handle, wraps; compare wrap-safe).
 * Only real rows are written (scales too); padding rows and rows past the
 * layout keep their contents.  FP8 with UE8M0 scales: per token and
 * 128-channel group, e = smallest integer in [-127,127] with amax <= 448*2^e
 * (NaN takes no part in amax); codes are x*2^-e rounded to nearest-even
 * e4m3fn.  With EP_DISPATCH_TILE_READY each tile's arrival count is raised as
 * its rows land and the dispatch that completes the tile release-stores the
 * sequence number into tile_ready[tile] (device scope), so a consumer on
 * another stream may acquire-load it and read the tile's rows.
 * Launch shape: a bf16 dispatch without EP_DISPATCH_TILE_READY, with top_k up
 * to 8 and at least 64 MiB of x, takes its shape from the current layout's
 * routing density as ep_combine does (and may wait for the layout kernel's
 * report on the host in the same way).  For dense routing that shape is two
 * launches on `stream`: a read pass over x, then the pool stores.  The pool
 * is the same in every shape. */
ep_status ep_dispatch(ep_handle* h, const void* x, int32_t hidden, void* pool,
                      void* pool_scales, uint32_t flags, hipStream_t stream,
                      uint32_t* seq_out);
/* EP_DISPATCH_BORROW ([BORROW]): nothing is copied or launched.  The rows are
 * lent as the view (slab = x, row indices = pool_recv_token of the current
 * layout): pool row r is row pool_recv_token[r] of x, -1 for padding.  Only a
 * bf16 dispatch with pool == NULL and pool_scales == NULL may borrow;
 * EP_DISPATCH_FP8 or EP_DISPATCH_TILE_READY with it is EP_ERR_UNSUPPORTED.
 * The handle then holds an exclusive lease: ep_layout, ep_dispatch,
 * ep_combine and ep_handle_destroy return EP_ERR_HANDLE_STATE until
 * ep_borrow_release.  The caller keeps x alive and unchanged meanwhile. */

/* ep_layout followed by ep_dispatch in one call, for batches small enough
 * that launch latency dominates (instagit DeepEP low-latency page,
 * "Low-Latency Dispatch Kernel" and "API Signature and Return Values": the
 * decoding dispatch takes x and topk_idx together and returns the per-expert
 * rows, their counts and the handle).  Arguments as for the two calls (x must have
 * num_tokens rows); EP_DISPATCH_BORROW is EP_ERR_UNSUPPORTED.  For at most
 * 2048 slots (num_tokens * top_k) and without EP_DISPATCH_TILE_READY the two
 * run as one kernel launch: one workgroup writes the layout while every other
 * workgroup builds the slot -> pool row map by itself from topk_idx and
 * dispatches its share; otherwise this calls ep_layout and then ep_dispatch.
 * The device results, the epoch (epoch_out) and the sequence number (seq_out,
 * may be NULL) are those of the two calls.  Every argument is checked before
 * anything is enqueued. */
ep_status ep_layout_dispatch(ep_handle* h, const int32_t* topk_idx, const float* topk_weights,
                             int32_t num_tokens, const void* x, int32_t hidden, void* pool,
                             void* pool_scales, uint32_t flags, hipStream_t stream,
                             uint32_t* epoch_out, uint32_t* seq_out);

/* Weighted sum back in original token order ([WEIGHTS], [ROUND]).
 *   epoch       the value ep_layout returned; else EP_ERR_HANDLE_STATE.
 *   expert_out  device bf16 [capacity_rows, hidden]; only real rows are read.
 *   y           device bf16 [num_tokens, hidden], fully written.
 * y[t,c] = bf16_rne( fp32 fma chain over k ascending of w[t,k] * o[row(t,k),c] )
 * starting from +0 and skipping masked slots; a token with no slot gets +0.
 * Launch shape: the layout kernel reports whether its routing averages 4 or
 * more real rows per token, tagged with its epoch, into a word of pinned host
 * memory that the handle owns; for batches too large to be resident at once
 * this call (and ep_dispatch_backward) runs fewer waves per compute unit for
 * dense routing.  It uses the current layout's word, and when the layout
 * kernel has not stored it yet the call waits for that store on the host (for
 * the layout kernel only, at most 200 ms; past that, or while the stream is
 * being captured into a HIP graph, it takes the dense shape).  So the shape
 * follows the routing, not the timing; y is the same in every shape. */
ep_status ep_combine(const ep_handle* h, uint32_t epoch, const void* expert_out,
                     int32_t hidden, void* y, hipStream_t stream);

/* ep_combine behind the per-token gate ([GATE]).  Before combining token t
 * the kernel waits (acquire, device scope) until y_done_per_token[t] has
 * reached round * n_t, n_t = unmasked slots of t (tokens with none do not
 * wait); the comparison is wrap-safe.  The producers of expert_out (on other
 * streams) make each row visible at device scope and then add 1 to the count
 * of that row's token, e.g. ep_tile_consume with EP_CONSUME_SIGNAL_DONE.
 *   round          >= 1: producer passes since ep_layout this call waits for.
 *   spin_limit_us  bound on one token's wait; past it, or once any wait of
 *                  this handle has timed out (in this call or an earlier one,
 *                  until ep_handle_sync_status clears the error word), the
 *                  remaining waiting tokens are skipped (their y rows are left
 *                  as they were) and EP_ERR_TIMEOUT is set in the error word.
 * Everything else as ep_combine: the result equals ep_combine's bit for bit. */
ep_status ep_combine_gated(const ep_handle* h, uint32_t epoch, const void* expert_out,
                           int32_t hidden, void* y, uint32_t round, uint32_t spin_limit_us,
                           hipStream_t stream);

/* Launch-shape hint of ep_combine, ep_dispatch_backward, ep_combine_backward
 * and the bf16 ep_dispatch.  EP_DENSITY_AUTO (the default) takes the current
 * layout's reported density as described at ep_combine (waiting for it if
 * needed; the dense shape under graph capture).  EP_DENSITY_SPARSE or EP_DENSITY_DENSE fix
 * the shape for the handle's later calls, which then never wait: for callers
 * that capture these calls in a HIP graph, that enqueue far ahead of the GPU
 * (whose calls would otherwise wait for the layout kernel to run), or that
 * know their routing.  Results never depend on the shape. */
#define EP_DENSITY_AUTO   0
#define EP_DENSITY_SPARSE 1     /* fewer than 4 real rows per token on average */
#define EP_DENSITY_DENSE  2     /* 4 or more */
ep_status ep_set_density_hint(ep_handle* h, int32_t hint);

/* BLOCKING (on the layout kernel only, as ep_combine waits): the density the
 * current layout reported, EP_DENSITY_SPARSE or EP_DENSITY_DENSE;
 * EP_DENSITY_AUTO when the handle has no layout or the report did not arrive
 * within 200 ms. */
int32_t ep_layout_density(ep_handle* h, hipStream_t stream);

/* per_token_cast_back ([FP8], example usage): bf16 rows from e4m3fn codes and
 * their scales, in any flavour and layout of the FP8 dispatch.
 *   q          device e4m3fn bytes [rows, hidden], hidden % 128 == 0.
 *   scales     device; layout and type as EP_SCALE_* in `flags` say, with row
 *              index r in [0, rows) (MN-major: column r of leading dimension
 *              scale_ld >= rows; ignored otherwise).
 *   out        device bf16 [rows, hidden], fully written.
 * out[r,c] = bf16_rne(value(q[r,c]) * s(r, c/128)): UE8M0 scales multiply
 * exactly; float32 scales give one float product first.  NaN codes (0x7F,
 * 0xFF), and NaN products, give a quiet NaN with the code's sign.  Needs no
 * handle. */
ep_status ep_fp8_cast_back(const void* q, const void* scales, uint32_t flags, int64_t rows,
                           int64_t scale_ld, int32_t hidden, void* out, hipStream_t stream);

/* Backward of ep_combine ([SEP] "What's in the box" names combine_grads; the
 * values are the derivatives of [WEIGHTS]'s y_t = sum_k w_{t,k} o_{row(t,k)}).
 *   epoch            the layout's epoch, else EP_ERR_HANDLE_STATE.
 *   grad_y           device bf16 [num_tokens, hidden].
 *   expert_out       device bf16 [capacity_rows, hidden] (combine's input).
 *   grad_expert_out  device bf16 [capacity_rows, hidden]: row(t,k) gets
 *                    bf16(fp32(w[t,k] * grad_y[t])); other rows untouched.
 *   grad_weights     device fp32 [num_tokens, top_k]: the dot product
 *                    <grad_y[t], expert_out[row(t,k)]> accumulated in double
 *                    (bf16 x bf16 products are exact) and rounded once to
 *                    float; 0 for masked slots.
 * hidden % 8 == 0.  Rejected while a borrowed view is out.  For top_k 5..8
 * on batches too large to be resident at once the launch shape follows the
 * layout's reported routing density exactly as at ep_combine (same wait, same
 * hint); the results are the same in every shape. */
ep_status ep_combine_backward(const ep_handle* h, uint32_t epoch, const void* grad_y,
                              const void* expert_out, int32_t hidden, void* grad_expert_out,
                              float* grad_weights, hipStream_t stream);

/* Backward of a bf16 ep_dispatch ([SEP] names dispatch_grads): each pool row
 * was a copy of its token's row, so
 *   grad_x[t] = bf16( fp32 sum over unmasked k ascending of grad_pool[row(t,k)] )
 * from +0 (a token with no unmasked slot gets +0); padding rows of grad_pool
 * are never read.  grad_pool device bf16 [capacity_rows, hidden], grad_x
 * device bf16 [num_tokens, hidden]; hidden % 8 == 0. */
ep_status ep_dispatch_backward(const ep_handle* h, uint32_t epoch, const void* grad_pool,
                               int32_t hidden, void* grad_x, hipStream_t stream);

/* End the lease of a borrowing dispatch ([BORROW]).  consumer_stream is the
 * stream the consumers of the view were enqueued on; the handle's next call
 * waits (on its own stream) until that stream's work enqueued so far is done,
 * so a new layout never overwrites the row indices under a delayed reader.
 * Returns EP_ERR_HANDLE_STATE when no lease is held. */
ep_status ep_borrow_release(ep_handle* h, hipStream_t consumer_stream);

/* Device pointers into the handle's metadata; valid until the next ep_layout
 * or ep_handle_destroy.  Lengths: counts E, offsets E+1, tile arrays
 * max_tiles, pool_recv_token capacity_rows, slot arrays num_tokens*top_k,
 * y_done_per_token num_tokens. */
typedef struct ep_handle_view {
    const int32_t* expert_counts;
    const int32_t* expert_pool_block_offset;
    const int32_t* num_tiles;
    const int32_t* tile_expert;
    const int32_t* pool_arrival_target;
    const uint32_t* pool_arrival_count;
    const uint32_t* tile_ready;
    const int32_t* slot_to_pool_row;
    const int32_t* pool_recv_token;
    const float* topk_weights;
    uint32_t* y_done_per_token;     /* [num_tokens], written by expert-output producers */
} ep_handle_view;

ep_status ep_handle_get_view(const ep_handle* h, ep_handle_view* out);

/* Which metadata array ep_copy_array copies. */
typedef enum ep_array {
    EP_ARRAY_EXPERT_COUNTS = 0,
    EP_ARRAY_BLOCK_OFFSET = 1,
    EP_ARRAY_NUM_TILES = 2,
    EP_ARRAY_TILE_EXPERT = 3,
    EP_ARRAY_ARRIVAL_TARGET = 4,
    EP_ARRAY_ARRIVAL_COUNT = 5,
    EP_ARRAY_TILE_READY = 6,
    EP_ARRAY_SLOT_TO_POOL_ROW = 7,
    EP_ARRAY_POOL_RECV_TOKEN = 8,
    EP_ARRAY_TOPK_WEIGHTS = 9,
    EP_ARRAY_Y_DONE = 10,
    EP_ARRAY_TILE_STAMP = 11        /* uint64 [max_tiles], see EP_CONSUME_STAMPS */
} ep_array;

/* Byte size of a metadata array for the current layout. */
int64_t ep_array_bytes(const ep_handle* h, ep_array which);

/* Stream-ordered device-to-device copy of one metadata array into dst
 * (device, dst_bytes >= ep_array_bytes). */
ep_status ep_copy_array(const ep_handle* h, ep_array which, void* dst, int64_t dst_bytes,
                        hipStream_t stream);

/* BLOCKING: copy expert_counts (E ints) and num_tiles into host memory
 * ("CPU counts" in DeepEP PR #769's wording). */
ep_status ep_counts_to_host(ep_handle* h, int32_t* counts_host, int32_t* num_tiles_host,
                            hipStream_t stream);

/* BLOCKING: wait for `stream`, read and clear the device error word.
 * Returns EP_ERR_BAD_ROUTING, EP_ERR_TIMEOUT or EP_OK. */
ep_status ep_handle_sync_status(ep_handle* h, hipStream_t stream);

/* Stand-in for the consumer of the streaming release ([SEP]: a consumer
 * kernel spins on an acquire-load of tile_ready[tile] >= dispatch_seq from a
 * different stream).  A bounded grid of `workgroups` (1..65536) walks tiles in order,
 * waits until tile_ready[tile] has reached `seq` (wrap-safe), then writes
 * every real row of the tile to `out` (device bf16 [capacity_rows, hidden]):
 * a copy of a bf16 pool, or with EP_DISPATCH_FP8 the dequantised value, as
 * ep_fp8_cast_back computes it, with the scales in the flavour and layout the
 * EP_SCALE_* flags name (as for the dispatch).  With EP_CONSUME_GATHER, `pool` is a
 * borrowed bf16 slab [num_tokens, hidden] and row r is read from slab row
 * pool_recv_token[r] (the indexed consumer of [BORROW]).  A wait longer than spin_limit_us gives up
 * on that tile and sets EP_ERR_TIMEOUT in the error word, so it always ends.
 * The caller orders it after ep_layout (e.g. with an event).  flags:
 * EP_DISPATCH_FP8 with any EP_SCALE_* flags, EP_CONSUME_GATHER (bf16 only),
 * EP_CONSUME_SIGNAL_DONE, EP_CONSUME_STAMPS. */
ep_status ep_tile_consume(const ep_handle* h, uint32_t seq, const void* pool,
                          const void* pool_scales, int32_t hidden, uint32_t flags,
                          void* out, int32_t workgroups, uint32_t spin_limit_us,
                          hipStream_t stream);

/* ep_layout without a handle and without any allocation, for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops
 * that forbid hipMalloc).  The routing metadata of ep_layout goes into arrays
 * the caller owns; the workspace of the multi-workgroup layout (one int32 per
 * workgroup of 2048 slots and expert) is a fixed 1 MiB device array of the
 * library, one per GPU, held until the process ends.
 *   topk_idx          device int32 [num_tokens, top_k]; -1 marks a masked slot.
 *   num_tokens 0..2^19, top_k 1..32, num_experts 1..1024, block_m 1..4096.
 *   capacity_rows     >= num_tokens*top_k + num_experts*(block_m-1), and
 *                     below 2^30; max_tiles = capacity_rows / block_m.
 *   outputs (device, caller-owned, 4-byte aligned), as ep_layout's arrays:
 *     expert_counts [E], expert_pool_block_offset [E+1], num_tiles [1],
 *     tile_expert [max_tiles], pool_arrival_target [max_tiles],
 *     slot_to_pool_row [num_tokens*top_k], pool_recv_token [capacity_rows].
 *   error_word        device uint32 or NULL: bit 0 is set (never cleared) when
 *                     an id outside [-1, num_experts) was seen; such slots are
 *                     treated as masked.
 * Returns EP_ERR_UNSUPPORTED when the workspace would exceed the fixed array
 * (ceil(num_tokens*top_k/2048) * num_experts > 262144 int32, e.g. more than
 * 524288 slots at 1024 experts), EP_ERR_INVALID_ARGUMENT for bad sizes or
 * pointers; nothing is enqueued then.  Calls that overlap on one GPU (on
 * different streams, or from different threads) share the array and race;
 * calls in stream order do not.  Nothing here touches a handle: no weights
 * copy, arrival counts, tile_ready stamps or done counts. */
ep_status ep_layout_noalloc(const int32_t* topk_idx, int32_t num_tokens, int32_t top_k,
                            int32_t num_experts, int32_t block_m, int64_t capacity_rows,
                            int32_t* expert_counts, int32_t* expert_pool_block_offset,
                            int32_t* num_tiles, int32_t* tile_expert,
                            int32_t* pool_arrival_target, int32_t* slot_to_pool_row,
                            int32_t* pool_recv_token, uint32_t* error_word,
                            hipStream_t stream);

/* Static description of a status code. */
const char* ep_status_string(ep_status s);

#ifdef __cplusplus
}
#endif

#endif /* EP_LAYOUT_H */
