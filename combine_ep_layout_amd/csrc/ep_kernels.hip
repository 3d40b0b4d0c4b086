// gfx950 kernels for one GPU's share of MoE expert-parallel dispatch/combine.
//
// Layout (StreamEP README, "Streaming dispatch in one paragraph"; blog
// "DeepEP MoE dispatch/combine", one DeepEP round): a per-expert histogram,
// an exclusive scan of BLOCK_M-padded tile counts into
// expert_pool_block_offset, per-tile arrival targets, and a stable rank of
// every (token, k) slot inside its expert.  Stable ranks come from wave64
// match-any masks built out of one ballot per key bit, so a slot's row
// depends only on how many earlier slots share its expert, never on timing.
// The layout is latency-bound (a few hundred KB), so every workgroup issues
// all of its loads before it waits on any of them, and the cross-workgroup
// scan is recomputed redundantly by each workgroup instead of being
// serialised through one of them.
//
// Dispatch is token-major: a wave reads one segment of a token's row of x
// once and writes it, as 16-byte vectors, to each of the token's pool rows
// (bf16), or quantises it once to e4m3fn with a scale per 128 channels and
// writes the codes (FP8; instagit DeepEP low-latency page, "FP8 and
// Quantization Support").  UE8M0 codes come from gfx950's scaled conversion
// instruction wherever it equals the exact integer encoder, which is kept for
// the rest.  With the streaming release, each workgroup takes one token, in
// token order, with one wave per row segment; it stores the rows with
// device-scope stores, and the last of its waves to see its own stores
// complete raises the arrival count of every tile the token wrote; the add
// that completes a tile stores the sequence number into tile_ready[tile].
//
// Combine is token-major too: a wave gathers one segment of the token's k
// expert rows, accumulates w * o in fp32 with one fused multiply-add per slot
// in slot order, and rounds once to bf16 (blog, router-weight section).  The
// gated variant waits per token on y_done_per_token (StreamEP README,
// opening paragraph).  The backward kernels, the FP8 cast back and the
// consumer stand-in (tests and benchmarks) follow.
//
// Nothing here is a dense contraction, so no matrix-core instructions are
// used; dispatch and combine are HBM-bound streaming kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <limits.h>

#include "ep_internal.h"

namespace epk {
namespace {

// Work shapes, each chosen by timing the alternatives on MI355X: 16-byte
// chunks or 16-channel units each lane handles per work item, and the
// streaming dispatch's chunk.
constexpr int kDispatchChunks = 2;      // bf16 dispatch: 16-byte chunks per lane per item
constexpr int kFp8Units = 1;            // FP8 dispatch: 16-channel units per lane per item
constexpr int kFp8StreamUnits = 1;      // the same with the streaming release
constexpr int kCombineChunks = 2;       // combine: 16-byte chunks per lane per item
constexpr int64_t kDenseDispatchMinBytes = int64_t(64) << 20;  // bf16 dispatch: dense-routing shape from this size of x
constexpr int kStreamTokens = 1;        // streaming dispatch: tokens per chunk (one workgroup, a wave per segment)
constexpr int kStageGrid = 8192;        // read pass over x before the dense-routing dispatch: workgroups
constexpr int kCombineResidentWaves = 8;   // combine grids up to this many waves per CU: full occupancy
constexpr int kCombineDenseLds = 55296;    // unused LDS per combine workgroup for dense routing: 2 per CU
constexpr int kBwdChunks = 2;           // combine backward: 16-byte chunks per lane in flight
constexpr int kBwdDenseLds = 55296;     // unused LDS per combine-backward workgroup for dense routing: 2 per CU
constexpr int kCastUnits = 2;           // cast back: 16-channel units per lane per item
constexpr int kGateTokens = 16;         // gated combine: most tokens per workgroup (<= 64)
constexpr int kGateWaves = 16;          // gated combine: most waves per workgroup
constexpr int kGateDefer = 4;           // gated combine: dense items computed before their stores

// Cache policy bits of buffer loads and stores on gfx950.
constexpr int kAuxNonTemporal = 2;      // nt: streaming, not kept in the caches
constexpr int kAuxDevice = 16;          // sc1: device scope (write-through / coherent read)


typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kLayoutThreads = 1024;                          // 16 waves
constexpr int kLayoutWaves = kLayoutThreads / kWave;
constexpr int kSlotsPerLane = kLayoutSlotsPerBlock / kLayoutThreads;   // slots per lane
constexpr int kWaveSlots = kLayoutSlotsPerBlock / kLayoutWaves;       // slots per wave

// Dynamic LDS of the rank launch: s_base, s_cnt, s_off, s_tmp and the per-wave counts.
inline size_t layout_rank_lds(int E) {
    return sizeof(int) * (size_t)(3 * E + 1 + kLayoutWaves) + sizeof(uint16_t) * (size_t)kLayoutWaves * E;
}

__device__ __forceinline__ int uniform_i(int v) { return __builtin_amdgcn_readfirstlane(v); }

// The hardware hands workgroup b to XCD b mod 8.  This bijection of [0, G)
// gives XCD x the contiguous blocks [x*G/8, (x+1)*G/8) instead (the first
// G mod 8 XCDs take one block more), so the tokens one XCD works on are
// consecutive.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_contiguous_block(int b, int G) {
    const int q = G / kXcds, r = G % kXcds, x = b % kXcds, j = b / kXcds;
    return x * q + (x < r ? x : r) + j;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int lane = threadIdx.x & (kWave - 1);
    return (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
}

// Lanes of the wave whose key equals this lane's key (all 64 lanes active).
__device__ __forceinline__ uint64_t match_any(int key, int nbits) {
    uint64_t m = ~0ull;
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t bal = __ballot(bit);
        m &= bit ? bal : ~bal;
    }
    return m;
}

template <bool NT, typename T>
__device__ __forceinline__ void store_v(T* p, const T& v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

template <bool NT, typename T>
__device__ __forceinline__ T load_v(const T* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}

// ---------------------------------------------------------------- layout ---

__device__ __forceinline__ int key_bits(int E) { return 32 - __clz(E); }

// Exclusive scan over a workgroup of NT threads; returns this thread's prefix
// and the total.  Every thread must call it.
template <int NT>
__device__ int block_exclusive_scan(int v, int* s_tmp, int& total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    int x = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(x, d, kWave);
        if (lane >= d) x += y;
    }
    if (lane == kWave - 1) s_tmp[w] = x;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / kWave; ++i) {
        const int c = s_tmp[i];
        before += (i < w) ? c : 0;
        tot += c;
    }
    __syncthreads();
    total = tot;
    return before + x - v;
}

// Exclusive scan over one wave; returns this lane's prefix and the wave total.
__device__ __forceinline__ int wave_exclusive_scan(int v, int& total) {
    const int lane = threadIdx.x & (kWave - 1);
    int x = v;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(x, d, kWave);
        if (lane >= d) x += y;
    }
    total = __shfl(x, kWave - 1, kWave);
    return x - v;
}

// Keys of this wave's kWaveSlots slots, slot = base + i*64 + lane: the expert id, or
// E for masked, invalid and past-the-end slots.  All loads are issued first.
__device__ __forceinline__ void load_keys(const int32_t* idx, int base, int S, int E,
                                          int (&key)[kSlotsPerLane], bool& bad) {
    const int lane = threadIdx.x & (kWave - 1);
    int raw[kSlotsPerLane];
#pragma unroll
    for (int i = 0; i < kSlotsPerLane; ++i) {
        const int s = base + i * kWave + lane;
        raw[i] = (s < S) ? idx[s] : -1;
    }
#pragma unroll
    for (int i = 0; i < kSlotsPerLane; ++i) {
        const bool ok = raw[i] >= 0 && raw[i] < E;
        bad |= !ok && raw[i] != -1;
        key[i] = ok ? raw[i] : E;
    }
}

// Launch 1 of the multi-workgroup layout: per-workgroup expert histograms.
__global__ __launch_bounds__(kLayoutThreads) void k_layout_count(LayoutArgs a) {
    extern __shared__ int smem[];
    int* hist = smem;                                   // [E]
    const int E = a.E, tid = threadIdx.x, lane = tid & (kWave - 1);
    const int w = uniform_i(tid / kWave);
    const int base = (int)blockIdx.x * kLayoutSlotsPerBlock + w * kWaveSlots;
    int key[kSlotsPerLane];
    bool bad = false;
    load_keys(a.topk_idx, base, a.S, E, key, bad);
    for (int i = tid; i < E; i += kLayoutThreads) hist[i] = 0;
    __syncthreads();
    const int nbits = key_bits(E);
#pragma unroll
    for (int i = 0; i < kSlotsPerLane; ++i) {
        if (base + i * kWave >= a.S) break;             // uniform per wave
        const uint64_t m = match_any(key[i], nbits);
        if (key[i] < E && lane == __ffsll((unsigned long long)m) - 1)
            atomicAdd(&hist[key[i]], __popcll(m));
    }
    if (a.error && __ballot(bad) && lane == 0) atomicOr(a.error, 1u);
    __syncthreads();
    for (int e = tid; e < E; e += kLayoutThreads)
        a.ws[(int64_t)blockIdx.x * E + e] = hist[e];
}

// The layout's routing density, for its combine's launch shape: 4 or more
// real rows per token on average is dense.  The word lives in pinned host
// memory and carries the layout's epoch, so the host can tell which layout
// it belongs to; the store is issued as early as the total is known, so that
// its trip to the host overlaps the rest of the kernel.
__device__ __forceinline__ void report_density(const LayoutArgs& a, int rows) {
    if (!a.density) return;
    const int64_t T = a.S / a.K;
    const uint32_t d = (int64_t)rows >= 4 * T ? (uint32_t)kDensityDense : (uint32_t)kDensitySparse;
    __hip_atomic_store(a.density, ((uint64_t)a.epoch << 32) | d, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_SYSTEM);
}

// Layout ranks, run by workgroup b of nb (kLayoutThreads threads).  FUSED:
// the whole layout in this one workgroup (nb == 1, b == 0, no histogram
// launch).  Otherwise launch 2 of the multi-workgroup layout: the workgroup
// sums the histograms of the workgroups before it and of all of them, scans
// tiles over experts, and ranks its own kLayoutSlotsPerBlock slots.  Every
// workgroup writes its share of the tile metadata and of the padding rows.
// ROWS_ONLY (with FUSED): only the pool row of every slot, into rows_out (LDS,
// S entries, -1 for a masked slot); nothing is written to global memory.
template <bool FUSED, bool ROWS_ONLY>
__device__ __forceinline__ void layout_rank_body(const LayoutArgs& a, int nb, int lg_tpe, int b,
                                                 int32_t* rows_out) {
    static_assert(FUSED || !ROWS_ONLY, "rows only for the one-workgroup layout");
    extern __shared__ int smem[];
    __shared__ int s_rows;                              // real rows (density report)
    const int E = a.E, BM = a.BM;
    int* s_base = smem;                                 // [E]   first row of e for this workgroup
    int* s_cnt = s_base + E;                            // [E]   rows of expert e
    int* s_off = s_cnt + E;                             // [E+1] first tile of expert e
    int* s_tmp = s_off + E + 1;                         // [16]
    uint16_t* wc = (uint16_t*)(s_tmp + kLayoutWaves);   // [16][E] per-wave counts, then next ranks
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int w = uniform_i(tid / kWave);
    const int nbits = key_bits(E);
    const int base = b * kLayoutSlotsPerBlock + w * kWaveSlots;
    if (tid == 0) s_rows = 0;                           // ordered before the adds by the barriers below

    int key[kSlotsPerLane];
    bool bad = false;
    load_keys(a.topk_idx, base, a.S, E, key, bad);
    float wv[kSlotsPerLane];                            // weights copied at the end, loaded now
#pragma unroll
    for (int j = 0; j < kSlotsPerLane; ++j) {
        const int s = base + j * kWave + lane;
        wv[j] = (!ROWS_ONLY && s < a.S && a.topk_w) ? a.topk_w[s] : 0.0f;
    }
    for (int i = tid; i < kLayoutWaves * E; i += kLayoutThreads) wc[i] = 0;

    int total = 0;
    if constexpr (!FUSED) {
        // rows of expert e in earlier workgroups (pre) and in all (tot); 2^lg_tpe threads per expert
        const int tpe = 1 << lg_tpe;
        const int e = tid >> lg_tpe, part = tid & (tpe - 1);
        int pre = 0, tot = 0;
        if (e < E) {
            // eight independent loads in flight per round
            for (int bb0 = part; bb0 < nb; bb0 += 8 * tpe) {
                int c[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int bb = bb0 + i * tpe;
                    c[i] = (bb < nb) ? a.ws[(int64_t)bb * E + e] : 0;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    tot += c[i];
                    pre += (bb0 + i * tpe < b) ? c[i] : 0;
                }
            }
        }
        for (int d = 1; d < tpe; d <<= 1) {
            pre += __shfl_xor(pre, d, kWave);
            tot += __shfl_xor(tot, d, kWave);
        }
        const bool owner = e < E && part == 0;
        const int tiles = owner ? (tot + BM - 1) / BM : 0;
        const int off = block_exclusive_scan<kLayoutThreads>(tiles, s_tmp, total);
        if (owner) {
            s_cnt[e] = tot;
            s_off[e] = off;
            s_base[e] = off * BM + pre;
        }
        if (b == 0) {                                   // all real rows, for the density report
            int v = owner ? tot : 0;
            for (int d = kWave / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, kWave);
            if (lane == 0 && v) atomicAdd(&s_rows, v);
        }
    }
    __syncthreads();
    if (!FUSED && b == 0 && tid == 0) report_density(a, s_rows);

    // per-wave counts; each iteration's match mask is kept for the ranking pass
    uint64_t m[kSlotsPerLane];
    int nvalid = 0;
#pragma unroll
    for (int i = 0; i < kSlotsPerLane; ++i) {
        m[i] = 0;
        if (base + i * kWave >= a.S) continue;          // uniform per wave
        m[i] = match_any(key[i], nbits);
        if (key[i] < E && lane == __ffsll((unsigned long long)m[i]) - 1)
            wc[w * E + key[i]] += (uint16_t)__popcll(m[i]);
        if constexpr (FUSED) nvalid += __popcll(__ballot(key[i] < E));
    }
    if (FUSED && !ROWS_ONLY && lane == 0 && nvalid) atomicAdd(&s_rows, nvalid);
    // The handle's copy of the weights (this wave's slots, as the keys).  On
    // gfx9 a wait for a load also waits for every store issued before it, so
    // global stores are kept after the last global load is consumed.
    if constexpr (!ROWS_ONLY) {
#pragma unroll
        for (int j = 0; j < kSlotsPerLane; ++j) {
            const int s = base + j * kWave + lane;
            if (s < a.S && a.weights) a.weights[s] = wv[j];
        }
    }
    __syncthreads();
    if (FUSED && !ROWS_ONLY && tid == 0) report_density(a, s_rows);

    // exclusive prefix of the per-wave counts over waves; the last running sum
    // is the expert's count in this workgroup (E <= kLayoutThreads)
    int run = 0;
    if (tid < E) {
        int c[kLayoutWaves];                            // every load issued before the stores
#pragma unroll
        for (int v = 0; v < kLayoutWaves; ++v) c[v] = wc[v * E + tid];
#pragma unroll
        for (int v = 0; v < kLayoutWaves; ++v) {
            wc[v * E + tid] = (uint16_t)run;
            run += c[v];
        }
    }
    if constexpr (FUSED) {
        if (!ROWS_ONLY && a.error && __ballot(bad) && lane == 0) atomicOr(a.error, 1u);
        const int tiles = (tid < E) ? (run + BM - 1) / BM : 0;
        // with E <= 64 wave 0 holds every expert and scans without a barrier
        const int off = E <= kWave ? wave_exclusive_scan(tiles, total)
                                   : block_exclusive_scan<kLayoutThreads>(tiles, s_tmp, total);
        if (tid < E) {
            s_cnt[tid] = run;
            s_off[tid] = off;
            s_base[tid] = off * BM;
        }
    }
    if (tid == 0) s_off[E] = total;
    __syncthreads();

    // pool row of every slot of this wave
#pragma unroll
    for (int i = 0; i < kSlotsPerLane; ++i) {
        if (base + i * kWave >= a.S) continue;          // uniform per wave
        const int s = base + i * kWave + lane;
        const int k = key[i];
        const int leader = __ffsll((unsigned long long)m[i]) - 1;
        int cur = 0;
        if (k < E && lane == leader) {
            cur = wc[w * E + k];
            wc[w * E + k] = (uint16_t)(cur + __popcll(m[i]));
        }
        cur = __shfl(cur, leader, kWave);
        if (s < a.S) {
            if (k < E) {
                const int row = s_base[k] + cur + __popcll(m[i] & lanemask_lt());
                if constexpr (ROWS_ONLY) {
                    rows_out[s] = row;
                } else {
                    a.slot_to_row[s] = row;
                    a.recv_token[row] = s / a.K;
                }
            } else {
                if constexpr (ROWS_ONLY) rows_out[s] = -1;
                else a.slot_to_row[s] = -1;
            }
        }
    }
    if constexpr (ROWS_ONLY) return;

    // Tile metadata and padding rows, expert by expert (expert e's tiles are
    // [s_off[e], s_off[e+1]) and its padding rows follow its s_cnt[e] real
    // rows): workgroup b takes experts b, b + nb, ..., one wave per expert.
    // (the next expert's bounds are read before this one's stores)
    const int estep = nb * kLayoutWaves;
    int e_n = b + nb * w;
    int j0_n = 0, j1_n = 0, cnt_n = 0;
    if (e_n < E) {
        j0_n = s_off[e_n];
        j1_n = s_off[e_n + 1];
        cnt_n = s_cnt[e_n];
    }
    for (int e = e_n; e < E; e += estep) {
        const int j0 = j0_n, nt = j1_n - j0_n, cnt = cnt_n;
        e_n = e + estep;
        if (e_n < E) {
            j0_n = s_off[e_n];
            j1_n = s_off[e_n + 1];
            cnt_n = s_cnt[e_n];
        }
        for (int i = lane; i < nt; i += kWave) {
            const int left = cnt - i * BM;
            a.tile_expert[j0 + i] = e;
            a.tile_target[j0 + i] = left < BM ? left : BM;
            if (a.arrival) {
                a.arrival[j0 + i] = 0u;
                // not ready for any dispatch after this layout (whose sequence
                // numbers come after seq_base), also when a graph replays both
                a.tile_ready[j0 + i] = a.seq_base;
            }
        }
        for (int r = j0 * BM + cnt + lane; r < (j0 + nt) * BM; r += kWave) a.recv_token[r] = -1;
    }
    // ... then the tiles and rows past the last tile, spread over all workgroups
    const int total_t = s_off[E];
    for (int j = total_t + b * kLayoutThreads + tid; j < a.max_tiles; j += nb * kLayoutThreads) {
        a.tile_expert[j] = -1;
        a.tile_target[j] = 0;
    }
    for (int r = total_t * BM + b * kLayoutThreads + tid; r < a.cap; r += nb * kLayoutThreads)
        a.recv_token[r] = -1;
    const int s1 = min(a.S, (b + 1) * kLayoutSlotsPerBlock);
    // and the per-token done counts of the tokens whose first slot is here
    const int T = a.S / a.K;
    const int tb0 = (b * kLayoutSlotsPerBlock + a.K - 1) / a.K;
    const int tb1 = min(T, (s1 + a.K - 1) / a.K);
    if (a.y_done)
        for (int t = tb0 + tid; t < tb1; t += kLayoutThreads) a.y_done[t] = 0u;
    // counts, first tiles and the tile total (workgroup 0)
    if (b == 0) {
        for (int e = tid; e <= E; e += kLayoutThreads) {
            if (e < E) a.counts[e] = s_cnt[e];
            a.offsets[e] = s_off[e];
        }
        if (tid == 0) *a.num_tiles = s_off[E];
    }
}

template <bool FUSED>
__global__ __launch_bounds__(kLayoutThreads) void k_layout_rank(LayoutArgs a, int nb, int lg_tpe) {
    layout_rank_body<FUSED, false>(a, nb, lg_tpe, (int)blockIdx.x, nullptr);
}

// ------------------------------------------------------------- dispatch ---

// Streaming release of one chunk (kStreamTokens consecutive tokens, one workgroup),
// without a workgroup barrier or a cache write-back.  All of a streaming
// dispatch's stores (pool rows and scales) are device-scope stores, which the
// XCD's L2 writes through, so a store counts as complete (vmcnt) only once it
// is visible to every XCD.  Each wave waits for its own stores, then counts
// itself done in LDS; the wave that completes the count has seen every other
// wave's stores complete and makes the chunk's arrival adds.  It groups the
// chunk's rows by tile with wave match masks (64 slots at a time), so a tile
// gets one add per chunk.  The add that brings a tile to round * target
// stores the sequence number into tile_ready[tile]; a consumer that
// acquire-loads it (which invalidates its own caches) then reads every row of
// the tile from the coherent level.
__device__ void release_chunk(const DispatchArgs& a, int t0, int t1, uint32_t* s_done) {
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t nw = blockDim.x / kWave;
    __builtin_amdgcn_s_waitcnt(0);                 // this wave's stores are complete
    __atomic_signal_fence(__ATOMIC_SEQ_CST);       // and no memory access moves across
    uint32_t old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(s_done, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_WORKGROUP);
    old = (uint32_t)__shfl((int)old, 0, kWave);
    if (old != nw - 1u) return;                    // not the last wave of the chunk
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const int nbits = 32 - __clz(a.max_tiles);     // tile ids and the no-row key max_tiles
    const int s0 = t0 * a.K, s1 = t1 * a.K;
    for (int b = s0; b < s1; b += kWave) {
        const int s = b + lane;
        const int r = s < s1 ? a.slot_to_row[s] : -1;
        const int tile = r >= 0 ? r / a.BM : a.max_tiles;
        const uint64_t m = match_any(tile, nbits);
        if (r >= 0 && lane == __ffsll((unsigned long long)m) - 1) {
            const uint32_t cnt = (uint32_t)__popcll(m);
            const uint32_t prev = __hip_atomic_fetch_add(&a.arrival[tile], cnt, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
            if (prev + cnt == a.round * (uint32_t)a.tile_target[tile])
                __hip_atomic_store(&a.tile_ready[tile], a.seq, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Stores of 16-byte chunk c of a row.  The pool, the gradient rows and y are
// written once and read by another kernel, so nothing is kept in the caches
// (non-temporal).  Device-scope stores are written through the XCD's L2: they
// leave no dirty line behind, which keeps a later device-scope release (and
// the end-of-kernel write-back) cheap, and they count as complete only once
// every XCD can see them, which the streaming release relies on.
enum StoreMode { kStoreNonTemporal, kStoreDeviceNonTemporal };

template <StoreMode MODE>
__device__ __forceinline__ void store_row(u32x4* row, int row_bytes, int c, const u32x4& v) {
    if constexpr (MODE == kStoreNonTemporal) {
        __builtin_nontemporal_store(v, row + c);
    } else {
        __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(row, (short)0, row_bytes, 0x00020000);
        __builtin_amdgcn_raw_buffer_store_b128(v, r, c * 16, 0, kAuxDevice | kAuxNonTemporal);
    }
}

// Pool rows, with or without the streaming release: device-scope
// non-temporal stores.  (Device-scope stores without the non-temporal hint
// made the streaming dispatch faster only when a cache flush ran between
// steps: they leave the rows dirty in the last-level cache, and the flush
// then writes them back; back to back they were 11 % slower.)
__device__ __forceinline__ void store_pool(u32x4* row, int row_bytes, int c, const u32x4& v) {
    store_row<kStoreDeviceNonTemporal>(row, row_bytes, c, v);
}

// Slot groups.  A kernel holds the pool rows (and weights) of at most KT <= 8
// slots of a token in registers.  With MANY (top_k above 8) it walks the
// token's slots in groups of KT, in ascending slot order, so the registers a
// wave needs do not grow with top_k and the fp32 sums keep their slot order.
constexpr int kSlotGroup = 8;

template <bool MANY, int KT>
__device__ __forceinline__ int slot_groups(int K) {
    return MANY ? (K + KT - 1) / KT : 1;
}

// Pool rows of slots k0 .. k0+KT-1 of token t (-1 past top_k); true when one
// of them is a real row.
template <int KT>
__device__ __forceinline__ bool load_rows(const int32_t* s2r, int t, int K, int k0, int (&rows)[KT]) {
    bool any = false;
#pragma unroll
    for (int k = 0; k < KT; ++k) {
        rows[k] = (k0 + k < K) ? s2r[t * K + k0 + k] : -1;
        any |= rows[k] >= 0;
    }
    return any;
}

// Work items are (token, segment) pairs, item = t * nseg + seg, handed out in
// order: workgroup b owns items [b * ipb, (b+1) * ipb) and its waves take them
// round-robin.  In streaming mode ipb is a whole number of tokens.  With MANY
// an item's first slot group is loaded ahead and the later groups' rows are
// read as they are stored (an item is never skipped).
// Workgroup bid of the dispatch; s2r is the slot -> pool row map (the
// handle's, or one a fused layout has just built in LDS).
// PRE: the x segment of the wave's first item is already in pre (loaded by
// the caller before it built s2r, so that the two waits overlap).
template <int KT, bool STREAM, bool MANY, bool PRE = false>
__device__ __forceinline__ void dispatch_bf16_body(const DispatchArgs& a, int nseg, int ipb, int bid,
                                                   const int32_t* s2r, const u32x4 (&pre)[kDispatchChunks]) {
    constexpr int U = kDispatchChunks;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = uniform_i(threadIdx.x / kWave);
    const int n16 = a.H / 8;
    const u32x4* x = (const u32x4*)a.x;
    u32x4* pool = (u32x4*)a.pool;
    const int nw = (int)blockDim.x / kWave;
    // streaming: the workgroup's items are the tokens of one chunk, released
    // as soon as they are stored; chunks follow token order
    __shared__ uint32_t s_done;
    if constexpr (STREAM) {
        if (threadIdx.x == 0) s_done = 0u;
        __syncthreads();
    }
    const int i0 = bid * ipb;
    const int i1 = min(a.T * nseg, i0 + ipb);
    // software-pipelined as in the FP8 dispatch: the next item's rows and x
    // segment are loaded before the current one is stored
    auto fetch = [&](int it_, int (&r)[KT], u32x4 (&v_)[U]) -> bool {
        const int t_ = it_ / nseg;
        const int seg_ = it_ - t_ * nseg;
        if (!load_rows<KT>(s2r, t_, a.K, 0, r) && !MANY) return false;
        const int c0_ = seg_ * (kWave * U) + lane;
        const u32x4* src_ = x + (int64_t)t_ * n16;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0_ + u * kWave;
            if (c < n16) v_[u] = src_[c];
        }
        return true;
    };
    int rows_n[KT];
    u32x4 v_n[U];
    bool any_n = false;
    if (i0 + w < i1) {
        if constexpr (PRE) {
            any_n = load_rows<KT>(s2r, (i0 + w) / nseg, a.K, 0, rows_n) || MANY;
#pragma unroll
            for (int u = 0; u < U; ++u) v_n[u] = pre[u];
        } else {
            any_n = fetch(i0 + w, rows_n, v_n);
        }
    }
    for (int it = i0 + w; it < i1; it += nw) {
        const int t = it / nseg;
        const int seg = it - t * nseg;
        int rows[KT];
        u32x4 v[U];
        const bool any = any_n;
#pragma unroll
        for (int k = 0; k < KT; ++k) rows[k] = rows_n[k];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = v_n[u];
        any_n = (it + nw < i1) && fetch(it + nw, rows_n, v_n);
        if (!any) continue;
        const int c0 = seg * (kWave * U) + lane;
        const int ngroups = slot_groups<MANY, KT>(a.K);
        for (int g = 0; g < ngroups; ++g) {
            if (MANY && g > 0) load_rows<KT>(s2r, t, a.K, g * KT, rows);
#pragma unroll
            for (int k = 0; k < KT; ++k) {
                if (rows[k] < 0) continue;
                u32x4* dst = pool + (int64_t)rows[k] * n16;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int c = c0 + u * kWave;
                    if (c < n16) store_pool(dst, a.H * 2, c, v[u]);
                }
            }
        }
    }
    if constexpr (STREAM) release_chunk(a, i0 / nseg, i1 / nseg, &s_done);
}

template <int KT, bool STREAM, bool MANY>
__global__ __launch_bounds__(1024) void k_dispatch_bf16(DispatchArgs a, int nseg, int ipb) {
    const u32x4 none[kDispatchChunks] = {};
    dispatch_bf16_body<KT, STREAM, MANY>(a, nseg, ipb, (int)blockIdx.x, a.slot_to_row, none);
}

// bf16 dispatch for dense routing (4 or more rows per token) without the
// streaming release, in two launches.  First a read pass streams x through
// the caches into the last-level cache (MALL); then one workgroup per (token,
// 1 KB row segment) has wave k store the segment to slot k's row, one 16-byte
// access per lane.  Each wave holds 1 KB of stores, so the workgroups in
// flight cover a narrow window of tokens and the pool is written at close to
// the rate of sequential writes; their x loads hit the MALL.  Without the
// read pass the same loads go to HBM in the middle of the write stream and
// stall the writers (16384 tokens x top-8, hidden 7168, caches flushed: 508
// against 345 us for both launches; back to back 304 / 338 us).  With
// sparse routing most of its waves would have nothing to store, so
// k_dispatch_bf16 serves that.

// The read pass: every 16-byte chunk of x loaded once with plain (cached)
// loads, several in flight per lane, and folded into a value nothing reads.
__global__ __launch_bounds__(256) void k_stage_x(const u32x4* x, int64_t n16) {
    u32x4 acc = {0u, 0u, 0u, 0u};
    const int64_t stride = (int64_t)gridDim.x * 256;
#pragma unroll 4
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < n16; c += stride) acc ^= x[c];
    // a data-dependent branch keeps the loads; it never writes memory
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) __builtin_amdgcn_s_sleep(1);
}

template <int KT>
__global__ __launch_bounds__(kWave * KT) void k_dispatch_bf16_dense(DispatchArgs a, int nseg) {
    const int lane = threadIdx.x & (kWave - 1);
    const int k = uniform_i(threadIdx.x / kWave);
    const int t = (int)blockIdx.x / nseg;
    const int seg = (int)blockIdx.x - t * nseg;
    if (k >= a.K) return;
    const int row = a.slot_to_row[t * a.K + k];
    if (row < 0) return;
    const int n16 = a.H / 8;
    const int c = seg * kWave + lane;
    if (c >= n16) return;
    const u32x4 v = ((const u32x4*)a.x)[(int64_t)t * n16 + c];
    store_pool((u32x4*)a.pool + (int64_t)row * n16, a.H * 2, c, v);
}

// --- FP8 e4m3fn with UE8M0 scales, from bf16 bit patterns, integer only ---

// Scale exponent of a group from the largest finite bf16 magnitude pattern:
// smallest e in [-127, 127] with amax <= 448 * 2^e (448 = 1.75 * 2^8).
__device__ __forceinline__ int ue8m0_exp(uint32_t amag) {
    if (amag == 0x7F80u) return 127;                 // infinite amax: no e fits
    const int eb = (int)(amag >> 7);
    if (eb == 0) return -127;                        // zero or subnormal amax
    const int e = eb - 135 + (((amag & 0x7Fu) > 0x60u) ? 1 : 0);
    return e < -127 ? -127 : e;
}

// e4m3fn code of (bf16 pattern b) * 2^-e, round to nearest even, sign kept.
__device__ __forceinline__ uint32_t e4m3_code(uint32_t b, int e) {
    const uint32_t sign = (b >> 8) & 0x80u;
    const uint32_t mag = b & 0x7FFFu;
    if (mag > 0x7F80u) return sign | 0x7Fu;          // NaN
    if (mag == 0x7F80u) return sign | 0x7Eu;         // infinity saturates
    if (mag == 0u) return sign;
    const int eb = (int)(mag >> 7);
    const uint32_t sig = eb ? (0x80u | (mag & 0x7Fu)) : (mag & 0x7Fu);   // value = sig * 2^p
    const int p = (eb ? eb - 134 : -133) - e;
    const int nb = 32 - __clz(sig);
    const int k = p + nb - 1;                        // unbiased exponent of the value
    uint32_t code;
    if (k >= -6) {                                   // normal: keep 4 significant bits
        const int sh = nb - 4;
        uint32_t m, up = 0;
        if (sh <= 0) {
            m = sig << (-sh);
        } else {
            m = sig >> sh;
            const uint32_t rem = sig & ((1u << sh) - 1u), half = 1u << (sh - 1);
            up = (rem > half || (rem == half && (m & 1u))) ? 1u : 0u;
        }
        code = ((uint32_t)(k + 7) << 3) + (m - 8u) + up;
        code = code > 0x7Eu ? 0x7Eu : code;
    } else {                                         // subnormal: multiples of 2^-9
        const int sh = -(p + 9);
        if (sh <= 0) {
            code = sig << (-sh);
        } else if (sh >= 10) {
            code = 0u;
        } else {
            const uint32_t m = sig >> sh;
            const uint32_t rem = sig & ((1u << sh) - 1u), half = 1u << (sh - 1);
            code = m + ((rem > half || (rem == half && (m & 1u))) ? 1u : 0u);
        }
    }
    return sign | code;
}

// e4m3fn code magnitude of a finite non-negative float32 (bit pattern v),
// round to nearest even, saturating at 448 (code 0x7E).
__device__ __forceinline__ uint32_t e4m3_code_f32(uint32_t v) {
    if (v >= 0x43E00000u) return 0x7Eu;             // >= 448
    const int eb = (int)(v >> 23);
    const uint32_t sig = eb ? (0x800000u | (v & 0x7FFFFFu)) : (v & 0x7FFFFFu);
    if (sig == 0u) return 0u;
    const int p = eb ? eb - 150 : -149;              // value = sig * 2^p
    const int nb = 32 - __clz(sig);
    const int k = p + nb - 1;
    if (k >= -6) {                                   // normal: keep 4 significant bits
        const int sh = nb - 4;                       // >= 1: sig has >= 5 bits here
        const uint32_t m = sig >> sh;
        const uint32_t rem = sig & ((1u << sh) - 1u), half = 1u << (sh - 1);
        const uint32_t up = (rem > half || (rem == half && (m & 1u))) ? 1u : 0u;
        const uint32_t code = ((uint32_t)(k + 7) << 3) + (m - 8u) + up;
        return code > 0x7Eu ? 0x7Eu : code;
    }
    const int sh = -(p + 9);                         // subnormal: multiples of 2^-9
    if (sh <= 0) return sig << (-sh);
    if (sh >= 25) return 0u;
    const uint32_t m = sig >> sh;
    const uint32_t rem = sig & ((1u << sh) - 1u), half = 1u << (sh - 1);
    return m + ((rem > half || (rem == half && (m & 1u))) ? 1u : 0u);
}

// Float32-scale flavour: code of float(x * f) for the bf16 pattern b, with
// the sign of x; a NaN product gives 0x7F.
__device__ __forceinline__ uint32_t e4m3_code_scaled(uint32_t b, float f) {
    const uint32_t sign = (b >> 8) & 0x80u;
    const float v = __uint_as_float(b << 16) * f;
    const uint32_t mag = __float_as_uint(v) & 0x7FFFFFFFu;
    if (mag > 0x7F800000u) return sign | 0x7Fu;
    return sign | e4m3_code_f32(mag);
}

// Four bf16 values (two per word) to four e4m3fn codes with gfx950's scaled
// conversion, the scale given as a power of two in a float's exponent field.
typedef __bf16 bf16x2_in_t __attribute__((ext_vector_type(2)));
typedef short shortx2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_fp8(uint32_t w0, uint32_t w1, float scale) {
    bf16x2_in_t a, b;
    __builtin_memcpy(&a, &w0, 4);
    __builtin_memcpy(&b, &w1, 4);
    shortx2_t r = {0, 0};
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, a, scale, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, b, scale, true);
    uint32_t out;
    __builtin_memcpy(&out, &r, 4);
    return out;
}

__device__ __forceinline__ uint32_t mag_for_max(uint32_t b) {
    const uint32_t m = b & 0x7FFFu;
    return m > 0x7F80u ? 0u : m;                     // NaN does not take part
}

// Scale stores of one 64-lane step (8 groups): every lane of a group holds
// its group's byte (UE8M0) and float (the other flavours).  When streaming,
// every scale store is a relaxed device-scope atomic store, written through
// the XCD's L2 like the pool rows, so the release needs no write-back; plain
// stores otherwise.
template <bool STREAM, typename V>
__device__ __forceinline__ void put_scale(V* p, V v) {
    if constexpr (STREAM)
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        *p = v;
}

template <int KT, bool STREAM>
__device__ __forceinline__ void store_scales(const DispatchArgs& a, const int (&rows)[KT], int c,
                                             int nunit, int ngrp, bool pack8, uint32_t sbyte,
                                             float sval) {
    const int lane = threadIdx.x & (kWave - 1);
    const int g = c >> 3;
    if (a.scale_kind == kScaleUe8m0 && a.scale_mn) {
        // packed words: group 4w + j in byte j; lanes 0 and 32 hold groups 4w
        const uint32_t word = sbyte | ((uint32_t)__shfl((int)sbyte, lane + 8, kWave) << 8) |
                              ((uint32_t)__shfl((int)sbyte, lane + 16, kWave) << 16) |
                              ((uint32_t)__shfl((int)sbyte, lane + 24, kWave) << 24);
        if ((lane & 31) == 0 && g < ngrp) {
            uint32_t* col = (uint32_t*)a.scales + (int64_t)(g >> 2) * a.scale_ld;
#pragma unroll
            for (int k = 0; k < KT; ++k)
                if (rows[k] >= 0) put_scale<STREAM>(col + rows[k], word);
        }
    } else if (a.scale_kind == kScaleUe8m0) {
        // the 8 bytes of a full step go out as one 64-bit store per row
        if (pack8 && c - lane + kWave <= nunit) {
            uint64_t word = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                word |= (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)sbyte, 8 * j) << (8 * j);
            const int g0 = (c - lane) >> 3;
#pragma unroll
            for (int k = 0; k < KT; ++k) {
                if (rows[k] < 0 || lane != k) continue;
                put_scale<STREAM>((uint64_t*)((uint8_t*)a.scales + (int64_t)rows[k] * ngrp + g0), word);
            }
        } else if (c < nunit && (lane & 7) == 0) {
#pragma unroll
            for (int k = 0; k < KT; ++k) {
                if (rows[k] < 0) continue;
                put_scale<STREAM>((uint8_t*)a.scales + (int64_t)rows[k] * ngrp + g,
                                                       (uint8_t)sbyte);
            }
        }
    } else if (c < nunit && (lane & 7) == 0) {
        float* sc = (float*)a.scales;
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            if (rows[k] < 0) continue;
            float* p = a.scale_mn ? sc + (int64_t)g * a.scale_ld + rows[k]
                                  : sc + (int64_t)rows[k] * ngrp + g;
            put_scale<STREAM>(p, sval);
        }
    }
}

// F32Q: float32 scale amax / 448 and codes of x * (448 / amax); otherwise the
// UE8M0 exponent (stored as a byte, or as the float 2^e).  U: 16-channel
// units per lane per work item.
// PRE: the x units of the wave's first item are already in pre_lo / pre_hi
// (loaded by the caller before it built s2r).
template <int KT, bool STREAM, bool F32Q, int U, bool MANY, bool PRE = false>
__device__ __forceinline__ void dispatch_fp8_body(const DispatchArgs& a, int nseg, int ipb, int bid, int nblk,
                                                  const int32_t* s2r, const u32x4 (&pre_lo)[U],
                                                  const u32x4 (&pre_hi)[U]) {
    const int lane = threadIdx.x & (kWave - 1);
    const int w = uniform_i(threadIdx.x / kWave);
    const int nunit = a.H / 16;          // 16 channels (32 bytes in, 16 bytes out) per unit
    const int ngrp = a.H / 128;
    // a row's 8 UE8M0 scale bytes of a 64-lane step go out as one 64-bit store
    const bool pack8 = (ngrp & 7) == 0 && ((uintptr_t)a.scales & 7) == 0;
    const u32x4* x = (const u32x4*)a.x;
    u32x4* pool = (u32x4*)a.pool;
    const int nw = (int)blockDim.x / kWave;
    __shared__ uint32_t s_done;                     // streaming: waves done with the chunk
    if constexpr (STREAM) {
        if (threadIdx.x == 0) s_done = 0u;
        __syncthreads();
    }
    // Float32 scales are 4-byte entries whose cache lines are shared by
    // consecutive pool rows of an expert, i.e. by consecutive tokens.  With
    // each XCD on a contiguous token range those lines are completed in one
    // L2 before they are written back, instead of in pieces from all eight
    // (measured 1-11 % faster for the float flavours at 16384 tokens; bf16
    // and UE8M0 keep the round-robin, which measured slightly faster there).
    const int blk = a.scale_kind != kScaleUe8m0 ? xcd_contiguous_block(bid, nblk) : bid;
    const int i0 = blk * ipb;
    const int i1 = min(a.T * nseg, i0 + ipb);
    // a wave's items are software-pipelined: the next item's rows and x
    // segment are loaded before the current one is quantised and stored
    auto fetch = [&](int it_, int (&r)[KT], u32x4 (&l)[U], u32x4 (&h)[U]) -> bool {
        const int t_ = it_ / nseg;
        const int seg_ = it_ - t_ * nseg;
        if (!load_rows<KT>(s2r, t_, a.K, 0, r) && !MANY) return false;
        const int u0_ = seg_ * (kWave * U) + lane;
        const u32x4* src_ = x + (int64_t)t_ * (a.H / 8);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = u0_ + u * kWave;
            if (c < nunit) {
                l[u] = src_[2 * c];
                h[u] = src_[2 * c + 1];
            } else {
                l[u] = u32x4{0, 0, 0, 0};
                h[u] = u32x4{0, 0, 0, 0};
            }
        }
        return true;
    };
    int rows_n[KT];
    u32x4 lo_n[U], hi_n[U];
    bool any_n = false;
    if (i0 + w < i1) {
        if constexpr (PRE) {
            any_n = load_rows<KT>(s2r, (i0 + w) / nseg, a.K, 0, rows_n) || MANY;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                lo_n[u] = pre_lo[u];
                hi_n[u] = pre_hi[u];
            }
        } else {
            any_n = fetch(i0 + w, rows_n, lo_n, hi_n);
        }
    }
    for (int it = i0 + w; it < i1; it += nw) {
        const int t = it / nseg;
        const int seg = it - t * nseg;
        int rows[KT];
        u32x4 lo[U], hi[U];
        const bool any = any_n;
#pragma unroll
        for (int k = 0; k < KT; ++k) rows[k] = rows_n[k];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            lo[u] = lo_n[u];
            hi[u] = hi_n[u];
        }
        any_n = (it + nw < i1) && fetch(it + nw, rows_n, lo_n, hi_n);
        if (!any) continue;
        const int u0 = seg * (kWave * U) + lane;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = u0 + u * kWave;
            if (c - lane >= nunit) break;            // whole wave past the row
            // 8 lanes hold one 128-channel group (groups never straddle lanes 8g..8g+7)
            uint32_t amax = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                amax = max(amax, max(mag_for_max(lo[u][i]), mag_for_max(lo[u][i] >> 16)));
                amax = max(amax, max(mag_for_max(hi[u][i]), mag_for_max(hi[u][i] >> 16)));
            }
            amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1, kWave));
            amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2, kWave));
            amax = max(amax, (uint32_t)__shfl_xor((int)amax, 4, kWave));
            u32x4 q;
            uint32_t sbyte = 0;
            float sval;
            if constexpr (F32Q) {
                // a = max(amax, 448 * 2^-126); s = a / 448; f = 448 / a (IEEE divisions)
                const float af = fmaxf(__uint_as_float(amax << 16), 448.0f * 0x1p-126f);
                sval = af / 448.0f;
                const float f = 448.0f / af;
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const uint32_t w0 = lo[u][2 * i], w1 = lo[u][2 * i + 1];
                    q[i] = e4m3_code_scaled(w0 & 0xFFFFu, f) | (e4m3_code_scaled(w0 >> 16, f) << 8) |
                           (e4m3_code_scaled(w1 & 0xFFFFu, f) << 16) |
                           (e4m3_code_scaled(w1 >> 16, f) << 24);
                    const uint32_t h0 = hi[u][2 * i], h1 = hi[u][2 * i + 1];
                    q[2 + i] = e4m3_code_scaled(h0 & 0xFFFFu, f) | (e4m3_code_scaled(h0 >> 16, f) << 8) |
                               (e4m3_code_scaled(h1 & 0xFFFFu, f) << 16) |
                               (e4m3_code_scaled(h1 >> 16, f) << 24);
                }
            } else {
                const int e = ue8m0_exp(amax);
                sbyte = (uint32_t)(e + 127);
                // 2^e as a float32 pattern (2^-127 is the subnormal 0x00400000)
                sval = __uint_as_float(e > -127 ? sbyte << 23 : 0x00400000u);
                // gfx950's scaled bf16 -> fp8 conversion (scale = the UE8M0 byte in a
                // float's exponent field) gives the integer encoder's codes for every
                // finite input within 448 * 2^e, which is every finite input here
                // (checked on the GPU for all bf16 patterns and scale bytes).  It differs
                // on NaN and infinity, so a unit holding one takes the integer path.
                uint32_t special = 0u;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    special |= ((lo[u][i] & 0x7F80u) == 0x7F80u) | ((lo[u][i] & 0x7F800000u) == 0x7F800000u);
                    special |= ((hi[u][i] & 0x7F80u) == 0x7F80u) | ((hi[u][i] & 0x7F800000u) == 0x7F800000u);
                }
                if (!special) {
                    const float hs = __uint_as_float(sbyte << 23);
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        q[i] = pk_fp8(lo[u][2 * i], lo[u][2 * i + 1], hs);
                        q[2 + i] = pk_fp8(hi[u][2 * i], hi[u][2 * i + 1], hs);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const uint32_t w0 = lo[u][2 * i], w1 = lo[u][2 * i + 1];
                        q[i] = e4m3_code(w0 & 0xFFFFu, e) | (e4m3_code(w0 >> 16, e) << 8) |
                               (e4m3_code(w1 & 0xFFFFu, e) << 16) | (e4m3_code(w1 >> 16, e) << 24);
                        const uint32_t h0 = hi[u][2 * i], h1 = hi[u][2 * i + 1];
                        q[2 + i] = e4m3_code(h0 & 0xFFFFu, e) | (e4m3_code(h0 >> 16, e) << 8) |
                                   (e4m3_code(h1 & 0xFFFFu, e) << 16) | (e4m3_code(h1 >> 16, e) << 24);
                    }
                }
            }
            const int ngroups = slot_groups<MANY, KT>(a.K);
            for (int g = 0; g < ngroups; ++g) {
                int rg[KT];
#pragma unroll
                for (int k = 0; k < KT; ++k) rg[k] = rows[k];
                if (MANY && g > 0) load_rows<KT>(s2r, t, a.K, g * KT, rg);
                if (c < nunit) {
#pragma unroll
                    for (int k = 0; k < KT; ++k) {
                        if (rg[k] < 0) continue;
                        store_pool(pool + (int64_t)rg[k] * nunit, a.H, c, q);
                    }
                }
                store_scales<KT, STREAM>(a, rg, c, nunit, ngrp, pack8, sbyte, sval);
            }
        }
    }
    if constexpr (STREAM) release_chunk(a, i0 / nseg, i1 / nseg, &s_done);
}

template <int KT, bool STREAM, bool F32Q, int U, bool MANY>
__global__ __launch_bounds__(1024) void k_dispatch_fp8(DispatchArgs a, int nseg, int ipb) {
    const u32x4 none[U] = {};
    dispatch_fp8_body<KT, STREAM, F32Q, U, MANY>(a, nseg, ipb, (int)blockIdx.x, (int)gridDim.x, a.slot_to_row,
                                                 none, none);
}

// -------------------------------------------------------------- combine ---


__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) & 0x8000u) | 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// A token's slot values (pool rows, weights) k0 .. k0+KT-1 for a wave that
// works on one token: the address is the same in every lane and the arrays
// are read-only while the kernel runs, so the reads go to the scalar unit, all
// issued before the first use.  Slots past top_k get `fill`.
template <int KT, typename V>
__device__ __forceinline__ void load_slots(const V* p, int t, int K, int k0, V fill, V (&out)[KT]) {
    typedef __attribute__((address_space(4))) const V CV;
    CV* q = (CV*)(p + (int64_t)t * K + k0);
#pragma unroll
    for (int k = 0; k < KT; ++k) out[k] = q[k0 + k < K ? k : 0];
#pragma unroll
    for (int k = 0; k < KT; ++k)
        if (k0 + k >= K) out[k] = fill;
}

// One combine work item: segment `seg` of token t (a wave gathers the token's
// expert rows for that segment, accumulates w * o in fp32 with one fused
// multiply-add per slot in slot order, and rounds once to bf16).  SCALAR: the
// slot values are read in one batch through the scalar unit, so a wave issues
// all its row loads at once (the plain combine; its launcher sets how many
// waves run at a time).  Otherwise they are read as vector loads, one slot
// after another (the gated combine).  With MANY the slots are taken in groups
// of KT, each group's rows loaded together, the accumulators carried over.
template <int KT, bool UNIT, bool SCALAR, bool MANY, bool COHERENT = false>
__device__ __forceinline__ int combine_compute(const CombineArgs& a, int t, int seg, int lane,
                                               u32x4 (&out)[kCombineChunks]) {
    constexpr int U = kCombineChunks;
    const int n16 = a.H / 8;
    const u32x4* eo = (const u32x4*)a.expert_out;
    const int c0 = seg * (kWave * U) + lane;
    float acc[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[u][i] = 0.0f;
    int nrows = 0;
    const int ngroups = slot_groups<MANY, KT>(a.K);
    for (int g = 0; g < ngroups; ++g) {
        const int k0 = g * KT;
        int rows[KT];
        float wt[KT];
        if constexpr (SCALAR) {
            load_slots<KT>(a.slot_to_row, t, a.K, k0, -1, rows);
            if constexpr (UNIT) {
#pragma unroll
                for (int k = 0; k < KT; ++k) wt[k] = 1.0f;
            } else {
                load_slots<KT>(a.weights, t, a.K, k0, 0.0f, wt);
            }
        } else {
#pragma unroll
            for (int k = 0; k < KT; ++k) {
                const bool in = k0 + k < a.K;
                rows[k] = in ? a.slot_to_row[t * a.K + k0 + k] : -1;
                wt[k] = UNIT ? 1.0f : (in ? a.weights[t * a.K + k0 + k] : 0.0f);
            }
        }
        u32x4 v[KT][U];
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            if (rows[k] < 0) continue;
            const u32x4* src = eo + (int64_t)rows[k] * n16;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * kWave;
                if (c >= n16) continue;
                if constexpr (COHERENT) {
                    // device-scope load: reads what another XCD's producer made
                    // visible, without an invalidation of this XCD's caches
                    __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                        (void*)src, (short)0, a.H * 2, 0x00020000);
                    v[k][u] = __builtin_amdgcn_raw_buffer_load_b128(rs, c * 16, 0, kAuxDevice);
                } else {
                    v[k][u] = load_v<true>(src + c);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int k = 0; k < KT; ++k) {
                if (rows[k] < 0) continue;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t p = v[k][u][i];
                    acc[u][2 * i] = __builtin_fmaf(wt[k], __uint_as_float(p << 16), acc[u][2 * i]);
                    acc[u][2 * i + 1] =
                        __builtin_fmaf(wt[k], __uint_as_float(p & 0xFFFF0000u), acc[u][2 * i + 1]);
                }
            }
        }
#pragma unroll
        for (int k = 0; k < KT; ++k) nrows += rows[k] >= 0 ? 1 : 0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            out[u][i] = f32_to_bf16_rne(acc[u][2 * i]) | (f32_to_bf16_rne(acc[u][2 * i + 1]) << 16);
    return nrows;
}

// Stores of one combine work item's outputs (row t of y, segment seg).
__device__ __forceinline__ void combine_store(const CombineArgs& a, int t, int seg, int lane,
                                              const u32x4 (&o)[kCombineChunks]) {
    constexpr int U = kCombineChunks;
    const int n16 = a.H / 8;
    const int c0 = seg * (kWave * U) + lane;
    u32x4* dst = (u32x4*)a.y + (int64_t)t * n16;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = c0 + u * kWave;
        if (c < n16) store_row<kStoreNonTemporal>(dst, a.H * 2, c, o[u]);
    }
}

template <int KT, bool UNIT, bool MANY>
__global__ __launch_bounds__(256) void k_combine(CombineArgs a, int nseg, int ipb) {
    const int lane = threadIdx.x & (kWave - 1);
    const int w = uniform_i(threadIdx.x / kWave);
    const int i0 = (int)blockIdx.x * ipb;
    const int i1 = min(a.T * nseg, i0 + ipb);
    for (int it = i0 + w; it < i1; it += 4) {
        const int t = it / nseg;
        const int seg = it - t * nseg;
        u32x4 o[kCombineChunks];
        combine_compute<KT, UNIT, true, MANY>(a, t, seg, lane, o);
        combine_store(a, t, seg, lane, o);
    }
}


// The items of a gated batch (token slot j < gtok, segment): wave w takes
// items w, w + nw, ...  On gfx9 a wait for a load also waits for every store
// issued before it, so a wave that owns several items computes D of them
// before issuing their stores: one store drain per D items, not per item.
// With few rows per token (a latency-bound batch) holding stores back was
// measured slower, so those batches use D = 1, and read a token's slots in
// one batch through the scalar unit, which measured faster there (and slower
// for dense batches, as in the plain combine at full occupancy).
template <int KT, int D, bool MANY, bool COHERENT>
__device__ __forceinline__ void gated_items(const CombineArgs& a, int nseg, int gtok, uint64_t mask,
                                            int w, int nw, int lane) {
    const int b = (int)blockIdx.x, nb = (int)gridDim.x;
    auto token_of = [&](int j) {
        return b + j * nb;
    };
    const int nit = gtok * nseg;
    for (int i0 = w; i0 < nit; i0 += D * nw) {
        u32x4 o[D][kCombineChunks];
        int tt[D], sg[D];
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int i = i0 + d * nw;
            const int j = i / nseg;
            tt[d] = -1;
            if (i < nit && token_of(j) < a.T && ((mask >> j) & 1ull)) {
                tt[d] = token_of(j);
                sg[d] = i - j * nseg;
                combine_compute<KT, false, D == 1, MANY, COHERENT>(a, tt[d], sg[d], lane, o[d]);
            }
        }
#pragma unroll
        for (int d = 0; d < D; ++d)
            if (tt[d] >= 0) combine_store(a, tt[d], sg[d], lane, o[d]);
    }
}

// Per-token gate (StreamEP README, y_done_per_token).  A workgroup takes
// kGateTokens tokens, strided by the grid size so that the workgroups in
// flight cover a compact window of tokens (their expert rows are then close
// together in each expert's block, as in the plain combine); one acquire per
// workgroup keeps the cache invalidations few.  Wave 0 waits, one lane per token, until
// every token's done count has reached round * (its unmasked slots), then
// acquires at device scope once for the batch, so the expert rows the
// producers released are seen; the workgroup then combines the batch.  The
// wait is bounded: past limit_ticks, or once another workgroup has timed out
// (error bit 2), it gives up, sets bit 2, and the batch's tokens that were
// not done are skipped (their y rows keep their contents).
template <int KT, bool MANY>
__global__ __launch_bounds__(64 * kGateWaves) void k_combine_gated(CombineArgs a, int nseg, int gtok) {
    __shared__ uint64_t s_done;
    __shared__ int s_dense;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = uniform_i(threadIdx.x / kWave);
    const int nw = (int)blockDim.x / kWave;
    const int b = (int)blockIdx.x, nb = (int)gridDim.x;
    // batch slot j < gtok holds token b + j * nb (strided: the workgroups in
    // flight cover a compact window of tokens) or b * gtok + j
    auto token_of = [&](int j) {
        return b + j * nb;
    };
    if (w == 0) {
        const int t = token_of(lane);
        const bool mine = lane < gtok && t < a.T;
        uint32_t target = 0;
        if (mine) {
            for (int g = 0; g < slot_groups<MANY, KT>(a.K); ++g) {
                int r[KT];                              // every load issued before the first use
                load_rows<KT>(a.slot_to_row, t, a.K, g * KT, r);
#pragma unroll
                for (int k = 0; k < KT; ++k) target += r[k] >= 0 ? 1u : 0u;
            }
        }
        // rows and tokens of the batch: an average of 4 or more rows per token
        // takes the path that holds stores back
        int rows = (int)target, toks = mine ? 1 : 0;
        for (int d = 1; d < kWave; d <<= 1) {
            rows += __shfl_xor(rows, d, kWave);
            toks += __shfl_xor(toks, d, kWave);
        }
        target *= a.round;
        auto done = [&]() {
            return !mine || target == 0 ||
                   (int32_t)(__hip_atomic_load(a.y_done + t, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT) - target) >= 0;
        };
        uint64_t mask = __ballot(done());
        if (mask != ~0ull) {
            const uint64_t start = wall_clock64();
            while (true) {
                __builtin_amdgcn_s_sleep(8);
                mask = __ballot(done());
                if (mask == ~0ull) break;
                const uint32_t err = (uint32_t)uniform_i((int)__hip_atomic_load(
                    a.error, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
                if ((err & 2u) || wall_clock64() - start > a.limit_ticks) {
                    if (lane == 0) atomicOr(a.error, 2u);
                    break;
                }
            }
        }
        // A dense batch acquires the producers' releases for the whole
        // workgroup (one cache invalidation per batch); a sparse batch reads
        // its few rows with device-scope loads instead, so workgroups do not
        // invalidate the caches the others are reading from.
        const bool dense = rows >= 4 * toks;
        if (dense) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        if (lane == 0) {
            s_done = mask;
            s_dense = dense;
        }
    }
    __syncthreads();
    const uint64_t mask = s_done;
    if (s_dense) gated_items<KT, MANY ? 1 : kGateDefer, MANY, false>(a, nseg, gtok, mask, w, nw, lane);
    else gated_items<KT, 1, MANY, true>(a, nseg, gtok, mask, w, nw, lane);
}

// ----------------------------------------------------- combine backward ---


// Backward of the combine for top_k above 8 (k_combine_bwd_slots serves the
// rest), one wave per token: grad_y[t] is read once per slot group; for each
// unmasked slot the gradient row bf16(fp32(w * g)) is stored and the exact
// bf16 x bf16 products are accumulated in double, per lane in ascending chunk
// order and then across lanes by a fixed butterfly (lane 0's sum is kept),
// then rounded once to float.
template <int KT, bool MANY>
__global__ __launch_bounds__(256) void k_combine_bwd(CombineBwdArgs a) {
    constexpr int U = kBwdChunks;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = uniform_i(threadIdx.x / kWave);
    const int t = (int)blockIdx.x * 4 + w;
    if (t >= a.T) return;
    const int n16 = a.H / 8;
    const u32x4* gy = (const u32x4*)a.grad_y + (int64_t)t * n16;
    const u32x4* eo = (const u32x4*)a.expert_out;
    u32x4* geo = (u32x4*)a.grad_eo;
    const int ngroups = slot_groups<MANY, KT>(a.K);
    for (int gi = 0; gi < ngroups; ++gi) {
        const int k0 = gi * KT;
        int rows[KT];
        float wt[KT];
        double acc[KT];
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            const bool in = k0 + k < a.K;
            rows[k] = in ? a.slot_to_row[t * a.K + k0 + k] : -1;
            wt[k] = in ? a.weights[t * a.K + k0 + k] : 0.0f;
            acc[k] = 0.0;
        }
        for (int c0 = lane; c0 < n16; c0 += kWave * U) {
            u32x4 g[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + u * kWave;
                if (c < n16) g[u] = gy[c];
            }
#pragma unroll
            for (int k = 0; k < KT; ++k) {
                if (rows[k] < 0) continue;
                u32x4 o[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int c = c0 + u * kWave;
                    if (c < n16) o[u] = load_v<true>(eo + (int64_t)rows[k] * n16 + c);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int c = c0 + u * kWave;
                    if (c >= n16) continue;
                    u32x4 q;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float g0 = __uint_as_float(g[u][i] << 16);
                        const float g1 = __uint_as_float(g[u][i] & 0xFFFF0000u);
                        const float o0 = __uint_as_float(o[u][i] << 16);
                        const float o1 = __uint_as_float(o[u][i] & 0xFFFF0000u);
                        q[i] = f32_to_bf16_rne(wt[k] * g0) | (f32_to_bf16_rne(wt[k] * g1) << 16);
                        acc[k] = __builtin_fma((double)g0, (double)o0, acc[k]);
                        acc[k] = __builtin_fma((double)g1, (double)o1, acc[k]);
                    }
                    // plain non-temporal: measured 0.8% faster than device scope here
                    store_row<kStoreNonTemporal>(geo + (int64_t)rows[k] * n16, a.H * 2, c, q);
                }
            }
        }
#pragma unroll
        for (int k = 0; k < KT; ++k) {
            double v = acc[k];
#pragma unroll
            for (int d = kWave / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, kWave);
            if (lane == 0 && k0 + k < a.K) a.grad_w[t * a.K + k0 + k] = rows[k] >= 0 ? (float)v : 0.0f;
        }
    }
}

// Backward of the combine for top_k up to 8: one workgroup per token, wave k
// taking slot k.  The wave walks the slot's row segment by segment, loading
// the next segment of grad_y and of the expert row before it stores the
// current gradient segment (on gfx9 a wait for a load also waits for every
// store issued before it), and keeps the same per-lane fp64 chain in
// ascending chunk order and the same butterfly as k_combine_bwd, so its
// results are identical.  grad_y's segment is read by every wave of the
// workgroup (once from memory, then from the caches).  With one row per wave
// the workgroups in flight write a narrower window of rows than one wave per
// token writing all its rows: prefill 736 against 760 us, the stream shape
// 810 against 854 us, share 32 against 40 us.
template <int KT>
__global__ __launch_bounds__(kWave * kSlotGroup) void k_combine_bwd_slots(CombineBwdArgs a, int nseg) {
    constexpr int U = kBwdChunks;
    const int lane = threadIdx.x & (kWave - 1);
    const int k = uniform_i(threadIdx.x / kWave);
    const int t = (int)blockIdx.x;
    if (k >= a.K) return;
    const int row = a.slot_to_row[t * a.K + k];
    if (row < 0) {
        if (lane == 0) a.grad_w[t * a.K + k] = 0.0f;
        return;
    }
    const int n16 = a.H / 8;
    const float wt = a.weights[t * a.K + k];
    const u32x4* gy = (const u32x4*)a.grad_y + (int64_t)t * n16;
    const u32x4* orow = (const u32x4*)a.expert_out + (int64_t)row * n16;
    u32x4* grow = (u32x4*)a.grad_eo + (int64_t)row * n16;
    double acc = 0.0;
    u32x4 g_n[U], o_n[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = lane + u * kWave;
        if (c < n16) {
            g_n[u] = gy[c];
            o_n[u] = load_v<true>(orow + c);
        }
    }
    for (int seg = 0; seg < nseg; ++seg) {
        const int c0 = seg * (kWave * U) + lane;
        u32x4 g[U], o[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            g[u] = g_n[u];
            o[u] = o_n[u];
        }
        if (seg + 1 < nseg) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + kWave * U + u * kWave;
                if (c < n16) {
                    g_n[u] = gy[c];
                    o_n[u] = load_v<true>(orow + c);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = c0 + u * kWave;
            if (c >= n16) continue;
            u32x4 q;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float g0 = __uint_as_float(g[u][i] << 16);
                const float g1 = __uint_as_float(g[u][i] & 0xFFFF0000u);
                const float o0 = __uint_as_float(o[u][i] << 16);
                const float o1 = __uint_as_float(o[u][i] & 0xFFFF0000u);
                q[i] = f32_to_bf16_rne(wt * g0) | (f32_to_bf16_rne(wt * g1) << 16);
                acc = __builtin_fma((double)g0, (double)o0, acc);
                acc = __builtin_fma((double)g1, (double)o1, acc);
            }
            store_row<kStoreNonTemporal>(grow, a.H * 2, c, q);
        }
    }
    double v = acc;
#pragma unroll
    for (int d = kWave / 2; d > 0; d >>= 1) v += __shfl_xor(v, d, kWave);
    if (lane == 0) a.grad_w[t * a.K + k] = (float)v;
}

// ------------------------------------------- consumer stand-in (tests) ---

__device__ __forceinline__ uint32_t e4m3_to_bf16(uint32_t code, int e) {
    const uint32_t sign = (code & 0x80u) << 8;
    const uint32_t mag = code & 0x7Fu;
    if (mag == 0x7Fu) return sign | 0x7FC0u;
    const int ef = (int)(mag >> 3);
    const uint32_t m = mag & 7u;
    const float v = ef ? __builtin_amdgcn_ldexpf((float)(8u + m), ef - 10 + e)
                       : __builtin_amdgcn_ldexpf((float)m, e - 9);
    return sign | f32_to_bf16_rne(v);
}

// The same value built directly as a bf16 pattern when the code is normal and
// the scaled value is a normal bf16: 1.m * 2^(ef-7+e) has 4 significant bits,
// so it is exact, with biased exponent ef + e + 120.  Everything else takes
// the general path above.
__device__ __forceinline__ uint32_t e4m3_to_bf16_fast(uint32_t code, int e) {
    const uint32_t mag = code & 0x7Fu;
    const uint32_t ef = mag >> 3;
    const uint32_t be = ef + (uint32_t)(e + 120);
    if (ef != 0u && mag != 0x7Fu && be - 1u < 254u)
        return ((code & 0x80u) << 8) | (be << 7) | ((mag & 7u) << 4);
    return e4m3_to_bf16(code, e);
}

// ---------------------------------------------------- FP8 decode helpers ---


// Exact float32 value of an e4m3fn code magnitude (0..0x7E).
__device__ __forceinline__ float e4m3_value_f32(uint32_t mag) {
    const uint32_t ef = mag >> 3, m = mag & 7u;
    return ef ? __uint_as_float(((ef + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
}

// bf16 of value(code) * s in float32 (one rounded product, then RNE); NaN
// codes and NaN products give a quiet NaN with the code's sign.
__device__ __forceinline__ uint32_t e4m3_scaled_to_bf16(uint32_t code, float s) {
    const uint32_t sign = (code & 0x80u) << 8;
    const uint32_t mag = code & 0x7Fu;
    if (mag == 0x7Fu) return sign | 0x7FC0u;
    const float v = e4m3_value_f32(mag);
    const float p = ((code & 0x80u) ? -v : v) * s;
    if ((__float_as_uint(p) & 0x7FFFFFFFu) > 0x7F800000u) return sign | 0x7FC0u;
    return f32_to_bf16_rne(p);
}

// Four codes with a power-of-two scale (a float whose exponent field is the
// UE8M0 byte; 2^-127 is field 0) through gfx950's scaled fp8 -> bf16
// conversion.  Checked on the GPU against the ldexp decode for every code and
// every scale byte: identical, apart from NaN codes, which it turns into
// 0xFFC0 whatever their sign.  Words holding a NaN code therefore take the
// ldexp path, which keeps the code's sign.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void decode_word_pow2(uint32_t word, float scale, int e, uint32_t& lo,
                                                 uint32_t& hi) {
    const uint32_t t = (word & 0x7F7F7F7Fu) ^ 0x7F7F7F7Fu;            // zero byte: a NaN code
    if (((t - 0x01010101u) & ~t & 0x80808080u) == 0u) {
        const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, scale, false);
        const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, scale, true);
        __builtin_memcpy(&lo, &a, 4);
        __builtin_memcpy(&hi, &b, 4);
    } else {
        lo = e4m3_to_bf16(word & 0xFFu, e) | (e4m3_to_bf16((word >> 8) & 0xFFu, e) << 16);
        hi = e4m3_to_bf16((word >> 16) & 0xFFu, e) | (e4m3_to_bf16(word >> 24, e) << 16);
    }
}

// Scales of an FP8 pool in any flavour and layout, and the bf16 decode of one
// 16-code unit of row r, group g, for the tile consumer (the cast back
// inlines the same decode; as a shared call it measured a few percent slower).
struct ScaleView {
    const void* p;
    int32_t kind;               // ScaleKind
    int32_t mn;                 // MN-major [G, ld] (UE8M0 packed 4 per word)
    int64_t ld;
    int32_t ngrp;               // groups per row
};

__device__ __forceinline__ void decode_unit(const ScaleView& sv, int64_t r, int g, const u32x4& q,
                                            u32x4& o0, u32x4& o1) {
    if (sv.kind == kScaleUe8m0) {
        const uint32_t byte =
            sv.mn ? (((const uint32_t*)sv.p)[(int64_t)(g >> 2) * sv.ld + r] >> (8 * (g & 3))) & 0xFFu
                  : ((const uint8_t*)sv.p)[r * sv.ngrp + g];
        const int e = (int)byte - 127;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t word = q[i];
            const uint32_t lo = e4m3_to_bf16_fast(word & 0xFFu, e) |
                                (e4m3_to_bf16_fast((word >> 8) & 0xFFu, e) << 16);
            const uint32_t hi = e4m3_to_bf16_fast((word >> 16) & 0xFFu, e) |
                                (e4m3_to_bf16_fast(word >> 24, e) << 16);
            if (i < 2) { o0[2 * i] = lo; o0[2 * i + 1] = hi; }
            else { o1[2 * (i - 2)] = lo; o1[2 * (i - 2) + 1] = hi; }
        }
    } else {
        const float sc = sv.mn ? ((const float*)sv.p)[(int64_t)g * sv.ld + r]
                               : ((const float*)sv.p)[r * sv.ngrp + g];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t word = q[i];
            const uint32_t lo = e4m3_scaled_to_bf16(word & 0xFFu, sc) |
                                (e4m3_scaled_to_bf16((word >> 8) & 0xFFu, sc) << 16);
            const uint32_t hi = e4m3_scaled_to_bf16((word >> 16) & 0xFFu, sc) |
                                (e4m3_scaled_to_bf16(word >> 24, sc) << 16);
            if (i < 2) { o0[2 * i] = lo; o0[2 * i + 1] = hi; }
            else { o1[2 * (i - 2)] = lo; o1[2 * (i - 2) + 1] = hi; }
        }
    }
}

__global__ __launch_bounds__(256) void k_tile_consume(ConsumeArgs a) {
    __shared__ int s_go;
    const ScaleView sv{a.scales, a.scale_kind, a.scale_mn, a.scale_ld, a.H / 128};
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = uniform_i(tid / kWave);
    const int nt = *a.num_tiles;
    for (int j = (int)blockIdx.x; j < nt; j += (int)gridDim.x) {
        if (tid == 0) {
            int go = 1;
            uint64_t waited = 0;
            const uint64_t start = wall_clock64();
            while ((int32_t)(__hip_atomic_load(&a.tile_ready[j], __ATOMIC_ACQUIRE,
                                               __HIP_MEMORY_SCOPE_AGENT) - a.seq) < 0) {
                waited = 1ull << 63;
                if (wall_clock64() - start > a.limit_ticks) {
                    go = 0;
                    atomicOr(a.error, 2u);
                    break;
                }
                __builtin_amdgcn_s_sleep(8);
            }
            if (a.stamps && go) a.stamps[j] = wall_clock64() | waited;
            s_go = go;
        }
        __syncthreads();
        if (!s_go) return;                    // timed out: give up on the remaining tiles too
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        for (int r = j * a.BM + w; r < (j + 1) * a.BM; r += 4) {
            const int src_tok = a.recv_token[r];
            if (src_tok < 0) continue;
            if (a.fp8) {
                const int nunit = a.H / 16;
                const u32x4* src = (const u32x4*)a.pool + (int64_t)r * nunit;
                u32x4* dst = (u32x4*)a.out + (int64_t)r * (a.H / 8);
                for (int c = lane; c < nunit; c += kWave) {
                    const u32x4 q = src[c];
                    u32x4 o0, o1;
                    decode_unit(sv, r, c >> 3, q, o0, o1);
                    dst[2 * c] = o0;
                    dst[2 * c + 1] = o1;
                }
            } else {
                const int n16 = a.H / 8;
                const int64_t src_row = a.gather ? (int64_t)src_tok : (int64_t)r;
                const u32x4* src = (const u32x4*)a.pool + src_row * n16;
                u32x4* dst = (u32x4*)a.out + (int64_t)r * n16;
                for (int c = lane; c < n16; c += kWave) dst[c] = src[c];
            }
        }
        if (a.y_done) {
            // producer side of the per-token gate: publish the tile's rows at
            // device scope, then count each real row for its token
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (w == 0) {
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                for (int r = j * a.BM + lane; r < (j + 1) * a.BM; r += kWave) {
                    const int tok = a.recv_token[r];
                    if (tok >= 0)
                        __hip_atomic_fetch_add(&a.y_done[tok], 1u, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------ cast back ---

// per_token_cast_back (instagit DeepEP low-latency page, example usage):
// bf16 rows from e4m3fn codes and their per-128-channel scales in any of the
// dispatch's flavours and layouts.  One work item is one wave over up to
// 64 * kCastUnits units of 16 channels of one row: 16 bytes of codes in,
// 32 bytes of bf16 out per unit, the group's scale read once per unit.
// A lane's 32 output bytes are not next to its neighbours', so the wave
// passes each group of 64 decoded units through LDS (its own 2 KB per group)
// and stores them as two 1 KB runs, one 16-byte chunk per lane: every store
// instruction then writes whole 128-byte lines (146048 rows at hidden 7168,
// UE8M0 scales: 588 -> 543 us; float32 scales 680 -> 656 us).  A wave's
// LDS accesses run in order, so between its writes and its reads only the
// compiler has to be kept from reordering them.
__global__ __launch_bounds__(256) void k_cast_back(CastBackArgs a, int nseg) {
    constexpr int U = kCastUnits;
    __shared__ u32x4 s_stage[4][U][2 * kWave];          // per wave and unit group
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int64_t items = a.rows * nseg;
    for (int64_t it = (int64_t)blockIdx.x * 4 + (threadIdx.x / kWave); it < items;
         it += (int64_t)gridDim.x * 4) {
        const int64_t r = it / nseg;
        const int seg = (int)(it - r * nseg);
        const int nunit = a.H / 16;
        const int ngrp = a.H / 128;
        const u32x4* src = (const u32x4*)a.q + r * nunit;
        u32x4* dst = (u32x4*)a.out + r * (a.H / 8);
        u32x4 q[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = seg * (kWave * U) + u * kWave + lane;
            if (c < nunit) q[u] = load_v<true>(src + c);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c0 = seg * (kWave * U) + u * kWave;    // first unit of the group
            if (c0 >= nunit) continue;                       // uniform per wave
            const int c = c0 + lane;
            const bool act = c < nunit;
            const int g = (act ? c : 0) >> 3;                // lanes past the row decode nothing stored
            u32x4 o0, o1;
            // a power-of-two scale goes through the hardware conversion: every
            // UE8M0 byte, and float scales that are exactly 2^e (the flavour's
            // own output; anything else takes the float product)
            uint32_t byte = 0;
            bool pow2 = true;
            float sc = 0.0f;
            if (a.scale_kind == kScaleUe8m0) {
                byte = a.scale_mn ? (((const uint32_t*)a.scales)[(int64_t)(g >> 2) * a.scale_ld + r] >>
                                     (8 * (g & 3))) & 0xFFu
                                  : ((const uint8_t*)a.scales)[r * ngrp + g];
                pow2 = byte != 255u;           // 0xFF is a NaN scale to the hardware
            } else {
                sc = a.scale_mn ? ((const float*)a.scales)[(int64_t)g * a.scale_ld + r]
                                : ((const float*)a.scales)[r * ngrp + g];
                const uint32_t sb = __float_as_uint(sc);
                byte = sb == 0x00400000u ? 0u : sb >> 23;
                pow2 = a.scale_kind == kScalePow2F32 &&
                       (sb == 0x00400000u || ((sb & 0x007FFFFFu) == 0u && byte - 1u < 254u));
            }
            if (pow2) {
                const float hs = __uint_as_float(byte << 23);
                const int e = (int)byte - 127;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    uint32_t lo, hi;
                    decode_word_pow2(q[u][i], hs, e, lo, hi);
                    if (i < 2) { o0[2 * i] = lo; o0[2 * i + 1] = hi; }
                    else { o1[2 * (i - 2)] = lo; o1[2 * (i - 2) + 1] = hi; }
                }
            } else if (a.scale_kind == kScaleUe8m0) {
                // byte 255: 2^128, beyond the hardware's scale range
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t word = q[u][i];
                    const uint32_t lo = e4m3_to_bf16(word & 0xFFu, 128) |
                                        (e4m3_to_bf16((word >> 8) & 0xFFu, 128) << 16);
                    const uint32_t hi = e4m3_to_bf16((word >> 16) & 0xFFu, 128) |
                                        (e4m3_to_bf16(word >> 24, 128) << 16);
                    if (i < 2) { o0[2 * i] = lo; o0[2 * i + 1] = hi; }
                    else { o1[2 * (i - 2)] = lo; o1[2 * (i - 2) + 1] = hi; }
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t word = q[u][i];
                    const uint32_t lo = e4m3_scaled_to_bf16(word & 0xFFu, sc) |
                                        (e4m3_scaled_to_bf16((word >> 8) & 0xFFu, sc) << 16);
                    const uint32_t hi = e4m3_scaled_to_bf16((word >> 16) & 0xFFu, sc) |
                                        (e4m3_scaled_to_bf16(word >> 24, sc) << 16);
                    if (i < 2) { o0[2 * i] = lo; o0[2 * i + 1] = hi; }
                    else { o1[2 * (i - 2)] = lo; o1[2 * (i - 2) + 1] = hi; }
                }
            }
            u32x4* st = s_stage[wv][u];
            st[2 * lane] = o0;                               // unit c0 + lane: chunks 2 lane, 2 lane + 1
            st[2 * lane + 1] = o1;
            // other lanes' writes are read next: keep the compiler from moving
            // the reads above the writes (the hardware runs them in order)
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_wave_barrier();
            const u32x4 r0 = st[lane];
            const u32x4 r1 = st[kWave + lane];
            const int n16 = 2 * nunit;                       // 16-byte chunks per row
            if (2 * c0 + lane < n16) store_row<kStoreNonTemporal>(dst, a.H * 2, 2 * c0 + lane, r0);
            if (2 * c0 + kWave + lane < n16)
                store_row<kStoreNonTemporal>(dst, a.H * 2, 2 * c0 + kWave + lane, r1);
        }
    }
}

// ----------------------------------- layout and dispatch in one launch ---

// For at most kLayoutSlotsPerBlock slots (decode-sized batches): workgroup 0
// runs the whole one-workgroup layout, writing every array the layout writes,
// while every other workgroup builds the slot -> pool row map by itself in
// LDS from topk_idx, with the same code (a slot's row depends only on the
// routing), and then dispatches its share of the items.  One launch and one
// trip through topk_idx instead of a layout kernel the dispatch has to wait
// for.
template <int KT, bool MANY>
__global__ __launch_bounds__(kLayoutThreads) void k_layout_dispatch_bf16(LayoutArgs la, DispatchArgs a, int nseg,
                                                                        int ipb) {
    constexpr int U = kDispatchChunks;
    __shared__ int32_t s2r[kLayoutSlotsPerBlock];
    if (blockIdx.x == 0) {
        layout_rank_body<true, false>(la, 1, 0, 0, nullptr);
        return;
    }
    // the x segment of this wave's first item is loaded before the layout's
    // keys, so that the two memory waits overlap
    const int lane = threadIdx.x & (kWave - 1);
    const int bid = (int)blockIdx.x - 1;
    const int it0 = bid * ipb + uniform_i(threadIdx.x / kWave);
    u32x4 pre[U] = {};
    if (it0 < a.T * nseg) {
        const int t = it0 / nseg, n16 = a.H / 8;
        const int c0 = (it0 - t * nseg) * (kWave * U) + lane;
        const u32x4* src = (const u32x4*)a.x + (int64_t)t * n16;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (c0 + u * kWave < n16) pre[u] = src[c0 + u * kWave];
    }
    layout_rank_body<true, true>(la, 1, 0, 0, s2r);
    __syncthreads();
    dispatch_bf16_body<KT, false, MANY, true>(a, nseg, ipb, bid, s2r, pre);
}

template <int KT, bool F32Q, int U, bool MANY>
__global__ __launch_bounds__(kLayoutThreads) void k_layout_dispatch_fp8(LayoutArgs la, DispatchArgs a, int nseg,
                                                                       int ipb) {
    __shared__ int32_t s2r[kLayoutSlotsPerBlock];
    if (blockIdx.x == 0) {
        layout_rank_body<true, false>(la, 1, 0, 0, nullptr);
        return;
    }
    // the x units of this wave's first item are loaded before the layout's
    // keys, so that the two memory waits overlap (the item as the dispatch
    // body assigns it)
    const int lane = threadIdx.x & (kWave - 1);
    const int bid = (int)blockIdx.x - 1, nblk = (int)gridDim.x - 1;
    const int blk = a.scale_kind != kScaleUe8m0 ? xcd_contiguous_block(bid, nblk) : bid;
    const int it0 = blk * ipb + uniform_i(threadIdx.x / kWave);
    u32x4 lo[U] = {}, hi[U] = {};
    if (it0 < a.T * nseg) {
        const int t = it0 / nseg, nunit = a.H / 16;
        const int u0 = (it0 - t * nseg) * (kWave * U) + lane;
        const u32x4* src = (const u32x4*)a.x + (int64_t)t * (a.H / 8);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = u0 + u * kWave;
            if (c < nunit) {
                lo[u] = src[2 * c];
                hi[u] = src[2 * c + 1];
            }
        }
    }
    layout_rank_body<true, true>(la, 1, 0, 0, s2r);
    __syncthreads();
    dispatch_fp8_body<KT, false, F32Q, U, MANY, true>(a, nseg, ipb, bid, nblk, s2r, lo, hi);
}

// ------------------------------------------------------------- launchers ---

// Items per workgroup: one per wave of 4, or every segment of the streaming chunk's tokens.
inline int items_per_block(int nseg, bool stream) {
    return stream ? kStreamTokens * nseg : 4;
}

template <int KT, bool MANY>
hipError_t dispatch_kt(const DispatchArgs& a, bool fp8, bool stream, hipStream_t st) {
    constexpr int FU = kFp8Units, FS = kFp8StreamUnits;
    const int fu = stream ? FS : FU;
    const int per_seg = fp8 ? kWave * fu * 16 : kWave * kDispatchChunks * 8;  // channels
    const int nseg = (a.H + per_seg - 1) / per_seg;
    const int ipb = items_per_block(nseg, stream);
    const int64_t items = (int64_t)a.T * nseg;
    int grid = (int)((items + ipb - 1) / ipb);
    const size_t lds = 0;
    // streaming: one wave per item of the chunk (at most 16)
    const dim3 block(stream ? kWave * (ipb < 16 ? ipb : 16) : 256);
    if (fp8) {
        const bool f32q = a.scale_kind == kScaleF32;
        if (stream && f32q)
            hipLaunchKernelGGL((k_dispatch_fp8<KT, true, true, FS, MANY>), dim3(grid), block, lds, st, a, nseg, ipb);
        else if (stream)
            hipLaunchKernelGGL((k_dispatch_fp8<KT, true, false, FS, MANY>), dim3(grid), block, lds, st, a, nseg, ipb);
        else if (f32q)
            hipLaunchKernelGGL((k_dispatch_fp8<KT, false, true, FU, MANY>), dim3(grid), block, lds, st, a, nseg, ipb);
        else
            hipLaunchKernelGGL((k_dispatch_fp8<KT, false, false, FU, MANY>), dim3(grid), block, lds, st, a, nseg, ipb);
    } else {
        if (stream) {
            hipLaunchKernelGGL((k_dispatch_bf16<KT, true, MANY>), dim3(grid), block, lds, st, a, nseg, ipb);
        } else if (!MANY && a.density == kDensityDense && dispatch_shape_uses_density(a.T, a.H, a.K)) {
            const int dseg = (a.H / 8 + kWave - 1) / kWave;
            hipLaunchKernelGGL(k_stage_x, dim3(kStageGrid), dim3(256), 0, st, (const u32x4*)a.x,
                               (int64_t)a.T * (a.H / 8));
            hipLaunchKernelGGL((k_dispatch_bf16_dense<KT>), dim3((unsigned)((int64_t)a.T * dseg)), dim3(kWave * KT), 0,
                               st, a, dseg);
        } else {
            hipLaunchKernelGGL((k_dispatch_bf16<KT, false, MANY>), dim3(grid), block, lds, st, a, nseg, ipb);
        }
    }
    return hipGetLastError();
}

template <int KT, bool UNIT, bool GATE, bool MANY>
hipError_t combine_kt(const CombineArgs& a, hipStream_t st) {
    const int per_seg = kWave * kCombineChunks * 8;
    const int nseg = (a.H + per_seg - 1) / per_seg;
    if constexpr (GATE) {
        // Tokens per workgroup: halved from kGateTokens until every wave has
        // at most kGateDefer items, so that a dense batch issues its stores
        // in one batch (prefill's 7 segments per token: 16 -> 8 tokens, 371 ->
        // 355 us; at 3 or 4 segments 16 tokens already fit); then fewer when
        // the batch would not give every compute unit two workgroups.  No
        // more waves than the batch has items.  (Sizes only: a batch's
        // density is decided inside the kernel.)
        int gtok = kGateTokens;
        while (gtok > 1 && gtok * nseg > kGateWaves * kGateDefer) gtok >>= 1;
        while (gtok > 1 && (a.T + gtok - 1) / gtok < 2 * a.num_cu) gtok >>= 1;
        const int gw = gtok * nseg < kGateWaves ? gtok * nseg : kGateWaves;
        const int grid = (a.T + gtok - 1) / gtok;
        hipLaunchKernelGGL((k_combine_gated<KT, MANY>), dim3(grid), dim3(64 * gw), 0, st, a, nseg, gtok);
        return hipGetLastError();
    }
    const int ipb = items_per_block(nseg, false);
    const int64_t items = (int64_t)a.T * nseg;
    const int grid = (int)((items + ipb - 1) / ipb);
    // Launch shape; the kernel and its results are the same in every shape.
    // A resident grid (one wave per item), or sparse routing, runs at full
    // occupancy.  Dense routing (4 or more rows per token) is capped at two
    // 4-wave workgroups per compute unit by unused LDS: with every wave
    // issuing all its row loads at once, that was the fastest shape for it
    // (345 against 375 us at full occupancy, 16384 tokens x top-8), while
    // sparse routing is latency-bound and wants every wave (23 against 38 us).
    // The density is the current layout's (the caller waits for it).
    const bool resident = items <= (int64_t)a.num_cu * kCombineResidentWaves;
    const size_t lds = (resident || a.density == kDensitySparse) ? 0 : kCombineDenseLds;
    hipLaunchKernelGGL((k_combine<KT, UNIT, MANY>), dim3(grid), dim3(256), lds, st, a, nseg, ipb);
    return hipGetLastError();
}

template <bool UNIT, bool GATE>
hipError_t combine_any(const CombineArgs& a, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    if (a.K <= 1) return combine_kt<1, UNIT, GATE, false>(a, stream);
    if (a.K <= 2) return combine_kt<2, UNIT, GATE, false>(a, stream);
    if (a.K <= 4) return combine_kt<4, UNIT, GATE, false>(a, stream);
    if (a.K <= kSlotGroup) return combine_kt<kSlotGroup, UNIT, GATE, false>(a, stream);
    return combine_kt<kSlotGroup, UNIT, GATE, true>(a, stream);
}

template <int KT, bool MANY>
hipError_t combine_bwd_kt(const CombineBwdArgs& a, hipStream_t st) {
    if constexpr (!MANY) {
        const int nseg = (a.H / 8 + kWave * kBwdChunks - 1) / (kWave * kBwdChunks);
        // Dense routing: at most two workgroups per compute unit, capped by
        // unused LDS, so fewer rows are written at once (16384 tokens x
        // top-8, hidden 7168: 734 -> 714 us back to back, 774 -> 759 us with
        // the caches flushed; 32768 x top-8, hidden 4096: 804 -> 794 us).
        // Sparse routing would lose half its speed that way (8192 tokens,
        // one row each on average: 31 -> 64 us) and keeps full occupancy.
        // The results are the same in both shapes.
        const size_t lds = KT == kSlotGroup && a.density == kDensityDense &&
                                   combine_bwd_shape_uses_density(a.T, a.K, a.num_cu)
                               ? kBwdDenseLds : 0;
        hipLaunchKernelGGL((k_combine_bwd_slots<KT>), dim3(a.T), dim3(kWave * KT), lds, st, a, nseg);
    } else {
        const int grid = (a.T + 3) / 4;
        hipLaunchKernelGGL((k_combine_bwd<KT, MANY>), dim3(grid), dim3(256), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_layout(const LayoutArgs& a, hipStream_t stream) {
    const size_t lds_rank = layout_rank_lds(a.E);
    if (a.S <= kLayoutSlotsPerBlock) {
        hipLaunchKernelGGL((k_layout_rank<true>), dim3(1), dim3(kLayoutThreads), lds_rank, stream,
                           a, 1, 0);
        return hipGetLastError();
    }
    const int nb = layout_blocks(a.S);
    hipLaunchKernelGGL(k_layout_count, dim3(nb), dim3(kLayoutThreads), sizeof(int) * (size_t)a.E,
                       stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    int epad = 1;
    while (epad < a.E) epad <<= 1;
    int tpe = kLayoutThreads / epad;
    if (tpe > kWave) tpe = kWave;
    int lg_tpe = 0;
    while ((1 << (lg_tpe + 1)) <= tpe) ++lg_tpe;
    hipLaunchKernelGGL((k_layout_rank<false>), dim3(nb), dim3(kLayoutThreads), lds_rank, stream, a,
                       nb, lg_tpe);
    return hipGetLastError();
}

template <int KT, bool MANY>
hipError_t layout_dispatch_kt(const LayoutArgs& la, const DispatchArgs& a, bool fp8, hipStream_t st) {
    const int per_seg = fp8 ? kWave * kFp8Units * 16 : kWave * kDispatchChunks * 8;  // channels
    const int nseg = (a.H + per_seg - 1) / per_seg;
    const int ipb = kLayoutWaves;                   // one item per wave
    const int64_t items = (int64_t)a.T * nseg;
    const int grid = 1 + (int)((items + ipb - 1) / ipb);
    const size_t lds = layout_rank_lds(la.E);
    if (fp8) {
        if (a.scale_kind == kScaleF32)
            hipLaunchKernelGGL((k_layout_dispatch_fp8<KT, true, kFp8Units, MANY>), dim3(grid), dim3(kLayoutThreads),
                               lds, st, la, a, nseg, ipb);
        else
            hipLaunchKernelGGL((k_layout_dispatch_fp8<KT, false, kFp8Units, MANY>), dim3(grid), dim3(kLayoutThreads),
                               lds, st, la, a, nseg, ipb);
    } else {
        hipLaunchKernelGGL((k_layout_dispatch_bf16<KT, MANY>), dim3(grid), dim3(kLayoutThreads), lds, st, la, a,
                           nseg, ipb);
    }
    return hipGetLastError();
}

hipError_t launch_dispatch(const DispatchArgs& a, bool fp8, bool tile_ready, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    if (a.K <= 1) return dispatch_kt<1, false>(a, fp8, tile_ready, stream);
    if (a.K <= 2) return dispatch_kt<2, false>(a, fp8, tile_ready, stream);
    if (a.K <= 4) return dispatch_kt<4, false>(a, fp8, tile_ready, stream);
    if (a.K <= kSlotGroup) return dispatch_kt<kSlotGroup, false>(a, fp8, tile_ready, stream);
    return dispatch_kt<kSlotGroup, true>(a, fp8, tile_ready, stream);
}

hipError_t launch_layout_dispatch(const LayoutArgs& la, const DispatchArgs& a, bool fp8, hipStream_t stream) {
    if (a.T == 0 || la.S > kLayoutSlotsPerBlock) return hipErrorInvalidValue;
    if (a.K <= 1) return layout_dispatch_kt<1, false>(la, a, fp8, stream);
    if (a.K <= 2) return layout_dispatch_kt<2, false>(la, a, fp8, stream);
    if (a.K <= 4) return layout_dispatch_kt<4, false>(la, a, fp8, stream);
    if (a.K <= kSlotGroup) return layout_dispatch_kt<kSlotGroup, false>(la, a, fp8, stream);
    return layout_dispatch_kt<kSlotGroup, true>(la, a, fp8, stream);
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
    return combine_any<false, false>(a, stream);
}

hipError_t launch_combine_gated(const CombineArgs& a, hipStream_t stream) {
    return combine_any<false, true>(a, stream);
}

hipError_t launch_combine_unit(const CombineArgs& a, hipStream_t stream) {
    return combine_any<true, false>(a, stream);
}

hipError_t launch_combine_bwd(const CombineBwdArgs& a, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    if (a.K <= 1) return combine_bwd_kt<1, false>(a, stream);
    if (a.K <= 2) return combine_bwd_kt<2, false>(a, stream);
    if (a.K <= 4) return combine_bwd_kt<4, false>(a, stream);
    if (a.K <= kSlotGroup) return combine_bwd_kt<kSlotGroup, false>(a, stream);
    return combine_bwd_kt<kSlotGroup, true>(a, stream);
}

hipError_t launch_cast_back(const CastBackArgs& a, hipStream_t stream) {
    if (a.rows == 0) return hipSuccess;
    const int nunit = a.H / 16;
    const int nseg = (nunit + kWave * kCastUnits - 1) / (kWave * kCastUnits);
    const int64_t items = a.rows * nseg;
    int64_t grid = (items + 3) / 4;
    if (grid > (1 << 20)) grid = 1 << 20;          // grid-stride beyond a million workgroups
    // Full occupancy: with whole-line stores the cast back measured fastest
    // with every wave it can get (UE8M0 543 us against 548 / 603 us at six /
    // five workgroups per compute unit).
    hipLaunchKernelGGL(k_cast_back, dim3((uint32_t)grid), dim3(256), 0, stream, a, nseg);
    return hipGetLastError();
}

bool dispatch_shape_uses_density(int T, int H, int K) {
    return T > 0 && K <= kSlotGroup && (int64_t)T * H * 2 >= kDenseDispatchMinBytes;
}

bool combine_bwd_shape_uses_density(int T, int K, int num_cu) {
    // one workgroup of kSlotGroup waves per token; four fit a compute unit
    return T > 0 && K > 4 && K <= kSlotGroup && (int64_t)T > (int64_t)num_cu * 4;
}

bool combine_shape_uses_density(int T, int H, int num_cu) {
    const int per_seg = kWave * kCombineChunks * 8;
    const int64_t items = (int64_t)T * ((H + per_seg - 1) / per_seg);
    return T > 0 && items > (int64_t)num_cu * kCombineResidentWaves;
}

hipError_t launch_consume(const ConsumeArgs& a, int workgroups, hipStream_t stream) {
    hipLaunchKernelGGL(k_tile_consume, dim3(workgroups), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace epk
