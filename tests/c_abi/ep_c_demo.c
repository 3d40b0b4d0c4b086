/*
 * The ep_layout C ABI used from plain C, with no Python and no torch in the
 * process: create a handle, lay out a seeded routing, dispatch bf16 rows into
 * the pool, combine with the pool itself as the expert output (identity
 * experts), and check the results against properties that hold exactly:
 *   - expert_counts equals a host histogram of topk_idx, and num_tiles the
 *     sum of ceil(count / BLOCK_M);
 *   - every unmasked slot has its own pool row inside the used tiles, and that
 *     row holds the token's row of x bit for bit;
 *   - with weight 1/2 on each of a token's two slots, y equals x exactly for a
 *     token with both slots unmasked, x / 2 for one, and +0 for none (the
 *     values of x are normal bf16 numbers, so halving them is exact).
 * Prints one "ok" line and exits 0, or names the first mismatch and exits 1.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ep_layout.h"

#define T 1000
#define K 2
#define E 16
#define BM 32
#define H 256

static int fail(const char* what, long where) {
    printf("c abi demo FAILED: %s (at %ld)\n", what, where);
    return 1;
}

#define HIP_OK(call)                                                        \
    do {                                                                    \
        hipError_t e_ = (call);                                             \
        if (e_ != hipSuccess) {                                             \
            printf("HIP error %d at line %d\n", (int)e_, __LINE__);          \
            return 1;                                                       \
        }                                                                   \
    } while (0)

#define EP_OK_(call)                                                        \
    do {                                                                    \
        ep_status s_ = (call);                                              \
        if (s_ != EP_OK) {                                                  \
            printf("ep error '%s' at line %d\n", ep_status_string(s_), __LINE__); \
            return 1;                                                       \
        }                                                                   \
    } while (0)

static uint32_t lcg(uint32_t* s) {
    *s = *s * 1664525u + 1013904223u;
    return *s >> 8;
}

int main(void) {
    static int32_t idx[T * K];
    static float w[T * K];
    static uint16_t x[T * H], y[T * H];
    uint32_t seed = 12345u;
    int valid[T];
    int32_t hist[E] = {0};

    /* routing: two distinct experts per token, each slot masked with
       probability 1/8; weights 1/2 */
    for (int t = 0; t < T; ++t) {
        const int e0 = (int)(lcg(&seed) % E);
        const int e1 = (e0 + 1 + (int)(lcg(&seed) % (E - 1))) % E;
        idx[t * K] = (lcg(&seed) % 8u) ? e0 : -1;
        idx[t * K + 1] = (lcg(&seed) % 8u) ? e1 : -1;
        valid[t] = 0;
        for (int k = 0; k < K; ++k) {
            w[t * K + k] = 0.5f;
            if (idx[t * K + k] >= 0) {
                hist[idx[t * K + k]] += 1;
                valid[t] += 1;
            }
        }
    }
    /* x: normal bf16 values +-(1 + m/128) * 2^e, e in [-10, 0] */
    for (int i = 0; i < T * H; ++i) {
        const uint32_t r = lcg(&seed);
        const uint32_t sign = r & 1u, m = (r >> 1) & 127u, e = (r >> 8) % 11u;
        x[i] = (uint16_t)((sign << 15) | ((127u - e) << 7) | m);
    }

    ep_config cfg = {T, K, E, BM};
    ep_handle* h = NULL;
    EP_OK_(ep_handle_create(&cfg, &h));
    const int64_t cap = ep_pool_capacity_rows(h);
    if (cap != (int64_t)T * K + (int64_t)E * (BM - 1)) return fail("capacity rows", (long)cap);

    int32_t *d_idx, *d_s2r;
    float* d_w;
    void *d_x, *d_pool, *d_y;
    HIP_OK(hipMalloc((void**)&d_idx, sizeof idx));
    HIP_OK(hipMalloc((void**)&d_w, sizeof w));
    HIP_OK(hipMalloc((void**)&d_s2r, sizeof idx));
    HIP_OK(hipMalloc(&d_x, sizeof x));
    HIP_OK(hipMalloc(&d_y, sizeof y));
    HIP_OK(hipMalloc(&d_pool, (size_t)cap * H * 2));
    HIP_OK(hipMemcpy(d_idx, idx, sizeof idx, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_w, w, sizeof w, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_x, x, sizeof x, hipMemcpyHostToDevice));
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));

    uint32_t epoch = 0, seq = 0;
    EP_OK_(ep_layout(h, d_idx, d_w, T, stream, &epoch));
    EP_OK_(ep_dispatch(h, d_x, H, d_pool, NULL, 0u, stream, &seq));
    EP_OK_(ep_combine(h, epoch, d_pool, H, d_y, stream));
    if (ep_array_bytes(h, EP_ARRAY_SLOT_TO_POOL_ROW) != (int64_t)sizeof idx)
        return fail("slot_to_pool_row size", (long)ep_array_bytes(h, EP_ARRAY_SLOT_TO_POOL_ROW));
    EP_OK_(ep_copy_array(h, EP_ARRAY_SLOT_TO_POOL_ROW, d_s2r, (int64_t)sizeof idx, stream));
    int32_t counts[E], num_tiles = 0;
    EP_OK_(ep_counts_to_host(h, counts, &num_tiles, stream));      /* blocking */
    EP_OK_(ep_handle_sync_status(h, stream));                      /* blocking */

    static int32_t s2r[T * K];
    uint16_t* pool = (uint16_t*)malloc((size_t)cap * H * 2);
    char* used = (char*)calloc((size_t)cap, 1);
    if (!pool || !used) return fail("host allocation", 0);
    HIP_OK(hipMemcpy(s2r, d_s2r, sizeof s2r, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(pool, d_pool, (size_t)cap * H * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(y, d_y, sizeof y, hipMemcpyDeviceToHost));

    int tiles = 0;
    for (int e = 0; e < E; ++e) {
        if (counts[e] != hist[e]) return fail("expert_counts", e);
        tiles += (hist[e] + BM - 1) / BM;
    }
    if (num_tiles != tiles) return fail("num_tiles", num_tiles);
    for (int s = 0; s < T * K; ++s) {
        const int t = s / K, r = s2r[s];
        if (idx[s] < 0) {
            if (r != -1) return fail("masked slot has a row", s);
            continue;
        }
        if (r < 0 || r >= num_tiles * BM) return fail("pool row outside the used tiles", s);
        if (used[r]) return fail("pool row given to two slots", s);
        used[r] = 1;
        if (memcmp(pool + (size_t)r * H, x + (size_t)t * H, H * 2) != 0) return fail("pool row != x row", s);
    }
    for (int t = 0; t < T; ++t) {
        for (int c = 0; c < H; ++c) {
            const uint16_t xv = x[t * H + c];
            /* halving a normal bf16 value: exponent field minus one */
            const uint16_t want = valid[t] == 2 ? xv : valid[t] == 1 ? (uint16_t)(xv - (1u << 7)) : 0;
            if (y[t * H + c] != want) return fail("combine output", (long)t * H + c);
        }
    }
    int n_two = 0, n_one = 0, n_none = 0;
    for (int t = 0; t < T; ++t) {
        n_two += valid[t] == 2;
        n_one += valid[t] == 1;
        n_none += valid[t] == 0;
    }
    printf("c abi demo ok: %d tokens (%d with both slots, %d with one, %d with none), %d tiles, epoch %u, seq %u\n",
           T, n_two, n_one, n_none, num_tiles, epoch, seq);

    free(pool);
    free(used);
    HIP_OK(hipStreamDestroy(stream));
    HIP_OK(hipFree(d_idx));
    HIP_OK(hipFree(d_w));
    HIP_OK(hipFree(d_s2r));
    HIP_OK(hipFree(d_x));
    HIP_OK(hipFree(d_y));
    HIP_OK(hipFree(d_pool));
    EP_OK_(ep_handle_destroy(h));
    return 0;
}
