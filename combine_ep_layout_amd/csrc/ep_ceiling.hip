// Bandwidth probes for the roofline's context (libep_ceiling.so, loaded only
// by the benchmark's ceiling leg; nothing on the dispatch/combine path uses
// it).  Each row of `row_bytes` bytes is moved in 16-byte chunks by 1, 2 or
// 4 waves of a 256-thread workgroup, or in 1 KB pieces by one wave each (one
// access per lane), rows taken from a list, so the same kernel measures
// sequential streams (rows 0, 1, 2, ...) and the pool's scattered-row pattern
// (rows in the order dispatch writes them, or combine reads them).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kAuxNonTemporal = 2;
constexpr int kAuxDevice = 16;

enum Op : int {
    kWriteNonTemporal = 0,        // dst[rows[i]] = pattern, non-temporal stores
    kWriteDeviceNonTemporal = 1,  // the same with device-scope non-temporal buffer stores
    kRead = 2,                    // fold src[rows[i]] into a word that is almost never stored
    kCopy = 3,                    // dst[rows[i]] = src[i] (sequential read, listed-row write)
    kWritePlain = 4,              // dst[rows[i]] = pattern, plain stores
    kWriteFlat = 5,               // the first n_rows rows of dst as one flat array, each
                                  // thread striding over it by the grid: non-temporal stores
    kWriteFlatPlain = 6,          // the same with plain stores
};

__global__ void __launch_bounds__(kThreads) k_rows(int op, int waves_per_row, u32x4* dst,
                                                   const u32x4* src, int64_t n_dst_rows, int n16,
                                                   const int32_t* rows, int64_t n_rows, uint32_t* sink) {
    if (op == kWriteFlat || op == kWriteFlatPlain) {
        const int64_t total = n_rows * n16, step = (int64_t)gridDim.x * kThreads;
        const u32x4 v = {1u, 2u, 0x3F803F80u, 0x3F803F80u};
        for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < total; c += step) {
            if (op == kWriteFlat) __builtin_nontemporal_store(v, dst + c);
            else dst[c] = v;
        }
        return;
    }
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    int64_t i;
    int first, stride;
    if (waves_per_row == 0) {               // one wave per 1 KB piece of a row
        const int pieces = (n16 + 63) / 64;
        const int64_t wv = (int64_t)blockIdx.x * (kThreads / 64) + wave;
        i = wv / pieces;
        first = (int)(wv - i * pieces) * 64 + lane;
        stride = n16;                       // one chunk per lane
    } else {
        i = (int64_t)blockIdx.x * (kThreads / 64 / waves_per_row) + wave / waves_per_row;
        first = (wave % waves_per_row) * 64 + lane;
        stride = waves_per_row * 64;
    }
    if (i >= n_rows) return;
    const int64_t r = rows[i];
    if (r < 0 || r >= n_dst_rows) return;
    if (op == kRead) {
        const u32x4* row = src + r * n16;
        u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll 4
        for (int c = first; c < n16; c += stride) acc ^= __builtin_nontemporal_load(row + c);
        // stores only if the row's chunks fold to this constant (the rows are
        // filled with a constant pattern that never does); keeps the loads
        if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) sink[i] = 1u;
        return;
    }
    u32x4* row = dst + r * n16;
    if (op == kCopy) {
        const u32x4* from = src + i * n16;
#pragma unroll 4
        for (int c = first; c < n16; c += stride)
            __builtin_nontemporal_store(__builtin_nontemporal_load(from + c), row + c);
        return;
    }
    const u32x4 v = {(uint32_t)r, (uint32_t)i, 0x3F803F80u, 0x3F803F80u};
    if (op == kWriteNonTemporal) {
        for (int c = first; c < n16; c += stride) __builtin_nontemporal_store(v, row + c);
    } else if (op == kWritePlain) {
        for (int c = first; c < n16; c += stride) row[c] = v;
    } else {
        __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(row, (short)0, n16 * 16, 0x00020000);
        for (int c = first; c < n16; c += stride)
            __builtin_amdgcn_raw_buffer_store_b128(v, rs, c * 16, 0, kAuxDevice | kAuxNonTemporal);
    }
}

}  // namespace

// Runs one probe over n_rows listed rows of row_bytes bytes.  The listed
// row numbers index dst (n_dst_rows rows), or src for kRead (then src holds
// n_dst_rows rows and dst is unused); for kCopy src holds n_rows rows, read
// in order.  row_bytes is a multiple of 16 and at most 2^30, pointers are
// 16-byte aligned, sink holds n_rows words for kRead, waves_per_row is 1, 2
// or 4, or 0 for one wave per 1 KB piece (the flat writes ignore it and the
// list's contents, and need n_rows <= n_dst_rows).  Listed rows outside [0, n_dst_rows) are skipped.
// Returns 0, -1 for an invalid argument, or the HIP error code.
extern "C" int ep_ceiling_rows(int op, int waves_per_row, void* dst, const void* src, int64_t n_dst_rows, int64_t row_bytes,
                               const int32_t* rows, int64_t n_rows, uint32_t* sink, hipStream_t stream) {
    if (op < kWriteNonTemporal || op > kWriteFlatPlain || row_bytes <= 0 || row_bytes % 16 || row_bytes > (1 << 30) ||
        n_rows < 0 || n_rows > INT32_MAX || n_dst_rows < 0 || !rows ||
        (waves_per_row != 0 && waves_per_row != 1 && waves_per_row != 2 && waves_per_row != 4))
        return -1;
    if (((uintptr_t)dst | (uintptr_t)src) & 15u) return -1;
    if ((op != kRead && !dst) || ((op == kRead || op == kCopy) && !src) || (op == kRead && !sink))
        return -1;
    if ((op == kWriteFlat || op == kWriteFlatPlain) && n_rows > n_dst_rows) return -1;
    if (n_rows == 0) return 0;
    const int64_t n16 = row_bytes / 16;
    const int64_t waves = waves_per_row == 0 ? n_rows * ((n16 + 63) / 64) : 0;
    if (waves_per_row == 0 && (waves + 3) / 4 > INT32_MAX) return -1;
    const int64_t rows_per_block = waves_per_row == 0 ? 1 : kThreads / 64 / waves_per_row;
    const unsigned blocks = waves_per_row == 0 ? (unsigned)((waves + 3) / 4)
                                               : (unsigned)((n_rows + rows_per_block - 1) / rows_per_block);
    hipLaunchKernelGGL(k_rows, dim3(blocks), dim3(kThreads), 0, stream, op, waves_per_row, (u32x4*)dst,
                       (const u32x4*)src, n_dst_rows, (int)(row_bytes / 16), rows, n_rows, sink);
    return (int)hipGetLastError();
}
