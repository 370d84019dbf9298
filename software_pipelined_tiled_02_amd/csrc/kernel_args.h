// kernel_args.h -- the by-value argument block of every GEMM kernel, and
// the registry entry the host uses to find a kernel instance.
#ifndef PIPEGEMM_KERNEL_ARGS_H
#define PIPEGEMM_KERNEL_ARGS_H

#include <stdint.h>

namespace pg {

// Split-K workspace: a fixed area of uint32 arrival counters, one per C tile
// (so a workspace reused for another shape finds its counters where the
// last call left them: zero), then the partial tiles.
constexpr int kSplitkCounters = 16384;
constexpr int64_t kSplitkCounterBytes = (int64_t)kSplitkCounters * 4;

struct GemmArgs {
    const void* A;      // row-major M x K
    const void* B;      // row-major K x N (RR) or column-major K x N (RC)
    void* C;            // row-major M x N
    int64_t lda, ldb, ldc;  // in elements
    int32_t M, N, K;
    int32_t tiles_m, tiles_n;
    int32_t splits;     // K splits per C tile (1: none)
    int32_t sk_tiles;   // the last sk_tiles tiles are shared out stream-K over the grid (0: none)
    void* ws;           // splits > 1 or sk_tiles > 0: per-tile arrival counters, then the partial tiles
};

struct KernelEntry {
    int dtype, layout, tile, stages, variant;
    const void* func;   // __global__ function, launched with hipLaunchKernel
};

// Instances compiled into each per-dtype translation unit.
const KernelEntry* kernels_i8(int* count);
const KernelEntry* kernels_f16(int* count);
const KernelEntry* kernels_bf16(int* count);
const KernelEntry* kernels_f32(int* count);

}  // namespace pg

#endif
