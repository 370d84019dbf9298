// Layout-RR direct-to-LDS kernel instances whose assembly the CPU test
// tests/test_rr_asm_waits.py reads: their transposing B-fragment reads are
// inline assembly the compiler does not track, so the kernel waits for them
// itself.  One instance per read schedule: 16x16 blocks in the split 3-stage
// ring and in the 2-stage ring, 32x32 blocks at 4 stages (half K-tile), the
// 128x128 tile, and the 32x64 tile with two k groups.
#include "gemm_kernel.h"

namespace pg {
template __global__ void pipegemm_kernel<DT_F16, LAYOUT_RR, TILE_L, 3, VAR_DIRECT>(GemmArgs);
template __global__ void pipegemm_kernel<DT_I8, LAYOUT_RR, TILE_L, 2, VAR_DIRECT>(GemmArgs);
template __global__ void pipegemm_kernel<DT_BF16, LAYOUT_RR, TILE_L, 4, VAR_DIRECT>(GemmArgs);
template __global__ void pipegemm_kernel<DT_F16, LAYOUT_RR, TILE_M, 2, VAR_DIRECT>(GemmArgs);
template __global__ void pipegemm_kernel<DT_I8, LAYOUT_RR, TILE_T, 3, VAR_DIRECT>(GemmArgs);
}  // namespace pg
