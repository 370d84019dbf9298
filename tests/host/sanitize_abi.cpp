// Runs the library's host code (csrc/abi.hip) under AddressSanitizer and
// UndefinedBehaviorSanitizer: gemm_query / gemm_query_splitk over a grid of
// shapes, dtypes, layouts, tiles, stages, variants, leading dimensions,
// pointer alignments and split counts, plus gemm_status_string and the NULL
// handle paths.  No HIP call is made (the query is pure host code); the
// kernel tables are stubbed out, since no launch happens.  Checks that every
// accepted configuration is self-consistent.  Exit status 0 on success.
#include <cstdint>
#include <cstdio>

#include "kernel_args.h"
#include "pipegemm.h"

namespace pg {
const KernelEntry* kernels_i8(int* n) { *n = 0; return nullptr; }
const KernelEntry* kernels_f16(int* n) { *n = 0; return nullptr; }
const KernelEntry* kernels_bf16(int* n) { *n = 0; return nullptr; }
const KernelEntry* kernels_f32(int* n) { *n = 0; return nullptr; }
}  // namespace pg

int main() {
    static const int64_t dims[] = {0, 1, 31, 64, 257, 1000, 4096, 8200};
    int ok = 0, fails = 0;
    for (int64_t M : dims)
        for (int64_t N : dims)
            for (int64_t K : dims)
                for (int dt = 0; dt < 4; ++dt)
                    for (int lay = 0; lay < 2; ++lay)
                        for (int tile = GEMM_TILE_AUTO; tile <= GEMM_TILE_256x256_W8; ++tile)
                            for (int st = 0; st <= 5; st += (st == 0 ? 1 : 2))
                                for (int var = 0; var < 2; ++var)
                                    for (int splits : {1, 0, 3}) {
                                        const int64_t ldb = (lay == GEMM_LAYOUT_RR ? N : K) + (K % 3);
                                        const uintptr_t base = (K % 2) ? 0x10001u : 0x10000u;
                                        gemm_config_info_t in;
                                        const int rc = gemm_query_splitk(M, N, K, dt, lay, st, var, tile, splits,
                                                                         (const void*)base, K + (M % 2),
                                                                         (const void*)(base + 0x100000), ldb,
                                                                         (const void*)0x40000000u, N + 4 - N % 4, &in);
                                        if (rc != GEMM_OK) continue;
                                        ++ok;
                                        const bool sane = in.splits >= 1 && in.grid >= 0 && in.threads > 0 &&
                                                          in.block_k > 0 && in.lds_bytes <= 160 * 1024 &&
                                                          (in.splits == 1) == (in.workspace_bytes == 0) &&
                                                          (M == 0 || N == 0 || in.grid > 0);
                                        if (!sane) {
                                            ++fails;
                                            std::printf("inconsistent plan %ld %ld %ld dt %d lay %d tile %d S %d v %d p %d\n",
                                                        (long)M, (long)N, (long)K, dt, lay, tile, st, var, splits);
                                        }
                                    }
    for (int s = -2; s < 8; ++s)
        if (gemm_status_string(s) == nullptr) ++fails;
    if (gemm_destroy(nullptr) != GEMM_OK) ++fails;
    if (gemm_set_tile(nullptr, 0) != GEMM_ERR_INVALID_ARG) ++fails;
    if (gemm_query(1, 1, 1, 0, 0, 1, 0, GEMM_TILE_AUTO, nullptr, 1, nullptr, 1, nullptr, 1, nullptr) !=
        GEMM_ERR_INVALID_ARG)
        ++fails;
    std::printf(fails ? "FAIL (%d)\n" : "host ABI under ASan/UBSan: OK (%d accepted configurations)\n",
                fails ? fails : ok);
    return fails ? 1 : 0;
}
