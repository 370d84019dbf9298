// abi.hip -- the C ABI declared in include/pipegemm.h: argument checks,
// configuration choice (tile class, K-tile, LDS ring, staging sets) and the
// kernel launch.  Host code only; the kernels live in kernels_*.hip.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "pipegemm.h"
#include "kernel_args.h"
#include "tile_layout.h"

struct gemm_handle_s {
    int device;
    int num_cus;
    int tile_override;  // GEMM_TILE_AUTO or a class
    void* scratch;      // this device's address of `scratch` (below)
};

// The split-K workspace of gemm_run_splitk_noalloc: one static array per
// device, for callers that cannot allocate device memory.  In host code its
// name is a host-side stand-in, not a device address: kernels get the
// address hipGetSymbolAddress returns for the device (scratch_setup).  Its
// first kSplitkCounterBytes are the arrival counters, cleared once per
// device at set-up; every completed split-K call leaves them zero again.
static __device__ __align__(256) uint8_t scratch[GEMM_NOALLOC_SCRATCH_BYTES];
static_assert(GEMM_NOALLOC_SCRATCH_BYTES > pg::kSplitkCounterBytes, "scratch holds the counters");

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kDefaultCus = 256;  // MI355X; used when no device is at hand

struct Plan {
    gemm_config_info_t info;
    int tile;
    int kernel_variant;   // pg::Variant of the instance launched
    int64_t tiles_m, tiles_n;
};

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int64_t kMaxSplits = 64;
constexpr int64_t kAutoSplits = 8;

// Split-K workspace: the fixed counter area, then every split's BM x BN
// tile of 4-byte accumulator words.
int64_t splitk_workspace(int64_t tiles, int64_t splits, const pg::TileShape& ts) {
    return pg::kSplitkCounterBytes + tiles * splits * ts.bm * ts.bn * 4;
}

bool instance_exists(int layout, int tile) {
    // both layouts are built at every tile class
    return (layout == pg::LAYOUT_RC || layout == pg::LAYOUT_RR) && tile >= 0 && tile < pg::TILE_COUNT;
}

// Every check of the ABI, then the configuration.  No HIP call.
// sk_grid: -1 for a call without stream-K; otherwise the stream-K grid (0:
// one workgroup per CU).
int plan_call(int64_t M, int64_t N, int64_t K, int dtype, int layout, int stages, int variant,
              int tile, int splits, int sk_grid, const void* A, int64_t lda, const void* B, int64_t ldb,
              const void* C, int64_t ldc, int num_cus, bool query, Plan* plan) {
    if (dtype < GEMM_I8 || dtype > GEMM_F32) return GEMM_ERR_INVALID_ARG;
    if (layout != GEMM_LAYOUT_RR && layout != GEMM_LAYOUT_RC) return GEMM_ERR_INVALID_ARG;
    if (variant != GEMM_VARIANT_REG && variant != GEMM_VARIANT_DIRECT) return GEMM_ERR_INVALID_ARG;
    if (stages < 1 || stages > pg::kMaxStages) return GEMM_ERR_INVALID_ARG;
    if (tile < GEMM_TILE_AUTO || tile >= pg::TILE_COUNT) return GEMM_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || K < 0) return GEMM_ERR_INVALID_ARG;
    if (splits < 0 || sk_grid < -1 || (sk_grid >= 0 && splits > 1)) return GEMM_ERR_INVALID_ARG;

    const bool has_c = M > 0 && N > 0;
    const bool reads_a = M > 0 && K > 0 && N > 0;
    const bool reads_b = N > 0 && K > 0 && M > 0;
    // A query may leave pointers NULL: then only their leading dimensions are checked.
    if (reads_a && ((A == nullptr && !query) || lda < K)) return GEMM_ERR_INVALID_ARG;
    if (reads_b && ((B == nullptr && !query) || ldb < (layout == GEMM_LAYOUT_RR ? N : K)))
        return GEMM_ERR_INVALID_ARG;
    if (has_c && ((C == nullptr && !query) || ldc < N)) return GEMM_ERR_INVALID_ARG;
    if (lda < 0 || ldb < 0 || ldc < 0) return GEMM_ERR_INVALID_ARG;

    const int sz = pg::in_size(dtype), epc = pg::epc(dtype);
    // Operands: element-aligned always; 16-byte aligned rows (base, ld and K
    // whole 16-byte chunks) for the direct-to-LDS variant, whose loads write
    // LDS in whole 16-byte chunks.  The register-staged variant takes any K
    // and leading dimension.
    if (reads_a && (uintptr_t)A % sz != 0) return GEMM_ERR_ALIGNMENT;
    if (reads_b && (uintptr_t)B % sz != 0) return GEMM_ERR_ALIGNMENT;
    const bool rows16 = (!reads_a || (aligned16(A) && (lda * sz) % 16 == 0)) &&
                        (!reads_b || (aligned16(B) && (ldb * sz) % 16 == 0)) && K % epc == 0;
    if (!rows16 && variant == GEMM_VARIANT_DIRECT) return GEMM_ERR_ALIGNMENT;
    if (has_c && (!aligned16(C) || ldc % 4 != 0)) return GEMM_ERR_ALIGNMENT;
    if (layout == GEMM_LAYOUT_RR && N % epc != 0) return GEMM_ERR_ALIGNMENT;
    if (M > INT_MAX || N > INT_MAX || K > INT_MAX) return GEMM_ERR_UNSUPPORTED;

    // Tile class: the largest whose grid still gives every CU a workgroup.
    // (The 8-wave 256x256 tile is only taken on request: with operands
    // streamed from HBM it measured level with the 4-wave one on 8192^2,
    // behind it on 4096^3, and ahead only with cache-resident operands.)
    int tc = tile;
    if (tc == GEMM_TILE_AUTO) {
        tc = pg::TILE_T;
        const int order[3] = {pg::TILE_L, pg::TILE_M, pg::TILE_T};
        for (int i = 0; i < 3; ++i) {
            const pg::TileShape ts = pg::tile_shape(order[i]);
            if (!instance_exists(layout, order[i])) continue;
            if (ceil_div(M, ts.bm) * ceil_div(N, ts.bn) >= num_cus) { tc = order[i]; break; }
        }
    }
    if (!instance_exists(layout, tc)) return GEMM_ERR_UNSUPPORTED;
    if (!pg::instance_fits(dtype, tc, stages, variant)) return GEMM_ERR_UNSUPPORTED;

    const pg::TileShape ts = pg::tile_shape(tc);
    const int bk = pg::block_k(dtype, tc, stages, variant);
    // 32-bit buffer offsets: one workgroup's operand rows (and, for a
    // row-major B, the whole K extent) must stay below 2^31 bytes.
    const int64_t lim = (int64_t)1 << 31;
    if ((int64_t)ts.bm * lda * sz >= lim || K * (int64_t)sz >= lim) return GEMM_ERR_UNSUPPORTED;
    if (layout == GEMM_LAYOUT_RC && (int64_t)ts.bn * ldb * sz >= lim) return GEMM_ERR_UNSUPPORTED;
    if (layout == GEMM_LAYOUT_RR && (K + bk) * ldb * (int64_t)sz >= lim) return GEMM_ERR_UNSUPPORTED;

    const int64_t tm = has_c ? ceil_div(M, ts.bm) : 0, tn = has_c ? ceil_div(N, ts.bn) : 0;
    if (tm * tn > INT_MAX) return GEMM_ERR_UNSUPPORTED;

    gemm_config_info_t& in = plan->info;
    memset(&in, 0, sizeof in);
    in.tile = tc;
    in.block_m = ts.bm;
    in.block_n = ts.bn;
    in.block_k = bk;
    in.waves_m = ts.wm;
    in.waves_n = ts.wn;
    in.waves_k = ts.wk;
    in.threads = pg::threads(tc);
    in.lds_slots = pg::lds_slots(variant, stages);
    in.reg_sets = pg::reg_sets(variant, stages);
    in.tiles_in_flight = pg::tiles_in_flight(variant, stages);
    in.lds_bytes = pg::lds_bytes(dtype, tc, stages, variant);
    in.loads_per_tile = pg::loads_a(dtype, tc, stages, variant) + pg::loads_b(dtype, tc, stages, variant);
    in.mfma_block = pg::mfma_block16(dtype, layout, tc, stages, variant) ? 16 : 32;
    // The 256x256 tiles run one workgroup per CU (their LDS ring and
    // registers allow no second one); with more tiles than CUs, a grid of
    // one workgroup per CU loops over the tiles, so that one tile's C stores
    // overlap the next tile's first loads.
    in.c_tiles = (int32_t)(tm * tn);
    // Split K: whole units of the class's largest K-tile per split, at most
    // kMaxSplits.  0 asks for the split that gives every CU a workgroup, at
    // most kAutoSplits and at least two units per split: the split that
    // arrives last reads every partial tile, so the final sum grows with the
    // split count (measured on 1024 x 1024 x 8192 bf16 with 256 x 256
    // tiles: 177 us at 8 splits, 320 us at 16, against 45 us for 128 x 128
    // tiles at 4).
    const int64_t units = K / pg::block_k(dtype, tc, 1, variant);
    int64_t P = splits;
    if (P == 0) {
        P = (tm * tn > 0 && tm * tn < num_cus) ? ceil_div(num_cus, tm * tn) : 1;
        if (P > kAutoSplits) P = kAutoSplits;
        if (P > units / 2) P = units / 2;
    }
    if (P > units) P = units;
    if (P > kMaxSplits) P = kMaxSplits;
    if (P < 1) P = 1;
    if (sk_grid >= 0) P = 1;
    if (P > 1 && tm * tn > pg::kSplitkCounters) return GEMM_ERR_UNSUPPORTED;
    in.splits = (int32_t)P;
    in.workspace_bytes = P > 1 ? splitk_workspace(tm * tn, P, ts) : 0;
    const int64_t work = tm * tn * P;
    if (work > INT_MAX) return GEMM_ERR_UNSUPPORTED;
    in.grid = ((tc == pg::TILE_L || tc == pg::TILE_W) && work > num_cus && num_cus % 8 == 0) ? num_cus : work;
    if (sk_grid >= 0 && tm * tn > 0) {
        // Stream-K: G workgroups; every full round of G tiles but the last
        // is data-parallel, and the rest (between one and two rounds' worth)
        // is shared out in units over all G workgroups, so each gets the
        // same number of units, give or take one.
        int64_t G = sk_grid > 0 ? sk_grid : num_cus;
        const int64_t U = units > 0 ? units : 1, full = tm * tn / G;
        const int64_t dp = full >= 2 ? (full - 1) * G : 0, sk = tm * tn - dp;
        if (G > sk * U) G = sk * U;
        if (tm * tn > pg::kSplitkCounters) return GEMM_ERR_UNSUPPORTED;
        if (2 * G * (int64_t)ts.bm * ts.bn * 4 >= ((int64_t)1 << 31)) return GEMM_ERR_UNSUPPORTED;
        in.sk_tiles = (int32_t)sk;
        in.grid = G;
        in.workspace_bytes = pg::kSplitkCounterBytes + 2 * G * (int64_t)ts.bm * ts.bn * 4;
    }
    in.k_tiles = ceil_div(K, bk);
    in.k_tail = (int32_t)(K % bk);
    plan->tile = tc;
    // A K that is not a multiple of 16 bytes reads its partial chunk with
    // exact-size loads, in instances of their own; the other instances are
    // not touched by it.
    plan->kernel_variant = (variant == GEMM_VARIANT_REG && K % epc != 0) ? (int)pg::VAR_REG_KTAIL : variant;
    plan->tiles_m = tm;
    plan->tiles_n = tn;
    return GEMM_OK;
}

struct Registry {
    const void* fn[4][2][pg::TILE_COUNT][pg::kMaxStages + 1][3];
    Registry() {
        memset(fn, 0, sizeof fn);
        const pg::KernelEntry* (*parts[4])(int*) = {pg::kernels_i8, pg::kernels_f16, pg::kernels_bf16,
                                                    pg::kernels_f32};
        for (int p = 0; p < 4; ++p) {
            int n = 0;
            const pg::KernelEntry* t = parts[p](&n);
            for (int i = 0; i < n; ++i)
                fn[t[i].dtype][t[i].layout][t[i].tile][t[i].stages][t[i].variant] = t[i].func;
        }
    }
};

const Registry& registry() {
    static const Registry r;
    return r;
}

int hip_fail(hipError_t e) {
    g_last_hip_error = (int)e;
    return GEMM_ERR_HIP;
}

// Writes zeros over n 32-bit words (clears the scratch counters with a
// kernel rather than a memset).
__global__ void zero_words(uint32_t* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];   // per device: address of `scratch`, once set up

// Once per device, with that device current: find this device's copy of
// `scratch` and clear its arrival counters.  *out receives the address.
hipError_t scratch_setup(int device, void** out) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (device >= kMaxDevices) return hipErrorInvalidDevice;
    if (g_scratch[device] != nullptr) {
        *out = g_scratch[device];
        return hipSuccess;
    }
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e == hipSuccess) {
        constexpr int words = (int)(pg::kSplitkCounterBytes / 4);
        hipLaunchKernelGGL(zero_words, dim3((words + 255) / 256), dim3(256), 0, nullptr, (uint32_t*)p, words);
        e = hipGetLastError();
        if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
    }
    if (cur != device) {
        const hipError_t r = hipSetDevice(cur);
        if (e == hipSuccess) e = r;
    }
    if (e == hipSuccess) {
        g_scratch[device] = p;
        *out = p;
    }
    return e;
}

// Launch the instance `plan` chose on the handle's device (ws: the split-K
// workspace when the plan has more than one split).
int launch(gemm_handle_t h, const Plan& plan, int64_t M, int64_t N, int64_t K, int dtype, int layout,
           int stages, const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, void* ws,
           void* stream) {
    if (plan.info.grid == 0) return GEMM_OK;
    const void* fn = registry().fn[dtype][layout][plan.tile][stages][plan.kernel_variant];
    if (fn == nullptr) return GEMM_ERR_UNSUPPORTED;

    pg::GemmArgs args;
    args.A = A;
    args.B = B;
    args.C = C;
    args.lda = lda;
    args.ldb = ldb;
    args.ldc = ldc;
    args.M = (int32_t)M;
    args.N = (int32_t)N;
    args.K = (int32_t)K;
    args.tiles_m = (int32_t)plan.tiles_m;
    args.tiles_n = (int32_t)plan.tiles_n;
    args.splits = plan.info.splits;
    args.sk_tiles = plan.info.sk_tiles;
    args.ws = (plan.info.splits > 1 || plan.info.sk_tiles > 0) ? ws : nullptr;

    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e);
    if (cur != h->device && (e = hipSetDevice(h->device)) != hipSuccess) return hip_fail(e);
    void* kargs[] = {&args};
    e = hipLaunchKernel(fn, dim3((unsigned)plan.info.grid), dim3((unsigned)plan.info.threads), kargs, 0,
                        (hipStream_t)stream);
    if (e == hipSuccess) e = hipGetLastError();
    if (cur != h->device) {
        // put the caller's device back; a failure here is reported unless
        // the launch itself already failed
        const hipError_t r = hipSetDevice(cur);
        if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return hip_fail(e);
    return GEMM_OK;
}

}  // namespace

extern "C" {

int gemm_create(gemm_handle_t* out, int device) {
    if (out == nullptr || device < 0) return GEMM_ERR_INVALID_ARG;
    *out = nullptr;
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess) return hip_fail(e);
    if (device >= count) return hip_fail(hipErrorInvalidDevice);
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess) return hip_fail(e);
    void* scr = nullptr;
    e = scratch_setup(device, &scr);
    if (e != hipSuccess) return hip_fail(e);
    gemm_handle_s* h = new (std::nothrow) gemm_handle_s;
    if (h == nullptr) return GEMM_ERR_INVALID_ARG;
    h->device = device;
    h->num_cus = cus > 0 ? cus : kDefaultCus;
    h->tile_override = GEMM_TILE_AUTO;
    h->scratch = scr;
    *out = h;
    return GEMM_OK;
}

int gemm_destroy(gemm_handle_t h) {
    delete h;
    return GEMM_OK;
}

int gemm_set_tile(gemm_handle_t h, int tile) {
    if (h == nullptr || tile < GEMM_TILE_AUTO || tile >= pg::TILE_COUNT) return GEMM_ERR_INVALID_ARG;
    h->tile_override = tile;
    return GEMM_OK;
}

int gemm_query_splitk(int64_t M, int64_t N, int64_t K, int dtype, int layout, int stages, int variant,
                      int tile, int splits, const void* A, int64_t lda, const void* B, int64_t ldb,
                      const void* C, int64_t ldc, gemm_config_info_t* info) {
    if (info == nullptr) return GEMM_ERR_INVALID_ARG;
    Plan plan;
    int rc = plan_call(M, N, K, dtype, layout, stages, variant, tile, splits, -1, A, lda, B, ldb, C, ldc,
                       kDefaultCus, true, &plan);
    if (rc == GEMM_OK) *info = plan.info;
    return rc;
}

int gemm_query_streamk(int64_t M, int64_t N, int64_t K, int dtype, int layout, int stages, int variant,
                       int tile, int grid, const void* A, int64_t lda, const void* B, int64_t ldb,
                       const void* C, int64_t ldc, gemm_config_info_t* info) {
    if (info == nullptr || grid < 0) return GEMM_ERR_INVALID_ARG;
    Plan plan;
    int rc = plan_call(M, N, K, dtype, layout, stages, variant, tile, 1, grid, A, lda, B, ldb, C, ldc,
                       kDefaultCus, true, &plan);
    if (rc == GEMM_OK) *info = plan.info;
    return rc;
}

int gemm_query(int64_t M, int64_t N, int64_t K, int dtype, int layout, int stages, int variant,
               int tile, const void* A, int64_t lda, const void* B, int64_t ldb, const void* C,
               int64_t ldc, gemm_config_info_t* info) {
    return gemm_query_splitk(M, N, K, dtype, layout, stages, variant, tile, 1, A, lda, B, ldb, C, ldc, info);
}

int gemm_run_splitk(gemm_handle_t h, int64_t M, int64_t N, int64_t K, int dtype, int layout, int stages,
                    int variant, int splits, const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                    int64_t ldc, void* workspace, int64_t workspace_bytes, void* stream) {
    if (h == nullptr || workspace_bytes < 0) return GEMM_ERR_INVALID_ARG;
    Plan plan;
    int rc = plan_call(M, N, K, dtype, layout, stages, variant, h->tile_override, splits, -1, A, lda, B, ldb, C,
                       ldc, h->num_cus, false, &plan);
    if (rc != GEMM_OK) return rc;
    if (plan.info.splits > 1) {
        if (workspace == nullptr || workspace_bytes < plan.info.workspace_bytes) return GEMM_ERR_INVALID_ARG;
        if (((uintptr_t)workspace & 255u) != 0) return GEMM_ERR_ALIGNMENT;
    }
    return launch(h, plan, M, N, K, dtype, layout, stages, A, lda, B, ldb, C, ldc, workspace, stream);
}

int gemm_run_streamk(gemm_handle_t h, int64_t M, int64_t N, int64_t K, int dtype, int layout, int stages,
                     int variant, int grid, const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                     int64_t ldc, void* workspace, int64_t workspace_bytes, void* stream) {
    if (h == nullptr || workspace_bytes < 0 || grid < 0) return GEMM_ERR_INVALID_ARG;
    Plan plan;
    int rc = plan_call(M, N, K, dtype, layout, stages, variant, h->tile_override, 1, grid, A, lda, B, ldb, C,
                       ldc, h->num_cus, false, &plan);
    if (rc != GEMM_OK) return rc;
    if (plan.info.sk_tiles > 0) {
        if (workspace == nullptr || workspace_bytes < plan.info.workspace_bytes) return GEMM_ERR_INVALID_ARG;
        if (((uintptr_t)workspace & 255u) != 0) return GEMM_ERR_ALIGNMENT;
    }
    return launch(h, plan, M, N, K, dtype, layout, stages, A, lda, B, ldb, C, ldc, workspace, stream);
}

int gemm_run_splitk_noalloc(gemm_handle_t h, int64_t M, int64_t N, int64_t K, int dtype, int layout,
                            int stages, int variant, int splits, const void* A, int64_t lda, const void* B,
                            int64_t ldb, void* C, int64_t ldc, void* stream) {
    if (h == nullptr) return GEMM_ERR_INVALID_ARG;
    Plan plan;
    int rc = plan_call(M, N, K, dtype, layout, stages, variant, h->tile_override, splits, -1, A, lda, B, ldb, C,
                       ldc, h->num_cus, false, &plan);
    if (rc != GEMM_OK) return rc;
    if (plan.info.workspace_bytes > (int64_t)GEMM_NOALLOC_SCRATCH_BYTES) return GEMM_ERR_SCRATCH;
    return launch(h, plan, M, N, K, dtype, layout, stages, A, lda, B, ldb, C, ldc, h->scratch, stream);
}

int gemm_run(gemm_handle_t h, int64_t M, int64_t N, int64_t K, int dtype, int layout, int stages,
             int variant, const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
             int64_t ldc, void* stream) {
    return gemm_run_splitk(h, M, N, K, dtype, layout, stages, variant, 1, A, lda, B, ldb, C, ldc, nullptr, 0,
                           stream);
}

int gemm_occupancy(gemm_handle_t h, int64_t M, int64_t N, int64_t K, int dtype, int layout, int stages,
                   int variant, gemm_occupancy_t* out) {
    if (h == nullptr || out == nullptr) return GEMM_ERR_INVALID_ARG;
    Plan plan;
    const int64_t ldb = layout == GEMM_LAYOUT_RR ? N : K;
    int rc = plan_call(M, N, K, dtype, layout, stages, variant, h->tile_override, 1, -1, nullptr, K, nullptr,
                       ldb, nullptr, N, h->num_cus, true, &plan);
    if (rc != GEMM_OK) return rc;
    const void* fn = registry().fn[dtype][layout][plan.tile][stages][plan.kernel_variant];
    if (fn == nullptr) return GEMM_ERR_UNSUPPORTED;
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e);
    if (cur != h->device && (e = hipSetDevice(h->device)) != hipSuccess) return hip_fail(e);
    hipFuncAttributes fa;
    int blocks = 0;
    e = hipFuncGetAttributes(&fa, fn);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fn, plan.info.threads, 0);
    if (cur != h->device) {
        const hipError_t r = hipSetDevice(cur);
        if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return hip_fail(e);
    memset(out, 0, sizeof *out);
    out->blocks_per_cu = blocks;
    out->waves_per_cu = blocks * (plan.info.threads / 64);
    out->num_regs = fa.numRegs;
    out->lds_bytes = (int32_t)fa.sharedSizeBytes;
    out->scratch_bytes = (int32_t)fa.localSizeBytes;
    out->threads = plan.info.threads;
    return GEMM_OK;
}

const char* gemm_status_string(int status) {
    switch (status) {
    case GEMM_OK: return "GEMM_OK";
    case GEMM_ERR_INVALID_ARG: return "GEMM_ERR_INVALID_ARG: invalid argument";
    case GEMM_ERR_ALIGNMENT: return "GEMM_ERR_ALIGNMENT: pointer, leading dimension or K not 16-byte aligned";
    case GEMM_ERR_UNSUPPORTED: return "GEMM_ERR_UNSUPPORTED: no kernel instance for this configuration";
    case GEMM_ERR_HIP: return "GEMM_ERR_HIP: HIP runtime error";
    case GEMM_ERR_SCRATCH:
        return "GEMM_ERR_SCRATCH: the split-K workspace this call needs exceeds the library's static scratch "
               "buffer (GEMM_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
    }
}

int gemm_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
